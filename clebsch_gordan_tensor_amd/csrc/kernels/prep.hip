// Per-graph preparation of the sender-ordered (transposed) edge index used
// by the backward pass, and the standalone harmonics kernel.
//
// The transposed index is a counting sort of the receiver-sorted CSR by
// sender, stable in edge id:  colptr[a] .. colptr[a+1] list the out-edges
// of sender a in increasing edge id, perm[j] is the edge id and recv[j] its
// receiver (the sender-keyed traversal of the e3j paper, E.4 backward).
// Padding edges (sender < 0) are left out and collected in padlist.
// Integer atomics only serve to count and to bucket; the final order inside
// every bucket is fixed by a rank sort, so the index is deterministic.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <mutex>

#include "common.h"
#include "harmonics_hi.h"
#include "registry.h"

namespace e3k {

namespace {

constexpr int kScanBlock = 256;
constexpr int kScanItems = 4;
constexpr int kScanTile = kScanBlock * kScanItems;
constexpr int kCellBitsHost = 18;  // cells: 6 bits per axis, 262,144 cells
constexpr int kBfsLevels = 64;       // traversal launches (levels) per graph

__global__ void __launch_bounds__(256) k_fill(int* __restrict__ p, int64_t n, int v) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

__global__ void __launch_bounds__(256)
    k_count(int n_edges, int n_nodes, const int* __restrict__ sender, int* __restrict__ cnt) {
  for (int64_t e = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; e < n_edges;
       e += int64_t(gridDim.x) * blockDim.x) {
    const int a = sender[e];
    if (a >= 0 && a < n_nodes) atomicAdd(cnt + a, 1);
  }
}

// Exclusive scan, pass 1: each block scans one tile in LDS, writes the
// tile-local exclusive prefix and the tile total.
__global__ void __launch_bounds__(kScanBlock)
    k_scan_tiles(const int* in, int64_t n, int* out, int* __restrict__ tile_sum) {
  // in and out may be the same array: a thread reads its own items before
  // it writes them and never touches another thread's items
  __shared__ int s[kScanBlock];
  const int64_t base = int64_t(blockIdx.x) * kScanTile + int64_t(threadIdx.x) * kScanItems;
  int v[kScanItems], t = 0;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    v[i] = (base + i < n) ? in[base + i] : 0;
    t += v[i];
  }
  s[threadIdx.x] = t;
  __syncthreads();
  for (int d = 1; d < kScanBlock; d <<= 1) {  // Hillis-Steele inclusive scan
    const int add = threadIdx.x >= d ? s[threadIdx.x - d] : 0;
    __syncthreads();
    s[threadIdx.x] += add;
    __syncthreads();
  }
  int run = s[threadIdx.x] - t;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    if (base + i < n) out[base + i] = run;
    run += v[i];
  }
  if (threadIdx.x == kScanBlock - 1) tile_sum[blockIdx.x] = s[threadIdx.x];
}

// Pass 2: one block turns the tile totals into exclusive tile offsets.
__global__ void __launch_bounds__(kScanBlock) k_scan_tile_sums(int* __restrict__ ts, int n_tiles) {
  __shared__ int s[kScanBlock];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < n_tiles; base += kScanBlock) {
    const int i = base + threadIdx.x;
    const int v = i < n_tiles ? ts[i] : 0;
    s[threadIdx.x] = v;
    __syncthreads();
    for (int d = 1; d < kScanBlock; d <<= 1) {
      const int add = threadIdx.x >= d ? s[threadIdx.x - d] : 0;
      __syncthreads();
      s[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < n_tiles) ts[i] = carry + s[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == kScanBlock - 1) carry += s[threadIdx.x];
    __syncthreads();
  }
}

// Pass 3: add the tile offsets.
__global__ void __launch_bounds__(kScanBlock)
    k_scan_add(int* __restrict__ out, int64_t n, const int* __restrict__ ts) {
  const int64_t base = int64_t(blockIdx.x) * kScanTile;
  const int off = ts[blockIdx.x];
  for (int i = threadIdx.x; i < kScanTile; i += kScanBlock)
    if (base + i < n) out[base + i] += off;
}

// One wavefront per receiver b: every real edge goes to its sender's bucket
// (slot from an integer atomic, so the order inside a bucket is arbitrary
// here and fixed by k_rank_buckets); padding edges go to padlist.
__global__ void __launch_bounds__(256)
    k_bucket(int n_nodes, int n_edges, const int* __restrict__ rowptr, const int* __restrict__ sender,
             const int* __restrict__ colptr, int* __restrict__ cursor, int* __restrict__ tmp_e,
             int* __restrict__ tmp_b, int* __restrict__ npad, int* __restrict__ padlist) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= n_nodes) return;
  const int lane = threadIdx.x & 63;
  const int beg = max(rowptr[b], 0), end = min(rowptr[b + 1], n_edges);
  for (int e = beg + lane; e < end; e += 64) {
    const int a = sender[e];
    if (a < 0 || a >= n_nodes) {
      const int k = atomicAdd(npad, 1);
      if (k < n_edges) padlist[k] = e;
    } else {
      const int slot = colptr[a] + atomicAdd(cursor + a, 1);
      if (slot < colptr[a + 1]) {  // holds for a well-formed CSR
        tmp_e[slot] = e;
        tmp_b[slot] = b;
      }
    }
  }
}

// One wavefront per sender: rank every bucket entry by edge id (ids are
// unique) and place it; O(d^2) per bucket of d entries.
__global__ void __launch_bounds__(256)
    k_rank_buckets(int n_nodes, const int* __restrict__ colptr, const int* __restrict__ tmp_e,
                   const int* __restrict__ tmp_b, int* __restrict__ perm, int* __restrict__ recv) {
  const int a = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (a >= n_nodes) return;
  const int lane = threadIdx.x & 63;
  const int beg = colptr[a], end = colptr[a + 1];
  for (int i = beg + lane; i < end; i += 64) {
    const int e = tmp_e[i];
    int rank = 0;
    for (int j = beg; j < end; ++j) rank += tmp_e[j] < e ? 1 : 0;
    perm[beg + rank] = e;
    recv[beg + rank] = tmp_b[i];
  }
}

// Breadth-first traversal over in-edges, one level per launch, the level's
// bounds on the device: lev[i] .. lev[i+1] of `order`.  Every wavefront takes
// a node of the level and claims its unvisited senders; claims are counted
// with one atomic per wavefront and appended to `order`.  The last workgroup
// to finish (a counter of finished workgroups; nothing waits on it) writes
// lev[i+2], the end of the next level, so the host never reads a bound and
// the launches queue back to back.  The order inside a level depends on
// timing; it only decides which wavefront handles which node later, never a
// result.  When edge vectors are given, a claimed sender also gets a position
// relative to the root along the traversal tree: pos[a] = pos[u] - r_e
// (r_e = pos[receiver] - pos[sender]).
__global__ void __launch_bounds__(256)
    k_bfs_level(int n_nodes, int n_edges, const int* __restrict__ rowptr,
                const int* __restrict__ sender, const float* __restrict__ evec,
                float* __restrict__ pos, int* __restrict__ order, int* __restrict__ visited,
                int* __restrict__ tail, int* __restrict__ lev, int* __restrict__ done, int i) {
  const int lane = threadIdx.x & 63;
  const int lb = max(lev[i], 0), le = min(lev[i + 1], n_nodes);
  for (int f = lb + blockIdx.x * 4 + (threadIdx.x >> 6); f < le; f += gridDim.x * 4) {
    const int u = order[f];
    const int beg = max(rowptr[u], 0), end = min(rowptr[u + 1], n_edges);
    for (int e0 = beg; e0 < end; e0 += 64) {  // wave-uniform bounds
      const int e = e0 + lane;
      int a = -1;
      if (e < end) {
        a = sender[e];
        if (a < 0 || a >= n_nodes) a = -1;
      }
      const bool claim = a >= 0 && atomicExch(visited + a, 1) == 0;
      const uint64_t mask = __ballot(claim);
      if (mask) {
        int base = 0;
        if (lane == 0) base = atomicAdd(tail, __popcll(mask));
        base = __shfl(base, 0, 64);
        if (claim) {
          order[base + __popcll(mask & ((uint64_t(1) << lane) - 1))] = a;
          if (evec) {
            pos[3 * a] = pos[3 * u] - evec[3 * int64_t(e)];
            pos[3 * a + 1] = pos[3 * u + 1] - evec[3 * int64_t(e) + 1];
            pos[3 * a + 2] = pos[3 * u + 2] - evec[3 * int64_t(e) + 2];
          }
        }
      }
    }
  }
  __syncthreads();  // this workgroup's claims are issued
  if (threadIdx.x == 0) {
    __threadfence();
    if (atomicAdd(done, 1) == int(gridDim.x) - 1) {
      lev[i + 2] = atomicAdd(tail, 0);
      *done = 0;
    }
  }
}

__global__ void k_bfs_seed(int* __restrict__ order, int* __restrict__ visited,
                           int* __restrict__ tail, int* __restrict__ lev, int* __restrict__ done,
                           float* __restrict__ pos, int s) {
  order[0] = s;
  visited[s] = 1;
  *tail = 1;
  lev[0] = 0;
  lev[1] = 1;
  *done = 0;
  if (pos) pos[3 * s] = pos[3 * s + 1] = pos[3 * s + 2] = 0.0f;
}

// Order-preserving int key of a float (for atomic min/max).
__device__ __forceinline__ int fkey(float f) {
  const int i = __float_as_int(f);
  return i >= 0 ? i : i ^ 0x7FFFFFFF;
}
__device__ __forceinline__ float kfloat(int k) {
  return __int_as_float(k >= 0 ? k : k ^ 0x7FFFFFFF);
}

// Bounding box of the reconstructed positions of order[0 .. n).
__global__ void __launch_bounds__(256)
    k_bbox(const int* __restrict__ n_ptr, int n_max, const int* __restrict__ order,
           const float* __restrict__ pos, int* __restrict__ box /* min xyz, max xyz as fkey */) {
  const int n = min(*n_ptr, n_max);
  int lo[3] = {INT_MAX, INT_MAX, INT_MAX}, hi[3] = {INT_MIN, INT_MIN, INT_MIN};
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const int v = order[i];
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      const int k = fkey(pos[3 * v + d]);
      lo[d] = min(lo[d], k);
      hi[d] = max(hi[d], k);
    }
  }
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    atomicMin(box + d, lo[d]);
    atomicMax(box + 3 + d, hi[d]);
  }
}

// Spread the low 6 bits of v to every third bit.
// Index along the 3-d Hilbert curve of the cell (x, y, z) of a 64^3 grid,
// by Skilling's transpose method ("Programming the Hilbert curve", AIP
// Conf. Proc. 707, 2004): undo the curve's excess rotations and
// reflections level by level from the top bit, Gray-encode across the axes,
// then read the index off the bits of the three transposed coordinates,
// most significant level first with x's bit above y's above z's.
// Consecutive indices are face-adjacent cells, so a range of the order is a
// connected piece of space (a Morton range can jump across the box).
__device__ __forceinline__ int hilbert_key6(unsigned x, unsigned y, unsigned z) {
  unsigned X[3] = {x, y, z};
  for (unsigned q = 32u; q > 1u; q >>= 1) {
    const unsigned p = q - 1u;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (X[i] & q) {
        X[0] ^= p;
      } else {
        const unsigned t = (X[0] ^ X[i]) & p;
        X[0] ^= t;
        X[i] ^= t;
      }
    }
  }
  X[1] ^= X[0];
  X[2] ^= X[1];
  unsigned t = 0;
  for (unsigned q = 32u; q > 1u; q >>= 1)
    if (X[2] & q) t ^= q - 1u;
  int key = 0;
#pragma unroll
  for (int b = 0; b < 6; ++b)
#pragma unroll
    for (int i = 0; i < 3; ++i) key |= int(((X[i] ^ t) >> b) & 1u) << (3 * b + 2 - i);
  return key;
}

// Hilbert index of the cell of each reached node; counts per cell.
__global__ void __launch_bounds__(256)
    k_cell_keys(const int* __restrict__ n_ptr, int n_max, const int* __restrict__ order,
                  const float* __restrict__ pos, const int* __restrict__ box,
                  int* __restrict__ key, int* __restrict__ hist) {
  const int n = min(*n_ptr, n_max);
  float lo[3], inv[3];
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    lo[d] = kfloat(box[d]);
    const float ext = kfloat(box[3 + d]) - lo[d];
    inv[d] = ext > 0.0f ? 63.999f / ext : 0.0f;
  }
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const int v = order[i];
    unsigned q[3];
#pragma unroll
    for (int d = 0; d < 3; ++d)
      q[d] = unsigned(min(63, max(0, int((pos[3 * v + d] - lo[d]) * inv[d]))));
    const int c = hilbert_key6(q[0], q[1], q[2]);
    key[i] = c;
    atomicAdd(hist + c, 1);
  }
}

// Scatter order[0 .. n) into cell order (cells by Hilbert index; inside a
// cell the order depends on timing, which only affects scheduling).
__global__ void __launch_bounds__(256)
    k_cell_scatter(const int* __restrict__ n_ptr, int n_max, const int* __restrict__ order,
                     const int* __restrict__ key, const int* __restrict__ start,
                     int* __restrict__ cursor, int* __restrict__ out) {
  const int n = min(*n_ptr, n_max);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const int c = key[i];
    const int k = start[c] + atomicAdd(cursor + c, 1);
    if (k < n) out[k] = order[i];
  }
}

__global__ void __launch_bounds__(256)
    k_copy_i32(const int* __restrict__ src, int* __restrict__ dst, const int* __restrict__ n_ptr,
               int n_max) {
  const int n = min(*n_ptr, n_max);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// flag[i] = 1 for nodes the traversal did not reach (flag[n] = 0).
__global__ void __launch_bounds__(256)
    k_unvisited_flags(int n_nodes, const int* __restrict__ visited, int* __restrict__ flag) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i <= n_nodes;
       i += int64_t(gridDim.x) * blockDim.x)
    flag[i] = (i < n_nodes && !visited[i]) ? 1 : 0;
}

// Unreached nodes go after the traversal (which reached *start nodes), in
// index order.
__global__ void __launch_bounds__(256)
    k_append_unvisited(int n_nodes, const int* __restrict__ visited, const int* __restrict__ pos,
                       const int* __restrict__ start_ptr, int* __restrict__ order) {
  const int start = *start_ptr;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n_nodes;
       i += int64_t(gridDim.x) * blockDim.x)
    if (!visited[i]) {
      const int k = start + pos[i];
      if (k < n_nodes) order[k] = int(i);
    }
}

template <int LMAX>
__global__ void __launch_bounds__(256)
    k_harmonics(int64_t n, const float* __restrict__ vec, float* __restrict__ Y) {
  constexpr int D = (LMAX + 1) * (LMAX + 1);
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x) {
    float h[D];
    harmonics_bank_of_vec_f64<LMAX>(vec[3 * i], vec[3 * i + 1], vec[3 * i + 2], h);
#pragma unroll
    for (int k = 0; k < D; ++k) Y[i * D + k] = h[k];
  }
}

// Gradient of the harmonics with respect to the unnormalised vector:
// dvec[i] = sum_k dY[i][k] dY_k/dr.  The polynomials of the unit vector u
// are differentiated by forward-mode arithmetic (dual numbers), and the chain
// rule through u = r/|r| projects out the radial part: dY/dr = (I - u u^T)
// dY/du / |r|.  Evaluated in fp64 and rounded once.  A zero vector gets 0.
template <int LMAX>
__global__ void __launch_bounds__(256)
    k_harmonics_grad(int64_t n, const float* __restrict__ vec, const float* __restrict__ dY,
                     float* __restrict__ dvec) {
  constexpr int D = (LMAX + 1) * (LMAX + 1);
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x) {
    double x = vec[3 * i], y = vec[3 * i + 1], z = vec[3 * i + 2];
    double g0 = 0.0, g1 = 0.0, g2 = 0.0;
    const double n2 = x * x + y * y + z * z;
    if (n2 > 0.0) {
      const double r = sqrt(n2), inv = 1.0 / r;
      x *= inv;
      y *= inv;
      z *= inv;
      const float* gy = dY + i * D;
      harmonics_grad_bank<LMAX>(x, y, z, [&](int k) { return gy[k]; }, g0, g1, g2);
      const double ug = x * g0 + y * g1 + z * g2;
      g0 = (g0 - x * ug) / r;
      g1 = (g1 - y * ug) / r;
      g2 = (g2 - z * ug) / r;
    }
    dvec[3 * i] = float(g0);
    dvec[3 * i + 1] = float(g1);
    dvec[3 * i + 2] = float(g2);
  }
}

// Position gradient from edge-vector gradients g[E][3], with r_e =
// pos[recv] - pos[sender]: dpos[b] = sum of g over b's in-edges (its CSR
// row) minus the sum over its out-edges (its column of the transposed
// index).  One wavefront per node; lanes take edges in a fixed stride and
// close with a fixed butterfly, so the result is reproducible.  Padding
// edges (sender outside [0, N)) are skipped.
__global__ void __launch_bounds__(256)
    k_edge_grad_to_nodes(int n_nodes, int n_edges, const int* __restrict__ rowptr,
                         const int* __restrict__ sender, const int* __restrict__ colptr,
                         const int* __restrict__ perm, const float* __restrict__ g,
                         float* __restrict__ dpos) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= n_nodes) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f;
  const int beg = max(rowptr[b], 0), end = min(rowptr[b + 1], n_edges);
  for (int e = beg + lane; e < end; e += 64) {
    const int a = sender[e];
    if (a < 0 || a >= n_nodes) continue;
    s0 += g[3 * int64_t(e)];
    s1 += g[3 * int64_t(e) + 1];
    s2 += g[3 * int64_t(e) + 2];
  }
  const int cb = max(colptr[b], 0), ce = min(colptr[b + 1], n_edges);
  for (int j = cb + lane; j < ce; j += 64) {
    const int e = perm[j];
    if (e < 0 || e >= n_edges) continue;
    s0 -= g[3 * int64_t(e)];
    s1 -= g[3 * int64_t(e) + 1];
    s2 -= g[3 * int64_t(e) + 2];
  }
  sfor<0, 6>([&](auto k) {
    constexpr int m = 32 >> k;
    s0 += shfl_xor_c<m>(s0);
    s1 += shfl_xor_c<m>(s1);
    s2 += shfl_xor_c<m>(s2);
  });
  if (lane == 0) {
    dpos[3 * int64_t(b)] = s0;
    dpos[3 * int64_t(b) + 1] = s1;
    dpos[3 * int64_t(b) + 2] = s2;
  }
}

unsigned grid_for(int64_t n, int per_block) {
  int64_t g = (n + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > (1 << 20)) g = 1 << 20;
  return unsigned(g);
}

}  // namespace

TransposeLayout transpose_layout(int64_t n_nodes, int64_t n_edges) {
  auto up = [](int64_t v) { return (v + 63) / 64 * 64; };  // 256-byte alignment
  TransposeLayout L{};
  int64_t o = 0;
  L.npad = o;
  o += 64;
  L.colptr = o;
  o += up(n_nodes + 1);
  L.cursor = o;
  o += up(n_nodes + 1);
  L.tmp_e = o;
  o += up(n_edges);
  L.tmp_b = o;
  o += up(n_edges);
  L.perm = o;
  o += up(n_edges);
  L.recv = o;
  o += up(n_edges);
  L.padlist = o;
  o += up(n_edges);
  L.order = o;
  o += up(n_nodes);
  L.flag = o;
  o += up(n_nodes + 1);
  L.pos = o;
  o += up(3 * n_nodes);
  L.key = o;
  o += up(n_nodes);
  L.order2 = o;
  o += up(n_nodes);
  L.box = o;
  o += 64;
  L.levels = o;
  o += up(kBfsLevels + 2);
  L.cell = o;
  o += up((int64_t(1) << kCellBitsHost) + 1);
  L.cell_cursor = o;
  o += up(int64_t(1) << kCellBitsHost);
  L.bsum = o;
  // tile sums of the largest scan (the cell counts or the node counts)
  o += up((std::max<int64_t>(n_nodes + 1, (int64_t(1) << kCellBitsHost) + 1) + kScanTile - 1) /
              kScanTile +
          1);
  L.total_words = o;
  return L;
}

// Traversal order of the nodes for the convolution kernels (ws + L.order):
// breadth-first from node 0 over in-edges; with edge vectors, the reached
// nodes are then re-sorted by the Hilbert-curve cell of their position rebuilt
// along the traversal tree; every unreached node follows in index order.
// Neighbouring nodes end up close in the order, so the wavefronts that run
// together gather overlapping node rows.  Nothing comes back to the host:
// the traversal is kBfsLevels launches whose level bounds live on the device
// (levels past the graph's depth are empty launches; nodes deeper than that
// join the unreached ones), and every later step reads the reached count
// from the device.
hipError_t build_locality_order(int n_nodes, int n_edges, const int* rowptr, const int* sender,
                                const float* evec, int* ws, const TransposeLayout& L,
                                hipStream_t s) {
  int* order = ws + L.order;
  int* visited = ws + L.cursor;  // free once the buckets are ranked
  int* tail = ws + L.npad + 1;
  int* done = ws + L.npad + 2;
  int* lev = ws + L.levels;
  float* pos = evec ? reinterpret_cast<float*>(ws + L.pos) : nullptr;
  const int64_t n1 = int64_t(n_nodes) + 1;
  hipLaunchKernelGGL(k_fill, dim3(grid_for(n1, 256)), dim3(256), 0, s, visited, n1, 0);
  hipLaunchKernelGGL(k_bfs_seed, dim3(1), dim3(1), 0, s, order, visited, tail, lev, done, pos, 0);
  // enough workgroups for a wide level, few enough that an empty one is cheap
  const unsigned g = unsigned(std::min<int64_t>((int64_t(n_nodes) + 63) / 64, 512));
  const int levels = int(std::min<int64_t>(kBfsLevels, n_nodes));
  for (int i = 0; i < levels; ++i)
    hipLaunchKernelGGL(k_bfs_level, dim3(g), dim3(256), 0, s, n_nodes, n_edges, rowptr, sender,
                       evec, pos, order, visited, tail, lev, done, i);
  const unsigned gn = grid_for(n_nodes, 256);
  if (pos) {
    // spatially compact order of the reached nodes: Hilbert cells of the
    // reconstructed positions, counting-sorted
    int* box = ws + L.box;
    int* key = ws + L.key;
    int* cell = ws + L.cell;
    int* cur = ws + L.cell_cursor;
    const int64_t ncell = int64_t(1) << kCellBitsHost;
    hipLaunchKernelGGL(k_fill, dim3(1), dim3(64), 0, s, box, int64_t(3), INT_MAX);
    hipLaunchKernelGGL(k_fill, dim3(1), dim3(64), 0, s, box + 3, int64_t(3), INT_MIN);
    hipLaunchKernelGGL(k_fill, dim3(grid_for(ncell + 1, 256)), dim3(256), 0, s, cell, ncell + 1, 0);
    hipLaunchKernelGGL(k_fill, dim3(grid_for(ncell, 256)), dim3(256), 0, s, cur, ncell, 0);
    hipLaunchKernelGGL(k_bbox, dim3(gn), dim3(256), 0, s, tail, n_nodes, order, pos, box);
    hipLaunchKernelGGL(k_cell_keys, dim3(gn), dim3(256), 0, s, tail, n_nodes, order, pos, box,
                       key, cell);
    const unsigned tiles = unsigned((ncell + 1 + kScanTile - 1) / kScanTile);
    hipLaunchKernelGGL(k_scan_tiles, dim3(tiles), dim3(kScanBlock), 0, s, cell, ncell + 1, cell,
                       ws + L.bsum);
    hipLaunchKernelGGL(k_scan_tile_sums, dim3(1), dim3(kScanBlock), 0, s, ws + L.bsum, int(tiles));
    hipLaunchKernelGGL(k_scan_add, dim3(tiles), dim3(kScanBlock), 0, s, cell, ncell + 1,
                       ws + L.bsum);
    hipLaunchKernelGGL(k_cell_scatter, dim3(gn), dim3(256), 0, s, tail, n_nodes, order, key, cell,
                       cur, ws + L.order2);
    hipLaunchKernelGGL(k_copy_i32, dim3(gn), dim3(256), 0, s, ws + L.order2, order, tail, n_nodes);
  }
  {
    int* flag = ws + L.flag;
    hipLaunchKernelGGL(k_unvisited_flags, dim3(grid_for(n1, 256)), dim3(256), 0, s, n_nodes, visited,
                       flag);
    const unsigned tiles = unsigned((n1 + kScanTile - 1) / kScanTile);
    hipLaunchKernelGGL(k_scan_tiles, dim3(tiles), dim3(kScanBlock), 0, s, flag, n1, flag,
                       ws + L.bsum);
    hipLaunchKernelGGL(k_scan_tile_sums, dim3(1), dim3(kScanBlock), 0, s, ws + L.bsum, int(tiles));
    hipLaunchKernelGGL(k_scan_add, dim3(tiles), dim3(kScanBlock), 0, s, flag, n1, ws + L.bsum);
    hipLaunchKernelGGL(k_append_unvisited, dim3(gn), dim3(256), 0, s, n_nodes, visited, flag, tail,
                       order);
  }
  return hipGetLastError();
}

hipError_t launch_prepare_transpose(int n_nodes, int n_edges, const int* rowptr, const int* sender,
                                    const float* evec, int* ws, hipStream_t s) {
  const TransposeLayout L = transpose_layout(n_nodes, n_edges);
  int* npad = ws + L.npad;
  int* colptr = ws + L.colptr;
  int* cnt = ws + L.cursor;
  const int64_t n1 = int64_t(n_nodes) + 1;
  // counts (cnt[n_nodes] stays 0, so the exclusive scan ends with the total)
  hipLaunchKernelGGL(k_fill, dim3(grid_for(n1, 256)), dim3(256), 0, s, cnt, n1, 0);
  hipLaunchKernelGGL(k_fill, dim3(1), dim3(64), 0, s, npad, int64_t(1), 0);
  if (n_edges > 0)
    hipLaunchKernelGGL(k_count, dim3(grid_for(n_edges, 256)), dim3(256), 0, s, n_edges, n_nodes,
                       sender, cnt);
  const unsigned tiles = unsigned((n1 + kScanTile - 1) / kScanTile);
  hipLaunchKernelGGL(k_scan_tiles, dim3(tiles), dim3(kScanBlock), 0, s, cnt, n1, colptr,
                     ws + L.bsum);
  hipLaunchKernelGGL(k_scan_tile_sums, dim3(1), dim3(kScanBlock), 0, s, ws + L.bsum, int(tiles));
  hipLaunchKernelGGL(k_scan_add, dim3(tiles), dim3(kScanBlock), 0, s, colptr, n1, ws + L.bsum);
  if (n_nodes > 0 && n_edges > 0) {
    hipLaunchKernelGGL(k_fill, dim3(grid_for(n1, 256)), dim3(256), 0, s, cnt, n1, 0);
    const unsigned wb = unsigned((int64_t(n_nodes) + 3) / 4);
    hipLaunchKernelGGL(k_fill, dim3(grid_for(n_edges, 256)), dim3(256), 0, s, ws + L.tmp_e,
                       int64_t(n_edges), -1);
    hipLaunchKernelGGL(k_bucket, dim3(wb), dim3(256), 0, s, n_nodes, n_edges, rowptr, sender,
                       colptr, cnt,
                       ws + L.tmp_e, ws + L.tmp_b, npad, ws + L.padlist);
    hipLaunchKernelGGL(k_rank_buckets, dim3(wb), dim3(256), 0, s, n_nodes, colptr, ws + L.tmp_e,
                       ws + L.tmp_b, ws + L.perm, ws + L.recv);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || n_nodes == 0) return err;
  return build_locality_order(n_nodes, n_edges, rowptr, sender, evec, ws, L, s);
}

// ------------------------------------------------ fixed scratch (no allocation)
//
// The index of e3_conv_backward_noalloc lives in one file-scope device array
// sized for kNoAllocMaxNodes nodes and kNoAllocMaxEdges edges (each GPU the
// library runs on holds its own copy until the process ends).  Host code
// never uses the array's name as an address: its device address is fetched
// once per device with hipGetSymbolAddress and kept.

namespace {

// transpose_layout's arrays at the limits (five per edge, nine per node, the
// cell counts twice, plus alignment); the entry point checks the layout of
// every call against it
constexpr int64_t kNoAllocWords =
    (int64_t(5) * kNoAllocMaxEdges + int64_t(9) * kNoAllocMaxNodes +
     2 * (int64_t(1) << kCellBitsHost) + 16384 + 63) / 64 * 64;

__device__ __align__(256) int scratch[kNoAllocWords];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

int64_t noalloc_scratch_words() { return kNoAllocWords; }

hipError_t noalloc_scratch(int** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<int*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_harmonics(int lmax, int64_t n, const float* vec, float* Y, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const dim3 g(grid_for(n, 256)), b(256);
  switch (lmax) {
    case 0: hipLaunchKernelGGL(k_harmonics<0>, g, b, 0, s, n, vec, Y); break;
    case 1: hipLaunchKernelGGL(k_harmonics<1>, g, b, 0, s, n, vec, Y); break;
    case 2: hipLaunchKernelGGL(k_harmonics<2>, g, b, 0, s, n, vec, Y); break;
    case 3: hipLaunchKernelGGL(k_harmonics<3>, g, b, 0, s, n, vec, Y); break;
    case 4: hipLaunchKernelGGL(k_harmonics<4>, g, b, 0, s, n, vec, Y); break;
    case 5: hipLaunchKernelGGL(k_harmonics<5>, g, b, 0, s, n, vec, Y); break;
    case 6: hipLaunchKernelGGL(k_harmonics<6>, g, b, 0, s, n, vec, Y); break;
    case 7: hipLaunchKernelGGL(k_harmonics<7>, g, b, 0, s, n, vec, Y); break;
    case 8: hipLaunchKernelGGL(k_harmonics<8>, g, b, 0, s, n, vec, Y); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_harmonics_grad(int lmax, int64_t n, const float* vec, const float* dY,
                                 float* dvec, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const dim3 g(grid_for(n, 256)), b(256);
  switch (lmax) {
    case 0: hipLaunchKernelGGL(k_harmonics_grad<0>, g, b, 0, s, n, vec, dY, dvec); break;
    case 1: hipLaunchKernelGGL(k_harmonics_grad<1>, g, b, 0, s, n, vec, dY, dvec); break;
    case 2: hipLaunchKernelGGL(k_harmonics_grad<2>, g, b, 0, s, n, vec, dY, dvec); break;
    case 3: hipLaunchKernelGGL(k_harmonics_grad<3>, g, b, 0, s, n, vec, dY, dvec); break;
    case 4: hipLaunchKernelGGL(k_harmonics_grad<4>, g, b, 0, s, n, vec, dY, dvec); break;
    case 5: hipLaunchKernelGGL(k_harmonics_grad<5>, g, b, 0, s, n, vec, dY, dvec); break;
    case 6: hipLaunchKernelGGL(k_harmonics_grad<6>, g, b, 0, s, n, vec, dY, dvec); break;
    case 7: hipLaunchKernelGGL(k_harmonics_grad<7>, g, b, 0, s, n, vec, dY, dvec); break;
    case 8: hipLaunchKernelGGL(k_harmonics_grad<8>, g, b, 0, s, n, vec, dY, dvec); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_edge_grad_to_nodes(int n_nodes, int n_edges, const int* rowptr,
                                     const int* sender, const int* ws, const float* g,
                                     float* dpos, hipStream_t s) {
  if (n_nodes <= 0) return hipSuccess;
  const TransposeLayout L = transpose_layout(n_nodes, n_edges);
  hipLaunchKernelGGL(k_edge_grad_to_nodes, dim3(unsigned((int64_t(n_nodes) + 3) / 4)), dim3(256),
                     0, s, n_nodes, n_edges, rowptr, sender, ws + L.colptr, ws + L.perm, g, dpos);
  return hipGetLastError();
}

// dst[i] += src[i] for n elements of float or bf16 storage (fp32 sum,
// one rounding for bf16).
template <class T>
__global__ void __launch_bounds__(256)
    k_add(int64_t n, T* __restrict__ dst, const T* __restrict__ src) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x) {
    float a[1], b[1];
    load_ch<T, 1>(dst + i, a);
    load_ch<T, 1>(src + i, b);
    a[0] += b[0];
    store_ch<T, 1>(dst + i, a);
  }
}

hipError_t launch_add(void* dst, const void* src, int64_t n, int bf16, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const dim3 g(grid_for(n, 256)), b(256);
  if (bf16)
    hipLaunchKernelGGL(k_add<bf16_t>, g, b, 0, s, n, static_cast<bf16_t*>(dst),
                       static_cast<const bf16_t*>(src));
  else
    hipLaunchKernelGGL(k_add<float>, g, b, 0, s, n, static_cast<float*>(dst),
                       static_cast<const float*>(src));
  return hipGetLastError();
}

}  // namespace e3k
