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
#include <cstdint>

#include "common.h"
#include "registry.h"

namespace e3k {

namespace {

constexpr int kScanBlock = 256;
constexpr int kScanItems = 4;
constexpr int kScanTile = kScanBlock * kScanItems;

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

// Breadth-first traversal over in-edges, one level per launch: every
// wavefront takes a node of the current level [lb, le) of `order` and claims
// its unvisited senders; claims are counted with one atomic per wavefront and
// appended to `order`.  The order inside a level depends on timing; it only
// decides which wavefront handles which node later, never a result.
__global__ void __launch_bounds__(256)
    k_bfs_expand(int n_nodes, int n_edges, const int* __restrict__ rowptr,
                 const int* __restrict__ sender, int* __restrict__ order,
                 int* __restrict__ visited, int* __restrict__ tail, int lb, int le) {
  const int lane = threadIdx.x & 63;
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
        if (claim) order[base + __popcll(mask & ((uint64_t(1) << lane) - 1))] = a;
      }
    }
  }
}

__global__ void k_bfs_seed(int* __restrict__ order, int* __restrict__ visited,
                           int* __restrict__ tail, int s) {
  order[0] = s;
  visited[s] = 1;
  *tail = 1;
}

// flag[i] = 1 for nodes the traversal did not reach (flag[n] = 0).
__global__ void __launch_bounds__(256)
    k_unvisited_flags(int n_nodes, const int* __restrict__ visited, int* __restrict__ flag) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i <= n_nodes;
       i += int64_t(gridDim.x) * blockDim.x)
    flag[i] = (i < n_nodes && !visited[i]) ? 1 : 0;
}

// Unreached nodes go after the traversal, in index order.
__global__ void __launch_bounds__(256)
    k_append_unvisited(int n_nodes, const int* __restrict__ visited, const int* __restrict__ pos,
                       int start, int* __restrict__ order) {
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
    float x = vec[3 * i], y = vec[3 * i + 1], z = vec[3 * i + 2];
    unit_vector(x, y, z);
    float h[D];
    sfor<0, LMAX + 1>([&](auto l) { harmonics_l<l>(x, y, z, h + l * l); });
#pragma unroll
    for (int k = 0; k < D; ++k) Y[i * D + k] = h[k];
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
  L.bsum = o;
  o += up((n_nodes + 1 + kScanTile - 1) / kScanTile + 1);
  L.total_words = o;
  return L;
}

// Traversal order of the nodes for the convolution kernels (ws + L.order):
// breadth-first from node 0 over in-edges, then every unreached node in
// index order.  Neighbouring nodes end up close in the order, so the
// wavefronts that run together gather overlapping node rows.  One host
// synchronisation per level (the level bounds come back to the host).
hipError_t build_locality_order(int n_nodes, int n_edges, const int* rowptr, const int* sender,
                                int* ws, const TransposeLayout& L, hipStream_t s) {
  int* order = ws + L.order;
  int* visited = ws + L.cursor;  // free once the buckets are ranked
  int* tail = ws + L.npad + 1;
  const int64_t n1 = int64_t(n_nodes) + 1;
  hipLaunchKernelGGL(k_fill, dim3(grid_for(n1, 256)), dim3(256), 0, s, visited, n1, 0);
  hipLaunchKernelGGL(k_bfs_seed, dim3(1), dim3(1), 0, s, order, visited, tail, 0);
  int lb = 0, le = 1, h_tail = 1;
  while (lb < le) {
    const unsigned g = unsigned(std::min<int64_t>((int64_t(le - lb) + 3) / 4, 1 << 16));
    hipLaunchKernelGGL(k_bfs_expand, dim3(g), dim3(256), 0, s, n_nodes, n_edges, rowptr, sender,
                       order, visited, tail, lb, le);
    hipError_t err = hipMemcpyAsync(&h_tail, tail, sizeof(int), hipMemcpyDeviceToHost, s);
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    if (err != hipSuccess) return err;
    if (h_tail < le || h_tail > n_nodes) return hipErrorUnknown;  // cannot happen
    lb = le;
    le = h_tail;
  }
  if (h_tail < n_nodes) {
    int* flag = ws + L.flag;
    hipLaunchKernelGGL(k_unvisited_flags, dim3(grid_for(n1, 256)), dim3(256), 0, s, n_nodes, visited,
                       flag);
    const unsigned tiles = unsigned((n1 + kScanTile - 1) / kScanTile);
    hipLaunchKernelGGL(k_scan_tiles, dim3(tiles), dim3(kScanBlock), 0, s, flag, n1, flag,
                       ws + L.bsum);
    hipLaunchKernelGGL(k_scan_tile_sums, dim3(1), dim3(kScanBlock), 0, s, ws + L.bsum, int(tiles));
    hipLaunchKernelGGL(k_scan_add, dim3(tiles), dim3(kScanBlock), 0, s, flag, n1, ws + L.bsum);
    hipLaunchKernelGGL(k_append_unvisited, dim3(grid_for(n_nodes, 256)), dim3(256), 0, s, n_nodes,
                       visited, flag, h_tail, order);
  }
  return hipGetLastError();
}

hipError_t launch_prepare_transpose(int n_nodes, int n_edges, const int* rowptr, const int* sender,
                                    int* ws, hipStream_t s) {
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
  return build_locality_order(n_nodes, n_edges, rowptr, sender, ws, L, s);
}

hipError_t launch_harmonics(int lmax, int64_t n, const float* vec, float* Y, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const dim3 g(grid_for(n, 256)), b(256);
  switch (lmax) {
    case 0: hipLaunchKernelGGL(k_harmonics<0>, g, b, 0, s, n, vec, Y); break;
    case 1: hipLaunchKernelGGL(k_harmonics<1>, g, b, 0, s, n, vec, Y); break;
    case 2: hipLaunchKernelGGL(k_harmonics<2>, g, b, 0, s, n, vec, Y); break;
    case 3: hipLaunchKernelGGL(k_harmonics<3>, g, b, 0, s, n, vec, Y); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace e3k
