// The channel-wise tensor product of high degree as dense products on the
// fp32 matrix cores.
//
// e3j (E.1, Eq.10-11) forms, per path P = (l1, l2 -> L) and channel q,
//   z_P[M][q] = sum_{m1,m2} C_P[M][m1][m2] y[m2] x[l1,m1][q],
// weights it per channel, z[L][M][q] += w[P][q] z_P[M][q], and sums the paths
// of each output block.  The coefficient sum over m2 does not depend on the
// channel: A_P[M][m1] = sum_{m2} C_P[M][m1][m2] y[m2] is one small matrix per
// row.  Folding the weight into x, xt_P[m1][q] = w[P][q] x[l1,m1][q], turns
// each output block into one matrix product over the concatenated (P, m1):
//   z[L][M][q] = sum_{(P,m1): P -> L} A_L[M][(P,m1)] xt[(P,m1)][q].
// The product runs on v_mfma_f32_16x16x4f32 (fp32 operands, exact products,
// fp32 accumulation): A_L is built per row in LDS, xt is formed per lane from
// the row's x and w staged in LDS, so the per-channel arithmetic is one
// multiply per product term instead of a walk over the coefficient records.
//
// Plan (host-built, see the GEMM table of the library):
//   header kGemmHeader words: magic, n_blocks, dx, dy, dout, P, n_klist,
//     n_groups, 0, a_floats, off_blocks, off_klist, off_groups, plan words
//   blocks [n_blocks][4]: output offset, rows (2L+1, at most 16: a degree-8
//     block is two, of 16 and 1 rows, on one K list), K-list start, K (x4)
//   klist  [n_klist]: (P << 16) | x component, or -1 for a padding column
//   groups [n_groups][4] in increasing A index: A index (block base + k * rows + M), the two y
//     components (y1 | y2 << 16), the two coefficients' bits (a real-basis
//     entry A[M][m1] couples at most two m2; an unused second term has c = 0)
// A is stored block after block, each transposed (A[k][M], stride rows;
// the MFMA's rows past them read zero), so a k-step's 64 reads fall in
// distinct banks; the staged x and w rows have a stride of 16 (mod 32)
// floats for the same reason (the four k of a step read four rows).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "harmonics_hi.h"
#include "registry.h"

namespace e3k {
namespace {

typedef float float4v __attribute__((ext_vector_type(4)));

// K steps [0, K) of one output block for NU tiles: D[u] += A[k][M] xt[k][c].
// Four steps per batch, all their LDS reads issued before the products (the
// w and x reads depend on the K-list read, so one step alone waits twice);
// BATCH = false keeps one step at a time (fewer registers).
template <int NU, bool BATCH = true>
__device__ __forceinline__ void gemm_ksteps(float4v (&D)[NU], const float* ap, const int* kp,
                                            int rows, bool aok, int K, const float* sw,
                                            const float* sx) {
  int k0 = 0;
  for (; BATCH && k0 + 16 <= K; k0 += 16) {
    int ent[4];
    float av[4], wv[4][NU], xv[4][NU];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ent[j] = kp[k0 + 4 * j];
      av[j] = ap[(k0 + 4 * j) * rows];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int wo = ent[j] & 0xFFFF, xo = int(unsigned(ent[j]) >> 16);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        wv[j][u] = sw[wo + 64 * u];
        xv[j][u] = sx[xo + 64 * u];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = aok ? av[j] : 0.0f;
#pragma unroll
      for (int u = 0; u < NU; ++u)
        D[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, wv[j][u] * xv[j][u], D[u], 0, 0, 0);
    }
  }
  for (; k0 < K; k0 += 4) {
    const float av = ap[k0 * rows];
    const float a = aok ? av : 0.0f;
    const int ent = kp[k0];
    const int wo = ent & 0xFFFF, xo = int(unsigned(ent) >> 16);
#pragma unroll
    for (int u = 0; u < NU; ++u)
      D[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sw[wo + 64 * u] * sx[xo + 64 * u], D[u], 0,
                                                  0, 0);
  }
}

// One workgroup (four wavefronts) per (row, slab of CS channels), rows in a
// grid-stride sequence.  LDS: A for every block (a_floats), the slab's x
// [dx][CS] and w [P][CS], the row's y and the K list.  A wavefront takes the
// NU 16-channel tiles wave, wave + 4 of the slab.  The sizes come from the
// host (built from the descriptor); every index read from the plan is
// clamped to them, so a plan of another descriptor gives wrong values but no
// access outside the arrays.
// PRE: 16-byte units per thread loaded one item ahead (12 for plans whose
// LDS leaves at most two workgroups per CU; 0 keeps the registers low so that
// small plans run more workgroups per CU).
// Windows of whole blocks over A, each starting at the first block that does
// not fit in the previous one (the partition the block loops walk), and,
// the plans' entries being sorted by A index, each window's run of entries:
// wq[i] = the first entry whose index is at least window i's start, wq[n] =
// n_groups; starts (if given) receives each window's A offset.  Run by one
// thread once per workgroup; returns the number of windows found (at most
// kMaxWindows: later windows scan every entry).
constexpr int kMaxWindows = 15;
template <class SizeOf>
__device__ int window_runs(int n_blocks, SizeOf size_of, int a_floats, int AW,
                           const int4* __restrict__ groups, int n_groups, int* wq,
                           int* starts = nullptr) {
  int nw = 0, abase = 0, w1 = 0;
  for (int b = 0; b < n_blocks && nw < kMaxWindows; ++b) {
    const int sz = size_of(b);
    if (abase + sz > a_floats) break;
    if (abase + sz > w1) {
      w1 = abase + AW;
      int lo = 0, hi = n_groups;  // first entry with index >= abase
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (groups[mid].x < abase) lo = mid + 1; else hi = mid;
      }
      if (starts) starts[nw] = abase;
      wq[nw++] = lo;
    }
    abase += sz;
  }
  wq[nw] = n_groups;
  return nw;
}

// WIN: A in windows of whole blocks (g.a_win > 0), built as the block loop
// reaches them; this form alone carries the window code.
template <int PRE, int NU, bool WIN>
__global__ void __launch_bounds__(256) k_tp_gemm(TpGemmArgs g) {
  extern __shared__ __align__(16) float gsm[];
  const int AW = WIN && g.a_win > 0 ? min(g.a_win, g.a_floats) : g.a_floats;
  const int* __restrict__ blocks = g.plan + g.off_blocks;
  const int* __restrict__ klist = g.plan + g.off_klist;
  const int4* __restrict__ groups = reinterpret_cast<const int4*>(g.plan + g.off_groups);
  const int CS = g.CS, C = g.C, XS = gemm_row_stride(CS);
  const int lg4 = __builtin_ctz(CS / 4);  // CS is a power of two
  float* s_a = gsm;
  float* s_x = s_a + AW;
  float* s_w = s_x + g.dx * XS;  // P rows and a zero row (the padding columns' weight)
  float* s_y = s_w + (g.P + 1) * XS;
  int* s_k = reinterpret_cast<int*>(s_y + g.dy);
  // the K list as LDS offsets of its w and x rows (clamped here, once)
  for (int i = threadIdx.x; i < g.n_klist; i += 256) {
    const int ent = klist[i];
    const int p = ent < 0 ? g.P : min(ent >> 16, g.P - 1);
    const int xi = ent < 0 ? 0 : min(ent & 0xFFFF, g.dx - 1);
    s_k[i] = p * XS | (xi * XS) << 16;
  }
  for (int i = threadIdx.x; i < XS; i += 256) s_w[g.P * XS + i] = 0.0f;
  // A's entries outside the plan's groups stay zero: every row (edge)
  // rewrites all the others, so A is cleared once (a window, per window)
  for (int i = threadIdx.x; i < AW; i += 256) s_a[i] = 0.0f;
  int* s_wq = s_k + g.n_klist;  // windows: their runs of entries, then their count
  if (WIN && threadIdx.x == 0) {
    auto size_of = [&](int b) {
      const int rows = min(max(blocks[4 * b + 1], 1), 16);
      const int kb = min(max(blocks[4 * b + 2], 0), g.n_klist);
      return rows * (min(max(blocks[4 * b + 3], 0), g.n_klist - kb) & ~3);
    };
    s_wq[kMaxWindows + 1] = window_runs(g.n_blocks, size_of, g.a_floats, AW, groups, g.n_groups, s_wq);
  }
  // wave-uniform (a scalar), so the tile tests below are scalar branches
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, kq = lane >> 4;
  const int n_slabs = C / CS, n_tiles = CS / 16;
  const bool active = wave < n_tiles;  // tiles wave + 4u, u < NU (n_tiles = 4 NU or fewer than 4)
  const int64_t n_items = g.n_rows * n_slabs;
  // The slab of x and w is 16-byte units u < U (x rows first): the first
  // 256 * PRE of them are loaded for the next item into registers while this
  // item's products run, the rest when the item is staged.
  const int U = (g.dx + g.P) << lg4;
  auto unit_src = [&](int u, int64_t row, int c0) {
    const int r = u >> lg4, c = 4 * (u & ((1 << lg4) - 1));
    return r < g.dx ? g.x + (row * g.dx + r) * C + c0 + c
                    : g.w + (row * g.P + (r - g.dx)) * C + c0 + c;
  };
  auto unit_dst = [&](int u) {
    const int r = u >> lg4, c = 4 * (u & ((1 << lg4) - 1));
    return r < g.dx ? s_x + r * XS + c : s_w + (r - g.dx) * XS + c;
  };
  float4v pre[PRE > 0 ? PRE : 1];
  float ypre = 0.0f;
  auto prefetch = [&](int64_t item) {
    const int64_t row = item / n_slabs;
    const int c0 = int(item - row * n_slabs) * CS;
#pragma unroll
    for (int j = 0; j < PRE; ++j) {
      const int u = threadIdx.x + 256 * j;
      if (u < U) pre[j] = *reinterpret_cast<const float4v*>(unit_src(u, row, c0));
    }
    if (threadIdx.x < g.dy) ypre = g.y[row * g.dy + threadIdx.x];
  };
  if (PRE > 0 && blockIdx.x < n_items) prefetch(blockIdx.x);
  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int64_t row = item / n_slabs;
    const int c0 = int(item - row * n_slabs) * CS;
    __syncthreads();  // the previous item's LDS reads are done (and s_k is written)
    // stage the slab of x and w and the row's y
#pragma unroll
    for (int j = 0; j < PRE; ++j) {
      const int u = threadIdx.x + 256 * j;
      if (u < U) *reinterpret_cast<float4v*>(unit_dst(u)) = pre[j];
    }
    for (int u = threadIdx.x + 256 * PRE; u < U; u += 256)
      *reinterpret_cast<float4v*>(unit_dst(u)) = *reinterpret_cast<const float4v*>(unit_src(u, row, c0));
    for (int i = threadIdx.x; i < g.dy; i += 256)
      s_y[i] = PRE > 0 && i < 256 ? ypre : g.y[row * g.dy + i];
    __syncthreads();
    // A[k][M] = c1 y[y1] + c2 y[y2]: one independent 16-byte load per entry
    // (in a window: the entries with A index in [a0, a1) at index - a0)
    auto build_a = [&](int a0, int a1, int q0, int q1) {
#pragma unroll 4
      for (int q = q0 + threadIdx.x; q < q1; q += 256) {
        const int4 e = groups[q];
        const int at = min(max(e.x, 0), g.a_floats - 1);
        const int y1 = min(e.y & 0xFFFF, g.dy - 1), y2 = min((e.y >> 16) & 0xFFFF, g.dy - 1);
        if (!WIN || (at >= a0 && at < a1))
          s_a[at - a0] = fmaf(__int_as_float(e.w), s_y[y2], __int_as_float(e.z) * s_y[y1]);
      }
    };
    if (!WIN) {
      build_a(0, g.a_floats, 0, g.n_groups);
      __syncthreads();
    }
    // the next item's operands load while this item's products run
    if (PRE > 0 && item + gridDim.x < n_items) prefetch(item + gridDim.x);
    int abase = 0, w0 = 0, w1 = WIN ? 0 : g.a_floats;  // A offsets [w0, w1) in LDS
    int wi = 0;                                          // window number
    for (int b = 0; b < g.n_blocks; ++b) {
      const int oo = blocks[4 * b], rows = min(max(blocks[4 * b + 1], 1), 16);
      const int kb = min(max(blocks[4 * b + 2], 0), g.n_klist);
      const int K = min(max(blocks[4 * b + 3], 0), g.n_klist - kb) & ~3;
      if (abase + rows * K > g.a_floats) break;
      if (WIN && abase + rows * K > w1) {  // the next window starts at this block (uniform)
        if (rows * K > AW) break;          // a block larger than the window: not built
        w0 = abase;
        w1 = abase + AW;
        __syncthreads();  // the previous window's reads are done
        for (int i = threadIdx.x; i < AW; i += 256) s_a[i] = 0.0f;
        __syncthreads();
        const int nw = s_wq[kMaxWindows + 1];
        if (wi < nw)
          build_a(w0, w1, s_wq[wi], s_wq[wi + 1]);
        else
          build_a(w0, w1, 0, g.n_groups);
        ++wi;
        __syncthreads();
      }
      // A[k = k0 + kq][M = li] at abase + k * rows + M; lanes past the rows read a
      // valid entry and take zero
      const bool aok = li < rows;
      const float* ap = s_a + (abase - w0) + kq * rows + min(li, rows - 1);
      const int* kp = s_k + kb + kq;
      if (active) {
        float4v D[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) D[u] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
        const float* sw = s_w + 16 * wave + li;
        const float* sx = s_x + 16 * wave + li;
        gemm_ksteps<NU>(D, ap, kp, rows, aok, K, sw, sx);
        // D[i][j] in register i % 4 of lane j + 16 (i / 4): row 4 kq + r, channel li
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * kq + r, o = oo + i;
            if (i < rows && o >= 0 && o < g.dout)
              g.z[(row * g.dout + o) * C + c0 + 16 * (wave + 4 * u) + li] = D[u][r];
          }
      }
      abase += rows * K;
    }
  }
}

// The harmonics of degree 0..LMAX of one edge vector into the LDS bank
// (component-normalised, l*l + m order).
template <int LMAX>
__device__ __forceinline__ void bank_of(const float* v, float* s_bank) {
  float Y[(LMAX + 1) * (LMAX + 1)];
  harmonics_bank_of_vec<LMAX>(v[0], v[1], v[2], Y);
#pragma unroll
  for (int i = 0; i < (LMAX + 1) * (LMAX + 1); ++i) s_bank[i] = Y[i];
}

__device__ __forceinline__ void edge_bank(int ly, const float* v, float* s_bank) {
  switch (ly) {
    case 0: bank_of<0>(v, s_bank); break;
    case 1: bank_of<1>(v, s_bank); break;
    case 2: bank_of<2>(v, s_bank); break;
    case 3: bank_of<3>(v, s_bank); break;
    case 4: bank_of<4>(v, s_bank); break;
    case 5: bank_of<5>(v, s_bank); break;
    case 6: bank_of<6>(v, s_bank); break;
    default: bank_of<7>(v, s_bank); break;  // 64 values: the bank's size
  }
}

// The convolution forward (e3j A.3 Eq.7 with E.1 Eq.10-12) in the same
// form: for receiver b, out[b][L] = sum over its in-edges e of A_{e,L} xt_e
// with xt_e[(P,m1)][q] = w[e][P][q] x[sender e][l1,m1][q].  One workgroup per
// (receiver, channel slab); per edge the slab of x[sender] and w[e] and Y[e]
// are staged and A_e built as for one tensor-product row, and every output
// block's tiles accumulate in registers over the edge list (at most NB
// blocks: collapsed outputs), so m is written once per receiver in edge
// order.  PRE as above, for the next edge of the same receiver (built with
// PRE = 0).  NB is 8, or kConvGemmMaxBlocks for plans of more blocks (the
// smaller form keeps the registers of the common case).
// WIN: A in windows of whole blocks (g.a_win > 0), each edge's A built and
// its blocks' products run one window at a time.
template <int PRE, int NU, bool BATCH, bool VEC, int NB, bool WIN>
__global__ void __launch_bounds__(256) k_conv_gemm(ConvGemmArgs cg) {
  constexpr int kConvGemmBlocks = NB;
  extern __shared__ __align__(16) float gsm[];
  const TpGemmArgs& g = cg.t;
  const int* __restrict__ blocks = g.plan + g.off_blocks;
  const int* __restrict__ klist = g.plan + g.off_klist;
  const int4* __restrict__ groups = reinterpret_cast<const int4*>(g.plan + g.off_groups);
  const int CS = g.CS, C = g.C, XS = gemm_row_stride(CS);
  const int lg4 = __builtin_ctz(CS / 4);
  const int AW = WIN && g.a_win > 0 ? min(g.a_win, g.a_floats) : g.a_floats;
  float* s_a = gsm;
  float* s_x = s_a + AW;
  float* s_w = s_x + g.dx * XS;
  float* s_y = s_w + (g.P + 1) * XS;
  int* s_k = reinterpret_cast<int*>(s_y + g.dy);
  float* s_bank = reinterpret_cast<float*>(s_k + g.n_klist);  // 64 floats
  int* s_ym = reinterpret_cast<int*>(s_bank + 64);             // y map, 16 words
  int* s_wq = s_ym + 16;  // windows: their runs of entries, then their count
  int* s_ws = s_wq + kMaxWindows + 2;  // and their A offsets
  for (int i = threadIdx.x; i < g.n_klist; i += 256) {
    const int ent = klist[i];
    const int p = ent < 0 ? g.P : min(ent >> 16, g.P - 1);
    const int xi = ent < 0 ? 0 : min(ent & 0xFFFF, g.dx - 1);
    s_k[i] = p * XS | (xi * XS) << 16;
  }
  for (int i = threadIdx.x; i < XS; i += 256) s_w[g.P * XS + i] = 0.0f;
  // A's entries outside the plan's groups stay zero: every row (edge)
  // rewrites all the others, so A is cleared once
  for (int i = threadIdx.x; i < AW; i += 256) s_a[i] = 0.0f;
  constexpr bool vec_y = VEC;  // harmonics from the edge vectors (cg.ly >= 0)
  if (threadIdx.x < 16) {
    int wd;
    __builtin_memcpy(&wd, cg.ym.idx + 4 * threadIdx.x, 4);
    s_ym[threadIdx.x] = wd;
  }
  const int nbank = (min(max(cg.ly, 0), 7) + 1) * (min(max(cg.ly, 0), 7) + 1);
  // y component i of the edge: given, or the bank entry the map names (clamped)
  auto yval = [&](int i) {
    if constexpr (!VEC) return s_y[i];
    const int b = reinterpret_cast<const signed char*>(s_ym)[i];
    return s_bank[min(max(b, 0), nbank - 1)];
  };
  // the blocks, read once
  int b_oo[kConvGemmBlocks], b_rows[kConvGemmBlocks], b_kb[kConvGemmBlocks], b_K[kConvGemmBlocks],
      b_ab[kConvGemmBlocks];
  {
    int abase = 0;
#pragma unroll
    for (int b = 0; b < kConvGemmBlocks; ++b) {
      const bool on = b < g.n_blocks;
      b_oo[b] = on ? blocks[4 * b] : 0;
      b_rows[b] = on ? min(max(blocks[4 * b + 1], 1), 16) : 1;
      b_kb[b] = on ? min(max(blocks[4 * b + 2], 0), g.n_klist) : 0;
      b_K[b] = on ? min(max(blocks[4 * b + 3], 0), g.n_klist - b_kb[b]) & ~3 : 0;
      if (abase + b_rows[b] * b_K[b] > g.a_floats) b_K[b] = 0;
      b_ab[b] = abase;
      abase += b_rows[b] * b_K[b];
    }
  }
  // windows of whole blocks (the partition of window_runs): block b in
  // window b_wi[b] at b_ab[b] - its start; n_win windows
  static_assert(NB <= kMaxWindows, "every window holds a block");
  int b_wi[kConvGemmBlocks], n_win = 1;
  if constexpr (WIN) {
    int w0 = 0, w1 = 0, wi = -1;
#pragma unroll
    for (int b = 0; b < kConvGemmBlocks; ++b) {
      const int sz = b_rows[b] * b_K[b];
      if (b < g.n_blocks && sz > 0 && b_ab[b] + sz > w1) {
        ++wi;
        w0 = b_ab[b];
        w1 = w0 + AW;
      }
      b_wi[b] = max(wi, 0);
      b_ab[b] -= w0;
      if (sz > AW) b_K[b] = 0;  // larger than a window: not computed
    }
    n_win = max(wi + 1, 1);
    if (threadIdx.x == 0) {
      auto size_of = [&](int b) {
        const int rows = min(max(blocks[4 * b + 1], 1), 16);
        const int kb = min(max(blocks[4 * b + 2], 0), g.n_klist);
        const int K = min(max(blocks[4 * b + 3], 0), g.n_klist - kb) & ~3;
        return rows * K;
      };
      s_wq[kMaxWindows + 1] =
          window_runs(g.n_blocks, size_of, g.a_floats, AW, groups, g.n_groups, s_wq, s_ws);
    }
  } else {
#pragma unroll
    for (int b = 0; b < kConvGemmBlocks; ++b) b_wi[b] = 0;
  }
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, kq = lane >> 4;
  const int n_slabs = C / CS, n_tiles = CS / 16;
  const bool active = wave < n_tiles;  // tiles wave + 4u, u < NU
  const int64_t n_items = int64_t(cg.n_nodes) * n_slabs;
  const int U = (g.dx + g.P) << lg4;
  auto unit_dst = [&](int u) {
    const int r = u >> lg4, c = 4 * (u & ((1 << lg4) - 1));
    return r < g.dx ? s_x + r * XS + c : s_w + (r - g.dx) * XS + c;
  };
  auto unit_src = [&](int u, int e, int a, int c0) {
    const int r = u >> lg4, c = 4 * (u & ((1 << lg4) - 1));
    return r < g.dx ? g.x + (int64_t(a) * g.dx + r) * C + c0 + c
                    : g.w + (int64_t(e) * g.P + (r - g.dx)) * C + c0 + c;
  };
  float4v pre[PRE > 0 ? PRE : 1];
  float ypre = 0.0f;
  // the edge id of CSR position j (its w and Y rows): j itself, or perm[j]
  // when the walk runs over another order (the transposed index); -1 when
  // perm names no edge
  auto edge_id = [&](int j) {
    if (!cg.perm) return j;
    const int e = cg.perm[j];
    return e >= 0 && e < cg.n_edges ? e : -1;
  };
  // a sender outside [0, n_nodes) marks a padding edge
  auto sender_of = [&](int j) {
    const int a = cg.sender[j];
    return a >= 0 && a < cg.n_nodes && edge_id(j) >= 0 ? a : -1;
  };
  auto prefetch = [&](int j, int c0) {
    const int a = max(sender_of(j), 0), e = max(edge_id(j), 0);
#pragma unroll
    for (int i = 0; i < PRE; ++i) {
      const int u = threadIdx.x + 256 * i;
      if (u < U) pre[i] = *reinterpret_cast<const float4v*>(unit_src(u, e, a, c0));
    }
    if (!vec_y && threadIdx.x < g.dy) ypre = g.y[int64_t(e) * g.dy + threadIdx.x];
  };
  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int node = int(item / n_slabs);
    const int c0 = int(item - int64_t(node) * n_slabs) * CS;
    // a malformed rowptr cannot move the walk outside [0, n_edges)
    const int e_lo = max(cg.rowptr[node], 0), e_hi = min(cg.rowptr[node + 1], cg.n_edges);
    float4v D[kConvGemmBlocks][NU];
#pragma unroll
    for (int b = 0; b < kConvGemmBlocks; ++b)
#pragma unroll
      for (int u = 0; u < NU; ++u) D[b][u] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    if (PRE > 0 && e_lo < e_hi) prefetch(e_lo, c0);
    for (int j = e_lo; j < e_hi; ++j) {
      const int a = sender_of(j);
      if (a < 0) {  // padding edge (the same for the whole workgroup): nothing to add
        if (PRE > 0 && j + 1 < e_hi) prefetch(j + 1, c0);
        continue;
      }
      const int e = edge_id(j);
      __syncthreads();  // the previous edge's LDS reads are done (and s_k is written)
#pragma unroll
      for (int j = 0; j < PRE; ++j) {
        const int u = threadIdx.x + 256 * j;
        if (u < U) *reinterpret_cast<float4v*>(unit_dst(u)) = pre[j];
      }
      for (int u = threadIdx.x + 256 * PRE; u < U; u += 256)
        *reinterpret_cast<float4v*>(unit_dst(u)) = *reinterpret_cast<const float4v*>(unit_src(u, e, a, c0));
      if constexpr (VEC) {
        if (threadIdx.x == 0) edge_bank(cg.ly, g.y + int64_t(e) * 3, s_bank);
      } else {
        for (int i = threadIdx.x; i < g.dy; i += 256)
          s_y[i] = PRE > 0 && i < 256 ? ypre : g.y[int64_t(e) * g.dy + i];
      }
      __syncthreads();
      if (PRE > 0 && j + 1 < e_hi) prefetch(j + 1, c0);
      for (int wi = 0; wi < n_win; ++wi) {  // one pass unless windowed (uniform)
      // (the window table is read after the edge's first barrier)
      const int w0 = WIN && wi < s_wq[kMaxWindows + 1] ? s_ws[wi] : 0;
      if (WIN) {
        if (wi > 0) __syncthreads();  // the previous window's reads are done
        for (int i = threadIdx.x; i < AW; i += 256) s_a[i] = 0.0f;
        __syncthreads();
      }
      {
        const int q0 = !WIN ? 0 : wi < s_wq[kMaxWindows + 1] ? s_wq[wi] : 0;
        const int q1 = !WIN ? g.n_groups : wi < s_wq[kMaxWindows + 1] ? s_wq[wi + 1] : g.n_groups;
#pragma unroll 4
        for (int q = q0 + threadIdx.x; q < q1; q += 256) {
          const int4 en = groups[q];
          const int at = min(max(en.x, 0), g.a_floats - 1) - w0;
          const int y1 = min(en.y & 0xFFFF, g.dy - 1), y2 = min((en.y >> 16) & 0xFFFF, g.dy - 1);
          if (!WIN || (at >= 0 && at < AW))
            s_a[at] = fmaf(__int_as_float(en.w), yval(y2), __int_as_float(en.z) * yval(y1));
        }
      }
      __syncthreads();
      // the same for the whole wavefront; windowed, it still meets the later windows' barriers
      if (!active) continue;
      const float* sw = s_w + 16 * wave + li;
      const float* sx = s_x + 16 * wave + li;
      // each edge's product starts from zero and joins the node's sum once,
      // so the long sum over the edge list rounds once per edge rather than
      // once per K step
#pragma unroll
      for (int b = 0; b < kConvGemmBlocks; ++b) {
        if (WIN && b_wi[b] != wi) continue;  // another window's block (uniform)
        const int rows = b_rows[b], K = b_K[b];
        const bool aok = li < rows;
        const float* ap = s_a + b_ab[b] + kq * rows + min(li, rows - 1);
        const int* kp = s_k + b_kb[b] + kq;
        float4v De[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) De[u] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
        gemm_ksteps<NU, BATCH>(De, ap, kp, rows, aok, K, sw, sx);
#pragma unroll
        for (int u = 0; u < NU; ++u) D[b][u] += De[u];
      }
      }  // windows
    }
    // D[i][j] in register i % 4 of lane j + 16 (i / 4): row 4 kq + r, channel li
#pragma unroll
    for (int b = 0; b < kConvGemmBlocks; ++b) {
      if (active && b < g.n_blocks) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = 4 * kq + r, o = b_oo[b] + i;
              if (i < b_rows[b] && o >= 0 && o < g.dout)
                cg.m[(int64_t(node) * g.dout + o) * C + c0 + 16 * (wave + 4 * u) + li] = D[b][u][r];
            }
          }
        }
      }
    }
  }
}

// Receiver of edge e in a CSR by receiver: the largest b with rowptr[b] <= e
// (so empty rows are passed over), clamped to [0, n_nodes).
__host__ __device__ constexpr int gemm_dy_row_stride(int CS) { return CS + 2; }

__device__ __forceinline__ int receiver_of(const int* __restrict__ rowptr, int n_nodes, int64_t e) {
  int lo = 0, hi = n_nodes;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (rowptr[mid] <= e) lo = mid; else hi = mid - 1;
  }
  return min(lo, n_nodes - 1);
}

// The gradient of w in the dense form (plan E3_GEN_GEMM_DW): per row (or
// edge) and path P,
//   dw[P][q] = sum_M dz[oo_P + M][q] (A_P x)[M][q].
// The plan stacks each path's rows (P, M) in quads of four (a path's last
// quad padded) into tiles of at most four quads, all of one x irrep and of
// one group of 16 paths.  Per tile, on the fp32 matrix cores: D = A x over
// the irrep's K steps (their x operand held in registers across the
// irrep's tiles, read from x in memory); the lane holding a quad's four
// rows forms
// sum_i D[row i] dz[row i] (in row order; padding rows read a zero row);
// and the quads' sums go into the group's 16 paths as a second product
// S E with S[P][quad] = 1 where the quad belongs to P, accumulated over the
// group's tiles and stored once the tiles have moved past it.  A is kept
// with a row stride of 16 (rows past a tile's end stay zero), so a K step's
// A read is one fixed offset.  One workgroup of NW wavefronts per (row,
// slab of CS = 16 NW NU channels).
__host__ __device__ constexpr int gemm_dw_a_slack() { return 256; }
// rows staged with a stride of 4 (mod 32) floats: a quad's rows four apart
// (the next quad of one path) then fall in the other half of the banks
__host__ __device__ constexpr int gemm_dw_row_stride(int CS) { return CS + 4; }

// WIN: A held in windows of whole tiles (a.a_win > 0; otherwise all of it,
// and this form has no window code in its tile loop)
template <int NU, int NW, bool WIN>
__global__ void __launch_bounds__(64 * NW) k_gemm_dw(GemmBwdArgs a) {
  constexpr int NT = 64 * NW;
  extern __shared__ __align__(16) float gsm[];
  const TpGemmArgs& g = a.t;
  const int* __restrict__ blocks = g.plan + g.off_blocks;
  const int* __restrict__ klist = g.plan + g.off_klist;
  const int* __restrict__ rowtab = g.plan + gemm_dw_rowtab_offset(g);
  const int4* __restrict__ groups = reinterpret_cast<const int4*>(g.plan + g.off_groups);
  const int CS = g.CS, C = g.C, XS = gemm_dw_row_stride(CS);
  const int lg4 = __builtin_ctz(CS / 4);
  // A of every tile at once, or (AW < a_floats) a window of whole tiles
  const int AW = WIN && a.a_win > 0 ? min(a.a_win, g.a_floats) : g.a_floats;
  const bool windowed = WIN && AW < g.a_floats;
  const int a4 = ((AW + 3) & ~3) + gemm_dw_a_slack();
  float* s_a = gsm;                         // A [tiles][K][16], then slack for reads past the last
  float* s_z = s_a + a4;                    // [dout + 1][XS]: a row of zeros, then the dz slab
  int* s_rt = reinterpret_cast<int*>(s_z + (g.dout + 1) * XS);  // rows [n_blocks][16], staged
  int* s_bd = s_rt + 16 * g.n_blocks;                              // descriptors [n_blocks][4]
  int* s_k = s_bd + 4 * g.n_blocks;                                // K list: x component or -1
  float* s_y = reinterpret_cast<float*>(s_k + g.n_klist);
  for (int i = threadIdx.x; i < g.n_klist; i += NT) {
    const int ent = klist[i];
    s_k[i] = ent < 0 || ent >= g.dx ? -1 : ent;
  }
  // rows: word offset in s_z of the row's dz row (row 0: zeros) | its path
  // in the group of 16 << 20 (16: none)
  for (int i = threadIdx.x; i < 16 * g.n_blocks; i += NT) {
    const int e = rowtab[i];
    const int z = e < 0 ? 0 : min(e >> 10, g.dout), rel = e < 0 ? 16 : min(e & 31, 16);
    s_rt[i] = z * XS | rel << 20;
  }
  for (int b = threadIdx.x; b < g.n_blocks; b += NT) {  // clamped to the plan's extents
    const int kb = min(max(blocks[4 * b + 2], 0), max(g.n_klist - 1, 0));
    const int K = min(min(max(blocks[4 * b + 3], 0), g.n_klist - kb), 16) & ~3;
    s_bd[4 * b] = blocks[4 * b];
    s_bd[4 * b + 1] = 0;
    s_bd[4 * b + 2] = kb;
    s_bd[4 * b + 3] = K;
  }
  for (int i = threadIdx.x; i < XS; i += NT) s_z[i] = 0.0f;
  for (int i = threadIdx.x; i < a4; i += NT) s_a[i] = 0.0f;
  int* s_wq = reinterpret_cast<int*>(s_y + g.dy);  // windows: their runs of entries, their count
  if (windowed && threadIdx.x == 0) {
    auto size_of = [&](int b) {  // as the s_bd entries above
      const int kb = min(max(blocks[4 * b + 2], 0), max(g.n_klist - 1, 0));
      return 16 * (min(min(max(blocks[4 * b + 3], 0), g.n_klist - kb), 16) & ~3);
    };
    s_wq[kMaxWindows + 1] = window_runs(g.n_blocks, size_of, g.a_floats, AW, groups, g.n_groups, s_wq);
  }
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, kq = lane >> 4;
  const int n_slabs = C / CS;
  const bool active = wave < CS / (16 * NU);
  const int64_t n_items = g.n_rows * n_slabs;
  const int U = g.dout << lg4;
  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int64_t row = item / n_slabs;
    const int c0 = int(item - row * n_slabs) * CS;
    const int xr = a.xrow ? a.xrow[row] : int(row);
    float* dwr = a.out + row * g.P * C + c0;
    __syncthreads();  // the previous item's LDS reads are done (and the tables are written)
    if (xr < 0 || xr >= a.n_x) {  // padding edge (uniform): zero gradient
      for (int i = threadIdx.x; i < g.P * CS; i += NT) dwr[(i / CS) * C + i % CS] = 0.0f;
      continue;
    }
    const int64_t zr = a.rowptr ? receiver_of(a.rowptr, a.n_zrows, row) : row;
    for (int u = threadIdx.x; u < U; u += NT) {
      const int r = u >> lg4, c = 4 * (u & ((1 << lg4) - 1));
      *reinterpret_cast<float4v*>(s_z + (r + 1) * XS + c) =
          *reinterpret_cast<const float4v*>(a.dz + (zr * g.dout + r) * C + c0 + c);
    }
    for (int i = threadIdx.x; i < g.dy; i += NT) s_y[i] = g.y[row * g.dy + i];
    __syncthreads();
    // A[at - a0] for the entries with at in [a0, a1)
    auto build_a = [&](int a0, int a1, int q0, int q1) {
#pragma unroll 4
      for (int q = q0 + threadIdx.x; q < q1; q += NT) {
        const int4 e = groups[q];
        const int at = min(max(e.x, 0), g.a_floats - 1);
        const int y1 = min(e.y & 0xFFFF, g.dy - 1), y2 = min((e.y >> 16) & 0xFFFF, g.dy - 1);
        if (at >= a0 && at < a1)
          s_a[at - a0] = fmaf(__int_as_float(e.w), s_y[y2], __int_as_float(e.z) * s_y[y1]);
      }
    };
    if (!windowed) {  // all of A, every entry
#pragma unroll 4
      for (int q = threadIdx.x; q < g.n_groups; q += NT) {
        const int4 e = groups[q];
        const int at = min(max(e.x, 0), g.a_floats - 1);
        const int y1 = min(e.y & 0xFFFF, g.dy - 1), y2 = min((e.y >> 16) & 0xFFFF, g.dy - 1);
        s_a[at] = fmaf(__int_as_float(e.w), s_y[y2], __int_as_float(e.z) * s_y[y1]);
      }
      __syncthreads();
    }
    // acc: paths 16 cur + [0, 16); register r of lane (li, kq) holds path
    // 16 cur + 4 kq + r at channel 16 (wave + NW u) + li
    float4v acc[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) acc[u] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    auto flush = [&](int t) {
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int P = 16 * t + 4 * kq + r;
          if (P >= 0 && P < g.P) dwr[int64_t(P) * C + 16 * (wave + NW * u) + li] = acc[u][r];
        }
    };
    const float* zl = s_z + 16 * wave + li;  // this lane's channel in a dz row
    const float* xl = g.x + int64_t(xr) * g.dx * C + c0 + 16 * wave + li;  // and in x
    int cur = 0, cur_kb = -1, cur_K = -1, abase = 0;
    int w0 = 0, w1 = windowed ? 0 : g.a_floats;  // A offsets [w0, w1) in LDS
    int wi = 0;                                   // window number
    float xb[4][NU];
    // the tiles' descriptors from LDS, the next one read while this one runs
    int4 bd = g.n_blocks > 0 ? *reinterpret_cast<const int4*>(s_bd) : int4{0, 0, 0, 0};
    for (int b = 0; b < g.n_blocks; ++b) {
      const int t = __builtin_amdgcn_readfirstlane(bd.x);
      const int kb = __builtin_amdgcn_readfirstlane(bd.z);
      const int K = __builtin_amdgcn_readfirstlane(bd.w);
      if (b + 1 < g.n_blocks) bd = *reinterpret_cast<const int4*>(s_bd + 4 * (b + 1));
      if (abase + 16 * K > g.a_floats) break;
      if (WIN && abase + 16 * K > w1) {  // windowed (uniform): the next window starts at this tile
        w0 = abase;
        w1 = abase + AW;
        __syncthreads();  // the previous window's reads are done
        for (int i = threadIdx.x; i < a4; i += NT) s_a[i] = 0.0f;
        __syncthreads();
        const int nw = s_wq[kMaxWindows + 1];
        if (wi < nw)
          build_a(w0, w1, s_wq[wi], s_wq[wi + 1]);
        else
          build_a(w0, w1, 0, g.n_groups);
        ++wi;
        __syncthreads();
      }
      if (!active) {  // the same for the whole wavefront (it still joins the barriers)
        abase += 16 * K;
        continue;
      }
      // A of the tile, its four K steps' reads issued together (past the
      // tile's K they read the next tile's A or the slack, unused)
      const float* ap = s_a + (abase - w0) + 16 * kq + li;
      float av[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) av[j] = ap[64 * j];
      const int4 rt = *reinterpret_cast<const int4*>(s_rt + 16 * b + 4 * kq);
      if (t != cur) {  // the tiles have moved past path group cur
        flush(cur);
#pragma unroll
        for (int u = 0; u < NU; ++u) acc[u] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
        cur = t;
      }
      if (kb != cur_kb || K != cur_K) {  // a new x irrep: its K steps' x operand
        int xi[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xi[j] = 4 * j < K ? s_k[min(kb + 4 * j + kq, g.n_klist - 1)] : -1;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int u = 0; u < NU; ++u)
            xb[j][u] = xi[j] >= 0 ? xl[int64_t(xi[j]) * C + 16 * NW * u] : 0.0f;
        cur_kb = kb;
        cur_K = K;
      }
      float4v D[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) D[u] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * j < K) {
#pragma unroll
          for (int u = 0; u < NU; ++u)
            D[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], xb[j][u], D[u], 0, 0, 0);
        }
      // D[u][r]: row 4 kq + r of the tile (quad kq), channel 16 (wave + NW u) + li
      const float sv = ((rt.x >> 20) & 31) == li ? 1.0f : 0.0f;
      const int zo[4] = {rt.x & 0xFFFFF, rt.y & 0xFFFFF, rt.z & 0xFFFFF, rt.w & 0xFFFFF};
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        float e = D[u][0] * zl[zo[0] + 16 * NW * u];
#pragma unroll
        for (int r = 1; r < 4; ++r) e = fmaf(D[u][r], zl[zo[r] + 16 * NW * u], e);
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(sv, e, acc[u], 0, 0, 0);
      }
      abase += 16 * K;
    }
    if (active) flush(cur);
  }
}

// The gradient of y in the dense form (plan E3_GEN_GEMM_DY): per row (or
// edge), one workgroup over every channel slab in turn:
//   G_P[M][m1] = sum_q w[P][q] dz[oo_P + M][q] x[xoff_P + m1][q]
// on the fp32 matrix cores with the channel sum as the product's K: per
// block, the columns are the components of one x irrep (rows (P, M)) or of
// one output irrep (rows (P, m1)); the A operand w times the row's own
// operand is formed per lane from the staged slab, B is the column operand.
// 16-row tiles of G are owned by one wavefront each and added up over the
// slabs in LDS, then dy[yi] = sum of c G over the plan's entries of yi, in
// the plan's order.
template <int NW>
__global__ void __launch_bounds__(64 * NW) k_gemm_dy(GemmBwdArgs a) {
  constexpr int NT = 64 * NW;
  extern __shared__ __align__(16) float gsm[];
  const TpGemmArgs& g = a.t;
  const int* __restrict__ blocks = g.plan + g.off_blocks;
  const int* __restrict__ grows = g.plan + a.off_rows;
  const int* __restrict__ yptr = g.plan + a.off_yptr;
  const int* __restrict__ yent = g.plan + a.off_yent;
  // rows staged with a stride of 2 (mod 32) floats: a K step's read takes
  // 16 rows at consecutive channels, and each half wavefront (two channels
  // of 16 rows) then falls in 32 distinct banks
  const int CS = g.CS, C = g.C, XS = gemm_dy_row_stride(CS);
  const int lg4 = __builtin_ctz(CS / 4);
  float* s_x = gsm;
  float* s_w = s_x + g.dx * XS;
  float* s_z = s_w + g.P * XS;
  // G rows in groups of g_rows (all of them at once when they fit)
  const int GR = min(max(a.g_rows, 16), a.n_grows) & ~15;
  float* s_g = s_z + g.dout * XS;                     // G [GR][16]: rows [gr0, gr0 + GR)
  int* s_r = reinterpret_cast<int*>(s_g + GR * 16);   // per G row: w row | own row << 16
  int* s_b = s_r + a.n_grows;  // per G row: its block's first column row | columns << 16
  float* s_dy = reinterpret_cast<float*>(s_b + a.n_grows);  // dy of the groups so far (two or more)
  const int n_srows = g.dx + g.P + g.dout;  // slab rows: x, w, dz
  for (int i = threadIdx.x; i < a.n_grows; i += NT) {
    const int ent = grows[i];
    const int P = ent < 0 ? 0 : min(ent & 0xFFFF, g.P - 1);
    const int own = ent < 0 ? 0 : min(ent >> 16, n_srows - 1);
    s_r[i] = ent < 0 ? -1 : P | own << 16;
    s_b[i] = 0;
  }
  __syncthreads();
  for (int b = threadIdx.x; b < g.n_blocks; b += NT) {
    const int xo = min(max(blocks[4 * b], 0), n_srows - 1);
    const int nc = min(max(blocks[4 * b + 1], 0), 16);
    const int r0 = max(blocks[4 * b + 2], 0), nr = max(blocks[4 * b + 3], 0);
    for (int r = r0; r < min(r0 + nr, a.n_grows); ++r) s_b[r] = xo | nc << 16;
  }
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, kq = lane >> 4;
  const int n_slabs = C / CS, n_gt = a.n_grows / 16;
  const int U = (g.dx + g.P + g.dout) << lg4;
  for (int64_t row = blockIdx.x; row < g.n_rows; row += gridDim.x) {
    const int xr = a.xrow ? a.xrow[row] : int(row);
    float* dyr = a.out + row * g.dy;
    __syncthreads();  // the previous row's LDS reads are done
    if (xr < 0 || xr >= a.n_x) {  // padding edge (uniform): zero gradient
      for (int i = threadIdx.x; i < g.dy; i += NT) dyr[i] = 0.0f;
      continue;
    }
    const int64_t zr = a.rowptr ? receiver_of(a.rowptr, a.n_zrows, row) : row;
    // (one pass when there are no G rows: dy is then written as zeros)
    for (int gr0 = 0; gr0 == 0 || gr0 < a.n_grows; gr0 += max(GR, 16)) {
    const int tg0 = gr0 / 16, tg1 = min(n_gt, (gr0 + GR) / 16);  // this group's tiles
    if (gr0 > 0) __syncthreads();  // the previous group's reads of G are done
    for (int i = threadIdx.x; i < GR * 16; i += NT) s_g[i] = 0.0f;
    for (int sl = 0; sl < n_slabs; ++sl) {
      const int c0 = sl * CS;
      __syncthreads();  // the previous slab's LDS reads are done (and s_g is cleared)
      for (int u = threadIdx.x; u < U; u += NT) {
        const int r = u >> lg4, c = 4 * (u & ((1 << lg4) - 1));
        const float* src = r < g.dx ? g.x + (int64_t(xr) * g.dx + r) * C
                         : r < g.dx + g.P ? g.w + (row * g.P + (r - g.dx)) * C
                                          : a.dz + (zr * g.dout + (r - g.dx - g.P)) * C;
        const float4v v = *reinterpret_cast<const float4v*>(src + c0 + c);
        float* d = s_x + r * XS + c;  // 8-byte aligned (XS is even)
        *reinterpret_cast<float2*>(d) = float2{v[0], v[1]};
        *reinterpret_cast<float2*>(d + 2) = float2{v[2], v[3]};
      }
      __syncthreads();
      // two tiles at a time (independent accumulators), four K steps per
      // batch with their LDS reads issued first
      for (int t0 = tg0 + 2 * wave; t0 < tg1; t0 += 2 * NW) {
        const float* wp[2];
        const float* zp[2];
        const float* xp[2];
        bool aok[2], bok[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int t = min(t0 + h, tg1 - 1);
          const int ro = s_r[16 * t + li];
          const int bx = s_b[16 * t];  // column block of the tile (uniform)
          const int xo = bx & 0xFFFF, nc = bx >> 16;
          wp[h] = s_w + (ro < 0 ? 0 : ro & 0xFFFF) * XS + kq;
          zp[h] = s_x + (ro < 0 ? 0 : ro >> 16) * XS + kq;
          xp[h] = s_x + min(xo + min(li, max(nc - 1, 0)), n_srows - 1) * XS + kq;
          aok[h] = ro >= 0 && t0 + h < tg1;
          bok[h] = li < nc;
        }
        float4v D[2] = {float4v{0.0f, 0.0f, 0.0f, 0.0f}, float4v{0.0f, 0.0f, 0.0f, 0.0f}};
        for (int q = 0; q < CS; q += 16) {
          float av[2][4], zv[2][4], bv[2][4];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              av[h][j] = wp[h][q + 4 * j];
              zv[h][j] = zp[h][q + 4 * j];
              bv[h][j] = xp[h][q + 4 * j];
            }
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h)
              D[h] = __builtin_amdgcn_mfma_f32_16x16x4f32(aok[h] ? av[h][j] * zv[h][j] : 0.0f,
                                                          bok[h] ? bv[h][j] : 0.0f, D[h], 0, 0, 0);
        }
        // D[h][r]: G row 16 t + 4 kq + r, column li
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (t0 + h < tg1)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              s_g[(16 * (t0 + h) - gr0 + 4 * kq + r) * 16 + li] += D[h][r];
      }
    }
    __syncthreads();
    // dy[y]: a wavefront per component, its entries (those in this group's
    // G rows) strided over the lanes, then the fixed-order wavefront sum,
    // added to the earlier groups' in group order
    const bool last = gr0 + GR >= a.n_grows;
    for (int y = wave; y < g.dy; y += NW) {
      float acc = 0.0f;
      const int k0 = max(yptr[y], 0), k1 = min(yptr[y + 1], a.n_ent);
      if (GR >= a.n_grows) {  // all of G in LDS (uniform)
        for (int k = k0 + lane; k < k1; k += 64) {
          const int gi = min(max(yent[2 * k], 0), a.n_grows * 16 - 1);
          acc = fmaf(__int_as_float(yent[2 * k + 1]), s_g[gi], acc);
        }
      } else {
        for (int k = k0 + lane; k < k1; k += 64) {
          const int gi = min(max(yent[2 * k], 0), a.n_grows * 16 - 1) - gr0 * 16;
          if (gi >= 0 && gi < GR * 16) acc = fmaf(__int_as_float(yent[2 * k + 1]), s_g[gi], acc);
        }
      }
      acc = wave_sum(acc);
      if (lane == 0) {
        const float v = gr0 == 0 ? acc : s_dy[y] + acc;
        if (last)
          dyr[y] = v;
        else
          s_dy[y] = v;
      }
    }
    }  // groups of G rows
  }
}

}  // namespace

size_t tp_gemm_lds_bytes(const TpGemmArgs& a) {
  const int XS = gemm_row_stride(a.CS);
  const int aw = a.a_win > 0 ? std::min(a.a_win, a.a_floats) : a.a_floats;
  // the windows' runs of entries and (the convolution) their A offsets
  const int wq = a.a_win > 0 ? 2 * kMaxWindows + 3 : 0;
  return size_t(aw + a.dx * XS + (a.P + 1) * XS + a.dy + a.n_klist + wq) * 4;
}

template <int PRE, int NU, bool WIN = false>
hipError_t launch_tp_gemm_pre(const TpGemmArgs& a, int per_cu, hipStream_t s) {
  // the attribute is per function: raised once, retried after a failure
  static std::atomic<bool> lds_set{false};
  if (const hipError_t e = set_max_lds_once(lds_set, reinterpret_cast<const void*>(&k_tp_gemm<PRE, NU, WIN>), 160 * 1024);
      e != hipSuccess)
    return e;
  const int64_t items = a.n_rows * (a.C / a.CS);
  const int grid = int(std::min<int64_t>(items, int64_t(256) * per_cu));
  hipLaunchKernelGGL((k_tp_gemm<PRE, NU, WIN>), dim3(grid), dim3(256), a.lds_bytes, s, a);
  return hipGetLastError();
}

template <int PRE, int NU, bool BATCH, bool VEC, int NB, bool WIN = false>
hipError_t launch_conv_gemm_nb(const ConvGemmArgs& a, int per_cu, hipStream_t s) {
  // the attribute is per function: raised once, retried after a failure
  static std::atomic<bool> lds_set{false};
  if (const hipError_t e = set_max_lds_once(lds_set, reinterpret_cast<const void*>(&k_conv_gemm<PRE, NU, BATCH, VEC, NB, WIN>), 160 * 1024);
      e != hipSuccess)
    return e;
  const int64_t items = int64_t(a.n_nodes) * (a.t.C / a.t.CS);
  const int grid = int(std::min<int64_t>(items, int64_t(256) * per_cu));
  hipLaunchKernelGGL((k_conv_gemm<PRE, NU, BATCH, VEC, NB, WIN>), dim3(grid), dim3(256), a.t.lds_bytes, s, a);
  return hipGetLastError();
}

template <int PRE, int NU, bool BATCH, bool VEC>
hipError_t launch_conv_gemm_pre(const ConvGemmArgs& a, int per_cu, hipStream_t s) {
  return a.t.n_blocks <= 8 ? launch_conv_gemm_nb<PRE, NU, BATCH, VEC, 8>(a, per_cu, s)
                           : launch_conv_gemm_nb<PRE, NU, BATCH, VEC, kConvGemmMaxBlocks>(a, per_cu, s);
}

hipError_t launch_conv_gemm(const ConvGemmArgs& a, hipStream_t s) {
  if (a.n_nodes <= 0) return hipSuccess;
  if (a.t.lds_bytes > 160 * 1024 || a.t.n_blocks > kConvGemmMaxBlocks || a.t.CS > 128 ||
      a.ly > 7 || (a.ly >= 0 && a.t.dy > 64))
    return hipErrorInvalidValue;
  const int per_cu = std::max<int>(1, int((160 * 1024) / std::max<size_t>(a.t.lds_bytes, 1)));
  if (a.t.a_win > 0) {  // A in windows: given harmonics, 64-channel slabs, one form
    if (a.ly >= 0 || a.t.CS != 64 || a.t.a_win < a.t.a_block_max) return hipErrorInvalidValue;
    return launch_conv_gemm_nb<0, 1, true, false, kConvGemmMaxBlocks, true>(a, per_cu, s);
  }
  // one 16-channel tile per wavefront (slabs of at most 64 channels).  The
  // next edge's operands are not prefetched here: with the per-block
  // accumulators the registers would leave one wavefront per SIMD.
  // Batched K steps for plans whose LDS leaves at most two workgroups per CU;
  // smaller plans keep the registers for a third wavefront per SIMD.
  if (a.t.CS > 64) return hipErrorInvalidValue;
  // The harmonics of the edge vectors are a variant of their own (the bank's
  // registers would otherwise cost the given-harmonics kernel its occupancy),
  // batched on the same rule.
  if (a.ly >= 0)
    return per_cu <= 2 ? launch_conv_gemm_pre<0, 1, true, true>(a, per_cu, s)
                       : launch_conv_gemm_pre<0, 1, false, true>(a, std::min(per_cu, 8), s);
  return per_cu <= 2 ? launch_conv_gemm_pre<0, 1, true, false>(a, per_cu, s)
                     : launch_conv_gemm_pre<0, 1, false, false>(a, std::min(per_cu, 8), s);
}

size_t gemm_dw_lds_bytes(const TpGemmArgs& a, int a_win) {
  const int XS = gemm_dw_row_stride(a.CS);
  const int aw = a_win > 0 ? std::min(a_win, a.a_floats) : a.a_floats;
  const int wq = a_win > 0 ? kMaxWindows + 2 : 0;  // the windows' runs of entries
  return size_t(((aw + 3) & ~3) + gemm_dw_a_slack() + (a.dout + 1) * XS + 20 * a.n_blocks +
                a.n_klist + a.dy + wq) * 4;
}

size_t gemm_dy_lds_bytes(const GemmBwdArgs& a) {
  const int XS = gemm_dy_row_stride(a.t.CS);
  const int gr = std::min(std::max(a.g_rows, 16), a.n_grows) & ~15;
  // dy's running sums only when G is walked in more than one group
  const int sdy = gr < a.n_grows ? a.t.dy : 0;
  return size_t((a.t.dx + a.t.P + a.t.dout) * XS + gr * 16 + 2 * a.n_grows + sdy) * 4;
}

template <int NU, int NW, bool WIN>
hipError_t launch_gemm_dw_win(const GemmBwdArgs& a, hipStream_t s) {
  static std::atomic<bool> lds_set{false};
  if (const hipError_t e = set_max_lds_once(
          lds_set, reinterpret_cast<const void*>(&k_gemm_dw<NU, NW, WIN>), 160 * 1024);
      e != hipSuccess)
    return e;
  const int per_cu = std::max<int>(1, int((160 * 1024) / std::max<size_t>(a.t.lds_bytes, 1)));
  const int64_t items = a.t.n_rows * (a.t.C / a.t.CS);
  const int grid = int(std::min<int64_t>(items, int64_t(256) * std::min(per_cu, 8)));
  hipLaunchKernelGGL((k_gemm_dw<NU, NW, WIN>), dim3(grid), dim3(64 * NW), a.t.lds_bytes, s, a);
  return hipGetLastError();
}

template <int NU, int NW>
hipError_t launch_gemm_dw_nu(const GemmBwdArgs& a, hipStream_t s) {
  if constexpr (NW >= 4)  // windows only with slabs of 64 or 128 channels
    if (a.a_win > 0) return launch_gemm_dw_win<NU, NW, true>(a, s);
  if (a.a_win > 0) return hipErrorInvalidValue;
  return launch_gemm_dw_win<NU, NW, false>(a, s);
}

// one 16-channel tile per wavefront
hipError_t launch_gemm_dw(const GemmBwdArgs& a, hipStream_t s) {
  if (a.t.n_rows <= 0) return hipSuccess;
  // a window holds at least one whole tile (16 x 16 floats)
  if (a.t.lds_bytes > 160 * 1024 || (a.a_win > 0 && a.a_win < 256)) return hipErrorInvalidValue;
  switch (a.t.CS) {
    case 128: return launch_gemm_dw_nu<1, 8>(a, s);
    case 64: return launch_gemm_dw_nu<1, 4>(a, s);
    case 32: return launch_gemm_dw_nu<1, 2>(a, s);
    case 16: return launch_gemm_dw_nu<1, 1>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// eight wavefronts: the LDS (slabs and G) allows about one workgroup per CU
hipError_t launch_gemm_dy(const GemmBwdArgs& a, hipStream_t s) {
  constexpr int NW = 8;
  if (a.t.n_rows <= 0) return hipSuccess;
  if (a.t.lds_bytes > 160 * 1024 || a.n_grows % 16 || a.g_rows < 16 || a.g_rows % 16)
    return hipErrorInvalidValue;
  static std::atomic<bool> lds_set{false};
  if (const hipError_t e =
          set_max_lds_once(lds_set, reinterpret_cast<const void*>(&k_gemm_dy<NW>), 160 * 1024);
      e != hipSuccess)
    return e;
  const int per_cu = std::max<int>(1, int((160 * 1024) / std::max<size_t>(a.t.lds_bytes, 1)));
  const int grid = int(std::min<int64_t>(a.t.n_rows, int64_t(256) * std::min(per_cu, 8)));
  hipLaunchKernelGGL(k_gemm_dy<NW>, dim3(grid), dim3(64 * NW), a.t.lds_bytes, s, a);
  return hipGetLastError();
}

hipError_t launch_tp_gemm(const TpGemmArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  if (a.lds_bytes > 160 * 1024) return hipErrorInvalidValue;
  const int per_cu = std::max<int>(1, int((160 * 1024) / std::max<size_t>(a.lds_bytes, 1)));
  if (a.a_win > 0) {  // A in windows: 64-channel slabs (a tile per wavefront), one form
    if (a.CS != 64 || a.a_win < a.a_block_max) return hipErrorInvalidValue;
    return launch_tp_gemm_pre<12, 1, true>(a, per_cu, s);
  }
  // tiles per wavefront: a 128-channel slab has 8 tiles (2 per wavefront),
  // smaller slabs at most 4 (1 per wavefront, some wavefronts idle below 64)
  if (a.CS > 64)
    return per_cu <= 2 ? launch_tp_gemm_pre<12, 2>(a, per_cu, s)
                       : launch_tp_gemm_pre<0, 2>(a, std::min(per_cu, 8), s);
  return per_cu <= 2 ? launch_tp_gemm_pre<12, 1>(a, per_cu, s)
                     : launch_tp_gemm_pre<0, 1>(a, std::min(per_cu, 8), s);
}

}  // namespace e3k
