// Channel-wise tensor product and message-passing convolution for any irreps
// signature with degrees up to 7 (harmonics from edge vectors to 6),
// interpreted from a coefficient table instead of compiled per signature.
//
// e3j describes its tensor product as a generic bilinear coupling driven by
// a sparse COO array of coefficients (E.1 Eq.10-11, B.1) and runs it to
// degree L = 6..8 (B.1 Figs 5-7).  The specialised kernels unroll every
// record at compile time, which stops scaling near L = 4 (the unrolled code
// outgrows the instruction cache); these kernels read the records from a
// table built on the host from the library's ladder CG
// (e3_generic_plan_build).
//
// Table (int32 words, built per descriptor and per cotangent):
//   header  [kGenMagic, operand dims, y dims, keys, weight rows,
//            n_contrib, n_rec, rec_off]
//   obeg    [keys + 1]         contributions of key k
//   contrib [n_contrib][3]     {weight row, first record, end record}
//   rec     [n_rec][2]         at word rec_off (32-byte aligned):
//                              {operand component | y component << 16,
//                               coefficient bits}
// Every record run is padded to a multiple of 4 with zero coefficients, so
// the kernels take records four at a time (one 32-byte scalar load, eight
// LDS reads in flight, two partial sums).  For every key k of a row
//   out[k][c] = sum_contributions wgt[row][c] sum_records c_r y[yi] op[oi][c]
// where y is one value per row (the harmonics) or, for the harmonic
// cotangent, one value per channel.  Every index read from the table is
// clamped to its array, so a table built for another descriptor gives wrong
// numbers, never an out-of-bounds access.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "harmonics_hi.h"
#include "registry.h"

namespace e3k {
namespace {

constexpr int kGenWaves = 4;
constexpr int kLdsBlockFloats = 16384;  // 64 KiB of LDS per workgroup at most

// A table with its counts checked against its length: counts that would
// read past the table are replaced by zero (no contributions).
struct Table {
  const int* obeg;
  const int* contrib;
  const int4* rec4;
  int n_contrib, n_rec;
};

__device__ __forceinline__ Table table_view(const int* prog, int64_t n_words, int keys) {
  Table t;
  t.n_contrib = prog[5];
  t.n_rec = prog[6];
  const int64_t rec_off = prog[7];
  const int64_t fixed = kGenHeader + int64_t(keys) + 1;
  if (t.n_contrib < 0 || t.n_rec < 0 || rec_off < fixed + 3 * int64_t(t.n_contrib) ||
      (rec_off & 7) || rec_off + 2 * int64_t(t.n_rec) > n_words)
    t.n_contrib = t.n_rec = 0;
  t.obeg = prog + kGenHeader;
  t.contrib = t.obeg + keys + 1;
  t.rec4 = reinterpret_cast<const int4*>(prog + (t.n_rec ? rec_off : 0));
  return t;
}

// Value of key k for this lane: sum over the key's contributions of
// wgt(row) * sum over the run's records of c * yv(y index) * ops[op index][lane].
// ops is the lane's operand column in LDS ([n_op][64]); yv reads the y
// operand (an LDS value shared by the wave or per lane).  The weight is
// requested before the records are walked so its latency overlaps them.
template <class WF, class YF>
__device__ __forceinline__ float key_sum(const Table& t, int k, int n_op, int n_y, int n_w,
                                         const float* ops, int lane, WF wgt, YF yv) {
  float acc = 0.0f;
  const int jb = max(t.obeg[k], 0), je = min(t.obeg[k + 1], t.n_contrib);
  for (int j = jb; j < je; ++j) {
    const float wv = wgt(min(max(t.contrib[3 * j], 0), n_w - 1));
    // runs are whole groups of 4 records: [rb, re) in units of 4
    const int gb = max(t.contrib[3 * j + 1], 0) >> 2, ge = min(t.contrib[3 * j + 2], t.n_rec) >> 2;
    float t0 = 0.0f, t1 = 0.0f;
#pragma unroll 2
    for (int g = gb; g < ge; ++g) {
      const int4 a = t.rec4[2 * g], b = t.rec4[2 * g + 1];  // 4 records, 32 bytes
      const int p0 = a.x, p1 = a.z, p2 = b.x, p3 = b.z;
      auto oi = [&](int pk) { return min(pk & 0xffff, n_op - 1); };
      auto yi = [&](int pk) { return min(int(unsigned(pk) >> 16), n_y - 1); };
      const float y0 = yv(yi(p0)), y1 = yv(yi(p1)), y2 = yv(yi(p2)), y3 = yv(yi(p3));
      const float x0 = ops[oi(p0) * 64 + lane], x1 = ops[oi(p1) * 64 + lane];
      const float x2 = ops[oi(p2) * 64 + lane], x3 = ops[oi(p3) * 64 + lane];
      t0 = fmaf(__int_as_float(a.y) * y0, x0, t0);
      t1 = fmaf(__int_as_float(a.w) * y1, x1, t1);
      t0 = fmaf(__int_as_float(b.y) * y2, x2, t0);
      t1 = fmaf(__int_as_float(b.w) * y3, x3, t1);
    }
    acc = fmaf(wv, t0 + t1, acc);
  }
  return acc;
}

// key_sum for two channels per lane: ops holds a float2 per lane and
// component ([n_op][64]), wgt returns the two channels' weights.  Each
// channel's sum is formed in the same order as key_sum's.
template <class WF, class YF>
__device__ __forceinline__ float2 key_sum2(const Table& t, int k, int n_op, int n_y, int n_w,
                                           const float2* ops, int lane, WF wgt, YF yv) {
  float a0 = 0.0f, a1 = 0.0f;
  const int jb = max(t.obeg[k], 0), je = min(t.obeg[k + 1], t.n_contrib);
  for (int j = jb; j < je; ++j) {
    const float2 wv = wgt(min(max(t.contrib[3 * j], 0), n_w - 1));
    const int gb = max(t.contrib[3 * j + 1], 0) >> 2, ge = min(t.contrib[3 * j + 2], t.n_rec) >> 2;
    float t00 = 0.0f, t01 = 0.0f, t10 = 0.0f, t11 = 0.0f;
#pragma unroll 2
    for (int g = gb; g < ge; ++g) {
      const int4 a = t.rec4[2 * g], b = t.rec4[2 * g + 1];
      const int p0 = a.x, p1 = a.z, p2 = b.x, p3 = b.z;
      auto oi = [&](int pk) { return min(pk & 0xffff, n_op - 1); };
      auto yi = [&](int pk) { return min(int(unsigned(pk) >> 16), n_y - 1); };
      const float c0 = __int_as_float(a.y) * yv(yi(p0)), c1 = __int_as_float(a.w) * yv(yi(p1));
      const float c2 = __int_as_float(b.y) * yv(yi(p2)), c3 = __int_as_float(b.w) * yv(yi(p3));
      const float2 x0 = ops[oi(p0) * 64 + lane], x1 = ops[oi(p1) * 64 + lane];
      const float2 x2 = ops[oi(p2) * 64 + lane], x3 = ops[oi(p3) * 64 + lane];
      t00 = fmaf(c0, x0.x, t00);
      t01 = fmaf(c0, x0.y, t01);
      t10 = fmaf(c1, x1.x, t10);
      t11 = fmaf(c1, x1.y, t11);
      t00 = fmaf(c2, x2.x, t00);
      t01 = fmaf(c2, x2.y, t01);
      t10 = fmaf(c3, x3.x, t10);
      t11 = fmaf(c3, x3.y, t11);
    }
    a0 = fmaf(wv.x, t00 + t10, a0);
    a1 = fmaf(wv.y, t01 + t11, a1);
  }
  return make_float2(a0, a1);
}

// Channels c and c + 1 of element p (c + 1 may be past C: then 0); a vector
// access when the pair is aligned (C even).
template <class T>
__device__ __forceinline__ float2 load_pair(const T* __restrict__ p, int c, int C) {
  float v[2] = {0.0f, 0.0f};
  if (c + 1 < C && !(C & 1)) {
    load_ch<T, 2>(p, v);
  } else {
    float u[1];
    if (c < C) {
      load_ch<T, 1>(p, u);
      v[0] = u[0];
    }
    if (c + 1 < C) {
      load_ch<T, 1>(p + 1, u);
      v[1] = u[0];
    }
  }
  return make_float2(v[0], v[1]);
}

template <class T>
__device__ __forceinline__ void store_pair(T* __restrict__ p, int c, int C, float2 v) {
  if (c + 1 < C && !(C & 1)) {
    const float o[2] = {v.x, v.y};
    store_ch<T, 2>(p, o);
  } else {
    const float o0[1] = {v.x}, o1[1] = {v.y};
    if (c < C) store_ch<T, 1>(p, o0);
    if (c + 1 < C) store_ch<T, 1>(p + 1, o1);
  }
}

// One channel per lane of row `row` (n components of C) into LDS [n][64];
// lanes past C get 0.
template <class T>
__device__ __forceinline__ void stage_rows(const T* __restrict__ src, int64_t row, int n, int C,
                                           int c, bool active, float* dst, int lane) {
  for (int i = 0; i < n; ++i) {
    float v[1] = {0.0f};
    if (active) load_ch<T, 1>(src + (row * n + i) * C + c, v);
    dst[i * 64 + lane] = v[0];
  }
}

template <class T>
__device__ __forceinline__ float load1(const T* __restrict__ p, bool active) {
  float v[1] = {0.0f};
  if (active) load_ch<T, 1>(p, v);
  return v[0];
}

// y operand of edge e into LDS: the given row Y[e][dy] (LY < 0), or the
// harmonics of the edge vector: every lane computes degrees 0..LY and lane
// i < dy stores the one its y component names (want = l*l + m, from the
// y irreps; -1 for lanes past dy).
template <int LY>
__device__ __forceinline__ void stage_edge_y(const float* __restrict__ src, int64_t e, int dy,
                                             int want, float* ys, int lane) {
  if constexpr (LY < 0) {
    for (int i = lane; i < dy; i += 64) ys[i] = src[e * dy + i];
  } else {
    constexpr int D = (LY + 1) * (LY + 1);
    float h[D];
    harmonics_bank_of_vec<LY>(src[3 * e], src[3 * e + 1], src[3 * e + 2], h);
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < D; ++q) v = want == q ? h[q] : v;
    if (want >= 0) ys[lane] = v;
  }
}

// ------------------------------------------------------------ tensor product

// Forward, dx and dw of the product (the table decides which): one
// wavefront per (row, 64 channels); the row's operand and y sit in LDS, the
// per-row weights come from global memory.
template <class T>
__global__ void __launch_bounds__(64 * kGenWaves)
    k_tp_generic(int64_t n_rows, int C, int dx, int dy, int dout, int np,
                 const int* __restrict__ prog, int64_t n_words, const T* __restrict__ x,
                 const float* __restrict__ y, const T* __restrict__ w, T* __restrict__ z) {
  const Table t = table_view(prog, n_words, dout);
  extern __shared__ float gsm[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* xs = gsm + wave * (dx * 64 + dy);
  float* ys = xs + dx * 64;
  const int cw = (C + 63) / 64;  // waves per row
  const int64_t total = n_rows * cw;
  for (int64_t item = int64_t(blockIdx.x) * kGenWaves + wave; item < total;
       item += int64_t(gridDim.x) * kGenWaves) {
    const int64_t row = item / cw;
    const int c = int(item % cw) * 64 + lane;
    const bool active = c < C;
    wave_lds_fence();  // the previous row's reads are done
    stage_rows<T>(x, row, dx, C, c, active, xs, lane);
    for (int i = lane; i < dy; i += 64) ys[i] = y[row * dy + i];
    wave_lds_fence();
    const T* wr = w + row * np * C + c;
    for (int o = 0; o < dout; ++o) {
      const float v = key_sum(
          t, o, dx, dy, np, xs, lane, [&](int p) { return load1<T>(wr + int64_t(p) * C, active); },
          [&](int i) { return ys[i]; });
      float out[1] = {v};
      if (active) store_ch<T, 1>(z + (row * dout + o) * C + c, out);
    }
  }
}

// k_tp_generic with two channels per lane (one wavefront per row and 128
// channels): the per-record scalar work, the index arithmetic and the
// harmonic reads are shared by the two channels.
template <class T>
__global__ void __launch_bounds__(256)
    k_tp_generic2(int64_t n_rows, int C, int dx, int dy, int dout, int np,
                  const int* __restrict__ prog, int64_t n_words, const T* __restrict__ x,
                  const float* __restrict__ y, const T* __restrict__ w, T* __restrict__ z) {
  const Table t = table_view(prog, n_words, dout);
  extern __shared__ float gsm2[];
  const int waves = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float2* xs = reinterpret_cast<float2*>(gsm2 + wave * (dx * 128 + ((dy + 1) & ~1)));
  float* ys = reinterpret_cast<float*>(xs + dx * 64);
  const int cw = (C + 127) / 128;  // waves per row
  const int64_t total = n_rows * cw;
  for (int64_t item = int64_t(blockIdx.x) * waves + wave; item < total;
       item += int64_t(gridDim.x) * waves) {
    const int64_t row = item / cw;
    const int c = int(item % cw) * 128 + 2 * lane;
    wave_lds_fence();  // the previous row's reads are done
    for (int i = 0; i < dx; ++i) xs[i * 64 + lane] = load_pair<T>(x + (row * dx + i) * C + c, c, C);
    for (int i = lane; i < dy; i += 64) ys[i] = y[row * dy + i];
    wave_lds_fence();
    const T* wr = w + row * np * C + c;
    for (int o = 0; o < dout; ++o) {
      const float2 v = key_sum2(
          t, o, dx, dy, np, xs, lane,
          [&](int p) { return load_pair<T>(wr + int64_t(p) * C, c, C); },
          [&](int i) { return ys[i]; });
      store_pair<T>(z + (row * dout + o) * C + c, c, C, v);
    }
  }
}

// Cotangent of y, summed over the channels, from the table keyed by the y
// component (records {x component | dz component << 16}, weight rows = the
// paths):  dy[i] = sum_c sum_P w[P][c] sum_records c x[xi][c] dz[o][c].
// One wavefront per row walks the channels 64 at a time; each key's lane
// values are added across the wave in a fixed order and the per-chunk sums
// are added in chunk order.
template <class T>
__global__ void __launch_bounds__(256)
    k_tp_generic_dy(int64_t n_rows, int C, int dx, int dy, int dout, int np,
                    const int* __restrict__ prog, int64_t n_words, const T* __restrict__ x,
                    const T* __restrict__ w, const T* __restrict__ dz, float* __restrict__ dyo) {
  const Table t = table_view(prog, n_words, dy);
  extern __shared__ float dsm[];
  const int waves = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* xs = dsm + wave * ((dx + dout) * 64 + dy);  // [dx][64]
  float* gs = xs + dx * 64;                           // [dout][64]
  float* acc = gs + dout * 64;                        // [dy]
  for (int64_t row = int64_t(blockIdx.x) * waves + wave; row < n_rows;
       row += int64_t(gridDim.x) * waves) {
    for (int c0 = 0; c0 < C; c0 += 64) {
      const int c = c0 + lane;
      const bool active = c < C;
      wave_lds_fence();
      stage_rows<T>(x, row, dx, C, c, active, xs, lane);
      stage_rows<T>(dz, row, dout, C, c, active, gs, lane);
      wave_lds_fence();
      const T* wr = w + row * np * C + c;
      for (int i = 0; i < dy; ++i) {
        const float v = key_sum(
            t, i, dx, dout, np, xs, lane,
            [&](int p) { return load1<T>(wr + int64_t(p) * C, active); },
            [&](int o) { return gs[o * 64 + lane]; });
        const float s = wave_sum(v);
        if (lane == 0) acc[i] = c0 == 0 ? s : acc[i] + s;
      }
    }
    wave_lds_fence();
    for (int i = lane; i < dy; i += 64) dyo[row * dy + i] = C > 0 ? acc[i] : 0.0f;
  }
}

// -------------------------------------------------------------- convolution

constexpr int kKeyBlock = 16;  // keys whose sums are held in registers per pass

// The keys [k0, k1) of work slice blockIdx.y of gridDim.y: a node's keys are
// split into slices of whole kKeyBlock blocks when the graph alone does not
// give the chip enough wavefronts (each slice re-stages its neighbours' rows).
__device__ __forceinline__ void key_slice(int keys, int& k0, int& k1) {
  const int blocks = (keys + kKeyBlock - 1) / kKeyBlock;
  const int per = (blocks + int(gridDim.y) - 1) / int(gridDim.y) * kKeyBlock;
  k0 = int(blockIdx.y) * per;
  k1 = min(keys, k0 + per);
}

// Segment sum over a node's edge list (e3j E.1 Eq.12-13):
//   out[node][k] = sum_{j in seg[node]..seg[node+1]} key_k(op[nbr[j]], Y_e, w[e]),
// e = emap[j] (or j).  With the forward table, seg = the receiver CSR and
// nbr = sender: the convolution.  With the dx table over the sender-ordered
// index (seg = colptr, emap = perm, nbr = recv, op = dm): the gradient of x.
// One wavefront per (node, 64 CPL channels).  e3j's CUDA convolution keeps
// the node's messages in a shared-memory buffer; here the sums of
// kKeyBlock keys at a time sit in registers and the edge list is walked
// once per block of keys (the neighbour rows come again from L2), which
// leaves LDS to the staged row alone and doubles the wavefronts per CU.
// The edges are taken in list order, so the result is reproducible.
// Entries whose neighbour is out of [0, n_nodes) (padding) are skipped.
template <class T, int LY, int CPL>
__global__ void __launch_bounds__(256)
    k_conv_generic_seg(int n_nodes, int n_edges, int C, int dop, int dy, int dkey, int np,
                       const int* __restrict__ prog, int64_t n_words,
                       const int* __restrict__ order, const int* __restrict__ seg,
                       const int* __restrict__ emap, const int* __restrict__ nbr,
                       const float* __restrict__ yv, YMap ym, const T* __restrict__ op,
                       const T* __restrict__ w, T* __restrict__ out) {
  static_assert(CPL == 1 || CPL == 2, "one or two channels per lane");
  const Table t = table_view(prog, n_words, dkey);
  extern __shared__ float csm[];
  const int waves = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* xs = csm + wave * (dop * 64 * CPL + ((dy + 1) & ~1));  // [dop][64] x CPL
  float* ys = xs + dop * 64 * CPL;                              // [dy]
  const int want = (LY >= 0 && lane < dy) ? ym.idx[lane] : -1;
  constexpr int CW = 64 * CPL;
  const int cw = (C + CW - 1) / CW;
  const int64_t total = int64_t(n_nodes) * cw;
  for (int64_t item = int64_t(blockIdx.x) * waves + wave; item < total;
       item += int64_t(gridDim.x) * waves) {
    const int slot = int(item / cw);
    int node = order ? order[slot] : slot;
    node = min(max(node, 0), n_nodes - 1);
    const int c = int(item % cw) * CW + CPL * lane;
    const bool active = c < C;
    const int jb = max(seg[node], 0), je = min(seg[node + 1], n_edges);
    int k0, k1;
    key_slice(dkey, k0, k1);
    for (int kb = k0; kb < k1; kb += kKeyBlock) {
      float acc[kKeyBlock][CPL] = {};
      for (int j = jb; j < je; ++j) {
        const int a = nbr[j];
        const int e = emap ? emap[j] : j;
        if (a < 0 || a >= n_nodes || e < 0 || e >= n_edges) continue;
        wave_lds_fence();  // the previous edge's reads of xs and ys are done
        if constexpr (CPL == 1) {
          stage_rows<T>(op, a, dop, C, c, active, xs, lane);
        } else {
          float2* x2 = reinterpret_cast<float2*>(xs);
          for (int i = 0; i < dop; ++i)
            x2[i * 64 + lane] = load_pair<T>(op + (int64_t(a) * dop + i) * C + c, c, C);
        }
        stage_edge_y<LY>(yv, e, dy, want, ys, lane);
        wave_lds_fence();
        const T* wr = w + int64_t(e) * np * C + c;
        sfor<0, kKeyBlock>([&](auto q) {
          if (kb + q < k1) {
            if constexpr (CPL == 1) {
              acc[q][0] += key_sum(
                  t, kb + q, dop, dy, np, xs, lane,
                  [&](int p) { return load1<T>(wr + int64_t(p) * C, active); },
                  [&](int i) { return ys[i]; });
            } else {
              const float2 v = key_sum2(
                  t, kb + q, dop, dy, np, reinterpret_cast<const float2*>(xs), lane,
                  [&](int p) { return load_pair<T>(wr + int64_t(p) * C, c, C); },
                  [&](int i) { return ys[i]; });
              acc[q][0] += v.x;
              acc[q][1] += v.y;
            }
          }
        });
      }
      sfor<0, kKeyBlock>([&](auto q) {
        if (kb + q < k1) {
          T* o = out + (int64_t(node) * dkey + kb + q) * C + c;
          if constexpr (CPL == 1) {
            const float v[1] = {acc[q][0]};
            if (active) store_ch<T, 1>(o, v);
          } else {
            store_pair<T>(o, c, C, make_float2(acc[q][0], acc[q][1]));
          }
        }
      });
    }
  }
}

// Weight cotangent of the convolution, receiver by receiver:
//   dw[e][P][c] = sum_o dm[b][o][c] sum_records c y_e[yi] x[a][xi][c]   (dw table)
// for every edge e = (a -> b).  One wavefront per (receiver b, 64 CPL
// channels) takes its edges in order; per edge only x[a] and the harmonics
// are staged in LDS, the weights dm[b][o] of the contributions come through
// the cache (the same row for all of b's edges).  Padding edges get dw = 0.
template <class T, int LY, int CPL>
__global__ void __launch_bounds__(256)
    k_conv_generic_dw(int n_nodes, int n_edges, int C, int dx, int dy, int dout, int np,
                      const int* __restrict__ pdw, int64_t dw_words,
                      const int* __restrict__ order, const int* __restrict__ rowptr,
                      const int* __restrict__ sender, const float* __restrict__ yv, YMap ym,
                      const T* __restrict__ x, const T* __restrict__ dm, T* __restrict__ dw) {
  static_assert(CPL == 1 || CPL == 2, "one or two channels per lane");
  const Table tw = table_view(pdw, dw_words, np);
  extern __shared__ float wsm[];
  const int waves = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* xs = wsm + wave * (dx * 64 * CPL + ((dy + 1) & ~1));  // [dx][64] x CPL
  float* ys = xs + dx * 64 * CPL;                              // [dy]
  const int want = (LY >= 0 && lane < dy) ? ym.idx[lane] : -1;
  constexpr int CW = 64 * CPL;
  const int cw = (C + CW - 1) / CW;
  const int64_t total = int64_t(n_nodes) * cw;
  for (int64_t item = int64_t(blockIdx.x) * waves + wave; item < total;
       item += int64_t(gridDim.x) * waves) {
    const int slot = int(item / cw);
    int b = order ? order[slot] : slot;
    b = min(max(b, 0), n_nodes - 1);
    const int c = int(item % cw) * CW + CPL * lane;
    const bool active = c < C;
    const T* gr = dm + int64_t(b) * dout * C + c;
    int p0, p1;  // this slice's paths
    key_slice(np, p0, p1);
    const int jb = max(rowptr[b], 0), je = min(rowptr[b + 1], n_edges);
    for (int e = jb; e < je; ++e) {
      const int a = sender[e];
      T* de = dw + int64_t(e) * np * C + c;
      if (a < 0 || a >= n_nodes) {  // padding
        for (int p = p0; p < p1; ++p) {
          if constexpr (CPL == 1) {
            const float z[1] = {0.0f};
            if (active) store_ch<T, 1>(de + int64_t(p) * C, z);
          } else {
            store_pair<T>(de + int64_t(p) * C, c, C, make_float2(0.0f, 0.0f));
          }
        }
        continue;
      }
      wave_lds_fence();  // the previous edge's reads are done
      if constexpr (CPL == 1) {
        stage_rows<T>(x, a, dx, C, c, active, xs, lane);
      } else {
        float2* x2 = reinterpret_cast<float2*>(xs);
        for (int i = 0; i < dx; ++i)
          x2[i * 64 + lane] = load_pair<T>(x + (int64_t(a) * dx + i) * C + c, c, C);
      }
      stage_edge_y<LY>(yv, e, dy, want, ys, lane);
      wave_lds_fence();
      for (int p = p0; p < p1; ++p) {
        if constexpr (CPL == 1) {
          const float v = key_sum(
              tw, p, dx, dy, dout, xs, lane,
              [&](int o) { return load1<T>(gr + int64_t(o) * C, active); },
              [&](int i) { return ys[i]; });
          const float o1[1] = {v};
          if (active) store_ch<T, 1>(de + int64_t(p) * C, o1);
        } else {
          const float2 v = key_sum2(
              tw, p, dx, dy, dout, reinterpret_cast<const float2*>(xs), lane,
              [&](int o) { return load_pair<T>(gr + int64_t(o) * C, c, C); },
              [&](int i) { return ys[i]; });
          store_pair<T>(de + int64_t(p) * C, c, C, v);
        }
      }
    }
  }
}

// Harmonic cotangent of the convolution, receiver by receiver:
//   dY[e][i] = sum_c sum_P w[e][P][c] sum_records c x[a][xi][c] dm[b][o][c]  (dy table)
// for every edge e = (a -> b).  One wavefront per receiver b takes its edges
// in order and, per edge, all channel chunks: x[a] and dm[b] are staged (both
// are per-lane factors of a record), each key is closed over the lanes with
// wave_sum and the chunk sums are added in chunk order.  Padding edges get
// dY = 0.
template <class T>
__global__ void __launch_bounds__(256)
    k_conv_generic_dY(int n_nodes, int n_edges, int C, int dx, int dy, int dout, int np,
                      const int* __restrict__ pdy, int64_t dy_words,
                      const int* __restrict__ order, const int* __restrict__ rowptr,
                      const int* __restrict__ sender, const T* __restrict__ x,
                      const T* __restrict__ w, const T* __restrict__ dm,
                      float* __restrict__ dY) {
  const Table ty = table_view(pdy, dy_words, dy);
  extern __shared__ float esm[];
  const int waves = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* xs = esm + wave * ((dx + dout) * 64 + dy);  // [dx][64]
  float* gs = xs + dx * 64;                           // [dout][64]
  float* accy = gs + dout * 64;                       // [dy]
  for (int64_t slot = int64_t(blockIdx.x) * waves + wave; slot < n_nodes;
       slot += int64_t(gridDim.x) * waves) {
    int b = order ? order[slot] : int(slot);
    b = min(max(b, 0), n_nodes - 1);
    int i0, i1;  // this slice's harmonic components
    key_slice(dy, i0, i1);
    const int jb = max(rowptr[b], 0), je = min(rowptr[b + 1], n_edges);
    for (int e = jb; e < je; ++e) {
      const int a = sender[e];
      if (a < 0 || a >= n_nodes) {  // padding
        for (int i = i0 + lane; i < i1; i += 64) dY[int64_t(e) * dy + i] = 0.0f;
        continue;
      }
      for (int c0 = 0; c0 < C; c0 += 64) {
        const int c = c0 + lane;
        const bool active = c < C;
        wave_lds_fence();  // the previous chunk's (or edge's) reads are done
        stage_rows<T>(x, a, dx, C, c, active, xs, lane);
        stage_rows<T>(dm, b, dout, C, c, active, gs, lane);
        wave_lds_fence();
        const T* wr = w + int64_t(e) * np * C + c;
        for (int i = i0; i < i1; ++i) {
          const float v = key_sum(
              ty, i, dx, dout, np, xs, lane,
              [&](int p) { return load1<T>(wr + int64_t(p) * C, active); },
              [&](int o) { return gs[o * 64 + lane]; });
          const float s = wave_sum(v);
          if (lane == 0) accy[i] = c0 == 0 ? s : accy[i] + s;
        }
      }
      wave_lds_fence();
      for (int i = i0 + lane; i < i1; i += 64) dY[int64_t(e) * dy + i] = C > 0 ? accy[i] : 0.0f;
    }
  }
}

// Key slices per (node, channel chunk) item: enough for about 16,384 work
// items on small graphs, at most one per block of kKeyBlock keys.
unsigned key_slices(int64_t node_items, int keys) {
  const int blocks = (keys + kKeyBlock - 1) / kKeyBlock;
  const int64_t want = (16384 + node_items - 1) / std::max<int64_t>(node_items, 1);
  return unsigned(std::max<int64_t>(1, std::min<int64_t>(blocks, want)));
}

// Waves per workgroup for a per-wave LDS need (floats), within 64 KiB.
int waves_for(int64_t per_wave) {
  return int(std::max<int64_t>(1, std::min<int64_t>(4, kLdsBlockFloats / per_wave)));
}

template <class T>
hipError_t launch_dy(const GenericTpArgs& a, const void* x, const void* w, const void* dz,
                     float* dyo, hipStream_t s) {
  const int64_t per_wave = int64_t(a.dx + a.dout) * 64 + a.dy;
  const int wv = waves_for(per_wave);
  const int64_t blocks = std::min<int64_t>((a.n_rows + wv - 1) / wv, 256 * 8);
  hipLaunchKernelGGL(k_tp_generic_dy<T>, dim3(unsigned(blocks)), dim3(64 * wv),
                     size_t(per_wave * wv) * sizeof(float), s, a.n_rows, a.C, a.dx, a.dy, a.dout,
                     a.np, a.prog, a.n_words, static_cast<const T*>(x),
                     static_cast<const T*>(w), static_cast<const T*>(dz), dyo);
  return hipGetLastError();
}

template <class T>
hipError_t launch2(const GenericTpArgs& a, hipStream_t s) {
  const int64_t per_wave = int64_t(a.dx) * 128 + ((a.dy + 1) & ~1);  // float2-aligned waves
  const int wv = waves_for(per_wave);
  const int64_t items = a.n_rows * ((a.C + 127) / 128);
  const int64_t blocks = std::min<int64_t>((items + wv - 1) / wv, 256 * 16);
  hipLaunchKernelGGL(k_tp_generic2<T>, dim3(unsigned(blocks)), dim3(64 * wv),
                     size_t(per_wave * wv) * sizeof(float), s, a.n_rows, a.C, a.dx, a.dy, a.dout,
                     a.np, a.prog, a.n_words, static_cast<const T*>(a.x), a.y,
                     static_cast<const T*>(a.w), static_cast<T*>(a.z));
  return hipGetLastError();
}

// Two channels per lane halve the per-record scalar and index work but
// double the LDS row; above 16 KB per wavefront (degree 5 and up with every
// irrep once) the lost occupancy costs more than that saves (measured).
template <class T>
hipError_t launch(const GenericTpArgs& a, hipStream_t s) {
  if (a.C > 64 && int64_t(a.dx) * 128 + a.dy <= 4096) return launch2<T>(a, s);
  const size_t lds = size_t(kGenWaves) * (a.dx * 64 + a.dy) * sizeof(float);
  const int64_t items = a.n_rows * ((a.C + 63) / 64);
  const int64_t blocks = std::min<int64_t>((items + kGenWaves - 1) / kGenWaves, 256 * 8);
  hipLaunchKernelGGL(k_tp_generic<T>, dim3(unsigned(blocks)), dim3(64 * kGenWaves), lds, s,
                     a.n_rows, a.C, a.dx, a.dy, a.dout, a.np, a.prog, a.n_words,
                     static_cast<const T*>(a.x), a.y, static_cast<const T*>(a.w),
                     static_cast<T*>(a.z));
  return hipGetLastError();
}

template <class T, int LY, int CPL>
hipError_t launch_seg_cpl(const GenericConvArgs& a, hipStream_t s) {
  const int64_t per_wave = int64_t(a.dop) * 64 * CPL + ((a.dy + 1) & ~1);
  const int wv = waves_for(per_wave);
  const int64_t items = int64_t(a.n_nodes) * ((a.C + 64 * CPL - 1) / (64 * CPL));
  const unsigned ks = key_slices(items, a.dkey);
  const int64_t blocks = std::min<int64_t>((items + wv - 1) / wv, 256 * 16 / ks + 1);
  hipLaunchKernelGGL((k_conv_generic_seg<T, LY, CPL>), dim3(unsigned(blocks), ks), dim3(64 * wv),
                     size_t(per_wave * wv) * sizeof(float), s, a.n_nodes, a.n_edges, a.C, a.dop,
                     a.dy, a.dkey, a.np, a.prog, a.n_words, a.order, a.seg, a.emap, a.nbr, a.yv,
                     a.ym, static_cast<const T*>(a.op), static_cast<const T*>(a.w),
                     static_cast<T*>(a.out));
  return hipGetLastError();
}

// Two channels per lane when the row fits 16 KB of LDS (as for the product).
template <class T, int LY>
hipError_t launch_seg(const GenericConvArgs& a, hipStream_t s) {
  if (a.C > 64 && int64_t(a.dop) * 128 + a.dy <= 4096) return launch_seg_cpl<T, LY, 2>(a, s);
  return launch_seg_cpl<T, LY, 1>(a, s);
}

template <class T, int LY, int CPL>
hipError_t launch_dw_cpl(const GenericConvEdgeArgs& a, hipStream_t s) {
  const int64_t per_wave = int64_t(a.dx) * 64 * CPL + ((a.dy + 1) & ~1);
  const int wv = waves_for(per_wave);
  const int64_t items = int64_t(a.n_nodes) * ((a.C + 64 * CPL - 1) / (64 * CPL));
  const unsigned ks = key_slices(items, a.np);
  const int64_t blocks = std::min<int64_t>((items + wv - 1) / wv, 256 * 16 / ks + 1);
  hipLaunchKernelGGL((k_conv_generic_dw<T, LY, CPL>), dim3(unsigned(blocks), ks), dim3(64 * wv),
                     size_t(per_wave * wv) * sizeof(float), s, a.n_nodes, a.n_edges, a.C, a.dx,
                     a.dy, a.dout, a.np, a.dw_prog, a.dw_words, a.order, a.rowptr, a.sender, a.yv,
                     a.ym, static_cast<const T*>(a.x), static_cast<const T*>(a.dm),
                     static_cast<T*>(a.dw));
  return hipGetLastError();
}

// dw (two channels per lane when the row fits, as for the forward), then dY.
template <class T, int LY>
hipError_t launch_edge(const GenericConvEdgeArgs& a, hipStream_t s) {
  hipError_t err = (a.C > 64 && int64_t(a.dx) * 128 + a.dy <= 4096)
                       ? launch_dw_cpl<T, LY, 2>(a, s)
                       : launch_dw_cpl<T, LY, 1>(a, s);
  if (err != hipSuccess) return err;
  const int64_t per_wave = int64_t(a.dx + a.dout) * 64 + a.dy;
  const int wv = waves_for(per_wave);
  const unsigned ksy = key_slices(a.n_nodes, a.dy);
  const int64_t blocks = std::min<int64_t>((int64_t(a.n_nodes) + wv - 1) / wv, 256 * 16 / ksy + 1);
  hipLaunchKernelGGL(k_conv_generic_dY<T>, dim3(unsigned(blocks), ksy), dim3(64 * wv),
                     size_t(per_wave * wv) * sizeof(float), s, a.n_nodes, a.n_edges, a.C, a.dx,
                     a.dy, a.dout, a.np, a.dy_prog, a.dy_words, a.order, a.rowptr, a.sender,
                     static_cast<const T*>(a.x), static_cast<const T*>(a.w),
                     static_cast<const T*>(a.dm), a.dY);
  return hipGetLastError();
}

// Degree of the harmonics computed in the kernel (-1: Y given) as a
// template argument.
template <class T, template <class, int> class F, class Args>
hipError_t by_degree(int ly, const Args& a, hipStream_t s) {
  switch (ly) {
    case -1: return F<T, -1>::run(a, s);
    case 0: return F<T, 0>::run(a, s);
    case 1: return F<T, 1>::run(a, s);
    case 2: return F<T, 2>::run(a, s);
    case 3: return F<T, 3>::run(a, s);
    case 4: return F<T, 4>::run(a, s);
    case 5: return F<T, 5>::run(a, s);
    case 6: return F<T, 6>::run(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <class T, int LY>
struct SegLaunch {
  static hipError_t run(const GenericConvArgs& a, hipStream_t s) { return launch_seg<T, LY>(a, s); }
};

template <class T, int LY>
struct EdgeLaunch {
  static hipError_t run(const GenericConvEdgeArgs& a, hipStream_t s) {
    return launch_edge<T, LY>(a, s);
  }
};

}  // namespace

hipError_t launch_tp_generic(const GenericTpArgs& a, int bf16, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  return bf16 ? launch<bf16_t>(a, s) : launch<float>(a, s);
}

hipError_t launch_tp_generic_dy(const GenericTpArgs& a, const void* dz, float* dy, int bf16,
                                hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  return bf16 ? launch_dy<bf16_t>(a, a.x, a.w, dz, dy, s)
              : launch_dy<float>(a, a.x, a.w, dz, dy, s);
}

hipError_t launch_conv_generic_seg(const GenericConvArgs& a, int bf16, hipStream_t s) {
  if (a.n_nodes <= 0) return hipSuccess;
  return bf16 ? by_degree<bf16_t, SegLaunch>(a.ly, a, s) : by_degree<float, SegLaunch>(a.ly, a, s);
}

hipError_t launch_conv_generic_edge(const GenericConvEdgeArgs& a, int bf16, hipStream_t s) {
  if (a.n_nodes <= 0 || a.n_edges <= 0) return hipSuccess;
  return bf16 ? by_degree<bf16_t, EdgeLaunch>(a.ly, a, s)
              : by_degree<float, EdgeLaunch>(a.ly, a, s);
}

}  // namespace e3k
