// gfx950 kernels of the fused equivariant convolution and the batched
// channel-wise tensor product, templated on the irreps signature S, the
// storage type T (float or bf16) and CPL, the channels held per lane.
//
// Work mapping: one 64-lane wavefront per receiver (forward) or per sender
// (backward).  The wavefront is split into 64/G edge groups of G = C/CPL
// lanes; group g walks edges g, g + 64/G, ... of the segment, each lane
// keeping CPL channels of the accumulator in registers.  Segments close with
// a fixed butterfly over the groups, so results are bitwise reproducible
// and no float atomics are used (e3j E.3: receiver-stationary aggregation;
// E.4: segmented reduction keyed on receivers, and on senders for dx).
#pragma once

#include "common.h"
#include "registry.h"

namespace e3k {

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = 64 * kWavesPerBlock;
constexpr int kXcds = 8;  // accelerator complex dies of an MI355X

// The forward keeps the next edge's x and w in flight (a second register
// buffer) only when that buffer is small.
template <class S, int CPL>
constexpr bool kFwdPrefetch = (Plan<S>::DX + Plan<S>::NP) * CPL <= 64;

// Node handled by this wavefront.  Workgroups are dispatched round-robin
// over the XCDs (workgroup i on XCD i % 8); each XCD is given a contiguous
// share of the traversal order, so the nodes that run together on one XCD
// are neighbours and share gathered rows in that XCD's L2.  The grid is a
// multiple of 8 workgroups; -1 for the waves past the end.
__device__ __forceinline__ int node_of_wave(int n_nodes, const int* __restrict__ order) {
  const int per_xcd = gridDim.x / kXcds;
  const int blk = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  const int w = blk * kWavesPerBlock + (threadIdx.x >> 6);
  if (w >= n_nodes) return -1;
  return order ? order[w] : w;
}

// ------------------------------------------------------------- forward
// m[b] = sum over the CSR segment of b of the weighted CG messages
// (e3j A.3 Eq.7, E.1 Eq.12-13).  Padding edges (a sender outside [0, N))
// are skipped.
template <class S, class T, int CPL, bool YG>
__global__ void __launch_bounds__(kBlock)
    k_conv_fwd(int n_nodes, int n_edges, int C, int G, const int* __restrict__ order,
               const int* __restrict__ rowptr,
               const int* __restrict__ sender, const float* __restrict__ ysrc,
               const T* __restrict__ x, const T* __restrict__ w, T* __restrict__ m) {
  using PL = Plan<S>;
  const int b = node_of_wave(n_nodes, order);
  if (b < 0 || b >= n_nodes) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const int NG = 64 / G;
  const int g = lane / G, ch0 = (lane - g * G) * CPL;

  float acc[PL::DO][CPL];
#pragma unroll
  for (int i = 0; i < PL::DO; ++i)
#pragma unroll
    for (int k = 0; k < CPL; ++k) acc[i][k] = 0.0f;

  // The segment is walked in chunks of 64 edges whose senders (and, from
  // edge vectors, the harmonics: one edge per lane) are
  // first staged in LDS, so every edge then costs a single round trip to
  // memory (x and w together) and no lane repeats another's harmonics.
  constexpr int DYS = (PL::DY + 3) & ~3;
  __shared__ int s_snd[kWavesPerBlock][64];
  __shared__ __align__(16) float s_y[kWavesPerBlock][YG ? 4 : 64 * DYS];
  int* snd = s_snd[threadIdx.x >> 6];
  float* ys = s_y[threadIdx.x >> 6];
  // a malformed rowptr cannot move the walk outside [0, n_edges)
  const int beg = max(rowptr[b], 0), end = min(rowptr[b + 1], n_edges);
  for (int c0 = beg; c0 < end; c0 += 64) {
    const int cn = min(64, end - c0);
    wave_lds_fence();  // every lane is done with the previous chunk
    if (lane < cn) {
      snd[lane] = sender[c0 + lane];
      if constexpr (!YG) {
        const float* r = ysrc + int64_t(c0 + lane) * 3;
        stage_y_from_vec<S>(r[0], r[1], r[2], ys + lane * DYS);
      }
    }
    wave_lds_fence();
    auto edge_yv = [&](int jj, float (&Y)[PL::DY]) {
      if constexpr (YG) {
        edge_y_given<S>(ysrc, c0 + jj, Y);
      } else {
        read_y_row<PL::DY>(ys + jj * DYS, Y);
      }
    };
    // software pipeline: the loads of the group's next edge are in flight
    // while the current edge is contracted
    auto valid = [&](int j) { return j < cn && snd[j] >= 0 && snd[j] < n_nodes; };
    auto issue = [&](int j, float (&xv)[PL::DX][CPL], float (&wv)[PL::NP][CPL]) {
      const T* xa = x + int64_t(snd[j]) * PL::DX * C + ch0;
#pragma unroll
      for (int i = 0; i < PL::DX; ++i) load_ch<T, CPL>(xa + int64_t(i) * C, xv[i]);
      const T* we = w + int64_t(c0 + j) * PL::NP * C + ch0;
#pragma unroll
      for (int p = 0; p < PL::NP; ++p) load_ch_stream<T, CPL>(we + int64_t(p) * C, wv[p]);
    };
    float xc[PL::DX][CPL], wc[PL::NP][CPL];
    int j = g;
    bool vc = valid(j);
    if constexpr (!kFwdPrefetch<S, CPL>) {
      for (; j < cn; j += NG) {
        if (!valid(j)) continue;
        issue(j, xc, wc);
        float Y[PL::DY];
        edge_yv(j, Y);
        edge_forward<S, CPL>(Y, xc, wc, acc);
      }
      continue;
    }
    if (vc) issue(j, xc, wc);
    while (j < cn) {
      const int jn = j + NG;
      const bool vn = valid(jn);
      float xn[PL::DX][CPL], wn[PL::NP][CPL];
      if (vn) issue(jn, xn, wn);
      if (vc) {
        float Y[PL::DY];
        edge_yv(j, Y);
        edge_forward<S, CPL>(Y, xc, wc, acc);
      }
#pragma unroll
      for (int i = 0; i < PL::DX; ++i)
#pragma unroll
        for (int k = 0; k < CPL; ++k) xc[i][k] = xn[i][k];
#pragma unroll
      for (int i = 0; i < PL::NP; ++i)
#pragma unroll
        for (int k = 0; k < CPL; ++k) wc[i][k] = wn[i][k];
      j = jn;
      vc = vn;
    }
  }

  T* mb = m + int64_t(b) * PL::DO * C + ch0;
  bool stored = false;
  if constexpr (PL::DO % 2 == 0) {
    if (G == 32) {  // two groups: halves trade their halves
      halves_reduce_scatter<PL::DO, CPL>(acc);
      const int off = g * (PL::DO / 2);
#pragma unroll
      for (int i = 0; i < PL::DO / 2; ++i)
        store_ch_stream<T, CPL>(mb + int64_t(off + i) * C, acc[i]);
      stored = true;
    }
  }
  if (!stored) {
    reduce_groups<PL::DO, CPL>(acc, G);
#pragma unroll
    for (int i = 0; i < PL::DO; ++i)
      if (i % NG == g) store_ch<T, CPL>(mb + int64_t(i) * C, acc[i]);
  }
}

// ------------------------------------------------------------ backward

// dst[0..N) = sum of v[0..N) over the G lanes of this lane's edge group (cl
// is the lane's index in the group): a reduce-scatter, after which the
// lanes that own distinct sums store them.  Lanes of other groups are never
// read, so groups past the end of the work may have returned already; with
// G = 64 the whole wavefront must be present.
template <int N>
__device__ __forceinline__ void store_group_sum(const float (&v)[N], int G, int lane, int cl,
                                                float* __restrict__ dst) {
  if (G == 64) {  // VALU-only cross-lane moves
    constexpr int NP = pow2_ceil_c(N);
    float t[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) t[i] = i < N ? v[i] : 0.0f;
    const int first = wave_reduce_scatter<N>(t, lane);
    if ((lane & 3) == 0 && first < N) dst[first] = t[0];
  } else {
    Scatter<N> sc;
    reduce_scatter<N>(v, G, lane, sc);
    constexpr int NP = Scatter<N>::NP;
    const int dup = (G > NP ? G / NP : 1) - 1;  // lanes holding copies
    if ((cl & dup) == 0) {
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int idx = sc.first + i;
        if (i < sc.count && idx < N) dst[idx] = sc.v[i];
      }
    }
  }
}

// Sender-ordered walk over the transposed index (colptr, perm, recv):
// dx[a] accumulates in registers over a's out-edges; dw[e] and dY[e] are
// edge-local and written once (e3j E.1 Eq.16; the sender-keyed reduction of
// E.4 replaces the atomics of E.3).
template <class S, class T, int CPL, bool YG>
__global__ void __launch_bounds__(kBlock)
    __attribute__((amdgpu_waves_per_eu(BwdWavesOf<S>::get(CPL == 1 ? 0 : CPL == 2 ? 1 : 2))))
    k_conv_bwd(int n_nodes, int n_edges, int C, int G, const int* __restrict__ order,
               const int* __restrict__ colptr,
               const int* __restrict__ perm, const int* __restrict__ recv,
               const float* __restrict__ ysrc, const T* __restrict__ x,
               const T* __restrict__ w, const T* __restrict__ dm, T* __restrict__ dx,
               T* __restrict__ dw, float* __restrict__ dY) {
  using PL = Plan<S>;
  const int a = node_of_wave(n_nodes, order);
  if (a < 0 || a >= n_nodes) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const int NG = 64 / G;
  const int g = lane / G, cl = lane - g * G, ch0 = cl * CPL;

  float xv[PL::DX][CPL], dxa[PL::DX][CPL];
  const T* xa = x + int64_t(a) * PL::DX * C + ch0;
#pragma unroll
  for (int i = 0; i < PL::DX; ++i) {
    load_ch<T, CPL>(xa + int64_t(i) * C, xv[i]);
#pragma unroll
    for (int k = 0; k < CPL; ++k) dxa[i][k] = 0.0f;
  }

  // Out-edges in chunks of 64: edge ids, receivers and (from edge vectors)
  // the harmonics, one edge per lane, are staged in LDS, then each edge
  // costs one round trip.
  // (Signatures that set kStageY false stage the edge vectors instead and
  // form the harmonics per edge in the loop, which their register budget
  // takes better.)
  constexpr bool SY = !YG && StageYOf<S>::value;
  constexpr int DYS = (PL::DY + 3) & ~3;
  constexpr int YROW = SY ? DYS : 3;
  __shared__ int s_e[kWavesPerBlock][64];
  __shared__ int s_b[kWavesPerBlock][64];
  __shared__ __align__(16) float s_y[kWavesPerBlock][YG ? 4 : 64 * YROW];
  int* se = s_e[threadIdx.x >> 6];
  int* sb = s_b[threadIdx.x >> 6];
  float* ys = s_y[threadIdx.x >> 6];
  // clamped so that a workspace built for another graph stays in bounds
  const int beg = max(colptr[a], 0), end = min(colptr[a + 1], n_edges);
  for (int c0 = beg; c0 < end; c0 += 64) {
    const int cn = min(64, end - c0);
    wave_lds_fence();
    if (lane < cn) {
      int e = perm[c0 + lane];
      const int b = recv[c0 + lane];
      if (e < 0 || e >= n_edges || b < 0 || b >= n_nodes) e = -1;  // only for malformed CSR
      se[lane] = e;
      sb[lane] = b;
      if constexpr (!YG) {
        const float* r = ysrc + int64_t(e < 0 ? 0 : e) * 3;
        if constexpr (SY) {
          stage_y_from_vec<S>(r[0], r[1], r[2], ys + lane * DYS);
        } else {
          ys[3 * lane] = r[0];
          ys[3 * lane + 1] = r[1];
          ys[3 * lane + 2] = r[2];
        }
      }
    }
    wave_lds_fence();
  for (int jj = g; jj < cn; jj += NG) {
    const int e = se[jj];
    const int b = sb[jj];
    if (e < 0) continue;
    float Y[PL::DY];
    if constexpr (YG)
      edge_y_given<S>(ysrc, e, Y);
    else if constexpr (SY)
      read_y_row<PL::DY>(ys + jj * DYS, Y);
    else
      edge_y_from_vec<S>(ys[3 * jj], ys[3 * jj + 1], ys[3 * jj + 2], Y);
    float wv[PL::NP][CPL], dmv[PL::DO][CPL];
    const T* we = w + int64_t(e) * PL::NP * C + ch0;
#pragma unroll
    for (int p = 0; p < PL::NP; ++p) load_ch_stream<T, CPL>(we + int64_t(p) * C, wv[p]);
    const T* dmb = dm + int64_t(b) * PL::DO * C + ch0;
#pragma unroll
    for (int i = 0; i < PL::DO; ++i) load_ch<T, CPL>(dmb + int64_t(i) * C, dmv[i]);

    float dYl[PL::DY];
#pragma unroll
    for (int i = 0; i < PL::DY; ++i) dYl[i] = 0.0f;
    edge_backward<S, CPL>(Y, xv, wv, dmv, dxa, dw + int64_t(e) * PL::NP * C + ch0, C, dYl);
    // dY[e] = sum over the group's channels
    store_group_sum<PL::DY>(dYl, G, lane, cl, dY + int64_t(e) * PL::DY);
  }
  }

  reduce_groups<PL::DX, CPL>(dxa, G);
  T* dxo = dx + int64_t(a) * PL::DX * C + ch0;
#pragma unroll
  for (int i = 0; i < PL::DX; ++i)
    if (i % NG == g) store_ch<T, CPL>(dxo + int64_t(i) * C, dxa[i]);
}

// Padding edges take no part in the transposed walk; their edge cotangents
// are zero.  npad and padlist come from the prepare step.
template <class T>
__global__ void __launch_bounds__(256)
    k_zero_padding_edges(const int* __restrict__ npad, const int* __restrict__ padlist,
                         int n_edges, int row, int dy, T* __restrict__ dw,
                         float* __restrict__ dY) {
  const int n = min(*npad, n_edges);
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    const int64_t e = padlist[i];
    if (e < 0 || e >= n_edges) continue;
    for (int k = threadIdx.x; k < row; k += blockDim.x) dw[e * row + k] = T{};
    for (int k = threadIdx.x; k < dy; k += blockDim.x) dY[e * dy + k] = 0.0f;
  }
}

// --------------------------------------------------- batched tensor product
// z[r] = sum_P w[r][P] (x[r] (x)_CG y[r])_P for independent rows (e3j E.1
// Eq.10-11); each edge group handles one row.
template <class S, class T, int CPL>
__global__ void __launch_bounds__(kBlock)
    k_tp_fwd(int64_t n_rows, int C, int G, const T* __restrict__ x, const float* __restrict__ y,
             const T* __restrict__ w, T* __restrict__ z) {
  using PL = Plan<S>;
  const int lane = threadIdx.x & 63;
  const int NG = 64 / G;
  const int g = lane / G, c0 = (lane - g * G) * CPL;
  const int64_t row =
      (int64_t(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6)) * NG + g;
  if (row >= n_rows) return;  // group-uniform; no shuffles follow

  float Y[PL::DY];
  edge_y_given<S>(y, row, Y);
  // every operand is read once and z written once: streaming accesses
  float xv[PL::DX][CPL];
  const T* xr = x + row * PL::DX * C + c0;
#pragma unroll
  for (int i = 0; i < PL::DX; ++i) load_ch_stream<T, CPL>(xr + int64_t(i) * C, xv[i]);
  float wv[PL::NP][CPL];
  const T* wr = w + row * PL::NP * C + c0;
#pragma unroll
  for (int p = 0; p < PL::NP; ++p) load_ch_stream<T, CPL>(wr + int64_t(p) * C, wv[p]);
  float acc[PL::DO][CPL];
#pragma unroll
  for (int i = 0; i < PL::DO; ++i)
#pragma unroll
    for (int k = 0; k < CPL; ++k) acc[i][k] = 0.0f;
  edge_forward<S, CPL>(Y, xv, wv, acc);
  T* zr = z + row * PL::DO * C + c0;
#pragma unroll
  for (int i = 0; i < PL::DO; ++i) store_ch_stream<T, CPL>(zr + int64_t(i) * C, acc[i]);
}

// Batched tensor-product backward (e3j E.1 Eq.14-16, one scalar per path):
// for the cotangent dz of z,
//   dx[r] = sum_P w[r][P] (y[r] (x)^T dz[r])_P,  dw[r][P] = <(x[r] (x) y[r])_P, dz[r]>,
//   dy[r] = sum over channels of sum_P w[r][P] (x[r] (x)^T dz[r])_P,
// in one pass over the row; each edge group handles one row.
template <class S, class T, int CPL>
__global__ void __launch_bounds__(kBlock)
    k_tp_bwd(int64_t n_rows, int C, int G, const T* __restrict__ x, const float* __restrict__ y,
             const T* __restrict__ w, const T* __restrict__ dz, T* __restrict__ dx,
             T* __restrict__ dw, float* __restrict__ dy) {
  using PL = Plan<S>;
  const int lane = threadIdx.x & 63;
  const int NG = 64 / G;
  const int g = lane / G, cl = lane - g * G, c0 = cl * CPL;
  const int64_t row =
      (int64_t(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6)) * NG + g;
  if (row >= n_rows) return;  // group-uniform (wave-uniform when G = 64)

  float Y[PL::DY];
  edge_y_given<S>(y, row, Y);
  float xv[PL::DX][CPL], wv[PL::NP][CPL], dzv[PL::DO][CPL];
  const T* xr = x + row * PL::DX * C + c0;
#pragma unroll
  for (int i = 0; i < PL::DX; ++i) load_ch_stream<T, CPL>(xr + int64_t(i) * C, xv[i]);
  const T* wr = w + row * PL::NP * C + c0;
#pragma unroll
  for (int p = 0; p < PL::NP; ++p) load_ch_stream<T, CPL>(wr + int64_t(p) * C, wv[p]);
  const T* dzr = dz + row * PL::DO * C + c0;
#pragma unroll
  for (int i = 0; i < PL::DO; ++i) load_ch_stream<T, CPL>(dzr + int64_t(i) * C, dzv[i]);

  float dxr[PL::DX][CPL], dYl[PL::DY];
#pragma unroll
  for (int i = 0; i < PL::DX; ++i)
#pragma unroll
    for (int k = 0; k < CPL; ++k) dxr[i][k] = 0.0f;
#pragma unroll
  for (int i = 0; i < PL::DY; ++i) dYl[i] = 0.0f;
  edge_backward<S, CPL>(Y, xv, wv, dzv, dxr, dw + row * PL::NP * C + c0, C, dYl);
  T* dxo = dx + row * PL::DX * C + c0;
#pragma unroll
  for (int i = 0; i < PL::DX; ++i) store_ch_stream<T, CPL>(dxo + int64_t(i) * C, dxr[i]);
  store_group_sum<PL::DY>(dYl, G, lane, cl, dy + row * PL::DY);
}

// ------------------------------------------------------------ launchers

template <int B, int E, class F>
void sfor_host(F&& f) {
  if constexpr (B < E) {
    f(ic<B>{});
    sfor_host<B + 1, E>(f);
  }
}

inline unsigned blocks_for(int64_t waves) {
  return unsigned((waves + kWavesPerBlock - 1) / kWavesPerBlock);
}

// One wavefront per node, rounded up to a whole number of XCD shares.
inline unsigned node_blocks(int64_t n_nodes) {
  const int64_t b = (n_nodes + kWavesPerBlock - 1) / kWavesPerBlock;
  return unsigned((b + kXcds - 1) / kXcds * kXcds);
}

template <class S, class T, int CPL, bool YG>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  if (a.n_nodes <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_conv_fwd<S, T, CPL, YG>), dim3(node_blocks(a.n_nodes)), dim3(kBlock), 0, s,
                     a.n_nodes, a.n_edges, a.C, a.G, a.order, a.rowptr, a.sender, a.ysrc,
                     static_cast<const T*>(a.x), static_cast<const T*>(a.w),
                     static_cast<T*>(a.m));
  return hipGetLastError();
}

template <class S, class T, int CPL, bool YG>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
  if (a.n_nodes <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_conv_bwd<S, T, CPL, YG>), dim3(node_blocks(a.n_nodes)), dim3(kBlock), 0, s,
                     a.n_nodes, int(a.n_edges), a.C, a.G, a.order, a.colptr, a.perm, a.recv, a.ysrc,
                     static_cast<const T*>(a.x), static_cast<const T*>(a.w),
                     static_cast<const T*>(a.dm), static_cast<T*>(a.dx), static_cast<T*>(a.dw),
                     a.dY);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.n_edges <= 0) return err;
  hipLaunchKernelGGL((k_zero_padding_edges<T>), dim3(256), dim3(256), 0, s, a.npad, a.padlist,
                     int(a.n_edges), Plan<S>::NP * a.C, Plan<S>::DY, static_cast<T*>(a.dw), a.dY);
  return hipGetLastError();
}

template <class S, class T, int CPL>
hipError_t launch_tp(const TpArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  const int64_t groups_per_wave = 64 / a.G;
  const int64_t waves = (a.n_rows + groups_per_wave - 1) / groups_per_wave;
  hipLaunchKernelGGL((k_tp_fwd<S, T, CPL>), dim3(blocks_for(waves)), dim3(kBlock), 0, s, a.n_rows,
                     a.C, a.G, static_cast<const T*>(a.x), a.y, static_cast<const T*>(a.w),
                     static_cast<T*>(a.z));
  return hipGetLastError();
}

template <class S, class T, int CPL>
hipError_t launch_tp_bwd(const TpBwdArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  const int64_t groups_per_wave = 64 / a.G;
  const int64_t waves = (a.n_rows + groups_per_wave - 1) / groups_per_wave;
  hipLaunchKernelGGL((k_tp_bwd<S, T, CPL>), dim3(blocks_for(waves)), dim3(kBlock), 0, s,
                     a.n_rows, a.C, a.G, static_cast<const T*>(a.x), a.y,
                     static_cast<const T*>(a.w), static_cast<const T*>(a.dz),
                     static_cast<T*>(a.dx), static_cast<T*>(a.dw), a.dy);
  return hipGetLastError();
}

template <class S>
KernelSet make_set(const char* name) {
  KernelSet k{};
  k.name = name;
  k.nx = S::NX;
  k.ny = S::NY;
  k.no = S::NO;
  for (int i = 0; i < S::NX; ++i) k.x[i] = IrSpec{S::X[i].l, S::X[i].p};
  for (int i = 0; i < S::NY; ++i) k.y[i] = IrSpec{S::Y[i].l, S::Y[i].p};
  for (int i = 0; i < S::NO; ++i) k.o[i] = IrSpec{S::O[i].l, S::O[i].p};
  k.dx = Plan<S>::DX;
  k.dy = Plan<S>::DY;
  k.dout = Plan<S>::DO;
  k.np = Plan<S>::NP;
  k.per_path = PerPathOf<S>::value ? 1 : 0;
  sfor_host<0, 3>([&](auto c) {
    constexpr int CPL = 1 << c;
    k.fwd[0][0][c] = &launch_fwd<S, float, CPL, false>;
    k.fwd[0][1][c] = &launch_fwd<S, float, CPL, true>;
    k.fwd[1][0][c] = &launch_fwd<S, bf16_t, CPL, false>;
    k.fwd[1][1][c] = &launch_fwd<S, bf16_t, CPL, true>;
    k.bwd[0][0][c] = &launch_bwd<S, float, CPL, false>;
    k.bwd[0][1][c] = &launch_bwd<S, float, CPL, true>;
    k.bwd[1][0][c] = &launch_bwd<S, bf16_t, CPL, false>;
    k.bwd[1][1][c] = &launch_bwd<S, bf16_t, CPL, true>;
    k.tpb[0][c] = &launch_tp_bwd<S, float, CPL>;
    k.tpb[1][c] = &launch_tp_bwd<S, bf16_t, CPL>;
  });
  sfor_host<0, 3>([&](auto c) {
    constexpr int CPL = 1 << c;
    k.tp[0][c] = &launch_tp<S, float, CPL>;
    k.tp[1][c] = &launch_tp<S, bf16_t, CPL>;
  });
  return k;
}

}  // namespace e3k
