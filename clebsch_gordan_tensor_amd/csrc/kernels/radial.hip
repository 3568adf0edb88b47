// Radial edge weights on the gfx950 matrix cores, and the convolution that
// computes them on the fly so that w never reaches HBM.
//
// The e3j paper (A.3, the edge scalars of Eq.7; E.1, message weighting with
// edge scalars) takes the per-edge, per-path, per-channel weights from an MLP
// applied to a radial basis embedding of |r|; its model table (Table 3) uses
// 8 basis functions.  The reading built here (the pages fix nothing else):
//   B_n(d) = sqrt(2/r_c) sin(n pi d / r_c) / d,  n = 1..8
//   h_k    = silu(sum_n B_n W1[n][k]),          k < 64
//   w[j]   = sum_k h_k W2[k][j],                j < P*C  (layout w[e][P][C])
//
// k_radial_mlp writes w with the same fp16 high/low product as the fused
// convolution below.
//
// k_conv_fwd_radial fuses it into the forward convolution.  One 512-thread
// workgroup per CU holds, for a 32-channel slab, W2 split into fp16 high and
// low parts (W2 = hi + lo to 22 bits) in LDS; h is split the same way and
// w = hi*hi + hi*lo + lo*hi is formed by three v_mfma_f32_16x16x32_f16 per
// K-step (the lo*lo term is below 2^-22 of the product), accurate to a few
// 1e-7 of |w| -- the fp32 convolution's tolerance holds.  Each wavefront
// walks one receiver's edges in tiles of 16: per path the MFMAs leave
// w[edge][channel] for 4 edges x 2 channels in every lane (rows 4*(lane/16)+r,
// columns lane%16 of two 16-column blocks), and the CG contraction of those
// 4 edges follows on the VALU with the weights still in registers.  Slabs
// are spread over the XCDs (slab = XCD mod slabs), and each XCD walks its
// share of the receivers in the locality order of the prepare step.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "common.h"
#include "partial_sums.h"
#include "registry.h"
#include "signatures.h"

namespace e3k {
namespace {

constexpr int kRadBasis = 8;
constexpr int kRadHidden = 64;
constexpr int kRadXcds = 8;
// Low parts of the fp16 splits are stored times 2^11 so that they stay
// normal numbers (a low part is ~2^-12 of its value, often below fp16's
// normal range); the cross products are scaled back once.
constexpr float kLoScale = 2048.0f;
constexpr float kLoUnscale = 1.0f / 2048.0f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

// B[n] = sqrt(2/rc) sin((n+1) pi d / rc) / d of the edge vector (vx, vy, vz),
// at d = 0 the limit sqrt(2/rc) (n+1) pi / rc.  Evaluated in fp64 and rounded
// once: the arguments (n+1) pi d / rc reach tens of radians, where an fp32
// argument alone is off by ~1e-6 absolute -- more than the MLP's outputs
// tolerate relative to their typical size.  sin((n+1)t) by the Chebyshev
// recurrence s_{n+1} = 2 cos(t) s_n - s_{n-1}.
__device__ __forceinline__ void bessel_basis(float vx, float vy, float vz, float rc,
                                             float (&B)[kRadBasis]) {
  const double d = sqrt(double(vx) * vx + double(vy) * vy + double(vz) * vz);
  const double pref = sqrt(2.0 / double(rc));
  if (d > 0.0) {
    double s, c;
    sincos(3.141592653589793 * d / double(rc), &s, &c);
    const double inv = pref / d;
    double sp = 0.0, sn = s;
#pragma unroll
    for (int n = 0; n < kRadBasis; ++n) {
      B[n] = float(sn * inv);
      const double nx = fma(2.0 * c, sn, -sp);
      sp = sn;
      sn = nx;
    }
  } else {
#pragma unroll
    for (int n = 0; n < kRadBasis; ++n)
      B[n] = float(pref * double(n + 1) * 3.141592653589793 / double(rc));
  }
}

// correctly rounded: a 1-ulp reciprocal here already moves the convolution's
// outputs by 1e-5 of their RMS on heavy-tailed graphs
__device__ __forceinline__ float silu(float t) { return t / (1.0f + expf(-t)); }

// ------------------------------------------------------------ radial MLP

constexpr int kMlpCols = 128;  // columns per workgroup slab (8 MFMA blocks)

// The A operand of one 16-edge tile: h of edge row lane%16 for hidden units
// 32*ks + 8*(lane/16) + (0..7), split into fp16 high and scaled low parts.
__device__ __forceinline__ void hidden_operands(const float (&B)[kRadBasis], bool valid,
                                                const float* __restrict__ s_w1, int gq,
                                                half8 (&ah)[2], half8 (&al)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    float pre[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) pre[q] = 0.0f;
#pragma unroll
    for (int n = 0; n < kRadBasis; ++n) {
      const float4* w1 = reinterpret_cast<const float4*>(s_w1 + n * kRadHidden + ks * 32 + 8 * gq);
      const float4 u = w1[0], v = w1[1];
      pre[0] = fmaf(B[n], u.x, pre[0]);
      pre[1] = fmaf(B[n], u.y, pre[1]);
      pre[2] = fmaf(B[n], u.z, pre[2]);
      pre[3] = fmaf(B[n], u.w, pre[3]);
      pre[4] = fmaf(B[n], v.x, pre[4]);
      pre[5] = fmaf(B[n], v.y, pre[5]);
      pre[6] = fmaf(B[n], v.z, pre[6]);
      pre[7] = fmaf(B[n], v.w, pre[7]);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float h = valid ? silu(pre[q]) : 0.0f;
      const _Float16 hh = static_cast<_Float16>(h);
      ah[ks][q] = hh;
      al[ks][q] = static_cast<_Float16>((h - static_cast<float>(hh)) * kLoScale);
    }
  }
}

// The hidden layer of every edge in the operand form the fused convolution
// reads (kRadialHiddenBytes per edge): the basis of the workgroup's 64 edges
// first (one thread per edge, into LDS), then thread (edge, quarter q) forms
// units 32 ks + 8 q + (0..7) for ks = 0, 1 exactly as the convolution would,
// and stores the fp16 high and scaled low parts at [e][ks][q][hi, lo].
// Every edge is written (its sender is not known here; the convolution
// zeroes the operands of padding edges itself).
__global__ void __launch_bounds__(256)
    k_radial_hidden(int n_edges, const float* __restrict__ vec, float rc,
                    const float* __restrict__ W1, half8* __restrict__ h) {
  __shared__ __align__(16) float s_w1[kRadBasis * kRadHidden];
  __shared__ float s_bas[64][kRadBasis + 1];
  for (int i = threadIdx.x; i < kRadBasis * kRadHidden; i += blockDim.x) s_w1[i] = W1[i];
  const int64_t e0 = int64_t(blockIdx.x) * 64;
  if (threadIdx.x < 64) {
    const int64_t e = e0 + threadIdx.x;
    float B[kRadBasis];
    if (e < n_edges)
      bessel_basis(vec[e * 3], vec[e * 3 + 1], vec[e * 3 + 2], rc, B);
    else
      bessel_basis(0.0f, 0.0f, 0.0f, rc, B);
#pragma unroll
    for (int n = 0; n < kRadBasis; ++n) s_bas[threadIdx.x][n] = B[n];
  }
  __syncthreads();
  const int64_t e = e0 + (threadIdx.x >> 2);
  const int q = int(threadIdx.x & 3);
  if (e >= n_edges) return;
  float B[kRadBasis];
#pragma unroll
  for (int n = 0; n < kRadBasis; ++n) B[n] = s_bas[threadIdx.x >> 2][n];
  half8 ah[2], al[2];
  hidden_operands(B, true, s_w1, q, ah, al);
  half8* o = h + e * 16;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    o[(ks * 4 + q) * 2] = ah[ks];
    o[(ks * 4 + q) * 2 + 1] = al[ks];
  }
}

// w[e][j] for all edges; workgroup = (column slab, edge-tile group), 4 waves,
// one 16-edge tile per wave at a time.  The product h W2 runs on the fp16
// matrix cores with the same high/low split as the fused convolution below
// (hi*hi + hi*lo + lo*hi, low parts scaled by 2^11): 6 v_mfma_f32_16x16x32_f16
// per 16 columns instead of 16 fp32 MFMAs at twice the cycles each.  W2's
// slab sits in LDS in the B operand order (k = 32*ks + 8*(lane/16) + t,
// column lane%16); the 16 x 128 result tile goes through LDS (rows padded by
// 4 floats against bank conflicts) so that every store instruction writes two
// 512-byte row segments, 16 bytes per lane.
constexpr int kMlpTileStride = kMlpCols + 4;

constexpr size_t mlp_lds_bytes() {
  return size_t(kMlpCols / 16) * 2 * 2 * 64 * sizeof(half8)  // W2 slab, [cb][ks][hi/lo][lane]
         + size_t(kRadBasis) * kRadHidden * sizeof(float)     // W1
         + size_t(4) * 16 * kMlpTileStride * sizeof(float);   // result tiles
}

// HG: the hidden layer's operands come from k_radial_hidden (hid) instead of
// being formed here for every column slab.
template <bool HG>
__global__ void __launch_bounds__(256)
    k_radial_mlp(int n_edges, int n_cols, int n_slabs, int n_groups, const float* __restrict__ vec,
                 float rc, const float* __restrict__ W1, const float* __restrict__ W2,
                 const half8* __restrict__ hid, float* __restrict__ w) {
  extern __shared__ __align__(16) unsigned char mlp_smem[];
  half8* s_w2 = reinterpret_cast<half8*>(mlp_smem);
  float* s_w1 = reinterpret_cast<float*>(mlp_smem + size_t(kMlpCols / 16) * 4 * 64 * sizeof(half8));
  float* s_t = s_w1 + kRadBasis * kRadHidden;  // [wave][16][stride]
  const int slab = blockIdx.x % n_slabs, group = blockIdx.x / n_slabs;
  for (int i = threadIdx.x; i < (kMlpCols / 16) * 2 * 64; i += blockDim.x) {
    const int cb = i / 128, ks = (i / 64) % 2, l = i % 64;
    const int col = slab * kMlpCols + cb * 16 + (l & 15);
    const int k0 = ks * 32 + 8 * (l >> 4);
    half8 hi, lo;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float v = col < n_cols ? W2[int64_t(k0 + t) * n_cols + col] : 0.0f;
      hi[t] = static_cast<_Float16>(v);
      lo[t] = static_cast<_Float16>((v - static_cast<float>(hi[t])) * kLoScale);
    }
    s_w2[(cb * 2 + ks) * 128 + l] = hi;
    s_w2[(cb * 2 + ks) * 128 + 64 + l] = lo;
  }
  for (int i = threadIdx.x; i < kRadBasis * kRadHidden; i += blockDim.x) s_w1[i] = W1[i];
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, gq = lane >> 4;
  float* tile_lds = s_t + wave * 16 * kMlpTileStride;
  const int ntiles = (n_edges + 15) / 16;
  const int width = min(kMlpCols, n_cols - slab * kMlpCols);  // multiple of 16
  const int ncb = width / 16;
  for (int tile = group * 4 + wave; tile < ntiles; tile += n_groups * 4) {
    const int er = tile * 16 + (lane & 15);
    half8 ah[2], al[2];
    if constexpr (HG) {
      const bool ok = er < n_edges;
      const half8* hp = hid + int64_t(ok ? er : 0) * 16 + gq * 2;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const half8 vh = hp[ks * 8], vl = hp[ks * 8 + 1];
        ah[ks] = ok ? vh : half8{};
        al[ks] = ok ? vl : half8{};
      }
      wave_lds_fence();  // the previous tile's LDS reads are done
    } else {
      float vx = 0.0f, vy = 0.0f, vz = 0.0f;
      if (er < n_edges) {
        const float* p = vec + int64_t(er) * 3;
        vx = p[0];
        vy = p[1];
        vz = p[2];
      }
      float B[kRadBasis];
      bessel_basis(vx, vy, vz, rc, B);
      wave_lds_fence();  // the previous tile's LDS reads are done; keeps W1 reads here
      hidden_operands(B, er < n_edges, s_w1, gq, ah, al);
    }
    for (int cb = 0; cb < ncb; ++cb) {
      float4v D = {0.0f, 0.0f, 0.0f, 0.0f}, X = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const half8 bh = s_w2[(cb * 2 + ks) * 128 + lane];
        const half8 bl = s_w2[(cb * 2 + ks) * 128 + 64 + lane];
        D = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[ks], bh, D, 0, 0, 0);
        X = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[ks], bl, X, 0, 0, 0);
        X = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[ks], bh, X, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        tile_lds[(4 * gq + r) * kMlpTileStride + cb * 16 + (lane & 15)] =
            fmaf(X[r], kLoUnscale, D[r]);
    }
    wave_lds_fence();
    // two rows per instruction: lanes 0..31 row 2i, lanes 32..63 row 2i+1
    const int q = lane & 31, half = lane >> 5;
    if (4 * q < width) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 2 * i + half;
        const int e = tile * 16 + row;
        if (e < n_edges) {
          const float4v v =
              *reinterpret_cast<const float4v*>(tile_lds + row * kMlpTileStride + 4 * q);
          __builtin_nontemporal_store(
              v, reinterpret_cast<float4v*>(w + int64_t(e) * n_cols + slab * kMlpCols) + q);
        }
      }
    }
  }
}

// ------------------------------------------- fused radial convolution

constexpr int kRadWaves = 8;  // 512-thread workgroups, one per CU

// One path of e3j E.1 Eq.13 for one edge and CPL channels, with the edge's
// harmonics of degree l2 in Yl (component m2 at Yl[m2]):
//   acc[oo+M][k] += w[k] sum_{m1,m2} c(M,m1,m2) Yl[m2] x[xo+m1][k]
// in the cheaper of the two orders (contract then weight, or weight x first).
template <class S, int PI, int CPL>
__device__ __forceinline__ void path_forward(const float* __restrict__ Yl,
                                             const float (&xv)[Plan<S>::DX][CPL],
                                             const float (&wp)[CPL],
                                             float (&acc)[CPL][Plan<S>::DO]) {
  constexpr PathC P = Plan<S>::paths.p[PI];
  constexpr int n1 = 2 * P.l1 + 1, nL = 2 * P.L + 1;
  float y[2 * P.l2 + 1];
#pragma unroll
  for (int i = 0; i < 2 * P.l2 + 1; ++i) y[i] = Yl[i];
  if constexpr (n1 < nL) {
    float u[n1][CPL];
#pragma unroll
    for (int a = 0; a < n1; ++a)
#pragma unroll
      for (int k = 0; k < CPL; ++k) u[a][k] = wp[k] * xv[P.xo + a][k];
    float A = 0.0f;
    sfor<0, P.rcnt>([&](auto r) {
      constexpr CgRec R = kRec[P.roff + r];
      if constexpr (group_first(P.roff, r))
        A = R.c * y[R.m2];
      else
        A = fmaf(R.c, y[R.m2], A);
      if constexpr (group_last(P.roff, P.rcnt, r)) {
#pragma unroll
        for (int k = 0; k < CPL; ++k) acc[k][P.oo + R.M] = fmaf(A, u[R.m1][k], acc[k][P.oo + R.M]);
      }
    });
  } else {
    float z[nL][CPL];
#pragma unroll
    for (int M = 0; M < nL; ++M)
#pragma unroll
      for (int k = 0; k < CPL; ++k) z[M][k] = 0.0f;
    float A = 0.0f;
    sfor<0, P.rcnt>([&](auto r) {
      constexpr CgRec R = kRec[P.roff + r];
      if constexpr (group_first(P.roff, r))
        A = R.c * y[R.m2];
      else
        A = fmaf(R.c, y[R.m2], A);
      if constexpr (group_last(P.roff, P.rcnt, r)) {
#pragma unroll
        for (int k = 0; k < CPL; ++k) z[R.M][k] = fmaf(A, xv[P.xo + R.m1][k], z[R.M][k]);
      }
    });
#pragma unroll
    for (int M = 0; M < nL; ++M)
#pragma unroll
      for (int k = 0; k < CPL; ++k) acc[k][P.oo + M] = fmaf(wp[k], z[M][k], acc[k][P.oo + M]);
  }
}

constexpr int kRadChunk = 64;  // edges staged per wavefront at a time (four 16-edge tiles)

template <class S>
constexpr size_t radial_lds_bytes() {
  using PL = Plan<S>;
  return size_t(PL::NP) * 8 * 64 * sizeof(half8)                           // W2 slab, hi and lo
         + size_t(kRadBasis) * kRadHidden * sizeof(float)                   // W1
         + size_t(kRadWaves) * kRadChunk * kRadBasis * sizeof(float)        // basis of a chunk
         + size_t(kRadWaves) * kRadChunk * (PL::DY + 1) * sizeof(float)     // harmonics
         + size_t(kRadWaves) * kRadChunk * sizeof(int);                     // senders
}

// HG: the hidden layer's operands come from k_radial_hidden (hid) instead of
// being formed here, once per 32-channel slab, from the edge's basis.
template <class S, bool HG>
__global__ void __launch_bounds__(64 * kRadWaves, 1)
    k_conv_fwd_radial(int n_nodes, int n_edges, int C, int n_slabs, const int* __restrict__ order,
                      const int* __restrict__ rowptr, const int* __restrict__ sender,
                      const float* __restrict__ vec, const float* __restrict__ x,
                      const float* __restrict__ W1, const float* __restrict__ W2, float rc,
                      const half8* __restrict__ hid, float* __restrict__ m) {
  using PL = Plan<S>;
  constexpr int NP = PL::NP, DX = PL::DX, DY = PL::DY, DO = PL::DO, YS = DY + 1;
  extern __shared__ __align__(16) unsigned char smem[];
  half8* s_w2 = reinterpret_cast<half8*>(smem);  // [NP][cb 2][ks 2][hi/lo 2][64 lanes]
  float* s_w1 = reinterpret_cast<float*>(smem + size_t(NP) * 8 * 64 * sizeof(half8));
  float* s_b = s_w1 + kRadBasis * kRadHidden;                  // [wave][64][8]
  float* s_y = s_b + kRadWaves * kRadChunk * kRadBasis;        // [wave][64][YS]
  int* s_snd = reinterpret_cast<int*>(s_y + kRadWaves * kRadChunk * YS);  // [wave][64]

  const int xcd = blockIdx.x % kRadXcds, slot = blockIdx.x / kRadXcds;
  const int slab = xcd % n_slabs, part = xcd / n_slabs, n_parts = kRadXcds / n_slabs;
  const int64_t ncols = int64_t(NP) * C;
  for (int i = threadIdx.x; i < NP * 4 * 64; i += blockDim.x) {
    const int p = i / 256, cb = (i / 128) % 2, ks = (i / 64) % 2, l = i % 64;
    const int64_t col = int64_t(p) * C + slab * 32 + cb * 16 + (l & 15);
    const int k0 = ks * 32 + 8 * (l >> 4);
    half8 hi, lo;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float v = W2[int64_t(k0 + t) * ncols + col];
      hi[t] = static_cast<_Float16>(v);
      lo[t] = static_cast<_Float16>((v - static_cast<float>(hi[t])) * kLoScale);
    }
    s_w2[(i / 64) * 128 + l] = hi;
    s_w2[(i / 64) * 128 + 64 + l] = lo;
  }
  for (int i = threadIdx.x; i < kRadBasis * kRadHidden; i += blockDim.x) s_w1[i] = W1[i];
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gq = lane >> 4, li = lane & 15;
  float* bs = s_b + wave * kRadChunk * kRadBasis;
  float* ys = s_y + wave * kRadChunk * YS;
  int* sn = s_snd + wave * kRadChunk;
  const int chan = slab * 32 + li;  // + 16 * cb
  const int per_part = (n_nodes + n_parts - 1) / n_parts;
  const int lo_pos = part * per_part, hi_pos = min(n_nodes, lo_pos + per_part);
  const int waves_here = (gridDim.x / kRadXcds) * kRadWaves;

  for (int pos = lo_pos + slot * kRadWaves + wave; pos < hi_pos; pos += waves_here) {
    const int b = order ? order[pos] : pos;
    float acc[2][DO];
#pragma unroll
    for (int o = 0; o < DO; ++o) acc[0][o] = acc[1][o] = 0.0f;
    const int beg = max(rowptr[b], 0), end = min(rowptr[b + 1], n_edges);
    for (int c0 = beg; c0 < end; c0 += kRadChunk) {
      // stage one edge per lane: sender, radial basis and harmonics
      wave_lds_fence();  // the previous chunk's reads are done
      {
        const int e = c0 + lane;
        int sr = -1;
        float vx = 0.0f, vy = 0.0f, vz = 0.0f;
        if (e < end) {
          sr = sender[e];
          vx = vec[int64_t(e) * 3];
          vy = vec[int64_t(e) * 3 + 1];
          vz = vec[int64_t(e) * 3 + 2];
        }
        sn[lane] = (sr >= 0 && sr < n_nodes) ? sr : -1;
        if constexpr (!HG) {
          float B[kRadBasis];
          bessel_basis(vx, vy, vz, rc, B);
#pragma unroll
          for (int n = 0; n < kRadBasis; ++n) bs[lane * kRadBasis + n] = B[n];
        }
        float Y[DY];
        edge_y_from_vec<S>(vx, vy, vz, Y);
#pragma unroll
        for (int i = 0; i < DY; ++i) ys[lane * YS + i] = Y[i];
      }
      wave_lds_fence();
      const int nt = (min(kRadChunk, end - c0) + 15) / 16;
      for (int t = 0; t < nt; ++t) {
        // keeps the tile's LDS reads (W1 above all) inside the loop instead of
        // hoisted into registers for the whole chunk
        wave_lds_fence();
        // A operand: h of edge row t*16 + li, units ks*32 + 8*gq + (0..7)
        half8 ah[2], al[2];
        {
          const int row = t * 16 + li;
          if constexpr (HG) {
            // a padding edge (or a row past the list) takes zero operands;
            // otherwise the row's edge c0 + row < end is in [0, n_edges)
            const bool ok = sn[row] >= 0;
            const half8* hp = hid + int64_t(ok ? c0 + row : 0) * 16 + gq * 2;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              const half8 vh = hp[ks * 8], vl = hp[ks * 8 + 1];
              ah[ks] = ok ? vh : half8{};
              al[ks] = ok ? vl : half8{};
            }
          } else {
            float B[kRadBasis];
#pragma unroll
            for (int n = 0; n < kRadBasis; ++n) B[n] = bs[row * kRadBasis + n];
            hidden_operands(B, sn[row] >= 0, s_w1, gq, ah, al);
          }
        }
        // x of this lane's contraction rows t*16 + 4*gq + rr, channels chan + 16*cb
        float xv[4][DX][2];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int sidx = sn[t * 16 + 4 * gq + rr];
#pragma unroll
          for (int i = 0; i < DX; ++i)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
              xv[rr][i][cb] = sidx >= 0 ? x[(int64_t(sidx) * DX + i) * C + chan + 16 * cb] : 0.0f;
        }
        // hi*hi in D, the two cross products (low parts scaled by 2^11) in X
        sfor<0, NP>([&](auto pi) {
          constexpr PathC P = PL::paths.p[pi];
          const half8* wb = s_w2 + size_t(pi) * 512;
          float4v D[2], X[2];
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            D[cb] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
            X[cb] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              const half8 bh = wb[(cb * 2 + ks) * 128 + lane];
              const half8 bl = wb[(cb * 2 + ks) * 128 + 64 + lane];
              D[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[ks], bh, D[cb], 0, 0, 0);
              X[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[ks], bl, X[cb], 0, 0, 0);
              X[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[ks], bh, X[cb], 0, 0, 0);
            }
          }
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const float wp[2] = {fmaf(X[0][rr], kLoUnscale, D[0][rr]),
                                 fmaf(X[1][rr], kLoUnscale, D[1][rr])};
            path_forward<S, pi, 2>(ys + (t * 16 + 4 * gq + rr) * YS + P.yo, xv[rr], wp, acc);
          }
        });
      }
    }
    // the four lane groups hold partial sums over different edges of the
    // same channels: fixed butterfly, then group gq stores components o = gq mod 4
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int o = 0; o < DO; ++o) {
        float v = acc[cb][o];
        v += shfl_xor_c<16>(v);
        v += shfl_xor_c<32>(v);
        acc[cb][o] = v;
      }
    float* mb = m + int64_t(b) * DO * C + chan;
#pragma unroll
    for (int o = 0; o < DO; ++o)
      if ((o & 3) == gq) {
        __builtin_nontemporal_store(acc[0][o], mb + int64_t(o) * C);
        __builtin_nontemporal_store(acc[1][o], mb + int64_t(o) * C + 16);
      }
  }
}

template <class S, bool HG>
hipError_t launch_fwd_radial_hg(const RadialConvArgs& a, hipStream_t s) {
  const size_t lds = radial_lds_bytes<S>();
  // the attribute is per function: raised once, retried after a failure
  static std::atomic<bool> lds_set{false};
  if (const hipError_t e = set_max_lds_once(
          lds_set, reinterpret_cast<const void*>(&k_conv_fwd_radial<S, HG>), int(lds));
      e != hipSuccess)
    return e;
  const int n_slabs = a.C / 32;
  hipLaunchKernelGGL((k_conv_fwd_radial<S, HG>), dim3(kRadXcds * 32), dim3(64 * kRadWaves), lds, s,
                     a.n_nodes, a.n_edges, a.C, n_slabs, a.order, a.rowptr, a.sender, a.vec, a.x,
                     a.W1, a.W2, a.cutoff, static_cast<const half8*>(a.hidden), a.m);
  return hipGetLastError();
}

template <class S>
hipError_t launch_fwd_radial(const RadialConvArgs& a, hipStream_t s) {
  return a.hidden ? launch_fwd_radial_hg<S, true>(a, s) : launch_fwd_radial_hg<S, false>(a, s);
}

// ------------------------------------------ fused radial convolution backward

// Backward of one edge for this lane's two channels chan and chan + 16 (as
// edge_backward, e3j E.1 Eq.16 with one scalar per path): dx gains
// w[P] B_P, dw[P] = sum_m1 x B_P is stored at dwe + P C (+16) after the
// last path, and dYl collects this lane's part of dY.
template <class S>
__device__ __forceinline__ void edge_backward_pair(const float (&Y)[Plan<S>::DY],
                                                   const float (&xv)[Plan<S>::DX][2],
                                                   const float (&wv)[Plan<S>::NP][2],
                                                   const float (&dmv)[Plan<S>::DO][2],
                                                   float (&dxa)[Plan<S>::DX][2],
                                                   float* __restrict__ dwe, int C, bool store,
                                                   float (&dYl)[Plan<S>::DY]) {
  using PL = Plan<S>;
  float t[PL::DX][2], dwv[PL::NP][2];
#pragma unroll
  for (int i = 0; i < PL::DX; ++i) t[i][0] = t[i][1] = 0.0f;
  sfor<0, PL::NP>([&](auto pi) {
    constexpr PathC P = PL::paths.p[pi];
    constexpr int n1 = 2 * P.l1 + 1;
    float B[n1][2], xw[n1][2];
#pragma unroll
    for (int a = 0; a < n1; ++a)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        B[a][k] = 0.0f;
        xw[a][k] = wv[pi][k] * xv[P.xo + a][k];
      }
    float A = 0.0f, T = 0.0f;
    sfor<0, P.rcnt>([&](auto r) {
      constexpr CgRec R = kRec[P.roff + r];
      if constexpr (group_first(P.roff, r)) {
        A = R.c * Y[P.yo + R.m2];
        T = fmaf(xw[R.m1][1], dmv[P.oo + R.M][1], xw[R.m1][0] * dmv[P.oo + R.M][0]);
      } else {
        A = fmaf(R.c, Y[P.yo + R.m2], A);
      }
      dYl[P.yo + R.m2] = fmaf(R.c, T, dYl[P.yo + R.m2]);
      if constexpr (group_last(P.roff, P.rcnt, r)) {
#pragma unroll
        for (int k = 0; k < 2; ++k) B[R.m1][k] = fmaf(A, dmv[P.oo + R.M][k], B[R.m1][k]);
      }
    });
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float s = 0.0f;
#pragma unroll
      for (int a = 0; a < n1; ++a) {
        t[P.xo + a][k] = fmaf(wv[pi][k], B[a][k], t[P.xo + a][k]);
        s = fmaf(xv[P.xo + a][k], B[a][k], s);
      }
      dwv[pi][k] = s;
    }
  });
  if (store) {  // one branch for the edge's stores
#pragma unroll
    for (int p = 0; p < PL::NP; ++p) {
      __builtin_nontemporal_store(dwv[p][0], dwe + int64_t(p) * C);
      __builtin_nontemporal_store(dwv[p][1], dwe + int64_t(p) * C + 16);
    }
  }
#pragma unroll
  for (int i = 0; i < PL::DX; ++i) {
    dxa[i][0] += t[i][0];
    dxa[i][1] += t[i][1];
  }
}

template <class S>
constexpr size_t radial_bwd_lds_bytes() {
  using PL = Plan<S>;
  return size_t(PL::NP) * 8 * 64 * sizeof(half8)                        // W2 slab, hi and lo
         + size_t(kRadWaves) * kRadChunk * (PL::DY + 1) * sizeof(float)  // harmonics
         + size_t(kRadWaves) * kRadChunk * 2 * sizeof(int);              // edge ids, receivers
}

// The convolution backward with w formed on the fly from the radial MLP's
// hidden layer (k_radial_hidden's operands), as the fused forward forms it:
// w never reaches HBM.  Sender-ordered walk over the transposed index (as
// k_conv_bwd: dx[a] sums over a's out-edges in registers, dw[e] and dY[e]
// are edge-local), one 32-channel slab per wavefront with W2's slab split
// into fp16 parts in LDS, slabs spread over the XCDs.  Per 16-edge tile of
// a sender's out-edges the MFMAs leave w for 4 edges x 2 channels in every
// lane (edges 4 (lane/16) + r, channels chan and chan + 16), so lane group
// g = lane / 16 takes edges 4g..4g+3 of the tile: it gathers their dm rows
// for its channels and runs the edge's backward.  dY of an edge is summed
// over the group's 16 lanes (a fixed reduce-scatter) and stored per slab
// (dY_part [slab][E][DY], added over the slabs afterwards); dx is summed
// over the four groups with a fixed butterfly.  Padding edges are not
// visited (zeroed afterwards).
template <class S>
__global__ void __launch_bounds__(64 * kRadWaves, 1)
    k_conv_bwd_radial(int n_nodes, int n_edges, int C, int n_slabs, const int* __restrict__ order,
                      const int* __restrict__ colptr, const int* __restrict__ perm,
                      const int* __restrict__ recv, const float* __restrict__ vec,
                      const float* __restrict__ x, const float* __restrict__ W2,
                      const half8* __restrict__ hid, const float* __restrict__ dm,
                      float* __restrict__ dx, float* __restrict__ dw,
                      float* __restrict__ dY_part) {
  using PL = Plan<S>;
  constexpr int NP = PL::NP, DX = PL::DX, DY = PL::DY, DO = PL::DO, YS = DY + 1;
  extern __shared__ __align__(16) unsigned char smem[];
  half8* s_w2 = reinterpret_cast<half8*>(smem);  // [NP][cb 2][ks 2][hi/lo 2][64 lanes]
  float* s_y = reinterpret_cast<float*>(smem + size_t(NP) * 8 * 64 * sizeof(half8));
  int* s_e = reinterpret_cast<int*>(s_y + kRadWaves * kRadChunk * YS);  // [wave][64]
  int* s_r = s_e + kRadWaves * kRadChunk;                                // [wave][64]

  const int xcd = blockIdx.x % kRadXcds, slot = blockIdx.x / kRadXcds;
  const int slab = xcd % n_slabs, part = xcd / n_slabs, n_parts = kRadXcds / n_slabs;
  const int64_t ncols = int64_t(NP) * C;
  for (int i = threadIdx.x; i < NP * 4 * 64; i += blockDim.x) {
    const int p = i / 256, cb = (i / 128) % 2, ks = (i / 64) % 2, l = i % 64;
    const int64_t col = int64_t(p) * C + slab * 32 + cb * 16 + (l & 15);
    const int k0 = ks * 32 + 8 * (l >> 4);
    half8 hi, lo;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float v = W2[int64_t(k0 + t) * ncols + col];
      hi[t] = static_cast<_Float16>(v);
      lo[t] = static_cast<_Float16>((v - static_cast<float>(hi[t])) * kLoScale);
    }
    s_w2[(i / 64) * 128 + l] = hi;
    s_w2[(i / 64) * 128 + 64 + l] = lo;
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gq = lane >> 4, li = lane & 15;
  float* ys = s_y + wave * kRadChunk * YS;
  int* se = s_e + wave * kRadChunk;
  int* sr = s_r + wave * kRadChunk;
  const int chan = slab * 32 + li;  // and chan + 16
  const int per_part = (n_nodes + n_parts - 1) / n_parts;
  const int lo_pos = part * per_part, hi_pos = min(n_nodes, lo_pos + per_part);
  const int waves_here = (gridDim.x / kRadXcds) * kRadWaves;

  for (int pos = lo_pos + slot * kRadWaves + wave; pos < hi_pos; pos += waves_here) {
    const int a = order ? order[pos] : pos;
    float xv[DX][2], dxa[DX][2];
#pragma unroll
    for (int i = 0; i < DX; ++i)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        xv[i][cb] = x[(int64_t(a) * DX + i) * C + chan + 16 * cb];
        dxa[i][cb] = 0.0f;
      }
    // clamped so that a workspace built for another graph stays in bounds
    const int beg = max(colptr[a], 0), end = min(colptr[a + 1], n_edges);
    for (int c0 = beg; c0 < end; c0 += kRadChunk) {
      // stage one out-edge per lane: edge id, receiver and harmonics
      wave_lds_fence();  // the previous chunk's reads are done
      {
        const int j = c0 + lane;
        int e = -1, b = -1;
        if (j < end) {
          e = perm[j];
          b = recv[j];
          if (e < 0 || e >= n_edges || b < 0 || b >= n_nodes) e = -1;  // only for malformed CSR
        }
        se[lane] = e;
        sr[lane] = e >= 0 ? b : a;  // an invalid row reads the sender's own dm row (not a shared one)
        float vx = 0.0f, vy = 0.0f, vz = 0.0f;
        if (e >= 0) {
          vx = vec[int64_t(e) * 3];
          vy = vec[int64_t(e) * 3 + 1];
          vz = vec[int64_t(e) * 3 + 2];
        }
        float Y[DY];
        edge_y_from_vec<S>(vx, vy, vz, Y);
#pragma unroll
        for (int i = 0; i < DY; ++i) ys[lane * YS + i] = Y[i];
      }
      wave_lds_fence();
      const int nt = (min(kRadChunk, end - c0) + 15) / 16;
      for (int t = 0; t < nt; ++t) {
        wave_lds_fence();
        // A operand: h of edge row t*16 + li (zeros for rows past the list)
        half8 ah[2], al[2];
        {
          const int er = se[t * 16 + li];
          const bool ok = er >= 0;
          const half8* hp = hid + int64_t(ok ? er : 0) * 16 + gq * 2;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const half8 vh = hp[ks * 8], vl = hp[ks * 8 + 1];
            ah[ks] = ok ? vh : half8{};
            al[ks] = ok ? vl : half8{};
          }
        }
        // w of edges t*16 + 4 gq + r, channels chan + 16 cb, for every path:
        // hi*hi in D, the two cross products (low parts scaled by 2^11) in X
        float4v wq[NP][2];
        sfor<0, NP>([&](auto pi) {
          const half8* wb = s_w2 + size_t(pi) * 512;
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            float4v D = {0.0f, 0.0f, 0.0f, 0.0f}, X = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              const half8 bh = wb[(cb * 2 + ks) * 128 + lane];
              const half8 bl = wb[(cb * 2 + ks) * 128 + 64 + lane];
              D = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[ks], bh, D, 0, 0, 0);
              X = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[ks], bl, X, 0, 0, 0);
              X = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[ks], bh, X, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) wq[pi][cb][r] = fmaf(X[r], kLoUnscale, D[r]);
          }
        });
        // one edge at a time (not unrolled: each copy of the edge's backward
        // would hold its own registers); wq rotates so that component 0 is
        // always the current edge's
#pragma unroll 1
        for (int rr = 0; rr < 4; ++rr) {
          const int jj = t * 16 + 4 * gq + rr;
          const int e = se[jj], b = sr[jj];
          const bool valid = e >= 0;
          // loaded unconditionally (an invalid row reads the sender's own
          // row) and zeroed after, so no load waits behind a branch
          float dmv[DO][2];
#pragma unroll
          for (int o = 0; o < DO; ++o)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
              const float v = dm[(int64_t(b) * DO + o) * C + chan + 16 * cb];
              dmv[o][cb] = valid ? v : 0.0f;
            }
          float Y[DY], dYl[DY];
#pragma unroll
          for (int i = 0; i < DY; ++i) {
            Y[i] = ys[jj * YS + i];
            dYl[i] = 0.0f;
          }
          float wv[NP][2];
#pragma unroll
          for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
              wv[p][cb] = wq[p][cb][0];
              wq[p][cb] = float4v{wq[p][cb][1], wq[p][cb][2], wq[p][cb][3], 0.0f};
            }
          edge_backward_pair<S>(Y, xv, wv, dmv, dxa,
                                dw + int64_t(valid ? e : 0) * NP * C + chan, C, valid, dYl);
          // this slab's part of dY[e]: the group's 16 lanes, fixed order
          Scatter<DY> sc;
          reduce_scatter<DY>(dYl, 16, lane, sc);
          if (valid && sc.first < DY)
            dY_part[(int64_t(slab) * n_edges + e) * DY + sc.first] = sc.v[0];
        }
      }
    }
    // the four lane groups hold partial sums over different edges of the
    // same channels: fixed butterfly, then group gq stores components i = gq mod 4
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int i = 0; i < DX; ++i) {
        float v = dxa[i][cb];
        v += shfl_xor_c<16>(v);
        v += shfl_xor_c<32>(v);
        dxa[i][cb] = v;
      }
    float* xb = dx + int64_t(a) * DX * C + chan;
#pragma unroll
    for (int i = 0; i < DX; ++i)
      if ((i & 3) == gq) {
        xb[int64_t(i) * C] = dxa[i][0];
        xb[int64_t(i) * C + 16] = dxa[i][1];
      }
  }
}

// dY[e] = the slabs' parts added in slab order (padding edges' rows are
// zeroed afterwards by the padding kernel).
__global__ void __launch_bounds__(256)
    k_sum_dy_slabs(int64_t n, int n_slabs, const float* __restrict__ part, float* __restrict__ dY) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float s = part[i];
  for (int q = 1; q < n_slabs; ++q) s += part[int64_t(q) * n + i];
  dY[i] = s;
}

// zero the dw and dY rows of padding edges (the walk does not visit them)
__global__ void __launch_bounds__(256)
    k_zero_padding_rows(const int* __restrict__ npad, const int* __restrict__ padlist,
                        int n_edges, int row, int dy, float* __restrict__ dw,
                        float* __restrict__ dY) {
  const int n = min(*npad, n_edges);
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    const int64_t e = padlist[i];
    if (e < 0 || e >= n_edges) continue;
    for (int k = threadIdx.x; k < row; k += blockDim.x) dw[e * row + k] = 0.0f;
    for (int k = threadIdx.x; k < dy; k += blockDim.x) dY[e * dy + k] = 0.0f;
  }
}

template <class S>
hipError_t launch_bwd_radial(const RadialBwdArgs& a, hipStream_t s) {
  using PL = Plan<S>;
  const size_t lds = radial_bwd_lds_bytes<S>();
  static std::atomic<bool> lds_set{false};
  if (const hipError_t e = set_max_lds_once(
          lds_set, reinterpret_cast<const void*>(&k_conv_bwd_radial<S>), int(lds));
      e != hipSuccess)
    return e;
  const int n_slabs = a.C / 32;
  hipLaunchKernelGGL((k_conv_bwd_radial<S>), dim3(kRadXcds * 32), dim3(64 * kRadWaves), lds, s,
                     a.n_nodes, a.n_edges, a.C, n_slabs, a.order, a.colptr, a.perm, a.recv, a.vec,
                     a.x, a.W2, static_cast<const half8*>(a.hidden), a.dm, a.dx, a.dw, a.dY_part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.n_edges <= 0) return err;
  const int64_t n = int64_t(a.n_edges) * PL::DY;
  hipLaunchKernelGGL(k_sum_dy_slabs, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, n, n_slabs,
                     a.dY_part, a.dY);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(k_zero_padding_rows, dim3(256), dim3(256), 0, s, a.npad, a.padlist,
                     a.n_edges, PL::NP * a.C, PL::DY, a.dw, a.dY);
  return hipGetLastError();
}

// ------------------------------------------------ radial MLP backward

constexpr int kTailBatch = 64;

// dh = the column slabs' partials added in slab order, into part 0:
// part[0][i] = part[0][i] + part[1][i] + ... (16 bytes per thread).
__global__ void __launch_bounds__(256)
    k_radial_sum_slabs(int64_t n4, int n_parts, int64_t stride4, float4v* __restrict__ part) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n4) return;
  float4v v[8];
  float4v acc = part[i];
  for (int q0 = 1; q0 < n_parts; q0 += 8) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q0 + q < n_parts) v[q] = __builtin_nontemporal_load(part + (q0 + q) * stride4 + i);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q0 + q < n_parts) acc += v[q];
  }
  part[i] = acc;
}

// Per edge, from dh = dw W2^T [E][64] and the basis with its derivative
// ([E][16], k_radial_basis):
// dpre = dh * silu'(pre), the radial part of
// the edge-vector gradient dvec = (sum_n B'_n(d) (dpre W1^T)_n) r / d, and
// this chunk's partial dW1[n][k] = sum_e B_n(e) dpre_k(e) (fixed order).
// One workgroup per chunk of edges, 64 edges per batch, in four phases: the
// basis and its derivative per edge (read); dpre with
// thread (k, g) taking hidden unit k of every fourth edge, so a wavefront
// reads an edge's dh row as one 256-byte access; g_n = sum_k dpre_k W1[n][k]
// with four threads per edge, two n each; dvec per edge.  Every sum keeps
// the order of a one-thread-per-edge evaluation.
__global__ void __launch_bounds__(256)
    k_radial_tail(int n_edges, int n_chunks, const float* __restrict__ vec,
                  const float* __restrict__ W1, const float* __restrict__ basis,
                  const float* __restrict__ dh, float* __restrict__ dvec,
                  float* __restrict__ dW1_part) {
  __shared__ float s_w1[kRadBasis * kRadHidden];
  __shared__ float s_b[kTailBatch][kRadBasis];
  __shared__ float s_bd[kTailBatch][kRadBasis + 1];
  __shared__ float s_g[kTailBatch][kRadBasis + 1];
  __shared__ float s_dp[kTailBatch][kRadHidden + 1];
  for (int i = threadIdx.x; i < kRadBasis * kRadHidden; i += blockDim.x) s_w1[i] = W1[i];
  __syncthreads();
  const int per = (n_edges + n_chunks - 1) / n_chunks;
  const int lo = blockIdx.x * per, hi = min(n_edges, lo + per);
  float acc0 = 0.0f, acc1 = 0.0f;  // pairs threadIdx.x and threadIdx.x + 256 of [8][64]
  const int p0 = threadIdx.x, p1 = threadIdx.x + 256;
  const int hk = threadIdx.x & 63, hg = threadIdx.x >> 6;  // phase 2: hidden unit, edge group
  const int ge = threadIdx.x >> 2, gq = threadIdx.x & 3;   // phase 3: edge, pair of n
  float w1c[kRadBasis];
#pragma unroll
  for (int n = 0; n < kRadBasis; ++n) w1c[n] = s_w1[n * kRadHidden + hk];
  for (int e0 = lo; e0 < hi; e0 += kTailBatch) {
    const int ne = min(kTailBatch, hi - e0);
    // dh of this thread's edges (unit hk of edges hg + 4j); the loads go out
    // before the basis is staged
    float g[kTailBatch / 4];
#pragma unroll
    for (int j = 0; j < kTailBatch / 4; ++j) {
      const int t = hg + 4 * j;
      g[j] = t < ne ? dh[(int64_t(e0) + t) * kRadHidden + hk] : 0.0f;
    }
    // the basis and its derivative of the batch's edges (16 floats each)
    for (int i = threadIdx.x; i < ne * 2 * kRadBasis; i += 256) {
      const int t = i >> 4, c = i & 15;
      const float v = basis[(int64_t(e0) + t) * 2 * kRadBasis + c];
      if (c < kRadBasis)
        s_b[t][c] = v;
      else
        s_bd[t][c - kRadBasis] = v;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kTailBatch / 4; ++j) {
      const int t = hg + 4 * j;
      if (t < ne) {
        float pre = 0.0f;
#pragma unroll
        for (int n = 0; n < kRadBasis; ++n) pre = fmaf(s_b[t][n], w1c[n], pre);
        const float sg = 1.0f / (1.0f + expf(-pre));
        s_dp[t][hk] = g[j] * sg * (1.0f + pre * (1.0f - sg));
      }
    }
    __syncthreads();
    if (ge < ne) {
      float g0 = 0.0f, g1 = 0.0f;
      const float* wa = s_w1 + (2 * gq) * kRadHidden;
      for (int k = 0; k < kRadHidden; ++k) {
        const float dp = s_dp[ge][k];
        g0 = fmaf(dp, wa[k], g0);
        g1 = fmaf(dp, wa[kRadHidden + k], g1);
      }
      s_g[ge][2 * gq] = g0;
      s_g[ge][2 * gq + 1] = g1;
    }
    __syncthreads();
    if (threadIdx.x < ne) {
      const int t = threadIdx.x;
      const int64_t e = e0 + t;
      float dd = 0.0f;
#pragma unroll
      for (int n = 0; n < kRadBasis; ++n) dd = fmaf(s_bd[t][n], s_g[t][n], dd);
      const float vx = vec[e * 3], vy = vec[e * 3 + 1], vz = vec[e * 3 + 2];
      const double d = sqrt(double(vx) * vx + double(vy) * vy + double(vz) * vz);
      const float inv = d > 0.0 ? float(1.0 / d) : 0.0f;
      dvec[e * 3] = dd * vx * inv;
      dvec[e * 3 + 1] = dd * vy * inv;
      dvec[e * 3 + 2] = dd * vz * inv;
    }
    {
      const int n0 = p0 / kRadHidden, k0 = p0 % kRadHidden;
      const int n1 = p1 / kRadHidden, k1 = p1 % kRadHidden;
      for (int t = 0; t < ne; ++t) {
        acc0 = fmaf(s_b[t][n0], s_dp[t][k0], acc0);
        acc1 = fmaf(s_b[t][n1], s_dp[t][k1], acc1);
      }
    }
    __syncthreads();
  }
  dW1_part[int64_t(blockIdx.x) * 512 + p0] = acc0;
  dW1_part[int64_t(blockIdx.x) * 512 + p1] = acc1;
}

// The two products of the second layer's backward, each reading dw once, on
// the bf16 matrix cores (v_mfma_f32_16x16x32_bf16).  Both operands are split
// into three bf16 parts, a = a0 + a1 + a2 with a1 the rounding error of a0
// and a2 that of a1: 24 significant bits and fp32's exponent range, so any
// cotangent is representable without scaling.  Six of the nine cross
// products are formed (a0b0, a0b1, a1b0, a0b2, a2b0, a1b1); the three left
// out and the split's own residue are each below 2^-24 of the product, the
// size of an fp32 rounding, and every product of two bf16 values is exact in
// the fp32 accumulator.  Six of these MFMAs (16 cycles each) do the work of
// sixteen v_mfma_f32_16x16x4f32 (32 cycles each), which leaves both products
// bound by their read of dw rather than by the matrix cores.
//
// Operand layout (that of the fp16 form above): A[i][k] is element k % 8 of
// lane i + 16 (k / 8), B[k][j] element k % 8 of lane j + 16 (k / 8), and
// D[i][j] register i % 4 of lane j + 16 (i / 4).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct Split3 {
  bf16x8 p[3];
};

__device__ __forceinline__ void split3(const float (&v)[8], Split3& s) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const __bf16 a = static_cast<__bf16>(v[t]);  // nearest even
    const float r = v[t] - static_cast<float>(a);  // exact
    const __bf16 b = static_cast<__bf16>(r);
    s.p[0][t] = a;
    s.p[1][t] = b;
    s.p[2][t] = static_cast<__bf16>(r - static_cast<float>(b));
  }
}

__device__ __forceinline__ u32x4 as_u4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }
__device__ __forceinline__ bf16x8 as_b8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float4v mfma_bf16(bf16x8 a, bf16x8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// the five smaller cross products, the smallest first
__device__ __forceinline__ float4v cross5(const Split3& a, const Split3& b, float4v c) {
  c = mfma_bf16(a.p[1], b.p[1], c);
  c = mfma_bf16(a.p[2], b.p[0], c);
  c = mfma_bf16(a.p[0], b.p[2], c);
  c = mfma_bf16(a.p[1], b.p[0], c);
  return mfma_bf16(a.p[0], b.p[1], c);
}

constexpr int kW2Units = 4 * 3 * 64;  // 16-byte units per 32-column block: [nt][part][lane]

// W2 [64][n_cols] in its three bf16 parts, in the B operand order of the dh
// product: unit [cb][nt][part][lane] holds W2[16 nt + lane % 16]
// [32 cb + 8 (lane / 16) + t], t = 0..7; blocks past n_cols / 32, up to a
// whole slab of the kernel below, are zeros.
constexpr int kDhwWaves = 8;
constexpr int kDhwCols = 32 * kDhwWaves;  // columns per slab: 32 per wavefront
constexpr int kDhwBlocks = kDhwCols / 32;  // 32-column blocks per slab

__host__ __device__ constexpr int w2_split_blocks(int n_cols) {
  return (n_cols / 32 + kDhwBlocks - 1) / kDhwBlocks * kDhwBlocks;
}

__global__ void __launch_bounds__(256)
    k_radial_split_w2(int n_cols, const float* __restrict__ W2, u32x4* __restrict__ w2s) {
  const int idx = blockIdx.x * 256 + threadIdx.x;  // (cb, nt, lane)
  if (idx >= w2_split_blocks(n_cols) * 256) return;
  const int lane = idx & 63, nt = (idx >> 6) & 3, cb = idx >> 8;
  float v[8];
  if (cb < n_cols / 32) {
    const float* src = W2 + int64_t(16 * nt + (lane & 15)) * n_cols + 32 * cb + 8 * (lane >> 4);
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = src[t];
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = 0.0f;
  }
  Split3 sp;
  split3(v, sp);
  u32x4* dst = w2s + int64_t(cb) * kW2Units + nt * 192 + lane;
#pragma unroll
  for (int q = 0; q < 3; ++q) dst[64 * q] = as_u4(sp.p[q]);
}

typedef float float2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// h of the backward's dW2 product.  Not the forward's correctly rounded
// SiLU: h enters only sums over thousands of edges, where its last bits do
// not show.
__device__ __forceinline__ float silu_sum_operand(float t) {
  return t * __builtin_amdgcn_rcpf(1.0f + __expf(-t));
}

// The radial basis of every edge and its derivative in d, [E][16] (B_n then
// dB_n/dd), for the backward's kernels to read instead of evaluating them in
// fp64 per column slab or batch:
//   B_n = sqrt(2/rc) sin(k_n d) / d,  dB_n/dd = sqrt(2/rc) (k_n cos(k_n d) - sin(k_n d) / d) / d
// with k_n = (n+1) pi / rc, in fp64 (sin and cos of (n+1) t by the
// angle-addition recurrence from one sincos, one division) and rounded once;
// at d = 0 the limits sqrt(2/rc) k_n and 0.
__global__ void __launch_bounds__(256)
    k_radial_basis(int n_edges, const float* __restrict__ vec, float rc, float* __restrict__ basis) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n_edges) return;
  const float vx = vec[int64_t(e) * 3], vy = vec[int64_t(e) * 3 + 1], vz = vec[int64_t(e) * 3 + 2];
  const double d = sqrt(double(vx) * vx + double(vy) * vy + double(vz) * vz);
  const double pref = sqrt(2.0 / double(rc)), k1 = 3.141592653589793 / double(rc);
  float B[2 * kRadBasis];
  if (d > 0.0) {
    double sn, cs;
    sincos(k1 * d, &sn, &cs);
    const double inv = 1.0 / d;
    double s_n = sn, c_n = cs;
#pragma unroll
    for (int n = 0; n < kRadBasis; ++n) {
      const double kn = double(n + 1) * k1;
      B[n] = float(pref * s_n * inv);
      B[kRadBasis + n] = float(pref * (kn * c_n - s_n * inv) * inv);
      const double s_next = s_n * cs + c_n * sn, c_next = c_n * cs - s_n * sn;
      s_n = s_next;
      c_n = c_next;
    }
  } else {
#pragma unroll
    for (int n = 0; n < kRadBasis; ++n) {
      B[n] = float(pref * double(n + 1) * k1);
      B[kRadBasis + n] = 0.0f;
    }
  }
  float4v* dst = reinterpret_cast<float4v*>(basis + int64_t(e) * 2 * kRadBasis);
#pragma unroll
  for (int q = 0; q < 4; ++q) dst[q] = float4v{B[4 * q], B[4 * q + 1], B[4 * q + 2], B[4 * q + 3]};
}

// LDS of the kernel below, per buffer (two of each, alternating by step):
// the step's dw in three bf16 parts [part][32 rows][256 columns] (rows of
// 528 bytes, 16-byte aligned for the dh operand reads, and each group of 8
// rows 64 bytes further on, so that the four row groups of a staging store
// fall in distinct banks), h's parts in the A
// operand order of the dW2 product, the basis of the step's edges, and the
// dh partials of the wavefronts (two halves per hidden tile).
constexpr int kDhwStep = 32;                        // edges per step
constexpr int kDhwMaxSteps = 256;                   // steps per edge range at most
constexpr int kDhwRowB = 2 * kDhwCols + 16;         // bytes per staged row of one part
constexpr int kDhwPartB = kDhwStep * kDhwRowB + kDhwStep / 8 * 64;  // one part of a step
constexpr int kDhwStageB = 3 * kDhwPartB;
constexpr int kDhwHB = 4 * 3 * 64 * 16;             // [tile][part][lane] x 16 bytes
constexpr int kDhwBasisB = kDhwStep * (kRadBasis + 1) * 4;
constexpr int kDhwRedB = 8 * 2 * 64 * 16;           // [wave][edge tile][lane] float4
constexpr int kDhwOffH = 2 * kDhwStageB;
constexpr int kDhwOffBasis = kDhwOffH + 2 * kDhwHB;
constexpr int kDhwOffRed = kDhwOffBasis + 2 * kDhwBasisB;
constexpr int kDhwLds = kDhwOffRed + 2 * kDhwRedB;  // 162,560 bytes
static_assert(kDhwLds <= 160 * 1024, "one workgroup's LDS");
static_assert(kDhwOffH % 16 == 0 && kDhwOffBasis % 16 == 0 && kDhwOffRed % 16 == 0, "alignment");

// Both products of the second layer's backward from one read of dw:
//   dh_part[slab][e][k] = sum_{j in slab} dw[e][j] W2[k][j]
//   part[range][k][j]   = sum_{e in range} h[e][k] dw[e][j]    (j in slab)
// Grid x = 256-column slabs, y = edge ranges; one 512-thread workgroup per
// CU (LDS), walking its range in steps of 32 edges.  Wavefront w loads the
// 32 x 32 block of dw at columns 32 w of the slab: lane (i, q) 8 bytes
// (columns 2i, 2i+1) of rows 8q..8q+7.  Splitting those values gives the B
// operand of its dW2 product directly (column 2i + t of MFMA t, K = the 32
// edges; A = h's parts, formed per step from the basis: thread (k, g) unit
// k of edges 4g..4g+3), and the same parts, stored once in LDS, are the A
// operand of the dh product (rows = edges, K = columns).  For dh,
// wavefront w owns hidden tile w % 4 over half w / 4 of the slab's columns,
// with W2's parts for them in registers for the whole kernel; the two
// halves go through LDS and are added in a fixed order one step later, each
// wavefront storing one edge tile of one hidden tile.
// One barrier per step: after it, step s's products run while step s+1's
// operands are formed (h, the split of dw) into the other buffers, so the
// matrix cores and the VALU work of the two steps overlap; dw is loaded
// three steps ahead of its products (two ahead of its split), the basis
// two.  The slabs' dh partials are added in a fixed order by the tail
// kernel, the ranges' dW2 partials by launch_sum_partials.  Rows past the
// range are loaded clamped and zeroed; columns past n_cols are zeros in dw
// and W2.
__global__ void __launch_bounds__(64 * kDhwWaves)
    k_radial_dhw2(int n_edges, int n_cols, const float* __restrict__ basis,
                  const float* __restrict__ W1, const float* __restrict__ dw,
                  const u32x4* __restrict__ w2s, float* __restrict__ dh_part,
                  float* __restrict__ part) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, kq = lane >> 4;
  const int sb = blockIdx.x;
  const int c2 = sb * kDhwCols + 32 * wave + 2 * li;  // this lane's 2 columns
  const bool cval = c2 < n_cols;                       // n_cols is a multiple of 32
  const int c2c = cval ? c2 : 0;
  const int kt = wave & 3, hf = wave >> 2;  // dh: hidden tile, half of the slab
  const int per = ((n_edges + int(gridDim.y) - 1) / int(gridDim.y) + kDhwStep - 1) / kDhwStep *
                  kDhwStep;
  const int lo = int(blockIdx.y) * per, hi = min(n_edges, lo + per);
  const int n_steps = lo < hi ? (hi - lo + kDhwStep - 1) / kDhwStep : 0;
  const int hk = threadIdx.x & 63, hg = threadIdx.x >> 6;  // hidden unit, group of 4 edges
  const int be = (threadIdx.x >> 3) & 31, bn = threadIdx.x & 7;  // basis value (edge, n)
  const float* __restrict__ w1c = W1 + hk;  // W1[n][hk] at w1c[n * 64] (cached; no registers held)
  Split3 W[4];  // W2's parts for the dh product: column blocks 4 hf + ks of the slab
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int cb = sb * kDhwBlocks + 4 * hf + ks;
#pragma unroll
    for (int p = 0; p < 3; ++p) W[ks].p[p] = as_b8(w2s[int64_t(cb) * kW2Units + kt * 192 + 64 * p + lane]);
  }
  // dW2 [hidden tile][t]: the leading products a0 b0 and the five smaller
  // ones in accumulators of their own.  A matrix-core accumulation drops the
  // bits of addends far below its accumulator's magnitude toward minus
  // infinity (a bias of one sign for every edge, which a sum over millions
  // of edges with cancelling signs does not hide); kept apart, each
  // accumulator's addends are within a few binades of it.
  float4v acc[4][2], axc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      acc[mt][t] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
      axc[mt][t] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    }
  auto s_p = [&](int u) { return reinterpret_cast<unsigned*>(lds + u * kDhwStageB); };
  auto s_h = [&](int u) { return reinterpret_cast<u32x2*>(lds + kDhwOffH + u * kDhwHB); };
  auto s_b = [&](int u) { return reinterpret_cast<float*>(lds + kDhwOffBasis + u * kDhwBasisB); };
  auto s_r = [&](int u) { return reinterpret_cast<float4v*>(lds + kDhwOffRed + u * kDhwRedB); };
  if (n_steps > 0) {  // the same for the whole workgroup
    // Every step issues its loads unconditionally and in the same order (the
    // steps past the range compute on zeroed rows), so each wait covers
    // exactly the loads it needs.
    float2v bq[2][8];
    float bv[2];
    int ld = 0;  // next step to load
    // Rows past the range are other ranges' (finite) rows, read but never
    // used: their h is zero and their dh is not stored; rows past the last
    // edge are clamped to it.  Columns past n_cols read columns 0 and 1
    // (finite), which meet zeros in W2 and whose dW2 is not stored.
    auto load_step = [&](float2v (&b)[8], float& v) {
      const int e0 = lo + kDhwStep * min(ld, n_steps - 1);
      ++ld;
      v = basis[int64_t(min(e0 + be, n_edges - 1)) * 2 * kRadBasis + bn];
      const float* base = dw + int64_t(e0) * n_cols;  // the same for the workgroup
      const int rlim = min(kDhwStep - 1, n_edges - 1 - e0);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const unsigned off = unsigned(min(8 * kq + s, rlim)) * unsigned(n_cols) + unsigned(c2c);
        b[s] = __builtin_nontemporal_load(reinterpret_cast<const float2v*>(base + off));
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the loads where they are issued
    };
    auto put_basis = [&](float v, float* sb_) {
      sb_[be * (kRadBasis + 1) + bn] = v;  // threads past 256 store the same values again
    };
    // h of the step's edges, split, in the A operand order of the dW2
    // product: lane hk % 16 + 16 (hg / 2) of tile hk / 16, elements 4 (hg % 2) .. +3
    auto hidden = [&](int st, const float* sb_, u32x2* sh) {
      const int e0 = lo + kDhwStep * st;
      float v8[8];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int el = 4 * hg + s;
        float pre = 0.0f;
#pragma unroll
        for (int n = 0; n < kRadBasis; ++n)
          pre = fmaf(sb_[el * (kRadBasis + 1) + n], w1c[n * kRadHidden], pre);
        v8[s] = e0 + el < hi ? silu_sum_operand(pre) : 0.0f;
        v8[4 + s] = 0.0f;
      }
      Split3 H;
      split3(v8, H);
#pragma unroll
      for (int p = 0; p < 3; ++p)
        sh[(((hk >> 4) * 3 + p) * 64 + (hk & 15) + 16 * (hg >> 1)) * 2 + (hg & 1)] =
            __builtin_bit_cast(u32x4, H.p[p]).xy;
    };
    // split the step's values (the dW2 product's B operands) and store the
    // parts; word i of a part holds rows 2i (low half) and 2i + 1 of one column
    auto stage = [&](const float2v (&b)[8], unsigned* sp, Split3 (&B)[2]) {
      float v[2][8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        v[0][s] = b[s].x;
        v[1][s] = b[s].y;
      }
      split3(v[0], B[0]);
      split3(v[1], B[1]);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const u32x4 x = as_u4(B[0].p[p]), y = as_u4(B[1].p[p]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          unsigned* row = sp + p * (kDhwPartB / 4) + (8 * kq + 2 * i) * (kDhwRowB / 4) + 16 * kq +
                          16 * wave + li;
          row[0] = __builtin_amdgcn_perm(y[i], x[i], 0x05040100u);             // low halves
          row[kDhwRowB / 4] = __builtin_amdgcn_perm(y[i], x[i], 0x07060302u);  // high halves
        }
      }
    };
    // dh of step st for hidden tile kt and edge tile hf: half 0 + half 1
    auto reduce = [&](int st, const float4v* sr) {
      const int e0 = lo + kDhwStep * st;
      const float4v k0 = sr[(kt * 2 + hf) * 64 + lane], o = sr[((kt + 4) * 2 + hf) * 64 + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = e0 + 16 * hf + 4 * kq + r;
        if (e < hi)
          dh_part[(int64_t(sb) * n_edges + e) * kRadHidden + 16 * kt + li] = k0[r] + o[r];
      }
    };
    // prologue: steps 0 and 1 loaded, their basis in LDS, step 0's operands
    // formed, step 2 loading
    Split3 B[2];
    load_step(bq[0], bv[0]);
    load_step(bq[1], bv[1]);
    put_basis(bv[0], s_b(0));
    put_basis(bv[1], s_b(1));
    __syncthreads();
    hidden(0, s_b(0), s_h(0));
    stage(bq[0], s_p(0), B);
    load_step(bq[0], bv[0]);  // step 2
    const int n_pad = (n_steps + 1) / 2 * 2;
    for (int s0 = 0; s0 < n_pad; s0 += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        // slot u holds step st + 2 (basis and dw), slot u ^ 1 step st + 1
        const int st = s0 + u;
        __syncthreads();  // step st's operands are in LDS; the halves of st - 1 too
        if (st > 0) reduce(st - 1, s_r(u ^ 1));
        // dW2: A = h's parts (hidden tile mt), B = this lane's columns
        const u32x2* sh = s_h(u);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          Split3 H;
#pragma unroll
          for (int p = 0; p < 3; ++p) {
            const u32x2 a = sh[((mt * 3 + p) * 64 + lane) * 2];
            const u32x2 b = sh[((mt * 3 + p) * 64 + lane) * 2 + 1];
            H.p[p] = as_b8(u32x4{a.x, a.y, b.x, b.y});
          }
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            acc[mt][t] = mfma_bf16(H.p[0], B[t].p[0], acc[mt][t]);
            axc[mt][t] = cross5(H, B[t], axc[mt][t]);
          }
        }
        // dh: A = the staged parts (rows = edges of tile et, K = columns), B = W2
        // (per edge tile the leading products and the smaller ones apart,
        // added at the end and stored for the reduction)
        const unsigned char* spb = reinterpret_cast<const unsigned char*>(s_p(u));
        float4v* sr = s_r(u);
#pragma unroll
        for (int et = 0; et < 2; ++et) {
          float4v dd = {0.0f, 0.0f, 0.0f, 0.0f}, de = {0.0f, 0.0f, 0.0f, 0.0f};
          const unsigned char* rowp = spb + (16 * et + li) * kDhwRowB + (2 * et + (li >> 3)) * 64;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            Split3 A;
#pragma unroll
            for (int p = 0; p < 3; ++p)
              A.p[p] = as_b8(*reinterpret_cast<const u32x4*>(
                  rowp + p * kDhwPartB + 2 * (32 * (4 * hf + ks) + 8 * kq)));
            dd = mfma_bf16(A.p[0], W[ks].p[0], dd);
            de = cross5(A, W[ks], de);
          }
          sr[(wave * 2 + et) * 64 + lane] = dd + de;
        }
        // step st + 1's operands into the other buffers, its slot reloaded
        // with step st + 3, and step st + 2's basis into LDS
        hidden(st + 1, s_b(u ^ 1), s_h(u ^ 1));
        stage(bq[u ^ 1], s_p(u ^ 1), B);
        load_step(bq[u ^ 1], bv[u ^ 1]);
        put_basis(bv[u], s_b(u));
      }
    }
    __syncthreads();
    reduce(n_pad - 1, s_r((n_pad - 1) & 1));
  }
  // D row = hidden unit 16 mt + 4 kq + r, column = c2 + t (lane li's columns)
  if (cval) {
    float* pr = part + int64_t(blockIdx.y) * kRadHidden * n_cols + c2;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float2v v = {acc[mt][0][r] + axc[mt][0][r], acc[mt][1][r] + axc[mt][1][r]};
        *reinterpret_cast<float2v*>(pr + int64_t(16 * mt + 4 * kq + r) * n_cols) = v;
      }
  }
}

}  // namespace

hipError_t launch_radial_tail(int n_edges, const float* vec, const float* W1,
                              const float* basis, float* dh, int n_parts, float* dvec,
                              float* dW1_part, float* dW1, hipStream_t s) {
  if (n_edges > 0 && n_parts > 1) {
    const int64_t n4 = int64_t(n_edges) * kRadHidden / 4;
    hipLaunchKernelGGL(k_radial_sum_slabs, dim3(unsigned((n4 + 255) / 256)), dim3(256), 0, s, n4,
                       n_parts, n4, reinterpret_cast<float4v*>(dh));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_radial_tail, dim3(kRadialTailChunks), dim3(256), 0, s, n_edges,
                     kRadialTailChunks, vec, W1, basis, dh, dvec, dW1_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return sum_partials_fixed(kRadialTailChunks, kRadBasis * kRadHidden, dW1_part, dW1, 0, s);
}

bool radial_conv_supported(const char* set_name) {
  return set_name && std::strcmp(set_name, "L1to3") == 0;
}

int radial_dw2_slabs(int n_cols) { return (n_cols + kDhwCols - 1) / kDhwCols; }

int radial_dw2_ranges(int n_edges, int n_cols) {
  // one workgroup per CU (LDS): slabs x ranges fills the 256 CUs at least
  // once, and no range is longer than kDhwMaxSteps steps (the rounding of
  // the matrix cores' long sums grows with the length of each range's)
  const int slabs = radial_dw2_slabs(n_cols);
  const int steps = std::max(1, (n_edges + kDhwStep - 1) / kDhwStep);
  const int wave = std::max(1, 256 / slabs);  // ranges of one round of workgroups
  const int by_length = (steps + kDhwMaxSteps - 1) / kDhwMaxSteps;
  return std::max(1, std::min(steps, (by_length + wave - 1) / wave * wave));
}

size_t radial_w2_split_bytes(int n_cols) {
  return size_t(w2_split_blocks(n_cols)) * kW2Units * 16;
}

hipError_t launch_radial_dh_dw2(int n_edges, int n_cols, const float* vec, float cutoff,
                                const float* W1, const float* W2, const float* dw,
                                float* dh_part, float* part, int ranges, void* w2s,
                                float* basis, hipStream_t s) {
  // the attribute is per function: raised once, retried after a failure
  static std::atomic<bool> lds_set{false};
  if (const hipError_t e =
          set_max_lds_once(lds_set, reinterpret_cast<const void*>(&k_radial_dhw2), kDhwLds);
      e != hipSuccess)
    return e;
  u32x4* w2u = static_cast<u32x4*>(w2s);
  hipLaunchKernelGGL(k_radial_split_w2, dim3(w2_split_blocks(n_cols)), dim3(256), 0, s, n_cols,
                     W2, w2u);
  if (n_edges > 0)
    hipLaunchKernelGGL(k_radial_basis, dim3(unsigned((int64_t(n_edges) + 255) / 256)), dim3(256), 0,
                       s, n_edges, vec, cutoff, basis);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // with no edges the dW2 partials are written as zeros
  hipLaunchKernelGGL(k_radial_dhw2, dim3(radial_dw2_slabs(n_cols), ranges),
                     dim3(64 * kDhwWaves), kDhwLds, s, n_edges, n_cols, basis, W1, dw, w2u,
                     dh_part, part);
  return hipGetLastError();
}

hipError_t launch_sum_partials(int n_chunks, int n, float* part, float* out, hipStream_t s) {
  return sum_partials_fixed(n_chunks, n, part, out, 0, s);
}

hipError_t launch_conv_fwd_radial(const char* set_name, const RadialConvArgs& a, hipStream_t s) {
  if (a.n_nodes <= 0) return hipSuccess;
  if (set_name && std::strcmp(set_name, "L1to3") == 0) return launch_fwd_radial<SigL1to3>(a, s);
  return hipErrorNotSupported;
}

size_t conv_bwd_radial_scratch_bytes(int n_edges, int C, int dy) {
  return size_t(C / 32) * size_t(n_edges) * size_t(dy) * sizeof(float);
}

hipError_t launch_conv_bwd_radial(const char* set_name, const RadialBwdArgs& a, hipStream_t s) {
  if (a.n_nodes <= 0) return hipSuccess;
  if (set_name && std::strcmp(set_name, "L1to3") == 0) return launch_bwd_radial<SigL1to3>(a, s);
  return hipErrorNotSupported;
}

hipError_t launch_radial_hidden(int n_edges, const float* vec, float cutoff, const float* W1,
                                void* h, hipStream_t s) {
  if (n_edges <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_radial_hidden, dim3(unsigned((int64_t(n_edges) + 63) / 64)), dim3(256), 0,
                     s, n_edges, vec, cutoff, W1, static_cast<half8*>(h));
  return hipGetLastError();
}

template <bool HG>
hipError_t launch_radial_mlp_hg(int n_edges, int n_cols, const float* vec, float cutoff,
                                const float* W1, const float* W2, const void* hidden, float* w,
                                hipStream_t s) {
  if (n_edges <= 0 || n_cols <= 0) return hipSuccess;
  const int n_slabs = (n_cols + kMlpCols - 1) / kMlpCols;
  const int ntiles = (n_edges + 15) / 16;
  int n_groups = (2048 + n_slabs - 1) / n_slabs;
  n_groups = max(1, min(n_groups, (ntiles + 3) / 4));
  // the attribute is per function: raised once, retried after a failure
  static std::atomic<bool> lds_set{false};
  if (const hipError_t e = set_max_lds_once(
          lds_set, reinterpret_cast<const void*>(&k_radial_mlp<HG>), int(mlp_lds_bytes()));
      e != hipSuccess)
    return e;
  hipLaunchKernelGGL(k_radial_mlp<HG>, dim3(n_slabs * n_groups), dim3(256), mlp_lds_bytes(), s,
                     n_edges, n_cols, n_slabs, n_groups, vec, cutoff, W1, W2,
                     static_cast<const half8*>(hidden), w);
  return hipGetLastError();
}

hipError_t launch_radial_mlp(int n_edges, int n_cols, const float* vec, float cutoff,
                             const float* W1, const float* W2, float* w, hipStream_t s,
                             const void* hidden) {
  return hidden ? launch_radial_mlp_hg<true>(n_edges, n_cols, vec, cutoff, W1, W2, hidden, w, s)
                : launch_radial_mlp_hg<false>(n_edges, n_cols, vec, cutoff, W1, W2, nullptr, w, s);
}

}  // namespace e3k
