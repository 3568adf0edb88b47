// Equivariant channel mixing within each irrep (e3j A.3 Eq.5): for a pair of
// blocks of equal degree and parity,
//   y[r][out_off + m][col] (+)= sum_k x[r][in_off + m][k] W[k][col],
// a GEMM whose rows are the (r, m) components of the block.  Dense and
// contraction-shaped, so it runs on the fp32 matrix cores: each wavefront
// computes 32-row tiles with v_mfma_f32_32x32x2_f32 against a slab of W
// held in LDS; workgroups are persistent over the row tiles so the slab is
// loaded once per workgroup.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"
#include "partial_sums.h"
#include "registry.h"

namespace e3k {
namespace {

typedef float f16v __attribute__((ext_vector_type(16)));

constexpr int kLinBlock = 256;   // 4 wavefronts
constexpr int kLinPad = 8;       // LDS row padding of the W slab (floats)

// LDS of one workgroup: a cin x (up to 128) slab of W, rows padded.
constexpr size_t linear_lds_bytes(int cin) { return size_t(cin) * (128 + kLinPad) * sizeof(float); }

// One 32-row x cw-column output tile per wavefront and iteration; the MFMA
// operand layouts (32x32x2, fp32): A[i][s] from lane s*32 + i, B[s][j] from
// lane s*32 + j, and D[i][j] in register r of lane j + 32*((i/4) % 2) for
// i = 8*(r/4) + 4*(lane/32) + r%4.  The two k slots s of one MFMA take
// k = kb + 4s + t for t = 0..3 over four MFMAs, so each lane reads four
// consecutive k of its row with one vector load.
//
// NK > 0 fixes cin = 8 NK: a lane then holds its row's whole A operand in
// registers and loads the next tile's while the matrix cores work on this
// one; NK = 0 streams A in steps of 8 k for any cin.
template <class T, int NCT, int NK>
__global__ void __launch_bounds__(kLinBlock)
    k_linear(int64_t n_rows, int din, int dout, int cin, int cout, int in_off, int out_off,
             int deg, int col0, const T* __restrict__ x, const float* __restrict__ W, int w_ld,
             int w_trans, T* __restrict__ y, int accumulate) {
  // W slab [cin][CW] with the columns of one lane adjacent: column
  // ct*32 + j sits at j*NCT + ct, so a lane reads its NCT B operands of
  // one k with one vector LDS load
  extern __shared__ float s_w[];  // [cin][NCT*32 + kLinPad]
  constexpr int CW = NCT * 32;
  constexpr int LD = CW + kLinPad;
  // Logical W[k][c] is W[k * w_ld + c] in memory, or W[c * w_ld + k] when
  // w_trans (the backward's W^T); either way read in 16-byte pieces.
  typedef float f4v __attribute__((ext_vector_type(4)));
  if (!w_trans) {
#pragma unroll 8
    for (int idx = threadIdx.x; idx < cin * (CW / 4); idx += kLinBlock) {
      const int k = idx / (CW / 4), c = 4 * (idx - k * (CW / 4));
      const f4v v = *reinterpret_cast<const f4v*>(W + int64_t(k) * w_ld + col0 + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) s_w[k * LD + ((c + e) % 32) * NCT + (c + e) / 32] = v[e];
    }
  } else {
#pragma unroll 8
    for (int idx = threadIdx.x; idx < CW * (cin / 4); idx += kLinBlock) {
      const int c = idx / (cin / 4), k = 4 * (idx - c * (cin / 4));
      const f4v v = *reinterpret_cast<const f4v*>(W + int64_t(col0 + c) * w_ld + k);
#pragma unroll
      for (int e = 0; e < 4; ++e) s_w[(k + e) * LD + (c % 32) * NCT + c / 32] = v[e];
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int i = lane & 31, s = lane >> 5;
  const int64_t n_comp = n_rows * deg;  // rows of this GEMM
  const int64_t n_tiles = (n_comp + 31) / 32;
  const int64_t waves = int64_t(gridDim.x) * (kLinBlock / 64);
  // this lane's A row of tile t (a zero row past the end)
  auto a_row = [&](int64_t t, bool& valid) {
    const int64_t q = t * 32 + i;
    valid = q < n_comp;
    const int64_t qq = valid ? q : 0;
    const int64_t r = qq / deg;
    const int m = int(qq - r * deg);
    return x + (r * din + in_off + m) * int64_t(cin) + 4 * s;
  };
  constexpr int NB = NK > 0 ? NK : 1;
  float abuf[NB][4];
  auto fetch = [&](int64_t t, float (&a)[NB][4]) {
    bool v;
    const T* xr = a_row(t, v);
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      load_ch<T, 4>(xr + 8 * kb, a[kb]);
      if (!v) a[kb][0] = a[kb][1] = a[kb][2] = a[kb][3] = 0.0f;
    }
  };
  int64_t t = int64_t(blockIdx.x) * (kLinBlock / 64) + (threadIdx.x >> 6);
  if (NK > 0 && t < n_tiles) fetch(t, abuf);
  for (; t < n_tiles; t += waves) {
    f16v acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = f16v{};
    // B operands of k = kb + 4s + u, u = 0..3
    auto load_b = [&](int kb, float (&b)[4][NCT]) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float* p = s_w + (kb + 4 * s + u) * LD + i * NCT;
        if constexpr (NCT == 4) {
          const f4v v = *reinterpret_cast<const f4v*>(p);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) b[u][ct] = v[ct];
        } else {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) b[u][ct] = p[ct];
        }
      }
    };
    auto mfma8 = [&](const float (&a)[4], const float (&b)[4][NCT]) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          acc[ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u], b[u][ct], acc[ct], 0, 0, 0);
    };
    if constexpr (NK > 0) {
      float anext[NB][4];
      if (t + waves < n_tiles) fetch(t + waves, anext);
      // B of the next 8 k is read from LDS while this 8 k is multiplied;
      // the scheduling fence keeps the compiler from hoisting more B reads
      // (which would cost registers and occupancy)
      float bc[4][NCT], bn[4][NCT];
      load_b(0, bc);
#pragma unroll
      for (int kb = 0; kb < NK; ++kb) {
        if (kb + 1 < NK) load_b(8 * (kb + 1), bn);
        mfma8(abuf[kb], bc);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) bc[u][ct] = bn[u][ct];
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int kb = 0; kb < NK; ++kb)
#pragma unroll
        for (int u = 0; u < 4; ++u) abuf[kb][u] = anext[kb][u];
    } else {
      bool v;
      const T* xr = a_row(t, v);
      for (int kb = 0; kb < cin; kb += 8) {
        float a[4], b[4][NCT];
        load_ch<T, 4>(xr + kb, a);
        if (!v) a[0] = a[1] = a[2] = a[3] = 0.0f;
        load_b(kb, b);
        mfma8(a, b);
      }
    }
    // D[i][j]: column j = lane % 32 of each 32-column tile; the tile's first
    // component (r0, m0) once, the rest by a 32-bit division of m0 + row
    const int64_t r0 = (t * 32) / deg;
    const int m0 = int(t * 32 - r0 * deg);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int row = 8 * (rr / 4) + 4 * s + (rr % 4);
      const int64_t qo = t * 32 + row;
      if (qo >= n_comp) continue;
      const unsigned mq = unsigned(m0 + row);
      const unsigned dr = mq / unsigned(deg);
      const int64_t ro = r0 + dr;
      const int mo = int(mq - dr * unsigned(deg));
      T* yr = y + (ro * dout + out_off + mo) * int64_t(cout) + col0 + i;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        float v[1] = {acc[ct][rr]};
        if (accumulate) {
          float o[1];
          load_ch<T, 1>(yr + ct * 32, o);
          v[0] += o[0];
        }
        store_ch<T, 1>(yr + ct * 32, v);
      }
    }
  }
}

// bf16 storage on the bf16 matrix cores: v_mfma_f32_32x32x16_bf16 with fp32
// accumulation, W rounded to bf16 (nearest even) once into the LDS slab.
// Operand layouts (checked on the hardware): A[i][k] from lane i + 32 (k / 8)
// element k % 8, B[k][j] from lane j + 32 (k / 8) element k % 8, D as for
// 32x32x2.  The slab is stored transposed, Wt[column][k], so a lane reads
// its eight k of one column with one 16-byte LDS load; rows padded by 8
// bf16.  A lane's eight k of an x row are one 16-byte global load.  NKB =
// cin / 16: a lane holds its row's whole A operand (NKB x 16 bytes) and
// loads the next tile's while the matrix cores work on this one.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
constexpr int kLinPadB = 8;  // bf16 padding of a slab row

template <int NCT, int NKB>
__global__ void __launch_bounds__(kLinBlock)
    k_linear_bf16(int64_t n_rows, int din, int dout, int cin, int cout, int in_off, int out_off,
                  int deg, int col0, const bf16_t* __restrict__ x, const float* __restrict__ W,
                  int w_ld, int w_trans, bf16_t* __restrict__ y, int accumulate) {
  extern __shared__ uint4 s_wt[];  // [CW][cin + kLinPadB] bf16, 16-byte units
  constexpr int CW = NCT * 32;
  constexpr int KL = 16 * NKB + kLinPadB;  // bf16 per slab row
  uint16_t* wt = reinterpret_cast<uint16_t*>(s_wt);
  for (int idx = threadIdx.x; idx < CW * 16 * NKB; idx += kLinBlock) {
    int c, k;
    if (!w_trans) {  // consecutive threads along the columns of W[k][.]
      k = idx / CW;
      c = idx - k * CW;
    } else {  // W^T: consecutive threads along k of W[c][.]
      c = idx / (16 * NKB);
      k = idx - c * (16 * NKB);
    }
    const float v = w_trans ? W[int64_t(col0 + c) * w_ld + k] : W[int64_t(k) * w_ld + col0 + c];
    wt[c * KL + k] = uint16_t(f32_to_bf16_rne(v));
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int i = lane & 31, kh = lane >> 5;
  const int64_t n_comp = n_rows * deg;
  const int64_t n_tiles = (n_comp + 31) / 32;
  const int64_t waves = int64_t(gridDim.x) * (kLinBlock / 64);
  auto fetch = [&](int64_t t, uint4 (&a)[NKB]) {
    const int64_t q = t * 32 + i;
    const bool valid = q < n_comp;
    const int64_t qq = valid ? q : 0;
    const int64_t r = qq / deg;
    const int m = int(qq - r * deg);
    const uint4* xr = reinterpret_cast<const uint4*>(x + (r * din + in_off + m) * int64_t(cin)) + kh;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) a[kb] = valid ? xr[2 * kb] : uint4{0u, 0u, 0u, 0u};
  };
  int64_t t = int64_t(blockIdx.x) * (kLinBlock / 64) + (threadIdx.x >> 6);
  uint4 abuf[NKB];
  if (t < n_tiles) fetch(t, abuf);
  for (; t < n_tiles; t += waves) {
    uint4 anext[NKB];
    if (t + waves < n_tiles) fetch(t + waves, anext);
    f16v acc[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[ct] = f16v{};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, abuf[kb]);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const uint4 bw = s_wt[((32 * ct + i) * KL + 16 * kb + 8 * kh) / 8];
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, bw), acc[ct],
                                                          0, 0, 0);
      }
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) abuf[kb] = anext[kb];
    // D[i][j]: column j = lane % 32 of each 32-column tile; the tile's first
    // component (r0, m0) once, the rest by a 32-bit division of m0 + row
    const int64_t r0 = (t * 32) / deg;
    const int m0 = int(t * 32 - r0 * deg);
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int row = 8 * (rr / 4) + 4 * kh + (rr % 4);
      const int64_t qo = t * 32 + row;
      if (qo >= n_comp) continue;
      const unsigned mq = unsigned(m0 + row);
      const unsigned dr = mq / unsigned(deg);
      const int64_t ro = r0 + dr;
      const int mo = int(mq - dr * unsigned(deg));
      bf16_t* yr = y + (ro * dout + out_off + mo) * int64_t(cout) + col0 + i;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        float v[1] = {acc[ct][rr]};
        if (accumulate) {
          float o[1];
          load_ch<bf16_t, 1>(yr + ct * 32, o);
          v[0] += o[0];
        }
        store_ch<bf16_t, 1>(yr + ct * 32, v);
      }
    }
  }
}

// Zero fill of one output block (no matching input block).
template <class T>
__global__ void __launch_bounds__(256)
    k_linear_zero(int64_t n_rows, int dout, int cout, int out_off, int deg, T* __restrict__ y) {
  const int64_t per_row = int64_t(deg) * cout;
  const int64_t n = n_rows * per_row;
  for (int64_t idx = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; idx < n;
       idx += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = idx / per_row;
    const int64_t rem = idx - r * per_row;
    y[(r * dout + out_off) * int64_t(cout) + rem] = T{};
  }
}

template <class T, int NCT, int NK>
hipError_t launch_one(const LinearBlockArgs& a, int col0, hipStream_t s) {
  const size_t lds = size_t(a.cin) * (NCT * 32 + kLinPad) * sizeof(float);
  // the attribute is per function: raised once, retried after a failure
  static std::atomic<bool> lds_set{false};
  if (const hipError_t e = set_max_lds_once(lds_set, reinterpret_cast<const void*>(&k_linear<T, NCT, NK>), int(linear_lds_bytes(256)));
      e != hipSuccess)
    return e;
  const int64_t tiles = (a.n_rows * a.deg + 31) / 32;
  // persistent: at most 2 workgroups per CU, 256 CUs
  int64_t blocks = (tiles + 3) / 4;
  if (blocks > 512) blocks = 512;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((k_linear<T, NCT, NK>), dim3(unsigned(blocks)), dim3(kLinBlock), lds, s,
                     a.n_rows, a.din, a.dout, a.cin, a.cout, a.in_off, a.out_off, a.deg, col0,
                     static_cast<const T*>(a.x), a.W, a.w_trans ? a.cin : a.cout, a.w_trans,
                     static_cast<T*>(a.y), a.accumulate);
  return hipGetLastError();
}

template <int NCT, int NKB>
hipError_t launch_bf16_one(const LinearBlockArgs& a, int col0, hipStream_t s) {
  const size_t lds = size_t(NCT * 32) * (16 * NKB + kLinPadB) * 2;
  // the attribute is per function: raised once, retried after a failure
  static std::atomic<bool> lds_set{false};
  if (const hipError_t e = set_max_lds_once(lds_set, reinterpret_cast<const void*>(&k_linear_bf16<NCT, NKB>), int(lds));
      e != hipSuccess)
    return e;
  const int64_t tiles = (a.n_rows * a.deg + 31) / 32;
  int64_t blocks = (tiles + 3) / 4;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((k_linear_bf16<NCT, NKB>), dim3(unsigned(blocks)), dim3(kLinBlock), lds, s,
                     a.n_rows, a.din, a.dout, a.cin, a.cout, a.in_off, a.out_off, a.deg, col0,
                     static_cast<const bf16_t*>(a.x), a.W, a.w_trans ? a.cin : a.cout, a.w_trans,
                     static_cast<bf16_t*>(a.y), a.accumulate);
  return hipGetLastError();
}

template <int NKB>
hipError_t launch_bf16_k(const LinearBlockArgs& a, hipStream_t s) {
  for (int col0 = 0; col0 < a.cout; col0 += 128) {
    const int cw = a.cout - col0 < 128 ? a.cout - col0 : 128;
    hipError_t e;
    switch (cw / 32) {
      case 1: e = launch_bf16_one<1, NKB>(a, col0, s); break;
      case 2: e = launch_bf16_one<2, NKB>(a, col0, s); break;
      case 3: e = launch_bf16_one<3, NKB>(a, col0, s); break;
      default: e = launch_bf16_one<4, NKB>(a, col0, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// bf16 storage with Cin in {64, 128, 256} (Cout a multiple of 32)
hipError_t launch_bf16(const LinearBlockArgs& a, hipStream_t s) {
  switch (a.cin) {
    case 64: return launch_bf16_k<4>(a, s);
    case 128: return launch_bf16_k<8>(a, s);
    default: return launch_bf16_k<16>(a, s);
  }
}

template <class T>
hipError_t launch_linear_t(const LinearBlockArgs& a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  if (a.zero) {
    const int64_t n = a.n_rows * a.deg * a.cout;
    int64_t g = (n + 255) / 256;
    if (g > (1 << 20)) g = 1 << 20;
    hipLaunchKernelGGL((k_linear_zero<T>), dim3(unsigned(g)), dim3(256), 0, s, a.n_rows, a.dout,
                       a.cout, a.out_off, a.deg, static_cast<T*>(a.y));
    return hipGetLastError();
  }
  if constexpr (std::is_same_v<T, bf16_t>) {
    if (a.cin == 64 || a.cin == 128 || a.cin == 256) return launch_bf16(a, s);
  }
  // column slabs of up to 128 channels
  for (int col0 = 0; col0 < a.cout; col0 += 128) {
    const int cw = a.cout - col0 < 128 ? a.cout - col0 : 128;
    hipError_t e;
    if (cw == 128 && a.cin == 128)
      e = launch_one<T, 4, 16>(a, col0, s);
    else if (cw == 128 && a.cin == 64)
      e = launch_one<T, 4, 8>(a, col0, s);
    else
      switch (cw / 32) {
        case 1: e = launch_one<T, 1, 0>(a, col0, s); break;
        case 2: e = launch_one<T, 2, 0>(a, col0, s); break;
        case 3: e = launch_one<T, 3, 0>(a, col0, s); break;
        default: e = launch_one<T, 4, 0>(a, col0, s); break;
      }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ------------------------------------------------------- weight gradient
// Partial dW over one chunk of the block's rows q = (r, m):
//   part[chunk][a][b] = sum_{q in chunk} x[q][a] dy[q][b],
// on the fp32 matrix cores with K = rows: wavefront w owns the 32 input
// channels [32w, 32w + 32) and all NTB 32-column tiles of the output
// channels; A[i][s] = x[q0 + s][32w + i], B[s][j] = dy[q0 + s][32 tb + j].
// Eight rows are loaded ahead of the eight being multiplied.
template <class T, int NTB>
__global__ void __launch_bounds__(kLinBlock)
    k_linear_dw(int64_t n_rows, int din, int dout, int cin, int cout, int in_off, int out_off,
                int deg, int64_t chunk, const T* __restrict__ x, const T* __restrict__ dy,
                float* __restrict__ part) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = lane & 31, s = lane >> 5;
  if (32 * w >= cin) return;  // wave-uniform; no block-wide barrier follows
  const int64_t n_comp = n_rows * deg;
  const int64_t q_beg = int64_t(blockIdx.x) * chunk;
  const int64_t q_end = q_beg + chunk < n_comp ? q_beg + chunk : n_comp;

  f16v acc[NTB];
#pragma unroll
  for (int t = 0; t < NTB; ++t) acc[t] = f16v{};
  // operands of rows q0 + 2u + s, u = 0..3
  auto fetch = [&](int64_t q0, float (&a)[4], float (&b)[4][NTB]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t q = q0 + 2 * u + s;
      const bool v = q < q_end;
      const int64_t qq = v ? q : q_beg;
      const int64_t r = qq / deg;
      const int m = int(qq - r * deg);
      float t1[1];
      load_ch<T, 1>(x + (r * din + in_off + m) * int64_t(cin) + 32 * w + i, t1);
      a[u] = v ? t1[0] : 0.0f;
      const T* dyr = dy + (r * dout + out_off + m) * int64_t(cout) + i;
#pragma unroll
      for (int t = 0; t < NTB; ++t) {
        load_ch<T, 1>(dyr + 32 * t, t1);
        b[u][t] = v ? t1[0] : 0.0f;
      }
    }
  };
  // a ring of four 8-row slots: the rows 24 ahead are requested while these
  // 8 are multiplied; the loop body covers all four slots, so every slot
  // keeps its registers (no copies that would wait on the loads).  Rows
  // past the chunk read as zero and add nothing.
  float ar[4][4], br[4][4][NTB];
#pragma unroll
  for (int sl = 0; sl < 3; ++sl) fetch(q_beg + 8 * sl, ar[sl], br[sl]);
  for (int64_t q0 = q_beg; q0 < q_end; q0 += 32) {
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      fetch(q0 + 8 * sl + 24, ar[(sl + 3) % 4], br[(sl + 3) % 4]);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int t = 0; t < NTB; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(ar[sl][u], br[sl][u][t], acc[t], 0, 0, 0);
    }
  }
  // D[i][j] -> part[chunk][32w + i'][32t + j]
  float* pc = part + int64_t(blockIdx.x) * cin * cout;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) {
    const int row = 8 * (rr / 4) + 4 * s + (rr % 4);
#pragma unroll
    for (int t = 0; t < NTB; ++t) pc[int64_t(32 * w + row) * cout + 32 * t + i] = acc[t][rr];
  }
}

template <class T, int NTB>
hipError_t launch_dw_t(const LinearDwArgs& a, int n_chunks, int64_t chunk, hipStream_t s) {
  hipLaunchKernelGGL((k_linear_dw<T, NTB>), dim3(unsigned(n_chunks)), dim3(kLinBlock), 0, s,
                     a.n_rows, a.din, a.dout, a.cin, a.cout, a.in_off, a.out_off, a.deg, chunk,
                     static_cast<const T*>(a.x), static_cast<const T*>(a.dy), a.part);
  return hipGetLastError();
}

template <class T>
hipError_t launch_dw(const LinearDwArgs& a, hipStream_t s) {
  const int64_t n_comp = a.n_rows * a.deg;
  const int64_t n_elem = int64_t(a.cin) * a.cout;
  if (n_comp <= 0) return sum_partials_fixed(0, n_elem, a.part, a.dW, a.accumulate, s);
  // chunks of a multiple of 8 rows, at most kLinDwChunks of them
  int64_t chunk = (n_comp + kLinDwChunks - 1) / kLinDwChunks;
  chunk = (chunk + 7) / 8 * 8;
  const int n_chunks = int((n_comp + chunk - 1) / chunk);
  hipError_t e;
  switch (a.cout / 32) {
    case 1: e = launch_dw_t<T, 1>(a, n_chunks, chunk, s); break;
    case 2: e = launch_dw_t<T, 2>(a, n_chunks, chunk, s); break;
    case 3: e = launch_dw_t<T, 3>(a, n_chunks, chunk, s); break;
    case 4: e = launch_dw_t<T, 4>(a, n_chunks, chunk, s); break;
    case 5: e = launch_dw_t<T, 5>(a, n_chunks, chunk, s); break;
    case 6: e = launch_dw_t<T, 6>(a, n_chunks, chunk, s); break;
    case 7: e = launch_dw_t<T, 7>(a, n_chunks, chunk, s); break;
    default: e = launch_dw_t<T, 8>(a, n_chunks, chunk, s); break;
  }
  if (e != hipSuccess) return e;
  return sum_partials_fixed(n_chunks, n_elem, a.part, a.dW, a.accumulate, s);
}

}  // namespace

hipError_t launch_linear(const LinearBlockArgs& a, int bf16, hipStream_t s) {
  return bf16 ? launch_linear_t<bf16_t>(a, s) : launch_linear_t<float>(a, s);
}

hipError_t launch_linear_dw(const LinearDwArgs& a, int bf16, hipStream_t s) {
  return bf16 ? launch_dw<bf16_t>(a, s) : launch_dw<float>(a, s);
}

}  // namespace e3k
