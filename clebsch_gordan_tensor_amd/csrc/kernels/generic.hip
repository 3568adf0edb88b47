// Channel-wise tensor product for any irreps signature with degrees up to 6,
// interpreted from a coefficient table instead of compiled per signature.
//
// e3j describes its tensor product as a generic bilinear coupling driven by
// a sparse COO array of coefficients (E.1 Eq.10-11, B.1) and runs it to
// degree L = 6..8 (B.1 Figs 5-6).  The specialised kernels unroll every
// record at compile time, which stops scaling near L = 4 (the unrolled code
// outgrows the instruction cache); this kernel reads the records from a
// table built on the host from the library's ladder CG (e3_generic_plan_build).
//
// Table (int32 words, built per descriptor):
//   header  [kGenMagic, dx, dy, dout, P, n_contrib, n_rec, rec_off]
//   obeg    [dout + 1]         contributions of output component o
//   contrib [n_contrib][3]     {path, first record, end record}
//   rec     [n_rec][2]         at word rec_off (32-byte aligned):
//                              {x component | y component << 16, coefficient bits}
// Every record run is padded to a multiple of 4 with zero coefficients, so
// the kernel takes records four at a time (one 32-byte scalar load, eight
// LDS reads in flight, two partial sums).
// Output-stationary: for every output component o of a row,
//   z[o][c] = sum_contributions w[P][c] sum_records c_r y[yi] x[xi][c]
// so each z element is written once and no accumulator is indexed at run
// time.  One wavefront handles one row and 64 channels: the row's x (one
// value per lane and component) and y sit in LDS; the records are
// wave-uniform and come through scalar loads.  Every index read from the
// table is clamped to its array, so a table built for another descriptor
// gives wrong numbers, never an out-of-bounds access.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "registry.h"

namespace e3k {
namespace {

constexpr int kGenWaves = 4;

// dx, dy, dout and np come from the caller's descriptor (they size the LDS
// and the arrays); the table's own counts are trusted only as far as the
// table's length (n_words) allows.
template <class T>
__global__ void __launch_bounds__(64 * kGenWaves)
    k_tp_generic(int64_t n_rows, int C, int dx, int dy, int dout, int np,
                 const int* __restrict__ prog, int64_t n_words, const T* __restrict__ x,
                 const float* __restrict__ y, const T* __restrict__ w, T* __restrict__ z) {
  int n_contrib = prog[5], n_rec = prog[6];
  const int64_t rec_off = prog[7];
  const int64_t fixed = kGenHeader + int64_t(dout) + 1;
  if (n_contrib < 0 || n_rec < 0 || rec_off < fixed + 3 * int64_t(n_contrib) || (rec_off & 7) ||
      rec_off + 2 * int64_t(n_rec) > n_words)
    n_contrib = n_rec = 0;
  const int* obeg = prog + kGenHeader;
  const int* contrib = obeg + dout + 1;
  const int4* rec4 = reinterpret_cast<const int4*>(prog + (n_rec ? rec_off : 0));
  extern __shared__ float gsm[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int stride = dx * 64 + dy;
  float* xs = gsm + wave * stride;
  float* ys = xs + dx * 64;
  const int cw = (C + 63) / 64;  // waves per row
  const int64_t total = n_rows * cw;
  for (int64_t item = int64_t(blockIdx.x) * kGenWaves + wave; item < total;
       item += int64_t(gridDim.x) * kGenWaves) {
    const int64_t row = item / cw;
    const int c = int(item % cw) * 64 + lane;
    const bool active = c < C;
    wave_lds_fence();  // the previous row's reads are done
    for (int i = 0; i < dx; ++i) {
      float v[1] = {0.0f};
      if (active) load_ch<T, 1>(x + (row * dx + i) * C + c, v);
      xs[i * 64 + lane] = v[0];
    }
    for (int i = lane; i < dy; i += 64) ys[i] = y[row * dy + i];
    wave_lds_fence();
    for (int o = 0; o < dout; ++o) {
      float acc = 0.0f;
      const int jb = max(obeg[o], 0), je = min(obeg[o + 1], n_contrib);
      for (int j = jb; j < je; ++j) {
        const int p = min(max(contrib[3 * j], 0), np - 1);
        float wv[1] = {0.0f};
        if (active) load_ch<T, 1>(w + (row * np + p) * C + c, wv);
        // runs are whole groups of 4 records: [rb, re) in units of 4
        const int gb = max(contrib[3 * j + 1], 0) >> 2, ge = min(contrib[3 * j + 2], n_rec) >> 2;
        float t0 = 0.0f, t1 = 0.0f;
#pragma unroll 2
        for (int g = gb; g < ge; ++g) {
          const int4 a = rec4[2 * g], b = rec4[2 * g + 1];  // 4 records, 32 bytes
          const int p0 = a.x, p1 = a.z, p2 = b.x, p3 = b.z;
          auto xi = [&](int pk) { return min(pk & 0xffff, dx - 1); };
          auto yi = [&](int pk) { return min(int(unsigned(pk) >> 16), dy - 1); };
          const float y0 = ys[yi(p0)], y1 = ys[yi(p1)], y2 = ys[yi(p2)], y3 = ys[yi(p3)];
          const float x0 = xs[xi(p0) * 64 + lane], x1 = xs[xi(p1) * 64 + lane];
          const float x2 = xs[xi(p2) * 64 + lane], x3 = xs[xi(p3) * 64 + lane];
          t0 = fmaf(__int_as_float(a.y) * y0, x0, t0);
          t1 = fmaf(__int_as_float(a.w) * y1, x1, t1);
          t0 = fmaf(__int_as_float(b.y) * y2, x2, t0);
          t1 = fmaf(__int_as_float(b.w) * y3, x3, t1);
        }
        acc = fmaf(wv[0], t0 + t1, acc);
      }
      float out[1] = {acc};
      if (active) store_ch<T, 1>(z + (row * dout + o) * C + c, out);
    }
  }
}

// dy[yi] = sum over channels of sum_records w[P][c] c_r x[xi][c] dz[o][c]
// (the channel-summed cotangent of y), from the forward table.  One
// wavefront per row walks the channels 64 at a time; per-lane partial sums
// sit in LDS and are added over the lanes in a fixed order at the end.
template <class T>
__global__ void __launch_bounds__(64)
    k_tp_generic_dy(int64_t n_rows, int C, int dx, int dy, int dout, int np,
                    const int* __restrict__ prog, int64_t n_words, const T* __restrict__ x,
                    const T* __restrict__ w, const T* __restrict__ dz, float* __restrict__ dyo) {
  int n_contrib = prog[5], n_rec = prog[6];
  const int64_t rec_off = prog[7];
  const int64_t fixed = kGenHeader + int64_t(dout) + 1;
  if (n_contrib < 0 || n_rec < 0 || rec_off < fixed + 3 * int64_t(n_contrib) || (rec_off & 7) ||
      rec_off + 2 * int64_t(n_rec) > n_words)
    n_contrib = n_rec = 0;
  const int* obeg = prog + kGenHeader;
  const int* contrib = obeg + dout + 1;
  const int4* rec4 = reinterpret_cast<const int4*>(prog + (n_rec ? rec_off : 0));
  extern __shared__ float dsm[];
  const int lane = threadIdx.x;
  float* xs = dsm;              // [dx][64]
  float* gs = xs + dx * 64;     // [dout][64]
  float* acc = gs + dout * 64;  // [dy][64]
  for (int64_t row = blockIdx.x; row < n_rows; row += gridDim.x) {
    wave_lds_fence();
    for (int i = 0; i < dy; ++i) acc[i * 64 + lane] = 0.0f;
    for (int c0 = 0; c0 < C; c0 += 64) {
      const int c = c0 + lane;
      const bool active = c < C;
      wave_lds_fence();
      for (int i = 0; i < dx; ++i) {
        float v[1] = {0.0f};
        if (active) load_ch<T, 1>(x + (row * dx + i) * C + c, v);
        xs[i * 64 + lane] = v[0];
      }
      for (int i = 0; i < dout; ++i) {
        float v[1] = {0.0f};
        if (active) load_ch<T, 1>(dz + (row * dout + i) * C + c, v);
        gs[i * 64 + lane] = v[0];
      }
      wave_lds_fence();
      for (int o = 0; o < dout; ++o) {
        const float g = gs[o * 64 + lane];
        const int jb = max(obeg[o], 0), je = min(obeg[o + 1], n_contrib);
        for (int j = jb; j < je; ++j) {
          const int p = min(max(contrib[3 * j], 0), np - 1);
          float wv[1] = {0.0f};
          if (active) load_ch<T, 1>(w + (row * np + p) * C + c, wv);
          const float wg = wv[0] * g;
          const int gb = max(contrib[3 * j + 1], 0) >> 2, ge = min(contrib[3 * j + 2], n_rec) >> 2;
          for (int gr = gb; gr < ge; ++gr) {
            const int4 a = rec4[2 * gr], b = rec4[2 * gr + 1];
            const int pk[4] = {a.x, a.z, b.x, b.z};
            const int cb[4] = {a.y, a.w, b.y, b.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int xi = min(pk[q] & 0xffff, dx - 1);
              const int yi = min(int(unsigned(pk[q]) >> 16), dy - 1);
              float* t = acc + yi * 64 + lane;
              *t = fmaf(__int_as_float(cb[q]) * xs[xi * 64 + lane], wg, *t);
            }
          }
        }
      }
    }
    wave_lds_fence();
    for (int i = lane; i < dy; i += 64) {
      float sum = 0.0f;
      for (int k = 0; k < 64; ++k) sum += acc[i * 64 + k];
      dyo[row * dy + i] = sum;
    }
  }
}

template <class T>
hipError_t launch_dy(const GenericTpArgs& a, const void* dz, float* dyo, hipStream_t s) {
  const size_t lds = size_t(a.dx + a.dout + a.dy) * 64 * sizeof(float);
  const int64_t blocks = std::min<int64_t>(a.n_rows, 256 * 16);
  hipLaunchKernelGGL(k_tp_generic_dy<T>, dim3(unsigned(blocks)), dim3(64), lds, s, a.n_rows, a.C,
                     a.dx, a.dy, a.dout, a.np, a.prog, a.n_words, static_cast<const T*>(a.x),
                     static_cast<const T*>(a.w), static_cast<const T*>(dz), dyo);
  return hipGetLastError();
}

template <class T>
hipError_t launch(const GenericTpArgs& a, hipStream_t s) {
  const size_t lds = size_t(kGenWaves) * (a.dx * 64 + a.dy) * sizeof(float);
  const int64_t items = a.n_rows * ((a.C + 63) / 64);
  const int64_t blocks = std::min<int64_t>((items + kGenWaves - 1) / kGenWaves, 256 * 8);
  hipLaunchKernelGGL(k_tp_generic<T>, dim3(unsigned(blocks)), dim3(64 * kGenWaves), lds, s,
                     a.n_rows, a.C, a.dx, a.dy, a.dout, a.np, a.prog, a.n_words,
                     static_cast<const T*>(a.x), a.y, static_cast<const T*>(a.w),
                     static_cast<T*>(a.z));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tp_generic(const GenericTpArgs& a, int bf16, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  return bf16 ? launch<bf16_t>(a, s) : launch<float>(a, s);
}

hipError_t launch_tp_generic_dy(const GenericTpArgs& a, const void* dz, float* dy, int bf16,
                                hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  return bf16 ? launch_dy<bf16_t>(a, dz, dy, s) : launch_dy<float>(a, dz, dy, s);
}

}  // namespace e3k
