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
//   header  [kGenMagic, dx, dy, dout, P, n_contrib, n_rec]
//   obeg    [dout + 1]         contributions of output component o
//   contrib [n_contrib][3]     {path, first record, end record}
//   rec     [n_rec][2]         {x component | y component << 16, coefficient bits}
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
  const int64_t fixed = kGenHeader + int64_t(dout) + 1;
  if (n_contrib < 0 || n_rec < 0 || fixed + 3 * int64_t(n_contrib) + 2 * int64_t(n_rec) > n_words)
    n_contrib = n_rec = 0;
  const int* obeg = prog + kGenHeader;
  const int* contrib = obeg + dout + 1;
  const int* rec = contrib + 3 * n_contrib;
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
        const int rb = max(contrib[3 * j + 1], 0), re = min(contrib[3 * j + 2], n_rec);
        float t = 0.0f;
        for (int r = rb; r < re; ++r) {
          const int packed = rec[2 * r];
          const float cf = __int_as_float(rec[2 * r + 1]);
          const int xi = min(packed & 0xffff, dx - 1), yi = min(int(unsigned(packed) >> 16), dy - 1);
          t = fmaf(cf * ys[yi], xs[xi * 64 + lane], t);
        }
        acc = fmaf(wv[0], t, acc);
      }
      float out[1] = {acc};
      if (active) store_ch<T, 1>(z + (row * dout + o) * C + c, out);
    }
  }
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

}  // namespace e3k
