// Device-side building blocks shared by the gfx950 kernels: compile-time
// path tables, unrolled per-path contractions, channel-vector loads/stores,
// the harmonics of an edge vector, and wavefront shuffles.
//
// Layouts (all row-major, channels innermost -- the "trailing channels"
// layout of the e3j paper, E.2.1):
//   node features   x[n][dx][C],  messages m[n][dout][C]
//   edge weights    w[e][P][C]    (P paths in canonical order)
//   harmonics       Y[e][dy]      (shared by all channels)
// A lane owns CPL consecutive channels; G = C / CPL lanes form an edge group
// and a 64-lane wavefront holds 64 / G groups.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "../generated/cg_table.inc"

namespace e3k {

// ------------------------------------------------------------ signatures

struct Ir {
  int l, p;
};

struct PathC {
  int l1, l2, L;   // degrees of the x, y and output irreps
  int xo, yo, oo;  // component offsets of those irreps
  int roff, rcnt;  // records of the real CG block in kRec
};

template <int N>
struct PathList {
  PathC p[N > 0 ? N : 1];
};

constexpr bool couples(Ir a, Ir b, Ir c) {
  const int lo = a.l > b.l ? a.l - b.l : b.l - a.l;
  return lo <= c.l && c.l <= a.l + b.l && a.p * b.p == c.p;
}

template <class S>
constexpr int count_paths() {
  int n = 0;
  for (int i = 0; i < S::NX; ++i)
    for (int j = 0; j < S::NY; ++j)
      for (int k = 0; k < S::NO; ++k) n += couples(S::X[i], S::Y[j], S::O[k]) ? 1 : 0;
  return n;
}

template <int N>
constexpr int dim_of(const Ir (&v)[N]) {
  int d = 0;
  for (int i = 0; i < N; ++i) d += 2 * v[i].l + 1;
  return d;
}

// Output mode of a signature: collapsed (paths landing on one output irrep
// are summed) unless S declares kPerPath, in which case every path keeps
// its own output block, in path order.
template <class S, class = void>
struct PerPathOf : std::false_type {};
template <class S>
struct PerPathOf<S, std::void_t<decltype(S::kPerPath)>> : std::bool_constant<S::kPerPath> {};

template <class S>
constexpr PathList<count_paths<S>()> make_paths() {
  PathList<count_paths<S>()> r{};
  int n = 0, xo = 0;
  for (int i = 0; i < S::NX; ++i) {
    int yo = 0;
    for (int j = 0; j < S::NY; ++j) {
      int oo = 0;
      for (int k = 0; k < S::NO; ++k) {
        if (couples(S::X[i], S::Y[j], S::O[k])) {
          const int l1 = S::X[i].l, l2 = S::Y[j].l, L = S::O[k].l;
          r.p[n++] = PathC{l1, l2, L, xo, yo, oo, kRecOff[l1][l2][L], kRecCnt[l1][l2][L]};
        }
        oo += 2 * S::O[k].l + 1;
      }
      yo += 2 * S::Y[j].l + 1;
    }
    xo += 2 * S::X[i].l + 1;
  }
  if (PerPathOf<S>::value) {
    int oo = 0;
    for (int i = 0; i < n; ++i) {
      r.p[i].oo = oo;
      oo += 2 * r.p[i].L + 1;
    }
  }
  return r;
}

// Occupancy hint of the convolution backward with 2^c channels per lane
// (see signatures.h); 1 when the signature gives none.
template <class S, class = void>
struct BwdWavesOf {
  static constexpr int get(int) { return 1; }
};
template <class S>
struct BwdWavesOf<S, std::void_t<decltype(S::kBwdWaves)>> {
  static constexpr int get(int c) { return S::kBwdWaves[c]; }
};

// Whether the convolution backward stages each chunk's harmonics in LDS
// (kStageY, default true) or forms them per edge in its loop.
template <class S, class = void>
struct StageYOf : std::true_type {};
template <class S>
struct StageYOf<S, std::void_t<decltype(S::kStageY)>> : std::bool_constant<S::kStageY> {};

template <class S>
constexpr int out_dim() {
  if (!PerPathOf<S>::value) return dim_of(S::O);
  int d = 0;
  const auto ps = make_paths<S>();
  for (int i = 0; i < count_paths<S>(); ++i) d += 2 * ps.p[i].L + 1;
  return d;
}

template <class S>
constexpr bool degrees_supported() {
  for (int i = 0; i < S::NX; ++i)
    if (S::X[i].l > kTabLmax) return false;
  for (int i = 0; i < S::NY; ++i)
    if (S::Y[i].l > kTabLmax) return false;
  for (int i = 0; i < S::NO; ++i)
    if (S::O[i].l > kTabLmax) return false;
  return true;
}

template <class S>
struct Plan {
  static_assert(degrees_supported<S>(), "irreps above the generated table's degree");
  static constexpr int DX = dim_of(S::X);
  static constexpr int DY = dim_of(S::Y);
  static constexpr int DO = out_dim<S>();
  static constexpr int NP = count_paths<S>();
  static constexpr PathList<NP> paths = make_paths<S>();
};

// Records of one path are sorted by (M, m1, m2); a "group" is a run of
// records with the same (M, m1), whose y-coefficients sum to one scalar.
constexpr bool same_pair(int i, int j) { return kRec[i].M == kRec[j].M && kRec[i].m1 == kRec[j].m1; }
constexpr bool group_first(int roff, int r) { return r == 0 || !same_pair(roff + r - 1, roff + r); }
constexpr bool group_last(int roff, int rcnt, int r) {
  return r == rcnt - 1 || !same_pair(roff + r, roff + r + 1);
}

constexpr int pow2_ceil_c(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// ------------------------------------------------------------- static for

template <int I>
using ic = std::integral_constant<int, I>;

template <int B, int E, class F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (B < E) {
    f(ic<B>{});
    sfor<B + 1, E>(f);
  }
}

// -------------------------------------------------------- storage types

struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Load CPL consecutive channels starting at p (p aligned to CPL elements).
template <class T, int CPL>
__device__ __forceinline__ void load_ch(const T* __restrict__ p, float (&v)[CPL]) {
  if constexpr (std::is_same_v<T, float>) {
    static_assert(CPL == 4 || CPL == 2 || CPL == 1, "fp32 channel vector");
    if constexpr (CPL == 4) {
      const float4 t = *reinterpret_cast<const float4*>(p);
      v[0] = t.x;
      v[1] = t.y;
      v[2] = t.z;
      v[3] = t.w;
    } else if constexpr (CPL == 2) {
      const float2 t = *reinterpret_cast<const float2*>(p);
      v[0] = t.x;
      v[1] = t.y;
    } else {
      v[0] = *p;
    }
  } else {
    static_assert(CPL == 1 || CPL == 2 || CPL == 4 || CPL == 8, "bf16 channel vector");
    if constexpr (CPL == 1) {
      v[0] = bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
    } else if constexpr (CPL == 2) {
      const uint32_t t = *reinterpret_cast<const uint32_t*>(p);
      v[0] = bf16_to_f32(t & 0xFFFFu);
      v[1] = bf16_to_f32(t >> 16);
    } else if constexpr (CPL == 4) {
      const uint2 t = *reinterpret_cast<const uint2*>(p);
      v[0] = bf16_to_f32(t.x & 0xFFFFu);
      v[1] = bf16_to_f32(t.x >> 16);
      v[2] = bf16_to_f32(t.y & 0xFFFFu);
      v[3] = bf16_to_f32(t.y >> 16);
    } else {
      const uint4 t = *reinterpret_cast<const uint4*>(p);
      const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
      }
    }
  }
}

template <class T, int CPL>
__device__ __forceinline__ void store_ch(T* __restrict__ p, const float (&v)[CPL]) {
  if constexpr (std::is_same_v<T, float>) {
    if constexpr (CPL == 4) {
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else if constexpr (CPL == 2) {
      *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    } else {
      *p = v[0];
    }
  } else {
    if constexpr (CPL == 1) {
      *reinterpret_cast<uint16_t*>(p) = uint16_t(f32_to_bf16_rne(v[0]));
    } else if constexpr (CPL == 2) {
      *reinterpret_cast<uint32_t*>(p) = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
    } else if constexpr (CPL == 4) {
      uint2 t;
      t.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
      t.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
      *reinterpret_cast<uint2*>(p) = t;
    } else {
      uint4 t;
      t.x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
      t.y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
      t.z = f32_to_bf16_rne(v[4]) | (f32_to_bf16_rne(v[5]) << 16);
      t.w = f32_to_bf16_rne(v[6]) | (f32_to_bf16_rne(v[7]) << 16);
      *reinterpret_cast<uint4*>(p) = t;
    }
  }
}

// Streaming variants for data touched once (edge weights in, edge and node
// outputs out): non-temporal hints keep them from evicting the gathered
// node rows from the caches.
typedef float vf4 __attribute__((ext_vector_type(4)));
typedef float vf2 __attribute__((ext_vector_type(2)));
typedef uint32_t vu2 __attribute__((ext_vector_type(2)));

template <class T, int CPL>
__device__ __forceinline__ void load_ch_stream(const T* __restrict__ p, float (&v)[CPL]) {
  if constexpr (std::is_same_v<T, float> && CPL == 4) {
    const vf4 t = __builtin_nontemporal_load(reinterpret_cast<const vf4*>(p));
    v[0] = t.x;
    v[1] = t.y;
    v[2] = t.z;
    v[3] = t.w;
  } else if constexpr (std::is_same_v<T, float> && CPL == 2) {
    const vf2 t = __builtin_nontemporal_load(reinterpret_cast<const vf2*>(p));
    v[0] = t.x;
    v[1] = t.y;
  } else if constexpr (!std::is_same_v<T, float> && CPL == 4) {
    const vu2 t = __builtin_nontemporal_load(reinterpret_cast<const vu2*>(p));
    v[0] = bf16_to_f32(t.x & 0xFFFFu);
    v[1] = bf16_to_f32(t.x >> 16);
    v[2] = bf16_to_f32(t.y & 0xFFFFu);
    v[3] = bf16_to_f32(t.y >> 16);
  } else if constexpr (!std::is_same_v<T, float> && CPL == 2) {
    const uint32_t t = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    v[0] = bf16_to_f32(t & 0xFFFFu);
    v[1] = bf16_to_f32(t >> 16);
  } else {
    load_ch<T, CPL>(p, v);
  }
}

template <class T, int CPL>
__device__ __forceinline__ void store_ch_stream(T* __restrict__ p, const float (&v)[CPL]) {
  if constexpr (std::is_same_v<T, float> && CPL == 4) {
    const vf4 t = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(t, reinterpret_cast<vf4*>(p));
  } else if constexpr (std::is_same_v<T, float> && CPL == 2) {
    const vf2 t = {v[0], v[1]};
    __builtin_nontemporal_store(t, reinterpret_cast<vf2*>(p));
  } else if constexpr (!std::is_same_v<T, float> && CPL == 4) {
    const vu2 t = {f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                   f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16)};
    __builtin_nontemporal_store(t, reinterpret_cast<vu2*>(p));
  } else if constexpr (!std::is_same_v<T, float> && CPL == 2) {
    __builtin_nontemporal_store(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                reinterpret_cast<uint32_t*>(p));
  } else {
    store_ch<T, CPL>(p, v);
  }
}

// ------------------------------------------------------------- harmonics

// Value and gradient along the three axes, for differentiating the
// harmonic polynomials below by forward-mode arithmetic (R: float or double).
template <class R>
struct DualT {
  R v, d0, d1, d2;
  __device__ DualT(R c = R(0)) : v(c), d0(R(0)), d1(R(0)), d2(R(0)) {}
  __device__ DualT(R c, R a, R b, R e) : v(c), d0(a), d1(b), d2(e) {}
};
template <class R>
__device__ __forceinline__ DualT<R> operator+(DualT<R> a, DualT<R> b) {
  return {a.v + b.v, a.d0 + b.d0, a.d1 + b.d1, a.d2 + b.d2};
}
template <class R>
__device__ __forceinline__ DualT<R> operator-(DualT<R> a, DualT<R> b) {
  return {a.v - b.v, a.d0 - b.d0, a.d1 - b.d1, a.d2 - b.d2};
}
template <class R>
__device__ __forceinline__ DualT<R> operator*(DualT<R> a, DualT<R> b) {
  return {a.v * b.v, fma(a.d0, b.v, a.v * b.d0), fma(a.d1, b.v, a.v * b.d1),
          fma(a.d2, b.v, a.v * b.d2)};
}
template <class R>
__device__ __forceinline__ DualT<R> operator*(R c, DualT<R> a) {
  return {c * a.v, c * a.d0, c * a.d1, c * a.d2};
}
using Dual3 = DualT<float>;
using Dual3d = DualT<double>;

// The real type under a scalar (the type of the polynomial coefficients).
template <class Sc>
struct RealOf {
  using type = Sc;
};
template <class R>
struct RealOf<DualT<R>> {
  using type = R;
};

// Component-normalised real harmonics of degree l (m = -l..l) of the unit
// vector (x, y, z), written into out[0..2l]; Sc is float or double, or a
// DualT of either to get the partial derivatives of each polynomial as well.
template <int L, class Sc>
__device__ __forceinline__ void harmonics_l(Sc x, Sc y, Sc z, Sc* out) {
  using R = typename RealOf<Sc>::type;
  if constexpr (L == 0) {
    out[0] = Sc(R(1));
  } else if constexpr (L == 1) {
    const R k = R(1.7320508075688772);  // sqrt(3)
    out[0] = k * y;
    out[1] = k * z;
    out[2] = k * x;
  } else if constexpr (L == 2) {
    const R k15 = R(3.872983346207417);        // sqrt(15)
    const R k5h = R(1.118033988749895);        // sqrt(5)/2
    const R k15h = R(1.9364916731037085);      // sqrt(15)/2
    const Sc xx = x * x, yy = y * y, zz = z * z;
    out[0] = k15 * (x * y);
    out[1] = k15 * (y * z);
    out[2] = k5h * (R(2) * zz - xx - yy);
    out[3] = k15 * (x * z);
    out[4] = k15h * (xx - yy);
  } else {
    static_assert(L == 3, "degree above 3");
    const R a = R(2.091650066335189);   // sqrt(35/8)
    const R b = R(10.246950765959598);  // sqrt(105)
    const R bh = R(5.123475382979799);  // sqrt(105)/2
    const R c = R(1.620185174601965);   // sqrt(21/8)
    const R d = R(1.3228756555322954);  // sqrt(7)/2
    const Sc xx = x * x, yy = y * y, zz = z * z;
    const Sc t = R(4) * zz - xx - yy;
    out[0] = a * ((R(3) * xx - yy) * y);
    out[1] = b * (x * y * z);
    out[2] = c * (y * t);
    out[3] = d * (z * (R(2) * zz - R(3) * xx - R(3) * yy));
    out[4] = c * (x * t);
    out[5] = bh * ((xx - yy) * z);
    out[6] = a * ((xx - R(3) * yy) * x);
  }
}

// r / |r| in float32 for any finite r: scaled first by the exact power of
// two of its largest component (the squared norm then lies in [1/4, 3/4],
// with no underflow or overflow), then a correctly rounded square root and
// one correctly rounded division per component.  0 stays 0.
__device__ __forceinline__ void unit_vector(float& x, float& y, float& z) {
  const float s = fmaxf(fabsf(x), fmaxf(fabsf(y), fabsf(z)));
  if (s > 0.0f) {
    int e;
    (void)frexpf(s, &e);
    x = ldexpf(x, -e);
    y = ldexpf(y, -e);
    z = ldexpf(z, -e);
    const float r = sqrtf(fmaf(x, x, fmaf(y, y, z * z)));
    x = x / r;
    y = y / r;
    z = z / r;
  }
}

template <class S>
constexpr int y_offset(int j) {
  int o = 0;
  for (int i = 0; i < j; ++i) o += 2 * S::Y[i].l + 1;
  return o;
}

// Direction of the edge vector (vx, vy, vz) in fp64: the products of fp32
// values are exact in fp64 and no fp32 input can underflow or overflow the
// squared norm, so no rescaling is needed.  The zero vector gives 0.
__device__ __forceinline__ void unit_dir_f64(float vx, float vy, float vz, double& x, double& y,
                                             double& z) {
  x = vx;
  y = vy;
  z = vz;
  const double n2 = x * x + y * y + z * z;
  const double inv = n2 > 0.0 ? 1.0 / sqrt(n2) : 0.0;
  x *= inv;
  y *= inv;
  z *= inv;
}

// Harmonics of every y irrep of S from one (unnormalised) edge vector,
// written to dst[0..DY): evaluated in fp64 on the fp64 direction and rounded
// once, so every value is the float32 nearest to the exact harmonic of the
// stored vector (up to rare ties).  In float32 throughout, the direction's
// rounding alone costs an ulp or two that the cubic harmonics triple, which
// heavy-tailed edge weights carry into the largest outputs.  The zero vector
// gives Y_0 = 1 and 0 for every l > 0.
template <class S, class Dst>
__device__ __forceinline__ void y_from_vec_f64(float vx, float vy, float vz, Dst&& dst) {
  double x, y, z;
  unit_dir_f64(vx, vy, vz, x, y, z);
  sfor<0, S::NY>([&](auto j) {
    constexpr int l = S::Y[j].l;
    constexpr int off = y_offset<S>(j);
    double h[2 * l + 1];
    harmonics_l<l>(x, y, z, h);
#pragma unroll
    for (int m = 0; m < 2 * l + 1; ++m) dst(off + m, float(h[m]));
  });
}

template <class S>
__device__ __forceinline__ void edge_y_from_vec(float vx, float vy, float vz,
                                                float (&Y)[Plan<S>::DY]) {
  y_from_vec_f64<S>(vx, vy, vz, [&](int i, float v) { Y[i] = v; });
}

// The same harmonics written straight to dst[0..DY) (an LDS row).
template <class S>
__device__ __forceinline__ void stage_y_from_vec(float vx, float vy, float vz,
                                                 float* __restrict__ dst) {
  y_from_vec_f64<S>(vx, vy, vz, [&](int i, float v) { dst[i] = v; });
}

// A staged harmonics row back from LDS (16-byte reads; DYS % 4 == 0).
template <int DY>
__device__ __forceinline__ void read_y_row(const float* __restrict__ src, float (&Y)[DY]) {
#pragma unroll
  for (int i = 0; i < DY; i += 4) {
    const float4 t = *reinterpret_cast<const float4*>(src + i);
    Y[i] = t.x;
    if (i + 1 < DY) Y[i + 1] = t.y;
    if (i + 2 < DY) Y[i + 2] = t.z;
    if (i + 3 < DY) Y[i + 3] = t.w;
  }
}

// Orders this wavefront's LDS accesses around a staging step: the compiler
// may not move LDS reads or writes across it, and the LDS queue drains.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// Given harmonics of edge or row e: Y[e][dy].
template <class S>
__device__ __forceinline__ void edge_y_given(const float* __restrict__ src, int64_t e,
                                             float (&Y)[Plan<S>::DY]) {
  constexpr int DY = Plan<S>::DY;
  const float* p = src + e * DY;
#pragma unroll
  for (int i = 0; i < DY; ++i) Y[i] = p[i];
}

// ------------------------------------------------------------ shuffles

// v from lane (lane ^ S): ds_swizzle in xor mode inside 32-lane halves,
// bpermute across the halves.
template <int S>
__device__ __forceinline__ float shfl_xor_c(float v) {
  if constexpr (S < 32)
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (S << 10) | 0x1F));
  else
    return __shfl_xor(v, 32, 64);
}

// Same with a wave-uniform runtime stride s in {1, 2, ..., 32}.
__device__ __forceinline__ float shfl_xor_rt(float v, int s) {
  switch (s) {
    case 1: return shfl_xor_c<1>(v);
    case 2: return shfl_xor_c<2>(v);
    case 4: return shfl_xor_c<4>(v);
    case 8: return shfl_xor_c<8>(v);
    case 16: return shfl_xor_c<16>(v);
    default: return shfl_xor_c<32>(v);
  }
}

// VALU cross-lane moves of gfx950 (lane layouts as documented for the ISA):
//  swap32(a, b): a's lanes 32..63 trade places with b's lanes 0..31;
//  swap16(a, b): a's odd 16-lane rows trade places with b's even rows;
//  dpp<CTRL>(v): v read through a DPP lane permutation (row_mirror 0x140,
//  row_half_mirror 0x141, quad_perm [3,2,1,0] 0x1B, quad_perm [1,0,3,2] 0xB1).
__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

__device__ __forceinline__ void swap16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum of v over the 64 lanes of a wavefront, returned in every lane:
// halves (swap32), 16-lane rows (swap16), then row mirror, half-row mirror
// and the two quad permutations.  Fixed pairing order: bitwise reproducible.
__device__ __forceinline__ float wave_sum(float v) {
  float a = v, b = v;
  swap32(a, b);
  v = a + b;
  a = v;
  b = v;
  swap16(a, b);
  v = a + b;
  v = v + dpp<0x140>(v);
  v = v + dpp<0x141>(v);
  v = v + dpp<0x1B>(v);
  return v + dpp<0xB1>(v);
}

// Sum of N values over all 64 lanes of a wavefront, scattered: on return
// v[0] of every lane with (lane & 3) == 0 holds the complete sum of value
// index `first` (the return value), for first < N.  Pairings: lane halves
// (swap32), 16-lane rows (swap16), then row mirror, half-row mirror and
// quad mirror; each halving step keeps one half of the live values, and once
// a single value is left the remaining pairings add it up.  Fixed order, so
// bitwise reproducible; no LDS traffic.
template <int N>
__device__ __forceinline__ int wave_reduce_scatter(float (&v)[pow2_ceil_c(N)], int lane) {
  constexpr int NP = pow2_ceil_c(N);
  static_assert(NP <= 16, "at most 16 values");
  int first = 0;
  sfor<0, 6>([&](auto j) {
    constexpr int L = NP >> j;  // live values before step j
    constexpr int H = L / 2;
    if constexpr (j == 0 || j == 1) {
      const bool upper = j == 0 ? lane >= 32 : (lane & 16) != 0;
      if constexpr (L >= 2) {
#pragma unroll
        for (int i = 0; i < H; ++i) {
          if constexpr (j == 0) swap32(v[i], v[i + H]); else swap16(v[i], v[i + H]);
          v[i] = v[i] + v[i + H];
        }
        first += upper ? H : 0;
      } else {
        float t = v[0];
        if constexpr (j == 0) swap32(v[0], t); else swap16(v[0], t);
        v[0] = v[0] + t;
      }
    } else {
      constexpr int CTRL = j == 2 ? 0x140 : j == 3 ? 0x141 : j == 4 ? 0x1B : 0xB1;
      constexpr int BIT = j == 2 ? 8 : j == 3 ? 4 : j == 4 ? 2 : 1;
      if constexpr (L >= 2) {
        const bool upper = (lane & BIT) != 0;
#pragma unroll
        for (int i = 0; i < H; ++i) {
          const float lo = v[i] + dpp<CTRL>(v[i]);
          const float hi = v[i + H] + dpp<CTRL>(v[i + H]);
          v[i] = upper ? hi : lo;
        }
        first += upper ? H : 0;
      } else {
        v[0] = v[0] + dpp<CTRL>(v[0]);
      }
    }
  });
  return first;
}

// Two edge groups of 32 lanes: sum acc over the two halves, scattered: the
// lower half ends with the totals of rows [0, N/2), the upper half with
// rows [N/2, N), both in acc[0 .. N/2).
template <int N, int CPL>
__device__ __forceinline__ void halves_reduce_scatter(float (&a)[N][CPL]) {
  static_assert(N % 2 == 0, "even row count");
#pragma unroll
  for (int i = 0; i < N / 2; ++i)
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      swap32(a[i][k], a[i + N / 2][k]);
      a[i][k] = a[i][k] + a[i + N / 2][k];
    }
}

// Sum over the 64/G edge groups of a wavefront (butterfly, fixed order):
// afterwards every group holds the total.
template <int N, int CPL>
__device__ __forceinline__ void reduce_groups(float (&a)[N][CPL], int G) {
  sfor<0, 6>([&](auto k) {
    constexpr int S = 1 << k;
    if (S >= G) {
#pragma unroll
      for (int i = 0; i < N; ++i)
#pragma unroll
        for (int c = 0; c < CPL; ++c) a[i][c] += shfl_xor_c<S>(a[i][c]);
    }
  });
}

constexpr int pow2_ceil(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Sum of N per-lane values over the G lanes of an edge group (G a power of
// two <= 64, groups aligned to G lanes), as a reduce-scatter: at each
// stride, from G/2 down, a lane pair splits the live values, each keeps one
// half and adds its partner's copy of that half; once one value is left,
// the remaining strides are plain butterfly adds.  On return the lane holds
// the complete sums of values first .. first+count-1 in v[0 .. count), and
// lanes that share `first` hold identical sums.  Fixed order: bitwise
// reproducible.
template <int N>
struct Scatter {
  static constexpr int NP = pow2_ceil(N);
  float v[NP];
  int first;  // index of v[0]
  int count;  // complete values held
};

template <int N>
__device__ __forceinline__ void reduce_scatter(const float (&a)[N], int G, int lane,
                                               Scatter<N>& r) {
  constexpr int NP = Scatter<N>::NP;
#pragma unroll
  for (int i = 0; i < NP; ++i) r.v[i] = i < N ? a[i] : 0.0f;
  int first = 0, live = NP;
  sfor<0, 6>([&](auto j) {
    constexpr int L = NP >> j;  // live values if every earlier step halved
    const int s = G >> (j + 1);
    if (s >= 1) {
      if constexpr (L >= 2) {
        const bool upper = (lane & s) != 0;
#pragma unroll
        for (int i = 0; i < L / 2; ++i) {
          const float keep = upper ? r.v[i + L / 2] : r.v[i];
          const float send = upper ? r.v[i] : r.v[i + L / 2];
          r.v[i] = keep + shfl_xor_rt(send, s);
        }
        first += upper ? L / 2 : 0;
        live = L / 2;
      } else {
        r.v[0] += shfl_xor_rt(r.v[0], s);
      }
    }
  });
  r.first = first;
  r.count = live;
}

// ------------------------------------------------- per-edge contractions

// Forward message of one edge added into acc (e3j E.1 Eq.13, with the edge
// scalar of each path factored out of its CG sum as in E.4):
//   acc[oo+M][k] += w[P][k] * sum_{m1,m2} c_P(M,m1,m2) Y[yo+m2] x[xo+m1][k]
// Per path the cheaper order is used: contract then weight (2L+1 products
// per channel) or weight x first (2l1+1 products per channel).
template <class S, int CPL>
__device__ __forceinline__ void edge_forward(const float (&Y)[Plan<S>::DY],
                                             const float (&xv)[Plan<S>::DX][CPL],
                                             const float (&wv)[Plan<S>::NP][CPL],
                                             float (&acc)[Plan<S>::DO][CPL]) {
  using PL = Plan<S>;
  sfor<0, PL::NP>([&](auto pi) {
    constexpr PathC P = PL::paths.p[pi];
    constexpr int n1 = 2 * P.l1 + 1, nL = 2 * P.L + 1;
    if constexpr (n1 < nL) {
      float u[n1][CPL];
#pragma unroll
      for (int a = 0; a < n1; ++a)
#pragma unroll
        for (int k = 0; k < CPL; ++k) u[a][k] = wv[pi][k] * xv[P.xo + a][k];
      float A = 0.0f;
      sfor<0, P.rcnt>([&](auto r) {
        constexpr int i = P.roff + r;
        constexpr CgRec R = kRec[i];
        if constexpr (group_first(P.roff, r))
          A = R.c * Y[P.yo + R.m2];
        else
          A = fmaf(R.c, Y[P.yo + R.m2], A);
        if constexpr (group_last(P.roff, P.rcnt, r)) {
#pragma unroll
          for (int k = 0; k < CPL; ++k) acc[P.oo + R.M][k] = fmaf(A, u[R.m1][k], acc[P.oo + R.M][k]);
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
        constexpr int i = P.roff + r;
        constexpr CgRec R = kRec[i];
        if constexpr (group_first(P.roff, r))
          A = R.c * Y[P.yo + R.m2];
        else
          A = fmaf(R.c, Y[P.yo + R.m2], A);
        if constexpr (group_last(P.roff, P.rcnt, r)) {
#pragma unroll
          for (int k = 0; k < CPL; ++k) z[R.M][k] = fmaf(A, xv[P.xo + R.m1][k], z[R.M][k]);
        }
      });
#pragma unroll
      for (int M = 0; M < nL; ++M)
#pragma unroll
        for (int k = 0; k < CPL; ++k) acc[P.oo + M][k] = fmaf(wv[pi][k], z[M][k], acc[P.oo + M][k]);
    }
  });
}

// Backward of one edge (e3j E.1 Eq.16 with one scalar per path; the scalar
// separates from the CG sum as in E.4):
//   B_P[m1][k]  = sum_{M,m2} c Y[yo+m2] dm[oo+M][k]
//   dx[xo+m1][k] += w[P][k] B_P[m1][k]
//   dw[P][k]      = sum_m1 x[xo+m1][k] B_P[m1][k]
//   dYl[yo+m2]   += sum_{M,m1} c sum_{k in lane} w[P][k] x[xo+m1][k] dm[oo+M][k]
// dYl holds this lane's partial sums over its own channels; dw[P] is stored
// to dwe + P*C as soon as the path is done.
template <class S, int CPL, class TS>
__device__ __forceinline__ void edge_backward(const float (&Y)[Plan<S>::DY],
                                              const float (&xv)[Plan<S>::DX][CPL],
                                              const float (&wv)[Plan<S>::NP][CPL],
                                              const float (&dmv)[Plan<S>::DO][CPL],
                                              float (&dxa)[Plan<S>::DX][CPL],
                                              TS* __restrict__ dwe, int C,
                                              float (&dYl)[Plan<S>::DY]) {
  using PL = Plan<S>;
  // this edge's dx contribution, summed over paths before it joins the
  // running per-sender sum (one rounding into the large sum per edge)
  float t[PL::DX][CPL];
#pragma unroll
  for (int i = 0; i < PL::DX; ++i)
#pragma unroll
    for (int k = 0; k < CPL; ++k) t[i][k] = 0.0f;
  sfor<0, PL::NP>([&](auto pi) {
    constexpr PathC P = PL::paths.p[pi];
    constexpr int n1 = 2 * P.l1 + 1;
    float B[n1][CPL], xw[n1][CPL];
#pragma unroll
    for (int a = 0; a < n1; ++a)
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        B[a][k] = 0.0f;
        xw[a][k] = wv[pi][k] * xv[P.xo + a][k];
      }
    float A = 0.0f, T = 0.0f;
    sfor<0, P.rcnt>([&](auto r) {
      constexpr int i = P.roff + r;
      constexpr CgRec R = kRec[i];
      constexpr bool first = group_first(P.roff, r);
      constexpr bool last = group_last(P.roff, P.rcnt, r);
      if constexpr (first) {
        A = R.c * Y[P.yo + R.m2];
        T = xw[R.m1][0] * dmv[P.oo + R.M][0];
#pragma unroll
        for (int k = 1; k < CPL; ++k) T = fmaf(xw[R.m1][k], dmv[P.oo + R.M][k], T);
      } else {
        A = fmaf(R.c, Y[P.yo + R.m2], A);
      }
      dYl[P.yo + R.m2] = fmaf(R.c, T, dYl[P.yo + R.m2]);
      if constexpr (last) {
#pragma unroll
        for (int k = 0; k < CPL; ++k) B[R.m1][k] = fmaf(A, dmv[P.oo + R.M][k], B[R.m1][k]);
      }
    });
    float dwp[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      float s = 0.0f;
#pragma unroll
      for (int a = 0; a < n1; ++a) {
        t[P.xo + a][k] = fmaf(wv[pi][k], B[a][k], t[P.xo + a][k]);
        s = fmaf(xv[P.xo + a][k], B[a][k], s);
      }
      dwp[k] = s;
    }
    store_ch_stream<TS, CPL>(dwe + int64_t(pi) * C, dwp);
  });
#pragma unroll
  for (int i = 0; i < PL::DX; ++i)
#pragma unroll
    for (int k = 0; k < CPL; ++k) dxa[i][k] += t[i][k];
}

}  // namespace e3k
