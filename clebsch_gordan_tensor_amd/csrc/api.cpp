// C-ABI entry points (include/e3hip.h): argument checks, signature dispatch
// and kernel launches.  No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <cmath>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "e3hip.h"
#include "host/cg_ladder.h"
#include "kernels/registry.h"

namespace {

thread_local std::string g_last_error;

e3_status fail(e3_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

e3_status ok() {
  g_last_error.clear();
  return E3_OK;
}

constexpr int kGenericLmax = 8;  // coefficient tables of the generic tensor product
constexpr int kTableHarmonicsLmax = 6;  // harmonics the coefficient-table kernels compute

e3_status check_graph_host(int32_t n_nodes, int32_t n_edges, const int32_t* rp,
                           const int32_t* sn);

// Host-side check of a receiver-sorted CSR graph (E3_CHECK): rowptr[0] = 0,
// rowptr non-decreasing, rowptr[N] = E, every sender in [-1, N) (-1 the
// padding mark).  The arrays are copied back on `stream` after the work
// already queued there, so the call synchronises that stream.
e3_status check_graph(int32_t n_nodes, int32_t n_edges, const int32_t* rowptr,
                      const int32_t* sender, hipStream_t stream) {
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  if (!rowptr || (n_edges > 0 && !sender)) return fail(E3_ERR_INVALID_ARG, "null pointer");
  std::vector<int32_t> rp(static_cast<size_t>(n_nodes) + 1), sn(static_cast<size_t>(n_edges));
  hipError_t e = hipMemcpyAsync(rp.data(), rowptr, rp.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess && n_edges > 0)
    e = hipMemcpyAsync(sn.data(), sender, sn.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess)
    return fail(E3_ERR_HIP, std::string("graph check copy: ") + hipGetErrorString(e));
  return check_graph_host(n_nodes, n_edges, rp.data(), sn.data());
}

e3_status check_graph_host(int32_t n_nodes, int32_t n_edges, const int32_t* rp,
                           const int32_t* sn) {
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  if (!rp || (n_edges > 0 && !sn)) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (rp[0] != 0) return fail(E3_ERR_GRAPH, "rowptr[0] = " + std::to_string(rp[0]) + ", not 0");
  for (int32_t b = 0; b < n_nodes; ++b)
    if (rp[b + 1] < rp[b])
      return fail(E3_ERR_GRAPH, "rowptr decreases at node " + std::to_string(b) + " (" +
                                    std::to_string(rp[b]) + " -> " + std::to_string(rp[b + 1]) +
                                    ")");
  if (rp[n_nodes] != n_edges)
    return fail(E3_ERR_GRAPH, "rowptr[N] = " + std::to_string(rp[n_nodes]) + ", E = " +
                                  std::to_string(n_edges));
  for (int32_t i = 0; i < n_edges; ++i)
    if (sn[i] < -1 || sn[i] >= n_nodes)
      return fail(E3_ERR_GRAPH, "sender[" + std::to_string(i) + "] = " + std::to_string(sn[i]) +
                                    " is outside [-1, N)");
  return E3_OK;
}

// E3_CHECK on a descriptor: the graph check before any launch.
e3_status maybe_check(const e3_desc* d, int32_t n_nodes, int32_t n_edges, const int32_t* rowptr,
                      const int32_t* sender, void* stream) {
  if (!d || !(d->flags & E3_CHECK)) return E3_OK;
  return check_graph(n_nodes, n_edges, rowptr, sender, hipStream_t(stream));
}

struct Parsed {
  int C = 0;
  int per_path = 0;  // E3_OUT_PER_PATH
  std::vector<e3k::IrSpec> x, y, o;
  int P = 0, dx = 0, dy = 0, dout = 0;
  std::vector<int> pix, piy, pio;
};

e3_status parse_list(const e3_irreps& in, const char* what, std::vector<e3k::IrSpec>& out,
                     std::vector<int>& muls) {
  if (in.n < 0 || (in.n > 0 && in.v == nullptr))
    return fail(E3_ERR_IRREPS, std::string(what) + ": bad irreps list");
  out.clear();
  for (int i = 0; i < in.n; ++i) {
    const e3_irrep& r = in.v[i];
    if (r.l < 0 || r.l > 64 || (r.parity != 1 && r.parity != -1) || r.mul <= 0)
      return fail(E3_ERR_IRREPS, std::string(what) + ": block " + std::to_string(i) +
                                     " needs mul > 0, l >= 0, parity +1 or -1");
    out.push_back({r.l, r.parity});
    muls.push_back(r.mul);
  }
  return E3_OK;
}

e3_status parse(const e3_desc* d, Parsed& p) {
  if (!d) return fail(E3_ERR_INVALID_ARG, "desc is null");
  std::vector<int> mx, my, mo;
  e3_status s;
  if ((s = parse_list(d->x, "x", p.x, mx)) != E3_OK) return s;
  if ((s = parse_list(d->y, "y", p.y, my)) != E3_OK) return s;
  if ((s = parse_list(d->out, "out", p.o, mo)) != E3_OK) return s;
  if (p.x.empty() || p.y.empty() || p.o.empty())
    return fail(E3_ERR_IRREPS, "x, y and out need at least one block each");
  p.C = mx[0];
  for (int m : mx)
    if (m != p.C) return fail(E3_ERR_IRREPS, "x blocks need one multiplicity (channel-wise)");
  for (int m : mo)
    if (m != p.C) return fail(E3_ERR_IRREPS, "out blocks need the multiplicity of x");
  for (int m : my)
    if (m != 1) return fail(E3_ERR_IRREPS, "y blocks need multiplicity 1");
  p.dx = p.dy = p.dout = 0;
  for (auto& r : p.x) p.dx += 2 * r.l + 1;
  for (auto& r : p.y) p.dy += 2 * r.l + 1;
  for (auto& r : p.o) p.dout += 2 * r.l + 1;
  p.pix.clear();
  p.piy.clear();
  p.pio.clear();
  for (size_t i = 0; i < p.x.size(); ++i)
    for (size_t j = 0; j < p.y.size(); ++j)
      for (size_t k = 0; k < p.o.size(); ++k) {
        const int l1 = p.x[i].l, l2 = p.y[j].l, L = p.o[k].l;
        const int lo = l1 > l2 ? l1 - l2 : l2 - l1;
        if (lo <= L && L <= l1 + l2 && p.x[i].p * p.y[j].p == p.o[k].p) {
          p.pix.push_back(int(i));
          p.piy.push_back(int(j));
          p.pio.push_back(int(k));
        }
      }
  p.P = int(p.pix.size());
  p.per_path = (d->flags & E3_OUT_PER_PATH) ? 1 : 0;
  if (p.per_path) {  // one output block per path
    p.dout = 0;
    for (int k : p.pio) p.dout += 2 * p.o[k].l + 1;
  }
  return E3_OK;
}

const e3k::KernelSet* const kSets[] = {&e3k::kSetL1,       &e3k::kSetL1to3,   &e3k::kSetL2to3,
                                       &e3k::kSetL3to3,     &e3k::kSetL1to3All, &e3k::kSetL1PP,
                                       &e3k::kSetL1to3PP,   &e3k::kSetL2to3PP};

bool same(const std::vector<e3k::IrSpec>& a, const e3k::IrSpec* b, int nb) {
  if (int(a.size()) != nb) return false;
  for (int i = 0; i < nb; ++i)
    if (a[i].l != b[i].l || a[i].p != b[i].p) return false;
  return true;
}

const e3k::KernelSet* find_set(const Parsed& p) {
  for (const e3k::KernelSet* k : kSets)
    if (k->per_path == p.per_path && same(p.x, k->x, k->nx) && same(p.y, k->y, k->ny) &&
        same(p.o, k->o, k->no))
      return k;
  return nullptr;
}

// Lanes per edge group for cpl channels per lane: G = C / cpl must be a
// power of two in [1, 64].
int group_lanes(int C, int cpl) {
  if (C <= 0 || C % cpl) return -1;
  const int G = C / cpl;
  if (G > 64 || (G & (G - 1))) return -1;
  return G;
}

enum class Kind { fwd, bwd, tp, tpb };

// Per-lane register estimate (fp32 words) of a kernel holding cpl channels
// per lane: feature, weight and accumulator vectors scale with cpl, the
// harmonics and the per-edge coefficient temporaries do not.
int register_estimate(const e3k::KernelSet& k, Kind kind, int cpl) {
  if (kind == Kind::bwd) return (3 * k.dx + k.np + k.dout) * cpl + 2 * k.dy + 48;
  if (kind == Kind::tpb) return (2 * k.dx + k.np + k.dout) * cpl + 2 * k.dy + 48;
  return (k.dx + k.np + k.dout) * cpl + k.dy + 40;
}

// Channels per lane: the largest of 4, 2, 1 whose register estimate keeps
// several wavefronts per SIMD (176 words), with G = C / cpl lanes per edge
// group a power of two <= 64; the backward passes try 2 first.  When no
// choice fits the estimate, the smallest valid one.  E3HIP_FWD_CPL,
// E3HIP_BWD_CPL and E3HIP_TP_CPL (1, 2 or 4) force a choice when it is
// valid, for tuning.
int choose_cpl(const e3k::KernelSet& k, Kind kind, int C) {
  static const int force_fwd = [] {
    const char* e = std::getenv("E3HIP_FWD_CPL");
    return e ? std::atoi(e) : 0;
  }();
  static const int force_bwd = [] {
    const char* e = std::getenv("E3HIP_BWD_CPL");
    return e ? std::atoi(e) : 0;
  }();
  static const int force_tp = [] {
    const char* e = std::getenv("E3HIP_TP_CPL");
    return e ? std::atoi(e) : 0;
  }();
  const int force = kind == Kind::fwd ? force_fwd : kind == Kind::tp ? force_tp : force_bwd;
  if ((force == 1 || force == 2 || force == 4) && group_lanes(C, force) > 0) return force;
  // the backward of the small signatures is best at two channels per lane
  // (one edge per wavefront at C = 128): prefer 2 there over 4
  const int first = kind == Kind::fwd || kind == Kind::tp ? 4 : 2;
  for (int cpl : {first, first == 4 ? 2 : 1, 1}) {
    if (group_lanes(C, cpl) <= 0) continue;
    if (register_estimate(k, kind, cpl) <= 176) return cpl;
  }
  for (int cpl : {1, 2, 4})
    if (group_lanes(C, cpl) > 0) return cpl;
  return -1;
}

e3_status select(const Parsed& p, e3_dtype dt, Kind kind, const e3k::KernelSet*& ks, int& G,
                 int& cpl_idx) {
  if (dt != E3_F32 && dt != E3_BF16) return fail(E3_ERR_INVALID_ARG, "unknown dtype");
  ks = find_set(p);
  if (!ks)
    return fail(E3_ERR_UNSUPPORTED,
                "no kernel for this irreps signature (supported: x in {0e+1o, 0e+1o+2e, "
                "0e+1o+2e+3o}, y = harmonics 0e+1o[+2e+3o], out = 0e+1o[+2e+3o])");
  const int cpl = choose_cpl(*ks, kind, p.C);
  if (cpl > 0) {
    G = group_lanes(p.C, cpl);
    cpl_idx = cpl == 1 ? 0 : cpl == 2 ? 1 : 2;
    return E3_OK;
  }
  return fail(E3_ERR_UNSUPPORTED,
              "channel count must be a power of two, 1 <= C <= 256, got " +
                  std::to_string(p.C));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

e3_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(E3_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

e3_status e3_num_paths(const e3_desc* desc, int32_t* n_paths) {
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  if (!n_paths) return fail(E3_ERR_INVALID_ARG, "n_paths is null");
  *n_paths = p.P;
  return ok();
}

e3_status e3_path_info(const e3_desc* desc, int32_t i, int32_t* ix, int32_t* iy, int32_t* iout) {
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  if (!ix || !iy || !iout) return fail(E3_ERR_INVALID_ARG, "null output pointer");
  if (i < 0 || i >= p.P) return fail(E3_ERR_INVALID_ARG, "path index out of range");
  *ix = p.pix[i];
  *iy = p.piy[i];
  *iout = p.pio[i];
  return ok();
}

int32_t e3_supported(const e3_desc* desc, e3_dtype dtype) {
  Parsed p;
  if (parse(desc, p) != E3_OK) return 0;
  const e3k::KernelSet* ks;
  int G, ci;
  return (select(p, dtype, Kind::fwd, ks, G, ci) == E3_OK &&
          select(p, dtype, Kind::bwd, ks, G, ci) == E3_OK)
             ? 1
             : 0;
}

e3_status e3_cg_block(int32_t l1, int32_t l2, int32_t L, double* out) {
  if (!out) return fail(E3_ERR_INVALID_ARG, "out is null");
  if (l1 < 0 || l2 < 0 || L < 0 || l1 > kGenericLmax || l2 > kGenericLmax || L > kGenericLmax)
    return fail(E3_ERR_INVALID_ARG, "degrees must be in 0..8");
  std::vector<double> T;
  if (!e3::cg_real_block(l1, l2, L, T)) return fail(E3_ERR_INVALID_ARG, "triple does not couple");
  for (size_t k = 0; k < T.size(); ++k) out[k] = T[k];
  return ok();
}

e3_status e3_spherical_harmonics(int32_t lmax, int64_t n, const float* vec, float* Y,
                                 void* stream) {
  if (lmax < 0 || lmax > 8) return fail(E3_ERR_INVALID_ARG, "lmax must be in 0..8");
  if (n < 0) return fail(E3_ERR_INVALID_ARG, "n < 0");
  if (n == 0) return ok();
  if (!vec || !Y) return fail(E3_ERR_INVALID_ARG, "null pointer");
  return hip_status(e3k::launch_harmonics(lmax, n, vec, Y, hipStream_t(stream)), "harmonics");
}

e3_status e3_tp_forward(const e3_desc* desc, int64_t n_rows, const void* x, const float* y,
                        const void* w, void* z, e3_dtype dtype, void* stream) {
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  const e3k::KernelSet* ks;
  int G, ci;
  if ((s = select(p, dtype, Kind::tp, ks, G, ci)) != E3_OK) return s;
  if (n_rows < 0) return fail(E3_ERR_INVALID_ARG, "n_rows < 0");
  if (n_rows == 0) return ok();
  if (!x || !y || !w || !z) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(x) || !aligned16(w) || !aligned16(z))
    return fail(E3_ERR_ALIGNMENT, "x, w and z must be 16-byte aligned");
  e3k::TpArgs a{n_rows, p.C, G, x, y, w, z};
  return hip_status(ks->tp[dtype][ci](a, hipStream_t(stream)), "tp_forward");
}

e3_status e3_tp_backward(const e3_desc* desc, int64_t n_rows, const void* x, const float* y,
                         const void* w, const void* dz, void* dx, void* dw, float* dy,
                         e3_dtype dtype, void* stream) {
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  const e3k::KernelSet* ks;
  int G, ci;
  if ((s = select(p, dtype, Kind::tpb, ks, G, ci)) != E3_OK) return s;
  if (n_rows < 0) return fail(E3_ERR_INVALID_ARG, "n_rows < 0");
  if (n_rows > INT32_MAX) return fail(E3_ERR_UNSUPPORTED, "more than 2^31 - 1 rows");
  if (n_rows == 0) return ok();
  if (!x || !y || !w || !dz || !dx || !dw || !dy) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(x) || !aligned16(w) || !aligned16(dz) || !aligned16(dx) || !aligned16(dw))
    return fail(E3_ERR_ALIGNMENT, "x, w, dz, dx and dw must be 16-byte aligned");
  e3k::TpBwdArgs a{n_rows, p.C, G, x, y, w, dz, dx, dw, dy};
  return hip_status(ks->tpb[dtype][ci](a, hipStream_t(stream)), "tp_backward");
}

e3_status e3_spherical_harmonics_backward(int32_t lmax, int64_t n, const float* vec,
                                          const float* dY, float* dvec, void* stream) {
  if (lmax < 0 || lmax > 8) return fail(E3_ERR_INVALID_ARG, "lmax must be in 0..8");
  if (n < 0) return fail(E3_ERR_INVALID_ARG, "n < 0");
  if (n == 0) return ok();
  if (!vec || !dY || !dvec) return fail(E3_ERR_INVALID_ARG, "null pointer");
  return hip_status(e3k::launch_harmonics_grad(lmax, n, vec, dY, dvec, hipStream_t(stream)),
                    "harmonics_backward");
}

e3_status e3_edge_grad_to_nodes(int32_t n_nodes, int32_t n_edges, const int32_t* rowptr,
                                const int32_t* sender, const void* workspace, size_t ws_bytes,
                                const float* edge_grad, float* node_grad, void* stream) {
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  if (n_nodes == 0) return ok();
  size_t need = 0;
  e3_conv_workspace_size(n_nodes, n_edges, &need);
  if (!workspace || ws_bytes < need)
    return fail(E3_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
  if (!rowptr || !node_grad || (n_edges > 0 && (!sender || !edge_grad)))
    return fail(E3_ERR_INVALID_ARG, "null pointer");
  return hip_status(e3k::launch_edge_grad_to_nodes(n_nodes, n_edges, rowptr, sender,
                                                   static_cast<const int*>(workspace), edge_grad,
                                                   node_grad, hipStream_t(stream)),
                    "edge_grad_to_nodes");
}

e3_status e3_conv_forward(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                          const int32_t* rowptr, const int32_t* sender, const void* workspace,
                          size_t ws_bytes, const float* edge_vec_or_Y, const void* x,
                          const void* w, void* m, e3_dtype dtype, void* stream) {
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  const e3k::KernelSet* ks;
  int G, ci;
  if ((s = select(p, dtype, Kind::fwd, ks, G, ci)) != E3_OK) return s;
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  if (n_nodes == 0) return ok();
  if ((s = maybe_check(desc, n_nodes, n_edges, rowptr, sender, stream)) != E3_OK) return s;
  if (!rowptr || !m || !x) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (n_edges > 0 && (!sender || !edge_vec_or_Y || !w))
    return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(x) || !aligned16(m) || (n_edges > 0 && !aligned16(w)))
    return fail(E3_ERR_ALIGNMENT, "x, w and m must be 16-byte aligned");
  const int* order = nullptr;
  if (workspace) {
    size_t need = 0;
    e3_conv_workspace_size(n_nodes, n_edges, &need);
    if (ws_bytes < need)
      return fail(E3_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
    order = static_cast<const int*>(workspace) + e3k::transpose_layout(n_nodes, n_edges).order;
  }
  const bool yg = (desc->flags & E3_Y_GIVEN) != 0;
  e3k::FwdArgs a{n_nodes, n_edges, p.C, G, order, rowptr, sender, edge_vec_or_Y, x, w, m};
  return hip_status(ks->fwd[dtype][yg][ci](a, hipStream_t(stream)), "conv_forward");
}

e3_status e3_conv_workspace_size(int32_t n_nodes, int32_t n_edges, size_t* bytes) {
  if (!bytes) return fail(E3_ERR_INVALID_ARG, "bytes is null");
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  *bytes = size_t(e3k::transpose_layout(n_nodes, n_edges).total_words) * sizeof(int32_t);
  return ok();
}

e3_status e3_conv_prepare_transpose(int32_t n_nodes, int32_t n_edges, const int32_t* rowptr,
                                    const int32_t* sender, const float* edge_vec, void* workspace,
                                    size_t ws_bytes, void* stream) {
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  size_t need = 0;
  e3_conv_workspace_size(n_nodes, n_edges, &need);
  if (!workspace || ws_bytes < need)
    return fail(E3_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
  if (!aligned16(workspace)) return fail(E3_ERR_ALIGNMENT, "workspace must be 16-byte aligned");
  if (n_nodes > 0 && !rowptr) return fail(E3_ERR_INVALID_ARG, "rowptr is null");
  if (n_edges > 0 && !sender) return fail(E3_ERR_INVALID_ARG, "sender is null");
  return hip_status(e3k::launch_prepare_transpose(n_nodes, n_edges, rowptr, sender,
                                                  n_edges > 0 ? edge_vec : nullptr,
                                                  static_cast<int*>(workspace), hipStream_t(stream)),
                    "prepare_transpose");
}

e3_status e3_conv_backward(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                           const int32_t* rowptr, const int32_t* sender, const void* workspace,
                           size_t ws_bytes, const float* edge_vec_or_Y, const void* x,
                           const void* w, const void* dm, void* dx, void* dw, float* dY,
                           e3_dtype dtype, void* stream) {
  (void)rowptr;
  (void)sender;
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  const e3k::KernelSet* ks;
  int G, ci;
  if ((s = select(p, dtype, Kind::bwd, ks, G, ci)) != E3_OK) return s;
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  if (n_nodes == 0) return ok();
  if ((s = maybe_check(desc, n_nodes, n_edges, rowptr, sender, stream)) != E3_OK) return s;
  size_t need = 0;
  e3_conv_workspace_size(n_nodes, n_edges, &need);
  if (!workspace || ws_bytes < need)
    return fail(E3_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
  if (!x || !dx || !dm) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (n_edges > 0 && (!edge_vec_or_Y || !w || !dw || !dY))
    return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(x) || !aligned16(dm) || !aligned16(dx) ||
      (n_edges > 0 && (!aligned16(w) || !aligned16(dw))))
    return fail(E3_ERR_ALIGNMENT, "x, w, dm, dx and dw must be 16-byte aligned");
  const e3k::TransposeLayout L = e3k::transpose_layout(n_nodes, n_edges);
  const int* ws = static_cast<const int*>(workspace);
  const bool yg = (desc->flags & E3_Y_GIVEN) != 0;
  e3k::BwdArgs a{n_nodes, p.C, G, ws + L.order, ws + L.colptr, ws + L.perm, ws + L.recv, ws + L.npad,
                 ws + L.padlist, n_edges, edge_vec_or_Y, x, w, dm, dx, dw, dY};
  return hip_status(ks->bwd[dtype][yg][ci](a, hipStream_t(stream)), "conv_backward");
}

e3_status e3_conv_backward_noalloc(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                   const int32_t* rowptr, const int32_t* sender,
                                   const float* edge_vec_or_Y, const void* x, const void* w,
                                   const void* dm, void* dx, void* dw, float* dY, e3_dtype dtype,
                                   void* stream) {
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  const e3k::KernelSet* ks;
  int G, ci;
  if ((s = select(p, dtype, Kind::bwd, ks, G, ci)) != E3_OK) return s;
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  if (n_nodes > e3k::kNoAllocMaxNodes || n_edges > e3k::kNoAllocMaxEdges)
    return fail(E3_ERR_UNSUPPORTED,
                "e3_conv_backward_noalloc takes at most " + std::to_string(e3k::kNoAllocMaxNodes) +
                    " nodes and " + std::to_string(e3k::kNoAllocMaxEdges) + " edges (got " +
                    std::to_string(n_nodes) + " and " + std::to_string(n_edges) +
                    "); use e3_conv_prepare_transpose and e3_conv_backward");
  if (n_nodes == 0) return ok();
  if (!rowptr || !x || !dx || !dm) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (n_edges > 0 && (!sender || !edge_vec_or_Y || !w || !dw || !dY))
    return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(x) || !aligned16(dm) || !aligned16(dx) ||
      (n_edges > 0 && (!aligned16(w) || !aligned16(dw))))
    return fail(E3_ERR_ALIGNMENT, "x, w, dm, dx and dw must be 16-byte aligned");
  if ((s = maybe_check(desc, n_nodes, n_edges, rowptr, sender, stream)) != E3_OK) return s;
  const e3k::TransposeLayout L = e3k::transpose_layout(n_nodes, n_edges);
  if (L.total_words > e3k::noalloc_scratch_words())
    return fail(E3_ERR_UNSUPPORTED, "the index does not fit the fixed scratch");
  int* ws = nullptr;  // the fixed scratch of the current device
  if ((s = hip_status(e3k::noalloc_scratch(&ws), "conv_backward_noalloc")) != E3_OK) return s;
  const hipStream_t st = hipStream_t(stream);
  const bool yg = (desc->flags & E3_Y_GIVEN) != 0;
  // the sender-ordered index of this graph into the scratch (the previous
  // call's contents are overwritten; every counter is cleared by a kernel)
  if ((s = hip_status(e3k::launch_prepare_transpose(n_nodes, n_edges, rowptr, sender,
                                                    (yg || n_edges == 0) ? nullptr : edge_vec_or_Y,
                                                    ws, st),
                      "conv_backward_noalloc")) != E3_OK)
    return s;
  e3k::BwdArgs a{n_nodes, p.C, G, ws + L.order, ws + L.colptr, ws + L.perm, ws + L.recv, ws + L.npad,
                 ws + L.padlist, n_edges, edge_vec_or_Y, x, w, dm, dx, dw, dY};
  return hip_status(ks->bwd[dtype][yg][ci](a, st), "conv_backward_noalloc");
}

namespace {

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Scratch of the double backward: one m-, x-, Y- and w-sized temporary.
size_t double_backward_scratch(const Parsed& p, int64_t n_nodes, int64_t n_edges, e3_dtype dt) {
  const size_t es = dt == E3_BF16 ? 2 : 4;
  return align256(size_t(n_nodes) * p.dout * p.C * es) +
         align256(size_t(n_nodes) * p.dx * p.C * es) + align256(size_t(n_edges) * p.dy * 4) +
         align256(size_t(n_edges) * p.P * p.C * es);
}

}  // namespace

e3_status e3_conv_double_backward_scratch_size(const e3_desc* desc, int32_t n_nodes,
                                               int32_t n_edges, e3_dtype dtype, size_t* bytes) {
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  if (!bytes) return fail(E3_ERR_INVALID_ARG, "bytes is null");
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  *bytes = double_backward_scratch(p, n_nodes, n_edges, dtype);
  return ok();
}

}  // extern "C"

namespace {

// The double backward of e3j E.1 Eq.17-18 composed from three forward and
// three backward calls (fwd, bwd) plus additions, the unused cotangents of
// each backward call going to the scratch.  Arguments checked by the caller.
template <class Fwd, class Bwd>
e3_status double_backward_composed(const Parsed& p, int32_t n_nodes, int32_t n_edges,
                                   const float* Y, const void* x, const void* w, const void* ddx,
                                   const float* ddY, const void* ddw, void* dx2, float* dY2,
                                   void* dw2, void* ddm, void* scratch, e3_dtype dtype,
                                   hipStream_t st, Fwd fwd, Bwd bwd) {
  const size_t es = dtype == E3_BF16 ? 2 : 4;
  char* sc = static_cast<char*>(scratch);
  void* t_m = sc;
  sc += align256(size_t(n_nodes) * p.dout * p.C * es);
  void* t_x = sc;
  sc += align256(size_t(n_nodes) * p.dx * p.C * es);
  float* t_Y = reinterpret_cast<float*>(sc);
  sc += align256(size_t(n_edges) * p.dy * 4);
  void* t_w = sc;
  const int bf = dtype == E3_BF16;
  const int64_t nm = int64_t(n_nodes) * p.dout * p.C, nx = int64_t(n_nodes) * p.dx * p.C;
  const int64_t nY = int64_t(n_edges) * p.dy, nw = int64_t(n_edges) * p.P * p.C;
  auto add = [&](void* dst, const void* src, int64_t n, int b16) {
    return hip_status(e3k::launch_add(dst, src, n, b16, st), "double_backward");
  };
  e3_status s;
  // ddm = conv(ddx, Y, w) + conv(x, ddY, w) + conv(x, Y, ddw)        (e3j Eq.17)
  if ((s = fwd(ddx, Y, w, ddm)) != E3_OK) return s;
  if ((s = fwd(x, ddY, w, t_m)) != E3_OK || (s = add(ddm, t_m, nm, bf)) != E3_OK) return s;
  if ((s = fwd(x, Y, ddw, t_m)) != E3_OK || (s = add(ddm, t_m, nm, bf)) != E3_OK) return s;
  // the three backward calls of e3j Eq.18, unused cotangents to scratch
  if ((s = bwd(ddx, Y, w, t_x, dw2, dY2)) != E3_OK) return s;
  if ((s = bwd(x, ddY, w, dx2, t_w, t_Y)) != E3_OK || (s = add(dw2, t_w, nw, bf)) != E3_OK)
    return s;
  if ((s = bwd(x, Y, ddw, t_x, t_w, t_Y)) != E3_OK || (s = add(dx2, t_x, nx, bf)) != E3_OK ||
      (s = add(dY2, t_Y, nY, 0)) != E3_OK)
    return s;
  return ok();
}

e3_status double_backward_checks(const e3_desc* desc, const Parsed& p, int32_t n_nodes,
                                 int32_t n_edges, const float* Y, const void* x, const void* w,
                                 const void* dm, const void* ddx, const float* ddY,
                                 const void* ddw, void* dx2, float* dY2, void* dw2, void* ddm,
                                 void* scratch, size_t scratch_bytes, e3_dtype dtype) {
  if (!(desc->flags & E3_Y_GIVEN))
    return fail(E3_ERR_INVALID_ARG, "the double backward takes given harmonics (E3_Y_GIVEN)");
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  if (n_nodes == 0) return ok();
  const size_t need = double_backward_scratch(p, n_nodes, n_edges, dtype);
  if (!scratch || scratch_bytes < need)
    return fail(E3_ERR_WORKSPACE, "scratch needs " + std::to_string(need) + " bytes");
  if (!aligned16(scratch)) return fail(E3_ERR_ALIGNMENT, "scratch must be 16-byte aligned");
  if (!x || !dm || !ddx || !dx2 || !ddm ||
      (n_edges > 0 && (!Y || !w || !ddY || !ddw || !dY2 || !dw2)))
    return fail(E3_ERR_INVALID_ARG, "null pointer");
  return ok();
}

}  // namespace

extern "C" {

e3_status e3_conv_double_backward(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                  const int32_t* rowptr, const int32_t* sender,
                                  const void* workspace, size_t ws_bytes, const float* Y,
                                  const void* x, const void* w, const void* dm, const void* ddx,
                                  const float* ddY, const void* ddw, void* dx2, float* dY2,
                                  void* dw2, void* ddm, void* scratch, size_t scratch_bytes,
                                  e3_dtype dtype, void* stream) {
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  if ((s = double_backward_checks(desc, p, n_nodes, n_edges, Y, x, w, dm, ddx, ddY, ddw, dx2, dY2,
                                  dw2, ddm, scratch, scratch_bytes, dtype)) != E3_OK ||
      n_nodes == 0)
    return s;
  if ((s = maybe_check(desc, n_nodes, n_edges, rowptr, sender, stream)) != E3_OK) return s;
  // the composed calls below run on the graph just checked
  e3_desc inner = *desc;
  inner.flags &= ~E3_CHECK;
  desc = &inner;
  auto fwd = [&](const void* xx, const float* yy, const void* ww, void* out) {
    return e3_conv_forward(desc, n_nodes, n_edges, rowptr, sender, workspace, ws_bytes, yy, xx,
                           ww, out, dtype, stream);
  };
  auto bwd = [&](const void* xx, const float* yy, const void* ww, void* ox, void* ow, float* oy) {
    return e3_conv_backward(desc, n_nodes, n_edges, rowptr, sender, workspace, ws_bytes, yy, xx,
                            ww, dm, ox, ow, oy, dtype, stream);
  };
  return double_backward_composed(p, n_nodes, n_edges, Y, x, w, ddx, ddY, ddw, dx2, dY2, dw2, ddm,
                                  scratch, dtype, hipStream_t(stream), fwd, bwd);
}

namespace {

// Block lists of a channel mixing: every block of a list has one
// multiplicity (the channel count of that side).
e3_status parse_linear(const e3_irreps* in, const e3_irreps* out, std::vector<e3k::IrSpec>& li,
                       std::vector<e3k::IrSpec>& lo, int& cin, int& cout) {
  if (!in || !out) return fail(E3_ERR_INVALID_ARG, "irreps pointer is null");
  std::vector<int> mi, mo;
  e3_status s;
  if ((s = parse_list(*in, "in", li, mi)) != E3_OK) return s;
  if ((s = parse_list(*out, "out", lo, mo)) != E3_OK) return s;
  if (li.empty() || lo.empty()) return fail(E3_ERR_IRREPS, "in and out need at least one block");
  cin = mi[0];
  cout = mo[0];
  for (int m : mi)
    if (m != cin) return fail(E3_ERR_IRREPS, "in blocks need one multiplicity");
  for (int m : mo)
    if (m != cout) return fail(E3_ERR_IRREPS, "out blocks need one multiplicity");
  return E3_OK;
}

}  // namespace

e3_status e3_linear_num_weights(const e3_irreps* in, const e3_irreps* out, int32_t* n_pairs) {
  std::vector<e3k::IrSpec> li, lo;
  int cin, cout;
  e3_status s = parse_linear(in, out, li, lo, cin, cout);
  if (s != E3_OK) return s;
  if (!n_pairs) return fail(E3_ERR_INVALID_ARG, "n_pairs is null");
  int n = 0;
  for (auto& a : li)
    for (auto& b : lo) n += (a.l == b.l && a.p == b.p);
  *n_pairs = n;
  return ok();
}

e3_status e3_linear(const e3_irreps* in, const e3_irreps* out, int64_t n_rows, const void* x,
                    const float* W, void* y, e3_dtype dtype, void* stream) {
  std::vector<e3k::IrSpec> li, lo;
  int cin, cout;
  e3_status s = parse_linear(in, out, li, lo, cin, cout);
  if (s != E3_OK) return s;
  if (dtype != E3_F32 && dtype != E3_BF16) return fail(E3_ERR_INVALID_ARG, "unknown dtype");
  if (cin % 8 != 0 || cin > 256 || cout % 32 != 0 || cout > 1024)
    return fail(E3_ERR_UNSUPPORTED, "channel mixing needs Cin a multiple of 8 up to 256 and "
                                    "Cout a multiple of 32 up to 1024");
  if (n_rows < 0) return fail(E3_ERR_INVALID_ARG, "n_rows < 0");
  if (n_rows == 0) return ok();
  if (!x || !W || !y) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(x) || !aligned16(y) || !aligned16(W))
    return fail(E3_ERR_ALIGNMENT, "x, W and y must be 16-byte aligned");
  int din = 0, dout = 0;
  for (auto& a : li) din += 2 * a.l + 1;
  for (auto& b : lo) dout += 2 * b.l + 1;
  // pair index of (i, o): input-block major, then output block
  std::vector<int> pair(li.size() * lo.size(), -1);
  int np = 0;
  for (size_t i = 0; i < li.size(); ++i)
    for (size_t o = 0; o < lo.size(); ++o)
      if (li[i].l == lo[o].l && li[i].p == lo[o].p) pair[i * lo.size() + o] = np++;
  int out_off = 0;
  for (size_t o = 0; o < lo.size(); ++o) {
    const int deg = 2 * lo[o].l + 1;
    int in_off = 0, used = 0;
    for (size_t i = 0; i < li.size(); ++i) {
      const int pi = pair[i * lo.size() + o];
      if (pi >= 0) {
        e3k::LinearBlockArgs a{n_rows, din, dout, cin, cout, in_off, out_off, deg,
                               x, W + int64_t(pi) * cin * cout, y, used > 0, 0, 0};
        if ((s = hip_status(e3k::launch_linear(a, dtype == E3_BF16, hipStream_t(stream)),
                            "linear")) != E3_OK)
          return s;
        ++used;
      }
      in_off += 2 * li[i].l + 1;
    }
    if (used == 0) {
      e3k::LinearBlockArgs a{n_rows, din, dout, cin, cout, 0, out_off, deg, x, W, y, 0, 1, 0};
      if ((s = hip_status(e3k::launch_linear(a, dtype == E3_BF16, hipStream_t(stream)),
                          "linear")) != E3_OK)
        return s;
    }
    out_off += deg;
  }
  return ok();
}

e3_status e3_linear_workspace_size(const e3_irreps* in, const e3_irreps* out, size_t* bytes) {
  std::vector<e3k::IrSpec> li, lo;
  int cin, cout;
  e3_status s = parse_linear(in, out, li, lo, cin, cout);
  if (s != E3_OK) return s;
  if (!bytes) return fail(E3_ERR_INVALID_ARG, "bytes is null");
  *bytes = size_t(e3k::kLinDwChunks) * cin * cout * sizeof(float);
  return ok();
}

e3_status e3_linear_backward(const e3_irreps* in, const e3_irreps* out, int64_t n_rows,
                             const void* x, const float* W, const void* dy, void* dx, float* dW,
                             void* workspace, size_t ws_bytes, e3_dtype dtype, void* stream) {
  std::vector<e3k::IrSpec> li, lo;
  int cin, cout;
  e3_status s = parse_linear(in, out, li, lo, cin, cout);
  if (s != E3_OK) return s;
  if (dtype != E3_F32 && dtype != E3_BF16) return fail(E3_ERR_INVALID_ARG, "unknown dtype");
  if (cin % 32 != 0 || cin > 128 || cout % 32 != 0 || cout > 256)
    return fail(E3_ERR_UNSUPPORTED, "channel-mixing backward needs Cin a multiple of 32 up to "
                                    "128 and Cout a multiple of 32 up to 256");
  if (n_rows < 0) return fail(E3_ERR_INVALID_ARG, "n_rows < 0");
  size_t need = 0;
  e3_linear_workspace_size(in, out, &need);
  if (!workspace || ws_bytes < need)
    return fail(E3_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
  if (!dW || (n_rows > 0 && (!x || !W || !dy || !dx)))
    return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(workspace) || !aligned16(dW) ||
      (n_rows > 0 && (!aligned16(x) || !aligned16(W) || !aligned16(dy) || !aligned16(dx))))
    return fail(E3_ERR_ALIGNMENT, "x, W, dy, dx, dW and the workspace must be 16-byte aligned");
  int din = 0, dout = 0;
  std::vector<int> ioff, ooff;
  for (auto& a : li) {
    ioff.push_back(din);
    din += 2 * a.l + 1;
  }
  for (auto& b : lo) {
    ooff.push_back(dout);
    dout += 2 * b.l + 1;
  }
  std::vector<int> pair(li.size() * lo.size(), -1);
  int np = 0;
  for (size_t i = 0; i < li.size(); ++i)
    for (size_t o = 0; o < lo.size(); ++o)
      if (li[i].l == lo[o].l && li[i].p == lo[o].p) pair[i * lo.size() + o] = np++;
  const hipStream_t st = hipStream_t(stream);
  const int bf = dtype == E3_BF16;
  // dx: per input block, dy of each matching output block times W^T
  if (n_rows > 0)
    for (size_t i = 0; i < li.size(); ++i) {
      const int deg = 2 * li[i].l + 1;
      int used = 0;
      for (size_t o = 0; o < lo.size(); ++o) {
        const int pi = pair[i * lo.size() + o];
        if (pi < 0) continue;
        e3k::LinearBlockArgs a{n_rows, dout, din, cout, cin, ooff[o], ioff[i], deg,
                               dy, W + int64_t(pi) * cin * cout, dx, used > 0, 0, 1};
        if ((s = hip_status(e3k::launch_linear(a, bf, st), "linear_backward")) != E3_OK) return s;
        ++used;
      }
      if (used == 0) {
        e3k::LinearBlockArgs a{n_rows, dout, din, cout, cin, 0, ioff[i], deg, dy, W, dx, 0, 1, 0};
        if ((s = hip_status(e3k::launch_linear(a, bf, st), "linear_backward")) != E3_OK) return s;
      }
    }
  // dW per pair, through the workspace's partial sums
  for (size_t i = 0; i < li.size(); ++i)
    for (size_t o = 0; o < lo.size(); ++o) {
      const int pi = pair[i * lo.size() + o];
      if (pi < 0) continue;
      e3k::LinearDwArgs a{n_rows, din, dout, cin, cout, ioff[i], ooff[o], 2 * li[i].l + 1,
                          x, dy, static_cast<float*>(workspace), dW + int64_t(pi) * cin * cout, 0};
      if ((s = hip_status(e3k::launch_linear_dw(a, bf, st), "linear_backward")) != E3_OK) return s;
    }
  return ok();
}

namespace {

e3_status check_radial(const e3_radial* mlp) {
  if (!mlp) return fail(E3_ERR_INVALID_ARG, "radial parameters are null");
  if (!(mlp->cutoff > 0.0f) || !std::isfinite(mlp->cutoff))
    return fail(E3_ERR_INVALID_ARG, "cutoff must be positive and finite");
  if (mlp->n_basis != 8 || mlp->hidden != 64)
    return fail(E3_ERR_UNSUPPORTED, "radial MLP must have 8 basis functions and 64 hidden units");
  if (!mlp->W1 || !mlp->W2) return fail(E3_ERR_INVALID_ARG, "W1 or W2 is null");
  return ok();
}

}  // namespace

e3_status e3_radial_mlp(const e3_radial* mlp, int32_t n_edges, int32_t n_cols,
                        const float* edge_vec, float* w, void* stream) {
  e3_status s = check_radial(mlp);
  if (s != E3_OK) return s;
  if (n_edges < 0 || n_cols <= 0) return fail(E3_ERR_INVALID_ARG, "bad size");
  if (n_cols % 16) return fail(E3_ERR_UNSUPPORTED, "n_cols must be a multiple of 16");
  if (n_edges == 0) return ok();
  if (!edge_vec || !w) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(w)) return fail(E3_ERR_ALIGNMENT, "w must be 16-byte aligned");
  return hip_status(e3k::launch_radial_mlp(n_edges, n_cols, edge_vec, mlp->cutoff, mlp->W1,
                                           mlp->W2, w, hipStream_t(stream)),
                    "radial_mlp");
}

e3_status e3_radial_mlp_hidden(const e3_radial* mlp, int32_t n_edges, int32_t n_cols,
                               const void* hidden, size_t h_bytes, float* w, void* stream) {
  e3_status s = check_radial(mlp);
  if (s != E3_OK) return s;
  if (n_edges < 0 || n_cols <= 0) return fail(E3_ERR_INVALID_ARG, "bad size");
  if (n_cols % 16) return fail(E3_ERR_UNSUPPORTED, "n_cols must be a multiple of 16");
  if (n_edges == 0) return ok();
  if (!hidden || !w) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (h_bytes < size_t(n_edges) * e3k::kRadialHiddenBytes)
    return fail(E3_ERR_WORKSPACE, "hidden needs " +
                                      std::to_string(size_t(n_edges) * e3k::kRadialHiddenBytes) +
                                      " bytes");
  if (!aligned16(w) || !aligned16(hidden))
    return fail(E3_ERR_ALIGNMENT, "w and hidden must be 16-byte aligned");
  return hip_status(e3k::launch_radial_mlp(n_edges, n_cols, nullptr, mlp->cutoff, mlp->W1,
                                           mlp->W2, w, hipStream_t(stream), hidden),
                    "radial_mlp_hidden");
}

e3_status e3_radial_hidden_size(int32_t n_edges, size_t* bytes) {
  if (!bytes) return fail(E3_ERR_INVALID_ARG, "bytes is null");
  if (n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  *bytes = size_t(n_edges) * e3k::kRadialHiddenBytes;
  return ok();
}

e3_status e3_radial_hidden(const e3_radial* mlp, int32_t n_edges, const float* edge_vec,
                           void* hidden, size_t h_bytes, void* stream) {
  e3_status s = check_radial(mlp);
  if (s != E3_OK) return s;
  if (n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  if (n_edges == 0) return ok();
  if (!edge_vec || !hidden) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (h_bytes < size_t(n_edges) * e3k::kRadialHiddenBytes)
    return fail(E3_ERR_WORKSPACE, "hidden needs " +
                                      std::to_string(size_t(n_edges) * e3k::kRadialHiddenBytes) +
                                      " bytes");
  if (!aligned16(hidden)) return fail(E3_ERR_ALIGNMENT, "hidden must be 16-byte aligned");
  return hip_status(e3k::launch_radial_hidden(n_edges, edge_vec, mlp->cutoff, mlp->W1, hidden,
                                              hipStream_t(stream)),
                    "radial_hidden");
}

}  // extern "C"

namespace {

e3_status conv_forward_radial_impl(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                   const int32_t* rowptr, const int32_t* sender,
                                   const void* workspace, size_t ws_bytes, const float* edge_vec,
                                   const float* x, const e3_radial* mlp, const void* hidden,
                                   size_t h_bytes, float* m, void* stream) {
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  if ((s = check_radial(mlp)) != E3_OK) return s;
  if (desc->flags & (E3_Y_GIVEN | E3_OUT_PER_PATH))
    return fail(E3_ERR_UNSUPPORTED, "the radial convolution takes edge vectors and collapsed outputs");
  const e3k::KernelSet* ks = find_set(p);
  if (!ks || !e3k::radial_conv_supported(ks->name))
    return fail(E3_ERR_UNSUPPORTED,
                "no radial convolution kernel for this signature (supported: 0e+1o x harmonics "
                "0e+1o+2e+3o -> 0e+1o+2e+3o)");
  if (p.C != 32 && p.C != 64 && p.C != 128 && p.C != 256)
    return fail(E3_ERR_UNSUPPORTED, "the radial convolution needs C in {32, 64, 128, 256}");
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  if (n_nodes == 0) return ok();
  if ((s = maybe_check(desc, n_nodes, n_edges, rowptr, sender, stream)) != E3_OK) return s;
  if (!rowptr || !x || !m) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (n_edges > 0 && (!sender || !edge_vec)) return fail(E3_ERR_INVALID_ARG, "null pointer");
  const int* order = nullptr;
  if (workspace) {
    size_t need = 0;
    e3_conv_workspace_size(n_nodes, n_edges, &need);
    if (ws_bytes < need)
      return fail(E3_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
    order = static_cast<const int*>(workspace) + e3k::transpose_layout(n_nodes, n_edges).order;
  }
  if (hidden) {
    if (h_bytes < size_t(n_edges) * e3k::kRadialHiddenBytes)
      return fail(E3_ERR_WORKSPACE, "hidden needs " +
                                        std::to_string(size_t(n_edges) * e3k::kRadialHiddenBytes) +
                                        " bytes");
    if (!aligned16(hidden)) return fail(E3_ERR_ALIGNMENT, "hidden must be 16-byte aligned");
  }
  e3k::RadialConvArgs a{n_nodes, n_edges, p.C, order, rowptr, sender, edge_vec, x,
                        mlp->W1, mlp->W2, mlp->cutoff, m, hidden};
  return hip_status(e3k::launch_conv_fwd_radial(ks->name, a, hipStream_t(stream)),
                    "conv_forward_radial");
}

}  // namespace

extern "C" {

e3_status e3_conv_forward_radial(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                 const int32_t* rowptr, const int32_t* sender,
                                 const void* workspace, size_t ws_bytes, const float* edge_vec,
                                 const float* x, const e3_radial* mlp, float* m, void* stream) {
  return conv_forward_radial_impl(desc, n_nodes, n_edges, rowptr, sender, workspace, ws_bytes,
                                  edge_vec, x, mlp, nullptr, 0, m, stream);
}

e3_status e3_conv_forward_radial_hidden(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                        const int32_t* rowptr, const int32_t* sender,
                                        const void* workspace, size_t ws_bytes,
                                        const float* edge_vec, const float* x,
                                        const e3_radial* mlp, const void* hidden, size_t h_bytes,
                                        float* m, void* stream) {
  if (!hidden) return fail(E3_ERR_INVALID_ARG, "hidden is null");
  return conv_forward_radial_impl(desc, n_nodes, n_edges, rowptr, sender, workspace, ws_bytes,
                                  edge_vec, x, mlp, hidden, h_bytes, m, stream);
}

e3_status e3_conv_backward_radial_scratch_size(const e3_desc* desc, int32_t n_edges,
                                               size_t* bytes) {
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  if (!bytes) return fail(E3_ERR_INVALID_ARG, "bytes is null");
  if (n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  if (p.C < 32 || p.C % 32) return fail(E3_ERR_UNSUPPORTED, "the radial convolution needs C in {32, 64, 128, 256}");
  *bytes = e3k::conv_bwd_radial_scratch_bytes(n_edges, p.C, p.dy);
  return ok();
}

e3_status e3_conv_backward_radial_hidden(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                         const int32_t* rowptr, const int32_t* sender,
                                         const void* workspace, size_t ws_bytes,
                                         const float* edge_vec, const float* x,
                                         const e3_radial* mlp, const void* hidden, size_t h_bytes,
                                         const float* dm, float* dx, float* dw, float* dY,
                                         void* scratch, size_t scratch_bytes, void* stream) {
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  if ((s = check_radial(mlp)) != E3_OK) return s;
  if (desc->flags & (E3_Y_GIVEN | E3_OUT_PER_PATH))
    return fail(E3_ERR_UNSUPPORTED, "the radial convolution takes edge vectors and collapsed outputs");
  const e3k::KernelSet* ks = find_set(p);
  if (!ks || !e3k::radial_conv_supported(ks->name))
    return fail(E3_ERR_UNSUPPORTED,
                "no radial convolution kernel for this signature (supported: 0e+1o x harmonics "
                "0e+1o+2e+3o -> 0e+1o+2e+3o)");
  if (p.C != 32 && p.C != 64 && p.C != 128 && p.C != 256)
    return fail(E3_ERR_UNSUPPORTED, "the radial convolution needs C in {32, 64, 128, 256}");
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  if (n_nodes == 0) return ok();
  if ((s = maybe_check(desc, n_nodes, n_edges, rowptr, sender, stream)) != E3_OK) return s;
  size_t need = 0;
  e3_conv_workspace_size(n_nodes, n_edges, &need);
  if (!workspace || ws_bytes < need)
    return fail(E3_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
  if (!x || !dm || !dx) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (n_edges > 0 && (!edge_vec || !hidden || !dw || !dY))
    return fail(E3_ERR_INVALID_ARG, "null pointer");
  const size_t sneed = e3k::conv_bwd_radial_scratch_bytes(n_edges, p.C, p.dy);
  if (n_edges > 0 && (!scratch || scratch_bytes < sneed))
    return fail(E3_ERR_WORKSPACE, "scratch needs " + std::to_string(sneed) + " bytes");
  if (n_edges > 0 && h_bytes < size_t(n_edges) * e3k::kRadialHiddenBytes)
    return fail(E3_ERR_WORKSPACE, "hidden needs " +
                                      std::to_string(size_t(n_edges) * e3k::kRadialHiddenBytes) +
                                      " bytes");
  if (!aligned16(x) || !aligned16(dm) || !aligned16(dx) ||
      (n_edges > 0 && (!aligned16(hidden) || !aligned16(dw))))
    return fail(E3_ERR_ALIGNMENT, "x, dm, dx, dw and hidden must be 16-byte aligned");
  const e3k::TransposeLayout L = e3k::transpose_layout(n_nodes, n_edges);
  const int* ws = static_cast<const int*>(workspace);
  e3k::RadialBwdArgs a{n_nodes, n_edges, p.C, ws + L.order, ws + L.colptr, ws + L.perm,
                       ws + L.recv, ws + L.npad, ws + L.padlist, edge_vec, x, mlp->W2, hidden,
                       dm, dx, dw, dY, static_cast<float*>(scratch)};
  return hip_status(e3k::launch_conv_bwd_radial(ks->name, a, hipStream_t(stream)),
                    "conv_backward_radial");
}

namespace {

// The radial MLP's second layer seen as a channel mixing: input 64x0e (h),
// output nb blocks of cb x 0e (the columns of w in blocks of cb <= 256).
struct RadialBwdPlan {
  int ranges = 0, slabs = 0;
  size_t off_dh = 0, off_part2 = 0, off_part = 0, off_w2s = 0, off_basis = 0, total = 0;
};

e3_status radial_bwd_plan(int n_edges, int n_cols, RadialBwdPlan& r) {
  if (n_cols <= 0 || n_cols % 32)
    return fail(E3_ERR_UNSUPPORTED, "the radial backward needs n_cols a multiple of 32");
  r.ranges = e3k::radial_dw2_ranges(n_edges, n_cols);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  r.slabs = e3k::radial_dw2_slabs(n_cols);
  r.off_dh = take(size_t(r.slabs) * size_t(n_edges) * 64 * 4);
  r.off_part2 = take(size_t(r.ranges) * 64 * n_cols * 4);
  r.off_part = take(size_t(e3k::kRadialTailChunks) * 512 * 4);
  r.off_w2s = take(e3k::radial_w2_split_bytes(n_cols));
  r.off_basis = take(size_t(n_edges) * 16 * 4);
  r.total = o;
  return ok();
}

}  // namespace

e3_status e3_radial_mlp_backward_workspace_size(const e3_radial* mlp, int32_t n_edges,
                                                int32_t n_cols, size_t* bytes) {
  e3_status s = check_radial(mlp);
  if (s != E3_OK) return s;
  if (!bytes) return fail(E3_ERR_INVALID_ARG, "bytes is null");
  if (n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  RadialBwdPlan r;
  if ((s = radial_bwd_plan(n_edges, n_cols, r)) != E3_OK) return s;
  *bytes = r.total;
  return ok();
}

e3_status e3_radial_mlp_backward(const e3_radial* mlp, int32_t n_edges, int32_t n_cols,
                                 const float* edge_vec, const float* dw, float* dW1, float* dW2,
                                 float* dvec, void* workspace, size_t ws_bytes, void* stream) {
  e3_status s = check_radial(mlp);
  if (s != E3_OK) return s;
  if (n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  RadialBwdPlan r;
  if ((s = radial_bwd_plan(n_edges, n_cols, r)) != E3_OK) return s;
  if (!dW1 || !dW2) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (n_edges > 0 && (!edge_vec || !dw || !dvec)) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (!workspace || ws_bytes < r.total)
    return fail(E3_ERR_WORKSPACE, "workspace needs " + std::to_string(r.total) + " bytes");
  if (!aligned16(workspace) || !aligned16(mlp->W2) || (n_edges > 0 && !aligned16(dw)))
    return fail(E3_ERR_ALIGNMENT, "workspace, W2 and dw must be 16-byte aligned");
  const hipStream_t st = hipStream_t(stream);
  char* ws = static_cast<char*>(workspace);
  float* dh = reinterpret_cast<float*>(ws + r.off_dh);
  float* part2 = reinterpret_cast<float*>(ws + r.off_part2);
  float* part = reinterpret_cast<float*>(ws + r.off_part);
  // dh = dw W2^T through per-slab partials, and dW2 = h^T dw through
  // per-range partials (bf16 matrix cores on three-part splits of the fp32
  // operands; one read of dw for both)
  if ((s = hip_status(e3k::launch_radial_dh_dw2(n_edges, n_cols, edge_vec, mlp->cutoff, mlp->W1,
                                                mlp->W2, dw, dh, part2, r.ranges, ws + r.off_w2s,
                                                reinterpret_cast<float*>(ws + r.off_basis), st),
                      "radial_mlp_backward")) != E3_OK)
    return s;
  if ((s = hip_status(e3k::launch_sum_partials(r.ranges, 64 * n_cols, part2, dW2, st),
                      "radial_mlp_backward")) != E3_OK)
    return s;
  // through SiLU and the first layer: dW1, and the radial part of dvec
  return hip_status(e3k::launch_radial_tail(n_edges, edge_vec, mlp->W1,
                                            reinterpret_cast<const float*>(ws + r.off_basis), dh,
                                            r.slabs, dvec, part, dW1, st),
                    "radial_mlp_backward");
}

namespace {

// The coefficient tables of a descriptor (layout in kernels/generic.hip),
// from the ladder-built real CG blocks.  Every nonzero coefficient c of
// path P couples output component o, x component xi and y component yi; a
// table keys the entries by what the kernel writes and names which array
// acts as its per-lane operand, which as its per-row weight and which as
// its second factor (the y slot of a record):
//   forward  z[o]   = sum_P w[P]  sum c y[yi] x[xi]    key o,  weight P, operand xi, y yi
//   dx       dx[xi] = sum_P w[P]  sum c y[yi] dz[o]    key xi, weight P, operand o,  y yi
//   dw       dw[P]  = sum_o dz[o] sum c y[yi] x[xi]    key P,  weight o, operand xi, y yi
//   dy       dy[yi] = sum_P w[P]  sum c dz[o] x[xi]    key yi, weight P, operand xi, y o
// (e3j E.1 Eq.14-16: each cotangent is the same coupling with the
// coefficient records permuted.)
struct GenEntry {
  int P, o, xi, yi;
  float c;
};

struct GenDims {
  int operand, y, keys, weights;  // kernel's view: x comps, y comps, outputs, w rows
};

e3_status generic_entries(const e3_desc* desc, Parsed& p, std::vector<GenEntry>& ent,
                          bool table_limits = true) {
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  for (const auto* v : {&p.x, &p.y, &p.o})
    for (const auto& r : *v)
      if (r.l > kGenericLmax) return fail(E3_ERR_UNSUPPORTED, "generic tables go to degree 8");
  if (p.dy >= 65536) return fail(E3_ERR_UNSUPPORTED, "too many y components");
  if (table_limits && (p.dx * 64 + p.dy > 4096 || p.dout * 64 + p.dy > 4096))
    return fail(E3_ERR_UNSUPPORTED,
                "too many components for the generic kernel (dx, dout <= 63)");
  std::vector<int> xoff(p.x.size()), yoff(p.y.size()), ooff(p.o.size());
  int o = 0;
  for (size_t i = 0; i < p.x.size(); ++i) xoff[i] = o, o += 2 * p.x[i].l + 1;
  o = 0;
  for (size_t i = 0; i < p.y.size(); ++i) yoff[i] = o, o += 2 * p.y[i].l + 1;
  o = 0;
  for (size_t i = 0; i < p.o.size(); ++i) ooff[i] = o, o += 2 * p.o[i].l + 1;
  ent.clear();
  int oo_pp = 0;  // output offset of the current path in per-path mode
  for (int pi = 0; pi < p.P; ++pi) {
    const int l1 = p.x[p.pix[pi]].l, l2 = p.y[p.piy[pi]].l, L = p.o[p.pio[pi]].l;
    const int xo = xoff[p.pix[pi]], yo = yoff[p.piy[pi]];
    const int oo = p.per_path ? oo_pp : ooff[p.pio[pi]];
    oo_pp += 2 * L + 1;
    std::vector<double> T;
    if (!e3::cg_real_block(l1, l2, L, T)) return fail(E3_ERR_IRREPS, "path does not couple");
    const int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1;
    for (int M = 0; M < 2 * L + 1; ++M)
      for (int a = 0; a < n1; ++a)
        for (int b = 0; b < n2; ++b) {
          const double c = T[(size_t(M) * n1 + a) * n2 + b];
          if (std::fabs(c) >= 1e-12) ent.push_back(GenEntry{pi, oo + M, xo + a, yo + b, float(c)});
        }
  }
  return ok();
}

GenDims generic_dims(const Parsed& p, int table) {
  if (table == E3_GEN_DX) return GenDims{p.dout, p.dy, p.dx, p.P};
  if (table == E3_GEN_DW) return GenDims{p.dx, p.dy, p.P, p.dout};
  if (table == E3_GEN_DY) return GenDims{p.dx, p.dout, p.dy, p.P};
  return GenDims{p.dx, p.dy, p.dout, p.P};
}

e3_status build_generic(const e3_desc* desc, int table, std::vector<int32_t>& out) {
  if (table != E3_GEN_FORWARD && table != E3_GEN_DX && table != E3_GEN_DW && table != E3_GEN_DY)
    return fail(E3_ERR_INVALID_ARG, "unknown table");
  Parsed p;
  std::vector<GenEntry> ent;
  e3_status s = generic_entries(desc, p, ent);
  if (s != E3_OK) return s;
  const GenDims dm = generic_dims(p, table);
  auto key = [&](const GenEntry& e) {
    return table == E3_GEN_DX ? e.xi : table == E3_GEN_DW ? e.P : table == E3_GEN_DY ? e.yi : e.o;
  };
  auto weight = [&](const GenEntry& e) { return table == E3_GEN_DW ? e.o : e.P; };
  auto operand = [&](const GenEntry& e) { return table == E3_GEN_DX ? e.o : e.xi; };
  auto second = [&](const GenEntry& e) { return table == E3_GEN_DY ? e.o : e.yi; };
  // group by (key, weight), keeping the coefficient order within a group
  std::stable_sort(ent.begin(), ent.end(), [&](const GenEntry& a, const GenEntry& b) {
    return key(a) != key(b) ? key(a) < key(b) : weight(a) < weight(b);
  });
  struct Contrib {
    int weight, rb, re;
  };
  std::vector<std::vector<Contrib>> per_key(dm.keys);
  std::vector<int32_t> rec;
  for (size_t i = 0; i < ent.size();) {
    size_t j = i;
    while (j < ent.size() && key(ent[j]) == key(ent[i]) && weight(ent[j]) == weight(ent[i])) ++j;
    const int rb = int(rec.size() / 2);
    for (size_t k = i; k < j; ++k) {
      int32_t bits;
      std::memcpy(&bits, &ent[k].c, 4);
      rec.push_back(int32_t(operand(ent[k]) | (second(ent[k]) << 16)));
      rec.push_back(bits);
    }
    while ((rec.size() / 2) % 4) {  // pad the run to whole groups of 4 (zero records)
      rec.push_back(int32_t(operand(ent[i]) | (second(ent[i]) << 16)));
      rec.push_back(0);
    }
    per_key[key(ent[i])].push_back(Contrib{weight(ent[i]), rb, int(rec.size() / 2)});
    i = j;
  }
  int n_contrib = 0;
  for (auto& v : per_key) n_contrib += int(v.size());
  const size_t rec_words = rec.size();
  size_t rec_off = size_t(e3k::kGenHeader) + dm.keys + 1 + 3 * size_t(n_contrib);
  rec_off = (rec_off + 7) / 8 * 8;  // records start on a 32-byte boundary
  out.assign(rec_off + rec_words, 0);
  const int32_t head[e3k::kGenHeader] = {int32_t(e3k::kGenMagic), int32_t(dm.operand),
                                         int32_t(dm.y),           int32_t(dm.keys),
                                         int32_t(dm.weights),     int32_t(n_contrib),
                                         int32_t(rec_words / 2),  int32_t(rec_off)};
  for (int i = 0; i < e3k::kGenHeader; ++i) out[i] = head[i];
  size_t w = e3k::kGenHeader;
  int acc = 0;
  for (int i = 0; i < dm.keys; ++i) out[w++] = acc, acc += int(per_key[i].size());
  out[w++] = acc;
  for (auto& v : per_key)
    for (auto& c : v) out[w++] = c.weight, out[w++] = c.rb, out[w++] = c.re;
  std::copy(rec.begin(), rec.end(), out.begin() + rec_off);
  return ok();
}

// The dense-product plan of the tensor product (kernels/gemm.hip).  Output
// blocks are the output irreps (one per path with E3_OUT_PER_PATH); a block's
// K list concatenates, in path order, the x components (P, m1) of its paths
// and pads to a multiple of 4; A[M][k] = sum_{m2} C_P[M][m1][m2] y[m2] is
// listed as groups of (y component, c) records, one group per nonzero entry.
// Dense-product plans.  Each is one matrix product per block over a K list
// of (path, input component) columns, A[k][M] built per row from y:
//   kind 0 (E3_GEN_GEMM, the forward): blocks = output irreps (or paths
//     with E3_OUT_PER_PATH), input x, out[o] += A w[P] x[xi];
//   kind 1 (E3_GEN_GEMM_DX, the gradient of x): the same entries with the
//     roles of x and the output swapped -- blocks = x irreps, input dz,
//     dx[xi] += A w[P] dz[o] (A'[m1][(P,M)] = sum_m2 C_P[M][m1][m2] y[m2]);
//   kind 2 (E3_GEN_GEMM_DW, the gradient of w): build_gemm_dw.
// Every block owns its rows (a block no path reaches gets K = 0).
// Groups {A index, y1 | y2 << 16, c1, c2} from (A index, y component, c)
// terms: one group per A element; the real basis couples each (M, m1) to at
// most two m2.
struct AGroupTerm {
  int at, yi;
  float c;
};
e3_status a_groups(std::vector<AGroupTerm>& ge, std::vector<int32_t>& groups) {
  std::stable_sort(ge.begin(), ge.end(),
                   [](const AGroupTerm& a, const AGroupTerm& b) { return a.at < b.at; });
  groups.clear();
  for (size_t i = 0; i < ge.size();) {
    size_t j = i;
    while (j < ge.size() && ge[j].at == ge[i].at) ++j;
    if (j - i > 2) return fail(E3_ERR_UNSUPPORTED, "an A entry with more than two terms");
    const AGroupTerm& a = ge[i];
    const AGroupTerm& b = j - i == 2 ? ge[i + 1] : AGroupTerm{a.at, a.yi, 0.0f};
    int32_t ca, cb;
    std::memcpy(&ca, &a.c, 4);
    std::memcpy(&cb, &b.c, 4);
    groups.insert(groups.end(), {a.at, int32_t(a.yi | (b.yi << 16)), ca, cb});
    i = j;
  }
  return ok();
}

e3_status build_gemm_dw(const e3_desc* desc, std::vector<int32_t>& out, e3k::TpGemmArgs& d);

e3_status build_gemm_kind(const e3_desc* desc, int kind, std::vector<int32_t>& out,
                          e3k::TpGemmArgs& d) {
  if (kind == 2) return build_gemm_dw(desc, out, d);
  Parsed p;
  std::vector<GenEntry> ent;
  e3_status s = generic_entries(desc, p, ent, false);
  if (s != E3_OK) return s;
  if (p.P > 32767 || p.dx > 65535 || p.dout > 65535)
    return fail(E3_ERR_UNSUPPORTED, "too many paths or components");
  std::vector<int> xoff(p.x.size()), ooff(p.o.size()), oo_path(p.P);
  for (size_t i = 0, o = 0; i < p.x.size(); ++i) xoff[i] = int(o), o += 2 * p.x[i].l + 1;
  for (size_t i = 0, o = 0; i < p.o.size(); ++i) ooff[i] = int(o), o += 2 * p.o[i].l + 1;
  for (int pi = 0, opp = 0; pi < p.P; ++pi) {
    oo_path[pi] = p.per_path ? opp : ooff[p.pio[pi]];
    opp += 2 * p.o[p.pio[pi]].l + 1;
  }
  const bool per_path_blocks = kind == 0 && p.per_path;
  const int nb = per_path_blocks ? p.P : kind == 1 ? int(p.x.size()) : int(p.o.size());
  auto block_of = [&](int pi) { return per_path_blocks ? pi : kind == 1 ? p.pix[pi] : p.pio[pi]; };
  auto in_off = [&](int pi) { return kind == 1 ? oo_path[pi] : xoff[p.pix[pi]]; };
  auto in_width = [&](int pi) {
    return 2 * (kind == 1 ? p.o[p.pio[pi]].l : p.x[p.pix[pi]].l) + 1;
  };
  auto out_comp = [&](const GenEntry& e) { return kind == 1 ? e.xi : e.o; };
  auto in_comp = [&](const GenEntry& e) { return kind == 1 ? e.o : e.xi; };
  std::vector<int> b_oo(nb), b_rows(nb), b_kb(nb), b_K(nb);
  for (int b = 0; b < nb; ++b) {
    if (per_path_blocks) {
      b_oo[b] = oo_path[b];
      b_rows[b] = 2 * p.o[p.pio[b]].l + 1;
    } else if (kind == 1) {
      b_oo[b] = xoff[b];
      b_rows[b] = 2 * p.x[b].l + 1;
    } else {
      b_oo[b] = ooff[b];
      b_rows[b] = 2 * p.o[b].l + 1;
    }
  }
  std::vector<int> path_koff(p.P);
  std::vector<std::vector<int>> bpaths(nb);
  for (int pi = 0; pi < p.P; ++pi) bpaths[block_of(pi)].push_back(pi);
  std::vector<int32_t> klist;
  for (int b = 0; b < nb; ++b) {
    b_kb[b] = int(klist.size());
    int k = 0;
    for (int pi : bpaths[b]) {
      path_koff[pi] = k;
      for (int m = 0; m < in_width(pi); ++m) klist.push_back((pi << 16) | (in_off(pi) + m));
      k += in_width(pi);
    }
    while (k % 4) klist.push_back(-1), ++k;
    b_K[b] = k;
  }
  // The matrix cores' products have 16 rows: a block of more rows (degree
  // 8: 17) is emitted as blocks of at most 16 rows sharing its K list, each
  // with its own part of A.
  struct Sub {
    int oo, rows, kb, K, abase;
  };
  std::vector<Sub> subs;
  std::vector<int> b_sub0(nb);
  int abase = 0;
  for (int b = 0; b < nb; ++b) {
    if (b_rows[b] > 64) return fail(E3_ERR_UNSUPPORTED, "an irrep of more than 64 components");
    b_sub0[b] = int(subs.size());
    for (int r0 = 0; r0 < b_rows[b]; r0 += 16) {
      const int rows = std::min(16, b_rows[b] - r0);
      subs.push_back(Sub{b_oo[b] + r0, rows, b_kb[b], b_K[b], abase});
      abase += rows * b_K[b];
    }
  }
  std::vector<AGroupTerm> ge;
  ge.reserve(ent.size());
  for (const GenEntry& e : ent) {
    const int b = block_of(e.P);
    const int M = out_comp(e) - b_oo[b];
    const int k = path_koff[e.P] + (in_comp(e) - in_off(e.P));
    const Sub& sb = subs[size_t(b_sub0[b] + M / 16)];
    ge.push_back(AGroupTerm{sb.abase + k * sb.rows + M % 16, e.yi, e.c});  // A[k][M]
  }
  const int nsub = int(subs.size());
  std::vector<int32_t> groups;
  if ((s = a_groups(ge, groups)) != E3_OK) return s;
  const int n_groups = int(groups.size() / 4);
  // the kernel's view: input components (dx), output components (dout)
  const int in_dim = kind == 1 ? p.dout : p.dx, out_dim = kind == 1 ? p.dx : p.dout;
  d = e3k::TpGemmArgs{};
  for (const Sub& sb : subs) d.a_block_max = std::max(d.a_block_max, sb.rows * sb.K);
  d.n_blocks = nsub;
  d.dx = in_dim;
  d.dy = p.dy;
  d.dout = out_dim;
  d.P = p.P;
  d.n_klist = int(klist.size());
  d.n_groups = n_groups;
  d.a_floats = std::max(abase, 1);
  d.off_blocks = e3k::kGemmHeader;
  d.off_klist = d.off_blocks + 4 * nsub;
  d.off_groups = (d.off_klist + d.n_klist + 3) / 4 * 4;  // 16-byte entries
  d.plan_words = d.off_groups + int(groups.size());
  out.assign(size_t(d.plan_words), 0);
  const int32_t head[14] = {e3k::kGemmMagic + kind, nsub,    in_dim,       p.dy,
                            out_dim,           p.P,          d.n_klist,    n_groups,
                            0,                 d.a_floats,   d.off_blocks, d.off_klist,
                            d.off_groups,      d.plan_words};
  std::copy(head, head + 14, out.begin());
  for (int b = 0; b < nsub; ++b) {
    out[d.off_blocks + 4 * b] = subs[size_t(b)].oo;
    out[d.off_blocks + 4 * b + 1] = subs[size_t(b)].rows;
    out[d.off_blocks + 4 * b + 2] = subs[size_t(b)].kb;
    out[d.off_blocks + 4 * b + 3] = subs[size_t(b)].K;
  }
  std::copy(klist.begin(), klist.end(), out.begin() + d.off_klist);
  std::copy(groups.begin(), groups.end(), out.begin() + d.off_groups);
  return ok();
}

e3_status build_gemm(const e3_desc* desc, std::vector<int32_t>& out, e3k::TpGemmArgs& d) {
  return build_gemm_kind(desc, 0, out, d);
}

// The gradient of w (E3_GEN_GEMM_DW): per row and path P,
//   dw[P][q] = sum_M dz[oo_P + M][q] (A_P x)[M][q],  A_P[M][m1] = sum_m2 C_P[M][m1][m2] y[m2].
// The rows (P, M) of each path, in runs of four (quads; a path's last quad
// padded with rows that read a zero dz row), are stacked in path order, so
// that the paths of one x irrep are consecutive, and cut into tiles of at
// most four quads that never mix x irreps or groups of 16 paths (16 t ..
// 16 t + 15): a tile is one product A x over its irrep's components (the K
// list, shared by the irrep's tiles; an irrep of more than 16 components,
// degree 8, gives each tile one block per K chunk of 16, consecutive, on
// the same rows), each quad's four rows are added up in the lane that holds
// them, and the quads' sums per path are a second product with a 0/1 matrix
// into the group's 16 paths.
// Layout: header kGemmHeader words (magic + 2, n_blocks, dx, dy, dout, P,
// n_klist, n_groups, off_rowtab, a_floats, off_blocks, off_klist,
// off_groups, words); blocks [nb][4]: path group t, rows (4 per quad), K
// list start, K (a multiple of 4, at most 16); K list: x components, -1 for
// padding; row table [nb][16] (16-byte aligned, after the K list):
// (P - 16 t) | (dz component + 1) << 10 per row, 0 in place of the
// component + 1 for a padding row, 16 for the rows of a missing quad;
// groups as in the other dense plans, A[k][row] at the tile's base +
// 16 k + row (the tiles' bases advance by 16 K).
e3_status build_gemm_dw(const e3_desc* desc, std::vector<int32_t>& out, e3k::TpGemmArgs& d) {
  Parsed p;
  std::vector<GenEntry> ent;
  e3_status s = generic_entries(desc, p, ent, false);
  if (s != E3_OK) return s;
  if (p.P > 32767 || p.dx > 65535 || p.dout > 65535)
    return fail(E3_ERR_UNSUPPORTED, "too many paths or components");
  std::vector<int> xoff(p.x.size()), oo_path(p.P);
  {
    std::vector<int> ooff(p.o.size());
    for (size_t i = 0, o = 0; i < p.x.size(); ++i) xoff[i] = int(o), o += 2 * p.x[i].l + 1;
    for (size_t i = 0, o = 0; i < p.o.size(); ++i) ooff[i] = int(o), o += 2 * p.o[i].l + 1;
    for (int pi = 0, opp = 0; pi < p.P; ++pi) {
      oo_path[pi] = p.per_path ? opp : ooff[p.pio[pi]];
      opp += 2 * p.o[p.pio[pi]].l + 1;
    }
  }
  for (int pi = 1; pi < p.P; ++pi)
    if (p.pix[pi] < p.pix[pi - 1]) return fail(E3_ERR_UNSUPPORTED, "paths not grouped by x irrep");
  std::vector<int32_t> blocks, klist, rowtab;
  std::vector<int> block_base;
  std::vector<std::vector<int>> tile_blocks;  // per tile: its block for each K chunk
  std::vector<std::vector<std::pair<int, int>>> path_rows(p.P);  // (P, M) -> tile, row
  for (int pi = 0; pi < p.P; ++pi) path_rows[pi].resize(size_t(2 * p.o[p.pio[pi]].l + 1));
  int abase = 0;
  for (int pa = 0; pa < p.P;) {
    int pb = pa;
    while (pb < p.P && p.pix[pb] == p.pix[pa]) ++pb;
    const int l1 = p.x[p.pix[pa]].l, width = 2 * l1 + 1;
    if (width > 64) return fail(E3_ERR_UNSUPPORTED, "an x irrep of more than 64 components");
    // K chunks of at most 16 components (degree 8: 16 + 1), each a K list
    // of its own: a tile is one block per chunk, consecutive, so the
    // chunks' partial products join the same path group's sums
    std::vector<std::pair<int, int>> chunks;  // (K list start, K)
    for (int c0 = 0; c0 < width; c0 += 16) {
      const int n = std::min(16, width - c0), K = (n + 3) / 4 * 4;
      chunks.push_back({int(klist.size()), K});
      for (int m = 0; m < K; ++m) klist.push_back(m < n ? xoff[p.pix[pa]] + c0 + m : -1);
    }
    // quads: each path's rows (P, M) in runs of four, the last one padded
    struct Quad {
      int P, M0, n;
    };
    std::vector<Quad> quads;
    for (int pi = pa; pi < pb; ++pi) {
      const int w = 2 * p.o[p.pio[pi]].l + 1;
      for (int M0 = 0; M0 < w; M0 += 4) quads.push_back(Quad{pi, M0, std::min(4, w - M0)});
    }
    // tiles: at most four quads, all of one group of 16 paths
    for (size_t q0 = 0; q0 < quads.size();) {
      const int t = quads[q0].P / 16;
      int n = 0;
      while (n < 4 && q0 + n < quads.size() && quads[q0 + n].P / 16 == t) ++n;
      const int tile = int(tile_blocks.size());
      std::vector<int32_t> rt;
      for (int j = 0; j < 4; ++j) {
        for (int i = 0; i < 4; ++i) {
          if (j >= n) {
            rt.push_back(16);  // no path, the zero row
            continue;
          }
          const Quad& qd = quads[q0 + j];
          const int rel = qd.P - 16 * t;
          if (i < qd.n) {
            const int M = qd.M0 + i;
            path_rows[qd.P][M] = {tile, 4 * j + i};
            rt.push_back(rel | ((oo_path[qd.P] + M + 1) << 10));
          } else {
            rt.push_back(rel);
          }
        }
      }
      tile_blocks.emplace_back();
      for (const auto& [kb, K] : chunks) {
        tile_blocks.back().push_back(int(blocks.size() / 4));
        block_base.push_back(abase);
        blocks.insert(blocks.end(), {t, 4 * n, kb, K});
        rowtab.insert(rowtab.end(), rt.begin(), rt.end());
        abase += 16 * K;
      }
      q0 += size_t(n);
    }
    pa = pb;
  }
  const int nb = int(blocks.size() / 4);
  std::vector<AGroupTerm> ge;
  ge.reserve(ent.size());
  for (const GenEntry& e : ent) {
    const auto [tile, r] = path_rows[e.P][size_t(e.o - oo_path[e.P])];
    const int k = e.xi - xoff[p.pix[e.P]];
    const int blk = tile_blocks[size_t(tile)][size_t(k / 16)];
    ge.push_back(AGroupTerm{block_base[size_t(blk)] + (k % 16) * 16 + r, e.yi, e.c});
  }
  std::vector<int32_t> groups;
  if ((s = a_groups(ge, groups)) != E3_OK) return s;
  d = e3k::TpGemmArgs{};
  d.n_blocks = nb;
  d.dx = p.dx;
  d.dy = p.dy;
  d.dout = p.dout;
  d.P = p.P;
  d.n_klist = int(klist.size());
  d.n_groups = int(groups.size() / 4);
  d.a_floats = std::max(abase, 4);
  d.off_blocks = e3k::kGemmHeader;
  d.off_klist = d.off_blocks + 4 * nb;
  const int off_rowtab = e3k::gemm_dw_rowtab_offset(d);
  d.off_groups = off_rowtab + 16 * nb;
  d.plan_words = d.off_groups + int(groups.size());
  out.assign(size_t(d.plan_words), 0);
  const int32_t head[14] = {e3k::kGemmMagic + 2, nb,          p.dx,         p.dy,
                            p.dout,              p.P,         d.n_klist,    d.n_groups,
                            off_rowtab,          d.a_floats,  d.off_blocks, d.off_klist,
                            d.off_groups,        d.plan_words};
  std::copy(head, head + 14, out.begin());
  std::copy(blocks.begin(), blocks.end(), out.begin() + d.off_blocks);
  std::copy(klist.begin(), klist.end(), out.begin() + d.off_klist);
  std::copy(rowtab.begin(), rowtab.end(), out.begin() + off_rowtab);
  std::copy(groups.begin(), groups.end(), out.begin() + d.off_groups);
  return ok();
}

// The gradient of y (E3_GEN_GEMM_DY): per row, the channel sums
//   G_P[M][m1] = sum_q w[P][q] dz[oo_P + M][q] x[xoff_P + m1][q]
// as matrix products with the channel sum as K, then
//   dy[yi] = sum over the CG entries (P, M, m1, yi, c) of c G_P[M][m1].
// A block is a group of paths sharing its columns: the components m1 of x
// irrep i, rows (P, M) for the paths from i with l1 >= l3 (every path with
// E3_OUT_PER_PATH); or the components M of output irrep k, rows (P, m1) for
// the paths into k with l1 < l3 -- so the 16 columns are the wider side.
// Rows are padded to a multiple of 16.  The operands come from one staged
// slab of rows: x [0, dx), w [dx, dx + P), dz [dx + P, dx + P + dout).
// Layout: header kGemmHeader words (magic + 7, n_blocks, dx, dy, dout, P,
// n_rows, n_ent, 0, 0, off_blocks, off_rows, off_yptr, words, off_yent);
// blocks [nb][4]: first column's slab row, columns, first G row, rows (x16);
// rows [n_rows]: P | (slab row of the row's own operand) << 16, -1 for
// padding; yptr [dy+1]; yent [n_ent][2]: G index (row * 16 + column),
// coefficient bits -- the entries of each y component in a fixed order.
e3_status build_gemm_dy(const e3_desc* desc, std::vector<int32_t>& out, int* dims) {
  Parsed p;
  std::vector<GenEntry> ent;
  e3_status s = generic_entries(desc, p, ent, false);
  if (s != E3_OK) return s;
  if (p.P > 32767 || p.dx + p.P + p.dout > 65535)
    return fail(E3_ERR_UNSUPPORTED, "too many paths or components");
  std::vector<int> xoff(p.x.size()), ooff(p.o.size()), oo_path(p.P);
  for (size_t i = 0, o = 0; i < p.x.size(); ++i) xoff[i] = int(o), o += 2 * p.x[i].l + 1;
  for (size_t i = 0, o = 0; i < p.o.size(); ++i) ooff[i] = int(o), o += 2 * p.o[i].l + 1;
  for (int pi = 0, opp = 0; pi < p.P; ++pi) {
    oo_path[pi] = p.per_path ? opp : ooff[p.pio[pi]];
    opp += 2 * p.o[p.pio[pi]].l + 1;
  }
  const int zrow0 = p.dx + p.P;  // slab row of dz component 0
  auto x_keyed = [&](int pi) { return p.per_path || p.x[p.pix[pi]].l >= p.o[p.pio[pi]].l; };
  std::vector<int32_t> blocks, rows;
  // path_row[c][pi]: first G row of path pi in its block's column chunk c
  // (16 columns per chunk: a block of more columns, degree 8, repeats its
  // rows once per chunk)
  std::vector<std::vector<int>> path_row(4, std::vector<int>(p.P));
  auto add_block = [&](int col_row, int ncols, auto&& member, auto&& own_row, auto&& n_own) {
    bool any = false;
    for (int pi = 0; pi < p.P; ++pi) any = any || member(pi);
    if (!any) return true;
    if (ncols > 64) return false;
    for (int c0 = 0, c = 0; c0 < ncols; c0 += 16, ++c) {
      const int r0 = int(rows.size());
      for (int pi = 0; pi < p.P; ++pi) {
        if (!member(pi)) continue;
        path_row[size_t(c)][pi] = int(rows.size());
        for (int i = 0; i < n_own(pi); ++i) rows.push_back(pi | own_row(pi, i) << 16);
      }
      while ((rows.size() - r0) % 16) rows.push_back(-1);
      blocks.insert(blocks.end(), {col_row + c0, std::min(16, ncols - c0), r0, int(rows.size()) - r0});
    }
    return true;
  };
  for (size_t i = 0; i < p.x.size(); ++i)
    if (!add_block(
            xoff[i], 2 * p.x[i].l + 1,
            [&](int pi) { return p.pix[pi] == int(i) && x_keyed(pi); },
            [&](int pi, int M) { return zrow0 + oo_path[pi] + M; },
            [&](int pi) { return 2 * p.o[p.pio[pi]].l + 1; }))
      return fail(E3_ERR_UNSUPPORTED, "an x irrep of more than 64 components");
  for (size_t k = 0; k < p.o.size(); ++k)
    if (!add_block(
            zrow0 + ooff[k], 2 * p.o[k].l + 1,
            [&](int pi) { return p.pio[pi] == int(k) && !x_keyed(pi); },
            [&](int pi, int m1) { return xoff[p.pix[pi]] + m1; },
            [&](int pi) { return 2 * p.x[p.pix[pi]].l + 1; }))
      return fail(E3_ERR_UNSUPPORTED, "an output irrep of more than 64 components");
  const int nb = int(blocks.size() / 4);
  std::vector<std::vector<std::pair<int, float>>> by_y(p.dy);
  for (const GenEntry& e : ent) {
    const int M = e.o - oo_path[e.P], m1 = e.xi - xoff[p.pix[e.P]];
    const int gi = x_keyed(e.P) ? (path_row[size_t(m1 / 16)][e.P] + M) * 16 + m1 % 16
                                : (path_row[size_t(M / 16)][e.P] + m1) * 16 + M % 16;
    by_y[e.yi].push_back({gi, e.c});
  }
  const int off_blocks = e3k::kGemmHeader, off_rows = off_blocks + 4 * nb;
  const int off_yptr = off_rows + int(rows.size());
  const int off_yent = off_yptr + p.dy + 1;
  int n_ent = 0;
  for (const auto& v : by_y) n_ent += int(v.size());
  const int words = off_yent + 2 * n_ent;
  out.assign(size_t(words), 0);
  const int32_t head[14] = {e3k::kGemmMagic + 7, nb, p.dx, p.dy, p.dout, p.P, int(rows.size()),
                            n_ent, 0, 0, off_blocks, off_rows, off_yptr, words};
  std::copy(head, head + 14, out.begin());
  out[e3k::kGemmHeader - 2] = off_yent;  // the header's last spare word
  std::copy(blocks.begin(), blocks.end(), out.begin() + off_blocks);
  std::copy(rows.begin(), rows.end(), out.begin() + off_rows);
  int k = 0;
  for (int y = 0; y < p.dy; ++y) {
    out[off_yptr + y] = k;
    for (const auto& [g, c] : by_y[y]) {
      int32_t cb;
      std::memcpy(&cb, &c, 4);
      out[off_yent + 2 * k] = g;
      out[off_yent + 2 * k + 1] = cb;
      ++k;
    }
  }
  out[off_yptr + p.dy] = k;
  if (dims) {
    dims[0] = nb;
    dims[1] = int(rows.size());
    dims[2] = n_ent;
    dims[3] = words;
  }
  return ok();
}

// The plan's sizes per descriptor, built once (the kernel takes them from
// the host, not from the caller's device copy).
std::mutex g_plan_mu;
std::map<std::string, std::pair<e3k::TpGemmArgs, size_t>> g_plan_cache;

e3_status gemm_dims(const e3_desc* desc, e3k::TpGemmArgs& d, size_t& bytes, int kind = 0) {
  std::mutex& mu = g_plan_mu;
  auto& cache = g_plan_cache;
  std::string key;
  if (!desc) return fail(E3_ERR_INVALID_ARG, "desc is null");
  for (const e3_irreps* v : {&desc->x, &desc->y, &desc->out}) {
    if (v->n < 0 || (v->n > 0 && !v->v)) return fail(E3_ERR_IRREPS, "bad irreps list");
    for (int i = 0; i < v->n; ++i)
      key += std::to_string(v->v[i].mul) + "x" + std::to_string(v->v[i].l) +
             (v->v[i].parity > 0 ? "e" : "o") + ",";
    key += "|";
  }
  key += std::to_string(desc->flags & E3_OUT_PER_PATH) + "/" + std::to_string(kind);
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = cache.find(key);
    if (it != cache.end()) {
      d = it->second.first;
      bytes = it->second.second;
      return ok();
    }
  }
  std::vector<int32_t> words;
  e3_status s = build_gemm_kind(desc, kind, words, d);
  if (s != E3_OK) return s;
  bytes = words.size() * 4;
  std::lock_guard<std::mutex> g(mu);
  cache[key] = {d, bytes};
  return ok();
}

// A dense tensor-product plan whose A fits beside the staged slabs only with
// slabs of fewer than 64 channels (degree 8: 16, one busy wavefront of
// four): 64-channel slabs with A in windows of whole blocks instead, if a
// window of at least a quarter of A (and the largest block) fits.
void tp_gemm_window(e3k::TpGemmArgs& t) {
  if (t.CS >= 64 || t.C % 64) return;
  e3k::TpGemmArgs w = t;
  w.CS = 64;
  w.a_win = 1;
  const long fixed = long(e3k::tp_gemm_lds_bytes(w)) - 4;
  const long win = (long(160) * 1024 - fixed) / 4;
  if (win < std::max<long>(t.a_block_max, t.a_floats / 4) || win >= t.a_floats) return;
  t.CS = 64;
  t.a_win = int(win);
  t.lds_bytes = e3k::tp_gemm_lds_bytes(t);
}

// The same for the dense convolution with given harmonics (its LDS adds the
// harmonic bank and the y map): 64-channel slabs with A in windows where
// all of A allows only narrower slabs.
void conv_gemm_window(e3k::TpGemmArgs& t) {
  if (t.CS >= 64 || t.C % 64) return;
  e3k::TpGemmArgs w = t;
  w.CS = 64;
  w.a_win = 1;
  const long fixed = long(e3k::tp_gemm_lds_bytes(w)) - 4 + 4L * e3k::kConvGemmExtraWords;
  const long win = (long(160) * 1024 - fixed) / 4;
  if (win < std::max<long>(t.a_block_max, t.a_floats / 4) || win >= t.a_floats) return;
  t.CS = 64;
  t.a_win = int(win);
  t.lds_bytes = e3k::tp_gemm_lds_bytes(t) + 4 * e3k::kConvGemmExtraWords;
}

e3_status build_table(const e3_desc* desc, int table, std::vector<int32_t>& out) {
  if (table == E3_GEN_GEMM || table == E3_GEN_GEMM_DX || table == E3_GEN_GEMM_DW) {
    e3k::TpGemmArgs d;
    return build_gemm_kind(desc, table == E3_GEN_GEMM ? 0 : table == E3_GEN_GEMM_DX ? 1 : 2, out,
                           d);
  }
  if (table == E3_GEN_GEMM_DY) return build_gemm_dy(desc, out, nullptr);
  return build_generic(desc, table, out);
}

}  // namespace

e3_status e3_generic_plan_size(const e3_desc* desc, int32_t table, size_t* bytes) {
  if (!bytes) return fail(E3_ERR_INVALID_ARG, "bytes is null");
  std::vector<int32_t> t;
  e3_status s = build_table(desc, table, t);
  if (s != E3_OK) return s;
  *bytes = t.size() * sizeof(int32_t);
  return ok();
}

e3_status e3_generic_plan_build(const e3_desc* desc, int32_t table, void* host_plan,
                                size_t bytes) {
  if (!host_plan) return fail(E3_ERR_INVALID_ARG, "host_plan is null");
  std::vector<int32_t> t;
  e3_status s = build_table(desc, table, t);
  if (s != E3_OK) return s;
  if (bytes < t.size() * sizeof(int32_t))
    return fail(E3_ERR_WORKSPACE, "plan needs " + std::to_string(t.size() * 4) + " bytes");
  std::memcpy(host_plan, t.data(), t.size() * sizeof(int32_t));
  return ok();
}

namespace {

e3_status generic_parse(const e3_desc* desc, e3_dtype dtype, Parsed& p) {
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  if (dtype != E3_F32 && dtype != E3_BF16) return fail(E3_ERR_INVALID_ARG, "unknown dtype");
  for (const auto* v : {&p.x, &p.y, &p.o})
    for (const auto& r : *v)
      if (r.l > kGenericLmax) return fail(E3_ERR_UNSUPPORTED, "generic tables go to degree 8");
  if (p.dx * 64 + p.dy > 4096 || p.dout * 64 + p.dy > 4096)
    return fail(E3_ERR_UNSUPPORTED, "too many components for the generic kernel (dx, dout <= 63)");
  return ok();
}

e3_status generic_table_ok(const void* plan, size_t bytes, const GenDims& dm) {
  const size_t min_words = size_t(e3k::kGenHeader) + dm.keys + 1;
  if (!plan || bytes < min_words * sizeof(int32_t) || (bytes % 4) != 0)
    return fail(E3_ERR_WORKSPACE, "plan is missing or too short for this descriptor");
  if (!aligned16(plan)) return fail(E3_ERR_ALIGNMENT, "plan must be 16-byte aligned");
  return ok();
}

}  // namespace

e3_status e3_tp_forward_generic(const e3_desc* desc, int64_t n_rows, const void* plan,
                                size_t plan_bytes, const void* x, const float* y, const void* w,
                                void* z, e3_dtype dtype, void* stream) {
  Parsed p;
  e3_status s = generic_parse(desc, dtype, p);
  if (s != E3_OK) return s;
  if (n_rows < 0) return fail(E3_ERR_INVALID_ARG, "n_rows < 0");
  if (n_rows == 0) return ok();
  if (!x || !y || !w || !z) return fail(E3_ERR_INVALID_ARG, "null pointer");
  const GenDims dm = generic_dims(p, E3_GEN_FORWARD);
  if ((s = generic_table_ok(plan, plan_bytes, dm)) != E3_OK) return s;
  e3k::GenericTpArgs a{n_rows, p.C, dm.operand, dm.y, dm.keys, dm.weights,
                       static_cast<const int*>(plan), int64_t(plan_bytes / 4), x, y, w, z};
  return hip_status(e3k::launch_tp_generic(a, dtype == E3_BF16, hipStream_t(stream)),
                    "tp_forward_generic");
}

e3_status e3_tp_forward_gemm(const e3_desc* desc, int64_t n_rows, const void* plan,
                             size_t plan_bytes, const float* x, const float* y, const float* w,
                             float* z, void* stream) {
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  e3k::TpGemmArgs a;
  size_t need = 0;
  if ((s = gemm_dims(desc, a, need)) != E3_OK) return s;
  if (p.C % 16) return fail(E3_ERR_UNSUPPORTED, "the dense-product kernel needs C % 16 == 0");
  if (n_rows < 0) return fail(E3_ERR_INVALID_ARG, "n_rows < 0");
  if (n_rows == 0) return ok();
  if (!plan || plan_bytes < need)
    return fail(E3_ERR_INVALID_ARG, "plan needs " + std::to_string(need) +
                                        " bytes (E3_GEN_GEMM table of this descriptor)");
  if (!x || !y || !w || !z) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(x) || !aligned16(w) || !aligned16(plan))
    return fail(E3_ERR_ALIGNMENT, "x, w and the plan must be 16-byte aligned");
  a.n_rows = n_rows;
  a.C = p.C;
  // the widest channel slab with two workgroups per CU, else with one
  a.CS = 0;
  for (size_t cap : {size_t(80) * 1024, size_t(160) * 1024}) {
    for (int cs : {128, 64, 32, 16}) {
      if (cs > p.C || p.C % cs) continue;
      a.CS = cs;
      if (e3k::tp_gemm_lds_bytes(a) <= cap) break;
      a.CS = 0;
    }
    if (a.CS) break;
  }
  tp_gemm_window(a);
  if (!a.CS) return fail(E3_ERR_UNSUPPORTED, "the dense-product plan does not fit in LDS");
  if ((a.P + 1) * e3k::gemm_row_stride(a.CS) > 65535 || a.dx * e3k::gemm_row_stride(a.CS) > 65535)
    return fail(E3_ERR_UNSUPPORTED, "too many x components or paths for the dense-product kernel");
  a.lds_bytes = e3k::tp_gemm_lds_bytes(a);
  a.plan = static_cast<const int*>(plan);
  a.x = x;
  a.y = y;
  a.w = w;
  a.z = z;
  return hip_status(e3k::launch_tp_gemm(a, hipStream_t(stream)), "tp_forward_gemm");
}

}  // extern "C"

namespace {

// Sizes of the dense backward's dy plan per descriptor (built once).
struct DyDims {
  int n_blocks, n_grows, n_ent, words, off_rows, off_yptr, off_yent;
};
std::map<std::string, DyDims> g_dy_cache;

e3_status gemm_dy_dims(const e3_desc* desc, DyDims& d) {
  std::string key;
  for (const e3_irreps* v : {&desc->x, &desc->y, &desc->out}) {
    if (v->n < 0 || (v->n > 0 && !v->v)) return fail(E3_ERR_IRREPS, "bad irreps list");
    for (int i = 0; i < v->n; ++i)
      key += std::to_string(v->v[i].mul) + "x" + std::to_string(v->v[i].l) +
             (v->v[i].parity > 0 ? "e" : "o") + ",";
    key += "|";
  }
  key += std::to_string(desc->flags & E3_OUT_PER_PATH);
  {
    std::lock_guard<std::mutex> g(g_plan_mu);
    auto it = g_dy_cache.find(key);
    if (it != g_dy_cache.end()) {
      d = it->second;
      return ok();
    }
  }
  std::vector<int32_t> words;
  int dims[4];
  e3_status s = build_gemm_dy(desc, words, dims);
  if (s != E3_OK) return s;
  d = DyDims{dims[0], dims[1], dims[2], dims[3], words[11], words[12], words[14]};
  std::lock_guard<std::mutex> g(g_plan_mu);
  g_dy_cache[key] = d;
  return ok();
}

// Widest channel slab (CS | C, CS <= 128) whose LDS leaves two workgroups per
// CU, else one; 0 when none fits.
template <class F>
int pick_slab(int C, F lds_of, bool widest = false) {
  for (size_t cap : {size_t(80) * 1024, size_t(160) * 1024}) {
    if (widest && cap < 160 * 1024) continue;
    for (int cs : {128, 64, 32, 16})
      if (cs <= C && C % cs == 0 && lds_of(cs) <= cap) return cs;
  }
  return 0;
}

// The three plans of the dense backward checked against the descriptor and
// set up: dx (TpGemmArgs on dz), dw and dy (GemmBwdArgs).
e3_status gemm_backward_setup(const e3_desc* desc, const Parsed& p, const void* plan_dx,
                              size_t dx_bytes, const void* plan_dw, size_t dw_bytes,
                              const void* plan_dy, size_t dy_bytes, e3k::TpGemmArgs& tdx,
                              e3k::GemmBwdArgs& bdw, e3k::GemmBwdArgs& bdy) {
  e3_status s;
  size_t need_dx = 0, need_dw = 0;
  if ((s = gemm_dims(desc, tdx, need_dx, 1)) != E3_OK) return s;
  bdw = e3k::GemmBwdArgs{};
  if ((s = gemm_dims(desc, bdw.t, need_dw, 2)) != E3_OK) return s;
  DyDims dd;
  if ((s = gemm_dy_dims(desc, dd)) != E3_OK) return s;
  if (p.C % 16) return fail(E3_ERR_UNSUPPORTED, "the dense-product kernels need C % 16 == 0");
  if (!plan_dx || dx_bytes < need_dx || !plan_dw || dw_bytes < need_dw || !plan_dy ||
      dy_bytes < size_t(dd.words) * 4)
    return fail(E3_ERR_INVALID_ARG,
                "plans need " + std::to_string(need_dx) + ", " + std::to_string(need_dw) + " and " +
                    std::to_string(size_t(dd.words) * 4) +
                    " bytes (tables E3_GEN_GEMM_DX, _DW, _DY of this descriptor)");
  if (!aligned16(plan_dx) || !aligned16(plan_dw) || !aligned16(plan_dy))
    return fail(E3_ERR_ALIGNMENT, "the plans must be 16-byte aligned");
  tdx.C = bdw.t.C = p.C;
  tdx.CS = pick_slab(p.C, [&](int cs) {
    e3k::TpGemmArgs t = tdx;
    t.CS = cs;
    return e3k::tp_gemm_lds_bytes(t);
  });
  // dw: the widest slab (A is built once per slab; the workgroup has a
  // wavefront per 16 channels)
  bdw.a_win = 0;
  bdw.t.CS = pick_slab(p.C, [&](int cs) {
    e3k::TpGemmArgs t = bdw.t;
    t.CS = cs;
    return e3k::gemm_dw_lds_bytes(t);
  }, true);
  if (bdw.t.CS < std::min(64, p.C)) {
    // A fits beside the dz slab only with narrow slabs, if at all (degree
    // 8: a 16-channel slab, one wavefront per CU): the widest slab of 64 or
    // more channels whose LDS leaves a window of at least a quarter of A,
    // the tiles walked in windows of whole tiles with A built per window
    for (int cs : {128, 64}) {
      if (cs > p.C || p.C % cs) continue;
      e3k::TpGemmArgs t = bdw.t;
      t.CS = cs;
      const long fixed = long(e3k::gemm_dw_lds_bytes(t, 4)) - 4 * 4;
      const long win = ((long(160) * 1024 - fixed) / 4) & ~3L;
      if (win >= std::max<long>(256, bdw.t.a_floats / 4)) {
        bdw.t.CS = cs;
        bdw.a_win = int(std::min<long>(win, bdw.t.a_floats));
        break;
      }
    }
  }
  bdy = e3k::GemmBwdArgs{};
  bdy.t.n_blocks = dd.n_blocks;
  bdy.t.dx = p.dx;
  bdy.t.dy = p.dy;
  bdy.t.dout = p.dout;
  bdy.t.P = p.P;
  bdy.t.C = p.C;
  bdy.t.off_blocks = e3k::kGemmHeader;
  bdy.n_grows = dd.n_grows;
  bdy.n_ent = dd.n_ent;
  bdy.off_rows = dd.off_rows;
  bdy.off_yptr = dd.off_yptr;
  bdy.off_yent = dd.off_yent;
  bdy.g_rows = std::max(16, dd.n_grows);  // all of G at once if it fits
  bdy.t.CS = pick_slab(p.C, [&](int cs) {
    e3k::GemmBwdArgs t = bdy;
    t.t.CS = cs;
    return e3k::gemm_dy_lds_bytes(t);
  });
  if (!bdy.t.CS && p.C % 16 == 0) {
    // 16-channel slabs and G in groups of as many rows as fit (degree 8):
    // the slabs are staged once per group
    e3k::GemmBwdArgs t = bdy;
    t.t.CS = 16;
    t.g_rows = 16;
    const long fixed = long(e3k::gemm_dy_lds_bytes(t)) - 16 * 16 * 4;
    const long rows = (long(160) * 1024 - fixed) / (16 * 4) / 16 * 16;
    if (rows >= 16) {
      bdy.t.CS = 16;
      bdy.g_rows = int(std::max<long>(16, std::min<long>(rows, dd.n_grows)));
    }
  }
  if (!tdx.CS || !bdw.t.CS || !bdy.t.CS)
    return fail(E3_ERR_UNSUPPORTED, "a dense-product backward plan does not fit in LDS");
  const int XS = e3k::gemm_row_stride(std::max(tdx.CS, bdw.t.CS));
  if ((p.P + 1) * XS > 65535 || std::max(p.dx, p.dout) * XS > 65535)
    return fail(E3_ERR_UNSUPPORTED, "too many components or paths for the dense-product kernels");
  tdx.lds_bytes = e3k::tp_gemm_lds_bytes(tdx);
  bdw.t.lds_bytes = e3k::gemm_dw_lds_bytes(bdw.t, bdw.a_win);
  bdy.t.lds_bytes = e3k::gemm_dy_lds_bytes(bdy);
  tdx.plan = static_cast<const int*>(plan_dx);
  bdw.t.plan = static_cast<const int*>(plan_dw);
  bdy.t.plan = static_cast<const int*>(plan_dy);
  return E3_OK;
}

}  // namespace

extern "C" {

e3_status e3_tp_backward_gemm(const e3_desc* desc, int64_t n_rows, const void* plan_dx,
                              size_t dx_bytes, const void* plan_dw, size_t dw_bytes,
                              const void* plan_dy, size_t dy_bytes, const float* x, const float* y,
                              const float* w, const float* dz, float* dx, float* dw, float* dy,
                              void* stream) {
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  e3k::TpGemmArgs tdx;
  e3k::GemmBwdArgs bdw, bdy;
  if ((s = gemm_backward_setup(desc, p, plan_dx, dx_bytes, plan_dw, dw_bytes, plan_dy, dy_bytes,
                               tdx, bdw, bdy)) != E3_OK)
    return s;
  if (n_rows < 0) return fail(E3_ERR_INVALID_ARG, "n_rows < 0");
  if (n_rows > INT32_MAX) return fail(E3_ERR_UNSUPPORTED, "more than 2^31 - 1 rows");
  if (n_rows == 0) return ok();
  if (!x || !y || !w || !dz || !dx || !dw || !dy) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(x) || !aligned16(w) || !aligned16(dz))
    return fail(E3_ERR_ALIGNMENT, "x, w and dz must be 16-byte aligned");
  const hipStream_t st = hipStream_t(stream);
  // dx: the forward's product with the roles of x and the output swapped
  tp_gemm_window(tdx);
  if ((tdx.P + 1) * e3k::gemm_row_stride(tdx.CS) > 65535 ||
      tdx.dx * e3k::gemm_row_stride(tdx.CS) > 65535)
    return fail(E3_ERR_UNSUPPORTED, "too many components or paths for the dense-product kernels");
  tdx.n_rows = n_rows;
  tdx.x = dz;
  tdx.y = y;
  tdx.w = w;
  tdx.z = dx;
  if ((s = hip_status(e3k::launch_tp_gemm(tdx, st), "tp_backward_gemm")) != E3_OK) return s;
  for (e3k::GemmBwdArgs* b : {&bdw, &bdy}) {
    b->t.n_rows = n_rows;
    b->t.x = x;
    b->t.y = y;
    b->t.w = w;
    b->dz = dz;
    b->n_x = int(n_rows);
    b->n_zrows = b->n_x;
  }
  bdw.out = dw;
  bdy.out = dy;
  if ((s = hip_status(e3k::launch_gemm_dw(bdw, st), "tp_backward_gemm")) != E3_OK) return s;
  return hip_status(e3k::launch_gemm_dy(bdy, st), "tp_backward_gemm");
}

e3_status e3_conv_backward_gemm(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                const int32_t* rowptr, const int32_t* sender,
                                const void* workspace, size_t ws_bytes, const void* plan_dx,
                                size_t dx_bytes, const void* plan_dw, size_t dw_bytes,
                                const void* plan_dy, size_t dy_bytes, const float* Y,
                                const float* x, const float* w, const float* dm, float* dx,
                                float* dw, float* dY, void* stream) {
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  if (!(desc->flags & E3_Y_GIVEN))
    return fail(E3_ERR_UNSUPPORTED,
                "the dense-product backward takes given harmonics (E3_Y_GIVEN); form them with "
                "e3_spherical_harmonics and chain dY with e3_spherical_harmonics_backward");
  if (p.per_path) return fail(E3_ERR_UNSUPPORTED, "the dense-product convolution has collapsed outputs");
  e3k::TpGemmArgs tdx;
  e3k::GemmBwdArgs bdw, bdy;
  if ((s = gemm_backward_setup(desc, p, plan_dx, dx_bytes, plan_dw, dw_bytes, plan_dy, dy_bytes,
                               tdx, bdw, bdy)) != E3_OK)
    return s;
  if (tdx.n_blocks > e3k::kConvGemmMaxBlocks)
    return fail(E3_ERR_UNSUPPORTED, "more than 10 x blocks (x irreps, degree 8 counting twice)");
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  if (n_nodes == 0) return ok();
  if ((s = maybe_check(desc, n_nodes, n_edges, rowptr, sender, stream)) != E3_OK) return s;
  size_t need = 0;
  e3_conv_workspace_size(n_nodes, n_edges, &need);
  if (!workspace || ws_bytes < need)
    return fail(E3_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
  if (!rowptr || !x || !dm || !dx) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (n_edges > 0 && (!sender || !Y || !w || !dw || !dY))
    return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (!aligned16(x) || !aligned16(dm) || (n_edges > 0 && !aligned16(w)))
    return fail(E3_ERR_ALIGNMENT, "x, w and dm must be 16-byte aligned");
  if (tdx.CS > 64) {  // the convolution's dense kernel keeps one 16-channel tile per wavefront
    tdx.CS = 64;
    tdx.lds_bytes = e3k::tp_gemm_lds_bytes(tdx) + 4 * e3k::kConvGemmExtraWords;
  } else {
    tdx.lds_bytes += 4 * e3k::kConvGemmExtraWords;
  }
  conv_gemm_window(tdx);
  if (p.C % tdx.CS || tdx.lds_bytes > 160 * 1024)
    return fail(E3_ERR_UNSUPPORTED, "the dense-product plan does not fit in LDS");
  if ((tdx.P + 1) * e3k::gemm_row_stride(tdx.CS) > 65535 ||
      tdx.dx * e3k::gemm_row_stride(tdx.CS) > 65535)
    return fail(E3_ERR_UNSUPPORTED, "too many components or paths for the dense-product kernels");
  const e3k::TransposeLayout L = e3k::transpose_layout(n_nodes, n_edges);
  const int* ws = static_cast<const int*>(workspace);
  const hipStream_t st = hipStream_t(stream);
  // dx: per sender over its out-edges (the transposed index), operand dm
  e3k::ConvGemmArgs a{};
  a.t = tdx;
  a.t.x = dm;
  a.t.y = Y;
  a.t.w = w;
  a.t.z = dx;
  a.n_nodes = n_nodes;
  a.n_edges = n_edges;
  a.rowptr = ws + L.colptr;
  a.sender = ws + L.recv;
  a.perm = ws + L.perm;
  a.m = dx;
  a.ly = -1;
  std::memset(&a.ym, 0xff, sizeof a.ym);
  if ((s = hip_status(e3k::launch_conv_gemm(a, st), "conv_backward_gemm")) != E3_OK) return s;
  if (n_edges == 0) return ok();
  for (e3k::GemmBwdArgs* b : {&bdw, &bdy}) {
    b->t.n_rows = n_edges;
    b->t.x = x;
    b->t.y = Y;
    b->t.w = w;
    b->dz = dm;
    b->xrow = sender;
    b->rowptr = rowptr;
    b->n_x = n_nodes;
    b->n_zrows = n_nodes;
  }
  bdw.out = dw;
  bdy.out = dY;
  if ((s = hip_status(e3k::launch_gemm_dw(bdw, st), "conv_backward_gemm")) != E3_OK) return s;
  return hip_status(e3k::launch_gemm_dy(bdy, st), "conv_backward_gemm");
}

e3_status e3_conv_forward_gemm(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                               const int32_t* rowptr, const int32_t* sender, const void* plan,
                               size_t plan_bytes, const float* edge_vec_or_Y, const float* x,
                               const float* w, float* m, void* stream) {
  const float* Y = edge_vec_or_Y;
  Parsed p;
  e3_status s = parse(desc, p);
  if (s != E3_OK) return s;
  if (p.per_path) return fail(E3_ERR_UNSUPPORTED, "the dense-product convolution has collapsed outputs");
  e3k::ConvGemmArgs a{};
  size_t need = 0;
  if ((s = gemm_dims(desc, a.t, need)) != E3_OK) return s;
  if (a.t.n_blocks > e3k::kConvGemmMaxBlocks)
    return fail(E3_ERR_UNSUPPORTED,
                "more than 10 output blocks (output irreps, degree 8 counting twice)");
  // the y operand: given rows, or the harmonics of the edge vectors (one bank
  // per y irrep, y component -> harmonic l*l + m)
  a.ly = -1;
  std::memset(&a.ym, 0xff, sizeof a.ym);
  if (!(desc->flags & E3_Y_GIVEN)) {
    if (p.dy > 64)
      return fail(E3_ERR_UNSUPPORTED, "harmonics from edge vectors need dy <= 64; use E3_Y_GIVEN");
    int i = 0;
    a.ly = 0;
    for (const auto& r : p.y) {
      a.ly = std::max(a.ly, r.l);
      for (int m = 0; m < 2 * r.l + 1; ++m) a.ym.idx[i++] = static_cast<signed char>(r.l * r.l + m);
    }
    if (a.ly > 7)  // the per-edge bank holds degrees 0..7 (64 values)
      return fail(E3_ERR_UNSUPPORTED,
                  "harmonics from edge vectors go to degree 7 here; use E3_Y_GIVEN");
  }
  if (p.C % 16) return fail(E3_ERR_UNSUPPORTED, "the dense-product kernel needs C % 16 == 0");
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  if (n_nodes == 0) return ok();
  if ((s = maybe_check(desc, n_nodes, n_edges, rowptr, sender, stream)) != E3_OK) return s;
  if (!rowptr || !x || !m) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (n_edges > 0 && (!sender || !Y || !w)) return fail(E3_ERR_INVALID_ARG, "null pointer");
  if (!plan || plan_bytes < need)
    return fail(E3_ERR_INVALID_ARG, "plan needs " + std::to_string(need) +
                                        " bytes (E3_GEN_GEMM table of this descriptor)");
  if (!aligned16(x) || (n_edges > 0 && !aligned16(w)) || !aligned16(plan))
    return fail(E3_ERR_ALIGNMENT, "x, w and the plan must be 16-byte aligned");
  a.t.C = p.C;
  // slabs of at most 64 channels (one tile per wavefront): the per-block
  // accumulators of two tiles would leave one wavefront per SIMD
  a.t.CS = 0;
  for (size_t cap : {size_t(80) * 1024, size_t(160) * 1024}) {
    for (int cs : {64, 32, 16}) {
      if (cs > p.C || p.C % cs) continue;
      a.t.CS = cs;
      if (e3k::tp_gemm_lds_bytes(a.t) + 4 * e3k::kConvGemmExtraWords <= cap) break;
      a.t.CS = 0;
    }
    if (a.t.CS) break;
  }
  if (a.ly < 0) conv_gemm_window(a.t);  // given harmonics
  if (!a.t.CS) return fail(E3_ERR_UNSUPPORTED, "the dense-product plan does not fit in LDS");
  const int XS = e3k::gemm_row_stride(a.t.CS);
  if ((a.t.P + 1) * XS > 65535 || a.t.dx * XS > 65535)
    return fail(E3_ERR_UNSUPPORTED, "too many x components or paths for the dense-product kernel");
  a.t.lds_bytes = e3k::tp_gemm_lds_bytes(a.t) + 4 * e3k::kConvGemmExtraWords;
  a.t.plan = static_cast<const int*>(plan);
  a.t.x = x;
  a.t.y = Y;  // Y [E][dy], or the edge vectors [E][3]
  a.t.w = w;
  a.t.z = m;
  a.n_nodes = n_nodes;
  a.n_edges = n_edges;
  a.rowptr = rowptr;
  a.sender = sender;
  a.m = m;
  return hip_status(e3k::launch_conv_gemm(a, hipStream_t(stream)), "conv_forward_gemm");
}

e3_status e3_tp_backward_generic(const e3_desc* desc, int64_t n_rows, const void* plan_dx,
                                 size_t dx_bytes, const void* plan_dw, size_t dw_bytes,
                                 const void* plan_dy, size_t dy_bytes, const void* x,
                                 const float* y, const void* w, const void* dz, void* dx, void* dw,
                                 float* dy, e3_dtype dtype, void* stream) {
  Parsed p;
  e3_status s = generic_parse(desc, dtype, p);
  if (s != E3_OK) return s;
  if (n_rows < 0) return fail(E3_ERR_INVALID_ARG, "n_rows < 0");
  if (n_rows > INT32_MAX) return fail(E3_ERR_UNSUPPORTED, "more than 2^31 - 1 rows");
  if (n_rows == 0) return ok();
  if (!x || !y || !w || !dz || !dx || !dw || !dy) return fail(E3_ERR_INVALID_ARG, "null pointer");
  const GenDims dyd = generic_dims(p, E3_GEN_DY), dxd = generic_dims(p, E3_GEN_DX),
                dwd = generic_dims(p, E3_GEN_DW);
  if ((s = generic_table_ok(plan_dx, dx_bytes, dxd)) != E3_OK ||
      (s = generic_table_ok(plan_dw, dw_bytes, dwd)) != E3_OK ||
      (s = generic_table_ok(plan_dy, dy_bytes, dyd)) != E3_OK)
    return s;
  const hipStream_t st = hipStream_t(stream);
  const int bf = dtype == E3_BF16;
  // dx: the dx table over dz, weights w
  e3k::GenericTpArgs ax{n_rows, p.C, dxd.operand, dxd.y, dxd.keys, dxd.weights,
                        static_cast<const int*>(plan_dx), int64_t(dx_bytes / 4), dz, y, w, dx};
  if ((s = hip_status(e3k::launch_tp_generic(ax, bf, st), "tp_backward_generic")) != E3_OK)
    return s;
  // dw: the dw table over x, with dz as the per-"path" array
  e3k::GenericTpArgs aw{n_rows, p.C, dwd.operand, dwd.y, dwd.keys, dwd.weights,
                        static_cast<const int*>(plan_dw), int64_t(dw_bytes / 4), x, y, dz, dw};
  if ((s = hip_status(e3k::launch_tp_generic(aw, bf, st), "tp_backward_generic")) != E3_OK)
    return s;
  // dy: summed over channels, from the table keyed by the y component
  e3k::GenericTpArgs ay{n_rows, p.C, p.dx, p.dy, p.dout, p.P,
                        static_cast<const int*>(plan_dy), int64_t(dy_bytes / 4), x, nullptr, w,
                        nullptr};
  return hip_status(e3k::launch_tp_generic_dy(ay, dz, dy, bf, st), "tp_backward_generic");
}

namespace {

// How the convolution gets its y operand: the given rows (E3_Y_GIVEN, ly =
// -1) or the harmonics of the edge vectors, one bank per y irrep (ly = the
// highest degree; ym maps each y component to the harmonic l*l + m).
e3_status generic_y_source(const e3_desc* desc, const Parsed& p, int& ly, e3k::YMap& ym) {
  ly = -1;
  std::memset(&ym, 0xff, sizeof ym);
  if (desc->flags & E3_Y_GIVEN) return ok();
  if (p.dy > 64)
    return fail(E3_ERR_UNSUPPORTED, "harmonics from edge vectors need dy <= 64; use E3_Y_GIVEN");
  int i = 0;
  ly = 0;
  for (const auto& r : p.y) {
    ly = std::max(ly, r.l);
    for (int m = 0; m < 2 * r.l + 1; ++m) ym.idx[i++] = static_cast<signed char>(r.l * r.l + m);
  }
  if (ly > kTableHarmonicsLmax)
    return fail(E3_ERR_UNSUPPORTED,
                "the coefficient-table convolution computes harmonics to degree 6; pass Y "
                "(E3_Y_GIVEN) or use the dense-product form");
  return ok();
}

// The graph arguments shared by both passes.
e3_status generic_graph(int32_t n_nodes, int32_t n_edges, const int32_t* rowptr,
                        const int32_t* sender, const float* yv) {
  if (n_nodes < 0 || n_edges < 0) return fail(E3_ERR_INVALID_ARG, "negative size");
  if (n_nodes > 0 && !rowptr) return fail(E3_ERR_INVALID_ARG, "rowptr is null");
  if (n_edges > 0 && (!sender || !yv)) return fail(E3_ERR_INVALID_ARG, "null pointer");
  return ok();
}

}  // namespace

e3_status e3_conv_forward_generic(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                  const int32_t* rowptr, const int32_t* sender,
                                  const void* workspace, size_t ws_bytes, const void* plan,
                                  size_t plan_bytes, const float* edge_vec_or_Y, const void* x,
                                  const void* w, void* m, e3_dtype dtype, void* stream) {
  Parsed p;
  e3_status s = generic_parse(desc, dtype, p);
  if (s != E3_OK) return s;
  int ly;
  e3k::YMap ym;
  if ((s = generic_y_source(desc, p, ly, ym)) != E3_OK) return s;
  if ((s = generic_graph(n_nodes, n_edges, rowptr, sender, edge_vec_or_Y)) != E3_OK) return s;
  if (n_nodes == 0) return ok();
  if ((s = maybe_check(desc, n_nodes, n_edges, rowptr, sender, stream)) != E3_OK) return s;
  if (!x || !m || (n_edges > 0 && !w)) return fail(E3_ERR_INVALID_ARG, "null pointer");
  const GenDims dm = generic_dims(p, E3_GEN_FORWARD);
  if ((s = generic_table_ok(plan, plan_bytes, dm)) != E3_OK) return s;
  const int* order = nullptr;
  if (workspace) {
    size_t need = 0;
    e3_conv_workspace_size(n_nodes, n_edges, &need);
    if (ws_bytes < need)
      return fail(E3_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
    order = static_cast<const int*>(workspace) + e3k::transpose_layout(n_nodes, n_edges).order;
  }
  e3k::GenericConvArgs a{n_nodes, n_edges, p.C, p.dx, p.dy, p.dout, p.P,
                         static_cast<const int*>(plan), int64_t(plan_bytes / 4), order, rowptr,
                         nullptr, sender, edge_vec_or_Y, ly, ym, x, w, m};
  return hip_status(e3k::launch_conv_generic_seg(a, dtype == E3_BF16, hipStream_t(stream)),
                    "conv_forward_generic");
}

e3_status e3_conv_backward_generic(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                   const int32_t* rowptr, const int32_t* sender,
                                   const void* workspace, size_t ws_bytes, const void* plan_dx,
                                   size_t dx_bytes, const void* plan_dw, size_t dw_bytes,
                                   const void* plan_dy, size_t dy_bytes,
                                   const float* edge_vec_or_Y, const void* x, const void* w,
                                   const void* dm, void* dx, void* dw, float* dY, e3_dtype dtype,
                                   void* stream) {
  Parsed p;
  e3_status s = generic_parse(desc, dtype, p);
  if (s != E3_OK) return s;
  int ly;
  e3k::YMap ym;
  if ((s = generic_y_source(desc, p, ly, ym)) != E3_OK) return s;
  if ((s = generic_graph(n_nodes, n_edges, rowptr, sender, edge_vec_or_Y)) != E3_OK) return s;
  if (n_nodes == 0) return ok();
  if ((s = maybe_check(desc, n_nodes, n_edges, rowptr, sender, stream)) != E3_OK) return s;
  size_t need = 0;
  e3_conv_workspace_size(n_nodes, n_edges, &need);
  if (!workspace || ws_bytes < need)
    return fail(E3_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
  if (!x || !dm || !dx || (n_edges > 0 && (!w || !dw || !dY)))
    return fail(E3_ERR_INVALID_ARG, "null pointer");
  const GenDims dxd = generic_dims(p, E3_GEN_DX), dwd = generic_dims(p, E3_GEN_DW),
                dyd = generic_dims(p, E3_GEN_DY);
  if ((s = generic_table_ok(plan_dx, dx_bytes, dxd)) != E3_OK ||
      (s = generic_table_ok(plan_dw, dw_bytes, dwd)) != E3_OK ||
      (s = generic_table_ok(plan_dy, dy_bytes, dyd)) != E3_OK)
    return s;
  const e3k::TransposeLayout L = e3k::transpose_layout(n_nodes, n_edges);
  const int* ws = static_cast<const int*>(workspace);
  const hipStream_t st = hipStream_t(stream);
  const int bf = dtype == E3_BF16;
  // dx: per sender over its out-edges (sender-ordered index), operand dm[receiver]
  e3k::GenericConvArgs ax{n_nodes, n_edges, p.C, p.dout, p.dy, p.dx, p.P,
                          static_cast<const int*>(plan_dx), int64_t(dx_bytes / 4), ws + L.order,
                          ws + L.colptr, ws + L.perm, ws + L.recv, edge_vec_or_Y, ly, ym, dm, w,
                          dx};
  if ((s = hip_status(e3k::launch_conv_generic_seg(ax, bf, st), "conv_backward_generic")) != E3_OK)
    return s;
  // dw and dY: per edge, receiver by receiver
  e3k::GenericConvEdgeArgs ae{n_nodes, n_edges, p.C, p.dx, p.dy, p.dout, p.P,
                              static_cast<const int*>(plan_dw), int64_t(dw_bytes / 4),
                              static_cast<const int*>(plan_dy), int64_t(dy_bytes / 4),
                              ws + L.order, rowptr, sender, edge_vec_or_Y, ly, ym, x, w, dm, dw,
                              dY};
  return hip_status(e3k::launch_conv_generic_edge(ae, bf, st), "conv_backward_generic");
}

e3_status e3_conv_double_backward_generic(
    const e3_desc* desc, int32_t n_nodes, int32_t n_edges, const int32_t* rowptr,
    const int32_t* sender, const void* workspace, size_t ws_bytes, const void* plan_fwd,
    size_t fwd_bytes, const void* plan_dx, size_t dx_bytes, const void* plan_dw, size_t dw_bytes,
    const void* plan_dy, size_t dy_bytes, const float* Y, const void* x, const void* w,
    const void* dm, const void* ddx, const float* ddY, const void* ddw, void* dx2, float* dY2,
    void* dw2, void* ddm, void* scratch, size_t scratch_bytes, e3_dtype dtype, void* stream) {
  Parsed p;
  e3_status s = generic_parse(desc, dtype, p);
  if (s != E3_OK) return s;
  if ((s = double_backward_checks(desc, p, n_nodes, n_edges, Y, x, w, dm, ddx, ddY, ddw, dx2, dY2,
                                  dw2, ddm, scratch, scratch_bytes, dtype)) != E3_OK ||
      n_nodes == 0)
    return s;
  if ((s = maybe_check(desc, n_nodes, n_edges, rowptr, sender, stream)) != E3_OK) return s;
  // the composed calls below run on the graph just checked
  e3_desc inner = *desc;
  inner.flags &= ~E3_CHECK;
  desc = &inner;
  auto fwd = [&](const void* xx, const float* yy, const void* ww, void* out) {
    return e3_conv_forward_generic(desc, n_nodes, n_edges, rowptr, sender, workspace, ws_bytes,
                                   plan_fwd, fwd_bytes, yy, xx, ww, out, dtype, stream);
  };
  auto bwd = [&](const void* xx, const float* yy, const void* ww, void* ox, void* ow, float* oy) {
    return e3_conv_backward_generic(desc, n_nodes, n_edges, rowptr, sender, workspace, ws_bytes,
                                    plan_dx, dx_bytes, plan_dw, dw_bytes, plan_dy, dy_bytes, yy, xx,
                                    ww, dm, ox, ow, oy, dtype, stream);
  };
  return double_backward_composed(p, n_nodes, n_edges, Y, x, w, ddx, ddY, ddw, dx2, dY2, dw2, ddm,
                                  scratch, dtype, hipStream_t(stream), fwd, bwd);
}

const char* e3_last_error(void) { return g_last_error.c_str(); }

e3_status e3_check_graph(int32_t n_nodes, int32_t n_edges, const int32_t* rowptr,
                         const int32_t* sender, void* stream) {
  const e3_status s = check_graph(n_nodes, n_edges, rowptr, sender, hipStream_t(stream));
  return s == E3_OK ? ok() : s;
}

e3_status e3_check_graph_host(int32_t n_nodes, int32_t n_edges, const int32_t* rowptr,
                              const int32_t* sender) {
  const e3_status s = check_graph_host(n_nodes, n_edges, rowptr, sender);
  return s == E3_OK ? ok() : s;
}

void e3_release_all(void) {
  std::lock_guard<std::mutex> g(g_plan_mu);
  g_plan_cache.clear();
  g_dy_cache.clear();
}

}  // extern "C"
