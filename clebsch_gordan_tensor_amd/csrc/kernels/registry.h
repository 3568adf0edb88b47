// Host-visible table of the specialised kernels: one KernelSet per irreps
// signature, holding launchers for every storage type and y mode.
#pragma once

#include <atomic>

#include <hip/hip_runtime.h>

#include <cstdint>

namespace e3k {

// Raises the dynamic-LDS limit of kernel f to `bytes` once per process: the
// flag is set only after a successful call, so a failure is returned and the
// next launch tries again.
inline hipError_t set_max_lds_once(std::atomic<bool>& done, const void* f, int bytes) {
  if (done.load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.store(true, std::memory_order_release);
  return e;
}


struct FwdArgs {
  int n_nodes, n_edges, C, G;
  const int* order;  // traversal order of the receivers, or null for 0..N-1
  const int* rowptr;
  const int* sender;
  const float* ysrc;  // edge vectors [E][3] or harmonics [E][dy]
  const void* x;
  const void* w;
  void* m;
};

struct BwdArgs {
  int n_nodes, C, G;
  const int* order;  // traversal order of the senders
  const int* colptr;
  const int* perm;
  const int* recv;
  const int* npad;
  const int* padlist;
  int64_t n_edges;
  const float* ysrc;
  const void* x;
  const void* w;
  const void* dm;
  void* dx;
  void* dw;
  float* dY;
};

struct TpArgs {
  int64_t n_rows;
  int C, G;
  const void* x;
  const float* y;
  const void* w;
  void* z;
};

struct TpBwdArgs {
  int64_t n_rows;
  int C, G;
  const void* x;
  const float* y;
  const void* w;
  const void* dz;
  void* dx;
  void* dw;
  float* dy;
};

using FwdFn = hipError_t (*)(const FwdArgs&, hipStream_t);
using BwdFn = hipError_t (*)(const BwdArgs&, hipStream_t);
using TpFn = hipError_t (*)(const TpArgs&, hipStream_t);
using TpBwdFn = hipError_t (*)(const TpBwdArgs&, hipStream_t);

struct IrSpec {
  int l, p;
};

struct KernelSet {
  const char* name;
  int nx, ny, no;
  IrSpec x[8], y[8], o[8];
  int dx, dy, dout, np;  // component and path counts of the signature
  int per_path;          // 1: one output block per path
  // [dtype: 0 f32, 1 bf16][y given][channels per lane: 0 -> 1, 1 -> 2, 2 -> 4]
  FwdFn fwd[2][2][3];
  BwdFn bwd[2][2][3];
  TpFn tp[2][3];       // [dtype][channels per lane]
  TpBwdFn tpb[2][3];
};

extern const KernelSet kSetL1;
extern const KernelSet kSetL1to3;
extern const KernelSet kSetL2to3;
extern const KernelSet kSetL3to3;
extern const KernelSet kSetL1to3All;
extern const KernelSet kSetL1PP;
extern const KernelSet kSetL1to3PP;
extern const KernelSet kSetL2to3PP;

// Prepare-transpose and harmonics launchers (prep.hip).
hipError_t launch_prepare_transpose(int n_nodes, int n_edges, const int* rowptr, const int* sender,
                                    const float* evec, int* ws, hipStream_t s);
hipError_t launch_harmonics(int lmax, int64_t n, const float* vec, float* Y, hipStream_t s);
// The fixed device scratch of the no-allocation backward: limits, its size in
// int32 words, and its address on the current device (fetched once per device).
constexpr int kNoAllocMaxNodes = 1 << 17;
constexpr int kNoAllocMaxEdges = 1 << 22;
int64_t noalloc_scratch_words();
hipError_t noalloc_scratch(int** out);
hipError_t launch_add(void* dst, const void* src, int64_t n, int bf16, hipStream_t s);

// Tensor product from a coefficient table (generic.hip); the table layout
// is documented there and built by the host (e3_generic_plan_build).
constexpr int kGenHeader = 8;
constexpr int kGenMagic = 0x31434745;
struct GenericTpArgs {
  int64_t n_rows;
  int C, dx, dy, dout, np;
  const int* prog;
  int64_t n_words;
  const void* x;
  const float* y;
  const void* w;
  void* z;
};
hipError_t launch_tp_generic(const GenericTpArgs& a, int bf16, hipStream_t s);
// dy of the generic tensor product from the table keyed by the y component
// (a.dx operand comps, a.dout dz comps, a.dy keys, a.np weight rows; a.y and
// a.z unused)
hipError_t launch_tp_generic_dy(const GenericTpArgs& a, const void* dz, float* dy, int bf16,
                                hipStream_t s);

// Harmonic index l*l + m of every y component when the convolution computes
// the harmonics of the edge vectors (dy <= 64).
struct YMap {
  signed char idx[64];
};

// Table-driven segment sum over a node's edge list: the convolution forward
// (seg = rowptr, nbr = sender, emap null) or its gradient of x (seg = colptr,
// emap = perm, nbr = recv of the sender-ordered index).
struct GenericConvArgs {
  int n_nodes, n_edges, C;
  int dop, dy, dkey, np;  // operand comps, y comps, output comps, weight rows
  const int* prog;
  int64_t n_words;
  const int* order;  // node visiting order, or null
  const int* seg;    // [n_nodes + 1]
  const int* emap;   // list position -> edge id, or null (identity)
  const int* nbr;    // list position -> neighbour node
  const float* yv;   // Y [E][dy] (ly < 0) or edge vectors [E][3]
  int ly;            // harmonics 0..ly computed from the vectors, or -1
  YMap ym;           // y component -> harmonic index (ly >= 0)
  const void* op;    // [N][dop][C]
  const void* w;     // [E][np][C]
  void* out;         // [N][dkey][C]
};
hipError_t launch_conv_generic_seg(const GenericConvArgs& a, int bf16, hipStream_t s);

// Table-driven per-edge cotangents dw [E][np][C] and dY [E][dy] of the
// convolution (dw table and dy table), receiver by receiver.
struct GenericConvEdgeArgs {
  int n_nodes, n_edges, C, dx, dy, dout, np;
  const int* dw_prog;
  int64_t dw_words;
  const int* dy_prog;
  int64_t dy_words;
  const int* order;
  const int* rowptr;
  const int* sender;
  const float* yv;
  int ly;
  YMap ym;
  const void* x;
  const void* w;
  const void* dm;
  void* dw;
  float* dY;
};
hipError_t launch_conv_generic_edge(const GenericConvEdgeArgs& a, int bf16, hipStream_t s);

// Radial edge weights and the convolution that computes them on the fly
// (radial.hip): 8 Bessel functions -> 64 SiLU units -> n_cols = P*C.
struct RadialConvArgs {
  int n_nodes, n_edges, C;
  const int* order;  // traversal order of the receivers, or null
  const int* rowptr;
  const int* sender;
  const float* vec;  // edge vectors [E][3]
  const float* x;    // [N][dx][C] float32
  const float* W1;   // [8][64]
  const float* W2;   // [64][P*C]
  float cutoff;
  float* m;          // [N][dout][C] float32
  const void* hidden = nullptr;  // the hidden layer's packed operands per edge, or null
};
bool radial_conv_supported(const char* set_name);
// The convolution backward with w formed from the hidden layer (never read
// or written): the transposed index of the prepare step, dY_part scratch of
// conv_bwd_radial_scratch_bytes (per 32-channel slab parts of dY).
struct RadialBwdArgs {
  int n_nodes, n_edges, C;
  const int* order;   // traversal order of the senders, or null
  const int* colptr;
  const int* perm;
  const int* recv;
  const int* npad;
  const int* padlist;
  const float* vec;   // edge vectors [E][3]
  const float* x;     // [N][dx][C] float32
  const float* W2;    // [64][P*C]
  const void* hidden; // the hidden layer's packed operands per edge
  const float* dm;    // [N][dout][C]
  float* dx;          // [N][dx][C]
  float* dw;          // [E][P][C]
  float* dY;          // [E][dy]
  float* dY_part;     // [C/32][E][dy]
};
size_t conv_bwd_radial_scratch_bytes(int n_edges, int C, int dy);
hipError_t launch_conv_bwd_radial(const char* set_name, const RadialBwdArgs& a, hipStream_t s);
// The radial MLP's hidden layer per edge in the fused convolution's operand
// form: [E][2 ks][4 quarters][hi, lo] fp16 x 8 (256 bytes per edge).
constexpr size_t kRadialHiddenBytes = 256;
hipError_t launch_radial_hidden(int n_edges, const float* vec, float cutoff, const float* W1,
                                void* h, hipStream_t s);
hipError_t launch_conv_fwd_radial(const char* set_name, const RadialConvArgs& a, hipStream_t s);
// hidden: the hidden layer from launch_radial_hidden, or null (formed per slab)
hipError_t launch_radial_mlp(int n_edges, int n_cols, const float* vec, float cutoff,
                             const float* W1, const float* W2, float* w, hipStream_t s,
                             const void* hidden = nullptr);
// pieces of the radial MLP's backward
constexpr int kRadialTailChunks = 4096;
// dh given as n_parts partials [n_parts][E][64] (added in part order, into
// part 0, which they overwrite); basis the per-edge basis and derivative
// [E][16] that launch_radial_dh_dw2 wrote
hipError_t launch_radial_tail(int n_edges, const float* vec, const float* W1, const float* basis,
                              float* dh, int n_parts, float* dvec, float* dW1_part,
                              float* dW1, hipStream_t s);
// The second layer's backward from dw [E][n_cols] (n_cols a multiple of
// 32), one read of dw: dh as per-slab partials dh_part [slabs][E][64]
// (slabs = radial_dw2_slabs(n_cols)) and dW2 as per-range partials part
// [ranges][64][n_cols] (add them with launch_sum_partials, which overwrites
// them).  w2s is device scratch of radial_w2_split_bytes(n_cols) bytes,
// basis of n_edges * 16 floats (written here: each edge's basis and its
// derivative, for launch_radial_tail), both 16-byte aligned.
int radial_dw2_slabs(int n_cols);
int radial_dw2_ranges(int n_edges, int n_cols);
size_t radial_w2_split_bytes(int n_cols);
hipError_t launch_radial_dh_dw2(int n_edges, int n_cols, const float* vec, float cutoff,
                                const float* W1, const float* W2, const float* dw,
                                float* dh_part, float* part, int ranges, void* w2s,
                                float* basis, hipStream_t s);
hipError_t launch_sum_partials(int n_chunks, int n, float* part, float* out, hipStream_t s);
// The tensor product as dense products per output block on the fp32 matrix
// cores (gemm.hip); sizes from the host-built plan, plan in device memory.
constexpr int kGemmHeader = 16;
constexpr int kGemmMagic = 0x4D4D4547;
struct TpGemmArgs {
  int64_t n_rows;
  int C, CS;  // channels; channel slab per workgroup (C % CS == 0, CS % 16 == 0)
  int n_blocks, dx, dy, dout, P, n_klist, n_groups, a_floats;
  int off_blocks, off_klist, off_groups, plan_words;  // word offsets in plan; its length
  const int* plan;
  const float* x;
  const float* y;
  const float* w;
  float* z;
  size_t lds_bytes;
  // the largest block's A (floats); A held in LDS in windows of whole blocks
  // of a_win floats (0: all of it; the tensor product's kernel only)
  int a_block_max = 0, a_win = 0;
};
// LDS row stride (floats) of a staged slab of CS channels: 16 (mod 32)
__host__ __device__ constexpr int gemm_row_stride(int CS) { return CS / 32 * 32 + 16 + (CS % 32 ? 32 : 0); }
size_t tp_gemm_lds_bytes(const TpGemmArgs& a);
hipError_t launch_tp_gemm(const TpGemmArgs& a, hipStream_t s);
// The convolution forward in the same form (t.n_rows unused; t.y = Y [E][dy];
// t.x = node features, t.w = edge weights; collapsed outputs, at most
// kConvGemmMaxBlocks blocks).
struct ConvGemmArgs {
  TpGemmArgs t;
  int n_nodes;
  int n_edges;
  const int* rowptr;
  const int* sender;
  const int* perm;  // edge id of CSR position j (nullptr: j); w and Y rows follow it
  float* m;
  int ly;   // -1: t.y is Y [E][dy]; else t.y is edge vectors [E][3], harmonics to degree ly
  YMap ym;  // y component -> harmonic l*l + m (ly >= 0)
};
// The dense-product backward's per-row (TP) or per-edge (convolution)
// kernels: dw (plan E3_GEN_GEMM_DW) and dy (plan E3_GEN_GEMM_DY).  Rows are
// TP rows, or edges with x gathered by sender and dz by receiver (found in
// rowptr); an edge whose sender is outside [0, n_x) gets zero outputs.
struct GemmBwdArgs {
  TpGemmArgs t;          // plan sizes (dw) and x, y, w; t.z unused
  const float* dz;       // [rows or nodes][dout][C]
  float* out;            // dw [rows][P][C] or dy [rows][dy]
  const int* xrow;       // convolution: sender of each edge (nullptr: x row = row)
  const int* rowptr;     // convolution: receiver CSR (nullptr: dz row = row)
  int n_x;               // rows of x (convolution: nodes)
  int n_zrows;           // rows of dz
  // dy plan; g_rows: G rows held in LDS at once (a multiple of 16; n_grows
  // when they all fit, else the kernel walks them in groups of g_rows)
  int n_grows, n_ent, off_rows, off_yptr, off_yent, g_rows;
  // dw plan: floats of A held in LDS at once (0: all of it; else the tiles
  // are walked in windows of whole tiles, A built per window)
  int a_win;
};
// dw plan: its row table [n_blocks][16] follows the K list, 16-byte aligned
constexpr int gemm_dw_rowtab_offset(const TpGemmArgs& a) { return (a.off_klist + a.n_klist + 3) / 4 * 4; }
size_t gemm_dw_lds_bytes(const TpGemmArgs& a, int a_win = 0);
size_t gemm_dy_lds_bytes(const GemmBwdArgs& a);
hipError_t launch_gemm_dw(const GemmBwdArgs& a, hipStream_t s);
hipError_t launch_gemm_dy(const GemmBwdArgs& a, hipStream_t s);
// LDS words the convolution adds to tp_gemm_lds_bytes: the harmonic bank and the y map
constexpr int kConvGemmExtraWords = 64 + 16;
// output blocks of the dense convolution (its per-block accumulators stay in
// registers): the irreps 0..8 once, the 17 rows of degree 8 as 16 + 1
constexpr int kConvGemmMaxBlocks = 10;
hipError_t launch_conv_gemm(const ConvGemmArgs& a, hipStream_t s);
hipError_t launch_harmonics_grad(int lmax, int64_t n, const float* vec, const float* dY,
                                 float* dvec, hipStream_t s);
hipError_t launch_edge_grad_to_nodes(int n_nodes, int n_edges, const int* rowptr,
                                     const int* sender, const int* ws, const float* g,
                                     float* dpos, hipStream_t s);

// One block pair of the per-irrep channel mixing (linear.hip): rows of x
// block [in_off, in_off + deg) times W [cin][cout] into y block
// [out_off, out_off + deg); `accumulate` adds to y, `zero` only clears the
// output block.
// With w_trans, W is read as the transpose of a [cout][cin] matrix (the
// backward's dy W^T).
struct LinearBlockArgs {
  int64_t n_rows;
  int din, dout, cin, cout, in_off, out_off, deg;
  const void* x;
  const float* W;
  void* y;
  int accumulate, zero, w_trans;
};
hipError_t launch_linear(const LinearBlockArgs& a, int bf16, hipStream_t s);

// Weight gradient of one block pair: dW [cin][cout] (+)= sum over the
// block's rows of x^T dy, through per-chunk partial sums in `part`
// (kLinDwChunks * cin * cout floats, overwritten) added in a fixed order.
constexpr int kLinDwChunks = 1024;
struct LinearDwArgs {
  int64_t n_rows;
  int din, dout, cin, cout, in_off, out_off, deg;
  const void* x;
  const void* dy;
  float* part;
  float* dW;
  int accumulate;
};
hipError_t launch_linear_dw(const LinearDwArgs& a, int bf16, hipStream_t s);

// Workspace layout of the transposed edge index (int32 words).
struct TransposeLayout {
  int64_t npad, colptr, cursor, tmp_e, tmp_b, perm, recv, padlist, order, flag, pos, key, order2,
      box, levels, cell, cell_cursor, bsum, total_words;
};
TransposeLayout transpose_layout(int64_t n_nodes, int64_t n_edges);

}  // namespace e3k
