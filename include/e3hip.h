/*
 * e3hip.h -- C ABI of the MI355X (gfx950) fused equivariant convolution.
 *
 * The library computes, on one AMD GPU, the hot path of E(3)-equivariant
 * message passing described in "e3j: An Efficient and Open-Source Backend for
 * Euclidean Equivariant Operations on GPU and TPU" (arXiv html version):
 *
 *   harmonics of edge vectors            (A.3 Eq.4, G.1)
 *   channel-wise Clebsch-Gordan product  (A.3 Eq.6, E.1 Eq.10)
 *   per-edge, per-path scalar weighting  (E.1 Eq.11)
 *   receiver segment sum                 (A.3 Eq.7, E.1 Eq.12-13)
 *   its vector-Jacobian product          (E.1 Eq.16)
 *
 * and the chain from the harmonic cotangent to per-atom position gradients
 * (conservative forces F = -dE/dpos, "Ab Initio Accuracy Beyond the Cutoff:
 * Distributed Message-Passing Equivariant Attention at Tens-of-Millions-of-
 * Atom Scale", cited as Tessera, 2.2 Eq.3).
 *
 * Conventions
 *   - An irreps list is a sequence of (l, parity) blocks; a block of degree l
 *     has 2l+1 components ordered m = -l..l.  Every x and output block has the
 *     same multiplicity C (channel-wise product); y has multiplicity 1.
 *   - Harmonics are real and component-normalised: sum_m Y_lm(r)^2 = 2l+1,
 *     with Y_1 = sqrt(3) (y, z, x) / |r|.
 *   - Coupling coefficients: Condon-Shortley CG moved to the real harmonic
 *     basis (a real block for l1+l2+L even, the imaginary part for odd).
 *   - Paths: for every x block, then every y block, then every output block,
 *     keep (x, y, out) when |l_x - l_y| <= l_out <= l_x + l_y and
 *     p_x p_y = p_out (parity rule, B.1).  Each path has its own weight per
 *     edge and channel; paths landing on the same output block are summed
 *     after weighting ("collapsed" output, one copy of each output block).
 *   - Layouts (row-major, channels innermost):
 *       x, dx      [rows][dx][C]       (dx = sum over x blocks of 2l+1)
 *       w, dw      [rows][P][C]        (P paths in the order above)
 *       m, dm, z   [rows][dout][C]
 *       y, Y, dY   [rows][dy]          (float32 always)
 *       edge_vec   [E][3]              (float32, r_e = pos[receiver] - pos[sender])
 *   - Graph: CSR by receiver.  rowptr[N+1] (rowptr[0] = 0, non-decreasing,
 *     rowptr[N] = E); sender[E]; edges of receiver b are
 *     rowptr[b] .. rowptr[b+1]-1.  A sender outside [0, N) marks a padding
 *     edge (the e3j paper, 3.1.2): it contributes nothing and its dw and dY
 *     are zero.
 *
 * Memory and streams
 *   - Every array argument is a DEVICE pointer unless stated otherwise; the
 *     caller owns all of them.  x, w, m, dm, dx, dw must be 16-byte aligned.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronise the host.  No call allocates device
 *     memory; the backward pass takes its index from a caller-owned workspace.
 *   - Outputs are fully overwritten; inputs are never modified.
 *   - Results are bitwise reproducible for the same inputs and device (no
 *     floating-point atomics).
 *
 * Errors
 *   - Every entry point returns an e3_status; E3_OK is 0.  On failure
 *     nothing is launched and e3_last_error() describes the problem.
 *     HIP launch errors come back as E3_ERR_HIP.
 *   - Supported signatures (irreps triples) are reported by e3_supported().
 */
#ifndef E3HIP_H
#define E3HIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  E3_OK = 0,
  E3_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad lmax */
  E3_ERR_IRREPS = -2,      /* malformed irreps (l < 0, parity not +-1, mixed multiplicities) */
  E3_ERR_UNSUPPORTED = -3, /* signature or channel count without a kernel */
  E3_ERR_ALIGNMENT = -4,   /* feature pointer not 16-byte aligned */
  E3_ERR_GRAPH = -5,       /* malformed CSR graph (found by E3_CHECK / e3_check_graph) */
  E3_ERR_WORKSPACE = -6,   /* workspace missing or too small */
  E3_ERR_HIP = -7          /* the HIP runtime reported an error */
} e3_status;

typedef enum { E3_F32 = 0, E3_BF16 = 1 } e3_dtype; /* storage; arithmetic is fp32 */

typedef struct {
  int32_t mul;    /* multiplicity (channels); 1 for y */
  int32_t l;      /* degree */
  int32_t parity; /* +1 even, -1 odd */
} e3_irrep;

typedef struct {
  int32_t n;          /* number of blocks */
  const e3_irrep* v;  /* HOST pointer to n blocks */
} e3_irreps;

enum {
  E3_Y_GIVEN = 1,      /* conv: edge_vec_or_Y holds harmonics Y[E][dy], not vectors */
  E3_OUT_PER_PATH = 2, /* one output block per path, in path order, instead of one
                          per output irrep (e3j's default layout; A.3, E.1):
                          m, dm, z, dz become [rows][sum over paths of 2L+1][C],
                          `out` still lists the irreps paths may land on */
  E3_CHECK = 4         /* debug: every convolution call first checks the graph as
                          e3_check_graph does (rowptr and sender are then required,
                          also by the backward) and returns E3_ERR_GRAPH, launching
                          nothing, when it is malformed.  The check copies rowptr
                          and sender to the host after the work queued on `stream`,
                          so such a call synchronises the host with that stream */
};

typedef struct {
  e3_irreps x, y, out;
  int32_t flags;
} e3_desc;

/* Checks a receiver-sorted CSR graph (the padding edges of e3j 3.1.2 marked
 * by sender -1): rowptr[0] = 0, rowptr non-decreasing, rowptr[N] = E and
 * every sender in [-1, N).  rowptr [N+1] and sender [E] are device arrays;
 * they are copied to the host on `stream` after the work already queued
 * there, so the call synchronises the host with that stream (debug use).
 * Returns E3_OK, E3_ERR_GRAPH (e3_last_error names the first violation),
 * E3_ERR_INVALID_ARG or E3_ERR_HIP. */
e3_status e3_check_graph(int32_t n_nodes, int32_t n_edges, const int32_t* rowptr,
                         const int32_t* sender, void* stream);
/* The same checks on HOST arrays rowptr [N+1] and sender [E] (no GPU work). */
e3_status e3_check_graph_host(int32_t n_nodes, int32_t n_edges, const int32_t* rowptr,
                              const int32_t* sender);

/* Frees the library's host-side cache (the dense-product plans' sizes per
 * descriptor; the library holds no device memory of its own).  Later calls
 * rebuild what they need.  Must not run concurrently with other calls. */
void e3_release_all(void);

/* Number of paths P of a descriptor (host only, no GPU work). */
e3_status e3_num_paths(const e3_desc* desc, int32_t* n_paths);

/* Indices into x, y, out of path i (host only). */
e3_status e3_path_info(const e3_desc* desc, int32_t i, int32_t* ix, int32_t* iy, int32_t* iout);

/* 1 if the descriptor, storage type and channel count have convolution
 * kernels: the irreps triple must be one of the specialised signatures
 * (x 0e+1o, 0e+1o+2e or 0e+1o+2e+3o; y the harmonic bank 0e+1o or
 * 0e+1o+2e+3o; out 0e+1o or 0e+1o+2e+3o; also x 0e+1o with out
 * 0e+1o+1e+2e+2o+3o+3e, pseudotensors included; with E3_OUT_PER_PATH the triples
 * 0e+1o / Y<=1 / 0e+1o, 0e+1o / Y<=3 / 0e+1o+2e+3o and
 * 0e+1o+2e / Y<=3 / 0e+1o+2e+3o) and C a power of two with 1 <= C <= 256.
 * The tensor-product calls accept the same. */
int32_t e3_supported(const e3_desc* desc, e3_dtype dtype);

/* Real coupling block T[M][m1][m2] of (l1, l2, L), l <= 7, written to the
 * HOST array out[(2L+1)(2l1+1)(2l2+1)] (the blocks the kernels' tables are
 * built from; e3j G.2 construction). */
e3_status e3_cg_block(int32_t l1, int32_t l2, int32_t L, double* out);

/* Harmonics Y[n][(lmax+1)^2] of vec[n][3] (e3j A.3 Eq.4), lmax <= 7: degrees
 * 0..3 from their closed forms, 4..7 by the coupling of Y_1 and Y_{L-1}
 * (Gaunt relation; recursion records generated and checked at build time). */
e3_status e3_spherical_harmonics(int32_t lmax, int64_t n, const float* vec, float* Y,
                                 void* stream);

/* Batched channel-wise tensor product (e3j E.1 Eq.10-11) over n_rows
 * independent rows:  z[r] = sum_P w[r][P] (x[r] (x) y[r])_P.
 * x [n][dx][C], y [n][dy] float32, w [n][P][C], z [n][dout][C]. */
e3_status e3_tp_forward(const e3_desc* desc, int64_t n_rows, const void* x, const float* y,
                        const void* w, void* z, e3_dtype dtype, void* stream);

/* Batched tensor-product backward (e3j E.1 Eq.14-16, with one scalar per
 * path as in Eq.11): for the cotangent dz [n][dout][C] of z,
 *   dx[r] = sum_P w[r][P] (y[r] (x)^T dz[r])_P            [n][dx][C]
 *   dw[r][P] = sum_M (x[r] (x) y[r])_P[M] dz[r][M]        [n][P][C]
 *   dy[r] = sum_channels sum_P w[r][P] (x[r] (x)^T dz[r])_P  [n][dy] float32
 * One pass per row; dx, dw, dy are overwritten.  x, w, dz, dx, dw must be
 * 16-byte aligned.  The signatures and channel counts of e3_supported. */
e3_status e3_tp_backward(const e3_desc* desc, int64_t n_rows, const void* x, const float* y,
                         const void* w, const void* dz, void* dx, void* dw, float* dy,
                         e3_dtype dtype, void* stream);

/* Gradient of the harmonics with respect to the vectors (chain rule from
 * the harmonic cotangent to the edge vector, toward conservative forces,
 * Tessera 2.2 Eq.3):
 *   dvec[i][k] = sum_j dY[i][j] dY_j(vec[i]) / dvec[i][k],
 * dY [n][(lmax+1)^2], vec and dvec [n][3], float32, lmax <= 7.  Since the
 * harmonics depend on the direction only, dvec is orthogonal to vec; a zero
 * vector gets 0.  Feed it the dY of e3_conv_backward. */
e3_status e3_spherical_harmonics_backward(int32_t lmax, int64_t n, const float* vec,
                                          const float* dY, float* dvec, void* stream);

/* Double backward of the convolution (e3j E.1 Eq.17-18) in the
 * given-harmonics form (desc->flags must hold E3_Y_GIVEN): for variations
 * ddx [N][dx][C], ddY [E][dy], ddw [E][P][C] of the backward's outputs, the
 * variations of its inputs
 *   ddm = conv(ddx, Y, w) + conv(x, ddY, w) + conv(x, Y, ddw)     [N][dout][C]
 *   dx2 = dx of conv_bwd(x, ddY, w, dm) + dx of conv_bwd(x, Y, ddw, dm)
 *   dY2 = dY of conv_bwd(ddx, Y, w, dm) + dY of conv_bwd(x, Y, ddw, dm)
 *   dw2 = dw of conv_bwd(ddx, Y, w, dm) + dw of conv_bwd(x, ddY, w, dm)
 * composed from the forward and backward kernels (three each) and additions.
 * workspace: from e3_conv_prepare_transpose; scratch: caller-owned,
 * e3_conv_double_backward_scratch_size bytes, 16-byte aligned.  Storage
 * type and alignment as for e3_conv_backward; Y, ddY, dY2 float32. */
e3_status e3_conv_double_backward_scratch_size(const e3_desc* desc, int32_t n_nodes,
                                               int32_t n_edges, e3_dtype dtype, size_t* bytes);
e3_status e3_conv_double_backward(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                  const int32_t* rowptr, const int32_t* sender,
                                  const void* workspace, size_t ws_bytes, const float* Y,
                                  const void* x, const void* w, const void* dm, const void* ddx,
                                  const float* ddY, const void* ddw, void* dx2, float* dY2,
                                  void* dw2, void* ddm, void* scratch, size_t scratch_bytes,
                                  e3_dtype dtype, void* stream);

/* Radial edge weights.  The e3j paper (A.3, the edge scalars s_ab of Eq.7;
 * E.1, message weighting with edge scalars) derives the per-edge weights
 * from an MLP on a radial basis embedding of |r_ab|, with 8 basis functions
 * in its model table (Table 3); the rest is this library's reading:
 *   B_n(d) = sqrt(2/cutoff) sin(n pi d / cutoff) / d   (n = 1..8; limit at d = 0)
 *   h_k    = silu(sum_n B_n(|r_e|) W1[n][k])           (k < 64; silu(t) = t/(1+e^-t))
 *   w[e][j] = sum_k h_k W2[k][j]                       (j < n_cols)
 * No envelope, no biases.  W1 [8][64] and W2 [64][n_cols] are float32
 * device arrays owned by the caller. */
typedef struct {
  float cutoff;     /* > 0 */
  int32_t n_basis;  /* must be 8 */
  int32_t hidden;   /* must be 64 */
  const float* W1;
  const float* W2;
} e3_radial;

/* w[E][n_cols] (float32, caller-owned) for the edge vectors edge_vec[E][3];
 * n_cols a multiple of 16 (P*C for a convolution's w[E][P][C]), w 16-byte
 * aligned.  The second layer runs on the fp16 matrix cores with operands
 * split into high and low fp16 parts (three products, fp32 accumulation),
 * which keeps w to a few 1e-7 of its size; |W2| and |h| must stay below the
 * fp16 range (65504).  The radial basis is evaluated in fp64.  E3_ERR_UNSUPPORTED for other basis or hidden
 * sizes. */
e3_status e3_radial_mlp(const e3_radial* mlp, int32_t n_edges, int32_t n_cols,
                        const float* edge_vec, float* w, void* stream);

/* The forward convolution (as e3_conv_forward, edge-vector mode, float32
 * storage) with w[e][P][C] = the radial MLP of edge e computed on the fly:
 * w never reaches memory.  The MLP's second layer runs on the fp16 matrix
 * cores with operands split into high and low fp16 parts (three products),
 * which keeps w to about 1e-6 of its size; |W2| and |h| must stay below the
 * fp16 range (65504).  Supported: x = Cx(0e+1o), harmonics 0e+1o+2e+3o,
 * out = Cx(0e+1o+2e+3o), C in {32, 64, 128, 256}; flags must be 0.  The
 * workspace (from e3_conv_prepare_transpose) is optional, as for the forward. */
e3_status e3_conv_forward_radial(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                 const int32_t* rowptr, const int32_t* sender,
                                 const void* workspace, size_t ws_bytes, const float* edge_vec,
                                 const float* x, const e3_radial* mlp, float* m, void* stream);

/* The radial MLP's hidden layer h = silu(B(|r_e|) W1) of every edge (e3j
 * A.3, Eq.7's edge scalars; the reading above), computed once per edge and
 * stored in the operand form e3_conv_forward_radial_hidden reads:
 * e3_radial_hidden_size bytes (256 per edge: per edge, for k-halves 0..1 and
 * quarters 0..3, the fp16 high part and the 2^11-scaled fp16 low part of
 * units 32 k + 8 q .. 32 k + 8 q + 7, each 8 halves).  It depends only on
 * the edge vectors, the cutoff and W1.  hidden: caller-owned device memory,
 * 16-byte aligned; E3_ERR_WORKSPACE when h_bytes is too small. */
e3_status e3_radial_hidden_size(int32_t n_edges, size_t* bytes);
e3_status e3_radial_hidden(const e3_radial* mlp, int32_t n_edges, const float* edge_vec,
                           void* hidden, size_t h_bytes, void* stream);
/* e3_radial_mlp with the hidden layer read from `hidden` (e3_radial_hidden of
 * the same edge vectors, cutoff and W1) instead of being formed again for
 * every 128-column slab of w: bitwise the same w.  No edge vectors needed;
 * sizes, alignment and errors as e3_radial_mlp, plus E3_ERR_WORKSPACE when
 * h_bytes is below e3_radial_hidden_size. */
e3_status e3_radial_mlp_hidden(const e3_radial* mlp, int32_t n_edges, int32_t n_cols,
                               const void* hidden, size_t h_bytes, float* w, void* stream);
/* e3_conv_forward_radial with the hidden layer read from `hidden` (written
 * by e3_radial_hidden for the same edge vectors, cutoff and W1) instead of
 * being formed again for every 32-channel slab of the output: bitwise the
 * same m.  The other arguments and limits are those of
 * e3_conv_forward_radial. */
e3_status e3_conv_forward_radial_hidden(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                        const int32_t* rowptr, const int32_t* sender,
                                        const void* workspace, size_t ws_bytes,
                                        const float* edge_vec, const float* x,
                                        const e3_radial* mlp, const void* hidden, size_t h_bytes,
                                        float* m, void* stream);

/* Convolution backward (as e3_conv_backward: e3j E.1 Eq.16 with one scalar
 * per path) with the per-edge weights formed on the fly from the radial
 * MLP's hidden layer, as e3_conv_forward_radial_hidden forms them (e3j A.3,
 * the edge scalars of Eq.7): w is neither read nor written.  For the dm of
 * the fused radial forward's m it gives dx [N][dx][C], dw [E][P][C] (the
 * cotangent of w, for e3_radial_mlp_backward) and dY [E][dy] (for
 * e3_spherical_harmonics_backward), all float32.  hidden: e3_radial_hidden
 * of the same edge vectors (h_bytes >= e3_radial_hidden_size); workspace:
 * from e3_conv_prepare_transpose on the same graph (required); scratch:
 * caller-owned device memory of e3_conv_backward_radial_scratch_size bytes
 * (per 32-channel slab partial sums of dY, added in slab order).  Same
 * signature, channel counts and flags as the fused forward; x, dm, dx, dw,
 * hidden 16-byte aligned; errors as e3_conv_backward plus E3_ERR_WORKSPACE
 * for a short hidden or scratch.  Padding edges get zero dw and dY. */
e3_status e3_conv_backward_radial_scratch_size(const e3_desc* desc, int32_t n_edges,
                                               size_t* bytes);
e3_status e3_conv_backward_radial_hidden(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                         const int32_t* rowptr, const int32_t* sender,
                                         const void* workspace, size_t ws_bytes,
                                         const float* edge_vec, const float* x,
                                         const e3_radial* mlp, const void* hidden, size_t h_bytes,
                                         const float* dm, float* dx, float* dw, float* dY,
                                         void* scratch, size_t scratch_bytes, void* stream);

/* Backward of e3_radial_mlp for the cotangent dw [E][n_cols] (n_cols a
 * multiple of 32): dW1 [8][64] and dW2 [64][n_cols] (summed over the edges
 * through fixed partials: reproducible) and dvec [E][3], the part of the
 * edge-vector gradient that flows through |r_e| (radial: dvec_e is parallel
 * to r_e, zero at r_e = 0); add it to e3_spherical_harmonics_backward's
 * for the full edge-vector gradient.  dh = dw W2^T and dW2 = h^T dw run on
 * the bf16 matrix cores with every fp32 operand split into three bf16 parts
 * (24 significant bits and fp32's exponent range, so any cotangent
 * magnitude is kept; six of the nine cross products, the others below
 * 2^-24 of a product), both from one read of dw (dh through per-slab
 * partials over 256-column slabs and dW2 through per-range partials, each
 * added in a fixed order; h recomputed from the edge vectors).
 * workspace: caller-owned,
 * e3_radial_mlp_backward_workspace_size bytes (about E * 256 bytes per
 * 256-column slab), 16-byte aligned; dw and W2 16-byte aligned.  All
 * arrays float32 on the device. */
e3_status e3_radial_mlp_backward_workspace_size(const e3_radial* mlp, int32_t n_edges,
                                                int32_t n_cols, size_t* bytes);
e3_status e3_radial_mlp_backward(const e3_radial* mlp, int32_t n_edges, int32_t n_cols,
                                 const float* edge_vec, const float* dw, float* dW1, float* dW2,
                                 float* dvec, void* workspace, size_t ws_bytes, void* stream);

/* Tensor product (as e3_tp_forward: e3j E.1 Eq.10-11, any channel-wise
 * signature, collapsed or per-path outputs) and its backward (as
 * e3_tp_backward, Eq.14-16) for irreps of degree up to 7, driven by
 * coefficient tables instead of compiled kernels (e3j treats the product as
 * a bilinear coupling given by a sparse COO array of coefficients, E.1 and
 * B.1; Figs 5-6 run it to L = 8).
 *   e3_generic_plan_size / e3_generic_plan_build: host-only; write table
 *     `table` for desc into a HOST buffer; the caller copies it to device
 *     memory it owns (16-byte aligned) and may reuse it for every call with
 *     the same descriptor.  One table per cotangent: E3_GEN_FORWARD (the
 *     forward), E3_GEN_DX (gradient of x), E3_GEN_DW (of w), E3_GEN_DY (of
 *     y; the records keyed by the y component).
 *   e3_tp_forward_generic: the forward table; x [n][dx][C], y [n][dy]
 *     float32, w [n][P][C], z [n][dout][C].
 *   e3_tp_backward_generic: the DX, DW and DY tables; for dz [n][dout][C]
 *     writes dx [n][dx][C], dw [n][P][C] and dy [n][dy] (float32, summed
 *     over the channels in a fixed order).
 * fp32 or bf16 storage, fp32 accumulation; no alignment beyond the element
 * size.  Needs every degree <= 7 and dx*64 + dy, dout*64 + dy <= 4096
 * (dx, dout <= 63: all irreps 0..L once fit up to L = 6).  A table built for another descriptor gives wrong
 * values but never an out-of-bounds access (every index read from it is
 * clamped). */
enum {
  E3_GEN_FORWARD = 0,
  E3_GEN_DX = 1,
  E3_GEN_DW = 2,
  E3_GEN_DY = 3,
  E3_GEN_GEMM = 4,    /* dense products: the forward */
  E3_GEN_GEMM_DX = 5, /* dense products: the gradient of x (the forward's roles swapped) */
  E3_GEN_GEMM_DW = 6, /* dense products: the gradient of w (one block per path) */
  E3_GEN_GEMM_DY = 7  /* dense products: the gradient of y (channel sums per x irrep) */
};
e3_status e3_generic_plan_size(const e3_desc* desc, int32_t table, size_t* bytes);
e3_status e3_generic_plan_build(const e3_desc* desc, int32_t table, void* host_plan,
                                size_t bytes);
e3_status e3_tp_forward_generic(const e3_desc* desc, int64_t n_rows, const void* plan,
                                size_t plan_bytes, const void* x, const float* y, const void* w,
                                void* z, e3_dtype dtype, void* stream);
/* The same tensor product forward on the fp32 matrix cores (degrees up to 7,
 * float32 only).  e3j E.1 Eq.10-11 contracted per output block as one dense
 * product: A_L[M][(P,m1)] = sum_{m2} C_P[M][m1][m2] y[m2] (per row, shared by
 * the channels) times xt[(P,m1)][q] = w[P][q] x[l1,m1][q], on
 * v_mfma_f32_16x16x4f32 (exact fp32 products, fp32 accumulation).
 *   plan: table E3_GEN_GEMM of e3_generic_plan_build for this descriptor,
 *     copied to device memory (16-byte aligned).
 *   x [n][dx][C], y [n][dy], w [n][P][C], z [n][dout][C] float32; x and w
 *     16-byte aligned; C % 16 == 0.
 * E3_ERR_UNSUPPORTED when C % 16 != 0 or a row's operands do not fit in one
 * workgroup's LDS (160 KB) even with 16-channel slabs.  Indices read from the
 * plan are clamped to the descriptor's sizes. */
e3_status e3_tp_forward_gemm(const e3_desc* desc, int64_t n_rows, const void* plan,
                             size_t plan_bytes, const float* x, const float* y, const float* w,
                             float* z, void* stream);
/* The convolution forward (e3j A.3 Eq.7, E.1 Eq.10-12) in the same dense
 * form: per receiver b and output block L, the sum over its in-edges e of
 * A_{e,L} xt_e (A from Y[e], xt from w[e] and x[sender e]) accumulates in the
 * matrix cores' registers over the edge list in CSR order, so m is written
 * once per node and reproducibly.  edge_vec_or_Y: edge vectors [E][3] (the
 * harmonics of every y irrep are computed per edge: needs dy <= 64 and
 * degrees <= 7) or, with E3_Y_GIVEN, Y [E][dy]; collapsed outputs with at
 * most 10 output blocks (an output irrep is one block, a degree-8 irrep
 * two: the irreps 0..8 once fit), C % 16 == 0, float32.  plan: table E3_GEN_GEMM (as
 * e3_tp_forward_gemm).  x [N][dx][C], w [E][P][C] (16-byte aligned),
 * m [N][dout][C]; padding edges (a sender outside [0, N)) add nothing, and a
 * row range outside [0, E) is clamped to it. */
e3_status e3_conv_forward_gemm(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                               const int32_t* rowptr, const int32_t* sender, const void* plan,
                               size_t plan_bytes, const float* edge_vec_or_Y, const float* x,
                               const float* w, float* m, void* stream);
/* The backward of e3_tp_forward_gemm (e3j E.1 Eq.14-16) as dense products
 * on the fp32 matrix cores, for the same descriptors (degrees up to 7,
 * float32, C % 16 == 0): with A_L[M][(P,m1)] = sum_m2 C_P[M][m1][m2] y[m2]
 * per row,
 *   dx   = the forward's product with the roles of x and the output swapped:
 *          dx[i][m1] = sum_{(P,M)} A'[m1][(P,M)] w[P] dz[L_P][M]  (table
 *          E3_GEN_GEMM_DX, one block per x irrep);
 *   dw[P] = sum_M dz[L_P][M] (A_P x)[M], the per-path product without weight
 *          and its sum over M in the product's epilogue (E3_GEN_GEMM_DW);
 *   dy[m2] = sum over the CG entries (P, M, m1, m2, c) of c G[(P,M)][m1],
 *          G[(P,M)][m1] = sum_q w[P][q] dz[L_P][M][q] x[l1][m1][q] on the
 *          matrix cores with the channel sum as K (E3_GEN_GEMM_DY).
 * Three launches on `stream`; every sum in a fixed order (reproducible).
 * Plans from e3_generic_plan_build with those tables (16-byte aligned device
 * copies); x [B][dx][C], y [B][dy], w [B][P][C], dz [B][dout][C] -> dx, dw,
 * dy of the same shapes (float32). */
e3_status e3_tp_backward_gemm(const e3_desc* desc, int64_t n_rows, const void* plan_dx,
                              size_t dx_bytes, const void* plan_dw, size_t dw_bytes,
                              const void* plan_dy, size_t dy_bytes, const float* x, const float* y,
                              const float* w, const float* dz, float* dx, float* dw, float* dy,
                              void* stream);
/* The backward of e3_conv_forward_gemm (e3j E.1 Eq.16) in the same dense
 * form, given harmonics only (E3_Y_GIVEN; from edge vectors, form Y with
 * e3_spherical_harmonics and chain dY with e3_spherical_harmonics_backward),
 * collapsed outputs, at most 10 x blocks (as the forward's output blocks):
 * dx per sender over its out-edges
 * (the workspace of e3_conv_prepare_transpose on this graph, required), the
 * products accumulated in registers in the index's order; dw and dY per
 * edge, x gathered by sender and dm by receiver.  Padding edges (a sender
 * outside [0, N)) get dw = 0 and dY = 0 and add nothing to dx. */
e3_status e3_conv_backward_gemm(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                const int32_t* rowptr, const int32_t* sender,
                                const void* workspace, size_t ws_bytes, const void* plan_dx,
                                size_t dx_bytes, const void* plan_dw, size_t dw_bytes,
                                const void* plan_dy, size_t dy_bytes, const float* Y,
                                const float* x, const float* w, const float* dm, float* dx,
                                float* dw, float* dY, void* stream);
e3_status e3_tp_backward_generic(const e3_desc* desc, int64_t n_rows, const void* plan_dx,
                                 size_t dx_bytes, const void* plan_dw, size_t dw_bytes,
                                 const void* plan_dy, size_t dy_bytes, const void* x,
                                 const float* y, const void* w, const void* dz, void* dx, void* dw,
                                 float* dy, e3_dtype dtype, void* stream);

/* Convolution forward and backward (as e3_conv_forward / e3_conv_backward:
 * e3j A.3 Eq.7, E.1 Eq.12-16) for irreps of degree up to 7, from the
 * coefficient tables above (e3j B.1 Fig 7 runs the convolution to L = 8).
 * The messages of a receiver accumulate in an on-chip buffer over its edge
 * list, as in the shared-memory accumulation of e3j's CUDA convolution
 * (E.1), so m is written once per node and the sum is reproducible.
 *   m[b]  = sum_{e in row b} sum_P w[e][P] (x[sender e] (x) Y_e)_P
 *   dx[a] = sum over out-edges of a (sender-ordered index), dw[e], dY[e]
 * edge_vec_or_Y: edge vectors [E][3] (the harmonics of every y irrep are
 * computed from them: needs dy <= 64 and degrees <= 6) or, with E3_Y_GIVEN,
 * Y [E][dy].
 * Forward: table E3_GEN_FORWARD; workspace optional (its node order, as
 * e3_conv_forward).  Backward: tables E3_GEN_DX, E3_GEN_DW, E3_GEN_DY;
 * workspace from e3_conv_prepare_transpose on the same graph (required);
 * dY float32 [E][dy] is the cotangent of Y (of the harmonics in edge-vector
 * mode; e3_spherical_harmonics_backward chains it to the vectors).  Padding
 * edges (a sender outside [0, N)) add nothing and get dw = 0, dY = 0.  Shapes, storage and limits as for the generic tensor product. */
e3_status e3_conv_forward_generic(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                  const int32_t* rowptr, const int32_t* sender,
                                  const void* workspace, size_t ws_bytes, const void* plan,
                                  size_t plan_bytes, const float* edge_vec_or_Y, const void* x,
                                  const void* w, void* m, e3_dtype dtype, void* stream);
e3_status e3_conv_backward_generic(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                   const int32_t* rowptr, const int32_t* sender,
                                   const void* workspace, size_t ws_bytes, const void* plan_dx,
                                   size_t dx_bytes, const void* plan_dw, size_t dw_bytes,
                                   const void* plan_dy, size_t dy_bytes,
                                   const float* edge_vec_or_Y, const void* x, const void* w,
                                   const void* dm, void* dx, void* dw, float* dY, e3_dtype dtype,
                                   void* stream);

/* Double backward (as e3_conv_double_backward, e3j E.1 Eq.17-18, given
 * harmonics: desc needs E3_Y_GIVEN) for degrees up to 7, composed from the
 * generic forward and backward with all four tables; scratch as
 * e3_conv_double_backward_scratch_size gives for desc. */
e3_status e3_conv_double_backward_generic(
    const e3_desc* desc, int32_t n_nodes, int32_t n_edges, const int32_t* rowptr,
    const int32_t* sender, const void* workspace, size_t ws_bytes, const void* plan_fwd,
    size_t fwd_bytes, const void* plan_dx, size_t dx_bytes, const void* plan_dw, size_t dw_bytes,
    const void* plan_dy, size_t dy_bytes, const float* Y, const void* x, const void* w,
    const void* dm, const void* ddx, const float* ddY, const void* ddw, void* dx2, float* dY2,
    void* dw2, void* ddm, void* scratch, size_t scratch_bytes, e3_dtype dtype, void* stream);

/* Per-node gradient from per-edge vector gradients, for r_e = pos[receiver]
 * - pos[sender]:
 *   node_grad[b] = sum_{e: receiver(e) = b} edge_grad[e]
 *                - sum_{e: sender(e) = b} edge_grad[e],
 * edge_grad [E][3], node_grad [N][3] float32 (the force on b is
 * -node_grad[b]; Tessera 2.2 Eq.3).
 * rowptr / sender as for the convolution; workspace from
 * e3_conv_prepare_transpose on the same graph.  Padding edges are skipped.
 * Deterministic (no atomics). */
e3_status e3_edge_grad_to_nodes(int32_t n_nodes, int32_t n_edges, const int32_t* rowptr,
                                const int32_t* sender, const void* workspace, size_t ws_bytes,
                                const float* edge_grad, float* node_grad, void* stream);

/* Fused convolution forward (e3j A.3 Eq.7, E.1 Eq.12-13):
 *   m[b] = sum_{e in row b} sum_P w[e][P] (x[sender[e]] (x) Y(r_e))_P.
 * edge_vec_or_Y: edge vectors [E][3], or Y [E][dy] with E3_Y_GIVEN.
 * workspace: optional (NULL allowed); when given it must come from
 * e3_conv_prepare_transpose on the same graph, and receivers are then
 * visited in its locality order (same results, better cache reuse).
 * Receivers without edges get m = 0. */
e3_status e3_conv_forward(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                          const int32_t* rowptr, const int32_t* sender, const void* workspace,
                          size_t ws_bytes, const float* edge_vec_or_Y, const void* x,
                          const void* w, void* m, e3_dtype dtype, void* stream);

/* Size in bytes of the workspace that holds the sender-ordered edge index. */
e3_status e3_conv_workspace_size(int32_t n_nodes, int32_t n_edges, size_t* bytes);

/* Build the per-graph index into the workspace:
 *  - the sender-ordered (transposed) edge list, a counting sort by sender
 *    stable in edge id (the sender-keyed traversal of the e3j backward, E.4),
 *    which the backward pass reads;
 *  - a locality order of the nodes in which both passes visit them:
 *    breadth-first over in-edges from node 0; when edge_vec [E][3] (device,
 *    r = pos[receiver] - pos[sender]) is given, the reached nodes are then
 *    sorted by the Hilbert-curve cell of their position rebuilt along the traversal
 *    tree; unreached nodes follow in index order.  edge_vec may be NULL.
 * The order only changes which wavefront handles which node: results are
 * the same with any order.  Once per graph.  ws_bytes must be >=
 * e3_conv_workspace_size().  Asynchronous on `stream`: no host
 * synchronisation (the traversal's level bounds stay on the device). */
e3_status e3_conv_prepare_transpose(int32_t n_nodes, int32_t n_edges, const int32_t* rowptr,
                                    const int32_t* sender, const float* edge_vec, void* workspace,
                                    size_t ws_bytes, void* stream);

/* Fused convolution backward (e3j E.1 Eq.16 with one scalar per path):
 *   dx[a]  = sum_{e: sender(e)=a} sum_P w[e][P] (Y(r_e) (x)^T dm[recv(e)])_P
 *   dw[e][P] = sum_M (x[sender] (x) Y(r_e))_P[M] dm[recv(e)][M]
 *   dY[e]  = sum_channels sum_P w[e][P] (x[sender] (x)^T dm[recv(e)])_P
 * dm is the cotangent of m.  workspace: from e3_conv_prepare_transpose on the
 * same graph.  dY is float32 [E][dy]; with E3_Y_GIVEN it is the cotangent of
 * the given Y, otherwise of the harmonics of the edge vectors. */
e3_status e3_conv_backward(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                           const int32_t* rowptr, const int32_t* sender, const void* workspace,
                           size_t ws_bytes, const float* edge_vec_or_Y, const void* x,
                           const void* w, const void* dm, void* dx, void* dw, float* dY,
                           e3_dtype dtype, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * backward as e3_conv_backward, with the sender-ordered index that
 * e3_conv_prepare_transpose would build made inside the call, in a fixed
 * device array the library holds on each GPU it runs on (87 MiB, for at
 * most 131,072 nodes and 4,194,304 edges; larger graphs return
 * E3_ERR_UNSUPPORTED).  No allocation of any kind happens in the call; the
 * index is rebuilt every call (about the cost of e3_conv_prepare_transpose)
 * and kept in the array until the next one.  rowptr and sender are required.
 * Calls that overlap on one GPU (two streams, or two threads) share the array
 * and race: serialise them.  Arguments, layouts and errors otherwise as
 * e3_conv_backward; results are bitwise those of e3_conv_backward. */
e3_status e3_conv_backward_noalloc(const e3_desc* desc, int32_t n_nodes, int32_t n_edges,
                                   const int32_t* rowptr, const int32_t* sender,
                                   const float* edge_vec_or_Y, const void* x, const void* w,
                                   const void* dm, void* dx, void* dw, float* dY, e3_dtype dtype,
                                   void* stream);

/* Number of weight matrices of the channel mixing from `in` to `out`: one
 * per (input block, output block) pair of equal degree and parity (host). */
e3_status e3_linear_num_weights(const e3_irreps* in, const e3_irreps* out, int32_t* n_pairs);

/* Equivariant channel mixing within each irrep (e3j A.3 Eq.5, with the
 * rotation- and inversion-commuting choice of the mixing tensor,
 * W^{km}_{k'm'} = W^k_{k'} delta_{mm'} between blocks of equal (l, parity)):
 *   y[r][o, m][k] = sum over input blocks i with (l_i, p_i) = (l_o, p_o) of
 *                   sum_{k'} x[r][i, m][k'] W_io[k'][k].
 * Every `in` block has multiplicity Cin (a multiple of 8, <= 256), every
 * `out` block Cout (a multiple of 32, <= 1024).  x [n_rows][din][Cin] and
 * y [n_rows][dout][Cout] in the storage type, W float32, all three 16-byte
 * aligned; W holds the e3_linear_num_weights matrices [Cin][Cout]
 * row-major, ordered by input block, then output block.  Output blocks
 * without a matching input block are zero.  fp32 storage runs on the fp32
 * matrix cores; bf16 storage with Cin in {64, 128, 256} on the bf16 matrix
 * cores (W rounded to bf16 inside the call), other Cin on the fp32 ones;
 * fp32 accumulation throughout.  y must not overlap x. */
e3_status e3_linear(const e3_irreps* in, const e3_irreps* out, int64_t n_rows, const void* x,
                    const float* W, void* y, e3_dtype dtype, void* stream);

/* Bytes of the workspace of e3_linear_backward (partial weight-gradient
 * sums; host only). */
e3_status e3_linear_workspace_size(const e3_irreps* in, const e3_irreps* out, size_t* bytes);

/* Backward of e3_linear for the cotangent dy [n_rows][dout][Cout]:
 *   dx[r][i, m][k'] = sum over output blocks o of the type of i of
 *                     sum_k dy[r][o, m][k] W_io[k'][k]          [n_rows][din][Cin]
 *   dW_io[k'][k]    = sum_r sum_m x[r][i, m][k'] dy[r][o, m][k]  float32, like W
 * dW is summed through fixed per-chunk partials in the caller's workspace
 * (e3_linear_workspace_size bytes), so the result is reproducible.
 * Needs Cin a multiple of 32 up to 128 and Cout a multiple of 32 up to 256;
 * every pointer 16-byte aligned.  n_rows = 0 gives dW = 0. */
e3_status e3_linear_backward(const e3_irreps* in, const e3_irreps* out, int64_t n_rows,
                             const void* x, const float* W, const void* dy, void* dx, float* dW,
                             void* workspace, size_t ws_bytes, e3_dtype dtype, void* stream);

/* Text of the last error on this thread ("" if none). */
const char* e3_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* E3HIP_H */
