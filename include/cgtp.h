/*
 * cgtp.h -- C ABI of the MI355X (gfx950) Clebsch-Gordan tensor-product
 * library: the CG tensor product of irrep feature vectors, fused with the
 * graph convolution that follows it, its gradient and its second
 * derivatives, plus the CSR, spherical-harmonic and force helpers the
 * convolution needs.
 *
 * Sources of the operations (the pages give no formulas; the plain
 * mathematical definitions are used, see each call):
 *   [KG]  "An Efficient Sparse Kernel Generator for O(3)-Equivariant Deep
 *         Networks", abstract: the CG tensor product contracts two dense
 *         feature vectors with a structured sparse tensor; it is fused with
 *         the following graph convolution; kernels for its gradient and for
 *         the higher partial derivatives needed for interatomic forces;
 *         static analysis at model compile time.
 *   [SE3] "Faster training and inference with NVIDIA's open-source
 *         SE(3)-Transformer" (TFN section): a degree-d feature has 2d+1
 *         components; pairwise products between degrees are summed per
 *         output degree; fused key/value channels; basis precomputation.
 *   [MACE] "Speeding Up MACE: Low-Precision Tricks for Equivariant Force
 *         Fields", abstract: FP64 / FP32 / BF16-with-FP32-accumulation
 *         policies; mismatched module layouts give wrong results, so the
 *         layout below is fixed and documented.
 *   [F3S] "Fused3S: Fast Sparse Attention on Tensor Cores", abstract:
 *         sparse attention as sampled dense-dense product, softmax and
 *         sparse-dense product, fused on the matrix units.
 *
 * Conventions (fixed; every call uses them):
 *   - Irreps strings: "MULxLp" terms joined by '+', p in {e,o} or absent
 *     (no parity label; labelled and unlabelled terms may not be mixed).
 *     Block b of a row holds MUL*(2L+1) entries, element (u, m) at
 *     offset_b + u*(2L+1) + (m+L), m = -L..L.  Blocks are kept in string
 *     order; nothing is sorted or merged.
 *   - Real spherical-harmonic basis, component normalisation
 *     (sum_m Y_lm^2 = 2l+1), l=1 ordered (y, z, x).
 *   - Real coupling tensor of path (l1,l2,l3): the complex CG tensor
 *     (Condon-Shortley phase) changed to the real basis; the real part is
 *     used when l1+l2+l3 is even, the imaginary part when odd.  This gives
 *     1x1->0 = -delta/sqrt(3) and 1x1->1 = +epsilon/sqrt(2).
 *   - No path or irrep normalisation factors; convolution sums are plain.
 *   - Weights, per path in path order: uvu -> [mul1][mul2]; uvw ->
 *     [mul1][mul2][mul_out].  Per-item weights are rows of weight_numel
 *     entries; CGTP_SHARED_WEIGHTS means one row shared by all items.
 *   - Graph arrays: edges are given in destination-sorted (CSR) order;
 *     edge t carries sh[t], w[t] and src[t]; the edges of node n are
 *     t in [dst_row_ptr[n], dst_row_ptr[n+1]).  Indices are int32.
 *
 * Ownership and execution: the caller owns every device buffer; calls are
 * asynchronous on the caller's stream (NULL = default stream); buffers must
 * stay alive until the stream has completed.  Execution calls allocate no
 * device memory: scratch space is passed in as `workspace`.  Outputs are
 * overwritten (rows of nodes with no edges are written as zero) unless a
 * call says otherwise.  A plan is immutable after creation and may be used
 * from several threads and streams at once.
 *
 * Errors: every call returns CGTP_OK (0) or a negative cgtp_status; a
 * description of the last error on the calling thread is returned by
 * cgtp_last_error().  No C++ exception crosses this boundary.
 */
#ifndef CGTP_H
#define CGTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *cgtp_stream_t; /* same handle as hipStream_t */
typedef struct cgtp_plan_s *cgtp_plan_t;

typedef enum {
    CGTP_OK = 0,
    CGTP_ERR_INVALID_ARGUMENT = -1, /* grammar, NULL, size, forbidden path, uvu mul mismatch */
    CGTP_ERR_UNSUPPORTED = -2,      /* l > 6, unsupported dtype/mode/flag combination */
    CGTP_ERR_COMPILE = -3,          /* kernel generation or compilation failed (log in last_error) */
    CGTP_ERR_HIP = -4,              /* HIP runtime error */
    CGTP_ERR_GRAPH = -5             /* malformed CSR input found by cgtp_validate_csr */
} cgtp_status;

typedef enum { CGTP_UVU = 0, CGTP_UVW = 1 } cgtp_mode;

typedef enum {
    CGTP_F32 = 0,         /* float inputs, float arithmetic and outputs */
    CGTP_F64 = 1,         /* double everywhere */
    CGTP_BF16_F32ACC = 2  /* bf16 x, sh, w; float accumulation; float outputs */
} cgtp_dtype;

enum {
    CGTP_SHARED_WEIGHTS = 1u << 0, /* one weight row for all items (uvw layers) */
    CGTP_PLAN_NO_LOAD = 1u << 1,   /* generate and compile into the on-disk cache only;
                                      no device contact; execution calls then fail */
    CGTP_BF16_WEIGHTS = 1u << 2,   /* uvu, CGTP_F32 only: every weight-shaped input (w,
                                      and gg_w of the double backward) is stored as
                                      bf16 (the upper half of a float); arithmetic,
                                      the other inputs and every output, g_w and d_w
                                      included, stay float.  Halves the dominant
                                      per-edge stream. */
};
/* Radial weights ([SE3]: the radial profile inside a TFN layer is a fully
 * connected network): a uvw, CGTP_BF16_F32ACC, CGTP_SHARED_WEIGHTS plan whose
 * input 2 is one SH row, with flag CGTP_RADIAL_HIDDEN(H), 1 <= H <= 64,
 * takes per-edge weights from a network of hidden width H on the edge
 * length (cgtp_conv_forward_radial). */
#define CGTP_RADIAL_HIDDEN(h) ((uint32_t)(h) << 16)

/* A path couples block i_in1 of input 1 with block i_in2 of input 2 into
 * block i_out of the output. */
typedef struct {
    int32_t i_in1, i_in2, i_out;
} cgtp_path;

typedef struct {
    int64_t dim_in1, dim_in2, dim_out; /* row lengths in elements */
    int64_t weight_numel;              /* weights per item (or shared) */
    int32_t n_paths;
    int32_t lmax_in2;  /* largest degree in input 2 (the SH degree in conv use) */
    int32_t n_kernels; /* generated kernels in the plan's code object */
    int32_t cached;    /* 1 if the code object came from the on-disk cache */
} cgtp_plan_dims;

/* ---------------------------------------------------------------------- */
/* Planning: the analysis done once per model before any launch ([KG]).  */
/* ---------------------------------------------------------------------- */

/* Parses the irreps, validates `paths` (n_paths > 0) or enumerates every
 * allowed path (n_paths == 0: |l1-l2| <= l3 <= l1+l2, parity p1*p2 == p3
 * when labelled, uvu needs mul_out == mul_in1; order i_in1, then i_in2,
 * then i_out), computes each path's real coupling tensor in FP64, keeps
 * its nonzeros, decides the kernels' work split from the register and LDS
 * budget, emits HIP source for gfx950 with the nonzeros as constants, and
 * compiles it (hipRTC) or loads it from the code-object cache
 * ($CGTP_CACHE_DIR, default "_kcache" beside the library).  Degrees are
 * limited to l <= 6.  Errors: INVALID_ARGUMENT, UNSUPPORTED, COMPILE, HIP.
 * On success *out owns the plan; release it with cgtp_plan_destroy. */
int cgtp_plan(const char *irreps_in1, const char *irreps_in2, const char *irreps_out,
              const cgtp_path *paths, int32_t n_paths, cgtp_mode mode, cgtp_dtype dtype,
              uint32_t flags, cgtp_plan_t *out);

int cgtp_plan_info(cgtp_plan_t plan, cgtp_plan_dims *dims);

/* Copies min(cap, n_paths) paths of the plan (after enumeration). */
int cgtp_plan_paths(cgtp_plan_t plan, cgtp_path *paths, int32_t cap);

/* Host copy of path p's real coupling tensor R[i][j][k] as used by the
 * kernels ((2l1+1)*(2l2+1)*(2l3+1) doubles; cap = capacity in doubles). */
int cgtp_plan_coupling(cgtp_plan_t plan, int32_t p, double *R, int64_t cap);

/* Generated HIP source (NUL-terminated; truncated to cap bytes).  Returns
 * the full length (excluding NUL) through *len when len != NULL. */
int cgtp_plan_source(cgtp_plan_t plan, char *buf, int64_t cap, int64_t *len);

void cgtp_plan_destroy(cgtp_plan_t plan);

/* ---------------------------------------------------------------------- */
/* Scratch.  Execution calls allocate nothing; the scratch they need comes   */
/* in as `workspace` (a 256-byte-aligned device buffer the caller owns and   */
/* does not touch while the call is in flight on its stream):                */
/*   - uvw forwards contract in two steps (per-item path tensors T_p =        */
/*     CG_p(x, y) summed over the item's edges and rounded to the MFMA        */
/*     operand type, then T . W per output block on the matrix cores, [SE3]:  */
/*     the TFN convolution with all paths into one output degree fused,       */
/*     concatenated along K); T and the partial tiles of long contractions    */
/*     live in the workspace (uvu forwards need none: NULL is accepted);      */
/*   - the backward calls keep per-edge x-messages, per-unit SH-gradient     */
/*     partials and per-edge force vectors there.                             */
/* cgtp_workspace_bytes returns a size that suffices for every execution     */
/* call of the plan on at most n_items items (destination nodes or samples)  */
/* and n_edges edges (0 for the single product, whose backward counts each   */
/* item as one edge).  Errors: INVALID_ARGUMENT (NULL, negative sizes).      */
/* ---------------------------------------------------------------------- */
int cgtp_workspace_bytes(cgtp_plan_t plan, int64_t n_items, int64_t n_edges, size_t *bytes);

/* ---------------------------------------------------------------------- */
/* Tensor product on independent items ([KG]: the CG tensor product).      */
/*   out[b] = sum_paths W . CG(x[b], y[b])                                 */
/* x [batch][dim_in1], y [batch][dim_in2], w [batch][weight_numel] (or     */
/* [weight_numel] shared), out [batch][dim_out]; element type per dtype.    */
/* workspace: cgtp_workspace_bytes(plan, batch, 0) bytes (may be NULL for   */
/* uvu plans).                                                              */
/* ---------------------------------------------------------------------- */
int cgtp_forward(cgtp_plan_t plan, const void *x, const void *y, const void *w, int64_t batch,
                 void *out, void *workspace, size_t workspace_bytes, cgtp_stream_t stream);

/* ---------------------------------------------------------------------- */
/* Fused graph convolution ([KG]: TP fused with the graph convolution).
 *   out[n] = sum_{t in [row_ptr[n], row_ptr[n+1])} TP(x[src[t]], sh[t], w[t])
 * x [n_nodes][dim_in1]; sh [n_edges][dim_in2]; w [n_edges][weight_numel]
 * (or shared); src [n_edges]; dst_row_ptr [n_nodes+1]; out
 * [n_nodes][dim_out].  Each destination row is reduced by one wavefront
 * per path group and written once; no atomics.  src values must lie in
 * [0, n_nodes) and row_ptr must be a monotone CSR with row_ptr[0] = 0,
 * row_ptr[n_nodes] = n_edges; check untrusted input with cgtp_validate_csr
 * first.  node_order [n_nodes] (may be NULL: natural order) is the order
 * in which destination rows are handed to the device, a permutation of
 * 0..n_nodes-1, normally from cgtp_build_csr_order or cgtp_node_order;
 * it changes timing only, never a result (an entry out of range leaves its
 * slot idle, so a node missing from it is not written).  workspace:
 * cgtp_workspace_bytes(plan, n_nodes, n_edges) (may be NULL for uvu plans).
 * uvw bf16 plans run the per-pair matrix-core kernel when x is 16-byte
 * aligned (and w too, where that kernel also does the channel mixing), else
 * the per-edge kernel: the same results, only the speed differs. */
int cgtp_conv_forward(cgtp_plan_t plan, const void *x, const void *sh, const void *w,
                      const int32_t *src, const int32_t *dst_row_ptr, const int32_t *node_order,
                      int64_t n_nodes, int64_t n_edges, void *out, void *workspace,
                      size_t workspace_bytes, cgtp_stream_t stream);

/* The same convolution with the SH of the edges computed inside the kernel
 * from the edge vectors ([SE3] basis computation, moved into the
 * convolution): edge t uses sh[t] = Y(vec[e] / |vec[e]|), e = vec_perm ?
 * vec_perm[t] : t, with the conventions of cgtp_sh; vec
 * [*][3] float (double for CGTP_F64 plans).  Needs a plan whose input 2 is
 * one SH row, 1x0+1x1+...+1xL with L <= 6 (parity labels absent or
 * (-1)^l); other plans return UNSUPPORTED.  The SH never reach memory. */
int cgtp_conv_forward_vec(cgtp_plan_t plan, const void *x, const void *vec, const int32_t *vec_perm,
                          const void *w, const int32_t *src, const int32_t *dst_row_ptr,
                          const int32_t *node_order, int64_t n_nodes, int64_t n_edges, void *out,
                          void *workspace, size_t workspace_bytes, cgtp_stream_t stream);

/* Convolution with per-edge weights from the radial network (plan flag
 * CGTP_RADIAL_HIDDEN(H)):
 *   phi_h(e) = silu(radial[h] r_e + radial[H + h]),  r_e = |vec[e]|,
 *   silu(z) = z / (1 + e^-z), h = 0..H-1;
 *   W_e = w[0] + sum_h phi_h(e) w[1 + h]     (w: bf16 [H+1][weight_numel])
 *   out[n] = sum_t TP_uvw(x[src[t]], Y(vec[t]), W_t)
 * radial: float [2][H] (first-layer slopes, then offsets).  The SH and
 * phi are computed inside the kernel from the edge vectors (as in
 * cgtp_conv_forward_vec).  Because the output layer is linear, the mixing
 * runs after aggregation: per node the path tensors are summed once per
 * row of w (phi-weighted), and the mixing on the matrix cores has an
 * (H+1)-fold contraction.  workspace: cgtp_workspace_bytes. */
int cgtp_conv_forward_radial(cgtp_plan_t plan, const void *x, const void *vec,
                             const int32_t *vec_perm, const float *radial, const void *w,
                             const int32_t *src, const int32_t *dst_row_ptr,
                             const int32_t *node_order, int64_t n_nodes, int64_t n_edges,
                             void *out, void *workspace, size_t workspace_bytes,
                             cgtp_stream_t stream);

/* Gradient of the convolution ([KG]: gradient kernels) for the output
 * cotangent g_out [n_nodes][dim_out]:
 *   g_x[s]  = sum over edges leaving s of d<g_out, out>/dx   [n_nodes][dim_in1]
 *   g_sh[t] = d<g_out, out>/dsh[t]                            [n_edges][dim_in2]
 *   g_w[t]  = d<g_out, out>/dw[t]                       [n_edges][weight_numel]
 * Edge arrays in dst-sorted order as in cgtp_conv_forward (x, sh, w, src,
 * dst_row_ptr, node_order have the meaning and layout given there);
 * src_row_ptr [n_nodes+1] and src_perm [n_edges] give, for each source node
 * s, the positions (into the dst-sorted arrays) of its edges:
 * src_perm[src_row_ptr[s] .. src_row_ptr[s+1]) (cgtp_build_csr with key =
 * the dst-sorted src array).  g_x is reduced per source node without
 * atomics.  Any of g_x, g_sh, g_w may be NULL (not computed); src_row_ptr and
 * src_perm may be NULL when g_x is.  The backward calls are provided for uvu
 * plans (CGTP_F32, CGTP_F64) with per-edge weights; other plans return
 * UNSUPPORTED.  workspace: cgtp_workspace_bytes(plan, n_nodes, n_edges).
 * Errors: INVALID_ARGUMENT (NULL buffer, sizes, short or misaligned
 * workspace), UNSUPPORTED, HIP. */
int cgtp_backward(cgtp_plan_t plan, const void *x, const void *sh, const void *w, const int32_t *src,
                  const int32_t *dst_row_ptr, const int32_t *node_order, const int32_t *src_row_ptr,
                  const int32_t *src_perm, const void *g_out, int64_t n_nodes, int64_t n_edges, void *g_x,
                  void *g_sh, void *g_w, void *workspace, size_t workspace_bytes, cgtp_stream_t stream);

/* Gradient of the single product cgtp_forward ([KG]: gradient kernels) on
 * batch independent items, for the cotangent g_out [batch][dim_out]:
 *   g_x[b] = d<g_out, out>/dx[b]  [batch][dim_in1],
 *   g_y[b] = d<g_out, out>/dy[b]  [batch][dim_in2],
 *   g_w[b] = d<g_out, out>/dw[b]  [batch][weight_numel].
 * Any of g_x, g_y, g_w may be NULL.  Same plans as cgtp_backward (uvu,
 * per-item weights).  workspace: cgtp_workspace_bytes(plan, batch, 0). */
int cgtp_tp_backward(cgtp_plan_t plan, const void *x, const void *y, const void *w, int64_t batch,
                     const void *g_out, void *g_x, void *g_y, void *g_w, void *workspace, size_t workspace_bytes,
                     cgtp_stream_t stream);

/* Backward with the SH computed from the edge vectors (as in
 * cgtp_conv_forward_vec) and, when F [n_nodes][3] is given, the forces of
 * the energy <g_out, out> on the atoms whose positions give the edge
 * vectors (vec = pos[dst] - pos[src]), without writing the SH gradient:
 *   F[a] = - sum_{t: dst=a} J_t^T g_sh[t] + sum_{t: src=a} J_t^T g_sh[t],
 * J_t = dY/dvec at vec_t, reduced per atom over dst_row_ptr and over
 * (src_row_ptr, src_perm) without atomics (as cgtp_sh_vjp_forces).  Any of g_x,
 * g_sh, g_w, F may be NULL.  Other arguments and the workspace as in
 * cgtp_backward. */
int cgtp_conv_backward_vec(cgtp_plan_t plan, const void *x, const void *vec, const int32_t *vec_perm,
                           const void *w, const int32_t *src, const int32_t *dst_row_ptr,
                           const int32_t *node_order, const int32_t *src_row_ptr,
                           const int32_t *src_perm, const void *g_out, int64_t n_nodes,
                           int64_t n_edges, void *g_x, void *g_sh, void *g_w, void *F,
                           void *workspace, size_t workspace_bytes, cgtp_stream_t stream);

/* Forward and backward in one pass over the edges, for an output cotangent
 * g_out that does not depend on out (an energy linear in the outputs, as
 * the sum of the 0e channels): out = the forward of cgtp_conv_forward, and
 * g_x, g_sh, g_w as cgtp_backward, each per-edge weight row read once
 * for both ([KG]: the gradient kernels; the fusion of the convolution).
 * out [n_nodes][dim_out] must not be NULL; g_x, g_sh, g_w may be NULL.
 * Other arguments and the workspace as in cgtp_backward.  FP64 plans
 * compute the same results with the forward and the backward as two
 * launches. */
int cgtp_conv_forward_backward(cgtp_plan_t plan, const void *x, const void *sh, const void *w,
                               const int32_t *src, const int32_t *dst_row_ptr,
                               const int32_t *node_order, const int32_t *src_row_ptr,
                               const int32_t *src_perm, const void *g_out, int64_t n_nodes,
                               int64_t n_edges, void *out, void *g_x, void *g_sh, void *g_w,
                               void *workspace, size_t workspace_bytes, cgtp_stream_t stream);

/* cgtp_conv_forward_backward with the SH computed from the edge vectors and
 * the forces F (may be NULL) as in cgtp_conv_backward_vec. */
int cgtp_conv_forward_backward_vec(cgtp_plan_t plan, const void *x, const void *vec,
                                   const int32_t *vec_perm, const void *w, const int32_t *src,
                                   const int32_t *dst_row_ptr, const int32_t *node_order,
                                   const int32_t *src_row_ptr, const int32_t *src_perm,
                                   const void *g_out, int64_t n_nodes, int64_t n_edges,
                                   void *out, void *g_x, void *g_sh, void *g_w, void *F,
                                   void *workspace, size_t workspace_bytes, cgtp_stream_t stream);

/* Second derivatives ([KG]: higher partial derivatives for forces).  The
 * convolution f(x, sh, w) is trilinear, so for cotangents (gg_x, gg_sh,
 * gg_w) on the backward's outputs the derivatives of
 *   S = <gg_x, g_x> + <gg_sh, g_sh> + <gg_w, g_w>
 * are forward and backward calls with substituted arguments:
 *   d_g_out = f(gg_x, sh, w) + f(x, gg_sh, w) + f(x, sh, gg_w)
 *   d_x     = fx*(g_out; gg_sh, w) + fx*(g_out; sh, gg_w)
 *   d_sh    = fsh*(g_out; gg_x, w) + fsh*(g_out; x, gg_w)
 *   d_w     = fw*(g_out; gg_x, sh) + fw*(g_out; x, gg_sh)
 * (Shapes: gg_x [n_nodes][dim_in1], gg_sh
 * [n_edges][dim_in2], gg_w [n_edges][weight_numel]; d_g_out has the shape of
 * g_out, d_x of x, d_sh of sh, d_w of w.)  NULL cotangents are zero; NULL
 * outputs are skipped; sh is read only for the gg_x and gg_w terms (may be
 * NULL when both are NULL); src_row_ptr and src_perm may be NULL when d_x
 * is.  Graph arguments, plans, workspace and errors as in cgtp_backward. */
int cgtp_double_backward(cgtp_plan_t plan, const void *x, const void *sh, const void *w, const void *g_out,
                         const void *gg_x, const void *gg_sh, const void *gg_w, const int32_t *src,
                         const int32_t *dst_row_ptr, const int32_t *node_order, const int32_t *src_row_ptr,
                         const int32_t *src_perm, int64_t n_nodes, int64_t n_edges, void *d_g_out, void *d_x,
                         void *d_sh, void *d_w, void *workspace, size_t workspace_bytes, cgtp_stream_t stream);

/* ---------------------------------------------------------------------- */
/* Helpers                                                                  */
/* ---------------------------------------------------------------------- */

/* Stable sort of edge ids by key (key[e] in [0, n_keys)):
 *   perm[t] = t-th edge id in (key, edge id) order; row_ptr[n] = #edges with
 *   key < n (n_keys+1 entries); sorted_key[t] = key[perm[t]] and
 *   sorted_val[t] = val[perm[t]] (each may be NULL; val carries a second
 *   per-edge index, e.g. the source node, into the sorted order).
 * Bit-exact and deterministic (the order within a key does not depend on
 * the order in which the device's atomics land).  Up to 65535 edges and
 * 2048 keys the sort takes two launches, linear in the edges.  Beyond, a
 * segment of d edges costs O(d^2 / 64) per wavefront, so very large
 * in-degrees are slow.
 * workspace: cgtp_csr_workspace_bytes.  Keys should lie in [0, n_keys):
 * an edge with a key outside it is left out (row_ptr[n_keys] then counts
 * only the edges kept, perm holds only that many ids, and
 * cgtp_validate_csr reports the shortfall). */
int cgtp_csr_workspace_bytes(int64_t n_edges, int64_t n_keys, size_t *bytes);
int cgtp_build_csr(const int32_t *key, const int32_t *val, int64_t n_edges, int64_t n_keys,
                   int32_t *perm, int32_t *row_ptr, int32_t *sorted_key, int32_t *sorted_val,
                   void *workspace, size_t workspace_bytes, cgtp_stream_t stream);

/* cgtp_build_csr that also writes order [n_keys], the rows' processing
 * order of cgtp_node_order (decreasing length, rows of 1023 or more edges
 * tie), from the row lengths the sort has already counted: with at most
 * 65,536 keys and at least one edge it costs no extra launch.  Same
 * arguments, workspace and errors as cgtp_build_csr; order may be NULL
 * (then the call is cgtp_build_csr). */
int cgtp_build_csr_order(const int32_t *key, const int32_t *val, int64_t n_edges, int64_t n_keys,
                         int32_t *perm, int32_t *row_ptr, int32_t *sorted_key, int32_t *sorted_val,
                         int32_t *order, void *workspace, size_t workspace_bytes, cgtp_stream_t stream);

/* cgtp_build_csr_order for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same results, with the scratch taken from a fixed array
 * of 32 MiB that the library holds on each device it runs on until the
 * process ends, instead of a caller workspace.  Nothing is allocated.  A
 * graph whose scratch (cgtp_csr_workspace_bytes, or the node order's when
 * it runs separately) exceeds 32 MiB -- about 8 million edges plus keys --
 * is refused with INVALID_ARGUMENT before any launch.  Every call on one
 * device shares that device's array: calls that overlap on one device (on
 * different streams or threads) race and give wrong results; serialise
 * them.  Other arguments and errors as cgtp_build_csr_order. */
int cgtp_build_csr_order_noalloc(const int32_t *key, const int32_t *val, int64_t n_edges, int64_t n_keys,
                                 int32_t *perm, int32_t *row_ptr, int32_t *sorted_key, int32_t *sorted_val,
                                 int32_t *order, cgtp_stream_t stream);

/* The transpose CSR (by source) that the backward calls take, for a
 * canonical edge list: edges sorted by source, ties by destination, every
 * source in [0, n_keys) and no repeated (source, destination) pair ([KG]'s
 * gradient needs the sum over each node's out-edges).  perm is the
 * destination CSR's permutation of that list (cgtp_build_csr with the
 * destinations as keys, all of them in range, so that perm is a
 * permutation of 0..n_edges-1; entries outside it are skipped).  Writes
 * src_row_ptr [n_keys+1] and src_perm
 * [n_edges], bit for bit what cgtp_build_csr gives when it sorts the
 * destination-sorted sources (its perm and row_ptr): the edges of source s
 * are the canonical run of s, in order of destination.  One launch, no
 * workspace, nothing allocated.  An edge list that is not canonical gives
 * undefined (in-range) results, in up to n_edges * n_keys steps; check with
 * cgtp_validate_csr where unsure.
 * Errors: INVALID_ARGUMENT (sizes, NULL). */
int cgtp_build_csr_transpose_canonical(const int32_t *src, const int32_t *perm, int64_t n_edges,
                                       int64_t n_keys, int32_t *src_perm, int32_t *src_row_ptr,
                                       cgtp_stream_t stream);

/* Processing order for the convolution calls: the n_nodes rows of a CSR
 * sorted by decreasing length (rows of 1023 or more edges tie), so that
 * the longest rows are started first and do not form the tail of a launch
 * (longest-processing-time-first scheduling).  The order among rows of
 * equal length is not fixed; it changes no result of any call.
 * order [n_nodes]; workspace: cgtp_node_order_workspace_bytes. */
int cgtp_node_order_workspace_bytes(int64_t n_nodes, size_t *bytes);
int cgtp_node_order(const int32_t *row_ptr, int64_t n_nodes, int32_t *order, void *workspace,
                    size_t workspace_bytes, cgtp_stream_t stream);

/* Graph sparse attention ([F3S]: sampled dense-dense product, softmax and
 * sparse-dense product fused in one kernel on the matrix cores):
 *   s_t = scale <q[i][h], k[col[t]][h]>   for t in [row_ptr[i], row_ptr[i+1])
 *   out[i][h] = sum_t (exp(s_t) / sum_t' exp(s_t')) v[col[t]][h]
 * Two calls.  cgtp_sparse_attention_prepare compacts the graph once: rows
 * are grouped in windows of 16, and each window's distinct columns are
 * listed with a 16-bit mask of the rows that hold them.  The layout goes into
 * a caller-owned buffer of cgtp_sparse_attention_layout_bytes(n_rows,
 * n_edges) bytes (256-byte aligned).  It depends only on (col, row_ptr), so
 * it serves every head, layer and call on the same graph.
 * cgtp_sparse_attention then computes
 * the attention from q [n_rows][n_heads][head_dim] and k, v
 * [n_cols][n_heads][head_dim], bf16 (dtype CGTP_BF16_F32ACC; q and k 8-byte
 * aligned), into out [n_rows][n_heads][head_dim] float; head_dim a multiple
 * of 16, at most 128.  Scores and probabilities stay on the chip; products
 * accumulate in float, the probabilities enter the second product rounded
 * to bf16.  A row may not list the same column twice; edges whose column
 * lies outside [0, n_cols) are ignored; rows without edges are zero;
 * n_cols < 2^28 - 1.  Both calls are asynchronous on the stream. */
int cgtp_sparse_attention_layout_bytes(int64_t n_rows, int64_t n_edges, size_t *bytes);
int cgtp_sparse_attention_prepare(const int32_t *col, const int32_t *row_ptr, int64_t n_rows,
                                  int64_t n_cols, int64_t n_edges, void *layout,
                                  size_t layout_bytes, cgtp_stream_t stream);
int cgtp_sparse_attention(cgtp_dtype dtype, int32_t n_heads, int32_t head_dim, float scale,
                          const void *q, const void *k, const void *v, const int32_t *row_ptr,
                          int64_t n_rows, int64_t n_edges, const void *layout, size_t layout_bytes,
                          void *out, cgtp_stream_t stream);

/* The same attention ([F3S]'s three sparse steps fused, scores on the chip)
 * in row form, straight from the CSR (col [n_edges], row_ptr [n_rows+1]; no
 * prepare call): each (row, head) is taken by head_dim/4 lanes, four head
 * dimensions per lane, and the row's edges are walked with an online
 * softmax; products, softmax and sums in FP32 (the probabilities are not
 * rounded).  Meant for graphs whose rows share few columns within 16-row
 * windows (random numbering), where the matrix-core tiles of
 * cgtp_sparse_attention stay nearly empty.  dtype CGTP_BF16_F32ACC; head_dim
 * 16, 32, 64 or 128; q, k, v 8-byte aligned, out 16-byte aligned; edges
 * whose column lies outside [0, n_cols) are ignored; rows without edges are
 * zero.  Asynchronous on the stream. */
int cgtp_sparse_attention_rows(cgtp_dtype dtype, int32_t n_heads, int32_t head_dim, float scale,
                               const void *q, const void *k, const void *v, const int32_t *col,
                               const int32_t *row_ptr, int64_t n_rows, int64_t n_cols, int64_t n_edges,
                               void *out, cgtp_stream_t stream);

/* Checks on the device that row_ptr is a monotone CSR over n_edges and that
 * every index in idx[n_edges] (may be NULL) lies in [0, n_idx_range).
 * Synchronises the stream.  Returns CGTP_OK or CGTP_ERR_GRAPH.
 * workspace: 16 bytes. */
int cgtp_validate_csr(const int32_t *row_ptr, int64_t n_rows, int64_t n_edges,
                      const int32_t *idx, int64_t n_idx_range, void *workspace,
                      cgtp_stream_t stream);

/* Real spherical harmonics of edge vectors (component normalisation, see
 * Conventions), degrees 0..lmax (lmax <= 6), [SE3] basis computation:
 *   sh[t][l*l + m + l] = Y_lm(vec[e] / |vec[e]|),  e = perm ? perm[t] : t.
 * vec [*][3] and sh [n][(lmax+1)^2] in dtype (F32 or F64; BF16_F32ACC
 * reads float vectors and writes bf16).  A zero vector gives undefined
 * values.  Errors: INVALID_ARGUMENT, UNSUPPORTED (dtype, lmax > 6). */
int cgtp_sh(int32_t lmax, cgtp_dtype dtype, const void *vec, const int32_t *perm, int64_t n, void *sh,
            cgtp_stream_t stream);

/* Vector-Jacobian product of the SH and the forces it implies ([KG]: the
 * derivatives needed for interatomic forces).  For a gradient g_sh
 * [n_edges][(lmax+1)^2] on the SH rows of the edges (edge order t as in the
 * convolution, vector of edge t = vec[perm ? perm[t] : t] = pos[dst] -
 * pos[src]):
 *   g_vec[t] = J_t^T g_sh[t]                               [n_edges][3]
 *   F[a] = - sum_{t: dst=a} g_vec[t] + sum_{t: src=a} g_vec[t]  [n_nodes][3]
 * with J_t = dY/dvec at vec_t (F = -dE/dpos for an energy E with
 * dE/dsh = g_sh).  F is reduced per atom over dst_row_ptr and over
 * (src_row_ptr, src_perm) without atomics.  Either output may be NULL.
 * workspace: n_edges * 3 elements of dtype (256-byte aligned) when F is
 * wanted and g_vec is NULL, else unused (may be NULL).  dtype F32 or F64.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (dtype, lmax > 6). */
int cgtp_sh_vjp_forces(int32_t lmax, cgtp_dtype dtype, const void *vec, const int32_t *perm, const void *g_sh,
                       const int32_t *dst_row_ptr, const int32_t *src_row_ptr, const int32_t *src_perm,
                       int64_t n_nodes, int64_t n_edges, void *g_vec, void *F, void *workspace,
                       size_t workspace_bytes, cgtp_stream_t stream);

/* Cotangent on the SH of the force loss L = 1/2 sum_a |F[a]|^2:
 *   gg_sh[t] = -J_t (F[dst[t]] - F[src[t]]).  dtype F32 or F64. */
int cgtp_force_loss_sh_cotangent(int32_t lmax, cgtp_dtype dtype, const void *vec,
                                 const int32_t *perm, const int32_t *src, const int32_t *dst,
                                 const void *F, int64_t n_edges, void *gg_sh,
                                 cgtp_stream_t stream);

/* Per-launch timing, a profiling aid.  While enabled, every kernel the
 * library launches is bracketed by two HIP events recorded on its launch
 * stream (the caller's stream).  cgtp_timing_collect waits for the recorded
 * events, writes up to cap records (kernel name, NUL-terminated in 64
 * bytes, and milliseconds) oldest first, returns their number in *n and
 * clears the record list.  Process-wide; thread-safe. */
int cgtp_timing_enable(int enable);
int cgtp_timing_collect(char (*names)[64], float *ms, int32_t cap, int32_t *n);

/* Streaming bandwidth probe, a measurement aid beside the kernels'
 * roofline (the ceiling the hardware reaches for plain streams, reported
 * next to the datasheet peak).  kind 0 reads `bytes` of src, 1 writes
 * `bytes` of dst (a fixed pattern), 2 copies src to dst; 16-byte
 * non-temporal loads and stores over a grid-stride loop.  bytes must be a
 * multiple of 16 and src, dst 16-byte aligned (kind 0 may store at most
 * 4 bytes at dst, which must be writable; src is unused for kind 1).  One
 * launch on stream, nothing allocated.  Errors: INVALID_ARGUMENT. */
int cgtp_stream_probe(int32_t kind, const void *src, void *dst, size_t bytes, cgtp_stream_t stream);

/* Description of the last error on this thread ("" if none). */
const char *cgtp_last_error(void);

/* Library version string. */
const char *cgtp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CGTP_H */
