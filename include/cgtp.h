/*
 * cgtp.h - C ABI of the MI355X (gfx950) Clebsch-Gordan tensor-product convolution.
 *
 * The operator (Sobek: Streaming Equivariant Tensor Product Convolutions, section 2.4,
 * Eqs. 7 and 11-12; LunaTP: Enabling Efficient and Scalable Tensor Product for
 * Equivariant MLIPs, section 2.1 Eq. 1 and section 2.2 Algorithm 1):
 *
 *   for every edge i <- j with vector r_ij = pos[j] - pos[i] + shift_ij,
 *   m_i = sum_j sum_paths sum_a W_ij,pi,a T_pi,a(x_j, Y(r_ij / |r_ij|)),
 *   W_ij,pi,a = sum_q phi_ij,q A_q,pi,a,
 *
 * where T_pi couples input block l1 of x_j with spherical-harmonic degree l2 into output
 * degree l3 through real Clebsch-Gordan coefficients.  Two schedules give the same result
 * up to rounding order (Sobek section 3.1, Eqs. 15-16): the conventional one forms the
 * per-edge weights w (in registers, never as an edge-sized tensor), the streamed one
 * accumulates the receiver state S_i = sum_j phi_ij (x) CG(x_j, Y_ij) and applies m = S A
 * (Sobek section 4.2, Eqs. 32-35).
 *
 * Conventions fixed by this library (the pages leave them open):
 *  - Irreps strings are "MULxLp" tokens joined by '+', p in {e, o}, e.g. "128x0e+128x1o".
 *    The spherical-harmonic irreps are one block of multiplicity 1 per degree 0..L in order,
 *    normally "1x0e+1x1o+...+1xLp" with parity (-1)^l.  The block values are always the real
 *    spherical harmonics of the edge direction; a block's parity label only enters path
 *    selection, so another label (LunaTP Appendix A.1 profile C1: "1x0e+1x1e+1x2e") is accepted
 *    as given.
 *  - Features use the ir_mul layout (Sobek section 4.5): block b of multiplicity C and
 *    degree l occupies C*(2l+1) consecutive values, component m (0..2l) major, channel minor.
 *    A node row holds its blocks back to back: x is N x C_in, out is N x C_out, row-major.
 *  - Real spherical harmonics of the unit edge direction, component normalised
 *    (sum_m Y_lm^2 = 2l+1), real combination of the Condon-Shortley complex harmonics,
 *    m = -l..l, so Y_1 = sqrt(3) (y, z, x).
 *  - Real Clebsch-Gordan tensors: unitary, first non-zero entry of each (l1,l2,l3) tensor in
 *    row-major (m1,m2,m3) order positive; no further path normalisation.
 *  - Paths are enumerated over (input block, SH block, output block) in lexicographic order;
 *    a path needs |l1-l2| <= l3 <= l1+l2 and parity_in * parity_sh == parity_out
 *    (Sobek section 2.2, Eq. 5); channelwise mode also needs mul_in == mul_out.  Paths into
 *    the same output block are summed.
 *  - A is K x N_w row-major.  Columns are path-major; within a path, channel u (channelwise,
 *    n_pi = C) or the pair (u, w) with u major (fully connected, n_pi = C_in C_out)
 *    (Sobek section 2.4, Eqs. 8-9 and 12).
 *  - Edges: the graph handle sorts the caller's edge list into receiver-major CSR order
 *    (LunaTP section 4.1).  Every per-edge array passed to a convolution call (shift, phi,
 *    grad_edge_vec, ...) is in that receiver-sorted order.
 *
 * Memory and calls: handles are opaque and owned by the library; every tensor argument is a
 * caller-owned device pointer in the plan's dtype (float or double) unless stated.  Calls
 * run asynchronously on the caller's HIP stream (`stream` is a hipStream_t, NULL = default
 * stream).  Outputs are overwritten, not accumulated.  The caller supplies a device
 * workspace of at least cgtp_workspace_size() bytes; the convolution calls never allocate
 * device memory and never synchronise, except for the one-off upload of a graph to a device
 * (cgtp_graph_upload; call it before the first convolution call) and the one-off compilation
 * and loading of a plan's kernels (cgtp_plan_compile).  Errors are returned as status codes;
 * nothing is thrown across the ABI.  cgtp_last_error() gives a readable message for the
 * calling thread.
 *
 * Zero-length edges: an edge whose vector pos[send] - pos[recv] + shift is exactly zero has no
 * direction, so its spherical harmonics are undefined.  The convolution calls do not test for
 * it (the test would need a synchronisation); such an edge turns the outputs it reaches into
 * NaN (its receiver's row, its sender's gradient row, its own per-edge gradients, grad_A).
 * cgtp_check_edges finds such edges on the device and returns CGTP_ERR_DEGENERATE_EDGE.
 */
#ifndef CGTP_H
#define CGTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cgtp_plan_s* cgtp_plan_t;
typedef struct cgtp_graph_s* cgtp_graph_t;

typedef enum { CGTP_CHANNELWISE = 0, CGTP_FULLY_CONNECTED = 1 } cgtp_mode_t;
typedef enum { CGTP_F32 = 0, CGTP_F64 = 1 } cgtp_dtype_t;
typedef enum { CGTP_STREAMED = 0, CGTP_CONVENTIONAL = 1 } cgtp_schedule_t;
typedef enum {
  CGTP_OP_FORWARD = 0,
  CGTP_OP_BACKWARD = 1,
  CGTP_OP_DOUBLE_BACKWARD = 2,
  CGTP_OP_TRIPLE_BACKWARD = 3
} cgtp_op_t;

typedef enum {
  CGTP_OK = 0,
  CGTP_ERR_INVALID_ARG = 1,    /* malformed irreps, bad sizes, null required pointer, bad CSR */
  CGTP_ERR_UNSUPPORTED = 2,    /* valid request the library does not implement (see message) */
  CGTP_ERR_WORKSPACE = 3,      /* workspace smaller than cgtp_workspace_size()                */
  CGTP_ERR_DEGENERATE_EDGE = 4,/* an edge of zero length was found by cgtp_check_edges        */
  CGTP_ERR_HIP = 5,            /* a HIP runtime call failed (message names it)                */
  CGTP_ERR_COMPILE = 6         /* run-time kernel compilation failed (message holds the log)  */
} cgtp_status_t;

typedef struct {
  int n_paths;       /* P, number of CG paths                                   */
  int n_weights;     /* N_w, columns of A                                       */
  int c_in;          /* C_in, values per node of x                              */
  int c_out;         /* C_out, values per node of out                           */
  int sh_dim;        /* (L+1)^2, spherical-harmonic components                  */
  int lmax_sh;       /* L                                                       */
  int num_radial;    /* K, rows of A and columns of phi                         */
  int mode;          /* cgtp_mode_t                                             */
  int dtype;         /* cgtp_dtype_t                                            */
  int n_in_blocks, n_out_blocks;
  int cg_nnz;        /* non-zero real CG coefficients summed over paths         */
  int g_nnz;         /* structural (m1, m3) pairs summed over paths: per-edge folded
                        coefficients G_pi[m1,m3] = sum_m2 c[m1,m2,m3] Y[m2]       */
} cgtp_plan_info_t;

/* ---------------------------------------------------------------- plans (host only) */

/* Build a plan: parse irreps, enumerate paths, compute the real CG tables.
 * Host only, no device needed.  Kernels are generated and compiled for gfx950 the first time
 * an operation needs them (or by cgtp_plan_compile).  Returns INVALID_ARG for malformed or
 * inconsistent irreps or num_radial < 1, UNSUPPORTED for degrees above 6 or no paths. */
cgtp_status_t cgtp_plan_create(const char* irreps_in, const char* irreps_sh, const char* irreps_out,
                               cgtp_mode_t mode, cgtp_dtype_t dtype, int num_radial, cgtp_plan_t* out);
cgtp_status_t cgtp_plan_destroy(cgtp_plan_t plan);
cgtp_status_t cgtp_plan_info(cgtp_plan_t plan, cgtp_plan_info_t* out);

/* Path descriptor: desc[0..8] = i_in, i_sh, i_out, l1, l2, l3, weight_offset, n_weights, cg_nnz. */
cgtp_status_t cgtp_plan_path(cgtp_plan_t plan, int path, int32_t* desc);

/* Sparse CG table of one path: up to `capacity` entries (m1, m2, m3) -> m123[3k..3k+2],
 * value -> val[k], indices 0..2l, row-major order; *nnz receives the full count. */
cgtp_status_t cgtp_plan_cg_table(cgtp_plan_t plan, int path, int32_t* m123, double* val,
                                 int capacity, int* nnz);

/* Generate and compile every kernel of `ops` (bit mask of 1 << cgtp_op_t) now.  Host only. */
cgtp_status_t cgtp_plan_compile(cgtp_plan_t plan, int ops);

/* Scratch budget in bytes for the per-edge folded coefficients and partial sums
 * (default 256 MiB, the size of the MI355X Infinity Cache).  Larger graphs are processed in
 * receiver chunks that fit it (Sobek Appendix B.2 bounds its scratch the same way). */
cgtp_status_t cgtp_plan_set_scratch_budget(cgtp_plan_t plan, size_t bytes);

/* Radial basis computed inside the kernels from the edge length r = |edge vector| instead of
 * being passed as phi (the pages give phi as an input, Sobek Eq. 12, and name an envelope option
 * without formulas; this is the plainest reading):
 *   kind 0  none: phi is an input (default)
 *   kind 1  Bessel: phi_n = sqrt(2/r_cut) sin(n pi r / r_cut) / r * u(r / r_cut), n = 1..K, with
 *           the polynomial envelope u(d) = 1 - 28 d^6 + 48 d^7 - 21 d^8 and phi = 0 for r >= r_cut
 *   kind 2  Gaussian: phi_k = exp(-(r - k D)^2 / (2 D^2)), D = r_cut / (K - 1), k = 0..K-1
 * With kind 1 or 2 the convolution calls take phi = NULL; no E x K tensor is read, the values
 * live in the per-chunk workspace rows; cgtp_conv_backward's grad_pos and grad_edge_vec include
 * the chain rule through phi(r) and grad_phi (optional) is the gradient with respect to the
 * computed values.  cgtp_conv_double_backward (both modes) takes phi = NULL and v_phi = NULL: the
 * radial direction is phi'(|r|) (r-hat . v_r) and its gg_edge_vec / gg_pos include the chain
 * through phi(r) and the basis' second derivative; the triple backward keeps phi as an input
 * (UNSUPPORTED with a radial kind).  Call before the plan compiles kernels (UNSUPPORTED
 * afterwards).  INVALID_ARG for an unknown kind, r_cut <= 0, or kind 2 with K < 2. */
cgtp_status_t cgtp_plan_set_radial(cgtp_plan_t plan, int kind, double r_cut);

/* ---------------------------------------------------------------- graphs */

/* Sort an edge list into receiver CSR order and build the source CSR (host only, exact).
 * Edge k is (recv[k] <- send[k]); image (E x 3 int32, may be NULL) holds the periodic image
 * index, used only to break ties.  Order: (recv, send, image_x, image_y, image_z, k) ascending.
 * perm_out (E int32, may be NULL) receives, for each sorted position, the caller's edge index.
 * INVALID_ARG for n_nodes < 1, n_edges < 0 or an index outside [0, n_nodes). */
cgtp_status_t cgtp_graph_build(int n_nodes, int n_edges, const int32_t* recv, const int32_t* send,
                               const int32_t* image, int32_t* perm_out, cgtp_graph_t* out);

/* Copy the CSR arrays to host memory: row_ptr[N+1], col[E] (sender of each sorted edge),
 * src_ptr[N+1], src_edge[E] (sorted edge positions grouped by sender, ascending). Any may be NULL. */
cgtp_status_t cgtp_graph_export(cgtp_graph_t g, int32_t* row_ptr, int32_t* col, int32_t* src_ptr,
                                int32_t* src_edge);
cgtp_status_t cgtp_graph_dims(cgtp_graph_t g, int* n_nodes, int* n_edges);

/* Node dispatch order of the channelwise kernels (LunaTP section 4.2, "task ordering": heavier
 * tasks first, so that a launch does not end on a tail of heavy workgroups):
 *   0  index order;
 *   1  by degree: a launch over every node deals the nodes to the 8 XCDs in contiguous index
 *      ranges of ceil(N / 8) (each XCD keeps its neighbourhood in its L2) and runs each range in
 *      descending in-degree (receiver passes) or out-degree (source passes), ties by index;
 *   2  automatic (default): 1 when the in-degrees are skewed (the largest above twice the mean),
 *      else 0.
 * Launches over part of the receivers (a graph split into receiver chunks by the scratch budget)
 * run in index order.  Tasks (feature blocks and path subsets) are always dispatched heaviest
 * first by their count of CG terms.  The order changes no result beyond the order of the
 * fixed-order grad_A partial sums.  Call before cgtp_graph_upload (UNSUPPORTED afterwards);
 * INVALID_ARG for another mode. */
cgtp_status_t cgtp_graph_set_order(cgtp_graph_t g, int mode);

/* Upload the CSR to the current device (once per device; later calls return at once).
 * The convolution calls do it themselves on first use; call it before a timed region. */
cgtp_status_t cgtp_graph_upload(cgtp_graph_t g);
cgtp_status_t cgtp_graph_destroy(cgtp_graph_t g);

/* ---------------------------------------------------------------- convolution (device) */

/* Workspace bytes needed by `op` for this plan and graph: at most the scratch budget (per-edge
 * rows, edge partials and grad_A partial slots of one receiver chunk) plus E x 3 edge-vector
 * values and 2 N int32 source-CSR bounds; never O(E x N_w).  A graph whose rows do not fit is
 * processed in receiver chunks; the receivers per chunk are also capped so that the grad_A
 * partial slots stay inside the budget at low in-degree.  The fully connected double backward
 * adds E x K values (a zero phi direction when v_phi is NULL; 4 E x K + E x 3 with a radial kind).  UNSUPPORTED for the triple
 * backward of a fully connected plan. */
cgtp_status_t cgtp_workspace_size(cgtp_plan_t plan, cgtp_graph_t g, cgtp_op_t op, size_t* bytes);

/* Forward.  x: N x C_in; pos: N x 3; shift: E x 3 receiver-sorted image shifts added to
 * pos[send] - pos[recv] (NULL = no shift); phi: E x K receiver-sorted (NULL exactly when the
 * plan computes the radial basis, cgtp_plan_set_radial); A: K x N_w;
 * out: N x C_out (overwritten). */
cgtp_status_t cgtp_conv_forward(cgtp_plan_t plan, cgtp_graph_t g, cgtp_schedule_t schedule,
                                const void* x, const void* pos, const void* shift, const void* phi,
                                const void* A, void* out, void* workspace, size_t ws_bytes, void* stream);

/* Backward of the forward map for the output cotangent grad_out (N x C_out) (Sobek section
 * 3.2, Eqs. 18-22).  Outputs, each overwritten and each optional (NULL = not requested):
 * grad_x (N x C_in), grad_pos (N x 3), grad_edge_vec (E x 3, gradient with respect to the
 * edge vectors r_ij), grad_phi (E x K), grad_A (K x N_w).  grad_pos = sum over out-edges of
 * grad_edge_vec minus sum over in-edges.  Reductions run in a fixed order: two identical
 * calls give bitwise identical results. */
cgtp_status_t cgtp_conv_backward(cgtp_plan_t plan, cgtp_graph_t g, const void* x, const void* pos,
                                 const void* shift, const void* phi, const void* A, const void* grad_out,
                                 void* grad_x, void* grad_pos, void* grad_edge_vec, void* grad_phi,
                                 void* grad_A, void* workspace, size_t ws_bytes, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments and results as
 * cgtp_conv_forward, without the workspace: the per-chunk rows of folded coefficients live in a
 * static device array of CGTP_STATIC_SCRATCH_BYTES held by the library on every GPU it runs on
 * until the process ends; receiver chunks are cut to fit it.  Channelwise plans only
 * (UNSUPPORTED for fully connected ones); both schedules.  Preconditions, checked on the host:
 * the graph is on the current device (cgtp_graph_upload; INVALID_ARG otherwise) and the plan's
 * forward kernels of `schedule` are loaded there (one cgtp_conv_forward call with that schedule on
 * this device; UNSUPPORTED otherwise).  The call then uploads, compiles, loads and allocates
 * nothing; the first call on a device looks up that device's copy of the array.  WORKSPACE when one
 * receiver's rows (in-degree x row width) exceed the array.  Calls on one GPU share its array: calls
 * that overlap in time on one GPU (different streams) race; calls on one stream do not.  Nothing in
 * the array needs clearing between calls (every row read is written first by the same call). */
#define CGTP_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
cgtp_status_t cgtp_conv_forward_static(cgtp_plan_t plan, cgtp_graph_t g, cgtp_schedule_t schedule, const void* x,
                                       const void* pos, const void* shift, const void* phi, const void* A, void* out,
                                       void* stream);

/* Kept forward state, for a backward with the same inputs.
 * Fully connected plans: the streamed forward accumulates per receiver the state
 * S_i = sum over in-edges of phi_ij (x) CG(x_j, Y_ij) (Sobek section 4, Eqs. 32-33) and the
 * backward needs it again for grad_A = S^T grad_out (Sobek section 3.2, Eq. 19 in receiver-state
 * form); the state is node-sized (N times the state width, e.g. 71.7 KB per node for
 * 64x(0e,1o,2e) with K = 8).
 * Channelwise plans: the state is the per-edge row of folded coefficients G = sum c Y and the
 * real SH Y that the forward and backward both derive from the edge vector (LunaTP section 4.3,
 * product reuse across passes); E times the row width (816 bytes per edge for the l <= 3
 * profile in fp32).  The state is never larger than E x N_w: cgtp_state_size returns
 * UNSUPPORTED when a row is longer than the N_w edge weights (e.g. 5,196 values against
 * N_w = 3,392 for 32x(0e..6e) with SH l <= 6); such plans let the backward recompute its rows.
 *   cgtp_state_size               bytes of the state buffer
 *   cgtp_conv_forward_keep_state  the forward (fully connected: CGTP_STREAMED; channelwise:
 *                                 CGTP_CONVENTIONAL, as cgtp_conv_forward) that also leaves the
 *                                 state of every node or edge in `state` (caller-owned device
 *                                 memory, state_bytes >= cgtp_state_size)
 *   cgtp_conv_backward_with_state as cgtp_conv_backward, reading the state instead of recomputing
 *                                 it; the state must come from cgtp_conv_forward_keep_state with
 *                                 the same plan, graph, x, pos, shift and phi (A does not enter
 *                                 it); results are bitwise those of cgtp_conv_backward.
 * WORKSPACE when `state` is NULL or smaller than cgtp_state_size; UNSUPPORTED when the plan keeps
 * no state (above); other errors as the plain calls.  The workspace requirements are those of the
 * plain calls. */
cgtp_status_t cgtp_state_size(cgtp_plan_t plan, cgtp_graph_t g, size_t* bytes);
cgtp_status_t cgtp_conv_forward_keep_state(cgtp_plan_t plan, cgtp_graph_t g, const void* x, const void* pos,
                                           const void* shift, const void* phi, const void* A, void* out,
                                           void* state, size_t state_bytes, void* workspace, size_t ws_bytes,
                                           void* stream);
cgtp_status_t cgtp_conv_backward_with_state(cgtp_plan_t plan, cgtp_graph_t g, const void* x, const void* pos,
                                            const void* shift, const void* phi, const void* A,
                                            const void* grad_out, const void* state, size_t state_bytes,
                                            void* grad_x, void* grad_pos, void* grad_edge_vec, void* grad_phi,
                                            void* grad_A, void* workspace, size_t ws_bytes, void* stream);

/* Double backward: the vector-Jacobian product of the backward map
 * (x, r, phi, A, grad_out) -> (grad_x, grad_edge_vec, grad_phi, grad_A) along the cotangent
 * directions (v_x, v_edge, v_phi, v_A), i.e. the gradient of
 *   <v_x, grad_x> + <v_edge, grad_edge_vec> + <v_phi, grad_phi> + <v_A, grad_A>
 * with respect to every input of the backward (Sobek section 3.3, Eqs. 23-31, which state the
 * same derivatives in tangent form).  Inputs as in cgtp_conv_backward; directions, each
 * optional (NULL = zero): v_x (N x C_in), v_pos (N x 3; a direction of the positions, entering
 * through the edge vectors as v_pos[send] - v_pos[recv]), v_edge_vec (E x 3, receiver-sorted),
 * v_phi (E x K), v_A (K x N_w).  Outputs, each optional and overwritten: gg_x (N x C_in),
 * gg_pos (N x 3, out-edge minus in-edge sums of gg_edge_vec), gg_edge_vec (E x 3), gg_phi
 * (E x K), gg_A (K x N_w) and gg_grad_out (N x C_out, the derivative with respect to grad_out,
 * which is the tangent of the forward output).  Fixed-order reductions: bitwise repeatable.
 * With an in-kernel radial basis (cgtp_plan_set_radial) phi and v_phi are NULL (INVALID_ARG
 * otherwise), the map differentiated is (x, r, A, grad_out) -> (grad_x, grad_edge_vec, grad_A)
 * with grad_edge_vec through phi(|r|) as in cgtp_conv_backward, and gg_phi (optional) is the
 * gradient with respect to the computed radial values.  Fully connected mode: evaluated by
 * linearity from the streamed first-order passes (Sobek Eqs. 37-39: m-dot = S-dot A + S A-dot,
 * Sbar-dot = mbar A-dot^T, A-bar-dot = S-dot^T mbar, and the edge and source passes with one
 * operand replaced by its direction); with a radial kind it runs on the plan's twin without a
 * basis, phi and phi-dot materialised per edge in the workspace (E x K each, plus E x K for the
 * gradient in phi and the first-order phi-bar), and adds the radial terms of gg_edge_vec. */
cgtp_status_t cgtp_conv_double_backward(cgtp_plan_t plan, cgtp_graph_t g, const void* x, const void* pos,
                                        const void* shift, const void* phi, const void* A,
                                        const void* grad_out, const void* v_x, const void* v_pos,
                                        const void* v_edge_vec, const void* v_phi, const void* v_A,
                                        void* gg_x, void* gg_pos, void* gg_edge_vec, void* gg_phi,
                                        void* gg_A, void* gg_grad_out, void* workspace, size_t ws_bytes,
                                        void* stream);

/* Triple backward (channelwise mode only): the third-order derivative of the convolution on the
 * operands of LunaTP Appendix F, Algorithm 4 ("Third-Order Derivative of Clebsch-Gordan Tensor
 * Product Convolution"): node features x, the angular edge operand Y, the edge weights
 * w = phi A (kept factored) and the output cotangent g = grad_out.  With the second-order map
 *   S2(x, Y, phi, A, g; v) = <v_x, grad_x> + <v_Y, grad_Y> + <v_phi, grad_phi> + <v_A, grad_A>
 * (the first-order outputs of <g, out> along the directions v) and the cotangents q of its
 * gradients, the outputs are the gradients of S3 = <q_x, dS2/dx> + <q_Y, dS2/dY> +
 * <q_phi, dS2/dphi> + <q_A, dS2/dA> + <q_grad_out, dS2/dg> with respect to x, Y, phi, A, g and the
 * directions v_x, v_Y, v_phi, v_A.  As in the page's algorithm the edge operand is an input: the
 * chain rule through the harmonics of the edge vectors is not applied (Y is normally the real
 * spherical harmonics of the edge directions, E x sh_dim, receiver-sorted, (L+1)^2 values per
 * edge in the plan's order; any values of that shape are accepted).
 * Inputs: x (N x C_in), Y (E x sh_dim), phi (E x K), A (K x N_w), grad_out (N x C_out); directions
 * v_x, v_Y, v_phi, v_A and cotangents q_x, q_Y, q_phi, q_A, q_grad_out of the same shapes, each
 * optional (NULL = zero).  Outputs, each optional (NULL = not requested) and overwritten: t_x, t_Y,
 * t_phi, t_A, t_grad_out (N x C_out), t_vx, t_vY, t_vphi, t_vA.  Workspace: cgtp_workspace_size
 * with CGTP_OP_TRIPLE_BACKWARD.  The passes run with 2K radial values (a weight phi_1 A_1 +
 * phi_2 A_2 as one product of stacked factors), so K must be at most 32.  Fixed-order reductions:
 * bitwise repeatable.  UNSUPPORTED for the fully connected mode, a plan with an in-kernel radial
 * basis, or K > 32. */
cgtp_status_t cgtp_conv_triple_backward(cgtp_plan_t plan, cgtp_graph_t g, const void* x, const void* Y,
                                        const void* phi, const void* A, const void* grad_out, const void* v_x,
                                        const void* v_Y, const void* v_phi, const void* v_A, const void* q_x,
                                        const void* q_Y, const void* q_phi, const void* q_A, const void* q_grad_out,
                                        void* t_x, void* t_Y, void* t_phi, void* t_A, void* t_grad_out, void* t_vx,
                                        void* t_vY, void* t_vphi, void* t_vA, void* workspace, size_t ws_bytes,
                                        void* stream);

/* Check on the device that no edge vector pos[send] - pos[recv] + shift is exactly zero (such an
 * edge has no direction, so its spherical harmonics are undefined).  workspace: device memory of
 * at least 4 bytes per 256 edges (any forward workspace of the plan serves).  Synchronises
 * `stream`.  *first_bad receives the smallest receiver-sorted index of a zero-length edge, else -1;
 * the status is then DEGENERATE_EDGE, else OK.  INVALID_ARG for null plan, graph, pos or
 * first_bad; WORKSPACE if the workspace is too small. */
cgtp_status_t cgtp_check_edges(cgtp_plan_t plan, cgtp_graph_t g, const void* pos, const void* shift,
                               void* workspace, size_t ws_bytes, void* stream, int* first_bad);

/* Feature layout conversion at the boundary.  The convolution entry points take node features
 * in the ir_mul layout (Sobek section 4.4: within an irrep block of multiplicity C and dimension
 * 2l+1 the component index m is the slower one, element offset + m C + u); libraries that store
 * mul_ir (offset + u (2l+1) + m, channel index slower) convert with this call.
 *   side       0: input features (N x C_in, the layout of x and grad_x); 1: output features
 *              (N x C_out, the layout of the output and of grad_out)
 *   direction  0: mul_ir -> ir_mul; 1: ir_mul -> mul_ir
 *   src, dst   device pointers of n_nodes rows in the plan's dtype; caller-owned; must not
 *              overlap (INVALID_ARG when src == dst)
 * Asynchronous on `stream`; a pure permutation of the elements (bit-exact).  INVALID_ARG for a
 * null plan or tensor, a side or direction other than 0/1, or n_nodes < 0. */
cgtp_status_t cgtp_layout_convert(cgtp_plan_t plan, int side, int direction, int n_nodes, const void* src, void* dst,
                                  void* stream);

/* ---------------------------------------------------------------- launch timing */

/* Start timing kernel launches: from now on every kernel the library launches (any plan, any
 * thread) is bracketed by two HIP events recorded on its launch stream.  Costs a few
 * microseconds per launch; leave it off in production timing. */
cgtp_status_t cgtp_profile_begin(void);
/* Stop timing, wait for the recorded events and total the elapsed time per kernel name. */
cgtp_status_t cgtp_profile_end(void);
/* Number of kernel names timed by the last begin/end pair, and the totals of entry `index`:
 * the kernel name (NUL-terminated, truncated to `capacity`), launch count and summed ms. */
int cgtp_profile_count(void);
cgtp_status_t cgtp_profile_get(int index, char* name, int capacity, long long* launches, double* total_ms);

/* ---------------------------------------------------------------- achievable peaks */

/* Measured ceilings of the current device, for roofline fractions beside the published peaks.
 * Plain kernels of this library, timed with HIP events on `stream` (the call synchronises it):
 *   kind 0  fp32 fused multiply-add throughput (16 independent chains per lane, eight waves per
 *           SIMD, no packed instructions), TFLOP/s (2 flop per FMA)
 *   kind 1  the same in fp64, TFLOP/s
 *   kind 2  device copy of `bytes` from src to dst in 16-byte units, counted as bytes read plus
 *           bytes written, GB/s
 * Two untimed launches raise the clocks; `reps` timed launches follow.  *best receives the highest
 * rate, *median (nullable) the median.  dst: caller-owned device memory, at least 8 bytes for
 * kinds 0 and 1 (never written for the values used, kept to make the chains live), `bytes` for
 * kind 2; src: `bytes` of device memory for kind 2 (unused otherwise).  INVALID_ARG for an
 * unknown kind, reps < 1, null best or dst, or (kind 2) null src or bytes not a positive
 * multiple of 16. */
cgtp_status_t cgtp_measure_peak(int kind, void* dst, const void* src, size_t bytes, int reps, void* stream,
                                double* best, double* median);

const char* cgtp_error_string(cgtp_status_t status);
const char* cgtp_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CGTP_H */
