/*
 * gdn_tree.h - C ABI of libgdntree: tree-structured gated-delta-rule (GDN)
 * speculative verification and accepted-path commit on AMD Instinct MI355X
 * (gfx950).
 *
 * What is computed (all citations name the page and the place on it):
 *
 *   Gated delta rule, state S in R^{d_v x d_k} (TreeWY: Speculative
 *   Verification for Gated DeltaNet Hybrids, Sec. 1; Bole review, Sec. 1,
 *   Eq. (1), which stores the same state transposed):
 *       S~ = a_i S_parent,  u = b_i (v_i - S~ k_i),  S_i = S~ + u k_i^T,  o_i = S_i q_i
 *   On a draft tree node i starts from the state of its parent pi(i), not of the
 *   previous packed row (Bole review, Sec. 3.1; GDN Tree-Scan review,
 *   "Background" and the packed-buffer example).  parent = -1 means the
 *   committed state S_pre.
 *
 *   Entry points, in the order one speculative step calls them:
 *     gdn_tree_desc_build   shared descriptor: validation, depth, strict-ancestor
 *                           mask, conv gather sources (LumoTree, Sec. III-C and V-C)
 *     conv_ancestry_gather  causal conv1d whose window for node i is its own
 *                           ancestry, then the conv history (LumoTree, Sec. V-C)
 *     gdn_tree_verify       every node's output o_i; S_pre is read, never written
 *                           (LumoTree, Sec. IV-A; Bole review, Algorithm 2 Phase A)
 *     gdn_tree_commit       replay the accepted root-to-frontier path from S_pre,
 *                           publish the state in place, and publish the conv
 *                           history along the same path (LumoTree, Sec. IV-B and
 *                           V-A; Bole review, Algorithm 2 Phase C)
 *     gdn_tree_commit_layers  the same commit for every layer in one launch
 *   The stored-U alternative to the replay commit:
 *     gdn_tree_verify_store_u, gdn_tree_commit_factored
 *   The steady-state step (commit of the previous path with the conv and the
 *   verify of the next tree), once per step for all layers:
 *     gdn_path_resolve      validate the previous path, resolve its rows
 *     gdn_step_prepare      gdn_tree_desc_build + gdn_path_resolve, one launch
 *   then per layer, either two launches
 *     conv_ancestry_gather_publish, gdn_tree_commit_verify
 *   or one:
 *     gdn_layer_step
 *   The softmax-attention layers of the same model, on the same descriptor:
 *     gdn_tree_attention (+ gdn_tree_attention_workspace_bytes)
 *     gdn_tree_attention_noalloc   the same without a workspace argument
 *     gdn_tree_kv_publish   the accepted path's KV entries after the prefix
 *   Host helpers: gdn_status_string, gdn_abi_version.
 *
 * Conventions shared by every call
 *   - Every pointer is device memory unless the comment says "host".  The
 *     caller owns every buffer; the library allocates nothing and keeps no
 *     mutable global state (reentrant), except the scratch array of
 *     gdn_tree_attention_noalloc (see there).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the library never synchronises with the host.  The caller orders
 *     desc_build -> conv -> verify -> commit on one stream.
 *   - Return value: GDN_OK, or a negative GDN_ERR_* found synchronously before
 *     any launch (bad argument / unsupported size), or GDN_ERR_HIP if a launch
 *     failed.  Nothing is launched when a negative value is returned.
 *   - Data-dependent errors are found on the device and OR-ed (atomic) into the
 *     int32 word `*err` as GDN_EV_* bits; the caller zeroes it.  The request at
 *     fault is skipped as a whole: none of its outputs, state or history is
 *     written, and no kernel reads or writes out of bounds.
 *   - Logical nodes: N per request, 1 <= N <= 64, topologically ordered
 *     (parent[i] < i).  Physical rows: R per request, node i lives in row
 *     node_row[i]; rows no node maps to (padding) are never read or written.
 *   - Row-major layouts; "[B][R][C]" means element (b, r, c) is at
 *     ((b*R + r)*C + c).
 */
#ifndef GDN_TREE_H
#define GDN_TREE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---------------------------------------------------- */
#define GDN_OK 0
#define GDN_ERR_ARG (-1)         /* null pointer, negative size, unknown enum */
#define GDN_ERR_UNSUPPORTED (-4) /* a size the kernels do not implement */
#define GDN_ERR_HIP (-5)         /* a kernel launch failed */

/* ---- device error bits (OR-ed into *err) ------------------------------- */
#define GDN_EV_PARENT 1 /* parent[i] outside [-1, i-1] */
#define GDN_EV_ROW 2    /* node_row[i] outside [0, R) or two nodes share a row */
#define GDN_EV_STATE 4  /* state_idx[b] outside [0, P); commit also: shared by two requests */
#define GDN_EV_PATH 8   /* path_len outside [0, Lmax] or path not a parent chain from a
                           node whose parent is -1 */
#define GDN_EV_CTX 16   /* tree attention / KV publication: ctx_len[b] outside [0, S - R] */

/* ---- operand dtypes and flags ----------------------------------------- */
#define GDN_DT_BF16 0 /* q, k, v are bfloat16 */
#define GDN_DT_F32 1  /* q, k, v are float32 */

#define GDN_F_NORM_QK 1  /* q, k <- x / sqrt(sum x^2 + 1e-6) inside verify and commit */
#define GDN_F_OUT_BF16 2 /* verify writes o as bfloat16 (default float32) */
#define GDN_F_VALU 4     /* verify: force the generic vector-ALU kernel (testing) */
/* Raw gate inputs (LumoTree, Sec. IV-B: the verifier takes raw gate inputs
 * and evaluates the gates in-kernel).  alpha and beta then hold the raw
 * per-node inputs a and b (same layout), and gate_params the per-value-head
 * parameters, float32 [2][Hv] (A_log, then dt_bias); every kernel uses
 *   alpha = exp(-exp(A_log[h]) * softplus(a + dt_bias[h])),
 *   beta  = 1 / (1 + exp(-b)),   softplus(x) = log(1 + exp(x)),
 * evaluated in fp32.  Without the flag gate_params is ignored (may be NULL);
 * with it a NULL gate_params is GDN_ERR_ARG. */
#define GDN_F_RAW_GATES 8
/* gdn_tree_verify_store_u: also write every node's state S_i (the state its
 * output is read from) into the dump argument (debug; see there). */
#define GDN_F_DUMP_STATES 16

#define GDN_ACT_NONE 0
#define GDN_ACT_SILU 1 /* z / (1 + exp(-z)) */

#define GDN_MAX_NODES 64
#define GDN_MAX_CONV_W 4

/* ---- shared tree descriptor (LumoTree, Sec. III-C: parents, depth and the
 *      logical->physical map read by every stage) -------------------------
 * The struct itself is host memory; its arrays are device memory.  With
 * shared = 1 the arrays hold one tree used by all B requests (T = 1),
 * otherwise one tree per request (T = B). */
typedef struct gdn_tree_desc {
    int32_t B;       /* requests, >= 1 */
    int32_t N;       /* logical nodes per request, 1..64 */
    int32_t R;       /* physical rows per request, >= N */
    int32_t W;       /* conv taps, 1..4 (W-1 history entries per request) */
    int32_t shared;  /* 1: one topology for all requests; 0: one per request */
    int32_t reserved;
    const int32_t *parent;   /* in  [T][N]: parent node, -1 = child of S_pre */
    const int32_t *node_row; /* in  [T][N]: physical row of each node */
    int32_t *depth;          /* out [T][N]: nodes on the root-to-i path (1 if parent is -1) */
    uint64_t *anc;           /* out [T][N]: bit j set iff j is a strict ancestor of i */
    int32_t *conv_src;       /* out [T][N][W-1] (may be NULL when W == 1): conv tap
                                sources, oldest first; r >= 0 is physical row r of the
                                request, -(s+1) is conv-history entry s (s = W-2 is the
                                most recent).  Walk: parent, grandparent, ..., then
                                history entries W-2, W-3, ... */
    int32_t *status;         /* out [T]: 0 = valid tree, else GDN_EV_PARENT/GDN_EV_ROW bits */
} gdn_tree_desc;

/* Validate each tree and build depth, anc, conv_src and status.  A tree with
 * a nonzero status gets depth = anc = conv_src = 0 and is skipped by every
 * later call (which then sets no further bit for it).
 * Cite: LumoTree, Sec. III-C (descriptor drives every stage), Sec. V-C (static
 * gather indices from the topology); Bole review, Sec. 3.1 (A(i), strict
 * ancestors) and Algorithm 1 step 4 (ancestor mask M-). */
int32_t gdn_tree_desc_build(const gdn_tree_desc *d, int32_t *err, void *stream);

/* Ancestry-gathered causal conv1d (LumoTree, Sec. V-C: windows from prior
 * conv history and candidate inputs, taps in order oldest -> newest, cast
 * point after the taps):
 *   y[b][row_i][c] = bf16( act( sum_{t<W-1} w[c][t] * X(conv_src[i][t])[c]
 *                               + w[c][W-1] * x[b][row_i][c] + bias[c] ) )
 * X(r >= 0) = x[b][r][c]; X(-(s+1)) = hist[state_idx[b]][s][c].  Accumulation
 * in float32 in that order, one round-to-nearest-even to bf16 at the end.
 *   x     bf16 [B][R][C]      hist bf16 [P][W-1][C] (read only here)
 *   w     bf16 [C][W]         bias float32 [C] or NULL
 *   y     bf16 [B][R][C]      only node rows written
 *   state_idx int32 [B]: history slot of each request (checked against P).
 * C must be a positive multiple of 4; x, hist, y 8-byte aligned.  act is
 * GDN_ACT_NONE or GDN_ACT_SILU. */
int32_t conv_ancestry_gather(const gdn_tree_desc *d, const void *x, const void *hist,
                             int32_t P, const int32_t *state_idx, const void *w,
                             const float *bias, void *y, int32_t C, int32_t act,
                             int32_t *err, void *stream);

/* Tree verify: o_i for every node i and value head h (TreeWY, Sec. 1; Bole
 * review, Sec. 1 Eq. (1) and Sec. 3.1-3.5: the result equals the sequential
 * recurrence from each node's parent, computed without materialising any
 * node's state).
 *   q, k   [B][R] rows; row (b, r) starts at ((b*R + r) * row_stride_qk) and
 *          holds Hqk heads of dk elements (head g at offset g*dk)
 *   v      [B][R] rows of stride row_stride_v, Hv heads of dv elements
 *          (strides let q/k/v alias the conv output: stride C, q at 0,
 *          k at Hqk*dk, v at 2*Hqk*dk)
 *   alpha, beta  float32 [B][R][Hv]: decay a_i and write strength b_i,
 *          already activated (or raw inputs with GDN_F_RAW_GATES)
 *   gate_params  float32 [2][Hv] with GDN_F_RAW_GATES, else ignored
 *   state_pool   float32 [P][Hv][dv][dk]: committed states, read only
 *   state_idx    int32 [B]: pool slot of each request
 *   out    [B][R][Hv][dv] float32 (bf16 with GDN_F_OUT_BF16); node rows only
 * Value head h reads qk head floor(h*Hqk/Hv).  dk == dv in {32, 64, 128};
 * Hv % Hqk == 0.  dtype GDN_DT_BF16 or GDN_DT_F32.  bf16 operands at d = 128
 * run on the matrix cores (fp32 state split into two bf16 halves, fp32
 * accumulation); other shapes, or GDN_F_VALU, run a vector-ALU kernel. */
int32_t gdn_tree_verify(const gdn_tree_desc *d, const void *q, const void *k, const void *v,
                        int64_t row_stride_qk, int64_t row_stride_v, const float *alpha,
                        const float *beta, const float *state_pool, int32_t P,
                        const int32_t *state_idx, void *out, int32_t Hqk, int32_t Hv,
                        int32_t dk, int32_t dv, int32_t dtype, int32_t flags,
                        const float *gate_params, int32_t *err, void *stream);

/* Accepted-path commit (LumoTree, Sec. IV-B: recorded accepted operands are
 * replayed through the gated delta update, in place into the fp32 state bank;
 * Sec. V-A: one device path drives recurrent replay and conv publication,
 * padded path entries never advance state; Bole review, Algorithm 2 step 8:
 * nothing accepted leaves the state as it was).
 *   path      int32 [B][Lmax]: logical node ids, root-level node first; must
 *             satisfy parent[path[0]] == -1 and parent[path[j]] == path[j-1]
 *   path_len  int32 [B]: 0..Lmax; 0 leaves state and history untouched
 *   k, v, alpha, beta, row strides, Hqk, Hv, dk, dv, dtype: as in verify (the
 *             same buffers verify read)
 *   state_pool float32 [P][Hv][dv][dk], updated in place for slot state_idx[b]
 *   x, hist   optional (both NULL or both set; ignored when the descriptor's
 *             W is 1): conv input bf16 [B][R][C] and conv history bf16
 *             [P][W-1][C]; the history of slot state_idx[b] becomes the last
 *             W-1 entries of (old history ++ x rows of the path).
 * flags: GDN_F_NORM_QK, GDN_F_RAW_GATES (both must match verify; gate_params
 * as in verify).  state_idx values must be distinct across requests (a
 * shared slot is GDN_EV_STATE for both). */
int32_t gdn_tree_commit(const gdn_tree_desc *d, const int32_t *path, const int32_t *path_len,
                        int32_t Lmax, const void *k, const void *v, int64_t row_stride_qk,
                        int64_t row_stride_v, const float *alpha, const float *beta,
                        float *state_pool, int32_t P, const int32_t *state_idx,
                        const void *x, void *hist, int32_t C, int32_t Hqk, int32_t Hv,
                        int32_t dk, int32_t dv, int32_t dtype, int32_t flags,
                        const float *gate_params, int32_t *err, void *stream);

/* ---- stored-U mode (alternative to the replay commit) ---------------------
 * Bole review, Sec. 5.2 (Algorithm 2 keeps the corrections U of its verify,
 * Phase A, and publishes the accepted frontier's state from them, Phase C,
 * by Eq. (10)); TreeWY, Sec. 3 (the same factored publish from
 * pseudo-values).  The verify writes, besides o, every node's delta
 * correction
 *     u_i = b_i (v_i - a_i S_parent k^_i)
 * (the rows of U in (I + G) U = R, Bole review, Lemma 2), and the commit
 * rebuilds the frontier's state without replaying the path:
 *     S_new = P_a S_pre + sum_{j on the path} (P_a / P_j) u_j k^_j^T
 * (a the frontier, P_x the product of the decays on the root-to-x path).
 * The stored U costs a write of B*R*Hv*dv*4 bytes per verify; the replay
 * commit stores nothing. */

/* gdn_tree_verify, plus u: float32 [B][R][Hv][dv], node rows written (the
 * layout of a float32 out).  bf16 operands at d = 128 with N <= 32 run on the
 * matrix cores (W = (I + G)^-1 solved along each root path beside M, then
 * U = W R), other shapes on the vector ALU.  Arguments, flags and errors as
 * gdn_tree_verify; u 4-byte aligned.
 *   dump  with GDN_F_DUMP_STATES (debug only; else ignored, may be NULL):
 *         float32 [B][N][Hv][dv][dk], indexed by logical node, 16-byte
 *         aligned; receives every node's state
 *             S_i = P_i S_pre + sum_{j on i's root path} (P_i / P_j) u_j k^_j^T,
 *         the state o_i = S_i q^_i is read from, rebuilt from the u just
 *         written by the factored commit's arithmetic (so a factored commit
 *         of i's root path reproduces dump[b][i] bit for bit, and a replay
 *         commit can be compared against it: LumoTree, Sec. IV-B, the replay
 *         and the verifier may differ numerically).  bf16 at d = 128 only
 *         (else GDN_ERR_UNSUPPORTED); k 8-byte aligned with row_stride_qk a
 *         multiple of 4, u 16-byte aligned.  Writes B*N*Hv*dv*dk*4 bytes. */
int32_t gdn_tree_verify_store_u(const gdn_tree_desc *d, const void *q, const void *k, const void *v,
                                int64_t row_stride_qk, int64_t row_stride_v, const float *alpha,
                                const float *beta, const float *state_pool, int32_t P,
                                const int32_t *state_idx, void *out, float *u, float *dump,
                                int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv, int32_t dtype,
                                int32_t flags, const float *gate_params, int32_t *err, void *stream);

/* Commit of the accepted path from stored corrections, in place: one rank-8
 * matrix-core update of P_a S_pre per 8 path nodes, no sequential replay.
 *   path, path_len, Lmax, state_pool, P, state_idx, err: as gdn_tree_commit
 *   (same validation and error bits; len 0 leaves the state untouched)
 *   k, row_stride_qk  the bf16 k rows the verify read (dk = dv = 128; k
 *            8-byte aligned, stride a multiple of 4)
 *   u        float32 [B][R][Hv][128] as gdn_tree_verify_store_u wrote it
 *            (16-byte aligned)
 *   alpha    float32 [B][R][Hv] (raw inputs with GDN_F_RAW_GATES)
 * flags: GDN_F_NORM_QK, GDN_F_RAW_GATES (as the verify; gate_params as
 * there).  No conv history: that publication goes through gdn_tree_commit
 * or the fused calls. */
int32_t gdn_tree_commit_factored(const gdn_tree_desc *d, const int32_t *path, const int32_t *path_len,
                                 int32_t Lmax, const void *k, int64_t row_stride_qk, const float *u,
                                 const float *alpha, float *state_pool, int32_t P,
                                 const int32_t *state_idx, int32_t Hqk, int32_t Hv, int32_t dk,
                                 int32_t dv, int32_t flags, const float *gate_params, int32_t *err,
                                 void *stream);

/* Commit of one accepted path into L layers' states in one launch (technical
 * review of Bole, Sec. 7, unified cross-layer state commit: one batched
 * launch after acceptance for every recurrent layer; LumoTree, Sec. IV-B and
 * V-A: one accepted path drives every layer's publication -- the same tree,
 * path and slots for every layer).  Layer
 * l's k, v, gates and state pool are the given buffers offset by l times the
 * layer strides, in elements; each layer's buffers follow gdn_tree_commit's
 * layouts and must not overlap the next layer's.  The result equals
 * gdn_tree_commit called once per layer (without conv history: x / hist are
 * per layer and go through gdn_tree_commit or the fused calls).
 *   layers            1..; B * Hv * layers < 2^31
 *   layer_stride_qk   >= B * R * row_stride_qk (k), layer_stride_v likewise
 *   layer_stride_gate >= B * R * Hv (alpha and beta)
 *   layer_stride_pool >= P * Hv * dv * dk, a multiple of 4 (16-byte alignment)
 *   gate_params       with GDN_F_RAW_GATES: float32 [layers][2][Hv], each
 *                     layer's A_log and dt_bias */
int32_t gdn_tree_commit_layers(const gdn_tree_desc *d, const int32_t *path,
                               const int32_t *path_len, int32_t Lmax, int32_t layers,
                               const void *k, const void *v, int64_t row_stride_qk,
                               int64_t row_stride_v, int64_t layer_stride_qk,
                               int64_t layer_stride_v, const float *alpha, const float *beta,
                               int64_t layer_stride_gate, float *state_pool,
                               int64_t layer_stride_pool, int32_t P, const int32_t *state_idx,
                               int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv, int32_t dtype,
                               int32_t flags, const float *gate_params, int32_t *err,
                               void *stream);

/* ---- fused steady-state step ---------------------------------------------
 * In a decode loop every step commits the previous step's accepted path and
 * then verifies a new tree from the committed state (LumoTree, Sec. IV-B and
 * V-A: the accepted path's recorded operands are replayed into the state
 * bank, and the same path drives the conv-history publication).  After
 * gdn_path_resolve (or gdn_step_prepare) of the previous tree and path, the
 * two calls below do exactly
 *     gdn_tree_commit(d_prev, path, ...);  conv_ancestry_gather(d, ...);
 *     gdn_tree_verify(d, ...)
 * in two launches instead of three, with the state read once and written
 * once per step instead of read twice and written once:
 *   conv_ancestry_gather_publish   publishes the conv history of the
 *                                  previous path, then convolves the new tree
 *   gdn_tree_commit_verify         replays the previous path into the state,
 *                                  writes it, and verifies the new tree from it
 * The previous path is passed resolved: path_rows [B][Lmax] and path_n [B]
 * as gdn_path_resolve wrote them for d_prev (values are clamped into range
 * before use).  The resolution reports the path's errors: a malformed
 * previous path (GDN_EV_PATH, n_b = 0) or a slot out of range or shared by
 * two requests (GDN_EV_STATE, n_b = -1) publishes and commits nothing for
 * that request, which is then convolved and verified from its unchanged
 * history and state; a malformed new tree still has its previous path
 * committed and published.  Other "previous" arguments are the operands
 * recorded for the previous tree (its q/k/v rows, gates and conv input). */

/* Conv with publication.  For each request with n_b > 0, hist[state_idx[b]]
 * first becomes the last W-1 entries of (hist ++ x_prev rows of the path);
 * then y is the conv of d's tree over that history, as in
 * conv_ancestry_gather.  hist is read and written in place.
 *   d_prev   the previous step's tree (d_prev->B == d->B, d_prev->W == d->W)
 *   path_rows [B][Lmax], path_n [B], Lmax: the previous path, resolved
 *   x_prev   bf16 [B][d_prev->R][C]: the previous step's conv input
 * Other arguments and requirements as in conv_ancestry_gather (x_prev 8-byte
 * aligned like x). */
int32_t conv_ancestry_gather_publish(const gdn_tree_desc *d, const void *x, void *hist,
                                     int32_t P, const int32_t *state_idx, const void *w,
                                     const float *bias, void *y, int32_t C, int32_t act,
                                     const gdn_tree_desc *d_prev, const int32_t *path_rows,
                                     const int32_t *path_n, int32_t Lmax, const void *x_prev,
                                     int32_t *err, void *stream);

/* Commit of the previous path, then verify of d's tree from the committed
 * state.  state_pool is updated in place (as gdn_tree_commit does, without
 * the history, which conv_ancestry_gather_publish handles) and out receives
 * d's outputs (as gdn_tree_verify).
 *   q, k, v, strides, alpha, beta, out, flags, gate_params: the new tree,
 *            as in verify (with GDN_F_RAW_GATES the previous tree's gates
 *            are raw inputs too, of the same layer's gate_params)
 *   k_prev, v_prev, row strides, alpha_prev, beta_prev: the operands
 *            recorded for the previous tree (same layout rules)
 *   d_prev, path_rows, path_n, Lmax: the previous tree and its path, resolved
 * bf16 operands at d = 128 run as one matrix-core kernel; other shapes run
 * the commit and verify kernels one after the other. */
int32_t gdn_tree_commit_verify(const gdn_tree_desc *d, const void *q, const void *k,
                               const void *v, int64_t row_stride_qk, int64_t row_stride_v,
                               const float *alpha, const float *beta, float *state_pool,
                               int32_t P, const int32_t *state_idx, void *out,
                               const gdn_tree_desc *d_prev, const int32_t *path_rows,
                               const int32_t *path_n, int32_t Lmax, const void *k_prev,
                               const void *v_prev, int64_t row_stride_qk_prev,
                               int64_t row_stride_v_prev, const float *alpha_prev,
                               const float *beta_prev, int32_t Hqk, int32_t Hv, int32_t dk,
                               int32_t dv, int32_t dtype, int32_t flags,
                               const float *gate_params, int32_t *err, void *stream);

/* ---- one launch per layer ------------------------------------------------
 * A model runs the same step for every GDN layer: commit the previous step's
 * accepted path, publish its conv history, convolve and verify the new tree.
 * Everything that depends only on the trees and the path (validation, the
 * path's physical rows) is done once per step by gdn_path_resolve; each
 * layer is then one launch of gdn_layer_step, which keeps a (request, head)
 * pair's whole step on one workgroup: the conv output q/k/v never goes to
 * memory, and the previous path's k/v are recomputed from its conv input
 * (the same conv, so the same bf16 values the previous step verified with)
 * instead of being stored (LumoTree, Sec. IV-B: replay of the accepted
 * operands; Sec. V-A: one path drives replay and conv publication; Sec. V-C:
 * the conv window of a node is its ancestry, then the history). */

/* Validate the previous step's accepted path against its tree and resolve it
 * to physical rows, once per step for all layers.
 *   d_prev      the previous step's descriptor (built; its status is read)
 *   path, path_len, Lmax: as in gdn_tree_commit (1 <= Lmax <= 64)
 *   state_idx   int32 [B], checked against P and for slots shared by two
 *               requests
 *   path_rows   out int32 [B][Lmax]: node_row of path[b][j] for j < n_b;
 *               other entries are left as they were
 *   path_n      out int32 [B]: n_b = path_len[b] when the path validates;
 *               0 when path_len[b] is 0, when the previous tree is malformed
 *               (reported by its own descriptor build) or when the path is
 *               malformed (GDN_EV_PATH); -1 when state_idx[b] is outside
 *               [0, P) or shared with another request (GDN_EV_STATE)
 * Cite: LumoTree, Sec. V-A (one device-produced path drives every
 * publication; padded entries never advance state). */
int32_t gdn_path_resolve(const gdn_tree_desc *d_prev, const int32_t *path,
                         const int32_t *path_len, int32_t Lmax, const int32_t *state_idx,
                         int32_t P, int32_t *path_rows, int32_t *path_n, int32_t *err,
                         void *stream);

/* gdn_tree_desc_build(d) and gdn_path_resolve(d_prev, ...) in one launch:
 * the step's shared work for every layer (d_prev->B == d->B).  Arguments,
 * outputs and errors are those of the two calls. */
int32_t gdn_step_prepare(const gdn_tree_desc *d, const gdn_tree_desc *d_prev,
                         const int32_t *path, const int32_t *path_len, int32_t Lmax,
                         const int32_t *state_idx, int32_t P, int32_t *path_rows,
                         int32_t *path_n, int32_t *err, void *stream);

/* One GDN layer's step in one launch.  With hist = hist_in copied to
 * hist_out first, it computes what these calls compute in order:
 *     y_prev = conv_ancestry_gather(d_prev, x_prev, hist)      (path rows only)
 *     gdn_tree_commit(d_prev, path, k/v of y_prev, alpha_prev, beta_prev,
 *                     state_pool, x_prev, hist)                 (state, history)
 *     y = conv_ancestry_gather(d, x, hist);  gdn_tree_verify(d, q/k/v of y, ...)
 * where the path is the one gdn_path_resolve resolved into path_rows/path_n.
 *   x         bf16 [B][d->R][C], C = 2*Hqk*128 + Hv*128, channels [q | k | v]
 *             head-major (qk head g: q at g*128, k at Hqk*128 + g*128; value
 *             head h: v at 2*Hqk*128 + h*128)
 *   w, bias, act: conv weights bf16 [C][W], bias float32 [C] or NULL,
 *             GDN_ACT_NONE / GDN_ACT_SILU; W = d->W
 *   hist_in   bf16 [P][W-1][C]: the history the previous step's tree was
 *             convolved with; read only
 *   hist_out  bf16 [P][W-1][C]: written for every request with n_b >= 0:
 *             the last W-1 entries of (hist_in ++ x_prev rows of the path);
 *             must not overlap hist_in.  The next step passes it as hist_in.
 *             Both may be NULL when W == 1.
 *   alpha, beta   float32 [B][d->R][Hv]: gates of the new tree
 *   state_pool float32 [P][Hv][128][128], slot state_idx[b]: read, and
 *             written with the committed state when n_b > 0
 *   out       [B][d->R][Hv][128] float32 (bf16 with GDN_F_OUT_BF16)
 *   y         optional (NULL: not written) bf16 [B][d->R][C]: the new tree's
 *             conv output, node rows only
 *   d_prev, x_prev bf16 [B][d_prev->R][C], alpha_prev, beta_prev float32
 *             [B][d_prev->R][Hv]: the previous step's tree, conv input and
 *             gates (read at path rows only, but must be valid buffers even
 *             when every n_b is 0)
 *   path_rows, path_n, Lmax: from gdn_path_resolve (values are clamped into
 *             range before use, so no access leaves the buffers)
 * Requirements: bf16, dk = dv = 128, d->N <= 32, d_prev->B == d->B,
 * 1 <= Lmax <= 64, x, x_prev, hist_in, hist_out 16-byte aligned, state_pool
 * 16-byte aligned.  flags: GDN_F_NORM_QK, GDN_F_OUT_BF16, GDN_F_RAW_GATES
 * (gate_params as in verify; both trees' gates raw).  Errors: a
 * malformed new tree gets no outputs (its path is still committed and its
 * history published); n_b = -1 writes neither state nor history. */
int32_t gdn_layer_step(const gdn_tree_desc *d, const void *x, const void *w, const float *bias,
                       int32_t act, const void *hist_in, void *hist_out, const float *alpha,
                       const float *beta, float *state_pool, int32_t P,
                       const int32_t *state_idx, void *out, void *y,
                       const gdn_tree_desc *d_prev, const void *x_prev,
                       const float *alpha_prev, const float *beta_prev,
                       const int32_t *path_rows, const int32_t *path_n, int32_t Lmax,
                       int32_t Hqk, int32_t Hv, int32_t dk, int32_t dv, int32_t flags,
                       const float *gate_params, int32_t *err, void *stream);

/* ---- tree attention (the softmax-attention layers of the same model) -----
 * LumoTree, Sec. III-C and V-B: query rows stay in logical node order; the
 * candidates' keys and values are written into the KV cache after the
 * committed prefix at physical slots given by the descriptor's slot map
 * (node_row), and the ancestry mask names which of them a node sees -- its
 * own slot and its ancestors' -- on top of the whole prefix.  Publication
 * moves the accepted path's entries through the same slot map to the
 * continuation positions right after the prefix. */

/* Bytes of the workspace gdn_tree_attention needs (split partial results). */
size_t gdn_tree_attention_workspace_bytes(int32_t B, int32_t N, int32_t Hq, int32_t D,
                                          int32_t splits);

/* o[b][i][h] = sum_j softmax_j(scale * q[b][i][h] . k_j) v_j over the keys
 * node i sees: positions 0 .. ctx_len[b]-1 and ctx_len[b] + node_row[a] for
 * every a on i's root path.  Query head h reads kv head h / (Hq / Hkv).
 *   q        bf16 [B][N][Hq][D], logical node rows
 *   k_cache, v_cache  bf16 [B][S][Hkv][D]; the candidates' entries are
 *            already written at ctx_len[b] + node_row
 *   ctx_len  int32 [B], each in [0, S - R] (else GDN_EV_CTX, request skipped)
 *   out      [B][N][Hq][D] float32 (bfloat16 with GDN_F_OUT_BF16); rows of
 *            skipped requests (malformed tree, bad ctx_len) are not written
 *   workspace, workspace_bytes: device scratch of at least
 *            gdn_tree_attention_workspace_bytes(B, N, Hq, D, splits) bytes,
 *            16-byte aligned, owned by the caller; its contents on entry do
 *            not matter
 *   splits   1..1024: partitions of the prefix (each an equal share of
 *            S - R positions), plus one for the candidates
 *   scale    softmax scale (e.g. 1 / sqrt(D)); positive, with scale * log2(e)
 *            finite (else GDN_ERR_ARG)
 * bf16, D in {128, 256}, N <= 64, R <= 64, Hq % Hkv == 0; q, k_cache,
 * v_cache 16-byte aligned.  flags: GDN_F_OUT_BF16. */
int32_t gdn_tree_attention(const gdn_tree_desc *d, const void *q, const void *k_cache,
                           const void *v_cache, int32_t S, const int32_t *ctx_len, void *out,
                           void *workspace, size_t workspace_bytes, int32_t splits, int32_t Hq,
                           int32_t Hkv, int32_t D, float scale, int32_t flags, int32_t *err,
                           void *stream);

/* gdn_tree_attention without the workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The split partial results go to
 * a scratch array inside the library (GDN_ATTN_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the library's load until the process ends); the call allocates
 * nothing.  Arguments and errors are those of gdn_tree_attention, plus
 * GDN_ERR_UNSUPPORTED (nothing launched) when
 * gdn_tree_attention_workspace_bytes(B, N, Hq, D, splits) exceeds the
 * scratch size.  Every call on one GPU uses the same scratch: calls that
 * overlap on a GPU (other streams, other threads) race and must be ordered
 * by the caller.  The scratch's contents on entry do not matter. */
#define GDN_ATTN_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
int32_t gdn_tree_attention_noalloc(const gdn_tree_desc *d, const void *q, const void *k_cache,
                                   const void *v_cache, int32_t S, const int32_t *ctx_len,
                                   void *out, int32_t splits, int32_t Hq, int32_t Hkv, int32_t D,
                                   float scale, int32_t flags, int32_t *err, void *stream);

/* KV publication of the accepted path: for every request with n_b =
 * path_n[b] > 0, cache positions ctx_len[b] + j (j < n_b) receive the
 * entries at ctx_len[b] + path_rows[b][j] (every source is read before any
 * destination is written), in k_cache and v_cache, all kv heads.
 *   d_prev   the tree the path was accepted from (its B and R)
 *   path_rows, path_n, Lmax: the path resolved by gdn_path_resolve or
 *            gdn_step_prepare (rows are clamped into [0, R) before use)
 *   k_cache, v_cache, S, ctx_len, Hkv, D: as in gdn_tree_attention
 * The caller then advances ctx_len by n_b.  ctx_len outside [0, S - R] is
 * GDN_EV_CTX and leaves the request's cache alone. */
int32_t gdn_tree_kv_publish(const gdn_tree_desc *d_prev, const int32_t *path_rows,
                            const int32_t *path_n, int32_t Lmax, void *k_cache, void *v_cache,
                            int32_t S, const int32_t *ctx_len, int32_t Hkv, int32_t D,
                            int32_t *err, void *stream);

/* Human-readable name of a return code (host; static string). */
const char *gdn_status_string(int32_t status);

/* ABI version of this header: 8 (1, plus the two fused-step calls in 2,
 * plus gdn_path_resolve, gdn_step_prepare and gdn_layer_step in 3, plus
 * gdn_tree_commit_layers in 4, plus GDN_F_RAW_GATES and the gate_params
 * argument of verify, commit and the fused calls in 5, plus tree attention
 * and KV publication in 6, plus gdn_tree_attention_noalloc in 7, plus
 * gdn_tree_verify_store_u and gdn_tree_commit_factored). */
int32_t gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_TREE_H */
