/*
 * tree_verify.h -- C ABI of libtreeverify.so: parallel verification of every
 * node of a speculative draft tree through one recurrent linear-attention
 * layer, and reconstruction of only the accepted node's state.  gfx950
 * (MI355X) only.
 *
 * Method (the pages this follows):
 *   - Twig (arXiv 2608.01651 v2) abstract / Bole (v1) abstract: a
 *     tree-structured factorization (closed form) of the linear-attention
 *     recurrence lets one kernel verify all draft nodes in parallel; speculative
 *     state updates are kept as token-level factors and only the accepted
 *     state is rebuilt.
 *   - TreeWY (arXiv 2608.20961) abstract: for the gated delta rule, a
 *     tree-structured WY transform gives every draft node's output from a
 *     single triangular solve and stores a small pseudo-value matrix instead
 *     of per-node states; the accepted state is reconstructed on commit.
 *   - Bole paper-daily auto-summary, core-formula section and worked example:
 *     scalar-decay linear attention S_t = lambda S_{t-1} + k_t v_t^T, its tree
 *     closed form, and the accepted-state rebuild from S_root.
 *
 * Layer (per sequence b and head h; S is d_k x d_v, d_v fastest):
 *   gated delta rule (mode TV_GDN):
 *     S_n = alpha_n (I - beta_n k_n k_n^T) S_parent(n) + beta_n k_n v_n^T
 *   scalar decay (mode TV_SCALAR_DECAY):
 *     S_n = alpha_n S_parent(n) + k_n v_n^T       (alpha_n = lambda_h)
 *   S_parent = S_root for a node whose parent is -1.
 *   output          o_n = S_n^T q_n  (state after node n's own update)
 *   pseudo-value    u_n = beta_n (v_n - alpha_n S_parent^T k_n)   (GDN)
 *                   u_n = v_n                                       (scalar)
 *   so that S_n = alpha_n S_parent + k_n u_n^T and the accepted state is
 *   gamma_a S_root + sum_{j on path(a)} (prod of alpha after j) k_j u_j^T.
 *
 * Conventions for every entry point:
 *   - Array arguments are DEVICE pointers owned by the caller; nothing is
 *     allocated, nothing is kept between calls, calls are re-entrant.
 *   - `stream` is a hipStream_t (NULL = the null stream).  On success the work
 *     is enqueued and the call returns; results are valid once the stream
 *     reaches that point.
 *   - The return value is host-side and synchronous: TV_OK, or a negative
 *     TV_ERR_* code; on any error nothing is launched.  A launch failure
 *     returns -(100 + hipError_t).
 *   - Data errors found on the device go to status[b] (TV_STATUS_*); that
 *     sequence's outputs are then unspecified, but no kernel reads or writes
 *     out of bounds (bad parents are treated as -1, a bad accepted index as 0).
 *   - Preconditions not checked: finite inputs, alpha in (0, 1]; in GDN mode
 *     ||k_n|| <= 1 keeps (I - beta k k^T) non-expansive.
 *   - q is used as given: an attention scale is folded in by the caller.
 *   - N <= TV_MAX_NODES; trees of any shape and depth up to that size are
 *     accepted (the per-node-snapshot baseline takes N <= 128).
 */
#ifndef TREE_VERIFY_H
#define TREE_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TV_MAX_NODES 512

/* dtype of q, k, v and o */
#define TV_F32 0
#define TV_BF16 1

/* layer */
#define TV_GDN 0
#define TV_SCALAR_DECAY 1

/* tree_verify_algo: which kernel solves the tree */
#define TV_ALGO_AUTO 0    /* N <= 128: matrix-core path where it applies, else level-scheduled;
                             N > 128: blocked */
#define TV_ALGO_LEVEL 1   /* level-scheduled forward substitution, fp32 FMA, any d; N <= 128 */
#define TV_ALGO_MFMA 2    /* bf16 matrix cores + per-node path solve; bf16, d_k = d_v = 128,
                             N <= 128 */
#define TV_ALGO_BLOCKED 3 /* one workgroup per (sequence, head): any tree up to TV_MAX_NODES,
                             any depth, any d (matrix-core contraction for bf16 at
                             d_k = d_v = 128).  Trees whose path entries fit on chip are solved
                             through the inverse of I + A (nonzero only on root paths), others
                             in depth-sorted chunks of entries */

/* host return codes */
#define TV_OK 0
#define TV_ERR_NULL (-1)     /* a required pointer is NULL */
#define TV_ERR_DIMS (-2)     /* B, H or N <= 0, N > TV_MAX_NODES (128 for the snapshot
                                baseline), or a size overflows (including one
                                sequence's N H max(d_k, d_v) 4-byte elements
                                past 2^32 bytes) */
#define TV_ERR_HEAD_DIM (-3) /* d_k or d_v not in {16, 32, 64, 128} */
#define TV_ERR_MODE (-4)     /* bad dtype or mode, or beta == NULL in GDN mode */
#define TV_ERR_ALIAS (-5)    /* an output overlaps an input it may not overlap */
#define TV_ERR_ALGO (-6)     /* bad algo, or TV_ALGO_MFMA where it does not apply */
#define TV_ERR_HIP_BASE (-100)

/* device status codes, status[b] */
#define TV_STATUS_OK 0
#define TV_STATUS_BAD_PARENTS 1  /* some parents[b][i] outside [-1, i-1] */
#define TV_STATUS_BAD_ACCEPTED 2 /* accepted[b] outside [0, N) */
#define TV_STATUS_BAD_PREFIX_LEN 3 /* tree_attention: prefix_len[b] outside [0, P_max] (clamped) */

/*
 * tree_verify -- outputs of all N draft nodes of B sequences x H heads in one
 * launch, plus the pseudo-value matrix U that tree_commit needs.
 * Defined by: TreeWY abstract (every draft node's output from one
 * tree-structured WY triangular solve; a small pseudo-value matrix kept in
 * place of per-node states) and Twig abstract (all draft nodes verified in
 * parallel by one kernel); for scalar decay, the Bole auto-summary's core
 * formulas and worked example (node state = decayed root state plus the
 * decayed k v^T terms of its root path).
 *
 *   q, k      [B, N, H, dk]  dtype, contiguous
 *   v         [B, N, H, dv]  dtype, contiguous
 *   alpha     [B, N, H] f32  decay per token (lambda_h broadcast in scalar mode)
 *   beta      [B, N, H] f32  write strength (GDN); ignored, may be NULL, in scalar mode
 *   parents   [B, N] int32   parents[b][i] in [-1, i-1]; -1 hangs node i off S_root
 *   S_root    [B, H, dk, dv] f32   state before the draft tree
 *   o         [B, N, H, dv]  OUT, dtype (bf16 is rounded to nearest even)
 *   U         [B, H, N, dv]  OUT, f32 (U = v in scalar mode)
 *   status    [B] int32      OUT, or NULL
 */
int tree_verify(int B, int H, int N, int dk, int dv, int dtype, int mode, const void* q,
                const void* k, const void* v, const float* alpha, const float* beta,
                const int32_t* parents, const float* S_root, void* o, float* U, int32_t* status,
                void* stream);

/* tree_verify with an explicit solver choice (TV_ALGO_*); same outputs within
 * floating-point rounding.  TV_ERR_ALGO when the choice does not apply to the
 * arguments.  Used by tests to exercise every solver on the same inputs.
 * Defined by: the TreeWY abstract, as tree_verify. */
int tree_verify_algo(int B, int H, int N, int dk, int dv, int dtype, int mode, const void* q,
                     const void* k, const void* v, const float* alpha, const float* beta,
                     const int32_t* parents, const float* S_root, void* o, float* U,
                     int32_t* status, int algo, void* stream);

/*
 * tree_commit -- state after the accepted node of each sequence, from S_root
 * and the token-level factors (k, alpha, U) of that node's root path only.
 * Defined by: TreeWY abstract (only the one accepted state is reconstructed,
 * on commit), Twig abstract (speculative updates kept as token-level factors,
 * only the accepted state rebuilt) and the Bole auto-summary's reconstruction
 * formula and its c3 worked example (the path's per-token factors applied to
 * the old root state).
 *
 *   k         [B, N, H, dk]  dtype     (as passed to tree_verify)
 *   alpha     [B, N, H] f32
 *   U         [B, H, N, dv] f32        (from tree_verify)
 *   parents   [B, N] int32
 *   accepted  [B] int32      node index in [0, N)
 *   S_root    [B, H, dk, dv] f32
 *   S_out     [B, H, dk, dv] f32 OUT;  S_out == S_root (in place) is allowed,
 *                                      any other overlap is TV_ERR_ALIAS
 *   path_out  [B, N] int32   OUT or NULL: accepted node's path, root side
 *                            first, padded with -1 (all -1 for a bad row)
 *   status    [B] int32      OUT or NULL: 1 bad parents, else 2 bad accepted, else 0
 * The caller keeps k, alpha, U and parents alive from tree_verify until this
 * call's work has run.
 */
int tree_commit(int B, int H, int N, int dk, int dv, int dtype, const void* k, const float* alpha,
                const float* U, const int32_t* parents, const int32_t* accepted,
                const float* S_root, float* S_out, int32_t* path_out, int32_t* status,
                void* stream);

/*
 * tree_index -- the tree bookkeeping both kernels do internally, exposed for
 * bit-exact testing.  Defined by: the Bole auto-summary's worked example
 * (each draft node's state follows its own root path; branches may hang
 * directly off the root state) and Twig abstract (the draft is a tree of
 * candidate tokens).
 *   parents [B, N] int32
 *   depth   [B, N] int32 OUT   (parent -1 -> depth 0)
 *   anc     [B, N, (N+63)/64] uint64 OUT: bit j%64 of word j/64 set when node j
 *           is on the root-to-n path, n included
 *   status  [B] int32 OUT or NULL (1 bad parents; that row's depth/anc are 0)
 */
int tree_index(int B, int N, const int32_t* parents, int32_t* depth, uint64_t* anc,
               int32_t* status, void* stream);

/*
 * Per-node-snapshot baseline: the verification method the pages measure
 * against (Twig abstract: existing engines verify the tree sequentially and
 * snapshot the full state of every node; Bole abstract: recurrent layers are
 * traversed branch by branch with a full state materialized per proposal
 * node).  Same layer, same outputs o as tree_verify; kept for comparison on
 * the same hardware and inputs, not as a fast path.
 *
 * tree_verify_snapshot -- visits the nodes of each (sequence, head) in index
 * order, computes S_n from its parent's snapshot (S_root for parent -1) and
 * writes it to snapshots, then o_n = S_n^T q_n.  N <= 128.
 *   q, k, v, alpha, beta, parents, S_root, o, status: as in tree_verify
 *   snapshots [B, H, N, dk, dv] f32 OUT (caller-allocated: B H N dk dv 4 bytes)
 * Bad parents are flagged in status and treated as -1.
 */
int tree_verify_snapshot(int B, int H, int N, int dk, int dv, int dtype, int mode, const void* q,
                         const void* k, const void* v, const float* alpha, const float* beta,
                         const int32_t* parents, const float* S_root, float* snapshots, void* o,
                         int32_t* status, void* stream);

/*
 * tree_commit_snapshot -- the baseline's commit: S_out[b, h] = snapshots[b, h,
 * accepted[b]] (node 0 for a bad accepted index), plus path_out and status
 * with the conventions of tree_commit.  S_out must not overlap snapshots
 * (TV_ERR_ALIAS).  Defined by: Twig abstract and Bole abstract (the engines
 * compared against keep a full state per draft node and take the accepted
 * node's snapshot).
 */
int tree_commit_snapshot(int B, int H, int N, int dk, int dv, const float* snapshots,
                         const int32_t* parents, const int32_t* accepted, float* S_out,
                         int32_t* path_out, int32_t* status, void* stream);

/*
 * tree_commit_verify -- one decoding step with the previous step's commit
 * deferred into this step's verification: exactly
 *
 *   tree_commit(B, H, N_prev, dk, dv, dtype, k_prev, alpha_prev, U_prev,
 *               parents_prev, accepted_prev, S_in, S_out, path_out, commit_status);
 *   tree_verify(B, H, N, dk, dv, dtype, mode, q, k, v, alpha, beta, parents,
 *               S_out, o, U, status);
 *
 * in one pass over the state (TreeWY abstract: only the accepted state is
 * rebuilt, from token-level factors kept at verification; Bole auto-summary,
 * reconstruction formula: that rebuild is the per-token factors of the path
 * applied to the old root state).  For bf16 at d_k = d_v = 128 a single kernel
 * reads S_in once, applies the accepted path's rank-len update in registers,
 * writes S_out and verifies the new tree against it when both trees have at
 * most 128 nodes; other shapes and sizes run the two kernels above in stream
 * order.  Outputs match the two calls within
 * floating-point rounding (S_out to ~2^-24 relative, as tree_commit).
 *
 *   N_prev, k_prev, alpha_prev, U_prev, parents_prev, accepted_prev,
 *   path_out, commit_status: as tree_commit's N, k, alpha, U, parents,
 *                            accepted, path_out, status (previous tree)
 *   S_in      [B, H, dk, dv] f32   state before the previous tree
 *   S_out     [B, H, dk, dv] f32 OUT: committed state, the new tree's root;
 *                                 S_out == S_in (in place) is allowed
 *   N, q, k, v, alpha, beta, parents, o, U, status: as tree_verify (new tree)
 * U must not overlap U_prev, and S_out must not partly overlap S_in
 * (TV_ERR_ALIAS).  Both trees' sizes are checked as in tree_verify.
 */
int tree_commit_verify(int B, int H, int N_prev, int N, int dk, int dv, int dtype, int mode,
                       const void* k_prev, const float* alpha_prev, const float* U_prev,
                       const int32_t* parents_prev, const int32_t* accepted_prev,
                       const float* S_in, float* S_out, int32_t* path_out, int32_t* commit_status,
                       const void* q, const void* k, const void* v, const float* alpha,
                       const float* beta, const int32_t* parents, void* o, float* U,
                       int32_t* status, void* stream);

/*
 * tree_attention -- the full-attention layers of the same hybrid model during
 * the same tree verification (Twig abstract and Bole abstract: full-attention
 * layers with a key/value cache of the committed context are interleaved with
 * the recurrent layers, and verification runs one forward over all draft
 * nodes).  Draft node n sees the committed prefix and the draft nodes on its
 * own root path, itself included, as its recurrent state does (Bole
 * auto-summary worked example); nothing else:
 *
 *   o[b, n, hq] = sum_j softmax_j(scale q[b, n, hq] . k_j) v_j
 *
 * over j in {cache entries 0 .. prefix_len[b]-1 of key/value head hq / (Hq/Hkv)}
 * followed by {draft nodes on n's root path}.  Grouped query heads: Hq must be
 * a multiple of Hkv.  bf16 q/k/v/o, D = 128 only (TV_ERR_HEAD_DIM otherwise,
 * TV_ERR_MODE for another dtype); softmax in fp32, probabilities rounded to
 * bf16 for the value product.
 *
 *   q         [B, N, Hq, D]       bf16
 *   k_cache,
 *   v_cache   [B, Hkv, P_max, D]  bf16, committed context; entries at and past
 *                                 prefix_len[b] are never read; may be NULL
 *                                 when P_max == 0
 *   prefix_len [B] int32          committed length per sequence, 0..P_max
 *   k_tree,
 *   v_tree    [B, N, Hkv, D]      bf16, the draft tokens' own keys and values
 *   parents   [B, N] int32        as tree_verify; N <= TV_MAX_NODES
 *   scale     softmax scale (e.g. 1/sqrt(D))
 *   o         [B, N, Hq, D]       OUT, bf16 (round to nearest even)
 *   status    [B] int32           OUT or NULL: 1 bad parents (treated as -1),
 *                                 else 3 prefix_len out of range (clamped), else 0
 */
int tree_attention(int B, int N, int Hq, int Hkv, int D, int P_max, int dtype, const void* q,
                   const void* k_cache, const void* v_cache, const int32_t* prefix_len,
                   const void* k_tree, const void* v_tree, const int32_t* parents, float scale,
                   void* o, int32_t* status, void* stream);

/* Text for a return code (negative) or a status code (0..3). Never NULL.
 * Library bookkeeping: defined by this header, no passage of the pages. */
const char* tv_status_string(int code);

/* ABI version: major * 100 + minor.
 * Library bookkeeping: defined by this header, no passage of the pages. */
int tv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TREE_VERIFY_H */
