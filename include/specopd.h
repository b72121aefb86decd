/*
 * libspecopd — branch-parallel target scoring for SpecOPD on MI355X (gfx950).
 *
 * The operations, all defined by the pages describing arXiv 2611.02846,
 * "SpecOPD: Branch-Parallel On-Policy Distillation for Speculative Decoding":
 *
 *   specopd_tree_attn_fwd   tree-masked GQA attention of every branch node
 *                           against a trunk key/value cache that was prefilled
 *                           once (jaehun.me review, §3.2(a) and Eq. 5; the
 *                           rustineverything.app summary, §2.1-§2.2).
 *   specopd_e2etv_fwd_bwd   the E2E-TV surrogate over the proposal tree and
 *                           its gradient with respect to the draft logits
 *                           (jaehun.me review, §1.1 and §3.3, Eqs. 8, 9, 13;
 *                           §3.2, Eq. 18; rustineverything.app summary, §2.3).
 *   specopd_prefill_fwd     the causal pass over each trunk that fills that
 *                           cache (jaehun.me review, §3.1 step 1, §3.2(a)).
 *   specopd_gdn_replay_fwd  branch scoring for a linear-attention (GDN)
 *                           target by indexed state replay from trunk
 *                           checkpoints (jaehun.me review, §3.2(c), Fig. 5).
 *   specopd_gdn_conv_fwd    that layer's short convolution for branch nodes,
 *                           its history following the branch's ancestors
 *                           (jaehun.me review, §3.2(c)).
 *   specopd_qsa_trunk_groups_fwd, specopd_qsa_select_fwd
 *                           block selection of a sparse-attention (QSA)
 *                           target with branch-consistent indexer groups
 *                           (jaehun.me review, §3.2(b) and Fig. 4).
 *   specopd_lmhead_e2etv_fwd_bwd
 *                           the E2E-TV surrogate computed from the two
 *                           models' LM heads without storing their logits
 *                           (jaehun.me review, §3.3 and the §3.2(a) reading
 *                           rule).
 *
 * Conventions shared by every entry point:
 *   - Every data pointer is DEVICE memory owned by the caller.  The library
 *     never allocates, frees or keeps a pointer after a call returns.
 *   - Work is enqueued on `stream` (NULL = the default stream) without
 *     synchronising; results are ready when the stream reaches that point.
 *   - Arrays are dense row-major in the layouts stated below.  Outputs are
 *     overwritten (never accumulated) and must not alias inputs.
 *   - Every error that the host can detect (null pointers, sizes, dtypes,
 *     unsupported head size, workspace too small, misalignment) is returned
 *     BEFORE any HIP call is made; nothing is enqueued in that case.
 *   - A failed kernel launch returns SPECOPD_ERR_HIP.  Faults inside kernels
 *     surface at the caller's next synchronisation.
 *   - Malformed tree inputs (anchor outside the trunk, a parent that does not
 *     precede its child, a semantic position that is not anchor + 1 + depth)
 *     are detected on the device: the affected branch's outputs are set to
 *     NaN and a count is kept in the workspace (specopd_*_device_status).
 *   - No global mutable state; calls on different streams may overlap as long
 *     as they use different workspaces.  No C++ exception crosses the ABI.
 */
#ifndef SPECOPD_H
#define SPECOPD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's own stream handle. */
typedef struct ihipStream_t* hipStream_t;

#define SPECOPD_VERSION 2

typedef enum {
  SPECOPD_OK = 0,
  SPECOPD_ERR_INVALID_ARGUMENT = -1, /* null pointer, bad size, bad dtype      */
  SPECOPD_ERR_UNSUPPORTED = -2,      /* valid but not implemented (e.g. D=96) */
  SPECOPD_ERR_WORKSPACE = -3,        /* workspace missing or too small         */
  SPECOPD_ERR_HIP = -4,              /* a HIP runtime call failed              */
  SPECOPD_ERR_DEVICE_VALIDATION = -5 /* malformed tree found on the device     */
} specopd_status;

typedef enum { SPECOPD_F32 = 0, SPECOPD_BF16 = 1 } specopd_dtype;

/* ------------------------------------------------------------------------ */
/* Tree attention                                                            */
/* ------------------------------------------------------------------------ */

/*
 * Problem sizes:  T trunks of length L; B branches per trunk (one anchor
 * each); Wn nodes per branch (1 <= Wn <= 64); Hq query heads and Hkv kv heads
 * (Hq % Hkv == 0, query head h reads kv head h / (Hq/Hkv)); head size D in
 * {64, 128, 256}.  bf16 calls need one trunk's K (L * Hkv * D elements) and
 * one trunk's branch-node keys (B * Wn * Hkv * D elements) under 4 GiB each,
 * else SPECOPD_ERR_UNSUPPORTED.
 */
typedef struct {
  int32_t T, L, B, Wn, Hq, Hkv, D;
  specopd_dtype dtype; /* of trunk_k, trunk_v, q, k, v and out               */
  float rope_base;     /* rotary base; <= 0 means 10000                       */
  float scale;         /* score scale; <= 0 means 1/sqrt(D)                   */
  uint32_t flags;      /* 0 or SPECOPD_TREE_BATCH_INVARIANT                   */
} specopd_tree_attn_desc;

/*
 * Batch-invariant scoring (the deterministic mode behind the jaehun.me
 * review's §3.2 "maintaining numerical consistency" and Table 4, where full
 * recomputation, single and batched cached scoring and merged tree execution
 * agree exactly): with this flag every output row is bitwise the same
 * whatever else is in the call -- its pack partners, the number of branches
 * or trunks, their order.  A row's keys are then always accumulated in one
 * pass over the same 32-key tiles (its trunk keys 0..a_b at their absolute
 * positions, then its own branch's nodes at fixed tile positions), never
 * split into key ranges merged afterwards.  Without the flag, calls with too
 * few (trunk, kv head, pack) units to fill the GPU split long packs into key
 * ranges for speed, and a row's result can then differ in its last bits
 * from the same row scored in another batch.  Calls that fill the GPU are
 * scored the same way with or without the flag.  bf16 matrix-core path only
 * (the fp32 path is batch-invariant always).
 */
#define SPECOPD_TREE_BATCH_INVARIANT 1u

/* Bytes of device workspace specopd_tree_attn_fwd needs for `desc`. */
specopd_status specopd_tree_attn_workspace_size(const specopd_tree_attn_desc* desc,
                                                size_t* bytes);

/*
 * Tree-masked attention (jaehun.me review §3.2(a), Eq. 5): the trunk is
 * prefilled once and cached; every branch node's query is attached to that
 * cache in one batch; node j of branch b in trunk t reads trunk positions
 * 0..anchors[t][b] (inclusive) and the nodes on its own parent chain
 * (itself included) — never a sibling branch, a sibling node or a reference
 * token after the anchor.  Rotary embedding is applied at the node's semantic
 * position pos[t][b][j] = anchors[t][b] + 1 + depth(j) (rustineverything.app
 * summary §2.1), with the rotate-half pairing (i, i + D/2) and angle
 * pos * base^(-2i/D).
 *
 *   trunk_k  [T][L][Hkv][D]     keys of the trunk, ALREADY rotated at their
 *                               trunk positions (a prefilled cache)
 *   trunk_v  [T][L][Hkv][D]     values of the trunk
 *   q        [T][B][Wn][Hq][D]  branch queries, NOT rotated
 *   k, v     [T][B][Wn][Hkv][D] branch keys (NOT rotated) and values
 *   anchors  [T][B]   int32     anchor position a_b, 0 <= a_b < L
 *   parent   [T][B][Wn] int32   -1 for the node attached to the anchor,
 *                               else the index (< j) of the parent node
 *   pos      [T][B][Wn] int32   semantic positions
 *   out      [T][B][Wn][Hq][D]  attention output (dtype of the inputs),
 *                               written for every node, the terminal ones too
 *   workspace / workspace_bytes  device scratch of at least
 *                               specopd_tree_attn_workspace_size bytes,
 *                               16-byte aligned; holds the per-call plan and
 *                               the device validation count
 *
 * bf16 inputs are multiplied on the matrix cores with fp32 accumulation;
 * fp32 inputs use fp32 arithmetic throughout.  All pointers 16-byte aligned.
 */
specopd_status specopd_tree_attn_fwd(const specopd_tree_attn_desc* desc,
                                     const void* trunk_k, const void* trunk_v,
                                     const void* q, const void* k, const void* v,
                                     const int32_t* anchors, const int32_t* parent,
                                     const int32_t* pos, void* out, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/*
 * Which attention row scores which branch token (jaehun.me review §3.2(a) and
 * Fig. 3; rustineverything.app summary §2.2): a row's output predicts the
 * token after it, so the target distribution of branch token j comes from
 * the row of its parent node, and for a token attached to the anchor from
 * the anchor's trunk row; siblings share their parent's row, and a leaf's
 * own row scores nothing.  Score rows are numbered as one matrix: the trunk
 * rows first, then the branch rows,
 *     trunk row s of trunk t       ->  t*L + s
 *     branch row (t, b, j)         ->  T*L + (t*B + b)*Wn + j
 * (the rows of specopd_prefill_fwd's `out` followed by those of
 * specopd_tree_attn_fwd's `out`).  Writes, for every node,
 *   rows  [T][B][Wn] int32   the index of the score row of that token, or
 *                            -1 when the branch is malformed (anchor outside
 *                            the trunk, a parent that does not precede its
 *                            child)
 * Only T, L, B and Wn of `desc` are used (the rest is validated as for
 * specopd_tree_attn_fwd).  `rows` can be passed to specopd_e2etv_fwd_bwd as
 * its target_row, with target_rows = T*L + T*B*Wn.  No workspace.
 */
specopd_status specopd_score_rows(const specopd_tree_attn_desc* desc, const int32_t* anchors,
                                  const int32_t* parent, int32_t* rows, hipStream_t stream);

/*
 * Reads back (synchronising `stream`) how many branches the last
 * specopd_tree_attn_fwd on this workspace found malformed.  Returns
 * SPECOPD_ERR_DEVICE_VALIDATION if that count is non-zero.  `bad_branches`
 * may be NULL.
 */
specopd_status specopd_tree_attn_device_status(const specopd_tree_attn_desc* desc,
                                               const void* workspace, size_t workspace_bytes,
                                               int32_t* bad_branches, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Trunk prefill                                                             */
/* ------------------------------------------------------------------------ */

/*
 * Problem sizes: T trunks of length L >= 1, Hq query heads and Hkv kv heads
 * (Hq % Hkv == 0), head size D in {64, 128, 256}; bf16 calls need one
 * trunk's K (L * Hkv * D elements) under 4 GiB, else SPECOPD_ERR_UNSUPPORTED.
 */
typedef struct {
  int32_t T, L, Hq, Hkv, D;
  specopd_dtype dtype; /* of q, k, v, cache_k, cache_v and out              */
  float rope_base;     /* rotary base; <= 0 means 10000                       */
  float scale;         /* score scale; <= 0 means 1/sqrt(D)                   */
  uint32_t flags;      /* reserved, must be 0                                 */
} specopd_prefill_desc;

specopd_status specopd_prefill_workspace_size(const specopd_prefill_desc* desc, size_t* bytes);

/*
 * The one pass over the reference trajectory that every branch attaches to
 * (jaehun.me review §3.1 step 1 and §3.2(a); rustineverything.app summary
 * §2.2): causal GQA self-attention of each trunk, token s reading tokens
 * 0..s, with rotary embedding at the trunk positions 0..L-1 (the same
 * rotate-half convention as specopd_tree_attn_fwd).  It also leaves the KV
 * cache that specopd_tree_attn_fwd takes as trunk_k / trunk_v.
 *
 *   q        [T][L][Hq][D]   queries, NOT rotated
 *   k, v     [T][L][Hkv][D]  keys (NOT rotated) and values
 *   cache_k  [T][L][Hkv][D]  out: keys rotated at their trunk positions
 *   cache_v  [T][L][Hkv][D]  out: the values, copied
 *   out      [T][L][Hq][D]   out: attention output of every token
 *   workspace / workspace_bytes  device scratch of at least
 *                            specopd_prefill_workspace_size bytes, 16-byte
 *                            aligned
 *
 * Row s >= 1 of a trunk is scored exactly as a one-node branch anchored at
 * s-1 whose key and value are token s's (the specopd_tree_attn_fwd kernels,
 * reading the branch key from the cache just written); row 0 is its own
 * value.  bf16 inputs use the matrix cores with fp32 accumulation; fp32
 * inputs use fp32 arithmetic throughout.  Outputs must not alias inputs or
 * each other.  All pointers 16-byte aligned.
 */
specopd_status specopd_prefill_fwd(const specopd_prefill_desc* desc, const void* q,
                                   const void* k, const void* v, void* cache_k, void* cache_v,
                                   void* out, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Linear-attention (GDN) branch scoring by indexed state replay             */
/* ------------------------------------------------------------------------ */

/*
 * Problem sizes: T trunks of length L, B branches per trunk (one anchor
 * each), Wn nodes per branch (1 <= Wn <= 64), H heads with key and value
 * size D in {64, 128}, a checkpoint after every C trunk tokens
 * (1 <= C <= 64; the pages use 64), so L / C checkpoints per trunk and head.
 * T * L must stay below 2^28.
 */
typedef struct {
  int32_t T, L, B, Wn, H, D, C;
  specopd_dtype dtype; /* of trunk_k, trunk_v, q, k, v; everything else fp32 */
  uint32_t flags;      /* reserved, must be 0                                  */
} specopd_gdn_desc;

/* Workspace bytes (a malformed-branch counter). */
specopd_status specopd_gdn_workspace_size(const specopd_gdn_desc* desc, size_t* bytes);

/*
 * A linear-attention target cannot rewind its recurrent state to an anchor
 * with a mask, so the trunk pass keeps immutable fp32 checkpoints of the
 * state every C tokens; each branch copies the last checkpoint at or before
 * its anchor, replays the trunk tokens after it up to the anchor, then runs
 * its own tokens on that private copy (jaehun.me review, §3.2(c), Fig. 5).
 * The recurrence, per head, is the gated delta rule as published for Gated
 * DeltaNet (the pages name GDN without stating it):
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,
 * with S of [D (value)][D (key)] and keys expected to be unit length.
 * A branch node's state is its parent's (the anchor state for a root)
 * updated with the node's token; its output reads that state with its query.
 *
 *   ckpt        [T][L/C][H][D][D] fp32  checkpoint m: the state after trunk
 *                                       tokens 0..(m+1)C-1 (rows = value
 *                                       dims); may be NULL when L < C
 *   trunk_k, trunk_v  [T][L][H][D]      trunk keys and values
 *   trunk_gate, trunk_beta  [T][L][H]   fp32 decay gate alpha and write
 *                                       strength beta of each trunk token
 *   anchors     [T][B] int32            anchor a: the branch follows trunk
 *                                       tokens 0..a
 *   parent      [T][B][Wn] int32        -1 = attached to the anchor, else an
 *                                       earlier node of the same branch
 *   q, k, v     [T][B][Wn][H][D]        branch node queries, keys, values
 *   gate, beta  [T][B][Wn][H] fp32      branch node alpha and beta
 *   out         [T][B][Wn][H][D] fp32   out: every node's output
 *   workspace / workspace_bytes         specopd_gdn_workspace_size bytes,
 *                                       16-byte aligned
 *
 * The state is replayed in fp32 (the checkpoints' precision); inputs are
 * converted to fp32 on load.  A branch whose anchor is outside [0, L) or
 * whose parent map has a node not preceded by its parent gets NaN outputs
 * and is counted (specopd_gdn_device_status).  All pointers 16-byte
 * aligned; out must not alias an input.
 */
specopd_status specopd_gdn_replay_fwd(const specopd_gdn_desc* desc, const float* ckpt,
                                      const void* trunk_k, const void* trunk_v,
                                      const float* trunk_gate, const float* trunk_beta,
                                      const int32_t* anchors, const int32_t* parent, const void* q,
                                      const void* k, const void* v, const float* gate,
                                      const float* beta, float* out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* Synchronises `stream`; reports how many branches the last
 * specopd_gdn_replay_fwd on this workspace found malformed (returning
 * SPECOPD_ERR_DEVICE_VALIDATION if any).  `bad_branches` may be NULL. */
specopd_status specopd_gdn_device_status(const specopd_gdn_desc* desc, const void* workspace,
                                         size_t workspace_bytes, int32_t* bad_branches,
                                         hipStream_t stream);

/*
 * The layer's short convolution for branch nodes (jaehun.me review, §3.2(c):
 * the convolution history, like the recurrent state, follows only the
 * branch's ancestors).  Gated DeltaNet convolves its projected q, k and v
 * per channel with a causal window of K inputs, applies SiLU (z sigmoid(z))
 * and scales q and k to unit length per head, before the recurrence above.
 * A branch node's K inputs are its own, its ancestors' (nearest first), then
 * trunk tokens a, a-1, ... of its anchor a (zeros before token 0).  One call
 * convolves one of q, k, v:
 *
 *   trunk_x   [T][L][H*D]       the trunk's projected inputs before the
 *                               convolution (tokens a-K+2..a are read)
 *   x         [T][B][Wn][H*D]   the nodes' projected inputs
 *   w         [H*D][K] fp32     w[c][i] multiplies channel c of the i-th
 *                               newest input (i = 0: the node itself)
 *   anchors, parent             as for specopd_gdn_replay_fwd
 *   out       [T][B][Wn][H*D]   out: SiLU(sum_i w[c][i] x_i[c]), computed in
 *                               fp32; with SPECOPD_GDN_CONV_L2NORM each
 *                               head's D values are then divided by
 *                               sqrt(sum of their squares + 1e-6)
 *
 * trunk_x, x and out share desc->dtype.  A node whose window meets a parent
 * that does not precede its child, or whose anchor is outside [0, L), gets
 * NaN outputs (specopd_gdn_replay_fwd on the same parent map counts such
 * branches).  No workspace.  All pointers 16-byte aligned; out must not alias
 * an input.
 */
typedef struct {
  int32_t T, L, B, Wn, H, D; /* as specopd_gdn_desc (D in {64, 128})           */
  int32_t K;                 /* convolution width, 1 <= K <= 8                 */
  specopd_dtype dtype;       /* of trunk_x, x and out                          */
  uint32_t flags;            /* 0 or SPECOPD_GDN_CONV_L2NORM                   */
} specopd_gdn_conv_desc;

#define SPECOPD_GDN_CONV_L2NORM 1u

specopd_status specopd_gdn_conv_fwd(const specopd_gdn_conv_desc* desc, const void* trunk_x,
                                    const void* x, const float* w, const int32_t* anchors,
                                    const int32_t* parent, void* out, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* E2E-TV surrogate                                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t R;                   /* branches                                   */
  int32_t Wn;                  /* nodes per branch, 1 <= Wn <= 64            */
  int32_t V;                   /* vocabulary size, >= 1                      */
  specopd_dtype logits_dtype;  /* draft and target logits                    */
  specopd_dtype grad_dtype;    /* gradient output                            */
  double norm_count;           /* <= 0: R*Wn; else the global count (Eq. 18) */
  float grad_scale;            /* factor applied to the gradient (1 = dLoss) */
  uint32_t flags;              /* 0 or SPECOPD_E2ETV_DEFER_ALL               */
  int32_t wait_polls;          /* bound on a row's polls for its branch; <= 0:
                                  2^20 (see specopd_e2etv_fwd_bwd)           */
  int32_t target_rows;         /* rows of target_logits when target_row is
                                  given (ignored otherwise)                  */
} specopd_e2etv_desc;

/* Every row that needs its branch's scan skips the wait for its siblings and
 * is finished by the follow-up kernel of the same call, exactly as a row
 * whose bounded wait gave up (see wait_polls); the outputs are the same.  It
 * makes that path run on every call, for tests; normal callers pass 0. */
#define SPECOPD_E2ETV_DEFER_ALL 1u

specopd_status specopd_e2etv_workspace_size(const specopd_e2etv_desc* desc, size_t* bytes);

/*
 * E2E-TV (jaehun.me review §3.3, Eqs. 8-9; rustineverything.app summary
 * §2.3).  For row n = r*Wn + j, q = softmax(draft[n]) and p = softmax(target[n])
 * over the FULL vocabulary (Eq. 13: target mass outside the drafter's support
 * is kept).  The acceptance probability is the overlap
 *     alpha_n = sum_v min(q_v, p_v) = 1 - TV(q, p)          (§1.1, Eq. 8)
 * Prefix products run along the parent chain:
 *     P_n = alpha_n * P_parent(n), P of the anchor = 1
 * and the loss is 1 - (sum_n P_n) / count, count = norm_count or R*Wn.
 * The gradient holds the sampled tokens and the target fixed and
 * differentiates only q (§3.3):
 *     grad[n][u] = grad_scale * dLoss/dalpha_n * q_u * ([q_u < p_u] - G_n),
 *     G_n = sum_{v: q_v < p_v} q_v,
 *     dLoss/dalpha_n = -P_parent(n) * S_n / count,
 *     S_n = 1 + sum over children c of n of alpha_c * S_c.
 * At an exact tie q_u == p_u the indicator is 0.
 *
 *   draft_logits [R][Wn][V]     (logits_dtype); -inf allowed
 *   target_logits               (logits_dtype): [R][Wn][V], row n the target
 *                               distribution of node n; or, with target_row,
 *                               [target_rows][V] score rows that nodes share
 *   target_row   [R][Wn] int32  NULL, or the row of target_logits scoring
 *                               each node (e.g. from specopd_score_rows:
 *                               siblings share their parent's row); a row
 *                               outside [0, target_rows) makes its branch
 *                               malformed
 *   parent       [R][Wn] int32  -1 = attached to the anchor, else < j
 *   alpha_out    [R][Wn] float  overlaps, or NULL
 *   prefix_out   [R][Wn] float  prefix products, or NULL
 *   loss_out     double[3]      {loss, numerator sum_n P_n, count}; the
 *                               numerator and count are kept apart so callers
 *                               can normalise across ranks (Eq. 18)
 *   grad_draft   [R][Wn][V]     (grad_dtype), or NULL for forward only
 *   workspace    >= specopd_e2etv_workspace_size bytes, 16-byte aligned
 *
 * Branches with a malformed parent map, a target row outside the target
 * matrix, or an undefined overlap (NaN logits, a row that is -inf
 * everywhere) get NaN alpha/prefix/gradient and are counted
 * (specopd_e2etv_device_status); the loss is then NaN.
 *
 * Scheduling.  Each row is reduced by one workgroup, and a row's gradient
 * needs the overlaps of every row of its branch, so a workgroup waits for
 * the other rows of its branch after posting its own.  That wait is bounded
 * by desc->wait_polls polls (each a few hundred nanoseconds): a row whose
 * branch has not fully posted by then -- because its rows could not run at
 * the same time, e.g. other kernels occupied the CUs -- hands its scan and
 * gradient to a second kernel of the same call, which runs once every row
 * has posted and re-reads that row.  Results are identical either way (the
 * deferred count is reported by specopd_e2etv_device_status); only the time
 * changes.  The wait never fails and never hangs.
 */
specopd_status specopd_e2etv_fwd_bwd(const specopd_e2etv_desc* desc,
                                     const void* draft_logits, const void* target_logits,
                                     const int32_t* target_row, const int32_t* parent,
                                     float* alpha_out,
                                     float* prefix_out, double* loss_out, void* grad_draft,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* Synchronises `stream`; reports how many branches had a malformed parent map
 * in the last specopd_e2etv_fwd_bwd on this workspace (returning
 * SPECOPD_ERR_DEVICE_VALIDATION if any did) and how many rows gave up their
 * wait for their branch and were finished by the second kernel (not an
 * error).  Either output pointer may be NULL. */
specopd_status specopd_e2etv_device_status(const specopd_e2etv_desc* desc,
                                           const void* workspace, size_t workspace_bytes,
                                           int32_t* bad_branches, int32_t* deferred_rows,
                                           hipStream_t stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: the same
 * computation as specopd_e2etv_fwd_bwd, with the workspace taken from a
 * static device array of SPECOPD_E2ETV_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on each GPU it runs on until the process ends.  The call
 * allocates nothing (no hipMalloc, no library allocation); its first call on
 * a GPU looks up that GPU's copy of the array.
 *
 *   Arguments are those of specopd_e2etv_fwd_bwd without the workspace.
 *   Returns SPECOPD_ERR_WORKSPACE, before any HIP call, when the call needs
 *   more than SPECOPD_E2ETV_NOALLOC_SCRATCH_BYTES of workspace
 *   (specopd_e2etv_workspace_size), e.g. more than ~200,000 rows.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (each call clears what must start at zero itself): calls that
 * overlap on one GPU -- on different streams, or from different threads --
 * race and must not be issued.  Malformed branches show as NaN outputs; the
 * device status of this call is not kept for specopd_e2etv_device_status.
 */
#define SPECOPD_E2ETV_NOALLOC_SCRATCH_BYTES (4u << 20)
specopd_status specopd_e2etv_fwd_bwd_noalloc(const specopd_e2etv_desc* desc,
                                             const void* draft_logits, const void* target_logits,
                                             const int32_t* target_row, const int32_t* parent,
                                             float* alpha_out,
                                             float* prefix_out, double* loss_out, void* grad_draft,
                                             hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Sparse attention (QSA): block selection with branch-consistent groups     */
/* ------------------------------------------------------------------------ */

/*
 * A QSA-style sparse layer picks, for each query, blocks of 4 consecutive
 * tokens ("groups") by a compressed indexer key and reads the top-k of them
 * (jaehun.me review, §3.2(b) and its Fig. 4 walk-through).  A group's key is
 * the mean of its 4 tokens' raw indexer keys, RMS-normalised
 * (u / sqrt(mean(u^2) + eps) * gamma), then rotated (rotate-half, base
 * rope_base, as for the attention) at the group's first position.  A query
 * at position p scores every group complete at p, g < floor((p + 1) / 4), by
 * the dot product of that key with its own indexer query rotated at p; the
 * k best are kept, ties going to the lower group, and are returned in
 * increasing group order (all of them when there are at most k).  The tokens
 * of p's incomplete group are the causal tail that attention reads without
 * selection.  One indexer head: the selection serves every attention head.
 *
 * specopd_qsa_trunk_groups_fwd -- the trunk pass's group cache:
 *   trunk_raw [T][L][Di] bf16   raw indexer keys of the trunk tokens
 *   gamma     [Di] fp32         RMSNorm gain
 *   trunk_gk  [T][L/4][Di] bf16 out: the key of every complete trunk group
 *
 * specopd_qsa_select_fwd -- selection for every branch node.  On a branch
 * with anchor a, groups complete at the anchor (g < floor((a + 1) / 4))
 * reuse trunk_gk as given; the group holding the anchor, when incomplete,
 * and every later group are compressed again from the node's own history
 * (itself, its ancestors, then trunk tokens a, a-1, ...), so reference tokens
 * after the anchor never enter a key and the sub-branches of a fork keep
 * groups of their own:
 *   trunk_gk  [T][L/4][Di] bf16 the trunk's group cache (entries of groups
 *                               not complete at an anchor are not read)
 *   trunk_raw [T][L][Di] bf16   trunk raw keys (the boundary groups' tokens)
 *   x, y      [T][B][Wn][Di] bf16  the nodes' raw indexer keys and their
 *                               indexer queries (unrotated)
 *   gamma     [Di] fp32         as above
 *   anchors [T][B], parent and pos [T][B][Wn] int32   as for tree attention
 *   sel       [T][B][Wn][topk] int32  out: selected groups, increasing;
 *                               -1 past the node's number of candidates
 *   score     [T][B][Wn][topk] fp32   out: their scores; -inf past it
 *   bkey      [T][B][Wn][Di] bf16 or NULL  out: the key of the group that
 *                               the node completes (position 3 mod 4), else 0
 * Scores are fp32 sums of products of the bf16-rounded rotated query and
 * key (the matrix cores' arithmetic).  A malformed branch (anchor outside
 * [0, L), a parent that does not precede its child, pos != anchor + 1 +
 * depth) gets sel = -1, NaN scores and zero bkey rows on every node and is counted in the
 * workspace (specopd_qsa_device_status).  Pointers 16-byte aligned; outputs
 * must not alias inputs.  (L + Wn) / 4 above 15360 (a row's candidate
 * scores are held in LDS) gives SPECOPD_ERR_UNSUPPORTED.
 */
typedef struct {
  int32_t T, L, B, Wn; /* Wn <= 64                                      */
  int32_t Di;          /* indexer key size: 64, 128 or 256              */
  int32_t topk;        /* groups kept per node, >= 1                    */
  float rope_base;     /* <= 0 means 10000                              */
  float eps;           /* RMSNorm epsilon; <= 0 means 1e-6              */
  uint32_t flags;      /* 0                                             */
} specopd_qsa_desc;

specopd_status specopd_qsa_trunk_groups_fwd(const specopd_qsa_desc* desc, const void* trunk_raw,
                                            const float* gamma, void* trunk_gk, hipStream_t stream);
specopd_status specopd_qsa_workspace_size(const specopd_qsa_desc* desc, size_t* bytes);
specopd_status specopd_qsa_select_fwd(const specopd_qsa_desc* desc, const void* trunk_gk,
                                      const void* trunk_raw, const void* x, const void* y,
                                      const float* gamma, const int32_t* anchors,
                                      const int32_t* parent, const int32_t* pos, int32_t* sel,
                                      float* score, void* bkey, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);
/* Waits for the stream; SPECOPD_ERR_DEVICE_VALIDATION with *bad_branches > 0
 * when the last select call on this workspace found malformed branches. */
specopd_status specopd_qsa_device_status(const specopd_qsa_desc* desc, const void* workspace,
                                         size_t workspace_bytes, int32_t* bad_branches,
                                         hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* LM head fused with the E2E-TV surrogate                                   */
/* ------------------------------------------------------------------------ */

/*
 * The E2E-TV surrogate of specopd_e2etv_fwd_bwd for logits that are the
 * outputs of two linear LM heads (jaehun.me review, §3.3, Eqs. 8, 9, 13):
 * z = h_draft W_draft^T and t = h_target[target_row] W_target^T, where a
 * node is scored against the target row of its parent, or of its anchor's
 * trunk position for a node on the anchor (the §3.2(a) reading rule, so
 * siblings share one row; specopd_score_rows computes that index).  The
 * logits are formed tile by tile on the matrix cores and never written: the
 * call recomputes them in each of its three passes over the vocabulary
 * (log-sum-exps, overlaps, gradient), three times the head products of
 * forming them once, in exchange for no [N][V] logit traffic or storage.
 *
 *   h_draft    [R][Wn][H] bf16   the drafter's last hidden state per node
 *   w_draft    [V][H] bf16       the drafter's head
 *   h_target   [M][H] bf16       the target's last hidden state per score row
 *   w_target   [V][H] bf16       the target's head (may equal w_draft)
 *   target_row [R][Wn] int32     row of h_target that scores each node
 *   parent     [R][Wn] int32     -1 on the anchor, else an earlier node
 *   alpha_out, prefix_out [R][Wn] fp32 or NULL
 *   loss_out   double[3]         loss, numerator, count (device memory)
 *   grad_draft [R][Wn][V] fp32 or NULL (forward only): dLoss/dz, which a
 *              linear head turns into the hidden-state gradient
 *              (dLoss/dz) W_draft
 * norm_count and grad_scale as for specopd_e2etv_desc.  Logits are fp32
 * sums of bf16 products.  A branch with a parent that does not precede its
 * child, or a node whose target row is outside [0, M), gets NaN outputs
 * and is counted (specopd_lmhead_e2etv_device_status).  H must be a
 * multiple of 16 and each of V*H, M*H and R*Wn*H below 2^31 (else
 * SPECOPD_ERR_UNSUPPORTED); pointers 16-byte aligned; outputs must not alias
 * inputs.
 */
typedef struct {
  int32_t R, Wn;        /* branches, nodes per branch (Wn <= 64)         */
  int32_t V, H;         /* vocabulary, hidden size                      */
  int32_t M;            /* rows of h_target                             */
  double norm_count;    /* <= 0: R * Wn                                 */
  float grad_scale;     /* 1 for the plain gradient                     */
  uint32_t flags;       /* 0                                            */
} specopd_lmhead_e2etv_desc;

specopd_status specopd_lmhead_e2etv_workspace_size(const specopd_lmhead_e2etv_desc* desc, size_t* bytes);
specopd_status specopd_lmhead_e2etv_fwd_bwd(const specopd_lmhead_e2etv_desc* desc, const void* h_draft,
                                            const void* w_draft, const void* h_target,
                                            const void* w_target, const int32_t* target_row,
                                            const int32_t* parent, float* alpha_out, float* prefix_out,
                                            double* loss_out, float* grad_draft, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream);
/* Waits for the stream; SPECOPD_ERR_DEVICE_VALIDATION with *bad > 0 when the
 * last call on this workspace found malformed branches or target rows. */
specopd_status specopd_lmhead_e2etv_device_status(const specopd_lmhead_e2etv_desc* desc,
                                                  const void* workspace, size_t workspace_bytes,
                                                  int32_t* bad, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Kernel timing, for measurement harnesses.
 *
 * specopd_kernel_timing(1) makes every later specopd_tree_attn_fwd,
 * specopd_e2etv_fwd_bwd, specopd_prefill_fwd and specopd_gdn_replay_fwd call
 * record a pair of HIP events on its stream around each launch of its main
 * kernel (the attention kernel proper, after the preparation kernel; the
 * E2E-TV kernel, without the small kernel that clears its counters; the
 * attention kernel of each prefilled trunk; the GDN replay kernel, without
 * the one that clears its counter; the GDN convolution kernel; the QSA
 * scoring kernel and the QSA top-k kernel; the LM head + E2E-TV call from
 * its first pass to its last), so that a harness can divide a kernel's algorithmic work
 * by that kernel's own duration.  specopd_kernel_timing(0) stops recording and
 * discards what was recorded.  The events belong to the library (a pool is
 * created when timing is switched on and kept for the process).
 *
 * specopd_kernel_time(which, &total_ms, &launches): which = 0 attention,
 * 1 E2E-TV, 2 prefill, 3 GDN replay, 4 GDN convolution, 5 QSA scores,
 * 6 QSA top-k, 7 LM head + E2E-TV.  Waits for the recorded events and returns the summed elapsed
 * milliseconds and the number of recorded launches.  Returns
 * SPECOPD_ERR_INVALID_ARGUMENT for another `which` or a null output pointer,
 * SPECOPD_ERR_HIP if an event cannot be created or read.  Not for use while
 * another thread is launching calls of this library. */
specopd_status specopd_kernel_timing(int enable);
specopd_status specopd_kernel_time(int which, double* total_ms, int* launches);

const char* specopd_status_string(specopd_status status);
int specopd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECOPD_H */
