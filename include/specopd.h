/*
 * libspecopd — branch-parallel target scoring for SpecOPD on MI355X (gfx950).
 *
 * Three operations, all defined by the pages describing arXiv 2611.02846,
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

#define SPECOPD_VERSION 1

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
 * {64, 128, 256}.
 */
typedef struct {
  int32_t T, L, B, Wn, Hq, Hkv, D;
  specopd_dtype dtype; /* of trunk_k, trunk_v, q, k, v and out               */
  float rope_base;     /* rotary base; <= 0 means 10000                       */
  float scale;         /* score scale; <= 0 means 1/sqrt(D)                   */
  uint32_t flags;      /* reserved, must be 0                                 */
} specopd_tree_attn_desc;

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
 * (Hq % Hkv == 0), head size D in {64, 128, 256}.
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
  uint32_t flags;              /* reserved, must be 0                        */
} specopd_e2etv_desc;

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
 *   draft_logits, target_logits [R][Wn][V]  (logits_dtype); -inf allowed
 *   parent       [R][Wn] int32  -1 = attached to the anchor, else < j
 *   alpha_out    [R][Wn] float  overlaps, or NULL
 *   prefix_out   [R][Wn] float  prefix products, or NULL
 *   loss_out     double[3]      {loss, numerator sum_n P_n, count}; the
 *                               numerator and count are kept apart so callers
 *                               can normalise across ranks (Eq. 18)
 *   grad_draft   [R][Wn][V]     (grad_dtype), or NULL for forward only
 *   workspace    >= specopd_e2etv_workspace_size bytes, 16-byte aligned
 *
 * Rows whose parent map is malformed get NaN alpha/prefix/gradient and are
 * counted (specopd_e2etv_device_status); the loss is then NaN.
 */
specopd_status specopd_e2etv_fwd_bwd(const specopd_e2etv_desc* desc,
                                     const void* draft_logits, const void* target_logits,
                                     const int32_t* parent, float* alpha_out,
                                     float* prefix_out, double* loss_out, void* grad_draft,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* Synchronises `stream`; reports how many branches had a malformed parent map
 * in the last specopd_e2etv_fwd_bwd on this workspace. */
specopd_status specopd_e2etv_device_status(const specopd_e2etv_desc* desc,
                                           const void* workspace, size_t workspace_bytes,
                                           int32_t* bad_branches, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Kernel timing, for measurement harnesses.
 *
 * specopd_kernel_timing(1) makes every later specopd_tree_attn_fwd,
 * specopd_e2etv_fwd_bwd and specopd_prefill_fwd call record a pair of HIP
 * events on its stream around each launch of its main kernel (the attention
 * kernel proper, after the preparation kernel; the E2E-TV kernel, without
 * the small kernel that clears its counters; the attention kernel of each
 * prefilled trunk), so that a harness can divide a kernel's algorithmic work
 * by that kernel's own duration.  specopd_kernel_timing(0) stops recording and
 * discards what was recorded.  The events belong to the library (a pool is
 * created when timing is switched on and kept for the process).
 *
 * specopd_kernel_time(which, &total_ms, &launches): which = 0 attention,
 * 1 E2E-TV, 2 prefill.  Waits for the recorded events and returns the summed elapsed
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
