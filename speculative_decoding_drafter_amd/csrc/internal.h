// Internal interface between the C-ABI front end (specopd_api.cpp) and the
// kernel launchers (*.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/specopd.h"

namespace specopd {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- tree attention
// Workspace layout (offsets in bytes, each 256-aligned):
//   anc        uint64 [T*B*Wn]   ancestor bitmask of every node (self included)
//   branch_ok  int32  [T*B]      1 = well formed, 0 = malformed (outputs NaN)
//   order      int32  [T*B]      branches of each trunk by anchor, longest first
//   rot        rotated branch queries and keys
//   pstart     int32  [T][npacks+1]  first key tile of each pack (prefix sums)
//   ctr        int32  [T][Hkv][npacks]  splits of a pack that finished
//   qctr       u64    [8]        unit-queue counters of the matrix-core kernel
//   part       partial results, one slot per (pack, split) when packs are split
struct TreeAttnWs {
  size_t anc, branch_ok, order, rot, pstart, ustart, umap, ctr, qctr, part, total;
};
TreeAttnWs tree_attn_ws_layout(const specopd_tree_attn_desc& d);

struct TreeAttnArgs {
  const void *trunk_k, *trunk_v, *q, *k, *v;
  const int32_t *anchors, *parent, *pos;
  void* out;
  char* ws;
  float rope_base, scale;
  int timing_kind;  // call kind the attention kernel is timed as (timing_mark)
};
hipError_t launch_tree_attn(const specopd_tree_attn_desc& d, const TreeAttnArgs& a, hipStream_t s);
// Score row of every branch node (specopd_score_rows).
hipError_t launch_score_rows(const specopd_tree_attn_desc& d, const int32_t* anchors,
                             const int32_t* parent, int32_t* rows, hipStream_t s);

// Matrix-core path (tree_attn_mfma.hip).  bf16 tensors are passed as uint16_t.
// Four waves per workgroup, one per SIMD, so that a wave may hold 512
// registers.  A wave owns two blocks of 32 rows for head sizes 64 and 128:
// each K and V operand read from LDS then feeds two matrix products, which
// halves the LDS traffic per flop (with one block per wave, LDS bandwidth
// and not the matrix cores sets the pace).  Head size 256 keeps one block:
// two would not fit the registers.
constexpr int mfma_waves(int) { return 4; }
constexpr int mfma_row_blocks(int D) { return D == 256 ? 1 : 2; }
constexpr int mfma_rows_per_wg(int D) { return mfma_waves(D) * 32 * mfma_row_blocks(D); }
size_t mfma_slot_bytes(int D);
// Key-range splits per pack: packs are split only when there are too few of
// them to give every CU one workgroup (a workgroup fills a CU, and merging
// split partials costs more than a second round of workgroups saves).
inline int mfma_nsplit(long long units, bool batch_invariant = false) {
  if (units >= 256 || batch_invariant) return 1;
  const long long s = (256 + units - 1) / units;
  return int(s < 16 ? s : 16);
}

struct MfmaParams {
  const uint16_t *trunk_k, *trunk_v;  // [T][L][Hkv][D]
  const uint16_t* qr;                 // rotated, scaled queries [T][B][Wn][Hq][D]
  const uint16_t* kr;                 // rotated branch keys [T][B][Wn][Hkv][D]
  const uint16_t* v;                  // branch values [T][B][Wn][Hkv][D]
  const int32_t* anchors;             // [T][B]
  const uint64_t* anc;                // ancestor bitmasks [T][B][Wn]
  const int32_t* branch_ok;           // [T][B]
  const int32_t* order;               // [T][B] branches by anchor, longest first
  const int32_t* pstart;              // [T][npacks+1]
  const int32_t* ustart;              // [T][npacks+1] first unit of each pack (per kv head)
  const int32_t* umap;                // [T][npacks*nsplit] pack of each unit
  int32_t* ctr;                       // [T][Hkv][npacks], zero on entry
  unsigned long long* qctr;           // [8] unit-queue counters, zero on entry
  char* part;                         // nunits slots of slot_bytes (nsplit > 1)
  size_t slot_bytes;
  uint16_t* out;                      // [T][B][Wn][Hq][D]
  int T, B, L, Wn, Hq, Hkv, G;
  int bpp;     // branches per pack
  int spb;     // packs per branch (> 1 when a branch has more rows than a workgroup; bpp is 1 then)
  int tstride; // tail keys per branch slot (Wn rounded up so each slot starts where a lone
               // branch's would: a row's tail keys sit at the same tile positions in any pack)
  int npacks;  // packs per trunk
  int nsplit;  // key-range splits per pack
  int ugp;      // units per (trunk, kv head) group, padded to a multiple of ilv
  int nunits;   // T * Hkv * ugp
  int nwg;      // workgroups: nunits rounded up to a multiple of 8
  int ilv;      // XCD blocks a group's units are dealt across (1: none)
  int chunked;  // 1: consecutive units to one XCD; 0: units by block index
};
// Tail keys per branch slot of a tree call: the branch's Wn nodes from a
// multiple of 16 (32, 64 for larger branches), so that in any pack a row's
// own nodes occupy the same positions of a 32-key tile and of its 16-key
// matrix-core steps as they would with the branch alone.
inline int mfma_tail_stride(int Wn) { return Wn <= 16 ? 16 : Wn <= 32 ? 32 : 64; }
// Key tiles of a pack whose longest anchor is `a` (-1: none well formed)
// holding `nbr` branch slots of `tstride` keys, the last one Wn keys.
__host__ __device__ inline int mfma_pack_tiles(int a, int nbr, int tstride, int Wn) {
  return (a + 32) / 32 + ((nbr - 1) * tstride + Wn + 31) / 32;
}

// Grid of the matrix-core kernel from T, Hkv, npacks and nsplit.  With a
// multiple of 8 (trunk, kv head) groups every XCD gets whole groups; with 1,
// 2 or 4 groups each spans 8/groups XCDs, its packs dealt to them
// alternately; any other count goes by block index, which balances the XCDs
// without keeping a group on one of them.
inline void mfma_grid(MfmaParams& p) {
  const int ug = p.npacks * p.nsplit, ng = p.T * p.Hkv;
  p.ilv = 1;
  p.ugp = ug;
  p.chunked = 1;
  if (ng % 8 != 0) {
    if (8 % ng == 0) {
      p.ilv = 8 / ng;
      p.ugp = (ug + p.ilv - 1) / p.ilv * p.ilv;
    } else {
      p.chunked = 0;
    }
  }
  p.nunits = ng * p.ugp;
  p.nwg = (p.nunits + 7) / 8 * 8;
}
// prefill: launch the kernel under its prefill name (same code)
hipError_t launch_tree_attn_mfma(int D, const MfmaParams& p, hipStream_t s, bool prefill = false);

// ---------------------------------------------------------------- trunk prefill
// Workspace layout (prefill.hip).  Matrix-core path (bf16):
//   anchors    int32  [L-1]           anchor of branch b (= token b+1) is b
//   qr         bf16   [T][L-1][Hq][D] rotated, scaled queries of tokens 1..L-1
//   branch_ok, order, anc, pstart, ustart, umap: the tree kernel's plan of the
//              L-1 one-node branches (the same for every trunk)
//   ctr        int32  [T][Hkv][npacks]
//   qctr       u64    [T][8]    unit-queue counters of each trunk's launch
//   part       split partials (one trunk's launch at a time)
// fp32 path: anchors, parent (-1), pos (b+1), then the tree workspace.
struct PrefillWs {
  size_t anchors, qr, branch_ok, order, anc, pstart, ustart, umap, ctr, qctr, part;
  size_t parent, pos, tree, total;
};
PrefillWs prefill_ws_layout(const specopd_prefill_desc& d);

struct PrefillArgs {
  const void *q, *k, *v;
  void *cache_k, *cache_v, *out;
  char* ws;
  float rope_base, scale;
};
hipError_t launch_prefill(const specopd_prefill_desc& d, const PrefillArgs& a, hipStream_t s);

// ---------------------------------------------------------------- E2E-TV
// Workspace layout:
//   slot       u64    [N]     (alpha, G) of every row, top bit set once posted
//   ticket     int32          next row to hand out, in order; 128 bytes on, the
//                             count of branches that reported their numerator;
//                             256 bytes on, the count of deferred rows
//   defer      int32  [N]     rows whose wait for their branch gave up
//   lse        float2 [N]     their -log2-sum-exp2 of draft and target
//   numer      double [R]     sum of prefix products of each branch
//   branch_ok  int32  [R]
struct E2etvWs {
  size_t slot, ticket, defer, lse, numer, branch_ok, total;
};
E2etvWs e2etv_ws_layout(const specopd_e2etv_desc& d);
// byte offsets of the count of reported branches and of deferred rows
inline size_t e2etv_done_offset(const E2etvWs& w) { return w.ticket + 128; }
inline size_t e2etv_ndefer_offset(const E2etvWs& w) { return w.ticket + 256; }


struct E2etvArgs {
  const void *draft, *target;
  const int32_t* target_row;
  const int32_t* parent;
  float *alpha_out, *prefix_out;
  double* loss_out;
  void* grad;
  char* ws;
};
hipError_t launch_e2etv(const specopd_e2etv_desc& d, const E2etvArgs& a, hipStream_t s);

// Static scratch of specopd_e2etv_fwd_bwd_noalloc (e2etv.hip): the device
// address of the current GPU's copy, looked up on first use per GPU.
constexpr size_t kE2etvScratchBytes = SPECOPD_E2ETV_NOALLOC_SCRATCH_BYTES;
hipError_t e2etv_scratch(void** ptr);

// ---------------------------------------------------------------- GDN replay
// Workspace: one int32, the count of malformed branches of the last call.
constexpr size_t kGdnWsBytes = 256;
struct GdnCallArgs {
  const float* ckpt;
  const void *trunk_k, *trunk_v;
  const float *trunk_gate, *trunk_beta;
  const int32_t *anchors, *parent;
  const void *q, *k, *v;
  const float *gate, *beta;
  float* out;
  char* ws;
};
hipError_t launch_gdn_replay(const specopd_gdn_desc& d, const GdnCallArgs& a, hipStream_t s);
hipError_t launch_gdn_conv(const specopd_gdn_conv_desc& d, const void* trunk_x, const void* x, const float* w,
                           const int32_t* anchors, const int32_t* parent, void* out, hipStream_t s);

// ---------------------------------------------------------------- QSA selection
// Workspace layout (offsets in bytes, each 256-aligned):
//   bad    int32  [1]           malformed branches of the last select call
//   ncand  int32  [T*B*Wn]      candidate groups of every node (-1: malformed)
//   sc     fp32   [T*B*Wn][Gs]  every candidate's score, Gs >= (L + Wn) / 4
struct QsaWs {
  size_t bad, ncand, sc, total;
  int Gs;
};
QsaWs qsa_ws_layout(const specopd_qsa_desc& d);
constexpr int kQsaMaxCand = 15360;  // a row's scores in LDS: 60 KiB
struct QsaCallArgs {
  const void *trunk_gk, *trunk_raw, *x, *y;
  const float* gamma;
  const int32_t *anchors, *parent, *pos;
  int32_t* sel;
  float* score;
  void* bkey;
  char* ws;
};
hipError_t launch_qsa_trunk_groups(const specopd_qsa_desc& d, const void* raw, const float* gamma, void* gk,
                                   hipStream_t s);
hipError_t launch_qsa_select(const specopd_qsa_desc& d, const QsaCallArgs& a, hipStream_t s);

// ---------------------------------------------------------------- LM head + E2E-TV
// Workspace layout (offsets in bytes, each 256-aligned):
//   bad    int32   [1]          malformed branches / out-of-range target rows
//   partA  f32x4   [N][nch]     per 64-entry chunk: max and 2^x-sum of z, t
//   nl     f32x2   [N]          log2-domain log-sum-exps
//   partB  f32x2   [N][nch]     per chunk: alpha, G
//   coef   f32x2   [N]          gradient coefficients
//   numer  double  [R]          branch numerators
//   bits   uint32  [N][nch][2]  the indicator [q < p] per element (pass B -> C)
struct LmhWs {
  size_t bad, partA, nl, partB, coef, numer, bits, total;
  int nch;
};
LmhWs lmhead_ws_layout(const specopd_lmhead_e2etv_desc& d);
struct LmhCallArgs {
  const void *h_draft, *w_draft, *h_target, *w_target;
  const int32_t *target_row, *parent;
  float *alpha_out, *prefix_out;
  double* loss_out;
  float* grad;
  char* ws;
};
hipError_t launch_lmhead_e2etv(const specopd_lmhead_e2etv_desc& d, const LmhCallArgs& a, hipStream_t s);

// Kernel timing (specopd_kernel_timing): records an event on s before
// (phase 0) or after (phase 1) the main kernel of call kind `which`
// (0 attention, 1 E2E-TV, 2 prefill, 3 GDN replay, 4 GDN convolution,
// 5 QSA scores, 6 QSA top-k, 7 LM head + E2E-TV from its first pass to its
// last) when timing is on;
// otherwise does nothing (also for a negative `which`).
constexpr int kTimingKinds = 8;
void timing_mark(int which, int phase, hipStream_t s);

}  // namespace specopd
