// C-ABI front end of libspecopd: argument validation (all of it before any
// HIP call), workspace sizing, dispatch to the kernel launchers, and the
// device-status readback.  Nothing here throws across the ABI.
#include <math.h>
#include <string.h>

#include <vector>

#include <mutex>
#include "internal.h"

using namespace specopd;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

specopd_status check_tree_desc(const specopd_tree_attn_desc* d) {
  if (!d) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->T < 1 || d->L < 1 || d->B < 1 || d->Wn < 1 || d->Hq < 1 || d->Hkv < 1 || d->D < 1)
    return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->Wn > 64) return SPECOPD_ERR_UNSUPPORTED;
  if (d->Hq % d->Hkv != 0) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->D != 64 && d->D != 128 && d->D != 256) return SPECOPD_ERR_UNSUPPORTED;
  if (d->dtype != SPECOPD_F32 && d->dtype != SPECOPD_BF16) return SPECOPD_ERR_INVALID_ARGUMENT;
  if ((d->flags & ~SPECOPD_TREE_BATCH_INVARIANT) != 0) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (!(isfinite(d->rope_base) && isfinite(d->scale))) return SPECOPD_ERR_INVALID_ARGUMENT;
  // element counts must stay within what the kernels index with 32/64-bit math
  const double nodes = double(d->T) * d->B * d->Wn;
  if (double(d->T) * d->B > 2147483647.0 || nodes * d->Hq > 2147483647.0 ||
      double(d->T) * d->L * d->Hkv * d->D > 9.0e15)
    return SPECOPD_ERR_UNSUPPORTED;
  // the matrix-core kernel addresses one trunk's K (and V), and the keys (and
  // values) of one trunk's branch nodes, with 32-bit offsets
  if (d->dtype == SPECOPD_BF16 && (double(d->L) * d->Hkv * d->D * 2.0 > 4294967295.0 ||
                                   double(d->B) * d->Wn * d->Hkv * d->D * 2.0 > 4294967295.0))
    return SPECOPD_ERR_UNSUPPORTED;
  return SPECOPD_OK;
}

specopd_status check_gdn_desc(const specopd_gdn_desc* d) {
  if (!d) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->T < 1 || d->L < 1 || d->B < 1 || d->Wn < 1 || d->H < 1 || d->C < 1 || d->D < 1)
    return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->dtype != SPECOPD_F32 && d->dtype != SPECOPD_BF16) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->flags != 0) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->D != 64 && d->D != 128) return SPECOPD_ERR_UNSUPPORTED;
  if (d->Wn > 64 || d->C > 64) return SPECOPD_ERR_UNSUPPORTED;  // the work list's bound
  // grid and element offsets
  if (double(d->T) * d->B * d->H > 2147483647.0 || double(d->T) * d->L >= double(1 << 28) ||
      double(d->T) * d->L * d->H * d->D > 9.0e15 || double(d->T) * d->B * d->Wn * d->H * d->D > 9.0e15)
    return SPECOPD_ERR_UNSUPPORTED;
  return SPECOPD_OK;
}

specopd_status check_gdn_conv_desc(const specopd_gdn_conv_desc* d) {
  if (!d) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->T < 1 || d->L < 1 || d->B < 1 || d->Wn < 1 || d->H < 1 || d->D < 1 || d->K < 1)
    return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->dtype != SPECOPD_F32 && d->dtype != SPECOPD_BF16) return SPECOPD_ERR_INVALID_ARGUMENT;
  if ((d->flags & ~SPECOPD_GDN_CONV_L2NORM) != 0) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->D != 64 && d->D != 128) return SPECOPD_ERR_UNSUPPORTED;
  if (d->Wn > 64 || d->K > 8) return SPECOPD_ERR_UNSUPPORTED;
  // grid (one workgroup per node) and element offsets
  if (double(d->T) * d->B * d->Wn > 2147483647.0 || double(d->T) * d->L >= double(1 << 28) ||
      double(d->T) * d->L * d->H * d->D > 9.0e15 || double(d->T) * d->B * d->Wn * d->H * d->D > 9.0e15)
    return SPECOPD_ERR_UNSUPPORTED;
  return SPECOPD_OK;
}

specopd_status check_qsa_desc(const specopd_qsa_desc* d) {
  if (!d) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->T < 1 || d->L < 1 || d->B < 1 || d->Wn < 1 || d->Di < 1 || d->topk < 1)
    return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->flags != 0) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (!(isfinite(d->rope_base) && isfinite(d->eps))) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->Di != 64 && d->Di != 128 && d->Di != 256) return SPECOPD_ERR_UNSUPPORTED;
  if (d->Wn > 64) return SPECOPD_ERR_UNSUPPORTED;
  if ((double(d->L) + d->Wn) / 4.0 > double(kQsaMaxCand)) return SPECOPD_ERR_UNSUPPORTED;
  // grids (one workgroup per branch, one per node) and element offsets
  const double rows = double(d->T) * d->B * d->Wn;
  if (rows > 2147483647.0 || rows * d->topk > 9.0e15 || rows * (double(d->L) + d->Wn) > 9.0e15 ||
      double(d->T) * d->L * d->Di > 9.0e15 || rows * d->Di > 9.0e15)
    return SPECOPD_ERR_UNSUPPORTED;
  return SPECOPD_OK;
}

specopd_status check_lmhead_desc(const specopd_lmhead_e2etv_desc* d) {
  if (!d) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->R < 1 || d->Wn < 1 || d->V < 1 || d->H < 16 || d->M < 1) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->H % 16 != 0) return SPECOPD_ERR_UNSUPPORTED;
  if (d->Wn > 64) return SPECOPD_ERR_UNSUPPORTED;
  if (d->flags != 0) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (!(isfinite(d->norm_count) && isfinite(d->grad_scale))) return SPECOPD_ERR_INVALID_ARGUMENT;
  // grid (vocabulary tiles x row tiles) and element offsets
  const double N = double(d->R) * d->Wn;
  if (N > 2147483647.0 || N * d->V > 9.0e15 || double(d->V) * d->H > 9.0e15 || double(d->M) * d->H > 9.0e15 ||
      N * d->H > 9.0e15 || (ceil(double(d->V) / 128) + 8) * ceil(N / 128) * 256.0 > 2147483647.0)
    return SPECOPD_ERR_UNSUPPORTED;  // the pass kernels' grid, in threads
  // the pass kernels address each operand with 32-bit element offsets
  if (double(d->V) * d->H >= 2147483648.0 || double(d->M) * d->H >= 2147483648.0 || N * d->H >= 2147483648.0)
    return SPECOPD_ERR_UNSUPPORTED;
  return SPECOPD_OK;
}

specopd_status check_prefill_desc(const specopd_prefill_desc* d) {
  if (!d) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->T < 1 || d->L < 1 || d->Hq < 1 || d->Hkv < 1 || d->D < 1) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->Hq % d->Hkv != 0) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->D != 64 && d->D != 128 && d->D != 256) return SPECOPD_ERR_UNSUPPORTED;
  if (d->dtype != SPECOPD_F32 && d->dtype != SPECOPD_BF16) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->flags != 0) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (!(isfinite(d->rope_base) && isfinite(d->scale))) return SPECOPD_ERR_INVALID_ARGUMENT;
  // one trunk is one tree call of L-1 one-node branches: the same index limits
  if (double(d->L) * d->Hq > 2147483647.0 || double(d->T) * d->L * (d->Hq + d->Hkv) * d->D > 9.0e15)
    return SPECOPD_ERR_UNSUPPORTED;
  if (d->dtype == SPECOPD_BF16 && double(d->L) * d->Hkv * d->D * 2.0 > 4294967295.0)
    return SPECOPD_ERR_UNSUPPORTED;
  return SPECOPD_OK;
}

specopd_status check_e2etv_desc(const specopd_e2etv_desc* d) {
  if (!d) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->R < 1 || d->Wn < 1 || d->V < 1) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->Wn > 64) return SPECOPD_ERR_UNSUPPORTED;
  if (d->logits_dtype != SPECOPD_F32 && d->logits_dtype != SPECOPD_BF16) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->grad_dtype != SPECOPD_F32 && d->grad_dtype != SPECOPD_BF16) return SPECOPD_ERR_INVALID_ARGUMENT;
  if ((d->flags & ~SPECOPD_E2ETV_DEFER_ALL) != 0) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (!isfinite(d->norm_count) || !isfinite(d->grad_scale)) return SPECOPD_ERR_INVALID_ARGUMENT;
  const double rows = double(d->R) * d->Wn;
  if (rows > 2147483647.0) return SPECOPD_ERR_UNSUPPORTED;
  if (double(d->V) * 16.0 > 2147483647.0) return SPECOPD_ERR_UNSUPPORTED;  // 32-bit unit indices
  return SPECOPD_OK;
}

// Pointer checks shared by the two E2E-TV calls (after the descriptor's).
specopd_status check_e2etv_call(const specopd_e2etv_desc* d, const void* draft, const void* target,
                                const int32_t* target_row, const int32_t* parent,
                                const float* alpha, const float* prefix, const double* loss,
                                const void* grad) {
  specopd_status st = check_e2etv_desc(d);
  if (st != SPECOPD_OK) return st;
  if (!draft || !target || !parent || !loss) return SPECOPD_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {draft, target, parent, loss};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SPECOPD_ERR_INVALID_ARGUMENT;
  if ((alpha && !aligned16(alpha)) || (prefix && !aligned16(prefix)) || (grad && !aligned16(grad)) ||
      (target_row && !aligned16(target_row)))
    return SPECOPD_ERR_INVALID_ARGUMENT;
  if (target_row && d->target_rows < 1) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (grad && (grad == draft || grad == target)) return SPECOPD_ERR_INVALID_ARGUMENT;
  return SPECOPD_OK;
}

}  // namespace

// ---- kernel timing
namespace {
struct TimingState {
  std::mutex mu;
  bool on = false;
  bool failed = false;
  std::vector<hipEvent_t> ev[kTimingKinds];  // per call kind: start, stop, start, stop, ...
  std::vector<hipEvent_t> pool;   // created up front, so recording costs no allocation
  void clear() {
    for (auto& v : ev) {
      for (hipEvent_t e : v) pool.push_back(e);
      v.clear();
    }
    failed = false;
  }
};
constexpr int kTimingPool = 256;
TimingState& timing() {
  static TimingState t;
  return t;
}
}  // namespace

namespace specopd {
void timing_mark(int which, int phase, hipStream_t s) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.on || which < 0 || which >= kTimingKinds) return;
  auto& v = t.ev[which];
  if (phase == 1 && v.size() % 2 == 0) return;  // no open start
  if (phase == 0 && v.size() % 2 == 1) return;  // already open
  hipEvent_t e = nullptr;
  if (!t.pool.empty()) {
    e = t.pool.back();
    t.pool.pop_back();
  } else if (hipEventCreate(&e) != hipSuccess) {
    t.failed = true;
    return;
  }
  if (hipEventRecord(e, s) != hipSuccess) {
    t.pool.push_back(e);
    t.failed = true;
    return;
  }
  v.push_back(e);
}
}  // namespace specopd

extern "C" {

const char* specopd_status_string(specopd_status s) {
  switch (s) {
    case SPECOPD_OK: return "ok";
    case SPECOPD_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SPECOPD_ERR_UNSUPPORTED: return "unsupported configuration";
    case SPECOPD_ERR_WORKSPACE: return "workspace missing or too small";
    case SPECOPD_ERR_HIP: return "HIP runtime error";
    case SPECOPD_ERR_DEVICE_VALIDATION: return "malformed tree detected on the device";
  }
  return "unknown status";
}

int specopd_version(void) { return SPECOPD_VERSION; }


specopd_status specopd_kernel_timing(int enable) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (hipDeviceSynchronize() != hipSuccess) return SPECOPD_ERR_HIP;
  t.clear();
  t.on = enable != 0;
  while (t.on && t.pool.size() < size_t(kTimingPool)) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return SPECOPD_ERR_HIP;
    t.pool.push_back(e);
  }
  return SPECOPD_OK;
}

specopd_status specopd_kernel_time(int which, double* total_ms, int* launches) {
  if (which < 0 || which >= kTimingKinds || !total_ms || !launches) return SPECOPD_ERR_INVALID_ARGUMENT;
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (t.failed) return SPECOPD_ERR_HIP;
  const auto& v = t.ev[which];
  double tot = 0.0;
  int n = 0;
  for (size_t i = 0; i + 1 < v.size(); i += 2) {
    if (hipEventSynchronize(v[i + 1]) != hipSuccess) return SPECOPD_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, v[i], v[i + 1]) != hipSuccess) return SPECOPD_ERR_HIP;
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return SPECOPD_OK;
}

specopd_status specopd_tree_attn_workspace_size(const specopd_tree_attn_desc* desc, size_t* bytes) {
  specopd_status st = check_tree_desc(desc);
  if (st != SPECOPD_OK) return st;
  if (!bytes) return SPECOPD_ERR_INVALID_ARGUMENT;
  *bytes = tree_attn_ws_layout(*desc).total;
  return SPECOPD_OK;
}

specopd_status specopd_tree_attn_fwd(const specopd_tree_attn_desc* desc, const void* trunk_k,
                                     const void* trunk_v, const void* q, const void* k,
                                     const void* v, const int32_t* anchors, const int32_t* parent,
                                     const int32_t* pos, void* out, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  specopd_status st = check_tree_desc(desc);
  if (st != SPECOPD_OK) return st;
  const void* ptrs[] = {trunk_k, trunk_v, q, k, v, anchors, parent, pos, out};
  for (const void* p : ptrs)
    if (!p) return SPECOPD_ERR_INVALID_ARGUMENT;
  for (const void* p : ptrs)
    if (!aligned16(p)) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (out == trunk_k || out == trunk_v || out == q || out == k || out == v)
    return SPECOPD_ERR_INVALID_ARGUMENT;
  const size_t need = tree_attn_ws_layout(*desc).total;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return SPECOPD_ERR_WORKSPACE;
  TreeAttnArgs a{};
  a.trunk_k = trunk_k; a.trunk_v = trunk_v; a.q = q; a.k = k; a.v = v;
  a.anchors = anchors; a.parent = parent; a.pos = pos; a.out = out;
  a.ws = static_cast<char*>(workspace);
  a.rope_base = desc->rope_base > 0.f ? desc->rope_base : 10000.f;
  a.scale = desc->scale > 0.f ? desc->scale : float(1.0 / sqrt(double(desc->D)));
  hipError_t e = launch_tree_attn(*desc, a, stream);
  return e == hipSuccess ? SPECOPD_OK : SPECOPD_ERR_HIP;
}

specopd_status specopd_prefill_workspace_size(const specopd_prefill_desc* desc, size_t* bytes) {
  specopd_status st = check_prefill_desc(desc);
  if (st != SPECOPD_OK) return st;
  if (!bytes) return SPECOPD_ERR_INVALID_ARGUMENT;
  *bytes = prefill_ws_layout(*desc).total;
  return SPECOPD_OK;
}

specopd_status specopd_prefill_fwd(const specopd_prefill_desc* desc, const void* q, const void* k,
                                   const void* v, void* cache_k, void* cache_v, void* out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  specopd_status st = check_prefill_desc(desc);
  if (st != SPECOPD_OK) return st;
  const void* ptrs[] = {q, k, v, cache_k, cache_v, out};
  for (const void* p : ptrs)
    if (!p) return SPECOPD_ERR_INVALID_ARGUMENT;
  for (const void* p : ptrs)
    if (!aligned16(p)) return SPECOPD_ERR_INVALID_ARGUMENT;
  // outputs may alias neither an input nor each other
  const void* outs[] = {cache_k, cache_v, out};
  for (const void* o : outs) {
    if (o == q || o == k || o == v) return SPECOPD_ERR_INVALID_ARGUMENT;
  }
  if (cache_k == cache_v || cache_k == out || cache_v == out) return SPECOPD_ERR_INVALID_ARGUMENT;
  const size_t need = prefill_ws_layout(*desc).total;
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return SPECOPD_ERR_WORKSPACE;
  PrefillArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.cache_k = cache_k; a.cache_v = cache_v; a.out = out;
  a.ws = static_cast<char*>(workspace);
  a.rope_base = desc->rope_base > 0.f ? desc->rope_base : 10000.f;
  a.scale = desc->scale > 0.f ? desc->scale : float(1.0 / sqrt(double(desc->D)));
  hipError_t e = launch_prefill(*desc, a, stream);
  return e == hipSuccess ? SPECOPD_OK : SPECOPD_ERR_HIP;
}

specopd_status specopd_gdn_workspace_size(const specopd_gdn_desc* desc, size_t* bytes) {
  specopd_status st = check_gdn_desc(desc);
  if (st != SPECOPD_OK) return st;
  if (!bytes) return SPECOPD_ERR_INVALID_ARGUMENT;
  *bytes = kGdnWsBytes;
  return SPECOPD_OK;
}

specopd_status specopd_gdn_replay_fwd(const specopd_gdn_desc* desc, const float* ckpt,
                                      const void* trunk_k, const void* trunk_v,
                                      const float* trunk_gate, const float* trunk_beta,
                                      const int32_t* anchors, const int32_t* parent, const void* q,
                                      const void* k, const void* v, const float* gate,
                                      const float* beta, float* out, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  specopd_status st = check_gdn_desc(desc);
  if (st != SPECOPD_OK) return st;
  const bool need_ckpt = desc->L / desc->C > 0;
  const void* ptrs[] = {trunk_k, trunk_v, trunk_gate, trunk_beta, anchors, parent, q, k, v, gate, beta, out};
  for (const void* p : ptrs)
    if (!p) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (need_ckpt && !ckpt) return SPECOPD_ERR_INVALID_ARGUMENT;
  for (const void* p : ptrs)
    if (!aligned16(p)) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (need_ckpt && !aligned16(ckpt)) return SPECOPD_ERR_INVALID_ARGUMENT;
  const void* ins[] = {ckpt, trunk_k, trunk_v, trunk_gate, trunk_beta, anchors, parent, q, k, v, gate, beta};
  for (const void* p : ins)
    if (p == out) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < kGdnWsBytes || !aligned16(workspace)) return SPECOPD_ERR_WORKSPACE;
  GdnCallArgs a{};
  a.ckpt = ckpt;
  a.trunk_k = trunk_k; a.trunk_v = trunk_v;
  a.trunk_gate = trunk_gate; a.trunk_beta = trunk_beta;
  a.anchors = anchors; a.parent = parent;
  a.q = q; a.k = k; a.v = v;
  a.gate = gate; a.beta = beta;
  a.out = out;
  a.ws = static_cast<char*>(workspace);
  hipError_t e = launch_gdn_replay(*desc, a, stream);
  return e == hipSuccess ? SPECOPD_OK : SPECOPD_ERR_HIP;
}

specopd_status specopd_gdn_conv_fwd(const specopd_gdn_conv_desc* desc, const void* trunk_x,
                                    const void* x, const float* w, const int32_t* anchors,
                                    const int32_t* parent, void* out, hipStream_t stream) {
  specopd_status st = check_gdn_conv_desc(desc);
  if (st != SPECOPD_OK) return st;
  const void* ins[] = {trunk_x, x, w, anchors, parent};
  for (const void* p : ins)
    if (!p || !aligned16(p) || p == out) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (!out || !aligned16(out)) return SPECOPD_ERR_INVALID_ARGUMENT;
  timing_mark(4, 0, stream);
  hipError_t e = launch_gdn_conv(*desc, trunk_x, x, w, anchors, parent, out, stream);
  timing_mark(4, 1, stream);
  return e == hipSuccess ? SPECOPD_OK : SPECOPD_ERR_HIP;
}

specopd_status specopd_gdn_device_status(const specopd_gdn_desc* desc, const void* workspace,
                                         size_t workspace_bytes, int32_t* bad_branches,
                                         hipStream_t stream) {
  specopd_status st = check_gdn_desc(desc);
  if (st != SPECOPD_OK) return st;
  if (!workspace || workspace_bytes < kGdnWsBytes || !aligned16(workspace)) return SPECOPD_ERR_WORKSPACE;
  int32_t bad = 0;
  if (hipStreamSynchronize(stream) != hipSuccess) return SPECOPD_ERR_HIP;
  if (hipMemcpy(&bad, workspace, sizeof(bad), hipMemcpyDeviceToHost) != hipSuccess) return SPECOPD_ERR_HIP;
  if (bad_branches) *bad_branches = bad;
  return bad != 0 ? SPECOPD_ERR_DEVICE_VALIDATION : SPECOPD_OK;
}

specopd_status specopd_qsa_trunk_groups_fwd(const specopd_qsa_desc* desc, const void* trunk_raw,
                                            const float* gamma, void* trunk_gk, hipStream_t stream) {
  specopd_status st = check_qsa_desc(desc);
  if (st != SPECOPD_OK) return st;
  if (!trunk_raw || !gamma || !trunk_gk) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (!aligned16(trunk_raw) || !aligned16(gamma) || !aligned16(trunk_gk)) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (trunk_gk == trunk_raw || trunk_gk == gamma) return SPECOPD_ERR_INVALID_ARGUMENT;
  return launch_qsa_trunk_groups(*desc, trunk_raw, gamma, trunk_gk, stream) == hipSuccess ? SPECOPD_OK
                                                                                           : SPECOPD_ERR_HIP;
}

specopd_status specopd_qsa_workspace_size(const specopd_qsa_desc* desc, size_t* bytes) {
  specopd_status st = check_qsa_desc(desc);
  if (st != SPECOPD_OK) return st;
  if (!bytes) return SPECOPD_ERR_INVALID_ARGUMENT;
  *bytes = qsa_ws_layout(*desc).total;
  return SPECOPD_OK;
}

specopd_status specopd_qsa_select_fwd(const specopd_qsa_desc* desc, const void* trunk_gk,
                                      const void* trunk_raw, const void* x, const void* y,
                                      const float* gamma, const int32_t* anchors,
                                      const int32_t* parent, const int32_t* pos, int32_t* sel,
                                      float* score, void* bkey, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  specopd_status st = check_qsa_desc(desc);
  if (st != SPECOPD_OK) return st;
  const void* ins[] = {trunk_gk, trunk_raw, x, y, gamma, anchors, parent, pos};
  const void* outs[] = {sel, score, bkey};
  for (const void* p : ins)
    if (!p || !aligned16(p)) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (!sel || !score) return SPECOPD_ERR_INVALID_ARGUMENT;
  for (const void* o : outs) {
    if (!o) continue;
    if (!aligned16(o)) return SPECOPD_ERR_INVALID_ARGUMENT;
    for (const void* p : ins)
      if (p == o) return SPECOPD_ERR_INVALID_ARGUMENT;
  }
  if (sel == static_cast<void*>(score) || bkey == static_cast<void*>(sel) || bkey == static_cast<void*>(score))
    return SPECOPD_ERR_INVALID_ARGUMENT;
  const QsaWs w = qsa_ws_layout(*desc);
  if (!workspace || workspace_bytes < w.total || !aligned16(workspace)) return SPECOPD_ERR_WORKSPACE;
  QsaCallArgs a{};
  a.trunk_gk = trunk_gk; a.trunk_raw = trunk_raw;
  a.x = x; a.y = y;
  a.gamma = gamma;
  a.anchors = anchors; a.parent = parent; a.pos = pos;
  a.sel = sel; a.score = score; a.bkey = bkey;
  a.ws = static_cast<char*>(workspace);
  return launch_qsa_select(*desc, a, stream) == hipSuccess ? SPECOPD_OK : SPECOPD_ERR_HIP;
}

specopd_status specopd_qsa_device_status(const specopd_qsa_desc* desc, const void* workspace,
                                         size_t workspace_bytes, int32_t* bad_branches,
                                         hipStream_t stream) {
  specopd_status st = check_qsa_desc(desc);
  if (st != SPECOPD_OK) return st;
  const QsaWs w = qsa_ws_layout(*desc);
  if (!workspace || workspace_bytes < w.total || !aligned16(workspace)) return SPECOPD_ERR_WORKSPACE;
  int32_t bad = 0;
  if (hipStreamSynchronize(stream) != hipSuccess) return SPECOPD_ERR_HIP;
  if (hipMemcpy(&bad, static_cast<const char*>(workspace) + w.bad, sizeof(bad), hipMemcpyDeviceToHost) != hipSuccess)
    return SPECOPD_ERR_HIP;
  if (bad_branches) *bad_branches = bad;
  return bad != 0 ? SPECOPD_ERR_DEVICE_VALIDATION : SPECOPD_OK;
}

specopd_status specopd_lmhead_e2etv_workspace_size(const specopd_lmhead_e2etv_desc* desc, size_t* bytes) {
  specopd_status st = check_lmhead_desc(desc);
  if (st != SPECOPD_OK) return st;
  if (!bytes) return SPECOPD_ERR_INVALID_ARGUMENT;
  *bytes = lmhead_ws_layout(*desc).total;
  return SPECOPD_OK;
}

specopd_status specopd_lmhead_e2etv_fwd_bwd(const specopd_lmhead_e2etv_desc* desc, const void* h_draft,
                                            const void* w_draft, const void* h_target,
                                            const void* w_target, const int32_t* target_row,
                                            const int32_t* parent, float* alpha_out, float* prefix_out,
                                            double* loss_out, float* grad_draft, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
  specopd_status st = check_lmhead_desc(desc);
  if (st != SPECOPD_OK) return st;
  const void* ins[] = {h_draft, w_draft, h_target, w_target, target_row, parent};
  for (const void* p : ins)
    if (!p || !aligned16(p)) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (!loss_out || !aligned16(loss_out)) return SPECOPD_ERR_INVALID_ARGUMENT;
  const void* outs[] = {alpha_out, prefix_out, loss_out, grad_draft};
  for (int i = 0; i < 4; ++i) {
    const void* o = outs[i];
    if (!o) continue;
    if (!aligned16(o)) return SPECOPD_ERR_INVALID_ARGUMENT;
    for (const void* p : ins)
      if (p == o) return SPECOPD_ERR_INVALID_ARGUMENT;
    for (int j = 0; j < i; ++j)
      if (outs[j] == o) return SPECOPD_ERR_INVALID_ARGUMENT;
  }
  const LmhWs w = lmhead_ws_layout(*desc);
  if (!workspace || workspace_bytes < w.total || !aligned16(workspace)) return SPECOPD_ERR_WORKSPACE;
  LmhCallArgs a{};
  a.h_draft = h_draft; a.w_draft = w_draft; a.h_target = h_target; a.w_target = w_target;
  a.target_row = target_row; a.parent = parent;
  a.alpha_out = alpha_out; a.prefix_out = prefix_out; a.loss_out = loss_out; a.grad = grad_draft;
  a.ws = static_cast<char*>(workspace);
  return launch_lmhead_e2etv(*desc, a, stream) == hipSuccess ? SPECOPD_OK : SPECOPD_ERR_HIP;
}

specopd_status specopd_lmhead_e2etv_device_status(const specopd_lmhead_e2etv_desc* desc,
                                                  const void* workspace, size_t workspace_bytes,
                                                  int32_t* bad_out, hipStream_t stream) {
  specopd_status st = check_lmhead_desc(desc);
  if (st != SPECOPD_OK) return st;
  const LmhWs w = lmhead_ws_layout(*desc);
  if (!workspace || workspace_bytes < w.total || !aligned16(workspace)) return SPECOPD_ERR_WORKSPACE;
  int32_t bad = 0;
  if (hipStreamSynchronize(stream) != hipSuccess) return SPECOPD_ERR_HIP;
  if (hipMemcpy(&bad, static_cast<const char*>(workspace) + w.bad, sizeof(bad), hipMemcpyDeviceToHost) != hipSuccess)
    return SPECOPD_ERR_HIP;
  if (bad_out) *bad_out = bad;
  return bad != 0 ? SPECOPD_ERR_DEVICE_VALIDATION : SPECOPD_OK;
}

specopd_status specopd_score_rows(const specopd_tree_attn_desc* desc, const int32_t* anchors,
                                  const int32_t* parent, int32_t* rows, hipStream_t stream) {
  specopd_status st = check_tree_desc(desc);
  if (st != SPECOPD_OK) return st;
  if (!anchors || !parent || !rows) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (!aligned16(anchors) || !aligned16(parent) || !aligned16(rows)) return SPECOPD_ERR_INVALID_ARGUMENT;
  // every score row index must fit an int32
  if (double(desc->T) * desc->L + double(desc->T) * desc->B * desc->Wn > 2147483647.0)
    return SPECOPD_ERR_UNSUPPORTED;
  return launch_score_rows(*desc, anchors, parent, rows, stream) == hipSuccess ? SPECOPD_OK
                                                                                 : SPECOPD_ERR_HIP;
}

specopd_status specopd_tree_attn_device_status(const specopd_tree_attn_desc* desc,
                                               const void* workspace, size_t workspace_bytes,
                                               int32_t* bad_branches, hipStream_t stream) {
  specopd_status st = check_tree_desc(desc);
  if (st != SPECOPD_OK) return st;
  const TreeAttnWs L = tree_attn_ws_layout(*desc);
  if (!workspace || workspace_bytes < L.total) return SPECOPD_ERR_WORKSPACE;
  const size_t TB = size_t(desc->T) * desc->B;
  std::vector<int32_t> ok(TB);
  if (hipStreamSynchronize(stream) != hipSuccess) return SPECOPD_ERR_HIP;
  if (hipMemcpy(ok.data(), static_cast<const char*>(workspace) + L.branch_ok, TB * sizeof(int32_t),
                hipMemcpyDeviceToHost) != hipSuccess)
    return SPECOPD_ERR_HIP;
  int32_t bad = 0;
  for (int32_t x : ok) bad += (x == 0);
  if (bad_branches) *bad_branches = bad;
  return bad ? SPECOPD_ERR_DEVICE_VALIDATION : SPECOPD_OK;
}

specopd_status specopd_e2etv_workspace_size(const specopd_e2etv_desc* desc, size_t* bytes) {
  specopd_status st = check_e2etv_desc(desc);
  if (st != SPECOPD_OK) return st;
  if (!bytes) return SPECOPD_ERR_INVALID_ARGUMENT;
  *bytes = e2etv_ws_layout(*desc).total;
  return SPECOPD_OK;
}

specopd_status specopd_e2etv_fwd_bwd(const specopd_e2etv_desc* desc, const void* draft_logits,
                                     const void* target_logits, const int32_t* target_row,
                                     const int32_t* parent, float* alpha_out, float* prefix_out,
                                     double* loss_out, void* grad_draft, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  specopd_status st = check_e2etv_call(desc, draft_logits, target_logits, target_row, parent,
                                       alpha_out, prefix_out, loss_out, grad_draft);
  if (st != SPECOPD_OK) return st;
  const size_t need = e2etv_ws_layout(*desc).total;
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return SPECOPD_ERR_WORKSPACE;
  E2etvArgs a{};
  a.draft = draft_logits; a.target = target_logits; a.target_row = target_row; a.parent = parent;
  a.alpha_out = alpha_out; a.prefix_out = prefix_out; a.loss_out = loss_out;
  a.grad = grad_draft; a.ws = static_cast<char*>(workspace);
  hipError_t e = launch_e2etv(*desc, a, stream);
  return e == hipSuccess ? SPECOPD_OK : SPECOPD_ERR_HIP;
}

specopd_status specopd_e2etv_fwd_bwd_noalloc(const specopd_e2etv_desc* desc, const void* draft_logits,
                                             const void* target_logits, const int32_t* target_row,
                                             const int32_t* parent, float* alpha_out,
                                             float* prefix_out, double* loss_out, void* grad_draft,
                                             hipStream_t stream) {
  specopd_status st = check_e2etv_call(desc, draft_logits, target_logits, target_row, parent,
                                       alpha_out, prefix_out, loss_out, grad_draft);
  if (st != SPECOPD_OK) return st;
  if (e2etv_ws_layout(*desc).total > kE2etvScratchBytes) return SPECOPD_ERR_WORKSPACE;
  void* ws = nullptr;
  if (e2etv_scratch(&ws) != hipSuccess) return SPECOPD_ERR_HIP;
  E2etvArgs a{};
  a.draft = draft_logits; a.target = target_logits; a.target_row = target_row; a.parent = parent;
  a.alpha_out = alpha_out; a.prefix_out = prefix_out; a.loss_out = loss_out;
  a.grad = grad_draft; a.ws = static_cast<char*>(ws);
  hipError_t e = launch_e2etv(*desc, a, stream);
  return e == hipSuccess ? SPECOPD_OK : SPECOPD_ERR_HIP;
}

specopd_status specopd_e2etv_device_status(const specopd_e2etv_desc* desc, const void* workspace,
                                           size_t workspace_bytes, int32_t* bad_branches,
                                           int32_t* deferred_rows, hipStream_t stream) {
  specopd_status st = check_e2etv_desc(desc);
  if (st != SPECOPD_OK) return st;
  const E2etvWs L = e2etv_ws_layout(*desc);
  if (!workspace || workspace_bytes < L.total) return SPECOPD_ERR_WORKSPACE;
  std::vector<int32_t> ok(size_t(desc->R));
  int32_t deferred = 0;
  const char* ws = static_cast<const char*>(workspace);
  if (hipStreamSynchronize(stream) != hipSuccess) return SPECOPD_ERR_HIP;
  if (hipMemcpy(ok.data(), ws + L.branch_ok, ok.size() * sizeof(int32_t), hipMemcpyDeviceToHost) !=
          hipSuccess ||
      hipMemcpy(&deferred, ws + e2etv_ndefer_offset(L), sizeof(int32_t), hipMemcpyDeviceToHost) !=
          hipSuccess)
    return SPECOPD_ERR_HIP;
  int32_t bad = 0;
  for (int32_t x : ok) bad += (x == 0);
  if (bad_branches) *bad_branches = bad;
  if (deferred_rows) *deferred_rows = deferred;
  return bad ? SPECOPD_ERR_DEVICE_VALIDATION : SPECOPD_OK;
}

}  // extern "C"
