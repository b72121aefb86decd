// C-ABI front end of libspecopd: argument validation (all of it before any
// HIP call), workspace sizing, dispatch to the kernel launchers, and the
// device-status readback.  Nothing here throws across the ABI.
#include <math.h>
#include <stdlib.h>
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
  if (d->flags != 0) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (!(isfinite(d->rope_base) && isfinite(d->scale))) return SPECOPD_ERR_INVALID_ARGUMENT;
  // element counts must stay within what the kernels index with 32/64-bit math
  const double nodes = double(d->T) * d->B * d->Wn;
  if (double(d->T) * d->B > 2147483647.0 || nodes * d->Hq > 2147483647.0 ||
      double(d->T) * d->L * d->Hkv * d->D > 9.0e15)
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
  return SPECOPD_OK;
}

specopd_status check_e2etv_desc(const specopd_e2etv_desc* d) {
  if (!d) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->R < 1 || d->Wn < 1 || d->V < 1) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->Wn > 64) return SPECOPD_ERR_UNSUPPORTED;
  if (d->logits_dtype != SPECOPD_F32 && d->logits_dtype != SPECOPD_BF16) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->grad_dtype != SPECOPD_F32 && d->grad_dtype != SPECOPD_BF16) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (d->flags != 0) return SPECOPD_ERR_INVALID_ARGUMENT;
  if (!isfinite(d->norm_count) || !isfinite(d->grad_scale)) return SPECOPD_ERR_INVALID_ARGUMENT;
  const double rows = double(d->R) * d->Wn;
  if (rows > 2147483647.0) return SPECOPD_ERR_UNSUPPORTED;
  if (double(d->V) * 16.0 > 2147483647.0) return SPECOPD_ERR_UNSUPPORTED;  // 32-bit unit indices
  return SPECOPD_OK;
}

}  // namespace

// ---- kernel timing
namespace {
struct TimingState {
  std::mutex mu;
  bool on = false;
  bool failed = false;
  std::vector<hipEvent_t> ev[3];  // per call kind: start, stop, start, stop, ...
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
  if (!t.on || which < 0 || which > 2) return;
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
  if (which < 0 || which > 2 || !total_ms || !launches) return SPECOPD_ERR_INVALID_ARGUMENT;
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
                                     const void* target_logits, const int32_t* parent,
                                     float* alpha_out, float* prefix_out, double* loss_out,
                                     void* grad_draft, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  specopd_status st = check_e2etv_desc(desc);
  if (st != SPECOPD_OK) return st;
  if (!draft_logits || !target_logits || !parent || !loss_out) return SPECOPD_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {draft_logits, target_logits, parent, loss_out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return SPECOPD_ERR_INVALID_ARGUMENT;
  if ((alpha_out && !aligned16(alpha_out)) || (prefix_out && !aligned16(prefix_out)) ||
      (grad_draft && !aligned16(grad_draft)))
    return SPECOPD_ERR_INVALID_ARGUMENT;
  if (grad_draft && (grad_draft == draft_logits || grad_draft == target_logits))
    return SPECOPD_ERR_INVALID_ARGUMENT;
  const size_t need = e2etv_ws_layout(*desc).total;
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return SPECOPD_ERR_WORKSPACE;
  E2etvArgs a{};
  a.draft = draft_logits; a.target = target_logits; a.parent = parent;
  a.alpha_out = alpha_out; a.prefix_out = prefix_out; a.loss_out = loss_out;
  a.grad = grad_draft; a.ws = static_cast<char*>(workspace);
  // Test hook: a small bound on the in-kernel wait forces the timeout path
  // (the affected branches are reported as malformed; nothing hangs).
  if (const char* sl = getenv("SPECOPD_E2ETV_SPIN_LIMIT")) a.spin_limit = atoi(sl);
  hipError_t e = launch_e2etv(*desc, a, stream);
  return e == hipSuccess ? SPECOPD_OK : SPECOPD_ERR_HIP;
}

specopd_status specopd_e2etv_device_status(const specopd_e2etv_desc* desc, const void* workspace,
                                           size_t workspace_bytes, int32_t* bad_branches,
                                           hipStream_t stream) {
  specopd_status st = check_e2etv_desc(desc);
  if (st != SPECOPD_OK) return st;
  const E2etvWs L = e2etv_ws_layout(*desc);
  if (!workspace || workspace_bytes < L.total) return SPECOPD_ERR_WORKSPACE;
  std::vector<int32_t> ok(size_t(desc->R));
  if (hipStreamSynchronize(stream) != hipSuccess) return SPECOPD_ERR_HIP;
  if (hipMemcpy(ok.data(), static_cast<const char*>(workspace) + L.branch_ok,
                ok.size() * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return SPECOPD_ERR_HIP;
  int32_t bad = 0;
  for (int32_t x : ok) bad += (x == 0);
  if (bad_branches) *bad_branches = bad;
  return bad ? SPECOPD_ERR_DEVICE_VALIDATION : SPECOPD_OK;
}

}  // extern "C"
