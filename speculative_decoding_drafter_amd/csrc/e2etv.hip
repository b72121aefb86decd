// E2E-TV surrogate forward + gradient over a proposal tree (gfx950).
//
// The loss follows the jaehun.me review of SpecOPD, §1.1 and §3.3 (Eqs. 8, 9,
// 13) and the rustineverything.app summary §2.3: per node the overlap
// alpha = sum_v min(q_v, p_v) = 1 - TV of the draft distribution q and the
// target distribution p (full-vocabulary softmaxes, target mass outside q's
// support kept), prefix products along the parent chain, loss = 1 - mean of
// the prefix products, gradient through q only.
//
// One fused kernel, one workgroup per row (row n = branch r, node j):
//   pass A   read the row: log-sum-exp of draft and target;
//   pass B   alpha = sum min(q, p) and G = sum_{q<p} q;
//   post     publish (alpha, G) in the row's slot;
//   scan     once every row of the branch has posted, compute prefix
//            products, suffix sums S and this row's coefficient
//            c = grad_scale * dLoss/dalpha in fp64 (every row of a branch
//            repeats the same tiny scan in the same order);
//   pass C   write grad[u] = c * q_u * ([q_u < p_u] - G).
// Two forms.  e2etv_resident_kernel (bf16 logits, 16-byte aligned rows)
// keeps most of the row in registers and LDS from pass A to pass C, so each
// row is read from memory about once (see the resident-rows section).
// e2etv_fused_kernel (fp32 logits or unaligned rows) streams the row in every
// pass with software-pipelined loads: the next batch of 16-byte vectors is in
// flight while the current one is reduced.  Rows are taken in order from an
// atomic ticket, so a workgroup only waits for rows of its own branch that
// were claimed just before or after it.  The wait is bounded: a row whose
// siblings have not all posted by then (they could not be resident at the
// same time, e.g. while other kernels hold the CUs) leaves its log-sum-exps
// in the workspace and hands its scan and gradient to e2etv_rescue_kernel,
// which runs after every row has posted; results are the same either way.
// The exchange uses device-scope relaxed atomic accesses (see the
// cross-workgroup exchange).
// The branch that reports last sums the branch numerators in a fixed order
// (loss), so no further kernel runs after the rows.
// No floating-point atomics: results are bitwise reproducible.
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace specopd {

namespace {

constexpr int kThreads = 1024;  // per workgroup (one row)
constexpr int kU = 2;           // 16-byte vectors per tensor per thread per batch

// One element's log2-probabilities.  The overlap pass and the gradient pass
// both call exactly this, so the indicator [q < p] is decided identically.
__device__ __forceinline__ void log2probs(float z, float t, float nlz, float nlt, float& lq,
                                          float& lp) {
  lq = __builtin_fmaf(z, kLog2e, nlz);
  lp = __builtin_fmaf(t, kLog2e, nlt);
}

// Running max / scaled sum over NV values.
template <int NV>
__device__ __forceinline__ void lse_update(float& m, float& s, const float (&x)[NV]) {
  float vm = x[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) vm = fmaxf(vm, x[i]);
  if (vm > m) {
    s *= fast_exp2((m - vm) * kLog2e);
    m = vm;
  }
  if (m != kNegInf) {
    const float nm = -m * kLog2e;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) acc += fast_exp2(__builtin_fmaf(x[i], kLog2e, nm));
    s += acc;
  }
}

// The same update with the reference moved only when it must be: the group
// is summed against the current reference m first, and that sum is kept
// unless it exceeds 2^64 (a value more than 64 binary orders of magnitude
// above m), is NaN or infinite (m still -inf, or infinite logits); then the
// group is redone by the exact update above.  s stays a sum of terms scaled
// by 2^(-m log2 e), so the log-sum-exp m + ln s is unchanged, and the common
// case needs no maximum and no rescaling.
constexpr float kLazyLimit = 0x1p64f;
template <int NV>
__device__ __forceinline__ void lse_update_lazy(float& m, float& s, const float (&x)[NV]) {
  const float nm = -m * kLog2e;
  float acc = fast_exp2(__builtin_fmaf(x[0], kLog2e, nm));
#pragma unroll
  for (int i = 1; i < NV; ++i) acc += fast_exp2(__builtin_fmaf(x[i], kLog2e, nm));
  if (__builtin_expect(acc <= kLazyLimit, 1))
    s += acc;
  else
    lse_update<NV>(m, s, x);
}

// Stream units [u0, u1) of a row (16-byte vectors, or single elements when
// the row is not 16-byte aligned), pairs (draft, target): thread tid takes
// u0 + tid + k * THREADS.  Two register batches alternate so the next
// batch's loads are in flight while f() consumes the current one.
template <bool VECTOR, bool NT, int THREADS = kThreads, int KU = kU, typename F>
__device__ __forceinline__ void stream_pairs(const void* zrow, const void* trow, int u0, int u1,
                                             int esize, F&& f) {
  constexpr int STEP = THREADS * KU;
  using T = typename std::conditional<VECTOR, u32x4, uint32_t>::type;
  const int base = u0 + int(threadIdx.x);
  T za[KU], ta[KU], zb[KU], tb[KU];
  auto ld = [&](const void* row, int u) -> T {
    if constexpr (VECTOR) {
      const u32x4* p = reinterpret_cast<const u32x4*>(row) + u;
      if constexpr (NT) return __builtin_nontemporal_load(p);
      return *p;
    } else {
      return esize == 2 ? uint32_t(reinterpret_cast<const uint16_t*>(row)[u])
                        : reinterpret_cast<const uint32_t*>(row)[u];
    }
  };
  auto load = [&](T(&z)[KU], T(&t)[KU], int b) {
#pragma unroll
    for (int k = 0; k < KU; ++k) {
      const int u = b + k * THREADS;
      if (u < u1) {
        z[k] = ld(zrow, u);
        t[k] = ld(trow, u);
      }
    }
  };
  auto run = [&](const T(&z)[KU], const T(&t)[KU], int b) {
#pragma unroll
    for (int k = 0; k < KU; ++k) {
      const int u = b + k * THREADS;
      if (u < u1) f(z[k], t[k], u);
    }
  };
  if (base < u1) load(za, ta, base);
  for (int b = base; b < u1; b += 2 * STEP) {
    if (b + STEP < u1) load(zb, tb, b + STEP);
    run(za, ta, b);
    if (b + 2 * STEP < u1) load(za, ta, b + 2 * STEP);
    if (b + STEP < u1) run(zb, tb, b + STEP);
  }
}

template <int BLOCK>
__device__ __forceinline__ void block_lse2(float& mz, float& sz, float& mt, float& st,
                                           float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float m2 = __shfl_xor(mz, o, 64), s2 = __shfl_xor(sz, o, 64);
    lse_merge(mz, sz, m2, s2);
    m2 = __shfl_xor(mt, o, 64);
    s2 = __shfl_xor(st, o, 64);
    lse_merge(mt, st, m2, s2);
  }
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int NW = BLOCK / 64;
  if (lane == 0) {
    red[4 * w + 0] = mz; red[4 * w + 1] = sz;
    red[4 * w + 2] = mt; red[4 * w + 3] = st;
  }
  __syncthreads();
  mz = red[0]; sz = red[1]; mt = red[2]; st = red[3];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    lse_merge(mz, sz, red[4 * i + 0], red[4 * i + 1]);
    lse_merge(mt, st, red[4 * i + 2], red[4 * i + 3]);
  }
  __syncthreads();
}

template <int BLOCK>
__device__ __forceinline__ void block_sum2(float& a, float& b, float* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int NW = BLOCK / 64;
  if (lane == 0) {
    red[2 * w] = a;
    red[2 * w + 1] = b;
  }
  __syncthreads();
  a = 0.f;
  b = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    a += red[2 * i];
    b += red[2 * i + 1];
  }
  __syncthreads();
}

// Cross-workgroup exchange.  The XCDs' L2 caches are not coherent with each
// other, and device-scope release/acquire would write back / invalidate a
// whole L2 per use.  Instead every exchanged word is a device-scope relaxed
// atomic access (individually coherent across the XCDs, no fence).  A row
// posts its (alpha, G) as one 64-bit word whose top bit marks it posted (the
// slots are cleared before the rows run; alpha >= 0 leaves its sign bit
// free), so a reader that sees the mark has the values in the same access.
// Numerators are posted and acknowledged before the branch is counted.
__device__ __forceinline__ void post_f64(double* p, double v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double peek_f64(const double* p) {
  return __hip_atomic_load(const_cast<double*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
constexpr unsigned long long kPosted = 1ull << 63;
__device__ __forceinline__ unsigned long long pack_slot(float al, float g) {
  return kPosted | (static_cast<unsigned long long>(__float_as_uint(al)) << 32) | __float_as_uint(g);
}

struct FusedArgs {
  const void* draft;
  const void* target;
  const int32_t* target_row;  // NULL: node n's target is row n
  int target_rows;
  const int32_t* parent;
  int Wn, V;
  double count;
  float grad_scale;
  int spin_limit;
  int defer_all;  // every row that may defer does so without waiting
  unsigned long long* slot;  // [N] posted (alpha, G) of every row, 0 until posted
  int32_t* ticket;
  int32_t* done;    // branches that reported their numerator
  int R;
  double* numer;
  double* loss_out;  // loss, numerator sum, count
  int32_t* branch_ok;
  float* alpha_out;
  float* prefix_out;
  void* grad;
  int32_t* ndefer;  // rows whose wait gave up
  int32_t* defer;   // [N] those rows, in the order they gave up
  float2* lse;      // [N] (-log2-sum-exp2) of draft and target of each deferred row
};

// The target-logit row of node n: row n, or the row target_row names.  An
// index outside the target matrix reads row 0 and marks the branch
// malformed (the row posts NaN, so its whole branch comes out NaN).
__device__ __forceinline__ size_t target_row_of(const FusedArgs& a, int n, bool& ok) {
  ok = true;
  if (!a.target_row) return size_t(n);
  const int tr = a.target_row[n];
  if (tr < 0 || tr >= a.target_rows) {
    ok = false;
    return 0;
  }
  return size_t(tr);
}

// Lane k of a wave holds node k of a branch (Wn <= 64).  Uniform-index
// reads of another lane's value.
__device__ __forceinline__ double lane_f64(double v, int l) {
  const unsigned long long u = __double_as_longlong(v);
  const unsigned lo = __builtin_amdgcn_readlane(unsigned(u), l);
  const unsigned hi = __builtin_amdgcn_readlane(unsigned(u >> 32), l);
  return __longlong_as_double((static_cast<unsigned long long>(hi) << 32) | lo);
}

// The first wave of a row's workgroup (all 64 lanes): publish the row's
// (alpha, G) (when `post`) and -- if the row needs the branch (gradient rows,
// and the branch's first row, which reports the branch) -- wait until every
// row of the branch has posted (lane k polls node k's slot; bounded), then
// scan the branch in fp64: prefix products P_k = alpha_k P_parent, suffix
// sums S_k = 1 + sum over children c of alpha_c S_c, and this row's gradient
// coefficients s_val[0] (where q < p) and s_val[1] (elsewhere).  The scan
// walks the nodes in index order (children come after their parents) with
// every value held by its node's lane, so every row of a branch does the
// same arithmetic in the same order, in whichever kernel it runs.
// When the wait gives up (or, with SPECOPD_E2ETV_DEFER_ALL, without waiting)
// and `can_defer`, the row records its log-sum-exps,
// appends itself to the deferred list and sets s_val[2]; its scan and
// gradient are then done by e2etv_rescue_kernel.
__device__ __forceinline__ void post_and_scan(const FusedArgs& a, int n, int r, int j,
                                              unsigned long long mine, bool post, bool need_scan,
                                              bool can_defer, float nlz, float nlt, float* s_val) {
  const int lane = int(threadIdx.x) & 63;
  const float qnan = __builtin_nanf("");
  if (post && lane == 0) __hip_atomic_store(a.slot + n, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!need_scan) return;
  const int Wn = a.Wn;
  unsigned long long* const bs = a.slot + size_t(r) * Wn;
  // this row's own slot is known when it was just posted; lanes past the
  // branch have nothing to wait for
  unsigned long long v = (post && lane == j) ? mine : 0ull;
  bool have = lane >= Wn || (post && lane == j);
  for (int spins = 0; !(can_defer && a.defer_all);) {
    if (!have) {
      v = __hip_atomic_load(bs + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      have = (v & kPosted) != 0;
    }
    if (__builtin_amdgcn_ballot_w64(!have) == 0 || ++spins > a.spin_limit) break;
    if (spins < 32)  // back off after the first polls
      __builtin_amdgcn_s_sleep(2);
    else
      __builtin_amdgcn_s_sleep(8);
  }
  if (can_defer && (a.defer_all || __builtin_amdgcn_ballot_w64(!have) != 0)) {
    if (lane == 0) {
      a.lse[n] = make_float2(nlz, nlt);
      const int at = __hip_atomic_fetch_add(a.ndefer, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a.defer[at] = n;
      s_val[2] = 1.f;
    }
    return;
  }
  bool lok = have;
  int pk = -1;
  double ak = 0.0;
  float gk = 0.f;
  if (lane < Wn) {
    pk = a.parent[size_t(r) * Wn + lane];
    if (pk < -1 || pk >= lane) {
      lok = false;
      pk = -1;
    }
    ak = double(__uint_as_float(unsigned(v >> 32) & 0x7fffffffu));
    gk = __uint_as_float(unsigned(v));
    if (!(ak == ak)) lok = false;  // undefined overlap (bad target row, NaN logits)
  }
  const bool ok = __builtin_amdgcn_ballot_w64(!lok) == 0;
  double P = 0.0, sum = 0.0;
  for (int k = 0; k < Wn; ++k) {
    const int pkk = __builtin_amdgcn_readlane(pk, k);
    const double Pk = lane_f64(ak, k) * (pkk < 0 ? 1.0 : lane_f64(P, pkk));
    if (lane == k) P = Pk;
    sum += Pk;
  }
  double S = 1.0;
  for (int k = Wn - 1; k > 0; --k) {
    const int pkk = __builtin_amdgcn_readlane(pk, k);
    if (pkk >= 0) {
      const double v = lane_f64(ak, k) * lane_f64(S, k);
      if (lane == pkk) S += v;
    }
  }
  const int pj = __builtin_amdgcn_readlane(pk, j);
  const double pp = pj >= 0 ? lane_f64(P, pj) : 1.0;
  const double Gj = double(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gk), j)));
  const double c = -double(a.grad_scale) * pp * lane_f64(S, j) / a.count;
  if (lane == 0) {
    s_val[0] = ok ? float(c * (1.0 - Gj)) : qnan;  // coefficient where q < p
    s_val[1] = ok ? float(-c * Gj) : qnan;         // elsewhere
    if (!ok) a.branch_ok[r] = 0;
  }
  if (j == 0) {
    if (lane < Wn) {
      if (a.alpha_out) a.alpha_out[size_t(r) * Wn + lane] = ok ? float(ak) : qnan;
      if (a.prefix_out) a.prefix_out[size_t(r) * Wn + lane] = ok ? float(P) : qnan;
    }
    // report the branch's numerator; the branch that reports last (its
    // count is the R-th) reads them all back and writes the loss
    int last = 0;
    if (lane == 0) {
      post_f64(&a.numer[r], ok ? sum : double(qnan));
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // numerator acknowledged first
      last = __hip_atomic_fetch_add(a.done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.R - 1;
    }
    if (__builtin_amdgcn_readfirstlane(last)) {
      // lane l adds branches l, l + 64, ... in order, then a butterfly over
      // the wave (both lanes of a pair add the same two values, so every lane
      // ends with the same sum, in an order fixed by the branch indices)
      double t = 0.0;
      for (int b = lane; b < a.R; b += 64) t += peek_f64(&a.numer[b]);
#pragma unroll
      for (int w = 32; w >= 1; w >>= 1) t += __shfl_xor(t, w, 64);
      if (lane == 0) {
        a.loss_out[0] = 1.0 - t / a.count;
        a.loss_out[1] = t;
        a.loss_out[2] = a.count;
      }
    }
  }
}

__global__ void e2etv_zero_kernel(int32_t* __restrict__ ticket, int32_t* __restrict__ done,
                                  int32_t* __restrict__ ndefer, unsigned long long* __restrict__ slot,
                                  int N, int32_t* __restrict__ branch_ok, int R) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) {
    *ticket = 0;
    *done = 0;
    *ndefer = 0;
  }
  if (i < N) slot[i] = 0;  // not posted
  if (i < R) branch_ok[i] = 1;  // cleared by any workgroup of the branch that finds a problem
}

// Elements of a streamed unit as fp32: a 16-byte vector, or one raw element.
template <bool BF16, bool VECTOR>
struct Unit {
  static constexpr int NV = VECTOR ? (BF16 ? 8 : 4) : 1;
  template <typename T>
  __device__ static __forceinline__ float get(const T& w, int i) {
    if constexpr (VECTOR) {
      if constexpr (BF16) return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
      else return __uint_as_float(w[i]);
    } else {
      if constexpr (BF16) return bf16_to_f32(uint16_t(w));
      else return __uint_as_float(w);
    }
  }
};

// Pass C of the streaming form: grad[u] = q_u * (c1 where q_u < p_u, else
// c0) over one row, all kThreads threads of the workgroup.
template <bool BF16, bool VECTOR, bool GBF16>
__device__ __forceinline__ void stream_grad(const FusedArgs& a, size_t row, const void* zrow,
                                            const void* trow, float nlz, float nlt, float c1,
                                            float c0) {
  using U = Unit<BF16, VECTOR>;
  constexpr int NV = U::NV;
  constexpr int ESZ = BF16 ? 2 : 4;
  const int tid = threadIdx.x;
  const int V = a.V;
  const int units = V / NV;
  const int e0 = units * NV;
  auto load1 = [&](const void* rowp, int e) -> float {
    if constexpr (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(rowp)[e]);
    else return reinterpret_cast<const float*>(rowp)[e];
  };
  auto gradv = [&](float z, float t) {
    float lq, lp;
    log2probs(z, t, nlz, nlt, lq, lp);
    return fast_exp2(lq) * (lq < lp ? c1 : c0);
  };
  stream_pairs<VECTOR, true>(zrow, trow, 0, units, ESZ, [&](const auto& zw, const auto& tw, int u) {
    float gv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) gv[i] = gradv(U::get(zw, i), U::get(tw, i));
    if constexpr (VECTOR) {
      if constexpr (GBF16) {
        uint16_t* o = reinterpret_cast<uint16_t*>(a.grad) + row + size_t(u) * NV;
        if constexpr (NV == 8) {
          const u32x4 w = {pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3]),
                           pack_bf16x2(gv[4], gv[5]), pack_bf16x2(gv[6], gv[7])};
          __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(o));
        } else {
          const u32x2 w = {pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3])};
          __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(o));
        }
      } else {
        float* o = reinterpret_cast<float*>(a.grad) + row + size_t(u) * NV;
#pragma unroll
        for (int i = 0; i < NV; i += 4)
          __builtin_nontemporal_store(f32x4{gv[i], gv[i + 1], gv[i + 2], gv[i + 3]},
                                      reinterpret_cast<f32x4*>(o + i));
      }
    } else {
      if constexpr (GBF16)
        reinterpret_cast<uint16_t*>(a.grad)[row + u] = f32_to_bf16(gv[0]);
      else
        reinterpret_cast<float*>(a.grad)[row + u] = gv[0];
    }
  });
  for (int e = e0 + tid; e < V; e += kThreads) {
    const float gv = gradv(load1(zrow, e), load1(trow, e));
    if constexpr (GBF16)
      reinterpret_cast<uint16_t*>(a.grad)[row + e] = f32_to_bf16(gv);
    else
      reinterpret_cast<float*>(a.grad)[row + e] = gv;
  }
}

template <bool BF16, bool VECTOR, bool GRAD, bool GBF16>
__global__ __launch_bounds__(kThreads) void e2etv_fused_kernel(const FusedArgs a) {
  using U = Unit<BF16, VECTOR>;
  constexpr int NV = U::NV;
  constexpr int ESZ = BF16 ? 2 : 4;
  __shared__ float red[4 * (kThreads / 64)];
  __shared__ int s_unit;
  __shared__ float s_val[4];

  const int tid = threadIdx.x;
  if (tid == 0) {
    s_unit = __hip_atomic_fetch_add(a.ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_val[2] = 0.f;
  }
  __syncthreads();
  const int n = s_unit;
  const int r = n / a.Wn;
  const int j = n - r * a.Wn;
  const int V = a.V;
  const size_t row = size_t(n) * size_t(V);
  bool tok;
  const size_t trw = target_row_of(a, n, tok) * size_t(V);
  const void* zrow = static_cast<const char*>(a.draft) + row * ESZ;
  const void* trow = static_cast<const char*>(a.target) + trw * ESZ;
  const int units = V / NV;  // whole units; a vector row's ragged tail is done element-wise
  const int e0 = units * NV;
  auto load1 = [&](const void* rowp, int e) -> float {
    if constexpr (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(rowp)[e]);
    else return reinterpret_cast<const float*>(rowp)[e];
  };

  // ---- pass A: log-sum-exp of both rows
  float mz = kNegInf, sz = 0.f, mt = kNegInf, st = 0.f;
  stream_pairs<VECTOR, false>(zrow, trow, 0, units, ESZ, [&](const auto& zw, const auto& tw, int) {
    float z[NV], t[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      z[i] = U::get(zw, i);
      t[i] = U::get(tw, i);
    }
    lse_update_lazy<NV>(mz, sz, z);
    lse_update_lazy<NV>(mt, st, t);
  });
  for (int e = e0 + tid; e < V; e += kThreads) {
    float z[1] = {load1(zrow, e)}, t[1] = {load1(trow, e)};
    lse_update<1>(mz, sz, z);
    lse_update<1>(mt, st, t);
  }
  block_lse2<kThreads>(mz, sz, mt, st, red);
  // -log2-sum-exp2 of the log2e-scaled logits; a row of only -inf gives NaN
  const float nlz = -(mz * kLog2e + log2f(sz));
  const float nlt = -(mt * kLog2e + log2f(st));

  // ---- pass B: alpha = sum min(q, p), G = sum_{q<p} q
  float al = 0.f, g = 0.f;
  auto overlap = [&](float z, float t) {
    float lq, lp;
    log2probs(z, t, nlz, nlt, lq, lp);
    const float e = fast_exp2(fminf(lq, lp));
    al += e;
    g += (lq < lp) ? e : 0.f;
  };
  stream_pairs<VECTOR, false>(zrow, trow, 0, units, ESZ, [&](const auto& zw, const auto& tw, int) {
#pragma unroll
    for (int i = 0; i < NV; ++i) overlap(U::get(zw, i), U::get(tw, i));
  });
  for (int e = e0 + tid; e < V; e += kThreads) overlap(load1(zrow, e), load1(trow, e));
  block_sum2<kThreads>(al, g, red);
  if (!tok) {
    al = __builtin_nanf("");
    if (tid == 0) a.branch_ok[r] = 0;
  }

  // ---- post, wait for the branch, scan
  if (tid < 64) post_and_scan(a, n, r, j, pack_slot(al, g), true, GRAD || j == 0, true, nlz, nlt, s_val);
  if constexpr (!GRAD) return;
  __syncthreads();
  if (s_val[2] != 0.f) return;  // handed to the rescue kernel

  // ---- pass C: gradient
  stream_grad<BF16, VECTOR, GBF16>(a, row, zrow, trow, nlz, nlt, s_val[0], s_val[1]);
}

// Rows whose wait for their branch gave up in the main kernel: every row has
// posted by now (this kernel runs after it on the same stream), so the scan
// finds every slot at once; the gradient is the streaming pass C with the
// row's stored log-sum-exps, i.e. the same arithmetic the row would have done.
template <bool BF16, bool VECTOR, bool GRAD, bool GBF16>
__global__ __launch_bounds__(kThreads) void e2etv_rescue_kernel(const FusedArgs a) {
  constexpr int ESZ = BF16 ? 2 : 4;
  __shared__ float s_val[4];
  const int cnt = *a.ndefer;
  const int tid = threadIdx.x;
  for (int i = blockIdx.x; i < cnt; i += gridDim.x) {
    const int n = a.defer[i];
    const int r = n / a.Wn;
    const int j = n - r * a.Wn;
    const float2 l = a.lse[n];
    if (tid < 64) post_and_scan(a, n, r, j, 0ull, false, true, false, l.x, l.y, s_val);
    if constexpr (GRAD) {
      __syncthreads();
      const size_t row = size_t(n) * size_t(a.V);
      bool tok;
      const size_t trw = target_row_of(a, n, tok) * size_t(a.V);
      stream_grad<BF16, VECTOR, GBF16>(a, row, static_cast<const char*>(a.draft) + row * ESZ,
                                       static_cast<const char*>(a.target) + trw * ESZ, l.x, l.y,
                                       s_val[0], s_val[1]);
      __syncthreads();  // s_val is rewritten by the next row
    }
  }
}

// ---------------------------------------------------------------- resident rows
// bf16 logits with 16-byte aligned rows: the same three passes, but most of
// the row stays on chip between them, so passes B and C re-read only the
// remainder.  One workgroup of 512 threads fills a CU (its registers and
// LDS).  Thread tid keeps the 8-element units k * 512 + tid, k < kResUnits,
// in registers (16-byte loads); the next kResLds blocks of 4096 elements go
// to LDS straight from memory (16 bytes per lane); the elements past those
// are streamed in every pass, 4 at a time.  Every gradient store is a
// contiguous 16 bytes per lane (1 KB per wave), which the memory system
// writes at full rate (per-lane stores 32 bytes apart do not combine as
// well): the LDS blocks and the streamed elements are read as quads of 4 in
// pass C, and the gradients of register units go through a per-wave LDS
// staging area (the space of the first LDS block, once it is done) that
// turns 8 consecutive values per lane into 4.  Pass A loads the streamed quads last and passes B and C
// take them first, so their re-reads find them in L2 while they are the
// most recently used lines; the resident elements are loaded with a
// non-temporal hint, which keeps them from pushing the streamed ones out.
constexpr int kResThreads = 512;
constexpr int kResUnits = 24;  // 8-element units per thread held in registers (192 VGPRs)
constexpr int kResLds = 9;     // LDS blocks of 4096 elements (144 KiB)
constexpr int kResRegElems = kResUnits * kResThreads * 8;
constexpr int kResElems = kResRegElems + kResLds * 4096;
constexpr int kStreamBatch = 4;  // streamed loads per thread in flight

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void unpack8(const u32x4& w, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16_lo(w[e]);
    x[2 * e + 1] = bf16_hi(w[e]);
  }
}
__device__ __forceinline__ void unpack4(const u32x2_t& w, float (&x)[4]) {
  x[0] = bf16_lo(w[0]);
  x[1] = bf16_hi(w[0]);
  x[2] = bf16_lo(w[1]);
  x[3] = bf16_hi(w[1]);
}

// Makes the compiler treat the resident registers as rewritten, so that each
// pass unpacks them afresh instead of keeping the fp32 values of an earlier
// pass alive (twice the registers).
template <int N>
__device__ __forceinline__ void reopen(u32x4 (&x)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) asm volatile("" : "+v"(x[k]));
}

// Raw buffer access: one per-lane offset register serves every quad (the
// quad's distance goes in the scalar offset).  Callers keep every access
// inside the row themselves.
constexpr int kBufFlags = 0x00020000;  // gfx9 raw buffer resource word 3
constexpr int kNT = 2;                 // non-temporal cache policy
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, kBufFlags);
}
template <int AUX>
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX));
}
template <int AUX>
__device__ __forceinline__ u32x2_t buf_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX));
}
// The same loads with the whole byte offset in the per-lane offset, which the
// buffer's range check covers (the scalar offset is not checked): past the
// row they return zeros without a memory access.  Issued unconditionally, so
// that the loads of a pass stay in one straight block; loads under per-unit
// conditions split it into blocks across which the compiler's wait
// bookkeeping loses count and waits for every load in flight at the first use.
template <int AUX>
__device__ __forceinline__ u32x4 buf_load16c(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}
template <int AUX>
__device__ __forceinline__ u32x2_t buf_load8c(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX));
}

// Gradient of elements [e, e + 4) of a row, e = 4 * (quad), through a buffer
// resource over the row's gradient: 16 bytes (fp32) or 8 bytes (bf16) per lane.
template <bool GBF16>
__device__ __forceinline__ void store_grad4(__amdgpu_buffer_rsrc_t r, int e, const float (&gv)[4]) {
  const int vo = int(threadIdx.x) * (GBF16 ? 8 : 16);
  const int so = (e - 4 * int(threadIdx.x)) * (GBF16 ? 2 : 4);
  if constexpr (GBF16) {
    const u32x2_t w = {pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3])};
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, w), r, vo, so, kNT);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{gv[0], gv[1], gv[2], gv[3]}), r,
                                           vo, so, kNT);
  }
}

// Calls f(integral_constant<k>) for k = 0 .. N-1, each after waiting until at
// most 2 (N - 1 - k) of this wave's vector-memory loads are in flight (the
// two loads of each later LDS block).
template <int N, int K = 0, typename F>
__device__ __forceinline__ void lds_blocks_in_order(F&& f) {
  if constexpr (K < N) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (N - 1 - K)) : "memory");
    f(std::integral_constant<int, K>{});
    lds_blocks_in_order<N, K + 1>(f);
  }
}

template <bool GRAD, bool GBF16>
__global__ __launch_bounds__(kResThreads, 1) void e2etv_resident_kernel(const FusedArgs a) {
  typedef __attribute__((address_space(3))) void lds_void;
  // LDS-resident elements: [block][tensor][4096 elements]
  __shared__ __attribute__((aligned(16))) uint16_t s_row[kResLds * 2 * 4096];
  __shared__ float red[4 * (kResThreads / 64)];
  __shared__ int s_unit;
  __shared__ float s_val[4];

  const int tid = threadIdx.x, wave = tid >> 6;
  if (tid == 0) {
    s_unit = __hip_atomic_fetch_add(a.ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_val[2] = 0.f;
  }
  __syncthreads();
  // uniform: the row's addresses and buffer resources stay in scalar registers
  const int n = __builtin_amdgcn_readfirstlane(s_unit);
  const int r = n / a.Wn;
  const int j = n - r * a.Wn;
  const int V = a.V;
  const size_t row = size_t(n) * size_t(V);
  bool tok;
  const size_t trw = target_row_of(a, n, tok) * size_t(V);
  const uint16_t* zrow = static_cast<const uint16_t*>(a.draft) + row;
  const uint16_t* trow = static_cast<const uint16_t*>(a.target) + trw;
  const __amdgpu_buffer_rsrc_t zres = buf_rsrc(zrow, V * 2), tres = buf_rsrc(trow, V * 2);
  const int sbeg = min(V, kResElems);  // first streamed element (a multiple of 4)

  // first element of register unit k
  auto reg_e = [&](int k) { return (k * kResThreads + tid) * 8; };
  // one pass over the streamed elements, W per lane per load (8: 16-byte
  // loads, 4: quads), kStreamBatch loads per thread at a time, the next
  // batch in flight while the current one is used.  Every access below is
  // guarded by the row length (the buffer range check is a second line only)
  auto stream = [&](auto wtag, auto&& f, int s0) {
    constexpr int W = decltype(wtag)::value;
    using VT = typename std::conditional<W == 8, u32x4, u32x2_t>::type;
    constexpr int SB = W == 8 ? kStreamBatch / 2 : kStreamBatch, STEP = kResThreads * W, BSTEP = STEP * SB;
    if (s0 + tid * W >= V) return;
    VT zc[SB], tc[SB], zn[SB], tn[SB];
    auto load = [&](VT(&z)[SB], VT(&t)[SB], int e0) {
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int off = (e0 + i * STEP + tid * W) * 2;  // past the row: zeros, no access
        if constexpr (W == 8) {
          z[i] = buf_load16c<0>(zres, off);
          t[i] = buf_load16c<0>(tres, off);
        } else {
          z[i] = buf_load8c<0>(zres, off);
          t[i] = buf_load8c<0>(tres, off);
        }
      }
    };
    load(zc, tc, s0);
    for (int e0 = s0; e0 < V; e0 += BSTEP) {
      load(zn, tn, e0 + BSTEP);
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int e = e0 + i * STEP + tid * W;
        if (e < V) f(zc[i], tc[i], e);
      }
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        zc[i] = zn[i];
        tc[i] = tn[i];
      }
    }
  };
  using W8 = std::integral_constant<int, 8>;
  using W4 = std::integral_constant<int, 4>;

  // ---- pass A: load the resident elements and the first streamed batch,
  // then the rest of the stream; log-sum-exps.  Loads go out in the order
  // register units, first streamed batch, LDS blocks, so that each LDS block
  // can be waited for on its own (the loads after it are the later blocks
  // only) and summed while the later ones arrive.
  // (every load is issued; units past the row read zeros and are not used)
  u32x4 zr[kResUnits], tr[kResUnits];
#pragma unroll
  for (int k = 0; k < kResUnits; ++k) {
    zr[k] = buf_load16c<kNT>(zres, reg_e(k) * 2);
    tr[k] = buf_load16c<kNT>(tres, reg_e(k) * 2);
  }
  constexpr int SB0 = kStreamBatch / 2, STEP0 = kResThreads * 8;  // the stream's first batch (16-byte units)
  u32x4 zs[SB0], ts[SB0];
#pragma unroll
  for (int i = 0; i < SB0; ++i) {
    zs[i] = buf_load16c<0>(zres, (sbeg + i * STEP0 + tid * 8) * 2);
    ts[i] = buf_load16c<0>(tres, (sbeg + i * STEP0 + tid * 8) * 2);
  }
#pragma unroll
  for (int k = 0; k < kResLds; ++k) {
    // straight into LDS; each lane's 16 bytes land at the wave's base + 16 * lane
    uint16_t* zb = s_row + (2 * k) * 4096 + wave * 512;
    const int off = (kResRegElems + k * 4096 + tid * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(zres, (lds_void*)zb, 16, off, 0, 0, kNT);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(tres, (lds_void*)(zb + 4096), 16, off, 0, 0, kNT);
  }
  float mz = kNegInf, sz = 0.f, mt = kNegInf, st = 0.f;
  auto lse8 = [&](const u32x4& zw, const u32x4& tw) {
    float z[8], t[8];
    unpack8(zw, z);
    unpack8(tw, t);
    lse_update_lazy<8>(mz, sz, z);
    lse_update_lazy<8>(mt, st, t);
  };
#pragma unroll
  for (int k = 0; k < kResUnits; ++k)
    if (reg_e(k) < V) lse8(zr[k], tr[k]);
  // each thread reads back the 16 bytes its own lane loaded
  auto lds8 = [&](int k, int x) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(s_row + (2 * k + x) * 4096 + tid * 8);
  };
  // block k is in once at most the 2 (kResLds - 1 - k) loads of the later
  // blocks are in flight
  lds_blocks_in_order<kResLds>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    if (kResRegElems + k * 4096 + tid * 8 < V) lse8(lds8(k, 0), lds8(k, 1));
  });
#pragma unroll
  for (int i = 0; i < SB0; ++i)
    if (sbeg + i * STEP0 + tid * 8 < V) lse8(zs[i], ts[i]);
  stream(W8{}, [&](const u32x4& zw, const u32x4& tw, int) { lse8(zw, tw); }, sbeg + SB0 * STEP0);
  block_lse2<kResThreads>(mz, sz, mt, st, red);
  const float nlz = -(mz * kLog2e + log2f(sz));
  const float nlt = -(mt * kLog2e + log2f(st));

  // ---- pass B: alpha = sum min(q, p), G = sum_{q<p} q; streamed quads first
  reopen(zr);
  reopen(tr);
  float al = 0.f, g = 0.f;
  auto overlap8 = [&](const u32x4& zw, const u32x4& tw) {
    float z[8], t[8];
    unpack8(zw, z);
    unpack8(tw, t);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float lq, lp;
      log2probs(z[i], t[i], nlz, nlt, lq, lp);
      const float e = fast_exp2(fminf(lq, lp));
      al += e;
      g += (lq < lp) ? e : 0.f;
    }
  };
  stream(W8{}, [&](const u32x4& zw, const u32x4& tw, int) { overlap8(zw, tw); }, sbeg);
#pragma unroll
  for (int k = 0; k < kResUnits; ++k)
    if (reg_e(k) < V) overlap8(zr[k], tr[k]);
#pragma unroll 1
  for (int k = 0; k < kResLds; ++k)
    if (kResRegElems + k * 4096 + tid * 8 < V) overlap8(lds8(k, 0), lds8(k, 1));
  block_sum2<kResThreads>(al, g, red);
  if (!tok) {
    al = __builtin_nanf("");
    if (tid == 0) a.branch_ok[r] = 0;
  }

  // ---- post, wait for the branch, scan
  if (tid < 64) post_and_scan(a, n, r, j, pack_slot(al, g), true, GRAD || j == 0, true, nlz, nlt, s_val);
  if constexpr (!GRAD) return;
  __syncthreads();
  if (s_val[2] != 0.f) return;  // handed to the rescue kernel

  // ---- pass C: gradient, streamed quads first
  reopen(zr);
  reopen(tr);
  const float c1 = s_val[0], c0 = s_val[1];
  const __amdgpu_buffer_rsrc_t gres =
      buf_rsrc(static_cast<char*>(a.grad) + row * (GBF16 ? 2 : 4), V * (GBF16 ? 2 : 4));
  auto grad4 = [&](const u32x2_t& zw, const u32x2_t& tw, int e) {
    float z[4], t[4], gv[4];
    unpack4(zw, z);
    unpack4(tw, t);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float lq, lp;
      log2probs(z[i], t[i], nlz, nlt, lq, lp);
      gv[i] = fast_exp2(lq) * (lq < lp ? c1 : c0);
    }
    store_grad4<GBF16>(gres, e, gv);
  };
  stream(W4{}, grad4, sbeg);
  // LDS blocks, read as quads here (any wave's block: every wave's loads
  // completed before the barriers of pass B); block 0 first, so that its
  // space can then stage the register units' gradients
  auto lds_block = [&](int k) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int o = h * 2048 + tid * 4;  // element within the block
      const int e = kResRegElems + k * 4096 + o;
      if (e < V) {
        const u32x2_t zw = *reinterpret_cast<const u32x2_t*>(s_row + (2 * k) * 4096 + o);
        const u32x2_t tw = *reinterpret_cast<const u32x2_t*>(s_row + (2 * k + 1) * 4096 + o);
        grad4(zw, tw, e);
      }
    }
  };
  lds_block(0);
  __syncthreads();  // block 0 is free
  // register units: a lane's 8 values go to the wave's 2 KB of staging and
  // come back as two quads, elements [4 l, 4 l + 4) and [256 + 4 l, ...) of
  // the wave's 512 (LDS operations of one wave complete in order)
  float* const stage = reinterpret_cast<float*>(s_row) + wave * 512;
  const int lane = tid & 63;
#pragma unroll
  for (int k = 0; k < kResUnits; ++k) {
    const int w0 = (k * kResThreads + wave * 64) * 8;  // first element of the wave's span
    if (w0 < V) {
      float z[4], t[4], gv[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        unpack4(u32x2_t{zr[k][2 * hh], zr[k][2 * hh + 1]}, z);
        unpack4(u32x2_t{tr[k][2 * hh], tr[k][2 * hh + 1]}, t);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float lq, lp;
          log2probs(z[i], t[i], nlz, nlt, lq, lp);
          gv[4 * hh + i] = fast_exp2(lq) * (lq < lp ? c1 : c0);
        }
      }
      *reinterpret_cast<f32x4*>(stage + lane * 8) = f32x4{gv[0], gv[1], gv[2], gv[3]};
      *reinterpret_cast<f32x4*>(stage + lane * 8 + 4) = f32x4{gv[4], gv[5], gv[6], gv[7]};
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int o = hh * 256 + lane * 4;
        if (w0 + o < V) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(stage + o);
          const float q4[4] = {x[0], x[1], x[2], x[3]};
          store_grad4<GBF16>(gres, w0 + o, q4);
        }
      }
    }
  }
#pragma unroll 1
  for (int k = 1; k < kResLds; ++k) lds_block(k);
}

template <bool BF16, bool VECTOR>
hipError_t launch_all(const specopd_e2etv_desc& d, const E2etvArgs& a, hipStream_t s, int spin_limit) {
  const E2etvWs L = e2etv_ws_layout(d);
  const int R = d.R, Wn = d.Wn;
  const int N = R * Wn;
  FusedArgs f{};
  f.draft = a.draft;
  f.target = a.target;
  f.target_row = a.target_row;
  f.target_rows = d.target_rows;
  f.parent = a.parent;
  f.Wn = Wn;
  f.V = d.V;
  f.count = d.norm_count > 0 ? d.norm_count : double(N);
  f.grad_scale = d.grad_scale;
  f.spin_limit = spin_limit;
  f.defer_all = (d.flags & SPECOPD_E2ETV_DEFER_ALL) != 0;
  f.slot = reinterpret_cast<unsigned long long*>(a.ws + L.slot);
  f.ticket = reinterpret_cast<int32_t*>(a.ws + L.ticket);
  f.done = reinterpret_cast<int32_t*>(a.ws + e2etv_done_offset(L));
  f.ndefer = reinterpret_cast<int32_t*>(a.ws + e2etv_ndefer_offset(L));
  f.R = R;
  f.numer = reinterpret_cast<double*>(a.ws + L.numer);
  f.loss_out = a.loss_out;
  f.branch_ok = reinterpret_cast<int32_t*>(a.ws + L.branch_ok);
  f.alpha_out = a.alpha_out;
  f.prefix_out = a.prefix_out;
  f.grad = a.grad;
  f.defer = reinterpret_cast<int32_t*>(a.ws + L.defer);
  f.lse = reinterpret_cast<float2*>(a.ws + L.lse);
  e2etv_zero_kernel<<<(N + 255) / 256, 256, 0, s>>>(f.ticket, f.done, f.ndefer, f.slot, N, f.branch_ok, R);
  const unsigned grid = unsigned(N);
  const unsigned rgrid = unsigned(N < 256 ? N : 256);
  timing_mark(1, 0, s);
  if constexpr (BF16 && VECTOR) {
    if (!a.grad)
      e2etv_resident_kernel<false, false><<<grid, kResThreads, 0, s>>>(f);
    else if (d.grad_dtype == SPECOPD_BF16)
      e2etv_resident_kernel<true, true><<<grid, kResThreads, 0, s>>>(f);
    else
      e2etv_resident_kernel<true, false><<<grid, kResThreads, 0, s>>>(f);
  } else if (!a.grad)
    e2etv_fused_kernel<BF16, VECTOR, false, false><<<grid, kThreads, 0, s>>>(f);
  else if (d.grad_dtype == SPECOPD_BF16)
    e2etv_fused_kernel<BF16, VECTOR, true, true><<<grid, kThreads, 0, s>>>(f);
  else
    e2etv_fused_kernel<BF16, VECTOR, true, false><<<grid, kThreads, 0, s>>>(f);
  timing_mark(1, 1, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // rows whose wait gave up (normally none: the launch finds an empty list)
  if (!a.grad)
    e2etv_rescue_kernel<BF16, VECTOR, false, false><<<rgrid, kThreads, 0, s>>>(f);
  else if (d.grad_dtype == SPECOPD_BF16)
    e2etv_rescue_kernel<BF16, VECTOR, true, true><<<rgrid, kThreads, 0, s>>>(f);
  else
    e2etv_rescue_kernel<BF16, VECTOR, true, false><<<rgrid, kThreads, 0, s>>>(f);
  return hipGetLastError();
}

}  // namespace

E2etvWs e2etv_ws_layout(const specopd_e2etv_desc& d) {
  const size_t N = size_t(d.R) * size_t(d.Wn);
  E2etvWs w{};
  size_t off = 0;
  w.slot = off;      off = align_up(off + N * sizeof(unsigned long long), 256);
  // ticket, then the count of reported branches and the count of deferred
  // rows, each on a 128-byte line of its own
  w.ticket = off;    off = align_up(off + 384, 256);
  w.defer = off;     off = align_up(off + N * sizeof(int32_t), 256);
  w.lse = off;       off = align_up(off + N * 2 * sizeof(float), 256);
  w.numer = off;     off = align_up(off + size_t(d.R) * sizeof(double), 256);
  w.branch_ok = off; off = align_up(off + size_t(d.R) * sizeof(int32_t), 256);
  w.total = off;
  return w;
}

// ---------------------------------------------------------------- static scratch
// The workspace of specopd_e2etv_fwd_bwd_noalloc: one array per GPU, held by
// the library until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol); the
// device address of each GPU's copy is looked up once, with that GPU
// current, and kept.
static __device__ __align__(256) char scratch[kE2etvScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t e2etv_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_e2etv(const specopd_e2etv_desc& d, const E2etvArgs& a, hipStream_t s) {
  const int spin_limit = d.wait_polls > 0 ? d.wait_polls : (1 << 20);
  const size_t esz = d.logits_dtype == SPECOPD_BF16 ? 2 : 4;
  const bool vec = (size_t(d.V) * esz) % 16 == 0 &&
                   (reinterpret_cast<uintptr_t>(a.draft) % 16) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.target) % 16) == 0 &&
                   (a.grad == nullptr || (reinterpret_cast<uintptr_t>(a.grad) % 16) == 0);
  if (d.logits_dtype == SPECOPD_BF16)
    return vec ? launch_all<true, true>(d, a, s, spin_limit) : launch_all<true, false>(d, a, s, spin_limit);
  return vec ? launch_all<false, true>(d, a, s, spin_limit) : launch_all<false, false>(d, a, s, spin_limit);
}

}  // namespace specopd
