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
//   pass A   stream the row: log-sum-exp of draft and target;
//   pass B   stream it again (the caches serve it: it was just read):
//            alpha = sum min(q, p) and G = sum_{q<p} q;
//   post     publish (alpha, G) and count the row into its branch;
//   scan     once every row of the branch has posted, compute prefix
//            products, suffix sums S and this row's coefficient
//            c = grad_scale * dLoss/dalpha in fp64 (every row of a branch
//            repeats the same tiny scan in the same order);
//   pass C   stream the row a third time and write
//            grad[u] = c * q_u * ([q_u < p_u] - G).
// Loads are software-pipelined: the next batch of 16-byte vectors is in
// flight while the current one is reduced.  Rows are taken in order from an
// atomic ticket, so a workgroup only waits for rows of its own branch that
// were claimed just before or after it; the wait is bounded and a timeout
// marks the branch malformed rather than hanging.  The exchange goes through
// memory with cache-bypassing accesses (see post_f32).
// A small kernel sums the branch numerators in a fixed order (loss).
// No floating-point atomics: results are bitwise reproducible.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace specopd {

namespace {

constexpr int kThreads = 1024;  // per workgroup (one row)
constexpr int kCtrStride = 64;  // branch counters 256 B apart, so polls of different
                                // branches do not all land on one memory channel
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

// Stream units [u0, u1) of a row (16-byte vectors, or single elements when
// the row is not 16-byte aligned), pairs (draft, target): thread tid takes
// u0 + tid + k * kThreads.  Two register batches alternate so the next
// batch's loads are in flight while f() consumes the current one.
template <bool VECTOR, bool NT, typename F>
__device__ __forceinline__ void stream_pairs(const void* zrow, const void* trow, int u0, int u1,
                                             int esize, F&& f) {
  constexpr int STEP = kThreads * kU;
  using T = typename std::conditional<VECTOR, u32x4, uint32_t>::type;
  const int base = u0 + int(threadIdx.x);
  T za[kU], ta[kU], zb[kU], tb[kU];
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
  auto load = [&](T(&z)[kU], T(&t)[kU], int b) {
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      const int u = b + k * kThreads;
      if (u < u1) {
        z[k] = ld(zrow, u);
        t[k] = ld(trow, u);
      }
    }
  };
  auto run = [&](const T(&z)[kU], const T(&t)[kU], int b) {
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      const int u = b + k * kThreads;
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
// whole L2 per use.  Instead every exchanged word goes through memory with
// system-scope relaxed accesses (write-through stores, cache-bypassing
// loads): a workgroup posts its partials, waits until those stores are
// acknowledged, and only then bumps the counter; a reader that sees the count
// reads the partials the same cache-bypassing way.
__device__ __forceinline__ void post_f32(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float peek_f32(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void post_count(int32_t* ctr) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // partials acknowledged first
  __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
// Bounded wait until *ctr reaches want.  False on timeout.
__device__ __forceinline__ bool wait_count(int32_t* ctr, int want, int spin_limit) {
  int spins = 0;
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) < want) {
    if (++spins > spin_limit) return false;
    if (spins < 8)  // back off after the first polls
      __builtin_amdgcn_s_sleep(4);
    else
      __builtin_amdgcn_s_sleep(32);
  }
  return true;
}

struct FusedArgs {
  const void* draft;
  const void* target;
  const int32_t* parent;
  int Wn, V;
  double count;
  float grad_scale;
  int spin_limit;
  float* segB;      // [N][2] (alpha, G) of every row
  int32_t* bcount;  // [R] rows of each branch that posted
  int32_t* ticket;
  double* numer;
  int32_t* branch_ok;
  float* alpha_out;
  float* prefix_out;
  void* grad;
};

__global__ void e2etv_zero_kernel(int32_t* __restrict__ ticket, int32_t* __restrict__ bcount,
                                  int32_t* __restrict__ branch_ok, int R) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) *ticket = 0;
  if (i < R) {
    bcount[size_t(i) * kCtrStride] = 0;
    branch_ok[i] = 1;  // cleared by any workgroup of the branch that finds a problem
  }
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

template <bool BF16, bool VECTOR, bool GRAD, bool GBF16>
__global__ __launch_bounds__(kThreads) void e2etv_fused_kernel(const FusedArgs a) {
  using U = Unit<BF16, VECTOR>;
  constexpr int NV = U::NV;
  constexpr int ESZ = BF16 ? 2 : 4;
  __shared__ float red[4 * (kThreads / 64)];
  __shared__ int s_unit;
  __shared__ float s_val[4];
  __shared__ double sA[64], sP[64], sS[64];

  const int tid = threadIdx.x;
  if (tid == 0)
    s_unit = __hip_atomic_fetch_add(a.ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __syncthreads();
  const int n = s_unit;
  const int r = n / a.Wn;
  const int j = n - r * a.Wn;
  const int V = a.V;
  const size_t row = size_t(n) * size_t(V);
  const void* zrow = static_cast<const char*>(a.draft) + row * ESZ;
  const void* trow = static_cast<const char*>(a.target) + row * ESZ;
  const int units = V / NV;  // whole units; a vector row's ragged tail is done element-wise
  const int e0 = units * NV;
  const float qnan = __builtin_nanf("");
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
    lse_update<NV>(mz, sz, z);
    lse_update<NV>(mt, st, t);
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

  // ---- post, wait for the branch, scan
  const bool lead = j == 0;
  const bool need_scan = GRAD || lead;
  if (tid == 0) {
    post_f32(a.segB + size_t(n) * 2 + 0, al);
    post_f32(a.segB + size_t(n) * 2 + 1, g);
    post_count(&a.bcount[size_t(r) * kCtrStride]);
    if (need_scan) {
      bool ok = wait_count(&a.bcount[size_t(r) * kCtrStride], a.Wn, a.spin_limit);
      const int32_t* par = a.parent + size_t(r) * a.Wn;
      const float* sb = a.segB + size_t(r) * a.Wn * 2;
      double sum = 0.0, Gj = 0.0;
      for (int k = 0; k < a.Wn; ++k) {
        int pk = par[k];
        if (pk < -1 || pk >= k) {
          ok = false;
          pk = -1;
        }
        const float ak = peek_f32(sb + 2 * k), gk = peek_f32(sb + 2 * k + 1);
        if (k == j) Gj = gk;
        sA[k] = double(ak);
        sP[k] = double(ak) * (pk < 0 ? 1.0 : sP[pk]);
        sS[k] = 1.0;
        sum += sP[k];
      }
      // suffix sums S_k = 1 + sum over children c of alpha_c S_c (children
      // come after their parent, so a backward sweep sees them complete)
      for (int k = a.Wn - 1; k >= 0; --k) {
        const int pk = par[k];
        if (pk >= 0 && pk < k) sS[pk] += sA[k] * sS[k];
      }
      const int pj = par[j];
      const double pp = (pj >= 0 && pj < j) ? sP[pj] : 1.0;
      const double c = -double(a.grad_scale) * pp * sS[j] / a.count;
      s_val[0] = ok ? float(c * (1.0 - Gj)) : qnan;  // coefficient where q < p
      s_val[1] = ok ? float(-c * Gj) : qnan;         // elsewhere
      if (!ok) a.branch_ok[r] = 0;
      if (lead) {
        a.numer[r] = ok ? sum : double(qnan);
        for (int k = 0; k < a.Wn; ++k) {
          if (a.alpha_out) a.alpha_out[size_t(r) * a.Wn + k] = ok ? float(sA[k]) : qnan;
          if (a.prefix_out) a.prefix_out[size_t(r) * a.Wn + k] = ok ? float(sP[k]) : qnan;
        }
      }
    }
  }
  if constexpr (!GRAD) return;
  __syncthreads();

  // ---- pass C: gradient
  const float c1 = s_val[0], c0 = s_val[1];
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

constexpr int kFinThreads = 256;

__global__ __launch_bounds__(kFinThreads) void e2etv_finalize_kernel(const double* __restrict__ numer,
                                                                     int R, double count,
                                                                     double* __restrict__ loss_out) {
  __shared__ double red[kFinThreads];
  double s = 0.0;
  for (int r = threadIdx.x; r < R; r += kFinThreads) s += numer[r];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kFinThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double tot = red[0];
    loss_out[0] = 1.0 - tot / count;
    loss_out[1] = tot;
    loss_out[2] = count;
  }
}



template <bool BF16, bool VECTOR>
hipError_t launch_all(const specopd_e2etv_desc& d, const E2etvArgs& a, hipStream_t s, int spin_limit) {
  const E2etvWs L = e2etv_ws_layout(d);
  const int R = d.R, Wn = d.Wn;
  const int N = R * Wn;
  FusedArgs f{};
  f.draft = a.draft;
  f.target = a.target;
  f.parent = a.parent;
  f.Wn = Wn;
  f.V = d.V;
  f.count = d.norm_count > 0 ? d.norm_count : double(N);
  f.grad_scale = d.grad_scale;
  f.spin_limit = spin_limit;
  f.segB = reinterpret_cast<float*>(a.ws + L.segB);
  f.bcount = reinterpret_cast<int32_t*>(a.ws + L.bcount);
  f.ticket = reinterpret_cast<int32_t*>(a.ws + L.ticket);
  f.numer = reinterpret_cast<double*>(a.ws + L.numer);
  f.branch_ok = reinterpret_cast<int32_t*>(a.ws + L.branch_ok);
  f.alpha_out = a.alpha_out;
  f.prefix_out = a.prefix_out;
  f.grad = a.grad;
  e2etv_zero_kernel<<<(R + 255) / 256, 256, 0, s>>>(f.ticket, f.bcount, f.branch_ok, R);
  const unsigned grid = unsigned(N);
  timing_mark(1, 0, s);
  if (!a.grad)
    e2etv_fused_kernel<BF16, VECTOR, false, false><<<grid, kThreads, 0, s>>>(f);
  else if (d.grad_dtype == SPECOPD_BF16)
    e2etv_fused_kernel<BF16, VECTOR, true, true><<<grid, kThreads, 0, s>>>(f);
  else
    e2etv_fused_kernel<BF16, VECTOR, true, false><<<grid, kThreads, 0, s>>>(f);
  timing_mark(1, 1, s);
  e2etv_finalize_kernel<<<1, kFinThreads, 0, s>>>(f.numer, R, f.count, a.loss_out);
  return hipGetLastError();
}

}  // namespace

E2etvWs e2etv_ws_layout(const specopd_e2etv_desc& d) {
  const size_t N = size_t(d.R) * size_t(d.Wn);
  E2etvWs w{};
  size_t off = 0;
  w.segB = off;      off = align_up(off + N * 2 * sizeof(float), 256);
  w.bcount = off;    off = align_up(off + size_t(d.R) * kCtrStride * sizeof(int32_t), 256);
  w.ticket = off;    off = align_up(off + sizeof(int32_t), 256);
  w.numer = off;     off = align_up(off + size_t(d.R) * sizeof(double), 256);
  w.branch_ok = off; off = align_up(off + size_t(d.R) * sizeof(int32_t), 256);
  w.total = off;
  return w;
}

hipError_t launch_e2etv(const specopd_e2etv_desc& d, const E2etvArgs& a, hipStream_t s) {
  const int spin_limit = a.spin_limit > 0 ? a.spin_limit : (1 << 20);
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
