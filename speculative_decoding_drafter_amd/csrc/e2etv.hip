// E2E-TV surrogate forward + gradient over a proposal tree (gfx950).
//
// The loss follows the jaehun.me review of SpecOPD, §1.1 and §3.3 (Eqs. 8, 9,
// 13) and the rustineverything.app summary §2.3: per node the overlap
// alpha = sum_v min(q_v, p_v) = 1 - TV of the draft distribution q and the
// target distribution p (full-vocabulary softmaxes, target mass outside q's
// support kept), prefix products along the parent chain, loss = 1 - mean of
// the prefix products, gradient through q only.
//
// Kernels (all vocab loops are coalesced 16-byte streams):
//   rows      one workgroup per row: pass A (log-sum-exp of draft and target),
//             then pass B over the same row (alpha and G = sum_{q<p} q).  The
//             re-read of pass B follows the first read closely, so it is
//             served from the caches.
//   scan      one thread per branch: prefix products, suffix sums S, the
//             per-row coefficient grad_scale * dLoss/dalpha, branch numerator.
//   finalize  fixed-order sum of the branch numerators -> loss, numer, count.
//   grad      grad[n][u] = coef_n * q_u * ([q_u < p_u] - G_n).
// No atomics: every reduction has a fixed order, so results are bitwise
// reproducible run to run.
#include <float.h>

#include "device_common.h"
#include "internal.h"

namespace specopd {

namespace {

constexpr int kRowThreads = 512;
constexpr int kGradThreads = 256;
constexpr int kGradUnroll = 4;

// Vector loads of logits widened to fp32.  BF16: 8 values per 16 bytes; FP32:
// 4 values per 16 bytes.
template <bool BF16>
struct Logits;

template <>
struct Logits<true> {
  static constexpr int NV = 8;
  __device__ static __forceinline__ void load(const void* base, size_t idx, float (&x)[8]) {
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
        reinterpret_cast<const uint16_t*>(base) + idx));
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
    x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
    x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  }
  __device__ static __forceinline__ void load_cached(const void* base, size_t idx, float (&x)[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + idx);
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
    x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
    x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  }
  __device__ static __forceinline__ float load1(const void* base, size_t idx) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
  }
};

template <>
struct Logits<false> {
  static constexpr int NV = 4;
  __device__ static __forceinline__ void load(const void* base, size_t idx, float (&x)[4]) {
    const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(
        reinterpret_cast<const float*>(base) + idx));
    x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
  }
  __device__ static __forceinline__ void load_cached(const void* base, size_t idx, float (&x)[4]) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + idx);
    x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
  }
  __device__ static __forceinline__ float load1(const void* base, size_t idx) {
    return reinterpret_cast<const float*>(base)[idx];
  }
};

// One element's log2-probabilities.  The overlap pass and the gradient pass
// both call exactly this, so the indicator [q < p] is decided identically.
__device__ __forceinline__ void log2probs(float z, float t, float nlz, float nlt, float& lq,
                                          float& lp) {
  lq = __builtin_fmaf(z, kLog2e, nlz);
  lp = __builtin_fmaf(t, kLog2e, nlt);
}

// Running max / scaled sum over a vector of NV values.
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

template <int NV>
__device__ __forceinline__ void overlap_update(float& al, float& g, const float (&z)[NV],
                                               const float (&t)[NV], float nlz, float nlt) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float lq, lp;
    log2probs(z[i], t[i], nlz, nlt, lq, lp);
    const float e = fast_exp2(fminf(lq, lp));
    al += e;
    g += (lq < lp) ? e : 0.f;
  }
}

template <int BLOCK>
__device__ __forceinline__ void block_lse2(float& mz, float& sz, float& mt, float& st,
                                           float* red) {
  // wave level
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

// Pass A + pass B for one row per workgroup.
template <bool BF16, bool VECTOR>
__global__ __launch_bounds__(kRowThreads) void e2etv_rows_kernel(const void* __restrict__ draft,
                                                                 const void* __restrict__ target,
                                                                 int V, float4* __restrict__ rowstat) {
  using LD = Logits<BF16>;
  constexpr int NV = LD::NV;
  constexpr int U = 2;
  __shared__ float red[4 * (kRowThreads / 64)];
  const size_t row = size_t(blockIdx.x) * size_t(V);
  const int tid = threadIdx.x;
  const int nvec = VECTOR ? V / NV : 0;

  // ---- pass A: log-sum-exp of both rows
  float mz = kNegInf, sz = 0.f, mt = kNegInf, st = 0.f;
  int i = tid;
  for (; i + (U - 1) * kRowThreads < nvec; i += U * kRowThreads) {
    float z[U][NV], t[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      LD::load_cached(draft, row + size_t(i + u * kRowThreads) * NV, z[u]);
      LD::load_cached(target, row + size_t(i + u * kRowThreads) * NV, t[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      lse_update<NV>(mz, sz, z[u]);
      lse_update<NV>(mt, st, t[u]);
    }
  }
  for (; i < nvec; i += kRowThreads) {
    float z[NV], t[NV];
    LD::load_cached(draft, row + size_t(i) * NV, z);
    LD::load_cached(target, row + size_t(i) * NV, t);
    lse_update<NV>(mz, sz, z);
    lse_update<NV>(mt, st, t);
  }
  for (int e = nvec * NV + tid; e < V; e += kRowThreads) {
    float z[1] = {LD::load1(draft, row + e)}, t[1] = {LD::load1(target, row + e)};
    lse_update<1>(mz, sz, z);
    lse_update<1>(mt, st, t);
  }
  block_lse2<kRowThreads>(mz, sz, mt, st, red);
  // -log2-sum-exp2 of the log2e-scaled logits; a row of only -inf gives NaN.
  const float nlz = -(mz * kLog2e + log2f(sz));
  const float nlt = -(mt * kLog2e + log2f(st));

  // ---- pass B: alpha = sum min(q, p), G = sum_{q<p} q
  float al = 0.f, g = 0.f;
  i = tid;
  for (; i + (U - 1) * kRowThreads < nvec; i += U * kRowThreads) {
    float z[U][NV], t[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      LD::load_cached(draft, row + size_t(i + u * kRowThreads) * NV, z[u]);
      LD::load_cached(target, row + size_t(i + u * kRowThreads) * NV, t[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) overlap_update<NV>(al, g, z[u], t[u], nlz, nlt);
  }
  for (; i < nvec; i += kRowThreads) {
    float z[NV], t[NV];
    LD::load_cached(draft, row + size_t(i) * NV, z);
    LD::load_cached(target, row + size_t(i) * NV, t);
    overlap_update<NV>(al, g, z, t, nlz, nlt);
  }
  for (int e = nvec * NV + tid; e < V; e += kRowThreads) {
    float z[1] = {LD::load1(draft, row + e)}, t[1] = {LD::load1(target, row + e)};
    overlap_update<1>(al, g, z, t, nlz, nlt);
  }
  block_sum2<kRowThreads>(al, g, red);
  if (tid == 0) rowstat[blockIdx.x] = make_float4(nlz, nlt, al, g);
}

// Prefix products, suffix sums and per-row coefficients; one thread per branch.
constexpr int kScanThreads = 32;

__global__ __launch_bounds__(kScanThreads) void e2etv_scan_kernel(
    const float4* __restrict__ rowstat, const int32_t* __restrict__ parent, int R, int Wn,
    double count, float grad_scale, float* __restrict__ coef, double* __restrict__ numer,
    int32_t* __restrict__ branch_ok, float* __restrict__ alpha_out, float* __restrict__ prefix_out) {
  __shared__ double P[64 * kScanThreads];
  __shared__ double S[64 * kScanThreads];
  const int tid = threadIdx.x;
  const int r = blockIdx.x * kScanThreads + tid;
  if (r >= R) return;
  const int32_t* par = parent + size_t(r) * Wn;
  const size_t n0 = size_t(r) * Wn;
  bool ok = true;
  double sum = 0.0;
  for (int j = 0; j < Wn; ++j) {
    int p = par[j];
    if (p < -1 || p >= j) {
      ok = false;
      p = -1;
    }
    const double a = double(rowstat[n0 + j].z);
    const double pp = (p < 0) ? 1.0 : P[p * kScanThreads + tid];
    const double pj = a * pp;
    P[j * kScanThreads + tid] = pj;
    S[j * kScanThreads + tid] = 1.0;
    sum += pj;
  }
  for (int j = Wn - 1; j >= 0; --j) {
    int p = par[j];
    if (p >= 0 && p < j)
      S[p * kScanThreads + tid] += double(rowstat[n0 + j].z) * S[j * kScanThreads + tid];
  }
  const float qnan = __builtin_nanf("");
  for (int j = 0; j < Wn; ++j) {
    int p = par[j];
    const double pp = (p >= 0 && p < j) ? P[p * kScanThreads + tid] : 1.0;
    const double c = -double(grad_scale) * pp * S[j * kScanThreads + tid] / count;
    coef[n0 + j] = ok ? float(c) : qnan;
    if (alpha_out) alpha_out[n0 + j] = ok ? rowstat[n0 + j].z : qnan;
    if (prefix_out) prefix_out[n0 + j] = ok ? float(P[j * kScanThreads + tid]) : qnan;
  }
  numer[r] = ok ? sum : double(qnan);
  branch_ok[r] = ok ? 1 : 0;
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

template <bool GBF16>
__device__ __forceinline__ void store_grad(void* grad, size_t idx, const float* g, int nv);

template <>
__device__ __forceinline__ void store_grad<false>(void* grad, size_t idx, const float* g, int nv) {
  float* o = reinterpret_cast<float*>(grad) + idx;
  if (nv == 8) {
    __builtin_nontemporal_store(f32x4{g[0], g[1], g[2], g[3]}, reinterpret_cast<f32x4*>(o));
    __builtin_nontemporal_store(f32x4{g[4], g[5], g[6], g[7]}, reinterpret_cast<f32x4*>(o + 4));
  } else if (nv == 4) {
    __builtin_nontemporal_store(f32x4{g[0], g[1], g[2], g[3]}, reinterpret_cast<f32x4*>(o));
  } else {
    for (int i = 0; i < nv; ++i) o[i] = g[i];
  }
}

template <>
__device__ __forceinline__ void store_grad<true>(void* grad, size_t idx, const float* g, int nv) {
  uint16_t* o = reinterpret_cast<uint16_t*>(grad) + idx;
  if (nv == 8) {
    const u32x4 w = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                     pack_bf16x2(g[6], g[7])};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(o));
  } else if (nv == 4) {
    const u32x2 w = {pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(o));
  } else {
    for (int i = 0; i < nv; ++i) o[i] = f32_to_bf16(g[i]);
  }
}

// Gradient pass.  Workgroup b covers row b / chunks, vocabulary chunk b % chunks.
template <bool BF16, bool VECTOR, bool GBF16>
__global__ __launch_bounds__(kGradThreads) void e2etv_grad_kernel(
    const void* __restrict__ draft, const void* __restrict__ target,
    const float4* __restrict__ rowstat, const float* __restrict__ coef, int V, int chunks,
    void* __restrict__ grad) {
  using LD = Logits<BF16>;
  constexpr int NV = VECTOR ? LD::NV : 1;
  constexpr int CHUNK = kGradThreads * kGradUnroll * NV;
  const int n = blockIdx.x / chunks;
  const int c = blockIdx.x - n * chunks;
  const float4 rs = rowstat[n];
  const float cf = coef[n];
  const size_t row = size_t(n) * size_t(V);
  const int e0 = c * CHUNK;
#pragma unroll
  for (int u = 0; u < kGradUnroll; ++u) {
    const int e = e0 + (u * kGradThreads + threadIdx.x) * NV;
    if (e >= V) break;
    float z[NV], t[NV], g[NV];
    if constexpr (VECTOR) {
      LD::load(draft, row + e, z);
      LD::load(target, row + e, t);
    } else {
      z[0] = LD::load1(draft, row + e);
      t[0] = LD::load1(target, row + e);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float lq, lp;
      log2probs(z[i], t[i], rs.x, rs.y, lq, lp);
      const float q = fast_exp2(lq);
      g[i] = cf * q * ((lq < lp ? 1.f : 0.f) - rs.w);
    }
    store_grad<GBF16>(grad, row + e, g, NV);
  }
}

template <bool BF16, bool VECTOR>
hipError_t launch_all(const specopd_e2etv_desc& d, const E2etvArgs& a, hipStream_t s) {
  const E2etvWs L = e2etv_ws_layout(d);
  const int R = d.R, Wn = d.Wn, V = d.V;
  const int N = R * Wn;
  float4* rowstat = reinterpret_cast<float4*>(a.ws + L.rowstat);
  float* coef = reinterpret_cast<float*>(a.ws + L.coef);
  double* numer = reinterpret_cast<double*>(a.ws + L.numer);
  int32_t* ok = reinterpret_cast<int32_t*>(a.ws + L.branch_ok);
  const double count = d.norm_count > 0 ? d.norm_count : double(N);

  e2etv_rows_kernel<BF16, VECTOR><<<N, kRowThreads, 0, s>>>(a.draft, a.target, V, rowstat);
  e2etv_scan_kernel<<<(R + kScanThreads - 1) / kScanThreads, kScanThreads, 0, s>>>(
      rowstat, a.parent, R, Wn, count, d.grad_scale, coef, numer, ok, a.alpha_out, a.prefix_out);
  e2etv_finalize_kernel<<<1, kFinThreads, 0, s>>>(numer, R, count, a.loss_out);
  if (a.grad) {
    constexpr int NV = VECTOR ? Logits<BF16>::NV : 1;
    constexpr int CHUNK = kGradThreads * kGradUnroll * NV;
    const int chunks = (V + CHUNK - 1) / CHUNK;
    const unsigned blocks = unsigned(N) * unsigned(chunks);
    if (d.grad_dtype == SPECOPD_BF16)
      e2etv_grad_kernel<BF16, VECTOR, true><<<blocks, kGradThreads, 0, s>>>(
          a.draft, a.target, rowstat, coef, V, chunks, a.grad);
    else
      e2etv_grad_kernel<BF16, VECTOR, false><<<blocks, kGradThreads, 0, s>>>(
          a.draft, a.target, rowstat, coef, V, chunks, a.grad);
  }
  return hipGetLastError();
}

}  // namespace

E2etvWs e2etv_ws_layout(const specopd_e2etv_desc& d) {
  const size_t N = size_t(d.R) * size_t(d.Wn);
  E2etvWs w{};
  size_t off = 0;
  w.rowstat = off;   off = align_up(off + N * sizeof(float4), 256);
  w.coef = off;      off = align_up(off + N * sizeof(float), 256);
  w.numer = off;     off = align_up(off + size_t(d.R) * sizeof(double), 256);
  w.branch_ok = off; off = align_up(off + size_t(d.R) * sizeof(int32_t), 256);
  w.total = off;
  return w;
}

hipError_t launch_e2etv(const specopd_e2etv_desc& d, const E2etvArgs& a, hipStream_t s) {
  const size_t esz = d.logits_dtype == SPECOPD_BF16 ? 2 : 4;
  const bool vec = (size_t(d.V) * esz) % 16 == 0 &&
                   (reinterpret_cast<uintptr_t>(a.draft) % 16) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.target) % 16) == 0 &&
                   (a.grad == nullptr || (reinterpret_cast<uintptr_t>(a.grad) % 16) == 0);
  if (d.logits_dtype == SPECOPD_BF16)
    return vec ? launch_all<true, true>(d, a, s) : launch_all<true, false>(d, a, s);
  return vec ? launch_all<false, true>(d, a, s) : launch_all<false, false>(d, a, s);
}

}  // namespace specopd
