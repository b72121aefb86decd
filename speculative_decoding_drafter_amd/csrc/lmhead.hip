// LM head fused with the E2E-TV surrogate (gfx950): the draft and target
// logits are formed tile by tile on the matrix cores and used in registers;
// the [N][V] logit matrices are never written to memory.
//
// What is computed (jaehun.me review of SpecOPD, §3.3, Eqs. 8, 9, 13, and the
// §3.2(a) reading rule): z = h_draft W_draft^T for every branch node,
// t = h_target[target_row] W_target^T (a node is scored against the target
// row of its parent, or of its anchor, so siblings read one row), then the
// E2E-TV surrogate of specopd_e2etv_fwd_bwd on (z, t): per row the
// log-sum-exps, alpha = sum min(q, p) and G = sum_{q<p} q, prefix products
// along the parent map, the loss, and the gradient with respect to z.
//
// The loss needs each row's full softmax twice before the gradient, so
// without stored logits every pass recomputes its logit tiles:
//   pass A       per (row, 64-entry vocabulary chunk): max and 2^x-sum of z
//                and of t (log2 units);
//   lse kernel   per row: the chunk partials merged in chunk order;
//   pass B       per (row, chunk): partial alpha and G;
//   scan kernel  per branch: alpha and G summed in chunk order (fp64), prefix
//                products, suffix sums, each row's gradient coefficients;
//   pass C       the gradient c q_u ([q_u < p_u] - G), written once;
//   final        the loss from the branch numerators in branch order.
// Every pass forms the same tiles in the same order, so the three passes see
// bitwise the same logits and the indicator [q < p] is decided identically.
//
// Matrix-core tiles (v_mfma_f32_32x32x16_bf16, lane l = r + 32h): a
// workgroup of four waves covers 128 rows x 128 vocabulary entries, a wave
// 64 rows x 64 entries of both z and t (eight 32 x 32 accumulators).  A = 32
// head rows (vocabulary entries) x 16 hidden values, B = 16 hidden values x
// 32 hidden-state rows, both loaded straight from memory in operand layout
// (16 contiguous bytes per lane: hidden states and heads are both
// hidden-contiguous), the next step's operands loaded while the current
// step's products run.  Lane (r, h) then holds row r's logits for
// vocabulary entries 8(i/4) + 4h + i%4 of each 32-entry block, so a row's
// reductions are in-lane sums plus one exchange with lane r + 32.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace specopd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kChunk = 64;   // vocabulary entries per partial (one wave's span)
constexpr int kTileV = 128;  // per workgroup
constexpr int kTileR = 128;

struct LmhArgs {
  const uint16_t *hd, *wd, *ht, *wt;
  const int32_t *trow, *parent;
  float *alpha_out, *prefix_out;
  double* loss_out;
  float* grad;
  int32_t* bad;
  f32x4* partA;  // [N][nch] (max z, sum z, max t, sum t), log2 units
  f32x2* nl;     // [N] log2-domain log-sum-exps of z and t
  f32x2* partB;  // [N][nch] (alpha, G)
  f32x2* coef;   // [N] gradient coefficients for [q<p] = 1 / 0
  double* numer; // [R]
  int R, Wn, V, H, M, N, nch, nrt;
  double count;
  float grad_scale;
};

__device__ __forceinline__ void lse2_merge(float& m, float& s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == kNegInf) {
    m = mm;
    s = 0.f;
    return;
  }
  s = s * fast_exp2(m - mm) + s2 * fast_exp2(m2 - mm);
  m = mm;
}

template <int PASS>
__global__ __launch_bounds__(256) void lmh_pass_kernel(const LmhArgs a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, r32 = lane & 31;
  const int rt = blockIdx.x % a.nrt, vt = blockIdx.x / a.nrt;
  const int row0 = rt * kTileR + 64 * (wave & 1);
  const int v0 = vt * kTileV + 64 * (wave >> 1);
  const int H = a.H;

  // operand rows of this lane, clamped into range (out-of-range results are
  // never used)
  const uint16_t *pwd[2], *pwt[2], *phd[2], *pht[2];
  int rowv[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int v = min(v0 + 32 * x + r32, a.V - 1);
    pwd[x] = a.wd + size_t(v) * H + 8 * h;
    pwt[x] = a.wt + size_t(v) * H + 8 * h;
    const int r = min(row0 + 32 * x + r32, a.N - 1);
    rowv[x] = r;
    int tr = a.trow[r];
    tr = (tr >= 0 && tr < a.M) ? tr : 0;  // an invalid row is reported by the lse kernel
    phd[x] = a.hd + size_t(r) * H + 8 * h;
    pht[x] = a.ht + size_t(tr) * H + 8 * h;
  }

  f32x16 zacc[2][2], tacc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      zacc[x][y] = f32x16{};
      tacc[x][y] = f32x16{};
    }
  bf16x8 Ad[2], At[2], Bd[2], Bt[2], nAd[2], nAt[2], nBd[2], nBt[2];
  auto load = [&](int k, bf16x8(&ad)[2], bf16x8(&at)[2], bf16x8(&bd)[2], bf16x8(&bt)[2]) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      ad[x] = *reinterpret_cast<const bf16x8*>(pwd[x] + k);
      at[x] = *reinterpret_cast<const bf16x8*>(pwt[x] + k);
      bd[x] = *reinterpret_cast<const bf16x8*>(phd[x] + k);
      bt[x] = *reinterpret_cast<const bf16x8*>(pht[x] + k);
    }
  };
  load(0, Ad, At, Bd, Bt);
  for (int k = 0; k < H; k += 16) {
    if (k + 16 < H) load(k + 16, nAd, nAt, nBd, nBt);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        zacc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ad[x], Bd[y], zacc[x][y], 0, 0, 0);
        tacc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(At[x], Bt[y], tacc[x][y], 0, 0, 0);
      }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      Ad[x] = nAd[x];
      At[x] = nAt[x];
      Bd[x] = nBd[x];
      Bt[x] = nBt[x];
    }
  }

  const int chunk = v0 / kChunk;
  // vocabulary entry of accumulator element i of block x
  auto vocab = [&](int x, int i) { return v0 + 32 * x + 8 * (i >> 2) + 4 * h + (i & 3); };
#pragma unroll
  for (int y = 0; y < 2; ++y) {
    const int row = row0 + 32 * y + r32;
    const bool rok = row < a.N && v0 < a.V;  // a wave past the vocabulary writes nothing
    if constexpr (PASS == 0) {
      float mz = kNegInf, mt = kNegInf;
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (vocab(x, i) < a.V) {
            mz = fmaxf(mz, zacc[x][y][i] * kLog2e);
            mt = fmaxf(mt, tacc[x][y][i] * kLog2e);
          }
      float sz = 0.f, st = 0.f;
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (vocab(x, i) < a.V) {
            sz += fast_exp2(__builtin_fmaf(zacc[x][y][i], kLog2e, -mz));
            st += fast_exp2(__builtin_fmaf(tacc[x][y][i], kLog2e, -mt));
          }
      if (mz == kNegInf) sz = 0.f;
      if (mt == kNegInf) st = 0.f;
      lse2_merge(mz, sz, __shfl_xor(mz, 32, 64), __shfl_xor(sz, 32, 64));
      lse2_merge(mt, st, __shfl_xor(mt, 32, 64), __shfl_xor(st, 32, 64));
      if (rok && h == 0) a.partA[size_t(row) * a.nch + chunk] = f32x4{mz, sz, mt, st};
    } else {
      const f32x2 l = a.nl[rowv[y]];
      const float nlz = -l[0], nlt = -l[1];
      if constexpr (PASS == 1) {
        float al = 0.f, g = 0.f;
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (vocab(x, i) < a.V) {
              const float lq = __builtin_fmaf(zacc[x][y][i], kLog2e, nlz);
              const float lp = __builtin_fmaf(tacc[x][y][i], kLog2e, nlt);
              const float e = fast_exp2(fminf(lq, lp));
              al += e;
              g += lq < lp ? e : 0.f;
            }
        al += __shfl_xor(al, 32, 64);
        g += __shfl_xor(g, 32, 64);
        if (rok && h == 0) a.partB[size_t(row) * a.nch + chunk] = f32x2{al, g};
      } else {
        const f32x2 c = a.coef[rowv[y]];
        float* grow = a.grad + size_t(rowv[y]) * a.V;
        const bool vec = (a.V & 3) == 0;
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            float gv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float lq = __builtin_fmaf(zacc[x][y][4 * q4 + e], kLog2e, nlz);
              const float lp = __builtin_fmaf(tacc[x][y][4 * q4 + e], kLog2e, nlt);
              gv[e] = fast_exp2(lq) * (lq < lp ? c[0] : c[1]);
            }
            const int vb = vocab(x, 4 * q4);
            if (!rok) continue;
            if (vec && vb + 3 < a.V) {
              *reinterpret_cast<f32x4*>(grow + vb) = f32x4{gv[0], gv[1], gv[2], gv[3]};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (vb + e < a.V) grow[vb + e] = gv[e];
            }
          }
      }
    }
  }
}

// Per row: the chunk partials merged in chunk order (lanes take strided
// chunks, then a fixed butterfly), log2-domain log-sum-exps; a row whose
// target row is out of range gets NaN and is counted.
__global__ __launch_bounds__(256) void lmh_lse_kernel(const LmhArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= a.N) return;
  float mz = kNegInf, sz = 0.f, mt = kNegInf, st = 0.f;
  for (int c = lane; c < a.nch; c += 64) {
    const f32x4 p = a.partA[size_t(row) * a.nch + c];
    lse2_merge(mz, sz, p[0], p[1]);
    lse2_merge(mt, st, p[2], p[3]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lse2_merge(mz, sz, __shfl_xor(mz, o, 64), __shfl_xor(sz, o, 64));
    lse2_merge(mt, st, __shfl_xor(mt, o, 64), __shfl_xor(st, o, 64));
  }
  if (lane == 0) {
    const int tr = a.trow[row];
    f32x2 l = {mz + log2f(sz), mt + log2f(st)};
    if (!(tr >= 0 && tr < a.M)) {
      l = f32x2{__builtin_nanf(""), __builtin_nanf("")};
      atomicAdd(a.bad, 1);
    }
    a.nl[row] = l;
  }
}

// Per branch: alpha and G of every node (chunk partials summed in fp64 in
// chunk order), the parent map checked, prefix products, suffix sums
// S_j = 1 + sum over children of alpha_c S_c, coefficients
// c_j = -grad_scale P_parent(j) S_j / count stored as (c (1 - G), -c G).
__global__ __launch_bounds__(64) void lmh_scan_kernel(const LmhArgs a) {
  __shared__ double s_al[64], s_g[64], s_P[64], s_S[64];
  __shared__ int s_par[64];
  const int r = blockIdx.x, lane = threadIdx.x, Wn = a.Wn;
  const size_t n0 = size_t(r) * Wn;
  if (lane < Wn) s_par[lane] = a.parent[n0 + lane];
  for (int j = 0; j < Wn; ++j) {
    double al = 0.0, g = 0.0;
    for (int c = lane; c < a.nch; c += 64) {
      const f32x2 p = a.partB[(n0 + j) * a.nch + c];
      al += p[0];
      g += p[1];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      al += __shfl_xor(al, o, 64);
      g += __shfl_xor(g, o, 64);
    }
    if (lane == 0) {
      s_al[j] = al;
      s_g[j] = g;
    }
  }
  __syncthreads();
  if (lane != 0) return;
  bool ok = true;
  for (int j = 0; j < Wn; ++j)
    if (!(s_par[j] >= -1 && s_par[j] < j)) ok = false;
  const double nan = __builtin_nan("");
  double numer = 0.0;
  for (int j = 0; j < Wn; ++j) {
    const double pp = (!ok || s_par[j] < 0) ? 1.0 : s_P[s_par[j]];
    s_P[j] = ok ? s_al[j] * pp : nan;
    s_S[j] = 1.0;
    numer += s_P[j];
  }
  for (int j = Wn - 1; j >= 0; --j)
    if (ok && s_par[j] >= 0) s_S[s_par[j]] += s_al[j] * s_S[j];
  for (int j = 0; j < Wn; ++j) {
    const double pp = !ok ? nan : (s_par[j] < 0 ? 1.0 : s_P[s_par[j]]);
    const double c = -double(a.grad_scale) * pp * s_S[j] / a.count;
    a.coef[n0 + j] = f32x2{float(c * (1.0 - s_g[j])), float(-c * s_g[j])};
    if (a.alpha_out) a.alpha_out[n0 + j] = ok ? float(s_al[j]) : __builtin_nanf("");
    if (a.prefix_out) a.prefix_out[n0 + j] = float(s_P[j]);
  }
  a.numer[r] = ok ? numer : nan;
  if (!ok) atomicAdd(a.bad, 1);
}

__global__ void lmh_final_kernel(const LmhArgs a) {
  double numer = 0.0;
  for (int r = 0; r < a.R; ++r) numer += a.numer[r];
  a.loss_out[0] = 1.0 - numer / a.count;
  a.loss_out[1] = numer;
  a.loss_out[2] = a.count;
}

__global__ void lmh_zero_kernel(int32_t* bad) { *bad = 0; }

}  // namespace

LmhWs lmhead_ws_layout(const specopd_lmhead_e2etv_desc& d) {
  LmhWs w{};
  const size_t N = size_t(d.R) * d.Wn;
  w.nch = (d.V + kChunk - 1) / kChunk;
  w.bad = 0;
  w.partA = 256;
  w.nl = align_up(w.partA + N * w.nch * 16, 256);
  w.partB = align_up(w.nl + N * 8, 256);
  w.coef = align_up(w.partB + N * w.nch * 8, 256);
  w.numer = align_up(w.coef + N * 8, 256);
  w.total = align_up(w.numer + size_t(d.R) * 8, 256);
  return w;
}

hipError_t launch_lmhead_e2etv(const specopd_lmhead_e2etv_desc& d, const LmhCallArgs& c, hipStream_t s) {
  const LmhWs w = lmhead_ws_layout(d);
  LmhArgs a{};
  a.hd = static_cast<const uint16_t*>(c.h_draft);
  a.wd = static_cast<const uint16_t*>(c.w_draft);
  a.ht = static_cast<const uint16_t*>(c.h_target);
  a.wt = static_cast<const uint16_t*>(c.w_target);
  a.trow = c.target_row;
  a.parent = c.parent;
  a.alpha_out = c.alpha_out;
  a.prefix_out = c.prefix_out;
  a.loss_out = c.loss_out;
  a.grad = c.grad;
  a.bad = reinterpret_cast<int32_t*>(c.ws + w.bad);
  a.partA = reinterpret_cast<f32x4*>(c.ws + w.partA);
  a.nl = reinterpret_cast<f32x2*>(c.ws + w.nl);
  a.partB = reinterpret_cast<f32x2*>(c.ws + w.partB);
  a.coef = reinterpret_cast<f32x2*>(c.ws + w.coef);
  a.numer = reinterpret_cast<double*>(c.ws + w.numer);
  a.R = d.R;
  a.Wn = d.Wn;
  a.V = d.V;
  a.H = d.H;
  a.M = d.M;
  a.N = d.R * d.Wn;
  a.nch = w.nch;
  a.nrt = (a.N + kTileR - 1) / kTileR;
  a.count = d.norm_count > 0.0 ? d.norm_count : double(a.N);
  a.grad_scale = d.grad_scale;
  const int nvt = (d.V + kTileV - 1) / kTileV;
  const dim3 grid(unsigned(size_t(nvt) * a.nrt));
  lmh_zero_kernel<<<1, 1, 0, s>>>(a.bad);
  timing_mark(7, 0, s);
  lmh_pass_kernel<0><<<grid, 256, 0, s>>>(a);
  lmh_lse_kernel<<<dim3(unsigned((a.N + 3) / 4)), 256, 0, s>>>(a);
  lmh_pass_kernel<1><<<grid, 256, 0, s>>>(a);
  lmh_scan_kernel<<<dim3(unsigned(d.R)), 64, 0, s>>>(a);
  if (a.grad) lmh_pass_kernel<2><<<grid, 256, 0, s>>>(a);
  timing_mark(7, 1, s);
  lmh_final_kernel<<<1, 1, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace specopd
