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
//   pass C       the gradient c q_u ([q_u < p_u] - G), written once; it forms
//                only z, reading the indicator from the bits pass B wrote;
//   final        the loss from the branch numerators in branch order.
// Every pass forms the same tiles in the same order, so the three passes see
// bitwise the same logits; the indicator [q < p] is decided once, in pass B.
//
// Matrix-core tiles (v_mfma_f32_32x32x16_bf16, lane l = r + 32h): a
// workgroup of four waves covers 128 rows x 128 vocabulary entries, a wave
// 64 rows x 64 entries of both z and t (eight 32 x 32 accumulators).  A = 32
// head rows (vocabulary entries) x 16 hidden values, B = 16 hidden values x
// 32 hidden-state rows, read from LDS in operand layout (16 contiguous
// bytes per lane: hidden states and heads are both
// hidden-contiguous, staged through LDS 32 hidden values at a time, the
// next stage loading while the current one's products run).  Lane (r, h)
// then holds row r's logits for
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
constexpr int kKc = 32;             // hidden values per LDS stage
constexpr int kSrow = kKc + 8;      // LDS row stride (elements): 80 bytes, so the
                                    // 32 rows an operand read touches spread over the banks

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
  uint32_t* bits;  // [N][nch][2] the indicator [q<p] of every element, from pass B
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

// Two workgroups per CU (2 x 80 KiB of LDS, at most 256 registers a wave),
// so one workgroup's loads and barriers overlap the other's products.
template <int PASS>
__global__ __launch_bounds__(256, PASS == 2 ? 3 : 2) void lmh_pass_kernel(const LmhArgs a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 5, r32 = lane & 31;
  // Workgroup b runs on XCD b mod 8.  The row tiles of one vocabulary tile
  // get consecutive slots of one XCD, so they run side by side and share the
  // head tile through that XCD's L2 instead of each fetching it.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int rt = slot % a.nrt, vt = 8 * (slot / a.nrt) + xcd;
  if (vt * kTileV >= a.V) return;  // padding of the vocabulary tiles to a multiple of 8
  const int row0 = rt * kTileR + 64 * (wave & 1);
  const int v0 = vt * kTileV + 64 * (wave >> 1);
  const int H = a.H;

  // Tiles of 128 rows x kKc hidden values of the four operands (draft and
  // target head rows, draft and gathered target hidden-state rows) are
  // staged in LDS, two stages deep: each thread loads 16 contiguous bytes of
  // 8 tile rows per stage (4 lanes per 64-byte row segment), so a wave's
  // load covers whole segments of 16 rows.  Out-of-range rows are clamped
  // into range (their results are never used); hidden values past H load
  // zeros.
  // pass C forms only z: the indicator [q < p] comes from pass B's bits, so
  // it stages two operands (half the LDS: three workgroups per CU)
  constexpr bool kT = PASS != 2;
  constexpr int NT = kT ? 4 : 2;
  __shared__ __attribute__((aligned(16))) uint16_t s_t[2][NT][kTileR * kSrow];
  // LDS slot of operand tile 0..3 (draft head, target head, draft hidden,
  // target hidden)
  auto lslot = [](int tile) { return kT ? tile : (tile == 0 ? 0 : 1); };
  // element offsets of this thread's 8 tile rows (32-bit: the host limits
  // every operand to 2^31 elements), from the four operands' bases
  const uint16_t* const bases[4] = {a.wd, a.wt, a.hd, a.ht};
  uint32_t off[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int tile = q >> 1, r = (q & 1) * 64 + (tid >> 2);
    int row;
    if (tile < 2) {
      row = min(vt * kTileV + r, a.V - 1);
    } else {
      row = min(rt * kTileR + r, a.N - 1);
      if (tile == 3) {
        const int tr = a.trow[row];
        row = (tr >= 0 && tr < a.M) ? tr : 0;  // an invalid row is reported by the lse kernel
      }
    }
    off[q] = uint32_t(row) * uint32_t(H) + uint32_t((tid & 3) * 8);
  }
  int rowv[2];
#pragma unroll
  for (int y = 0; y < 2; ++y) rowv[y] = min(row0 + 32 * y + r32, a.N - 1);

  f32x16 zacc[2][2], tacc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      zacc[x][y] = f32x16{};
      tacc[x][y] = f32x16{};
    }
  auto used = [&](int q) { return kT || (q >> 1) == 0 || (q >> 1) == 2; };
  u32x4 st[8];
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (used(q))
        st[q] = k0 + (tid & 3) * 8 < H ? *reinterpret_cast<const u32x4*>(bases[q >> 1] + off[q] + k0)
                                       : u32x4{0u, 0u, 0u, 0u};
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (!used(q)) continue;
      const int tile = q >> 1, r = (q & 1) * 64 + (tid >> 2);
      *reinterpret_cast<u32x4*>(&s_t[buf][lslot(tile)][r * kSrow + (tid & 3) * 8]) = st[q];
    }
  };
  const int ra = 64 * (wave >> 1) + r32;  // this lane's head row in the tile (+ 32 x)
  const int rb = 64 * (wave & 1) + r32;   // this lane's hidden-state row (+ 32 y)
  gload(0);
  lstore(0);
  __syncthreads();
  const int nst = (H + kKc - 1) / kKc;
  for (int sidx = 0; sidx < nst; ++sidx) {
    const int buf = sidx & 1;
    if (sidx + 1 < nst) gload((sidx + 1) * kKc);
#pragma unroll
    for (int ks = 0; ks < kKc / 16; ++ks) {
      bf16x8 Ad[2], At[2], Bd[2], Bt[2];
      const int ko = 16 * ks + 8 * h;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        Ad[x] = *reinterpret_cast<const bf16x8*>(&s_t[buf][0][(ra + 32 * x) * kSrow + ko]);
        Bd[x] = *reinterpret_cast<const bf16x8*>(&s_t[buf][lslot(2)][(rb + 32 * x) * kSrow + ko]);
        if constexpr (kT) {
          At[x] = *reinterpret_cast<const bf16x8*>(&s_t[buf][1][(ra + 32 * x) * kSrow + ko]);
          Bt[x] = *reinterpret_cast<const bf16x8*>(&s_t[buf][3][(rb + 32 * x) * kSrow + ko]);
        }
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          zacc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ad[x], Bd[y], zacc[x][y], 0, 0, 0);
          if constexpr (kT)
            tacc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(At[x], Bt[y], tacc[x][y], 0, 0, 0);
        }
    }
    if (sidx + 1 < nst) lstore(buf ^ 1);
    __syncthreads();
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
        uint32_t ind = 0u;  // bit 16 x + i: [q < p] of accumulator element (x, i)
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
              ind |= uint32_t(lq < lp) << (16 * x + i);
            }
        al += __shfl_xor(al, 32, 64);
        g += __shfl_xor(g, 32, 64);
        if (rok) a.bits[(size_t(row) * a.nch + chunk) * 2 + h] = ind;
        if (rok && h == 0) a.partB[size_t(row) * a.nch + chunk] = f32x2{al, g};
      } else {
        const f32x2 c = a.coef[rowv[y]];
        float* grow = a.grad + size_t(rowv[y]) * a.V;
        const bool vec = (a.V & 3) == 0;
        const uint32_t ind = rok ? a.bits[(size_t(row) * a.nch + chunk) * 2 + h] : 0u;
        (void)nlt;
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            float gv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float lq = __builtin_fmaf(zacc[x][y][4 * q4 + e], kLog2e, nlz);
              gv[e] = fast_exp2(lq) * (((ind >> (16 * x + 4 * q4 + e)) & 1u) ? c[0] : c[1]);
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
  w.bits = align_up(w.numer + size_t(d.R) * 8, 256);
  w.total = align_up(w.bits + N * w.nch * 8, 256);
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
  a.bits = reinterpret_cast<uint32_t*>(c.ws + w.bits);
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
  const dim3 grid(unsigned(size_t((nvt + 7) / 8 * 8) * a.nrt));
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
