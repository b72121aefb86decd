// Linear-attention (GDN) branch scoring by indexed state replay (gfx950).
//
// What is computed (jaehun.me review of SpecOPD, §3.2(c) and Fig. 5): a
// linear-attention target keeps one recurrent state per head, which a mask
// cannot rewind to an anchor.  The trunk pass stores the state as immutable
// fp32 checkpoints every C trunk tokens; a branch restores its anchor's state
// by copying the nearest checkpoint at or before the anchor into private
// registers and replaying only the trunk tokens after it, then updates and
// reads that copy with its own tokens.  The recurrence is the gated delta
// rule as published for Gated DeltaNet (the pages name GDN without stating
// it): per head, with a state S of [Dv][Dk] and unit keys,
//     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
//         = alpha_t S_{t-1} + u_t k_t^T,  u_t = beta_t (v_t - alpha_t S_{t-1} k_t),
//     o_t = S_t q_t.
// A branch node's state is its parent's state (the anchor's for a root)
// updated with the node's own token.
//
// One workgroup per (trunk, branch, head), D/32 waves.  The D x D state
// lives in registers: lanes l and l + 32 of wave w hold row 32 w + (l mod 32),
// the first and the second half of its columns, as S / g with one running
// scale g for the whole state, so a token's decay costs one scalar multiply
// and its update one fused multiply-add per element.  Key and query rows are
// read as per-lane slices (four or two consecutive elements per lane, each
// 16-lane row of the wave holding one half of the row) and reach every lane
// through DPP row broadcasts in the FMAs' operands; a token's value is one
// element per row.  Per token each lane updates its columns and, in the same
// pass, forms its part of S k for the next token and of S q for its output;
// the two halves of a row are summed by a lane swap within the wave, so the
// waves of a workgroup never wait for each other after the list is built.
// The next token's rows are loaded while the current one is processed.
//
// The order of work is a list built by one thread from the parent map:
// replay the trunk suffix, then the nodes in index order; a node whose
// parent is not the node just processed starts again from the checkpoint
// and replays the trunk suffix and the path down to its parent (no
// outputs), so no state copy is ever stored.  Malformed branches (anchor
// outside the trunk, a parent that does not precede its node) get NaN
// outputs and are counted in the workspace.
#include "device_common.h"
#include "internal.h"

namespace specopd {

namespace {

// Work-list entries (16 bits): the offset of a trunk token from the first
// token after the checkpoint, or kNode | j for branch node j; kRestore on the
// first token after which the state restarts from the checkpoint.
constexpr int kNode = 1 << 8;
constexpr int kRestore = 1 << 9;

// Uniform loads through the constant address space become scalar loads (a
// plain global pointer would be read by vector loads, since the kernel also
// stores to global memory); the inputs are never written while it runs.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* cptr(const void* p) {
  return (const __attribute__((address_space(4))) T*)(p);
}

// A lane's slice of a key or query row: V consecutive elements of its half,
// starting at column V * (lane mod 16), raw as loaded and as fp32.
template <typename IN, int V>
struct Slice;
template <>
struct Slice<uint16_t, 4> {
  using raw = u32x2;
  static __device__ __forceinline__ raw load(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }
  static __device__ __forceinline__ void cvt(raw w, float (&x)[4]) {
    x[0] = bf16_lo(w[0]);
    x[1] = bf16_hi(w[0]);
    x[2] = bf16_lo(w[1]);
    x[3] = bf16_hi(w[1]);
  }
};
template <>
struct Slice<uint16_t, 2> {
  using raw = uint32_t;
  static __device__ __forceinline__ raw load(const uint16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
  static __device__ __forceinline__ void cvt(raw w, float (&x)[2]) {
    x[0] = bf16_lo(w);
    x[1] = bf16_hi(w);
  }
};
template <>
struct Slice<float, 4> {
  using raw = f32x4;
  static __device__ __forceinline__ raw load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  static __device__ __forceinline__ void cvt(raw w, float (&x)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = w[i];
  }
};
template <>
struct Slice<float, 2> {
  using raw = f32x2;
  static __device__ __forceinline__ raw load(const float* p) { return *reinterpret_cast<const f32x2*>(p); }
  static __device__ __forceinline__ void cvt(raw w, float (&x)[2]) {
    x[0] = w[0];
    x[1] = w[1];
  }
};

// One token's pass over a lane's NCOL columns as a single block of
// v_fmac_f32_dpp: the DPP row broadcast (row_newbcast:X) hands every lane
// the slice element of lane X of its 16-lane row, i.e. the row element of
// column V * X + j, in the FMA's own operand fetch.  Per column c:
//   St[c] += k[c] w;   y += k'[c] St[c];   o += q[c] St[c]
// (k the token's key, k' the next token's, q its query), two columns at a
// time with two accumulators each.  A DPP source must not be written by a
// VALU instruction in the two wait states before, nor EXEC by a SALU one in
// the five before: each block starts with five.  (The compiler neither folds
// a broadcast move into v_fmac_f32 nor knows the hazards inside an asm
// block, hence one block per pass.)
#define GDN_BC(X) " row_newbcast:" #X " row_mask:0xf bank_mask:0xf\n\t"
#define GDN_FULL(A, B, JA, JB, X)                     \
  "v_fmac_f32_dpp %" #A ", %[k" #JA "], %[w]" GDN_BC(X) \
  "v_fmac_f32_dpp %" #B ", %[k" #JB "], %[w]" GDN_BC(X) \
  "v_fmac_f32_dpp %[y0], %[n" #JA "], %" #A GDN_BC(X)   \
  "v_fmac_f32_dpp %[y1], %[n" #JB "], %" #B GDN_BC(X)   \
  "v_fmac_f32_dpp %[o0], %[q" #JA "], %" #A GDN_BC(X)   \
  "v_fmac_f32_dpp %[o1], %[q" #JB "], %" #B GDN_BC(X)
// a trunk token has no output: the update and S k'
#define GDN_NOQ(A, B, JA, JB, X)                      \
  "v_fmac_f32_dpp %" #A ", %[k" #JA "], %[w]" GDN_BC(X) \
  "v_fmac_f32_dpp %" #B ", %[k" #JB "], %[w]" GDN_BC(X) \
  "v_fmac_f32_dpp %[y0], %[n" #JA "], %" #A GDN_BC(X)   \
  "v_fmac_f32_dpp %[y1], %[n" #JB "], %" #B GDN_BC(X)
// S k alone (after a restore)
#define GDN_DOT(A, B, JA, JB, X)                    \
  "v_fmac_f32_dpp %[y0], %[k" #JA "], %" #A GDN_BC(X) \
  "v_fmac_f32_dpp %[y1], %[k" #JB "], %" #B GDN_BC(X)
// column pairs: 64 columns, 4 slice elements per lane (D = 128)
#define GDN_COLS64(M)                                                                              \
  M(0, 1, 0, 1, 0) M(2, 3, 2, 3, 0) M(4, 5, 0, 1, 1) M(6, 7, 2, 3, 1) M(8, 9, 0, 1, 2)             \
  M(10, 11, 2, 3, 2) M(12, 13, 0, 1, 3) M(14, 15, 2, 3, 3) M(16, 17, 0, 1, 4) M(18, 19, 2, 3, 4)   \
  M(20, 21, 0, 1, 5) M(22, 23, 2, 3, 5) M(24, 25, 0, 1, 6) M(26, 27, 2, 3, 6) M(28, 29, 0, 1, 7)   \
  M(30, 31, 2, 3, 7) M(32, 33, 0, 1, 8) M(34, 35, 2, 3, 8) M(36, 37, 0, 1, 9) M(38, 39, 2, 3, 9)   \
  M(40, 41, 0, 1, 10) M(42, 43, 2, 3, 10) M(44, 45, 0, 1, 11) M(46, 47, 2, 3, 11)                   \
  M(48, 49, 0, 1, 12) M(50, 51, 2, 3, 12) M(52, 53, 0, 1, 13) M(54, 55, 2, 3, 13)                   \
  M(56, 57, 0, 1, 14) M(58, 59, 2, 3, 14) M(60, 61, 0, 1, 15) M(62, 63, 2, 3, 15)
// column pairs: 32 columns, 2 slice elements per lane (D = 64)
#define GDN_COLS32(M)                                                                              \
  M(0, 1, 0, 1, 0) M(2, 3, 0, 1, 1) M(4, 5, 0, 1, 2) M(6, 7, 0, 1, 3) M(8, 9, 0, 1, 4)             \
  M(10, 11, 0, 1, 5) M(12, 13, 0, 1, 6) M(14, 15, 0, 1, 7) M(16, 17, 0, 1, 8) M(18, 19, 0, 1, 9)   \
  M(20, 21, 0, 1, 10) M(22, 23, 0, 1, 11) M(24, 25, 0, 1, 12) M(26, 27, 0, 1, 13)                   \
  M(28, 29, 0, 1, 14) M(30, 31, 0, 1, 15)
#define GDN_ST16(S, o)                                                                              \
  "+v"(S[o]), "+v"(S[o + 1]), "+v"(S[o + 2]), "+v"(S[o + 3]), "+v"(S[o + 4]), "+v"(S[o + 5]),        \
      "+v"(S[o + 6]), "+v"(S[o + 7]), "+v"(S[o + 8]), "+v"(S[o + 9]), "+v"(S[o + 10]), "+v"(S[o + 11]), \
      "+v"(S[o + 12]), "+v"(S[o + 13]), "+v"(S[o + 14]), "+v"(S[o + 15])
#define GDN_IN4(N, x) [N##0] "v"(x[0]), [N##1] "v"(x[1]), [N##2] "v"(x[2]), [N##3] "v"(x[3])
#define GDN_IN2(N, x) [N##0] "v"(x[0]), [N##1] "v"(x[1])

// St += w k^T with the partial sums of S k' and, when out is nonzero (a
// branch node), of S q; the choice is a branch inside the block, so both
// paths keep the state in the same registers
__device__ __forceinline__ void token_pass(float (&St)[64], const float (&kr)[4], const float (&kn)[4],
                                           const float (&q)[4], float w, float (&y)[2], float (&o)[2], int out) {
  asm("s_nop 4\n\t"
      "s_cmp_eq_u32 %[out], 0\n\t"
      "s_cbranch_scc1 1f\n\t" GDN_COLS64(GDN_FULL) "s_branch 2f\n"
      "1:\n\t" GDN_COLS64(GDN_NOQ) "2:"
      : GDN_ST16(St, 0), GDN_ST16(St, 16), GDN_ST16(St, 32), GDN_ST16(St, 48), [y0] "+v"(y[0]), [y1] "+v"(y[1]),
        [o0] "+v"(o[0]), [o1] "+v"(o[1])
      : GDN_IN4(k, kr), GDN_IN4(n, kn), GDN_IN4(q, q), [w] "v"(w), [out] "s"(out)
      : "scc");
}
__device__ __forceinline__ void token_pass(float (&St)[32], const float (&kr)[2], const float (&kn)[2],
                                           const float (&q)[2], float w, float (&y)[2], float (&o)[2], int out) {
  asm("s_nop 4\n\t"
      "s_cmp_eq_u32 %[out], 0\n\t"
      "s_cbranch_scc1 1f\n\t" GDN_COLS32(GDN_FULL) "s_branch 2f\n"
      "1:\n\t" GDN_COLS32(GDN_NOQ) "2:"
      : GDN_ST16(St, 0), GDN_ST16(St, 16), [y0] "+v"(y[0]), [y1] "+v"(y[1]), [o0] "+v"(o[0]), [o1] "+v"(o[1])
      : GDN_IN2(k, kr), GDN_IN2(n, kn), GDN_IN2(q, q), [w] "v"(w), [out] "s"(out)
      : "scc");
}
// the partial sums of S k
__device__ __forceinline__ void dot_pass(float (&St)[64], const float (&kr)[4], float (&y)[2]) {
  asm("s_nop 4\n\t" GDN_COLS64(GDN_DOT)
      : GDN_ST16(St, 0), GDN_ST16(St, 16), GDN_ST16(St, 32), GDN_ST16(St, 48), [y0] "+v"(y[0]), [y1] "+v"(y[1])
      : GDN_IN4(k, kr));
}
__device__ __forceinline__ void dot_pass(float (&St)[32], const float (&kr)[2], float (&y)[2]) {
  asm("s_nop 4\n\t" GDN_COLS32(GDN_DOT)
      : GDN_ST16(St, 0), GDN_ST16(St, 16), [y0] "+v"(y[0]), [y1] "+v"(y[1])
      : GDN_IN2(k, kr));
}

struct GdnArgs {
  const float* __restrict__ ckpt;
  const void *trunk_k, *trunk_v, *q, *k, *v;
  const float *trunk_gate, *trunk_beta, *gate, *beta;
  const int32_t *anchors, *parent;
  float* out;
  int32_t* bad;
  int T, L, B, Wn, H, C, NC;
};

// The longest work list: with C <= 64 (host check), at most Wn restarts, each
// replaying at most C - 1 trunk tokens and a path of at most Wn - 1 nodes,
// plus the Wn nodes themselves.
constexpr int kMaxList = 64 * (63 + 63) + 64;

template <int D, typename IN>
__device__ __forceinline__ void gdn_replay(const GdnArgs& a) {
  constexpr int NCOL = D / 2;   // columns per lane
  constexpr int V = NCOL / 16;  // slice elements per lane
  using SL = Slice<IN, V>;
  __shared__ uint16_t s_list[kMaxList];
  __shared__ int s_par[64];
  __shared__ int s_n;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, r = wave * 32 + (lane & 31);
  const int c0 = half * NCOL + V * (lane & 15);  // this lane's slice of a row
  const int h = blockIdx.x % a.H;
  const int tb = blockIdx.x / a.H;  // trunk * B + branch
  const int t = tb / a.B;
  const int Wn = a.Wn;
  const int anc = a.anchors[tb];
  const IN* const tk = static_cast<const IN*>(a.trunk_k);
  const IN* const tv = static_cast<const IN*>(a.trunk_v);
  const IN* const bq = static_cast<const IN*>(a.q);
  const IN* const bk = static_cast<const IN*>(a.k);
  const IN* const bv = static_cast<const IN*>(a.v);

  // ---- the work list (one thread, from the parent map staged in LDS)
  if (tid < Wn) s_par[tid] = a.parent[size_t(tb) * Wn + tid];
  __syncthreads();
  if (tid == 0) {
    bool ok = anc >= 0 && anc < a.L;
    for (int j = 0; j < Wn && ok; ++j) ok = s_par[j] >= -1 && s_par[j] < j;
    int n = -1;
    if (ok) {
      const int t0 = (anc + 1) / a.C * a.C;  // first trunk token after the checkpoint
      n = 0;
      int cur = -2;                          // state held: -1 the anchor's, j node j's
      for (int j = 0; j < Wn; ++j) {
        const int p = s_par[j];
        const int first = n;
        if (p != cur) {
          // checkpoint, trunk suffix, then the path from the root down to p
          for (int x = 0; t0 + x <= anc; ++x) s_list[n++] = uint16_t(x);
          int depth = 0;
          for (int x = p; x >= 0; x = s_par[x]) ++depth;
          for (int d = depth - 1; d >= 0; --d) {
            int x = p;
            for (int k = 0; k < d; ++k) x = s_par[x];
            s_list[n++] = uint16_t(kNode | x);
          }
        }
        s_list[n++] = uint16_t(kNode | j);
        if (p != cur) s_list[first] |= uint16_t(kRestore);
        cur = j;
      }
    }
    s_n = n;
    if (!ok && h == 0) atomicAdd(a.bad, 1);
  }
  __syncthreads();
  const int n = s_n;
  float* const orow0 = a.out + size_t(tb) * Wn * a.H * D;
  if (n < 0) {
    if (half == 0)
      for (int j = 0; j < Wn; ++j) orow0[(size_t(j) * a.H + h) * D + r] = __builtin_nanf("");
    return;
  }

  // token e: e >= 0 trunk token e, e < 0 branch node -1-e
  const int t0 = (anc + 1) / a.C * a.C;
  auto token = [&](int i) -> int {
    const int x = __builtin_amdgcn_readfirstlane(int(s_list[i < n ? i : n - 1])) & ~kRestore;
    return (x & kNode) ? -1 - (x & (kNode - 1)) : t0 + x;
  };
  auto krow = [&](int e) -> const IN* {
    return e >= 0 ? tk + ((size_t(t) * a.L + e) * a.H + h) * D
                  : bk + ((size_t(tb) * Wn + (-1 - e)) * a.H + h) * D;
  };
  // a node's query row; a trunk token has none, so any valid row
  auto qrow = [&](int e) -> const IN* {
    return e < 0 ? bq + ((size_t(tb) * Wn + (-1 - e)) * a.H + h) * D : krow(e);
  };
  auto vval = [&](int e) -> float {
    return load_f32((e >= 0 ? tv + ((size_t(t) * a.L + e) * a.H + h) * D
                            : bv + ((size_t(tb) * Wn + (-1 - e)) * a.H + h) * D) + r);
  };
  auto gate = [&](int e) -> float {
    return e >= 0 ? cptr<float>(a.trunk_gate)[(size_t(t) * a.L + e) * a.H + h]
                  : cptr<float>(a.gate)[(size_t(tb) * Wn + (-1 - e)) * a.H + h];
  };
  auto strength = [&](int e) -> float {
    return e >= 0 ? cptr<float>(a.trunk_beta)[(size_t(t) * a.L + e) * a.H + h]
                  : cptr<float>(a.beta)[(size_t(tb) * Wn + (-1 - e)) * a.H + h];
  };

  float St[NCOL];
  float g = 1.f;  // the state is g * St
  // the sum of the two column halves' partials of this lane's row (lanes l
  // and l + 32): v_permlane32_swap trades the upper half of one register
  // with the lower half of the other, so with both holding x each ends with
  // x[l mod 32] in one and x[l mod 32 + 32] in the other
  auto halves = [&](float x) -> float {
    float p = x, q = x;
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(p), "+v"(q));
    return p + q;
  };
  // the checkpoint at or before the anchor (the zero state if none)
  auto restore = [&]() {
    const int c = (anc + 1) / a.C - 1;
    if (c >= 0) {
      const float* src = a.ckpt + ((size_t(t) * a.NC + c) * a.H + h) * size_t(D) * D + size_t(r) * D + half * NCOL;
#pragma unroll
      for (int i = 0; i < NCOL; i += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(src + i);
        St[i] = x[0];
        St[i + 1] = x[1];
        St[i + 2] = x[2];
        St[i + 3] = x[3];
      }
    } else {
#pragma unroll
      for (int i = 0; i < NCOL; ++i) St[i] = 0.f;
    }
    g = 1.f;
  };

  // the token about to be processed: e, its key kr, the next token's key kn,
  // its query q (nodes), gate, strength, value element and y = S_{t-1} k_t
  int e = token(0);
  float kr[V], kn[V], q[V];
  SL::cvt(SL::load(krow(e) + c0), kr);
  SL::cvt(SL::load(krow(token(1)) + c0), kn);
  SL::cvt(SL::load(qrow(e) + c0), q);
  float al = gate(e), be = strength(e), vr = vval(e), y = 0.f;
  for (int i = 0; i < n; ++i) {
    const bool rst = __builtin_amdgcn_readfirstlane(int(s_list[i])) & kRestore;
    // the next iteration's rows and scalars, loaded during this one
    const int e1 = token(i + 1), e2 = token(i + 2);
    const typename SL::raw rk = SL::load(krow(e2) + c0);
    const typename SL::raw rq = SL::load(qrow(e1) + c0);
    const float al1 = gate(e1), be1 = strength(e1), vr1 = vval(e1);
    if (rst) {
      restore();
      float a2[2] = {0.f, 0.f};
      dot_pass(St, kr, a2);
      y = halves(a2[0] + a2[1]);
    }
    // S_t = alpha S_{t-1} + u k^T, u = beta (v - alpha y); as g St with
    // g <- alpha g and St += (u / g) k, the scale folded into St when small
    const float u = be * (vr - al * y);
    float gn = al * g;
    float w;
    if (gn < 0x1p-30f) {
#pragma unroll
      for (int c = 0; c < NCOL; ++c) St[c] *= gn;
      gn = 1.f;
      w = u;
    } else {
      w = u * __builtin_amdgcn_rcpf(gn);
    }
    g = gn;
    float ay[2] = {0.f, 0.f}, ao[2] = {0.f, 0.f};
    token_pass(St, kr, kn, q, w, ay, ao, e < 0);
    y = halves(g * (ay[0] + ay[1]));
    if (e < 0) {
      const float o = halves(g * (ao[0] + ao[1]));
      if (half == 0) orow0[(size_t(-1 - e) * a.H + h) * D + r] = o;
    }
    e = e1;
    al = al1;
    be = be1;
    vr = vr1;
#pragma unroll
    for (int j = 0; j < V; ++j) kr[j] = kn[j];
    SL::cvt(rk, kn);
    SL::cvt(rq, q);
  }
}

template <int D, typename IN>
__global__ __launch_bounds__(D / 32 * 64) void gdn_replay_kernel(const GdnArgs a) {
  gdn_replay<D, IN>(a);
}
// bf16 slices leave the D = 128 kernel at 96 VGPRs: five workgroups per CU
template <>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void gdn_replay_kernel<128, uint16_t>(
    const GdnArgs a) {
  gdn_replay<128, uint16_t>(a);
}

__global__ void gdn_zero_kernel(int32_t* __restrict__ bad) {
  if (threadIdx.x == 0) *bad = 0;
}

}  // namespace

hipError_t launch_gdn_replay(const specopd_gdn_desc& d, const GdnCallArgs& c, hipStream_t s) {
  GdnArgs a{};
  a.ckpt = c.ckpt;
  a.trunk_k = c.trunk_k;
  a.trunk_v = c.trunk_v;
  a.q = c.q;
  a.k = c.k;
  a.v = c.v;
  a.trunk_gate = c.trunk_gate;
  a.trunk_beta = c.trunk_beta;
  a.gate = c.gate;
  a.beta = c.beta;
  a.anchors = c.anchors;
  a.parent = c.parent;
  a.out = c.out;
  a.bad = reinterpret_cast<int32_t*>(c.ws);
  a.T = d.T; a.L = d.L; a.B = d.B; a.Wn = d.Wn; a.H = d.H; a.C = d.C; a.NC = d.L / d.C;
  gdn_zero_kernel<<<1, 64, 0, s>>>(a.bad);
  const dim3 grid(unsigned(size_t(d.T) * d.B * d.H));
  timing_mark(3, 0, s);
  const bool bf = d.dtype == SPECOPD_BF16;
  if (d.D == 128) {
    if (bf) gdn_replay_kernel<128, uint16_t><<<grid, 256, 0, s>>>(a);
    else gdn_replay_kernel<128, float><<<grid, 256, 0, s>>>(a);
  } else {
    if (bf) gdn_replay_kernel<64, uint16_t><<<grid, 128, 0, s>>>(a);
    else gdn_replay_kernel<64, float><<<grid, 128, 0, s>>>(a);
  }
  timing_mark(3, 1, s);
  return hipGetLastError();
}

}  // namespace specopd
