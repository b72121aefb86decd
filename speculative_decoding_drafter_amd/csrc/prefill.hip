// Trunk prefill on gfx950: causal GQA attention of a trunk over itself that
// leaves the rotated KV cache the branch calls read.
//
// What is computed (jaehun.me review of SpecOPD, §3.1 step 1 and §3.2(a);
// rustineverything.app summary §2.2): the reference trajectory is run through
// the target once; its keys (rotated at trunk positions 0..L-1) and values
// are cached; token s attends to tokens 0..s.
//
// Formulation.  Row s >= 1 is exactly a one-node branch anchored at s-1: it
// sees trunk keys 0..s-1 and its own key, rotated at position s.  So the
// matrix-core tree kernel does the work, with branch b = token b+1, one node
// per branch, anchors b, and branch keys read straight from the cache it has
// just written (cache row s is token s's rotated key).  The plan the tree
// kernel needs is known in closed form here (branches sorted by anchor are
// simply the tokens in reverse order), so no sort runs.  Row 0 sees only
// itself: its output is its value.
//
// fp32 inputs take the exact fp32 tree path per trunk instead.
#include <algorithm>
#include <cmath>

#include "device_common.h"
#include "internal.h"

namespace specopd {

namespace {

struct PrefillRopeParams {
  const void *q, *k, *v;
  void *cache_k, *cache_v, *out;
  uint16_t* qr;  // bf16 path: rotated queries of tokens 1..L-1, times qmul
  int T, L, Hq, Hkv, D;
  double log2_base;
  float qmul;
};

constexpr int kPfTokens = 4;  // tokens per pass of a rotary workgroup

// Eight consecutive elements as fp32, from and to bf16 (uint16_t) or fp32.
struct F8 {
  float x[8];
};
__device__ __forceinline__ F8 ld8(const uint16_t* p) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
  F8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r.x[2 * e] = bf16_lo(w[e]);
    r.x[2 * e + 1] = bf16_hi(w[e]);
  }
  return r;
}
__device__ __forceinline__ F8 ld8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
  return F8{{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}};
}
__device__ __forceinline__ void st8(uint16_t* p, const F8& v) {
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(v.x[2 * e], v.x[2 * e + 1]);
  *reinterpret_cast<u32x4*>(p) = w;
}
__device__ __forceinline__ void st8(float* p, const F8& v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v.x[0], v.x[1], v.x[2], v.x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v.x[4], v.x[5], v.x[6], v.x[7]};
}
// raw copy of eight elements
template <typename E>
__device__ __forceinline__ void cp8(E* dst, const E* src) {
#pragma unroll
  for (int o = 0; o < int(8 * sizeof(E)); o += 16)
    *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(dst) + o) =
        *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(src) + o);
}

// Rotates pairs (i, i + D/2), i in [i0, i0 + 8), of one head row by the
// angles in cs, times mul.
template <typename E, typename O>
__device__ __forceinline__ void rotate8(const E* src, O* dst, int i0, int half, const float2* cs,
                                       float mul) {
  const F8 a = ld8(src + i0), b = ld8(src + i0 + half);
  F8 ya, yb;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float2 c = cs[i0 + e];
    ya.x[e] = (a.x[e] * c.x - b.x[e] * c.y) * mul;
    yb.x[e] = (b.x[e] * c.x + a.x[e] * c.y) * mul;
  }
  st8(dst + i0, ya);
  st8(dst + i0 + half, yb);
}

// Rotary pre-pass, kPfTokens tokens per workgroup pass.  The angles of a
// pass's tokens are formed once (fp64, reduced modulo 2 pi, sine and cosine
// in fp32 on the reduced argument) and shared by every head; the threads
// then take (token, head, eight pairs) units of the query, key and value
// heads: keys rotated into the cache, values copied into it, queries of
// tokens >= 1 rotated and scaled into qr (matrix-core path), and token 0's
// row, which reads only itself, written as its value.
template <typename E>
__global__ __launch_bounds__(256) void prefill_rope_kernel(const PrefillRopeParams p) {
  __shared__ double s_theta[128];              // D/2 <= 128
  __shared__ float2 s_cs[kPfTokens * 128];     // (cos, sin)
  const int tid = threadIdx.x, half = p.D / 2, octs = p.D / 16;
  const int G = p.Hq / p.Hkv, H = p.Hq + 2 * p.Hkv;  // query, key, value heads
  const size_t ntok = size_t(p.T) * p.L;
  if (tid < half) s_theta[tid] = exp2(-(2.0 * tid / p.D) * p.log2_base);
  for (size_t n0 = size_t(blockIdx.x) * kPfTokens; n0 < ntok; n0 += size_t(gridDim.x) * kPfTokens) {
    const int nn = int(min(size_t(kPfTokens), ntok - n0));
    __syncthreads();  // the table is written / the previous pass's angles are no longer read
    for (int idx = tid; idx < nn * half; idx += 256) {
      const int ln = idx / half, i = idx - ln * half;
      const int s = int((n0 + ln) % size_t(p.L));
      const double ang = double(s) * s_theta[i];
      const double k = rint(ang * 0.15915494309189535);  // 1 / (2 pi)
      float sn, cs;
      sincosf(float(fma(-k, 6.283185307179586, ang)), &sn, &cs);
      s_cs[idx] = make_float2(cs, sn);
    }
    __syncthreads();
    for (int u = tid; u < nn * H * octs; u += 256) {
      const int lnh = u / octs;
      const int i0 = (u - lnh * octs) * 8;
      const int ln = lnh / H, hd = lnh - ln * H;
      const size_t ts = n0 + ln;  // t * L + s
      const int s = int(ts % size_t(p.L));
      const float2* cs = s_cs + ln * half;
      if (hd >= p.Hq + p.Hkv) {
        const size_t row = (ts * p.Hkv + (hd - p.Hq - p.Hkv)) * p.D;
        const E* v = static_cast<const E*>(p.v) + row;
        E* cv = static_cast<E*>(p.cache_v) + row;
        cp8(cv + i0, v + i0);
        cp8(cv + i0 + half, v + i0 + half);
      } else if (hd >= p.Hq) {
        const size_t row = (ts * p.Hkv + (hd - p.Hq)) * p.D;
        rotate8(static_cast<const E*>(p.k) + row, static_cast<E*>(p.cache_k) + row, i0, half, cs, 1.0f);
      } else if (s == 0) {
        const E* v = static_cast<const E*>(p.v) + (ts * p.Hkv + hd / G) * p.D;
        E* o = static_cast<E*>(p.out) + (ts * p.Hq + hd) * p.D;
        cp8(o + i0, v + i0);
        cp8(o + i0 + half, v + i0 + half);
      } else if (p.qr) {
        const size_t t = ts / p.L;
        uint16_t* dst = p.qr + ((t * (p.L - 1) + (s - 1)) * p.Hq + hd) * p.D;
        rotate8(static_cast<const E*>(p.q) + (ts * p.Hq + hd) * p.D, dst, i0, half, cs, p.qmul);
      }
    }
  }
}

struct PrefillPlanParams {
  int32_t *anchors, *parent, *pos, *branch_ok, *order, *pstart, *ustart, *umap, *ctr;
  unsigned long long* qctr;
  uint64_t* anc;
  int T, B, Hkv, bpp, npacks, nsplit;
};

// The plan of B = L-1 one-node branches (branch b = token b+1, anchor b),
// shared by every trunk: validity, masks, order (anchors descending: tokens
// in reverse), the packs' key-tile prefix sums, the units' pack table, and
// every trunk's split counters cleared.  One workgroup.
__global__ __launch_bounds__(256) void prefill_plan_kernel(const PrefillPlanParams p) {
  const int tid = threadIdx.x, B = p.B, np = p.npacks;
  for (int b = tid; b < B; b += 256) {
    p.anchors[b] = b;
    if (p.parent) p.parent[b] = -1;
    if (p.pos) p.pos[b] = b + 1;
    if (p.branch_ok) {
      p.branch_ok[b] = 1;
      p.anc[b] = 1ull;
      p.order[b] = B - 1 - b;
    }
  }
  if (!p.pstart) return;
  // key tiles of pack pk: trunk tiles up to its longest anchor, then one or
  // more tail tiles of its branches' nodes
  auto tiles = [&](int pk) {
    const int b0 = pk * p.bpp, nbr = min(p.bpp, B - b0);
    const int amax = B - 1 - b0;
    return mfma_pack_tiles(amax, nbr, 1, 1);
  };
  __shared__ int run[256];
  const int per = (np + 255) / 256;
  const int lo = min(tid * per, np), hi = min(lo + per, np);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += tiles(i);
  run[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < 256; ++i) {
      const int x = run[i];
      run[i] = acc;
      acc += x;
    }
    p.pstart[np] = acc;
  }
  __syncthreads();
  int acc = run[tid];
  for (int i = lo; i < hi; ++i) {
    p.pstart[i] = acc;
    acc += tiles(i);
  }
  __syncthreads();
  // units per kv head: one per pack plus the rest dealt in proportion to the
  // packs' key tiles
  const int U = np * p.nsplit, extra = U - np;
  const long long NT = p.pstart[np];
  for (int i = tid; i <= np; i += 256) {
    const long long e = NT > 0 ? (long long)extra * p.pstart[i] / NT : 0;
    p.ustart[i] = i == np ? U : i + int(e);
  }
  for (int i = tid; i < np; i += 256) {
    const long long e0 = NT > 0 ? (long long)extra * p.pstart[i] / NT : 0;
    const long long e1 = i + 1 == np ? extra : (NT > 0 ? (long long)extra * p.pstart[i + 1] / NT : 0);
    for (int u = i + int(e0); u < i + 1 + int(e1); ++u) p.umap[u] = i;
  }
  for (int i = tid; i < p.T * p.Hkv * np; i += 256) p.ctr[i] = 0;
  for (int i = tid; i < p.T * 8; i += 256) p.qctr[i] = 0;
}

// Matrix-core geometry of the one-node-branch problem of a trunk.
struct PrefillGeo {
  bool mfma;
  int B, bpp, np, nsplit;
};

PrefillGeo prefill_geo(const specopd_prefill_desc& d) {
  PrefillGeo g{};
  g.B = d.L - 1;
  g.mfma = d.dtype == SPECOPD_BF16 && g.B >= 1;
  if (g.mfma) {
    const int G = d.Hq / d.Hkv;
    g.bpp = mfma_rows_per_wg(d.D) / G;
    const double lim = 2147483647.0;
    if (g.bpp < 1 || double(d.L) * d.Hkv * d.D > lim || double(g.B) * d.Hq * d.D > lim) g.mfma = false;
  }
  if (g.mfma) {
    g.np = (g.B + g.bpp - 1) / g.bpp;
    g.nsplit = mfma_nsplit((long long)d.Hkv * g.np);
  }
  return g;
}

specopd_tree_attn_desc trunk_tree_desc(const specopd_prefill_desc& d) {
  specopd_tree_attn_desc t{};
  t.T = 1; t.L = d.L; t.B = d.L - 1; t.Wn = 1; t.Hq = d.Hq; t.Hkv = d.Hkv; t.D = d.D;
  t.dtype = d.dtype; t.rope_base = d.rope_base; t.scale = d.scale; t.flags = 0;
  return t;
}

}  // namespace

PrefillWs prefill_ws_layout(const specopd_prefill_desc& d) {
  const PrefillGeo g = prefill_geo(d);
  const size_t B = size_t(std::max(g.B, 0));
  PrefillWs w{};
  size_t off = 0;
  w.anchors = off;   off = align_up(off + B * sizeof(int32_t), 256);
  if (g.mfma) {
    w.qr = off;        off = align_up(off + size_t(d.T) * B * d.Hq * d.D * sizeof(uint16_t), 256);
    w.branch_ok = off; off = align_up(off + B * sizeof(int32_t), 256);
    w.order = off;     off = align_up(off + B * sizeof(int32_t), 256);
    w.anc = off;       off = align_up(off + B * sizeof(uint64_t), 256);
    w.pstart = off;    off = align_up(off + size_t(g.np + 1) * sizeof(int32_t), 256);
    w.ustart = off;    off = align_up(off + size_t(g.np + 1) * sizeof(int32_t), 256);
    w.umap = off;      off = align_up(off + size_t(g.np) * g.nsplit * sizeof(int32_t), 256);
    w.ctr = off;       off = align_up(off + size_t(d.T) * d.Hkv * g.np * sizeof(int32_t), 256);
    w.qctr = off;      off = align_up(off + size_t(d.T) * 8 * sizeof(unsigned long long), 256);
    const size_t units = size_t(d.Hkv) * g.np;
    w.part = off;      off = align_up(off + (g.nsplit > 1 ? units * g.nsplit * mfma_slot_bytes(d.D) : 0), 256);
  } else if (B > 0) {
    w.parent = off;    off = align_up(off + B * sizeof(int32_t), 256);
    w.pos = off;       off = align_up(off + B * sizeof(int32_t), 256);
    w.tree = off;      off = align_up(off + tree_attn_ws_layout(trunk_tree_desc(d)).total, 256);
  }
  w.total = off;
  return w;
}

hipError_t launch_prefill(const specopd_prefill_desc& d, const PrefillArgs& a, hipStream_t s) {
  const PrefillGeo g = prefill_geo(d);
  const PrefillWs L = prefill_ws_layout(d);
  const bool bf16 = d.dtype == SPECOPD_BF16;
  const size_t esz = bf16 ? 2 : 4;
  PrefillRopeParams rp{};
  rp.q = a.q; rp.k = a.k; rp.v = a.v;
  rp.cache_k = a.cache_k; rp.cache_v = a.cache_v; rp.out = a.out;
  rp.qr = g.mfma ? reinterpret_cast<uint16_t*>(a.ws + L.qr) : nullptr;
  rp.T = d.T; rp.L = d.L; rp.Hq = d.Hq; rp.Hkv = d.Hkv; rp.D = d.D;
  rp.log2_base = std::log2(double(a.rope_base));
  rp.qmul = a.scale * kLog2e;
  const size_t ntok = size_t(d.T) * d.L;
  const unsigned blocks = unsigned(std::min<size_t>((ntok + kPfTokens - 1) / kPfTokens, 16384));
  if (bf16) prefill_rope_kernel<uint16_t><<<blocks, 256, 0, s>>>(rp);
  else prefill_rope_kernel<float><<<blocks, 256, 0, s>>>(rp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.B < 1) return e;

  PrefillPlanParams pp{};
  pp.anchors = reinterpret_cast<int32_t*>(a.ws + L.anchors);
  pp.T = d.T; pp.B = g.B; pp.Hkv = d.Hkv;
  if (g.mfma) {
    pp.branch_ok = reinterpret_cast<int32_t*>(a.ws + L.branch_ok);
    pp.order = reinterpret_cast<int32_t*>(a.ws + L.order);
    pp.anc = reinterpret_cast<uint64_t*>(a.ws + L.anc);
    pp.pstart = reinterpret_cast<int32_t*>(a.ws + L.pstart);
    pp.ustart = reinterpret_cast<int32_t*>(a.ws + L.ustart);
    pp.umap = reinterpret_cast<int32_t*>(a.ws + L.umap);
    pp.ctr = reinterpret_cast<int32_t*>(a.ws + L.ctr);
    pp.qctr = reinterpret_cast<unsigned long long*>(a.ws + L.qctr);
    pp.bpp = g.bpp; pp.npacks = g.np; pp.nsplit = g.nsplit;
  } else {
    pp.parent = reinterpret_cast<int32_t*>(a.ws + L.parent);
    pp.pos = reinterpret_cast<int32_t*>(a.ws + L.pos);
  }
  prefill_plan_kernel<<<1, 256, 0, s>>>(pp);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  const size_t kv_tok = size_t(d.Hkv) * d.D, q_tok = size_t(d.Hq) * d.D;
  for (int t = 0; t < d.T; ++t) {
    const size_t t0 = size_t(t) * d.L;
    if (g.mfma) {
      MfmaParams p{};
      p.trunk_k = static_cast<const uint16_t*>(a.cache_k) + t0 * kv_tok;
      p.trunk_v = static_cast<const uint16_t*>(a.cache_v) + t0 * kv_tok;
      p.qr = reinterpret_cast<const uint16_t*>(a.ws + L.qr) + size_t(t) * g.B * q_tok;
      p.kr = static_cast<const uint16_t*>(a.cache_k) + (t0 + 1) * kv_tok;  // token b+1's rotated key
      p.v = static_cast<const uint16_t*>(a.cache_v) + (t0 + 1) * kv_tok;
      p.anchors = pp.anchors;
      p.anc = pp.anc;
      p.branch_ok = pp.branch_ok;
      p.order = pp.order;
      p.pstart = pp.pstart;
      p.ustart = pp.ustart;
      p.umap = pp.umap;
      p.ctr = pp.ctr + size_t(t) * d.Hkv * g.np;
      p.qctr = pp.qctr + size_t(t) * 8;
      p.part = a.ws + L.part;  // launches on one stream run in turn
      p.slot_bytes = mfma_slot_bytes(d.D);
      p.out = static_cast<uint16_t*>(a.out) + (t0 + 1) * q_tok;
      p.T = 1; p.B = g.B; p.L = d.L; p.Wn = 1; p.Hq = d.Hq; p.Hkv = d.Hkv; p.G = d.Hq / d.Hkv;
      p.bpp = g.bpp;
      p.spb = 1;
      p.tstride = 1;  // one-node branches: each token's own key, packed densely
      p.npacks = g.np;
      p.nsplit = g.nsplit;
      mfma_grid(p);
      timing_mark(2, 0, s);
      e = launch_tree_attn_mfma(d.D, p, s, true);
      timing_mark(2, 1, s);
    } else {
      TreeAttnArgs ta{};
      ta.trunk_k = static_cast<const char*>(a.cache_k) + t0 * kv_tok * esz;
      ta.trunk_v = static_cast<const char*>(a.cache_v) + t0 * kv_tok * esz;
      ta.q = static_cast<const char*>(a.q) + (t0 + 1) * q_tok * esz;
      ta.k = static_cast<const char*>(a.k) + (t0 + 1) * kv_tok * esz;
      ta.v = static_cast<const char*>(a.v) + (t0 + 1) * kv_tok * esz;
      ta.anchors = pp.anchors;
      ta.parent = pp.parent;
      ta.pos = pp.pos;
      ta.out = static_cast<char*>(a.out) + (t0 + 1) * q_tok * esz;
      ta.ws = a.ws + L.tree;
      ta.rope_base = a.rope_base;
      ta.scale = a.scale;
      ta.timing_kind = 2;
      e = launch_tree_attn(trunk_tree_desc(d), ta, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace specopd
