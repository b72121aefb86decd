// Tree-masked GQA attention of branch nodes against a prefilled trunk cache:
// planning, rotary embedding of the branch queries/keys, and the fp32-math
// path (used for fp32 inputs, and for bf16 inputs whose head size the matrix
// core path does not cover).
//
// Mask (jaehun.me review of SpecOPD, §3.2(a), Eq. 5): node j of branch b
// reads trunk positions 0..a_b and the nodes on its own parent chain, itself
// included.  Rotary embedding at the semantic position a_b + 1 + depth(j)
// (rustineverything.app summary, §2.1), rotate-half pairing (i, i + D/2),
// angle pos * base^(-2i/D).
#include <math.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace specopd {

// ---------------------------------------------------------------- planning

// One thread per branch: validate the anchor, the parent map and the semantic
// positions, and record each node's ancestor bitmask (bit k set when node k
// is the node itself or one of its ancestors; depth = popcount - 1).
__global__ void tree_plan_kernel(const int32_t* __restrict__ anchors,
                                 const int32_t* __restrict__ parent,
                                 const int32_t* __restrict__ pos, int TB, int Wn, int L,
                                 uint64_t* __restrict__ anc, int32_t* __restrict__ branch_ok) {
  const int tb = blockIdx.x * blockDim.x + threadIdx.x;
  if (tb >= TB) return;
  const int a = anchors[tb];
  bool ok = (a >= 0) && (a < L);
  const int32_t* par = parent + size_t(tb) * Wn;
  const int32_t* ps = pos + size_t(tb) * Wn;
  uint64_t* an = anc + size_t(tb) * Wn;
  for (int j = 0; j < Wn; ++j) {
    const int p = par[j];
    uint64_t m = uint64_t(1) << j;
    if (p >= 0 && p < j) {
      m |= an[p];
    } else if (p != -1) {
      ok = false;
    }
    an[j] = m;
    const int depth = __popcll(m) - 1;
    if (ps[j] != a + 1 + depth) ok = false;
  }
  branch_ok[tb] = ok ? 1 : 0;
}

// ---------------------------------------------------------------- score rows

// One thread per node: the score row of branch token j is its parent's row,
// or the anchor's trunk row for a token attached to the anchor (jaehun.me
// review §3.2(a), Fig. 3).  Rows: trunk rows t*L + s first, then branch rows
// T*L + (t*B + b)*Wn + j.  A malformed branch gets -1 for every node.
__global__ void score_rows_kernel(const int32_t* __restrict__ anchors,
                                  const int32_t* __restrict__ parent, int T, int L, int B, int Wn,
                                  int32_t* __restrict__ rows) {
  const long long n = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long nodes = (long long)T * B * Wn;
  if (n >= nodes) return;
  const long long tb = n / Wn;
  const int j = int(n - tb * Wn);
  const int t = int(tb / B);
  const int a = anchors[tb];
  bool ok = a >= 0 && a < L;
  const int32_t* par = parent + tb * Wn;
  for (int k = 0; k < Wn; ++k) {
    const int pk = par[k];
    ok = ok && pk >= -1 && pk < k;
  }
  const int p = par[j];
  long long r = p < 0 ? (long long)t * L + a : (long long)T * L + tb * Wn + p;
  rows[n] = ok ? int32_t(r) : -1;
}

hipError_t launch_score_rows(const specopd_tree_attn_desc& d, const int32_t* anchors,
                             const int32_t* parent, int32_t* rows, hipStream_t s) {
  const long long nodes = (long long)d.T * d.B * d.Wn;
  score_rows_kernel<<<unsigned((nodes + 255) / 256), 256, 0, s>>>(anchors, parent, d.T, d.L, d.B,
                                                                 d.Wn, rows);
  return hipGetLastError();
}

// ---------------------------------------------------------------- rotary

// Rotates every branch query and key at its node's semantic position.  One
// thread per (node, pair i), looping over the heads, so each angle is formed
// once.  The angle is formed and reduced in fp64: positions reach tens of
// thousands of radians, where an fp32 angle would be off by ~1e-3.  Queries
// are also multiplied by `qmul`.
template <typename T, typename O>
__global__ void rope_branch_kernel(const T* __restrict__ x, const int32_t* __restrict__ pos,
                                   int nodes, int H, int D, double log2_base, float qmul,
                                   O* __restrict__ out) {
  const int half = D >> 1;
  const size_t total = size_t(nodes) * half;
  for (size_t idx = size_t(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += size_t(gridDim.x) * blockDim.x) {
    const int i = int(idx % half);
    const size_t node = idx / half;
    const double theta = exp2(-(2.0 * i / D) * log2_base);
    const double ang = double(pos[node]) * theta;
    double sn, cs;
    sincos(ang, &sn, &cs);
    const float c = float(cs), s = float(sn);
    for (int hd = 0; hd < H; ++hd) {
      const size_t nh = node * H + hd;
      const T* src = x + nh * D;
      const float x1 = load_f32(src + i), x2 = load_f32(src + i + half);
      O* dst = out + nh * D;
      store_f32(dst + i, (x1 * c - x2 * s) * qmul);
      store_f32(dst + i + half, (x2 * c + x1 * s) * qmul);
    }
  }
}

// ---------------------------------------------------------------- preparation (bf16 path)

struct PrepParams {
  const int32_t *anchors, *parent, *pos;
  const uint16_t *q, *k;
  uint64_t* anc;
  int32_t *branch_ok, *order, *pstart, *ustart, *umap, *ctr;
  unsigned long long* qctr;
  uint16_t *qr, *kr;
  int T, B, L, Wn, Hq, Hkv, D, bpp, spb, tstride, npacks, nsplit;
  double log2_base;
  float qmul;
};

constexpr int kSortLds = 2048;  // branches per trunk planned and sorted in LDS
constexpr int kPlanLds = 8192;  // nodes per trunk whose parents are staged in LDS
constexpr int kRopeNodes = 4;   // nodes per rotary pass of a workgroup
constexpr int kRopeBatch = 6;   // rotary units per thread whose loads are in flight together

__device__ void plan_branch(const PrepParams& p, size_t tb) {
  const int a = p.anchors[tb];
  bool ok = (a >= 0) && (a < p.L);
  const int32_t* par = p.parent + tb * p.Wn;
  const int32_t* ps = p.pos + tb * p.Wn;
  uint64_t* an = p.anc + tb * p.Wn;
  for (int j = 0; j < p.Wn; ++j) {
    const int pj = par[j];
    uint64_t m = uint64_t(1) << j;
    if (pj >= 0 && pj < j) {
      m |= an[pj];  // written by this thread above
    } else if (pj != -1) {
      ok = false;
    }
    an[j] = m;
    const int depth = __popcll(m) - 1;
    if (ps[j] != a + 1 + depth) ok = false;
  }
  p.branch_ok[tb] = ok ? 1 : 0;
}

// One launch prepares everything the matrix-core kernel reads:
//   workgroups [0, T): one trunk each -- validate its branches and record
//     ancestor masks, order the branches by anchor (longest first, malformed
//     last, ties by index; rank sort), tabulate the packs' key tiles as prefix
//     sums, and clear the trunk's split-pack counters;
//   the other workgroups: rotary embedding of branch queries (times qmul) and
//     keys, a few nodes at a time, angles in fp64.
__global__ __launch_bounds__(256) void tree_prep_kernel(const PrepParams p) {
  const int tid = threadIdx.x;
  if (int(blockIdx.x) < p.T) {
    const int t = blockIdx.x;
    const size_t tB = size_t(t) * p.B;
    const int B = p.B, Wn = p.Wn;
    __shared__ int8_t s_par[kPlanLds];  // parent of every node of the trunk
    __shared__ int8_t s_dep[kPlanLds];  // depth its position implies (-1: none in 0..63)
    __shared__ __attribute__((aligned(16))) int s_key[kSortLds + 4];  // anchor, then sort key (-1: malformed)
    __shared__ int s_bad[kSortLds];
    __shared__ int s_ord[kSortLds];
    __shared__ int run[256];
    const int nodes = B * Wn;
    const bool staged = B <= kSortLds && nodes <= kPlanLds;
    if (staged) {
      for (int b = tid; b < B; b += 256) {
        s_key[b] = p.anchors[tB + b];
        s_bad[b] = 0;
      }
      // parents, positions and anchors are read in one pass (independent
      // loads), so the walk below touches only LDS
#pragma unroll 4
      for (int i = tid; i < nodes; i += 256) {
        const int pj = p.parent[tB * Wn + i];
        s_par[i] = int8_t((pj >= -1 && pj < 64) ? pj : -2);  // -2: invalid
        const long long e = (long long)p.pos[tB * Wn + i] - p.anchors[tB + i / Wn] - 1;
        s_dep[i] = int8_t((e >= 0 && e < 64) ? e : -1);
      }
      __syncthreads();
      // ancestor masks by pointer jumping: one lane per node, a branch's
      // nodes in a group of gsz lanes (the power of two >= Wn); each round a
      // node takes in the mask of the node its link points to and links on
      // to that node's link, so after r rounds the mask holds the ancestors
      // less than 2^r steps up (a parent must be an earlier node, so a
      // node's depth is below Wn).  A node whose own parent is out of range
      // marks its branch malformed and counts as a root.  The mask's size
      // fixes the depth.
      {
        int gsz = 1, rounds = 0;
        while (gsz < Wn) {
          gsz <<= 1;
          ++rounds;
        }
        const int lane = tid & 63, wv = tid >> 6;
        const int j = lane & (gsz - 1);
        const int bpw = 64 / gsz;  // branches per wave and pass
        for (int b0 = wv * bpw; b0 < B; b0 += 4 * bpw) {
          const int b = b0 + lane / gsz;
          const bool live = b < B && j < Wn;
          int pj = live ? int(s_par[b * Wn + j]) : -1;
          bool ok = true;
          if (pj < -1 || pj >= j) {
            ok = false;
            pj = -1;
          }
          uint64_t m = live ? uint64_t(1) << j : 0;
          int link = pj >= 0 ? lane - j + pj : -1;  // the parent's lane
          for (int rd = 0; rd < rounds; ++rd) {
            const int src = (link >= 0 ? link : lane) << 2;
            const unsigned lo = __builtin_amdgcn_ds_bpermute(src, unsigned(m));
            const unsigned hi = __builtin_amdgcn_ds_bpermute(src, unsigned(m >> 32));
            const int nl = __builtin_amdgcn_ds_bpermute(src, link);
            if (link >= 0) {
              m |= (uint64_t(hi) << 32) | lo;
              link = nl;
            }
          }
          if (live) {
            const int i = b * Wn + j;
            if (s_dep[i] != __popcll(m) - 1) ok = false;
            p.anc[tB * Wn + i] = m;
            if (!ok) s_bad[b] = 1;
          }
        }
      }
      __syncthreads();
      for (int b = tid; b < B; b += 256) {
        const int a = s_key[b];
        const bool ok = !s_bad[b] && a >= 0 && a < p.L;
        p.branch_ok[tB + b] = ok ? 1 : 0;
        s_key[b] = ok ? a : -1;
      }
      __syncthreads();
      // rank sort; keys are read four at a time (s_key is padded with keys
      // that rank below every branch)
      for (int b = B + tid; b < ((B + 3) & ~3); b += 256) s_key[b] = -2;
      __syncthreads();
      for (int b = tid; b < B; b += 256) {
        const int kb = s_key[b];
        int rank = 0;
#pragma unroll 4
        for (int o = 0; o < B; o += 4) {
          const int4 ko = *reinterpret_cast<const int4*>(s_key + o);
          rank += (ko.x > kb) || (ko.x == kb && o < b);
          rank += (ko.y > kb) || (ko.y == kb && o + 1 < b);
          rank += (ko.z > kb) || (ko.z == kb && o + 2 < b);
          rank += (ko.w > kb) || (ko.w == kb && o + 3 < b);
        }
        s_ord[rank] = b;
        p.order[tB + rank] = b;
      }
      __syncthreads();
    } else {
      for (int b = tid; b < B; b += 256) plan_branch(p, tB + b);
      __syncthreads();
      for (int b = tid; b < B; b += 256) {
        const int kb = p.branch_ok[tB + b] ? p.anchors[tB + b] : -1;
        int rank = 0;
        for (int o = 0; o < B; ++o) {
          const int ko = p.branch_ok[tB + o] ? p.anchors[tB + o] : -1;
          rank += (ko > kb) || (ko == kb && o < b);
        }
        p.order[tB + rank] = b;
      }
      __syncthreads();
    }
    // key tiles of pack pk: trunk tiles up to its longest anchor, then tail
    // tiles holding the pack's branch nodes (a branch split over spb packs
    // gives each of them its trunk and its nodes)
    auto tiles = [&](int pk) {
      const int b0 = (pk / p.spb) * p.bpp;
      const int nbr = min(p.bpp, B - b0);
      int a;
      if (staged) {
        a = s_key[s_ord[b0]];
      } else {
        const int bl = p.order[tB + b0];
        a = p.branch_ok[tB + bl] ? p.anchors[tB + bl] : -1;
      }
      return mfma_pack_tiles(a, nbr, p.tstride, Wn);
    };
    // exclusive prefix sums of the packs' tiles: per-thread runs, then a scan
    // of the 256 run totals
    const int np = p.npacks;
    const int per = (np + 255) / 256;
    const int lo = min(tid * per, np), hi = min(lo + per, np);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += tiles(i);
    run[tid] = sum;
    __syncthreads();
    int32_t* ps = p.pstart + size_t(t) * (np + 1);
    __shared__ int wsum[4];
    {
      // exclusive scan of the 256 run totals: within each wave by shuffles,
      // then across the four waves
      const int lane = tid & 63, w = tid >> 6;
      int x = run[tid];
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (lane == 63) wsum[w] = x;
      __syncthreads();
      int base = 0;
      for (int i = 0; i < w; ++i) base += wsum[i];
      const int excl = base + x - run[tid];
      __syncthreads();
      run[tid] = excl;
      if (tid == 255) ps[np] = base + x;
    }
    __syncthreads();
    // each thread's run of packs: tile offsets, and the matrix-core kernel's
    // units per (trunk, kv head): U = npacks * nsplit, one per pack plus the
    // other U - npacks dealt to the packs in proportion to their key tiles
    // (cumulatively, so they add up exactly)
    {
      const long long NT = (long long)wsum[0] + wsum[1] + wsum[2] + wsum[3];
      const int U = np * p.nsplit, extra = U - np;
      int32_t* us = p.ustart + size_t(t) * (np + 1);
      int32_t* um = p.umap + size_t(t) * U;
      auto share = [&](long long tiles_before) {
        return NT > 0 ? int((long long)extra * tiles_before / NT) : 0;
      };
      int acc = run[tid];
      for (int i = lo; i < hi; ++i) {
        const int ti = tiles(i);
        ps[i] = acc;
        const int e0 = share(acc), e1 = i + 1 == np ? extra : share(acc + ti);
        us[i] = i + e0;
        for (int u = i + e0; u < i + 1 + e1; ++u) um[u] = i;
        acc += ti;
      }
      if (tid == 255) us[np] = U;
    }
    int32_t* c = p.ctr + size_t(t) * p.Hkv * np;
    for (int i = tid; i < p.Hkv * np; i += 256) c[i] = 0;
    if (t == 0 && tid < 8) p.qctr[tid] = 0;
    return;
  }
  // rotary: kRopeNodes nodes per workgroup pass.  Frequencies are tabulated
  // once per workgroup (fp64); an angle is formed and reduced modulo 2 pi in
  // fp64 (positions reach tens of thousands of radians) and its sine and
  // cosine taken in fp32 on the reduced argument.  The workgroup's threads
  // then take (node, head, eight pairs) units of all query and key heads.
  __shared__ double s_theta[128];            // D/2 <= 128
  __shared__ float2 s_cs[kRopeNodes * 128];  // (cos, sin)
  const int half = p.D / 2;
  const int octs = p.D / 16;
  const int H = p.Hq + p.Hkv;
  const size_t nodes = size_t(p.T) * p.B * p.Wn;
  if (tid < half) s_theta[tid] = exp2(-(2.0 * tid / p.D) * p.log2_base);
  for (size_t n0 = size_t(blockIdx.x - p.T) * kRopeNodes; n0 < nodes;
       n0 += size_t(gridDim.x - p.T) * kRopeNodes) {
    const int nn = int(min(size_t(kRopeNodes), nodes - n0));
    __syncthreads();  // the previous pass's angles are no longer read
    for (int idx = tid; idx < nn * half; idx += 256) {
      const int ln = idx / half, i = idx - ln * half;
      const double ang = double(p.pos[n0 + ln]) * s_theta[i];
      const double k = rint(ang * 0.15915494309189535);  // 1 / (2 pi)
      const float r = float(fma(-k, 6.283185307179586, ang));
      float sn, cs;
      sincosf(r, &sn, &cs);
      s_cs[idx] = make_float2(cs, sn);
    }
    __syncthreads();
    // kRopeBatch units per thread at a time: their loads are all issued
    // before any of them is rotated, so a pass costs one memory round trip
    // per batch rather than one per unit
    const int units = nn * H * octs;
    for (int u0 = tid; u0 < units; u0 += 256 * kRopeBatch) {
      u32x4 a[kRopeBatch], b[kRopeBatch];
#pragma unroll
      for (int r = 0; r < kRopeBatch; ++r) {
        const int u = u0 + r * 256;
        if (u < units) {
          const int lnh = u / octs;
          const int i0 = (u - lnh * octs) * 8;
          const int ln = lnh / H, hd = lnh - ln * H;
          const size_t node = n0 + ln;
          const uint16_t* src =
              hd < p.Hq ? p.q + (node * p.Hq + hd) * p.D : p.k + (node * p.Hkv + (hd - p.Hq)) * p.D;
          a[r] = *reinterpret_cast<const u32x4*>(src + i0);
          b[r] = *reinterpret_cast<const u32x4*>(src + i0 + half);
        }
      }
#pragma unroll
      for (int r = 0; r < kRopeBatch; ++r) {
        const int u = u0 + r * 256;
        if (u < units) {
          const int lnh = u / octs;
          const int i0 = (u - lnh * octs) * 8;
          const int ln = lnh / H, hd = lnh - ln * H;
          const size_t node = n0 + ln;
          const bool isq = hd < p.Hq;
          uint16_t* dst = isq ? p.qr + (node * p.Hq + hd) * p.D : p.kr + (node * p.Hkv + (hd - p.Hq)) * p.D;
          const float mul = isq ? p.qmul : 1.0f;
          u32x4 ya, yb;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float2 c0 = s_cs[ln * half + i0 + 2 * e], c1 = s_cs[ln * half + i0 + 2 * e + 1];
            const float x10 = bf16_lo(a[r][e]), x11 = bf16_hi(a[r][e]);
            const float x20 = bf16_lo(b[r][e]), x21 = bf16_hi(b[r][e]);
            ya[e] = pack_bf16x2((x10 * c0.x - x20 * c0.y) * mul, (x11 * c1.x - x21 * c1.y) * mul);
            yb[e] = pack_bf16x2((x20 * c0.x + x10 * c0.y) * mul, (x21 * c1.x + x11 * c1.y) * mul);
          }
          *reinterpret_cast<u32x4*>(dst + i0) = ya;
          *reinterpret_cast<u32x4*>(dst + i0 + half) = yb;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- fp32 path

// One workgroup per (trunk, branch, kv head); each wave takes rows
// (node j, head h in the kv group) in turn; lanes take keys 64 at a time for
// the scores and dimensions for the weighted sum.  Online softmax in fp32.
template <typename T, int D>
__global__ __launch_bounds__(256) void tree_attn_generic_kernel(
    const T* __restrict__ trunk_k, const T* __restrict__ trunk_v, const float* __restrict__ qr,
    const float* __restrict__ kr, const T* __restrict__ v, const int32_t* __restrict__ anchors,
    const uint64_t* __restrict__ anc, const int32_t* __restrict__ branch_ok, int B, int L,
    int Wn, int Hq, int Hkv, T* __restrict__ out) {
  constexpr int DL = D / 64;  // dims per lane
  __shared__ float qs[4][D];
  __shared__ float pb[4][64];
  const int G = Hq / Hkv;
  const int g = blockIdx.x % Hkv;
  const int tb = blockIdx.x / Hkv;  // t*B + b
  const int t = tb / B;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int a = anchors[tb];
  const bool ok = branch_ok[tb] != 0;
  const size_t kv_stride = size_t(Hkv) * D;  // between consecutive trunk positions
  const T* tk = trunk_k + size_t(t) * L * kv_stride + size_t(g) * D;
  const T* tv = trunk_v + size_t(t) * L * kv_stride + size_t(g) * D;
  const float* kb = kr + size_t(tb) * Wn * kv_stride + size_t(g) * D;
  const T* vb = v + size_t(tb) * Wn * kv_stride + size_t(g) * D;

  for (int r = w; r < Wn * G; r += 4) {
    const int j = r / G;
    const int h = g * G + (r - j * G);
    const size_t orow = (size_t(tb) * Wn + j) * Hq + h;
    if (!ok) {
      for (int i = 0; i < DL; ++i) store_f32(out + orow * D + lane + 64 * i, __builtin_nanf(""));
      continue;
    }
    const float* qrow = qr + orow * D;
    for (int i = 0; i < DL; ++i) qs[w][lane + 64 * i] = qrow[lane + 64 * i];
    __builtin_amdgcn_wave_barrier();
    float m = kNegInf, l = 0.f, o[DL];
#pragma unroll
    for (int i = 0; i < DL; ++i) o[i] = 0.f;
    const uint64_t am = anc[size_t(tb) * Wn + j];
    // key tiles: trunk 0..a, then the branch's own nodes (one tile, Wn <= 64)
    const int ntrunk_tiles = (a + 1 + 63) / 64;
    for (int tile = 0; tile <= ntrunk_tiles; ++tile) {
      const bool branch_tile = tile == ntrunk_tiles;
      const int key = branch_tile ? lane : tile * 64 + lane;
      const bool valid = branch_tile ? (lane < Wn && ((am >> lane) & 1)) : (key <= a);
      float sc = kNegInf;
      if (valid) {
        float acc = 0.f;
        if (branch_tile) {
          const float* kk = kb + size_t(key) * kv_stride;
          for (int d = 0; d < D; ++d) acc = __builtin_fmaf(qs[w][d], kk[d], acc);
        } else {
          const T* kk = tk + size_t(key) * kv_stride;
          for (int d = 0; d < D; ++d) acc = __builtin_fmaf(qs[w][d], load_f32(kk + d), acc);
        }
        sc = acc;  // queries carry the score scale
      }
      const float tmax = wave_max(sc);
      const float mn = fmaxf(m, tmax);
      const float p = valid ? __expf(sc - mn) : 0.f;
      const float corr = (m == kNegInf) ? 0.f : __expf(m - mn);
      l = l * corr + wave_sum(p);
#pragma unroll
      for (int i = 0; i < DL; ++i) o[i] *= corr;
      m = mn;
      pb[w][lane] = p;
      __builtin_amdgcn_wave_barrier();
      const int nk = branch_tile ? Wn : min(64, a + 1 - tile * 64);
      for (int k = 0; k < nk; ++k) {
        const float pk = pb[w][k];
        if (pk != 0.f) {
          const T* vv = branch_tile ? vb + size_t(k) * kv_stride : tv + size_t(tile * 64 + k) * kv_stride;
#pragma unroll
          for (int i = 0; i < DL; ++i) o[i] = __builtin_fmaf(pk, load_f32(vv + lane + 64 * i), o[i]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    const float inv = 1.f / l;
#pragma unroll
    for (int i = 0; i < DL; ++i) store_f32(out + orow * D + lane + 64 * i, o[i] * inv);
  }
}

// ---------------------------------------------------------------- launch

// Matrix-core plan: branches per pack, packs per branch and packs per trunk;
// false for fp32 inputs.  A pack fills one workgroup with the rows (node x
// query head of a kv group) of whole branches; a branch with more rows than
// a workgroup holds is split over several packs, each scoring a slice of its
// rows against all of its keys.
struct MfmaPlan {
  int bpp, spb, npacks, nsplit;
};
static bool mfma_plan(const specopd_tree_attn_desc& d, MfmaPlan* pl) {
  if (d.dtype != SPECOPD_BF16) return false;
  // per-trunk element offsets are formed in 32 bits
  const double lim = 2147483647.0;
  if (double(d.L) * d.Hkv * d.D > lim || double(d.B) * d.Wn * d.Hq * d.D > lim) return false;
  const int rows_per_branch = d.Wn * (d.Hq / d.Hkv);
  const int rpw = mfma_rows_per_wg(d.D);
  if (rows_per_branch <= rpw) {
    pl->bpp = rpw / rows_per_branch;
    pl->spb = 1;
    pl->npacks = (d.B + pl->bpp - 1) / pl->bpp;
  } else {
    pl->bpp = 1;
    pl->spb = (rows_per_branch + rpw - 1) / rpw;
    if (double(d.B) * pl->spb > lim) return false;
    pl->npacks = d.B * pl->spb;
  }
  pl->nsplit = mfma_nsplit((long long)d.T * d.Hkv * pl->npacks,
                           (d.flags & SPECOPD_TREE_BATCH_INVARIANT) != 0);
  return true;
}

TreeAttnWs tree_attn_ws_layout(const specopd_tree_attn_desc& d) {
  const size_t TB = size_t(d.T) * d.B, nodes = TB * d.Wn;
  MfmaPlan pl{};
  const bool mf = mfma_plan(d, &pl);
  const int np = mf ? pl.npacks : 0;
  TreeAttnWs w{};
  size_t off = 0;
  w.anc = off;        off = align_up(off + nodes * sizeof(uint64_t), 256);
  w.branch_ok = off;  off = align_up(off + TB * sizeof(int32_t), 256);
  w.order = off;      off = align_up(off + TB * sizeof(int32_t), 256);
  // rotated branch queries then keys: bf16 for the matrix-core path, fp32 otherwise
  const size_t esz = mf ? sizeof(uint16_t) : sizeof(float);
  w.rot = off;        off = align_up(off + nodes * (size_t(d.Hq) + d.Hkv) * d.D * esz, 256);
  w.pstart = off;     off = align_up(off + (mf ? size_t(d.T) * (np + 1) * sizeof(int32_t) : 0), 256);
  const long long units = mf ? (long long)d.T * d.Hkv * np : 0;
  const int nsplit = mf ? pl.nsplit : 1;
  w.ustart = off;     off = align_up(off + (mf ? size_t(d.T) * (np + 1) * sizeof(int32_t) : 0), 256);
  w.umap = off;       off = align_up(off + (mf ? size_t(d.T) * np * nsplit * sizeof(int32_t) : 0), 256);
  w.ctr = off;        off = align_up(off + (mf ? size_t(d.T) * d.Hkv * np * sizeof(int32_t) : 0), 256);
  w.qctr = off;       off = align_up(off + (mf ? 8 * sizeof(unsigned long long) : 0), 256);
  w.part = off;       off = align_up(off + (nsplit > 1 ? size_t(units) * nsplit * mfma_slot_bytes(d.D) : 0), 256);
  w.total = off;
  return w;
}

template <typename T>
static hipError_t launch_generic(const specopd_tree_attn_desc& d, const TreeAttnArgs& a,
                                 const uint64_t* anc, const int32_t* ok, float* qr, float* kr,
                                 hipStream_t s) {
  const int TB = d.T * d.B;
  const unsigned blocks = unsigned(TB) * d.Hkv;
#define SPECOPD_GEN(DD)                                                                         \
  tree_attn_generic_kernel<T, DD><<<blocks, 256, 0, s>>>(                                      \
      static_cast<const T*>(a.trunk_k), static_cast<const T*>(a.trunk_v), qr, kr,              \
      static_cast<const T*>(a.v), a.anchors, anc, ok, d.B, d.L, d.Wn, d.Hq, d.Hkv,             \
      static_cast<T*>(a.out))
  timing_mark(a.timing_kind, 0, s);
  switch (d.D) {
    case 64: SPECOPD_GEN(64); break;
    case 128: SPECOPD_GEN(128); break;
    case 256: SPECOPD_GEN(256); break;
    default: return hipErrorInvalidValue;
  }
#undef SPECOPD_GEN
  timing_mark(a.timing_kind, 1, s);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_rope_fp32(const specopd_tree_attn_desc& d, const TreeAttnArgs& a,
                                   float* qr, float* kr, hipStream_t s) {
  const int nodes = d.T * d.B * d.Wn;
  const double lb = log2(double(a.rope_base));
  auto grid = [](size_t n) { return unsigned(std::min<size_t>((n + 255) / 256, 65536)); };
  rope_branch_kernel<T, float><<<grid(size_t(nodes) * d.D / 2), 256, 0, s>>>(
      static_cast<const T*>(a.q), a.pos, nodes, d.Hq, d.D, lb, a.scale, qr);
  rope_branch_kernel<T, float><<<grid(size_t(nodes) * d.D / 2), 256, 0, s>>>(
      static_cast<const T*>(a.k), a.pos, nodes, d.Hkv, d.D, lb, 1.0f, kr);
  return hipGetLastError();
}

hipError_t launch_tree_attn(const specopd_tree_attn_desc& d, const TreeAttnArgs& a, hipStream_t s) {
  const TreeAttnWs L = tree_attn_ws_layout(d);
  uint64_t* anc = reinterpret_cast<uint64_t*>(a.ws + L.anc);
  int32_t* ok = reinterpret_cast<int32_t*>(a.ws + L.branch_ok);
  int32_t* order = reinterpret_cast<int32_t*>(a.ws + L.order);
  const int TB = d.T * d.B;
  const int nodes = TB * d.Wn;
  hipError_t e;
  MfmaPlan pl{};
  if (mfma_plan(d, &pl)) {
    uint16_t* qr = reinterpret_cast<uint16_t*>(a.ws + L.rot);
    uint16_t* kr = qr + size_t(nodes) * d.Hq * d.D;
    PrepParams pp{};
    pp.anchors = a.anchors; pp.parent = a.parent; pp.pos = a.pos;
    pp.q = static_cast<const uint16_t*>(a.q);
    pp.k = static_cast<const uint16_t*>(a.k);
    pp.anc = anc; pp.branch_ok = ok; pp.order = order;
    pp.pstart = reinterpret_cast<int32_t*>(a.ws + L.pstart);
    pp.ustart = reinterpret_cast<int32_t*>(a.ws + L.ustart);
    pp.umap = reinterpret_cast<int32_t*>(a.ws + L.umap);
    pp.nsplit = pl.nsplit;
    pp.ctr = reinterpret_cast<int32_t*>(a.ws + L.ctr);
    pp.qctr = reinterpret_cast<unsigned long long*>(a.ws + L.qctr);
    pp.qr = qr; pp.kr = kr;
    pp.T = d.T; pp.B = d.B; pp.L = d.L; pp.Wn = d.Wn; pp.Hq = d.Hq; pp.Hkv = d.Hkv; pp.D = d.D;
    pp.bpp = pl.bpp; pp.spb = pl.spb; pp.tstride = mfma_tail_stride(d.Wn); pp.npacks = pl.npacks;
    pp.log2_base = log2(double(a.rope_base));
    pp.qmul = a.scale * kLog2e;
    const unsigned rope_blocks = unsigned(std::min<size_t>((size_t(nodes) + kRopeNodes - 1) / kRopeNodes, 16384));
    tree_prep_kernel<<<unsigned(d.T) + rope_blocks, 256, 0, s>>>(pp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    MfmaParams p{};
    p.trunk_k = static_cast<const uint16_t*>(a.trunk_k);
    p.trunk_v = static_cast<const uint16_t*>(a.trunk_v);
    p.qr = qr;
    p.kr = kr;
    p.v = static_cast<const uint16_t*>(a.v);
    p.anchors = a.anchors;
    p.anc = anc;
    p.branch_ok = ok;
    p.order = order;
    p.pstart = pp.pstart;
    p.ustart = pp.ustart;
    p.umap = pp.umap;
    p.ctr = pp.ctr;
    p.qctr = pp.qctr;
    p.part = a.ws + L.part;
    p.slot_bytes = mfma_slot_bytes(d.D);
    p.out = static_cast<uint16_t*>(a.out);
    p.T = d.T; p.B = d.B; p.L = d.L; p.Wn = d.Wn; p.Hq = d.Hq; p.Hkv = d.Hkv; p.G = d.Hq / d.Hkv;
    p.bpp = pl.bpp;
    p.spb = pl.spb;
    p.tstride = pp.tstride;
    p.npacks = pl.npacks;
    p.nsplit = pp.nsplit;
    mfma_grid(p);
    timing_mark(a.timing_kind, 0, s);
    e = launch_tree_attn_mfma(d.D, p, s);
    timing_mark(a.timing_kind, 1, s);
    return e;
  }
  tree_plan_kernel<<<(TB + 255) / 256, 256, 0, s>>>(a.anchors, a.parent, a.pos, TB, d.Wn, d.L, anc, ok);
  float* qr = reinterpret_cast<float*>(a.ws + L.rot);
  float* kr = qr + size_t(nodes) * d.Hq * d.D;
  if (d.dtype == SPECOPD_BF16) {
    if ((e = launch_rope_fp32<uint16_t>(d, a, qr, kr, s)) != hipSuccess) return e;
    return launch_generic<uint16_t>(d, a, anc, ok, qr, kr, s);
  }
  if ((e = launch_rope_fp32<float>(d, a, qr, kr, s)) != hipSuccess) return e;
  return launch_generic<float>(d, a, anc, ok, qr, kr, s);
}

}  // namespace specopd
