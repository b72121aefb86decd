// Block selection of a sparse-attention (QSA) target with branch-consistent
// indexer groups (gfx950).
//
// What is computed (jaehun.me review of SpecOPD, §3.2(b) and the Fig. 4
// walk-through): tokens form groups of 4 consecutive positions; a group's
// indexer key is the mean of its tokens' raw indexer keys, RMS-normalised,
// then rotated at the group's first position.  A query at position p scores
// every group complete at p against its own rotated indexer query and keeps
// the top k.  On a branch, groups complete at the anchor reuse the trunk's
// cached keys unchanged; the group that holds the anchor (when the anchor
// does not complete it) and every later group are compressed again from the
// node's own history, so no reference token after the anchor enters a key
// and each sub-branch of a fork keeps groups of its own.
//
// Kernels:
//   qsa_trunk_groups_kernel  one wave per trunk group: the trunk pass's cache.
//   qsa_score_kernel         a few workgroups per branch (each every
//                            nsplit-th trunk tile): validates the tree,
//                            rotates the nodes' queries (bf16, LDS),
//                            compresses the groups its nodes complete (one
//                            wave per node; the boundary group's trunk tokens
//                            stand in the four raw slots), scores the cached
//                            trunk groups on the matrix cores
//                            (v_mfma_f32_32x32x16_bf16, A = 32 group keys
//                            staged per wave through LDS from whole-row
//                            loads, B = the rotated queries,
//                            32 nodes per row block) and the branch's own
//                            groups with wave dot products; every row's
//                            candidate scores go to the workspace.
//   qsa_topk_kernel          one workgroup per node: the row's scores into LDS
//                            as order-preserving integer keys, the k-th
//                            largest key by up to four 8-bit radix passes
//                            (histograms with LDS atomics, digit found by a
//                            wave suffix scan), then the kept groups written
//                            in increasing group order by ballot prefix sums
//                            (keys equal to the k-th go to the lowest groups).
#include <math.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace specopd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int kGroup = 4;
// workgroups the scoring kernel aims for (branches x splits); measured: more
// splits add their own prologues (tree walk, query rotation) for little gain
constexpr long long kQsaScoreWgs = 1024;

struct QsaKArgs {
  const uint16_t *trunk_gk, *trunk_raw, *x, *y;
  const float* gamma;
  const int32_t *anchors, *parent, *pos;
  int32_t* sel;
  float* score;
  uint16_t* bkey;
  int32_t* bad;    // malformed branches of the call
  int32_t* ncand;  // [rows] candidates of every node, -1 for a malformed branch
  float* sc;       // [rows][Gs] candidate scores
  int L, B, Wn, ng, Gs, topk;
  int nsplit;  // workgroups per branch, each taking every nsplit-th trunk tile
  double log2_base;
  float eps;
};

// Rotation frequencies theta_i = base^(-2i/Di), i < Di/2, in fp64 into an
// LDS table (by the whole workgroup; a barrier must follow).
template <int DI>
__device__ __forceinline__ void fill_theta(double* s_theta, double log2_base) {
  for (int i = threadIdx.x; i < DI / 2; i += blockDim.x) s_theta[i] = exp2(-(2.0 * i / DI) * log2_base);
}

// cos and sin of pos * theta: the angle formed and reduced modulo 2 pi in
// fp64 (2 pi in two parts), then the fp32 functions on [-pi, pi]
__device__ __forceinline__ void rot_cs(int pos, double theta, float& c, float& s) {
  const double ang = double(pos) * theta;
  const double k = rint(ang * 0.15915494309189535);  // 1 / (2 pi)
  const double r = __builtin_fma(-k, 2.4492935982947064e-16, __builtin_fma(-k, 6.283185307179586, ang));
  sincosf(float(r), &s, &c);
}

// One wave compresses one group: the four rows r[0..3] (bf16, DI values,
// oldest first) are averaged, RMS-normalised with gain gamma, rotated at
// `first` (rotate-half pairs i, i + DI/2) and written to out as bf16.
// Lane l owns the pairs l, l + 64, ...
template <int DI>
__device__ void compress_group_wave(const uint16_t* const (&r)[kGroup], const float* __restrict__ gamma,
                                    int first, const double* s_theta, float eps, uint16_t* out) {
  constexpr int H = DI / 2, NP = (H + 63) / 64;
  const int lane = threadIdx.x & 63;
  float u1[NP], u2[NP];
  float ss = 0.f;
#pragma unroll
  for (int m = 0; m < NP; ++m) {
    const int i = lane + 64 * m;
    u1[m] = u2[m] = 0.f;
    if (i < H) {
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int k = 0; k < kGroup; ++k) {
        s1 += bf16_to_f32(r[k][i]);
        s2 += bf16_to_f32(r[k][i + H]);
      }
      u1[m] = s1 * 0.25f;
      u2[m] = s2 * 0.25f;
      ss += u1[m] * u1[m] + u2[m] * u2[m];
    }
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / float(DI) + eps);
#pragma unroll
  for (int m = 0; m < NP; ++m) {
    const int i = lane + 64 * m;
    if (i < H) {
      const float v1 = u1[m] * inv * gamma[i], v2 = u2[m] * inv * gamma[i + H];
      float c, s;
      rot_cs(first, s_theta[i], c, s);
      out[i] = f32_to_bf16(v1 * c - v2 * s);
      out[i + H] = f32_to_bf16(v2 * c + v1 * s);
    }
  }
}

template <int DI>
__global__ __launch_bounds__(256) void qsa_trunk_groups_kernel(const uint16_t* __restrict__ raw,
                                                               const float* __restrict__ gamma,
                                                               uint16_t* __restrict__ gk, int T, int L, int ng,
                                                               double log2_base, float eps) {
  __shared__ double s_theta[DI / 2];
  fill_theta<DI>(s_theta, log2_base);
  __syncthreads();
  const long long gid = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);  // t * ng + g
  if (gid >= (long long)T * ng) return;                                  // whole waves
  const int t = int(gid / ng), g = int(gid - (long long)t * ng);
  const uint16_t* b0 = raw + (size_t(t) * L + size_t(kGroup) * g) * DI;
  const uint16_t* r[kGroup] = {b0, b0 + DI, b0 + 2 * DI, b0 + 3 * DI};
  compress_group_wave<DI>(r, gamma, kGroup * g, s_theta, eps, gk + size_t(gid) * DI);
}

__global__ void qsa_zero_kernel(int32_t* bad) { *bad = 0; }

// LDS row stride of the rotated queries: padded by 16 bytes so that the 32
// rows a matrix-core operand read touches spread over the banks.
template <int DI>
constexpr int qsa_sy_stride() { return DI + 8; }

template <int DI>
__global__ __launch_bounds__(256) void qsa_score_kernel(const QsaKArgs a) {
  constexpr int H = DI / 2, NS = DI / 16, SY = qsa_sy_stride<DI>(), SK = qsa_sy_stride<DI>();
  extern __shared__ __attribute__((aligned(16))) uint16_t qsa_smem[];
  __shared__ int s_par[64], s_pos[64];
  __shared__ unsigned char s_at[64][64];  // s_at[j][d]: j's ancestor at depth d (self at depth(j))
  __shared__ double s_theta[H];
  __shared__ int s_ok;

  const int tb = blockIdx.x / a.nsplit;  // t * B + b
  const int split = blockIdx.x - tb * a.nsplit;
  const int t = tb / a.B;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int Wn = a.Wn, Wp = (Wn + 31) & ~31;
  uint16_t* const sy = qsa_smem;          // [Wp][SY] rotated queries (zero rows past Wn)
  uint16_t* const sk = sy + Wp * SY;      // [Wn][DI] keys of the groups nodes complete
  uint16_t* const sk_tiles = sk + Wn * DI;  // [4 waves][32][SK] each wave's staged trunk tile
  const int anchor = a.anchors[tb];
  const size_t node0 = size_t(tb) * Wn;

  if (tid == 0) s_ok = (anchor >= 0 && anchor < a.L) ? 1 : 0;
  fill_theta<DI>(s_theta, a.log2_base);
  if (tid < Wn) {
    s_par[tid] = a.parent[node0 + tid];
    s_pos[tid] = a.pos[node0 + tid];
  }
  __syncthreads();
  if (tid < Wn) {
    // walk to the anchor; every step must go to an earlier node, so the walk ends
    int k = tid, d = 0;
    bool ok = true;
    for (;;) {
      const int p = s_par[k];
      if (p == -1) break;
      if (p < -1 || p >= k) {
        ok = false;
        break;
      }
      k = p;
      ++d;
    }
    if (ok) {
      k = tid;
      for (int dd = d; dd >= 0; --dd) {
        s_at[tid][dd] = (unsigned char)k;
        k = s_par[k];
      }
    }
    if (!ok || s_pos[tid] != anchor + 1 + d) s_ok = 0;
  }
  __syncthreads();
  if (!s_ok) {
    if (split != 0) return;  // the branch's first workgroup reports it
    if (tid == 0) atomicAdd(a.bad, 1);
    if (tid < Wn) a.ncand[node0 + tid] = -1;
    if (a.bkey)
      for (int e = tid; e < Wn * DI; e += 256) a.bkey[node0 * DI + e] = 0;
    return;
  }

  // rotated queries, bf16 (the operands the matrix cores see); zero rows pad
  // the last block of 32.  A thread takes 8 pairs (i, i + H) of one node,
  // read as two 16-byte loads.
  for (int e = tid; e < Wp * (H / 8); e += 256) {
    const int j = e / (H / 8), i0 = (e - j * (H / 8)) * 8;
    u32x4 w1 = {0u, 0u, 0u, 0u}, w2 = {0u, 0u, 0u, 0u};
    if (j < Wn) {
      const uint16_t* yr = a.y + (node0 + j) * DI;
      const u32x4 v1 = *reinterpret_cast<const u32x4*>(yr + i0);
      const u32x4 v2 = *reinterpret_cast<const u32x4*>(yr + i0 + H);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float c0, s0, c1, s1;
        rot_cs(s_pos[j], s_theta[i0 + 2 * q], c0, s0);
        rot_cs(s_pos[j], s_theta[i0 + 2 * q + 1], c1, s1);
        const float a0 = bf16_lo(v1[q]), a1 = bf16_hi(v1[q]), b0 = bf16_lo(v2[q]), b1 = bf16_hi(v2[q]);
        w1[q] = pack_bf16x2(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
        w2[q] = pack_bf16x2(b0 * c0 + a0 * s0, b1 * c1 + a1 * s1);
      }
    }
    *reinterpret_cast<u32x4*>(sy + j * SY + i0) = w1;
    *reinterpret_cast<u32x4*>(sy + j * SY + i0 + H) = w2;
  }
  // keys of the groups the nodes complete: the four tokens ending at the
  // node along its own path, trunk tokens up to the anchor for the boundary
  // group (the branch's raw slots); the branch's first workgroup scores the
  // branch's own groups, the others only trunk groups
  for (int j = wave; j < Wn && split == 0; j += 4) {
    const int p = s_pos[j];
    if ((p & 3) != 3) continue;
    const uint16_t* r[kGroup];
#pragma unroll
    for (int m = 0; m < kGroup; ++m) {
      const int q = p - 3 + m;
      r[m] = q > anchor ? a.x + (node0 + s_at[j][q - anchor - 1]) * DI
                        : a.trunk_raw + (size_t(t) * a.L + q) * DI;
    }
    compress_group_wave<DI>(r, a.gamma, p - 3, s_theta, a.eps, sk + j * DI);
  }
  __syncthreads();
  if (a.bkey && split == 0)
    for (int e = tid; e < Wn * DI; e += 256) {
      const int j = e / DI;
      a.bkey[node0 * DI + e] = (s_pos[j] & 3) == 3 ? sk[e] : (uint16_t)0;
    }

  // cached trunk groups g < gT on the matrix cores: S^T[group][node] =
  // K[group][:] . Y[node][:]; lane (r, h) holds node r's scores for groups
  // 8(i/4) + 4h + i%4 of the tile
  const int gT = (anchor + 1) >> 2;
  const int ntile = (gT + 31) >> 5;
  const int nb = Wp >> 5;
  const int h = lane >> 5, r32 = lane & 31;
  float* const sc0 = a.sc + node0 * size_t(a.Gs);
  if (ntile > 0) {
    bf16x8 qop[2][NS];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int s = 0; s < NS; ++s)
        qop[rb][s] = rb < nb ? *reinterpret_cast<const bf16x8*>(sy + (rb * 32 + r32) * SY + 16 * s + 8 * h)
                             : bf16x8{};
    const uint16_t* gkt = a.trunk_gk + size_t(t) * a.ng * DI;
    // tiles split + nsplit * (wave + 4 m).  A tile's 32 group keys are read
    // with whole-row loads (DI / 8 lanes per key row, so a wave load covers
    // 512 / DI complete rows) into registers, written to this wave's LDS
    // block, and read back in operand layout; the next tile's rows are in
    // flight while the current one is multiplied.  Waves run different tile
    // counts, so the block is private to the wave and only the wave's own
    // LDS accesses are ordered (lgkmcnt waits), never a workgroup barrier.
    constexpr int LPR = DI / 8, RPL = 64 / LPR, NLD = 32 / RPL;  // lanes per row, rows per load, loads
    uint16_t* const kw = sk_tiles + wave * (32 * SK);
    const int lrow = lane / LPR, lcol = (lane % LPR) * 8;
    u32x4 kreg[NLD];
    auto gload = [&](int tt) {
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int g = min(tt * 32 + j * RPL + lrow, a.ng - 1);  // gT <= ng, so ng >= 1 here
        kreg[j] = *reinterpret_cast<const u32x4*>(gkt + size_t(g) * DI + lcol);
      }
    };
    const int tstep = 4 * a.nsplit;
    int tt = split + a.nsplit * wave;
    if (tt < ntile) gload(tt);
    for (; tt < ntile; tt += tstep) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the previous tile's operand reads are done
#pragma unroll
      for (int j = 0; j < NLD; ++j) *reinterpret_cast<u32x4*>(kw + (j * RPL + lrow) * SK + lcol) = kreg[j];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (tt + tstep < ntile) gload(tt + tstep);
      bf16x8 kop[NS];
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) kop[s2] = *reinterpret_cast<const bf16x8*>(kw + r32 * SK + 16 * s2 + 8 * h);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        if (rb >= nb) break;
        f32x16 acc = {};
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[s2], qop[rb][s2], acc, 0, 0, 0);
        const int row = rb * 32 + r32;
        if (row < Wn) {
          float* dst = sc0 + size_t(row) * a.Gs;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int g0 = tt * 32 + 8 * q4 + 4 * h;
            if (g0 + 3 < gT) {
              *reinterpret_cast<f32x4*>(dst + g0) = f32x4{acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (g0 + e < gT) dst[g0 + e] = acc[4 * q4 + e];
            }
          }
        }
      }
    }
  }
  // the branch's own groups g in [gT, G_j): the key the ancestor at position
  // 4g + 3 completed
  if (split != 0) return;
  const int maxnb = (Wn + 3) / 4 + 1;
  for (int it = wave; it < Wn * maxnb; it += 4) {
    const int j = it / maxnb, g = gT + (it - j * maxnb);
    if (g >= ((s_pos[j] + 1) >> 2)) continue;
    const int node = s_at[j][4 * g + 3 - anchor - 1];
    float acc = 0.f;
    for (int e = lane; e < DI; e += 64) acc += bf16_to_f32(sy[j * SY + e]) * bf16_to_f32(sk[node * DI + e]);
    acc = wave_sum(acc);
    if (lane == 0) sc0[size_t(j) * a.Gs + g] = acc;
  }
  if (tid < Wn) a.ncand[node0 + tid] = (s_pos[tid] + 1) >> 2;
}

// fp32 -> unsigned key with the same order (-0 taken as +0), and back
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

__global__ __launch_bounds__(256) void qsa_topk_kernel(const QsaKArgs a) {
  extern __shared__ uint32_t qsa_keys[];  // [Gs]
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_cnt[2][4];
  __shared__ uint32_t s_dig, s_rem, s_all;
  const size_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = a.topk;
  int32_t* const so = a.sel + row * size_t(k);
  float* const vo = a.score + row * size_t(k);
  const int n = a.ncand[row];
  const float* const sc = a.sc + row * size_t(a.Gs);
  if (n < 0) {
    for (int i = tid; i < k; i += 256) {
      so[i] = -1;
      vo[i] = __builtin_nanf("");
    }
    return;
  }
  if (n <= k) {
    for (int i = tid; i < k; i += 256) {
      if (i < n) {
        so[i] = i;
        vo[i] = sc[i];
      } else {
        so[i] = -1;
        vo[i] = kNegInf;
      }
    }
    return;
  }
  constexpr int kLoadBatch = 8;  // loads in flight per thread
  for (int i0 = tid; i0 < n; i0 += 256 * kLoadBatch) {
    float v[kLoadBatch];
#pragma unroll
    for (int e = 0; e < kLoadBatch; ++e) {
      const int i = i0 + 256 * e;
      v[e] = i < n ? sc[i] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < kLoadBatch; ++e) {
      const int i = i0 + 256 * e;
      if (i < n) qsa_keys[i] = order_key(v[e]);
    }
  }
  // the k-th largest key, 8 bits at a time from the top; when every key of
  // the bin that holds it is kept, its lower bits do not matter and the
  // passes stop
  uint32_t prefix = 0u, pmask = 0u, rem = uint32_t(k);
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const uint32_t u = qsa_keys[i];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t c[4], s = 0u;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        c[b] = hist[4 * lane + b];
        s += c[b];
      }
      uint32_t v = s;  // count in lanes >= this one
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t w = __shfl_down(v, o, 64);
        if (lane + o < 64) v += w;
      }
      uint32_t cum = v - s;  // count in higher bins
#pragma unroll
      for (int b = 3; b >= 0; --b) {
        if (cum < rem && rem <= cum + c[b]) {
          s_dig = uint32_t(4 * lane + b);
          s_rem = rem - cum;
          s_all = rem == cum + c[b];
        }
        cum += c[b];
      }
    }
    __syncthreads();
    prefix |= s_dig << shift;
    pmask |= 0xffu << shift;
    rem = s_rem;
    if (s_all) break;
  }
  // keys whose resolved bits are above prefix, then the first `rem` keys
  // whose resolved bits equal it, in group order: k in all
  uint32_t gt_seen = 0u, eq_seen = 0u;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < n; c0 += 256) {
    const int i = c0 + tid;
    const uint32_t u = i < n ? qsa_keys[i] : 0u;
    const uint32_t um = u & pmask;
    const bool gt = i < n && um > prefix, eq = i < n && um == prefix;
    const unsigned long long bg = __ballot(gt), be = __ballot(eq);
    if (lane == 0) {
      s_cnt[0][wave] = uint32_t(__popcll(bg));
      s_cnt[1][wave] = uint32_t(__popcll(be));
    }
    __syncthreads();
    uint32_t og = 0u, oe = 0u, tg = 0u, te = 0u;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w < wave) {
        og += s_cnt[0][w];
        oe += s_cnt[1][w];
      }
      tg += s_cnt[0][w];
      te += s_cnt[1][w];
    }
    const uint32_t gb = gt_seen + og + uint32_t(__popcll(bg & below));
    const uint32_t eb = eq_seen + oe + uint32_t(__popcll(be & below));
    if (gt || (eq && eb < rem)) {
      // below k by construction; the bound keeps a row's writes in its own
      // k slots whatever the keys
      const uint32_t o = min(gb + (eb < rem ? eb : rem), uint32_t(k - 1));
      so[o] = i;
      vo[o] = key_value(u);
    }
    gt_seen += tg;
    eq_seen += te;
    __syncthreads();
  }
}

// Statically declared LDS of the two kernels (bytes), for the dynamic limit.
constexpr size_t kScoreStaticLds = 6656;   // s_par, s_pos, s_at, s_theta, s_ok (<= 5,648 bytes as built) and room
constexpr size_t kTopkStaticLds = 1536;    // hist, s_cnt, s_dig, s_rem (1,064 bytes as built) and room

// Raises a kernel's dynamic LDS limit when static + dynamic LDS passes the
// 64 KiB a workgroup gets without asking (gfx950 has 160 KiB per CU).
hipError_t allow_lds(const void* kernel, size_t dyn, size_t stat) {
  if (dyn + stat <= 65536) return hipSuccess;
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, int(dyn));
}

template <int DI>
size_t score_lds_bytes(int Wn) {
  const int Wp = (Wn + 31) & ~31;
  return size_t(Wp) * qsa_sy_stride<DI>() * 2 + size_t(Wn) * DI * 2 + size_t(4 * 32) * qsa_sy_stride<DI>() * 2;
}

template <int DI>
hipError_t launch_select_di(const specopd_qsa_desc& d, const QsaKArgs& k, hipStream_t s) {
  const size_t lds = score_lds_bytes<DI>(d.Wn);
  hipError_t e = allow_lds(reinterpret_cast<const void*>(&qsa_score_kernel<DI>), lds, kScoreStaticLds);
  if (e != hipSuccess) return e;
  timing_mark(5, 0, s);
  qsa_score_kernel<DI><<<dim3(unsigned(size_t(d.T) * d.B * k.nsplit)), 256, lds, s>>>(k);
  timing_mark(5, 1, s);
  return hipGetLastError();
}

}  // namespace

QsaWs qsa_ws_layout(const specopd_qsa_desc& d) {
  QsaWs w{};
  const size_t rows = size_t(d.T) * d.B * d.Wn;
  w.Gs = int(align_up(size_t(std::max(1, (d.L + d.Wn) / kGroup)), 4));
  w.bad = 0;
  w.ncand = 256;
  w.sc = align_up(w.ncand + rows * 4, 256);
  w.total = align_up(w.sc + rows * size_t(w.Gs) * 4, 256);
  return w;
}

hipError_t launch_qsa_trunk_groups(const specopd_qsa_desc& d, const void* raw, const float* gamma, void* gk,
                                   hipStream_t s) {
  const int ng = d.L / kGroup;
  const long long groups = (long long)d.T * ng;
  if (groups == 0) return hipSuccess;
  const dim3 grid(unsigned((groups + 3) / 4));
  const double lb = log2(double(d.rope_base > 0.f ? d.rope_base : 10000.f));
  const float eps = d.eps > 0.f ? d.eps : 1e-6f;
  const uint16_t* r = static_cast<const uint16_t*>(raw);
  uint16_t* o = static_cast<uint16_t*>(gk);
  if (d.Di == 64) qsa_trunk_groups_kernel<64><<<grid, 256, 0, s>>>(r, gamma, o, d.T, d.L, ng, lb, eps);
  else if (d.Di == 128) qsa_trunk_groups_kernel<128><<<grid, 256, 0, s>>>(r, gamma, o, d.T, d.L, ng, lb, eps);
  else qsa_trunk_groups_kernel<256><<<grid, 256, 0, s>>>(r, gamma, o, d.T, d.L, ng, lb, eps);
  return hipGetLastError();
}

hipError_t launch_qsa_select(const specopd_qsa_desc& d, const QsaCallArgs& a, hipStream_t s) {
  const QsaWs w = qsa_ws_layout(d);
  QsaKArgs k{};
  k.trunk_gk = static_cast<const uint16_t*>(a.trunk_gk);
  k.trunk_raw = static_cast<const uint16_t*>(a.trunk_raw);
  k.x = static_cast<const uint16_t*>(a.x);
  k.y = static_cast<const uint16_t*>(a.y);
  k.gamma = a.gamma;
  k.anchors = a.anchors;
  k.parent = a.parent;
  k.pos = a.pos;
  k.sel = a.sel;
  k.score = a.score;
  k.bkey = static_cast<uint16_t*>(a.bkey);
  k.bad = reinterpret_cast<int32_t*>(a.ws + w.bad);
  k.ncand = reinterpret_cast<int32_t*>(a.ws + w.ncand);
  k.sc = reinterpret_cast<float*>(a.ws + w.sc);
  k.L = d.L;
  k.B = d.B;
  k.Wn = d.Wn;
  k.ng = d.L / kGroup;
  k.Gs = w.Gs;
  k.topk = d.topk;
  // enough workgroups to fill the GPU several times over: the longest
  // branch's trunk tiles, not the branch count, set the kernel's length
  {
    const long long br = (long long)d.T * d.B;
    k.nsplit = int(std::min<long long>(8, std::max<long long>(1, (kQsaScoreWgs + br - 1) / br)));
  }
  k.log2_base = log2(double(d.rope_base > 0.f ? d.rope_base : 10000.f));
  k.eps = d.eps > 0.f ? d.eps : 1e-6f;
  qsa_zero_kernel<<<1, 1, 0, s>>>(k.bad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (d.Di == 64) e = launch_select_di<64>(d, k, s);
  else if (d.Di == 128) e = launch_select_di<128>(d, k, s);
  else e = launch_select_di<256>(d, k, s);
  if (e != hipSuccess) return e;
  const size_t rows = size_t(d.T) * d.B * d.Wn;
  e = allow_lds(reinterpret_cast<const void*>(&qsa_topk_kernel), size_t(w.Gs) * 4, kTopkStaticLds);
  if (e != hipSuccess) return e;
  timing_mark(6, 0, s);
  qsa_topk_kernel<<<dim3(unsigned(rows)), 256, size_t(w.Gs) * 4, s>>>(k);
  timing_mark(6, 1, s);
  return hipGetLastError();
}

}  // namespace specopd
