// Tree-masked GQA attention on the gfx950 matrix cores (bf16 in, fp32
// accumulate).
//
// What is computed (jaehun.me review of SpecOPD, §3.2(a), Eq. 5): every node
// j of branch b attends to trunk keys 0..a_b of the shared prefilled cache
// and to the nodes on its own parent chain; rotary embedding at the node's
// semantic position has already been applied to its query/key by
// rope_branch_kernel (queries also carry scale * log2(e), so scores come out
// of the matrix cores in log2 units).
//
// Work unit = (trunk t, kv head g, pack of branches).  Branches of a trunk are
// sorted by anchor (longest first) and consecutive ones are packed so that
// the pack's rows (node x query head of the kv group) fill the workgroup.  All
// rows of a pack share trunk keys 0..max anchor, so one K/V tile feeds every
// row; rows whose anchor is shorter mask the tail of the last tiles.  The
// branches' own nodes form extra "tail" tiles masked by the ancestor bitmask
// and by branch identity.
//
// Wave layout (8 waves, two per SIMD so one wave's softmax overlaps the
// other's matrix work): KS key slices x (8/KS) row groups.  A row group is NB
// blocks of 32 rows (one wave).  Waves of the same slice share one
// double-buffered K/V tile in LDS; waves of different slices take interleaved
// tiles and are merged at the end through LDS in a fixed order
// (deterministic).
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16, lane l = r + 32h):
//   S^T[key][row] = K[key][:] . Q[row][:]      A = K tile (LDS, 16 B reads),
//                                              B = Q^T (registers)
//   lane (r, h) holds row r's scores for keys 8(i/4) + 4h + i%4, i = 0..15,
//   which is exactly the B operand P^T of the second product for k-steps of
//   16 keys (elements 8s..8s+7 -> keys 16s + 8(e/4) + 4h + e%4), so P never
//   leaves registers;
//   O^T[dim][row] += V^T[dim][key] . P^T[key][row]
//                                              A = V^T read from the row-major
//                                              V tile with ds_read_b64_tr_b16
//                                              (each 16-lane group turns four
//                                              4-element rows into columns).
// Softmax is online in log2 units with a lazily moved reference maximum: the
// accumulators are rescaled only when a row's maximum grows by more than
// 2^8, so the common tile costs no rescale.
#include "device_common.h"
#include "internal.h"

namespace specopd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int KT = 32;            // keys per tile
constexpr float kRescale = 8.0f;  // log2 headroom before the reference max moves
constexpr float kFarNeg = -1.0e30f;

// Waves per workgroup: 8 (two per SIMD) where a wave fits in 256 registers;
// 4 for D = 256, whose accumulators and query operand need more.
template <int D>
constexpr int waves_for() { return D == 256 ? 4 : 8; }

template <int D, int NB, int KS>
struct Shape {
  static constexpr int NW = waves_for<D>();
  static constexpr int RG = NW / KS;         // row groups per workgroup
  static constexpr int ROWS_G = 32 * NB;     // rows per row group (one wave)
  static constexpr int RW = RG * ROWS_G;     // rows per workgroup
  static constexpr int LDK = D + 8;          // LDS row stride (elements); +16 B spreads banks
  static constexpr int TILE = KT * LDK;      // elements of one K (or V) tile
  static constexpr int SLICE = 2 * 2 * TILE; // double-buffered K and V
  static constexpr int TILES_BYTES = KS * SLICE * 2;
  static constexpr int OREGS = NB * D / 2;   // fp32 accumulator registers per lane
  static constexpr int COMB_WORDS = (KS > 1) ? (KS - 1) * RG * (OREGS + 2 * NB) * 64 : 0;
  static constexpr int LDS_BYTES = TILES_BYTES > COMB_WORDS * 4 ? TILES_BYTES : COMB_WORDS * 4;
  static constexpr int CHUNKS = 2 * KT * D / 8;  // 16-byte pieces of a K+V tile
  // threads filling one slice's tile (capped so every loader has a K and a V piece)
  static constexpr int LOADERS = 64 * RG < CHUNKS / 2 ? 64 * RG : CHUNKS / 2;
  static constexpr int CPT = CHUNKS / LOADERS;   // pieces per loader (first half K)
  static_assert(CHUNKS % LOADERS == 0 && CPT % 2 == 0, "tile must split evenly over loaders");
};

__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

// Visible tail keys of a row within tail tile [tau0, tau0 + 32): the row's own
// branch occupies tail keys slot*Wn .. slot*Wn + Wn - 1 and it sees the nodes
// set in its ancestor mask.  Bit q of the result = tail key tau0 + q.
__device__ __forceinline__ uint32_t tail_window(uint64_t anc, int slot, int Wn, int tau0) {
  const int base = slot * Wn - tau0;  // tile position of the row's node 0
  if (anc == 0 || base >= KT || base <= -64) return 0u;
  const uint64_t w = base >= 0 ? (anc << base) : (anc >> (-base));
  return uint32_t(w);
}

template <int D, int NB, int KS>
__global__ __launch_bounds__(waves_for<D>() * 64, 1) void tree_attn_mfma_kernel(const MfmaParams p) {
  using S = Shape<D, NB, KS>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::LDS_BYTES / 2];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int slice = wave % KS, rgrp = wave / KS;
  const int h = lane >> 5, r32 = lane & 31;

  // XCD-aware unit order: workgroups are dealt to the 8 XCDs round robin, so
  // consecutive units (same trunk and kv head, hence same K/V) land on one XCD.
  const int bid = blockIdx.x;
  const int u = (bid & 7) * p.per + (bid >> 3);
  if (u >= p.nunits) return;
  const int pk = u % p.npacks;
  const int tg = u / p.npacks;
  const int g = tg % p.Hkv, t = tg / p.Hkv;
  const int rows_per_branch = p.Wn * p.G;
  const size_t tB = size_t(t) * p.B;
  const int32_t* ord = p.order + tB;
  const int b0 = pk * p.bpp;
  const int nbr = min(p.bpp, p.B - b0);

  int amax = -1, amin = 0x7fffffff;
  for (int i = 0; i < nbr; ++i) {
    const int b = ord[b0 + i];
    const int a = p.branch_ok[tB + b] ? p.anchors[tB + b] : -1;
    amax = max(amax, a);
    amin = min(amin, a);
  }

  // ---- this lane's rows: metadata and the Q^T operand
  int ra[NB], rslot[NB];
  uint64_t rmask[NB];
  bf16x8 qop[NB][D / 16];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int rho = rgrp * S::ROWS_G + nb * 32 + r32;
    const int slot = rho / rows_per_branch;
    const int within = rho - slot * rows_per_branch;
    const int j = within / p.G;
    const int hh = within - j * p.G;
    const bool exists = slot < nbr;
    const int b = exists ? ord[b0 + slot] : 0;
    const bool ok = exists && p.branch_ok[tB + b];
    ra[nb] = ok ? p.anchors[tB + b] : -1;
    rslot[nb] = slot;
    rmask[nb] = ok ? p.anc[(tB + b) * p.Wn + j] : 0ull;
    const uint16_t* qrow = p.qr + ((((tB + b) * p.Wn + j) * p.Hq) + size_t(g) * p.G + hh) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qop[nb][s] = ok ? *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * h) : bf16x8{};
  }

  const int ntrunk = (amax + 1 + KT - 1) / KT;
  const int nt_total = nbr * p.Wn;
  const int ntail = (nt_total + KT - 1) / KT;
  const int nvt = ntrunk + ntail;
  const int iters = (nvt + KS - 1) / KS;

  // ---- tile staging (global -> registers -> LDS), two tiles ahead.  Piece c
  // of a loader: the first CPT/2 are K, the rest V (compile-time split).
  uint16_t* sbase = smem + slice * S::SLICE;
  const int li = rgrp * 64 + lane;
  constexpr int HALF = S::CPT / 2;
  u32x4 stage[S::CPT];
  auto load_tile = [&](int vt) {
    const bool trunk = vt < ntrunk;
    if (li >= S::LOADERS) return;
#pragma unroll
    for (int c = 0; c < S::CPT; ++c) {
      const int rem = li + (c % HALF) * S::LOADERS;
      const int key = rem / (D / 8);
      const int part = rem - key * (D / 8);
      size_t row;
      if (trunk) {
        row = (size_t(t) * p.L + min(vt * KT + key, p.L - 1)) * p.Hkv + g;
      } else {
        int tau = (vt - ntrunk) * KT + key;
        if (tau >= nt_total) tau = 0;
        const int sl = tau / p.Wn;
        const int node = tau - sl * p.Wn;
        row = ((tB + size_t(ord[b0 + sl])) * p.Wn + node) * p.Hkv + g;
      }
      const uint16_t* base = c < HALF ? (trunk ? p.trunk_k : p.kr) : (trunk ? p.trunk_v : p.v);
      stage[c] = *reinterpret_cast<const u32x4*>(base + row * D + part * 8);
    }
  };
  auto store_tile = [&](int buf) {
    if (li >= S::LOADERS) return;
#pragma unroll
    for (int c = 0; c < S::CPT; ++c) {
      const int rem = li + (c % HALF) * S::LOADERS;
      const int key = rem / (D / 8);
      const int part = rem - key * (D / 8);
      *reinterpret_cast<u32x4*>(sbase + (buf * 2 + c / HALF) * S::TILE + key * S::LDK + part * 8) =
          stage[c];
    }
  };

  // ---- accumulators
  f32x16 oacc[NB][D / 32];
  float mref[NB], lsum[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    mref[nb] = kFarNeg;
    lsum[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[nb][db] = f32x16{};
  }

  if (slice < nvt) {
    load_tile(slice);
    store_tile(0);
  }
  if (KS + slice < nvt) load_tile(KS + slice);
  __syncthreads();

  const int gi = lane >> 4, rq = lane & 15;
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  for (int it = 0; it < iters; ++it) {
    const int vt = it * KS + slice;
    const int buf = it & 1;
    if (vt < nvt) {
      const uint16_t* Kt = sbase + (buf * 2) * S::TILE;
      const uint16_t* Vt = Kt + S::TILE;
      f32x16 sacc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sacc[nb] = f32x16{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(Kt + r32 * S::LDK + 16 * s + 8 * h);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[nb][s], sacc[nb], 0, 0, 0);
      }
      // masks: trunk keys beyond a row's anchor (edge tiles only); tail keys
      // of other branches or outside the row's ancestor chain
      if (vt < ntrunk) {
        const int k0 = vt * KT;
        if (k0 + KT - 1 > amin) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int lim = ra[nb] - k0 - 4 * h;  // element i visible iff 8(i/4)+(i%4) <= lim
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (8 * (i >> 2) + (i & 3) > lim) sacc[nb][i] = kNegInf;
          }
        }
      } else {
        const int tau0 = (vt - ntrunk) * KT;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint32_t vis = tail_window(rmask[nb], rslot[nb], p.Wn, tau0) >> (4 * h);
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (!((vis >> (8 * (i >> 2) + (i & 3))) & 1u)) sacc[nb][i] = kNegInf;
        }
      }
      // online softmax (log2 units), lazily rescaled
      bool need[NB];
      bool any = false;
      float mt[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float m = sacc[nb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) m = fmaxf(m, sacc[nb][i]);
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        mt[nb] = m;
        need[nb] = m > mref[nb] + kRescale;
        any |= need[nb];
      }
      if (__any(any)) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const float alpha = need[nb] ? fast_exp2(mref[nb] - mt[nb]) : 1.0f;
          mref[nb] = need[nb] ? mt[nb] : mref[nb];
          lsum[nb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) oacc[nb][db] *= alpha;
        }
      }
      bf16x8 pop[NB][2];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float ps = lsum[nb];
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const bf16x2 e2 = {static_cast<__bf16>(fast_exp2(sacc[nb][i] - mref[nb])),
                             static_cast<__bf16>(fast_exp2(sacc[nb][i + 1] - mref[nb]))};
          pop[nb][i >> 3][i & 7] = e2[0];
          pop[nb][i >> 3][(i & 7) + 1] = e2[1];
          ps = __builtin_amdgcn_fdot2_f32_bf16(e2, ones, ps, false);  // sums the bf16 weights used below
        }
        lsum[nb] = ps;
      }
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const uint16_t* vb = Vt + (16 * s2 + 4 * (gi >> 1) + (rq >> 2)) * S::LDK + 32 * db +
                               16 * (gi & 1) + 4 * (rq & 3);
          const s16x4 va = lds_read_tr(vb);
          const s16x4 vc = lds_read_tr(vb + 8 * S::LDK);
          const bf16x8 vop = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(va, vc, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            oacc[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[nb][s2], oacc[nb][db], 0, 0, 0);
        }
      }
    }
    if (it + 1 < iters) {
      if (vt + KS < nvt) store_tile(buf ^ 1);
      if (vt + 2 * KS < nvt) load_tile(vt + 2 * KS);
    }
    __syncthreads();
  }

  // ---- merge key slices (fixed order), then normalise and write
  if constexpr (KS > 1) {
    float* comb = reinterpret_cast<float*>(smem);
    constexpr int PER = S::OREGS + 2 * NB;  // O registers, then (m, l), per row block
    if (slice > 0) {
      float* dst = comb + size_t((rgrp * (KS - 1) + (slice - 1)) * PER) * 64;
      int k = 0;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) dst[(k++) * 64 + lane] = oacc[nb][db][i];
        dst[(k++) * 64 + lane] = mref[nb];
        dst[(k++) * 64 + lane] = lsum[nb];
      }
    }
    __syncthreads();
    if (slice == 0) {
#pragma unroll 1
      for (int o = 1; o < KS; ++o) {
        const float* src = comb + size_t((rgrp * (KS - 1) + (o - 1)) * PER) * 64;
        int k = 0;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int kb = k;
          k += S::OREGS / NB;
          const float m2 = src[(k++) * 64 + lane];
          const float l2 = src[(k++) * 64 + lane];
          const float mn = fmaxf(mref[nb], m2);
          const float a0 = fast_exp2(mref[nb] - mn), a1 = fast_exp2(m2 - mn);
          int kk = kb;
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              oacc[nb][db][i] = oacc[nb][db][i] * a0 + src[(kk++) * 64 + lane] * a1;
          lsum[nb] = lsum[nb] * a0 + l2 * a1;
          mref[nb] = mn;
        }
      }
    }
  }
  if (slice != 0) return;

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float lt = lsum[nb] + __shfl_xor(lsum[nb], 32, 64);
    const int rho = rgrp * S::ROWS_G + nb * 32 + r32;
    const int slot = rho / rows_per_branch;
    if (slot >= nbr) continue;
    const int within = rho - slot * rows_per_branch;
    const int j = within / p.G;
    const int hh = within - j * p.G;
    const size_t b = size_t(ord[b0 + slot]);
    const bool ok = p.branch_ok[tB + b] != 0;
    const float inv = ok ? 1.0f / lt : __builtin_nanf("");
    uint16_t* orow = p.out + ((((tB + b) * p.Wn + j) * p.Hq) + size_t(g) * p.G + hh) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int dim = 32 * db + 8 * q + 4 * h;
        const f32x16& o = oacc[nb][db];
        u32x2 w = {pack_bf16x2(o[4 * q] * inv, o[4 * q + 1] * inv),
                   pack_bf16x2(o[4 * q + 2] * inv, o[4 * q + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + dim) = w;
      }
  }
}

template <int D, int NB, int KS>
hipError_t launch_shape(const MfmaParams& p, hipStream_t s) {
  tree_attn_mfma_kernel<D, NB, KS><<<8 * p.per, waves_for<D>() * 64, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace

int mfma_rows_per_wg(int D, int KS) {
  const int NB = D == 64 ? 2 : 1;
  const int nw = D == 256 ? waves_for<256>() : waves_for<128>();
  return (nw / KS) * 32 * NB;
}

hipError_t launch_tree_attn_mfma(int D, int KS, const MfmaParams& p, hipStream_t s) {
  switch (D) {
    case 64:
      return KS == 1 ? launch_shape<64, 2, 1>(p, s)
                     : KS == 2 ? launch_shape<64, 2, 2>(p, s) : launch_shape<64, 2, 4>(p, s);
    case 128:
      return KS == 1 ? launch_shape<128, 1, 1>(p, s)
                     : KS == 2 ? launch_shape<128, 1, 2>(p, s) : launch_shape<128, 1, 4>(p, s);
    case 256:
      return KS == 1 ? launch_shape<256, 1, 1>(p, s) : launch_shape<256, 1, 2>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace specopd
