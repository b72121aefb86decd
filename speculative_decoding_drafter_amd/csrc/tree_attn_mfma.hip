// Tree-masked GQA attention on the gfx950 matrix cores (bf16 in, fp32
// accumulate).
//
// What is computed (jaehun.me review of SpecOPD, §3.2(a), Eq. 5): every node
// j of branch b attends to trunk keys 0..a_b of the shared prefilled cache
// and to the nodes on its own parent chain.  Rotary embedding at the node's
// semantic position has already been applied to its query and key by the
// preparation kernel; queries also carry scale * log2(e), so scores come out
// of the matrix cores in log2 units.
//
// Packs.  Branches of a trunk are sorted by anchor (longest first) and
// consecutive ones are packed so that the pack's rows (node x query head of
// one kv group) fill a workgroup.  All rows of a pack share trunk keys
// 0..max anchor, so one K/V tile feeds every row; rows whose anchor is shorter
// mask the tail of the last tiles.  The branches' own nodes form extra "tail"
// tiles masked by the ancestor bitmask and by branch identity.  A pack's key
// tiles (trunk tiles, then tail tiles) are its units of work.
//
// Work split.  A workgroup takes one pack, or one key range of a pack when
// there are too few packs to fill the chip; packs get key ranges in
// proportion to their key tiles (at least one each), so ranges are of like
// length.  A split pack leaves partial results (unnormalised output in bf16,
// running max and sum in fp32) in the workspace, exchanged with device-scope
// accesses; the workgroup that finishes last merges them in range order, so
// the result does not depend on timing.  Packs of one kv head are
// consecutive units and run side by side on one XCD, reading the same trunk
// tiles at about the same time, so the trunk is fetched into that XCD's L2
// about once.  The trunk prefill launches this same kernel (under a second
// name) on one-node branches, one per trunk token.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16, lane l = r + 32h):
//   S^T[key][row] = K[key][:] . Q[row][:]      A = K tile (LDS, 16-byte
//                                              reads), B = Q^T (registers)
//   lane (r, h) holds row r's scores for keys 8(i/4) + 4h + i%4, i = 0..15,
//   which is exactly the B operand P^T of the second product for k-steps of
//   16 keys, so P never leaves registers;
//   O^T[dim][row] += V^T[dim][key] . P^T[key][row]
//                                              A = V^T read from the row-major
//                                              V tile with ds_read_b64_tr_b16.
// LDS rows are padded (K by 16 bytes, V by 32) so that both read patterns hit
// distinct banks of the 64-bank LDS.
//
// Pipeline per wave (four waves, one per SIMD, each owning 64 rows for head
// sizes up to 128, so that every K and V operand read from LDS feeds two
// products): the score product of tile i + 1 is issued step by step together
// with the exponentials of tile i, the LDS reads of tile i's V operands and
// the wave's loads of a later tile; the products with V of tile i follow,
// at whose start the K operands of tile i + 2 are read.  Tiles go from
// global memory straight into LDS (each lane of a wave-wide load writes 16
// bytes at base + 16 * lane), through six LDS buffers (four for head size
// 256), one barrier per tile.  Lanes whose 16 bytes land on a row's pad
// chunk load a harmless in-bounds chunk that is never read.  Tiles that need
// no mask for any row of the wave run through a branch-free copy of the
// step; the last tiles of a unit (edge and tail tiles) through a second copy
// that masks the scores it forms inside the step.
//
// Softmax is online in log2 units.  The score product starts from -m (m the
// row's reference maximum), so scores arrive already shifted; the reference
// moves only when a score exceeds it by more than 2^8, so the common tile
// costs no rescale.
#include "device_common.h"
#include "internal.h"

namespace specopd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const char lds_cchar;

namespace {

constexpr int KT = 32;            // keys per tile
constexpr int kMergeBatch = 4;    // split partials loaded per merge round trip
constexpr float kRescale = 8.0f;  // log2 headroom before the reference max moves
constexpr float kUnset = -3.0e38f;

template <int D>
struct Geo {
  static constexpr int NW = mfma_waves(D);       // waves per workgroup
  static constexpr int NB = mfma_row_blocks(D);  // 32-row blocks per wave
  static constexpr int OREG = D / 32;            // 16-register accumulator blocks per row block
  static constexpr int CH = D / 8;               // 16-byte chunks of a key row
  static constexpr int KROW = 2 * D + 16;        // LDS bytes per K row (one pad chunk)
  static constexpr int VROW = 2 * D + 32;        // LDS bytes per V row (two pad chunks)
  static constexpr int SK = KROW / 16, SV = VROW / 16;
  static constexpr int KBYTES = KT * KROW;
  // the V rows start on a 1 KB boundary, so each wave-wide 1 KB write of a
  // tile is all K or all V (one source tensor per load instruction)
  static constexpr int VBASE = (KBYTES + 1023) / 1024 * 1024;
  static constexpr int NJ = (VBASE + KT * VROW + 1023) / 1024;  // 1 KB writes a tile needs
  static constexpr int JPW = (NJ + NW - 1) / NW; // wave writes per tile (every wave the same)
  static constexpr int BUFB = JPW * NW * 1024;   // bytes of one staged K+V tile, with slack
  // staged tiles: up to six where they fit in LDS, at least four.  With
  // five or more, the K operands of a tile are read one tile early.
  static constexpr int NBUF = (6 * BUFB + 16 <= 160 * 1024) ? 6 : (5 * BUFB + 16 <= 160 * 1024) ? 5 : 4;
  static constexpr bool EARLYK = NBUF >= 5;
  // tiles ahead of the accumulated one that must be readable after a
  // tile's barrier, and tiles whose loads may stay in flight across it
  static constexpr int NEED = EARLYK ? 3 : 2;
  static constexpr int INFL = NBUF - 1 - NEED;
};

// Visible tail keys of a row within tail tile [tau0, tau0 + 32): the row's own
// branch occupies tail keys slot*ts .. slot*ts + Wn - 1 and it sees the nodes
// set in its ancestor mask.  Bit q of the result = tail key tau0 + q.
__device__ __forceinline__ uint32_t tail_window(uint64_t anc, int slot, int ts, int tau0) {
  const int base = slot * ts - tau0;  // tile position of the row's node 0
  if (anc == 0 || base >= KT || base <= -64) return 0u;
  const uint64_t w = base >= 0 ? (anc << base) : (anc >> (-base));
  return uint32_t(w);
}

// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait until at most k tiles' loads (JPW each) of this wave are in flight,
// k in [0, 3] (wave-uniform).
template <int JPW>
__device__ __forceinline__ void wait_tiles(int k) {
  static_assert(3 * JPW <= 63, "vmcnt holds at most 63");
  switch (k) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<JPW>(); break;
    case 2: wait_vm<2 * JPW>(); break;
    default: wait_vm<3 * JPW>(); break;
  }
}
// Workgroup barrier for LDS traffic: this wave's LDS reads and writes are
// done, global-to-LDS loads are waited for separately (wait_vm), so loads of
// later tiles stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Split partials and their counters are exchanged across workgroups with
// device-scope relaxed atomic accesses: individually coherent across the
// XCDs' L2 caches, with no fence (a device-scope release / acquire would
// write back or invalidate a whole L2).
__device__ __forceinline__ float peek_f32(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void post_f32(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte accesses to a split partial with the same cache policy as the
// device-scope accesses above (sc1: coherent across the XCDs of the device),
// through a buffer resource over the partial's slot.
constexpr int kDevPolicy = 16;  // sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const char* slot, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(slot), (short)0, int(bytes), 0x00020000);
}
__device__ __forceinline__ void post16(__amdgpu_buffer_rsrc_t r, int off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kDevPolicy);
}
__device__ __forceinline__ u32x4 peek16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDevPolicy));
}

// Scores (log2 units) of a staged K tile against this wave's queries, shifted
// by -m (the product starts from cinit = -m).
template <int D>
__device__ __forceinline__ void tile_scores(const char* kl,
                                            const bf16x8 (&qop)[Geo<D>::NB][D / 16],
                                            const f32x16 (&cinit)[Geo<D>::NB],
                                            f32x16 (&S)[Geo<D>::NB]) {
  constexpr int NB = Geo<D>::NB;
#pragma unroll
  for (int s2 = 0; s2 < D / 16; ++s2) {
    const bf16x8 kop = *reinterpret_cast<const bf16x8*>(kl + 32 * s2);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      S[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[nb][s2], s2 == 0 ? cinit[nb] : S[nb], 0, 0, 0);
  }
}

// Load q of this wave for a whole trunk tile (every key < L) of the current
// (trunk, kv head): a buffer load from the trunk's K or V (uniform per load:
// its 1 KB of the tile is all K or all V) at this lane's fixed offset into
// the tile plus the tile's offset as a scalar, straight into LDS buffer lb.
template <int D>
__device__ __forceinline__ void dma_whole_q(int q, int v, int kvrow, int wave, char* lb,
                                            const uint16_t* kbase, const uint16_t* vbase, int tbytes,
                                            int toffq) {
  using Gm = Geo<D>;
  const int w = wave + Gm::NW * q;
  const int so = int(uint32_t(v) * uint32_t(KT * 2) * uint32_t(kvrow));  // < 4 GiB (host check)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(w * 1024 >= Gm::VBASE ? vbase : kbase), (short)0, tbytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lb + w * 1024), 16,
                                           toffq, so, 0, 0);
}
template <int D>
__device__ __forceinline__ void dma_whole(int v, int kvrow, int wave, char* lb, const uint16_t* kbase,
                                          const uint16_t* vbase, int tbytes, const int (&toff)[Geo<D>::JPW]) {
#pragma unroll
  for (int q = 0; q < Geo<D>::JPW; ++q) dma_whole_q<D>(q, v, kvrow, wave, lb, kbase, vbase, tbytes, toff[q]);
}

// Loads key tile v (trunk tile, or tail tile of branch nodes) of the current
// pack into LDS buffer b: this wave's share of the wave-wide 1 KB writes.
// A plain function rather than a lambda: a lambda's closure here stays in
// private memory.
// With FROM_LDS the branch of a tail slot comes from the pack's branch table
// in LDS (s_ord, written in the unit's prologue and published by its first
// barrier), read in inline assembly that waits for LDS only: a load from
// global memory there waits for every tile load in flight, and so would an
// LDS read the compiler sees (it cannot tell the table from the tiles being
// loaded).  The prologue's own tile loads take the global path.
template <int D, bool FROM_LDS>
__device__ __forceinline__ void dma_tile(int v, int ntrunk, int nt_total, int Lk, int kvrow, int Wn,
                                         int ts, int wave, const uint16_t* tk, const uint16_t* tv,
                                         const uint16_t* bk, const uint16_t* bv,
                                         const int32_t* pord, const int* s_ord, char* lb,
                                         const int (&dcode)[Geo<D>::JPW],
                                         const uint16_t* kbase, const uint16_t* vbase, int tbytes,
                                         const int (&toff)[Geo<D>::JPW]) {
  using Gm = Geo<D>;
  const bool trunk = v < ntrunk;
  if (trunk && (v + 1) * KT <= Lk) {
    dma_whole<D>(v, kvrow, wave, lb, kbase, vbase, tbytes, toff);
    return;
  }
#pragma unroll
  for (int q = 0; q < Gm::JPW; ++q) {
    const int code = dcode[q];
    const int key = code & 31, c = (code >> 5) & 127;
    const bool isv = (code >> 12) & 1;
    const uint16_t* src;
    if (trunk) {
      const int off = min(v * KT + key, Lk - 1) * kvrow + c * 8;
      src = (isv ? tv : tk) + off;
    } else {
      int tau = (v - ntrunk) * KT + key;
      if (tau >= nt_total) tau = 0;
      const int sl = tau / ts;
      int node = tau - sl * ts;
      if (node >= Wn) node = 0;  // a slot's padding: a valid key that every row masks
      int br;
      if constexpr (FROM_LDS) {
        const __attribute__((address_space(3))) int* lp = (const __attribute__((address_space(3))) int*)(s_ord) + sl;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(br) : "v"(lp) : "memory");
      } else {
        br = pord[sl];
      }
      const int off = (br * Wn + node) * kvrow + c * 8;
      src = (isv ? bv : bk) + off;
    }
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(
                                              lb + (wave + Gm::NW * q) * 1024), 16, 0, 0);
  }
}

// Reads N entries of the pack's branch table in LDS (one per lane and load),
// in inline assembly that waits for LDS only (see dma_tile): all N reads go
// out before the one wait.
typedef const __attribute__((address_space(3))) int* lds_cint;
template <int N>
struct OrdGather;
template <>
struct OrdGather<3> {
  static __device__ __forceinline__ void run(int (&r)[3], lds_cint const (&a)[3]) {
    asm volatile("ds_read_b32 %0, %3\n\tds_read_b32 %1, %4\n\tds_read_b32 %2, %5\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2])
                 : "memory");
  }
};
template <>
struct OrdGather<5> {
  static __device__ __forceinline__ void run(int (&r)[5], lds_cint const (&a)[5]) {
    asm volatile(
        "ds_read_b32 %0, %5\n\tds_read_b32 %1, %6\n\tds_read_b32 %2, %7\n\tds_read_b32 %3, %8\n\t"
        "ds_read_b32 %4, %9\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4])
        : "memory");
  }
};
template <>
struct OrdGather<9> {
  static __device__ __forceinline__ void run(int (&r)[9], lds_cint const (&a)[9]) {
    asm volatile(
        "ds_read_b32 %0, %9\n\tds_read_b32 %1, %10\n\tds_read_b32 %2, %11\n\tds_read_b32 %3, %12\n\t"
        "ds_read_b32 %4, %13\n\tds_read_b32 %5, %14\n\tds_read_b32 %6, %15\n\tds_read_b32 %7, %16\n\t"
        "ds_read_b32 %8, %17\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
          "=&v"(r[7]), "=&v"(r[8])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8])
        : "memory");
  }
};

// LDS address of this lane's first transposed V read in a staged tile, as an
// opaque value: the tile's reads then share one base register with immediate
// offsets (otherwise the compiler hoists one address register per read out of
// the loop and adds the buffer offset to each).  The callee takes it as a
// restrict parameter, which tells the compiler that these reads do not touch
// the tiles still being loaded.
__device__ __forceinline__ lds_cchar* v_base(const char* p) {
  lds_cchar* b = (lds_cchar*)(p);
  asm("" : "+v"(b));
  return b;
}

// K operands of a staged tile (this lane's 16-byte reads).
template <int D>
__device__ __forceinline__ void load_k(const char* kl, bf16x8 (&kop)[D / 16]) {
#pragma unroll
  for (int s2 = 0; s2 < D / 16; ++s2) kop[s2] = *reinterpret_cast<const bf16x8*>(kl + 32 * s2);
}

// The matrix-core work of one steady-state tile, in an explicit order (one
// wave per SIMD, so the wave's own instruction stream has to keep the matrix
// core busy while the vector unit forms the probabilities).  The exponentials
// of the current tile are spread over the matrix products: between the
// k-steps of the next tile's score product (K operands kop, already in
// registers), together with the reads of the current tile's V operands and
// this wave's loads of a later tile; with two row blocks, the second block's
// half between the first V products, which are ordered by (row block, key
// half) so that each waits only for its own probabilities.  The second half
// of the V products covers the maxima of the next tile's scores.  When
// knext is given, the K operands of the tile after next are read into kop
// at the start of the V products.  sched_barrier(0) keeps the compiler from
// regrouping the steps.  The row sums (v_dot2) are left where instruction
// selection puts them, after the last product: between the products each
// one stalls the matrix pipe (measured ~16 cycles apiece).
// A whole trunk tile's loads (dma_whole_q) that tile_compute issues among its
// score products.  With tbytes = 0 (no tile left to load) every lane is out
// of the buffer's range and the loads fetch nothing: the step stays free of
// branches, which would let the compiler move the exponentials out of the
// score products.
template <int D>
struct TileLoads {
  int v, kvrow, wave;
  char* lb;
  const uint16_t *kbase, *vbase;
  int tbytes;
  int toff[Geo<D>::JPW];
};

// With MASK the maxima are taken after the next tile's scores are masked:
// score i of row block nb stays where bit 8(i/4) + i%4 of vis[nb] is set
// (vis already shifted by this lane's 4h keys) and becomes -inf elsewhere.
template <int D, bool KNEXT, bool MX, bool DMA, bool MASK = false>
__device__ __forceinline__ void tile_compute(bf16x8 (&kop)[D / 16], const char* knext,
                                             lds_cchar* __restrict__ vl,
                                             const bf16x8 (&qop)[Geo<D>::NB][D / 16],
                                             const f32x16 (&cinit)[Geo<D>::NB],
                                             const f32x16 (&Scur)[Geo<D>::NB], f32x16 (&Snext)[Geo<D>::NB],
                                             float (&lsum)[Geo<D>::NB],
                                             f32x16 (&oacc)[Geo<D>::NB][Geo<D>::OREG],
                                             const TileLoads<D>& dma, float (&mx)[Geo<D>::NB],
                                             const uint32_t (&vis)[Geo<D>::NB]) {
  using Gm = Geo<D>;
  constexpr int NB = Gm::NB, KS = D / 16, OREG = Gm::OREG;
  constexpr int NPAIR = NB * 8;                    // pairs of probabilities per lane
  // pairs formed during the V products: half of them with two row blocks
  // (the score products' exponentials otherwise saturate the vector unit;
  // measured 1,687 -> 1,611 cycles per tile from 4 to 8 of 16, flat to 10)
  constexpr int LATE = NB == 2 ? 8 : 0;
  constexpr int EARLY = NPAIR - LATE;              // pairs formed during the score product
  constexpr int NVO = OREG * 2;                    // V operands (two transposed reads each)
  constexpr int VPS = (NVO + KS - 1) / KS;         // V operands per k-step
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  bf16x8 vop[NVO];
  bf16x8 P[NB][2];
  float acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = lsum[nb];
  auto pair = [&](int q) __attribute__((always_inline)) {
    const int nb = q >> 3, i = 2 * (q & 7);
    const bf16x2 e2 = {static_cast<__bf16>(fast_exp2(Scur[nb][i])),
                       static_cast<__bf16>(fast_exp2(Scur[nb][i + 1]))};
    P[nb][i >> 3][i & 7] = e2[0];
    P[nb][i >> 3][(i & 7) + 1] = e2[1];
    acc[nb] = __builtin_amdgcn_fdot2_f32_bf16(e2, ones, acc[nb], false);  // sums the bf16 weights used
  };
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      Snext[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[s2], qop[nb][s2], s2 == 0 ? cinit[nb] : Snext[nb],
                                                          0, 0, 0);
#pragma unroll
    for (int o = s2 * VPS; o < (s2 + 1) * VPS && o < NVO; ++o) {
      const int db = o >> 1, h2 = o & 1;
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vl + 16 * h2 * Gm::VROW + 64 * db));
      const s16x4 vc = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vl + (16 * h2 + 8) * Gm::VROW + 64 * db));
      vop[o] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vc, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int q = s2 * EARLY / KS; q < (s2 + 1) * EARLY / KS; ++q) pair(q);
    // this wave's loads of a later tile, spread over the k-steps (the CU's
    // vector memory path takes a wave-wide 16-byte load into LDS every 16
    // cycles; issued in one burst by every wave they would queue and hold
    // the waves at the issue)
#pragma unroll
    for (int q = s2 * Gm::JPW / KS; q < (s2 + 1) * Gm::JPW / KS; ++q)
      if constexpr (DMA)
        dma_whole_q<D>(q, dma.v, dma.kvrow, dma.wave, dma.lb, dma.kbase, dma.vbase, dma.tbytes, dma.toff[q]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // V products by (row block, key half); the late pairs go between the first
  // half of them
  constexpr int NPV = NB * 2 * OREG;
#pragma unroll
  for (int g = 0; g < NB * 2; ++g) {
    const int nb = g >> 1, h2 = g & 1;
#pragma unroll
    for (int db = 0; db < OREG; ++db) {
      const int sl = g * OREG + db;  // V product slot
      oacc[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[2 * db + h2], P[nb][h2], oacc[nb][db], 0, 0, 0);
      if constexpr (LATE > 0) {
        if (sl < NPV / 2) {
#pragma unroll
          for (int q = EARLY + sl * LATE / (NPV / 2); q < EARLY + (sl + 1) * LATE / (NPV / 2); ++q) pair(q);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // the maxima of the next tile's scores (for the reference check) over
      // the second half of the V products
      if constexpr (MX) {
        if (sl >= NPV / 2) {
          constexpr int NE = NB * 16, H = NPV / 2;
#pragma unroll
          for (int k = (sl - H) * NE / H; k < (sl - H + 1) * NE / H; ++k) {
            const int nb = k >> 4, e = k & 15;
            if constexpr (MASK) {
              // all ones where the key is visible, else zero; then a bit
              // select in inline assembly (the compiler's own form of this
              // select on matrix-core results gave every element the first
              // element's value).  The scores were written several products
              // earlier, so the read needs no wait states.
              const int keep = __builtin_amdgcn_sbfe(int(vis[nb]), 8 * (e >> 2) + (e & 3), 1);
              float r;
              asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(keep), "v"(Snext[nb][e]), "s"(0xff800000u));
              Snext[nb][e] = r;
            }
            mx[nb] = e == 0 ? Snext[nb][0] : fmaxf(mx[nb], Snext[nb][e]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if (KNEXT && g == 0) load_k<D>(knext, kop);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) lsum[nb] = acc[nb];
}

// PREFILL changes nothing in the code: the kernel is instantiated under a
// second name for trunk prefills, so that profiles attribute tree calls and
// prefills separately.
template <int D, bool PREFILL>
__global__ __launch_bounds__(mfma_waves(D) * 64, 1) void tree_attn_mfma_kernel(const MfmaParams p) {
  using Gm = Geo<D>;
  constexpr int NB = Gm::NB, OREG = Gm::OREG;
  // The kernel's only LDS object (tile buffers, then one flag word): with a
  // second __shared__ variable the compiler tags LDS accesses with alias
  // scopes and then waits for every global-to-LDS load before any LDS read.
  __shared__ __attribute__((aligned(1024))) char smem[Gm::NBUF * Gm::BUFB + 16 + 1024];
  int* const s_last = reinterpret_cast<int*>(smem + Gm::NBUF * Gm::BUFB);
  int* const s_unit = s_last + 1;
  int* const s_ord = s_last + 4;  // the current pack's branches (at most 256)

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int h = lane >> 5, r32 = lane & 31;
  const int gi = lane >> 4, rq = lane & 15;

  // Work unit u = (t * Hkv + g) * ugp + j, j < npacks * nsplit the j-th split
  // of the (trunk, kv head) group in pack order; ugp >= that count pads the
  // group to a multiple of ilv.  In chunked mode the groups are queued to the
  // XCDs in consecutive blocks (workgroups go to the 8 XCDs round robin), so
  // the packs of a kv head run on one XCD and stream its trunk rows through
  // that XCD's L2; when a group spans `ilv` XCD blocks, its packs are dealt
  // to those blocks alternately, so that each XCD gets a like share of long
  // and short packs.  The workgroups are persistent (one per CU): each
  // takes the front unit of its XCD's queue (packs come longest first) until
  // that queue is empty, then the back units -- the shortest left -- of the
  // other XCDs' queues, so XCDs whose trunks hold less work help the others
  // finish.  A queue's counter keeps the front count in its low half and the
  // back count in its high half: one atomic add both claims an entry and
  // tells whether it was still free, so every entry is taken exactly once.
  // Otherwise (no XCD structure) units are claimed in order from one queue.
  const int nq = p.nwg >> 3;  // entries per XCD queue
  for (;;) {
  __syncthreads();  // every wave is done with the previous unit and its claim
  if (tid == 0) {
    int u = -1;
    if (p.chunked) {
      const int x = blockIdx.x & 7;
      for (int k = 0; k < 8 && u < 0; ++k) {
        const int y = (x + k) & 7;
        const unsigned long long old = __hip_atomic_fetch_add(
            p.qctr + y, k == 0 ? 1ull : (1ull << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const long long f = (long long)(old & 0xffffffffull), bk = (long long)(old >> 32);
        if (f + bk < nq) u = y * nq + int(k == 0 ? f : nq - 1 - bk);
      }
    } else {
      const int v = int(__hip_atomic_fetch_add(p.qctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      u = v < p.nwg ? v : -1;
    }
    *s_unit = u;
  }
  __syncthreads();
  const int ub = *s_unit;
  if (ub < 0) break;             // every queue is empty
  if (ub >= p.nunits) continue;  // padding
  const int np = p.npacks;
  const int ug = np * p.nsplit;            // units per (trunk, kv head)
  // Queue entry -> (group, unit of the group).  A queue holding whole groups
  // deals them by unit rank (every group's longest pack first, its shortest
  // last), so the units claimed at the end of the kernel are the shortest
  // ones of every group, not one group's packs of all lengths; likewise the
  // single queue of the unchunked mode.
  int tg, jj;
  if (!p.chunked) {
    const int ng = p.T * p.Hkv;
    tg = ub % ng;
    jj = ub / ng;
  } else if (p.ilv == 1) {
    const int gpx = (p.T * p.Hkv) >> 3;  // groups per XCD queue
    const int y = ub / nq, e = ub - y * nq;
    tg = y * gpx + e % gpx;
    jj = e / gpx;
  } else {
    tg = ub / p.ugp;
    jj = ub - tg * p.ugp;
    const int c = p.ugp / p.ilv;
    jj = (jj % c) * p.ilv + jj / c;
  }
  if (jj >= ug) continue;  // padding
  const int g = tg % p.Hkv, t = tg / p.Hkv;
  // the pack of this unit and its splits: packs get units in proportion to
  // their key tiles (at least one each), so splits are of similar length
  const int pk = p.umap[size_t(t) * ug + jj];
  const int* us = p.ustart + size_t(t) * (np + 1);
  const int u0 = us[pk];
  const int S = us[pk + 1] - u0;  // splits of this pack
  const int rsp = jj - u0;
  const int upk = tg * np + pk;
  const int* ps = p.pstart + size_t(t) * (np + 1);
  const int nvt = ps[pk + 1] - ps[pk];
  // split rsp takes the pack's key tiles [rsp * nvt / S, (rsp + 1) * nvt / S)
  auto split_begin = [=](int r2) __attribute__((always_inline)) { return int((long long)r2 * nvt / S); };
  const int v0 = split_begin(rsp);
  const int n = split_begin(rsp + 1) - v0;
  if (n == 0) continue;  // pack shorter than its split count

  const int rows_per_branch = p.Wn * p.G;
  // scalars the helper lambdas use, copied so that no lambda takes the
  // address of the kernel argument block (that would move it to scratch)
  const int Lk = p.L, Wn = p.Wn, ts = p.tstride;
  char* const part = p.part;
  const size_t slot_bytes = p.slot_bytes;

  // This lane's 16-byte slot in each of its wave's tile loads: key row,
  // chunk, K or V.  Pad chunks, the gap before the V rows and the slack after
  // them load chunk 0 of a valid row (of K or V, as the rest of the load).
  int dcode[Gm::JPW];
#pragma unroll
  for (int q = 0; q < Gm::JPW; ++q) {
    const int w = wave + Gm::NW * q;
    const int pos = w * 64 + lane;
    int key = 0, c = 0;
    const int isv = w * 1024 >= Gm::VBASE;
    if (pos < KT * Gm::SK) {
      key = pos / Gm::SK;
      c = pos - key * Gm::SK;
    } else if (isv && pos < Gm::VBASE / 16 + KT * Gm::SV) {
      const int pv = pos - Gm::VBASE / 16;
      key = pv / Gm::SV;
      c = pv - key * Gm::SV;
    }
    if (c >= Gm::CH) c = 0;
    dcode[q] = key | (c << 5) | (isv << 12);
  }

  {
    // ---- pack geometry: its trunk tiles are its tile count less the tail
    // tiles of its branch nodes, so the tile loads can start before any
    // per-branch metadata has arrived
    const size_t tB = size_t(t) * p.B;
    const int32_t* ord = p.order + tB;
    // sorted branches [b0, b0 + nbr) in slots of ts tail keys; with a branch
    // split over spb packs, this pack's rows start at row ro of the branch
    const int b0 = (pk / p.spb) * p.bpp;
    const int nbr = min(p.bpp, p.B - b0);
    const int ro = (pk % p.spb) * mfma_rows_per_wg(D);
    const int nt_total = (nbr - 1) * ts + Wn;
    const int ntrunk = nvt - (nt_total + KT - 1) / KT;

    // per-segment bases (uniform); per-lane offsets below stay in 32 bits
    const uint16_t* tk = p.trunk_k + (size_t(t) * p.L * p.Hkv + g) * D;
    const uint16_t* tv = p.trunk_v + (size_t(t) * p.L * p.Hkv + g) * D;
    const uint16_t* bk = p.kr + (tB * p.Wn * p.Hkv + g) * D;
    const uint16_t* bv = p.v + (tB * p.Wn * p.Hkv + g) * D;
    const int kvrow = p.Hkv * D;  // elements between consecutive keys
    // whole trunk tiles: buffer resources over trunk t's K and V (under 4 GiB
    // each, checked on the host) and this lane's byte offset in each of its
    // tile loads for trunk tile 0
    const size_t tbase = size_t(t) * p.L * p.Hkv * D;
    const int tbytes = int(uint32_t(size_t(p.L) * kvrow * 2));
    const uint16_t* const kbase = p.trunk_k + tbase;
    const uint16_t* const vbase = p.trunk_v + tbase;
    int toff[Gm::JPW];
#pragma unroll
    for (int q = 0; q < Gm::JPW; ++q) {
      const int code = dcode[q];
      toff[q] = ((code & 31) * kvrow + ((code >> 5) & 127) * 8 + g * D) * 2;
    }

    // tail tiles in the loop: buffer resources over the trunk's branch-node
    // K and V from this kv head's first element on (under 4 GiB, checked on
    // the host); slots are a power of two keys apart
    const int bbytes = int(uint32_t((size_t(p.B) * Wn * kvrow - size_t(g) * D) * 2));
    const int lts = 31 - __builtin_clz(ts);

    // ---- tile loads: global -> LDS buffer b
#define DMA_TILE_(v, b, LDS)                                                                                 \
  dma_tile<D, LDS>(v, ntrunk, nt_total, Lk, kvrow, Wn, ts, wave, tk, tv, bk, bv, ord + b0, s_ord,            \
                   smem + (b) * Gm::BUFB, dcode, kbase, vbase, tbytes, toff)
#define DMA_TILE(v, b) DMA_TILE_(v, b, true)
    const int koff = r32 * Gm::KROW + 16 * h;  // this lane's K read in a tile
    const int voff = Gm::VBASE + (4 * (gi >> 1) + (rq >> 2)) * Gm::VROW + 32 * (gi & 1) + 8 * (rq & 3);

    // ---- staging.  Tile j of this range goes to LDS buffer j % NBUF and is
    // loaded AH = NBUF - 1 tiles ahead of the tile being accumulated, in
    // iteration j - AH (the buffer's previous tile, j - NBUF, had its last
    // reads in iteration j - NBUF).  Iteration i needs tiles up to i + NEED
    // readable after its barrier (K of tile i + NEED is read one tile early
    // when EARLYK), so the loads of the INFL tiles after that may stay in
    // flight across the barrier.
    constexpr int NBUF = Gm::NBUF, AH = NBUF - 1, NEED = Gm::NEED, INFL = Gm::INFL;
    constexpr bool EK = Gm::EARLYK;
    auto buf = [&](int j) __attribute__((always_inline)) { return smem + (j % NBUF) * Gm::BUFB; };
    // tiles issued beyond tile `last`, capped at INFL
    auto inflight = [&](int last) __attribute__((always_inline)) { return max(0, min(INFL, n - 1 - last)); };

    // the pack's branch table for the tail loads of the loop (loaded before
    // the first tiles, so that waiting for it does not wait for them)
    static_assert(mfma_waves(D) * 64 >= 256, "one thread per table entry");
    const int ordv = tid < nbr ? ord[b0 + tid] : 0;
#pragma unroll
    for (int q = 0; q < AH; ++q)
      if (q < n) DMA_TILE_(v0 + q, q, false);
    if (tid < nbr) s_ord[tid] = ordv;
    // ---- this lane's rows: metadata and the Q^T operand
    int ra[NB], rslot[NB], rbr[NB];  // anchor, pack slot and branch of each row block's row
    bool rok[NB];                     // the row's branch is well formed
    uint64_t rmask[NB];
    bf16x8 qop[NB][D / 16];
    int wmin = 0x7fffffff;
    {
      const uint16_t* qb = p.qr + (tB * p.Wn * p.Hq + size_t(g) * p.G) * D;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int rho = (wave * NB + nb) * 32 + r32 + ro;
        const int slot = rho / rows_per_branch;
        const int within = rho - slot * rows_per_branch;
        const int j = within / p.G;
        const int hh = within - j * p.G;
        const bool exists = slot < nbr;
        const int b = exists ? ord[b0 + slot] : 0;
        const bool ok = exists && p.branch_ok[tB + b];
        ra[nb] = ok ? p.anchors[tB + b] : ntrunk * KT - 1;  // rows without output never force a mask
        rslot[nb] = slot;
        rbr[nb] = b;
        rok[nb] = ok;
        rmask[nb] = ok ? p.anc[(tB + b) * p.Wn + j] : 0ull;
        wmin = min(wmin, ra[nb]);
        const uint16_t* qrow = qb + ((b * p.Wn + j) * p.Hq + hh) * D;
#pragma unroll
        for (int s2 = 0; s2 < D / 16; ++s2)
          qop[nb][s2] = ok ? *reinterpret_cast<const bf16x8*>(qrow + 16 * s2 + 8 * h) : bf16x8{};
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) wmin = min(wmin, __shfl_xor(wmin, o, 64));
    const int wave_amin = __builtin_amdgcn_readfirstlane(wmin);

    // ---- running state
    f32x16 oacc[NB][OREG], cinit[NB];
    float mref[NB], lim[NB], lsum[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      mref[nb] = 0.f;
      lim[nb] = kUnset;
      lsum[nb] = 0.f;
      cinit[nb] = f32x16{};
#pragma unroll
      for (int db = 0; db < OREG; ++db) oacc[nb][db] = f32x16{};
    }

    // trunk keys beyond a row's anchor (edge tiles only); tail keys of other
    // branches or outside the row's ancestor chain
    auto mask = [&](int v, f32x16 (&S)[NB]) __attribute__((always_inline)) {
      if (v < ntrunk) {
        const int k0 = v * KT;
        if (k0 + KT - 1 > wave_amin) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int lm = ra[nb] - k0 - 4 * h;  // element i visible iff 8(i/4)+(i%4) <= lm
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (8 * (i >> 2) + (i & 3) > lm) S[nb][i] = kNegInf;
          }
        }
      } else {
        const int tau0 = (v - ntrunk) * KT;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint32_t vis = tail_window(rmask[nb], rslot[nb], ts, tau0) >> (4 * h);
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (!((vis >> (8 * (i >> 2) + (i & 3))) & 1u)) S[nb][i] = kNegInf;
        }
      }
    };
    // move the reference maximum of rows that need it (rare)
    // (mx: the maxima of each row block's scores in this lane)
    auto settle_mx = [&](f32x16 (&S)[NB], const float (&mx)[NB]) __attribute__((always_inline)) {
      bool any = false;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) any |= mx[nb] > lim[nb];
      if (__any(any)) {
        // keeps this rare path a branch: without a side effect the compiler
        // would fold it into the common path as unconditional multiplies
        asm volatile("; rescale" ::: "memory");
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const float m = fmaxf(mx[nb], __shfl_xor(mx[nb], 32, 64));  // whole row, relative to mref
          const bool nd = m > lim[nb];
          const float delta = nd ? m : 0.f;
          const float f = (nd && lim[nb] != kUnset) ? fast_exp2(-delta) : 1.0f;
#pragma unroll
          for (int i = 0; i < 16; ++i) S[nb][i] -= delta;
          lsum[nb] *= f;
#pragma unroll
          for (int db = 0; db < OREG; ++db) oacc[nb][db] *= f;
          mref[nb] += delta;
          lim[nb] = nd ? kRescale : lim[nb];
          const float c = -mref[nb];
#pragma unroll
          for (int i = 0; i < 16; ++i) cinit[nb][i] = c;
        }
      }
    };
    auto settle = [&](f32x16 (&S)[NB]) __attribute__((always_inline)) {
      float mx[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float m = S[nb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) m = fmaxf(m, S[nb][i]);
        mx[nb] = m;
      }
      settle_mx(S, mx);
    };

    wait_tiles<Gm::JPW>(inflight(NEED - 1));  // tiles 0 .. NEED-1 have landed
    lds_barrier();

    f32x16 Sa[NB], Sb[NB];
    tile_scores<D>(smem + koff, qop, cinit, Sa);
    mask(v0, Sa);
    settle(Sa);
    bf16x8 kop[D / 16];
    if constexpr (EK) load_k<D>(smem + Gm::BUFB + koff, kop);  // tile 1 (stale data if n == 1: unused)

    // Fast iterations (every one but the last): the straight-code step.  In
    // the first ones the scored tile needs no mask for this wave's rows and
    // the tile loaded (if any) is a whole trunk tile (the lane's offset into
    // tile 0 plus the tile's offset as a scalar); tiles [0, nomask) of the
    // pack are visible to every row of the wave.  The later ones (`fastx`)
    // load tail tiles and trunk tiles that end past L too (the lane's whole
    // offset in the range-checked part: keys past L read zeros), and mask
    // the scored tile after the products where a row of the wave needs it.
    const int nomask = min(ntrunk, (wave_amin + 1) / KT);
    const int nwhole = min(ntrunk, Lk / KT);
    int nplain = min(nomask - v0 - 1, n - 1);
    if (v0 + n > nwhole) nplain = min(nplain, nwhole - v0 - AH);
    // the fixed wait in the steps counts on AH tiles in flight from the start
    const int nfast = n < AH ? 0 : n - 1;
    if (n < AH) nplain = 0;
    auto fast = [&](int i, const f32x16 (&Sc)[NB], f32x16 (&Sn)[NB]) __attribute__((always_inline)) {
      if constexpr (!EK) load_k<D>(buf(i + 1) + koff, kop);
      TileLoads<D> tl;
      const bool on = i + AH < n;
      tl.v = on ? v0 + i + AH : v0;
      tl.kvrow = kvrow;
      tl.wave = wave;
      tl.lb = buf(i + AH);
      tl.kbase = kbase;
      tl.vbase = vbase;
      tl.tbytes = on ? tbytes : 0;
#pragma unroll
      for (int q = 0; q < Gm::JPW; ++q) tl.toff[q] = toff[q];
      float mx[NB];
      const uint32_t vis[NB] = {};
      tile_compute<D, EK, true, true>(kop, buf(i + 2) + koff, v_base(buf(i) + voff), qop, cinit, Sc, Sn, lsum,
                                      oacc, tl, mx, vis);
      settle_mx(Sn, mx);
      // every fast iteration issues JPW loads (zero-record ones at the end),
      // so exactly INFL tiles' loads follow those of tile i + NEED
      wait_vm<INFL * Gm::JPW>();
      lds_barrier();
    };
    auto fastx = [&](int i, const f32x16 (&Sc)[NB], f32x16 (&Sn)[NB]) __attribute__((always_inline)) {
      if constexpr (!EK) load_k<D>(buf(i + 1) + koff, kop);
      TileLoads<D> tl;
      const int vl = v0 + i + AH;  // the tile this step loads
      const bool on = i + AH < n;
      tl.kvrow = kvrow;
      tl.wave = wave;
      tl.lb = buf(i + AH);
      if (on && vl >= nwhole) {
        tl.v = 0;
        if (vl < ntrunk) {
          const uint32_t to = uint32_t(vl) * uint32_t(KT * 2) * uint32_t(kvrow);
          tl.kbase = kbase;
          tl.vbase = vbase;
          tl.tbytes = tbytes;
#pragma unroll
          for (int q = 0; q < Gm::JPW; ++q) tl.toff[q] = int(uint32_t(toff[q]) + to);
        } else {
          // tail key tau of the pack: slot tau / ts, node tau % ts (a slot's
          // padding and keys past the last node load node 0 of a valid slot,
          // which every row masks)
          lds_cint la[Gm::JPW];
          int node[Gm::JPW], br[Gm::JPW];
#pragma unroll
          for (int q = 0; q < Gm::JPW; ++q) {
            int tau = (vl - ntrunk) * KT + (dcode[q] & 31);
            if (tau >= nt_total) tau = 0;
            node[q] = tau & (ts - 1);
            if (node[q] >= Wn) node[q] = 0;
            la[q] = (lds_cint)(s_ord) + (tau >> lts);
          }
          OrdGather<Gm::JPW>::run(br, la);
          tl.kbase = bk;
          tl.vbase = bv;
          tl.tbytes = bbytes;
#pragma unroll
          for (int q = 0; q < Gm::JPW; ++q)
            tl.toff[q] = ((br[q] * Wn + node[q]) * kvrow + ((dcode[q] >> 5) & 127) * 8) * 2;
        }
      } else {
        tl.v = on ? vl : v0;
        tl.kbase = kbase;
        tl.vbase = vbase;
        tl.tbytes = on ? tbytes : 0;
#pragma unroll
        for (int q = 0; q < Gm::JPW; ++q) tl.toff[q] = toff[q];
      }
      // visible keys of the tile whose scores the step forms, per row block
      const int vn = v0 + i + 1;
      uint32_t vis[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (vn < ntrunk) {
          const int lm = ra[nb] - vn * KT - 4 * h;  // key offsets 0..lm of the lane's keys are visible
          vis[nb] = lm >= 31 ? ~0u : lm < 0 ? 0u : (2u << lm) - 1u;
        } else {
          vis[nb] = tail_window(rmask[nb], rslot[nb], ts, (vn - ntrunk) * KT) >> (4 * h);
        }
      }
      float mx[NB];
      tile_compute<D, EK, true, true, true>(kop, buf(i + 2) + koff, v_base(buf(i) + voff), qop, cinit, Sc, Sn,
                                            lsum, oacc, tl, mx, vis);
      settle_mx(Sn, mx);
      // every fast iteration issues JPW loads (zero-record ones at the end),
      // so exactly INFL tiles' loads follow those of tile i + NEED
      wait_vm<INFL * Gm::JPW>();
      lds_barrier();
    };
    int i = 0;
    for (; i + 1 < nplain; i += 2) {
      fast(i, Sa, Sb);
      fast(i + 1, Sb, Sa);
    }
    for (; i + 1 < nfast; i += 2) {
      fastx(i, Sa, Sb);
      fastx(i + 1, Sb, Sa);
    }
    // remaining iterations: scores of tile i+1 overlap the probabilities of
    // tile i; after the last tile the scores are unused (they keep the block
    // straight)
    for (; i < n; ++i) {
      if (i + AH < n) DMA_TILE(v0 + i + AH, (i + AH) % NBUF);
      if constexpr (!EK) load_k<D>(buf(i + 1) + koff, kop);
      float mxu[NB];
      TileLoads<D> tl{};
      const uint32_t visu[NB] = {};
      tile_compute<D, EK, false, false>(kop, buf(i + 2) + koff, v_base(buf(i) + voff), qop, cinit, Sa, Sb, lsum,
                                        oacc, tl, mxu, visu);
      if (i + 1 < n) {
        mask(v0 + i + 1, Sb);
        settle(Sb);
      }
      wait_tiles<Gm::JPW>(inflight(i + NEED));
      lds_barrier();
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) Sa[nb] = Sb[nb];
    }

#undef DMA_TILE
#undef DMA_TILE_

    // ---- finish the pack (or this split of it)
    const int nseg = min(S, nvt);  // non-empty splits of the pack
    const bool whole = nseg == 1;
    bool write = whole;
    if (!whole) {
      const size_t ctr_i = upk;  // one counter per (trunk, kv head, pack)
      auto slot_of = [=](int r2) __attribute__((always_inline)) -> char* {
        return part + (size_t(tg) * ug + u0 + r2) * slot_bytes;
      };
      // a slot holds each wave's outputs as 16-byte chunks, chunk c of lane l
      // at ((wave * OCH + c) * 64 + l) * 16 (four bf16 pairs), then the
      // waves' (m, l) per row block
      constexpr int OWORDS = NB * OREG * 8;  // bf16 pairs per lane
      constexpr int OCH = OWORDS / 4;
      char* mine = slot_of(rsp);
      const __amdgpu_buffer_rsrc_t mres = slot_rsrc(mine, slot_bytes);
      float* pm = reinterpret_cast<float*>(mine + Gm::NW * OWORDS * 64 * 4) + wave * NB * 128 + lane;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int db = 0; db < OREG; ++db)
#pragma unroll
          for (int k4 = 0; k4 < 2; ++k4) {
            const f32x16& o = oacc[nb][db];
            const int k = 4 * k4;
            const u32x4 w = {pack_bf16x2(o[2 * k], o[2 * k + 1]), pack_bf16x2(o[2 * k + 2], o[2 * k + 3]),
                             pack_bf16x2(o[2 * k + 4], o[2 * k + 5]), pack_bf16x2(o[2 * k + 6], o[2 * k + 7])};
            const int c = (nb * OREG + db) * 2 + k4;
            post16(mres, ((wave * OCH + c) * 64 + lane) * 16, w);
          }
        post_f32(pm + nb * 128, lim[nb] == kUnset ? kNegInf : mref[nb]);
        post_f32(pm + nb * 128 + 64, lsum[nb]);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // partials acknowledged first
      __syncthreads();
      if (tid == 0) {
        const int old = __hip_atomic_fetch_add(p.ctr + ctr_i, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        *s_last = old == nseg - 1;
      }
      __syncthreads();
      write = *s_last != 0;
      if (write) {
        // merge every non-empty segment, this one included, from the stored
        // values in segment order, so the result does not depend on who
        // merges.  Each step is a round trip to memory, so the loads are
        // batched: every segment's (m, l) first, then the outputs of
        // kMergeBatch segments at a time.
        // a segment that does not exist reads this workgroup's own slot, so
        // every load stays inside the workspace (its values are not used)
        const char* const sbase = part + (size_t(tg) * ug + u0) * slot_bytes;
        auto present = [&](int r2) __attribute__((always_inline)) {
          return r2 < S && split_begin(r2 + 1) > split_begin(r2);
        };
        float mx[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          mx[nb] = kNegInf;
          lsum[nb] = 0.f;
#pragma unroll
          for (int db = 0; db < OREG; ++db) oacc[nb][db] = f32x16{};
        }
        for (int r0 = 0; r0 < S; r0 += kMergeBatch) {
          bool f[kMergeBatch];
          float m2[kMergeBatch][NB], l2[kMergeBatch][NB];
          u32x4 wv[kMergeBatch][OCH];
#pragma unroll
          for (int e = 0; e < kMergeBatch; ++e) {
            f[e] = present(r0 + e);
            const char* sl = sbase + size_t(f[e] ? r0 + e : rsp) * slot_bytes;
            const __amdgpu_buffer_rsrc_t sres = slot_rsrc(sl, slot_bytes);
            const float* qm = reinterpret_cast<const float*>(sl + Gm::NW * OWORDS * 64 * 4) + wave * NB * 128 + lane;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              m2[e][nb] = peek_f32(qm + nb * 128);
              l2[e][nb] = peek_f32(qm + nb * 128 + 64);
            }
#pragma unroll
            for (int c = 0; c < OCH; ++c) wv[e][c] = peek16(sres, ((wave * OCH + c) * 64 + lane) * 16);
          }
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            // new reference max over the running one and this batch
            float mn = mx[nb];
#pragma unroll
            for (int e = 0; e < kMergeBatch; ++e)
              if (f[e]) mn = fmaxf(mn, m2[e][nb]);
            const float a0 = mx[nb] == kNegInf ? 0.f : fast_exp2(mx[nb] - mn);
            lsum[nb] *= a0;
#pragma unroll
            for (int db = 0; db < OREG; ++db) oacc[nb][db] *= a0;
            mx[nb] = mn;
#pragma unroll
            for (int e = 0; e < kMergeBatch; ++e) {
              const float a = (!f[e] || m2[e][nb] == kNegInf) ? 0.f : fast_exp2(m2[e][nb] - mn);
              if (a == 0.f) continue;
              lsum[nb] += a * l2[e][nb];
#pragma unroll
              for (int db = 0; db < OREG; ++db)
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                  const uint32_t w2 = wv[e][((nb * OREG + db) * 8 + k) >> 2][k & 3];
                  oacc[nb][db][2 * k] += bf16_lo(w2) * a;
                  oacc[nb][db][2 * k + 1] += bf16_hi(w2) * a;
                }
            }
          }
        }
      }
    }
    if (write) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float lt = lsum[nb] + __shfl_xor(lsum[nb], 32, 64);
        const int rho = (wave * NB + nb) * 32 + r32 + ro;
        const int slot = rho / rows_per_branch;
        if (slot >= nbr) continue;
        const int within = rho - slot * rows_per_branch;
        const int j = within / p.G;
        const int hh = within - j * p.G;
        const size_t b = size_t(rbr[nb]);  // kept from the setup: no reload at the end
        const bool ok = rok[nb];
        const float inv = ok ? 1.0f / lt : __builtin_nanf("");
        uint16_t* orow = p.out + (tB * p.Wn * p.Hq + size_t(g) * p.G) * D +
                         ((int(b) * p.Wn + j) * p.Hq + hh) * D;
#pragma unroll
        for (int db = 0; db < OREG; ++db)
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
  }
  }  // next unit
}

}  // namespace

size_t mfma_slot_bytes(int D) {
  const int nw = mfma_waves(D), nb = mfma_row_blocks(D);
  return align_up(size_t(nw) * nb * (D / 32) * 8 * 64 * 4 + size_t(nw) * nb * 128 * 4, 256);
}

// Compute units of the current device (cached per device): the persistent
// matrix-core kernel runs one workgroup per CU.
static int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    cus[dev] = c;
  }
  return cus[dev];
}

hipError_t launch_tree_attn_mfma(int D, const MfmaParams& p, hipStream_t s, bool prefill) {
  // one workgroup per CU (a multiple of 8, so every XCD runs workgroups of
  // its own queue), or fewer when there are fewer queue entries
  const int cus = device_cus() / 8 * 8;
  const dim3 grid(unsigned(p.nwg < cus ? p.nwg : (cus > 0 ? cus : 8))), block(mfma_waves(D) * 64);
  switch (D) {
    case 64:
      if (prefill) tree_attn_mfma_kernel<64, true><<<grid, block, 0, s>>>(p);
      else tree_attn_mfma_kernel<64, false><<<grid, block, 0, s>>>(p);
      break;
    case 128:
      if (prefill) tree_attn_mfma_kernel<128, true><<<grid, block, 0, s>>>(p);
      else tree_attn_mfma_kernel<128, false><<<grid, block, 0, s>>>(p);
      break;
    case 256:
      if (prefill) tree_attn_mfma_kernel<256, true><<<grid, block, 0, s>>>(p);
      else tree_attn_mfma_kernel<256, false><<<grid, block, 0, s>>>(p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace specopd
