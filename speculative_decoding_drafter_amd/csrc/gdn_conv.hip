// The short convolution of a linear-attention (GDN) layer for branch nodes
// (gfx950).
//
// What is computed (jaehun.me review of SpecOPD, §3.2(c)): like the
// recurrent state, the convolution history of a branch token follows only
// the branch's ancestors.  Gated DeltaNet convolves its projected q, k and v
// per channel over the last K inputs, applies SiLU and scales q and k to unit
// length per head (the pages name GDN without stating it).  For branch node
// j the K inputs are j's own, its ancestors' (nearest first), then the trunk
// tokens a, a-1, ... of its anchor a, and zeros before the trunk's start.
//
// One workgroup of four waves per node: thread 0 walks the parent map once
// for the node's window (which tensor and row each of the K inputs comes
// from) into LDS; then each wave takes whole heads (wave w: heads w, w+4,
// ...), each lane D/64 consecutive channels of the head, so a window row is
// one contiguous read per wave and a head's sum of squares one wave
// reduction.  Memory-bound: each node's row is read by the up to K nodes
// whose windows hold it (the repeats hit the caches) and written once.
#include "device_common.h"
#include "internal.h"

namespace specopd {

namespace {

constexpr int kConvMaxK = 8;
constexpr int kConvWaves = 4;

struct ConvArgs {
  const void *trunk_x, *x;
  const float* w;
  const int32_t *anchors, *parent;
  void* out;
  int L, B, Wn, H, K;
  bool l2norm;
};

// CPL consecutive values of a row as fp32, and back
template <typename IO, int CPL>
struct Chan;
template <>
struct Chan<uint16_t, 2> {
  static __device__ __forceinline__ void load(const uint16_t* p, float (&v)[2]) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    v[0] = bf16_lo(w);
    v[1] = bf16_hi(w);
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float (&v)[2]) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(v[0], v[1]);
  }
};
template <>
struct Chan<uint16_t, 1> {
  static __device__ __forceinline__ void load(const uint16_t* p, float (&v)[1]) { v[0] = bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(uint16_t* p, const float (&v)[1]) { *p = f32_to_bf16(v[0]); }
};
template <>
struct Chan<float, 2> {
  static __device__ __forceinline__ void load(const float* p, float (&v)[2]) {
    const f32x2 w = *reinterpret_cast<const f32x2*>(p);
    v[0] = w[0];
    v[1] = w[1];
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[2]) {
    *reinterpret_cast<f32x2*>(p) = f32x2{v[0], v[1]};
  }
};
template <>
struct Chan<float, 1> {
  static __device__ __forceinline__ void load(const float* p, float (&v)[1]) { v[0] = *p; }
  static __device__ __forceinline__ void store(float* p, const float (&v)[1]) { *p = v[0]; }
};

template <int D, typename IO>
__global__ __launch_bounds__(kConvWaves * 64) void gdn_conv_kernel(const ConvArgs a) {
  constexpr int CPL = D / 64;  // channels per lane
  using CH = Chan<IO, CPL>;
  const int C = a.H * D;
  // window input i: s_src[i] 0 none (zeros), 1 a node row of x, 2 a trunk
  // row of trunk_x; s_row[i] that row's index
  __shared__ long long s_row[kConvMaxK];
  __shared__ int s_src[kConvMaxK];
  __shared__ int s_ok;
  const int node = blockIdx.x;  // (trunk * B + branch) * Wn + j
  const int tb = node / a.Wn, j = node - tb * a.Wn;
  const int t = tb / a.B;
  if (threadIdx.x == 0) {
    const int32_t* par = a.parent + size_t(tb) * a.Wn;
    const int anc = a.anchors[tb];
    bool ok = anc >= 0 && anc < a.L;
    int x = j, s = anc;
    for (int i = 0; i < a.K; ++i) {
      int src = 0;
      long long row = 0;
      if (x >= 0) {
        src = 1;
        row = (long long)tb * a.Wn + x;
        const int p = par[x];
        ok = ok && p >= -1 && p < x;  // a parent precedes its child
        x = ok ? p : -1;
      } else if (s >= 0) {
        src = 2;
        row = (long long)t * a.L + s;
        --s;
      }
      s_src[i] = ok ? src : 0;
      s_row[i] = row;
    }
    s_ok = ok;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const bool ok = s_ok;
  const IO* const xb = static_cast<const IO*>(a.x);
  const IO* const tx = static_cast<const IO*>(a.trunk_x);
  IO* const ob = static_cast<IO*>(a.out) + size_t(node) * C;
  for (int h = wave; h < a.H; h += kConvWaves) {
    const int c0 = h * D + lane * CPL;  // this lane's first channel
    float z[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) z[e] = 0.f;
    for (int i = 0; i < a.K; ++i) {
      const int src = s_src[i];
      if (src == 0) continue;
      float v[CPL];
      CH::load((src == 1 ? xb : tx) + size_t(s_row[i]) * C + c0, v);
#pragma unroll
      for (int e = 0; e < CPL; ++e) z[e] = __builtin_fmaf(a.w[size_t(c0 + e) * a.K + i], v[e], z[e]);
    }
    float y[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) y[e] = z[e] / (1.f + fast_exp2(-z[e] * kLog2e));  // SiLU
    if (a.l2norm) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < CPL; ++e) ss = __builtin_fmaf(y[e], y[e], ss);
      ss = wave_sum(ss);
      const float sc = 1.f / __builtin_sqrtf(ss + 1e-6f);
#pragma unroll
      for (int e = 0; e < CPL; ++e) y[e] *= sc;
    }
    if (!ok) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) y[e] = __builtin_nanf("");
    }
    CH::store(ob + c0, y);
  }
}

}  // namespace

hipError_t launch_gdn_conv(const specopd_gdn_conv_desc& d, const void* trunk_x, const void* x, const float* w,
                           const int32_t* anchors, const int32_t* parent, void* out, hipStream_t s) {
  ConvArgs a{};
  a.trunk_x = trunk_x;
  a.x = x;
  a.w = w;
  a.anchors = anchors;
  a.parent = parent;
  a.out = out;
  a.L = d.L; a.B = d.B; a.Wn = d.Wn; a.H = d.H; a.K = d.K;
  a.l2norm = (d.flags & SPECOPD_GDN_CONV_L2NORM) != 0;
  const dim3 grid(unsigned(size_t(d.T) * d.B * d.Wn));
  const bool bf = d.dtype == SPECOPD_BF16;
  if (d.D == 128) {
    if (bf) gdn_conv_kernel<128, uint16_t><<<grid, kConvWaves * 64, 0, s>>>(a);
    else gdn_conv_kernel<128, float><<<grid, kConvWaves * 64, 0, s>>>(a);
  } else {
    if (bf) gdn_conv_kernel<64, uint16_t><<<grid, kConvWaves * 64, 0, s>>>(a);
    else gdn_conv_kernel<64, float><<<grid, kConvWaves * 64, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace specopd
