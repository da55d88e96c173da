// DFlash2's dynamic grouped convolution around attention and MLP [NIF,
// DFlash2 layer equations]: for the branch's normalised input X,
//   Conv_s(X)[i, g, j] = (base[s,0,g,j] + delta[i,s,0,g]) X[i,g,j]
//                      + [i >= 1] (base[s,1,g,j] + delta[i,s,1,g]) X[i-1,g,j]
// with delta = W_delta X (a streamed GEMM), increments shared by the
// channels of a group and no tap before a block's row 0.  The prepare side
// (s = 0) feeds the branch's projections; the finish side (s = 1) applies
// the same delta to the branch output and adds it to the residual.
// One workgroup per row; four consecutive channels per thread (a group
// holds a multiple of four channels).
#include "conv_internal.hpp"
#include "dspine_device.hpp"

namespace dspine {

constexpr int kConvThreads = 256;
constexpr int kConvBatch = 8;            // float4 steps per thread held in flight (H <= 8192)

__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
template <typename T>
__device__ __forceinline__ f32x4 load4t(const T* p, int k) {
  return f32x4{Elt<T>::load(p, k), Elt<T>::load(p, k + 1), Elt<T>::load(p, k + 2), Elt<T>::load(p, k + 3)};
}

// row scale rsqrt(S / H + eps) of row m from its statistics lists
__device__ __forceinline__ float norm_scale(const ConvParams& p, int m) {
  float v = 0.f;
  for (int t = threadIdx.x & 63; t < p.lists; t += 64) v += p.stats[(size_t)t * p.ld + m];
  return rsqrtf(wave_sum(v) / p.H + p.eps);
}

template <typename TW>
__global__ __launch_bounds__(kConvThreads) void conv_prepare_kernel(const ConvParams p) {
  using TA = typename ActOf<TW>::type;
  const int m = blockIdx.x, i = m % p.W, H = p.H;
  const float s_cur = norm_scale(p, m);
  const float s_prev = i > 0 ? norm_scale(p, m - 1) : 0.f;
  const TW* base = reinterpret_cast<const TW*>(p.base);
  const TW* gain = reinterpret_cast<const TW*>(p.gain);
  const float* d = p.delta + (size_t)m * 4 * p.G;
  TA* out = reinterpret_cast<TA*>(p.act) + (size_t)m * H;
#pragma unroll
  for (int q = 0; q < kConvBatch; ++q) {
    const int k = 4 * (threadIdx.x + q * kConvThreads);
    if (k >= H) continue;
    const int g = k / p.cg;
    const f32x4 gn = load4t(gain, k);
    const f32x4 xc = load4(p.x + (size_t)m * H + k) * (s_cur * gn);
    f32x4 r = (load4t(base, k) + d[g]) * xc;
    if (i > 0) {
      const f32x4 xp = load4(p.x + (size_t)(m - 1) * H + k) * (s_prev * gn);
      r += (load4t(base, H + k) + d[p.G + g]) * xp;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) Elt<TA>::store(out, k + e, r[e]);
  }
}

template <typename TW>
__global__ __launch_bounds__(kConvThreads) void conv_finish_kernel(const ConvParams p) {
  __shared__ float red[kConvThreads / 64];
  const int m = blockIdx.x, i = m % p.W, H = p.H;
  const TW* base = reinterpret_cast<const TW*>(p.base);
  const float* d = p.delta + (size_t)m * 4 * p.G;
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < kConvBatch; ++q) {
    const int k = 4 * (threadIdx.x + q * kConvThreads);
    if (k >= H) continue;
    const int g = k / p.cg;
    f32x4 v = load4(p.x_out + (size_t)m * H + k) + (load4t(base, 2 * H + k) + d[2 * p.G + g]) * load4(p.o + (size_t)m * H + k);
    if (i > 0) v += (load4t(base, 3 * H + k) + d[3 * p.G + g]) * load4(p.o + (size_t)(m - 1) * H + k);
    *reinterpret_cast<f32x4*>(p.x_out + (size_t)m * H + k) = v;
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  const float tot = block_sum<kConvThreads>(ss, red);
  if (threadIdx.x == 0) p.stats_out[m] = tot;
}

hipError_t launch_conv_prepare(const ConvParams& p, int dtype, hipStream_t s) {
  if (p.H > 4 * kConvThreads * kConvBatch || p.H % 4 || p.cg % 4) return hipErrorInvalidValue;
  if (dtype == DT_BF16) DSPINE_LAUNCH(conv_prepare_kernel<bf16_t>, dim3(p.M), dim3(kConvThreads), 0, s, p);
  else DSPINE_LAUNCH(conv_prepare_kernel<float>, dim3(p.M), dim3(kConvThreads), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_conv_finish(const ConvParams& p, int dtype, hipStream_t s) {
  if (p.H > 4 * kConvThreads * kConvBatch || p.H % 4 || p.cg % 4) return hipErrorInvalidValue;
  if (dtype == DT_BF16) DSPINE_LAUNCH(conv_finish_kernel<bf16_t>, dim3(p.M), dim3(kConvThreads), 0, s, p);
  else DSPINE_LAUNCH(conv_finish_kernel<float>, dim3(p.M), dim3(kConvThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dspine
