// Row-wise kernels: the block input gather (a4), plain RMSNorm (a12 and the
// context norm of long materialize blocks), row statistics, and the context
// K/V store epilogue (a2).
// One workgroup per row; statistics in fp32.
#include <algorithm>

#include "dspine_device.hpp"
#include "dspine_internal.hpp"

namespace dspine {

constexpr int kRowThreads = 256;

// (cos, sin) of position * theta^(-2j/D), angle formed in double precision so
// that positions of tens of thousands keep full float accuracy.
__device__ __forceinline__ void rope_pair(int64_t pos, int j, int D, float theta, float& c, float& s) {
  const double inv_freq = exp2(-(2.0 * j / D) * log2((double)theta));
  const double ang = (double)pos * inv_freq;
  double sd, cd;
  sincos(ang, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

// a4 [NIF, draft input]: x[m] = embed[token(m)], row 0 of each request the
// anchor and rows 1..W-1 the mask token.  Also the row's sum of squares (one
// statistics tile, from which the first input norm is formed in the QKV
// projection, or, with `act`, that norm itself as the projection's operand)
// and the rotation table of the row's position F + i.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void embed_kernel(const RowParams p) {
  __shared__ float red[kRowThreads / 64];
  const int m = blockIdx.x, b = m / p.W, i = m % p.W;
  const int tok = i == 0 ? p.anchor[b] : p.mask_id;
  const gptr<T> e = as_global(reinterpret_cast<const T*>(p.embed)) + (size_t)tok * p.H;
  float ss = 0.f;
#pragma unroll 4
  for (int k = threadIdx.x; k < p.H; k += kRowThreads) {
    const float v = Elt<T>::gload(e, k);
    p.x_out[(size_t)m * p.H + k] = v;
    ss += v * v;
  }
  ss = block_sum<kRowThreads>(ss, red);
  if (threadIdx.x == 0) p.stats[m] = ss;
  if (p.act) {
    // the first input norm as the q|k|v operand, (x * rsqrt(S / H + eps)) *
    // gain, with the factor the pre-scale kernel forms from this one list
    using TA = typename ActOf<T>::type;
    const float inv = rsqrtf(ss / p.H + p.eps);
    const gptr<T> gn = as_global(reinterpret_cast<const T*>(p.gain));
    TA* out = reinterpret_cast<TA*>(p.act) + (size_t)m * p.H;
#pragma unroll 4
    for (int k = threadIdx.x; k < p.H; k += kRowThreads)
      Elt<TA>::store(out, k, p.x_out[(size_t)m * p.H + k] * inv * Elt<T>::gload(gn, k));
  }
  for (int j = threadIdx.x; j < p.head_dim / 2; j += kRowThreads) {
    float c, s;
    rope_pair(p.F[b] + i, j, p.head_dim, p.rope_theta, c, s);
    p.rope[(size_t)m * p.head_dim + 2 * j] = c;
    p.rope[(size_t)m * p.head_dim + 2 * j + 1] = s;
  }
}

// Sum of squares of each row of x (one statistics tile): the bridge called
// on its own receives x without statistics.
__global__ __launch_bounds__(kRowThreads) void rowstats_kernel(const RowParams p) {
  __shared__ float red[kRowThreads / 64];
  const int m = blockIdx.x;
  const gptr<float> x = as_global(p.x) + (size_t)m * p.H;
  float ss = 0.f;
#pragma unroll 4
  for (int k = threadIdx.x; k < p.H; k += kRowThreads) ss += x[k] * x[k];
  ss = block_sum<kRowThreads>(ss, red);
  if (threadIdx.x == 0) p.stats[m] = ss;
}

// act[m, k] = x[m, k] * s[m] (* gain[k]) in the operand type.  One wave per
// row forms s[m] from the row's statistics lists (a fixed split over lanes
// and a fixed reduction order); grid (column blocks of 2048, rows).
template <typename T>
__global__ __launch_bounds__(256) void scale_rows_kernel(const ScaleParams p) {
  __shared__ float s_row;
  const int m = blockIdx.y;
  if (threadIdx.x < 64) {
    float v = 0.f;
    if (p.mode != SCALE_ONE)
      for (int t = threadIdx.x; t < p.lists; t += 64) v += p.stats[(size_t)t * p.ld + m];
    v = wave_sum(v);
    if (threadIdx.x == 0)
      s_row = p.mode == SCALE_ONE ? 1.f : row_scale(p.mode, v, p.n, p.eps, p.code_scale, m % p.W == 0);
  }
  __syncthreads();
  const float sc = s_row;
  using TA = typename ActOf<T>::type;
  constexpr int EPC = 8;
  const int k = (blockIdx.x * 256 + threadIdx.x) * EPC;
  if (k >= p.K) return;
  const gptr<float> x = as_global(p.x) + (size_t)m * p.ldx + k;
  const gptr<T> gn = as_global(reinterpret_cast<const T*>(p.gain)) + k;
  TA* out = reinterpret_cast<TA*>(p.act) + (size_t)m * p.ld_act + k;
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    const float g = p.gain ? Elt<T>::gload(gn, e) : 1.f;
    const float v = x[e] * sc * g;
    Elt<TA>::store(out, e, p.round_bf16 ? round_bf16(v) : v);
  }
}

// act[t, k] = sigmoid(P[t, k] + Pp[tp, a + k] + b[k]) * Pp[tp, 2a + k] for
// receiver rows t (tp = t - 1, or t with an override), zero at anchor rows
// [FLZ, "The bridge"]; grid (column blocks of 256, rows).
template <typename T>
__global__ __launch_bounds__(256) void bridge_msg_kernel(const ScaleParams p) {
  const int m = blockIdx.y;
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= p.K) return;
  using TA = typename ActOf<T>::type;
  TA* out = reinterpret_cast<TA*>(p.act) + (size_t)m * p.ld_act;
  if (m % p.W == 0) {
    Elt<TA>::store(out, k, 0.f);
    return;
  }
  const int tp = p.pred_shift ? m - 1 : m;
  const int a = p.K, a3 = 3 * p.K;
  const float gpre = p.P[(size_t)m * a3 + k] + p.Ppred[(size_t)tp * a3 + a + k] +
                     Elt<T>::load(reinterpret_cast<const T*>(p.bias), k);
  Elt<TA>::store(out, k, sigmoid(gpre) * p.Ppred[(size_t)tp * a3 + 2 * a + k]);
}

// plain_rmsnorm [NIF]: out = g * x / sqrt(mean(x^2) + eps); out in the model
// dtype (GEMM operand), bf16 (operand of the tile GEMM's bf16 x bf16 path)
// or fp32 (final hidden states).
template <typename T, bool F32OUT>
__global__ __launch_bounds__(kRowThreads) void rmsnorm_kernel(const RowParams p) {
  __shared__ float red[kRowThreads / 64];
  const int m = blockIdx.x;
  const gptr<float> x = as_global(p.x) + (size_t)m * p.H;
  float ss = 0.f;
  if (p.nlists > 0) {
    // the row's sum of squares from the statistics lists of x, summed as the
    // pre-scale kernel and the fused bridge sum them (so that a norm formed
    // there and one formed here are the same bits)
    if (threadIdx.x < 64) {
      for (int t = threadIdx.x; t < p.nlists; t += 64) ss += p.lists[(size_t)t * p.ld + m];
      ss = wave_sum(ss);
      if (threadIdx.x == 0) red[0] = ss;
    }
    __syncthreads();
    ss = red[0];
  } else {
#pragma unroll 4
    for (int k = threadIdx.x; k < p.H; k += kRowThreads) ss += x[k] * x[k];
    ss = block_sum<kRowThreads>(ss, red);
  }
  const float inv = rsqrtf(ss / p.H + p.eps);
  const gptr<T> gw = as_global(reinterpret_cast<const T*>(p.gain));
#pragma unroll 4
  for (int k = threadIdx.x; k < p.H; k += kRowThreads) {
    const float v = x[k] * inv * Elt<T>::gload(gw, k);
    if (F32OUT) p.f32_out[(size_t)m * p.H + k] = v;
    else if (p.act_bf16) Elt<bf16_t>::store(reinterpret_cast<bf16_t*>(p.act), (size_t)m * p.H + k, v);
    else Elt<typename ActOf<T>::type>::store(reinterpret_cast<typename ActOf<T>::type*>(p.act), (size_t)m * p.H + k, v);
  }
}

// a2 epilogue [NIF, context K/V; fused context materializer], for every
// layer of the launch at once (grid: rows x layers): k =
// rope_1d(head_rmsnorm(k_raw, gk), t) stored BF16 (no rounding before the
// norm); v stored FP16_RNE(BF16(v_raw)).  F32 models store float.  Rows at
// positions below keep_lo are not stored (chunk truncation); position t
// goes to ring slot t mod S (t for a full layer).  Each thread holds 4
// consecutive elements of a head; a head's sum of squares is reduced over
// its D/4 threads in a fixed butterfly order.
template <typename T>
__global__ __launch_bounds__(kRowThreads) void kv_store_kernel(const KvStoreParams p) {
  extern __shared__ __align__(16) float sm[];   // (cos, sin) x D/2, then nkv*D raw keys, then nkv head sums
  const int row = blockIdx.x;
  int b = 0;
  while (b + 1 < p.n_req && row >= p.row0[b + 1]) ++b;
  const int64_t t = p.pos0[b] + (row - p.row0[b]);
  const int D = p.D, half = D / 2, n = p.nkv * D;
  float* cs = sm;
  float* kraw = sm + D;
  for (int j = threadIdx.x; j < half; j += kRowThreads) rope_pair(t, j, D, p.rope_theta, cs[2 * j], cs[2 * j + 1]);
  // layers [l0, l1) of this row (the rotation table is shared by them)
  const int l0 = blockIdx.y * p.lpw, l1 = l0 + p.lpw < p.n_layers ? l0 + p.lpw : p.n_layers;
  for (int l = l0; l < l1; ++l) {
    if (t < p.keep_lo[l][b]) continue;                        // uniform over the workgroup
    const float* kr = p.kv + (size_t)row * p.ld + p.col[l];
    const float* vr = kr + n;
    const int S = p.S[l];
    const size_t slot = (size_t)ring_slot(t, S);
    const size_t cap = (size_t)p.cap[l][b];
    const T* gk = reinterpret_cast<const T*>(p.gk[l]);
    // the head sum needs the D/4 threads of a head inside one wave: 4 * 64 >= D
    for (int e0 = 4 * threadIdx.x; e0 < n; e0 += 4 * kRowThreads) {
      const float4 kv4 = *reinterpret_cast<const float4*>(kr + e0);
      *reinterpret_cast<float4*>(kraw + e0) = kv4;
      float ss = ((kv4.x * kv4.x + kv4.y * kv4.y) + kv4.z * kv4.z) + kv4.w * kv4.w;
      for (int o = 1; o < D / 4; o <<= 1) ss += __shfl_xor(ss, o, 64);
      kraw[n + e0 / D] = ss;                                  // per-head sum (same in all its threads)
      // v: FP16_RNE(BF16(v)) (or float), 4 consecutive elements in one store
      const float4 v4 = *reinterpret_cast<const float4*>(vr + e0);
      const int hh = e0 / D, d = e0 % D;
      const size_t vi = ((size_t)hh * cap + slot) * D + d;
      if constexpr (Elt<T>::kBytes == 2) {
        auto h = [](float v) { return (uint32_t)f32_to_f16_bits(bf16_bits_to_f32(f32_to_bf16_bits(v))); };
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.vring[l][b]) + vi) =
            uint2{h(v4.x) | (h(v4.y) << 16), h(v4.z) | (h(v4.w) << 16)};
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.vring[l][b]) + vi) = v4;
      }
    }
    __syncthreads();
    // k: head norm, rotation of the pairs (j, j + D/2), two consecutive j per thread
    for (int e = threadIdx.x; e < p.nkv * half / 2; e += kRowThreads) {
      const int hh = e / (half / 2), j = 2 * (e % (half / 2));
      const float inv = rsqrtf(kraw[n + hh] / D + p.eps);
      float lo[2], hi[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float a = kraw[hh * D + j + u] * inv * Elt<T>::load(gk, j + u);
        const float c = kraw[hh * D + j + u + half] * inv * Elt<T>::load(gk, j + u + half);
        const float co = cs[2 * (j + u)], si = cs[2 * (j + u) + 1];
        lo[u] = a * co - c * si;
        hi[u] = c * co + a * si;
      }
      const size_t base = ((size_t)hh * cap + slot) * D;
      if constexpr (Elt<T>::kBytes == 2) {
        uint16_t* K = reinterpret_cast<uint16_t*>(p.kring[l][b]);
        *reinterpret_cast<uint32_t*>(K + base + j) =
            (uint32_t)f32_to_bf16_bits(lo[0]) | ((uint32_t)f32_to_bf16_bits(lo[1]) << 16);
        *reinterpret_cast<uint32_t*>(K + base + j + half) =
            (uint32_t)f32_to_bf16_bits(hi[0]) | ((uint32_t)f32_to_bf16_bits(hi[1]) << 16);
      } else {
        float* K = reinterpret_cast<float*>(p.kring[l][b]);
        *reinterpret_cast<float2*>(K + base + j) = float2{lo[0], lo[1]};
        *reinterpret_cast<float2*>(K + base + j + half) = float2{hi[0], hi[1]};
      }
    }
    __syncthreads();                                          // kraw is rewritten by the next layer
  }
}

// Fragment order of a projection matrix W [R, K] (R % 16 == 0, K % 32 == 0):
// block b (rows 16b..16b+15) keeps its place; inside it, 32-wide K step ks
// holds 64 lane fragments, lane l = row 16b + l%16, columns ks*32 + 8*(l/16)
// .. +8, at element offset (b*(K/32) + ks)*512 + 8*l.  This is the order in
// which a wave's MFMA fragments are loaded, so each load reads 1 KB
// (bf16; 2 KB for float) of consecutive memory.
// *out = max(*out, |x|) over bf16 values, compared as float bits (for
// non-negative floats the bit order is the value order; NaN ranks highest)
__global__ __launch_bounds__(256) void absmax_bf16_kernel(const uint16_t* src, size_t n, uint32_t* out) {
  uint32_t m = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    m = max(m, ((uint32_t)src[i] & 0x7fffu) << 16);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  if ((threadIdx.x & 63) == 0) atomicMax(out, m);
}

hipError_t launch_absmax_bf16(const void* src, size_t n, uint32_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  DSPINE_LAUNCH(absmax_bf16_kernel, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0, s,
                static_cast<const uint16_t*>(src), n, out);
  return hipGetLastError();
}

// words [0, n) of p <- 0 (a plain kernel, not a memset node, so that it can
// sit in a captured graph)
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_zero_words(void* p, size_t n_words, hipStream_t s) {
  if (n_words == 0) return hipSuccess;
  const size_t blocks = (n_words + 255) / 256;
  DSPINE_LAUNCH(zero_words_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s,
                static_cast<uint32_t*>(p), n_words);
  return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(const T* src, T* dst, int R, int K) {
  const size_t nfrag = (size_t)(R / 16) * (K / 32) * 64;
  for (size_t f = blockIdx.x * (size_t)blockDim.x + threadIdx.x; f < nfrag; f += (size_t)gridDim.x * blockDim.x) {
    const size_t blk = f / 64;
    const int l = (int)(f % 64);
    const size_t rb = blk / (K / 32);
    const int ks = (int)(blk % (K / 32));
    const T* s = src + (rb * 16 + (l & 15)) * (size_t)K + ks * 32 + 8 * (l >> 4);
    T* d = dst + blk * 512 + l * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = s[j];
  }
}

// a3 as evaluated by the attention kernel (same device predicate)
__global__ void debug_visible_kernel(const VisibleParams p) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= p.B * p.W) return;
  const int b = m / p.W, i = m % p.W;
  const int64_t F = p.F[b];
  const int64_t lo = ctx_row_lo(F, p.S, i);
  p.lo_hi[2 * m] = lo;
  p.lo_hi[2 * m + 1] = F;
  p.first_slot[m] = lo < F ? (int32_t)ring_slot(lo, p.S) : -1;
  int n = 0;
  for (int j = 0; j < p.W; ++j) n += block_key_visible(p.S, p.causal, i, j) ? 1 : 0;
  p.n_block[m] = n;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#define DSPINE_DISPATCH(dtype, KERNEL, ...)                                               \
  do {                                                                                    \
    if ((dtype) == DT_BF16) DSPINE_LAUNCH((KERNEL<bf16_t>), __VA_ARGS__);            \
    else DSPINE_LAUNCH((KERNEL<float>), __VA_ARGS__);                                \
  } while (0)

hipError_t launch_embed(const RowParams& p, int dtype, hipStream_t s) {
  DSPINE_DISPATCH(dtype, embed_kernel, dim3(p.M), dim3(kRowThreads), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_rmsnorm(const RowParams& p, int dtype, bool f32_output, hipStream_t s) {
  if (dtype == DT_BF16) {
    if (f32_output) DSPINE_LAUNCH((rmsnorm_kernel<bf16_t, true>), dim3(p.M), dim3(kRowThreads), 0, s, p);
    else DSPINE_LAUNCH((rmsnorm_kernel<bf16_t, false>), dim3(p.M), dim3(kRowThreads), 0, s, p);
  } else {
    if (f32_output) DSPINE_LAUNCH((rmsnorm_kernel<float, true>), dim3(p.M), dim3(kRowThreads), 0, s, p);
    else DSPINE_LAUNCH((rmsnorm_kernel<float, false>), dim3(p.M), dim3(kRowThreads), 0, s, p);
  }
  return hipGetLastError();
}
hipError_t launch_scale_rows(const ScaleParams& p, int dtype, hipStream_t s) {
  if (p.K % 8) return hipErrorInvalidValue;
  DSPINE_DISPATCH(dtype, scale_rows_kernel, dim3((p.K / 8 + 255) / 256, p.M), dim3(256), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_bridge_msg(const ScaleParams& p, int dtype, hipStream_t s) {
  DSPINE_DISPATCH(dtype, bridge_msg_kernel, dim3((p.K + 255) / 256, p.M), dim3(256), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_rowstats(const RowParams& p, hipStream_t s) {
  DSPINE_LAUNCH(rowstats_kernel, dim3(p.M), dim3(kRowThreads), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_kv_store(const KvStoreParams& p, int dtype, hipStream_t s) {
  if (p.n_layers < 1 || p.n_layers > kKvLayers || p.D % 4 || 4 * 64 < p.D) return hipErrorInvalidValue;
  const size_t smem = (size_t)(p.D + p.nkv * p.D + p.nkv) * sizeof(float);
  // many rows: one workgroup per row walks every layer (one rotation table,
  // a fifth of the workgroups); few rows: one per row and layer, for width
  KvStoreParams q = p;
  q.lpw = p.rows >= 1024 ? p.n_layers : 1;
  DSPINE_DISPATCH(dtype, kv_store_kernel, dim3(p.rows, (p.n_layers + q.lpw - 1) / q.lpw), dim3(kRowThreads), smem, s, q);
  return hipGetLastError();
}
hipError_t launch_pack(const void* src, void* dst, int rows, int cols, int dtype, hipStream_t s) {
  const size_t nfrag = (size_t)(rows / 16) * (cols / 32) * 64;
  const int grid = (int)std::min<size_t>((nfrag + 255) / 256, 8192);
  if (dtype == DT_BF16)
    DSPINE_LAUNCH((pack_kernel<uint16_t>), dim3(grid), dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), rows, cols);
  else
    DSPINE_LAUNCH((pack_kernel<float>), dim3(grid), dim3(256), 0, s,
                       static_cast<const float*>(src), static_cast<float*>(dst), rows, cols);
  return hipGetLastError();
}

hipError_t launch_debug_visible(const VisibleParams& p, hipStream_t s) {
  const int n = p.B * p.W;
  DSPINE_LAUNCH(debug_visible_kernel, dim3((n + 63) / 64), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace dspine
