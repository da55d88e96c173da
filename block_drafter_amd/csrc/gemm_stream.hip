// Weight-streaming GEMM for the draft forward and decode-round materialization.
//
//   out[m, n] (op)= sum_k A[m, k] * W[n, k]     m < M <= 128, n < N, k < K
//
// The block has only B*W <= 128 activation rows, so every projection of the
// draft layers is bound by reading W once from HBM.  Design for gfx950:
//  * W rows stream straight from HBM into registers as MFMA fragments (16 B
//    per lane per 32 K) and are double-buffered in registers across
//    iterations; A (tiny) is staged once per workgroup iteration in LDS and
//    shared by the four waves.
//  * Stream-K: the (tile, k-iteration) space is cut into equal contiguous
//    ranges, one per workgroup, so every CU streams the same number of bytes
//    whatever N and K are.  A tile split between workgroups is finished by the
//    last one to arrive (device-scope counter), which adds the published
//    partials and runs the epilogue: no accumulator buffer needs zeroing and
//    epilogues (residual add, SwiGLU) stay fused.
//  * Weights are the MFMA A operand (16 rows = 16 output columns n) and the
//    activations the B operand (16 columns = 16 rows m), so each lane ends up
//    with 4 consecutive n of one m: 16-byte epilogue stores.
//  * Operand types: a BF16 model multiplies FP16 activations by its bf16
//    weights widened to fp16 in registers (exact); bf16 target features are
//    used as they are (bf16 x bf16).  A float32 model uses fp32 MFMAs.
#include "dspine_device.hpp"
#include "dspine_internal.hpp"

namespace dspine {

namespace {

__device__ __forceinline__ int64_t iter_begin(int g, int64_t TI, int G) {
  return (int64_t)g * TI / G;
}
// workgroup whose range holds iteration i
__device__ __forceinline__ int owner_of(int64_t i, int64_t TI, int G) {
  return (int)(((i + 1) * (int64_t)G - 1) / TI);
}

template <typename T>
__device__ __forceinline__ const T* seg_row_ptr(const GemmParams& p, int vb, int& valid) {
  valid = 0;
  if (vb >= p.nblk) return nullptr;
  valid = 1;
  if (p.interleave) {
    return reinterpret_cast<const T*>(p.seg_ptr[vb & 1]) + (size_t)(vb >> 1) * 16 * p.K;
  }
  int s = 0;
#pragma unroll 1
  while (s + 1 < p.nseg && vb >= p.seg_blk0[s + 1]) ++s;
  return reinterpret_cast<const T*>(p.seg_ptr[s]) + (size_t)(vb - p.seg_blk0[s]) * 16 * p.K;
}

// Fill one 16-byte chunk of the A tile: row m, columns k..k+EPC (TA elements).
template <typename TW, typename TA>
__device__ __forceinline__ u32x4 load_a_chunk(const GemmParams& p, int m, int k) {
  constexpr int EPC = 16 / Elt<TA>::kBytes;
  u32x4 r = {0, 0, 0, 0};
  if (m >= p.M || k >= p.K) return r;
  if (p.pro == PRO_COPY) {
    const TA* a = reinterpret_cast<const TA*>(p.a) + (size_t)m * p.lda + k;
    return *reinterpret_cast<const u32x4*>(a);
  }
  if (p.pro == PRO_GATHER) {
    int s = 0;
#pragma unroll 1
    while (s + 1 < p.g_n && m >= p.g_row0[s + 1]) ++s;
    const TA* a = reinterpret_cast<const TA*>(p.g_src[s]) +
                  (size_t)(m - p.g_row0[s] + p.g_skip[s]) * p.lda + k;
    return *reinterpret_cast<const u32x4*>(a);
  }
  // PRO_BRIDGE_MSG: A[t, k] = sigmoid(P[t, k] + Pp[tp, a + k] + b[k]) * Pp[tp, 2a + k]
  // (the receiver's rms multiplies the product in the epilogue)
  const int i = m % p.W;
  if (i == 0) return r;                       // anchors receive no message
  const int tp = p.pred_shift ? m - 1 : m;
  const int a3 = 3 * p.a_dim;
  const float* P = p.P + (size_t)m * a3;
  const float* Pp = p.Ppred + (size_t)tp * a3;
  const TW* bias = reinterpret_cast<const TW*>(p.bias);
  float v[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    const int kk = k + e;
    const float gpre = P[kk] + Pp[p.a_dim + kk] + Elt<TW>::load(bias, kk);
    v[e] = sigmoid(gpre) * Pp[2 * p.a_dim + kk];
  }
  TA* out = reinterpret_cast<TA*>(&r);
#pragma unroll
  for (int e = 0; e < EPC; ++e) Elt<TA>::store(out, e, v[e]);
  return r;
}

}  // namespace

template <typename TW, typename TA, int MT, int NWB, int KSUB>
__global__ __launch_bounds__(256) void gemm_stream_kernel(const GemmParams p) {
  using T = TA;                                 // LDS / MFMA operand type
  constexpr int EB = Elt<TA>::kBytes;
  constexpr int KS = 32 * KSUB;                 // K elements per iteration
  constexpr int EPC = 16 / EB;                  // elements per 16-byte chunk
  constexpr int LDA = KS + EPC;                 // LDS row stride (16 B padding)
  constexpr int MP = MT * 16;
  constexpr int CPR = KS / EPC;                 // chunks per A row
  constexpr int NCH = MP * CPR / 256;           // chunks per thread
  static_assert(NCH >= 1 && (MP * CPR) % 256 == 0, "A tile must split over 256 threads");
  constexpr int WG_BLKS = 4 * NWB;              // 16-row weight blocks per tile

  __shared__ __attribute__((aligned(16))) T lds[2][MP * LDA];
  __shared__ uint32_t s_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int G = gridDim.x;
  int g = blockIdx.x;
  if (p.xcd_remap) g = (g % 8) * (G / 8) + g / 8;   // neighbours in k-space share an XCD

  const int64_t TI = (int64_t)p.tiles * p.ipt;
  const int64_t it_beg = iter_begin(g, TI, G);
  const int64_t it_end = iter_begin(g + 1, TI, G);
  if (it_beg >= it_end) return;

  f32x4 acc[NWB][MT];
#pragma unroll
  for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) acc[nb][mb] = f32x4{0, 0, 0, 0};

  Frag<TW> wf0[NWB][KSUB], wf1[NWB][KSUB];
  u32x4 areg[NCH];

  auto load_iter = [&](int64_t it, Frag<TW> (&wf)[NWB][KSUB]) {
    const int tile = (int)(it / p.ipt);
    const int k0 = (int)(it % p.ipt) * KS;
    // A tile chunks first: the LDS store waits only for these (older) loads
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int c = tid + q * 256;
      areg[q] = load_a_chunk<TW, TA>(p, c / CPR, k0 + (c % CPR) * EPC);
    }
#pragma unroll
    for (int nb = 0; nb < NWB; ++nb) {
      int valid;
      const TW* wr = seg_row_ptr<TW>(p, tile * WG_BLKS + wave * NWB + nb, valid);
#pragma unroll
      for (int s = 0; s < KSUB; ++s) {
        const int k = k0 + s * 32 + 8 * (lane >> 4);
        if (valid && k < p.K) wf[nb][s].load(wr + (size_t)(lane & 15) * p.K + k);
        else wf[nb][s].zero();
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int c = tid + q * 256;
      *reinterpret_cast<u32x4*>(&lds[buf][(c / CPR) * LDA + (c % CPR) * EPC]) = areg[q];
    }
  };
  auto compute = [&](int buf, Frag<TW> (&wf)[NWB][KSUB]) {
#pragma unroll
    for (int s = 0; s < KSUB; ++s) {
      Frag<T> wo[NWB];
#pragma unroll
      for (int nb = 0; nb < NWB; ++nb) wo[nb] = AsOperand<T, TW>::cvt(wf[nb][s]);
#pragma unroll
      for (int mb = 0; mb < MT; ++mb) {
        Frag<T> af;
        af.load(&lds[buf][(mb * 16 + (lane & 15)) * LDA + s * 32 + 8 * (lane >> 4)]);
#pragma unroll
        for (int nb = 0; nb < NWB; ++nb) mma16(acc[nb][mb], wo[nb], af);
      }
    }
  };

  // Finish tile `tile` whose iterations [kb, ke) this workgroup has accumulated.
  auto finish = [&](int tile, int kb, int ke) {
    const bool whole = (kb == 0 && ke == p.ipt);
    if (!whole) {
      const int64_t t0 = (int64_t)tile * p.ipt;
      const int g_first = owner_of(t0, TI, G);
      const int g_last = owner_of(t0 + p.ipt - 1, TI, G);
      const int ncontrib = g_last - g_first + 1;
      auto slot_of = [&](int gg) {
        const int first_tile = (int)(iter_begin(gg, TI, G) / p.ipt);
        return 2 * gg + (first_tile == tile ? 0 : 1);
      };
      float* mine = p.partials + (size_t)slot_of(g) * (NWB * MT * 256 * 4);
#pragma unroll
      for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MT; ++mb)
          *reinterpret_cast<f32x4*>(mine + ((nb * MT + mb) * 256 + tid) * 4) = acc[nb][mb];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      if (tid == 0) s_flag = arrive(p.counters + tile);
      __syncthreads();
      if ((int)s_flag != ncontrib - 1) {
#pragma unroll
        for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
          for (int mb = 0; mb < MT; ++mb) acc[nb][mb] = f32x4{0, 0, 0, 0};
        return;
      }
      acquire_partials();
      // add the contributions in workgroup order, whoever finishes, so the
      // result does not depend on arrival order (bit-reproducible runs)
      f32x4 sum[NWB][MT];
#pragma unroll
      for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) sum[nb][mb] = f32x4{0, 0, 0, 0};
      for (int gg = g_first; gg <= g_last; ++gg) {
        const float* other = p.partials + (size_t)slot_of(gg) * (NWB * MT * 256 * 4);
#pragma unroll
        for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
          for (int mb = 0; mb < MT; ++mb) {
            if (gg == g) sum[nb][mb] += acc[nb][mb];
            else sum[nb][mb] += *reinterpret_cast<const f32x4*>(other + ((nb * MT + mb) * 256 + tid) * 4);
          }
      }
#pragma unroll
      for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) acc[nb][mb] = sum[nb][mb];
      if (tid == 0) reset_counter(p.counters + tile);
    }
    // epilogue: lane holds D[n = 4*(lane/16) + v][m = lane%16] per (nb, mb)
    const int nl = 4 * (lane >> 4);
    if (p.epi == EPI_SWIGLU) {
      const int j = tile * (WG_BLKS / 2) + wave;      // gate/up row block (NWB == 2)
      if (2 * j < p.nblk) {
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) {
          const int m = mb * 16 + (lane & 15);
          if (m < p.M) {
            T* o = reinterpret_cast<T*>(p.out_act) + (size_t)m * p.ld_act + j * 16 + nl;
#pragma unroll
            for (int v = 0; v < 4; ++v) Elt<T>::store(o, v, silu(acc[0][mb][v]) * acc[1][mb][v]);
          }
        }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NWB; ++nb) {
        const int vb = tile * WG_BLKS + wave * NWB + nb;
        if (vb >= p.nblk) continue;
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) {
          const int m = mb * 16 + (lane & 15);
          if (m >= p.M) continue;
          f32x4* o = reinterpret_cast<f32x4*>(p.out + (size_t)m * p.ldo + vb * 16 + nl);
          if (p.epi == EPI_ADD) *o = *o + acc[nb][mb];
          else if (p.epi == EPI_ADD_ROWSCALE) *o = *o + p.row_scale[m] * acc[nb][mb];
          else *o = acc[nb][mb];
        }
      }
    }
#pragma unroll
    for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MT; ++mb) acc[nb][mb] = f32x4{0, 0, 0, 0};
  };

  // prologue: first iteration's data
  load_iter(it_beg, wf0);
  store_a(0);
  __syncthreads();

  int64_t it = it_beg;
  int buf = 0;
  int seg_k0 = (int)(it_beg % p.ipt);
  // one pipeline step: compute `it` from (buf, cur) while loading it+1 into nxt
  auto step = [&](Frag<TW> (&cur)[NWB][KSUB], Frag<TW> (&nxt)[NWB][KSUB]) -> bool {
    const bool has_next = it + 1 < it_end;
    if (has_next) load_iter(it + 1, nxt);
    compute(buf, cur);
    const int tile = (int)(it / p.ipt);
    const int kk = (int)(it % p.ipt);
    if (!has_next || kk == p.ipt - 1) {
      finish(tile, seg_k0, kk + 1);
      seg_k0 = 0;
    }
    if (has_next) store_a(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    ++it;
    return has_next;
  };
  while (true) {
    if (!step(wf0, wf1)) break;
    if (!step(wf1, wf0)) break;
  }
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------
template <typename TW, typename TA, int MT, int NWB, int KSUB>
static hipError_t launch_t(GemmParams p, int grid_cap, hipStream_t s) {
  constexpr int KS = 32 * KSUB;
  p.ipt = (p.K + KS - 1) / KS;
  p.tiles = (p.nblk + 4 * NWB - 1) / (4 * NWB);
  const int64_t TI = (int64_t)p.tiles * p.ipt;
  int G = (int)(TI < grid_cap ? TI : grid_cap);
  p.xcd_remap = (G % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((gemm_stream_kernel<TW, TA, MT, NWB, KSUB>), dim3(G), dim3(256), 0, s, p);
  return hipGetLastError();
}

int gemm_stream_grid_cap(int num_cus) { return 2 * num_cus < kMaxGrid ? 2 * num_cus : kMaxGrid; }

size_t gemm_stream_partial_floats(int grid_cap) {
  // 2 slots per workgroup, each NWB*MT*256*4 floats at most (NWB = 2, MT = 8)
  return (size_t)2 * grid_cap * (2 * 8 * 256 * 4);
}

template <typename TW, typename TA>
static hipError_t launch_mt(const GemmParams& p, int grid_cap, hipStream_t s) {
  const int mt = (p.M + 15) / 16;
  constexpr bool kHalf = Elt<TA>::kBytes == 2;
  if (mt <= 1) return launch_t<TW, TA, 1, 2, kHalf ? 8 : 4>(p, grid_cap, s);
  if (mt <= 2) return launch_t<TW, TA, 2, 2, kHalf ? 8 : 4>(p, grid_cap, s);
  if (mt <= 4) return launch_t<TW, TA, 4, 2, kHalf ? 4 : 2>(p, grid_cap, s);
  return launch_t<TW, TA, 8, 2, kHalf ? 4 : 1>(p, grid_cap, s);
}

hipError_t launch_gemm_stream(const GemmParams& p, int dtype, int num_cus, hipStream_t s) {
  const int grid_cap = gemm_stream_grid_cap(num_cus);
  if (dtype == DT_BF16) {
    if (p.a_bf16) return launch_mt<bf16_t, bf16_t>(p, grid_cap, s);
    return launch_mt<bf16_t, f16_t>(p, grid_cap, s);
  }
  return launch_mt<float, float>(p, grid_cap, s);
}

}  // namespace dspine
