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
//  * Weights are stored fragment-ordered (see the packing kernel): inside a
//    16-row block, each 32-wide K step is 64 lane fragments of 16 bytes laid
//    out contiguously, so every wave load reads 1 KB of consecutive memory.
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

__device__ __forceinline__ int iter_begin(int g, int TI, int G) {
  return (int)((int64_t)g * TI / G);
}
// workgroup whose range holds iteration i
__device__ __forceinline__ int owner_of(int i, int TI, int G) {
  return (int)(((int64_t)(i + 1) * G - 1) / TI);
}

// Weight segment table, copied to LDS at kernel start: looking a segment up
// inside the streaming loop must not issue global loads, whose completion
// counter is shared with the in-flight weight prefetch.
struct SegTable {
  const void* ptr[kMaxSeg];
  int32_t blk0[kMaxSeg];
};

// First weight row of 16-row block vb; blocks past the end read the last
// block (in bounds, results discarded) so loads need no branch.
template <typename T>
__device__ __forceinline__ gptr<T> seg_row_ptr(const GemmParams& p, const SegTable& t, int vb) {
  vb = vb < p.nblk ? vb : p.nblk - 1;
  if (p.interleave) return as_global(reinterpret_cast<const T*>(t.ptr[vb & 1]) + (size_t)(vb >> 1) * 16 * p.K);
  int s = 0;
#pragma unroll 1
  while (s + 1 < p.nseg && vb >= t.blk0[s + 1]) ++s;
  return as_global(reinterpret_cast<const T*>(t.ptr[s]) + (size_t)(vb - t.blk0[s]) * 16 * p.K);
}

// Row pointer of activation row m (clamped to a valid row: rows >= M only
// feed MFMA columns that are never stored).
template <int PRO, typename TA>
__device__ __forceinline__ const TA* a_row_ptr(const GemmParams& p, int m) {
  m = m < p.M ? m : p.M - 1;
  if constexpr (PRO == PRO_GATHER) {
    int s = 0;
#pragma unroll 1
    while (s + 1 < p.g_n && m >= p.g_row0[s + 1]) ++s;
    return reinterpret_cast<const TA*>(p.g_src[s]) + (size_t)(m - p.g_row0[s] + p.g_skip[s]) * p.lda;
  } else {
    return reinterpret_cast<const TA*>(p.a) + (size_t)m * p.lda;
  }
}

// PRO_BRIDGE_MSG chunk: A[t, k] = sigmoid(P[t, k] + Pp[tp, a + k] + b[k]) * Pp[tp, 2a + k]
// for receivers t (zero at anchors); the receiver's rms scales the product
// in the epilogue.
template <typename TW, typename TA>
__device__ __forceinline__ u32x4 bridge_msg_chunk(const GemmParams& p, int m, int k) {
  constexpr int EPC = 16 / Elt<TA>::kBytes;
  u32x4 r = {0, 0, 0, 0};
  if (m >= p.M || k >= p.K || m % p.W == 0) return r;
  const int tp = p.pred_shift ? m - 1 : m;
  const int a3 = 3 * p.a_dim;
  const float* P = p.P + (size_t)m * a3;
  const float* Pp = p.Ppred + (size_t)tp * a3;
  const TW* bias = reinterpret_cast<const TW*>(p.bias);
  TA* out = reinterpret_cast<TA*>(&r);
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    const int kk = k + e;
    const float gpre = P[kk] + Pp[p.a_dim + kk] + Elt<TW>::load(bias, kk);
    Elt<TA>::store(out, e, sigmoid(gpre) * Pp[2 * p.a_dim + kk]);
  }
  return r;
}

}  // namespace

template <typename TW, typename TA, int MT, int NWB, int KSUB, int PRO, int EPI>
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
  __shared__ SegTable s_seg;

  const int tid = threadIdx.x;
  if (tid < p.nseg) {
    s_seg.ptr[tid] = p.seg_ptr[tid];
    s_seg.blk0[tid] = p.seg_blk0[tid];
  }
  __syncthreads();
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int G = gridDim.x;
  int g = blockIdx.x;
  if (p.xcd_remap) g = (g % 8) * (G / 8) + g / 8;   // neighbours in k-space share an XCD

  const int ipt = p.ipt;
  const int TI = p.tiles * ipt;
  const int it_beg = iter_begin(g, TI, G);
  const int it_end = iter_begin(g + 1, TI, G);
  if (it_beg >= it_end) return;

  f32x4 acc[NWB][MT];
#pragma unroll
  for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) acc[nb][mb] = f32x4{0, 0, 0, 0};

  // per-thread A rows (fixed for the whole kernel)
  gptr<TA> arow[NCH];
#pragma unroll
  for (int q = 0; q < NCH; ++q) arow[q] = as_global(a_row_ptr<PRO, TA>(p, (tid + q * 256) / CPR));

  Frag<TW> wf0[NWB][KSUB], wf1[NWB][KSUB];
  u32x4 areg[NCH];

  // Nothing may consume a prefetched weight fragment before the MFMAs that
  // need it: a use would make the wave wait for the whole prefetch.  So past
  // the end of K the weight address is clamped (finite data, in bounds) and
  // the matching activation chunk is zeroed when it is written to LDS.
  auto load_iter = [&](int it, Frag<TW> (&wf)[NWB][KSUB]) {
    const int tile = it / ipt;
    const int k0 = (it - tile * ipt) * KS;
    // A tile chunks first: the LDS store waits only for these (older) loads
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int c = tid + q * 256;
      const int k = k0 + (c % CPR) * EPC;
      if constexpr (PRO == PRO_BRIDGE_MSG) {
        areg[q] = bridge_msg_chunk<TW, TA>(p, c / CPR, k);
      } else {
        areg[q] = gload16((gptr<void>)(arow[q] + (k < p.K ? k : p.K - EPC)));
      }
    }
#pragma unroll
    for (int nb = 0; nb < NWB; ++nb) {
      // fragment-ordered block: 32-K step ks of the block is 64 lanes x 8
      // elements, contiguous; a step past the end of K re-reads the last one
      const gptr<TW> wr = seg_row_ptr<TW>(p, s_seg, tile * WG_BLKS + wave * NWB + nb) + lane * 8;
#pragma unroll
      for (int s = 0; s < KSUB; ++s) {
        const int ks = k0 / 32 + s;
        wf[nb][s].gload(wr + (size_t)(ks < p.K / 32 ? ks : p.K / 32 - 1) * 512);
      }
    }
  };
  auto store_a = [&](int buf, int it) {
    const int k0 = (it - (it / ipt) * ipt) * KS;
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int c = tid + q * 256;
      const int k = k0 + (c % CPR) * EPC;
      *reinterpret_cast<u32x4*>(&lds[buf][(c / CPR) * LDA + (c % CPR) * EPC]) =
          k < p.K ? areg[q] : u32x4{0, 0, 0, 0};
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
    if (!(kb == 0 && ke == ipt)) {
      const int t0 = tile * ipt;
      const int g_first = owner_of(t0, TI, G);
      const int g_last = owner_of(t0 + ipt - 1, TI, G);
      const int ncontrib = g_last - g_first + 1;
      auto slot_of = [&](int gg) {
        const int first_tile = iter_begin(gg, TI, G) / ipt;
        return 2 * gg + (first_tile == tile ? 0 : 1);
      };
      float* mine = p.partials + (size_t)slot_of(g) * (NWB * MT * 256 * 4);
#pragma unroll
      for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) store_coherent(mine + ((nb * MT + mb) * 256 + tid) * 4, acc[nb][mb]);
      drain_own_stores();
      __syncthreads();
      if (tid == 0) s_flag = count_arrival(p.counters + tile);
      __syncthreads();
      if ((int)s_flag != ncontrib - 1) {
#pragma unroll
        for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
          for (int mb = 0; mb < MT; ++mb) acc[nb][mb] = f32x4{0, 0, 0, 0};
        return;
      }
      // Add the contributions in workgroup order, whoever finishes, so the
      // result does not depend on arrival order (bit-reproducible runs).  The
      // own partial is read back like the others (the same values).  Loads go
      // out FB contributors at a time so their latencies overlap; indexes past
      // the last contributor repeat it and are not added.
      constexpr int FB = NWB * MT <= 2 ? 8 : NWB * MT <= 4 ? 4 : NWB * MT <= 8 ? 2 : 1;
      f32x4 sum[NWB][MT];
#pragma unroll
      for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) sum[nb][mb] = f32x4{0, 0, 0, 0};
      for (int g0 = g_first; g0 <= g_last; g0 += FB) {
        f32x4 part[FB][NWB][MT];
#pragma unroll
        for (int j = 0; j < FB; ++j) {
          const int gg = g0 + j <= g_last ? g0 + j : g_last;
          const float* other = p.partials + (size_t)slot_of(gg) * (NWB * MT * 256 * 4);
#pragma unroll
          for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
            for (int mb = 0; mb < MT; ++mb) part[j][nb][mb] = load_coherent4(other + ((nb * MT + mb) * 256 + tid) * 4);
        }
#pragma unroll
        for (int j = 0; j < FB; ++j) {
          if (g0 + j > g_last) break;
#pragma unroll
          for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
            for (int mb = 0; mb < MT; ++mb) sum[nb][mb] += part[j][nb][mb];
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
    if constexpr (EPI == EPI_SWIGLU) {
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
          if constexpr (EPI == EPI_ADD) *o = *o + acc[nb][mb];
          else if constexpr (EPI == EPI_ADD_ROWSCALE) *o = *o + p.row_scale[m] * acc[nb][mb];
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
  store_a(0, it_beg);
  __syncthreads();

  // Stream the workgroup's range.  The register prefetch of iteration it+1
  // overlaps the MFMAs of iteration it; two iterations per trip so that the
  // two register buffers swap statically.  A tile is finished when its last
  // iteration in this range has been accumulated.
  int it = it_beg;
  int buf = 0;
  int seg_k0 = it_beg % ipt;
  // The prefetch is issued on every iteration (the last one re-reads its own
  // data, which sits in L2): with the same number of loads in flight on every
  // path, the wait before the MFMAs covers exactly the previous iteration.
  auto step = [&](Frag<TW> (&cur)[NWB][KSUB], Frag<TW> (&nxt)[NWB][KSUB]) -> bool {
    const bool has_next = it + 1 < it_end;
    const int it_next = has_next ? it + 1 : it;
    load_iter(it_next, nxt);
    compute(buf, cur);
    const int tile = it / ipt;
    const int kk = it - tile * ipt;
    if (!has_next || kk == ipt - 1) {
      finish(tile, seg_k0, kk + 1);
      seg_k0 = 0;
    }
    store_a(buf ^ 1, it_next);
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
template <typename TW, typename TA, int MT, int NWB, int KSUB, int PRO, int EPI>
static hipError_t launch_t(GemmParams p, int grid_cap, hipStream_t s) {
  constexpr int KS = 32 * KSUB;
  p.ipt = (p.K + KS - 1) / KS;
  p.tiles = (p.nblk + 4 * NWB - 1) / (4 * NWB);
  const int64_t TI = (int64_t)p.tiles * p.ipt;
  int G = (int)(TI < grid_cap ? TI : grid_cap);
  p.xcd_remap = (G % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((gemm_stream_kernel<TW, TA, MT, NWB, KSUB, PRO, EPI>), dim3(G), dim3(256), 0, s, p);
  return hipGetLastError();
}

int gemm_stream_grid_cap(int num_cus) { return 2 * num_cus < kMaxGrid ? 2 * num_cus : kMaxGrid; }

size_t gemm_stream_partial_floats(int grid_cap) {
  // 2 slots per workgroup, each NWB*MT*256*4 floats at most (NWB = 2, MT = 8)
  return (size_t)2 * grid_cap * (2 * 8 * 256 * 4);
}

template <typename TW, typename TA, int PRO, int EPI>
static hipError_t launch_mt(const GemmParams& p, int grid_cap, hipStream_t s) {
  const int mt = (p.M + 15) / 16;
  constexpr bool kHalf = Elt<TA>::kBytes == 2;
  if (mt <= 1) return launch_t<TW, TA, 1, 2, kHalf ? 8 : 4, PRO, EPI>(p, grid_cap, s);
  if (mt <= 2) return launch_t<TW, TA, 2, 2, kHalf ? 8 : 4, PRO, EPI>(p, grid_cap, s);
  if (mt <= 4) return launch_t<TW, TA, 4, 2, kHalf ? 4 : 2, PRO, EPI>(p, grid_cap, s);
  return launch_t<TW, TA, 8, 2, kHalf ? 4 : 1, PRO, EPI>(p, grid_cap, s);
}

template <typename TW, typename TA>
static hipError_t launch_kind(const GemmParams& p, int grid_cap, hipStream_t s) {
  if (p.pro == PRO_BRIDGE_MSG) {
    if (p.epi != EPI_ADD_ROWSCALE) return hipErrorInvalidValue;
    return launch_mt<TW, TA, PRO_BRIDGE_MSG, EPI_ADD_ROWSCALE>(p, grid_cap, s);
  }
  if (p.pro != PRO_COPY) return hipErrorInvalidValue;
  switch (p.epi) {
    case EPI_STORE: return launch_mt<TW, TA, PRO_COPY, EPI_STORE>(p, grid_cap, s);
    case EPI_ADD: return launch_mt<TW, TA, PRO_COPY, EPI_ADD>(p, grid_cap, s);
    case EPI_SWIGLU: return launch_mt<TW, TA, PRO_COPY, EPI_SWIGLU>(p, grid_cap, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_stream(const GemmParams& p, int dtype, int num_cus, hipStream_t s) {
  const int grid_cap = gemm_stream_grid_cap(num_cus);
  if (p.pro == PRO_GATHER) {          // target features, stored output only
    if (p.epi != EPI_STORE) return hipErrorInvalidValue;
    if (dtype == DT_BF16) return launch_mt<bf16_t, bf16_t, PRO_GATHER, EPI_STORE>(p, grid_cap, s);
    return launch_mt<float, float, PRO_GATHER, EPI_STORE>(p, grid_cap, s);
  }
  if (dtype == DT_BF16) return launch_kind<bf16_t, f16_t>(p, grid_cap, s);
  return launch_kind<float, float>(p, grid_cap, s);
}

}  // namespace dspine
