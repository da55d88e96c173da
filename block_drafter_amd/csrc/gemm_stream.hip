// Weight-streaming GEMM for the draft forward and decode-round materialization.
//
//   out[m, n] (op)= sum_k A[m, k] * W[n, k]     m < M <= 128, n < N, k < K
//
// The block has only B*W <= 128 activation rows, so every projection of the
// draft layers is bound by reading W once from HBM.  Design for gfx950:
//  * Weights are stored fragment-ordered (see the packing kernel): inside a
//    16-row block, each 32-wide K step is 64 lane fragments of 16 bytes laid
//    out contiguously, so every wave load reads 1 KB of consecutive memory.
//    They are the MFMA A operand (16 rows = 16 output columns n); activations
//    are the B operand (16 columns = 16 rows m), so each lane ends with 4
//    consecutive n of one m: 16-byte epilogue stores.
//  * Each wave streams NWB 16-row blocks.  Its weight fragments go through a
//    ring of PD + 1 register stages: PD iterations are in flight while one is
//    multiplied.  The activation chunk of an iteration travels in the same
//    stage as its weights (the vector-memory counter retires in issue order,
//    so a load issued after the weights could not be waited for alone), and
//    is staged through LDS for the four waves.
//  * With 128 rows the registers cannot hold the accumulators and several
//    weight stages at once, so both operands move global -> LDS directly
//    (global_load_lds_dwordx4) into a ring of 64-K stages: weights as their
//    1 KB fragment blocks, activations as full-line blocks of 8 rows x 128
//    bytes.  The registers then hold only the accumulators and the
//    fragments being multiplied.  All shared state lives in one array: with
//    several __shared__ objects the compiler makes every LDS read wait for
//    all direct-to-LDS loads in flight.
//  * A tile (4 * NWB blocks) is either streamed over its whole K by one
//    workgroup (no reduction at all), or, when N has fewer tiles than there
//    are CUs (one CU alone cannot pull its share of HBM bandwidth), the
//    (tile, k-iteration) space is cut into equal contiguous ranges
//    (stream-K).  A tile split between workgroups is finished by the
//    last one to arrive, which adds the published partials in workgroup
//    order (bit-reproducible) and runs the epilogue.
//  * Prologues form the A operand: as stored, gathered bf16 target
//    features, a row-scaled (and gained) fp32 residual whose norm comes from
//    per-64-column sums of squares written by the producing GEMM, or the
//    bridge gate * message.  Epilogues: store, residual add, SwiGLU (gate/up
//    blocks interleaved), row-scaled add; the stored rows' sums of squares
//    go out per 64 columns for the next norm.
//  * Operand types: a BF16 model multiplies FP16 activations by its bf16
//    weights widened to fp16 in registers (exact); bf16 target features are
//    used as they are (bf16 x bf16).  A float32 model uses fp32 MFMAs.
#include <type_traits>

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

// Per-row scale from the row's sum of squares S (see the SCALE_* modes).
__device__ __forceinline__ float row_scale_of(const GemmParams& p, int m, float S) {
  return row_scale(p.scale_mode, S, p.scale_n, p.eps, p.code_scale, m % p.W == 0);
}

// 16-byte registers one activation chunk (EPC elements) occupies in a stage
template <int PRO, int EPC>
constexpr int a_regs() {
  return PRO == PRO_NORM ? (EPC == 8 ? 3 : 2)           // fp32 x (+ gain)
       : PRO == PRO_SCALE ? (EPC == 8 ? 2 : 1)          // fp32 x
       : PRO == PRO_BRIDGE_MSG ? (EPC == 8 ? 7 : 4)     // P, Pp gate, Pp message (fp32) + bias
       : 1;
}

}  // namespace

// TL: row-block launches, whose blocks read the same weights, load them
// with the ordinary cache policy (single-block launches: non-temporal)
template <typename TW, typename TA, int MT, int NWB, int KSUB, int PD, int PRO, int EPI, bool DMA, bool WD, bool TL>
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
  constexpr int NST = PD + 1;                   // register (WD: LDS) stages
  static_assert(NST >= 1 && NST <= (WD ? 8 : 4), "stages");
  constexpr int AR = a_regs<PRO, EPC>();
  constexpr bool kScaledA = PRO == PRO_NORM || PRO == PRO_SCALE;
  // DMA: the activation chunk of a stage goes global -> LDS directly
  // (global_load_lds_dwordx4) into a ring slot in MFMA operand order, so the
  // register stages hold weights only; K must be a multiple of KS.
  static_assert(!DMA || ((PRO == PRO_COPY || PRO == PRO_GATHER) && EB == 2 && (MT * KSUB) % 4 == 0 && NST >= 2),
                "direct-to-LDS activations: 16-bit copy or gather operands");
  constexpr int SLOT = MT * KSUB * 1024;        // DMA: one stage's chunk, 1 KB blocks [mb][ks]
  constexpr int DBLK = MT * KSUB / 4;           // DMA: blocks per wave per stage
  // weight loads per wave per stage (one 16-byte load per fragment, or per
  // pair of FP8 fragments); the direct-to-LDS waits count them exactly
  constexpr int WLD = sizeof(TW) == 1 ? NWB * KSUB / 2 : NWB * KSUB;
  static_assert(!DMA || (256 / MP) * MP * 4 <= SLOT, "row-scale scratch fits a ring slot");
  // WD: the weight blocks of a stage also go global -> LDS directly (1 KB
  // blocks [wave][nb][ks] after the activation chunk), so the registers hold
  // only accumulators and the fragments being multiplied, and the ring can
  // be deeper than the register file would allow.
  static_assert(!WD || (DMA && sizeof(TW) == 2), "weights through LDS: with direct-to-LDS activations, 16-bit weights");
  constexpr int WSLOT = WD ? 4 * NWB * KSUB * 1024 : 0;
  constexpr int STG = SLOT + WSLOT;             // DMA: bytes of one ring stage

  // All shared state is carved out of one array.  With several __shared__
  // objects the compiler tags their accesses with alias scopes, and then
  // makes every LDS read wait for all direct-to-LDS loads in flight
  // (vmcnt(0) before the fragment reads), which serialises the ring.
  constexpr int kLdsA = DMA ? 8 : MP * LDA;     // activation staging, elements per buffer
  constexpr int OFF_LDS = DMA ? NST * STG : 16;
  constexpr int OFF_RED = OFF_LDS + ((2 * kLdsA * (int)sizeof(T) + 15) & ~15);
  constexpr int OFF_SCALE = OFF_RED + 4 * MP * 4;
  constexpr int OFF_SEG = OFF_SCALE + MP * 4;
  constexpr int OFF_FLAG = OFF_SEG + (((int)sizeof(SegTable) + 15) & ~15);
  __shared__ __attribute__((aligned(1024))) char smem[OFF_FLAG + 16];
  char* const adma = smem;                                               // DMA ring
  T (*const lds)[kLdsA] = reinterpret_cast<T (*)[kLdsA]>(smem + OFF_LDS);
  float (*const s_red)[MP] = reinterpret_cast<float (*)[MP]>(smem + OFF_RED);  // per-wave row sums of squares
  float* const s_scale = reinterpret_cast<float*>(smem + OFF_SCALE);    // per-row scale (SCALE_* modes)
  SegTable& s_seg = *reinterpret_cast<SegTable*>(smem + OFF_SEG);
  uint32_t& s_flag = *reinterpret_cast<uint32_t*>(smem + OFF_FLAG);

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

  // row block of this workgroup (blocks of MP rows along y; one block: 0)
  const int m_base = blockIdx.y * MP;
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
  const void* arow[NCH];
#pragma unroll
  for (int q = 0; q < NCH; ++q) {
    const int m = m_base + (tid + q * 256) / CPR;
    if constexpr (kScaledA) arow[q] = p.xa + (size_t)(m < p.M ? m : p.M - 1) * p.lda;
    else if constexpr (PRO == PRO_BRIDGE_MSG) arow[q] = nullptr;
    else arow[q] = a_row_ptr<PRO, TA>(p, m);
  }

  // DMA: lane l of block (mb, ks) fetches row mb*16 + l%16, K 8 (l/16) of
  // the block's 32-K step; this wave takes blocks wave, wave + 4, ...
  // Full-line layout (WD with 64-K stages): block b holds rows 8 b .. 8 b + 7
  // over the stage's whole 128 bytes, so every L2 request is a whole line.
  constexpr bool kFullLine = WD && KSUB == 2;
  const TA* drow[DMA ? DBLK : 1];
  if constexpr (DMA) {
#pragma unroll
    for (int q = 0; q < DBLK; ++q) {
      const int bi = wave + 4 * q;
      if constexpr (kFullLine) {
        const int r = lane >> 3;
        drow[q] = a_row_ptr<PRO, TA>(p, m_base + bi * 8 + r) + ((lane & 7) ^ act_swz(r, bi & 1)) * 8;
      } else {
        drow[q] = a_row_ptr<PRO, TA>(p, m_base + (bi / KSUB) * 16 + (lane & 15)) + (bi % KSUB) * 32 + 8 * (lane >> 4);
      }
    }
  }
  // full-line fragment offsets in a stage's activation chunk, per 32-K half
  int aoff[2] = {0, 0};
  if constexpr (kFullLine) {
    const int bb = (lane & 15) >> 3, r = lane & 7;
#pragma unroll
    for (int h = 0; h < 2; ++h) aoff[h] = bb * 1024 + (r * 8 + ((4 * h + (lane >> 4)) ^ act_swz(r, bb))) * 16;
  }

  Frag<TW> wf[WD ? 1 : NST][NWB][KSUB];
  // WD: this wave's weight rows of the tile being loaded (looked up once
  // per tile, not per stage)
  int wtile = -1;
  gptr<TW> wrow[NWB];
  u32x4 areg[DMA ? 1 : NST][NCH][AR];

  // Stage j <- iteration it: activation chunk(s) first, then the weights.
  // Nothing may consume a prefetched value before it is needed: past the
  // end of K the addresses are clamped (finite data, in bounds) and the
  // activation chunk is zeroed when it is written to LDS.
  auto load_stage = [&](int j, int it) __attribute__((always_inline)) {
    const int tile = it / ipt;
    const int k0 = (it - tile * ipt) * KS;
    if constexpr (DMA) {
      char* slot = adma + j * STG;
#pragma unroll
      for (int q = 0; q < DBLK; ++q)
        __builtin_amdgcn_global_load_lds((const void*)(drow[q] + k0), (lds_void*)(slot + (wave + 4 * q) * 1024), 16,
                                         0, 0);
    }
#pragma unroll
    for (int q = 0; q < (DMA ? 0 : NCH); ++q) {
      const int c = tid + q * 256;
      const int k = k0 + (c % CPR) * EPC;
      const int kc = k < p.K ? k : p.K - EPC;
      if constexpr (kScaledA) {
        const gptr<float> x = as_global(reinterpret_cast<const float*>(arow[q])) + kc;
        areg[j][q][0] = gload16((gptr<void>)x);
        if constexpr (EPC == 8) areg[j][q][1] = gload16((gptr<void>)(x + 4));
        if constexpr (PRO == PRO_NORM)
          areg[j][q][AR - 1] = gload16((gptr<void>)(as_global(reinterpret_cast<const TW*>(p.gain)) + kc));
      } else if constexpr (PRO == PRO_BRIDGE_MSG) {
        // A[t, k] = sigmoid(P[t, k] + Pp[tp, a + k] + b[k]) * Pp[tp, 2a + k]
        int m = m_base + c / CPR;
        m = m < p.M ? m : p.M - 1;
        int tp = p.pred_shift ? m - 1 : m;
        tp = tp < 0 ? 0 : tp;
        const int a3 = 3 * p.a_dim;
        const gptr<float> P = as_global(p.P) + (size_t)m * a3 + kc;
        const gptr<float> Pg = as_global(p.Ppred) + (size_t)tp * a3 + p.a_dim + kc;
        const gptr<float> Pm = as_global(p.Ppred) + (size_t)tp * a3 + 2 * p.a_dim + kc;
        constexpr int H4 = EPC / 4;                // 16-byte pieces of EPC floats
#pragma unroll
        for (int h = 0; h < H4; ++h) {
          areg[j][q][h] = gload16((gptr<void>)(P + 4 * h));
          areg[j][q][H4 + h] = gload16((gptr<void>)(Pg + 4 * h));
          areg[j][q][2 * H4 + h] = gload16((gptr<void>)(Pm + 4 * h));
        }
        areg[j][q][3 * H4] = gload16((gptr<void>)(as_global(reinterpret_cast<const TW*>(p.bias)) + kc));
      } else {
        areg[j][q][0] = gload16((gptr<void>)(as_global(reinterpret_cast<const TA*>(arow[q])) + kc));
      }
    }
    if constexpr (WD) {
      if (tile != wtile) {
        wtile = tile;
#pragma unroll
        for (int nb = 0; nb < NWB; ++nb) wrow[nb] = seg_row_ptr<TW>(p, s_seg, tile * WG_BLKS + wave * NWB + nb) + lane * 8;
      }
    }
#pragma unroll
    for (int nb = 0; nb < NWB; ++nb) {
      if constexpr (sizeof(TW) == 1) {
        // FP8 codes: each 64-wide K step of a block is 64 lanes x 16 bytes,
        // lane l holding its 8 codes of the two 32-wide steps in a row (one
        // 16-byte load feeds two fragments); K is a multiple of 64
        static_assert(KSUB % 2 == 0, "FP8 fragments come in pairs of 32-K steps");
        const gptr<TW> wr = seg_row_ptr<TW>(p, s_seg, tile * WG_BLKS + wave * NWB + nb) + lane * 16;
#pragma unroll
        for (int s = 0; s < KSUB; s += 2) {
          const int kp = k0 / 64 + s / 2;
          const u32x4 q = gload16_nt((gptr<void>)(wr + (size_t)(kp < p.K / 64 ? kp : p.K / 64 - 1) * 1024));
          wf[j][nb][s].v[0] = q[0];
          wf[j][nb][s].v[1] = q[1];
          wf[j][nb][s + 1].v[0] = q[2];
          wf[j][nb][s + 1].v[1] = q[3];
        }
        continue;
      }
      // fragment-ordered block: 32-K step ks of the block is 64 lanes x 8
      // elements, contiguous; a step past the end of K re-reads the last one
      const gptr<TW> wr = WD ? wrow[nb] : seg_row_ptr<TW>(p, s_seg, tile * WG_BLKS + wave * NWB + nb) + lane * 8;
#pragma unroll
      for (int s = 0; s < KSUB; ++s) {
        const int ks = k0 / 32 + s;
        const gptr<TW> src = wr + (size_t)(ks < p.K / 32 ? ks : p.K / 32 - 1) * 512;
        // weights are read once: non-temporal (cache policy NT), so the L2
        // keeps the activation lines every workgroup re-reads (128 rows: the
        // L2 missed 57 % of requests with the weights cached; B=8 forward
        // 1.79 -> 1.69 ms)
        if constexpr (WD)
          __builtin_amdgcn_global_load_lds((const void*)src,
                                           (lds_void*)(adma + j * STG + SLOT + ((wave * NWB + nb) * KSUB + s) * 1024),
                                           16, 0, 2);
        else if constexpr (TL)    // row blocks: the siblings of this tile read the same lines from L2
          wf[j][nb][s].gload(src);
        else
          wf[j][nb][s].gload_nt(src);
      }
    }
  };
  // activation chunk of stage j (iteration it) -> LDS buffer buf
  auto store_a = [&](int buf, int j, int it) __attribute__((always_inline)) {
    if constexpr (DMA) return;
    const int k0 = (it - (it / ipt) * ipt) * KS;
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int c = tid + q * 256;
      const int m = c / CPR;
      const int k = k0 + (c % CPR) * EPC;
      u32x4 v = u32x4{0, 0, 0, 0};
      if constexpr (kScaledA) {
        if (k < p.K) {
          const float sc = s_scale[m];
          alignas(16) float xv[EPC];
          *reinterpret_cast<u32x4*>(&xv[0]) = areg[j][q][0];
          if constexpr (EPC == 8) *reinterpret_cast<u32x4*>(&xv[4]) = areg[j][q][1];
          alignas(16) TW gv[EPC];
          if constexpr (PRO == PRO_NORM) *reinterpret_cast<u32x4*>(gv) = areg[j][q][AR - 1];
          alignas(16) T tv[EPC];
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            const float gn = (PRO == PRO_NORM) ? Elt<TW>::load(gv, e) : 1.f;
            const float av = xv[e] * sc * gn;
            Elt<T>::store(tv, e, p.act_round_bf16 ? round_bf16(av) : av);
          }
          v = *reinterpret_cast<const u32x4*>(tv);
        }
      } else if constexpr (PRO == PRO_BRIDGE_MSG) {
        // receivers only: zero at anchors (m % W == 0) and past M / K
        if (k < p.K && m_base + m < p.M && (m_base + m) % p.W != 0) {
          constexpr int H4 = EPC / 4;
          alignas(16) float P[EPC], Pg[EPC], Pm[EPC];
#pragma unroll
          for (int h = 0; h < H4; ++h) {
            *reinterpret_cast<u32x4*>(&P[4 * h]) = areg[j][q][h];
            *reinterpret_cast<u32x4*>(&Pg[4 * h]) = areg[j][q][H4 + h];
            *reinterpret_cast<u32x4*>(&Pm[4 * h]) = areg[j][q][2 * H4 + h];
          }
          alignas(16) TW bv[EPC];
          *reinterpret_cast<u32x4*>(bv) = areg[j][q][3 * H4];
          alignas(16) T tv[EPC];
#pragma unroll
          for (int e = 0; e < EPC; ++e)
            Elt<T>::store(tv, e, sigmoid(P[e] + Pg[e] + Elt<TW>::load(bv, e)) * Pm[e]);
          v = *reinterpret_cast<const u32x4*>(tv);
        }
      } else {
        v = k < p.K ? areg[j][q][0] : u32x4{0, 0, 0, 0};
      }
      *reinterpret_cast<u32x4*>(&lds[buf][m * LDA + (c % CPR) * EPC]) = v;
    }
  };
  // One stage's products.  Wide row tiles (64 and 128 rows) read every LDS
  // fragment of the stage before the first MFMA: with one wave per SIMD
  // nothing else hides an LDS round trip, and reads issued one group at a
  // time (read, wait, multiply) stall the wave once per group and hold back
  // the next stage's loads (128 rows: gate/up 105.6 -> 103.2 us, the B=8
  // forward 2.021 -> 1.954 ms).  Narrow tiles keep one read per product,
  // which the compiler interleaves with the next stage's weight loads (the
  // batched order made the 16-row q|k|v 8 % slower).  Each accumulator sums
  // its 32-K steps in order either way.
  auto compute = [&](int buf, int j) __attribute__((always_inline)) {
    auto a_frag = [&](Frag<T>& af, int s, int mb) __attribute__((always_inline)) {
      if constexpr (kFullLine)
        af.v = *reinterpret_cast<const u32x4*>(adma + j * STG + mb * 2048 + aoff[s]);
      else if constexpr (DMA)
        af.v = *reinterpret_cast<const u32x4*>(adma + j * STG + (mb * KSUB + s) * 1024 + lane * 16);
      else
        af.load(&lds[buf][(mb * 16 + (lane & 15)) * LDA + s * 32 + 8 * (lane >> 4)]);
    };
    auto w_frag = [&](int s, int nb) __attribute__((always_inline)) -> Frag<TW> {
      Frag<TW> w{};
      if constexpr (WD)   // 16-bit weights only
        w.v = *reinterpret_cast<const u32x4*>(adma + j * STG + SLOT + ((wave * NWB + nb) * KSUB + s) * 1024 + lane * 16);
      return w;
    };
    if constexpr (MT >= 4) {
      Frag<T> af[KSUB][MT];
      Frag<TW> wl[WD ? KSUB : 1][NWB];
#pragma unroll
      for (int s = 0; s < KSUB; ++s) {
        if constexpr (WD) {
#pragma unroll
          for (int nb = 0; nb < NWB; ++nb) wl[s][nb] = w_frag(s, nb);
        }
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) a_frag(af[s][mb], s, mb);
      }
      // keep the scheduler from sinking the reads back between the products
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < KSUB; ++s) {
        Frag<T> wo[NWB];
#pragma unroll
        for (int nb = 0; nb < NWB; ++nb) {
          if constexpr (WD) wo[nb] = AsOperand<T, TW>::cvt(wl[s][nb]);
          else wo[nb] = AsOperand<T, TW>::cvt(wf[j][nb][s]);
        }
#pragma unroll
        for (int mb = 0; mb < MT; ++mb)
#pragma unroll
          for (int nb = 0; nb < NWB; ++nb) mma16(acc[nb][mb], wo[nb], af[s][mb]);
      }
    } else {
#pragma unroll
      for (int s = 0; s < KSUB; ++s) {
        Frag<T> wo[NWB];
#pragma unroll
        for (int nb = 0; nb < NWB; ++nb) {
          if constexpr (WD) wo[nb] = AsOperand<T, TW>::cvt(w_frag(s, nb));
          else wo[nb] = AsOperand<T, TW>::cvt(wf[j][nb][s]);
        }
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) {
          Frag<T> af;
          a_frag(af, s, mb);
#pragma unroll
          for (int nb = 0; nb < NWB; ++nb) mma16(acc[nb][mb], wo[nb], af);
        }
      }
    }
  };

  // Finish tile `tile` whose iterations [kb, ke) this workgroup has accumulated.
  auto finish = [&](int tile, int kb, int ke) __attribute__((always_inline)) {
    if (!(kb == 0 && ke == ipt)) {
      const int t0 = tile * ipt;
      const int g_first = owner_of(t0, TI, G);
      const int g_last = owner_of(t0 + ipt - 1, TI, G);
      const int ncontrib = g_last - g_first + 1;
      // two slots per workgroup of each row block
      auto slot_of = [&](int gg) __attribute__((always_inline)) {
        const int first_tile = iter_begin(gg, TI, G) / ipt;
        return 2 * ((int)blockIdx.y * G + gg) + (first_tile == tile ? 0 : 1);
      };
      float* mine = p.partials + (size_t)slot_of(g) * (NWB * MT * 256 * 4);
#pragma unroll
      for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) store_coherent(mine + ((nb * MT + mb) * 256 + tid) * 4, acc[nb][mb]);
      drain_own_stores();
      __syncthreads();
      if (tid == 0) s_flag = count_arrival(p.counters + blockIdx.y * p.tiles + tile);
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
      // the last contributor repeat it and are not added.  The partials are
      // read with agent-scope loads, from the device coherence point the
      // writers stored them to: this workgroup's L2 may still hold a line of
      // the same slot from an earlier launch that reused the workspace, and
      // the loads are issued only after the arrival count (whose value they
      // depend on) has returned.
      if constexpr (WD) {
        // One weight block at a time, FB contributors per load batch: the
        // registers hold the accumulators plus FB x MT partial fragments,
        // not a second full tile (the same additions in the same order).
        constexpr int FB = MT <= 4 ? 4 : 2;
#pragma unroll
        for (int nb = 0; nb < NWB; ++nb) {
          f32x4 sum[MT];
#pragma unroll
          for (int mb = 0; mb < MT; ++mb) sum[mb] = f32x4{0, 0, 0, 0};
          for (int g0 = g_first; g0 <= g_last; g0 += FB) {
            f32x4 part[FB][MT];
#pragma unroll
            for (int j = 0; j < FB; ++j) {
              const int gg = g0 + j <= g_last ? g0 + j : g_last;
              const float* other = p.partials + (size_t)slot_of(gg) * (NWB * MT * 256 * 4);
#pragma unroll
              for (int mb = 0; mb < MT; ++mb)
                part[j][mb] = load_coherent4(other + ((nb * MT + mb) * 256 + tid) * 4);
            }
#pragma unroll
            for (int j = 0; j < FB; ++j) {
              if (g0 + j > g_last) break;
#pragma unroll
              for (int mb = 0; mb < MT; ++mb) sum[mb] += part[j][mb];
            }
          }
#pragma unroll
          for (int mb = 0; mb < MT; ++mb) acc[nb][mb] = sum[mb];
        }
        if (tid == 0) reset_counter(p.counters + blockIdx.y * p.tiles + tile);
        // the repeated loads past the last contributor are never used: wait
        // for them here, or the compiler's wait before the next reuse of
        // their registers (an LDS fragment read of the next tile) would
        // also wait for every stage in flight
        wait_vmcnt<0>();
      } else {
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
            for (int mb = 0; mb < MT; ++mb)
              part[j][nb][mb] = load_coherent4(other + ((nb * MT + mb) * 256 + tid) * 4);
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
      if (tid == 0) reset_counter(p.counters + blockIdx.y * p.tiles + tile);
      wait_vmcnt<0>();                             // as above
      }
    }
    // epilogue: lane holds D[n = 4*(lane/16) + v][m = lane%16] per (nb, mb)
    const int nl = 4 * (lane >> 4);
    if constexpr (EPI == EPI_SWIGLU) {
      // blocks nb = 2 i, 2 i + 1 of a wave are gate and up of row block j
#pragma unroll
      for (int i = 0; i < NWB / 2; ++i) {
        const int j = (tile * WG_BLKS + wave * NWB) / 2 + i;
        if (2 * j >= p.nblk) continue;
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) {
          const int m = mb * 16 + (lane & 15);
          if (m_base + m < p.M) {
            const size_t e = (size_t)(m_base + m) * p.ld_act + j * 16 + nl;
            const float rs = p.post_scale ? s_scale[m] * p.post_mult : 1.f;   // the norm after the product
            if (p.out_act_bf16) {
#pragma unroll
              for (int v = 0; v < 4; ++v)
                Elt<bf16_t>::store(reinterpret_cast<bf16_t*>(p.out_act) + e, v,
                                   silu(rs * acc[2 * i][mb][v]) * (rs * acc[2 * i + 1][mb][v]));
            } else {
#pragma unroll
              for (int v = 0; v < 4; ++v)
                Elt<T>::store(reinterpret_cast<T*>(p.out_act) + e, v,
                              silu(rs * acc[2 * i][mb][v]) * (rs * acc[2 * i + 1][mb][v]));
            }
          }
        }
      }
    } else {
      float sq[MT];
#pragma unroll
      for (int mb = 0; mb < MT; ++mb) sq[mb] = 0.f;
#pragma unroll
      for (int nb = 0; nb < NWB; ++nb) {
        const int vb = tile * WG_BLKS + wave * NWB + nb;
        if (vb >= p.nblk) continue;
        // the copy's gains go out with the residual loads below
        float cg[4] = {1.f, 1.f, 1.f, 1.f};
        if (p.out_copy && p.copy_gain) {
          const gptr<bf16_t> gp = as_global(reinterpret_cast<const bf16_t*>(p.copy_gain)) + vb * 16 + nl;
#pragma unroll
          for (int v = 0; v < 4; ++v) cg[v] = Elt<bf16_t>::gload(gp, v);
        }
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) {
          const int m = mb * 16 + (lane & 15);               // row in the block (s_scale)
          const int mg = m_base + m;                            // row of the matrix
          if (mg >= p.M) continue;
          f32x4* o = reinterpret_cast<f32x4*>(p.out + (size_t)mg * p.ldo + vb * 16 + nl);
          f32x4 val;
          if constexpr (EPI == EPI_ADD) {
            val = *o + acc[nb][mb];
          } else if constexpr (EPI == EPI_ADD_ROWSCALE) {
            val = *o + s_scale[m] * acc[nb][mb];
          } else {
            val = acc[nb][mb];
            if (p.post_scale) {                       // the operand's row norm, after the product
              const float rs = s_scale[m] * p.post_mult;
              val = f32x4{val[0] * rs, val[1] * rs, val[2] * rs, val[3] * rs};
            }
            if constexpr (sizeof(TW) == 1) {          // FP8 rows: codes read as value / 256
              const f32x4 cs = *as_global(reinterpret_cast<const f32x4*>(p.col_scale + vb * 16 + nl));
              val = f32x4{val[0] * cs[0], val[1] * cs[1], val[2] * cs[2], val[3] * cs[3]};
            }
            if (p.code_anchor && mg % p.W == 0) {     // anchor code: sqrt(r) C[anchor]
              const gptr<TW> cb = as_global(reinterpret_cast<const TW*>(p.codebook)) +
                                  (size_t)p.anchor[mg / p.W] * p.ldo + vb * 16 + nl;
#pragma unroll
              for (int v = 0; v < 4; ++v) val[v] = p.code_scale * Elt<TW>::gload(cb, v);
            }
          }
          *o = val;
          if (p.out_copy) {                           // the next GEMM's 16-bit operand
            float cv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) cv[v] = val[v] * p.copy_mult * cg[v];
            const size_t e = (size_t)mg * p.ld_copy + vb * 16 + nl;
            uint32_t w0, w1;
            if (p.copy_bf16) {
              w0 = (uint32_t)f32_to_bf16_bits(cv[0]) | ((uint32_t)f32_to_bf16_bits(cv[1]) << 16);
              w1 = (uint32_t)f32_to_bf16_bits(cv[2]) | ((uint32_t)f32_to_bf16_bits(cv[3]) << 16);
            } else {
              w0 = (uint32_t)f32_to_f16_bits(cv[0]) | ((uint32_t)f32_to_f16_bits(cv[1]) << 16);
              w1 = (uint32_t)f32_to_f16_bits(cv[2]) | ((uint32_t)f32_to_f16_bits(cv[3]) << 16);
            }
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out_copy) + e) = uint2{w0, w1};
          }
          sq[mb] += sumsq4(val[0], val[1], val[2], val[3]);
        }
      }
      // Sums of squares per row over each 64 output columns, in a fixed
      // order: lane values, the four lane groups, then the waves of the list.
      if (p.stats_out != nullptr) {
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) {
          sq[mb] += __shfl_xor(sq[mb], 16, 64);
          sq[mb] += __shfl_xor(sq[mb], 32, 64);
          if (lane < 16) s_red[wave][mb * 16 + lane] = sq[mb];
        }
        __syncthreads();
        constexpr int WPL = 4 / NWB;                   // waves per 64-column list
        const int nlists = (p.nblk + 3) / 4;
        if (m_base + tid < p.M && tid < MP) {
#pragma unroll
          for (int jl = 0; jl < NWB; ++jl) {
            const int list = tile * NWB + jl;
            if (list >= nlists) break;
            float sum = s_red[jl * WPL][tid];
#pragma unroll
            for (int w = 1; w < WPL; ++w) sum += s_red[jl * WPL + w][tid];
            p.stats_out[(size_t)list * p.stats_out_ld + m_base + tid] = sum;
          }
        }
        __syncthreads();
      }
    }
#pragma unroll
    for (int nb = 0; nb < NWB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MT; ++mb) acc[nb][mb] = f32x4{0, 0, 0, 0};
  };

  // prologue: the per-row scales and the first NST iterations.  A row's
  // statistics lists are split over Q = 256 / MP threads (thread jq takes
  // lists jq, jq + Q, ...) and the Q partial sums are added in order, so the
  // sum does not depend on timing.  The first batch of statistics loads goes
  // out before the weight stages, so that waiting for it does not wait for
  // the weights (the memory counter retires in issue order).
  constexpr int Q = 256 / MP;
  // statistics loads per batch: with 64 rows and more a thread takes 40 of
  // its row's lists at once (80 lists at H = 5120 otherwise cost five
  // serial round trips before the first weight stage)
  constexpr int LB = MP >= 64 ? 40 : 8;
  const bool scaled = p.scale_mode != SCALE_NONE && p.scale_mode != SCALE_ONE;
  const int sm = tid % MP, sq0 = tid / MP;
  const gptr<float> st = as_global(p.stats_in) + (m_base + sm < p.M ? m_base + sm : 0);
  float sv[LB];
  if (scaled) {
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int t = sq0 + u * Q;
      sv[u] = st[(size_t)(t < p.stats_tiles ? t : 0) * p.stats_ld];
    }
  }
#pragma unroll
  for (int j = 0; j < (DMA ? NST - 1 : NST); ++j) load_stage(j, it_beg + j < it_end ? it_beg + j : it_end - 1);
  if (p.scale_mode == SCALE_ONE) {
    if (tid < MP) s_scale[tid] = 1.f;
    __syncthreads();
  } else if (scaled) {
    float part = 0.f;
#pragma unroll
    for (int u = 0; u < LB; ++u)
      if (sq0 + u * Q < p.stats_tiles) part += sv[u];
    for (int t0 = sq0 + LB * Q; t0 < p.stats_tiles; t0 += LB * Q) {    // large M only
#pragma unroll
      for (int u = 0; u < LB; ++u) {
        const int t = t0 + u * Q;
        sv[u] = st[(size_t)(t < p.stats_tiles ? t : 0) * p.stats_ld];
      }
#pragma unroll
      for (int u = 0; u < LB; ++u)
        if (t0 + u * Q < p.stats_tiles) part += sv[u];
    }
    // [Q][MP] scratch, free until the first step: the second activation
    // buffer, or (direct-to-LDS) the ring slot the prologue leaves empty
    float* s_part = DMA ? reinterpret_cast<float*>(adma + (NST - 1) * STG) : reinterpret_cast<float*>(lds[1]);
    s_part[sq0 * MP + sm] = part;
    __syncthreads();
    if (tid < MP) {
      float S = 0.f;
#pragma unroll
      for (int q = 0; q < Q; ++q) S += s_part[q * MP + tid];
      s_scale[tid] = m_base + tid < p.M ? row_scale_of(p, m_base + tid, S) : 0.f;
    }
    __syncthreads();
  }
  if constexpr (WD) {
    // Ring of NST LDS stages, NST - 1 in flight; nothing lives in registers
    // across steps but the accumulators, so the slot index is a plain
    // counter and the loop runs one tile's part of the range at a time,
    // finishing the tile after it.  Step: wait for this wave's loads of the
    // slot (only the NST - 2 later stages may remain in flight), barrier
    // (every wave's part landed, every wave done with the previous slot),
    // refill the previous slot with iteration it + NST - 1, multiply.
    int it = it_beg;
    int j = 0;
    while (true) {
      const int tile = it / ipt;
      const int kb = it - tile * ipt;
      const int seg_end = (tile + 1) * ipt < it_end ? (tile + 1) * ipt : it_end;
      for (; it < seg_end; ++it) {
        wait_vmcnt<(NST - 2) * (DBLK + WLD)>();
        __builtin_amdgcn_s_barrier();
        load_stage(j == 0 ? NST - 1 : j - 1, it + NST - 1 < it_end ? it + NST - 1 : it_end - 1);
        compute(0, j);
        j = j == NST - 1 ? 0 : j + 1;
      }
      finish(tile, kb, it - tile * ipt);
      if (it >= it_end) break;
    }
    wait_vmcnt<0>();                               // no load into LDS outlives the workgroup
    return;
  }
  if constexpr (DMA) {
    // Ring of NST stages, NST - 1 in flight.  Step `it` (stage j = it % NST):
    // wait for this wave's part of stage j (the loads issued after it are
    // stage j's register weights, unless they too went to LDS, and the
    // NST - 2 later stages; anything the epilogue issues only adds to
    // that), then the barrier makes every wave's part visible and says
    // every wave is done with stage j - 1, whose slot and registers then
    // take iteration it + NST - 1.
    int it = it_beg;
    int seg_k0 = it_beg % ipt;
    auto dstep = [&](auto J) __attribute__((always_inline)) -> bool {
      constexpr int j = decltype(J)::value;
      wait_vmcnt<(WD ? 0 : WLD) + (NST - 2) * (DBLK + WLD)>();
      __builtin_amdgcn_s_barrier();
      load_stage((j + NST - 1) % NST, it + NST - 1 < it_end ? it + NST - 1 : it_end - 1);
      compute(0, j);
      const bool has_next = it + 1 < it_end;
      const int tile = it / ipt;
      const int kk = it - tile * ipt;
      if (!has_next || kk == ipt - 1) {
        finish(tile, seg_k0, kk + 1);
        seg_k0 = 0;
      }
      if (!has_next) return false;
      ++it;
      return true;
    };
    while (true) {
      if (!dstep(std::integral_constant<int, 0>{})) break;
      if (!dstep(std::integral_constant<int, 1 % NST>{})) break;
      if constexpr (NST > 2) {
        if (!dstep(std::integral_constant<int, 2 % NST>{})) break;
      }
      if constexpr (NST > 3) {
        if (!dstep(std::integral_constant<int, 3 % NST>{})) break;
      }
      if constexpr (NST > 4) {
        if (!dstep(std::integral_constant<int, 4 % NST>{})) break;
      }
      if constexpr (NST > 5) {
        if (!dstep(std::integral_constant<int, 5 % NST>{})) break;
      }
      if constexpr (NST > 6) {
        if (!dstep(std::integral_constant<int, 6 % NST>{})) break;
      }
      if constexpr (NST > 7) {
        if (!dstep(std::integral_constant<int, 7 % NST>{})) break;
      }
    }
    wait_vmcnt<0>();                               // no load into LDS outlives the workgroup
    return;
  }
  store_a(0, 0, it_beg);
  __syncthreads();

  // Stream the workgroup's range.  Step `it` uses stage it % NST: multiply,
  // finish a tile whose last iteration this was, stage the next iteration's
  // activations, then refill the stage with iteration it + NST (clamped to
  // the range: a re-read of data this wave just fetched, an L2 hit).  The
  // loop is unrolled over the stages so that every register index is static.
  int it = it_beg;
  int buf = 0;
  int seg_k0 = it_beg % ipt;
  auto step = [&](auto J) __attribute__((always_inline)) -> bool {
    constexpr int j = decltype(J)::value;
    constexpr int jn = (j + 1) % NST;
    const bool has_next = it + 1 < it_end;
    compute(buf, j);
    const int tile = it / ipt;
    const int kk = it - tile * ipt;
    if (!has_next || kk == ipt - 1) {
      finish(tile, seg_k0, kk + 1);
      seg_k0 = 0;
    }
    if (!has_next) return false;
    store_a(buf ^ 1, jn, it + 1);
    load_stage(j, it + NST < it_end ? it + NST : it_end - 1);
    __syncthreads();
    buf ^= 1;
    ++it;
    return true;
  };
  while (true) {
    if (!step(std::integral_constant<int, 0>{})) break;
    if constexpr (NST > 1) {
      if (!step(std::integral_constant<int, 1 % NST>{})) break;
    }
    if constexpr (NST > 2) {
      if (!step(std::integral_constant<int, 2 % NST>{})) break;
    }
    if constexpr (NST > 3) {
      if (!step(std::integral_constant<int, 3 % NST>{})) break;
    }
  }
}

// ---------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------
// Stream-K and whole-K tiles both assume every workgroup of the grid is
// resident at once: the grid is capped at what the kernel's occupancy
// allows on all CUs.
template <typename TW, typename TA, int MT, int NWB, int KSUB, int PD, int PRO, int EPI, bool DMA, bool WD, bool TL>
static int resident_cap(int grid_cap, int num_cus) {
  static int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_stream_kernel<TW, TA, MT, NWB, KSUB, PD, PRO, EPI, DMA, WD, TL>,
                                                      256, 0) != hipSuccess ||
        n < 1)
      n = 1;
    per_cu = n;
  }
  const int cap = per_cu * num_cus;
  return cap < grid_cap ? cap : grid_cap;
}

constexpr int kMaxSplitWide = 6;   // contributors per tile for MT x NWB >= 8
constexpr int kWholeKSteps = 16;   // MT x NWB >= 8: K iterations up to which tiles run whole-K
constexpr int kMaxSplitSmall = 8;  // contributors per tile for MT <= 2 (one load batch of the finisher)

template <typename TW, typename TA, int MT, int NWB, int KSUB, int PD, int PRO, int EPI, bool DMA = false,
          bool WD = false, bool TL = false>
static hipError_t launch_t(GemmParams p, int grid_cap, int num_cus, hipStream_t s) {
  static_assert(NWB == 1 || NWB == 2 || (WD && NWB == 4), "tile widths");
  static_assert(EPI != EPI_SWIGLU || NWB % 2 == 0, "SwiGLU pairs gate and up blocks");
  constexpr int KS = 32 * KSUB;
  grid_cap = resident_cap<TW, TA, MT, NWB, KSUB, PD, PRO, EPI, DMA, WD, TL>(grid_cap, num_cus);
  // row blocks share the resident grid and the CUs; over at most 20 MB of
  // weights they take two workgroups per CU between them (B=8 per forward:
  // the 27B bridge's three GEMMs 217 -> 208 us, the 35B-style O 119 -> 112;
  // the 25 MB q|k|v went 118 -> 135 and keeps one)
  const int RB = p.rb_rows > 0 ? (p.M + MT * 16 - 1) / (MT * 16) : 1;
  if (p.rb_rows > 0 && (p.rb_rows != MT * 16 || !TL)) return hipErrorInvalidValue;
  grid_cap = (grid_cap + RB - 1) / RB;
  if (RB > 1) {
    const int64_t wbytes = (int64_t)p.nblk * 16 * p.K * (int64_t)sizeof(TW);
    num_cus = ((wbytes <= ((int64_t)20 << 20) ? 2 : 1) * num_cus + RB - 1) / RB;
  }
  p.ipt = (p.K + KS - 1) / KS;
  p.tiles = (p.nblk + 4 * NWB - 1) / (4 * NWB);
  const int64_t TI = (int64_t)p.tiles * p.ipt;
  // One CU streams only about 25 GB/s, so every CU must take part: whole-K
  // tiles when there are at least as many tiles as CUs (and all fit at
  // once), or when a tile's whole K fits in the register stages (its loads
  // all go out at once and no partials have to be combined); otherwise
  // stream-K over the resident grid.
  // A split tile is finished by one workgroup that reads every contributor's
  // partial tile (MT x NWB x 4 KB); for the wide tiles of large blocks that
  // read dominates past a few contributors, so their splits are capped.
  // Small tiles take one workgroup per CU (a second one per CU only adds
  // contributors) and at most as many contributors as the finisher loads in
  // one batch (the 16-row bridge projection onto 1024 codes ran 15 us split
  // 20 ways, 10 us split 8 ways).
  // Wide tiles over a short K (the bridge's [G; G_p; A] and W_l at 128
  // rows): whole-K tiles; a split's partial tiles (MT x NWB x 4 KB each)
  // would outweigh the few weights each contributor streams.
  int G;
  if (p.tiles <= grid_cap && (p.tiles >= num_cus || p.ipt <= PD + 1 || (MT * NWB >= 8 && p.ipt <= kWholeKSteps))) {
    G = p.tiles;
  } else {
    int64_t g = TI < grid_cap ? TI : grid_cap;
    if (MT * NWB >= 8 && g > (int64_t)p.tiles * kMaxSplitWide) g = (int64_t)p.tiles * kMaxSplitWide;
    if (MT <= 2) {
      // one workgroup per CU (a second one only adds contributors: O and
      // down at 16 rows ran 7 and 4 % slower with two), except for one-byte
      // weights, whose kernel holds two (the FP8 head 1 % faster per call)
      const int per_cu = (DMA && sizeof(TW) == 1) ? 2 : 1;
      if (g > per_cu * num_cus) g = per_cu * num_cus;
      if (g > (int64_t)p.tiles * kMaxSplitSmall) g = (int64_t)p.tiles * kMaxSplitSmall;
    }
    G = (int)g;
  }
  // two partial slots per workgroup, each NWB * MT * 4 KB; a counter per
  // tile of every row block
  if ((size_t)2 * G * RB * (NWB * MT * 256 * 4) > p.partial_floats || (int64_t)RB * p.tiles > kMaxTiles)
    return hipErrorInvalidValue;
  p.xcd_remap = (G % 8 == 0) ? 1 : 0;
  DSPINE_LAUNCH((gemm_stream_kernel<TW, TA, MT, NWB, KSUB, PD, PRO, EPI, DMA, WD, TL>), dim3(G, RB), dim3(256), 0, s,
                p);
  return hipGetLastError();
}

int gemm_stream_grid_cap(int num_cus) { return 2 * num_cus < kMaxGrid ? 2 * num_cus : kMaxGrid; }

int gemm_stream_row_tile(int M) {
  const int mt = (M + 15) / 16;
  return 16 * (mt <= 1 ? 1 : mt <= 2 ? 2 : mt <= 4 ? 4 : 8);
}

size_t gemm_stream_partial_floats(int rows) {
  // 2 slots per workgroup of a grid of at most kMaxGrid, each NWB*MT*256*4
  // floats with NWB <= 2 and MT the row tile of `rows` (see launch_mt)
  const int mt = gemm_stream_row_tile(rows < 1 ? 1 : rows > kMaxRows ? kMaxRows : rows) / 16;
  return (size_t)2 * kMaxGrid * (2 * mt * 256 * 4);
}

// statistics lists a GEMM of N output columns writes (one per 64 columns)
int gemm_stream_stat_lists(int n) { return (n + 63) / 64; }

// largest M whose prologues form scaled operands themselves
int gemm_stream_fused_rows() { return 32; }

// Tile shape and pipeline depth per row-tile count: a wave keeps about 32 KB
// of weights in flight when M is small; large M spends its registers on the
// accumulators and the activation stages instead.
template <typename TW, typename TA, int PRO, int EPI>
static hipError_t launch_mt(const GemmParams& p, int grid_cap, int num_cus, hipStream_t s) {
  const int mt = ((p.rb_rows > 0 ? p.rb_rows : p.M) + 15) / 16;
  constexpr bool kHalf = Elt<TA>::kBytes == 2;
  // row blocks (16 or 32 rows each): 16-bit copy operands, the small tile
  // shapes, weights loaded with the ordinary cache policy
  if (p.rb_rows > 0) {
    if constexpr (kHalf && sizeof(TW) == 2 && PRO == PRO_COPY && EPI != EPI_SWIGLU) {
      if (mt <= 1) {
        if (p.K % 512 == 0) return launch_t<TW, TA, 1, 1, 16, 1, PRO, EPI, true, false, true>(p, grid_cap, num_cus, s);
        if (p.K % 256 == 0) return launch_t<TW, TA, 1, 1, 8, 3, PRO, EPI, true, false, true>(p, grid_cap, num_cus, s);
        return launch_t<TW, TA, 1, 1, 8, 3, PRO, EPI, false, false, true>(p, grid_cap, num_cus, s);
      }
      if (mt <= 2) {
        if (p.K % 256 == 0) return launch_t<TW, TA, 2, 1, 8, 2, PRO, EPI, true, false, true>(p, grid_cap, num_cus, s);
        return launch_t<TW, TA, 2, 1, 8, 3, PRO, EPI, false, false, true>(p, grid_cap, num_cus, s);
      }
    }
    return hipErrorInvalidValue;
  }
  if constexpr (sizeof(TW) == 1 && PRO == PRO_COPY) {
    // One-byte FP8 weights: 512-K stages (16 fragments of 8 bytes per
    // lane, as many bytes in flight as 16-bit weights in 256-K stages) with
    // the activation chunks going global -> LDS directly, so that the
    // registers hold only weight stages and two workgroups fit on a CU
    if (p.K % 512 == 0) {
      if (mt <= 1) return launch_t<TW, TA, 1, 1, 16, 3, PRO, EPI, true>(p, grid_cap, num_cus, s);
      if (mt <= 2) return launch_t<TW, TA, 2, 1, 16, 2, PRO, EPI, true>(p, grid_cap, num_cus, s);
    }
  }
  constexpr int NWB1 = EPI == EPI_SWIGLU ? 2 : 1;   // narrow tiles: more of them
  constexpr int PD_SMALL = PRO == PRO_BRIDGE_MSG ? 1 : (NWB1 == 2 ? 2 : 3);
  if constexpr (kHalf && sizeof(TW) == 2 && PRO == PRO_COPY && EPI != EPI_SWIGLU) {
    // operands already in memory as 16-bit rows: they go global -> LDS
    // directly, the registers hold only the weight stages.  16 rows: two
    // stages of 512 K (16 KB of weights per wave each; two workgroups per
    // CU); the LM head at B=1 runs 0.69 of HBM this way against 0.59 with
    // four stages of 256 K in registers and the operand staged by the waves
    if (mt <= 1 && p.K % 512 == 0) return launch_t<TW, TA, 1, 1, 16, 1, PRO, EPI, true>(p, grid_cap, num_cus, s);
    if (p.K % 256 == 0) {
      if (mt <= 1) return launch_t<TW, TA, 1, 1, 8, 3, PRO, EPI, true>(p, grid_cap, num_cus, s);
      if (mt <= 2) return launch_t<TW, TA, 2, 1, 8, 2, PRO, EPI, true>(p, grid_cap, num_cus, s);
    }
  }
  if (mt <= 1) return launch_t<TW, TA, 1, NWB1, kHalf ? 8 : 4, PD_SMALL, PRO, EPI>(p, grid_cap, num_cus, s);
  if (mt <= 2) return launch_t<TW, TA, 2, NWB1, kHalf ? 8 : 4, PD_SMALL, PRO, EPI>(p, grid_cap, num_cus, s);
  if constexpr (PRO == PRO_COPY || PRO == PRO_GATHER) {
    // 64 and 128 rows take pre-scaled operands (the launcher's caller forms
    // them), in 128-column tiles so that each staged activation chunk feeds
    // twice the weights
    // 16-bit operands with K a multiple of the stage move the activation
    // chunks global -> LDS directly, leaving the registers to four weight
    // stages
    if constexpr (kHalf) {
      if (p.K % 128 == 0) {
        if (mt <= 4) return launch_t<TW, TA, 4, 2, 4, 3, PRO, EPI, true>(p, grid_cap, num_cus, s);
        // 128 rows: weights move global -> LDS too (a 4-stage ring of 64-K
        // stages, full-line activation blocks); 1.2-1.3x faster than
        // weights in registers, whose stages the allocator cannot keep.
        // One-byte FP8 weights keep their (half as large) stages in registers.
        // Narrow outputs take 64-column tiles: twice the workgroups, and
        // half the partial tile each finisher reads.  At the 27B geometry
        // that is q|k|v, O and the bridge's three projections (B=8 forward
        // 1.953 -> 1.79 ms; 35B B=8 1.49 -> 1.33 ms); over a long K and
        // N > 2048 (the 27B down and feature projections) the wide tiles
        // stay faster.
        if constexpr (sizeof(TW) == 2) {
          if constexpr (EPI != EPI_SWIGLU)
            if (p.nblk <= 128 || (p.nblk <= 384 && p.K <= 8192))
              return launch_t<TW, TA, 8, 1, 2, 3, PRO, EPI, true, true>(p, grid_cap, num_cus, s);
          return launch_t<TW, TA, 8, 2, 2, 3, PRO, EPI, true, true>(p, grid_cap, num_cus, s);
        }
        else return launch_t<TW, TA, 8, 2, 4, 3, PRO, EPI, true>(p, grid_cap, num_cus, s);
      }
    }
    if (mt <= 4) return launch_t<TW, TA, 4, 2, kHalf ? 4 : 2, 1, PRO, EPI>(p, grid_cap, num_cus, s);
    return launch_t<TW, TA, 8, 2, kHalf ? 4 : 1, 1, PRO, EPI>(p, grid_cap, num_cus, s);
  }
  return hipErrorInvalidValue;
}

// The (prologue, epilogue) pairs the hot path uses.
template <typename TW, typename TA>
static hipError_t launch_kind(const GemmParams& p, int grid_cap, int num_cus, hipStream_t s) {
  switch (p.pro) {
    case PRO_BRIDGE_MSG:
      if (p.epi == EPI_ADD_ROWSCALE)
        return launch_mt<TW, TA, PRO_BRIDGE_MSG, EPI_ADD_ROWSCALE>(p, grid_cap, num_cus, s);
      break;
    case PRO_COPY:
      if (p.epi == EPI_STORE) return launch_mt<TW, TA, PRO_COPY, EPI_STORE>(p, grid_cap, num_cus, s);
      if (p.epi == EPI_ADD) return launch_mt<TW, TA, PRO_COPY, EPI_ADD>(p, grid_cap, num_cus, s);
      if (p.epi == EPI_SWIGLU) return launch_mt<TW, TA, PRO_COPY, EPI_SWIGLU>(p, grid_cap, num_cus, s);
      if (p.epi == EPI_ADD_ROWSCALE) return launch_mt<TW, TA, PRO_COPY, EPI_ADD_ROWSCALE>(p, grid_cap, num_cus, s);
      break;
    case PRO_NORM:
      if (p.epi == EPI_STORE) return launch_mt<TW, TA, PRO_NORM, EPI_STORE>(p, grid_cap, num_cus, s);
      if (p.epi == EPI_SWIGLU) return launch_mt<TW, TA, PRO_NORM, EPI_SWIGLU>(p, grid_cap, num_cus, s);
      break;
    case PRO_SCALE:
      if (p.epi == EPI_STORE) return launch_mt<TW, TA, PRO_SCALE, EPI_STORE>(p, grid_cap, num_cus, s);
      break;
    default:
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_stream(const GemmParams& p, int dtype, int num_cus, hipStream_t s) {
  const int grid_cap = gemm_stream_grid_cap(num_cus);
  if (p.w_fp8) {                      // the LM head's FP8 copy: scores of fp16 rows only
    if (dtype != DT_BF16 || p.epi != EPI_STORE || !p.col_scale || p.code_anchor || p.pro != PRO_COPY || p.K % 64)
      return hipErrorInvalidValue;
    return launch_mt<fp8_t, f16_t, PRO_COPY, EPI_STORE>(p, grid_cap, num_cus, s);
  }
  if (p.pro == PRO_COPY && p.a_bf16) {   // bf16 rows (the SwiGLU hidden) x bf16 weights
    if (dtype != DT_BF16) return hipErrorInvalidValue;
    if (p.epi == EPI_ADD) return launch_mt<bf16_t, bf16_t, PRO_COPY, EPI_ADD>(p, grid_cap, num_cus, s);
    if (p.epi == EPI_STORE) return launch_mt<bf16_t, bf16_t, PRO_COPY, EPI_STORE>(p, grid_cap, num_cus, s);
    return hipErrorInvalidValue;
  }
  if (p.pro == PRO_GATHER) {          // target features, stored output only
    if (p.epi != EPI_STORE) return hipErrorInvalidValue;
    if (dtype == DT_BF16) return launch_mt<bf16_t, bf16_t, PRO_GATHER, EPI_STORE>(p, grid_cap, num_cus, s);
    return launch_mt<float, float, PRO_GATHER, EPI_STORE>(p, grid_cap, num_cus, s);
  }
  if (dtype == DT_BF16) return launch_kind<bf16_t, f16_t>(p, grid_cap, num_cus, s);
  return launch_kind<float, float>(p, grid_cap, num_cus, s);
}

}  // namespace dspine
