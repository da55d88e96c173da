// Block attention over ring context + block rows (a6), with the q/k head
// RMSNorm and RoPE of the block (a5 tail) fused into the prologue.
//
// [NIF, layer equations]: a = attention(q, concat(K_ctx, k), concat(V_ctx,
// v), scale 1/sqrt(D), layer mask); q, k are head-RMSNormed then rotated.
// [NIF, draft attention]: the mask keeps |p_key - p_query| < S on local
// layers; block keys are all visible (bidirectional) unless block_causal.
//
// Layout on gfx950.  A workgroup serves one (key split, KV head, request):
// GRP waves, one per query head of the GQA group, times NSUB key
// sub-streams.  Each sub-stream (GRP waves) takes every NSUB-th 32-key tile
// of the split, stages it in its own LDS buffers and keeps several tiles in
// flight in registers, so the CU always has waves with work while loads are
// outstanding.  A wave holds the block's (<= 16) rows of its head and
// computes S^T = K Q^T with 16x16x32 MFMAs: each lane then owns one query
// row (lane % 16), which makes the online-softmax rescale of the
// O^T = V^T P^T accumulators lane-local.  Sub-streams are combined through
// LDS with their log-sum-exp; splits over context keys publish partials
// that a second, small kernel merges (one wave per request, query head and
// quarter of the head dims).  Ring slots advance in int32 from one modulo per
// workgroup; the window and tail masks run only on the tiles that straddle
// an edge.
#include "dspine_device.hpp"
#include "dspine_internal.hpp"

namespace dspine {

// Operand types: a BF16 model keeps Q and K in LDS as fp16 (context keys are
// stored bf16 and widen to fp16 exactly), P and V as fp16 (context values are
// stored fp16); a float32 model uses float throughout.  Block values are
// scratch of this forward and are rounded straight to the fp16 operand.
__device__ __forceinline__ void put_v(f16_t* d, float v) { d->bits = f32_to_f16_bits(v); }
__device__ __forceinline__ void put_v(float* d, float v) { *d = v; }

// one 16-byte chunk of stored keys -> the LDS operand type
__device__ __forceinline__ u32x4 key_chunk(u32x4 v, bf16_t*, f16_t*) { return bf16x8_to_f16x8(v); }
__device__ __forceinline__ u32x4 key_chunk(u32x4 v, float*, float*) { return v; }

// P fragment (8 probabilities of one row) in the PV operand type
__device__ __forceinline__ void pack_p(Frag<f16_t>& f, float (&pv)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint16_t lo = f32_to_f16_bits(pv[2 * e]);
    const uint16_t hi = f32_to_f16_bits(pv[2 * e + 1]);
    pv[2 * e] = f16_bits_to_f32(lo);       // normalise with the rounded weights
    pv[2 * e + 1] = f16_bits_to_f32(hi);
    f.v[e] = (uint32_t)lo | ((uint32_t)hi << 16);
  }
}
__device__ __forceinline__ void pack_p(Frag<float>& f, float (&pv)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e >> 2][e & 3] = __float_as_uint(pv[e]);
}
// V^T fragment: d row `d`, keys {4q..4q+3} then {16+4q..16+4q+3}
__device__ __forceinline__ void load_vt(Frag<f16_t>& f, const f16_t* row, int q) {
  const uint2 a = *reinterpret_cast<const uint2*>(row + 4 * q);
  const uint2 b = *reinterpret_cast<const uint2*>(row + 16 + 4 * q);
  f.v = u32x4{a.x, a.y, b.x, b.y};
}
__device__ __forceinline__ void load_vt(Frag<float>& f, const float* row, int q) {
  f.v[0] = *reinterpret_cast<const u32x4*>(row + 4 * q);
  f.v[1] = *reinterpret_cast<const u32x4*>(row + 16 + 4 * q);
}

// Compile-time shape of one attention instantiation.
template <typename TQ, typename TV, int D, int GRP>
struct AttnShape {
  static constexpr int EQ = (int)sizeof(TQ), EV = (int)sizeof(TV);
  // padded row of Q / K tiles: with 16 halves of padding (72 words at D =
  // 128) the 16 lanes that one cycle of a 128-bit LDS read serves land on
  // distinct banks (8 halves left pairs of them on one bank)
  static constexpr int LDQ = D + (EQ == 2 ? 16 : 16 / EQ);
  static constexpr int LDV = 32 + 16 / EV;              // padded row of V^T tiles (32 keys)
  static constexpr int K_BYTES = 32 * LDQ * EQ;
  static constexpr int V_BYTES = D * LDV * EV;
  static constexpr int TILE = K_BYTES + V_BYTES;        // one K tile + one V^T tile
  static constexpr int Q_BYTES = GRP * 16 * LDQ * EQ;
  static constexpr int PART = 64 * (D / 4 + 2) * 4;     // one wave's (o, m, l) in LDS
  static constexpr int LIMIT = 156 * 1024;
  // slots tile slots per key sub-stream and the block's tile
  static constexpr bool fits(int n, int slots) {
    return Q_BYTES + (slots * n + 1) * TILE <= LIMIT && GRP * (n - 1) * PART <= Q_BYTES + (slots * n + 1) * TILE;
  }
  // at most 8 waves (512 threads): 256 registers per wave, two workgroups per CU
  static constexpr int NSUB_MAX = 8 / GRP < 1 ? 1 : 8 / GRP < 4 ? 8 / GRP : 4;
  static constexpr int NSUB = (NSUB_MAX >= 4 && fits(4, 1)) ? 4 : (NSUB_MAX >= 2 && fits(2, 1)) ? 2 : 1;
  // two slots per sub-stream where they fit: a round stages its tile while
  // other waves may still read the previous round's (one barrier a round)
  static constexpr int NSLOT = fits(NSUB, 2) ? 2 : 1;
  static constexpr int NT = 64 * GRP * NSUB;
  static constexpr int SMEM = Q_BYTES + (NSLOT * NSUB + 1) * TILE;
  static_assert(fits(NSUB, NSLOT), "attention LDS");
  static_assert((D / 16) % NSUB == 0, "merge split of the head dimension");
};

// KVNT: the context K/V tiles are read with non-temporal loads (a layer's
// context is read once; large ones otherwise evict lines that are re-read)
template <typename TW, typename TQ, typename TV, int D, int GRP, bool KVNT = false>
__global__ __launch_bounds__((AttnShape<TQ, TV, D, GRP>::NT)) void attention_kernel(const AttnParams p) {
  using Sh = AttnShape<TQ, TV, D, GRP>;
  static_assert(sizeof(TW) == sizeof(TQ), "stored keys and key operands have one element size");
  constexpr int EQ = Sh::EQ, EV = Sh::EV, LDQ = Sh::LDQ, LDV = Sh::LDV;
  constexpr int NSUB = Sh::NSUB, NSLOT = Sh::NSLOT;
  constexpr int GT = 64 * GRP;                          // threads of one sub-stream
  constexpr int PSZ = 64 * (D / 4) + 32;                // floats of one split partial in HBM

  __shared__ __attribute__((aligned(16))) char smem[Sh::SMEM];
  TQ* const sQ = reinterpret_cast<TQ*>(smem);           // [GRP][16][LDQ]
  auto sK = [&](int t) { return reinterpret_cast<TQ*>(smem + Sh::Q_BYTES + t * Sh::TILE); };
  auto sVt = [&](int t) { return reinterpret_cast<TV*>(smem + Sh::Q_BYTES + t * Sh::TILE + Sh::K_BYTES); };

  const int b = blockIdx.z, g = blockIdx.y, split = blockIdx.x;
  // the wave index is uniform per wave: keeping it scalar keeps the role
  // branches and the parameter loads they select (gains, columns) scalar,
  // instead of vector loads queued behind the tile prefetch
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = w % GRP, sub = w / GRP;                // head within the group, sub-stream
  const int h = g * GRP + hl;
  const int gtid = tid - sub * GT;                      // thread index within the sub-stream
  const int W = p.W, S = p.S;
  const int64_t F = p.F[b];
  const int64_t cbeg = p.lo0[b] + (int64_t)split * p.kps[b];
  const int64_t cend = (cbeg + p.kps[b] < F) ? cbeg + p.kps[b] : F;
  const int nkeys = cend > cbeg ? (int)(cend - cbeg) : 0;
  const bool has_block = split == p.nsplit - 1;
  const int row_base = b * W;

  // ---- context keys [cbeg, cend) in tiles of 32 --------------------------
  const gptr<TW> kring = as_global(reinterpret_cast<const TW*>(p.kring[b]));
  const gptr<TV> vring = as_global(reinterpret_cast<const TV*>(p.vring[b]));
  const size_t head_base = (size_t)g * (size_t)p.cap[b];
  const int slot0 = S > 0 ? (int)ring_slot(cbeg, S) : 0;   // slot of cbeg; later keys advance in int32
  constexpr int KCH = D * EQ / 16, KEPC = 16 / EQ;      // 16-byte chunks per key row
  constexpr int VCH = D * EV / 16, VEPC = 16 / EV;
  // chunks per thread of the sub-stream; spare threads re-load a chunk and store nothing
  constexpr int KPT = (32 * KCH + GT - 1) / GT, VPT = (32 * VCH + GT - 1) / GT;
  constexpr int PFR = 16 / (KPT + VPT);
  constexpr int PF = PFR < 1 ? 1 : PFR > 4 ? 4 : PFR;   // tiles in flight per sub-stream
  u32x4 kreg[PF][KPT], vreg[PF][VPT];
  const int n_tiles = (nkeys + 31) / 32;
  const int rounds = (n_tiles + NSUB - 1) / NSUB;       // sub-stream `sub` takes tiles r*NSUB + sub

  // key row kr of tile i -> element offset of its ring row (positions past
  // the split's end re-read its last key: in bounds, masked later)
  auto key_row = [&](int i, int kr) -> size_t {
    int rel = 32 * i + kr;
    rel = rel < nkeys ? rel : nkeys - 1;
    int64_t slot;
    if (S > 0) {
      const int sl = slot0 + rel;
      slot = sl >= S ? sl - S : sl;
    } else {
      slot = cbeg + rel;
    }
    return (head_base + (size_t)slot) * D;
  };
  // V chunks: with 16-bit values and an even count per thread, a thread
  // takes keys 2m and 2m+1 of one 8-value part (pair index pi = gtid +
  // (q/2) GT, m = pi % 16, part = pi / 16), so that the transposed store
  // writes both keys of a head dim as one 32-bit word; otherwise chunk c =
  // gtid + q GT is key c / VCH, part c % VCH.
  constexpr bool kPairV = EV == 2 && VPT % 2 == 0;
  auto v_chunk = [&](int q, int& kr, int& part) __attribute__((always_inline)) -> bool {
    if constexpr (kPairV) {
      const int pi = gtid + (q >> 1) * GT;
      kr = 2 * (pi % 16) + (q & 1);
      part = pi / 16;
      return pi < 16 * VCH;
    } else {
      const int c = gtid + q * GT;
      kr = c / VCH;
      part = c % VCH;
      return c < 32 * VCH;
    }
  };
  auto load_tile = [&](u32x4 (&kr_)[KPT], u32x4 (&vr_)[VPT], int i) {
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const int c = (gtid + q * GT) % (32 * KCH);
      const gptr<void> src = (gptr<void>)(kring + key_row(i, c / KCH) + (c % KCH) * KEPC);
      if constexpr (KVNT) kr_[q] = gload16_nt(src);
      else kr_[q] = gload16(src);
    }
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
      int kr, part;
      if (!v_chunk(q, kr, part)) kr = part = 0;          // spare thread: re-load chunk 0
      const gptr<void> src = (gptr<void>)(vring + key_row(i, kr) + part * VEPC);
      if constexpr (KVNT) vr_[q] = gload16_nt(src);
      else vr_[q] = gload16(src);
    }
  };
  auto store_tile = [&](const u32x4 (&kr_)[KPT], const u32x4 (&vr_)[VPT], int i, int slot) {
    TQ* k_t = sK(NSLOT * sub + slot);
    TV* v_t = sVt(NSLOT * sub + slot);
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const int c = gtid + q * GT;
      if (c < 32 * KCH)
        *reinterpret_cast<u32x4*>(&k_t[(c / KCH) * LDQ + (c % KCH) * KEPC]) =
            key_chunk(kr_[q], (TW*)nullptr, (TQ*)nullptr);
    }
    if constexpr (kPairV) {
      // both keys of a head dim in one 32-bit word; lanes whose part has bit
      // 1 set take the dims in the order 4..7, 0..3, which puts the 64 lanes
      // of a wave on distinct banks (a V^T row is LDV/2 words)
#pragma unroll
      for (int q = 0; q < VPT; q += 2) {
        int kr, part;
        if (!v_chunk(q, kr, part)) continue;
        u32x4 a = 32 * i + kr < nkeys ? vr_[q] : u32x4{0, 0, 0, 0};
        u32x4 b = 32 * i + kr + 1 < nkeys ? vr_[q + 1] : u32x4{0, 0, 0, 0};
        const bool rot = (part >> 1) & 1;
        if (rot) {
          a = u32x4{a[2], a[3], a[0], a[1]};
          b = u32x4{b[2], b[3], b[0], b[1]};
        }
        uint32_t* row = reinterpret_cast<uint32_t*>(v_t) + kr / 2;
#pragma unroll
        for (int e = 0; e < VEPC; ++e) {
          const int dim = part * VEPC + ((e + (rot ? 4 : 0)) & 7);
          const uint32_t lo = e & 1 ? a[e >> 1] >> 16 : a[e >> 1] & 0xffffu;
          const uint32_t hi = e & 1 ? b[e >> 1] >> 16 : b[e >> 1] & 0xffffu;
          row[dim * (LDV / 2)] = lo | (hi << 16);
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < VPT; ++q) {
        int kr, part;
        if (!v_chunk(q, kr, part)) continue;
        alignas(16) TV val[VEPC];
        *reinterpret_cast<u32x4*>(val) = 32 * i + kr < nkeys ? vr_[q] : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < VEPC; ++e) v_t[(part * VEPC + e) * LDV + kr] = val[e];
      }
    }
  };
  // ---- prologue: head RMSNorm + RoPE of the block's q (and k) rows --------
  // Round 0's tile goes out first, then the prologue's rows, then the tiles
  // of rounds 1 .. PF-1 (all clamped, in bounds): the prologue waits for its
  // rows and the first tile only (the memory counter retires in issue
  // order), while the later tiles stream in behind.
  constexpr int NP = D / 8;                   // rotation pairs per lane
  struct PrepIn {
    float xa[NP], xb[NP], ga[NP], gb[NP], co[NP], si[NP];
  };
  auto prep_load = [&](int col0, const void* gain, PrepIn& in) {
    const int r = lane >> 2, part = lane & 3;
    const bool live = r < W;
    const gptr<float> src = as_global(p.qkv) + (size_t)(row_base + (live ? r : 0)) * p.ld_qkv + col0;
    const gptr<float> cs = as_global(p.rope) + (size_t)(row_base + (live ? r : 0)) * D;   // (cos, sin) x D/2
    const gptr<TW> gw = as_global(reinterpret_cast<const TW*>(gain));
#pragma unroll
    for (int jj = 0; jj < NP; ++jj) {
      const int j = part * NP + jj;
      in.xa[jj] = src[j];
      in.xb[jj] = src[j + D / 2];
      in.ga[jj] = Elt<TW>::gload(gw, j);
      in.gb[jj] = Elt<TW>::gload(gw, j + D / 2);
      in.co[jj] = cs[2 * j];
      in.si[jj] = cs[2 * j + 1];
    }
  };
  auto prep_store = [&](const PrepIn& in, TQ* dst) {
    const int r = lane >> 2, part = lane & 3;
    const bool live = r < W;
    float ss = 0.f;
#pragma unroll
    for (int jj = 0; jj < NP; ++jj) ss += in.xa[jj] * in.xa[jj] + in.xb[jj] * in.xb[jj];
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    const float inv = rsqrtf(ss / D + p.eps);
#pragma unroll
    for (int jj = 0; jj < NP; ++jj) {
      const int j = part * NP + jj;
      const float a = in.xa[jj] * inv * in.ga[jj];
      const float c = in.xb[jj] * inv * in.gb[jj];
      Elt<TQ>::store(dst, r * LDQ + j, live ? a * in.co[jj] - c * in.si[jj] : 0.f);
      Elt<TQ>::store(dst, r * LDQ + j + D / 2, live ? c * in.co[jj] + a * in.si[jj] : 0.f);
    }
  };
  // wave roles: sub-stream 0 prepares its head's q rows; in the split that
  // owns the block, the last sub-stream's first wave its k rows and its
  // second wave (or the first, for one head per group) its v rows
  const bool do_q = sub == 0;
  const bool do_k = has_block && sub == NSUB - 1 && hl == 0;
  const bool do_v = has_block && sub == NSUB - 1 && hl == (GRP > 1 ? 1 : 0);
  const int kcol = p.nq * D + g * D;
  const int vcol = p.nq * D + p.nkv * D + g * D;
  if (n_tiles > 0) load_tile(kreg[0], vreg[0], sub < n_tiles ? sub : n_tiles - 1);
  PrepIn pin;
  if (do_q) prep_load(h * D, p.gq, pin);
  else if (do_k) prep_load(kcol, p.gk, pin);
  float vv[D / 4];
  if (do_v && !do_k) {
    const int r = lane >> 2, part = lane & 3;
    const bool live = r < W;
    const gptr<float> src =
        as_global(p.qkv) + (size_t)(row_base + (live ? r : 0)) * p.ld_qkv + vcol + part * (D / 4);
#pragma unroll
    for (int d = 0; d < D / 4; ++d) vv[d] = src[d];
  }
  if (n_tiles > 0) {
#pragma unroll
    for (int j = 1; j < PF; ++j) {
      const int i = j * NSUB + sub;
      load_tile(kreg[j], vreg[j], i < n_tiles ? i : n_tiles - 1);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (do_q) prep_store(pin, sQ + hl * 16 * LDQ);
  if (do_k) {
    if (do_q) prep_load(kcol, p.gk, pin);        // (only with one sub-stream)
    prep_store(pin, sK(NSLOT * NSUB));
    for (int e = lane; e < 16 * D; e += 64) Elt<TQ>::store(sK(NSLOT * NSUB), (16 + e / D) * LDQ + e % D, 0.f);
  }
  if (do_v) {
    const int r = lane >> 2, part = lane & 3;
    const bool live = r < W;
    if (do_k) {                                   // one head per group: this wave does k and v
      const gptr<float> src =
          as_global(p.qkv) + (size_t)(row_base + (live ? r : 0)) * p.ld_qkv + vcol + part * (D / 4);
#pragma unroll
      for (int d = 0; d < D / 4; ++d) vv[d] = src[d];
    }
#pragma unroll
    for (int d = 0; d < D / 4; ++d) put_v(&sVt(NSLOT * NSUB)[(part * (D / 4) + d) * LDV + r], live ? vv[d] : 0.f);
    for (int e = lane; e < 16 * D; e += 64) put_v(&sVt(NSLOT * NSUB)[(e / 16) * LDV + 16 + (e % 16)], 0.f);
  }
  __syncthreads();

  Frag<TQ> qf[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) qf[c].load(&sQ[(hl * 16 + (lane & 15)) * LDQ + c * 32 + 8 * (lane >> 4)]);

  const float scale_log2 = 1.4426950408889634f * rsqrtf((float)D);
  const int qrow = lane & 15;
  // first visible key of a row, relative to cbeg (clamped into int range)
  auto rel_lo = [&](int row) -> int {
    const int64_t d = ctx_row_lo(F, S, row) - cbeg;
    return d < -(1 << 30) ? -(1 << 30) : d > (1 << 30) ? (1 << 30) : (int)d;
  };
  const int lo_rel = rel_lo(qrow);
  const int lo_rel_max = rel_lo(W - 1);      // the last row starts latest
  float m_run = -INFINITY, l_lane = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0, 0, 0, 0};

  // One 32-key tile from LDS tile t: context keys k0.. (relative to cbeg),
  // with the window / tail mask only when the tile straddles an edge, or the
  // block's keys.
  auto process = [&](int t, int k0, bool is_block, bool mask) {
    f32x4 s[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
    const TQ* k_t = sK(t);
    const TV* v_t = sVt(t);
    // every fragment of the tile is read before the first multiply, so the
    // LDS latencies overlap (the V^T reads with the softmax)
    Frag<TQ> kf[D / 32][2];
    Frag<TV> vf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) kf[c][kt].load(&k_t[(kt * 16 + (lane & 15)) * LDQ + c * 32 + 8 * (lane >> 4)]);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) load_vt(vf[dt], &v_t[(dt * 16 + (lane & 15)) * LDV], lane >> 4);
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) mma16(s[kt], kf[c][kt], qf[c]);
    float sv[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int kidx = kt * 16 + 4 * (lane >> 4) + v;
        bool vis = true;
        if (is_block) {
          vis = qrow < W && kidx < W && block_key_visible(S, p.causal, qrow, kidx);
        } else if (mask) {
          const int rel = k0 + kidx;
          vis = rel < nkeys && rel >= lo_rel;
        }
        const float x = vis ? s[kt][v] * scale_log2 : -INFINITY;
        sv[kt * 4 + v] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    // Branch-free: a row with nothing visible yet (m_new = -inf) shifts by 0,
    // so its weights exp2(-inf) and its rescale exp2(-inf) are 0 (its o and
    // l are still 0).  The hardware exp2 flushes results below 2^-126
    // (weights that small relative to the row maximum are negligible).
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(sv[e] - m_use);
    Frag<TV> pf;
    pack_p(pf, pv);
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) psum += pv[e];
    l_lane = l_lane * alpha + psum;
    m_run = m_new;
    // once the row maxima settle, most tiles change none of them
    const bool rescale = !__all(alpha == 1.f);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      if (rescale) o[dt] *= alpha;
      mma16(o[dt], vf[dt], pf);
    }
  };

  // Round r stages register slot r % PF and refills it with round r + PF
  // while there is one (the number of rounds is the same for every
  // sub-stream of the workgroup, so the barriers match).  Its tile goes to
  // LDS slot r % NSLOT of the sub-stream.  With two slots one barrier per
  // round suffices: the slot a round overwrites was last read two rounds
  // before, and every wave has passed the barrier of the round in between.  Passes whose refills are all needed
  // run without any exit or condition around the loads: with a break or a
  // skipped refill inside the unrolled pass, the compiler routes every slot
  // through one set of registers, and the copy waits for the load just
  // issued, so each round would cost a full memory round trip.
  int r0 = 0;
  for (; r0 + 2 * PF <= rounds; r0 += PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int r = r0 + j;
      const int i = r * NSUB + sub;
      const bool live = i < n_tiles;
      if (live) store_tile(kreg[j], vreg[j], i, r % NSLOT);
      __syncthreads();
      const int inext = (r + PF) * NSUB + sub;
      load_tile(kreg[j], vreg[j], inext < n_tiles ? inext : n_tiles - 1);
      if (live) {
        const bool edge = 32 * i + 32 > nkeys || 32 * i < lo_rel_max;
        process(NSLOT * sub + r % NSLOT, 32 * i, false, edge);
      }
      if constexpr (NSLOT == 1) __syncthreads();   // the one slot is rewritten next round
    }
  }
  for (; r0 < rounds; r0 += PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int r = r0 + j;
      if (r >= rounds) break;
      const int i = r * NSUB + sub;
      const bool live = i < n_tiles;
      if (live) store_tile(kreg[j], vreg[j], i, r % NSLOT);
      __syncthreads();
      if (r + PF < rounds) {
        const int inext = (r + PF) * NSUB + sub;
        load_tile(kreg[j], vreg[j], inext < n_tiles ? inext : n_tiles - 1);
      }
      if (live) {
        const bool edge = 32 * i + 32 > nkeys || 32 * i < lo_rel_max;
        process(NSLOT * sub + r % NSLOT, 32 * i, false, edge);
      }
      if constexpr (NSLOT == 1) __syncthreads();   // the one slot is rewritten next round
    }
  }
  if (has_block && sub == NSUB - 1) process(NSLOT * NSUB, -1, true, true);
  __syncthreads();                                      // all tiles and Q done: LDS reused below

  // ---- combine the sub-streams of each head (lane-wise, through LDS) ------
  float* part = reinterpret_cast<float*>(smem);
  auto part_of = [&](int s, int head) { return part + (size_t)((s - 1) * GRP + head) * (64 * (D / 4 + 2)); };
  if (sub > 0) {
    float* pp = part_of(sub, hl);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int v = 0; v < 4; ++v) pp[(dt * 4 + v) * 64 + lane] = o[dt][v];
    pp[(D / 4) * 64 + lane] = m_run;
    pp[(D / 4 + 1) * 64 + lane] = l_lane;
  }
  __syncthreads();
  if (sub == 0) {
    float mstar = m_run;
#pragma unroll
    for (int s = 1; s < NSUB; ++s) mstar = fmaxf(mstar, part_of(s, hl)[(D / 4) * 64 + lane]);
    if (mstar != -INFINITY) {
      const float w0 = m_run == -INFINITY ? 0.f : exp2f(m_run - mstar);
      l_lane *= w0;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[dt] *= w0;
#pragma unroll
      for (int s = 1; s < NSUB; ++s) {
        const float* pp = part_of(s, hl);
        const float ms = pp[(D / 4) * 64 + lane];
        const float ws = ms == -INFINITY ? 0.f : exp2f(ms - mstar);
        l_lane += ws * pp[(D / 4 + 1) * 64 + lane];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
          for (int v = 0; v < 4; ++v) o[dt][v] += ws * pp[(dt * 4 + v) * 64 + lane];
      }
    }
    m_run = mstar;
  }

  // ---- finish: write, or publish a partial and let the last workgroup merge
  TQ* out = reinterpret_cast<TQ*>(p.out);
  float lrow = l_lane + __shfl_xor(l_lane, 16, 64);
  lrow += __shfl_xor(lrow, 32, 64);
  if (p.nsplit == 1) {
    if (sub == 0 && qrow < W && lrow > 0.f) {
      const float inv = 1.f / lrow;
      TQ* dst = out + (size_t)(row_base + qrow) * p.ld_out + h * D + 4 * (lane >> 4);
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int v = 0; v < 4; ++v) Elt<TQ>::store(dst, dt * 16 + v, o[dt][v] * inv);
    }
    return;
  }
  // publish this split's partial (o unnormalised, row max, row sum); the
  // merge kernel that follows on the stream combines the splits
  float* base = p.partials + (size_t)(b * p.nq + g * GRP) * p.nsplit * PSZ;   // [GRP][nsplit][PSZ]
  if (sub == 0) {
    float* mine = base + (size_t)(hl * p.nsplit + split) * PSZ;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<f32x4*>(mine + (dt * 64 + lane) * 4) = o[dt];
    if (lane < 16) {
      mine[64 * (D / 4) + lane] = m_run;
      mine[64 * (D / 4) + 16 + lane] = lrow;
    }
  }
}

// Split merge: one wave per (head-dim quarter, query head, request), each
// combining its 2 x 16 head dims over every split of the head, MB splits at
// a time in split order, rescaling the running sum whenever the running
// maximum grows (the same order on every run: bit-reproducible).
template <typename TQ, int D>
__global__ __launch_bounds__(64) void attn_merge_kernel(const AttnParams p) {
  constexpr int PSZ = 64 * (D / 4) + 32;                // floats of one split partial
  constexpr int DPW = 2;                                // 16-wide head-dim tiles per wave
  constexpr int NPART = (D / 16) / DPW;
  constexpr int MB = 16;                                // splits per load batch (kMaxSplit / 2)
  static_assert((D / 16) % DPW == 0, "head-dim parts");
  const int part = blockIdx.x % NPART, h = blockIdx.x / NPART, b = blockIdx.y;
  const int lane = threadIdx.x, qrow = lane & 15;
  const int wv = part;                                  // head-dim tiles [wv DPW, (wv + 1) DPW)
  const float* hb = p.partials + (size_t)(b * p.nq + h) * p.nsplit * PSZ;
  float mstar = -INFINITY, L = 0.f;
  f32x4 acc[DPW];
#pragma unroll
  for (int d = 0; d < DPW; ++d) acc[d] = f32x4{0, 0, 0, 0};
  for (int sp0 = 0; sp0 < p.nsplit; sp0 += MB) {
    float mv[MB], lv[MB];
    f32x4 ov[MB][DPW];
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      mv[j] = -INFINITY;
      lv[j] = 0.f;
#pragma unroll
      for (int d = 0; d < DPW; ++d) ov[j][d] = f32x4{0, 0, 0, 0};
      if (sp0 + j >= p.nsplit) continue;                // uniform: nothing to load past the last split
      const int sp = sp0 + j;
      const gptr<float> pt = as_global(hb + (size_t)sp * PSZ);
      mv[j] = pt[64 * (D / 4) + qrow];
      lv[j] = pt[64 * (D / 4) + 16 + qrow];
#pragma unroll
      for (int d = 0; d < DPW; ++d)
        ov[j][d] = *as_global(reinterpret_cast<const f32x4*>(hb + (size_t)sp * PSZ) + (wv * DPW + d) * 64 + lane);
    }
    float bm = mstar;
#pragma unroll
    for (int j = 0; j < MB; ++j)
      if (sp0 + j < p.nsplit) bm = fmaxf(bm, mv[j]);
    if (bm == -INFINITY) continue;
    const float rescale = mstar == -INFINITY ? 0.f : exp2f(mstar - bm);
    L *= rescale;
#pragma unroll
    for (int d = 0; d < DPW; ++d) acc[d] *= rescale;
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      if (sp0 + j >= p.nsplit || mv[j] == -INFINITY) continue;
      const float wgt = exp2f(mv[j] - bm);
      L += wgt * lv[j];
#pragma unroll
      for (int d = 0; d < DPW; ++d) acc[d] += wgt * ov[j][d];
    }
    mstar = bm;
  }
  if (qrow < p.W && L > 0.f) {
    const float inv = 1.f / L;
    TQ* dst = reinterpret_cast<TQ*>(p.out) + (size_t)(b * p.W + qrow) * p.ld_out + h * D + 4 * (lane >> 4);
#pragma unroll
    for (int d = 0; d < DPW; ++d)
#pragma unroll
      for (int v = 0; v < 4; ++v) Elt<TQ>::store(dst, (wv * DPW + d) * 16 + v, acc[d][v] * inv);
  }
}

size_t attn_partial_floats(int max_b, int nq, int head_dim) {
  return (size_t)max_b * nq * kMaxSplit * (64 * (head_dim / 4) + 32);
}

template <typename TW, typename TQ, typename TV, int D, int GRP>
static hipError_t launch_g(const AttnParams& p, hipStream_t s) {
  const dim3 grid(p.nsplit, p.nkv, p.B);
  if constexpr (sizeof(TW) == 2) {
    if (p.kv_nt) {
      DSPINE_LAUNCH((attention_kernel<TW, TQ, TV, D, GRP, true>), grid, dim3(AttnShape<TQ, TV, D, GRP>::NT), 0, s, p);
    } else {
      DSPINE_LAUNCH((attention_kernel<TW, TQ, TV, D, GRP>), grid, dim3(AttnShape<TQ, TV, D, GRP>::NT), 0, s, p);
    }
  } else {
    DSPINE_LAUNCH((attention_kernel<TW, TQ, TV, D, GRP>), grid, dim3(AttnShape<TQ, TV, D, GRP>::NT), 0, s, p);
  }
  if (p.nsplit > 1) DSPINE_LAUNCH((attn_merge_kernel<TQ, D>), dim3(p.nq * (D / 32), p.B), dim3(64), 0, s, p);
  return hipGetLastError();
}

template <typename TW, typename TQ, typename TV, int D>
static hipError_t launch_d(const AttnParams& p, hipStream_t s) {
  switch (p.nq / p.nkv) {
    case 1: return launch_g<TW, TQ, TV, D, 1>(p, s);
    case 2: return launch_g<TW, TQ, TV, D, 2>(p, s);
    case 4: return launch_g<TW, TQ, TV, D, 4>(p, s);
    case 8: return launch_g<TW, TQ, TV, D, 8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention(const AttnParams& p, int dtype, int head_dim, hipStream_t s) {
  if (dtype == DT_BF16) {
    if (head_dim == 128) return launch_d<bf16_t, f16_t, f16_t, 128>(p, s);
    return launch_d<bf16_t, f16_t, f16_t, 64>(p, s);
  }
  if (head_dim == 128) return launch_d<float, float, float, 128>(p, s);
  return launch_d<float, float, float, 64>(p, s);
}

}  // namespace dspine
