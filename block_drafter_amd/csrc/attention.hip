// Block attention over ring context + block rows (a6), with the q/k head
// RMSNorm and RoPE of the block (a5 tail) fused into the prologue.
//
// [NIF, layer equations]: a = attention(q, concat(K_ctx, k), concat(V_ctx,
// v), scale 1/sqrt(D), layer mask); q, k are head-RMSNormed then rotated.
// [NIF, draft attention]: the mask keeps |p_key - p_query| < S on local
// layers; block keys are all visible (bidirectional) unless block_causal.
//
// Layout on gfx950: one workgroup per (key split, KV head, request), one
// wave per query head of the GQA group, so every K/V tile staged in LDS is
// used by all heads that share it.  A wave holds the block's (<= 16) rows of
// its head and computes S^T = K Q^T with 16x16x32 MFMAs: each lane then owns
// one query row (lane % 16), which makes the online-softmax rescale of the
// O^T = V^T P^T accumulators lane-local.  Splits over context keys are merged
// with their log-sum-exp by the last wave to finish each (request, head).
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

template <typename TW, typename TQ, typename TV, int D, int GRP>
__global__ __launch_bounds__(64 * GRP) void attention_kernel(const AttnParams p) {
  static_assert(sizeof(TW) == sizeof(TQ), "stored keys and key operands have one element size");
  constexpr int EQ = (int)sizeof(TQ);
  constexpr int EV = (int)sizeof(TV);
  constexpr int LDQ = D + 16 / EQ;          // padded row of Q / K tiles
  constexpr int LDV = 32 + 4;               // padded row of V^T tiles (32 keys)
  constexpr int NT = 64 * GRP;
  constexpr int PSZ = 64 * (D / 4) + 32;    // floats per split partial

  __shared__ __attribute__((aligned(16))) TQ sQ[GRP][16 * LDQ];
  __shared__ __attribute__((aligned(16))) TQ sK[2][32 * LDQ];
  __shared__ __attribute__((aligned(16))) TV sVt[2][D * LDV];

  const int b = blockIdx.z, g = blockIdx.y, split = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = g * GRP + w;
  const int W = p.W, S = p.S;
  const int64_t F = p.F[b];
  const int64_t cbeg = p.lo0[b] + (int64_t)split * p.kps[b];
  const int64_t cend = (cbeg + p.kps[b] < F) ? cbeg + p.kps[b] : F;
  const bool has_block = split == p.nsplit - 1;
  const int row_base = b * W;
  const float* rope = p.rope;

  // ---- context keys [cbeg, cend) in tiles of 32 ---------------------------
  // PF tiles are in flight in registers at any time: the slot of tile i is
  // refilled with tile i + PF as soon as tile i is in LDS, so a split's keys
  // cost about one memory latency, not one per tile.  Loads past cend read
  // position cend-1 (in bounds); those keys are masked and their values
  // zeroed when the tile is written to LDS.
  const gptr<TW> kring = as_global(reinterpret_cast<const TW*>(p.kring[b]));
  const gptr<TV> vring = as_global(reinterpret_cast<const TV*>(p.vring[b]));
  const int64_t cap = p.cap[b];
  constexpr int KCH = D * EQ / 16, KEPC = 16 / EQ;     // 16-byte chunks per key row
  constexpr int VCH = D * EV / 16, VEPC = 16 / EV;
  // chunks per thread; with more threads than chunks the spare threads load
  // a duplicate chunk and store nothing
  constexpr int KPT = (32 * KCH + NT - 1) / NT, VPT = (32 * VCH + NT - 1) / NT;
  constexpr int PF = (16 / (KPT + VPT)) < 1 ? 1 : (16 / (KPT + VPT)) > 8 ? 8 : 16 / (KPT + VPT);
  u32x4 kreg[PF][KPT], vreg[PF][VPT];
  const int n_tiles = cend > cbeg ? (int)((cend - cbeg + 31) / 32) : 0;
  auto load_tile = [&](u32x4 (&kr_)[KPT], u32x4 (&vr_)[VPT], int i) {
    const int64_t t0 = cbeg + 32 * (int64_t)i;
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const int c = (tid + q * NT) % (32 * KCH), kr = c / KCH, part = c % KCH;
      const int64_t pos = t0 + kr < cend ? t0 + kr : cend - 1;
      kr_[q] = gload16((gptr<void>)(kring + ((size_t)g * cap + ring_slot(pos, S)) * D + part * KEPC));
    }
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
      const int c = (tid + q * NT) % (32 * VCH), kr = c / VCH, part = c % VCH;
      const int64_t pos = t0 + kr < cend ? t0 + kr : cend - 1;
      vr_[q] = gload16((gptr<void>)(vring + ((size_t)g * cap + ring_slot(pos, S)) * D + part * VEPC));
    }
  };
  auto store_tile = [&](const u32x4 (&kr_)[KPT], const u32x4 (&vr_)[VPT], int i) {
    const int64_t t0 = cbeg + 32 * (int64_t)i;
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
      const int c = tid + q * NT, kr = c / KCH, part = c % KCH;
      if (c < 32 * KCH)
        *reinterpret_cast<u32x4*>(&sK[0][kr * LDQ + part * KEPC]) = key_chunk(kr_[q], (TW*)nullptr, (TQ*)nullptr);
    }
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
      const int c = tid + q * NT, kr = c / VCH, part = c % VCH;
      if (c >= 32 * VCH) continue;
      alignas(16) TV val[VEPC];
      *reinterpret_cast<u32x4*>(val) = t0 + kr < cend ? vr_[q] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < VEPC; ++e) sVt[0][(part * VEPC + e) * LDV + kr] = val[e];
    }
  };
  // first PF tiles in flight during the prologue below (clamped, in bounds)
  if (n_tiles > 0) {
#pragma unroll
    for (int j = 0; j < PF; ++j) load_tile(kreg[j], vreg[j], j < n_tiles ? j : n_tiles - 1);
  }

  // ---- prologue: head RMSNorm + RoPE of this wave's query head ------------
  // Every operand is loaded into registers before the first use, through
  // global-address-space pointers, so the row's loads share one latency.
  auto prep_rows = [&](int col0, const void* gain, TQ* dst) {
    const int r = lane >> 2, part = lane & 3;
    constexpr int NP = D / 8;               // rotation pairs per lane
    const bool live = r < W;
    const gptr<float> src = as_global(p.qkv) + (size_t)(row_base + (live ? r : 0)) * p.ld_qkv + col0;
    const gptr<float> cs = as_global(rope) + (size_t)(row_base + (live ? r : 0)) * D;   // (cos, sin) x D/2
    const gptr<TW> gw = as_global(reinterpret_cast<const TW*>(gain));
    float xa[NP], xb[NP], ga[NP], gb[NP], co[NP], si[NP];
#pragma unroll
    for (int jj = 0; jj < NP; ++jj) {
      const int j = part * NP + jj;
      xa[jj] = src[j];
      xb[jj] = src[j + D / 2];
      ga[jj] = Elt<TW>::gload(gw, j);
      gb[jj] = Elt<TW>::gload(gw, j + D / 2);
      co[jj] = cs[2 * j];
      si[jj] = cs[2 * j + 1];
    }
    float ss = 0.f;
#pragma unroll
    for (int jj = 0; jj < NP; ++jj) ss += xa[jj] * xa[jj] + xb[jj] * xb[jj];
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    const float inv = rsqrtf(ss / D + p.eps);
#pragma unroll
    for (int jj = 0; jj < NP; ++jj) {
      const int j = part * NP + jj;
      const float a = xa[jj] * inv * ga[jj];
      const float c = xb[jj] * inv * gb[jj];
      Elt<TQ>::store(dst, r * LDQ + j, live ? a * co[jj] - c * si[jj] : 0.f);
      Elt<TQ>::store(dst, r * LDQ + j + D / 2, live ? c * co[jj] + a * si[jj] : 0.f);
    }
  };
  prep_rows(h * D, p.gq, sQ[w]);

  if (has_block) {
    const int kcol = p.nq * D + g * D;
    const int vcol = p.nq * D + p.nkv * D + g * D;
    if (w == 0) {
      prep_rows(kcol, p.gk, sK[1]);
      for (int e = lane; e < 16 * D; e += 64) Elt<TQ>::store(sK[1], (16 + e / D) * LDQ + e % D, 0.f);
    }
    if (w == (GRP > 1 ? 1 : 0)) {
      const int r = lane >> 2, part = lane & 3;
      const bool live = r < W;
      const gptr<float> src = as_global(p.qkv) + (size_t)(row_base + (live ? r : 0)) * p.ld_qkv + vcol + part * (D / 4);
      float vv[D / 4];
#pragma unroll
      for (int d = 0; d < D / 4; ++d) vv[d] = src[d];
#pragma unroll
      for (int d = 0; d < D / 4; ++d) put_v(&sVt[1][(part * (D / 4) + d) * LDV + r], live ? vv[d] : 0.f);
      for (int e = lane; e < 16 * D; e += 64) put_v(&sVt[1][(e / 16) * LDV + 16 + (e % 16)], 0.f);
    }
  }
  __syncthreads();

  Frag<TQ> qf[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    qf[c].load(&sQ[w][(lane & 15) * LDQ + c * 32 + 8 * (lane >> 4)]);

  const float scale_log2 = 1.4426950408889634f * rsqrtf((float)D);
  const int qrow = lane & 15;
  const int64_t row_lo = ctx_row_lo(F, S, qrow);
  float m_run = -INFINITY, l_lane = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0, 0, 0, 0};

  auto process = [&](int which, int64_t p0, bool is_block) {
    f32x4 s[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        Frag<TQ> kf;
        kf.load(&sK[which][(kt * 16 + (lane & 15)) * LDQ + c * 32 + 8 * (lane >> 4)]);
        mma16(s[kt], kf, qf[c]);
      }
    float sv[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int kidx = kt * 16 + 4 * (lane >> 4) + v;
        bool vis;
        if (!is_block) {
          const int64_t pos = p0 + kidx;
          vis = qrow < W && pos < cend && pos >= row_lo;
        } else {
          vis = qrow < W && kidx < W && block_key_visible(S, p.causal, qrow, kidx);
        }
        const float x = vis ? s[kt][v] * scale_log2 : -INFINITY;
        sv[kt * 4 + v] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    float pv[8];
    float alpha = 1.f;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = 0.f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = exp2f(sv[e] - m_new);
    }
    Frag<TV> pf;
    pack_p(pf, pv);
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) psum += pv[e];
    l_lane = l_lane * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      o[dt] *= alpha;
      Frag<TV> vf;
      load_vt(vf, &sVt[which][(dt * 16 + (lane & 15)) * LDV], lane >> 4);
      mma16(o[dt], vf, pf);
    }
  };

  // Every trip issues the same loads (refills past the end re-read the last
  // tile), so the wait before each LDS store covers exactly one slot.
  for (int i0 = 0; i0 < n_tiles; i0 += PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int i = i0 + j;
      const bool live = i < n_tiles;
      if (live) store_tile(kreg[j], vreg[j], i);
      __syncthreads();
      load_tile(kreg[j], vreg[j], i + PF < n_tiles ? i + PF : n_tiles - 1);
      if (live) process(0, cbeg + 32 * (int64_t)i, false);
      __syncthreads();
    }
  }
  if (has_block) process(1, 0, true);

  // ---- finish: write, or publish a partial and let the last wave merge ----
  float lrow = l_lane + __shfl_xor(l_lane, 16, 64);
  lrow += __shfl_xor(lrow, 32, 64);
  TQ* out = reinterpret_cast<TQ*>(p.out);
  auto write_row = [&](const f32x4 (&acc)[D / 16], float inv_l) {
    if (qrow >= W) return;
    TQ* dst = out + (size_t)(row_base + qrow) * p.ld_out + h * D + 4 * (lane >> 4);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int v = 0; v < 4; ++v) Elt<TQ>::store(dst, dt * 16 + v, acc[dt][v] * inv_l);
  };
  if (p.nsplit == 1) {
    if (lrow > 0.f) write_row(o, 1.f / lrow);
    return;
  }
  float* base = p.partials + (size_t)((b * p.nq + h) * p.nsplit) * PSZ;
  float* mine = base + (size_t)split * PSZ;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) store_coherent(mine + (dt * 64 + lane) * 4, o[dt]);
  if (lane < 16) {
    store_coherent(mine + 64 * (D / 4) + lane, m_run);
    store_coherent(mine + 64 * (D / 4) + 16 + lane, lrow);
  }
  drain_own_stores();
  uint32_t old = 0;
  if (lane == 0) old = count_arrival(p.counters + b * p.nq + h);
  old = __shfl(old, 0, 64);
  if ((int)old != p.nsplit - 1) return;
  // Merge: the splits' row maxima first (8 loads in flight at a time), then
  // their partial sums four splits at a time, every load issued before use.
  // Indexes past the last split repeat it; those copies are not added.
  float mstar = -INFINITY;
  for (int sp0 = 0; sp0 < p.nsplit; sp0 += 8) {
    float mv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sp = sp0 + j < p.nsplit ? sp0 + j : p.nsplit - 1;
      mv[j] = load_coherent(base + (size_t)sp * PSZ + 64 * (D / 4) + qrow);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) mstar = fmaxf(mstar, mv[j]);
  }
  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0, 0, 0, 0};
  float L = 0.f;
  if (mstar != -INFINITY) {
    constexpr int MB = 256 / D;              // splits merged per batch of loads
    for (int sp0 = 0; sp0 < p.nsplit; sp0 += MB) {
      float mv[MB], lv[MB];
      f32x4 ov[MB][D / 16];
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int sp = sp0 + j < p.nsplit ? sp0 + j : p.nsplit - 1;
        const float* part = base + (size_t)sp * PSZ;
        mv[j] = load_coherent(part + 64 * (D / 4) + qrow);
        lv[j] = load_coherent(part + 64 * (D / 4) + 16 + qrow);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) ov[j][dt] = load_coherent4(part + (dt * 64 + lane) * 4);
      }
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        if (sp0 + j >= p.nsplit || mv[j] == -INFINITY) continue;
        const float wgt = exp2f(mv[j] - mstar);
        L += wgt * lv[j];
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) acc[dt] += wgt * ov[j][dt];
      }
    }
  }
  if (L > 0.f) write_row(acc, 1.f / L);
  if (lane == 0) reset_counter(p.counters + b * p.nq + h);
}

size_t attn_partial_floats(int max_b, int nq, int head_dim) {
  return (size_t)max_b * nq * kMaxSplit * (64 * (head_dim / 4) + 32);
}

template <typename TW, typename TQ, typename TV, int D>
static hipError_t launch_d(const AttnParams& p, hipStream_t s) {
  const int grp = p.nq / p.nkv;
  const dim3 grid(p.nsplit, p.nkv, p.B);
  switch (grp) {
    case 1: hipLaunchKernelGGL((attention_kernel<TW, TQ, TV, D, 1>), grid, dim3(64), 0, s, p); break;
    case 2: hipLaunchKernelGGL((attention_kernel<TW, TQ, TV, D, 2>), grid, dim3(128), 0, s, p); break;
    case 4: hipLaunchKernelGGL((attention_kernel<TW, TQ, TV, D, 4>), grid, dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((attention_kernel<TW, TQ, TV, D, 8>), grid, dim3(512), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
