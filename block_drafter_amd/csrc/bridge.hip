// Fused bridge (a9-a11) of one layer for blocks of at most 32 rows, in one
// launch.  [FLZ, "The bridge"]; [PHY, 统一转移空间; 门控与写回; 融合 kernel]:
//
//   rho_t = rms(x_t),  z_t = R_l x_t / (rho_t + eps),
//   c_t = sqrt(r) z_t / (||z_t|| + eps)        (anchor rows: c_0 = sqrt(r) C[a]),
//   g_t = sigmoid(G c_t + G_p c_{t-1} + b),   m_t = g_t * (A c_{t-1}),  m_0 = 0,
//   x_t += rho_t W_l m_t.
//
// The three contractions are small (10.5 + 3.1 + 5.2 MB of bf16 weights at
// the 27B geometry) and each depends on the whole result of the one before,
// so as three streamed GEMMs they cost mostly fixed latency: entering, the
// first load round trip, the split-K hand-off.  Here one grid does all three:
//
//   - group 1 (4 r/16 workgroups): 16 rows of R and one quarter of K = H
//     each, wave w taking every fourth 32-wide K step of the quarter (the
//     waves' products are added through LDS in wave order); each quarter
//     publishes its partial, and the last of a block's four to arrive adds
//     them in quarter order, writes z (fp16) and each row's sum of squares
//     over the 16 columns, then counts the block on sync[0];
//   - group 2 (a/16 workgroups): the same 16 rows of G, G_p and A each (K
//     steps split over the waves the same way);
//     waits for sync[0] = r/16, forms the code norm from the sums of
//     squares (c = s z with s = sqrt(r) / (||z|| + eps), 1 at anchor rows:
//     the scale is a per-row factor, so it multiplies the products), writes
//     P = [G; G_p; A] c and the gate * message of its 16 columns (rows t
//     and t-1 are both in the workgroup), then counts itself on sync[1];
//   - group 3 (H/64 workgroups): 64 rows of W_l each (16 per wave, K = a);
//     waits for sync[1] = a/16, adds rho W_l m to its 64 columns of x and
//     writes their per-row sums of squares (the next norm's statistics).
//
// Optionally (next_act / next_out) group 3 also forms the next RMS norm of
// its columns once every group-3 workgroup has published its statistics (a
// fourth wait), so that no separate norm or pre-scale kernel follows; or
// (copy_out) it stores its columns of x times the next norm's gain as fp16
// at once, and the next q|k|v GEMM applies the norm after its product.
//
// Every workgroup loads its weights into registers before it waits, so the
// three groups' HBM reads overlap.  Results that cross workgroups travel by
// write-through agent-scope stores, drained before the count, and are read
// with agent-scope loads.  The grid (4 r/16 + a/16 + H/64 workgroups) must be
// resident at once: the launcher checks it against the CU count, and every
// wait is bounded (a timeout sets sync[3] and the workgroup skips its work,
// so no wave waits forever).  The last group-3 workgroup resets the counters.
// Counter i (sync[i] above) is the word i kBridgeLine: each on a 128-byte line
// of its own, so that the 64 block arrivals, the hand-off counts and the
// waiting workgroups' polls do not queue behind one another (packed into two
// lines, the last block's hand-off ended about 5 us later).
#include "dspine_device.hpp"
#include "dspine_internal.hpp"

namespace dspine {

namespace {

constexpr int kS1 = 4;      // group 1: workgroups (K quarters) per block of 16 codes
constexpr int kF1 = 10;     // group 1: K steps of 32 per wave (H <= 5120)
constexpr int kF2 = 8;      // group 2: K steps per wave (r <= 1024)
constexpr int kF3 = 16;     // group 3: K steps of each wave's 16 rows (a <= 512)
constexpr int kSpin = 1 << 17;
constexpr int kBlk0 = 5;    // first per-block arrival counter in sync

// Thread 0: wait until *c >= target (bounded); false after a timeout, which
// is also recorded in *flag.
__device__ bool wait_count(uint32_t* c, uint32_t target, uint32_t* flag) {
  for (int it = 0; it < kSpin; ++it) {
    if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return true;
    __builtin_amdgcn_s_sleep(4);
  }
  __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

// 8 fp16 values read at agent scope (written by another workgroup of this launch)
__device__ __forceinline__ u32x4 load_coherent_u32x4(const void* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
}

// out[m] = the sum of row m's statistics lists st[t][m], t < lists, for the
// ROWS rows of the block (rows past M repeat row M - 1).  The lists are split
// over Q = 256 / ROWS threads per row, eight loads in flight per thread, and
// the Q partial sums added in order (fixed order; no thread waits for one
// list at a time).  COH: the lists were written by other workgroups of this
// launch (agent-scope loads).  All threads must call it.
template <int ROWS, bool COH>
__device__ __forceinline__ void row_sums(const float* st, int lists, int ld, int M, float* out, float* scratch) {
  constexpr int Q = 256 / ROWS;
  const int tid = threadIdx.x, m = tid % ROWS, q = tid / ROWS;
  const float* col = st + (m < M ? m : M - 1);
  float part = 0.f;
  for (int t0 = q; t0 < lists; t0 += 8 * Q) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + u * Q;
      const float* a = col + (size_t)(t < lists ? t : 0) * ld;
      v[u] = COH ? load_coherent(a) : *a;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (t0 + u * Q < lists) part += v[u];
  }
  scratch[q * ROWS + m] = part;
  __syncthreads();
  if (tid < ROWS) {
    float S = 0.f;
    for (int j = 0; j < Q; ++j) S += scratch[j * ROWS + tid];
    out[tid] = S;
  }
  __syncthreads();
}

// Reduce the four waves' accumulators (red[w] holds wave w's NB x MT
// fragments, 256 floats each) in wave order; wave 0's lanes get the sums.
template <int NB, int MT>
__device__ __forceinline__ void reduce_waves(f32x4 (&acc)[NB][MT], float* red, int wave, int lane) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<f32x4*>(red + ((wave * NB + nb) * MT + mt) * 256 + 4 * lane) = acc[nb][mt];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 s = acc[nb][mt];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          const f32x4 o = *reinterpret_cast<const f32x4*>(red + ((w * NB + nb) * MT + mt) * 256 + 4 * lane);
          s = f32x4{s[0] + o[0], s[1] + o[1], s[2] + o[2], s[3] + o[3]};
        }
        acc[nb][mt] = s;
      }
  }
}

}  // namespace

template <int MT>
__global__ __launch_bounds__(256) void bridge_fused_kernel(const BridgeParams p) {
  __shared__ __align__(16) float red[4 * 3 * MT * 256];
  __shared__ float s_scale[MT * 16];
  __shared__ __align__(16) float s_P[3][MT * 16][16];
  __shared__ float s_sq[4][MT * 16];
  __shared__ float s_nrm[MT * 16];
  // group 3: the message rows, staged once for the four waves (row stride
  // kF3 * 32 + 8 halves: the 16 rows of a fragment read land on distinct banks)
  __shared__ __align__(16) f16_t s_msg[MT * 16 * (kF3 * 32 + 8)];
  __shared__ int s_ok;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int U1 = p.r / 16, U2 = p.a / 16;
  const int g = blockIdx.x;
  const int nl = 4 * (lane >> 4);                     // first output column of this lane's 4
  uint32_t* const sync = p.sync;
  auto ctr = [sync](int i) { return sync + i * kBridgeLine; };   // counter i, on a line of its own

  if (g < kS1 * U1) {
    // ---- group 1: z = R x / (rho + eps) for 16 codes ----------------------
    // block j of 16 codes, K quarter s (steps [s NQ, (s + 1) NQ) of the H/32
    // steps); wave w takes the quarter's steps w, w + 4, ...
    const int j = g / kS1, sp = g % kS1;
    const int NK = p.H / 32, NQ = (NK + kS1 - 1) / kS1;
    const int k_lo = sp * NQ, k_hi = min(NK, k_lo + NQ);
    const gptr<bf16_t> R = as_global(reinterpret_cast<const bf16_t*>(p.R)) + (size_t)j * 16 * p.H + 8 * lane;
    Frag<bf16_t> wf[kF1];
#pragma unroll
    for (int f = 0; f < kF1; ++f)
      if (k_lo + wave + 4 * f < k_hi) wf[f].gload_nt(R + (size_t)(k_lo + wave + 4 * f) * 512);
    // activation rows (fp32 x) of every step, all in flight together
    u32x4 xv[kF1][MT][2];
#pragma unroll
    for (int f = 0; f < kF1; ++f)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + (lane & 15);
        const int ks = k_lo + wave + 4 * f;
        if (ks < k_hi) {
          const gptr<float> src = as_global(p.x + (size_t)(m < p.M ? m : p.M - 1) * p.H + 32 * ks + 8 * (lane >> 4));
          xv[f][mt][0] = gload16((gptr<void>)src);
          xv[f][mt][1] = gload16((gptr<void>)(src + 4));
        }
      }
    row_sums<MT * 16, false>(p.xst, p.xst_lists, p.ld, p.M, s_scale, red);
    if (tid < MT * 16) s_scale[tid] = 1.f / (sqrtf(s_scale[tid] / p.H) + p.eps);
    __syncthreads();
    float sc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sc[mt] = s_scale[mt * 16 + (lane & 15)];
    f32x4 acc[1][MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[0][mt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int f = 0; f < kF1; ++f) {
      if (k_lo + wave + 4 * f < k_hi) {
        const Frag<f16_t> w = AsOperand<f16_t, bf16_t>::cvt(wf[f]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          Frag<f16_t> bq;
          bq.v = u32x4{pack_f16x2(__uint_as_float(xv[f][mt][0][0]) * sc[mt], __uint_as_float(xv[f][mt][0][1]) * sc[mt]),
                       pack_f16x2(__uint_as_float(xv[f][mt][0][2]) * sc[mt], __uint_as_float(xv[f][mt][0][3]) * sc[mt]),
                       pack_f16x2(__uint_as_float(xv[f][mt][1][0]) * sc[mt], __uint_as_float(xv[f][mt][1][1]) * sc[mt]),
                       pack_f16x2(__uint_as_float(xv[f][mt][1][2]) * sc[mt], __uint_as_float(xv[f][mt][1][3]) * sc[mt])};
          mma16(acc[0][mt], w, bq);
        }
      }
    }
    reduce_waves<1, MT>(acc, red, wave, lane);
    if (wave == 0) {
      // the anchor rows' codebook values, loaded before the arrival (only
      // the block's last quarter uses them)
      float cbv[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + (lane & 15);
        if (m % p.W == 0) {
          const gptr<bf16_t> cb = as_global(reinterpret_cast<const bf16_t*>(p.codebook)) +
                                  (size_t)p.anchor[(m < p.M ? m : 0) / p.W] * p.r + 16 * j + nl;
#pragma unroll
          for (int v = 0; v < 4; ++v) cbv[mt][v] = Elt<bf16_t>::gload(cb, v);
        }
      }
      // publish this quarter's partial; the last quarter of the block to
      // arrive adds the four in quarter order and finishes the block
      float* part = p.zpart + (size_t)(j * kS1) * MT * 256;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) store_coherent(part + ((size_t)sp * MT + mt) * 256 + 4 * lane, acc[0][mt]);
      drain_own_stores();
      uint32_t prev = 0;
      if (lane == 0) prev = __hip_atomic_fetch_add(ctr(kBlk0 + j), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      prev = __shfl(prev, 0, 64);
      if (prev != (uint32_t)kS1 - 1) return;
      if (lane == 0) __hip_atomic_store(ctr(kBlk0 + j), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      f32x4 q[kS1][MT];
#pragma unroll
      for (int t = 0; t < kS1; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) q[t][mt] = load_coherent4(part + ((size_t)t * MT + mt) * 256 + 4 * lane);
      const int col = 16 * j + nl;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + (lane & 15);
        f32x4 z = q[0][mt];
#pragma unroll
        for (int t = 1; t < kS1; ++t) z = f32x4{z[0] + q[t][mt][0], z[1] + q[t][mt][1], z[2] + q[t][mt][2], z[3] + q[t][mt][3]};
        if (m % p.W == 0) {                           // anchor code sqrt(r) C[anchor]
#pragma unroll
          for (int v = 0; v < 4; ++v) z[v] = p.code_scale * cbv[mt][v];
        }
        float ss = ((z[0] * z[0] + z[1] * z[1]) + z[2] * z[2]) + z[3] * z[3];
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        if (m < p.M) {
          const uint64_t h = (uint64_t)pack_f16x2(z[0], z[1]) | ((uint64_t)pack_f16x2(z[2], z[3]) << 32);
          __hip_atomic_store(reinterpret_cast<uint64_t*>(reinterpret_cast<f16_t*>(p.z) + (size_t)m * p.r + col), h,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (lane < 16) store_coherent(p.ssz + (size_t)j * p.ld + m, ss);
        }
      }
      drain_own_stores();
      if (lane == 0) __hip_atomic_fetch_add(ctr(0), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }

  if (g < kS1 * U1 + U2) {
    // ---- group 2: P = [G; G_p; A] c, gate * message, for 16 columns --------
    const int i = g - kS1 * U1;
    const int NK = p.r / 32;                          // wave w takes steps w, w + 4, ...
    Frag<bf16_t> wf[3][kF2];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const gptr<bf16_t> Wm = as_global(reinterpret_cast<const bf16_t*>(s == 0 ? p.G : s == 1 ? p.Gp : p.A)) +
                              (size_t)i * 16 * p.r + 8 * lane;
#pragma unroll
      for (int f = 0; f < kF2; ++f)
        if (wave + 4 * f < NK) wf[s][f].gload_nt(Wm + (size_t)(wave + 4 * f) * 512);
    }
    if (tid == 0) s_ok = wait_count(ctr(0), (uint32_t)U1, ctr(3)) ? 1 : 0;
    __syncthreads();
    const bool ok = s_ok != 0;
    if (ok) {
      // z goes out first, the code-norm sums of squares behind it: one
      // memory round trip for both
      u32x4 zv[kF2][MT];
#pragma unroll
      for (int f = 0; f < kF2; ++f)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = mt * 16 + (lane & 15);
          if (wave + 4 * f < NK)
            zv[f][mt] = load_coherent_u32x4(reinterpret_cast<const f16_t*>(p.z) + (size_t)(m < p.M ? m : p.M - 1) * p.r +
                                            32 * (wave + 4 * f) + 8 * (lane >> 4));
        }
      // code-norm scale of each row from the sums of squares of z
      row_sums<MT * 16, true>(p.ssz, U1, p.ld, p.M, s_scale, red);
      if (tid < MT * 16) {
        const int m = tid < p.M ? tid : p.M - 1;
        s_scale[tid] = (m % p.W == 0) ? 1.f : p.code_scale / (sqrtf(s_scale[tid]) + p.eps);
      }
      __syncthreads();
      f32x4 acc[3][MT];
#pragma unroll
      for (int s = 0; s < 3; ++s)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[s][mt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int f = 0; f < kF2; ++f) {
        if (wave + 4 * f >= NK) continue;
#pragma unroll
        for (int s = 0; s < 3; ++s) {
          const Frag<f16_t> w = AsOperand<f16_t, bf16_t>::cvt(wf[s][f]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            Frag<f16_t> b;
            b.v = zv[f][mt];
            mma16(acc[s][mt], w, b);
          }
        }
      }
      reduce_waves<3, MT>(acc, red, wave, lane);
      if (wave == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = mt * 16 + (lane & 15);
          const float sc = s_scale[mt * 16 + (lane & 15)];
#pragma unroll
          for (int s = 0; s < 3; ++s) {
            const f32x4 v = f32x4{acc[s][mt][0] * sc, acc[s][mt][1] * sc, acc[s][mt][2] * sc, acc[s][mt][3] * sc};
            *reinterpret_cast<f32x4*>(&s_P[s][mt * 16 + (lane & 15)][nl]) = v;
            if (m < p.M) *reinterpret_cast<f32x4*>(p.P + (size_t)m * 3 * p.a + s * p.a + 16 * i + nl) = v;
          }
        }
      }
      __syncthreads();
      // gate * message of row t from P of rows t and t - 1 (zero at anchors)
      for (int e = tid; e < MT * 16 * 8; e += 256) {
        const int m = e >> 3, c = 2 * (e & 7);
        if (m >= p.M) continue;
        float o[2] = {0.f, 0.f};
        if (m % p.W != 0) {
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const float b = Elt<bf16_t>::load(reinterpret_cast<const bf16_t*>(p.bias), 16 * i + c + d);
            o[d] = sigmoid(s_P[0][m][c + d] + s_P[1][m - 1][c + d] + b) * s_P[2][m - 1][c + d];
          }
        }
        __hip_atomic_store(reinterpret_cast<uint32_t*>(reinterpret_cast<f16_t*>(p.msg) + (size_t)m * p.a + 16 * i + c),
                           pack_f16x2(o[0], o[1]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      drain_own_stores();
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(ctr(1), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }

  // ---- group 3: x += rho W_l m for 64 columns; their statistics ------------
  const int c3 = g - kS1 * U1 - U2;
  const int F = p.a / 32;
  const gptr<bf16_t> Wl = as_global(reinterpret_cast<const bf16_t*>(p.Wl)) + (size_t)(4 * c3 + wave) * 16 * p.a + 8 * lane;
  Frag<bf16_t> wf[kF3];
#pragma unroll
  for (int f = 0; f < kF3; ++f)
    if (f < F) wf[f].gload_nt(Wl + (size_t)f * 512);
  const int U3 = p.H / 64;
  const bool fold = p.next_act != nullptr || p.next_out != nullptr;
  const int col = 16 * (4 * c3 + wave) + nl;
  // this lane's 4 columns of x (the other groups do not write x) and of the
  // next norm's gain, loaded before the wait
  f32x4 xn[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + (lane & 15);
    xn[mt] = *reinterpret_cast<const f32x4*>(p.x + (size_t)(m < p.M ? m : p.M - 1) * p.H + col);
  }
  float gv[4] = {0.f, 0.f, 0.f, 0.f};
  if (fold || p.copy_out) {
    const gptr<bf16_t> gn = as_global(reinterpret_cast<const bf16_t*>(fold ? p.next_gain : p.copy_gain)) + col;
#pragma unroll
    for (int e = 0; e < 4; ++e) gv[e] = Elt<bf16_t>::gload(gn, e);
  }
  row_sums<MT * 16, false>(p.xst, p.xst_lists, p.ld, p.M, s_scale, red);
  if (tid < MT * 16) s_scale[tid] = sqrtf(s_scale[tid] / p.H);        // rho
  if (tid == 0) s_ok = wait_count(ctr(1), (uint32_t)U2, ctr(3)) ? 1 : 0;
  __syncthreads();
  if (s_ok) {
    // every wave multiplies all of m: the workgroup reads it from memory
    // once (8 values per thread and pass) and the waves take their
    // fragments from LDS
    constexpr int LDM = kF3 * 32 + 8;
    const int cpr = p.a / 8;                          // 8-value chunks per row
    for (int c = tid; c < MT * 16 * cpr; c += 256) {
      const int m = c / cpr, k8 = c % cpr;
      const u32x4 v = load_coherent_u32x4(reinterpret_cast<const f16_t*>(p.msg) + (size_t)(m < p.M ? m : p.M - 1) * p.a +
                                          8 * k8);
      *reinterpret_cast<u32x4*>(&s_msg[m * LDM + 8 * k8]) = v;
    }
    __syncthreads();
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int f = 0; f < kF3; ++f) {
      if (f >= F) continue;
      const Frag<f16_t> w = AsOperand<f16_t, bf16_t>::cvt(wf[f]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        Frag<f16_t> b;
        b.v = *reinterpret_cast<const u32x4*>(&s_msg[(mt * 16 + (lane & 15)) * LDM + 32 * f + 8 * (lane >> 4)]);
        mma16(acc[mt], w, b);
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + (lane & 15);
      float sq = 0.f;
      if (m < p.M) {
        const float rho = s_scale[mt * 16 + (lane & 15)];
        f32x4 v = xn[mt];
        v = f32x4{v[0] + rho * acc[mt][0], v[1] + rho * acc[mt][1], v[2] + rho * acc[mt][2], v[3] + rho * acc[mt][3]};
        *reinterpret_cast<f32x4*>(p.x + (size_t)m * p.H + col) = v;
        xn[mt] = v;
        if (p.copy_out) {                             // the next layer's raw operand
          float c[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) c[e] = v[e] * p.copy_mult * gv[e];
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.copy_out) + (size_t)m * p.H + col) =
              uint2{pack_f16x2(c[0], c[1]), pack_f16x2(c[2], c[3])};
        }
        sq = sumsq4(v[0], v[1], v[2], v[3]);
      }
      sq += __shfl_xor(sq, 16, 64);
      sq += __shfl_xor(sq, 32, 64);
      if (lane < 16) s_sq[wave][mt * 16 + lane] = sq;
    }
    __syncthreads();
    if (tid < p.M) {
      const float st = ((s_sq[0][tid] + s_sq[1][tid]) + s_sq[2][tid]) + s_sq[3][tid];
      if (fold) store_coherent(p.st_out + (size_t)c3 * p.ld + tid, st);   // read by the other workgroups
      else p.st_out[(size_t)c3 * p.ld + tid] = st;
    }
  }
  if (!fold) {
    if (s_ok && tid == 0) {
      // the last group-3 workgroup resets the counters for the next launch
      const uint32_t done = __hip_atomic_fetch_add(ctr(2), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (done == (uint32_t)U3 - 1) {
        __hip_atomic_store(ctr(0), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ctr(1), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ctr(2), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return;
  }

  // ---- fourth phase: the next RMS norm of these 64 columns ------------------
  // Every group-3 workgroup counts itself on sync[2] (also one that timed
  // out above, so that the wait below ends), waits for all of them, sums each
  // row's H/64 statistics lists exactly as the pre-scale kernel does (lane t
  // takes lists t, t + 64, ...; then a wave butterfly), and writes
  // (x * rsqrt(S / H + eps)) * gain.  sync[4] counts the workgroups past the
  // wait; the last one resets the counters.
  drain_own_stores();
  __syncthreads();
  if (tid == 0) {
    __hip_atomic_fetch_add(ctr(2), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_ok = (s_ok && wait_count(ctr(2), (uint32_t)U3, ctr(3))) ? 1 : 0;
  }
  __syncthreads();
  if (s_ok) {
    // rows wave, wave + 4, ...: every row's loads go out before any is summed
    constexpr int RPW = MT * 16 / 4;
    float v[RPW];
    const float* srow[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int rr = wave + 4 * i;
      srow[i] = p.st_out + (rr < p.M ? rr : p.M - 1);
      v[i] = 0.f;
    }
    for (int t = lane; t < U3; t += 64) {
      float l[RPW];
#pragma unroll
      for (int i = 0; i < RPW; ++i) l[i] = load_coherent(srow[i] + (size_t)t * p.ld);
#pragma unroll
      for (int i = 0; i < RPW; ++i) v[i] += l[i];
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const float S = wave_sum(v[i]);
      if (lane == 0) s_nrm[wave + 4 * i] = rsqrtf(S / p.H + p.eps);
    }
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + (lane & 15);
      if (m >= p.M) continue;
      const float sc = s_nrm[m];
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = xn[mt][e] * sc * gv[e];
      if (p.next_out) *reinterpret_cast<f32x4*>(p.next_out + (size_t)m * p.H + col) = f32x4{o[0], o[1], o[2], o[3]};
      if (p.next_act) {
        f16_t* d = reinterpret_cast<f16_t*>(p.next_act) + (size_t)m * p.H + col;
#pragma unroll
        for (int e = 0; e < 4; ++e) Elt<f16_t>::store(d, e, o[e]);
      }
    }
  }
  if (tid == 0) {
    const uint32_t done = __hip_atomic_fetch_add(ctr(4), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (uint32_t)U3 - 1) {
      __hip_atomic_store(ctr(0), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctr(1), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctr(2), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctr(4), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

int bridge_fused_grid(int H, int r, int a) { return kS1 * (r / 16) + a / 16 + H / 64; }

// workgroups of the fused kernel one CU holds at once (occupancy)
static int bridge_per_cu(int M) {
  static int cache[2] = {0, 0};
  int& n = cache[M <= 16 ? 0 : 1];
  if (n == 0) {
    int v = 0;
    const hipError_t e = M <= 16 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, bridge_fused_kernel<1>, 256, 0)
                                 : hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, bridge_fused_kernel<2>, 256, 0);
    n = (e == hipSuccess && v > 0) ? v : 1;
  }
  return n;
}

bool bridge_fused_fits(int H, int r, int a, int M, int num_cus) {
  if (M < 1 || M > 32) return false;
  if (H % 64 || H / 32 > kS1 * 4 * kF1 || r % 32 || r / 32 > 4 * kF2 || a % 32 || a / 32 > kF3 ||
      r / 16 > kBridgeSyncWords / kBridgeLine - kBlk0)
    return false;
  // the whole grid resident at once
  return bridge_fused_grid(H, r, a) <= bridge_per_cu(M) * num_cus;
}

hipError_t launch_bridge_fused(const BridgeParams& p, hipStream_t s) {
  const dim3 grid(bridge_fused_grid(p.H, p.r, p.a));
  if (p.M <= 16) DSPINE_LAUNCH(bridge_fused_kernel<1>, grid, dim3(256), 0, s, p);
  else DSPINE_LAUNCH(bridge_fused_kernel<2>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dspine
