// Proposal tail after the draft forward: top-K candidates of the shared LM
// head's scores, the candidates' codes and bridge messages for the last-write
// refinement, the refined states' scores (the transition table) and the
// conditional walk.  [FLZ, "The last write is refined using discrete
// candidates"]; [PHY, 前驱条件解码与 transition cache].
//
// The head scores themselves and the two projections of the refinement
// ([G_p; A] of the candidate codes, W_l of the messages) run on the GEMM
// kernels; this file holds the row kernels around them.
#include <climits>

#include "dspine_device.hpp"
#include "dspine_internal.hpp"
#include "propose_internal.hpp"

namespace dspine {

constexpr int kTopkThreads = 256;
constexpr int kScoreThreads = 256;
constexpr int kMaxHidden = 8192;       // refined state kept in LDS

// Ranking of (score, token): a higher score first, equal scores the smaller
// token first.  A NaN score never ranks ahead of anything.
__device__ __forceinline__ bool ranks_before(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// logits row of proposal row r (rows 1..W-1 of every request)
__device__ __forceinline__ int score_row(int r, int W) { return (r / (W - 1)) * W + 1 + r % (W - 1); }

// Rank of pair (v, i) among the n4 pairs (cv, ci) in LDS: how many rank
// before it.  n4 is a multiple of 4 and the arrays are 16-byte aligned (read
// four pairs at a time, several reads in flight); padding pairs (-inf,
// INT_MAX) rank before nothing.
__device__ __forceinline__ int rank_among(float v, int i, const float* cv, const int* ci, int n4) {
  int r = 0;
#pragma unroll 4
  for (int u = 0; u < n4; u += 4) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(cv + u);
    const int4 b = *reinterpret_cast<const int4*>(ci + u);
    r += (ranks_before(a[0], b.x, v, i) ? 1 : 0) + (ranks_before(a[1], b.y, v, i) ? 1 : 0) +
         (ranks_before(a[2], b.z, v, i) ? 1 : 0) + (ranks_before(a[3], b.w, v, i) ? 1 : 0);
  }
  return r;
}

// Partial top-K: block (c, r) ranks slice c (kSliceValues scores, kVpt per
// thread, held in registers) of proposal row r's scores and writes the
// slice's best kMaxTopK pairs in order.  A NaN score ranks as -inf.
//
// Selection by threshold: tau = the kMaxTopK-th best of the 256 per-thread
// best pairs.  Those are kMaxTopK distinct slice pairs ranking at or before
// tau, so every pair of the slice's top kMaxTopK ranks at or before tau too.
// The pairs at or before tau (usually a few dozen) are gathered in LDS and
// placed by counting how many of them rank before each.  A pair qualifies
// only if its thread's best pair does, i.e. only from the kMaxTopK threads
// whose best pairs rank at or before tau, and tau's own thread adds only tau:
// at most (kMaxTopK - 1) * kVpt + 1 pairs.  (With fewer than kMaxTopK
// threads holding a score, tau is (-inf, INT_MAX) and every score of the
// slice qualifies: fewer than kMaxTopK * kVpt.)
constexpr int kVpt = 32;
constexpr int kSliceValues = kVpt * kTopkThreads;
constexpr int kGather = kMaxTopK * kVpt;
static_assert((kMaxTopK - 1) * kVpt + 1 <= kGather, "gather buffer below the bound on qualifying pairs");
__global__ __launch_bounds__(kTopkThreads) void topk_partial_kernel(const ProposeParams p) {
  __shared__ __align__(16) float sv[kGather + 4];    // the gathered pairs (+ padding)
  __shared__ __align__(16) int si[kGather + 4];
  __shared__ __align__(16) float mv[kTopkThreads];
  __shared__ __align__(16) int mi[kTopkThreads];
  __shared__ __align__(16) float wv[kTopkThreads / 64 * kMaxTopK];   // each wave's best maxima
  __shared__ __align__(16) int wi[kTopkThreads / 64 * kMaxTopK];
  __shared__ float tau_v;
  __shared__ int tau_i, count;
  const int c = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int lo = c * kSliceValues, hi = min(p.vocab, lo + kSliceValues);
  const gptr<float> row = as_global(p.scores) + (size_t)score_row(r, p.W) * p.vocab;
  float x[kVpt];
#pragma unroll
  for (int u = 0; u < kVpt; ++u) {
    const int v = lo + tid + u * kTopkThreads;
    const float s = v < hi ? row[v] : -INFINITY;
    x[u] = s == s ? s : -INFINITY;
  }
  // this thread's best pair
  float bv = -INFINITY;
  int bi = INT_MAX;
#pragma unroll
  for (int u = 0; u < kVpt; ++u) {
    const int v = lo + tid + u * kTopkThreads;
    if (v < hi && ranks_before(x[u], v, bv, bi)) {
      bv = x[u];
      bi = v;
    }
  }
  mv[tid] = bv;
  mi[tid] = bi;
  if (tid < kTopkThreads / 64 * kMaxTopK) {
    wv[tid] = -INFINITY;
    wi[tid] = INT_MAX;
  }
  if (tid == 0) {
    count = 0;
    tau_v = -INFINITY;      // kept when fewer than kMaxTopK threads hold a score
    tau_i = INT_MAX;
  }
  __syncthreads();
  // tau in two steps: each wave keeps its kMaxTopK best maxima (the
  // kMaxTopK best of all 256 are among them), then tau is the kMaxTopK-th
  // best of those.  Real pairs have distinct ranks; empty threads' pairs
  // (-inf, INT_MAX) all rank after them and write identical values.
  const int wave = tid >> 6;
  const int rw = rank_among(bv, bi, mv + 64 * wave, mi + 64 * wave, 64);
  if (rw < kMaxTopK) {
    wv[wave * kMaxTopK + rw] = bv;
    wi[wave * kMaxTopK + rw] = bi;
  }
  __syncthreads();
  if (tid < kTopkThreads / 64 * kMaxTopK && wi[tid] != INT_MAX &&
      rank_among(wv[tid], wi[tid], wv, wi, kTopkThreads / 64 * kMaxTopK) == kMaxTopK - 1) {
    tau_v = wv[tid];
    tau_i = wi[tid];
  }
  __syncthreads();
  const float tv = tau_v;
  const int ti = tau_i;
#pragma unroll
  for (int u = 0; u < kVpt; ++u) {
    const int v = lo + tid + u * kTopkThreads;
    if (v < hi && !ranks_before(tv, ti, x[u], v)) {   // at or before tau
      const int slot = atomicAdd(&count, 1);
      if (slot < kGather) {                             // always (bound above)
        sv[slot] = x[u];
        si[slot] = v;
      }
    }
  }
  __syncthreads();
  const int n = count;                                // <= kGather (see above)
  const int n4 = (n + 3) & ~3;
  const size_t out0 = ((size_t)r * gridDim.x + c) * kMaxTopK;
  if (tid < kMaxTopK) {
    p.part_v[out0 + tid] = -INFINITY;                  // slots no pair fills
    p.part_i[out0 + tid] = INT_MAX;
  }
  if (tid < n4 - n) {
    sv[n + tid] = -INFINITY;
    si[n + tid] = INT_MAX;
  }
  __syncthreads();
  for (int e = tid; e < n; e += kTopkThreads) {
    const int rk = rank_among(sv[e], si[e], sv, si, n4);
    if (rk < kMaxTopK) {
      p.part_v[out0 + rk] = sv[e];
      p.part_i[out0 + rk] = si[e];
    }
  }
}

// Final top-K of proposal row r from its partial lists (one sorted list of
// kMaxTopK pairs per slice, at most kMaxSlices).  Same selection as above
// with the lists' heads as the groups: tau = the kMaxTopK-th best head; only
// lists whose head ranks at or before tau contribute, tau's list only its
// head, so at most (kMaxTopK - 1) * kMaxTopK + 1 pairs are gathered and
// ranked.  Slots that no ranked pair fills (fewer than K finite scores) get
// token -1.
constexpr int kMaxSlices = 32;
__global__ __launch_bounds__(kTopkThreads) void topk_merge_kernel(const ProposeParams p, int slices) {
  __shared__ __align__(16) float sv[kMaxSlices * kMaxTopK];
  __shared__ __align__(16) int si[kMaxSlices * kMaxTopK];
  __shared__ __align__(16) float gv[kMaxTopK * kMaxTopK + 4];
  __shared__ __align__(16) int gi[kMaxTopK * kMaxTopK + 4];
  __shared__ __align__(16) float hv[kMaxSlices];
  __shared__ __align__(16) int hi_[kMaxSlices];
  __shared__ float tau_v;
  __shared__ int tau_i, count;
  const int r = blockIdx.x, n = slices * kMaxTopK, tid = threadIdx.x;
  for (int e = tid; e < n; e += kTopkThreads) {
    sv[e] = p.part_v[(size_t)r * n + e];
    si[e] = p.part_i[(size_t)r * n + e];
  }
  if (tid < kMaxSlices) {                 // heads (padding lists rank last)
    hv[tid] = tid < slices ? p.part_v[(size_t)r * n + tid * kMaxTopK] : -INFINITY;
    hi_[tid] = tid < slices ? p.part_i[(size_t)r * n + tid * kMaxTopK] : INT_MAX;
  }
  if (tid < p.K) {
    p.cand[r * p.K + tid] = -1;
    p.cand_scores[r * p.K + tid] = -INFINITY;
  }
  if (tid == 0) {
    count = 0;
    tau_v = -INFINITY;                    // kept with fewer than kMaxTopK real heads
    tau_i = INT_MAX;
  }
  __syncthreads();
  if (tid < slices && hi_[tid] != INT_MAX && rank_among(hv[tid], hi_[tid], hv, hi_, kMaxSlices) == kMaxTopK - 1) {
    tau_v = hv[tid];
    tau_i = hi_[tid];
  }
  __syncthreads();
  const float tv = tau_v;
  const int ti = tau_i;
  for (int e = tid; e < n; e += kTopkThreads) {
    if (si[e] != INT_MAX && !ranks_before(tv, ti, sv[e], si[e])) {   // at or before tau
      const int slot = atomicAdd(&count, 1);
      if (slot < kMaxTopK * kMaxTopK) {                              // always (bound above)
        gv[slot] = sv[e];
        gi[slot] = si[e];
      }
    }
  }
  __syncthreads();
  const int m = count, m4 = (m + 3) & ~3;
  if (tid < m4 - m) {
    gv[m + tid] = -INFINITY;
    gi[m + tid] = INT_MAX;
  }
  __syncthreads();
  for (int e = tid; e < m; e += kTopkThreads) {
    const int rk = rank_among(gv[e], gi[e], gv, gi, m4);
    if (rk < p.K) {
      p.cand[r * p.K + rk] = gi[e];
      p.cand_scores[r * p.K + rk] = gv[e];
    }
  }
}

// candidate row (b, t, i), t = 1..W-1, i = 0..K-1, of the refinement
struct CandRow {
  int b, t, i;
};
__device__ __forceinline__ CandRow cand_row(int row, int W, int K) {
  CandRow c;
  c.b = row / ((W - 1) * K);
  const int rem = row % ((W - 1) * K);
  c.t = 1 + rem / K;
  c.i = rem % K;
  return c;
}
__device__ __forceinline__ int clamp_token(int v, int vocab) { return v < 0 ? 0 : (v >= vocab ? vocab - 1 : v); }

// Predecessor code of candidate row (b, t, i): sqrt(r) C[s], s the anchor for
// t = 1, else candidate i of row t-1.  Written as the GEMM operand type.
template <typename TW, typename TA>
__global__ __launch_bounds__(128) void cand_code_kernel(const ProposeParams p) {
  const CandRow c = cand_row(blockIdx.x, p.W, p.K);
  const int s = c.t == 1 ? p.anchor[c.b] : p.cand[(c.b * (p.W - 1) + c.t - 2) * p.K + c.i];
  const gptr<TW> src = as_global(reinterpret_cast<const TW*>(p.codebook)) + (size_t)clamp_token(s, p.vocab) * p.r;
  TA* dst = reinterpret_cast<TA*>(p.codes) + (size_t)blockIdx.x * p.r;
  for (int k = threadIdx.x; k < p.r; k += blockDim.x) Elt<TA>::store(dst, k, p.code_scale * Elt<TW>::gload(src, k));
}

// Message of candidate row (b, t, i): sigmoid(G c_t + G_p s + b) * (A s), with
// G c_t the receiver's own projection from the forward's last bridge and
// [G_p s, A s] the candidate code's projections.
template <typename TW, typename TA>
__global__ __launch_bounds__(128) void cand_msg_kernel(const ProposeParams p) {
  const CandRow c = cand_row(blockIdx.x, p.W, p.K);
  const float* own = p.P_own + (size_t)(c.b * p.W + c.t) * 3 * p.a;
  const float* pc = p.P_cand + (size_t)blockIdx.x * 2 * p.a;
  const TW* bias = reinterpret_cast<const TW*>(p.bias);
  TA* dst = reinterpret_cast<TA*>(p.msg) + (size_t)blockIdx.x * p.a;
  for (int k = threadIdx.x; k < p.a; k += blockDim.x) {
    const float gate = sigmoid(own[k] + pc[k] + Elt<TW>::load(bias, k));
    Elt<TA>::store(dst, k, gate * pc[p.a + k]);
  }
}

// the 8 elements of a lane fragment as floats
__device__ __forceinline__ void frag_to_float(const Frag<bf16_t>& f, float* w) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    w[2 * d] = __uint_as_float(f.v[d] << 16);
    w[2 * d + 1] = __uint_as_float(f.v[d] & 0xffff0000u);
  }
}
__device__ __forceinline__ void frag_to_float(const Frag<float>& f, float* w) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    w[d] = __uint_as_float(f.v[0][d]);
    w[4 + d] = __uint_as_float(f.v[1][d]);
  }
}

// Row (b, t, i) of the transition table: x' = u_t + rho_t Y, h = g_final x' /
// rms(x'), T[b, t-1, i, j] = E[cand_j] . h for the K candidates j of row t.
// Head rows are read from the row-major head (each row one contiguous read;
// in the fragment-ordered copy a row's pieces share cache lines with seven
// other rows).
template <typename TW>
__global__ __launch_bounds__(kScoreThreads) void cand_score_kernel(const ProposeParams p) {
  __shared__ float h[kMaxHidden];
  __shared__ float red[kScoreThreads / 64];
  __shared__ float dots[kScoreThreads / 64][kMaxTopK];
  const CandRow c = cand_row(blockIdx.x, p.W, p.K);
  const int H = p.H;
  const float* u = p.u + (size_t)(c.b * p.W + c.t) * H;
  const float* y = p.Y + (size_t)blockIdx.x * H;
  // u, Y and the gain in one batch of loads (H <= kMaxHidden: 32 per thread),
  // then x' = u + rho Y and h = g_final x' / rms(x') from registers
  constexpr int kBatch = kMaxHidden / kScoreThreads;
  const TW* gain = reinterpret_cast<const TW*>(p.g_final);
  float uu[kBatch], yy[kBatch], gg[kBatch];
#pragma unroll
  for (int q = 0; q < kBatch; ++q) {
    const int k = threadIdx.x + q * kScoreThreads;
    uu[q] = k < H ? u[k] : 0.f;
    yy[q] = k < H ? y[k] : 0.f;
    gg[q] = k < H ? Elt<TW>::load(gain, k) : 0.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < kBatch; ++q) ss += uu[q] * uu[q];
  const float rho = sqrtf(block_sum<kScoreThreads>(ss, red) / H);
  float sx = 0.f;
#pragma unroll
  for (int q = 0; q < kBatch; ++q) {
    uu[q] += rho * yy[q];                // x'
    sx += uu[q] * uu[q];
  }
  const float inv = rsqrtf(block_sum<kScoreThreads>(sx, red) / H + p.eps);
#pragma unroll
  for (int q = 0; q < kBatch; ++q) {
    const int k = threadIdx.x + q * kScoreThreads;
    if (k < H) h[k] = uu[q] * inv * gg[q];
  }
  __syncthreads();

  const int* cj = p.cand + (size_t)(c.b * (p.W - 1) + c.t - 1) * p.K;
  const TW* E = reinterpret_cast<const TW*>(p.head);
  size_t rowbase[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) rowbase[j] = (size_t)clamp_token(j < p.K ? cj[j] : cj[0], p.vocab) * H;
  float acc[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) acc[j] = 0.f;
  const int nchunk = H / 8;              // 8 consecutive columns of one lane fragment
  for (int ch = threadIdx.x; ch < nchunk; ch += kScoreThreads) {
    const size_t off = (size_t)8 * ch;
    Frag<TW> f[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) f[j].gload(as_global(E + rowbase[j] + off));
    float hk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) hk[e] = h[8 * ch + e];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      float w[8];
      frag_to_float(f[j], w);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += w[e] * hk[e];
      acc[j] += s;
    }
  }
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    const float s = wave_sum(acc[j]);
    if ((threadIdx.x & 63) == 0) dots[w][j] = s;
  }
  __syncthreads();
  if (threadIdx.x < p.K) {
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < kScoreThreads / 64; ++ww) s += dots[ww][threadIdx.x];
    p.table[(size_t)blockIdx.x * p.K + threadIdx.x] = s;
  }
}

// The walk of request b: one wave; the request's tables go to LDS in one
// pass, then the rows are taken in order.  Row 1 uses table row 0 (the
// anchor), row t the row chosen at t-1.  Lane j holds candidate j's score.
// Greedy: the first maximum.  Sampled: float64 p = softmax(T / temperature);
// the normaliser and the cumulative sum are taken left to right (every lane
// forms the same sums), and the choice is the first j whose cumulative
// probability exceeds the uniform (the last j if none does).
__global__ __launch_bounds__(64) void walk_kernel(const ProposeParams p) {
  __shared__ float tab[(DSPINE_MAX_WIDTH - 1) * kMaxTopK * kMaxTopK];
  __shared__ int cand[(DSPINE_MAX_WIDTH - 1) * kMaxTopK];
  __shared__ double uni[DSPINE_MAX_WIDTH - 1];
  const int b = blockIdx.x, n = p.W - 1, K = p.K, lane = threadIdx.x;
  // the request's candidates and uniforms come in with the tables, so the
  // serial walk below touches only LDS
#pragma unroll
  for (int q = 0; q < ((DSPINE_MAX_WIDTH - 1) * kMaxTopK + 63) / 64; ++q) {
    const int e = lane + 64 * q;
    if (e < n * K) cand[e] = p.cand[(size_t)b * n * K + e];
  }
  if (p.walk != DSPINE_WALK_GREEDY && lane < n) uni[lane] = p.uniforms[b * n + lane];
  const gptr<float> src = as_global(p.table) + (size_t)b * n * K * K;
  constexpr int kBatch = ((DSPINE_MAX_WIDTH - 1) * kMaxTopK * kMaxTopK + 63) / 64;   // the largest table in one batch
  for (int e0 = lane; e0 < n * K * K; e0 += 64 * kBatch) {
    float x[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) x[u] = e0 + 64 * u < n * K * K ? src[e0 + 64 * u] : 0.f;
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (e0 + 64 * u < n * K * K) tab[e0 + 64 * u] = x[u];
  }
  __syncthreads();
  const bool on = lane < K;
  int i = 0;
  for (int t = 0; t < n; ++t) {
    const float v = on ? tab[(t * K + i) * K + lane] : -INFINITY;
    int j = 0;
    double q = 1.0;
    if (p.walk == DSPINE_WALK_GREEDY) {
      // first maximum: larger score, then smaller index
      float bv = v;
      int bj = on ? lane : INT_MAX;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oj = __shfl_xor(bj, o, 64);
        if (ov > bv || (ov == bv && oj < bj)) {
          bv = ov;
          bj = oj;
        }
      }
      j = bj;
    } else {
      const double sv = (double)v / p.temperature;
      double mx = sv;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
      const double e = on ? exp(sv - mx) : 0.0;
      double total = 0.0;
      for (int jj = 0; jj < K; ++jj) total += __shfl(e, jj, 64);
      const double pj = e / total;
      const double u = uni[t];
      double cdf = 0.0;
      j = K - 1;
      for (int jj = 0; jj < K; ++jj) {
        cdf += __shfl(pj, jj, 64);
        if (u < cdf) {
          j = jj;
          break;
        }
      }
      q = __shfl(pj, j, 64);
    }
    if (lane == 0) {
      p.choice[b * n + t] = j;
      p.tokens[b * n + t] = cand[t * K + j];
      if (p.q) p.q[b * n + t] = q;
    }
    i = j;
  }
}

// ---------------------------------------------------------------------------
// FP8 row-scaled retrieval [FLZ, "The last write is refined using discrete
// candidates": the optimized path scores the vocabulary approximately with a
// row-scaled FP8 head, keeps 128 candidates, rescores them with the BF16 head
// and retains 16]
// ---------------------------------------------------------------------------
// E4M3 code of x (finite, |x| <= 448), round to nearest, ties to even.  At or
// above 2^-6 the float's exponent and top 3 fraction bits are the code's
// (rebiased from 127 to 7) after rounding away the 20 lower bits; below it
// the code is the number of 2^-9 steps.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (a >= 0.015625f) {
    const uint32_t b = __float_as_uint(a);
    code = ((b + 0x7ffffu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
  } else {
    code = (uint32_t)rintf(a * 512.0f);
  }
  return sign | code;
}

// One workgroup per block of 16 head rows: each row's absolute maximum m
// (16 threads per row), its scale exponent k (2^k the smallest power of two
// >= m / 448; 0 for a zero row), then the codes of E / 2^k in fragment order
// with two 32-column steps per lane: for 64-column step kp, lane l holds row
// l % 16, columns 64 kp + 8 (l / 16) .. + 8 and then 64 kp + 32 + 8 (l / 16)
// .. + 8, 16 bytes at byte (blk K/64 + kp) 1024 + 16 l.
__global__ __launch_bounds__(256) void quant_head_fp8_kernel(const bf16_t* head, uint8_t* codes, float* col_scale,
                                                             int H) {
  __shared__ int s_k[16];
  const int blk = blockIdx.x, tid = threadIdx.x;
  const int r = tid >> 4, j = tid & 15;
  const gptr<bf16_t> row = as_global(head) + (size_t)(16 * blk + r) * H;
  float m = 0.f;
  for (int c = j; c < H / 8; c += 16) {
    const u32x4 v = gload16((gptr<void>)(row + 8 * c));
#pragma unroll
    for (int d = 0; d < 4; ++d)
      m = fmaxf(m, fmaxf(fabsf(__uint_as_float(v[d] << 16)), fabsf(__uint_as_float(v[d] & 0xffff0000u))));
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (j == 0) {
    int k = 0;
    if (m > 0.f) {
      int ex = 0;
      const float mant = frexpf(m / 448.0f, &ex);      // m / 448 = mant 2^ex, mant in [0.5, 1)
      k = mant == 0.5f ? ex - 1 : ex;
    }
    s_k[r] = k;
    col_scale[16 * blk + r] = ldexpf(1.0f, k + 8);
  }
  __syncthreads();
  const int steps = H / 32;
  for (int f = tid; f < steps * 64; f += 256) {
    const int ks = f >> 6, lane = f & 63;
    const int rr = lane & 15;
    const int k = s_k[rr];
    const u32x4 v = gload16((gptr<void>)(as_global(head) + (size_t)(16 * blk + rr) * H + 32 * ks + 8 * (lane >> 4)));
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t lo = e4m3_code(ldexpf(__uint_as_float(v[d] << 16), -k));
      const uint32_t hi = e4m3_code(ldexpf(__uint_as_float(v[d] & 0xffff0000u), -k));
      w[d >> 1] |= (lo | (hi << 8)) << (16 * (d & 1));
    }
    *reinterpret_cast<uint64_t*>(codes + ((size_t)blk * (steps / 2) + ks / 2) * 1024 + 16 * lane + 8 * (ks & 1)) =
        (uint64_t)w[0] | ((uint64_t)w[1] << 32);
  }
}

// Partial top-R of the FP8 scores: block (c, r) keeps the R best pairs of
// slice c of proposal row r, in order.  Same threshold selection as
// topk_partial_kernel with kMaxRetrieve for kMaxTopK and tau taken in one
// step (the kMaxRetrieve-th best of the 256 per-thread best pairs): at most
// (kMaxRetrieve - 1) * kVpt + 1 pairs are gathered.
constexpr int kRGather = kMaxRetrieve * kVpt;
static_assert((kMaxRetrieve - 1) * kVpt + 1 <= kRGather, "gather buffer below the bound on qualifying pairs");
__global__ __launch_bounds__(kTopkThreads) void retrieve_partial_kernel(const ProposeParams p) {
  __shared__ __align__(16) float sv[kRGather + 4];
  __shared__ __align__(16) int si[kRGather + 4];
  __shared__ __align__(16) float mv[kTopkThreads];
  __shared__ __align__(16) int mi[kTopkThreads];
  __shared__ float tau_v;
  __shared__ int tau_i, count;
  const int c = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int lo = c * kSliceValues, hi = min(p.vocab, lo + kSliceValues);
  const gptr<float> row = as_global(p.scores) + (size_t)score_row(r, p.W) * p.vocab;
  float x[kVpt];
#pragma unroll
  for (int u = 0; u < kVpt; ++u) {
    const int v = lo + tid + u * kTopkThreads;
    const float sc = v < hi ? row[v] : -INFINITY;
    x[u] = sc == sc ? sc : -INFINITY;
  }
  float bv = -INFINITY;
  int bi = INT_MAX;
#pragma unroll
  for (int u = 0; u < kVpt; ++u) {
    const int v = lo + tid + u * kTopkThreads;
    if (v < hi && ranks_before(x[u], v, bv, bi)) {
      bv = x[u];
      bi = v;
    }
  }
  mv[tid] = bv;
  mi[tid] = bi;
  if (tid == 0) {
    count = 0;
    tau_v = -INFINITY;        // kept when fewer than kMaxRetrieve threads hold a score
    tau_i = INT_MAX;
  }
  __syncthreads();
  if (bi != INT_MAX && rank_among(bv, bi, mv, mi, kTopkThreads) == kMaxRetrieve - 1) {
    tau_v = bv;
    tau_i = bi;
  }
  __syncthreads();
  const float tv = tau_v;
  const int ti = tau_i;
#pragma unroll
  for (int u = 0; u < kVpt; ++u) {
    const int v = lo + tid + u * kTopkThreads;
    if (v < hi && !ranks_before(tv, ti, x[u], v)) {
      const int slot = atomicAdd(&count, 1);
      if (slot < kRGather) {                            // always (bound above)
        sv[slot] = x[u];
        si[slot] = v;
      }
    }
  }
  __syncthreads();
  const int n = count;
  const int n4 = (n + 3) & ~3;
  const size_t out0 = ((size_t)r * gridDim.x + c) * kMaxRetrieve;
  if (tid < kMaxRetrieve) {
    p.part_v[out0 + tid] = -INFINITY;
    p.part_i[out0 + tid] = INT_MAX;
  }
  if (tid < n4 - n) {
    sv[n + tid] = -INFINITY;
    si[n + tid] = INT_MAX;
  }
  __syncthreads();
  for (int e = tid; e < n; e += kTopkThreads) {
    const int rk = rank_among(sv[e], si[e], sv, si, n4);
    if (rk < kMaxRetrieve) {
      p.part_v[out0 + rk] = sv[e];
      p.part_i[out0 + rk] = si[e];
    }
  }
}

// Final top-R of proposal row r from its slice lists (sorted, kMaxRetrieve
// each).  tau = the kMaxRetrieve-th best of the lists' first J = ceil(R /
// slices) pairs: those are distinct pairs of the row, so the row's R best all
// rank at or before tau; every pair at or before tau is gathered and placed by
// counting.  (With fewer than kMaxRetrieve real pairs among them, tau is
// (-inf, INT_MAX) and every pair qualifies.)  Ids beyond the real pairs are -1.
__global__ __launch_bounds__(kTopkThreads) void retrieve_merge_kernel(const ProposeParams p, int slices) {
  __shared__ __align__(16) float sv[kMaxSlices * kMaxRetrieve];
  __shared__ __align__(16) int si[kMaxSlices * kMaxRetrieve];
  __shared__ __align__(16) float gv[kMaxSlices * kMaxRetrieve + 4];
  __shared__ __align__(16) int gi[kMaxSlices * kMaxRetrieve + 4];
  __shared__ float tau_v;
  __shared__ int tau_i, count;
  const int r = blockIdx.x, n = slices * kMaxRetrieve, tid = threadIdx.x;
  for (int e = tid; e < n; e += kTopkThreads) {
    sv[e] = p.part_v[(size_t)r * n + e];
    si[e] = p.part_i[(size_t)r * n + e];
  }
  if (tid == 0) {
    tau_v = -INFINITY;
    tau_i = INT_MAX;
    count = 0;
  }
  __syncthreads();
  // the subset: the first J pairs of every list, compacted into gv/gi
  const int J = (kMaxRetrieve + slices - 1) / slices;
  const int ns = J * slices, ns4 = (ns + 3) & ~3;
  for (int e = tid; e < ns4; e += kTopkThreads) {
    const bool in = e < ns;
    gv[e] = in ? sv[(e / J) * kMaxRetrieve + e % J] : -INFINITY;
    gi[e] = in ? si[(e / J) * kMaxRetrieve + e % J] : INT_MAX;
  }
  __syncthreads();
  for (int e = tid; e < ns; e += kTopkThreads)
    if (gi[e] != INT_MAX && rank_among(gv[e], gi[e], gv, gi, ns4) == kMaxRetrieve - 1) {
      tau_v = gv[e];
      tau_i = gi[e];
    }
  __syncthreads();
  const float tv = tau_v;
  const int ti = tau_i;
  for (int e = tid; e < n; e += kTopkThreads) {
    if (si[e] != INT_MAX && !ranks_before(tv, ti, sv[e], si[e])) {
      const int slot = atomicAdd(&count, 1);
      gv[slot] = sv[e];                        // slot < n: at most every pair
      gi[slot] = si[e];
    }
  }
  __syncthreads();
  const int m = count, m4 = (m + 3) & ~3;
  if (tid < m4 - m) {
    gv[m + tid] = -INFINITY;
    gi[m + tid] = INT_MAX;
  }
  if (tid < p.R) p.retrieved[(size_t)r * p.R + tid] = -1;
  __syncthreads();
  for (int e = tid; e < m; e += kTopkThreads) {
    const int rk = rank_among(gv[e], gi[e], gv, gi, m4);
    if (rk < p.R) p.retrieved[(size_t)r * p.R + rk] = gi[e];
  }
}

// BF16 rescoring: grid (R / 16, rows); wave w scores candidates 16 x + 4 w ..
// + 3 of proposal row r: E_v . h with h the forward's final-normed row (in
// LDS), each lane's 8-column pieces summed in order, then a wave sum.
// Empty retrieval slots (-1) score -inf.
__global__ __launch_bounds__(256) void rescore_kernel(const ProposeParams p) {
  __shared__ __align__(16) float h[kMaxHidden];
  const int r = blockIdx.y, H = p.H;
  const float* hr = p.h + (size_t)score_row(r, p.W) * H;
  for (int k = threadIdx.x; k < H; k += 256) h[k] = hr[k];
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i0 = blockIdx.x * 16 + 4 * w;
  int id[4];
  gptr<bf16_t> e[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = i0 + j;
    id[j] = i < p.R ? p.retrieved[(size_t)r * p.R + i] : -1;
    e[j] = as_global(reinterpret_cast<const bf16_t*>(p.head)) + (size_t)clamp_token(id[j], p.vocab) * H;
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int ch = lane; ch < H / 8; ch += 64) {
    u32x4 f[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = gload16((gptr<void>)(e[j] + 8 * ch));
    const f32x4 h0 = *reinterpret_cast<const f32x4*>(&h[8 * ch]);
    const f32x4 h1 = *reinterpret_cast<const f32x4*>(&h[8 * ch + 4]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float hl = d < 2 ? h0[2 * d] : h1[2 * d - 4];
        const float hh = d < 2 ? h0[2 * d + 1] : h1[2 * d - 3];
        s += __uint_as_float(f[j][d] << 16) * hl;
        s += __uint_as_float(f[j][d] & 0xffff0000u) * hh;
      }
      acc[j] += s;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float sc = wave_sum(acc[j]);
    const int i = i0 + j;
    if (lane == 0 && i < p.R) p.rescored[(size_t)r * p.R + i] = id[j] < 0 ? -INFINITY : sc;
  }
}

// The K best rescored candidates of proposal row r, best first (equal scores:
// the smaller token first; NaN ranks last); slots no candidate fills get -1.
__global__ __launch_bounds__(kMaxRetrieve) void retrieve_keep_kernel(const ProposeParams p) {
  __shared__ __align__(16) float v[kMaxRetrieve];
  __shared__ __align__(16) int id[kMaxRetrieve];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int t = tid < p.R ? p.retrieved[(size_t)r * p.R + tid] : -1;
  const float x = tid < p.R ? p.rescored[(size_t)r * p.R + tid] : -INFINITY;
  v[tid] = (t < 0 || x != x) ? -INFINITY : x;
  id[tid] = t < 0 ? INT_MAX : t;
  if (tid < p.K) {
    p.cand[(size_t)r * p.K + tid] = -1;
    p.cand_scores[(size_t)r * p.K + tid] = -INFINITY;
  }
  __syncthreads();
  if (id[tid] != INT_MAX) {
    const int rk = rank_among(v[tid], id[tid], v, id, kMaxRetrieve);
    if (rk < p.K) {
      p.cand[(size_t)r * p.K + rk] = id[tid];
      p.cand_scores[(size_t)r * p.K + rk] = v[tid];
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_quant_head_fp8(const void* head, void* codes, float* col_scale, int V, int H, hipStream_t s) {
  if (V % 16 || H % 64) return hipErrorInvalidValue;
  DSPINE_LAUNCH(quant_head_fp8_kernel, dim3(V / 16), dim3(256), 0, s, static_cast<const bf16_t*>(head),
                static_cast<uint8_t*>(codes), col_scale, H);
  return hipGetLastError();
}
size_t retrieve_partial_entries(int rows, int vocab) {
  return (size_t)rows * ((vocab + kSliceValues - 1) / kSliceValues) * kMaxRetrieve;
}
hipError_t launch_retrieve(const ProposeParams& p, hipStream_t s) {
  const int rows = p.B * (p.W - 1), slices = (p.vocab + kSliceValues - 1) / kSliceValues;
  if (slices > kMaxSlices || p.R < p.K || p.R > kMaxRetrieve || p.H > kMaxHidden || p.H % 8)
    return hipErrorInvalidValue;
  DSPINE_LAUNCH(retrieve_partial_kernel, dim3(slices, rows), dim3(kTopkThreads), 0, s, p);
  DSPINE_LAUNCH(retrieve_merge_kernel, dim3(rows), dim3(kTopkThreads), 0, s, p, slices);
  DSPINE_LAUNCH(rescore_kernel, dim3((p.R + 15) / 16, rows), dim3(256), 0, s, p);
  DSPINE_LAUNCH(retrieve_keep_kernel, dim3(rows), dim3(kMaxRetrieve), 0, s, p);
  return hipGetLastError();
}
int topk_slices(int vocab) { return (vocab + kSliceValues - 1) / kSliceValues; }
hipError_t launch_topk(const ProposeParams& p, hipStream_t s) {
  const int rows = p.B * (p.W - 1), slices = topk_slices(p.vocab);
  if (slices > kMaxSlices) return hipErrorInvalidValue;
  DSPINE_LAUNCH(topk_partial_kernel, dim3(slices, rows), dim3(kTopkThreads), 0, s, p);
  DSPINE_LAUNCH(topk_merge_kernel, dim3(rows), dim3(kTopkThreads), 0, s, p, slices);
  return hipGetLastError();
}
size_t topk_partial_entries(int rows, int vocab) { return (size_t)rows * topk_slices(vocab) * kMaxTopK; }
int topk_max_vocab() { return kMaxSlices * kSliceValues; }
int propose_max_hidden() { return kMaxHidden; }

hipError_t launch_cand_codes(const ProposeParams& p, int dtype, hipStream_t s) {
  const int rows = p.B * (p.W - 1) * p.K;
  if (dtype == DT_BF16) DSPINE_LAUNCH((cand_code_kernel<bf16_t, f16_t>), dim3(rows), dim3(128), 0, s, p);
  else DSPINE_LAUNCH((cand_code_kernel<float, float>), dim3(rows), dim3(128), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_cand_msg(const ProposeParams& p, int dtype, hipStream_t s) {
  const int rows = p.B * (p.W - 1) * p.K;
  if (dtype == DT_BF16) DSPINE_LAUNCH((cand_msg_kernel<bf16_t, f16_t>), dim3(rows), dim3(128), 0, s, p);
  else DSPINE_LAUNCH((cand_msg_kernel<float, float>), dim3(rows), dim3(128), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_cand_score(const ProposeParams& p, int dtype, hipStream_t s) {
  const int rows = p.B * (p.W - 1) * p.K;
  if (dtype == DT_BF16) DSPINE_LAUNCH((cand_score_kernel<bf16_t>), dim3(rows), dim3(kScoreThreads), 0, s, p);
  else DSPINE_LAUNCH((cand_score_kernel<float>), dim3(rows), dim3(kScoreThreads), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_walk(const ProposeParams& p, hipStream_t s) {
  DSPINE_LAUNCH(walk_kernel, dim3(p.B), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace dspine
