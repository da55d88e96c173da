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

namespace dspine {

constexpr int kTopkThreads = 256;
constexpr int kTopkChunks = 64;        // vocabulary slices of one row's partial top-K
constexpr int kScoreThreads = 256;
constexpr int kMaxHidden = 8192;       // refined state kept in LDS

// Ranking of (score, token): a higher score first, equal scores the smaller
// token first.  A NaN score never ranks ahead of anything.
__device__ __forceinline__ bool ranks_before(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// A sorted list of the best kMaxTopK (score, token) pairs in registers.
struct TopList {
  float v[kMaxTopK];
  int i[kMaxTopK];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
      v[s] = -INFINITY;
      i[s] = INT_MAX;
    }
  }
  __device__ __forceinline__ void insert(float nv, int ni) {
    if (!ranks_before(nv, ni, v[kMaxTopK - 1], i[kMaxTopK - 1])) return;
    // walk up from the last slot: entries the new pair beats move down one
    bool placed = false;
#pragma unroll
    for (int s = kMaxTopK - 1; s >= 1; --s) {
      const bool up = !placed && ranks_before(nv, ni, v[s - 1], i[s - 1]);
      const float wv = up ? v[s - 1] : (placed ? v[s] : nv);
      const int wi = up ? i[s - 1] : (placed ? i[s] : ni);
      placed = placed || !up;
      v[s] = wv;
      i[s] = wi;
    }
    if (!placed) {
      v[0] = nv;
      i[0] = ni;
    }
  }
};

// Tree merge of n sorted lists held in LDS (list t at sv/si[t*kMaxTopK ..]):
// at each level thread t < half merges lists t and t + half into list t.
// Leaves the best kMaxTopK pairs in list 0.  Every thread of the block calls.
__device__ void merge_lists(float* sv, int* si, int n) {
  for (int half = n / 2; half >= 1; half /= 2) {
    __syncthreads();
    const int t = threadIdx.x;
    float ov[kMaxTopK];
    int oi[kMaxTopK];
    if (t < half) {
      const float* av = sv + t * kMaxTopK;
      const int* ai = si + t * kMaxTopK;
      const float* bv = sv + (t + half) * kMaxTopK;
      const int* bi = si + (t + half) * kMaxTopK;
      // both lists hold kMaxTopK entries and kMaxTopK are taken, so neither
      // runs out before the last step; the read indices stay clamped anyway
      int ia = 0, ib = 0;
#pragma unroll
      for (int s = 0; s < kMaxTopK; ++s) {
        const bool take_a = ranks_before(av[ia], ai[ia], bv[ib], bi[ib]);
        ov[s] = take_a ? av[ia] : bv[ib];
        oi[s] = take_a ? ai[ia] : bi[ib];
        ia = min(ia + (take_a ? 1 : 0), kMaxTopK - 1);
        ib = min(ib + (take_a ? 0 : 1), kMaxTopK - 1);
      }
    }
    __syncthreads();
    if (t < half) {
#pragma unroll
      for (int s = 0; s < kMaxTopK; ++s) {
        sv[t * kMaxTopK + s] = ov[s];
        si[t * kMaxTopK + s] = oi[s];
      }
    }
  }
  __syncthreads();
}

// logits row of proposal row r (rows 1..W-1 of every request)
__device__ __forceinline__ int score_row(int r, int W) { return (r / (W - 1)) * W + 1 + r % (W - 1); }

// Partial top-K: block (c, r) ranks slice c of the vocabulary of proposal row r.
__global__ __launch_bounds__(kTopkThreads) void topk_partial_kernel(const ProposeParams p) {
  __shared__ float sv[kTopkThreads * kMaxTopK];
  __shared__ int si[kTopkThreads * kMaxTopK];
  const int c = blockIdx.x, r = blockIdx.y;
  const int slice = (p.vocab + kTopkChunks - 1) / kTopkChunks;
  const int lo = c * slice, hi = min(p.vocab, lo + slice);
  const gptr<float> row = as_global(p.scores) + (size_t)score_row(r, p.W) * p.vocab;
  TopList L;
  L.clear();
  for (int v = lo + threadIdx.x; v < hi; v += kTopkThreads) L.insert(row[v], v);
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) {
    sv[threadIdx.x * kMaxTopK + s] = L.v[s];
    si[threadIdx.x * kMaxTopK + s] = L.i[s];
  }
  merge_lists(sv, si, kTopkThreads);
  if (threadIdx.x < kMaxTopK) {
    const size_t o = ((size_t)r * kTopkChunks + c) * kMaxTopK + threadIdx.x;
    p.part_v[o] = sv[threadIdx.x];
    p.part_i[o] = si[threadIdx.x];
  }
}

// Final top-K of proposal row r from its kTopkChunks partial lists.  Slots
// that no finite score filled (fewer than K ranked tokens) get token -1.
__global__ __launch_bounds__(kTopkChunks) void topk_merge_kernel(const ProposeParams p) {
  __shared__ float sv[kTopkChunks * kMaxTopK];
  __shared__ int si[kTopkChunks * kMaxTopK];
  const int r = blockIdx.x;
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) {
    const size_t o = ((size_t)r * kTopkChunks + threadIdx.x) * kMaxTopK + s;
    sv[threadIdx.x * kMaxTopK + s] = p.part_v[o];
    si[threadIdx.x * kMaxTopK + s] = p.part_i[o];
  }
  merge_lists(sv, si, kTopkChunks);
  if (threadIdx.x < p.K) {
    const int tok = si[threadIdx.x];
    p.cand[r * p.K + threadIdx.x] = tok == INT_MAX ? -1 : tok;
    p.cand_scores[r * p.K + threadIdx.x] = sv[threadIdx.x];
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

// Row (b, t, i) of the transition table: x' = u_t + rho_t Y, h = g_final x' /
// rms(x'), T[b, t-1, i, j] = E[cand_j] . h for the K candidates j of row t.
// Head rows are read from the fragment-ordered copy: element (v, k) sits at
// ((v/16)*(H/32) + k/32)*512 + 8*((v%16) + 16*((k%32)/8)) + k%8.
template <typename TW>
__global__ __launch_bounds__(kScoreThreads) void cand_score_kernel(const ProposeParams p) {
  __shared__ float h[kMaxHidden];
  __shared__ float red[kScoreThreads / 64];
  __shared__ float dots[kScoreThreads / 64][kMaxTopK];
  const CandRow c = cand_row(blockIdx.x, p.W, p.K);
  const int H = p.H;
  const float* u = p.u + (size_t)(c.b * p.W + c.t) * H;
  const float* y = p.Y + (size_t)blockIdx.x * H;
  float ss = 0.f;
  for (int k = threadIdx.x; k < H; k += kScoreThreads) ss += u[k] * u[k];
  const float rho = sqrtf(block_sum<kScoreThreads>(ss, red) / H);
  float sx = 0.f;
  for (int k = threadIdx.x; k < H; k += kScoreThreads) {
    const float x = u[k] + rho * y[k];
    h[k] = x;
    sx += x * x;
  }
  const float inv = rsqrtf(block_sum<kScoreThreads>(sx, red) / H + p.eps);
  const TW* gain = reinterpret_cast<const TW*>(p.g_final);
  for (int k = threadIdx.x; k < H; k += kScoreThreads) h[k] = h[k] * inv * Elt<TW>::load(gain, k);
  __syncthreads();

  const int* cj = p.cand + (size_t)(c.b * (p.W - 1) + c.t - 1) * p.K;
  const gptr<TW> E = as_global(reinterpret_cast<const TW*>(p.head_packed));
  float acc[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) acc[j] = 0.f;
  const int nchunk = H / 8;              // 8 consecutive columns of one lane fragment
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < p.K) {
      const int v = clamp_token(cj[j], p.vocab);
      const size_t rowbase = (size_t)(v / 16) * (H / 32) * 512 + 8 * (v % 16);
      for (int ch = threadIdx.x; ch < nchunk; ch += kScoreThreads) {
        const size_t o = rowbase + (size_t)(ch / 4) * 512 + 128 * (ch % 4);
        const float* hk = h + 8 * ch;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s += Elt<TW>::gload(E, o + e) * hk[e];
        acc[j] += s;
      }
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

// The walk of request b, serial over its rows (one thread): row 1 uses table
// row 0 (the anchor), row t the row chosen at t-1.  Greedy: the first
// maximum.  Sampled: float64 p = softmax(T / temperature) with the normaliser
// and the cumulative sum taken left to right, the first j whose cumulative
// probability exceeds the uniform (the last j if none does).
__global__ __launch_bounds__(64) void walk_kernel(const ProposeParams p) {
  if (threadIdx.x != 0) return;
  const int b = blockIdx.x, n = p.W - 1, K = p.K;
  int i = 0;
  for (int t = 0; t < n; ++t) {
    const float* row = p.table + ((size_t)(b * n + t) * K + i) * K;
    int j = 0;
    double q = 1.0;
    if (p.walk == DSPINE_WALK_GREEDY) {
      float best = row[0];
      for (int jj = 1; jj < K; ++jj)
        if (row[jj] > best) {
          best = row[jj];
          j = jj;
        }
    } else {
      double mx = (double)row[0] / p.temperature;
      for (int jj = 1; jj < K; ++jj) mx = fmax(mx, (double)row[jj] / p.temperature);
      double total = 0.0;
      for (int jj = 0; jj < K; ++jj) total += exp((double)row[jj] / p.temperature - mx);
      const double u = p.uniforms[b * n + t];
      double cdf = 0.0;
      j = K - 1;
      for (int jj = 0; jj < K; ++jj) {
        cdf += exp((double)row[jj] / p.temperature - mx) / total;
        if (u < cdf) {
          j = jj;
          break;
        }
      }
      q = exp((double)row[j] / p.temperature - mx) / total;
    }
    p.choice[b * n + t] = j;
    p.tokens[b * n + t] = p.cand[(b * n + t) * K + j];
    if (p.q) p.q[b * n + t] = q;
    i = j;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_topk(const ProposeParams& p, hipStream_t s) {
  const int rows = p.B * (p.W - 1);
  DSPINE_LAUNCH(topk_partial_kernel, dim3(kTopkChunks, rows), dim3(kTopkThreads), 0, s, p);
  DSPINE_LAUNCH(topk_merge_kernel, dim3(rows), dim3(kTopkChunks), 0, s, p);
  return hipGetLastError();
}
size_t topk_partial_entries(int rows) { return (size_t)rows * kTopkChunks * kMaxTopK; }
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
