// C ABI of the DSpine draft-block library: argument checks, workspace plan and
// the launch sequences of the three hot-path calls.  All arithmetic runs in
// the HIP kernels; this file only validates and enqueues.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dspine_internal.hpp"
#include "propose_internal.hpp"
#include "conv_internal.hpp"

struct dspine_model {
  dspine_geometry g;
  dspine_weights w;    // as given: projection matrices row-major [out, in]
  dspine_weights pw;   // the same with projection matrices in fragment order
  const void* head_fp8 = nullptr;        // the LM head's E4M3 codes in fragment order (BF16 models)
  const float* head_fp8_scale = nullptr; // 256 x its power-of-two row scales
  bool packed = false;
};

using namespace dspine;

namespace {

thread_local std::string t_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  t_err = buf;
  return code;
}
int ok() {
  t_err.clear();
  return DSPINE_OK;
}
#define HIP_TRY(expr)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess) return fail(DSPINE_E_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
int elt_bytes(const dspine_geometry& g) { return g.dtype == DSPINE_BF16 ? 2 : 4; }
// activation (MFMA operand) bytes: fp16 for BF16 models, float for F32 models
int act_bytes(const dspine_geometry& g) { return g.dtype == DSPINE_BF16 ? 2 : 4; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// CU count of the current device, cached per device.
int num_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// ---------------------------------------------------------------------------
// kernel timing: event pairs around launches of selected classes
// ---------------------------------------------------------------------------
struct Profiler {
  std::mutex mu;
  uint32_t mask = 0;
  uint32_t stride = 1;                          // time every stride-th scope of a class
  uint64_t seen[DSPINE_PROF_KINDS] = {};        // scopes opened per class since the stride was set
  std::vector<std::pair<hipEvent_t, hipEvent_t>> rec[DSPINE_PROF_KINDS];
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Profiler& prof() {
  static Profiler p;
  return p;
}
// Records a start event now and a stop event when it goes out of scope.
// The events the launches of an open profiling scope on this thread record
// (see DSPINE_LAUNCH): the first launch records `start` at its own start,
// every launch records `stop` at its end (the last one counts).
thread_local LaunchTimer t_scope{nullptr, nullptr};
thread_local LaunchTimer t_give{nullptr, nullptr};
thread_local bool t_scope_open = false;
thread_local int t_scope_launches = 0;

// Times the kernels launched while it is alive, from the first one's start
// to the last one's end.
class ProfScope {
 public:
  ProfScope(int kind, hipStream_t s) : kind_(kind) {
    (void)s;
    Profiler& p = prof();
    if (!(p.mask & (1u << kind)) || t_scope_open) return;
    std::lock_guard<std::mutex> lk(p.mu);
    if (p.seen[kind]++ % p.stride != 0) return;
    a_ = p.get();
    b_ = p.get();
    if (a_ && b_) {
      t_scope = LaunchTimer{a_, b_};
      t_scope_open = true;
      t_scope_launches = 0;
    }
  }
  ~ProfScope() {
    if (!a_ || !b_) return;
    const bool launched = t_scope_launches > 0;
    t_scope_open = false;
    Profiler& p = prof();
    std::lock_guard<std::mutex> lk(p.mu);
    if (launched) {
      p.rec[kind_].emplace_back(a_, b_);
    } else {
      p.pool.push_back(a_);
      p.pool.push_back(b_);
    }
  }
 private:
  int kind_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
};

// first context position block row 0 sees (host twin of ctx_row_lo)
int64_t row0_lo(int64_t F, int S) {
  if (S == 0) return 0;
  return std::min(F, std::max<int64_t>(0, F - S + 1));
}
// live interval start of a layer after frontier F [NIF, ring storage]
int64_t live_lo(int S, int64_t F) { return S == 0 ? 0 : std::max<int64_t>(0, F - S); }

// ---------------------------------------------------------------------------
// workspace plan.  Counters sit first at fixed offsets so that they stay
// zero from call to call whatever else the calls put in the buffer.
// ---------------------------------------------------------------------------
struct Plan {
  size_t gemm_cnt;                        // u32 tile counters
  size_t bridge_sync;                     // u32 hand-off counters of the fused bridge
  size_t counters_end;                    // every counter lies below this offset
  size_t ssz;                             // fused bridge: sums of squares of z per 16 columns
  size_t gemm_part, attn_part;            // f32 partials
  size_t x, act_q, act_f, qkv, z, P, P2, rope;
  size_t act_h, act_r, act_m;             // pre-scaled operands (large blocks)
  size_t st0, st1, stz, stc;              // row statistics [lists][kMaxRows]
  size_t c_raw, c_act, kv_raw;            // materialize, per row block
  size_t conv_da, conv_dm, o_tmp;         // DFlash2 convolution deltas and branch output
  size_t gemm_part_floats;                // capacity of gemm_part
  size_t total;
};
// row-statistics lists a GEMM writes for `width` output columns (one per 64)
int stat_tiles(int width) { return gemm_stream_stat_lists(width); }

// Workspace of a call over B requests of width W (forward, bridge, propose)
// or of a materialize call whose row blocks hold up to `rows` positions:
// the streamed GEMMs' split partials are sized for the most rows one of
// them multiplies (B*W, or a materialize chunk of at most kMaxRows), the
// attention's for B requests.
Plan make_plan(const dspine_geometry& g, int64_t B, int64_t W, int64_t rows) {
  Plan p{};
  const size_t eb = elt_bytes(g);
  const int64_t M = B * W;
  const int64_t Mp = ((std::max<int64_t>(M, 1) + 15) / 16) * 16;
  const int gemm_rows = (int)std::max<int64_t>(M, std::min<int64_t>(rows, kMaxRows));
  const int qd = g.n_q_heads * g.head_dim, kvd = g.n_kv_heads * g.head_dim;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  p.gemm_cnt = take(sizeof(uint32_t) * kMaxTiles);
  p.bridge_sync = take(sizeof(uint32_t) * kBridgeSyncWords);
  p.counters_end = off;
  p.gemm_part_floats = gemm_stream_partial_floats(gemm_rows);
  p.gemm_part = take(sizeof(float) * p.gemm_part_floats);
  p.attn_part = take(sizeof(float) * attn_partial_floats((int)std::max<int64_t>(B, 1), g.n_q_heads, g.head_dim));
  p.x = take(4 * Mp * g.hidden);
  p.act_q = take(eb * Mp * qd);
  p.act_f = take(eb * Mp * g.ffn);
  const int r = std::max(g.code_dim, 1), a = std::max(g.msg_dim, 1);
  p.qkv = take(4 * Mp * (qd + 2 * kvd));
  p.z = take(4 * Mp * r);
  p.P = take(4 * Mp * 3 * a);
  p.P2 = take(4 * Mp * 3 * a);
  p.rope = take(4 * Mp * g.head_dim);
  p.act_h = take(eb * Mp * g.hidden);
  p.act_r = take(eb * Mp * r);
  p.act_m = take(eb * Mp * a);
  p.st0 = take(4 * (size_t)kMaxRows * stat_tiles(g.hidden));
  p.st1 = take(4 * (size_t)kMaxRows * stat_tiles(g.hidden));
  p.stz = take(4 * (size_t)kMaxRows * stat_tiles(r));
  p.stc = take(4 * (size_t)kMaxRows * stat_tiles(g.hidden));
  p.ssz = take(4 * (size_t)kMaxRows * (r / 16 + 1));
  const size_t cg = g.conv_group > 0 ? (size_t)g.hidden / g.conv_group : 0;
  p.conv_da = take(4 * Mp * 4 * cg);
  p.conv_dm = take(4 * Mp * 4 * cg);
  p.o_tmp = take(cg ? 4 * Mp * g.hidden : 0);
  const int64_t R = std::max<int64_t>(rows, 0);
  p.c_raw = take(4 * R * g.hidden);
  p.c_act = take(eb * R * g.hidden);
  p.kv_raw = take(4 * R * (int64_t)g.n_layers * 2 * kvd);
  p.total = off;
  return p;
}
// materialize row-block capacity of a workspace of `bytes`: the most rows
// whose plan fits (the plan grows with the rows)
int64_t rows_capacity(const dspine_geometry& g, size_t bytes) {
  if (make_plan(g, 1, 1, 1).total > bytes) return 0;
  int64_t lo = 1, hi = 1;
  while (hi < (int64_t(1) << 40) && make_plan(g, 1, 1, 2 * hi).total <= bytes) hi *= 2;
  hi *= 2;                                             // plan(lo) fits, plan(hi) does not
  while (hi - lo > 1) {
    const int64_t mid = lo + (hi - lo) / 2;
    (make_plan(g, 1, 1, mid).total <= bytes ? lo : hi) = mid;
  }
  return lo;
}

int check_geometry(const dspine_geometry& g) {
  if (g.dtype != DSPINE_F32 && g.dtype != DSPINE_BF16) return fail(DSPINE_E_UNSUPPORTED, "dtype %d", g.dtype);
  if (g.n_layers < 1 || g.n_layers > DSPINE_MAX_LAYERS)
    return fail(DSPINE_E_UNSUPPORTED, "n_layers %d not in 1..%d", g.n_layers, DSPINE_MAX_LAYERS);
  if (g.hidden <= 0 || g.hidden % 64) return fail(DSPINE_E_UNSUPPORTED, "hidden %d not a positive multiple of 64", g.hidden);
  if (g.head_dim != 64 && g.head_dim != 128) return fail(DSPINE_E_UNSUPPORTED, "head_dim %d not 64 or 128", g.head_dim);
  if (g.n_kv_heads < 1 || g.n_q_heads < g.n_kv_heads || g.n_q_heads % g.n_kv_heads)
    return fail(DSPINE_E_UNSUPPORTED, "heads %d/%d", g.n_q_heads, g.n_kv_heads);
  const int grp = g.n_q_heads / g.n_kv_heads;
  if (grp != 1 && grp != 2 && grp != 4 && grp != 8)
    return fail(DSPINE_E_UNSUPPORTED, "query heads per KV head %d not in {1,2,4,8}", grp);
  if (g.n_q_heads > 256) return fail(DSPINE_E_UNSUPPORTED, "n_q_heads %d > 256", g.n_q_heads);
  if (g.ffn <= 0 || g.ffn % 64) return fail(DSPINE_E_UNSUPPORTED, "ffn %d not a positive multiple of 64", g.ffn);
  if (g.n_feat_layers < 1) return fail(DSPINE_E_UNSUPPORTED, "n_feat_layers %d", g.n_feat_layers);
  if ((g.code_dim == 0) != (g.msg_dim == 0) || g.code_dim < 0 || g.msg_dim < 0)
    return fail(DSPINE_E_UNSUPPORTED, "code_dim %d / msg_dim %d: both zero or both positive", g.code_dim, g.msg_dim);
  if (g.code_dim % 32 || g.msg_dim % 32)
    return fail(DSPINE_E_UNSUPPORTED, "code_dim %d and msg_dim %d must be multiples of 32", g.code_dim, g.msg_dim);
  if (g.vocab < 1 || g.mask_token_id < 0 || g.mask_token_id >= g.vocab)
    return fail(DSPINE_E_UNSUPPORTED, "vocab %d / mask_token_id %d", g.vocab, g.mask_token_id);
  if (g.block_causal != 0 && g.block_causal != 1) return fail(DSPINE_E_UNSUPPORTED, "block_causal %d", g.block_causal);
  for (int l = 0; l < g.n_layers; ++l)
    if (g.window[l] < 0) return fail(DSPINE_E_UNSUPPORTED, "window[%d] = %d", l, g.window[l]);
  if (!(g.eps >= 0.f) || !(g.rope_theta > 0.f)) return fail(DSPINE_E_UNSUPPORTED, "eps / rope_theta");
  if (g.conv_group < 0 || (g.conv_group > 0 && (g.conv_group % 4 || g.hidden % g.conv_group ||
                                                (g.hidden / g.conv_group) % 16 || g.hidden > 8192)))
    return fail(DSPINE_E_UNSUPPORTED, "conv_group %d: a multiple of 4 dividing hidden into a multiple of 16 groups "
                "(hidden <= 8192)", g.conv_group);
  return DSPINE_OK;
}

int check_weights(const dspine_geometry& g, const dspine_weights& w) {
  auto need = [&](const void* p, const char* name, int layer) -> int {
    if (!p) return fail(DSPINE_E_ARG, "weight %s (layer %d) is NULL", name, layer);
    if (!aligned16(p)) return fail(DSPINE_E_ARG, "weight %s (layer %d) not 16-byte aligned", name, layer);
    return DSPINE_OK;
  };
  int rc;
#define NEED(ptr, name, layer) if ((rc = need(ptr, name, layer)) != DSPINE_OK) return rc
  NEED(w.embed, "embed", -1);
  NEED(w.w_feat, "w_feat", -1);
  NEED(w.g_ctx, "g_ctx", -1);
  NEED(w.g_final, "g_final", -1);
  if (g.code_dim > 0) {
    NEED(w.codebook, "codebook", -1);
    NEED(w.bridge_G, "bridge_G", -1);
    NEED(w.bridge_Gp, "bridge_Gp", -1);
    NEED(w.bridge_A, "bridge_A", -1);
    NEED(w.bridge_b, "bridge_b", -1);
  }
  for (int l = 0; l < g.n_layers; ++l) {
    const dspine_layer_weights& L = w.layer[l];
    NEED(L.g_in, "g_in", l);
    NEED(L.wq, "wq", l);
    NEED(L.wk, "wk", l);
    NEED(L.wv, "wv", l);
    NEED(L.gq, "gq", l);
    NEED(L.gk, "gk", l);
    NEED(L.wo, "wo", l);
    NEED(L.g_post, "g_post", l);
    NEED(L.w_gate, "w_gate", l);
    NEED(L.w_up, "w_up", l);
    NEED(L.w_down, "w_down", l);
    if (g.code_dim > 0) {
      NEED(L.R, "R", l);
      NEED(L.W_l, "W_l", l);
    }
    if (g.conv_group > 0) {
      NEED(L.attn_conv_w, "attn_conv_w", l);
      NEED(L.attn_conv_base, "attn_conv_base", l);
      NEED(L.mlp_conv_w, "mlp_conv_w", l);
      NEED(L.mlp_conv_base, "mlp_conv_base", l);
    }
  }
#undef NEED
  if (w.lm_head) {
    if (!aligned16(w.lm_head)) return fail(DSPINE_E_ARG, "weight lm_head not 16-byte aligned");
    if (g.vocab % 16) return fail(DSPINE_E_UNSUPPORTED, "lm_head needs vocab %d to be a multiple of 16", g.vocab);
  }
  return DSPINE_OK;
}

int check_ctx_rings(const dspine_model& m, const dspine_ctx& c, int b, int64_t need_full) {
  const dspine_geometry& g = m.g;
  if (c.frontier < 0) return fail(DSPINE_E_STATE, "request %d: frontier %lld < 0", b, (long long)c.frontier);
  for (int l = 0; l < g.n_layers; ++l) {
    if (!c.k_ring[l] || !c.v_ring[l]) return fail(DSPINE_E_ARG, "request %d layer %d: ring pointer NULL", b, l);
    if (!aligned16(c.k_ring[l]) || !aligned16(c.v_ring[l]))
      return fail(DSPINE_E_ARG, "request %d layer %d: ring not 16-byte aligned", b, l);
    const int S = g.window[l];
    if (S > 0 && c.capacity[l] != S)
      return fail(DSPINE_E_STATE, "request %d layer %d: ring capacity %lld != window %d", b, l,
                  (long long)c.capacity[l], S);
    if (S == 0 && c.capacity[l] < need_full)
      return fail(DSPINE_E_STATE, "request %d layer %d: full-layer capacity %lld < %lld", b, l,
                  (long long)c.capacity[l], (long long)need_full);
  }
  return DSPINE_OK;
}

// Projection matrices of a model (the operands streamed by the GEMMs), each
// with its rows and columns; `global` / `layer` select the pointer field.
struct Proj {
  const void* dspine_weights::*global;
  const void* dspine_layer_weights::*layer;
  int rows, cols;
  const char* name;
};
std::vector<Proj> projections(const dspine_geometry& g) {
  const int H = g.hidden, qd = g.n_q_heads * g.head_dim, kvd = g.n_kv_heads * g.head_dim;
  std::vector<Proj> v = {
      {nullptr, &dspine_layer_weights::wq, qd, H, "wq"},      {nullptr, &dspine_layer_weights::wk, kvd, H, "wk"},
      {nullptr, &dspine_layer_weights::wv, kvd, H, "wv"},     {nullptr, &dspine_layer_weights::wo, H, qd, "wo"},
      {nullptr, &dspine_layer_weights::w_gate, g.ffn, H, "w_gate"},
      {nullptr, &dspine_layer_weights::w_up, g.ffn, H, "w_up"},
      {nullptr, &dspine_layer_weights::w_down, H, g.ffn, "w_down"}};
  if (g.code_dim > 0) {
    v.push_back({nullptr, &dspine_layer_weights::R, g.code_dim, H, "R"});
    v.push_back({nullptr, &dspine_layer_weights::W_l, H, g.msg_dim, "W_l"});
  }
  if (g.conv_group > 0) {
    v.push_back({nullptr, &dspine_layer_weights::attn_conv_w, 4 * (H / g.conv_group), H, "attn_conv_w"});
    v.push_back({nullptr, &dspine_layer_weights::mlp_conv_w, 4 * (H / g.conv_group), H, "mlp_conv_w"});
  }
  v.push_back({&dspine_weights::w_feat, nullptr, H, g.n_feat_layers * H, "w_feat"});
  if (g.code_dim > 0) {
    v.push_back({&dspine_weights::bridge_G, nullptr, g.msg_dim, g.code_dim, "bridge_G"});
    v.push_back({&dspine_weights::bridge_Gp, nullptr, g.msg_dim, g.code_dim, "bridge_Gp"});
    v.push_back({&dspine_weights::bridge_A, nullptr, g.msg_dim, g.code_dim, "bridge_A"});
  }
  return v;
}
// bytes of the fragment-ordered copy (the shared LM head too when given)
size_t packed_bytes(const dspine_geometry& g, bool head) {
  size_t total = 0;
  for (const Proj& pr : projections(g)) {
    const size_t one = align256((size_t)pr.rows * pr.cols * elt_bytes(g));
    total += pr.layer ? one * g.n_layers : one;
  }
  if (head) total += align256((size_t)g.vocab * g.hidden * elt_bytes(g));
  if (head && g.dtype == DSPINE_BF16)          // the head's FP8 copy and its row scales
    total += align256((size_t)g.vocab * g.hidden) + align256(sizeof(float) * (size_t)g.vocab);
  if (g.dtype == DSPINE_BF16) total += 256;    // the range check's maxima
  return total;
}

// Projections whose bf16 weights a BF16 model's GEMMs widen to fp16 (every
// projection but w_feat and w_down, which multiply bf16 x bf16): their
// magnitudes must stay within fp16's range.
bool widened_to_fp16(const Proj& pr) {
  return pr.layer != &dspine_layer_weights::w_down && pr.global != &dspine_weights::w_feat;
}
constexpr float kF16Max = 65504.f;

// streamed GEMM helpers -------------------------------------------------------
GemmParams gemm_base(const Plan& P, char* ws, int K, int M) {
  GemmParams gp;
  memset(&gp, 0, sizeof gp);
  gp.K = K;
  gp.M = M;
  gp.partials = reinterpret_cast<float*>(ws + P.gemm_part);
  gp.partial_floats = P.gemm_part_floats;
  gp.counters = reinterpret_cast<uint32_t*>(ws + P.gemm_cnt);
  return gp;
}
void set_segments(GemmParams& gp, std::initializer_list<std::pair<const void*, int>> segs) {
  int blk = 0, s = 0;
  for (const auto& sg : segs) {
    gp.seg_ptr[s] = sg.first;
    gp.seg_blk0[s] = blk;
    blk += sg.second / 16;
    ++s;
  }
  gp.nseg = s;
  gp.nblk = blk;
}

// A operand of a streamed GEMM: fp32 rows x[m, :K] (stride ldx) times the
// per-row scale `mode` formed from the row statistics `st` (`lists` lists),
// times `gain` when given.  Small blocks form it in the GEMM prologue; large
// ones through the pre-scale kernel into `act` (stride K).
int set_scaled_a(GemmParams& gp, const dspine_geometry& g, int M, int W, const float* x, int ldx, int K, int mode,
                 const float* st, int lists, float n, const void* gain, void* act, hipStream_t stream,
                 bool round_bf16 = false) {
  gp.scale_n = n;
  gp.eps = g.eps;
  gp.code_scale = sqrtf((float)std::max(g.code_dim, 1));
  gp.W = W;
  if (M <= gemm_stream_fused_rows()) {
    gp.pro = gain ? PRO_NORM : PRO_SCALE;
    gp.xa = x;
    gp.lda = ldx;
    gp.gain = gain;
    gp.scale_mode = mode;
    gp.stats_in = st;
    gp.stats_tiles = lists;
    gp.stats_ld = kMaxRows;
    gp.act_round_bf16 = round_bf16 ? 1 : 0;
    return DSPINE_OK;
  }
  ScaleParams sp;
  memset(&sp, 0, sizeof sp);
  sp.M = M;
  sp.K = K;
  sp.W = W;
  sp.mode = mode;
  sp.stats = st;
  sp.lists = lists;
  sp.ld = kMaxRows;
  sp.n = n;
  sp.eps = g.eps;
  sp.code_scale = gp.code_scale;
  sp.x = x;
  sp.ldx = ldx;
  sp.gain = gain;
  sp.round_bf16 = round_bf16 ? 1 : 0;
  sp.act = act;
  sp.ld_act = K;
  HIP_TRY(launch_scale_rows(sp, g.dtype, stream));
  gp.pro = PRO_COPY;
  gp.a = act;
  gp.lda = K;
  return DSPINE_OK;
}

// act = the scaled operand of x (mode `mode`, rows' statistics `st`), then
// a copy prologue: for BF16 models at 16 rows and under, whose copy GEMMs
// stream their operand straight into LDS in long stages
int set_prescaled_a(GemmParams& gp, const dspine_geometry& g, int M, int W, const float* x, int K, int mode,
                    const float* st, int lists, const void* gain, void* act, hipStream_t stream,
                    bool round_bf16 = false) {
  ScaleParams sp;
  memset(&sp, 0, sizeof sp);
  sp.M = M;
  sp.K = K;
  sp.W = W;
  sp.mode = mode;
  sp.stats = st;
  sp.lists = lists;
  sp.ld = kMaxRows;
  sp.n = (float)K;
  sp.eps = g.eps;
  sp.code_scale = sqrtf((float)std::max(g.code_dim, 1));
  sp.x = x;
  sp.ldx = K;
  sp.gain = gain;
  sp.round_bf16 = round_bf16 ? 1 : 0;
  sp.act = act;
  sp.ld_act = K;
  HIP_TRY(launch_scale_rows(sp, g.dtype, stream));
  gp.pro = PRO_COPY;
  gp.a = act;
  gp.lda = K;
  return DSPINE_OK;
}
bool prescale_pays(const dspine_geometry& g, int M, int K) { return g.dtype == DSPINE_BF16 && M <= 16 && K % 512 == 0; }

// The norm of a raw-row operand applied after the product: the epilogue
// multiplies row m's products by its row scale (mode, from the statistics
// lists st), a per-row factor of the contraction
void set_post_scale(GemmParams& gp, const dspine_geometry& g, int W, int mode, const float* st, int lists, float n,
                    float mult = 1.f) {
  gp.post_scale = 1;
  gp.post_mult = mult;
  gp.scale_mode = mode;
  gp.stats_in = st;
  gp.stats_tiles = lists;
  gp.stats_ld = kMaxRows;
  gp.scale_n = n;
  gp.eps = g.eps;
  gp.code_scale = sqrtf((float)std::max(g.code_dim, 1));
  gp.W = W;
}
// The epilogue also stores a 16-bit copy of its output (times mult and
// gain[n]) as the next GEMM's operand
void set_copy(GemmParams& gp, void* dst, int ld, bool bf16, const void* gain, float mult = 1.f) {
  gp.out_copy = dst;
  gp.ld_copy = ld;
  gp.copy_bf16 = bf16 ? 1 : 0;
  gp.copy_gain = gain;
  gp.copy_mult = mult;
}
// Blocks of more than 32 rows (BF16): GEMMs with at most 32 MB of weights
// run as row blocks side by side, each with a stream-K split of its own,
// instead of one 128-row tile row whose few column tiles are split deep over
// K: blocks of 16 rows up to 12 MB of weights, of 32 rows above and where K
// is a single 512-K stage (W_l: the 16-row blocks left 80 column tiles to 64
// workgroups a block, 32-row blocks give each its own; bridge 208 -> 204 us
// per B=8 forward).  The row
// blocks of one column range run on one XCD (grid widths that are multiples
// of 8) and read the weights through its L2 (ordinary loads, not
// non-temporal ones); larger matrices still pay for the extra reads.  B=8
// per forward: at the 27B geometry the bridge's R, [G; G_p; A] and W_l
// 315 -> 239 us in 32-row blocks, 216 in 16-row ones, while q|k|v (63 MB)
// went 167 -> 195 and O (42 MB) 149 -> 157 in 32-row blocks; at the
// 35B-style geometry q|k|v (25 MB) 141 -> 121 in 32-row blocks (161 in
// 16-row ones) and O (17 MB) 140 -> 120.
void set_row_blocks(GemmParams& gp, const dspine_geometry& g, int M, int64_t N, int64_t K) {
  if (g.dtype != DSPINE_BF16 || M <= gemm_stream_fused_rows()) return;
  const int64_t bytes = N * K * 2;
  if (bytes <= ((int64_t)12 << 20) && K > 512) gp.rb_rows = 16;
  else if (bytes <= ((int64_t)32 << 20)) gp.rb_rows = 32;
}
// Raw residual rows (not yet normalised) travel as fp16 times 2^-8: fp16's
// 11-bit precision (bf16 copies, with 8 bits, took the 27B B=8 forward's
// error against the oracle from about 0.009 to 0.021) with headroom up to
// |x g| of about 1.7e7;
// entries below 2^-6 lose relative precision but keep an absolute error
// under 2^-16.  The consuming GEMM multiplies its products back by 2^8.
constexpr float kRawCopy = 1.f / 256.f, kRawPost = 256.f;

}  // namespace

const LaunchTimer* dspine::take_launch_timer() {
  if (!t_scope_open) return nullptr;
  t_give = LaunchTimer{t_scope_launches == 0 ? t_scope.start : nullptr, t_scope.stop};
  ++t_scope_launches;
  return &t_give;
}

// =============================================================================
extern "C" {

const char* dspine_last_error(void) { return t_err.c_str(); }

int dspine_profile_enable(uint32_t kind_mask) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  p.mask = kind_mask & ((1u << DSPINE_PROF_KINDS) - 1);
  return ok();
}

int dspine_profile_stride(uint32_t stride) {
  if (stride == 0) return fail(DSPINE_E_ARG, "profile_stride: stride must be >= 1");
  Profiler& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  p.stride = stride;
  for (uint64_t& n : p.seen) n = 0;
  return ok();
}

int dspine_profile_read(int kind, double* total_ms, int64_t* launches) {
  if (kind < 0 || kind >= DSPINE_PROF_KINDS || !total_ms || !launches)
    return fail(DSPINE_E_ARG, "profile_read: bad argument");
  Profiler& p = prof();
  std::vector<std::pair<hipEvent_t, hipEvent_t>> rec;
  {
    std::lock_guard<std::mutex> lk(p.mu);
    rec.swap(p.rec[kind]);
  }
  double sum = 0.0;
  int rc = DSPINE_OK;
  for (auto& ab : rec) {
    float ms = 0.f;
    if (hipEventSynchronize(ab.second) != hipSuccess || hipEventElapsedTime(&ms, ab.first, ab.second) != hipSuccess)
      rc = fail(DSPINE_E_HIP, "profile_read: event query failed");
    sum += ms;
  }
  {
    std::lock_guard<std::mutex> lk(p.mu);
    for (auto& ab : rec) {
      p.pool.push_back(ab.first);
      p.pool.push_back(ab.second);
    }
  }
  *total_ms = sum;
  *launches = (int64_t)rec.size();
  return rc ? rc : ok();
}
const char* dspine_version(void) { return "dspine-mi355x 0.1 (gfx950)"; }

int dspine_model_create(const dspine_geometry* geom, const dspine_weights* weights, dspine_model** out) {
  if (!geom || !weights || !out) return fail(DSPINE_E_ARG, "model_create: NULL argument");
  *out = nullptr;
  int rc = check_geometry(*geom);
  if (rc) return rc;
  if ((rc = check_weights(*geom, *weights))) return rc;
  dspine_model* m = new (std::nothrow) dspine_model;
  if (!m) return fail(DSPINE_E_ARG, "out of host memory");
  m->g = *geom;
  m->w = *weights;
  *out = m;
  return ok();
}

void dspine_model_destroy(dspine_model* model) { delete model; }

size_t dspine_packed_bytes(const dspine_model* model) {
  if (!model) {
    fail(DSPINE_E_ARG, "packed_bytes: NULL model");
    return 0;
  }
  return packed_bytes(model->g, model->w.lm_head != nullptr);
}

int dspine_pack_weights(dspine_model* model, void* dst, size_t dst_bytes, dspine_stream_t stream) {
  if (!model || !dst) return fail(DSPINE_E_ARG, "pack_weights: NULL argument");
  if (((uintptr_t)dst & 255u) != 0) return fail(DSPINE_E_ARG, "pack_weights: dst not 256-byte aligned");
  const size_t need = packed_bytes(model->g, model->w.lm_head != nullptr);
  if (dst_bytes < need) return fail(DSPINE_E_WORKSPACE, "pack_weights: %zu bytes < %zu needed", dst_bytes, need);
  const dspine_geometry& g = model->g;
  dspine_weights pw = model->w;
  char* out = static_cast<char*>(dst);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (const Proj& pr : projections(g)) {
    const size_t one = align256((size_t)pr.rows * pr.cols * elt_bytes(g));
    if (pr.layer) {
      for (int l = 0; l < g.n_layers; ++l) {
        HIP_TRY(launch_pack(model->w.layer[l].*pr.layer, out, pr.rows, pr.cols, g.dtype, s));
        pw.layer[l].*pr.layer = out;
        out += one;
      }
    } else {
      HIP_TRY(launch_pack(model->w.*pr.global, out, pr.rows, pr.cols, g.dtype, s));
      pw.*pr.global = out;
      out += one;
    }
  }
  if (model->w.lm_head) {
    HIP_TRY(launch_pack(model->w.lm_head, out, g.vocab, g.hidden, g.dtype, s));
    pw.lm_head = out;
    out += align256((size_t)g.vocab * g.hidden * elt_bytes(g));
    if (g.dtype == DSPINE_BF16) {
      float* scale = reinterpret_cast<float*>(out + align256((size_t)g.vocab * g.hidden));
      HIP_TRY(launch_quant_head_fp8(model->w.lm_head, out, scale, g.vocab, g.hidden, s));
      model->head_fp8 = out;
      model->head_fp8_scale = scale;
      out += align256((size_t)g.vocab * g.hidden) + align256(sizeof(float) * (size_t)g.vocab);
    }
  }
  if (g.dtype == DSPINE_BF16) {
    // range check of the weights the GEMMs widen to fp16 operands: the
    // largest magnitude of each projection kind (and of the LM head, whose
    // direct score GEMM widens it too); this waits for the kernels
    const std::vector<Proj> prs = projections(g);
    const int nk = (int)prs.size() + 1;
    uint32_t* mx = reinterpret_cast<uint32_t*>(out);
    HIP_TRY(launch_zero_words(mx, nk, s));
    for (int k = 0; k < (int)prs.size(); ++k) {
      if (!widened_to_fp16(prs[k])) continue;
      const size_t n = (size_t)prs[k].rows * prs[k].cols;
      if (prs[k].layer)
        for (int l = 0; l < g.n_layers; ++l) HIP_TRY(launch_absmax_bf16(model->w.layer[l].*prs[k].layer, n, mx + k, s));
      else
        HIP_TRY(launch_absmax_bf16(model->w.*prs[k].global, n, mx + k, s));
    }
    if (model->w.lm_head) HIP_TRY(launch_absmax_bf16(model->w.lm_head, (size_t)g.vocab * g.hidden, mx + nk - 1, s));
    std::vector<uint32_t> host(nk, 0u);
    HIP_TRY(hipMemcpyAsync(host.data(), mx, sizeof(uint32_t) * nk, hipMemcpyDeviceToHost, s));
    HIP_TRY(hipStreamSynchronize(s));
    for (int k = 0; k < nk; ++k) {
      float v;
      memcpy(&v, &host[k], sizeof v);
      if (!(v <= kF16Max))
        return fail(DSPINE_E_UNSUPPORTED, "pack_weights: %s has a weight of magnitude %g, beyond the fp16 range "
                    "(65504) of the GEMM operands it is widened to", k + 1 < nk ? prs[k].name : "lm_head", v);
    }
  }
  model->pw = pw;
  model->packed = true;
  return ok();
}

size_t dspine_ring_bytes(const dspine_model* model, int layer, int64_t capacity) {
  if (!model || layer < 0 || layer >= model->g.n_layers || capacity < 0) {
    fail(DSPINE_E_ARG, "ring_bytes: bad argument");
    return 0;
  }
  const int S = model->g.window[layer];
  if (S > 0 && capacity != S) {
    fail(DSPINE_E_STATE, "ring_bytes: local layer %d needs capacity %d", layer, S);
    return 0;
  }
  return (size_t)model->g.n_kv_heads * capacity * model->g.head_dim * elt_bytes(model->g);
}

size_t dspine_workspace_bytes(const dspine_model* model, int max_batch, int max_width, int64_t max_rows) {
  if (!model || max_batch < 1 || max_batch > DSPINE_MAX_BATCH || max_width < DSPINE_MIN_WIDTH ||
      max_width > DSPINE_MAX_WIDTH || max_rows < 0) {
    fail(DSPINE_E_ARG, "workspace_bytes: bad argument");
    return 0;
  }
  return make_plan(model->g, max_batch, max_width, max_rows).total;
}

// -----------------------------------------------------------------------------
// a1-a3
// -----------------------------------------------------------------------------
int dspine_ctx_materialize(const dspine_model* model, int n_req, dspine_ctx* ctx, const void* const* feats,
                           const int64_t* n_tok, void* workspace, size_t workspace_bytes,
                           dspine_stream_t stream_) {
  if (!model || !ctx || !feats || !n_tok) return fail(DSPINE_E_ARG, "materialize: NULL argument");
  if (n_req < 1 || n_req > DSPINE_MAX_BATCH) return fail(DSPINE_E_UNSUPPORTED, "materialize: n_req %d", n_req);
  const dspine_geometry& g = model->g;
  const dspine_weights& wt = model->w;
  const dspine_weights& pw = model->pw;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  const int L = g.n_layers, H = g.hidden, kvd = g.n_kv_heads * g.head_dim;

  // rows each request must compute: [need_lo, F1)
  int64_t need_lo[DSPINE_MAX_BATCH], F1[DSPINE_MAX_BATCH], total_rows = 0;
  for (int b = 0; b < n_req; ++b) {
    if (n_tok[b] < 0) return fail(DSPINE_E_ARG, "materialize: n_tok[%d] = %lld", b, (long long)n_tok[b]);
    const int64_t F0 = ctx[b].frontier;
    F1[b] = F0 + n_tok[b];
    int rc = check_ctx_rings(*model, ctx[b], b, F1[b]);
    if (rc) return rc;
    if (n_tok[b] > 0 && !feats[b]) return fail(DSPINE_E_ARG, "materialize: feats[%d] is NULL", b);
    if (n_tok[b] > 0 && !aligned16(feats[b])) return fail(DSPINE_E_ARG, "materialize: feats[%d] not aligned", b);
    int64_t lo = F1[b];
    for (int l = 0; l < L; ++l) lo = std::min(lo, std::max(F0, live_lo(g.window[l], F1[b])));
    need_lo[b] = lo;
    total_rows += F1[b] - lo;
  }
  if (total_rows > 0) {
    if (!workspace || !aligned16(workspace)) return fail(DSPINE_E_ARG, "materialize: workspace NULL or unaligned");
    const int64_t cap_rows = rows_capacity(g, workspace_bytes);
    if (cap_rows < 1)
      return fail(DSPINE_E_WORKSPACE, "materialize: workspace of %zu bytes holds no row block", workspace_bytes);
    if (!model->packed) return fail(DSPINE_E_STATE, "weights not packed: call dspine_pack_weights first");
    char* ws = static_cast<char*>(workspace);
    const int cus = num_cus();
    const int64_t blk_rows = std::min<int64_t>(cap_rows, total_rows);
    const Plan P = make_plan(g, 1, 1, blk_rows);
    float* c_raw = reinterpret_cast<float*>(ws + P.c_raw);
    void* c_act = ws + P.c_act;
    float* kv_raw = reinterpret_cast<float*>(ws + P.kv_raw);
    float* stc = reinterpret_cast<float*>(ws + P.stc);
    const int ldkv = L * 2 * kvd;

    // walk the concatenated row list in blocks
    int64_t done = 0;
    while (done < total_rows) {
      const int64_t nrows = std::min(blk_rows, total_rows - done);
      // requests intersecting [done, done + nrows)
      int nsrc = 0;
      const void* src[DSPINE_MAX_BATCH];
      int32_t row0[DSPINE_MAX_BATCH + 1];
      int64_t skip[DSPINE_MAX_BATCH], pos0[DSPINE_MAX_BATCH];
      int req_of[DSPINE_MAX_BATCH];
      int64_t acc = 0;
      for (int b = 0; b < n_req; ++b) {
        const int64_t rb = F1[b] - need_lo[b];
        const int64_t s0 = std::max(acc, done), s1 = std::min(acc + rb, done + nrows);
        if (s1 > s0) {
          src[nsrc] = feats[b];
          row0[nsrc] = (int32_t)(s0 - done);
          const int64_t first_pos = need_lo[b] + (s0 - acc);
          skip[nsrc] = first_pos - ctx[b].frontier;      // feature row of that position
          pos0[nsrc] = first_pos;
          req_of[nsrc] = b;
          ++nsrc;
        }
        acc += rb;
      }
      row0[nsrc] = (int32_t)nrows;

      // a1: c_raw = W_feat s; a2: every layer's K and V projections of
      // c = plain_rmsnorm(c_raw, g_ctx)
      const bool tile = g.dtype == DSPINE_BF16 && nrows > kMaxRows && gemm_tile_fits(H, g.n_feat_layers * H) &&
                        gemm_tile_fits(kvd, H);
      if (tile) {
        // long blocks: MFMA tile GEMMs with the norm between them
        TileGemmParams tp;
        memset(&tp, 0, sizeof tp);
        tp.seg_ptr[0] = pw.w_feat;
        tp.seg_rows0[0] = 0;
        tp.seg_rows0[1] = H;
        tp.nseg = 1;
        tp.N = H;
        tp.K = g.n_feat_layers * H;
        tp.M = (int)nrows;
        tp.pro = PRO_GATHER;
        tp.a_bf16 = 1;
        tp.lda = g.n_feat_layers * H;
        for (int s = 0; s < nsrc; ++s) {
          tp.g_src[s] = src[s];
          tp.g_row0[s] = row0[s];
          tp.g_skip[s] = skip[s];
        }
        tp.g_row0[nsrc] = row0[nsrc];
        tp.g_n = nsrc;
        tp.out = c_raw;
        tp.ldo = H;
        {
          ProfScope ps(DSPINE_PROF_CTX_GEMM, stream);
          HIP_TRY(launch_gemm_tile(tp, g.dtype, cus, stream));
        }
        RowParams rp;
        memset(&rp, 0, sizeof rp);
        rp.M = (int)nrows;
        rp.H = H;
        rp.x = c_raw;
        rp.act = c_act;
        rp.act_bf16 = 1;                  // the K/V tile GEMM multiplies bf16 x bf16
        rp.gain = wt.g_ctx;
        rp.eps = g.eps;
        {
          ProfScope ps(DSPINE_PROF_CTX_STORE, stream);
          HIP_TRY(launch_rmsnorm(rp, g.dtype, false, stream));
        }
        memset(&tp, 0, sizeof tp);
        for (int l = 0; l < L; ++l) {
          tp.seg_ptr[2 * l] = pw.layer[l].wk;
          tp.seg_ptr[2 * l + 1] = pw.layer[l].wv;
          tp.seg_rows0[2 * l] = 2 * l * kvd;
          tp.seg_rows0[2 * l + 1] = (2 * l + 1) * kvd;
        }
        tp.seg_rows0[2 * L] = 2 * L * kvd;
        tp.nseg = 2 * L;
        tp.N = ldkv;
        tp.K = H;
        tp.M = (int)nrows;
        tp.pro = PRO_COPY;
        tp.a_bf16 = 1;
        tp.a = c_act;
        tp.lda = H;
        tp.out = kv_raw;
        tp.ldo = ldkv;
        ProfScope ps(DSPINE_PROF_CTX_GEMM, stream);
        HIP_TRY(launch_gemm_tile(tp, g.dtype, cus, stream));
      } else {
        // short blocks, in chunks of at most kMaxRows rows: streamed GEMMs,
        // the norm formed in the K/V GEMM from the first one's statistics
        for (int64_t r0 = 0; r0 < nrows; r0 += kMaxRows) {
          const int mr = (int)std::min<int64_t>(kMaxRows, nrows - r0);
          GemmParams gp = gemm_base(P, ws, g.n_feat_layers * H, mr);
          set_segments(gp, {{pw.w_feat, H}});
          gp.pro = PRO_GATHER;
          gp.a_bf16 = 1;                    // target features are bf16 inputs
          gp.lda = g.n_feat_layers * H;
          int n = 0;
          for (int s = 0; s < nsrc; ++s) {
            const int64_t a0 = std::max<int64_t>(row0[s], r0), a1 = std::min<int64_t>(row0[s + 1], r0 + mr);
            if (a1 <= a0) continue;
            gp.g_src[n] = src[s];
            gp.g_row0[n] = (int32_t)(a0 - r0);
            gp.g_skip[n] = skip[s] + (a0 - row0[s]);
            ++n;
          }
          gp.g_row0[n] = mr;
          gp.g_n = n;
          gp.epi = EPI_STORE;
          gp.out = c_raw + r0 * H;
          gp.ldo = H;
          gp.stats_out = stc;
          gp.stats_out_ld = kMaxRows;
          {
            ProfScope ps(DSPINE_PROF_CTX_GEMM, stream);
            HIP_TRY(launch_gemm_stream(gp, g.dtype, cus, stream));
          }
          gp = gemm_base(P, ws, H, mr);
          int blk = 0;
          for (int l = 0; l < L; ++l) {
            gp.seg_ptr[2 * l] = pw.layer[l].wk;
            gp.seg_blk0[2 * l] = blk;
            blk += kvd / 16;
            gp.seg_ptr[2 * l + 1] = pw.layer[l].wv;
            gp.seg_blk0[2 * l + 1] = blk;
            blk += kvd / 16;
          }
          gp.nseg = 2 * L;
          gp.nblk = blk;
          // c passes through bf16, as the long-block path stores it, so that
          // both paths project the same operand values.  At 16 rows and
          // under the pre-scale kernel forms it (the GEMM then streams it
          // into LDS in long stages: 47 -> 36 us per 16-row step at the 27B
          // geometry, the kernel counted)
          int rc2;
          {
            ProfScope ps(DSPINE_PROF_CTX_GEMM, stream);
            rc2 = prescale_pays(g, mr, H)
                      ? set_prescaled_a(gp, g, mr, 1, c_raw + r0 * H, H, SCALE_RMSNORM, stc, stat_tiles(H), wt.g_ctx,
                                        c_act, stream, g.dtype == DSPINE_BF16)
                      : set_scaled_a(gp, g, mr, 1, c_raw + r0 * H, H, H, SCALE_RMSNORM, stc, stat_tiles(H), (float)H,
                                     wt.g_ctx, c_act, stream, g.dtype == DSPINE_BF16);
          }
          if (rc2) return rc2;
          gp.epi = EPI_STORE;
          gp.out = kv_raw + r0 * ldkv;
          gp.ldo = ldkv;
          ProfScope ps(DSPINE_PROF_CTX_GEMM, stream);
          HIP_TRY(launch_gemm_stream(gp, g.dtype, cus, stream));
        }
      }
      // every layer: head norm + RoPE + storage rounding + ring scatter
      for (int l0 = 0; l0 < L; l0 += kKvLayers) {
        KvStoreParams kp;
        memset(&kp, 0, sizeof kp);
        kp.rows = (int)nrows;
        kp.nkv = g.n_kv_heads;
        kp.D = g.head_dim;
        kp.n_req = nsrc;
        kp.n_layers = std::min(kKvLayers, L - l0);
        kp.kv = kv_raw;
        kp.ld = ldkv;
        kp.eps = g.eps;
        kp.rope_theta = g.rope_theta;
        for (int s = 0; s <= nsrc; ++s) kp.row0[s] = row0[s];
        for (int s = 0; s < nsrc; ++s) kp.pos0[s] = pos0[s];
        for (int j = 0; j < kp.n_layers; ++j) {
          const int l = l0 + j;
          kp.S[j] = g.window[l];
          kp.col[j] = 2 * l * kvd;
          kp.gk[j] = wt.layer[l].gk;
          for (int s = 0; s < nsrc; ++s) {
            const int b = req_of[s];
            kp.keep_lo[j][s] = std::max(ctx[b].frontier, live_lo(g.window[l], F1[b]));
            kp.kring[j][s] = ctx[b].k_ring[l];
            kp.vring[j][s] = ctx[b].v_ring[l];
            kp.cap[j][s] = ctx[b].capacity[l];
          }
        }
        ProfScope ps(DSPINE_PROF_CTX_STORE, stream);
        HIP_TRY(launch_kv_store(kp, g.dtype, stream));
      }
      done += nrows;
    }
  }
  for (int b = 0; b < n_req; ++b) ctx[b].frontier = F1[b];
  return ok();
}

// -----------------------------------------------------------------------------
// bridge (a9-a11) on x [M, H] fp32 in place
// -----------------------------------------------------------------------------
namespace {
// x [M, H] fp32 in place; `xst` holds the sums of squares of x's rows as
// `xst_tiles` partial lists (ld kMaxRows).  Writes the new rows' statistics
// to `st_out` (stat_tiles(H) lists).
// The bridge (a9-a11) of `layer` on x.  With the fused kernel (blocks of up to
// 32 rows, BF16) it can also form the next RMS norm of the written x (gain
// next_gain): as the fp16 operand next_act and/or the fp32 rows next_out;
// *folded then says that it did (otherwise the caller forms that norm).
int run_bridge(const dspine_model& m, int layer, int B, int W, float* x, const float* xst, int xst_tiles,
               float* st_out, const int32_t* anchor_ids, const float* pred_codes, char* ws, const Plan& P,
               int cus, hipStream_t stream, const void* next_gain = nullptr, void* next_act = nullptr,
               float* next_out = nullptr, bool* folded = nullptr, const void* x16 = nullptr,
               void* copy_out = nullptr, const void* copy_gain = nullptr) {
  const dspine_geometry& g = m.g;
  const dspine_weights& wt = m.w;
  const int M = B * W, H = g.hidden, r = g.code_dim, a = g.msg_dim;
  if (folded) *folded = false;
  if (!pred_codes && g.dtype == DSPINE_BF16 && bridge_fused_fits(H, r, a, M, cus)) {
    // blocks of up to 32 rows: the whole bridge in one launch
    BridgeParams bp;
    memset(&bp, 0, sizeof bp);
    bp.M = M;
    bp.W = W;
    bp.H = H;
    bp.r = r;
    bp.a = a;
    bp.eps = g.eps;
    bp.code_scale = sqrtf((float)r);
    bp.x = x;
    bp.xst = xst;
    bp.xst_lists = xst_tiles;
    bp.st_out = st_out;
    bp.ld = kMaxRows;
    bp.R = m.pw.layer[layer].R;
    bp.G = m.pw.bridge_G;
    bp.Gp = m.pw.bridge_Gp;
    bp.A = m.pw.bridge_A;
    bp.Wl = m.pw.layer[layer].W_l;
    bp.bias = wt.bridge_b;
    bp.codebook = wt.codebook;
    for (int b = 0; b < B; ++b) bp.anchor[b] = anchor_ids[b];
    bp.zpart = reinterpret_cast<float*>(ws + P.gemm_part);
    bp.z = ws + P.act_r;
    bp.ssz = reinterpret_cast<float*>(ws + P.ssz);
    bp.P = reinterpret_cast<float*>(ws + P.P);
    bp.msg = ws + P.act_m;
    bp.sync = reinterpret_cast<uint32_t*>(ws + P.bridge_sync);
    if (next_gain && (next_act || next_out)) {
      bp.next_gain = next_gain;
      bp.next_act = next_act;
      bp.next_out = next_out;
      if (folded) *folded = true;
    } else if (copy_out) {
      bp.copy_out = copy_out;
      bp.copy_gain = copy_gain;
      bp.copy_mult = kRawCopy;
    }
    HIP_TRY(launch_bridge_fused(bp, stream));
    return DSPINE_OK;
  }
  float* z = reinterpret_cast<float*>(ws + P.z);
  float* stz = reinterpret_cast<float*>(ws + P.stz);
  float* Pb = reinterpret_cast<float*>(ws + P.P);
  float* P2 = reinterpret_cast<float*>(ws + P.P2);

  // z = R (x / (rho + eps)), rho = rms(x); the anchor rows of z take
  // sqrt(r) C[anchor] (their code); statistics of z for the code norm
  GemmParams gp = gemm_base(P, ws, H, M);
  set_segments(gp, {{m.pw.layer[layer].R, r}});
  int rc = DSPINE_OK;
  if (x16) {
    // fp16 rows of x (stored by the down projection); 1 / (rho + eps) after
    // the product, and fp16(z) stored beside z as the next operand
    gp.pro = PRO_COPY;
    gp.a = x16;
    gp.lda = H;
    set_post_scale(gp, g, W, SCALE_RHO_INV, xst, xst_tiles, (float)H, kRawPost);
    set_copy(gp, ws + P.act_r, r, false, nullptr);
  } else if ((rc = set_scaled_a(gp, g, M, W, x, H, H, SCALE_RHO_INV, xst, xst_tiles, (float)H, nullptr, ws + P.act_h,
                                stream))) {
    return rc;
  }
  gp.epi = EPI_STORE;
  gp.out = z;
  gp.ldo = r;
  gp.stats_out = stz;
  gp.stats_out_ld = kMaxRows;
  if (x16) set_row_blocks(gp, g, M, r, H);
  gp.code_anchor = 1;
  gp.codebook = wt.codebook;
  gp.code_scale = sqrtf((float)r);
  gp.W = W;
  for (int b = 0; b < B; ++b) gp.anchor[b] = anchor_ids[b];
  HIP_TRY(launch_gemm_stream(gp, g.dtype, cus, stream));

  // [G; G_p; A] c with c = sqrt(r) z / (||z|| + eps) (anchor rows: z as is)
  gp = gemm_base(P, ws, r, M);
  set_segments(gp, {{m.pw.bridge_G, a}, {m.pw.bridge_Gp, a}, {m.pw.bridge_A, a}});
  if (x16) {
    // fp16(z) from the R projection; the code norm after the product
    gp.pro = PRO_COPY;
    gp.a = ws + P.act_r;
    gp.lda = r;
    set_post_scale(gp, g, W, SCALE_CODE, stz, stat_tiles(r), (float)r);
  } else if ((rc = set_scaled_a(gp, g, M, W, z, r, r, SCALE_CODE, stz, stat_tiles(r), (float)r, nullptr,
                                ws + P.act_r, stream))) {
    return rc;
  }
  gp.epi = EPI_STORE;
  gp.out = Pb;
  gp.ldo = 3 * a;
  if (x16) set_row_blocks(gp, g, M, 3 * a, r);
  HIP_TRY(launch_gemm_stream(gp, g.dtype, cus, stream));

  const float* Ppred = Pb;
  int shift = 1;
  if (pred_codes) {                                                    // predecessor override
    gp = gemm_base(P, ws, r, M);
    set_segments(gp, {{m.pw.bridge_G, a}, {m.pw.bridge_Gp, a}, {m.pw.bridge_A, a}});
    rc = set_scaled_a(gp, g, M, W, pred_codes, r, r, SCALE_ONE, nullptr, 0, (float)r, nullptr, ws + P.act_r, stream);
    if (rc) return rc;
    gp.epi = EPI_STORE;
    gp.out = P2;
    gp.ldo = 3 * a;
    HIP_TRY(launch_gemm_stream(gp, g.dtype, cus, stream));
    Ppred = P2;
    shift = 0;
  }

  // x += rho W_l (g * m), rho from the same statistics of x
  gp = gemm_base(P, ws, a, M);
  set_segments(gp, {{m.pw.layer[layer].W_l, H}});
  if (M <= gemm_stream_fused_rows()) {
    gp.pro = PRO_BRIDGE_MSG;
    gp.P = Pb;
    gp.Ppred = Ppred;
    gp.bias = wt.bridge_b;
    gp.a_dim = a;
    gp.pred_shift = shift;
  } else {
    ScaleParams sp;
    memset(&sp, 0, sizeof sp);
    sp.M = M;
    sp.K = a;
    sp.W = W;
    sp.P = Pb;
    sp.Ppred = Ppred;
    sp.bias = wt.bridge_b;
    sp.pred_shift = shift;
    sp.act = ws + P.act_m;
    sp.ld_act = a;
    HIP_TRY(launch_bridge_msg(sp, g.dtype, stream));
    gp.pro = PRO_COPY;
    gp.a = ws + P.act_m;
    gp.lda = a;
  }
  gp.W = W;
  gp.scale_mode = SCALE_RHO;
  gp.stats_in = xst;
  gp.stats_tiles = xst_tiles;
  gp.stats_ld = kMaxRows;
  gp.scale_n = (float)H;
  gp.epi = EPI_ADD_ROWSCALE;
  gp.out = x;
  gp.ldo = H;
  gp.stats_out = st_out;
  gp.stats_out_ld = kMaxRows;
  if (copy_out) set_copy(gp, copy_out, H, false, copy_gain, kRawCopy);   // the next layer's operand
  if (x16) set_row_blocks(gp, g, M, H, a);
  HIP_TRY(launch_gemm_stream(gp, g.dtype, cus, stream));
  return DSPINE_OK;
}

// checks of a call over B requests of width W, workspace aside
int check_call_args(const dspine_model* model, int B, int W, const int32_t* anchor_ids) {
  if (!model || !anchor_ids) return fail(DSPINE_E_ARG, "NULL argument");
  if (B < 1 || B > DSPINE_MAX_BATCH) return fail(DSPINE_E_UNSUPPORTED, "B = %d not in 1..%d", B, DSPINE_MAX_BATCH);
  if (W < DSPINE_MIN_WIDTH || W > DSPINE_MAX_WIDTH)
    return fail(DSPINE_E_UNSUPPORTED, "W = %d not in %d..%d", W, DSPINE_MIN_WIDTH, DSPINE_MAX_WIDTH);
  for (int b = 0; b < B; ++b)
    if (anchor_ids[b] < 0 || anchor_ids[b] >= model->g.vocab)
      return fail(DSPINE_E_ARG, "anchor_ids[%d] = %d outside [0, %d)", b, anchor_ids[b], model->g.vocab);
  return DSPINE_OK;
}
int check_call(const dspine_model* model, int B, int W, const int32_t* anchor_ids, const void* ws,
               size_t ws_bytes, size_t* need) {
  int rc = check_call_args(model, B, W, anchor_ids);
  if (rc) return rc;
  *need = make_plan(model->g, B, W, 0).total;
  if (!ws || !aligned16(ws)) return fail(DSPINE_E_ARG, "workspace NULL or not 16-byte aligned");
  if (ws_bytes < *need) return fail(DSPINE_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, *need);
  return DSPINE_OK;
}
// last check before the first launch of a call
int check_packed(const dspine_model* model) {
  if (!model->packed) return fail(DSPINE_E_STATE, "weights not packed: call dspine_pack_weights first");
  return DSPINE_OK;
}
}  // namespace

int dspine_bridge(const dspine_model* model, int layer, int B, int W, float* x, const int32_t* anchor_ids,
                  const float* pred_codes, void* workspace, size_t workspace_bytes, dspine_stream_t stream) {
  size_t need = 0;
  int rc = check_call(model, B, W, anchor_ids, workspace, workspace_bytes, &need);
  if (rc) return rc;
  if (model->g.code_dim == 0) return fail(DSPINE_E_UNSUPPORTED, "bridge: the geometry has no bridge (code_dim 0)");
  if (layer < 0 || layer >= model->g.n_layers) return fail(DSPINE_E_ARG, "bridge: layer %d", layer);
  if (!x || !aligned16(x)) return fail(DSPINE_E_ARG, "bridge: x NULL or unaligned");
  if (pred_codes && !aligned16(pred_codes)) return fail(DSPINE_E_ARG, "bridge: pred_codes unaligned");
  if ((rc = check_packed(model))) return rc;
  const Plan P = make_plan(model->g, B, W, 0);
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* st1 = reinterpret_cast<float*>(ws + P.st1);
  RowParams rp;
  memset(&rp, 0, sizeof rp);
  rp.M = B * W;
  rp.H = model->g.hidden;
  rp.x = x;
  rp.stats = st1;
  HIP_TRY(launch_rowstats(rp, s));
  rc = run_bridge(*model, layer, B, W, x, st1, 1, reinterpret_cast<float*>(ws + P.st0), anchor_ids, pred_codes, ws,
                  P, num_cus(), s);
  return rc ? rc : ok();
}

// -----------------------------------------------------------------------------
// a4-a12
// -----------------------------------------------------------------------------
// checks shared by the forward calls and the propose call, workspace aside
static int check_forward_args(const dspine_model* model, int B, int W, const dspine_ctx* ctx,
                              const int32_t* anchor_ids, const float* out) {
  int rc = check_call_args(model, B, W, anchor_ids);
  if (rc) return rc;
  if (!ctx) return fail(DSPINE_E_ARG, "forward: ctx NULL");
  if (!out || !aligned16(out)) return fail(DSPINE_E_ARG, "forward: out NULL or unaligned");
  for (int b = 0; b < B; ++b)
    if ((rc = check_ctx_rings(*model, ctx[b], b, ctx[b].frontier))) return rc;
  return DSPINE_OK;
}
static int check_forward(const dspine_model* model, int B, int W, const dspine_ctx* ctx, const int32_t* anchor_ids,
                         const float* out, void* workspace, size_t workspace_bytes) {
  size_t need = 0;
  int rc = check_call(model, B, W, anchor_ids, workspace, workspace_bytes, &need);
  if (rc) return rc;
  if (!ctx) return fail(DSPINE_E_ARG, "forward: ctx NULL");
  if (!out || !aligned16(out)) return fail(DSPINE_E_ARG, "forward: out NULL or unaligned");
  for (int b = 0; b < B; ++b)
    if ((rc = check_ctx_rings(*model, ctx[b], b, ctx[b].frontier))) return rc;
  return DSPINE_OK;
}

// DFlash2 convolution of one branch (side 0 "prepare" or side 1 "finish")
static ConvParams conv_params(const dspine_geometry& g, int M, int W, const float* delta, const void* base) {
  ConvParams cp;
  memset(&cp, 0, sizeof cp);
  cp.M = M;
  cp.W = W;
  cp.H = g.hidden;
  cp.cg = g.conv_group;
  cp.G = g.hidden / g.conv_group;
  cp.delta = delta;
  cp.base = base;
  cp.eps = g.eps;
  return cp;
}

// The forward's launches (arguments already checked).  save_u, when given,
// receives the last layer's state before its bridge write [B*W, H].
// want_head_act: also leave fp16(out) in the act_h buffer when the last
// bridge can form it (*head_act_ready then says it did).
static int run_forward(const dspine_model* model, int B, int W, const dspine_ctx* ctx, const int32_t* anchor_ids,
                       float* out, void* workspace, hipStream_t stream, float* save_u, bool want_head_act = false,
                       bool* head_act_ready = nullptr) {
  int rc = DSPINE_OK;
  const dspine_geometry& g = model->g;
  const dspine_weights& wt = model->w;
  char* ws = static_cast<char*>(workspace);
  const int M = B * W, H = g.hidden, D = g.head_dim;
  const int qd = g.n_q_heads * D, kvd = g.n_kv_heads * D;
  const Plan P = make_plan(g, B, W, 0);
  const int cus = num_cus();
  float* x = reinterpret_cast<float*>(ws + P.x);
  void* act_q = ws + P.act_q;
  void* act_f = ws + P.act_f;
  float* qkv = reinterpret_cast<float*>(ws + P.qkv);
  float* rope = reinterpret_cast<float*>(ws + P.rope);
  float* st0 = reinterpret_cast<float*>(ws + P.st0);
  float* st1 = reinterpret_cast<float*>(ws + P.st1);
  const int tH = stat_tiles(H);
  const bool conv = g.conv_group > 0;
  const int G4 = conv ? 4 * (H / g.conv_group) : 0;
  float* conv_da = reinterpret_cast<float*>(ws + P.conv_da);
  float* conv_dm = reinterpret_cast<float*>(ws + P.conv_dm);
  float* o_tmp = reinterpret_cast<float*>(ws + P.o_tmp);

  // a4: x, its row statistics (one list) and the rotation table of F_b + i
  RowParams rp;
  memset(&rp, 0, sizeof rp);
  rp.M = M;
  rp.W = W;
  rp.H = H;
  rp.x_out = x;
  rp.stats = st1;
  rp.embed = wt.embed;
  for (int b = 0; b < B; ++b) {
    rp.anchor[b] = anchor_ids[b];
    rp.F[b] = ctx[b].frontier;
  }
  rp.mask_id = g.mask_token_id;
  rp.rope = rope;
  rp.head_dim = D;
  rp.rope_theta = g.rope_theta;
  // Blocks whose q|k|v takes a pre-scaled operand (16 rows and fewer, and
  // more than 32) get it from the kernel that writes x: the embedding for
  // layer 0, the fused bridge (up to 32 rows) for the layers after it.
  // act_ready: act_h holds this layer's operand.
  const bool fold_norm = !conv && (prescale_pays(g, M, H) || M > gemm_stream_fused_rows());
  bool act_ready = false;
  // Blocks of more than 32 rows of a BF16 model (no convolution): after
  // layer 0, every norm is applied after the product that consumes it (a
  // per-row factor of the contraction), to raw rows times the norm's gain
  // that the GEMM writing those rows stores beside them as fp16 (scaled by
  // 2^-8), so no pre-scale kernel runs.  copy_ready: act_h holds that copy
  // of x g_in for this layer.
  const bool post = !conv && g.dtype == DSPINE_BF16 && M > gemm_stream_fused_rows();
  // 16 rows and fewer (BF16): the bridge stores the same kind of copy for
  // the layers after the first, instead of waiting for every column to form
  // the next norm itself, and O stores y g_post for gate/up, which then reads
  // 16-bit rows instead of forming the norm from fp32 ones (27B B=1 gate/up
  // 384 -> 345 us per forward, O 85 -> 87)
  const bool copy16 = !conv && prescale_pays(g, M, H);
  bool copy_ready = false;
  if (head_act_ready) *head_act_ready = false;
  if (fold_norm) {
    rp.act = ws + P.act_h;
    rp.gain = wt.layer[0].g_in;
    rp.eps = g.eps;
    act_ready = true;
  }
  {
    ProfScope ps(DSPINE_PROF_NORM, stream);
    HIP_TRY(launch_embed(rp, g.dtype, stream));
  }
  // statistics of the current x: list and its length
  const float* xst = st1;
  int xst_tiles = 1;

  for (int l = 0; l < g.n_layers; ++l) {
    const dspine_layer_weights& Lw = wt.layer[l];
    const dspine_layer_weights& Pw = model->pw.layer[l];
    // a5: q | k | v projections of n = input_norm(x) (norm formed in the GEMM)
    GemmParams gp = gemm_base(P, ws, H, M);
    if (conv) {
      // DFlash2: delta of the attention branch from n = input_norm(x), then
      // the prepared input Conv_0(n) as the projections' operand
      GemmParams dg = gemm_base(P, ws, H, M);
      set_segments(dg, {{Pw.attn_conv_w, G4}});
      if ((rc = set_scaled_a(dg, g, M, W, x, H, H, SCALE_RMSNORM, xst, xst_tiles, (float)H, Lw.g_in, ws + P.act_h,
                             stream)))
        return rc;
      dg.epi = EPI_STORE;
      dg.out = conv_da;
      dg.ldo = G4;
      ProfScope ps(DSPINE_PROF_CONV, stream);
      HIP_TRY(launch_gemm_stream(dg, g.dtype, cus, stream));
      ConvParams cp = conv_params(g, M, W, conv_da, Lw.attn_conv_base);
      cp.x = x;
      cp.stats = xst;
      cp.lists = xst_tiles;
      cp.ld = kMaxRows;
      cp.gain = Lw.g_in;
      cp.act = ws + P.act_h;
      HIP_TRY(launch_conv_prepare(cp, g.dtype, stream));
    }
    set_segments(gp, {{Pw.wq, qd}, {Pw.wk, kvd}, {Pw.wv, kvd}});
    if (conv) {
      gp.pro = PRO_COPY;
      gp.a = ws + P.act_h;
      gp.lda = H;
    } else if (act_ready) {
      // the input norm as a pre-scaled operand, already formed by the kernel
      // that wrote x: the q|k|v GEMM streams it into LDS in long stages
      gp.pro = PRO_COPY;
      gp.a = ws + P.act_h;
      gp.lda = H;
    } else if (copy_ready) {
      gp.pro = PRO_COPY;
      gp.a = ws + P.act_h;
      gp.lda = H;
      set_post_scale(gp, g, W, SCALE_RMSNORM, xst, xst_tiles, (float)H, kRawPost);
    } else if (prescale_pays(g, M, H)) {
      // the same operand from the pre-scale kernel (at B=1 the q|k|v GEMM
      // went 142 -> 103 us per forward with these kernels counted)
      ProfScope ps(DSPINE_PROF_NORM, stream);
      if ((rc = set_prescaled_a(gp, g, M, W, x, H, SCALE_RMSNORM, xst, xst_tiles, Lw.g_in, ws + P.act_h, stream)))
        return rc;
    } else if ((rc = set_scaled_a(gp, g, M, W, x, H, H, SCALE_RMSNORM, xst, xst_tiles, (float)H, Lw.g_in,
                                  ws + P.act_h, stream))) {
      return rc;
    }
    gp.epi = EPI_STORE;
    gp.out = qkv;
    gp.ldo = qd + 2 * kvd;
    if (post) set_row_blocks(gp, g, M, qd + 2 * kvd, H);
    {
      ProfScope ps(DSPINE_PROF_GEMM_QKV, stream);
      HIP_TRY(launch_gemm_stream(gp, g.dtype, cus, stream));
    }
    act_ready = false;                    // act_h is reused below
    copy_ready = false;

    // a6 (with the q/k head norm + RoPE of a5)
    AttnParams ap;
    memset(&ap, 0, sizeof ap);
    ap.B = B;
    ap.W = W;
    ap.nq = g.n_q_heads;
    ap.nkv = g.n_kv_heads;
    ap.M = M;
    ap.qkv = qkv;
    ap.ld_qkv = qd + 2 * kvd;
    ap.gq = Lw.gq;
    ap.gk = Lw.gk;
    ap.eps = g.eps;
    ap.rope = rope;
    ap.S = g.window[l];
    ap.causal = g.block_causal;
    // Key splits: enough workgroups to spread the reads over the CUs (about
    // 256, or more on long contexts, below) but at least 128 keys per split,
    // so that each of a workgroup's key sub-streams has a tile.
    int64_t max_ctx = 0, min_ctx = INT64_MAX;
    for (int b = 0; b < B; ++b) {
      ap.kring[b] = ctx[b].k_ring[l];
      ap.vring[b] = ctx[b].v_ring[l];
      ap.cap[b] = ctx[b].capacity[l];
      ap.F[b] = ctx[b].frontier;
      ap.lo0[b] = row0_lo(ctx[b].frontier, g.window[l]);
      max_ctx = std::max(max_ctx, ap.F[b] - ap.lo0[b]);
      min_ctx = std::min(min_ctx, ap.F[b] - ap.lo0[b]);
    }
    // Long contexts: splits of up to 8192 keys when the requests' contexts
    // are within a factor of two (each wave then holds like work, and fewer
    // waves pay fewer prologues: 35B-style full layer at B=8 in one wave of
    // 256 workgroups, attention 512 -> 483 us per forward), else of 2048 so
    // that the short requests' workgroups fill in behind the long ones
    const int64_t per_split = 2 * min_ctx >= max_ctx ? 8192 : 2048;
    const int64_t spread = std::max(ceil_div(256, (int64_t)B * g.n_kv_heads), ceil_div(max_ctx, per_split));
    ap.nsplit = (int)std::max<int64_t>(1, std::min<int64_t>({spread, ceil_div(max_ctx, 128), (int64_t)kMaxSplit}));
    {
      // One workgroup fills a CU (its LDS), so a grid of several waves runs
      // a whole number of them: the split count goes to the nearest multiple
      // of the splits that fill one wave (35B-style full layer at B=8: 17 ->
      // 16 splits, 1088 -> 1024 workgroups, instead of a quarter-full fifth
      // wave)
      const int64_t heads = (int64_t)B * g.n_kv_heads;
      const int64_t per = cus % heads == 0 ? cus / heads : 0;
      if (per > 0 && ap.nsplit > per) {
        int64_t n = (ap.nsplit + per / 2) / per * per;
        while (n > kMaxSplit || n > ceil_div(max_ctx, 128)) n -= per;
        if (n >= per) ap.nsplit = (int)n;
      }
    }
    int64_t kv_bytes = 0;
    for (int b = 0; b < B; ++b) {
      const int64_t nctx = ap.F[b] - ap.lo0[b];
      ap.kps[b] = (int32_t)(ceil_div(ceil_div(nctx, ap.nsplit), 32) * 32);
      kv_bytes += nctx * g.n_kv_heads * D * 4;
    }
    // a layer's context K/V is read once: non-temporal loads keep it from
    // evicting reused lines when it is large (27B B=8: 1.3 % faster, 35B
    // B=8 2.5 %); at 27B B=1 (8.4 MB) the cached loads measured faster
    ap.kv_nt = kv_bytes > ((int64_t)16 << 20) ? 1 : 0;
    ap.out = act_q;
    ap.ld_out = qd;
    ap.partials = reinterpret_cast<float*>(ws + P.attn_part);
    {
      ProfScope ps(DSPINE_PROF_ATTENTION, stream);
      HIP_TRY(launch_attention(ap, g.dtype, D, stream));
    }

    // a7: y = x + W_o a, with the row statistics of y
    gp = gemm_base(P, ws, qd, M);
    set_segments(gp, {{Pw.wo, H}});
    gp.pro = PRO_COPY;
    gp.a = act_q;
    gp.lda = qd;
    gp.epi = conv ? EPI_STORE : EPI_ADD;
    gp.out = conv ? o_tmp : x;
    gp.ldo = H;
    gp.stats_out = conv ? nullptr : st0;
    gp.stats_out_ld = kMaxRows;
    if (post || copy16) set_copy(gp, ws + P.act_h, H, false, Lw.g_post, kRawCopy);     // y g_post for gate/up
    if (post) set_row_blocks(gp, g, M, H, qd);
    {
      ProfScope ps(DSPINE_PROF_GEMM_O, stream);
      HIP_TRY(launch_gemm_stream(gp, g.dtype, cus, stream));
    }
    int yst_tiles = tH;                   // statistics lists of y in st0
    if (conv) {
      // y = x + Conv_1(W_o a) with the prepare's delta; one statistics list
      ConvParams cp = conv_params(g, M, W, conv_da, Lw.attn_conv_base);
      cp.o = o_tmp;
      cp.x_out = x;
      cp.stats_out = st0;
      ProfScope ps(DSPINE_PROF_CONV, stream);
      HIP_TRY(launch_conv_finish(cp, g.dtype, stream));
      yst_tiles = 1;
    }

    // a8: x = y + W_down(SiLU(W_gate m) * W_up m), m = post_norm(y) formed
    // in the gate/up GEMM
    gp = gemm_base(P, ws, H, M);
    gp.seg_ptr[0] = Pw.w_gate;
    gp.seg_ptr[1] = Pw.w_up;
    gp.nseg = 2;
    gp.interleave = 1;
    gp.nblk = 2 * (g.ffn / 16);
    if (conv) {
      // DFlash2: delta of the MLP branch from m = post_norm(y), then Conv_0(m)
      GemmParams dg = gemm_base(P, ws, H, M);
      set_segments(dg, {{Pw.mlp_conv_w, G4}});
      if ((rc = set_scaled_a(dg, g, M, W, x, H, H, SCALE_RMSNORM, st0, yst_tiles, (float)H, Lw.g_post,
                             ws + P.act_h, stream)))
        return rc;
      dg.epi = EPI_STORE;
      dg.out = conv_dm;
      dg.ldo = G4;
      ProfScope ps(DSPINE_PROF_CONV, stream);
      HIP_TRY(launch_gemm_stream(dg, g.dtype, cus, stream));
      ConvParams cp = conv_params(g, M, W, conv_dm, Lw.mlp_conv_base);
      cp.x = x;
      cp.stats = st0;
      cp.lists = yst_tiles;
      cp.ld = kMaxRows;
      cp.gain = Lw.g_post;
      cp.act = ws + P.act_h;
      HIP_TRY(launch_conv_prepare(cp, g.dtype, stream));
      gp.pro = PRO_COPY;
      gp.a = ws + P.act_h;
      gp.lda = H;
    } else if (post || copy16) {
      gp.pro = PRO_COPY;
      gp.a = ws + P.act_h;
      gp.lda = H;
      set_post_scale(gp, g, W, SCALE_RMSNORM, st0, tH, (float)H, kRawPost);
    } else if ((rc = set_scaled_a(gp, g, M, W, x, H, H, SCALE_RMSNORM, st0, tH, (float)H, Lw.g_post, ws + P.act_h,
                                  stream))) {
      return rc;
    }
    // the SwiGLU hidden is the one operand no norm bounds: a BF16 model keeps
    // it in bf16 (fp32's range) and the down projection multiplies bf16 x bf16
    gp.epi = EPI_SWIGLU;
    gp.out_act = act_f;
    gp.ld_act = g.ffn;
    gp.out_act_bf16 = g.dtype == DSPINE_BF16;
    {
      ProfScope ps(DSPINE_PROF_GEMM_GATE_UP, stream);
      HIP_TRY(launch_gemm_stream(gp, g.dtype, cus, stream));
    }
    gp = gemm_base(P, ws, g.ffn, M);
    set_segments(gp, {{Pw.w_down, H}});
    gp.pro = PRO_COPY;
    gp.a = act_f;
    gp.a_bf16 = g.dtype == DSPINE_BF16;
    gp.lda = g.ffn;
    gp.epi = conv ? EPI_STORE : EPI_ADD;
    gp.out = conv ? o_tmp : x;
    gp.ldo = H;
    gp.stats_out = conv ? nullptr : st1;
    gp.stats_out_ld = kMaxRows;
    const bool more = l + 1 < g.n_layers;
    if (post && g.code_dim > 0) set_copy(gp, ws + P.act_h, H, false, nullptr, kRawCopy);   // x for R
    else if (post && more) set_copy(gp, ws + P.act_h, H, false, wt.layer[l + 1].g_in, kRawCopy);
    {
      ProfScope ps(DSPINE_PROF_GEMM_DOWN, stream);
      HIP_TRY(launch_gemm_stream(gp, g.dtype, cus, stream));
    }
    xst = st1;
    xst_tiles = tH;
    copy_ready = post && g.code_dim == 0 && more;
    if (conv) {
      // x_next = y + Conv_1(z) with the MLP prepare's delta
      ConvParams cp = conv_params(g, M, W, conv_dm, Lw.mlp_conv_base);
      cp.o = o_tmp;
      cp.x_out = x;
      cp.stats_out = st1;
      ProfScope ps(DSPINE_PROF_CONV, stream);
      HIP_TRY(launch_conv_finish(cp, g.dtype, stream));
      xst_tiles = 1;
    }

    if (save_u && l == g.n_layers - 1)
      HIP_TRY(hipMemcpyAsync(save_u, x, sizeof(float) * (size_t)M * H, hipMemcpyDeviceToDevice, stream));
    // a9-a11 (statistics of the written rows go to st0); the fused bridge
    // also forms the next norm: the next layer's q|k|v operand, or after the
    // last layer the final norm (a12) into `out` (and fp16(out) on request)
    if (g.code_dim > 0) {
      ProfScope ps(DSPINE_PROF_BRIDGE, stream);
      const bool last = l == g.n_layers - 1;
      bool folded = false;
      if (last)
        rc = run_bridge(*model, l, B, W, x, xst, xst_tiles, st0, anchor_ids, nullptr, ws, P, cus, stream, wt.g_final,
                        want_head_act ? ws + P.act_h : nullptr, out, &folded, post ? ws + P.act_h : nullptr);
      else if (post)
        rc = run_bridge(*model, l, B, W, x, xst, xst_tiles, st0, anchor_ids, nullptr, ws, P, cus, stream, nullptr,
                        nullptr, nullptr, nullptr, ws + P.act_h, ws + P.act_h, wt.layer[l + 1].g_in);
      else if (copy16)
        // the next layer's operand as a raw copy: its norm is applied after
        // the q|k|v product, so the bridge does not wait for every column
        rc = run_bridge(*model, l, B, W, x, xst, xst_tiles, st0, anchor_ids, nullptr, ws, P, cus, stream, nullptr,
                        nullptr, nullptr, nullptr, nullptr, ws + P.act_h, wt.layer[l + 1].g_in);
      else
        rc = run_bridge(*model, l, B, W, x, xst, xst_tiles, st0, anchor_ids, nullptr, ws, P, cus, stream);
      if (rc) return rc;
      xst = st0;                          // the write GEMM's lists, one per 64 columns
      xst_tiles = tH;
      if (last && folded) {
        if (head_act_ready) *head_act_ready = want_head_act;
        return DSPINE_OK;
      }
      act_ready = folded;
      copy_ready = (post || copy16) && !last;
    }
  }
  // a12
  RowParams fp;
  memset(&fp, 0, sizeof fp);
  fp.M = M;
  fp.H = H;
  fp.x = x;
  fp.f32_out = out;
  fp.gain = wt.g_final;
  fp.eps = g.eps;
  fp.lists = xst;                         // the same bits as the fused bridge's folded norm
  fp.nlists = xst_tiles;
  fp.ld = kMaxRows;
  {
    ProfScope ps(DSPINE_PROF_NORM, stream);
    HIP_TRY(launch_rmsnorm(fp, g.dtype, true, stream));
  }
  return DSPINE_OK;
}

int dspine_draft_forward(const dspine_model* model, int B, int W, const dspine_ctx* ctx, const int32_t* anchor_ids,
                         float* out, void* workspace, size_t workspace_bytes, dspine_stream_t stream) {
  int rc = check_forward(model, B, W, ctx, anchor_ids, out, workspace, workspace_bytes);
  if (rc) return rc;
  if ((rc = check_packed(model))) return rc;
  rc = run_forward(model, B, W, ctx, anchor_ids, out, workspace, reinterpret_cast<hipStream_t>(stream), nullptr);
  return rc ? rc : ok();
}

// -----------------------------------------------------------------------------
// allocation-free forward: the workspace is a static device array
// -----------------------------------------------------------------------------
// One copy of the array lives on every device the library runs on, until the
// process ends.  On the host, `scratch` only names the symbol: its device
// address on the current device comes from hipGetSymbolAddress, and only that
// address is ever handed to a kernel.
static __device__ __align__(256) char scratch[DSPINE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// 32-bit words at the start of every workspace plan that hold counters
size_t counter_words() {
  dspine_geometry g0;
  memset(&g0, 0, sizeof g0);
  return make_plan(g0, 1, 2, 0).counters_end / sizeof(uint32_t);
}

// Device address of the current device's copy of `scratch`.  The first call
// on a device looks it up and clears the counters (stream-K tiles, fused
// bridge hand-offs; at the start of every plan) on `stream`; every forward
// leaves them at zero again.
int scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(DSPINE_E_UNSUPPORTED, "device index %d not below %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p || ((uintptr_t)p & 255u)) return fail(DSPINE_E_HIP, "static scratch: bad device address");
    HIP_TRY(launch_zero_words(p, counter_words(), stream));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSPINE_OK;
}
}  // namespace

int dspine_draft_forward_noalloc(const dspine_model* model, int B, int W, const dspine_ctx* ctx,
                                 const int32_t* anchor_ids, float* out, dspine_stream_t stream) {
  int rc = check_forward_args(model, B, W, ctx, anchor_ids, out);
  if (rc) return rc;
  const size_t need = make_plan(model->g, B, W, 0).total;
  if (need > DSPINE_NOALLOC_SCRATCH_BYTES)
    return fail(DSPINE_E_WORKSPACE, "forward_noalloc: B = %d, W = %d needs %zu bytes of scratch, more than the "
                "static %zu", B, W, need, (size_t)DSPINE_NOALLOC_SCRATCH_BYTES);
  if ((rc = check_packed(model))) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((rc = scratch_for_current_device(s, &ws))) return rc;
  rc = run_forward(model, B, W, ctx, anchor_ids, out, ws, s, nullptr);
  return rc ? rc : ok();
}

// -----------------------------------------------------------------------------
// proposal tail
// -----------------------------------------------------------------------------
namespace {
struct ProposePlan {
  size_t u, scores, part_v, part_i, codes, Pc, msg, Y, retr, resc, total;
};
ProposePlan make_propose_plan(const dspine_geometry& g, int B, int W, int K) {
  ProposePlan p{};
  const size_t eb = act_bytes(g);
  const int64_t M = (int64_t)B * W, Mp = (int64_t)B * (W - 1);
  const int64_t Mc = Mp * K + kMaxRows;      // the GEMMs may read a padded last row block
  const int r = std::max(g.code_dim, 1), a = std::max(g.msg_dim, 1);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  p.u = take(4 * (size_t)M * g.hidden);
  p.scores = take(4 * (size_t)M * g.vocab);
  const size_t parts = std::max(topk_partial_entries((int)Mp, g.vocab), retrieve_partial_entries((int)Mp, g.vocab));
  p.part_v = take(4 * parts);
  p.part_i = take(4 * parts);
  p.retr = take(4 * (size_t)Mp * kMaxRetrieve);
  p.resc = take(4 * (size_t)Mp * kMaxRetrieve);
  p.codes = take(eb * Mc * r);
  p.Pc = take(4 * Mc * 2 * a);
  p.msg = take(eb * Mc * a);
  p.Y = take(4 * Mc * g.hidden);
  p.total = off;
  return p;
}
// tiles of the head GEMM must fit its tile counters
bool head_fits(const dspine_geometry& g) {
  return (int64_t)g.vocab / 16 <= 4LL * kMaxTiles && g.vocab <= topk_max_vocab();
}
}  // namespace

size_t dspine_propose_workspace_bytes(const dspine_model* model, int max_batch, int max_width, int topk) {
  if (!model || max_batch < 1 || max_batch > DSPINE_MAX_BATCH || max_width < DSPINE_MIN_WIDTH ||
      max_width > DSPINE_MAX_WIDTH || topk < 1 || topk > DSPINE_MAX_TOPK || !model->w.lm_head) {
    fail(DSPINE_E_ARG, "propose_workspace_bytes: bad argument or no lm_head");
    return 0;
  }
  return make_propose_plan(model->g, max_batch, max_width, topk).total;
}

int dspine_draft_propose(const dspine_model* model, int B, int W, const dspine_ctx* ctx, const int32_t* anchor_ids,
                         float* out, const dspine_proposal* prop, void* workspace, size_t workspace_bytes,
                         void* propose_ws, size_t propose_ws_bytes, dspine_stream_t stream_) {
  int rc = check_forward(model, B, W, ctx, anchor_ids, out, workspace, workspace_bytes);
  if (rc) return rc;
  const dspine_geometry& g = model->g;
  if (g.code_dim == 0) return fail(DSPINE_E_UNSUPPORTED, "propose: the refinement needs the bridge (code_dim 0)");
  if (!model->w.lm_head) return fail(DSPINE_E_UNSUPPORTED, "propose: the model has no lm_head");
  if (g.hidden > propose_max_hidden())
    return fail(DSPINE_E_UNSUPPORTED, "propose: hidden %d > %d", g.hidden, propose_max_hidden());
  if (!head_fits(g)) return fail(DSPINE_E_UNSUPPORTED, "propose: vocab %d too large for the head GEMM", g.vocab);
  if (!prop) return fail(DSPINE_E_ARG, "propose: prop NULL");
  const int K = prop->topk;
  if (K < 1 || K > DSPINE_MAX_TOPK || K > g.vocab)
    return fail(DSPINE_E_ARG, "propose: topk %d not in 1..%d (and <= vocab)", K, DSPINE_MAX_TOPK);
  if (prop->walk != DSPINE_WALK_GREEDY && prop->walk != DSPINE_WALK_SAMPLED)
    return fail(DSPINE_E_ARG, "propose: walk %d", prop->walk);
  const int R = prop->retrieve;
  if (R != 0) {
    if (R < K || R > DSPINE_MAX_RETRIEVE || R > g.vocab)
      return fail(DSPINE_E_ARG, "propose: retrieve %d not in K = %d..%d (and <= vocab)", R, K, DSPINE_MAX_RETRIEVE);
    if (g.dtype != DSPINE_BF16)
      return fail(DSPINE_E_UNSUPPORTED, "propose: the FP8 retrieval needs a BF16 model (its head's FP8 copy)");
    if ((prop->retrieved && !aligned16(prop->retrieved)) || (prop->rescored && !aligned16(prop->rescored)))
      return fail(DSPINE_E_ARG, "propose: retrieved or rescored unaligned");
  }
  if (prop->walk == DSPINE_WALK_SAMPLED) {
    if (!(prop->temperature > 0.0) || !std::isfinite(prop->temperature))
      return fail(DSPINE_E_ARG, "propose: temperature must be finite and > 0");
    if (!prop->uniforms || ((uintptr_t)prop->uniforms & 7u)) return fail(DSPINE_E_ARG, "propose: uniforms NULL or unaligned");
    if (!prop->q) return fail(DSPINE_E_ARG, "propose: the sampled walk needs q (the choices' probabilities)");
  }
  if (!prop->cand || !prop->cand_scores || !prop->table || !prop->choice || !prop->tokens)
    return fail(DSPINE_E_ARG, "propose: an output pointer is NULL");
  if ((prop->scores && !aligned16(prop->scores)) || ((uintptr_t)prop->q & 7u))
    return fail(DSPINE_E_ARG, "propose: scores or q unaligned");
  const ProposePlan PP = make_propose_plan(g, B, W, K);
  if (!propose_ws || !aligned16(propose_ws)) return fail(DSPINE_E_ARG, "propose: propose workspace NULL or unaligned");
  if (propose_ws_bytes < PP.total)
    return fail(DSPINE_E_WORKSPACE, "propose: propose workspace %zu bytes < %zu needed", propose_ws_bytes, PP.total);
  if ((rc = check_packed(model))) return rc;
  if (R != 0 && !model->head_fp8) return fail(DSPINE_E_STATE, "propose: the model has no FP8 head copy");

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  char* pws = static_cast<char*>(propose_ws);
  char* ws = static_cast<char*>(workspace);
  const int M = B * W, H = g.hidden, V = g.vocab, r = g.code_dim, a = g.msg_dim, L = g.n_layers;
  const int Mc = B * (W - 1) * K;
  const size_t eb = act_bytes(g);
  const int cus = num_cus();
  const Plan P = make_plan(g, B, W, 0);
  float* u = reinterpret_cast<float*>(pws + PP.u);
  float* scores = prop->scores ? prop->scores : reinterpret_cast<float*>(pws + PP.scores);

  // the head's fp16 operand (h itself) comes from the last bridge when it can
  const bool head_prescaled = R != 0 || prescale_pays(g, M, H);
  bool head_act_ready = false;
  if ((rc = run_forward(model, B, W, ctx, anchor_ids, out, workspace, stream, u, head_prescaled, &head_act_ready)))
    return rc;

  // head scores E h of every row (h = the forward's final-normed output), or
  // their FP8 approximation s_v (q_v . h); one timed span holds the operand
  // conversion (when there is one) and the score GEMM
  GemmParams gp = gemm_base(P, ws, H, M);
  {
    ProfScope head_scope(DSPINE_PROF_HEAD, stream);
    if (R != 0) {
      set_segments(gp, {{model->head_fp8, V}});
      gp.w_fp8 = 1;
      gp.col_scale = model->head_fp8_scale;
    } else {
      set_segments(gp, {{model->pw.lm_head, V}});
    }
    if (head_act_ready) {
      gp.pro = PRO_COPY;                  // fp16(h), written by the last bridge
      gp.a = ws + P.act_h;
      gp.lda = H;
    } else if (head_prescaled) {
      // h converted once to fp16 rows (the FP8 GEMM's copy prologue, and the
      // 16-row BF16 head's direct-to-LDS stages)
      if ((rc = set_prescaled_a(gp, g, M, W, out, H, SCALE_ONE, nullptr, 0, nullptr, ws + P.act_h, stream))) return rc;
    } else if ((rc = set_scaled_a(gp, g, M, W, out, H, H, SCALE_ONE, nullptr, 0, (float)H, nullptr, ws + P.act_h,
                                  stream))) {
      return rc;
    }
    gp.epi = EPI_STORE;
    gp.out = scores;
    gp.ldo = V;
    HIP_TRY(launch_gemm_stream(gp, g.dtype, cus, stream));
  }
  ProfScope tail_scope(DSPINE_PROF_TAIL, stream);

  ProposeParams pp;
  memset(&pp, 0, sizeof pp);
  pp.B = B;
  pp.W = W;
  pp.K = K;
  pp.vocab = V;
  pp.H = H;
  pp.r = r;
  pp.a = a;
  pp.walk = prop->walk;
  pp.temperature = prop->temperature;
  pp.eps = g.eps;
  pp.code_scale = sqrtf((float)r);
  for (int b = 0; b < B; ++b) pp.anchor[b] = anchor_ids[b];
  pp.scores = scores;
  pp.part_v = reinterpret_cast<float*>(pws + PP.part_v);
  pp.part_i = reinterpret_cast<int32_t*>(pws + PP.part_i);
  pp.cand = prop->cand;
  pp.cand_scores = prop->cand_scores;
  pp.codebook = model->w.codebook;
  pp.codes = pws + PP.codes;
  pp.P_own = reinterpret_cast<const float*>(ws + P.P);
  pp.P_cand = reinterpret_cast<const float*>(pws + PP.Pc);
  pp.bias = model->w.bridge_b;
  pp.msg = pws + PP.msg;
  pp.u = u;
  pp.Y = reinterpret_cast<const float*>(pws + PP.Y);
  pp.g_final = model->w.g_final;
  pp.head = model->w.lm_head;             // row-major: the candidates' rows are gathered
  pp.table = prop->table;
  pp.uniforms = prop->uniforms;
  pp.choice = prop->choice;
  pp.tokens = prop->tokens;
  pp.q = prop->q;
  if (R != 0) {
    pp.R = R;
    pp.retrieved = prop->retrieved ? prop->retrieved : reinterpret_cast<int32_t*>(pws + PP.retr);
    pp.rescored = prop->rescored ? prop->rescored : reinterpret_cast<float*>(pws + PP.resc);
    pp.h = out;
    HIP_TRY(launch_retrieve(pp, stream));
  } else {
    HIP_TRY(launch_topk(pp, stream));
  }
  HIP_TRY(launch_cand_codes(pp, g.dtype, stream));

  // [G_p; A] of the candidate codes, then W_l of their messages
  float* Pc = reinterpret_cast<float*>(pws + PP.Pc);
  float* Y = reinterpret_cast<float*>(pws + PP.Y);
  const bool tile = g.dtype == DSPINE_BF16 && gemm_tile_fits(a, r) && gemm_tile_fits(H, a);
  const int chunk = gemm_stream_row_tile(M);
  if (tile) {
    TileGemmParams tp;
    memset(&tp, 0, sizeof tp);
    tp.seg_ptr[0] = model->pw.bridge_Gp;
    tp.seg_ptr[1] = model->pw.bridge_A;
    tp.seg_rows0[0] = 0;
    tp.seg_rows0[1] = a;
    tp.seg_rows0[2] = 2 * a;
    tp.nseg = 2;
    tp.N = 2 * a;
    tp.K = r;
    tp.M = Mc;
    tp.pro = PRO_COPY;
    tp.a = pws + PP.codes;
    tp.lda = r;
    tp.out = Pc;
    tp.ldo = 2 * a;
    HIP_TRY(launch_gemm_tile(tp, g.dtype, cus, stream));
  } else {
    // chunks of at most the rows whose split partials the forward's
    // workspace holds (the streamed GEMM's row tile of M = B*W)
    for (int r0 = 0; r0 < Mc; r0 += chunk) {
      const int mr = std::min(chunk, Mc - r0);
      gp = gemm_base(P, ws, r, mr);
      set_segments(gp, {{model->pw.bridge_Gp, a}, {model->pw.bridge_A, a}});
      gp.pro = PRO_COPY;
      gp.a = pws + PP.codes + (size_t)r0 * r * eb;
      gp.lda = r;
      gp.epi = EPI_STORE;
      gp.out = Pc + (size_t)r0 * 2 * a;
      gp.ldo = 2 * a;
      HIP_TRY(launch_gemm_stream(gp, g.dtype, cus, stream));
    }
  }
  HIP_TRY(launch_cand_msg(pp, g.dtype, stream));
  if (tile) {
    TileGemmParams tp;
    memset(&tp, 0, sizeof tp);
    tp.seg_ptr[0] = model->pw.layer[L - 1].W_l;
    tp.seg_rows0[0] = 0;
    tp.seg_rows0[1] = H;
    tp.nseg = 1;
    tp.N = H;
    tp.K = a;
    tp.M = Mc;
    tp.pro = PRO_COPY;
    tp.a = pws + PP.msg;
    tp.lda = a;
    tp.out = Y;
    tp.ldo = H;
    HIP_TRY(launch_gemm_tile(tp, g.dtype, cus, stream));
  } else {
    for (int r0 = 0; r0 < Mc; r0 += chunk) {
      const int mr = std::min(chunk, Mc - r0);
      gp = gemm_base(P, ws, a, mr);
      set_segments(gp, {{model->pw.layer[L - 1].W_l, H}});
      gp.pro = PRO_COPY;
      gp.a = pws + PP.msg + (size_t)r0 * a * eb;
      gp.lda = a;
      gp.epi = EPI_STORE;
      gp.out = Y + (size_t)r0 * H;
      gp.ldo = H;
      HIP_TRY(launch_gemm_stream(gp, g.dtype, cus, stream));
    }
  }
  HIP_TRY(launch_cand_score(pp, g.dtype, stream));
  HIP_TRY(launch_walk(pp, stream));
  return ok();
}

int dspine_debug_visible(const dspine_model* model, int layer, int B, int W, const dspine_ctx* ctx,
                         int64_t* lo_hi, int32_t* first_slot, int32_t* n_block, dspine_stream_t stream) {
  if (!model || !ctx || !lo_hi || !first_slot || !n_block) return fail(DSPINE_E_ARG, "debug_visible: NULL argument");
  if (layer < 0 || layer >= model->g.n_layers) return fail(DSPINE_E_ARG, "debug_visible: layer %d", layer);
  if (B < 1 || B > DSPINE_MAX_BATCH || W < DSPINE_MIN_WIDTH || W > DSPINE_MAX_WIDTH)
    return fail(DSPINE_E_UNSUPPORTED, "debug_visible: B %d W %d", B, W);
  VisibleParams vp;
  memset(&vp, 0, sizeof vp);
  vp.B = B;
  vp.W = W;
  vp.S = model->g.window[layer];
  vp.causal = model->g.block_causal;
  for (int b = 0; b < B; ++b) {
    if (ctx[b].frontier < 0) return fail(DSPINE_E_STATE, "debug_visible: frontier < 0");
    vp.F[b] = ctx[b].frontier;
  }
  vp.lo_hi = lo_hi;
  vp.first_slot = first_slot;
  vp.n_block = n_block;
  HIP_TRY(launch_debug_visible(vp, reinterpret_cast<hipStream_t>(stream)));
  return ok();
}

}  // extern "C"
