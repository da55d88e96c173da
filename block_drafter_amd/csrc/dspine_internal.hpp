// Internal interfaces between the C ABI (dspine_api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "/root/repo/include/dspine.h"

namespace dspine {

enum { DT_F32 = DSPINE_F32, DT_BF16 = DSPINE_BF16 };
// A-operand prologues of the streamed GEMM
enum {
  PRO_COPY = 0,        // activations as stored (model operand type)
  PRO_GATHER = 1,      // bf16 target features gathered from several requests
  PRO_BRIDGE_MSG = 2,  // bridge gate * message from the [G; G_p; A] projections
  PRO_NORM = 3,        // fp32 rows x per-row scale x per-column gain
  PRO_SCALE = 4,       // fp32 rows x per-row scale
};
enum { EPI_STORE = 0, EPI_ADD = 1, EPI_SWIGLU = 2, EPI_ADD_ROWSCALE = 3 };
// per-row scale s[m] formed in the kernel from the sum S of squares of the
// row (a list of per-tile partial sums), over rows of width n:
// (the values are the mode numbers of row_scale in dspine_device.hpp)
enum {
  SCALE_NONE = 0,
  SCALE_RMSNORM = 1,   // 1 / sqrt(S / n + eps)              plain RMSNorm
  SCALE_RHO_INV = 2,   // 1 / (sqrt(S / n) + eps)            bridge read
  SCALE_CODE = 3,      // sqrt(r) / (sqrt(S) + eps); 1 at anchor rows (m % W == 0)
  SCALE_RHO = 4,       // sqrt(S / n)                        bridge write
  SCALE_ONE = 5,       // 1
};

constexpr int kMaxSeg = 32;        // weight segments of one streamed GEMM
constexpr int kMaxGrid = 512;      // workgroups of one streamed GEMM
constexpr int kMaxTiles = 8192;    // tile counters of one GEMM
constexpr int kMaxSplit = 32;      // key splits of one attention launch
constexpr int kMaxRows = 128;      // B*W rows of one forward

// ---------------------------------------------------------------------------
// streamed (skinny) GEMM: out[m, n] (op)= sum_k A[m, k] W[n, k]
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Kernel timing: while a profiling scope is open on this thread, each launch
// takes events to record at the kernel's own start (the first launch) and
// end (hipExtLaunchKernelGGL), so that a timed span holds no queueing before
// its first kernel.
// ---------------------------------------------------------------------------
struct LaunchTimer {
  hipEvent_t start, stop;
};
// the events for the next launch on this thread (either may be NULL); NULL
// when no profiling scope is open
const LaunchTimer* take_launch_timer();
#define DSPINE_LAUNCH(kernel, grid, block, smem, stream, ...)                                       \
  do {                                                                                              \
    const ::dspine::LaunchTimer* lt_ = ::dspine::take_launch_timer();                               \
    if (lt_) hipExtLaunchKernelGGL(kernel, grid, block, smem, stream, lt_->start, lt_->stop, 0, __VA_ARGS__); \
    else hipLaunchKernelGGL(kernel, grid, block, smem, stream, __VA_ARGS__);                        \
  } while (0)

struct GemmParams {
  // weights: the virtual N space is a list of segments (or gate/up pairs)
  const void* seg_ptr[kMaxSeg];   // each [rows_s, K] row-major, model dtype
  int32_t seg_blk0[kMaxSeg];      // first 16-row block of each segment
  int32_t nseg;
  int32_t interleave;             // 1: block vb -> segment vb&1, row block vb>>1
  int32_t nblk;                   // 16-row blocks in N
  int32_t K, M;
  // rows per row block (16 or 32), or 0: all M rows in one tile row.  Row
  // blocks run side by side (grid y), each with its own stream-K split:
  // small outputs of many rows get more independent tiles
  int32_t rb_rows;
  // A operand: activation type of the model (fp16 for BF16 models), or bf16
  // target features when a_bf16 is set
  int32_t pro;
  int32_t a_bf16;                 // PRO_GATHER / PRO_COPY of a BF16 model: bf16 x bf16 MFMAs
  const void* a;                  // PRO_COPY / PRO_GATHER: row stride lda
  int32_t lda;
  const void* g_src[DSPINE_MAX_BATCH];   // PRO_GATHER: rows [g_row0[s], g_row0[s+1])
  int32_t g_row0[DSPINE_MAX_BATCH + 1];  //   come from g_src[s] starting at row g_skip[s]
  int32_t g_n;
  int64_t g_skip[DSPINE_MAX_BATCH];
  const float* P;                 // PRO_BRIDGE_MSG: own-code projections [M, 3a]
  const float* Ppred;             //   predecessor-code projections
  const void* bias;               //   [a] model dtype
  int32_t a_dim, W, pred_shift;
  const float* xa;                // PRO_NORM / PRO_SCALE: fp32 rows, stride lda
  const void* gain;               // PRO_NORM: [K] model dtype
  int32_t act_round_bf16;         // PRO_NORM / PRO_SCALE: operand values pass through bfloat16
                                  //   (RNE) before the fp16 store, as the tile GEMM's bf16 operands do
  // per-row scale (prologue of PRO_NORM / PRO_SCALE, or EPI_ADD_ROWSCALE)
  int32_t scale_mode;
  const float* stats_in;          // [stats_tiles][stats_ld] per-64-column sums of squares
  int32_t stats_tiles, stats_ld;
  float scale_n, eps, code_scale;
  // epilogue
  int32_t epi;
  float* out;                     // EPI_STORE / EPI_ADD(_ROWSCALE): fp32 [M, ldo]
  int32_t ldo;
  void* out_act;                  // EPI_SWIGLU: operand type [M, ld_act] (bf16 when out_act_bf16)
  int32_t ld_act;
  int32_t out_act_bf16;           // EPI_SWIGLU of a BF16 model: store bf16 (the hidden's full range)
  float* stats_out;               // or NULL: [n / 64][stats_out_ld] sums of squares of the stored rows
  int32_t stats_out_ld;
  // EPI_STORE / EPI_SWIGLU with post_scale: the products of row m times its
  // row scale (scale_mode, from stats_in) before the epilogue's operation;
  // the norm of an operand applied after the contraction (it is a per-row
  // factor), so that the operand can be the raw rows
  int32_t post_scale;
  float post_mult;                // and times post_mult (the inverse of the operand copy's copy_mult)
  // EPI_STORE / EPI_ADD / EPI_ADD_ROWSCALE: a 16-bit copy of the stored
  // values times copy_mult (and copy_gain[n] when given) into out_copy
  // [M, ld_copy], bf16 when copy_bf16 (else fp16): the next GEMM's operand
  void* out_copy;
  int32_t ld_copy, copy_bf16;
  float copy_mult;
  const void* copy_gain;          // [N] bf16, or NULL
  // FP8 weights (w_fp8): E4M3 codes in fragment order, read as value / 256;
  // EPI_STORE multiplies output column n by col_scale[n]
  int32_t w_fp8;
  const float* col_scale;
  // EPI_STORE: rows m % W == 0 store code_scale * codebook[anchor[m / W]] instead
  int32_t code_anchor;
  const void* codebook;           // [vocab, N] model dtype
  int32_t anchor[DSPINE_MAX_BATCH];
  // filled by the launcher
  int32_t tiles, ipt, xcd_remap;
  float* partials;
  size_t partial_floats;          // capacity of `partials` (gemm_stream_partial_floats of the rows)
  uint32_t* counters;
};
hipError_t launch_gemm_stream(const GemmParams& p, int dtype, int num_cus, hipStream_t s);
// split partials (floats) of streamed GEMMs of up to `rows` rows
size_t gemm_stream_partial_floats(int rows);
// rows of the row tile a streamed GEMM of M rows runs (16, 32, 64 or 128)
int gemm_stream_row_tile(int M);
int gemm_stream_grid_cap(int num_cus);
int gemm_stream_stat_lists(int n_columns);
int gemm_stream_fused_rows();

// ---------------------------------------------------------------------------
// tiled MFMA GEMM for many rows (prefill): out[m, n] = sum_k A[m, k] W[n, k]
// ---------------------------------------------------------------------------
struct TileGemmParams {
  const void* seg_ptr[kMaxSeg];
  int32_t seg_rows0[kMaxSeg + 1]; // first N row of each segment (prefix)
  int32_t nseg;
  int32_t N, K, M;
  int32_t pro;                    // PRO_COPY or PRO_GATHER (same fields as above)
  int32_t a_bf16;                 // 1: bf16 x bf16 (features); 0: fp16 operands
  const void* a;
  int32_t lda;
  const void* g_src[DSPINE_MAX_BATCH];
  int32_t g_row0[DSPINE_MAX_BATCH + 1];
  int32_t g_n;
  int64_t g_skip[DSPINE_MAX_BATCH];
  float* out;                     // fp32 [M, ldo]
  int32_t ldo;
};
hipError_t launch_gemm_tile(const TileGemmParams& p, int dtype, int num_cus, hipStream_t s);
// true if the tile GEMM takes segments of n_seg output rows and K = k
bool gemm_tile_fits(int n_seg, int k);

// ---------------------------------------------------------------------------
// attention over ring context + block
// ---------------------------------------------------------------------------
struct AttnParams {
  int32_t B, W, nq, nkv, M;
  const float* qkv;               // raw projections [M, ld_qkv]: q | k | v
  int32_t ld_qkv;
  const void* gq;                 // [D] model dtype
  const void* gk;
  float eps;
  const float* rope;              // [M, D/2, 2] cos, sin of each row's angles
  int32_t S, causal;
  const void* kring[DSPINE_MAX_BATCH];
  const void* vring[DSPINE_MAX_BATCH];
  int64_t cap[DSPINE_MAX_BATCH];
  int64_t F[DSPINE_MAX_BATCH];
  int64_t lo0[DSPINE_MAX_BATCH];  // first context position row 0 sees
  int32_t kps[DSPINE_MAX_BATCH];  // context keys per split (multiple of 32)
  int32_t nsplit;
  int32_t kv_nt;                  // context K/V read with non-temporal loads
  void* out;                      // model dtype [M, ld_out]
  int32_t ld_out;
  float* partials;                // [B][nq][nsplit] split partials, merged by a second kernel
};
hipError_t launch_attention(const AttnParams& p, int dtype, int head_dim, hipStream_t s);
size_t attn_partial_floats(int max_b, int nq, int head_dim);

// ---------------------------------------------------------------------------
// row kernels
// ---------------------------------------------------------------------------
struct RowParams {
  int32_t M, W, H;
  const float* x;                 // fp32 [M, H] input
  float* x_out;                   // fp32 residual written by embed gather
  void* act;                      // model dtype [M, H] output
  float* f32_out;                 // fp32 output (final norm)
  const void* gain;               // [H] model dtype
  float eps;
  // embedding gather
  const void* embed;
  int32_t anchor[DSPINE_MAX_BATCH];
  int32_t mask_id;
  // rope table side job
  float* rope;                    // [M, D/2, 2]
  int64_t F[DSPINE_MAX_BATCH];
  int32_t head_dim;
  float rope_theta;
  float* stats;                   // [M] sum of squares of each row (one stats tile)
  int32_t act_bf16;               // rmsnorm: act is bfloat16 (the tile GEMM's bf16 x bf16 path)
  // rmsnorm: with nlists > 0 the rows' sums of squares come from the
  // statistics lists of x ([nlists][ld]) instead of from x itself
  const float* lists;
  int32_t nlists, ld;
};
// Operand pre-scale for large blocks: act[m, k] = x[m, k] * s[m] (* gain[k]),
// s[m] from the row's statistics lists; or the bridge message
// act[t, k] = sigmoid(P[t, k] + Pp[tp, a + k] + b[k]) * Pp[tp, 2a + k]
// (zero at anchor rows).  act is in the model's operand type.
struct ScaleParams {
  int32_t M, K, W;
  int32_t mode;                   // SCALE_* (scale_rows)
  const float* stats;             // [lists][ld]
  int32_t lists, ld;
  float n, eps, code_scale;
  const float* x;                 // fp32 [M, ldx]
  int32_t ldx;
  const void* gain;               // [K] model dtype, or NULL
  int32_t round_bf16;             // scale_rows: values pass through bfloat16 (RNE) first
  const float* P;                 // bridge_msg: [M, 3a]
  const float* Ppred;
  const void* bias;               // [a] model dtype
  int32_t pred_shift;
  void* act;                      // [M, ld_act]
  int32_t ld_act;
};
hipError_t launch_scale_rows(const ScaleParams& p, int dtype, hipStream_t s);
hipError_t launch_bridge_msg(const ScaleParams& p, int dtype, hipStream_t s);

// a4: x = embedding rows, their sums of squares, and the rotation table
hipError_t launch_embed(const RowParams& p, int dtype, hipStream_t s);
hipError_t launch_rmsnorm(const RowParams& p, int dtype, bool f32_output, hipStream_t s);
// sums of squares of the rows of x (one stats tile)
hipError_t launch_rowstats(const RowParams& p, hipStream_t s);

constexpr int kKvLayers = 8;       // draft layers stored by one K/V store launch
struct KvStoreParams {
  int32_t rows, nkv, D, n_req, n_layers;
  int32_t lpw;                    // layers per workgroup (set by the launcher)
  const float* kv;                // fp32 [rows, ld]: layer l's k at l*2*kvd, v at (2l+1)*kvd
  int32_t ld;
  float eps, rope_theta;
  int32_t row0[DSPINE_MAX_BATCH + 1];
  int64_t pos0[DSPINE_MAX_BATCH];      // position of the request's first row
  // per layer of this launch
  int32_t S[kKvLayers];
  int32_t col[kKvLayers];              // column of the layer's k block in kv
  const void* gk[kKvLayers];
  int64_t keep_lo[kKvLayers][DSPINE_MAX_BATCH];   // rows at positions below are not stored
  void* kring[kKvLayers][DSPINE_MAX_BATCH];
  void* vring[kKvLayers][DSPINE_MAX_BATCH];
  int64_t cap[kKvLayers][DSPINE_MAX_BATCH];
};
hipError_t launch_kv_store(const KvStoreParams& p, int dtype, hipStream_t s);

struct VisibleParams {
  int32_t B, W, S, causal;
  int64_t F[DSPINE_MAX_BATCH];
  int64_t* lo_hi;
  int32_t* first_slot;
  int32_t* n_block;
};
hipError_t launch_debug_visible(const VisibleParams& p, hipStream_t s);

// ---------------------------------------------------------------------------
// fused bridge (a9-a11) for blocks of at most 32 rows: one launch whose
// workgroups form three groups (R x, [G; G_p; A] c with gate and message,
// W_l m with the residual add), handing results on through agent-scope
// counters
// ---------------------------------------------------------------------------
struct BridgeParams {
  int32_t M, W, H, r, a;
  float eps, code_scale;          // sqrt(r)
  float* x;                       // fp32 [M, H], updated in place
  const float* xst;               // statistics lists of x: [xst_lists][ld]
  int32_t xst_lists;
  float* st_out;                  // statistics lists of the written x: [H / 64][ld]
  int32_t ld;                     // list stride (kMaxRows)
  const void* R;                  // packed [r, H] (layer)
  const void* G;                  // packed [a, r] (shared)
  const void* Gp;
  const void* A;
  const void* Wl;                 // packed [H, a] (layer)
  const void* bias;               // [a]
  const void* codebook;           // [vocab, r]
  int32_t anchor[DSPINE_MAX_BATCH];
  float* zpart;                   // [r / 16][4][2][256] partial products of the K quarters
  void* z;                        // fp16 [M, r]: R x / (rho + eps), anchor rows sqrt(r) C[anchor]
  float* ssz;                     // [r / 16][ld]: sums of squares of z over each 16 columns
  float* P;                       // fp32 [M, 3a]: [G; G_p; A] c (read by the proposal tail)
  void* msg;                      // fp16 [M, a]: gate * message, zero at anchor rows
  uint32_t* sync;                 // [kBridgeSyncWords]: two hand-off counters, a completion counter, a
                                  // timeout flag, the fourth phase's completion counter, then one
                                  // arrival counter per block of 16 codes, each kBridgeLine words apart
  // Optional fourth phase, the next RMS norm folded in: once every column of
  // x is written, each group-3 workgroup scales its 64 columns by the row's
  // factor rsqrt(S / H + eps) (S from the statistics lists just written,
  // summed in the pre-scale kernel's order) and by next_gain; next_act
  // receives the result as fp16 (the next projection's operand), next_out as
  // fp32 (the final norm).  Both NULL: no fourth phase.
  const void* next_gain;          // [H] bf16
  void* next_act;                 // fp16 [M, H] or NULL
  float* next_out;                // fp32 [M, H] or NULL
  // Or (copy_out): group 3 stores fp16(x * copy_gain * copy_mult) of its
  // columns, the next layer's raw operand, whose norm its q|k|v GEMM applies
  // after the product; no fourth phase
  void* copy_out;                 // fp16 [M, H] or NULL
  const void* copy_gain;          // [H] bf16
  float copy_mult;
};
hipError_t launch_bridge_fused(const BridgeParams& p, hipStream_t s);
// true if the fused bridge takes this geometry and M rows on num_cus CUs
bool bridge_fused_fits(int H, int r, int a, int M, int num_cus);
// The fused bridge's counters sit kBridgeLine words (128 bytes) apart, so
// that the arrivals and polls on one counter do not queue behind those on
// another in the same line.
constexpr int kBridgeLine = 32;
constexpr int kBridgeSyncWords = (5 + 64) * kBridgeLine;

// words [0, n_words) of p <- 0 with a kernel
hipError_t launch_zero_words(void* p, size_t n_words, hipStream_t s);

// *out = max(*out, max |src[i]|) over n bf16 values, as float bits (NaN
// counts above every finite value)
hipError_t launch_absmax_bf16(const void* src, size_t n, uint32_t* out, hipStream_t s);

// projection matrix [rows, cols] row-major -> fragment order (see pack_kernel)
hipError_t launch_pack(const void* src, void* dst, int rows, int cols, int dtype, hipStream_t s);

}  // namespace dspine
