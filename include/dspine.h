/*
 * dspine.h -- C ABI of the DSpine draft-block library for AMD Instinct MI355X (gfx950).
 *
 * The library computes one speculative-decoding draft round on the GPU:
 *   - dspine_ctx_materialize: fuse committed target features into context
 *     features and store every draft layer's context K/V in per-request rings;
 *   - dspine_draft_forward:   one masked-block forward (anchor + masks) over
 *     B requests, with the DSpine gated predecessor bridge after every layer;
 *   - dspine_bridge:          the bridge alone on one layer's block states;
 *   - dspine_draft_propose:   the forward, then candidates from the shared LM
 *     head, the transition table of the last-write refinement and the walk.
 *
 * Sources, cited by tag in the comments below:
 *   [FLZ] "DSpine for Qwen3.8-27B: Causal Features Through Depth" (flozi.net guide)
 *   [PHY] "DSpine 完全拆解：相邻因果注入如何让并行草稿沿网络深度建立 token 依赖"
 *         (pinghaoyang.com.cn article)
 *   [DSP] "DSpark, every bolt and rivet" (lab-artifacts tutorial)
 *   [NIF] NInfer maintainer notes, "DFlash" (docs/maintainer/dflash.md)
 *
 * Conventions for every call:
 *   - "device" pointers address GPU memory of the current HIP device; "host"
 *     pointers address CPU memory read during the call only.
 *   - The caller owns every buffer (weights, rings, features, outputs,
 *     workspace).  The library never allocates or frees; calls only enqueue
 *     kernels on the given stream and return (dspine_pack_weights, a one-time
 *     set-up call, also waits for its range check; dspine_profile_read waits
 *     for its events).
 *   - Matrices are row-major [out, in] (y = W x).  BF16 tensors are IEEE
 *     bfloat16 bit patterns; FP16 is IEEE binary16.
 *   - Return value: DSPINE_OK (0) or a negative DSPINE_E_* code.  Every
 *     argument check happens before the first launch: on error nothing is
 *     enqueued and no context frontier changes.  dspine_last_error() gives
 *     a message for the calling thread's last failure.
 *   - A kernel fault surfaces as DSPINE_E_HIP on a later call (or on the
 *     caller's own stream synchronisation).
 */
#ifndef DSPINE_H
#define DSPINE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* dspine_stream_t;   /* same object as hipStream_t */

#define DSPINE_MAX_LAYERS 16
#define DSPINE_MAX_BATCH 8
#define DSPINE_MIN_WIDTH 2
#define DSPINE_MAX_WIDTH 16

/* status codes */
#define DSPINE_OK 0
#define DSPINE_E_ARG (-1)          /* null pointer, negative size, bad index */
#define DSPINE_E_UNSUPPORTED (-2)  /* geometry, B or W outside what the kernels implement */
#define DSPINE_E_WORKSPACE (-3)    /* workspace smaller than dspine_workspace_bytes() */
#define DSPINE_E_STATE (-4)        /* context state inconsistent with the request */
#define DSPINE_E_HIP (-5)          /* a HIP runtime call failed */

/* element type of weights, features and the residual stream's inputs */
#define DSPINE_F32 0
#define DSPINE_BF16 1

/*
 * Draft geometry.  [NIF, draft config table]: hidden width, layers, FFN
 * width, Q/KV heads and head width, norm epsilon, 1-D RoPE theta, per-layer
 * attention type and window, target feature layers, mask token.  [FLZ, "The
 * bridge"]: code width r and message width a (r = a = 0: no bridge, which
 * is plain DFlash).
 *
 * Kernel limits (DSPINE_E_UNSUPPORTED otherwise): hidden, ffn, code_dim and
 * n_q_heads*head_dim multiples of 32 (hidden and ffn also of 64); msg_dim a
 * multiple of 32; head_dim 64 or 128; n_q_heads/n_kv_heads in {1,2,4,8};
 * 1 <= n_layers <= DSPINE_MAX_LAYERS; window[l] >= 0 (0 = full attention).
 */
typedef struct {
    int32_t hidden;            /* H */
    int32_t n_layers;          /* L */
    int32_t n_q_heads;         /* nq */
    int32_t n_kv_heads;        /* nkv */
    int32_t head_dim;          /* D */
    int32_t ffn;               /* SwiGLU intermediate width */
    int32_t n_feat_layers;     /* Lf: target layers concatenated into features */
    int32_t code_dim;          /* r; 0 disables the bridge */
    int32_t msg_dim;           /* a; 0 iff code_dim == 0 */
    int32_t vocab;             /* rows of the embedding table and the codebook */
    int32_t mask_token_id;     /* embedding row used for every mask position */
    int32_t block_causal;      /* 0: bidirectional block [NIF]; 1: block-causal [PHY, 块因果注意力] */
    int32_t window[DSPINE_MAX_LAYERS];  /* S_l; 0 = full attention layer */
    float eps;                 /* RMSNorm epsilon, also the bridge floor */
    float rope_theta;
    int32_t dtype;             /* DSPINE_F32 or DSPINE_BF16 */
    int32_t conv_group;        /* DFlash2 dynamic grouped convolution [NIF, DFlash2 layer
                                  equations]: group width (16), 0 = none; hidden/conv_group
                                  must be a multiple of 16 */
} dspine_geometry;

/* Per-layer weights (device, borrowed; element type = geometry.dtype). */
typedef struct {
    const void* g_in;          /* [H]    input RMSNorm gain */
    const void* wq;            /* [nq*D, H] */
    const void* wk;            /* [nkv*D, H]  used for block and context keys [NIF] */
    const void* wv;            /* [nkv*D, H]  used for block and context values */
    const void* gq;            /* [D]    query head-norm gain */
    const void* gk;            /* [D]    key head-norm gain */
    const void* wo;            /* [H, nq*D] */
    const void* g_post;        /* [H]    post-attention RMSNorm gain */
    const void* w_gate;        /* [ffn, H] */
    const void* w_up;          /* [ffn, H] */
    const void* w_down;        /* [H, ffn] */
    const void* R;             /* [r, H]  bridge read [FLZ]; NULL when r == 0 */
    const void* W_l;           /* [H, a]  bridge write;     NULL when r == 0 */
    /* DFlash2 convolutions (NULL when conv_group == 0), G = H / conv_group groups:
     * W_delta [4G, H], output row (side*2 + tap)*G + g; base [4, H], row side*2 + tap.
     * Conv_side(X)[i] = (base[side,0] + delta[i,side,0,g]) X[i]
     *                 + [i >= 1] (base[side,1] + delta[i,side,1,g]) X[i-1]
     * on the branch's normalised input X (side 0, "prepare") and on the branch
     * output with the same delta (side 1, "finish"). */
    const void* attn_conv_w;
    const void* attn_conv_base;
    const void* mlp_conv_w;
    const void* mlp_conv_base;
} dspine_layer_weights;

/* All model weights (device, borrowed, element type = geometry.dtype).  They
 * must stay valid and unchanged while the model handle is used. */
typedef struct {
    const void* embed;         /* [vocab, H]  target input embedding */
    const void* w_feat;        /* [H, Lf*H]   context feature projection, no bias [NIF] */
    const void* g_ctx;         /* [H]         context_norm gain */
    const void* g_final;       /* [H]         final RMSNorm gain */
    const void* codebook;      /* [vocab, r]  token codes C [FLZ]; NULL when r == 0 */
    const void* bridge_G;      /* [a, r]  receiver gate, shared by layers [FLZ] */
    const void* bridge_Gp;     /* [a, r]  predecessor gate, shared */
    const void* bridge_A;      /* [a, r]  predecessor value map, shared */
    const void* bridge_b;      /* [a]     gate bias, shared */
    dspine_layer_weights layer[DSPINE_MAX_LAYERS];
    const void* lm_head;       /* [vocab, H]  shared LM head for dspine_draft_propose (vocab a
                                  multiple of 16); NULL when proposals are not used.  Packed
                                  like the projections for the score GEMM, and also read
                                  row-major (candidate rows): unlike the projections it must
                                  stay valid while the model is used */
} dspine_weights;

/*
 * One request's draft context (host struct).  [NIF, ring storage]: a local
 * layer of window S keeps positions [max(0, F-S), F) in a ring of exactly S
 * slots, position p in slot p mod S; a full layer keeps [0, F) with
 * position p at index p (capacity >= every frontier it will reach).
 *
 * Ring layout per layer, head-major: K [n_kv_heads][capacity][head_dim] and
 * V [n_kv_heads][capacity][head_dim].  Element types [NIF, fused context
 * materializer]: BF16 model -> K bfloat16, V binary16 (FP16_RNE(BF16(v)));
 * F32 model -> both float32.  Only live slots are ever read.
 *
 * frontier F: positions [0, F) are processed and materialized; the anchor
 * token sits at position F [NIF, frontier].  dspine_ctx_materialize
 * advances it; nothing else changes it.
 */
typedef struct {
    void* k_ring[DSPINE_MAX_LAYERS];
    void* v_ring[DSPINE_MAX_LAYERS];
    int64_t capacity[DSPINE_MAX_LAYERS];
    int64_t frontier;
} dspine_ctx;

typedef struct dspine_model dspine_model;

/* Checks the geometry and weight pointers and makes a host-side handle that
 * borrows them.  Errors: E_ARG (null), E_UNSUPPORTED (limits above). */
int dspine_model_create(const dspine_geometry* geom, const dspine_weights* weights,
                        dspine_model** out);
void dspine_model_destroy(dspine_model* model);

/*
 * Projection weights in fragment order.  The GEMMs stream every projection
 * matrix (wq, wk, wv, wo, w_gate, w_up, w_down, R, W_l, attn/mlp_conv_w per layer; w_feat,
 * bridge_G, bridge_Gp, bridge_A; lm_head when given) in the order their MFMA fragments are
 * loaded: inside each block of 16 rows, 32-wide column step ks holds the 64
 * lane fragments (row 16b + l%16, columns 32ks + 8(l/16) .. +8) in
 * consecutive memory.  dspine_pack_weights writes that copy into `dst`
 * (device, 256-byte aligned, dspine_packed_bytes bytes, caller-owned) with
 * kernels on `stream`; from then on the model reads projections only from
 * `dst`, which must outlive the model (the row-major matrices may be freed
 * once those kernels have run).
 *
 * Operand range (BF16 models).  The GEMMs multiply fp16 operands by the bf16
 * weights widened to fp16, except the feature projection w_feat and the
 * down projection w_down (bf16 x bf16: the SwiGLU hidden is the one operand
 * no norm bounds, so it is kept in bf16).  A widened weight must therefore
 * lie within fp16's range: dspine_pack_weights measures the largest
 * magnitude of every widened projection (and of lm_head), waits for that
 * check, and fails with DSPINE_E_UNSUPPORTED (naming the matrix) beyond
 * 65504.  Weights below 2^-14 become fp16 subnormals (rounded toward zero,
 * an absolute error below 2^-24).  This is the one call that synchronises.
 *
 * With an lm_head on a BF16 model, `dst` also
 * receives the head's row-scaled FP8 copy for the retrieval of
 * dspine_draft_propose (one E4M3 code per element, fragment order with two
 * 32-wide column steps per lane fragment, and a float32 scale per row:
 * vocab * (hidden + 4) bytes more).  Every other
 * call returns DSPINE_E_STATE until the model is packed.  Errors: E_ARG,
 * E_WORKSPACE (dst too small), E_UNSUPPORTED (a weight out of range, above),
 * E_HIP.
 */
size_t dspine_packed_bytes(const dspine_model* model);
int dspine_pack_weights(dspine_model* model, void* dst, size_t dst_bytes, dspine_stream_t stream);

/* Bytes of one ring (K or V, same size) of `layer` for one request with the
 * given capacity (must be window[layer] for a local layer).  0 on error. */
size_t dspine_ring_bytes(const dspine_model* model, int layer, int64_t capacity);

/* Workspace bytes a call needs for up to max_batch requests of width up to
 * max_width and up to max_rows materialized positions per call (summed over
 * the call's requests, after truncation to the live windows).  The buffer
 * must be zero-filled once before its first use; the library leaves its
 * internal counters at zero when each call's work completes.  Calls that
 * share a workspace must be ordered on one stream.  0 on error. */
size_t dspine_workspace_bytes(const dspine_model* model, int max_batch, int max_width,
                              int64_t max_rows);

/*
 * a1-a3: materialize committed target features into the draft context.
 * [NIF, context conditioning / context K/V / fused context materializer]:
 *   c_t = plain_rmsnorm(W_feat s_t, g_ctx);
 *   per layer: k = rope_1d(head_rmsnorm(W_k c_t, gk), t) stored BF16,
 *              v = W_v c_t stored FP16_RNE(BF16(v)).
 * A chunk longer than a local ring stores only its final live window; the
 * frontier still advances by the whole chunk.
 *
 *   n_req          number of requests (1..DSPINE_MAX_BATCH)
 *   ctx            host [n_req]; ctx[b].frontier += n_tok[b] on success
 *   feats          host [n_req] of device pointers, each [n_tok[b], Lf*H]
 *                  in the model dtype (positions F..F+n-1 in order)
 *   n_tok          host [n_req], each >= 0
 * Errors: E_ARG, E_STATE (local capacity != window, full capacity < F+n),
 * E_WORKSPACE (rows after truncation exceed the workspace's max_rows).
 */
int dspine_ctx_materialize(const dspine_model* model, int n_req, dspine_ctx* ctx,
                           const void* const* feats, const int64_t* n_tok,
                           void* workspace, size_t workspace_bytes, dspine_stream_t stream);

/*
 * a4-a12: one masked-block draft forward for B requests of width W.
 * [NIF, draft input]: row i of request b is the embedding of the anchor
 * (i = 0) or of the mask token (i > 0), at position F_b + i.
 * [NIF, layer equations] per layer (with conv_group > 0, DFlash2's dynamic
 * grouped convolution around attention and MLP [NIF, DFlash2 layer
 * equations]), then the bridge [FLZ, "The bridge"] after every layer when
 * code_dim > 0, then the final plain RMSNorm.
 * Attention [NIF, draft attention]: key at position p is visible to the
 * row at q iff |p - q| < S (local) plus, with block_causal, block key j <=
 * row i; context keys are the ring positions [max(0, q-S+1), F).
 *
 *   B, W           1..8 and 2..16
 *   ctx            host [B]; read only (frontiers and rings)
 *   anchor_ids     host [B], each in [0, vocab)
 *   out            device float32 [B, W, H]: final-normed hidden states
 * Errors: E_ARG, E_UNSUPPORTED, E_STATE (full-layer capacity < F + W is
 * allowed; a frontier < 0 is not), E_WORKSPACE.
 */
int dspine_draft_forward(const dspine_model* model, int B, int W, const dspine_ctx* ctx,
                         const int32_t* anchor_ids, float* out,
                         void* workspace, size_t workspace_bytes, dspine_stream_t stream);

/*
 * dspine_draft_forward for callers that cannot allocate (code under graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * forward and the same kernels, with the workspace replaced by a static
 * device array of DSPINE_NOALLOC_SCRATCH_BYTES held by the library on every
 * GPU it runs on until the process ends.  The call allocates nothing.
 *
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents: calls that overlap on one GPU (other streams, other
 *     threads) race and must be ordered by the caller.
 *   - The first call on a device looks the array up and clears its tile
 *     counters on `stream` before the forward.
 *   - B * W and the geometry must fit the array: the 27B geometry takes up to
 *     B * W = 32 rows (B = 2 at W = 16).  Larger calls fail with
 *     DSPINE_E_WORKSPACE before any launch.
 * Arguments and errors otherwise as dspine_draft_forward.
 */
#define DSPINE_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)
int dspine_draft_forward_noalloc(const dspine_model* model, int B, int W, const dspine_ctx* ctx,
                                 const int32_t* anchor_ids, float* out, dspine_stream_t stream);

/*
 * a9-a11 alone on one layer's block states.  [FLZ, "The bridge"]:
 *   rho_t = rms(x_t), z_t = R_l x_t / (rho_t + eps),
 *   c_t = sqrt(r) z_t / (||z_t|| + eps), anchor row: c_0 = sqrt(r) C[a_b];
 *   x_t += rho_t W_l (sigmoid(G c_t + G_p p_t + b) * (A p_t)) for t >= 1,
 * with predecessor code p_t = c_{t-1}, or pred_codes[b][t] when given (the
 * hook for redoing the last write with a chosen predecessor token [PHY,
 * last-write refinement]).  Row 0 is never written.
 *
 *   layer          0..L-1 (selects R_l and W_l)
 *   x              device float32 [B, W, H], updated in place
 *   anchor_ids     host [B]
 *   pred_codes     device float32 [B, W, r] or NULL; entry t = 0 unused
 * Errors: E_ARG, E_UNSUPPORTED (no bridge in the geometry), E_WORKSPACE.
 */
int dspine_bridge(const dspine_model* model, int layer, int B, int W, float* x,
                  const int32_t* anchor_ids, const float* pred_codes,
                  void* workspace, size_t workspace_bytes, dspine_stream_t stream);

/*
 * Proposal tail after the draft forward.  [FLZ, "The last write is refined
 * using discrete candidates"]; [PHY, 前驱条件解码与 transition cache]:
 *   - candidates: the K best tokens of the shared LM head's scores E_v . h_t
 *     of every proposal row t = 1..W-1 (h = the forward's final-normed
 *     state), best first, equal scores by smaller token id (direct BF16 path);
 *     or, with retrieve = R > 0 (BF16 models), by FP8 row-scaled retrieval:
 *     the vocabulary is scored with the head's FP8 copy, s_v (q_v . h_t), the
 *     R best of those (same order rule) are rescored with the BF16 head and
 *     the K best rescored kept.  The FP8 copy (made by dspine_pack_weights):
 *     q_v = E4M3 codes (OCP, round to nearest even) of E_v / s_v, s_v the
 *     smallest power of two with max_k |E_v[k]| / s_v <= 448;
 *   - transition table T_t[i, j]: the last layer's bridge write is redone
 *     from its pre-write state u_t with the predecessor code replaced by
 *     sqrt(r) C[s], s = candidate i of row t-1 (the anchor for t = 1, so the
 *     K rows of T_1 are equal); the result is final-normed and scored by the
 *     head on row t's candidates j;
 *   - walk: row 1 picks from T_1's row 0, row t from the row of T_t chosen at
 *     t-1.  Greedy: the largest score (smaller index on ties).  Sampled:
 *     p = softmax(T_t[i*, :] / temperature) in float64, the first j whose
 *     cumulative probability exceeds the given uniform u (the last j if
 *     rounding leaves u above the total); q = p[j] is kept.
 */
#define DSPINE_MAX_TOPK 16
#define DSPINE_MAX_RETRIEVE 128
#define DSPINE_WALK_GREEDY 0
#define DSPINE_WALK_SAMPLED 1

typedef struct {
    int32_t topk;              /* K, 1..DSPINE_MAX_TOPK */
    int32_t walk;              /* DSPINE_WALK_GREEDY or DSPINE_WALK_SAMPLED */
    int32_t retrieve;          /* 0: direct BF16 head scores; R in K..DSPINE_MAX_RETRIEVE (and <=
                                  vocab): FP8 retrieval of R candidates per row, BF16 rescoring */
    double temperature;        /* sampled walk: > 0 */
    const double* uniforms;    /* sampled walk: device float64 [B, W-1], each in [0, 1) */
    /* outputs, device */
    float* scores;             /* optional (NULL: kept in the workspace): float32 [B*W, vocab]
                                  head scores of every row (anchor rows included); the FP8
                                  scores when retrieve > 0 */
    int32_t* retrieved;        /* optional, retrieve > 0: int32 [B, W-1, R] the retrieved ids,
                                  best FP8 score first (-1 beyond the finite scores) */
    float* rescored;           /* optional, retrieve > 0: float32 [B, W-1, R] their BF16 scores */
    int32_t* cand;             /* int32 [B, W-1, K] candidate token ids of rows 1..W-1 (-1 in
                                  slots beyond the number of finite scores; NaN ranks as -inf) */
    float* cand_scores;        /* float32 [B, W-1, K] their BF16 head scores */
    float* table;              /* float32 [B, W-1, K, K]: entry [b, t-1, i, j] = T_t[i, j] */
    int32_t* choice;           /* int32 [B, W-1] chosen candidate index of each row */
    int32_t* tokens;           /* int32 [B, W-1] chosen token ids */
    double* q;                 /* float64 [B, W-1] probability of each choice: required for the
                                  sampled walk (it is kept for verification); for the greedy
                                  walk NULL or written as 1 */
} dspine_proposal;

/* Bytes of the second workspace dspine_draft_propose needs for up to
 * max_batch requests of width up to max_width and top-k up to topk.  It needs
 * no zero fill.  0 on error (or when the model has no lm_head). */
size_t dspine_propose_workspace_bytes(const dspine_model* model, int max_batch, int max_width, int topk);

/*
 * One draft forward (exactly dspine_draft_forward: same arguments, same
 * `out`) followed by the proposal tail above.  Needs a bridge (code_dim > 0)
 * and lm_head.  `workspace` is the forward's; `propose_ws` the tail's.
 * Errors: those of dspine_draft_forward, E_ARG (NULL output, K, R or walk
 * out of range, temperature <= 0, uniforms or q NULL for the sampled walk),
 * E_UNSUPPORTED (no bridge or no lm_head; retrieval on a float32 model),
 * E_WORKSPACE.
 */
int dspine_draft_propose(const dspine_model* model, int B, int W, const dspine_ctx* ctx,
                         const int32_t* anchor_ids, float* out, const dspine_proposal* prop,
                         void* workspace, size_t workspace_bytes,
                         void* propose_ws, size_t propose_ws_bytes, dspine_stream_t stream);

/*
 * a3 as the attention kernel evaluates it, for exact comparison: for every
 * block row, the half-open interval of visible context positions, the ring
 * slot of its first position, and the number of visible block keys.  The
 * values come from the same device predicate the attention kernel uses.
 *
 *   lo_hi          device int64 [B, W, 2]
 *   first_slot     device int32 [B, W]   (-1 for an empty interval)
 *   n_block        device int32 [B, W]
 */
int dspine_debug_visible(const dspine_model* model, int layer, int B, int W,
                         const dspine_ctx* ctx, int64_t* lo_hi, int32_t* first_slot,
                         int32_t* n_block, dspine_stream_t stream);

/*
 * Kernel timing (tracing).  While enabled, the calls record a pair of HIP
 * events on their stream around every launch of the selected kernel classes;
 * dspine_profile_read waits for the recorded events of one class, returns
 * their summed duration and count, and forgets them.  Intended for
 * measurement runs: the event records add a few microseconds per launch.
 */
#define DSPINE_PROF_GEMM_QKV 0      /* a5 q|k|v projection */
#define DSPINE_PROF_ATTENTION 1     /* a6 */
#define DSPINE_PROF_GEMM_O 2        /* a7 output projection + residual */
#define DSPINE_PROF_GEMM_GATE_UP 3  /* a8 gate/up projection + SwiGLU */
#define DSPINE_PROF_GEMM_DOWN 4     /* a8 down projection + residual */
#define DSPINE_PROF_BRIDGE 5        /* a9-a11, all kernels of one bridge */
#define DSPINE_PROF_NORM 6          /* input/post/final norms and the embedding gather */
#define DSPINE_PROF_CTX_GEMM 7      /* a1-a2 feature and K/V projections */
#define DSPINE_PROF_CTX_STORE 8     /* a1 norm, a2 head norm + RoPE + ring scatter */
#define DSPINE_PROF_HEAD 9          /* proposal: the LM head's scores of every row */
#define DSPINE_PROF_TAIL 10         /* proposal: top-K, refinement table and walk */
#define DSPINE_PROF_CONV 11         /* DFlash2 convolution deltas, prepare and finish */
#define DSPINE_PROF_KINDS 12

/* kind_mask: bit k enables class k; 0 disables recording.  Process-wide. */
int dspine_profile_enable(uint32_t kind_mask);
/* Records only every stride-th launch scope of each enabled class (counted
 * per class from this call; 1, the default, records all), so that a
 * measurement over many launches pays the event overhead on a sample of
 * them.  stride 0 is DSPINE_E_ARG.  Process-wide. */
int dspine_profile_stride(uint32_t stride);
/* Waits for the recorded events of class `kind` (host-blocking), writes the
 * summed milliseconds and the number of launches, and clears the class. */
int dspine_profile_read(int kind, double* total_ms, int64_t* launches);

/* Message for the calling thread's last nonzero status ("" if none). */
const char* dspine_last_error(void);

/* Library version string. */
const char* dspine_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DSPINE_H */
