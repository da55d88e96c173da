// Internal interface of the proposal tail kernels (propose.hip) for the C ABI.
#pragma once
#include "dspine_internal.hpp"

namespace dspine {

// ---------------------------------------------------------------------------
// proposal tail (candidates, refinement rows, walk)
// ---------------------------------------------------------------------------
constexpr int kMaxTopK = DSPINE_MAX_TOPK;
struct ProposeParams {
  int32_t B, W, K, vocab, H, r, a, walk;
  double temperature;
  float eps, code_scale;
  int32_t anchor[DSPINE_MAX_BATCH];
  const float* scores;            // [B*W, vocab] head scores
  float* part_v;                  // partial top-K lists [rows][chunks][kMaxTopK]
  int32_t* part_i;
  int32_t* cand;                  // [B, W-1, K]
  float* cand_scores;
  const void* codebook;           // [vocab, r] model dtype
  void* codes;                    // [B*(W-1)*K, r] operand type
  const float* P_own;             // [B*W, 3a]: the forward's last [G; G_p; A] c
  const float* P_cand;            // [B*(W-1)*K, 2a]: [G_p; A] of the candidate codes
  const void* bias;               // [a] model dtype
  void* msg;                      // [B*(W-1)*K, a] operand type
  const float* u;                 // [B*W, H] last layer's pre-write state
  const float* Y;                 // [B*(W-1)*K, H] W_l msg
  const void* g_final;            // [H] model dtype
  const void* head;               // [vocab, H] row-major
  float* table;                   // [B, W-1, K, K]
  const double* uniforms;         // [B, W-1]
  int32_t* choice;                // [B, W-1]
  int32_t* tokens;                // [B, W-1]
  double* q;                      // [B, W-1] or NULL
  // FP8 row-scaled retrieval (R > 0): the R best of the FP8 scores (in
  // `scores`), rescored with the BF16 head, the best K kept
  int32_t R;
  int32_t* retrieved;             // [B*(W-1), R] ids, best FP8 score first
  float* rescored;                // [B*(W-1), R] their BF16 head scores
  const float* h;                 // [B*W, H] the forward's final-normed output
};
hipError_t launch_topk(const ProposeParams& p, hipStream_t s);
size_t topk_partial_entries(int rows, int vocab);
int topk_max_vocab();
int propose_max_hidden();
hipError_t launch_cand_codes(const ProposeParams& p, int dtype, hipStream_t s);
hipError_t launch_cand_msg(const ProposeParams& p, int dtype, hipStream_t s);
hipError_t launch_cand_score(const ProposeParams& p, int dtype, hipStream_t s);
hipError_t launch_walk(const ProposeParams& p, hipStream_t s);

// FP8 retrieval: candidates kept by the FP8 scores of one row (at most)
constexpr int kMaxRetrieve = DSPINE_MAX_RETRIEVE;
hipError_t launch_retrieve(const ProposeParams& p, hipStream_t s);
size_t retrieve_partial_entries(int rows, int vocab);
// Row-scaled FP8 copy of a bf16 head [V, H] (V a multiple of 16, H of 64):
// E4M3 codes in fragment order, each lane's 16 bytes holding its codes of
// two consecutive 32-wide column steps (one byte per element), and
// col_scale[v] = 256 s_v, s_v the smallest power of two with max|E_v| / s_v
// <= 448 (256: the GEMM reads each code as its value / 256).
hipError_t launch_quant_head_fp8(const void* head, void* codes, float* col_scale, int V, int H, hipStream_t s);

}  // namespace dspine
