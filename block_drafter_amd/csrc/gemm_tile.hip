// Tiled MFMA GEMM for context prefill (a1 feature fusion, a2 K/V projection):
//
//   out[m, n] = sum_k A[m, k] * W[n, k]     (16-bit operands, fp32 accumulate)
//
// With thousands of rows this is a dense contraction bound by the matrix
// cores.  gfx950 design:
//  * 256 x 256 output tile per workgroup of eight waves (two per SIMD, so
//    that one multiplies while the other waits at the barrier or on LDS);
//    each wave owns 128 x 64 = 8 x 4 MFMA 16x16x32 tiles, accumulators in
//    the register file.
//  * Operands move global -> LDS with the direct-to-LDS loads of gfx950
//    (global_load_lds_dwordx4): no registers are spent on staging.
//  * LDS holds 1 KB blocks in the MFMA operand order (16 rows x 32 K; lane l
//    owns row l % 16, K 8 (l / 16) .. + 8): a wave reads a fragment as one
//    contiguous, conflict-free ds_read_b128.  The weights are stored in that
//    order already (each block is one coalesced 1 KB copy); an activation
//    block is 16 row pieces of 64 contiguous bytes.
//  * A ring of four K slices of 32 (32 KB each): the direct-to-LDS loads
//    run three slices ahead of the multiply, one barrier per slice.  Within
//    a slice each B fragment is read one group of 8 multiplies ahead.
//  * Tiles are numbered so that each XCD (which receives every 8th
//    workgroup) walks a contiguous range of tiles, in groups of 8 row tiles
//    (each group row tiles first, then the next column): the workgroups
//    resident on one XCD form an 8 x 4 block of tiles that shares activation
//    and weight slices in that XCD's L2.
// Operands: bf16 target features x bf16 weights (F16 = false), or fp16
// context features x bf16 weights widened to fp16 after they are read from
// LDS (F16 = true).
#include "dspine_device.hpp"
#include "dspine_internal.hpp"

namespace dspine {


constexpr int kGroupM = 8;          // row tiles per group of the tile order
constexpr int kTileM = 256, kTileN = 256;

template <bool F16>
__global__ __launch_bounds__(512, 1) void gemm_tile_kernel(const TileGemmParams p) {
  constexpr int BM = kTileM, BN = kTileN, SB = (BM + BN) / 16 * 1024;   // 32 KB per slice
  constexpr int LOADS = (BM + BN) / 16 / 8;                        // DMA loads per wave per slice
  constexpr int ABLK = BM / 16;
  __shared__ __attribute__((aligned(1024))) char smem[4 * SB];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wn = w >> 1;                               // rows wm*128, cols wn*64
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = p.N / BN;
  const int T = gridDim.x;
  int id = blockIdx.x;
  if (T % 8 == 0) id = (id % 8) * (T / 8) + id / 8;
  const int per_group = kGroupM * tiles_n;
  const int g0 = (id / per_group) * kGroupM;
  const int gm = tiles_m - g0 < kGroupM ? tiles_m - g0 : kGroupM;
  const int tm = g0 + (id % per_group) % gm, tn = (id % per_group) / gm;
  const int n0 = tn * BN;

  int s = 0;
  while (s + 1 < p.nseg && n0 >= p.seg_rows0[s + 1]) ++s;
  const bf16_t* wbase = reinterpret_cast<const bf16_t*>(p.seg_ptr[s]) + (size_t)(n0 - p.seg_rows0[s]) * p.K;

  // wave w loads A row blocks w, w + 8 and B row blocks w, w + 8
  const uint16_t* arow[2];
  const uint16_t* brow[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    int m = tm * BM + (w + 8 * q) * 16 + (lane & 15);
    m = m < p.M ? m : p.M - 1;
    const uint16_t* r;
    if (p.pro == PRO_GATHER) {
      int g = 0;
      while (g + 1 < p.g_n && m >= p.g_row0[g + 1]) ++g;
      r = reinterpret_cast<const uint16_t*>(p.g_src[g]) + (size_t)(m - p.g_row0[g] + p.g_skip[g]) * p.lda;
    } else {
      r = reinterpret_cast<const uint16_t*>(p.a) + (size_t)m * p.lda;
    }
    arow[q] = r + 8 * (lane >> 4);
    brow[q] = reinterpret_cast<const uint16_t*>(wbase) + (size_t)(w + 8 * q) * 16 * p.K + lane * 8;
  }
  auto issue = [&](int kt, int b) __attribute__((always_inline)) {
    char* st = smem + b * SB;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_global_load_lds(arow[q] + kt * 32, (lds_void*)(st + (w + 8 * q) * 1024), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_global_load_lds(brow[q] + (size_t)kt * 512, (lds_void*)(st + (ABLK + w + 8 * q) * 1024), 16, 0,
                                       0);
  };

  f32x4 acc[4][8];                                     // [n block][m block]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = f32x4{0, 0, 0, 0};

  const int nk = p.K / 32;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  if (nk > 2) issue(2, 2);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 2 < nk) wait_vmcnt<2 * LOADS>();
    else if (kt + 1 < nk) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (kt + 3 < nk) issue(kt + 3, (kt + 3) & 3);
    // the 8 A fragments and B fragment 0, then per B fragment j: wait for
    // the reads so far, read fragment j + 1, multiply with fragment j
    const char* st = smem + (kt & 3) * SB;
    u32x4 af[8], bw[4];
#pragma unroll
    for (int t = 0; t < 8; ++t) af[t] = *reinterpret_cast<const u32x4*>(st + (wm * 8 + t) * 1024 + lane * 16);
    bw[0] = *reinterpret_cast<const u32x4*>(st + (ABLK + wn * 4) * 1024 + lane * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      if (j + 1 < 4) bw[j + 1] = *reinterpret_cast<const u32x4*>(st + (ABLK + wn * 4 + j + 1) * 1024 + lane * 16);
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 b = F16 ? bf16x8_to_f16x8(bw[j]) : bw[j];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (F16)
          acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, b),
                                                             __builtin_bit_cast(f16x8, af[i]), acc[j][i], 0, 0, 0);
        else
          acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b),
                                                              __builtin_bit_cast(bf16x8, af[i]), acc[j][i], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = tm * BM + (wm * 8 + i) * 16 + (lane & 15);
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + (wn * 4 + j) * 16 + 4 * (lane >> 4);
      *reinterpret_cast<f32x4*>(p.out + (size_t)m * p.ldo + n) = acc[j][i];
    }
  }
}

bool gemm_tile_fits(int n_seg, int k) { return n_seg > 0 && n_seg % kTileN == 0 && k > 0 && k % 32 == 0; }

hipError_t launch_gemm_tile(const TileGemmParams& p, int dtype, int num_cus, hipStream_t s) {
  (void)num_cus;
  if (dtype != DT_BF16 || p.M < 1 || p.K % 32 != 0 || p.N % kTileN != 0 || p.ldo % 4 != 0) return hipErrorInvalidValue;
  for (int i = 1; i < p.nseg; ++i)
    if (p.seg_rows0[i] % kTileN != 0) return hipErrorInvalidValue;      // a tile never crosses a segment
  const int tiles = ((p.M + kTileM - 1) / kTileM) * (p.N / kTileN);
  if (p.a_bf16) DSPINE_LAUNCH(gemm_tile_kernel<false>, dim3(tiles), dim3(512), 0, s, p);
  else DSPINE_LAUNCH(gemm_tile_kernel<true>, dim3(tiles), dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace dspine
