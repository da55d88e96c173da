// Tiled MFMA GEMM for context prefill (a1 feature fusion, a2 K/V projection):
//
//   out[m, n] = sum_k A[m, k] * W[n, k]     (bf16 operands, fp32 accumulate)
//
// With thousands of rows this is a dense contraction bound by the matrix
// cores.  gfx950 design: 256 x 128 output tile per workgroup of four waves
// (each wave 128 x 64 = 4 x 2 MFMA 32x32x16 tiles, accumulators in the
// register file), K slices of 64 double-buffered in LDS through registers,
// 16-byte padded LDS rows.  Tiles are numbered so that each XCD (which
// receives every 8th workgroup) walks a contiguous block of tiles with the
// row index fastest: the workgroups resident on one XCD share weight rows
// and activation slices in that XCD's L2.
// Operands: bf16 target features x bf16 weights as they are (F16 = false),
// or fp16 context features x bf16 weights widened to fp16 while they are
// staged into LDS (F16 = true).
#include "dspine_device.hpp"
#include "dspine_internal.hpp"

namespace dspine {

template <int BM, int BN, int WM, int WN, bool F16>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tile_kernel(const TileGemmParams p) {
  constexpr int NT = 64 * WM * WN;
  constexpr int BK = 64, LDK = BK + 8;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int ACH = BM * (BK / 8) / NT;
  constexpr int BCH = BN * (BK / 8) / NT;
  static_assert(ACH * NT == BM * BK / 8 && BCH * NT == BN * BK / 8, "tile split");

  __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w % WM, wn = w / WM;
  const int tiles_m = (p.M + BM - 1) / BM;
  const int T = gridDim.x;
  int id = blockIdx.x;
  if (T % 8 == 0) id = (id % 8) * (T / 8) + id / 8;
  const int tm = id % tiles_m, tn = id / tiles_m;
  const int n0 = tn * BN;

  // weight rows of this tile (a tile never crosses a segment)
  int s = 0;
  while (s + 1 < p.nseg && n0 >= p.seg_rows0[s + 1]) ++s;
  const bf16_t* wbase = reinterpret_cast<const bf16_t*>(p.seg_ptr[s]) + (size_t)(n0 - p.seg_rows0[s]) * p.K;

  // activation row pointers of this thread's chunks (fixed across K)
  const bf16_t* arow[ACH];
#pragma unroll
  for (int q = 0; q < ACH; ++q) {
    const int c = tid + q * NT;
    const int m = tm * BM + c / (BK / 8);
    const bf16_t* r = nullptr;
    if (m < p.M) {
      if (p.pro == PRO_GATHER) {
        int g = 0;
        while (g + 1 < p.g_n && m >= p.g_row0[g + 1]) ++g;
        r = reinterpret_cast<const bf16_t*>(p.g_src[g]) + (size_t)(m - p.g_row0[g] + p.g_skip[g]) * p.lda;
      } else {
        r = reinterpret_cast<const bf16_t*>(p.a) + (size_t)m * p.lda;
      }
    }
    arow[q] = r;
  }

  u32x4 ra[ACH], rb[BCH];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int q = 0; q < ACH; ++q) {
      const int c = tid + q * NT;
      const int col = (c % (BK / 8)) * 8;
      ra[q] = arow[q] ? *reinterpret_cast<const u32x4*>(arow[q] + k0 + col) : u32x4{0, 0, 0, 0};
    }
    // weights are fragment-ordered: block i (16 rows), 32-K step ks holds 64
    // lane fragments (row i*16 + l%16, K 8*(l/16)..+8) in 1 KB
#pragma unroll
    for (int q = 0; q < BCH; ++q) {
      const int c = tid + q * NT;
      const int blk = c / 128, sub = (c / 64) % 2, l = c % 64;
      rb[q] = *reinterpret_cast<const u32x4*>(wbase + (size_t)blk * 16 * p.K + (size_t)(k0 / 32 + sub) * 512 + l * 8);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int q = 0; q < ACH; ++q) {
      const int c = tid + q * NT;
      *reinterpret_cast<u32x4*>(&sA[buf][(c / (BK / 8)) * LDK + (c % (BK / 8)) * 8]) = ra[q];
    }
#pragma unroll
    for (int q = 0; q < BCH; ++q) {
      const int c = tid + q * NT;
      const int blk = c / 128, sub = (c / 64) % 2, l = c % 64;
      *reinterpret_cast<u32x4*>(&sB[buf][(blk * 16 + (l & 15)) * LDK + sub * 32 + 8 * (l >> 4)]) =
          F16 ? bf16x8_to_f16x8(rb[q]) : rb[q];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const u32x4*>(
            &sA[buf][(wm * TM + i * 32 + (lane & 31)) * LDK + ks * 16 + 8 * (lane >> 5)]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const u32x4*>(
            &sB[buf][(wn * TN + j * 32 + (lane & 31)) * LDK + ks * 16 + 8 * (lane >> 5)]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma32<F16>(acc[i][j], af[i], bfr[j]);
    }
  };

  const int nk = p.K / BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  int buf = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) load_stage((kt + 1) * BK);
    compute(buf);
    if (more) store_stage(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // D[i = 8*(v/4) + 4*(lane/32) + v%4][n = lane%32]
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = tm * BM + wm * TM + i * 32 + 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
        const int n = n0 + wn * TN + j * 32 + (lane & 31);
        if (m < p.M) p.out[(size_t)m * p.ldo + n] = acc[i][j][v];
      }
}

hipError_t launch_gemm_tile(const TileGemmParams& p, int dtype, int num_cus, hipStream_t s) {
  (void)num_cus;
  if (dtype != DT_BF16) return hipErrorInvalidValue;
  constexpr int BM = 256, BN = 128;
  const int tiles = ((p.M + BM - 1) / BM) * (p.N / BN);
  if (p.a_bf16) hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, 2, 2, false>), dim3(tiles), dim3(256), 0, s, p);
  else hipLaunchKernelGGL((gemm_tile_kernel<BM, BN, 2, 2, true>), dim3(tiles), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dspine
