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
//    (global_load_lds_dwordx4): no registers are spent on staging.  Each
//    such load writes 1 KB of LDS, lane l at byte 16 l.
//  * Weights (already stored in MFMA operand order: 16 rows x 32 K per 1 KB
//    block) move in K slices of 32, one coalesced 1 KB copy per block.
//  * Activations move in half-units of 128 rows x 64 K (16 KB): one load
//    covers 8 rows x 128 B, so every L2 request is a whole cache line.  With
//    64 B row pieces (K slices of 32) the L2 sees half-line requests and the
//    loads run about a third slower.  Inside a 1 KB block, row r's 16-byte
//    chunk c sits at slot 8 r + (c ^ swz(r, block parity)); the XOR keeps a
//    wave's fragment reads free of bank conflicts under the lane grouping
//    of gfx950's 128-bit LDS reads (lanes 0-3, 12-15, 20-23, 24-27 share a
//    cycle, as do 4-11, 16-19, 28-31; likewise + 32).
//  * Ring: 6 activation half-units + 4 weight slices = 160 KB of LDS.  Step
//    kt issues half-unit kt + 4 and weight slice kt + 3 (the slots of
//    consumed data) and multiplies slice kt, one barrier per step.
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
  constexpr int BM = kTileM, BN = kTileN;
  constexpr int AH = 16 * 1024, BS = 16 * 1024;      // activation half-unit, weight slice
  __shared__ __attribute__((aligned(1024))) char smem[6 * AH + 4 * BS];
  char* const sa = smem;
  char* const sb = smem + 6 * AH;

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

  auto row_ptr = [&](int m) -> const uint16_t* {
    m = m < p.M ? m : p.M - 1;
    if (p.pro == PRO_GATHER) {
      int g = 0;
      while (g + 1 < p.g_n && m >= p.g_row0[g + 1]) ++g;
      return reinterpret_cast<const uint16_t*>(p.g_src[g]) + (size_t)(m - p.g_row0[g] + p.g_skip[g]) * p.lda;
    }
    return reinterpret_cast<const uint16_t*>(p.a) + (size_t)m * p.lda;
  };
  // wave w loads blocks w, w + 8 of every activation half-unit (rows 8 b ..
  // 8 b + 7 of the half; this lane: row r, chunk c) and weight row blocks
  // w, w + 8 of every slice
  const uint16_t* arow[2];
  long ahalf[2];                                   // elements from the first half's row to the second's
  const uint16_t* brow[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int b = w + 8 * q, r = lane >> 3, c = (lane & 7) ^ act_swz(r, b & 1);
    const int m0 = tm * BM + b * 8 + r;
    const uint16_t* r0 = row_ptr(m0);
    arow[q] = r0 + c * 8;
    ahalf[q] = ((intptr_t)row_ptr(m0 + 128) - (intptr_t)r0) / 2;   // rows may sit in different sources
    brow[q] = reinterpret_cast<const uint16_t*>(wbase) + (size_t)b * 16 * p.K + lane * 8;
  }
  const int nk = p.K / 32;                         // weight slices = activation half-units
  // Batch of step kt: activation half-unit kt + 4 (pair (kt + 4) / 2, rows
  // 128 ((kt + 4) & 1) ..) and weight slice kt + 3, clamped to the last one
  // at the end (the re-read lands in a free slot, keeping every batch at
  // four loads per wave).
  auto issue = [&](int kt, int aslot, int bslot) __attribute__((always_inline)) {
    const int a = kt + 4 < nk ? kt + 4 : nk - 1;
    const long off = (long)(a >> 1) * 64;
    char* da = sa + aslot * AH;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(arow[q] + ((a & 1) ? ahalf[q] : 0) + off),
                                       (lds_void*)(da + (w + 8 * q) * 1024), 16, 0, 0);
    const int bk = kt + 3 < nk ? kt + 3 : nk - 1;
    char* db = sb + bslot * BS;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(brow[q] + (size_t)bk * 512), (lds_void*)(db + (w + 8 * q) * 1024),
                                       16, 0, 0);
  };
  // fragment reads: lane l takes block 2 t + (l & 15) / 8, row l & 7, chunk
  // 4 h + l / 16 of the wave's half-unit, h = K half of the pair
  int aoff0, aoff1;
  {
    const int bb = (lane & 15) >> 3, r = lane & 7, c = lane >> 4;
    aoff0 = bb * 1024 + (r * 8 + (c ^ act_swz(r, bb))) * 16;
    aoff1 = bb * 1024 + (r * 8 + ((c + 4) ^ act_swz(r, bb))) * 16;
  }

  f32x4 acc[4][8];                                     // [n block][m block]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = f32x4{0, 0, 0, 0};

  // prologue: the batches of steps -4 .. -1 (half-units 0 .. 3, weight
  // slices 0 .. 2; step -4 has no weight slice)
#pragma unroll
  for (int q = 0; q < 2; ++q)
    __builtin_amdgcn_global_load_lds((const void*)arow[q], (lds_void*)(sa + (w + 8 * q) * 1024), 16, 0, 0);
  issue(-3, 1, 0);
  issue(-2, 2, 1);
  issue(-1, 3, 2);
  int aslot = 4, bslot = 3, cbase = 0;             // slots for step kt's batch; half-unit slot of pair kt / 2
  for (int kt = 0; kt < nk; ++kt) {
    // the batch of step kt - 3 (half-units up to pair kt / 2, weight slice
    // kt) has landed when at most the two later batches are outstanding
    wait_vmcnt<8>();
    __builtin_amdgcn_s_barrier();
    issue(kt, aslot, bslot);
    aslot = aslot == 5 ? 0 : aslot + 1;
    bslot = (bslot + 1) & 3;
    const char* at = sa + (cbase + wm) * AH + ((kt & 1) ? aoff1 : aoff0);
    const char* bt = sb + (kt & 3) * BS + wn * 4 * 1024 + lane * 16;
    // the 8 A fragments and B fragment 0, then per B fragment j: wait for
    // the reads so far, read fragment j + 1, multiply with fragment j
    u32x4 af[8], bw[4];
#pragma unroll
    for (int t = 0; t < 8; ++t) af[t] = *reinterpret_cast<const u32x4*>(at + t * 2048);
    bw[0] = *reinterpret_cast<const u32x4*>(bt);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      if (j + 1 < 4) bw[j + 1] = *reinterpret_cast<const u32x4*>(bt + (j + 1) * 1024);
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
    if (kt & 1) cbase = cbase == 4 ? 0 : cbase + 2;
  }
  wait_vmcnt<0>();                                 // no load into LDS outlives the workgroup

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

bool gemm_tile_fits(int n_seg, int k) { return n_seg > 0 && n_seg % kTileN == 0 && k > 0 && k % 64 == 0; }

hipError_t launch_gemm_tile(const TileGemmParams& p, int dtype, int num_cus, hipStream_t s) {
  (void)num_cus;
  if (dtype != DT_BF16 || p.M < 1 || p.K % 64 != 0 || p.N % kTileN != 0 || p.ldo % 4 != 0) return hipErrorInvalidValue;
  for (int i = 1; i < p.nseg; ++i)
    if (p.seg_rows0[i] % kTileN != 0) return hipErrorInvalidValue;      // a tile never crosses a segment
  const int tiles = ((p.M + kTileM - 1) / kTileM) * (p.N / kTileN);
  if (p.a_bf16) DSPINE_LAUNCH(gemm_tile_kernel<false>, dim3(tiles), dim3(512), 0, s, p);
  else DSPINE_LAUNCH(gemm_tile_kernel<true>, dim3(tiles), dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace dspine
