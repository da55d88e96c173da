// Device-side helpers shared by the DSpine HIP kernels (gfx950 / CDNA4).
//
// MFMA lane layouts used throughout (checked on hardware):
//   v_mfma_f32_16x16x32_{bf16,f16}: lane l holds A[i = l%16][k = 8*(l/16) + j]
//     and B[k = 8*(l/16) + j][n = l%16], j = 0..7; result element v of lane l
//     is D[i = 4*(l/16) + v][n = l%16].
//   v_mfma_f32_16x16x4_f32: one element per lane, A[i = l%16][k = l/16].  Eight
//     of them consume the same 8-element lane fragment as one 16x16x32 op
//     (element j of every lane forms step j); the order of a dot product's
//     terms is free, so both paths share one fragment layout.
//   v_mfma_f32_32x32x16_bf16: A[i = l%32][k = 8*(l/32) + j]; element v of the
//     result is D[i = 8*(v/4) + 4*(l/32) + v%4][n = l%32].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspine {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };
struct fp8_t { uint8_t bits; };      // OCP FP8 E4M3 code (the row-scaled LM head copy)

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// float -> the nearest bfloat16 value (RNE), as a float
__device__ __forceinline__ float round_bf16(float f) { return bf16_bits_to_f32(f32_to_bf16_bits(f)); }
// Sum of squares of four values in one fixed evaluation (explicit fused
// multiply-adds): the kernels whose row statistics must agree bit for bit
// (a GEMM epilogue and the fused bridge) do not depend on how the compiler
// would contract the plain expression in each of them
__device__ __forceinline__ float sumsq4(float a, float b, float c, float d) {
  return __builtin_fmaf(d, d, __builtin_fmaf(c, c, __builtin_fmaf(b, b, a * a)));
}
// float -> IEEE half bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// Model dtype -> activation (MFMA operand) type.  BF16 models use FP16
// operands: bf16 weights widen to fp16 exactly, and an 11-bit significand
// keeps the operand rounding 4x below bf16's at the same MFMA rate.
template <typename TW> struct ActOf;

// Element traits: the storage type of weights/activations for each model dtype.
// Global-address-space view of a pointer.  Loads through it are global_load
// (vector-memory counter only); loads through a generic pointer become
// flat_load, which also counts on the LDS counter, so any later LDS wait
// would drain every in-flight global load with it.
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;
template <typename T>
__device__ __forceinline__ gptr<T> as_global(const T* p) {
  return (gptr<T>)(p);
}
__device__ __forceinline__ u32x4 gload16(gptr<void> p) { return *(gptr<u32x4>)(p); }
// A load of data read once (streamed weights): non-temporal, so that the L2
// keeps the lines that are re-read (the activations every workgroup reads)
// instead of the stream's
__device__ __forceinline__ u32x4 gload16_nt(gptr<void> p) { return __builtin_nontemporal_load((gptr<u32x4>)(p)); }

template <typename T> struct Elt;
template <> struct Elt<float> {
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  __device__ static __forceinline__ float gload(gptr<float> p, size_t i) { return p[i]; }
  __device__ static __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elt<f16_t> {
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ float load(const f16_t* p, size_t i) { return f16_bits_to_f32(p[i].bits); }
  __device__ static __forceinline__ float gload(gptr<f16_t> p, size_t i) { return f16_bits_to_f32(p[i].bits); }
  __device__ static __forceinline__ void store(f16_t* p, size_t i, float v) { p[i].bits = f32_to_f16_bits(v); }
};
template <> struct Elt<fp8_t> {    // (the FP8 head has no gain, bias or codebook operand)
  static constexpr int kBytes = 1;
  __device__ static __forceinline__ float load(const fp8_t*, size_t) { return 0.f; }
  __device__ static __forceinline__ float gload(gptr<fp8_t>, size_t) { return 0.f; }
};
template <> struct Elt<bf16_t> {
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ float load(const bf16_t* p, size_t i) {
    return bf16_bits_to_f32(p[i].bits);
  }
  __device__ static __forceinline__ float gload(gptr<bf16_t> p, size_t i) { return bf16_bits_to_f32(p[i].bits); }
  __device__ static __forceinline__ void store(bf16_t* p, size_t i, float v) {
    p[i].bits = f32_to_bf16_bits(v);
  }
};


// ---------------------------------------------------------------------------
// MFMA fragments: 8 consecutive K elements of one row, per lane.
// ---------------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
  u32x4 v;  // 8 bf16
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void gload(gptr<bf16_t> p) { v = gload16((gptr<void>)p); }
  __device__ __forceinline__ void gload_nt(gptr<bf16_t> p) { v = gload16_nt((gptr<void>)p); }
  __device__ __forceinline__ void zero() { v = u32x4{0, 0, 0, 0}; }
};
template <> struct Frag<float> {
  u32x4 v[2];  // 8 floats
  __device__ __forceinline__ void load(const float* p) {
    v[0] = reinterpret_cast<const u32x4*>(p)[0];
    v[1] = reinterpret_cast<const u32x4*>(p)[1];
  }
  __device__ __forceinline__ void gload(gptr<float> p) {
    v[0] = gload16((gptr<void>)p);
    v[1] = gload16((gptr<void>)(p + 4));
  }
  __device__ __forceinline__ void gload_nt(gptr<float> p) {
    v[0] = gload16_nt((gptr<void>)p);
    v[1] = gload16_nt((gptr<void>)(p + 4));
  }
  __device__ __forceinline__ void zero() { v[0] = u32x4{0, 0, 0, 0}; v[1] = v[0]; }
};

template <> struct Frag<f16_t> {
  u32x4 v;  // 8 halves
  __device__ __forceinline__ void load(const f16_t* p) { v = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void zero() { v = u32x4{0, 0, 0, 0}; }
};
// 8 E4M3 codes (8 bytes) of one lane's fragment
template <> struct Frag<fp8_t> {
  uint32_t v[2];
  __device__ __forceinline__ void gload(gptr<fp8_t> p) {
    const uint64_t q = *(gptr<uint64_t>)(p);
    v[0] = (uint32_t)q;
    v[1] = (uint32_t)(q >> 32);
  }
  __device__ __forceinline__ void gload_nt(gptr<fp8_t> p) {
    const uint64_t q = __builtin_nontemporal_load((gptr<uint64_t>)(p));
    v[0] = (uint32_t)q;
    v[1] = (uint32_t)(q >> 32);
  }
  __device__ __forceinline__ void zero() { v[0] = v[1] = 0u; }
};
template <> struct ActOf<bf16_t> { using type = f16_t; };
template <> struct ActOf<float> { using type = float; };

// two bf16 (one dword) -> two fp16 (one dword); exact for |x| in the fp16
// normal range, round toward zero below it.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t d) {
  const float lo = __uint_as_float(d << 16);
  const float hi = __uint_as_float(d & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}
// Full-line activation blocks (8 rows x 128 bytes of 16-bit values, 1 KB of
// LDS): row r's 16-byte chunk c sits at slot 8 r + (c ^ act_swz(r, bb)), bb
// the block's parity.  The XOR keeps the MFMA fragment reads (lane l: row
// l & 7 of block 2 t + (l & 15) / 8, chunk 4 h + l / 16) free of bank
// conflicts under the lane grouping of gfx950's 128-bit LDS reads (lanes
// 0-3, 12-15, 20-23, 24-27 share a cycle, as do 4-11, 16-19, 28-31;
// likewise + 32).
__device__ __forceinline__ int act_swz(int r, int bb) { return (((r >> 1) & 1) << 2) ^ ((r >> 2) * 3) ^ (bb << 1); }

__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  return u32x4{bf16x2_to_f16x2(v[0]), bf16x2_to_f16x2(v[1]), bf16x2_to_f16x2(v[2]), bf16x2_to_f16x2(v[3])};
}
// Two E4M3 codes (bytes 0 and 1 of d) -> two fp16 whose values are the codes'
// values / 256, exactly: the sign moves to bit 15 and the 4 exponent + 3
// fraction bits to bits 13..7, so exponent field e (bias 7) reads as e with
// bias 15 (a factor 2^-8) and a subnormal code m (m/8 x 2^-6) as the fp16
// subnormal m x 2^-17.  The 256 goes into the row scale.
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2_div256(uint32_t d) {
  const uint32_t t = (d & 0xffu) | ((d & 0xff00u) << 8);      // byte 0 -> bits 0..7, byte 1 -> 16..23
  return ((t << 7) & 0x3f803f80u) | ((t << 8) & 0x80008000u);
}
__device__ __forceinline__ u32x4 e4m3x8_to_f16x8_div256(const uint32_t v[2]) {
  return u32x4{e4m3x2_to_f16x2_div256(v[0]), e4m3x2_to_f16x2_div256(v[0] >> 16),
               e4m3x2_to_f16x2_div256(v[1]), e4m3x2_to_f16x2_div256(v[1] >> 16)};
}

// weight fragment in the MFMA operand type
template <typename TA, typename TW> struct AsOperand;
template <typename T> struct AsOperand<T, T> {
  __device__ static __forceinline__ Frag<T> cvt(const Frag<T>& w) { return w; }
};
template <> struct AsOperand<f16_t, fp8_t> {
  __device__ static __forceinline__ Frag<f16_t> cvt(const Frag<fp8_t>& w) {
    Frag<f16_t> r;
    r.v = e4m3x8_to_f16x8_div256(w.v);
    return r;
  }
};
template <> struct AsOperand<f16_t, bf16_t> {
  __device__ static __forceinline__ Frag<f16_t> cvt(const Frag<bf16_t>& w) {
    Frag<f16_t> r;
    r.v = bf16x8_to_f16x8(w.v);
    return r;
  }
};

// acc += A_frag (rows i) x B_frag (cols n), 16x16 tile, 32 K elements.
__device__ __forceinline__ void mma16(f32x4& acc, const Frag<f16_t>& a, const Frag<f16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a.v),
                                               __builtin_bit_cast(f16x8, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                __builtin_bit_cast(bf16x8, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.v[h][j]),
                                                __uint_as_float(b.v[h][j]), acc, 0, 0, 0);
}

// acc += A (32 rows) x B (32 cols), 16 K elements (8 per lane).
template <bool F16>
__device__ __forceinline__ void mma32(f32x16& acc, const u32x4& a, const u32x4& b) {
  if constexpr (F16)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  else
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// Sum over a block of NT threads (NT multiple of 64); `red` holds NT/64 floats.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += red[i];
  __syncthreads();
  return s;
}

// LDS address space (the destination of direct-to-LDS loads)
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt with only the vector-memory count set (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt and lgkmcnt at their "no wait" maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------------------
// Cross-workgroup handoff of partial results (last arriver finishes).
//
// Each XCD has its own L2, so a plain store from one workgroup need not be
// visible to a workgroup on another XCD.  An agent-scope release/acquire
// fence pair would write back and invalidate a whole L2 per handoff, which
// stalls every wave of that XCD.  Instead the partials travel with
// agent-scope relaxed atomic stores and loads (global_store/global_load with
// the sc1 bit: written through to, and read from, the device coherence
// point), the writer waits until its own stores have completed before it
// counts its arrival, and the counter is an agent-scope atomic.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_coherent(float* p, const f32x4& v) {
  uint64_t* q = reinterpret_cast<uint64_t*>(p);
  const uint64_t a = ((uint64_t)__float_as_uint(v[1]) << 32) | __float_as_uint(v[0]);
  const uint64_t b = ((uint64_t)__float_as_uint(v[3]) << 32) | __float_as_uint(v[2]);
  __hip_atomic_store(q, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 load_coherent4(const float* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return f32x4{__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
               __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32))};
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed (its
// write-through stores included).  The empty asm keeps the compiler from
// moving memory operations across the wait.
__device__ __forceinline__ void drain_own_stores() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ uint32_t count_arrival(uint32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_counter(uint32_t* counter) {
  __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// a3: visibility rule shared by the attention kernel and the debug export.
// [NIF, draft attention]: a key at position p is visible to the query at q
// iff |p - q| < S for a local layer (S > 0); a full layer (S == 0) sees
// every populated key.  Context keys are positions [0, F); the block rows
// sit at F + i.  With block_causal, block key j is hidden from rows i < j.
// ---------------------------------------------------------------------------
// first context position visible to block row i (equals F when none)
__device__ __forceinline__ int64_t ctx_row_lo(int64_t F, int S, int i) {
  if (S == 0) return 0;
  int64_t lo = F + i - S + 1;
  if (lo < 0) lo = 0;
  return lo < F ? lo : F;
}
__device__ __forceinline__ bool block_key_visible(int S, int causal, int i, int j) {
  const int d = i > j ? i - j : j - i;
  if (S > 0 && d >= S) return false;
  if (causal && j > i) return false;
  return true;
}
// ring slot of a stored position: p mod S for a local layer, p for a full one
__device__ __forceinline__ int64_t ring_slot(int64_t p, int S) { return S > 0 ? p % S : p; }

// Per-row scale of a row with sum of squares S (the SCALE_* modes of the
// streamed GEMM and the row pre-scale kernel), rows of width n.
__device__ __forceinline__ float row_scale(int mode, float S, float n, float eps, float code_scale, bool anchor) {
  switch (mode) {
    case 1: return rsqrtf(S / n + eps);                              // plain RMSNorm
    case 2: return 1.f / (sqrtf(S / n) + eps);                       // bridge read 1/(rho+eps)
    case 3: return anchor ? 1.f : code_scale / (sqrtf(S) + eps);     // bridge code
    case 4: return sqrtf(S / n);                                     // rho
    default: return 1.f;
  }
}

__device__ __forceinline__ float silu(float x) { return x / (1.f + __expf(-x)); }
__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

}  // namespace dspine
