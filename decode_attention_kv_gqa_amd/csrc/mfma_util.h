// Register types and wave-level helpers shared by the attention kernels on
// the gfx950 matrix cores (v_mfma_f32_16x16x32_f16): f16 hi + lo splitting
// of fp32 operands, cross-lane reductions with the permlane swaps, and
// range-checked buffer resources for the cache reads.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gqa_kern {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

#define GQA_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// fp32 -> f16 high part and the f16 of what it leaves out: hi + lo keeps
// ~22 bits of x.
__device__ __forceinline__ void split_hi_lo(const float (&x)[8], half8& hi, half8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const _Float16 h = (_Float16)x[e];
    hi[e] = h;
    lo[e] = (_Float16)(x[e] - (float)h);
  }
}

// Power of two that normalises a query row: with m = max |q| of the row and
// qscale = qmant * 2^qexp, q * qmant * 2^(15 - e) with e = exponent of m
// (clamped to [-100, 128] so the factor stays a normal float) has its largest
// magnitude in [2^13, 2^15).  Returns that factor; *rs = 2^(e + qexp - 15)
// turns a score of normalised rows back into q . k * qscale (exponent
// clamped to the normal range; only rows with max |q * qscale| below
// ~2^-111, whose scores are ~0 anyway, reach the clamp).
__device__ __forceinline__ float q_row_factor(float m, float qmant, int qexp, float* rs) {
  int e = __builtin_amdgcn_frexp_expf(m);
  e = e < -100 ? -100 : (e > 128 ? 128 : e);
  int es = e + qexp - 15;
  es = es < -126 ? -126 : (es > 127 ? 127 : es);
  *rs = __builtin_amdgcn_ldexpf(1.0f, es);
  return __builtin_amdgcn_ldexpf(qmant, 15 - e);
}

// Largest value of a 5-bit field (0..31) over the wave, by bisection on
// ballots: five wave votes, no LDS round trip.
__device__ __forceinline__ int wave_max_u5(int x) {
  int m = 0;
#pragma unroll
  for (int b = 4; b >= 0; --b) {
    const int c = m | (1 << b);
    if (__any(x >= c)) m = c;
  }
  return m;
}

// Butterfly steps across lane distance 16 and 32 of a wave64 with the gfx950
// permlane swaps (VALU, no LDS round trip).  With both operands equal,
// permlane16_swap returns (rows 0,0,2,2) and (rows 1,1,3,3) of x, and
// permlane32_swap returns (low, low) and (high, high) halves, so combining
// the two results gives every lane the reduction over its xor-16 / xor-32
// partner.  The two results pass through an empty asm statement: without it
// this compiler folds the second result into the first when both operands
// are the same value (it emitted r0 + r0 for r0 + r1).
__device__ __forceinline__ void swap16(float x, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  uint32_t r0 = r[0], r1 = r[1];
  asm volatile("" : "+v"(r0), "+v"(r1));
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  uint32_t r0 = r[0], r1 = r[1];
  asm volatile("" : "+v"(r0), "+v"(r1));
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float max_x16(float x) { float a, b; swap16(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float max_x32(float x) { float a, b; swap32(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float sum_x16(float x) { float a, b; swap16(x, a, b); return a + b; }
__device__ __forceinline__ float sum_x32(float x) { float a, b; swap32(x, a, b); return a + b; }

__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Cache policy of the K/V row loads: non-temporal (each row is read once per
// split and never again in the step).
constexpr int kNT = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer: stride 0, num_records in bytes; reads past the end return 0
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

}  // namespace gqa_kern
