// Quantize-on-append for the int8 KV cache on gfx950: new fp32 K and V rows
// are written into the cache as int8 codes with one f16 scale per 64-element
// group, the format the int8 attention reads.
//
// Per group of 64 consecutive elements x (FORWARD_MSL, kernel kv_append_q8,
// with the group widened from 32 to the cache's 64; qsa2.metal's cache
// format), in fp32 as the page computes:
//   d = max|x| / 127,  code = clamp(rint(x / d), -127, 127) if d > 0 else 0,
//   scale = f16(d).
// The divisions are IEEE round-to-nearest and rint rounds halves to even, so
// the codes match any other IEEE fp32 evaluation bit for bit.
//
// Mapping: one wave per workgroup, eight lanes per group, eight elements
// (two 16-byte loads) per lane, so a workgroup covers eight consecutive groups
// = 2 KB of contiguous input and writes 512 contiguous code bytes; the group
// max is three xor-shuffles inside the eight lanes.  The workgroups of one
// (side, sequence) pair walk that sequence's new rows in order.  The rows go
// to consecutive cells, and a cell holds [Hk][D] like a new row, so a group's
// place in the cache is its place in the input plus one per-sequence offset:
// no lane divides.  One grid covers K and V.  This is a streaming kernel: 4
// bytes read and ~1 byte written per element.
//
// Codes without a per-element IEEE division.  Let q = fl(x / d) be the IEEE
// quotient, r = v_rcp_f32(d) (within 1 ulp of 1 / d) and n = the code taken
// from y = fl(x * r): y clamped to [-127, 127] (v_med3) and rounded to
// nearest even by adding 1.5 * 2^23, whose sum's low byte is n in two's
// complement.  Since |x / d| <= 127 (1 + 2^-24), |x * r - x / d| < 1.6e-5 and
// |q - x / d| <= 2^-17, so |q - x * r| < 2.4e-5.  The code is accepted when
// the exact product (one FMA) lies within 0.4999 of n: then q lies within
// 0.4999 + 2.4e-5 < 1/2 of n, so clamp(rint(q)) = n (for |n| = 127 the clamp
// absorbs the side beyond it).  A lane with any code not accepted (ties,
// non-finite products) or with max |x| below 2^-100 (where d and 1 / d may
// leave the normal range) recomputes its eight codes from IEEE quotients:
// about 2e-4 of the elements of random data.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gqa_decode.h"

namespace {

constexpr int kAppGroupsPerBlock = 8;    // one wave: 8 groups x 8 lanes

struct AppendArgs {
  const float* src[2];      // k_new, v_new   [S][Tn][Hk][D]
  int8_t* codes[2];         // k, v           [S][Lmax][Hk][D]
  uint16_t* scales[2];      // k_scales, v_scales [S][Lmax][Hk][D/64]
  const int32_t* pos;       // [S]
  int64_t gps;              // groups per sequence and side = Tn * Hk * (D / 64)
  int bps;                  // workgroups per sequence and side
  int S, Tn, Lmax, Hk, D;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// IEEE code of x for the group scale d (d = 0: every code is 0)
__device__ __forceinline__ uint32_t code_ieee(float x, float d) {
  float q = d > 0.f ? rintf(__fdiv_rn(x, d)) : 0.f;
  q = fminf(fmaxf(q, -127.f), 127.f);
  return (uint32_t)(uint8_t)(int8_t)(int)q;
}

__global__ __launch_bounds__(64) void append_i8(AppendArgs a) {
  const int lane = threadIdx.x;
  const int sub = lane & 7;                      // lane within the group
  const int ss = blockIdx.x / a.bps;             // side * S + sequence
  const int blk = blockIdx.x - ss * a.bps;
  const int side = ss >= a.S ? 1 : 0;
  const int s = ss - side * a.S;
  const int64_t gpc = (int64_t)a.Hk * (a.D / 64);      // groups per cache cell
  const int64_t pos = a.pos[s];
  // groups [lo, hi) of the sequence land on cells inside [0, Lmax): a bad
  // position only truncates
  const int64_t lo = pos < 0 ? -pos * gpc : 0;
  int64_t hi = ((int64_t)a.Lmax - pos) * gpc;
  hi = hi < 0 ? 0 : (hi > a.gps ? a.gps : hi);
  const int64_t lg = (int64_t)blk * kAppGroupsPerBlock + (lane >> 3);

  f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = x0;
  if (lg < a.gps) {
    const f32x4* p = reinterpret_cast<const f32x4*>(a.src[side] + ((int64_t)s * a.gps + lg) * 64 + sub * 8);
    x0 = p[0];
    x1 = p[1];
  }
  const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  m = fmaxf(m, __shfl_xor(m, 4, 64));
  if (lg < lo || lg >= hi) return;               // whole 8-lane groups exit together

  const float d = __fdiv_rn(m, 127.0f);
  const float r = __builtin_amdgcn_rcpf(d);
  constexpr float kMagic = 12582912.0f;          // 1.5 * 2^23
  bool slow = !(m >= 0x1p-100f);
  uint32_t b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float z = __builtin_amdgcn_fmed3f(x[e] * r, -127.f, 127.f) + kMagic;
    slow |= !(fabsf(__builtin_fmaf(x[e], r, -(z - kMagic))) <= 0.4999f);
    b[e] = __builtin_bit_cast(uint32_t, z);
  }
  uint32_t w[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)   // low bytes of four sums -> one word
    w[c] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[4 * c + 3], b[4 * c + 2], 0x0c0c0400u),
                                 __builtin_amdgcn_perm(b[4 * c + 1], b[4 * c], 0x0c0c0400u),
                                 0x05040100u);
  if (slow) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
      w[c] = code_ieee(x[4 * c], d) | code_ieee(x[4 * c + 1], d) << 8 |
             code_ieee(x[4 * c + 2], d) << 16 | code_ieee(x[4 * c + 3], d) << 24;
  }
  const int64_t cg = ((int64_t)s * a.Lmax + pos) * gpc + lg;   // cache group index
  *reinterpret_cast<u32x2*>(a.codes[side] + cg * 64 + sub * 8) = u32x2{w[0], w[1]};
  if (sub == 0) a.scales[side][cg] = __builtin_bit_cast(uint16_t, (_Float16)d);
}

}  // namespace

extern "C" int gqa_decode_append_i8(const float* k_new, const float* v_new, const int32_t* pos,
                                    int8_t* k, int8_t* v, uint16_t* k_scales, uint16_t* v_scales,
                                    int S, int Tn, int Lmax, int Hk, int D, void* stream) {
  if (S < 1 || Tn < 0 || Lmax < 0 || Hk < 1) return GQA_ERR_SHAPE;
  if (D < 64 || D % 64 != 0) return GQA_ERR_HEAD_DIM;
  if (Tn == 0 || Lmax == 0) return GQA_OK;       // nothing to write
  if (!k_new || !v_new || !pos || !k || !v || !k_scales || !v_scales) return GQA_ERR_NULL;
  AppendArgs a;
  a.src[0] = k_new; a.src[1] = v_new;
  a.codes[0] = k; a.codes[1] = v;
  a.scales[0] = k_scales; a.scales[1] = v_scales;
  a.pos = pos;
  a.gps = (int64_t)Tn * Hk * (D / 64);
  a.S = S; a.Tn = Tn; a.Lmax = Lmax; a.Hk = Hk; a.D = D;
  const int64_t bps = (a.gps + kAppGroupsPerBlock - 1) / kAppGroupsPerBlock;
  const int64_t blocks = (int64_t)2 * S * bps;    // K and V, every sequence
  if (bps > 0x7fffffff || blocks > 0x7fffffff) return GQA_ERR_SHAPE;
  a.bps = (int)bps;
  hipLaunchKernelGGL(append_i8, dim3((unsigned)blocks), dim3(64), 0,
                     reinterpret_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? GQA_OK : (int)e;
}
