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
// Mapping: eight lanes per group, eight elements (two 16-byte loads) per
// lane, so a wave covers eight groups = 2 KB of contiguous input and writes
// 512 contiguous code bytes; the group max is three xor-shuffles inside the
// eight lanes.  One grid covers K and V.  This is a streaming kernel: 4 bytes
// read and ~1 byte written per element.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gqa_decode.h"

namespace {

constexpr int kAppThreads = 256;

struct AppendArgs {
  const float* src[2];      // k_new, v_new   [S][Tn][Hk][D]
  int8_t* codes[2];         // k, v           [S][Lmax][Hk][D]
  uint16_t* scales[2];      // k_scales, v_scales [S][Lmax][Hk][D/64]
  const int32_t* pos;       // [S]
  int64_t groups;           // groups per side = S * Tn * Hk * (D / 64)
  int S, Tn, Lmax, Hk, D;
};

__global__ __launch_bounds__(kAppThreads) void append_i8(AppendArgs a) {
  const int64_t gt = (int64_t)blockIdx.x * kAppThreads + threadIdx.x;
  const int sub = (int)(gt & 7);                 // lane within the group
  const int64_t grp_all = gt >> 3;
  if (grp_all >= 2 * a.groups) return;           // whole 8-lane groups exit together
  const int side = grp_all >= a.groups ? 1 : 0;
  const int64_t gidx = grp_all - side * a.groups;
  const int ng = a.D / 64;
  const int64_t row = gidx / ng;                 // (s, i, g) over [S][Tn][Hk]
  const int grp = (int)(gidx % ng);
  const int g = (int)(row % a.Hk);
  const int i = (int)((row / a.Hk) % a.Tn);
  const int s = (int)(row / ((int64_t)a.Hk * a.Tn));

  const float* src = a.src[side] + gidx * 64 + sub * 8;
  const float4 x0 = *reinterpret_cast<const float4*>(src);
  const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
  const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  m = fmaxf(m, __shfl_xor(m, 4, 64));

  const int64_t cell = (int64_t)a.pos[s] + i;
  if (cell < 0 || cell >= a.Lmax) return;        // a bad position only truncates
  const float d = __fdiv_rn(m, 127.0f);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float q = d > 0.f ? rintf(__fdiv_rn(x[e], d)) : 0.f;
    q = fminf(fmaxf(q, -127.f), 127.f);
    const uint32_t b = (uint32_t)(uint8_t)(int8_t)(int)q;
    w[e >> 2] |= b << (8 * (e & 3));
  }
  const int64_t drow = ((int64_t)s * a.Lmax + cell) * a.Hk + g;
  *reinterpret_cast<uint2*>(a.codes[side] + drow * a.D + grp * 64 + sub * 8) = make_uint2(w[0], w[1]);
  if (sub == 0)
    a.scales[side][drow * ng + grp] = __builtin_bit_cast(uint16_t, (_Float16)d);
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
  a.groups = (int64_t)S * Tn * Hk * (D / 64);
  a.S = S; a.Tn = Tn; a.Lmax = Lmax; a.Hk = Hk; a.D = D;
  const int64_t threads = 2 * a.groups * 8;
  const int64_t blocks = (threads + kAppThreads - 1) / kAppThreads;
  if (blocks > 0x7fffffff) return GQA_ERR_SHAPE;
  hipLaunchKernelGGL(append_i8, dim3((unsigned)blocks), dim3(kAppThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? GQA_OK : (int)e;
}
