// Shared device helpers and kernel argument blocks.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace gqa_kern {

__device__ __forceinline__ float h2f(uint16_t bits) {
  return (float)__builtin_bit_cast(_Float16, bits);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Arguments of the chunk kernel.  Query rows of a unit (one sequence, one KV
// head and, with ids, one token) are r = t * G + j (dense: all T tokens) or
// r = j (ids: the grid's token), j = query head within the group.
struct AttnArgs {
  const float* q;
  const void* k;
  const void* v;
  const uint16_t* ksc;
  const uint16_t* vsc;
  const int32_t* ids;
  const int32_t* seq_lens;
  float* part_o;     // [S][T][H][P][D]
  float* part_ml;    // [S][T][H][P][2]  (running max in base-2 units, running sum)
  int S, T, Lmax, B, H, Hk, G, R, nrb, P, chunk;
  int seq_fast;      // 1: grid order with the sequence varying fastest, else the KV head
  float qscale;      // scale * log2(e)
  float qmant;       // qscale = qmant * 2^qexp, |qmant| in [0.5, 1) (0 when qscale is 0)
  int qexp;
};

// Arguments of the merge kernel: one output row per workgroup, P partial
// slots per row, every slot written by the attention call.
struct MergeArgs {
  const float* part_o;     // [rows][P][D]
  const float* part_ml;    // [rows][P][2]
  float* out;              // [rows][D]
  const float* gate;       // row r's gate at gate + r * gate_stride, or null (no gate)
  int64_t gate_stride;
  int P;
};

}  // namespace gqa_kern
