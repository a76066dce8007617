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

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const int y = __shfl_xor(x, o, 64);
    x = y < x ? y : x;
  }
  return x;
}

__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const int y = __shfl_xor(x, o, 64);
    x = y > x ? y : x;
  }
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan_i(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Balanced partition of dense windows (a negative chunk in the C ABI).  The
// windows w_s = clamp(seq_lens[s], 0, Lmax) of all sequences are laid end to
// end, each non-empty one preceded by `pad` virtual cells that stand for the
// cost of starting a sequence inside a workgroup (its query rows staged, its
// first tile's latency, its partial written), so a piece's cost is its
// cells plus its sequence starts.  The total, W = sum over non-empty windows
// of (pad + w_s) < 2^31, is cut into Pe = min(P, W) pieces of near-equal
// length: piece j = [flat_bound(j), flat_bound(j + 1)) with flat_bound(j) =
// floor(j W / Pe), so no piece is empty.  Each KV head (and row block) is cut
// the same way; a piece yields one partial per sequence whose real cells it
// touches.
__device__ __forceinline__ int flat_window(int seq_len, int Lmax) {
  return seq_len < 0 ? 0 : (seq_len > Lmax ? Lmax : seq_len);
}
// The concatenation is cut in units of kFlatQ cells (a round of 32-cell
// tiles over four waves): pads are whole units and windows are rounded up to
// whole units, so sequences start on unit boundaries and a piece boundary
// inside a sequence never splits a round of tiles.
constexpr int kFlatQ = 128;
// Cells a window takes in the concatenation: its pad and its cells rounded
// up to whole units, or none.
__device__ __forceinline__ int flat_span(int seq_len, int Lmax, int pad) {
  const int w = flat_window(seq_len, Lmax);
  return w > 0 ? (w + kFlatQ - 1) / kFlatQ * kFlatQ + pad : 0;
}
// Piece j of Pe over a span of W cells (both in whole units).
__device__ __forceinline__ int flat_bound(int j, int W, int Pe) {
  return (int)((int64_t)j * (W / kFlatQ) / Pe) * kFlatQ;
}
// The piece holding position x in [0, W): the largest j with flat_bound(j)
// <= x.
__device__ __forceinline__ int flat_piece(int x, int W, int Pe) {
  const int64_t Wu = W / kFlatQ;
  return (int)(((int64_t)(x / kFlatQ + 1) * Pe + Wu - 1) / Wu) - 1;
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
  int flat;          // 1: balanced partition, P pieces per (KV head, row block)
  int wide;          // gather mode: 1 when a sequence's rows of all KV heads span >= 2^31 bytes
  int flat_pad;      // balanced partition: virtual cells before each non-empty window
  int* flat_n;       // balanced partition: [S] partial slots each sequence fills
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
  // balanced partition (flat != 0): row r belongs to sequence r / TH, whose
  // partials fill its first flat_n[r / TH] slots (written by the attention
  // call)
  int flat;
  const int32_t* flat_n;
  int TH;
};

}  // namespace gqa_kern
