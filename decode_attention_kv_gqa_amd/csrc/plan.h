// Host-side argument checks and launch planning for the decode-attention
// kernels.  Pure C++ (no HIP calls), so it can be exercised without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

#include "gqa_decode.h"

namespace gqa {

// Largest number of query rows one workgroup holds.  A workgroup serves the
// query rows of one KV head (all G heads of the group, times the T tokens of
// a dense window), so K/V rows are streamed once for all of them; groups
// with more rows than this are cut into row blocks that each stream K/V.
// 64 rows (four 16-row MFMA blocks) for head_dim 64 and 128, whose
// accumulators fit one wave per SIMD; 32 for head_dim 256 and the
// TurboQuant kernel.
constexpr int kMaxRowsPerBlock = 64;

struct Shape {
  int S, T, Lmax, B, H, Hk, D;
  bool ids;   // gather through a budget of cell ids
  bool i8;    // int8 rows with f16 group scales
  bool tq = false;   // TurboQuant-compressed cache (gqa_decode_attn_tq)
};

inline int max_rows_per_block(const Shape& s) { return (!s.tq && s.D <= 128) ? 64 : 32; }

// Positions a split can cover: min(B, Lmax) with ids, else Lmax.
inline int64_t width_cap(const Shape& s) {
  if (s.ids) return s.B < s.Lmax ? s.B : s.Lmax;
  return s.Lmax;
}

// Most pieces per (KV head, row block) of the balanced partition.
constexpr int kMaxPieces = 1 << 16;

// A negative chunk selects the balanced partition with -chunk pieces per
// (KV head, row block): the dense windows of all sequences, laid end to end,
// cut into equal pieces (no ids; the total window, at most S * Lmax cells,
// below 2^31).
// (The total span, windows rounded up to 128-cell units plus their pad
// cells, stays below 2^31: the pad is at most 1024 cells.)
inline bool balanced_ok(const Shape& s, int chunk) {
  return chunk < 0 && -(int64_t)chunk <= kMaxPieces && !s.ids && !s.tq &&
         (int64_t)s.S * ((int64_t)s.Lmax + 1152) < ((int64_t)1 << 31);
}

// Partial slots per query row: the split count, or the piece count of the
// balanced partition (a sequence's partials fill its first slots).
inline int64_t num_splits(const Shape& s, int chunk) {
  int64_t w = width_cap(s);
  if (w <= 0) return 0;
  if (chunk < 0) return -(int64_t)chunk;
  return (w + chunk - 1) / chunk;
}

// Query rows served by one (sequence, KV head[, token]) unit.  64-bit: the
// shape checks use it before they have bounded G * T (check_shape then
// guarantees S * T * H <= 2^31 - 1, so after it the value fits an int).
inline int64_t rows_per_unit(const Shape& s) {
  const int64_t G = s.H / s.Hk;
  return s.ids ? G : G * s.T;
}

inline int64_t row_blocks(const Shape& s) {
  const int m = max_rows_per_block(s);
  return (rows_per_unit(s) + m - 1) / m;
}

// Rows per block rounded up to the kernel instance (4, 8, 16, 32 or 64).
inline int block_rows(const Shape& s) {
  int64_t R = rows_per_unit(s);
  if (R > max_rows_per_block(s)) R = max_rows_per_block(s);
  if (R <= 4) return 4;
  if (R <= 8) return 8;
  if (R <= 16) return 16;
  if (R <= 32) return 32;
  return 64;
}

// Largest split the kernels accept: one split's K (or V) rows of a KV head
// span chunk * Hk * row bytes, addressed with 31-bit buffer offsets.
// In gather mode the split's cell ids are staged in LDS: at most
// kMaxIdsChunk cells per split.
constexpr int64_t kMaxIdsChunk = 4096;
inline int64_t max_chunk(const Shape& s) {
  const int64_t row = (int64_t)s.Hk * s.D * (s.i8 ? 1 : 2);
  const int64_t m = ((int64_t)1 << 31) / row - 1;
  return s.ids && m > kMaxIdsChunk ? kMaxIdsChunk : m;
}

// Waves per attention workgroup.  Each wave streams its own 32-cell tiles
// of the split (wave w: tiles w, w+NW, ...), so a split of at most two tiles
// gets a one-wave workgroup (no idle waves, no cross-wave combine); longer
// splits get four waves, one per SIMD.
inline int waves_per_block(const Shape& s, int chunk) {
  (void)s;
  return (chunk > 0 && chunk <= 64) ? 1 : 4;
}

int check_shape(const Shape& s);               // GQA_OK or GQA_ERR_*
int auto_chunk(const Shape& s);                // > 0, or GQA_ERR_*
int auto_pieces(const Shape& s);               // -P (balanced partition), or GQA_ERR_*
size_t part_bytes(const Shape& s, int chunk);  // 0 on bad arguments

// Offsets (in floats) of the two regions of the partial workspace:
//   o  [S][T][H][P][D]   unnormalised outputs
//   ml [S][T][H][P][2]   running max (base-2 domain) and running sum
inline size_t part_o_floats(const Shape& s, int64_t P) {
  return (size_t)s.S * s.T * s.H * (size_t)P * s.D;
}
// Balanced partition: after the two regions, n [S] int32, the partial slots
// each sequence fills (written by the attention call, read by the merge).
inline size_t flat_n_offset_floats(const Shape& s, int64_t P) {
  return (size_t)s.S * s.T * s.H * (size_t)P * (s.D + 2);
}

// Virtual cells charged for each non-empty window in the balanced
// partition: the cost of starting a sequence inside a workgroup, as the
// cells that stream in that time.  f16 rows: 64 KB of K + V rows of one KV
// head per sequence start (f16 batch, head_dim 128: 32 KB 58.2-58.5, 64 KB
// 57.5-57.6, 128 KB 57.6-57.7 us).  int8 rows, whose tiles cost more
// arithmetic to drain and refill: 256 cells whatever the head_dim (int8
// batch, head_dim 256: 128 cells 54.9, 256 cells 53.3-53.6, 384 cells
// 53.3-53.8 us; head_dim 128: 256 cells 43.2, 512 cells 45.0-45.2, 768
// cells 47.8-47.9 us).
constexpr int64_t kFlatPadBytes = 64 * 1024;
constexpr int64_t kFlatPadCellsI8 = 256;
inline int flat_pad_cells(const Shape& s) {
  const int64_t cell = 4 * (int64_t)s.D;      // K + V bytes of one KV head, f16
  const int64_t pad = s.i8 ? kFlatPadCellsI8 : kFlatPadBytes / cell;
  return (int)((pad + 127) / 128 * 128);      // whole 128-cell units
}

}  // namespace gqa
