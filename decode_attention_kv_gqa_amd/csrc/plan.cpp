// Host-side argument checks and launch planning (no HIP calls).
#include "plan.h"

#include <cstdint>

namespace gqa {

int check_shape(const Shape& s) {
  if (s.S < 1 || s.T < 1 || s.H < 1 || s.Hk < 1 || s.Lmax < 0) return GQA_ERR_SHAPE;
  if (s.H % s.Hk != 0) return GQA_ERR_GROUP;
  if (s.D != 64 && s.D != 128 && s.D != 256) return GQA_ERR_HEAD_DIM;
  if (s.ids && s.B < 1) return GQA_ERR_BUDGET;
  // The merge grid has one workgroup per output row: S * T * H of them
  // (bounded in two steps, each product below 2^62).
  const int64_t st = (int64_t)s.S * s.T;
  if (st > 0x7fffffff || st * s.H > 0x7fffffff) return GQA_ERR_SHAPE;
  // The attention grid is 1-D: S * Hk * row blocks (* T when gathering)
  // workgroups per split (below S * T * H + S * Hk, so no overflow here).
  const int64_t units = (int64_t)s.S * s.Hk * row_blocks(s) * (s.ids ? s.T : 1);
  if (units > 0x7fffffff) return GQA_ERR_SHAPE;
  return GQA_OK;
}

// Cells per split.  The attention grid is S * Hk * row-blocks (* T with ids)
// units times the split count.  Long splits stream best: one four-wave
// workgroup per compute unit (256 of them), each running through a long
// split with its K/V pipeline full, beats more and shorter workgroups that
// share a compute unit.  So the split is sized for about 256 workgroups
// when every sequence is full length, but at most an eighth of the window,
// so that batches of uneven lengths (unknown on the host) still spread over
// the compute units; and at least 64 cells.
int auto_chunk(const Shape& s) {
  int rc = check_shape(s);
  if (rc != GQA_OK) return rc;
  // The TurboQuant kernel is bound by decode latency, not by the stream:
  // eight of its workgroups per compute unit (four waves per SIMD) hide it
  // (int8-shaped 128K cache, 8 KV heads: 292 us at one workgroup per unit,
  // 195 us at eight).
  const int64_t kTargetWorkgroups = s.tq ? 2048 : 256;
  const int64_t kMinSplitsPerUnit = 8;
  const int64_t kMinChunk = 64;
  int64_t W = width_cap(s);
  if (W <= 0) return (int)kMinChunk;
  int64_t units = (int64_t)s.S * s.Hk * row_blocks(s) * (s.ids ? s.T : 1);
  int64_t chunk = (W * units + kTargetWorkgroups - 1) / kTargetWorkgroups;
  const int64_t eighth = (W + kMinSplitsPerUnit - 1) / kMinSplitsPerUnit;
  if (chunk > eighth) chunk = eighth;
  if (chunk < kMinChunk) chunk = kMinChunk;
  chunk = (chunk + 63) / 64 * 64;
  const int64_t cap = max_chunk(s) / 64 * 64;
  if (chunk > cap) chunk = cap;
  return (int)chunk;
}

// Pieces per (KV head, row block) of the balanced partition: one four-wave
// workgroup per compute unit (256 of them), measured best on uneven batches
// (f16 batch at 32 pieces per KV head: 57.5 us against 60.1 at 64 and
// 61.7 at 28), rounded down to a multiple of the 8 XCDs when that is at
// least 8.  Returned negated, as the chunk argument that selects it.
int auto_pieces(const Shape& s) {
  int rc = check_shape(s);
  if (rc != GQA_OK) return rc;
  if (s.ids || s.tq) return GQA_ERR_CHUNK;       // the partition covers dense windows
  const int64_t units = (int64_t)s.Hk * row_blocks(s);
  int64_t P = 256 / units;
  if (P >= 8) P = P / 8 * 8;
  if (P < 1) P = 1;
  if (P > kMaxPieces) P = kMaxPieces;
  if (!balanced_ok(s, (int)-P)) return GQA_ERR_CHUNK;
  return (int)-P;
}

size_t part_bytes(const Shape& s, int chunk) {
  if (chunk == 0 || (chunk < 0 && !balanced_ok(s, chunk)) || check_shape(s) != GQA_OK) return 0;
  const int64_t P = num_splits(s, chunk);
  // rows (< 2^31) x splits (< 2^31) x (D + 2) floats: computed in 128 bits;
  // a workspace beyond half the address space is refused (0), never wrapped
  unsigned __int128 b = (unsigned __int128)((int64_t)s.S * s.T * s.H) * (uint64_t)P *
                        (uint64_t)(s.D + 2) * sizeof(float);
  // balanced partition: the per-sequence slot counts follow, 16-byte rounded
  if (chunk < 0) b += ((uint64_t)s.S * 4 + 15) / 16 * 16;
  if (b > (unsigned __int128)(SIZE_MAX >> 1)) return 0;
  return (size_t)b;
}

}  // namespace gqa

extern "C" {

size_t gqa_decode_part_bytes(int S, int T, int Lmax, int B, int H, int D, int chunk) {
  // Hk does not change the workspace size; H is a valid stand-in here.
  gqa::Shape s{S, T, Lmax, B, H, H, D, B > 0, false};
  return gqa::part_bytes(s, chunk);
}

int gqa_decode_auto_chunk(int S, int T, int Lmax, int B, int H, int Hk, int D, int kv_kind) {
  if (kv_kind < 0 || kv_kind > 2) return GQA_ERR_SHAPE;
  gqa::Shape s{S, T, Lmax, B, H, Hk, D, B > 0, kv_kind != 0, kv_kind == 2};
  return gqa::auto_chunk(s);
}

int gqa_decode_auto_pieces(int S, int T, int Lmax, int H, int Hk, int D, int kv_kind) {
  if (kv_kind < 0 || kv_kind > 1) return GQA_ERR_SHAPE;
  gqa::Shape s{S, T, Lmax, 0, H, Hk, D, false, kv_kind == 1, false};
  return gqa::auto_pieces(s);
}

const char* gqa_decode_strerror(int code) {
  switch (code) {
    case GQA_OK: return "ok";
    case GQA_ERR_NULL: return "a required pointer is NULL";
    case GQA_ERR_SHAPE: return "invalid shape (S, T, H, Hk >= 1, Lmax >= 0, grid within limits)";
    case GQA_ERR_GROUP: return "n_heads must be a multiple of n_kv_heads";
    case GQA_ERR_HEAD_DIM: return "head_dim must be 64, 128 or 256";
    case GQA_ERR_BUDGET: return "ids given with a budget B < 1";
    case GQA_ERR_CHUNK:
      return "chunk must be >= 1 cells per split, or -P for the balanced partition (dense "
             "windows, S * Lmax < 2^31, Lmax within a split's limit); the merge takes the "
             "resolved chunk";
    case GQA_ERR_WORKSPACE: return "partial workspace smaller than gqa_decode_part_bytes()";
    case GQA_ERR_STATIC_LIMIT:
      return "the partials exceed the static buffer of gqa_decode_step_static "
             "(GQA_STATIC_PART_BYTES); use a larger chunk or the workspace calls";
    default: return code > 0 ? "HIP launch error (hipError_t)" : "unknown error";
  }
}

}  // extern "C"
