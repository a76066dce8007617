/*
 * gqa_decode.h — C ABI of libgqa_decode.so: split-KV flash-decoding of
 * grouped-query attention over a KV cache on AMD Instinct MI355X (gfx950).
 *
 * One decode step is two calls on the same stream:
 *
 *   gqa_decode_attn_f16 / gqa_decode_attn_i8   chunk partials (o, m, l)
 *   gqa_decode_merge                            log-sum-exp merge -> out
 *   gqa_decode_merge_gated                      the merge times sigmoid(gate)
 *   gqa_decode_attn_tq / gqa_decode_merge_tq     the same step over a
 *                                               TurboQuant-compressed cache
 *
 * preceded, for budgeted attention, by gqa_decode_select_ids (the B cell ids
 * of every token from per-block scores); gqa_decode_append_i8 writes new K/V
 * rows into the int8 cache the int8 call reads.
 *
 * What is computed, for sequence s, query token t and query head h
 * (G = H / Hk query heads share KV head g = h / G):
 *
 *   L_t   = clamp(seq_lens[s] - (T - 1 - t), 0, Lmax)
 *   cells = [0, L_t)                      when ids == NULL
 *         = ids[s][t][0 .. min(L_t, B))   otherwise
 *   K[c]  = k[s][c][g][:]                 (f16)
 *         = int8 k[s][c][g][d] * f16 k_scales[s][c][g][d / 64]   (int8)
 *   out[s][t][h][:] = sum_c softmax_c(scale * q[s][t][h][:] . K[c]) V[c]
 *   out[s][t][h][:] = 0 when `cells` is empty.
 *
 * Sources: the GQA head mapping and the whole-group workgroup that reads
 * K/V once come from cera's attention_gqa.metal (header and Phase 1); the
 * chunk partials with a chunk-local softmax and their log-sum-exp merge from
 * qsa2.metal (qsa_attn2, qsa_merge2); the int8 row format with one f16
 * scale per 64 elements and the budget of cell ids (width = min(n_kv,
 * budget)) from qsa2.metal (qsa_attn2, qsa_attn3); the per-token causal
 * window that bad parameters can only truncate from cera's
 * flash_attention_tq.metal (flash_attention_tq); the online softmax and
 * the zero output of an empty window from cera's flash_attention.metal
 * (flash_attention_impl).
 *
 * Conventions for every call:
 *  - Array arguments are DEVICE pointers to C-contiguous arrays owned by the
 *    caller; the library never frees, keeps or allocates memory on these
 *    paths and holds no state between calls.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream);
 *    the library never synchronises.  The merge must be enqueued after the
 *    attention call whose workspace it reads (same stream, or an event).
 *  - Return 0 on success; a negative GQA_ERR_* code when the arguments are
 *    rejected on the host, in which case nothing was enqueued; a positive
 *    hipError_t when a launch failed.  gqa_decode_strerror() names codes.
 *  - Device-side preconditions that are not checked: seq_lens[s] >= 0 is not
 *    required (negative counts clamp to an empty window); ids must be
 *    distinct cells of the token's window [0, L_t).  An id outside [0, Lmax)
 *    is clamped into range, so a bad id yields a wrong row, never an
 *    out-of-bounds read.
 *  - Size limits: any Lmax with ids (a sequence whose rows span 2^31 bytes
 *    or more is addressed with 64-bit row pointers); a dense split's K rows
 *    must span less than 2^31 bytes (see `chunk`).
 *  - K/V traffic: one workgroup serves every query row of a KV head (the
 *    H / Hk heads of the group, times the T tokens of a dense window), so
 *    each K/V row is read once per split, up to 64 rows per KV head for
 *    head_dim 64 and 128 and up to 32 for head_dim 256.  More rows are cut
 *    into blocks of that size that each read the KV head's rows again (with
 *    ids: one token per block, each token's own cells).
 *  - Numerics: scores, softmax sums and outputs are fp32; the products run
 *    on the matrix cores as f16 hi + lo operand pairs (~22 bits each).  A
 *    query row may hold any finite fp32 values: it is scaled by a power of
 *    two before its split (scores are scaled back exactly), so rows with
 *    max |q * scale| from ~1e-33 up to where q . k overflows fp32 keep full
 *    precision.  The softmax weights are held near the top of f16's range
 *    (int8 V: with a power of two taken from the largest V scale), so a
 *    weight is resolved to within ~2^-31 of the largest weight of its wave's
 *    cells: over the ~1e4-1e5 cells a wave streams, the output's error
 *    stays below ~1e-4 of max |V| even when most of the softmax mass sits in
 *    cells far below the maximum.
 */
#ifndef GQA_DECODE_H
#define GQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  GQA_OK = 0,
  GQA_ERR_NULL = -1,       /* a required pointer is NULL                         */
  GQA_ERR_SHAPE = -2,      /* S, T, H, Hk < 1, Lmax < 0, or sizes overflow       */
  GQA_ERR_GROUP = -3,      /* H % Hk != 0                                        */
  GQA_ERR_HEAD_DIM = -4,   /* D not in {64, 128, 256}                            */
  GQA_ERR_BUDGET = -5,     /* ids given with B < 1                               */
  GQA_ERR_CHUNK = -6,      /* chunk 0 in the merge, a split wider than 2^31
                              bytes of K rows (chunk * Hk * D * elem >= 2^31),
                              or a balanced partition (chunk < 0) outside its
                              limits (ids, P > 65536, S * (Lmax + 1152) >= 2^31,
                              Lmax * Hk * D * elem >= 2^31)                      */
  GQA_ERR_WORKSPACE = -7,  /* part_bytes < gqa_decode_part_bytes(...)            */
  GQA_ERR_STATIC_LIMIT = -8 /* gqa_decode_step_static: the partials need more than
                              GQA_STATIC_PART_BYTES                              */
};

/* Size of the static partial buffer of gqa_decode_step_static, per GPU. */
#define GQA_STATIC_PART_BYTES ((size_t)16 << 20)

/* Partial workspace size in bytes for one attention call: one partial
 * (D unnormalised output floats + running max + running sum) per query row
 * and split, splits = ceil(min(B or Lmax, Lmax) / chunk).  `B` is the budget
 * (0 when no ids are used); `chunk` is the resolved cells-per-split (> 0),
 * or -P for the balanced partition (see the attention calls): P partial
 * slots per query row, followed by S int32 slot counts rounded up to 16
 * bytes.  Returns 0 for invalid arguments.  Pure host function. */
size_t gqa_decode_part_bytes(int S, int T, int Lmax, int B, int H, int D, int chunk);

/* The split size the attention calls use when passed chunk == 0.  A pure,
 * deterministic host function of the shapes: it picks the cells per split so
 * that the grid gives every one of the 256 compute units several
 * workgroups, while the partials stay a small fraction of the KV bytes.
 * `kv_kind` names the cache: 0 f16, 1 int8 (both stream best with one
 * long-running four-wave workgroup per compute unit), 2 TurboQuant
 * (gqa_decode_attn_tq: decoding is latency-bound, so its splits are sized
 * for several workgroups per compute unit).  Returns a positive chunk, or a
 * negative GQA_ERR_* code. */
int gqa_decode_auto_chunk(int S, int T, int Lmax, int B, int H, int Hk, int D, int kv_kind);

/* The balanced partition's piece count for dense windows (no ids), as the
 * chunk argument that selects it (-P): one workgroup per compute unit,
 * P = 256 / (Hk * row blocks) rounded down to a multiple of 8 when at least
 * 8 (32 for 8 KV heads, 128 for 2).  Worth choosing when the lengths of a
 * batch differ (on one MI355X an f16 batch of 32 lengths U[512, 4096] steps
 * in 61 µs against 66 with the automatic split, an int8 head_dim 256 batch
 * of 32 lengths U[2048, 16384] in 57 µs against 87); on equal lengths the
 * automatic split is as fast or faster.  kv_kind 0 f16, 1 int8.
 * Returns -P, or a negative GQA_ERR_* code (GQA_ERR_CHUNK where the
 * partition's limits are not met).  Pure host function. */
int gqa_decode_auto_pieces(int S, int T, int Lmax, int H, int Hk, int D, int kv_kind);

/* Chunk partials over an f16 cache.
 *   q         [S][T][H][D]       float32
 *   k, v      [S][Lmax][Hk][D]   IEEE binary16 bit patterns
 *   ids       NULL (dense causal windows) or [S][T][B] int32 cell ids
 *   seq_lens  [S] int32: cells visible to the LAST query token of sequence s
 *   part      workspace of part_bytes >= gqa_decode_part_bytes(S,T,Lmax,B,H,D,chunk')
 *             where chunk' is the resolved chunk; contents are overwritten
 *   scale     score scale (typically 1/sqrt(D))
 *   chunk     cells per split (> 0): each (sequence, KV head) window is cut
 *             into splits of `chunk` cells, one workgroup each;
 *             0 selects gqa_decode_auto_chunk(...);
 *             -P (dense windows only) selects the balanced partition for
 *             batches of uneven lengths: the windows of all S sequences are
 *             laid end to end, each non-empty one preceded by a fixed number
 *             of virtual cells that stand for the cost of starting a
 *             sequence (f16: 64 KB of its K + V rows, 128 cells at
 *             head_dim 128; int8: 256 cells; none when every non-empty
 *             window has the same length),
 *             and the total is cut into P near-equal pieces per KV head
 *             (and row block), one workgroup each, that may cross sequence
 *             boundaries; a piece writes one partial per sequence it
 *             touches.  The windows are rounded up, and the pieces cut, in
 *             whole units of 128 cells (a round of 32-cell tiles over a
 *             workgroup's four waves).  Needs ids == NULL, P <= 65536 and
 *             S * (Lmax + 1152) < 2^31.  (qsa2.metal's chunk partials and
 *             log-sum-exp merge do not depend on where the chunks start, so
 *             any cut of a window gives the same result up to rounding.)
 *             chunk * Hk * D * (bytes per element) must stay below 2^31
 *             (balanced: Lmax in its place).
 * Errors: GQA_ERR_NULL, _SHAPE, _GROUP, _HEAD_DIM, _BUDGET, _CHUNK, _WORKSPACE. */
int gqa_decode_attn_f16(const float *q, const uint16_t *k, const uint16_t *v,
                        const int32_t *ids, const int32_t *seq_lens,
                        float *part, size_t part_bytes,
                        int S, int T, int Lmax, int B, int H, int Hk, int D,
                        float scale, int chunk, void *stream);

/* Chunk partials over an int8 cache with one f16 scale per 64 elements.
 *   k, v                [S][Lmax][Hk][D]      int8 codes
 *   k_scales, v_scales  [S][Lmax][Hk][D/64]   binary16 bit patterns
 * Element value = float(int8) * float(scale of its 64-element group), which
 * is exact in fp32.  Other arguments as gqa_decode_attn_f16. */
int gqa_decode_attn_i8(const float *q, const int8_t *k, const int8_t *v,
                       const uint16_t *k_scales, const uint16_t *v_scales,
                       const int32_t *ids, const int32_t *seq_lens,
                       float *part, size_t part_bytes,
                       int S, int T, int Lmax, int B, int H, int Hk, int D,
                       float scale, int chunk, void *stream);

/* Log-sum-exp merge of the partials written by the attention call with the
 * same S, T, Lmax, B, H, D and the same RESOLVED chunk (> 0, or the same -P
 * for the balanced partition, where each row's slot count is read from the
 * workspace):
 *   M = max_j m_j,  out = sum_j e^(m_j - M) o_j / sum_j e^(m_j - M) l_j
 * (qsa2.metal, qsa_merge2).  The attention call writes every (row, split)
 * slot of the workspace; a split holding no visible cell of a row carries
 * m = -inf and weighs 0, so the merge reads only the workspace.
 *   part          workspace written by gqa_decode_attn_*
 *   seq_lens      [S] int32, as passed to the attention call (must be
 *                 non-NULL; not dereferenced)
 *   ids_or_null   the attention call's ids pointer (only its NULL-ness is
 *                 used: with ids the split count follows min(B, Lmax))
 *   out           [S][T][H][D] float32; rows with an empty window get zeros
 * Errors: GQA_ERR_NULL, _SHAPE, _HEAD_DIM, _BUDGET, _CHUNK. */
int gqa_decode_merge(const float *part, const int32_t *seq_lens, const int32_t *ids_or_null,
                     float *out, int S, int T, int Lmax, int B, int H, int D, int chunk,
                     void *stream);

/* The merge of gqa_decode_merge followed by the output gate (qsa2.metal,
 * end of qsa_merge2; FORWARD_MSL, end of attn_combine):
 *   out[r][d] = merged[r][d] * 1 / (1 + exp(-gate[r][d]))
 * for every output row r = (s * T + t) * H + h.  The gate is fp32 and row r
 * starts at gate + r * gate_stride (in floats, gate_stride >= D): a separate
 * [S][T][H][D] tensor has gate_stride = D; the pages' layout, one
 * [query | gate] row of 2 * D floats per (token, head), is passed as
 * gate = qfull + D with gate_stride = 2 * D.  Rows with an empty window stay
 * zero.  The gate is read only; the caller owns it.  Other arguments and
 * errors as gqa_decode_merge, plus GQA_ERR_NULL for a NULL gate and
 * GQA_ERR_SHAPE for gate_stride < D. */
int gqa_decode_merge_gated(const float *part, const int32_t *seq_lens, const int32_t *ids_or_null,
                           const float *gate, int64_t gate_stride, float *out,
                           int S, int T, int Lmax, int B, int H, int D, int chunk,
                           void *stream);

/* Chunk partials over a TurboQuant-compressed cache (cera 0.4.0,
 * flash_attention_tq.metal: header formulas, kernel flash_attention_tq).
 * Keys and values are never rebuilt; for cell c of KV head g, in the page's
 * notation:
 *   polar_dot  = sum_d q_rot[d] * centroid[idx_k[d]]
 *   signed_sum = 2 * sum_{d: jl_bit[d] = 1} q_jl[d] - sum_d q_jl[d]
 *   score      = scale * (norm * polar_dot
 *                         + norm * residual_norm * qjl_scale * signed_sum)
 * softmax over the causal window (L_t as for the other attention calls), and
 * the value accumulator stays in the rotated basis:
 *   o[d] = sum_c p_c * vnorm_c * centroid[idx_v[c][d]]
 * so the partials are rotated; gqa_decode_merge_tq merges them and applies
 * the inverse rotation.
 *   q_rot, q_jl  [S][T][H][D] float32: the query rotated by the key rotation,
 *                and its JL projection (both prepared by the caller)
 *   k_polar      [S][Hk][Lmax][D/16] uint32: 2-bit centroid indices, dim
 *                16w + i in bits 2i, 2i+1 of word w (per cell, head-major as
 *                the page's slot = kv_head * cache_cap + t)
 *   k_jl         [S][Hk][Lmax][D/32] uint32: sign bits, dim 32w + i in bit i
 *   k_norms      [S][Hk][Lmax] uint32: f16 norm (low half), f16 residual
 *                norm (high half)
 *   v_polar      [S][Hk][Lmax][D/16] uint32, v_norms [S][Hk][Lmax] uint32
 *                (f16 value norm in the low half)
 *   c0 .. c3     the four centroids; qjl_scale (the page uses
 *                sqrt(pi/2) / head_dim); scale the score scale
 * D must be 64 or 128 (the page: at most 128); no ids.  Workspace, chunk,
 * stream and errors as gqa_decode_attn_f16.  Numerics as for the other
 * calls; a row's q_rot and q_jl are scaled together by one power of two
 * before their f16 hi + lo split. */
int gqa_decode_attn_tq(const float *q_rot, const float *q_jl, const uint32_t *k_polar,
                       const uint32_t *k_jl, const uint32_t *k_norms, const uint32_t *v_polar,
                       const uint32_t *v_norms, const int32_t *seq_lens,
                       float *part, size_t part_bytes,
                       int S, int T, int Lmax, int H, int Hk, int D,
                       float c0, float c1, float c2, float c3, float qjl_scale, float scale,
                       int chunk, void *stream);

/* Merge of gqa_decode_attn_tq's rotated partials followed by the inverse
 * randomized Hadamard rotation (flash_attention_tq.metal, epilogue):
 *   out = signs * (H_D @ merged) / sqrt(D)
 * where H_D is the Sylvester Walsh-Hadamard matrix (the page's butterfly
 * passes) and signs [D] float32 is the key rotation's sign flips (+-1).
 * Rows with an empty window get zeros.  Other arguments and errors as
 * gqa_decode_merge (no ids; D 64 or 128). */
int gqa_decode_merge_tq(const float *part, const int32_t *seq_lens, const float *signs,
                        float *out, int S, int T, int Lmax, int H, int D, int chunk,
                        void *stream);

/* Budget selection: the ids a budgeted token attends (qsa2.metal, kernel
 * qsa_topk2).  Cells come in blocks of 4 with one score per block; with
 * n = L_t visible cells (the causal window of token t, as in the attention
 * calls), block b < n/4 holds cells 4b..4b+3 and block n/4 the n%4 remaining
 * ones.  ids[s][t][0..B) = the first B cells ranked by (block score
 * descending, cell index ascending), in ascending order; when n <= B,
 * ids[s][t][0..n) = 0..n-1 and the rest of the row is left untouched.
 * Scores compare as floats (an order-preserving key; -0 below +0).
 *   block_scores  [S][T][Lmax/4 + 1] float32
 *   seq_lens      [S] int32, as for the attention calls
 *   ids           [S][T][B] int32 (written)
 * The output feeds gqa_decode_attn_* (ids, B).  Errors: GQA_ERR_NULL,
 * _SHAPE, _BUDGET. */
int gqa_decode_select_ids(const float *block_scores, const int32_t *seq_lens, int32_t *ids,
                          int S, int T, int Lmax, int B, void *stream);

/* Quantize-on-append: new fp32 K and V rows written into the int8 cache
 * (FORWARD_MSL, kernel kv_append_q8, with 64-element groups as the cache the
 * attention reads).  For every 64-element group x of a new row, in fp32:
 *   d = max|x| / 127,  code = clamp(rint(x / d), -127, 127) (0 when d == 0),
 *   stored scale = f16(d)   (IEEE division, rint rounds halves to even).
 *   k_new, v_new        [S][Tn][Hk][D] float32, D a multiple of 64
 *   pos                 [S] int32: cell of the first new row of sequence s;
 *                       row i goes to cell pos[s] + i, and cells outside
 *                       [0, Lmax) are skipped (a bad position only truncates)
 *   k, v                [S][Lmax][Hk][D] int8 caches (rows written in place)
 *   k_scales, v_scales  [S][Lmax][Hk][D/64] f16 bits (written in place)
 * The new rows must be finite (codes and scales of a group holding inf or
 * NaN are unspecified).  Tn == 0 or Lmax == 0 enqueues nothing.  Errors:
 * GQA_ERR_NULL, _SHAPE (also when the 2 S Tn Hk D/64 groups need more than
 * 2^31 - 1 eight-group workgroups), _HEAD_DIM (D not a positive multiple of
 * 64). */
int gqa_decode_append_i8(const float *k_new, const float *v_new, const int32_t *pos,
                         int8_t *k, int8_t *v, uint16_t *k_scales, uint16_t *v_scales,
                         int S, int Tn, int Lmax, int Hk, int D, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): one whole decode step,
 * gqa_decode_attn_f16 / gqa_decode_attn_i8 followed by gqa_decode_merge,
 * with the partials in a buffer the library owns instead of a caller
 * workspace.  The buffer is a static device array of GQA_STATIC_PART_BYTES
 * (16 MiB), one per GPU the library runs on, held until the process ends;
 * the call allocates and frees nothing.  Its address on the current device
 * is looked up on the first call with that device current (the only call
 * that may block), so a caller that captures the step should make one call
 * first.
 *   kv_kind   0: k, v are f16 bit patterns (k_scales, v_scales unused)
 *             1: k, v are int8 codes with f16 k_scales, v_scales
 *   out       [S][T][H][D] float32, as gqa_decode_merge
 *   chunk     0 selects gqa_decode_auto_chunk(..., kv_kind); -P the
 *             balanced partition, as the attention calls
 * Other arguments as gqa_decode_attn_f16 / _i8.  Every call on one GPU uses
 * that GPU's one buffer: calls that overlap on a GPU (other streams, other
 * threads, without ordering between them) race and give wrong results.
 * Each call writes every partial slot it then reads, so nothing needs
 * clearing between calls.  Errors: those of the two calls it makes, and
 * GQA_ERR_STATIC_LIMIT, before anything is enqueued, when
 * gqa_decode_part_bytes(S, T, Lmax, B or 0, H, D, resolved chunk) exceeds
 * GQA_STATIC_PART_BYTES (use a larger chunk, or the workspace calls). */
int gqa_decode_step_static(const float *q, const void *k, const void *v,
                           const uint16_t *k_scales, const uint16_t *v_scales,
                           const int32_t *ids, const int32_t *seq_lens, float *out,
                           int S, int T, int Lmax, int B, int H, int Hk, int D,
                           float scale, int chunk, int kv_kind, void *stream);

/* Static text for a return code. */
const char *gqa_decode_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* GQA_DECODE_H */
