// Split-KV flash-decoding of grouped-query attention for gfx950 (MI355X).
//
// Kernels:
//   attn_mfma   (attn_mfma.h) one workgroup per (split, KV head [x row block]
//               [x token], seq): streams the K/V rows of its cell range once
//               for every query row of the GQA group (all G heads, and all T
//               tokens of a dense causal window), runs an online softmax per
//               row and writes one partial (o unnormalised, m, l) per row.
// The log-sum-exp merge of the partials is in merge.hip.
// The attention grid is one-dimensional and ordered so that consecutive
// workgroups, which the hardware hands to different XCDs, carry equal work.
//
// Sources: the whole-group workgroup that loads K/V once (cera,
// attention_gqa.metal, header and Phase 1); the online softmax with a running
// max, running sum and a correction that is zero before the first visible
// cell (cera, flash_attention.metal, flash_attention_impl); chunk partials and
// their log-sum-exp merge (qsa2.metal, qsa_attn2 and qsa_merge2); int8 rows
// with one f16 scale per 64 elements and gathering through cell ids
// (qsa2.metal, qsa_attn2 and qsa_attn3); the per-token causal window
// (cera, flash_attention_tq.metal, flash_attention_tq).
//
// Scores are kept in the base-2 domain: q is pre-multiplied by
// scale * log2(e) so the exponentials are exp2, which is the hardware's
// native v_exp_f32.  exp2(x * log2 e) = exp(x), so this is the same
// natural-base softmax.  The running max stored in a partial is therefore
// in base-2 units; only the merge reads it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "attn_mfma.h"
#include "common.h"
#include "gqa_decode.h"
#include "plan.h"

namespace {

using gqa_kern::AttnArgs;

constexpr float kLog2e = 1.4426950408889634f;

// IDS: 0 dense, 1 gather, 2 gather over a plane of 2 GiB or more.  FLAT:
// the balanced-partition grid (dense windows only).
template <int D, bool I8, int IDS, int NRB, int NW, bool FLAT = false>
hipError_t launch_one(const AttnArgs& a, dim3 grid, hipStream_t st) {
  static_assert(!(FLAT && IDS != 0), "the balanced partition covers dense windows");
  using L = gqa_kern::AttnLds<D, I8, NRB, NW>;
  // gather mode: the split's ids follow the fixed part, 16-byte aligned
  const int bytes = L::BYTES + (IDS ? (a.chunk * 4 + 15) / 16 * 16 : 0);
  constexpr int most = L::BYTES + (IDS ? L::IDSB : 0);
  auto* fn = &gqa_kern::attn_mfma<D, I8, IDS, NRB, NW>;
  if constexpr (FLAT) fn = &gqa_kern::attn_mfma_flat<D, I8, NRB, NW>;
  if constexpr (most > 65536) {
    // more than 64 KB of dynamic LDS must be allowed once per device
    static std::atomic<uint64_t> attr_set{0};   // bit per device, per instance
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (!(attr_set.load(std::memory_order_acquire) & bit)) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                              hipFuncAttributeMaxDynamicSharedMemorySize, most);
      if (e != hipSuccess) return e;
      attr_set.fetch_or(bit, std::memory_order_acq_rel);
    }
  }
  hipLaunchKernelGGL(fn, grid, dim3(64 * NW), bytes, st, a);
  return hipGetLastError();
}

// LDS of one compute unit (gfx950).
constexpr int kLdsPerCu = 160 * 1024;

template <int D, bool I8, int NRB, int NW>
constexpr bool fits_lds() {
  return gqa_kern::AttnLds<D, I8, NRB, NW>::BYTES + gqa_kern::AttnLds<D, I8, NRB, NW>::IDSB <=
         kLdsPerCu;
}

// One-wave workgroups for splits of at most two tiles, four waves otherwise.
template <int D, bool I8, int NRB>
hipError_t launch_attn_nw(const AttnArgs& a, bool ids, int nw, dim3 grid, hipStream_t st) {
  static_assert(fits_lds<D, I8, NRB, 4>() && fits_lds<D, I8, NRB, 1>(), "LDS budget");
  if (a.flat) return launch_one<D, I8, 0, NRB, 4, true>(a, grid, st);
  if (nw == 1) {
    if (!ids) return launch_one<D, I8, 0, NRB, 1>(a, grid, st);
    return a.wide ? launch_one<D, I8, 2, NRB, 1>(a, grid, st) : launch_one<D, I8, 1, NRB, 1>(a, grid, st);
  }
  if (!ids) return launch_one<D, I8, 0, NRB, 4>(a, grid, st);
  return a.wide ? launch_one<D, I8, 2, NRB, 4>(a, grid, st) : launch_one<D, I8, 1, NRB, 4>(a, grid, st);
}

template <int D, bool I8>
hipError_t launch_attn(const AttnArgs& a, bool ids, int nrows, int nw, dim3 grid, hipStream_t st) {
  if (nrows <= 16) return launch_attn_nw<D, I8, 1>(a, ids, nw, grid, st);
  if constexpr (D <= 128) {
    if (nrows > 32) return launch_attn_nw<D, I8, 4>(a, ids, nw, grid, st);
  }
  return launch_attn_nw<D, I8, 2>(a, ids, nw, grid, st);
}

template <bool I8>
hipError_t launch_attn_d(const AttnArgs& a, int D, bool ids, int nrows, int nw, dim3 grid,
                         hipStream_t st) {
  switch (D) {
    case 64: return launch_attn<64, I8>(a, ids, nrows, nw, grid, st);
    case 128: return launch_attn<128, I8>(a, ids, nrows, nw, grid, st);
    default: return launch_attn<256, I8>(a, ids, nrows, nw, grid, st);
  }
}

int attn_common(bool i8, const float* q, const void* k, const void* v, const uint16_t* ksc,
                const uint16_t* vsc, const int32_t* ids, const int32_t* seq_lens, float* part,
                size_t part_bytes, int S, int T, int Lmax, int B, int H, int Hk, int D,
                float scale, int chunk, void* stream) {
  // K/V (and scales) may be NULL only for an empty cache (Lmax == 0).
  if (!q || !seq_lens || !part) return GQA_ERR_NULL;
  if (Lmax > 0 && (!k || !v || (i8 && (!ksc || !vsc)))) return GQA_ERR_NULL;
  gqa::Shape sh{S, T, Lmax, ids ? B : 0, H, Hk, D, ids != nullptr, i8};
  int rc = gqa::check_shape(sh);
  if (rc != GQA_OK) return rc;
  if (chunk == 0) chunk = gqa::auto_chunk(sh);
  // balanced partition: a segment lies inside one window, so Lmax bounds it
  const bool flat = chunk < 0;
  if (flat ? (!gqa::balanced_ok(sh, chunk) || Lmax > gqa::max_chunk(sh))
           : (chunk <= 0 || chunk > gqa::max_chunk(sh)))
    return GQA_ERR_CHUNK;
  const size_t need = gqa::part_bytes(sh, chunk);
  const int64_t P = gqa::num_splits(sh, chunk);
  if (P > 0 && need == 0) return GQA_ERR_SHAPE;   // the partials would not fit any address space
  if (part_bytes < need) return GQA_ERR_WORKSPACE;
  if (P == 0) return GQA_OK;                 // Lmax == 0: every row is empty
  if (P > 0x7fffffff) return GQA_ERR_SHAPE;

  AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.ksc = ksc; a.vsc = vsc; a.ids = ids; a.seq_lens = seq_lens;
  a.part_o = part;
  a.part_ml = part + gqa::part_o_floats(sh, P);
  a.S = S; a.T = T; a.Lmax = Lmax; a.B = sh.B; a.H = H; a.Hk = Hk; a.G = H / Hk;
  a.R = (int)gqa::rows_per_unit(sh); a.nrb = (int)gqa::row_blocks(sh); a.P = (int)P; a.chunk = chunk;
  a.flat = flat ? 1 : 0;
  // gather over a sequence whose rows of all KV heads span 2^31 bytes or
  // more: 64-bit row addresses instead of 32-bit buffer offsets
  a.wide = (ids && (int64_t)Lmax * Hk * D * (i8 ? 1 : 2) >= ((int64_t)1 << 31)) ? 1 : 0;
  a.flat_pad = gqa::flat_pad_cells(sh);
  a.flat_n = reinterpret_cast<int*>(part + gqa::flat_n_offset_floats(sh, P));
  a.qscale = scale * kLog2e;
  a.qmant = std::frexp(a.qscale, &a.qexp);
  // int8 rows: the KV heads of a sequence share an XCD (sequence-fastest
  // grid) when S is a multiple of the 8 XCDs.  Measured on one MI355X: int8
  // 32K 49.1 -> 48.6 us, budgeted int8 13.9 -> 13.5 us.  f16 keeps the
  // head-fastest order, which spreads every sequence over the XCDs and
  // balances uneven batches (f16 batch 62.6 us, 64.5 sequence-fastest).
  a.seq_fast = (i8 && S % 8 == 0) ? 1 : 0;
  const int nrows = gqa::block_rows(sh);
  const int64_t nwg = flat ? P * Hk * a.nrb : P * Hk * a.nrb * (ids ? T : 1) * S;
  if (nwg > 0x7fffffff) return GQA_ERR_SHAPE;
  dim3 grid((unsigned)nwg);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int nw = gqa::waves_per_block(sh, chunk);
  hipError_t e = i8 ? launch_attn_d<true>(a, D, ids != nullptr, nrows, nw, grid, st)
                    : launch_attn_d<false>(a, D, ids != nullptr, nrows, nw, grid, st);
  return e == hipSuccess ? GQA_OK : (int)e;
}

}  // namespace

extern "C" {

int gqa_decode_attn_f16(const float* q, const uint16_t* k, const uint16_t* v, const int32_t* ids,
                        const int32_t* seq_lens, float* part, size_t part_bytes, int S, int T,
                        int Lmax, int B, int H, int Hk, int D, float scale, int chunk,
                        void* stream) {
  return attn_common(false, q, k, v, nullptr, nullptr, ids, seq_lens, part, part_bytes, S, T, Lmax,
                     B, H, Hk, D, scale, chunk, stream);
}

int gqa_decode_attn_i8(const float* q, const int8_t* k, const int8_t* v, const uint16_t* k_scales,
                       const uint16_t* v_scales, const int32_t* ids, const int32_t* seq_lens,
                       float* part, size_t part_bytes, int S, int T, int Lmax, int B, int H,
                       int Hk, int D, float scale, int chunk, void* stream) {
  return attn_common(true, q, k, v, k_scales, v_scales, ids, seq_lens, part, part_bytes, S, T,
                     Lmax, B, H, Hk, D, scale, chunk, stream);
}

}  // extern "C"
