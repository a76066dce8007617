// Chunk kernel on the gfx950 matrix cores (v_mfma_f32_16x16x32_f16).
//
// One workgroup = one (split, KV head [, row block] [, token], sequence): it
// holds every query row that reads this KV head (the G heads of the group,
// times the T tokens of a dense causal window, up to 32 rows), so each K/V
// row is fetched from HBM exactly once per split (cera, attention_gqa.metal:
// one threadgroup per KV head for all Q heads of the group).
//
// The NW (1 or 4) waves of the workgroup stream 32-cell tiles independently
// (wave w takes tiles w, w+NW, ...) with their own online-softmax state, and combine
// at the end through LDS into ONE partial (o unnormalised, m, l) per query
// row — the chunk partial of qsa2.metal (qsa_attn2), merged later by the
// log-sum-exp merge (qsa_merge2).
//
// Per 32-cell tile and wave:
//   QK   S^T[cell][row] = K[cell][:] . Q[row][:]   MFMA with A = K straight
//        from HBM into registers (lane: one cell, 8 dims per k-step), B = the
//        query rows (registers, loaded once).  q is fp32; it is split into
//        f16 hi + lo (hi = f16(q), lo = f16(q - hi)) and both halves are
//        multiplied, so the product keeps ~22 bits of q.  Before the split
//        each query row is multiplied by a power of two that puts its largest
//        |q * scale * log2 e| in [2^13, 2^15): the hi part is then a normal
//        f16 for every element that matters, whatever the range of q, and
//        the row's scores are multiplied back by the inverse power (exact).
//        f16 K and int8 K are exact in f16.  int8 K: one accumulator per 64-element group,
//        multiplied by that group's f16 scale after the dot (qsa2.metal,
//        qsa_attn3: raw int8 dot per group, then the scale).
//   softmax  online, per query row, base 2 (q carries scale * log2 e): the
//        running max/sum update of cera, flash_attention.metal
//        (flash_attention_impl), with no correction before the first visible
//        cell.  The row's reference max moves only when a tile's max exceeds
//        it by more than 8 (so p <= 256), which skips most accumulator
//        rescales; any reference gives the same (o, m, l) partial up to
//        rounding.  Cross-lane max/sum use the gfx950 permlane swaps.
//   PV   O[row][dim] += P[row][cell] V[cell][dim]  MFMA with A = P taken
//        directly from the QK accumulators (no shuffle: the QK output layout
//        is the PV input layout up to a fixed permutation of the 32 cells),
//        B = V read from LDS with ds_read_b64_tr_b16 / _b8, which deliver the
//        cell-major fragments out of the row-major tile.  P is split hi + lo
//        like q.  int8 V: the per-(cell, group) scale is folded into P.
//        The f16 hi + lo pair resolves values only down to f16's subnormal
//        step (2^-24), while the softmax sum l keeps every weight in fp32, so
//        P is kept near the top of f16's range instead of near 1: f16 V takes
//        p = 2^(s - m + 7) <= 2^15; int8 V folds a per-wave power of two 2^E
//        into the staged scales, E set from the largest V-scale exponent seen
//        so far, so that p * scale * 2^E <= 2^15 (the accumulators are
//        rescaled, rarely, when a larger scale arrives).  The partial is
//        written in the same units: (o, m - 7, l) or (o, m - E, l * 2^E),
//        which is the same partial for the merge.
//
// V tiles are staged per wave in LDS with 16-byte chunks XOR-swizzled per
// row so that both the row-major writes and the transposed reads are free of
// bank conflicts.  K, V and the int8 scales of the next tile are loaded into
// registers while the current tile is computed.
#pragma once

#include <type_traits>

#include "common.h"
#include "mfma_util.h"

namespace gqa_kern {

// Four int8 (one dword) -> four f16 (two dwords), exact: bias each byte to
// unsigned (x ^ 0x80 = x + 128), place it as the low mantissa byte of
// f16 1024 (0x6400 | u = 1024 + u), then subtract 1152.
__device__ __forceinline__ void i8x4_to_f16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = w ^ 0x80808080u;
  const half2v bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u);
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x07030602u);
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, a) - bias);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, b) - bias);
}

__device__ __forceinline__ half8 i8x8_to_half8(uint32_t w0, uint32_t w1) {
  uint32_t r0, r1, r2, r3;
  i8x4_to_f16(w0, r0, r1);
  i8x4_to_f16(w1, r2, r3);
  const u32x4 r = {r0, r1, r2, r3};
  return __builtin_bit_cast(half8, r);
}

// Largest f16 exponent field among the f16 values packed in w (their
// magnitudes are below 2^(field - 14)).
__device__ __forceinline__ uint32_t f16x2_max_expfield(uint32_t w) {
  const uint32_t a = w & 0x7fff7fffu;
  const uint32_t lo = a & 0xffffu, hi = a >> 16;
  return (lo > hi ? lo : hi) >> 10;
}

template <int D, bool I8>
struct TileGeom {
  static constexpr int ES = I8 ? 1 : 2;      // bytes per element
  static constexpr int RBY = D * ES;         // bytes per K/V row
  static constexpr int CH = RBY / 16;        // 16-byte chunks per row
  static constexpr int NG = D / 64;          // int8 scale groups per row
  static constexpr int KS = D / 32;          // MFMA k-steps over head_dim
  static constexpr int NB = D / 16;          // 16-dim output blocks
  static constexpr int KLD = RBY / 64;       // 16-byte K loads per lane per 16-cell block
  static constexpr int TC = 32;              // cells per wave tile
  static constexpr int VLD = TC * RBY / 1024;  // 16-byte V loads per lane per tile
  static constexpr int RPI = 1024 / RBY;     // V rows per wave-wide load
  // log2(16 / CH) for CH <= 16 (0 above): aligns the row key with the bank
  // group of a chunk when rows are narrower than the 256-byte bank period.
  static constexpr int SH = CH >= 16 ? 0 : (CH == 8 ? 1 : 2);
  static_assert(RBY >= 64 && RBY <= 512, "row size");
  // chunk swizzle of row r (bank-conflict-free writes and transposed reads)
  __device__ static int swz(int r) {
    if constexpr (I8) {
      const int key = (r & 7) | (((r >> 4) & 1) << 3);
      return (key >> SH) & (CH - 1);
    } else {
      return ((2 * (r & 7)) >> SH) & (CH - 1);
    }
  }
  __device__ static int lds_off(int r, int c) { return r * RBY + ((c ^ swz(r)) << 4); }
  // K tile swizzle: the 16-byte chunks of consecutive rows rotate through the
  // 16 bank groups of a 256-byte period, so the row-major writes and the
  // MFMA-operand reads (16 rows x 4 chunks per instruction) are both
  // conflict-free.
  static constexpr int SHK = RBY >= 256 ? 0 : (RBY == 128 ? 1 : 2);
  __device__ static int swzk(int r) { return (r >> SHK) & (CH < 16 ? CH - 1 : 15); }
  __device__ static int lds_offk(int r, int c) { return r * RBY + ((c ^ swzk(r)) << 4); }
};

// Largest split (cells) in gather mode: the split's cell ids are staged in LDS.
constexpr int kMaxIdsChunk = 4096;

// Dynamic LDS bytes of one workgroup of NW waves (plus the split's cell ids,
// 4 bytes each, in gather mode).
template <int D, bool I8, int NRB, int NW>
struct AttnLds {
  using G = TileGeom<D, I8>;
  static constexpr int RB = 16 * NRB;
  static constexpr int VT = NW * G::TC * G::RBY;         // per-wave V tiles (and K tiles)
  // Combine buffers hold rows of RS = D + 4 floats: the accumulators are
  // parked with one lane per dim, four rows per lane group, and a row stride
  // of 4 mod 8 dwords puts the two lane groups of a half-wave in different
  // halves of the 32 banks (a stride of D put them in the same banks).
  static constexpr int RS = D + 4;
  static constexpr int BUF2 = NW / 2 * RB * RS * 4;      // two-stage cross-wave combine buffers
  static constexpr int QB = NRB * G::KS * 2 * 64 * 16;   // query B operands, hi and lo
  static constexpr int SC = I8 ? NW * 2 * G::NG * G::TC * 4 : 0;  // per-wave K/V scales (fp32)
  static constexpr int ML = NW * RB * 2 * 4;             // per-wave (m, l)
  static constexpr int IDSB = kMaxIdsChunk * 4;          // most the split's cell ids take
  static constexpr int CAP = 160 * 1024;                 // LDS of one compute unit
  // f16 K rows are staged through LDS like V when both tiles fit: then K is
  // read from HBM in whole rows (fully used cache lines) and the next tile's
  // K and V are both requested as soon as the current ones are staged
  // (measured: multi-query causal 128K 356 -> 330 us, uneven batch 76 ->
  // 64 us).  int8 K, whose path is already bound by the vector ALU, and
  // tiles that do not fit load each lane's K operand fragment straight into
  // registers (int8 32K: 50 us that way, 55 us through LDS).
  static constexpr int MAIN_KL = 2 * VT > BUF2 ? 2 * VT : BUF2;
  static constexpr bool KL = !I8 && MAIN_KL + QB + SC + ML + IDSB <= CAP;
  static constexpr int TILES = KL ? 2 * VT : VT;
  // The waves combine in one pass (each parks its unscaled accumulators in a
  // buffer of its own, one barrier, every output element sums the NW
  // buffers) when NW buffers fit beside everything else; otherwise in two
  // (half the waves park, the other half add, then the sums are added).
  // The buffers alias the tiles either way.
  static constexpr int BUF1 = NW * RB * RS * 4;
  static constexpr bool ONE_PASS =
      NW > 1 && (TILES > BUF1 ? TILES : BUF1) + QB + SC + ML + IDSB <= CAP;
  static constexpr int BUF = ONE_PASS ? BUF1 : BUF2;     // cross-wave combine buffers (alias tiles)
  static constexpr int MAIN = TILES > BUF ? TILES : BUF;
  static constexpr int BYTES = MAIN + QB + SC + ML;
};

// Waves per SIMD the register budget is sized for: 2, except for the
// instances whose accumulators and operands do not fit half the register
// file (head_dim 256 with two row blocks or f16 K, f16 head_dim 128 with two
// row blocks, and every four-block instance), which get the whole file
// (accumulation registers included) instead of spilling.
template <int D, bool I8, int NRB>
constexpr int attn_occupancy() {
  return (NRB >= 4 || (D == 256 && (NRB == 2 || !I8)) || (D == 128 && NRB == 2 && !I8)) ? 1 : 2;
}

// Query-operand slots (row block x k-step x lane) of one row block, and how
// many each thread of an NW-wave workgroup holds.  When they divide evenly
// (at most eight per thread) a caller can request a unit's query rows before
// it knows the unit's window, so their latency overlaps that read.
template <int D, int NRB, int NW>
struct QSlots {
  static constexpr int QSLOTS = NRB * (D / 32) * 64;
  static constexpr int NT = 64 * NW;
  static constexpr int QPT = QSLOTS / NT;
  static constexpr bool QPRE = QSLOTS % NT == 0 && QPT <= 8;
  static constexpr int N = QPRE ? QPT : 1;
};

// Eight fp32 query elements of operand slot `slot` (slot = (row block k,
// k-step ks, lane ln) of the MFMA B-operand layout) of the row block whose
// first unit row is r0, in unit (sequence s, KV head g[, token tq]).  Rows
// past the unit's last read that last row (always valid; they are zeroed
// when stored).
template <int D, bool I8, bool IDS>
__device__ __forceinline__ void q_load_slot(const AttnArgs& a, int s, int g, int tq, int r0,
                                            int slot, float4& u0, float4& u1) {
  using G = TileGeom<D, I8>;
  const int ln = slot & 63, kks = slot >> 6;
  const int ks = kks % G::KS, k = kks / G::KS;
  const int r = r0 + 16 * k + (ln & 15);
  // dims of k-step ks held by lane group ln / 16 (must match the K loads)
  const int lb2 = ln >> 4;
  const int d0 = I8 ? (64 * (ks >> 1) + 16 * lb2 + 8 * (ks & 1)) : (32 * ks + 8 * lb2);
  const int rc = r < a.R ? r : a.R - 1;
  const int t = IDS ? tq : rc / a.G;
  const int h = g * a.G + (IDS ? rc : rc % a.G);
  const float* qrow = a.q + ((size_t)(s * a.T + t) * a.H + h) * D + d0;
  u0 = *reinterpret_cast<const float4*>(qrow);
  u1 = *reinterpret_cast<const float4*>(qrow + 4);
}

// One unit's split: every query row of row block rbl of (sequence s, KV head
// g[, token tq]) against the cells [c0l, min(cap_end, window)) of its
// window, written as partial slot p of each row.  seq_len is seq_lens[s];
// id_first (gather mode) the split's first NT cell ids as requested by the
// caller; qv the block's query slots when QSlots::QPRE (requested by the
// caller).  Called by every thread of the workgroup; returns with the
// partial written (LDS may be reused after a barrier).
// IDS: 0 dense windows, 1 gather through cell ids, 2 gather through cell ids
// over a plane of 2 GiB or more (64-bit row addresses).
template <int D, bool I8, int IDS, int NRB, int NW, bool IN_LOOP = false>
__device__ __forceinline__ void attn_unit(const AttnArgs& a, int g, int s, int rbl, int tq, int p,
                                          int64_t c0l, int64_t cap_end, int seq_len,
                                          int id_first,
                                          const float4 (&qv)[QSlots<D, NRB, NW>::N][2]) {
  using G = TileGeom<D, I8>;
  using L = AttnLds<D, I8, NRB, NW>;
  using Q = QSlots<D, NRB, NW>;
  constexpr int NT = 64 * NW;                    // threads per workgroup
  constexpr int RB = 16 * NRB;
  constexpr int TC = G::TC;
  constexpr int RBY = G::RBY;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  int tid = threadIdx.x;
  // Called in a loop: the lane index is made opaque at each call, so the
  // compiler cannot hoist the body's lane-dependent addressing out of the
  // loop and hold it in registers across the whole body; and the unit's
  // coordinates, uniform by construction, are read from the first lane, so
  // that the buffer resources built from them sit in scalar registers (a
  // resource in vector registers costs a loop over the lanes at every load:
  // balanced int8 32K 63.3 -> 53.2 us).
  if constexpr (IN_LOOP) {
    asm volatile("" : "+v"(tid));
    g = __builtin_amdgcn_readfirstlane(g);
    s = __builtin_amdgcn_readfirstlane(s);
    rbl = __builtin_amdgcn_readfirstlane(rbl);
    p = __builtin_amdgcn_readfirstlane(p);
    c0l = __builtin_amdgcn_readfirstlane((int)c0l);
    cap_end = __builtin_amdgcn_readfirstlane((int)cap_end);
    seq_len = __builtin_amdgcn_readfirstlane(seq_len);
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15, lb = lane >> 4;
  auto row_t = [&](int r) -> int { return IDS ? tq : r / a.G; };
  auto row_h = [&](int r) -> int { return g * a.G + (IDS ? r : r % a.G); };
  const int r0 = rbl * RB;                       // first unit row of this block

  // ---- query rows as MFMA B operands (f16 hi + lo), staged once in LDS. ----
  constexpr int QSLOTS = Q::QSLOTS;
  constexpr int QPT = Q::QPT;
  constexpr bool QPRE = Q::QPRE;
  auto q_load = [&](int slot, float4& u0, float4& u1) {
    q_load_slot<D, I8, (IDS != 0)>(a, s, g, tq, r0, slot, u0, u1);
  };
  // Per-row max |q| of the block.  A lane's slots all belong to its rows
  // 16k + lr; each wave reduces its slots in registers (qmx).  A one-wave
  // workgroup of one row block then has its rows' maxima in registers;
  // otherwise they meet in LDS, qred[wave][row] (the (m, l) area, unused
  // until the epilogue).
  constexpr bool QREG = NW == 1 && NRB == 1;
  float* qred = reinterpret_cast<float*>(smem + L::MAIN + L::QB + L::SC);
  float qmx[NRB];
  auto row_max = [&](int row) -> float {
    if constexpr (QREG) {
      (void)row;
      return qmx[0];
    } else {
      float m = qred[row];
#pragma unroll
      for (int w = 1; w < NW; ++w) m = fmaxf(m, qred[w * RB + row]);
      return m;
    }
  };
#pragma unroll
  for (int k = 0; k < NRB; ++k) qmx[k] = 0.f;
  // max |q| of a slot's eight elements, over the four lane groups that hold
  // the same row (wave-wide: every lane of the wave passes a slot)
  auto q_note = [&](int slot, const float4& u0, const float4& u1) {
    const int kb = (slot >> 6) / G::KS;
    float m = fmaxf(fmaxf(fmaxf(fabsf(u0.x), fabsf(u0.y)), fmaxf(fabsf(u0.z), fabsf(u0.w))),
                    fmaxf(fmaxf(fabsf(u1.x), fabsf(u1.y)), fmaxf(fabsf(u1.z), fabsf(u1.w))));
    m = max_x32(max_x16(m));
#pragma unroll
    for (int k = 0; k < NRB; ++k) qmx[k] = (kb == k) ? fmaxf(qmx[k], m) : qmx[k];
  };
  auto q_store = [&](int slot, const float4& u0, const float4& u1) {
    const int ln = slot & 63, kks = slot >> 6;
    const int row = 16 * (kks / G::KS) + (ln & 15);
    const bool real = r0 + row < a.R;
    float rs_unused;
    const float f = q_row_factor(row_max(row), a.qmant, a.qexp, &rs_unused);
    float x[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = real ? x[e] * f : 0.f;
    half8 hi, lo;
    split_hi_lo(x, hi, lo);
    u32x4* qlds = reinterpret_cast<u32x4*>(smem + L::MAIN);
    qlds[(kks * 2 + 0) * 64 + ln] = __builtin_bit_cast(u32x4, hi);
    qlds[(kks * 2 + 1) * 64 + ln] = __builtin_bit_cast(u32x4, lo);
  };

  auto width_of = [&](int r) -> int {   // r: row index within the unit
    if (r >= a.R) return 0;
    const int t = IDS ? tq : r / a.G;
    int Lt = seq_len - (a.T - 1 - t);
    Lt = Lt < 0 ? 0 : (Lt > a.Lmax ? a.Lmax : Lt);
    if (IDS) Lt = Lt < a.B ? Lt : a.B;
    return Lt;
  };

  const int rlast = (a.R - 1 < r0 + RB - 1) ? a.R - 1 : r0 + RB - 1;
  const int wmax = width_of(rlast);
  if (c0l >= wmax) {
    // nothing visible in this split for any row of the block: its partials
    // carry weight 0 (m = -inf, l = 0), and the merge skips their o
    if (tid < RB && r0 + tid < a.R) {
      const int r = r0 + tid;
      const size_t prow = ((size_t)(s * a.T + row_t(r)) * a.H + row_h(r)) * a.P + p;
      a.part_ml[prow * 2] = -INFINITY;
      a.part_ml[prow * 2 + 1] = 0.f;
    }
    return;
  }
  const int c0 = (int)c0l;
  const int cend = (int)((cap_end < wmax) ? cap_end : wmax);
  // Tiles ending at or before lim_lo are fully visible to every real row.
  const int lim_lo = width_of(r0) < cend ? width_of(r0) : cend;

  uint8_t* vt = smem + wave * TC * RBY;                       // this wave's V tile
  uint8_t* kt = smem + L::VT + wave * TC * RBY;               // this wave's K tile (L::KL)
  u32x4* qlds = reinterpret_cast<u32x4*>(smem + L::MAIN);
  // int8: this wave's K scales [NG][TC] then V scales [NG][TC], fp32
  float* sclf = reinterpret_cast<float*>(smem + L::MAIN + L::QB) + wave * 2 * G::NG * TC;
  float* mls = reinterpret_cast<float*>(smem + L::MAIN + L::QB + L::SC);

  int lim[NRB];                                  // visible limit of this lane's rows
#pragma unroll
  for (int k = 0; k < NRB; ++k) {
    const int wr = width_of(r0 + 16 * k + lr);
    lim[k] = wr < cend ? wr : cend;
  }

  // ---- K/V addressing through buffer resources: every offset is 32-bit and
  // a read at or past the resource's size returns zeros without touching
  // memory.  The whole per-cell offset goes in the per-lane offset, which
  // the range check covers; the scalar offset is always 0.  dense: the
  // resource starts at this split's first cell and ends at its last, so the
  // ragged end of the last tile, and tiles past the split's end, read
  // zeros.  gather: the resource spans the sequence's rows of this KV head;
  // a lane adds its cell's row offset (the split's ids are staged in LDS)
  // and list positions past the split map to kOut, past every resource.
  // Loads are therefore issued unconditionally, which keeps the compiler's
  // wait counts exact.  Wide gather (IDS 2: the sequence's rows of all KV
  // heads span 2^31 bytes or more, past a 32-bit offset): plain 64-bit
  // addresses, and a list position at or past the split's end reads the
  // split's last row again, a row this split attends anyway, whose weight
  // the softmax's edge mask sets to 0. ----
  const uint32_t rowstride = (uint32_t)a.Hk * RBY;           // bytes between cells of a KV head
  const uint32_t srow = (uint32_t)a.Hk * G::NG * 2;           // scale bytes between cells
  const size_t first_row = ((size_t)s * a.Lmax + (IDS ? 0 : c0)) * a.Hk + g;
  const uint32_t ncells = IDS ? (uint32_t)a.Lmax : (uint32_t)(cend - c0);
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(reinterpret_cast<const uint8_t*>(a.k) + first_row * RBY, ncells * rowstride);
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(reinterpret_cast<const uint8_t*>(a.v) + first_row * RBY, ncells * rowstride);
  const __amdgpu_buffer_rsrc_t rks = make_rsrc(I8 ? a.ksc + first_row * G::NG : nullptr, ncells * srow);
  const __amdgpu_buffer_rsrc_t rvs = make_rsrc(I8 ? a.vsc + first_row * G::NG : nullptr, ncells * srow);
  constexpr uint32_t kOut = 0x80000000u;                     // past every resource (< 2^31 bytes)
  constexpr bool WIDE = IDS == 2;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k) + first_row * RBY;
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v) + first_row * RBY;
  const uint8_t* ksbase = reinterpret_cast<const uint8_t*>(I8 ? a.ksc + first_row * G::NG : nullptr);
  const uint8_t* vsbase = reinterpret_cast<const uint8_t*>(I8 ? a.vsc + first_row * G::NG : nullptr);
  int32_t* idl = reinterpret_cast<int32_t*>(smem + L::BYTES);  // gather mode: ids of [c0, cend)
  if constexpr (IDS) {
    const int32_t* idrow = a.ids + ((size_t)s * a.T + tq) * a.B;
    for (int i = tid; i < cend - c0; i += NT) {
      // position c0 + tid < cend <= B and tid < chunk: id_first holds it
      int c = i == tid ? id_first : idrow[c0 + i];
      idl[i] = c < 0 ? 0 : (c >= a.Lmax ? a.Lmax - 1 : c);
    }
  }
  // Byte offset, from the resource base, of the row of list position pos
  // (pos >= c0; positions at or past cend land out of range).
  auto cell_off = [&](int pos, uint32_t stride) -> uint32_t {
    if constexpr (IDS) {
      const int i = (pos < cend ? pos : cend - 1) - c0;
      return pos < cend ? (uint32_t)idl[i] * stride : kOut;
    } else {
      return (uint32_t)(pos - c0) * stride;
    }
  };
  // Wide gather: byte offset of list position pos's row (the split's last
  // row for positions at or past cend).
  auto cell_off64 = [&](int pos, uint32_t stride) -> size_t {
    const int i = (pos < cend ? pos : cend - 1) - c0;
    return (size_t)(uint32_t)idl[i] * stride;
  };
  auto ld16 = [](const uint8_t* p) -> u32x4 {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  };

  struct KRegs {
    u32x4 k[L::KL ? G::VLD : 2 * G::KLD];
  };
  struct VRegs {
    u32x4 v[G::VLD];
    u32x2 ks, vs;
  };
  // Lazy rescaling: a row's reference max moves only when a tile's max
  // exceeds it by more than kTau (base-2 units), so 2^(s - m) <= 2^kTau.
  constexpr float kTau = 8.0f;
  // f16 V: the weights are p = 2^(s - m + kPShift) <= 2^15, near the top of
  // f16's range, so the f16 hi + lo pair resolves them down to 2^-31 of the
  // row's largest weight.
  constexpr float kPShift = 7.0f;
  // int8 V: the staged V scales carry a factor 2^(21 - vexp), vexp = the
  // largest f16 exponent field of the V scales this wave has seen (scales
  // below 2^(vexp - 14)), so p * scale * 2^(21 - vexp) < 2^15.  vexp only
  // grows; when it does, the accumulators are rescaled by vf = 2^(old - new)
  // together with the next softmax correction.
  int vexp = 0;
  float vf = 1.0f;

  f32x4 O[NRB][G::NB];
  float m_run[NRB], l_run[NRB];
  float rs[NRB];                                 // score factor of this lane's rows 16k+lr
#pragma unroll
  for (int k = 0; k < NRB; ++k) {
    m_run[k] = -INFINITY;
    l_run[k] = 0.f;
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) O[k][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto issue_k = [&](int ts, KRegs& R) {
    if constexpr (L::KL) {       // whole rows, as V
#pragma unroll
      for (int u = 0; u < G::VLD; ++u) {
        const int rr = u * G::RPI + lane / G::CH;
        if constexpr (WIDE) {
          R.k[u] = ld16(kbase + cell_off64(ts + rr, rowstride) + 16 * (lane % G::CH));
        } else {
          const uint32_t vo = cell_off(ts + rr, rowstride) + 16 * (lane % G::CH);
          R.k[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, vo, 0, kNT);
        }
      }
    } else {                     // the lane's MFMA operand fragments
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        if constexpr (WIDE) {
          const uint8_t* row = kbase + cell_off64(ts + 16 * cb + lr, rowstride) + 16 * lb;
#pragma unroll
          for (int j = 0; j < G::KLD; ++j) R.k[cb * G::KLD + j] = ld16(row + 64 * j);
        } else {
          const uint32_t vo = cell_off(ts + 16 * cb + lr, rowstride) + 16 * lb;
#pragma unroll
          for (int j = 0; j < G::KLD; ++j)
            R.k[cb * G::KLD + j] = __builtin_amdgcn_raw_buffer_load_b128(rk, vo + 64 * j, 0, kNT);
        }
      }
    }
  };

  auto issue_v = [&](int ts, VRegs& R) {
#pragma unroll
    for (int u = 0; u < G::VLD; ++u) {
      const int rr = u * G::RPI + lane / G::CH;
      if constexpr (WIDE) {
        R.v[u] = ld16(vbase + cell_off64(ts + rr, rowstride) + 16 * (lane % G::CH));
      } else {
        const uint32_t vo = cell_off(ts + rr, rowstride) + 16 * (lane % G::CH);
        R.v[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo, 0, kNT);
      }
    }
    if constexpr (I8 && WIDE) {
      const size_t so = cell_off64(ts + (lane & 31), srow);
      if constexpr (G::NG == 4) {
        R.ks = *reinterpret_cast<const u32x2*>(ksbase + so);
        R.vs = *reinterpret_cast<const u32x2*>(vsbase + so);
      } else if constexpr (G::NG == 2) {
        R.ks[0] = *reinterpret_cast<const uint32_t*>(ksbase + so);
        R.vs[0] = *reinterpret_cast<const uint32_t*>(vsbase + so);
      } else {
        R.ks[0] = *reinterpret_cast<const uint16_t*>(ksbase + so);
        R.vs[0] = *reinterpret_cast<const uint16_t*>(vsbase + so);
      }
    } else if constexpr (I8) {
      const uint32_t vo = cell_off(ts + (lane & 31), srow);
      if constexpr (G::NG == 4) {
        R.ks = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rks, vo, 0, 0));
        R.vs = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rvs, vo, 0, 0));
      } else if constexpr (G::NG == 2) {
        R.ks[0] = __builtin_amdgcn_raw_buffer_load_b32(rks, vo, 0, 0);
        R.vs[0] = __builtin_amdgcn_raw_buffer_load_b32(rvs, vo, 0, 0);
      } else {
        R.ks[0] = __builtin_amdgcn_raw_buffer_load_b16(rks, vo, 0, 0);
        R.vs[0] = __builtin_amdgcn_raw_buffer_load_b16(rvs, vo, 0, 0);
      }
    }
  };

  auto stage = [&](const VRegs& R, const KRegs& RK) {
#pragma unroll
    for (int u = 0; u < G::VLD; ++u) {
      const int rr = u * G::RPI + lane / G::CH;
      *reinterpret_cast<u32x4*>(vt + G::lds_off(rr, lane % G::CH)) = R.v[u];
      if constexpr (L::KL)
        *reinterpret_cast<u32x4*>(kt + G::lds_offk(rr, lane % G::CH)) = RK.k[u];
    }
    if constexpr (I8) {
      // every lane holds the scales of cell lane % 32
      int ef = (int)f16x2_max_expfield(R.vs[0]);
      if constexpr (G::NG == 4) {
        const int e1 = (int)f16x2_max_expfield(R.vs[1]);
        ef = ef > e1 ? ef : e1;
      }
      if (__any(ef > vexp)) {                    // a larger V scale: fewer guard bits
        const int vn = wave_max_u5(ef);
        vf = __builtin_amdgcn_ldexpf(vf, vexp - vn);
        vexp = vn;
      }
      // lanes 0-31 store the K scales of cells 0-31, lanes 32-63 the V
      // scales times 2^(21 - vexp), both as fp32, group-major
      const float fac = lane < 32 ? 1.0f : __builtin_amdgcn_ldexpf(1.0f, 21 - vexp);
      const u32x2 sv = lane < 32 ? R.ks : R.vs;
      float* dst = sclf + (lane >> 5) * G::NG * TC + (lane & 31);
#pragma unroll
      for (int gi = 0; gi < G::NG; ++gi) {
        const uint16_t h = (uint16_t)(sv[gi >> 1] >> (16 * (gi & 1)));
        dst[gi * TC] = (float)__builtin_bit_cast(_Float16, h) * fac;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  };

  // K operand fragment of lane (lr, lb) for cell block cb, 16-byte chunk
  // lb + 4j of the row: dims 8lb + 32j .. +7 (f16) or 16lb + 64j .. +15 (int8)
  auto kfrag = [&](const KRegs& R, int cb, int j) -> u32x4 {
    if constexpr (L::KL)
      return *reinterpret_cast<const u32x4*>(kt + G::lds_offk(16 * cb + lr, lb + 4 * j));
    else
      return R.k[cb * G::KLD + j];
  };

  // ---- QK: S[cb][k][i] = score of cell ts+16cb+4lb+i for row 16k+lr ----
  auto qk = [&](const KRegs& R, f32x4 (&S)[2][NRB]) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int k = 0; k < NRB; ++k) S[cb][k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (!I8) {
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) {
#pragma unroll
        for (int k = 0; k < NRB; ++k) {
          const half8 qh = __builtin_bit_cast(half8, qlds[((k * G::KS + ks) * 2 + 0) * 64 + lane]);
          const half8 ql = __builtin_bit_cast(half8, qlds[((k * G::KS + ks) * 2 + 1) * 64 + lane]);
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            const half8 ka = __builtin_bit_cast(half8, kfrag(R, cb, ks));
            S[cb][k] = mfma16(ka, qh, S[cb][k]);
            S[cb][k] = mfma16(ka, ql, S[cb][k]);
          }
        }
      }
    } else {
#pragma unroll
      for (int gi = 0; gi < G::NG; ++gi) {
        half8 k0[2], k1[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          const u32x4 w = kfrag(R, cb, gi);
          k0[cb] = i8x8_to_half8(w[0], w[1]);
          k1[cb] = i8x8_to_half8(w[2], w[3]);
        }
#pragma unroll
        for (int k = 0; k < NRB; ++k) {
          const int b0 = (k * G::KS + 2 * gi) * 2;
          const half8 qh0 = __builtin_bit_cast(half8, qlds[(b0 + 0) * 64 + lane]);
          const half8 ql0 = __builtin_bit_cast(half8, qlds[(b0 + 1) * 64 + lane]);
          const half8 qh1 = __builtin_bit_cast(half8, qlds[(b0 + 2) * 64 + lane]);
          const half8 ql1 = __builtin_bit_cast(half8, qlds[(b0 + 3) * 64 + lane]);
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            f32x4 C = f32x4{0.f, 0.f, 0.f, 0.f};
            C = mfma16(k0[cb], qh0, C);
            C = mfma16(k0[cb], ql0, C);
            C = mfma16(k1[cb], qh1, C);
            C = mfma16(k1[cb], ql1, C);
            // K scales of this lane's four output cells 16cb+4lb+i, group gi
            const f32x4 ksv = *reinterpret_cast<const f32x4*>(sclf + gi * TC + 16 * cb + 4 * lb);
#pragma unroll
            for (int i = 0; i < 4; ++i) S[cb][k][i] = __builtin_fmaf(C[i], ksv[i], S[cb][k][i]);
          }
        }
      }
    }

  };

  // ---- online softmax per query row (this lane: row 16k+lr, 8 cells), then PV ----
  auto softmax_pv = [&](int ts, const f32x4 (&S)[2][NRB]) {
    const bool edge = ts + TC > lim_lo;          // wave-uniform
    float pr[NRB][8];
#pragma unroll
    for (int k = 0; k < NRB; ++k) {
      float x[8];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * cb + i] = S[cb][k][i];
      if (edge) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (ts + 16 * cb + 4 * lb + i >= lim[k]) x[4 * cb + i] = -INFINITY;
      }
      // x holds the scores of the normalised query row: the score is x * rs
      float tmax = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, x[e]);
      tmax = max_x32(max_x16(tmax)) * rs[k];
      // The reference max m_run moves only when this tile's max exceeds it
      // by more than kTau (always on a row's first visible cell); the
      // accumulators are rescaled only then.  exp2 of the reference offset is
      // exact math: (o, m, l) stays a valid partial for any reference m.
      const float mold = m_run[k];
      const bool bump = tmax > mold + kTau;
      const float mnew = bump ? tmax : mold;
      const float corr = bump && mold != -INFINITY ? __builtin_amdgcn_exp2f(mold - mnew) : 1.0f;
      const float mref = I8 ? mnew : mnew - kPShift;
      float psum = 0.f;
      if (edge) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe =
              (x[e] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], rs[k], -mref));
          pr[k][e] = pe;
          psum += pe;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], rs[k], -mref));
          pr[k][e] = pe;
          psum += pe;
        }
      }
      psum = sum_x32(sum_x16(psum));
      l_run[k] = l_run[k] * corr + psum;
      m_run[k] = mnew;
      // rescale the accumulator rows 16k+4lb+i by their row's correction
      // (int8: times the pending V-exponent factor)
      if (__any(corr != 1.0f) || (I8 && vf != 1.0f)) {
        float cf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cf[i] = __shfl(corr, 4 * lb + i, 64) * (I8 ? vf : 1.0f);
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[k][nb][i] *= cf[i];
      }
    }
    if constexpr (I8) vf = 1.0f;

    // ---- PV ----
    const int lam = lane & 15;
    if constexpr (!I8) {
      half8 phi[NRB], plo[NRB];
#pragma unroll
      for (int k = 0; k < NRB; ++k) split_hi_lo(pr[k], phi[k], plo[k]);
      // ds_read_b64_tr_b16: source lane (j = lam/4, q = lam%4) points at
      // row cell(j) and dims 16nb + 4q .. +3; result lane i gets 4 cells of dim i.
      const int j = lam >> 2, q = lam & 3;
      const int ra = 4 * lb + j, rb2 = 16 + 4 * lb + j;
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) {
        const int c = 2 * nb + (q >> 1);
        const int off = 8 * (q & 1);
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            GQA_LDS(s16x4, vt + G::lds_off(ra, c) + off));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            GQA_LDS(s16x4, vt + G::lds_off(rb2, c) + off));
        // whole-vector bit casts only: a bit cast of a single vector element
        // reads element 0 with this compiler
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo4);
        const u32x2 hi2 = __builtin_bit_cast(u32x2, hi4);
        const u32x4 w = {lo2[0], lo2[1], hi2[0], hi2[1]};
        const half8 b = __builtin_bit_cast(half8, w);
#pragma unroll
        for (int k = 0; k < NRB; ++k) {
          O[k][nb] = mfma16(phi[k], b, O[k][nb]);
          O[k][nb] = mfma16(plo[k], b, O[k][nb]);
        }
      }
    } else {
      // ds_read_b64_tr_b8: source lane (j = lam/2, h = lam%2) points at row
      // cell(j) and bytes 16nb + 8h .. +7; result lane i gets 8 cells of dim i.
      const int j = lam >> 1, h = lam & 1;
      const int rr = (j < 4) ? 4 * lb + j : 16 + 4 * lb + (j - 4);
      const float* vs_l = sclf + G::NG * TC;
#pragma unroll
      for (int gi = 0; gi < G::NG; ++gi) {
        // V scales (times 2^(21 - vexp)) of cells 4lb..4lb+3 and 16+4lb..16+4lb+3
        const f32x4 va = *reinterpret_cast<const f32x4*>(vs_l + gi * TC + 4 * lb);
        const f32x4 vb = *reinterpret_cast<const f32x4*>(vs_l + gi * TC + 16 + 4 * lb);
        half8 phi[NRB], plo[NRB];
#pragma unroll
        for (int k = 0; k < NRB; ++k) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pv[e] = pr[k][e] * va[e];
            pv[4 + e] = pr[k][4 + e] * vb[e];
          }
          split_hi_lo(pv, phi[k], plo[k]);
        }
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) {
          const int nb = 4 * gi + nn;
          const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              GQA_LDS(i32x2, vt + G::lds_off(rr, nb) + 8 * h));
          const half8 b = i8x8_to_half8((uint32_t)raw[0], (uint32_t)raw[1]);
#pragma unroll
          for (int k = 0; k < NRB; ++k) {
            O[k][nb] = mfma16(phi[k], b, O[k][nb]);
            O[k][nb] = mfma16(plo[k], b, O[k][nb]);
          }
        }
      }
    }
  };

  // ---- main loop over this wave's tiles.  One register set each for K and
  // V: V(t+1) is requested as soon as V(t) is in LDS, K(t+1) as soon as QK(t)
  // has consumed K(t); the second wave on the SIMD covers the rest. ----
  {
    KRegs RK;
    VRegs RV;
    int ts = c0 + TC * wave;
    if constexpr (IDS) __syncthreads();   // the split's ids are staged
    // The first tile is requested before the query operands are staged, so
    // its latency overlaps that work.  Same issue order as inside the loop
    // (V, then K), so the wait counts at the loop head hold on both paths
    // into it.
    issue_v(ts, RV);
    issue_k(ts, RK);
    if constexpr (QPRE) {
#pragma unroll
      for (int i = 0; i < QPT; ++i) q_note(tid + NT * i, qv[i][0], qv[i][1]);
    } else {
      for (int slot = tid; slot < QSLOTS; slot += NT) {
        float4 u0, u1;
        q_load(slot, u0, u1);
        q_note(slot, u0, u1);
      }
    }
    if constexpr (!QREG) {
      if (lane < 16) {
#pragma unroll
        for (int k = 0; k < NRB; ++k) qred[wave * RB + 16 * k + lane] = qmx[k];
      }
      __syncthreads();   // row maxima of q staged
    }
#pragma unroll
    for (int k = 0; k < NRB; ++k) (void)q_row_factor(row_max(16 * k + lr), a.qmant, a.qexp, &rs[k]);
    if constexpr (QPRE) {
#pragma unroll
      for (int i = 0; i < QPT; ++i) q_store(tid + NT * i, qv[i][0], qv[i][1]);
    } else {
      for (int slot = tid; slot < QSLOTS; slot += NT) {
        float4 u0, u1;
        q_load(slot, u0, u1);
        q_store(slot, u0, u1);
      }
    }
    __syncthreads();   // query operands staged
    // One tile; MORE: request the wave's next tile (the last tile requests
    // nothing, so the combine's barrier does not wait on loads past the
    // split).  Two copies of the body rather than a branch around the
    // requests, which would leave the loop head's wait counts inexact.
    auto step = [&](int t0, auto more) {
      constexpr bool MORE = decltype(more)::value;
      const int tn = t0 + NW * TC;
      stage(RV, RK);
      if constexpr (MORE) issue_v(tn, RV);
      f32x4 S[2][NRB];
      if constexpr (L::KL) {
        if constexpr (MORE) issue_k(tn, RK);
        qk(RK, S);
      } else {
        qk(RK, S);
        if constexpr (MORE) issue_k(tn, RK);
      }
      softmax_pv(t0, S);
    };
    if (ts < cend) {
#pragma unroll 1
      while (ts + NW * TC < cend) {
        step(ts, std::integral_constant<bool, true>{});
        ts += NW * TC;
      }
      step(ts, std::integral_constant<bool, false>{});
    }
  }

  // The accumulators hold o * 2^kPShift (f16 V, whose l carries the same
  // factor) or o * 2^(21 - vexp) (int8 V, whose l does not): written as the
  // equivalent partial (o * 2^x, m - x, l * 2^x).
#pragma unroll
  for (int k = 0; k < NRB; ++k) {
    if constexpr (I8) {
      m_run[k] -= (float)(21 - vexp);
      l_run[k] = __builtin_amdgcn_ldexpf(l_run[k], 21 - vexp);
    } else {
      m_run[k] -= kPShift;
    }
  }

  if constexpr (NW == 1) {
    // ---- a single wave: its state is the partial.  Lane (lr, lb) holds
    // rows 16k+4lb+i at dims 16nb+lr, and m, l of row 16k+lr. ----
#pragma unroll
    for (int k = 0; k < NRB; ++k) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 16 * k + 4 * lb + i;
        if (r < a.R) {
          float* dst = a.part_o + (((size_t)(s * a.T + row_t(r)) * a.H + row_h(r)) * a.P + p) * D + lr;
#pragma unroll
          for (int nb = 0; nb < G::NB; ++nb) dst[16 * nb] = O[k][nb][i];
        }
      }
      const int r = r0 + 16 * k + lr;
      if (lb == 0 && r < a.R) {
        const size_t prow = ((size_t)(s * a.T + row_t(r)) * a.H + row_h(r)) * a.P + p;
        a.part_ml[prow * 2] = m_run[k];
        a.part_ml[prow * 2 + 1] = l_run[k];
      }
    }
    return;
  }

  // ---- combine the NW waves: one partial per query row. ----
  if constexpr (L::ONE_PASS) {
    // Every wave parks its (m, l) and its unscaled accumulators in its own
    // buffer; after one barrier each output element is the sum over the
    // waves of exp2(m_w - M) * o_w, with M the rows' common max.
    __syncthreads();                               // the tiles the buffers alias are done with
    if (lb == 0) {
#pragma unroll
      for (int k = 0; k < NRB; ++k) {
        mls[(wave * RB + 16 * k + lr) * 2] = m_run[k];
        mls[(wave * RB + 16 * k + lr) * 2 + 1] = l_run[k];
      }
    }
    constexpr int RS = L::RS;
    float* bw = reinterpret_cast<float*>(smem) + wave * RB * RS;
#pragma unroll
    for (int k = 0; k < NRB; ++k)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) bw[(16 * k + 4 * lb + i) * RS + 16 * nb + lr] = O[k][nb][i];
    __syncthreads();
    const float* b0 = reinterpret_cast<const float*>(smem);
#pragma unroll
    for (int idx = tid; idx < RB * D / 4; idx += NT) {
      const int row = idx / (D / 4);
      const int d4 = idx % (D / 4);
      const int r = r0 + row;
      if (r < a.R) {
        float mw[NW], M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          mw[w] = mls[(w * RB + row) * 2];
          M = fmaxf(M, mw[w]);
        }
        float4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float f = (mw[w] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
          const float4 y = *reinterpret_cast<const float4*>(b0 + w * RB * RS + row * RS + 4 * d4);
          x.x = __builtin_fmaf(f, y.x, x.x);
          x.y = __builtin_fmaf(f, y.y, x.y);
          x.z = __builtin_fmaf(f, y.z, x.z);
          x.w = __builtin_fmaf(f, y.w, x.w);
        }
        const size_t prow = ((size_t)(s * a.T + row_t(r)) * a.H + row_h(r)) * a.P + p;
        *reinterpret_cast<float4*>(a.part_o + prow * D + 4 * d4) = x;
      }
    }
  } else {
    // Two passes: each wave rescales its accumulators to the rows' common max,
    // the upper half of the waves parks them in LDS, the lower half adds
    // theirs, and the NW/2 sums are added while the partial is written.
    constexpr int HALF = NW / 2 > 0 ? NW / 2 : 1;
    constexpr int RS = L::RS;
    __syncthreads();
    if (lb == 0) {
#pragma unroll
      for (int k = 0; k < NRB; ++k) {
        mls[(wave * RB + 16 * k + lr) * 2] = m_run[k];
        mls[(wave * RB + 16 * k + lr) * 2 + 1] = l_run[k];
      }
    }
    __syncthreads();
    float* buf = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int k = 0; k < NRB; ++k) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * k + 4 * lb + i;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, mls[(w * RB + row) * 2]);
        const float ms = mls[(wave * RB + row) * 2];
        const float f = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) O[k][nb][i] *= f;
      }
    }
    if (wave >= HALF) {
      float* b = buf + (wave - HALF) * RB * RS;
#pragma unroll
      for (int k = 0; k < NRB; ++k)
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) b[(16 * k + 4 * lb + i) * RS + 16 * nb + lr] = O[k][nb][i];
    }
    __syncthreads();
    if (wave < HALF) {
      float* b = buf + wave * RB * RS;
#pragma unroll
      for (int k = 0; k < NRB; ++k)
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* x = b + (16 * k + 4 * lb + i) * RS + 16 * nb + lr;
            *x = *x + O[k][nb][i];
          }
    }
    __syncthreads();
    for (int idx = tid; idx < RB * D / 4; idx += NT) {
      const int row = idx / (D / 4);
      const int d4 = idx % (D / 4);
      const int r = r0 + row;
      if (r < a.R) {
        float4 x = *reinterpret_cast<const float4*>(buf + row * RS + 4 * d4);
#pragma unroll
        for (int w = 1; w < HALF; ++w) {
          const float4 y = *reinterpret_cast<const float4*>(buf + w * RB * RS + row * RS + 4 * d4);
          x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
        }
        const size_t prow = ((size_t)(s * a.T + row_t(r)) * a.H + row_h(r)) * a.P + p;
        *reinterpret_cast<float4*>(a.part_o + prow * D + 4 * d4) = x;
      }
    }
  }
  if (tid < RB && r0 + tid < a.R) {
    const int row = tid;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mls[(w * RB + row) * 2]);
    float Ls = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = mls[(w * RB + row) * 2];
      if (mw != -INFINITY) Ls += mls[(w * RB + row) * 2 + 1] * __builtin_amdgcn_exp2f(mw - M);
    }
    const int r = r0 + row;
    const size_t prow = ((size_t)(s * a.T + row_t(r)) * a.H + row_h(r)) * a.P + p;
    a.part_ml[prow * 2] = M;
    a.part_ml[prow * 2 + 1] = Ls;
  }
}


// Split grid: one workgroup per (split p, KV head [, row block] [, token],
// sequence), 1-D and XCD-aware.  Consecutive workgroups are dispatched to
// different XCDs (8 of them, each with its own L2 and its own share of the
// fabric), so the index that varies fastest must carry equal work: the KV
// head, then the sequence; the split index varies slowest, because the last
// splits of short sequences are empty and would otherwise all land on the
// same XCDs.  With a.seq_fast the sequence varies fastest instead: with S a
// multiple of 8 every KV head of a (sequence, split) then runs on the same
// XCD, so the heads' reads of the same cells (int8: the scale lines they
// share, the neighbouring halves of each cell's K/V run) meet in one L2.
template <int D, bool I8, int IDS, int NRB, int NW>
__global__ __launch_bounds__(64 * NW, (attn_occupancy<D, I8, NRB>())) void attn_mfma(AttnArgs a) {
  using Q = QSlots<D, NRB, NW>;
  const int tid = threadIdx.x;
  int id = blockIdx.x;
  int g, s;
  if (a.seq_fast) {
    s = id % a.S;
    id /= a.S;
    g = id % a.Hk;
    id /= a.Hk;
  } else {
    g = id % a.Hk;
    id /= a.Hk;
    s = id % a.S;
    id /= a.S;
  }
  const int nu = a.nrb * (IDS ? a.T : 1);
  const int rbl = (id % nu) % a.nrb;
  const int tq = (id % nu) / a.nrb;
  const int p = id / nu;
  // The query rows are requested before anything waits on memory, so their
  // latency overlaps the sequence-length read and the first tile's requests.
  float4 qv[Q::N][2];
  if constexpr (Q::QPRE) {
#pragma unroll
    for (int i = 0; i < Q::QPT; ++i)
      q_load_slot<D, I8, (IDS != 0)>(a, s, g, tq, rbl * 16 * NRB, tid + Q::NT * i, qv[i][0], qv[i][1]);
  }
  // Gather mode: the split's first NT cell ids do not depend on the
  // sequence length, so they are requested with it and the two reads
  // overlap.
  int id_first = 0;
  if constexpr (IDS) {
    const int64_t pos = (int64_t)p * a.chunk + tid;
    if (tid < a.chunk && pos < a.B) id_first = a.ids[((size_t)s * a.T + tq) * a.B + pos];
  }
  const int seq_len = a.seq_lens[s];
  const int64_t c0l = (int64_t)p * a.chunk;
  attn_unit<D, I8, IDS, NRB, NW>(a, g, s, rbl, tq, p, c0l, c0l + a.chunk, seq_len, id_first, qv);
}

// Balanced grid (dense windows): one workgroup per (KV head, row block,
// piece j), KV head fastest; a.P pieces per (KV head, row block).  The
// piece's real cells are visited sequence by sequence, each sequence's
// segment being one split of that sequence's unit, written as partial slot
// j - (piece of the sequence's first real cell): a sequence's partials fill
// its slots 0 .. n-1, n = the number of pieces holding its real cells, which
// workgroup (0, 0, 0) writes to a.flat_n for the merge.  Every wave walks
// the lengths itself (no LDS, no barrier), so all waves agree on the
// segments; the walk keeps its state in scalar registers (the sequence index
// and the span start), so nothing lane-dependent stays live across units.
template <int D, bool I8, int NRB, int NW>
__global__ __launch_bounds__(64 * NW, (attn_occupancy<D, I8, NRB>())) void attn_mfma_flat(AttnArgs a) {
  using Q = QSlots<D, NRB, NW>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // Piece order.  With a piece count divisible by the 8 XCDs, for int8 rows
  // or fewer than 8 (KV head, row block) pairs: XCD x (workgroup id mod 8)
  // takes the contiguous pieces [x P/8, (x+1) P/8) with every KV head and
  // row block of each (their ids differ by multiples of 8), so the scale
  // lines the heads of a cell share (int8) and the rows around a piece
  // boundary meet in one L2.  Otherwise (f16 with 8 or more pairs, or P not
  // a multiple of 8) the KV head varies fastest: XCD x streams the same
  // heads of every piece.
  int id = blockIdx.x;
  int g, rbl, j;
  if (a.P % 8 == 0 && (I8 || a.Hk * a.nrb < 8)) {
    const int li = id / 8;
    g = li % a.Hk;
    rbl = li / a.Hk % a.nrb;
    j = (id % 8) * (a.P / 8) + li / (a.Hk * a.nrb);
  } else {
    g = id % a.Hk;
    id /= a.Hk;
    rbl = id % a.nrb;
    j = id / a.nrb;
  }
  // The first 64 lengths stay in registers (one per lane) for the whole
  // walk: the plan needs one round trip to memory before the first unit's
  // requests, and the walk reads them with lane reads.  Batches of more
  // than 64 sequences read the rest in passes of 64.
  const int L0 = lane < a.S ? a.seq_lens[lane] : 0;
  // Windows all of one length (empty ones aside): pieces can align with the
  // sequences, and a pad would only shift them off, so none is charged.
  int wlo, whi;
  {
    const int x = flat_window(L0, a.Lmax);
    wlo = x > 0 ? x : 0x7fffffff;
    whi = x;
    for (int c = 64; c < a.S; c += 64) {
      const int y = c + lane < a.S ? flat_window(a.seq_lens[c + lane], a.Lmax) : 0;
      wlo = y > 0 && y < wlo ? y : wlo;
      whi = y > whi ? y : whi;
    }
    wlo = wave_min_i(wlo);
    whi = wave_max_i(whi);
  }
  const int pad = wlo >= whi ? 0 : a.flat_pad;
  const int w0 = lane < a.S ? flat_span(L0, a.Lmax, pad) : 0;
  int W = wave_sum_i(w0);                       // total span
  for (int c = 64; c < a.S; c += 64) {
    const int si = c + lane;
    W += wave_sum_i(si < a.S ? flat_span(a.seq_lens[si], a.Lmax, pad) : 0);
  }
  const int Pe = a.P < W / kFlatQ ? a.P : W / kFlatQ;
  const int end0 = wave_incl_scan_i(w0);        // span ends of sequences 0..63
  if (blockIdx.x == 0 && tid < 64) {
    // every sequence's slot count, for the merge
    int base = 0;
    for (int c = 0; c < a.S; c += 64) {
      const int si = c + lane;
      const int Ls = c == 0 ? L0 : (si < a.S ? a.seq_lens[si] : 0);
      const int w = c == 0 ? w0 : (si < a.S ? flat_span(Ls, a.Lmax, pad) : 0);
      const int end = c == 0 ? end0 : base + wave_incl_scan_i(w);
      const int first = end - w + pad;         // the window's first real cell
      if (si < a.S)
        a.flat_n[si] = w > 0 ? flat_piece(first + flat_window(Ls, a.Lmax) - 1, W, Pe) -
                                   flat_piece(first, W, Pe) + 1
                             : 0;
      base = __builtin_amdgcn_readlane(end, 63);
    }
  }
  if (j >= Pe) return;                          // also W == 0: nothing visible anywhere
  const int b0 = flat_bound(j, W, Pe), b1 = flat_bound(j + 1, W, Pe);
  // the first sequence whose span reaches past b0, and where its span starts
  int s = a.S, st = 0;
  {
    const uint64_t m = __ballot(w0 > 0 && end0 > b0);
    if (m) {
      const int l = __builtin_ctzll(m);
      s = l;
      st = __builtin_amdgcn_readlane(end0, l) - __builtin_amdgcn_readlane(w0, l);
    } else {
      int base = __builtin_amdgcn_readlane(end0, 63);
      for (int c = 64; c < a.S; c += 64) {
        const int si = c + lane;
        const int w = si < a.S ? flat_span(a.seq_lens[si], a.Lmax, pad) : 0;
        const int end = base + wave_incl_scan_i(w);
        const uint64_t mc = __ballot(w > 0 && end > b0);
        if (mc) {
          const int l = __builtin_ctzll(mc);
          s = c + l;
          st = __builtin_amdgcn_readlane(end, l) - __builtin_amdgcn_readlane(w, l);
          break;
        }
        base = __builtin_amdgcn_readlane(end, 63);
      }
    }
  }
  s = __builtin_amdgcn_readfirstlane(s);
  st = __builtin_amdgcn_readfirstlane(st);
  for (; s < a.S && st < b1; ++s) {
    const int L = s < 64 ? __builtin_amdgcn_readlane(L0, s) : a.seq_lens[s];
    const int ws = flat_window(L, a.Lmax);
    if (ws == 0) continue;
    const int c0 = st + pad;                    // the window's first real cell
    const int lo = c0 > b0 ? c0 : b0;
    const int hi = c0 + ws < b1 ? c0 + ws : b1;
    if (lo < hi) {
      const int p = j - flat_piece(c0, W, Pe);
      float4 qv[Q::N][2];
      if constexpr (Q::QPRE) {
#pragma unroll
        for (int i = 0; i < Q::QPT; ++i)
          q_load_slot<D, I8, false>(a, s, g, 0, rbl * 16 * NRB, tid + Q::NT * i, qv[i][0], qv[i][1]);
      }
      attn_unit<D, I8, 0, NRB, NW, true>(a, g, s, rbl, 0, p, lo - c0, hi - c0, L, 0, qv);
      __syncthreads();                          // LDS is restaged by the next segment
    }
    st = c0 + (ws + kFlatQ - 1) / kFlatQ * kFlatQ;
  }
}

}  // namespace gqa_kern
