// Chunk kernel over a TurboQuant-compressed KV cache (cera 0.4.0,
// flash_attention_tq.metal) on the gfx950 matrix cores.
//
// Per cell c of a KV head the cache holds, as the page lays it out:
//   K: D/16 words of 2-bit polar indices, D/32 words of QJL sign bits, and one
//      word holding the f16 key norm (low half) and f16 residual norm (high);
//   V: D/16 words of 2-bit polar indices and one word with the f16 value norm.
// The query arrives rotated (q_rot) and JL-projected (q_jl).  Score and value
// (the page's header):
//   score = scale * norm * (sum_d q_rot[d] c[idx_k[d]]
//                           + residual * qjl_scale * sum_d q_jl[d] (2 bit[d] - 1))
//   acc[d] += p * vnorm * c[idx_v[d]]        (rotated basis; the inverse
//                                             rotation runs after the merge)
// Keys and values are never rebuilt in the original basis.
//
// Layout of the work is that of the dense attention kernel: one workgroup per
// (split, KV head, row block, sequence), four waves streaming their own
// 32-cell tiles with their own online softmax (base 2, lazy rescale),
// combined into one partial (o in the rotated basis, m, l) per query row.
//
// QK on v_mfma_f32_16x16x32_f16: A = decoded key fragments, B = the query
// rows.  Lane group lb (lanes 16 lb .. 16 lb + 15) owns dims [lb D/4, (lb+1)
// D/4) of every cell -- D/64 polar words and D/4 sign bits -- and covers
// 8 of them per k-step; the query operands use the same dim assignment.
//   polar:  each pair of 2-bit indices looks up the f16 high and low parts
//           of its two centroids in 16-entry LDS tables, so q_rot . c[idx]
//           keeps ~22 bits: hi*hi + hi*lo + lo*hi.
//   QJL:    each nibble of sign bits looks up four f16 2 / 0 values; the
//           MFMA, its accumulator started at -sum_d q_jl[d], gives the page's
//           signed sum 2 * (sum over set bits) - sum_d q_jl[d] directly.
// PV on the same MFMA: A = p * vnorm (f16 hi + lo) straight from the score
// accumulators, B = decoded value fragments: a lane needs one dim of eight
// cells, so the tile's V index words are restaged in LDS as ready lookup
// addresses (two cells' fields interleaved per 4-bit group), one byte
// extract per lookup.
// Up to 8 query rows per KV head (packed instances): the f16 hi parts of the
// query (and of p * vnorm) take MFMA columns (rows) 0-7 and the lo parts
// 8-15, and centroid pairs are looked up as [hi lo] with one two-dword read,
// the other operand laid out against that alternation: 40 instead of 64
// MFMAs and 115 instead of 182 LDS instructions per 32-cell tile.
// Ranges, as in the dense kernel: each query row (q_rot and q_jl together)
// is multiplied by a power of two that puts its largest element in
// [2^13, 2^14) before its f16 hi + lo split (the scores take the inverse
// power inside the exponent), and p * vnorm carries a per-wave factor
// 2^(21 - vexp), vexp the largest f16 exponent field of the value norms seen
// so far, so that it stays below 2^15 and far above f16's subnormal step;
// the partial is written as (o, m - x, l * 2^x).
#pragma once

#include "common.h"
#include "mfma_util.h"

namespace gqa_kern {

struct TqArgs {
  const float* q_rot;        // [S][T][H][D]
  const float* q_jl;         // [S][T][H][D]
  const uint32_t* k_polar;   // [S][Hk][Lmax][D/16]
  const uint32_t* k_jl;      // [S][Hk][Lmax][D/32]
  const uint32_t* k_norms;   // [S][Hk][Lmax]
  const uint32_t* v_polar;   // [S][Hk][Lmax][D/16]
  const uint32_t* v_norms;   // [S][Hk][Lmax]
  const int32_t* seq_lens;
  float* part_o;             // [S][T][H][P][D]  (rotated basis)
  float* part_ml;            // [S][T][H][P][2]
  uint32_t chi_lo, chi_hi;   // f16 high parts of centroids 0,1 and 2,3 (perm table)
  uint32_t clo_lo, clo_hi;   // f16 low parts (c - f16(c))
  float qjl_scale;
  float qscale;              // scale * log2(e)
  int S, T, Lmax, H, Hk, G, R, nrb, P, chunk;
};

// LDS of one TurboQuant workgroup (four waves).
template <int D, int NRB, bool PK>
struct TqLds {
  static constexpr int NW = 4;
  static constexpr int TC = 32;
  static constexpr int RB = 16 * NRB;
  static constexpr int KS = D / 32;
  static constexpr int VW = D / 16;                          // V index words per cell
  // per-wave V index words staged as lookup addresses, VS dwords per word
  // (see the staging)
  static constexpr int VS = 2 * TC + 16 / VW;                 // (VW / 2) VS = 8 mod 32
  static constexpr int VT = NW * VW * VS * 4;
  static constexpr int NM = NW * 3 * TC * 4;                 // per-wave (n, rq) per cell and value norms
  // q_rot and q_jl operands: hi and lo separately, or (packed) hi parts in
  // columns 0-7 and lo parts in 8-15, q_rot as two operands per k-step laid
  // out against keys whose hi and lo pairs alternate
  static constexpr int QB = (PK ? 3 * KS : 2 * NRB * KS * 2) * 64 * 16;
  static constexpr int QS = RB * 4;                          // per-row sum of q_jl
  static constexpr int ML = NW * RB * 2 * 4;
  // cross-wave combine (aliases VT, NM, QB), rows of RS = D + 4 floats: a
  // stride of 4 mod 8 dwords keeps the parking stores of a half-wave's two
  // lane groups in different halves of the 32 banks
  static constexpr int RS = D + 4;
  static constexpr int BUF = NW / 2 * RB * RS * 4;
  static constexpr int MAIN = VT + NM + QB;
  static constexpr int BYTES = (MAIN > BUF ? MAIN : BUF) + QS + ML;
};

// Decoding goes through 16-entry tables in the kernel's static LDS (at fixed
// addresses, so a lookup's address is a 4-bit group of the cache word scaled
// to the entry size), built once per workgroup; a lookup replaces the bit
// arithmetic:
//   chi[u], u = (b << 2) | a for two 2-bit indices a, b: the f16 high parts
//           of centroids a and b (one dword of the MFMA operand);
//   clo[u]  their f16 low parts -- 1028 bytes after chi: farther than a
//           paired dword read reaches and not a multiple of 256 bytes, so the
//           compiler cannot fuse a chi and a clo read into one two-dword read
//           (whose two results land in adjacent registers and then need a move
//           each into the hi and lo operand registers);
//   jtab[u], u = four sign bits: four f16 values, 2 where the bit is set and
//           0 elsewhere;
//   chl[u]  chi[u] and clo[u] side by side, one two-dword read for both
//           (the packed instances, whose other operand is laid out to take
//           hi and lo pairs alternately).
// Each table's entries sit in distinct banks, so a wave's lookups never
// conflict (equal entries broadcast; larger tables indexed by a whole byte
// would conflict on random codes).  The address of a 4-bit group is the
// group moved to bits 2-5 (chi, clo) or 3-6 (jtab, chl) of a byte and masked: each
// word is shifted once per direction, after which every group of it sits at
// those bits of some byte of one of the two shifted copies, and one masked
// byte select gives its address.
constexpr int kTqCtabHi = 0, kTqJtab = 64, kTqCtabHL = 192, kTqCtabLo = 1028, kTqTabBytes = 1104;

__device__ __forceinline__ uint32_t lds_u32(const uint8_t* base, uint32_t byte) {
  return *reinterpret_cast<const uint32_t*>(base + byte);
}

// x & m restricted to byte b of x (b a compile-time constant after
// unrolling): one VALU operation with an SDWA byte select, which this compiler
// does not form by itself from a shift and a mask.
__device__ __forceinline__ uint32_t and_byte(uint32_t x, uint32_t m, int b) {
  uint32_t r;
  switch (b) {
    case 0: r = x & m; break;
    case 1:
      asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
          : "=v"(r) : "v"(m), "v"(x));
      break;
    case 2:
      asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
          : "=v"(r) : "v"(m), "v"(x));
      break;
    default:
      asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
          : "=v"(r) : "v"(m), "v"(x));
      break;
  }
  return r;
}

// A polar word prepared for lookups: e = w << 2 holds the even 4-bit groups
// (index pairs 0, 2, 4, 6) at bits 2-5 of bytes 0..3, o = w >> 2 the odd ones.
struct PolarWord {
  uint32_t e, o;
};
__device__ __forceinline__ PolarWord polar_word(uint32_t w) { return PolarWord{w << 2, w >> 2}; }
__device__ __forceinline__ uint32_t polar_addr(const PolarWord& p, int i) {   // group i = 0..7
  return and_byte((i & 1) ? p.o : p.e, 0x3Cu, i >> 1);
}

// Eight 2-bit indices (4-bit groups g0 .. g0+3 of the word) -> f16 high and
// low parts of their centroids.
__device__ __forceinline__ void tq_polar8(const PolarWord& p, int g0, const uint8_t* tab,
                                          half8& hi, half8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t a4 = polar_addr(p, g0 + j);
    h[j] = lds_u32(tab + kTqCtabHi, a4);
    l[j] = lds_u32(tab + kTqCtabLo, a4);
  }
  hi = __builtin_bit_cast(half8, h);
  lo = __builtin_bit_cast(half8, l);
}

// A sign word prepared for lookups: lo = w << 3 holds the low 4 bits of each
// byte at bits 3-6 of that byte, hi = w >> 1 the high 4 bits.
struct SignWord {
  uint32_t lo, hi;
};
__device__ __forceinline__ SignWord sign_word(uint32_t w) { return SignWord{w << 3, w >> 1}; }

// Eight sign bits (byte b of the word) -> f16 2.0 where set, 0 elsewhere.
__device__ __forceinline__ half8 tq_bits8(const SignWord& p, int b, const uint8_t* tab) {
  const uint32_t a0 = and_byte(p.lo, 0x78u, b);
  const uint32_t a1 = and_byte(p.hi, 0x78u, b);
  const u32x2 e0 = *reinterpret_cast<const u32x2*>(tab + kTqJtab + a0);
  const u32x2 e1 = *reinterpret_cast<const u32x2*>(tab + kTqJtab + a1);
  const u32x4 r = {e0[0], e0[1], e1[0], e1[1]};
  return __builtin_bit_cast(half8, r);
}

// Eight 2-bit indices (4-bit groups g0 .. g0+3 of a polar word prepared like
// a sign word, so that each group's address is the group scaled by 8) -> two
// operands whose dwords alternate the f16 high and low parts of the centroid
// pairs: a = [hi lo] of groups g0 and g0 + 1, b = [hi lo] of groups g0 + 2
// and g0 + 3.
__device__ __forceinline__ void tq_polar8_hl(const SignWord& p, int g0, const uint8_t* tab,
                                             half8& a, half8& b) {
  u32x2 e[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int g = g0 + j;
    const uint32_t a8 = and_byte((g & 1) ? p.hi : p.lo, 0x78u, g >> 1);
    e[j] = *reinterpret_cast<const u32x2*>(tab + kTqCtabHL + a8);
  }
  a = __builtin_bit_cast(half8, u32x4{e[0][0], e[0][1], e[1][0], e[1][1]});
  b = __builtin_bit_cast(half8, u32x4{e[2][0], e[2][1], e[3][0], e[3][1]});
}

// x of lane l ^ 8 (a rotation by 8 within each row of 16 lanes, DPP).
__device__ __forceinline__ float ror8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, true));
}

__device__ __forceinline__ float f16lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float f16hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

template <int D, int NRB, bool PK>
__global__ __launch_bounds__(256, 2) void attn_tq(TqArgs a) {
  using L = TqLds<D, NRB, PK>;
  constexpr int NW = L::NW, NT = 64 * NW, TC = L::TC, RB = L::RB, KS = L::KS, VW = L::VW;
  constexpr int NB = D / 16;                     // 16-dim output blocks
  constexpr int KW = D / 64;                     // polar words per lane group and cell
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(!PK || NRB == 1, "packed operands hold at most 8 rows");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ __attribute__((aligned(16))) uint8_t tab[kTqTabBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15, lb = lane >> 4;

  // 1-D grid: KV head fastest, then sequence, then row block, split slowest
  int id = blockIdx.x;
  const int g = id % a.Hk;
  id /= a.Hk;
  const int s = id % a.S;
  id /= a.S;
  const int rbl = id % a.nrb;
  const int p = id / a.nrb;
  const int r0 = rbl * RB;
  auto row_t = [&](int r) -> int { return r / a.G; };
  auto row_h = [&](int r) -> int { return g * a.G + r % a.G; };

  const int seq_len = a.seq_lens[s];
  auto width_of = [&](int r) -> int {
    if (r >= a.R) return 0;
    int Lt = seq_len - (a.T - 1 - row_t(r));
    return Lt < 0 ? 0 : (Lt > a.Lmax ? a.Lmax : Lt);
  };
  const int rlast = (a.R - 1 < r0 + RB - 1) ? a.R - 1 : r0 + RB - 1;
  const int wmax = width_of(rlast);
  const int64_t c0l = (int64_t)p * a.chunk;
  if (c0l >= wmax) {                             // empty split: weight 0
    if (tid < RB && r0 + tid < a.R) {
      const int r = r0 + tid;
      const size_t prow = ((size_t)(s * a.T + row_t(r)) * a.H + row_h(r)) * a.P + p;
      a.part_ml[prow * 2] = -INFINITY;
      a.part_ml[prow * 2 + 1] = 0.f;
    }
    return;
  }
  const int c0 = (int)c0l;
  const int cend = (int)((c0l + a.chunk < wmax) ? c0l + a.chunk : wmax);
  const int lim_lo = width_of(r0) < cend ? width_of(r0) : cend;

  uint8_t* work = smem;
  uint32_t* vtw = reinterpret_cast<uint32_t*>(work) + wave * VW * L::VS;
  // per cell of this wave's tile: (n, rq) = (key norm * qscale, residual norm
  // * qjl_scale), then the value norm times 2^(21 - vexp)
  float* knf = reinterpret_cast<float*>(work + L::VT) + wave * 3 * TC;
  float* vnf = knf + 2 * TC;
  u32x4* qlds = reinterpret_cast<u32x4*>(work + L::VT + L::NM);
  const int tail = L::MAIN > L::BUF ? L::MAIN : L::BUF;
  float* qsum = reinterpret_cast<float*>(work + tail);
  float* mls = reinterpret_cast<float*>(work + tail + L::QS);
  if (tid < 16) {
    // entry u = (b << 2) | a: the byte selector [2a, 2a+1, 2b, 2b+1] picks
    // the two f16 halves of centroids a and b out of each 8-byte table
    const uint32_t sel = ((uint32_t)(tid & 3) | ((uint32_t)(tid >> 2) << 16)) * 0x0202u + 0x01000100u;
    const uint32_t h = __builtin_amdgcn_perm(a.chi_hi, a.chi_lo, sel);
    const uint32_t l = __builtin_amdgcn_perm(a.clo_hi, a.clo_lo, sel);
    reinterpret_cast<uint32_t*>(tab + kTqCtabHi)[tid] = h;
    reinterpret_cast<uint32_t*>(tab + kTqCtabLo)[tid] = l;
    reinterpret_cast<u32x2*>(tab + kTqCtabHL)[tid] = u32x2{h, l};
  } else if (tid < 32) {
    const uint32_t u = (uint32_t)(tid - 16);
    auto f = [](uint32_t bit) -> uint32_t { return bit ? 0x4000u : 0u; };   // f16 2.0
    reinterpret_cast<u32x2*>(tab + kTqJtab)[u] =
        u32x2{f(u & 1) | (f((u >> 1) & 1) << 16), f((u >> 2) & 1) | (f((u >> 3) & 1) << 16)};
  }

  // ---- query operands: q_rot and q_jl rows as f16 hi + lo, both parts of a
  // row normalised by one power of two (the max |element| of each part per
  // wave first, into qred[which][wave][row], the (m, l) area that the
  // epilogue uses later), and each row's sum of q_jl (fp32) ----
  float* qred = mls;
  // the row of the block that MFMA column (or row) c = 0..15 carries: with
  // packed operands columns 0-7 hold the hi parts of rows 0-7 and columns
  // 8-15 their lo parts
  auto crow = [](int c) -> int { return PK ? (c & 7) : c; };
  auto q_slot = [&](int slot, int& which, int& kks, int& row, float (&x)[8]) {
    which = slot / (NRB * KS * 64);              // 0: q_rot, 1: q_jl
    const int sl = slot % (NRB * KS * 64);
    const int ln = sl & 63;
    kks = sl >> 6;
    const int ks = kks % KS, k = kks / KS;
    row = 16 * k + crow(ln & 15);
    const int r = r0 + row;
    const int d0 = (ln >> 4) * (D / 4) + 8 * ks;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.f;
    if (r < a.R) {
      const float* src = (which ? a.q_jl : a.q_rot) +
                         ((size_t)(s * a.T + row_t(r)) * a.H + row_h(r)) * D + d0;
      const float4 u0 = *reinterpret_cast<const float4*>(src);
      const float4 u1 = *reinterpret_cast<const float4*>(src + 4);
      x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
      x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
    }
  };
  auto row_max = [&](int row) -> float {       // over both parts and all waves
    float m = qred[row];
#pragma unroll
    for (int w = 1; w < 2 * NW; ++w) m = fmaxf(m, qred[w * RB + row]);
    return m;
  };
  {
    float qmx[2][NRB];
#pragma unroll
    for (int w2 = 0; w2 < 2; ++w2)
#pragma unroll
      for (int k = 0; k < NRB; ++k) qmx[w2][k] = 0.f;
    // every lane of a wave passes the same number of slots (wave-wide reductions)
    for (int slot = tid; slot < 2 * NRB * KS * 64; slot += NT) {
      int which, kks, row;
      float x[8];
      q_slot(slot, which, kks, row, x);
      float m = fabsf(x[0]);
#pragma unroll
      for (int e = 1; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
      m = max_x32(max_x16(m));
      const int kb = kks / KS;
#pragma unroll
      for (int w2 = 0; w2 < 2; ++w2)
#pragma unroll
        for (int k = 0; k < NRB; ++k)
          qmx[w2][k] = (which == w2 && kb == k) ? fmaxf(qmx[w2][k], m) : qmx[w2][k];
    }
    if (lane < 16) {
#pragma unroll
      for (int w2 = 0; w2 < 2; ++w2)
#pragma unroll
        for (int k = 0; k < NRB; ++k) qred[(w2 * NW + wave) * RB + 16 * k + lane] = qmx[w2][k];
    }
  }
  auto q_stage = [&]() {
    for (int slot = tid; slot < 2 * NRB * KS * 64; slot += NT) {
      int which, kks, row;
      float x[8];
      q_slot(slot, which, kks, row, x);
      float rs_unused;
      const float f = q_row_factor(row_max(row), 0.5f, 1, &rs_unused);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= f;
      half8 hi, lo;
      split_hi_lo(x, hi, lo);
      if constexpr (PK) {
        const bool hic = (slot & 15) < 8;        // column of a hi part
        const u32x4 h = __builtin_bit_cast(u32x4, hi), l = __builtin_bit_cast(u32x4, lo);
        if (which == 0) {
          // against keys [hi lo hi lo] of dims (0,1), (2,3) and of (4,5),
          // (6,7): hi columns give (c_hi + c_lo) q_hi, lo columns c_hi q_lo
          qlds[(2 * kks) * 64 + (slot & 63)] = hic ? u32x4{h[0], h[0], h[1], h[1]} : u32x4{l[0], 0u, l[1], 0u};
          qlds[(2 * kks + 1) * 64 + (slot & 63)] = hic ? u32x4{h[2], h[2], h[3], h[3]} : u32x4{l[2], 0u, l[3], 0u};
        } else {
          qlds[(2 * KS + kks) * 64 + (slot & 63)] = hic ? h : l;
        }
      } else {
        const int base = ((which * NRB * KS + kks) * 2) * 64;
        qlds[base + (slot & 63)] = __builtin_bit_cast(u32x4, hi);
        qlds[base + 64 + (slot & 63)] = __builtin_bit_cast(u32x4, lo);
      }
    }
  };
  if (tid < RB) {
    const int r = r0 + tid;
    float t = 0.f;
    if (r < a.R) {
      const float* src = a.q_jl + ((size_t)(s * a.T + row_t(r)) * a.H + row_h(r)) * D;
#pragma unroll 8
      for (int d = 0; d < D; d += 4) {
        const float4 u = *reinterpret_cast<const float4*>(src + d);
        t += (u.x + u.y) + (u.z + u.w);
      }
    }
    qsum[tid] = t;
  }

  int lim[NRB];
#pragma unroll
  for (int k = 0; k < NRB; ++k) {
    const int wr = width_of(r0 + 16 * k + crow(lr));
    lim[k] = wr < cend ? wr : cend;
  }

  // ---- compressed rows of this split through range-checked buffer
  // resources: reads past the split's last cell return zeros ----
  const size_t first = ((size_t)s * a.Hk + g) * a.Lmax + c0;
  const uint32_t ncells = (uint32_t)(cend - c0);
  const __amdgpu_buffer_rsrc_t rkp = make_rsrc(a.k_polar + first * VW, ncells * VW * 4);
  const __amdgpu_buffer_rsrc_t rkj = make_rsrc(a.k_jl + first * (D / 32), ncells * (D / 32) * 4);
  const __amdgpu_buffer_rsrc_t rkn = make_rsrc(a.k_norms + first, ncells * 4);
  const __amdgpu_buffer_rsrc_t rvp = make_rsrc(a.v_polar + first * VW, ncells * VW * 4);
  const __amdgpu_buffer_rsrc_t rvn = make_rsrc(a.v_norms + first, ncells * 4);

  struct KRegs {
    uint32_t pol[2][KW];       // this lane's polar words of cells 16 cb + lr
    uint32_t jl[2];            // the sign-bit word holding this lane group's dims
  };
  struct VRegs {
    uint32_t pol[VW / 2];      // lane l: cell l / 2, words (l % 2) * VW/2 ..
    uint32_t nrm;              // lanes 0-31: K norm word of cell l; 32-63: V norm word of cell l - 32
  };

  auto issue_k = [&](int ts, KRegs& R) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const uint32_t cell = (uint32_t)(ts + 16 * cb + lr - c0);
      if constexpr (KW == 2) {
        const u32x2 w = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(rkp, (cell * VW + 2 * lb) * 4, 0, kNT));
        R.pol[cb][0] = w[0];
        R.pol[cb][1] = w[1];
      } else {
        R.pol[cb][0] = __builtin_amdgcn_raw_buffer_load_b32(rkp, (cell * VW + lb) * 4, 0, kNT);
      }
      R.jl[cb] = __builtin_amdgcn_raw_buffer_load_b32(
          rkj, (cell * (D / 32) + (lb * (D / 4)) / 32) * 4, 0, kNT);
    }
  };
  auto issue_v = [&](int ts, VRegs& R) {
    const uint32_t cell = (uint32_t)(ts + (lane >> 1) - c0);
    const uint32_t off = (cell * VW + (lane & 1) * (VW / 2)) * 4;
    if constexpr (VW == 8) {
      const u32x4 w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rvp, off, 0, kNT));
#pragma unroll
      for (int j = 0; j < 4; ++j) R.pol[j] = w[j];
    } else {
      const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rvp, off, 0, kNT));
      R.pol[0] = w[0];
      R.pol[1] = w[1];
    }
    // both norm words of cell l % 32 in every lane (a lane-dependent choice
    // of resource would need a loop over the distinct resources)
    const uint32_t nc = (uint32_t)(ts + (lane & 31) - c0);
    const uint32_t kn = __builtin_amdgcn_raw_buffer_load_b32(rkn, nc * 4, 0, 0);
    const uint32_t vn = __builtin_amdgcn_raw_buffer_load_b32(rvn, nc * 4, 0, 0);
    R.nrm = lane < 32 ? kn : vn;
  };

  constexpr float kTau = 8.0f;
  // p * vnorm carries 2^(21 - vexp), vexp = the largest f16 exponent field
  // of the value norms this wave has seen (norms below 2^(vexp - 14)), so
  // that it stays below 2^8 * 2^7 = 2^15; when vexp grows the accumulators
  // are rescaled by vf with the next softmax correction.
  int vexp = 0;
  float vf = 1.0f;
  auto stage = [&](const VRegs& R) {
    const int cell = lane >> 1;
    {
      // A value lookup takes field f (dim 16 nb + f) of the words of two
      // cells (2i, 2i+1).  Interleave the two words so that 4-bit group m
      // holds field 2m + t of both cells (t = f's parity; the even cell's
      // field in the low bits): the group is the lookup's index.  The even
      // cell's lane builds t = 0 from its word and the odd cell's (lane ^ 2),
      // the odd cell's lane t = 1: a rotation of the other word by 2 bits and
      // a bit-field select.  Each result is stored as two words whose bytes
      // hold the even and the odd groups scaled by the entry size (8 bytes
      // for the packed instances' [hi lo] entries, else 4), so that one byte
      // extract gives a lookup's address.  Layout per word:
      // [pair / 8][parity][half][pair % 8], VS dwords apart with VS VW / 2 =
      // 8 mod 32, so that the stores of a wave and the two-dword reads of
      // the lookups each fall in distinct banks of the 32.
      const bool odd = cell & 1;
      const uint32_t msk = odd ? 0xCCCCCCCCu : 0x33333333u;
#pragma unroll
      for (int j = 0; j < VW / 2; ++j) {
        const uint32_t w = R.pol[j];
        const uint32_t p = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0x4E, 0xF, 0xF, true);   // lane ^ 2
        const uint32_t rot = __builtin_amdgcn_alignbit(p, p, odd ? 2 : 30);
        const uint32_t x = (w & msk) | (rot & ~msk);
        const int pr = cell >> 1;                  // cell pair
        uint32_t* dst = vtw + ((lane & 1) * (VW / 2) + j) * L::VS + (pr >> 3) * 32 + (cell & 1) * 16 + (pr & 7);
        if constexpr (PK) {
          dst[0] = (x << 3) & 0x78787878u;         // groups 0, 2, 4, 6, times 8
          dst[8] = (x >> 1) & 0x78787878u;         // groups 1, 3, 5, 7
        } else {
          dst[0] = (x << 2) & 0x3C3C3C3Cu;         // times 4
          dst[8] = (x >> 2) & 0x3C3C3C3Cu;
        }
      }
    }
    const int ef = lane >= 32 ? (int)((R.nrm & 0x7fffu) >> 10) : 0;
    if (__any(ef > vexp)) {
      const int vn = wave_max_u5(ef);
      vf = __builtin_amdgcn_ldexpf(vf, vexp - vn);
      vexp = vn;
    }
    if (lane < 32) {
      knf[2 * lane] = f16lo(R.nrm) * a.qscale;
      knf[2 * lane + 1] = f16hi(R.nrm) * a.qjl_scale;
    } else {
      vnf[lane - 32] = __builtin_amdgcn_ldexpf(f16lo(R.nrm), 21 - vexp);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  };

  f32x4 O[NRB][NB];
  float m_run[NRB], l_run[NRB];
#pragma unroll
  for (int k = 0; k < NRB; ++k) {
    m_run[k] = -INFINITY;
    l_run[k] = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) O[k][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float qs[NRB];                                 // normalised sum of q_jl of this lane's rows 16k + crow(lr)
  float rs[NRB];                                 // inverse of the rows' normalising factor

  // ---- QK: S[cb][k][i] = score (base 2) of cell ts+16cb+4lb+i for row
  // 16k+crow(lr), times the row's normalising factor.  Packed: the hi and lo
  // parts of a row's query land in columns c and c + 8 of the accumulators,
  // which one rotation of each 16-lane row adds up (lanes c and c + 8 then
  // hold the same row) ----
  auto qk = [&](const KRegs& R, f32x4 (&S)[2][NRB]) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x4 Sp[2][NRB], Sj[2][NRB];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int k = 0; k < NRB; ++k) {
        const float q0 = (!PK || lr < 8) ? -qs[k] : 0.f;
        Sp[cb][k] = f32x4{0.f, 0.f, 0.f, 0.f};
        Sj[cb][k] = f32x4{q0, q0, q0, q0};
      }
    PolarWord pw[2][KW];
    SignWord pw8[2][KW];                         // packed: polar groups scaled by 8
    SignWord sw[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
#pragma unroll
      for (int w = 0; w < KW; ++w) {
        if constexpr (PK) pw8[cb][w] = sign_word(R.pol[cb][w]);
        else pw[cb][w] = polar_word(R.pol[cb][w]);
      }
      // D = 64: the lane group's 16 sign bits are the low or high half of the word
      sw[cb] = sign_word(D == 64 ? R.jl[cb] >> (16 * (lb & 1)) : R.jl[cb]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      half8 ch[2], cl[2], jb[2];
      const int dl = 8 * ks;                     // dim offset inside the lane group's span
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        if constexpr (PK)                        // ch, cl: [hi lo hi lo] of dims 0-3 and of 4-7
          tq_polar8_hl(pw8[cb][dl / 16], (dl % 16) / 2, tab, ch[cb], cl[cb]);
        else
          tq_polar8(pw[cb][dl / 16], (dl % 16) / 2, tab, ch[cb], cl[cb]);
        jb[cb] = tq_bits8(sw[cb], dl / 8, tab);
      }
      if constexpr (PK) {
        // columns 0-7: hi parts, 8-15: lo parts
        const half8 qa = __builtin_bit_cast(half8, qlds[(2 * ks) * 64 + lane]);
        const half8 qb = __builtin_bit_cast(half8, qlds[(2 * ks + 1) * 64 + lane]);
        const half8 jp = __builtin_bit_cast(half8, qlds[(2 * KS + ks) * 64 + lane]);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          Sp[cb][0] = mfma16(ch[cb], qa, Sp[cb][0]);
          Sp[cb][0] = mfma16(cl[cb], qb, Sp[cb][0]);
          Sj[cb][0] = mfma16(jb[cb], jp, Sj[cb][0]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < NRB; ++k) {
          const int br = ((0 * NRB * KS + k * KS + ks) * 2) * 64;
          const int bj = ((1 * NRB * KS + k * KS + ks) * 2) * 64;
          const half8 qh = __builtin_bit_cast(half8, qlds[br + lane]);
          const half8 ql = __builtin_bit_cast(half8, qlds[br + 64 + lane]);
          const half8 jh = __builtin_bit_cast(half8, qlds[bj + lane]);
          const half8 jl = __builtin_bit_cast(half8, qlds[bj + 64 + lane]);
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            Sp[cb][k] = mfma16(ch[cb], qh, Sp[cb][k]);
            Sp[cb][k] = mfma16(ch[cb], ql, Sp[cb][k]);
            Sp[cb][k] = mfma16(cl[cb], qh, Sp[cb][k]);
            Sj[cb][k] = mfma16(jb[cb], jh, Sj[cb][k]);
            Sj[cb][k] = mfma16(jb[cb], jl, Sj[cb][k]);
          }
        }
      }
    }
    if constexpr (PK) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Sp[cb][0][i] += ror8(Sp[cb][0][i]);
          Sj[cb][0][i] += ror8(Sj[cb][0][i]);
        }
    }
    // score = qscale * norm * (polar + residual * qjl_scale * signed sum)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const f32x4 f0 = *reinterpret_cast<const f32x4*>(knf + 2 * (16 * cb + 4 * lb));
      const f32x4 f1 = *reinterpret_cast<const f32x4*>(knf + 2 * (16 * cb + 4 * lb) + 4);
      const float n[4] = {f0[0], f0[2], f1[0], f1[2]};
      const float rq[4] = {f0[1], f0[3], f1[1], f1[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < NRB; ++k)
          S[cb][k][i] = n[i] * __builtin_fmaf(rq[i], Sj[cb][k][i], Sp[cb][k][i]);
    }
  };

  // ---- online softmax per row, then PV in the rotated basis ----
  auto softmax_pv = [&](int ts, const f32x4 (&S)[2][NRB]) {
    const bool edge = ts + TC > lim_lo;
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
      float tmax = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, x[e]);
      tmax = max_x32(max_x16(tmax)) * rs[k];
      const float mold = m_run[k];
      const bool bump = tmax > mold + kTau;
      const float mnew = bump ? tmax : mold;
      const float corr = bump && mold != -INFINITY ? __builtin_amdgcn_exp2f(mold - mnew) : 1.0f;
      // a row with no visible cell yet has every x = -inf: any finite
      // reference gives its weights exp2(-inf) = 0
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], rs[k], -mref));
        pr[k][e] = pe;
        psum += pe;
      }
      psum = sum_x32(sum_x16(psum));
      l_run[k] = l_run[k] * corr + psum;
      m_run[k] = mnew;
      if (__any(corr != 1.0f) || vf != 1.0f) {
        float cf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) cf[i] = __shfl(corr, crow(4 * lb + i), 64) * vf;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[k][nb][i] *= cf[i];
      }
    }
    vf = 1.0f;
    // P' = p * vnorm of each of this lane's eight cells (A operand k = 8 lb + e)
    half8 phi[NRB], plo[NRB];
    {
      const f32x4 va = *reinterpret_cast<const f32x4*>(vnf + 4 * lb);
      const f32x4 vb = *reinterpret_cast<const f32x4*>(vnf + 16 + 4 * lb);
      float vn[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vn[i] = va[i];
        vn[4 + i] = vb[i];
      }
#pragma unroll
      for (int k = 0; k < NRB; ++k) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = pr[k][e] * vn[e];
        split_hi_lo(pv, phi[k], plo[k]);
      }
    }
    // value fragments: lane (dim 16 nb + lr, k-group lb) takes field lr of the
    // index words of cells 4lb .. 4lb+3 and 16+4lb .. 16+4lb+3: its staged
    // addresses are at parity lr & 1, group lr >> 1 -> half (lr >> 1) & 1,
    // byte lr >> 2
    const uint32_t* vsrc = vtw + (lr & 1) * 16 + ((lr >> 1) & 1) * 8 + 2 * lb;
    const uint32_t boff = 8 * (lr >> 2);
    if constexpr (PK) {
      // values as [hi lo hi lo] of cell pairs (4lb, 4lb+1), (4lb+2, 4lb+3)
      // and of the same pairs 16 cells on; the weights against them: rows
      // 0-7 (hi parts of rows 0-7) [hi hi hi hi] of the pairs, giving
      // p_hi (v_hi + v_lo), rows 8-15 (their lo parts) [lo 0 lo 0], giving
      // p_lo v_hi
      const u32x4 ph = __builtin_bit_cast(u32x4, phi[0]), pl = __builtin_bit_cast(u32x4, plo[0]);
      const bool hir = lr < 8;
      const half8 pa = __builtin_bit_cast(half8, hir ? u32x4{ph[0], ph[0], ph[1], ph[1]} : u32x4{pl[0], 0u, pl[1], 0u});
      const half8 pb = __builtin_bit_cast(half8, hir ? u32x4{ph[2], ph[2], ph[3], ph[3]} : u32x4{pl[2], 0u, pl[3], 0u});
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x2 x0 = *reinterpret_cast<const u32x2*>(vsrc + nb * L::VS);        // pairs 2lb, 2lb+1
        const u32x2 x1 = *reinterpret_cast<const u32x2*>(vsrc + nb * L::VS + 32);   // pairs 8+2lb, 9+2lb
        const uint32_t xs[4] = {x0[0], x0[1], x1[0], x1[1]};
        u32x2 e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          e[j] = *reinterpret_cast<const u32x2*>(tab + kTqCtabHL + __builtin_amdgcn_ubfe(xs[j], boff, 8));
        const half8 va = __builtin_bit_cast(half8, u32x4{e[0][0], e[0][1], e[1][0], e[1][1]});
        const half8 vb = __builtin_bit_cast(half8, u32x4{e[2][0], e[2][1], e[3][0], e[3][1]});
        O[0][nb] = mfma16(pa, va, O[0][nb]);
        O[0][nb] = mfma16(pb, vb, O[0][nb]);
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x2 x0 = *reinterpret_cast<const u32x2*>(vsrc + nb * L::VS);        // pairs 2lb, 2lb+1
        const u32x2 x1 = *reinterpret_cast<const u32x2*>(vsrc + nb * L::VS + 32);   // pairs 8+2lb, 9+2lb
        const uint32_t xs[4] = {x0[0], x0[1], x1[0], x1[1]};
        u32x4 h, l;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t a4 = __builtin_amdgcn_ubfe(xs[j], boff, 8);
          h[j] = lds_u32(tab + kTqCtabHi, a4);
          l[j] = lds_u32(tab + kTqCtabLo, a4);
        }
        const half8 vh = __builtin_bit_cast(half8, h);
        const half8 vl = __builtin_bit_cast(half8, l);
#pragma unroll
        for (int k = 0; k < NRB; ++k) {
          O[k][nb] = mfma16(phi[k], vh, O[k][nb]);
          O[k][nb] = mfma16(plo[k], vh, O[k][nb]);
          O[k][nb] = mfma16(phi[k], vl, O[k][nb]);
        }
      }
    }
  };

  // ---- main loop: the first tile is requested before the query operands are
  // staged; then K and V of tile t+1 are in flight while tile t computes ----
  {
    KRegs RK;
    VRegs RV;
    int ts = c0 + TC * wave;
    issue_v(ts, RV);
    issue_k(ts, RK);
    __syncthreads();                             // row maxima, q_jl sums and tables staged
#pragma unroll
    for (int k = 0; k < NRB; ++k)
      qs[k] = qsum[16 * k + crow(lr)] * q_row_factor(row_max(16 * k + crow(lr)), 0.5f, 1, &rs[k]);
    q_stage();
    __syncthreads();                             // query operands staged
#pragma unroll 1
    while (ts < cend) {
      const int tn = ts + NW * TC;
      stage(RV);
      issue_v(tn, RV);
      f32x4 S[2][NRB];
      qk(RK, S);
      issue_k(tn, RK);
      softmax_pv(ts, S);
      ts = tn;
    }
  }

  // The accumulators hold o * 2^(21 - vexp): written as the equivalent
  // partial (o * 2^x, m - x, l * 2^x).
#pragma unroll
  for (int k = 0; k < NRB; ++k) {
    m_run[k] -= (float)(21 - vexp);
    l_run[k] = __builtin_amdgcn_ldexpf(l_run[k], 21 - vexp);
  }
  if constexpr (PK) {
    // packed: accumulator rows 0-7 hold the hi-weight sums of rows 0-7 (lane
    // groups 0, 1), rows 8-15 the lo-weight sums of the same rows (groups 2,
    // 3); their sum is the row's o, left in both halves so that rows 8-15
    // stay copies of rows 0-7 with the same (m, l)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float u, v;
        swap32(O[0][nb][i], u, v);
        O[0][nb][i] = u + v;
      }
  }

  // ---- combine the four waves into one partial per query row (as the
  // dense kernel) ----
  __syncthreads();
  if (lb == 0) {
#pragma unroll
    for (int k = 0; k < NRB; ++k) {
      mls[(wave * RB + 16 * k + lr) * 2] = m_run[k];
      mls[(wave * RB + 16 * k + lr) * 2 + 1] = l_run[k];
    }
  }
  __syncthreads();
  float* buf = reinterpret_cast<float*>(work);
  constexpr int HALF = NW / 2;
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
      for (int nb = 0; nb < NB; ++nb) O[k][nb][i] *= f;
    }
  }
  constexpr int RS = L::RS;
  if (wave >= HALF) {
    float* b = buf + (wave - HALF) * RB * RS;
#pragma unroll
    for (int k = 0; k < NRB; ++k)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) b[(16 * k + 4 * lb + i) * RS + 16 * nb + lr] = O[k][nb][i];
  }
  __syncthreads();
  if (wave < HALF) {
    float* b = buf + wave * RB * RS;
#pragma unroll
    for (int k = 0; k < NRB; ++k)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
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

}  // namespace gqa_kern
