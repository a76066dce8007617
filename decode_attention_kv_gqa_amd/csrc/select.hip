// Budget selection for the gathered (budgeted) decode attention on gfx950:
// for every query token, the ids of the B cells it attends.
//
// What is selected (qsa2.metal, kernel qsa_topk2): cells come in blocks of
// four, each block with one score.  With n visible cells, block b < n/4 holds
// 4 cells and block n/4 holds the n%4 remaining ones.  The chosen cells are
// the first B when ranked by (block score descending, cell index ascending),
// written in ascending order; with n <= B the ids are 0 .. n-1.
//
// How (one workgroup of 1024 threads per token):
//   1. Three radix passes (12, 10 and 10 bits) over the blocks' order-
//      preserving 32-bit keys find the key Tk of the block where the running
//      cell count, from the highest key down, reaches B, and how many cells
//      `need` must still come from blocks whose key equals Tk.  Each pass
//      counts cells per digit with LDS atomics into a histogram region of
//      its own (zeroed once, so no pass clears for the next), over the
//      blocks that match the digits found so far; after one barrier every
//      wave finds the digit itself (lane sums of 64 or 16 counters, a wave
//      prefix sum to find the lane, a second one over that lane's counters).
//      Up to 16 keys per thread stay in registers across the passes.
//   2. Emission: every thread owns a contiguous block range and marks, one
//      bit per block, the blocks above and at Tk; popcounts of the two masks
//      and one block-wide prefix sum give each thread its share of the Tk
//      blocks (in block order) and its output offset, so the ids come out
//      ascending.  The keys come from LDS, and the ids are gathered in LDS
//      and written to memory in one coalesced pass.
// The page's kernel makes the same two phases on Apple simdgroups; here the
// scans are wave64 DPP moves and the histogram lives in LDS.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "gqa_decode.h"

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kKeysInRegs = 16;         // blocks per thread kept in registers (radix passes)
constexpr int kKeysInLds = 28672;       // block keys staged in LDS (112 KB) for the emission
constexpr int kSelOutLds = 4096;        // budgets up to this are written through LDS
constexpr int kMaxPer = (kKeysInLds + kSelThreads - 1) / kSelThreads;  // blocks per thread, emission
constexpr int kKeyPad = 32;             // LDS keys past the last block (read, never used)
static_assert(kMaxPer <= 32 && kMaxPer <= kKeyPad, "emission block mask / key padding");

// Order-preserving map of a float's bits to an unsigned key (floats compare
// like their keys; -0 sorts below +0).
__device__ __forceinline__ uint32_t okey(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave, with DPP moves (no LDS
// round trips): shifts by 1, 2, 4 and 8 lanes inside each row of 16, then
// row 0's total into row 1 and row 2's into row 3 (row_bcast:15), then the
// total of rows 0-1 into rows 2-3 (row_bcast:31).  Lanes whose source is
// outside the row, and rows the row mask leaves out, add 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

struct SelArgs {
  const float* scores;   // [S][T][nbs]
  const int32_t* seq_lens;
  int32_t* ids;          // [S][T][B]
  int S, T, Lmax, B, nbs;
};

// Exclusive prefix sums of two values per thread over the workgroup, in
// thread order; wsum is a 2 * kSelWaves-entry LDS scratch array.  Every
// wave reads all the wave totals at once and scans them itself.
__device__ __forceinline__ void block_excl_scan2(uint32_t x, uint32_t y, uint32_t* wsum, int tid,
                                                 uint32_t& xe, uint32_t& ye) {
  const int lane = tid & 63, wave = tid >> 6;
  const uint32_t xi = wave_incl_scan(x), yi = wave_incl_scan(y);
  if (lane == 63) {
    wsum[wave] = xi;
    wsum[kSelWaves + wave] = yi;
  }
  __syncthreads();
  const uint32_t xt = wave_incl_scan(lane < kSelWaves ? wsum[lane] : 0u);
  const uint32_t yt = wave_incl_scan(lane < kSelWaves ? wsum[kSelWaves + lane] : 0u);
  const uint32_t xb = wave > 0 ? (uint32_t)__shfl((int)xt, wave - 1, 64) : 0u;
  const uint32_t yb = wave > 0 ? (uint32_t)__shfl((int)yt, wave - 1, 64) : 0u;
  xe = xb + xi - x;
  ye = yb + yi - y;
}

// Radix digits, most significant first: 12, 10 and 10 bits of the key.
// Each pass counts into its own region of one LDS histogram (zeroed once),
// so no pass waits for another's counts to be cleared.
constexpr int kPasses = 3;
constexpr int kDigitShift[kPasses] = {20, 10, 0};
constexpr int kDigitBins[kPasses] = {4096, 1024, 1024};
constexpr int kHistBase[kPasses] = {0, 4096, 5120};
constexpr int kHistBins = 6144;

// The digit of the threshold within one pass's histogram h of `bins`
// counters, ranked from the top: the digit whose counter takes the running
// count, from the highest digit down, to `need` cells, and how many cells
// `need` still asks of blocks with that digit.  Every wave computes it
// itself: lane l sums the bins/64 counters of digits from the top (l * w ..
// l * w + w - 1 places down), a wave prefix sum finds the lane where the
// count reaches `need`, and the wave's lanes then read that lane's w
// counters one each and prefix-sum them to find the digit.
template <int BINS>
__device__ __forceinline__ void find_digit(const uint32_t* h, uint32_t need, int lane,
                                           uint32_t& digit, uint32_t& left) {
  constexpr int W = BINS / 64;
  // lane l's counters are h[BINS - (l+1) W .. BINS - l W), read four at a
  // time (16-byte reads); lane l starts its walk l (or l / 2) chunks in, so
  // that any eight consecutive lanes of one read cover all 32 banks (without
  // the skew every lane would read the same bank)
  const uint32_t* mine = h + BINS - (lane + 1) * W;
  constexpr int NC = W / 4;
  const int sk = NC >= 8 ? lane : (lane >> 1);
  uint32_t lsum = 0;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const u4 v = *reinterpret_cast<const u4*>(mine + 4 * ((j + sk) & (NC - 1)));
    lsum += v[0] + v[1] + v[2] + v[3];
  }
  const uint32_t above = wave_incl_scan(lsum) - lsum;   // cells in higher digits
  const uint64_t hit = __ballot(above < need && above + lsum >= need);
  const int L = hit ? __builtin_ctzll(hit) : 0;
  const uint32_t aboveL = (uint32_t)__shfl((int)above, L, 64);
  // lane j < W takes the counter j places below the top of lane L's range
  const uint32_t c = lane < W ? h[BINS - 1 - L * W - lane] : 0u;
  const uint32_t ci = wave_incl_scan(c), ce = ci - c;
  const uint64_t hit2 = __ballot(lane < W && aboveL + ce < need && aboveL + ci >= need);
  const int J = hit2 ? __builtin_ctzll(hit2) : 0;
  digit = hit ? (uint32_t)(BINS - 1 - L * W - J) : 0u;
  left = hit ? need - aboveL - (uint32_t)__shfl((int)ce, J, 64) : need;
}

__global__ __launch_bounds__(kSelThreads) void select_ids(SelArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kHistBins];
  __shared__ uint32_t wsum[2 * kSelWaves];
  __shared__ int32_t obuf[kSelOutLds];   // the token's ids before the coalesced write
  extern __shared__ uint32_t keyl[];     // block keys (first kKeysInLds blocks)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tok = blockIdx.x;            // s * T + t
  const int s = tok / a.T, t = tok % a.T;
  const int len = a.seq_lens[s];
  const float* sc = a.scores + (size_t)tok * a.nbs;

  // Keys: 16 blocks per thread (b = tid + 1024 i) in registers for the radix
  // passes, and the first kKeysInLds blocks also in LDS for the emission;
  // blocks past both are re-read from memory.  The 16 loads are unconditional
  // (indices clamped to the row), so all are in flight at once; they cover
  // the whole score row and do not wait for the sequence length, so the two
  // memory round trips overlap; keys past the window are never counted.
  uint32_t kr[kKeysInRegs];
  float kv[kKeysInRegs];
#pragma unroll
  for (int i = 0; i < kKeysInRegs; ++i) {   // unconditional (clamped) loads, all in flight
    const int b = tid + kSelThreads * i;
    kv[i] = sc[b < a.nbs ? b : a.nbs - 1];
  }
#pragma unroll
  for (int i = 0; i < kKeysInRegs; ++i) {
    const int b = tid + kSelThreads * i;
    kr[i] = b < a.nbs ? okey(kv[i]) : 0u;
    if (b < a.nbs && b < kKeysInLds) keyl[b] = kr[i];
  }
  for (int b = tid + kSelThreads * kKeysInRegs; b < a.nbs && b < kKeysInLds; b += kSelThreads)
    keyl[b] = okey(sc[b]);

  int n = len - (a.T - 1 - t);
  n = n < 0 ? 0 : (n > a.Lmax ? a.Lmax : n);
  int32_t* out = a.ids + (size_t)tok * a.B;
  if (n <= a.B) {                        // the whole window fits the budget
    for (int c = tid; c < n; c += kSelThreads) out[c] = c;
    return;
  }
  const int n_bid = n >> 2, rem = n & 3, nb = n_bid + 1;
  auto cells_of = [&](int b) -> uint32_t { return b < n_bid ? 4u : (uint32_t)rem; };
  auto key = [&](int b) -> uint32_t { return b < kKeysInLds ? keyl[b] : okey(sc[b]); };
  for (int i = tid; i < kHistBins; i += kSelThreads) hist[i] = 0;
  __syncthreads();

  // ---- 1. radix select of the threshold key: one barrier per pass ----
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)a.B;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int shift = kDigitShift[pass];
    const uint32_t dmask = (uint32_t)kDigitBins[pass] - 1u;
    uint32_t* h = hist + kHistBase[pass];
#pragma unroll
    for (int i = 0; i < kKeysInRegs; ++i) {
      const int b = tid + kSelThreads * i;
      if (b < nb && (kr[i] & pmask) == prefix && cells_of(b))
        atomicAdd(&h[(kr[i] >> shift) & dmask], cells_of(b));
    }
    for (int b = tid + kSelThreads * kKeysInRegs; b < nb; b += kSelThreads) {
      const uint32_t k = key(b);
      if ((k & pmask) == prefix && cells_of(b)) atomicAdd(&h[(k >> shift) & dmask], cells_of(b));
    }
    __syncthreads();
    uint32_t digit, left;
    if (pass == 0)
      find_digit<4096>(h, need, lane, digit, left);
    else
      find_digit<1024>(h, need, lane, digit, left);
    need = left;
    prefix |= digit << shift;
    pmask |= dmask << shift;
  }
  const uint32_t Tk = prefix;

  // ---- 2. emission from contiguous block ranges into LDS, then one
  // coalesced write of the row ----
  const int per = (nb + kSelThreads - 1) / kSelThreads;
  const int b0 = tid * per < nb ? tid * per : nb;
  const int b1 = b0 + per < nb ? b0 + per : nb;
  const bool staged = a.B <= kSelOutLds;
  auto put = [&](uint32_t pos, int id) {
    if (pos < (uint32_t)a.B) {           // never past the row
      if (staged) obuf[pos] = id;
      else out[pos] = id;
    }
  };
  if (staged && nb <= kKeysInLds) {
    // every key is in LDS, a thread's range has at most kMaxPer blocks, and
    // the ids go to LDS.  The counting loop runs `per` times for every thread
    // (a range's reads may run up to per - 1 keys past the last block, into
    // the kKeyPad padding; the `valid` mask drops them) and only sets bits;
    // the counts are popcounts, and the writing loop visits only the blocks
    // with a key >= Tk -- a few per thread when B is a small part of the
    // window.
    // bit i of cand / eqm: block b0 + i has a key >= Tk / == Tk; per is
    // uniform, so the loop is a scalar loop with no divergence
    uint32_t cand = 0, eqm = 0;
#pragma unroll 4
    for (int i = 0; i < per; ++i) {
      const uint32_t k = keyl[b0 + i];
      cand |= (k >= Tk ? 1u : 0u) << i;
      eqm |= (k == Tk ? 1u : 0u) << i;
    }
    const int cnt = b1 - b0;
    const uint32_t valid = cnt >= 32 ? ~0u : ((1u << cnt) - 1u);
    cand &= valid;
    eqm &= valid;
    uint32_t gt = 4u * (uint32_t)__builtin_popcount(cand & ~eqm);
    uint32_t eq = 4u * (uint32_t)__builtin_popcount(eqm);
    if (n_bid >= b0 && n_bid < b1) {     // this range holds the partial block n_bid (rem cells)
      const uint32_t bit = 1u << (n_bid - b0);
      const uint32_t d = 4u - (uint32_t)rem;
      if (cand & ~eqm & bit) gt -= d;
      if (eqm & bit) eq -= d;
      if (rem == 0) { cand &= ~bit; eqm &= ~bit; }   // no cells: never emitted
    }
    uint32_t gt_before, eq_before;
    block_excl_scan2(gt, eq, wsum, tid, gt_before, eq_before);
    // the Tk blocks are taken in block order until `need` cells are taken,
    // so the threads before this one took min(eq_before, need) of them
    uint32_t left = eq_before >= need ? 0u : (eq < need - eq_before ? eq : need - eq_before);
    uint32_t off = gt_before + (eq_before < need ? eq_before : need);
    while (cand) {
      const int i = __builtin_ctz(cand);
      cand &= cand - 1;
      const int b = b0 + i;
      const uint32_t k = keyl[b];
      const uint32_t cells = cells_of(b);
      uint32_t take = cells;
      if (k == Tk) {
        take = cells < left ? cells : left;
        left -= take;
      }
      // off + take never passes B; the clamp only keeps a stray write in LDS
#pragma unroll
      for (uint32_t c = 0; c < 4; ++c) {
        const uint32_t pos = off + c < (uint32_t)(kSelOutLds - 1) ? off + c : (uint32_t)(kSelOutLds - 1);
        if (c < take) obuf[pos] = 4 * b + (int)c;
      }
      off += take;
    }
  } else {
    uint32_t gt = 0, eq = 0;
    for (int b = b0; b < b1; ++b) {
      const uint32_t k = key(b);
      if (k > Tk) gt += cells_of(b);
      else if (k == Tk) eq += cells_of(b);
    }
    uint32_t gt_before, eq_before;
    block_excl_scan2(gt, eq, wsum, tid, gt_before, eq_before);
    uint32_t left = eq_before >= need ? 0u : (eq < need - eq_before ? eq : need - eq_before);
    uint32_t off = gt_before + (eq_before < need ? eq_before : need);
    for (int b = b0; b < b1; ++b) {
      const uint32_t k = key(b);
      const uint32_t cells = cells_of(b);
      uint32_t take = 0;
      if (k > Tk) {
        take = cells;
      } else if (k == Tk) {
        take = cells < left ? cells : left;
        left -= take;
      }
      for (uint32_t c = 0; c < take; ++c) put(off + c, 4 * b + (int)c);
      off += take;
    }
  }
  if (staged) {
    __syncthreads();
    for (int i = tid; i < a.B; i += kSelThreads) out[i] = obuf[i];
  }
}

}  // namespace

extern "C" int gqa_decode_select_ids(const float* block_scores, const int32_t* seq_lens,
                                     int32_t* ids, int S, int T, int Lmax, int B, void* stream) {
  if (!block_scores || !seq_lens || !ids) return GQA_ERR_NULL;
  if (S < 1 || T < 1 || Lmax < 0) return GQA_ERR_SHAPE;
  if (B < 1) return GQA_ERR_BUDGET;
  if ((int64_t)S * T > 0x7fffffff) return GQA_ERR_SHAPE;
  SelArgs a{block_scores, seq_lens, ids, S, T, Lmax, B, Lmax / 4 + 1};
  const int nl = a.nbs < kKeysInLds ? a.nbs : kKeysInLds;
  const int bytes = (nl + kKeyPad) * 4;
  if (bytes > 65536) {
    // more than 64 KB of dynamic LDS must be allowed once per device
    static std::atomic<uint64_t> attr_set{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (!(attr_set.load(std::memory_order_acquire) & bit)) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_ids),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (kKeysInLds + kKeyPad) * 4);
      if (e != hipSuccess) return (int)e;
      attr_set.fetch_or(bit, std::memory_order_acq_rel);
    }
  }
  hipLaunchKernelGGL(select_ids, dim3((unsigned)(S * T)), dim3(kSelThreads), bytes,
                     reinterpret_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? GQA_OK : (int)e;
}
