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
//   1. Four 8-bit radix passes over the blocks' order-preserving 32-bit keys
//      find the key Tk of the block where the running cell count, from the
//      highest key down, reaches B, and how many cells `need` must still come
//      from blocks whose key equals Tk.  Each pass builds a 256-bin histogram
//      of cell counts in LDS (ds_add, one histogram per wave, then summed)
//      over the blocks that match the digits found so far; every wave scans
//      the bins from the top with a wave-wide prefix sum and finds the digit
//      itself, so a pass needs two barriers.  Up to 16 keys per thread stay
//      in registers across the passes.
//   2. Emission: every thread owns a contiguous block range; block-wide
//      prefix sums give each thread its share of the Tk blocks (in block
//      order) and its output offset, so the ids come out ascending.  The
//      keys come from LDS, and the ids are gathered in LDS and written to
//      memory in one coalesced pass.
// The page's kernel makes the same two phases on Apple simdgroups; here the
// scans are wave64 shuffles and the histogram lives in LDS.
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

// Order-preserving map of a float's bits to an unsigned key (floats compare
// like their keys; -0 sorts below +0).
__device__ __forceinline__ uint32_t okey(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

struct SelArgs {
  const float* scores;   // [S][T][nbs]
  const int32_t* seq_lens;
  int32_t* ids;          // [S][T][B]
  int S, T, Lmax, B, nbs;
};

// Exclusive prefix sum of one value per thread over the workgroup, in
// thread order; wsum is a kSelWaves-entry LDS scratch array.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* wsum, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const uint32_t inc = wave_incl_scan(x, lane);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  __syncthreads();                      // wsum is reused by the next scan
  return before + inc - x;
}

__global__ __launch_bounds__(kSelThreads) void select_ids(SelArgs a) {
  // one 256-bin histogram per wave (summed per pass): the top key bytes of
  // real scores take few values, and one shared histogram would serialise
  // every wave's adds on the same bins
  __shared__ uint32_t hist[kSelWaves][256];
  __shared__ uint32_t tot[256];
  __shared__ uint32_t wsum[kSelWaves];
  __shared__ int32_t obuf[kSelOutLds];   // the token's ids before the coalesced write
  extern __shared__ uint32_t keyl[];     // block keys (first kKeysInLds blocks)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int tok = blockIdx.x;            // s * T + t
  const int s = tok / a.T, t = tok % a.T;
  int n = a.seq_lens[s] - (a.T - 1 - t);
  n = n < 0 ? 0 : (n > a.Lmax ? a.Lmax : n);
  int32_t* out = a.ids + (size_t)tok * a.B;
  if (n <= a.B) {                        // the whole window fits the budget
    for (int c = tid; c < n; c += kSelThreads) out[c] = c;
    return;
  }
  const int n_bid = n >> 2, rem = n & 3, nb = n_bid + 1;
  const float* sc = a.scores + (size_t)tok * a.nbs;
  auto cells_of = [&](int b) -> uint32_t { return b < n_bid ? 4u : (uint32_t)rem; };

  // Keys: 16 blocks per thread (b = tid + 1024 i) in registers for the radix
  // passes, and the first kKeysInLds blocks also in LDS for the emission;
  // blocks past both are re-read from memory.
  uint32_t kr[kKeysInRegs];
#pragma unroll
  for (int i = 0; i < kKeysInRegs; ++i) {
    const int b = tid + kSelThreads * i;
    kr[i] = b < nb ? okey(sc[b]) : 0u;
    if (b < nb && b < kKeysInLds) keyl[b] = kr[i];
  }
  for (int b = tid + kSelThreads * kKeysInRegs; b < nb && b < kKeysInLds; b += kSelThreads)
    keyl[b] = okey(sc[b]);
  auto key = [&](int b) -> uint32_t { return b < kKeysInLds ? keyl[b] : okey(sc[b]); };
#pragma unroll
  for (int j = 0; j < 4; ++j) hist[wave][lane + 64 * j] = 0;
  __syncthreads();

  // ---- 1. radix select of the threshold key: two barriers per pass ----
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)a.B;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    uint32_t* h = hist[wave];
#pragma unroll
    for (int i = 0; i < kKeysInRegs; ++i) {
      const int b = tid + kSelThreads * i;
      if (b < nb && (kr[i] & pmask) == prefix && cells_of(b))
        atomicAdd(&h[(kr[i] >> shift) & 255u], cells_of(b));
    }
    for (int b = tid + kSelThreads * kKeysInRegs; b < nb; b += kSelThreads) {
      const uint32_t k = key(b);
      if ((k & pmask) == prefix && cells_of(b)) atomicAdd(&h[(k >> shift) & 255u], cells_of(b));
    }
    __syncthreads();
    if (tid < 256) {                     // sum the wave histograms, clear them for the next pass
      uint32_t x = 0;
#pragma unroll
      for (int w = 0; w < kSelWaves; ++w) {
        x += hist[w][tid];
        hist[w][tid] = 0;
      }
      tot[tid] = x;
    }
    __syncthreads();
    // every wave finds the digit itself: lane l holds digits 255-4l .. 252-4l
    uint32_t c[4], lsum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) { c[j] = tot[255 - 4 * lane - j]; lsum += c[j]; }
    uint32_t above = wave_incl_scan(lsum, lane) - lsum;   // cells in higher digits
    uint32_t dsel = 0, nsel = 0;
    bool found = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (above < need && above + c[j] >= need) {
        found = true;
        dsel = 255u - 4u * lane - j;
        nsel = need - above;
      }
      above += c[j];
    }
    const uint64_t who = __ballot(found);
    const int src = who ? __builtin_ctzll(who) : 0;
    const uint32_t digit = who ? (uint32_t)__shfl((int)dsel, src, 64) : 0u;
    need = who ? (uint32_t)__shfl((int)nsel, src, 64) : need;
    prefix |= digit << shift;
    pmask |= 255u << shift;
  }
  const uint32_t Tk = prefix;

  // ---- 2. emission from contiguous block ranges into LDS, then one
  // coalesced write of the row ----
  const int per = (nb + kSelThreads - 1) / kSelThreads;
  const int b0 = tid * per < nb ? tid * per : nb;
  const int b1 = b0 + per < nb ? b0 + per : nb;
  uint32_t gt = 0, eq = 0;
  for (int b = b0; b < b1; ++b) {
    const uint32_t k = key(b);
    if (k > Tk) gt += cells_of(b);
    else if (k == Tk) eq += cells_of(b);
  }
  const uint32_t eq_before = block_excl_scan(eq, wsum, tid);
  const uint32_t eq_take = eq_before >= need ? 0u : (eq < need - eq_before ? eq : need - eq_before);
  uint32_t off = block_excl_scan(gt + eq_take, wsum, tid);
  const bool staged = a.B <= kSelOutLds;
  uint32_t left = eq_take;
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
    for (uint32_t c = 0; c < take; ++c) {
      if (off + c < (uint32_t)a.B) {     // never past the row
        if (staged) obuf[off + c] = 4 * b + (int)c;
        else out[off + c] = 4 * b + (int)c;
      }
    }
    off += take;
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
  const int bytes = nl * 4;
  if (bytes > 65536) {
    // more than 64 KB of dynamic LDS must be allowed once per device
    static std::atomic<uint64_t> attr_set{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (!(attr_set.load(std::memory_order_acquire) & bit)) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_ids),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kKeysInLds * 4);
      if (e != hipSuccess) return (int)e;
      attr_set.fetch_or(bit, std::memory_order_acq_rel);
    }
  }
  hipLaunchKernelGGL(select_ids, dim3((unsigned)(S * T)), dim3(kSelThreads), bytes,
                     reinterpret_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? GQA_OK : (int)e;
}
