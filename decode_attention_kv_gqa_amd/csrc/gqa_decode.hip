// Split-KV flash-decoding of grouped-query attention for gfx950 (MI355X).
//
// Kernels:
//   attn_mfma   (attn_mfma.h) one workgroup per (split, KV head [x row block]
//               [x token], seq): streams the K/V rows of its cell range once
//               for every query row of the GQA group (all G heads, and all T
//               tokens of a dense causal window), runs an online softmax per
//               row and writes one partial (o unnormalised, m, l) per row.
//   merge_rows  one workgroup per output row: log-sum-exp merge of the
//               partials of that row's splits.
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
// in base-2 units; only the merge below reads it.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn_mfma.h"
#include "common.h"
#include "gqa_decode.h"
#include "plan.h"

namespace {

using gqa_kern::AttnArgs;
using gqa_kern::MergeArgs;
using gqa_kern::wave_max;
using gqa_kern::wave_sum;

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

// One workgroup per output row (s, t, h).
template <int D>
__global__ __launch_bounds__(kThreads) void merge_rows(MergeArgs a) {
  __shared__ float wgt[kThreads];
  __shared__ float red[kThreads / 64];
  __shared__ float bcast;
  const int tid = threadIdx.x;
  const int row = blockIdx.x;             // ((s * T) + t) * H + h
  const int h = row % a.H;
  const int t = (row / a.H) % a.T;
  const int s = row / (a.H * a.T);
  (void)h;
  int L = a.seq_lens[s] - (a.T - 1 - t);
  L = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
  if (a.ids) L = L < a.B ? L : a.B;
  int nv = (L + a.chunk - 1) / a.chunk;
  nv = nv < a.P ? nv : a.P;
  float* out = a.out + (size_t)row * D;
  if (nv == 0) {
    for (int d = tid; d < D; d += kThreads) out[d] = 0.f;
    return;
  }
  const float* ml = a.part_ml + (size_t)row * a.P * 2;
  const float* po = a.part_o + (size_t)row * a.P * D;

  // M = max_j m_j
  float m = -INFINITY;
  for (int j = tid; j < nv; j += kThreads) m = fmaxf(m, ml[2 * j]);
  m = wave_max(m);
  if (tid % 64 == 0) red[tid / 64] = m;
  __syncthreads();
  if (tid == 0) {
    float M = red[0];
    for (int w = 1; w < kThreads / 64; ++w) M = fmaxf(M, red[w]);
    bcast = M;
  }
  __syncthreads();
  const float M = bcast;
  if (M == -INFINITY) {
    for (int d = tid; d < D; d += kThreads) out[d] = 0.f;
    return;
  }
  // L = sum_j exp2(m_j - M) * l_j ; out = sum_j exp2(m_j - M) * o_j / L
  float lsum = 0.f;
  float acc = 0.f;
  for (int jb = 0; jb < nv; jb += kThreads) {
    const int j = jb + tid;
    float e = 0.f;
    if (j < nv) {
      const float mj = ml[2 * j];
      e = (mj == -INFINITY) ? 0.f : exp2f(mj - M);
      lsum = fmaf(e, ml[2 * j + 1], lsum);
    }
    wgt[tid] = e;
    __syncthreads();
    const int jn = (nv - jb < kThreads) ? nv - jb : kThreads;
    if (tid < D) {
      for (int jj = 0; jj < jn; ++jj) acc = fmaf(wgt[jj], po[(size_t)(jb + jj) * D + tid], acc);
    }
    __syncthreads();
  }
  lsum = wave_sum(lsum);
  if (tid % 64 == 0) red[tid / 64] = lsum;
  __syncthreads();
  if (tid == 0) {
    float Ls = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) Ls += red[w];
    bcast = Ls;
  }
  __syncthreads();
  if (tid < D) out[tid] = acc / bcast;
}


template <int D, bool I8, bool IDS, int NRB>
hipError_t launch_one(const AttnArgs& a, dim3 grid, hipStream_t st) {
  constexpr int bytes = gqa_kern::AttnLds<D, I8, NRB>::BYTES +
                        (IDS ? gqa_kern::AttnLds<D, I8, NRB>::IDSB : 0);
  auto* fn = &gqa_kern::attn_mfma<D, I8, IDS, NRB>;
  if (bytes > 65536) {
    static bool attr_set = false;   // per instance; set before the first launch
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
  }
  hipLaunchKernelGGL(fn, grid, dim3(kThreads), bytes, st, a);
  return hipGetLastError();
}

template <int D, bool I8>
hipError_t launch_attn(const AttnArgs& a, bool ids, int nrows, dim3 grid, hipStream_t st) {
  if (nrows <= 16)
    return ids ? launch_one<D, I8, true, 1>(a, grid, st) : launch_one<D, I8, false, 1>(a, grid, st);
  return ids ? launch_one<D, I8, true, 2>(a, grid, st) : launch_one<D, I8, false, 2>(a, grid, st);
}

template <bool I8>
hipError_t launch_attn_d(const AttnArgs& a, int D, bool ids, int nrows, dim3 grid, hipStream_t st) {
  switch (D) {
    case 64: return launch_attn<64, I8>(a, ids, nrows, grid, st);
    case 128: return launch_attn<128, I8>(a, ids, nrows, grid, st);
    default: return launch_attn<256, I8>(a, ids, nrows, grid, st);
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
  if (chunk <= 0) chunk = gqa::auto_chunk(sh);
  if (chunk <= 0 || chunk > gqa::max_chunk(sh)) return GQA_ERR_CHUNK;
  if (ids && (int64_t)Lmax * Hk * D * (i8 ? 1 : 2) >= ((int64_t)1 << 31)) return GQA_ERR_SHAPE;
  const size_t need = gqa::part_bytes(sh, chunk);
  if (part_bytes < need) return GQA_ERR_WORKSPACE;
  const int64_t P = gqa::num_splits(sh, chunk);
  if (P == 0) return GQA_OK;                 // Lmax == 0: every row is empty
  if (P > 0x7fffffff) return GQA_ERR_SHAPE;

  AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.ksc = ksc; a.vsc = vsc; a.ids = ids; a.seq_lens = seq_lens;
  a.part_o = part;
  a.part_ml = part + gqa::part_o_floats(sh, P);
  a.S = S; a.T = T; a.Lmax = Lmax; a.B = sh.B; a.H = H; a.Hk = Hk; a.G = H / Hk;
  a.R = gqa::rows_per_unit(sh); a.nrb = gqa::row_blocks(sh); a.P = (int)P; a.chunk = chunk;
  a.qscale = scale * kLog2e;
  const int nrows = gqa::block_rows(sh);
  dim3 grid((unsigned)P, (unsigned)(Hk * a.nrb * (ids ? T : 1)), (unsigned)S);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = i8 ? launch_attn_d<true>(a, D, ids != nullptr, nrows, grid, st)
                    : launch_attn_d<false>(a, D, ids != nullptr, nrows, grid, st);
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

int gqa_decode_merge(const float* part, const int32_t* seq_lens, const int32_t* ids_or_null,
                     float* out, int S, int T, int Lmax, int B, int H, int D, int chunk,
                     void* stream) {
  if (!part || !seq_lens || !out) return GQA_ERR_NULL;
  const bool ids = ids_or_null != nullptr;
  gqa::Shape sh{S, T, Lmax, ids ? B : 0, H, H, D, ids, false};
  int rc = gqa::check_shape(sh);
  if (rc != GQA_OK) return rc;
  if (chunk < 1) return GQA_ERR_CHUNK;
  const int64_t P = gqa::num_splits(sh, chunk);
  MergeArgs a;
  a.part_o = part;
  a.part_ml = part + gqa::part_o_floats(sh, P);
  a.seq_lens = seq_lens; a.out = out;
  a.S = S; a.T = T; a.Lmax = Lmax; a.B = sh.B; a.H = H; a.P = (int)P; a.chunk = chunk; a.ids = ids;
  const size_t rows = (size_t)S * T * H;
  if (rows > 0x7fffffffu) return GQA_ERR_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  dim3 grid((unsigned)rows);
  switch (D) {
    case 64: hipLaunchKernelGGL(merge_rows<64>, grid, dim3(kThreads), 0, st, a); break;
    case 128: hipLaunchKernelGGL(merge_rows<128>, grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL(merge_rows<256>, grid, dim3(kThreads), 0, st, a); break;
  }
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? GQA_OK : (int)e;
}

}  // extern "C"
