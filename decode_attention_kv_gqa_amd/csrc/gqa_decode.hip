// Split-KV flash-decoding of grouped-query attention for gfx950 (MI355X).
//
// Kernels:
//   attn_chunk  one workgroup per (split, KV head [x row block] [x token], seq):
//               streams the K/V rows of its cell range once for every query
//               row of the GQA group (all G heads, and all T tokens of a
//               dense causal window), runs an online softmax per row and
//               writes one partial (o unnormalised, m, l) per row.
//   merge       one workgroup per output row: log-sum-exp merge of the
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

#include "gqa_decode.h"
#include "plan.h"

namespace {

constexpr int kThreads = 256;   // 4 waves of 64
constexpr int kTile = 64;       // cells per inner tile (one per lane in the softmax)
constexpr float kLog2e = 1.4426950408889634f;

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

struct AttnArgs {
  const float* q;
  const void* k;
  const void* v;
  const uint16_t* ksc;
  const uint16_t* vsc;
  const int32_t* ids;
  const int32_t* seq_lens;
  float* part_o;
  float* part_ml;
  int S, T, Lmax, B, H, Hk, G, R, nrb, P, chunk;
  float qscale;  // scale * log2(e)
};

// Loads 16 bytes of a K row and widens them to fp32 (8 f16 or 16 int8
// elements; int8 elements times their group's f16 scale, exact in fp32).
template <bool I8>
struct Row16;

template <>
struct Row16<false> {
  static constexpr int E = 8;
  __device__ static void load(const void* base, size_t elem_off, int part, const uint16_t*, size_t,
                              float (&x)[E]) {
    const uint4 w = *reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(base) + elem_off + part * 8);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = h2f((uint16_t)(u[i] & 0xffffu));
      x[2 * i + 1] = h2f((uint16_t)(u[i] >> 16));
    }
  }
};

template <>
struct Row16<true> {
  static constexpr int E = 16;
  __device__ static void load(const void* base, size_t elem_off, int part, const uint16_t* sc,
                              size_t sc_off, float (&x)[E]) {
    const uint4 w = *reinterpret_cast<const uint4*>(
        reinterpret_cast<const int8_t*>(base) + elem_off + part * 16);
    const float s = h2f(sc[sc_off + (part * 16) / 64]);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int b = 0; b < 4; ++b) x[4 * i + b] = (float)(int8_t)((u[i] >> (8 * b)) & 0xffu) * s;
    }
  }
};

// Four consecutive V elements of a row, widened to fp32.
template <bool I8>
__device__ __forceinline__ void load_v4(const void* base, size_t elem_off, const uint16_t* sc,
                                        size_t sc_off, int d0, float (&x)[4]) {
  if constexpr (I8) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(
        reinterpret_cast<const int8_t*>(base) + elem_off + d0);
    const float s = h2f(sc[sc_off + d0 / 64]);
#pragma unroll
    for (int b = 0; b < 4; ++b) x[b] = (float)(int8_t)((w >> (8 * b)) & 0xffu) * s;
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(
        reinterpret_cast<const uint16_t*>(base) + elem_off + d0);
    x[0] = h2f((uint16_t)(w.x & 0xffffu));
    x[1] = h2f((uint16_t)(w.x >> 16));
    x[2] = h2f((uint16_t)(w.y & 0xffffu));
    x[3] = h2f((uint16_t)(w.y >> 16));
  }
}

// D: head_dim.  I8: int8 rows.  IDS: gather through cell ids.  RB: query
// rows held by the workgroup (4, 8, 16 or 32; rows past the unit's R are
// zero and never written).
template <int D, bool I8, bool IDS, int RB>
__global__ __launch_bounds__(kThreads) void attn_chunk(AttnArgs a) {
  constexpr int ES = I8 ? 1 : 2;                 // bytes per element
  constexpr int LPC = D * ES / 16;               // lanes per cell row (16 B each)
  constexpr int CPP = kThreads / LPC;            // cells per QK pass
  constexpr int EPT = 16 / ES;                   // elements per lane in QK
  constexpr int TPR = D / 4;                     // PV threads per row group
  constexpr int RG = kThreads / TPR;             // PV row groups
  constexpr int KR = (RB + RG - 1) / RG;         // rows per PV thread
  static_assert(CPP <= kTile && kTile % CPP == 0, "tile must be whole QK passes");
  static_assert(LPC <= 64, "a cell row must fit in one wave");

  __shared__ float qs[RB][D];
  __shared__ float sc[RB][kTile];
  __shared__ int cid[kTile];
  __shared__ float rowm[RB], rowl[RB], rowcorr[RB];
  __shared__ int roww[RB];

  const int tid = threadIdx.x;
  const int p = blockIdx.x;
  int y = blockIdx.y;
  const int g = y % a.Hk;
  y /= a.Hk;
  const int rb = y % a.nrb;
  const int tq = y / a.nrb;    // token (gather mode only)
  const int s = blockIdx.z;
  const int seq_len = a.seq_lens[s];

  // Visible width of a local row (0 for padding rows).
  auto row_width = [&](int i) -> int {
    const int r = rb * RB + i;
    if (r >= a.R) return 0;
    const int t = IDS ? tq : r / a.G;
    int L = seq_len - (a.T - 1 - t);
    L = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
    if (IDS) L = L < a.B ? L : a.B;
    return L;
  };
  auto row_t = [&](int i) -> int { return IDS ? tq : (rb * RB + i) / a.G; };
  auto row_h = [&](int i) -> int {
    const int r = rb * RB + i;
    return g * a.G + (IDS ? r : r % a.G);
  };

  // Widest row of the block: the last real row (widths grow with the token).
  int last = a.R - 1 - rb * RB;
  last = last < RB - 1 ? last : RB - 1;
  const int wmax = row_width(last);
  const int c0 = p * a.chunk;
  if (c0 >= wmax) return;   // no row of this block has cells here; the merge skips it
  const int cend = (c0 + a.chunk < wmax) ? c0 + a.chunk : wmax;

  for (int idx = tid; idx < RB * D; idx += kThreads) {
    const int i = idx / D, d = idx % D;
    float val = 0.f;
    if (rb * RB + i < a.R)
      val = a.q[((size_t)(s * a.T + row_t(i)) * a.H + row_h(i)) * D + d] * a.qscale;
    qs[i][d] = val;
  }
  if (tid < RB) {
    rowm[tid] = -INFINITY;
    rowl[tid] = 0.f;
    roww[tid] = row_width(tid);
  }

  float acc[KR][4];
#pragma unroll
  for (int k = 0; k < KR; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[k][e] = 0.f;

  const size_t seq_row0 = (size_t)s * a.Lmax;  // first cell row of the sequence
  const int32_t* idrow = IDS ? a.ids + ((size_t)s * a.T + tq) * a.B : nullptr;

  for (int cb = c0; cb < cend; cb += kTile) {
    const int n = (cend - cb < kTile) ? cend - cb : kTile;
    if (tid < kTile) {
      int c = 0;
      if (tid < n) {
        c = IDS ? idrow[cb + tid] : cb + tid;
        c = c < 0 ? 0 : (c >= a.Lmax ? a.Lmax - 1 : c);
      }
      cid[tid] = c;
    }
    __syncthreads();

    // ---- scores: LPC lanes per cell, each 16 bytes of the K row ----
    {
      const int part = tid % LPC;
#pragma unroll 1
      for (int pass = 0; pass < kTile / CPP; ++pass) {
        const int j = pass * CPP + tid / LPC;
        const size_t row = (seq_row0 + cid[j]) * a.Hk + g;
        float kx[EPT];
        Row16<I8>::load(a.k, row * D, part, a.ksc, row * (D / 64), kx);
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < EPT; ++e) d = fmaf(qs[i][part * EPT + e], kx[e], d);
#pragma unroll
          for (int o = LPC / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o, 64);
          if (part == 0) sc[i][j] = d;
        }
      }
    }
    __syncthreads();

    // ---- online softmax update: one wave per row, one lane per cell ----
    {
      const int w = tid / 64, lane = tid % 64;
      for (int i = w; i < RB; i += kThreads / 64) {
        const bool vis = lane < n && cb + lane < roww[i];
        const float x = vis ? sc[i][lane] : -INFINITY;
        const float mold = rowm[i];
        const float mnew = fmaxf(mold, wave_max(x));
        const float corr = (mold == -INFINITY) ? 0.f : exp2f(mold - mnew);
        const float pr = vis ? exp2f(x - mnew) : 0.f;
        const float tsum = wave_sum(pr);
        sc[i][lane] = pr;
        if (lane == 0) {
          rowm[i] = mnew;
          rowl[i] = rowl[i] * corr + tsum;
          rowcorr[i] = corr;
        }
      }
    }
    __syncthreads();

    // ---- P.V: thread owns 4 dims of KR rows ----
    {
      const int rg = tid / TPR;
      const int d0 = (tid % TPR) * 4;
#pragma unroll
      for (int k = 0; k < KR; ++k) {
        const int i = rg + k * RG;
        const float cf = (i < RB) ? rowcorr[i] : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[k][e] *= cf;
      }
#pragma unroll 2
      for (int j = 0; j < n; ++j) {
        const size_t row = (seq_row0 + cid[j]) * a.Hk + g;
        float vx[4];
        load_v4<I8>(a.v, row * D, a.vsc, row * (D / 64), d0, vx);
#pragma unroll
        for (int k = 0; k < KR; ++k) {
          const int i = rg + k * RG;
          if (i < RB) {
            const float pr = sc[i][j];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[k][e] = fmaf(pr, vx[e], acc[k][e]);
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- write the partials of the real rows ----
  {
    const int rg = tid / TPR;
    const int d0 = (tid % TPR) * 4;
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      const int i = rg + k * RG;
      if (i < RB && rb * RB + i < a.R) {
        const size_t prow = ((size_t)(s * a.T + row_t(i)) * a.H + row_h(i)) * a.P + p;
        float4 o = make_float4(acc[k][0], acc[k][1], acc[k][2], acc[k][3]);
        *reinterpret_cast<float4*>(a.part_o + prow * D + d0) = o;
      }
    }
    if (tid < RB && rb * RB + tid < a.R) {
      const size_t prow = ((size_t)(s * a.T + row_t(tid)) * a.H + row_h(tid)) * a.P + p;
      a.part_ml[prow * 2] = rowm[tid];
      a.part_ml[prow * 2 + 1] = rowl[tid];
    }
  }
}

struct MergeArgs {
  const float* part_o;
  const float* part_ml;
  const int32_t* seq_lens;
  float* out;
  int S, T, Lmax, B, H, P, chunk;
  bool ids;
};

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

template <int D, bool I8, bool IDS>
hipError_t launch_attn_rb(const AttnArgs& a, int RB, dim3 grid, hipStream_t st) {
  switch (RB) {
    case 4: hipLaunchKernelGGL((attn_chunk<D, I8, IDS, 4>), grid, dim3(kThreads), 0, st, a); break;
    case 8: hipLaunchKernelGGL((attn_chunk<D, I8, IDS, 8>), grid, dim3(kThreads), 0, st, a); break;
    case 16: hipLaunchKernelGGL((attn_chunk<D, I8, IDS, 16>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((attn_chunk<D, I8, IDS, 32>), grid, dim3(kThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

template <bool I8>
hipError_t launch_attn(const AttnArgs& a, int D, bool ids, int RB, dim3 grid, hipStream_t st) {
  switch (D) {
    case 64: return ids ? launch_attn_rb<64, I8, true>(a, RB, grid, st)
                        : launch_attn_rb<64, I8, false>(a, RB, grid, st);
    case 128: return ids ? launch_attn_rb<128, I8, true>(a, RB, grid, st)
                         : launch_attn_rb<128, I8, false>(a, RB, grid, st);
    default: return ids ? launch_attn_rb<256, I8, true>(a, RB, grid, st)
                        : launch_attn_rb<256, I8, false>(a, RB, grid, st);
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
  if (chunk <= 0) return GQA_ERR_CHUNK;
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
  const int RB = gqa::block_rows(sh);
  dim3 grid((unsigned)P, (unsigned)(Hk * a.nrb * (ids ? T : 1)), (unsigned)S);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = i8 ? launch_attn<true>(a, D, ids != nullptr, RB, grid, st)
                    : launch_attn<false>(a, D, ids != nullptr, RB, grid, st);
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
