// Decode attention over a TurboQuant-compressed KV cache (cera 0.4.0,
// flash_attention_tq.metal) on gfx950: the host entry points, and the merge
// whose epilogue rotates the merged rows back to the original basis.
//
// The page runs one threadgroup per (head, query) over the whole window; here
// the window is cut into splits like the other decode paths, and because the
// inverse rotation is linear, the splits' partials stay in the rotated basis,
// the log-sum-exp merge combines them there, and the rotation runs once per
// output row after the merge: out = signs * (H_D @ merged) / sqrt(D), with H_D
// the Walsh-Hadamard matrix applied as the page's butterfly passes.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "attn_tq.h"
#include "gqa_decode.h"
#include "plan.h"

namespace {

using gqa_kern::TqArgs;

constexpr int kMergeThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

struct TqMergeArgs {
  const float* part_o;     // [rows][P][D]  rotated basis
  const float* part_ml;    // [rows][P][2]
  const float* signs;      // [D]
  float* out;              // [rows][D]
  int P;
};

// One workgroup (four waves) per output row: the online merge of the
// row's partials as in the other merge, then the inverse randomized Hadamard
// rotation by wave 0 -- lane l holds dims l*V .. l*V+V-1 (V = D/64), so a
// butterfly at stride s < V stays inside the lane and one at s >= V pairs
// lane l with lane l ^ (s / V).  U splits per wave have their loads in
// flight together (4 waves x U covers up to 16, 32 or 64 splits in one round
// trip).
template <int D, int U>
__global__ __launch_bounds__(kMergeThreads) void merge_rows_tq(TqMergeArgs a) {
  constexpr int V = D / 64;
  __shared__ float red_o[4][D];
  __shared__ float red_ml[4][2];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int row = blockIdx.x;
  const float* ml = a.part_ml + (size_t)row * a.P * 2;
  const float* po = a.part_o + (size_t)row * a.P * D + lane * V;
  float M = -INFINITY, lsum = 0.f;
  float acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.f;
  for (int j0 = wave; j0 < a.P; j0 += 4 * U) {
    float mj[U], lj[U], oj[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + 4 * u;
      mj[u] = -INFINITY;
      lj[u] = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) oj[u][e] = 0.f;
      if (j < a.P) {
        mj[u] = ml[2 * j];
        lj[u] = ml[2 * j + 1];
#pragma unroll
        for (int e = 0; e < V; ++e) oj[u][e] = po[(size_t)j * D + e];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (mj[u] == -INFINITY) continue;        // split without a visible cell: weight 0
      if (mj[u] > M) {
        const float c = (M == -INFINITY) ? 0.f : exp2f(M - mj[u]);
        lsum *= c;
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] *= c;
        M = mj[u];
      }
      const float w = exp2f(mj[u] - M);
      lsum = fmaf(w, lj[u], lsum);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = fmaf(w, oj[u][e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < V; ++e) red_o[wave][lane * V + e] = acc[e];
  if (lane == 0) {
    red_ml[wave][0] = M;
    red_ml[wave][1] = lsum;
  }
  __syncthreads();
  if (wave != 0) return;
  float* out = a.out + (size_t)row * D + lane * V;
  float Mt = red_ml[0][0];
#pragma unroll
  for (int w = 1; w < 4; ++w) Mt = fmaxf(Mt, red_ml[w][0]);
  if (Mt == -INFINITY) {                       // empty window: zeros
#pragma unroll
    for (int e = 0; e < V; ++e) out[e] = 0.f;
    return;
  }
  float f[4], Ls = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = red_ml[w][0];
    f[w] = (mw == -INFINITY) ? 0.f : exp2f(mw - Mt);
    Ls = fmaf(f[w], red_ml[w][1], Ls);
  }
  float x[V];
#pragma unroll
  for (int e = 0; e < V; ++e) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) t = fmaf(f[w], red_o[w][lane * V + e], t);
    x[e] = t / Ls;
  }
  // Walsh-Hadamard butterflies: (a, b) -> (a + b, a - b) at strides 1 .. D/2
#pragma unroll
  for (int st = 1; st < D; st <<= 1) {
    if (st < V) {
#pragma unroll
      for (int e = 0; e < V; ++e)
        if ((e & st) == 0) {
          const float u = x[e], v = x[e + st];
          x[e] = u + v;
          x[e + st] = u - v;
        }
    } else {
      const int lx = st / V;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float y = __shfl_xor(x[e], lx, 64);
        x[e] = (lane & lx) ? y - x[e] : x[e] + y;
      }
    }
  }
  const float inv = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int e = 0; e < V; ++e) out[e] = x[e] * inv * a.signs[lane * V + e];
}

template <int D, int NRB, bool PK = false>
hipError_t launch_tq(const TqArgs& a, dim3 grid, hipStream_t st) {
  using L = gqa_kern::TqLds<D, NRB, PK>;
  static_assert(L::BYTES <= 65536, "TurboQuant LDS budget");
  hipLaunchKernelGGL((gqa_kern::attn_tq<D, NRB, PK>), grid, dim3(256), L::BYTES, st, a);
  return hipGetLastError();
}

template <int U>
void launch_merge_tq(const TqMergeArgs& a, int D, dim3 grid, hipStream_t st) {
  if (D == 64) hipLaunchKernelGGL((merge_rows_tq<64, U>), grid, dim3(kMergeThreads), 0, st, a);
  else hipLaunchKernelGGL((merge_rows_tq<128, U>), grid, dim3(kMergeThreads), 0, st, a);
}

uint16_t f16_bits(_Float16 h) {
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}

}  // namespace

extern "C" {

int gqa_decode_attn_tq(const float* q_rot, const float* q_jl, const uint32_t* k_polar,
                       const uint32_t* k_jl, const uint32_t* k_norms, const uint32_t* v_polar,
                       const uint32_t* v_norms, const int32_t* seq_lens, float* part,
                       size_t part_bytes, int S, int T, int Lmax, int H, int Hk, int D,
                       float c0, float c1, float c2, float c3, float qjl_scale, float scale,
                       int chunk, void* stream) {
  if (!q_rot || !q_jl || !seq_lens || !part) return GQA_ERR_NULL;
  if (Lmax > 0 && (!k_polar || !k_jl || !k_norms || !v_polar || !v_norms)) return GQA_ERR_NULL;
  gqa::Shape sh{S, T, Lmax, 0, H, Hk, D, false, true, true};
  int rc = gqa::check_shape(sh);
  if (rc != GQA_OK) return rc;
  if (D != 64 && D != 128) return GQA_ERR_HEAD_DIM;
  if (chunk <= 0) chunk = gqa::auto_chunk(sh);
  // one split of one KV head spans chunk * D/16 words in the largest region
  if (chunk <= 0 || (int64_t)chunk * (D / 16) * 4 >= ((int64_t)1 << 31)) return GQA_ERR_CHUNK;
  const size_t need = gqa::part_bytes(sh, chunk);
  const int64_t P = gqa::num_splits(sh, chunk);
  if (P > 0 && need == 0) return GQA_ERR_SHAPE;   // the partials would not fit any address space
  if (part_bytes < need) return GQA_ERR_WORKSPACE;
  if (P == 0) return GQA_OK;
  if (P > 0x7fffffff) return GQA_ERR_SHAPE;

  TqArgs a;
  a.q_rot = q_rot; a.q_jl = q_jl;
  a.k_polar = k_polar; a.k_jl = k_jl; a.k_norms = k_norms;
  a.v_polar = v_polar; a.v_norms = v_norms; a.seq_lens = seq_lens;
  a.part_o = part;
  a.part_ml = part + gqa::part_o_floats(sh, P);
  // centroid tables for the byte permutes: f16 high parts and the f16 of
  // what they leave out
  const float c[4] = {c0, c1, c2, c3};
  uint16_t hb[4], lb[4];
  for (int i = 0; i < 4; ++i) {
    const _Float16 h = (_Float16)c[i];
    hb[i] = f16_bits(h);
    lb[i] = f16_bits((_Float16)(c[i] - (float)h));
  }
  a.chi_lo = hb[0] | ((uint32_t)hb[1] << 16);
  a.chi_hi = hb[2] | ((uint32_t)hb[3] << 16);
  a.clo_lo = lb[0] | ((uint32_t)lb[1] << 16);
  a.clo_hi = lb[2] | ((uint32_t)lb[3] << 16);
  a.qjl_scale = qjl_scale;
  a.qscale = scale * kLog2e;
  a.S = S; a.T = T; a.Lmax = Lmax; a.H = H; a.Hk = Hk; a.G = H / Hk;
  a.R = (int)gqa::rows_per_unit(sh); a.nrb = (int)gqa::row_blocks(sh); a.P = (int)P; a.chunk = chunk;
  const int64_t nwg = P * Hk * a.nrb * S;
  if (nwg > 0x7fffffff) return GQA_ERR_SHAPE;
  const dim3 grid((unsigned)nwg);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // up to 8 rows per KV head: hi and lo query parts share one MFMA operand
  // (3 instead of 5 MFMAs per k-step of QK, 2 instead of 3 per PV block)
  const bool packed = a.R <= 8;
  const bool two = gqa::block_rows(sh) > 16;
  hipError_t e;
  if (D == 64)
    e = packed ? launch_tq<64, 1, true>(a, grid, st) : two ? launch_tq<64, 2>(a, grid, st) : launch_tq<64, 1>(a, grid, st);
  else
    e = packed ? launch_tq<128, 1, true>(a, grid, st) : two ? launch_tq<128, 2>(a, grid, st) : launch_tq<128, 1>(a, grid, st);
  return e == hipSuccess ? GQA_OK : (int)e;
}

int gqa_decode_merge_tq(const float* part, const int32_t* seq_lens, const float* signs, float* out,
                        int S, int T, int Lmax, int H, int D, int chunk, void* stream) {
  if (!part || !seq_lens || !signs || !out) return GQA_ERR_NULL;
  gqa::Shape sh{S, T, Lmax, 0, H, H, D, false, true};
  int rc = gqa::check_shape(sh);
  if (rc != GQA_OK) return rc;
  if (D != 64 && D != 128) return GQA_ERR_HEAD_DIM;
  if (chunk < 1) return GQA_ERR_CHUNK;
  const int64_t P = gqa::num_splits(sh, chunk);
  if (P > 0 && gqa::part_bytes(sh, chunk) == 0) return GQA_ERR_SHAPE;   // no workspace could hold it
  const size_t rows = (size_t)S * T * H;
  if (rows > 0x7fffffffu) return GQA_ERR_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  TqMergeArgs a;                               // P == 0 (empty cache): every row merges to zeros
  a.part_o = part;
  a.part_ml = part + gqa::part_o_floats(sh, P);
  a.signs = signs;
  a.out = out;
  a.P = (int)P;
  const dim3 grid((unsigned)rows);
  if (P <= 16) launch_merge_tq<4>(a, D, grid, st);
  else if (P <= 32) launch_merge_tq<8>(a, D, grid, st);
  else launch_merge_tq<16>(a, D, grid, st);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? GQA_OK : (int)e;
}

}  // extern "C"
