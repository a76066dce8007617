// Log-sum-exp merge of the split-KV partials on gfx950 (MI355X): one
// workgroup per output row combines the (o unnormalised, m, l) partials of
// that row's splits (qsa2.metal, qsa_merge2), optionally multiplying the
// result by sigmoid(gate) (qsa2.metal, end of qsa_merge2; FORWARD_MSL, end of
// attn_combine).  The partials' running max is in base-2 units (the
// attention kernels fold log2(e) into the query), so the weights are exp2.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "common.h"
#include "gqa_decode.h"
#include "plan.h"

namespace {

using gqa_kern::MergeArgs;

constexpr int kThreads = 256;

// One workgroup per output row (s, t, h); its four waves split the row's
// partials (wave w takes splits w, w+4, ...) and lane l holds dims
// l*V .. l*V+V-1 (V = D/64), so one split's o is one 16/8/4-byte load per
// lane, 1 KB / 512 B / 256 B per wave, coalesced.  Each wave merges its
// splits online (a running max with rescaling, the same update as the
// attention's softmax but over partials), so every load of the row is issued
// up front and no wave waits for another before reading o; the four waves'
// (max, sum, o) are then combined through LDS.  U splits per wave have their
// loads in flight together: U = 4 covers 16 splits in one round trip, and
// longer rows (budgeted windows cut into 32-cell splits: 64 of them) get
// U = 8 or 16 so that they also take one.
template <int D, int U>
__global__ __launch_bounds__(kThreads) void merge_rows(MergeArgs a) {
  constexpr int V = D / 64;
  __shared__ float red_o[4][D];
  __shared__ float red_ml[4][2];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int row = blockIdx.x;             // ((s * T) + t) * H + h
  // The attention call writes every (row, split) slot; a split without a
  // visible cell of the row carries m = -inf and is skipped, so the row's
  // window need not be recomputed here and every load is issued at once.
  const int nv = a.P;
  const float* ml = a.part_ml + (size_t)row * a.P * 2;
  const float* po = a.part_o + (size_t)row * a.P * D + lane * V;
  // output gate (qsa2.metal, qsa_merge2; FORWARD_MSL, attn_combine): the
  // merged row is multiplied by sigmoid(gate) elementwise.  Wave 0 writes
  // the row, so it requests its gate elements first.
  float gt[V];
  const bool gated = a.gate != nullptr;
  if (gated && wave == 0) {
    const float* gsrc = a.gate + (size_t)row * a.gate_stride + lane * V;
#pragma unroll
    for (int e = 0; e < V; ++e) gt[e] = gsrc[e];
  }

  float M = -INFINITY, lsum = 0.f;
  float acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.f;
  for (int j0 = wave; j0 < nv; j0 += 4 * U) {
    float mj[U], lj[U], oj[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + 4 * u;
      mj[u] = -INFINITY;
      lj[u] = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) oj[u][e] = 0.f;
      if (j < nv) {
        mj[u] = ml[2 * j];
        lj[u] = ml[2 * j + 1];
        const float* src = po + (size_t)j * D;
        if constexpr (V == 4) {
          const float4 x = *reinterpret_cast<const float4*>(src);
          oj[u][0] = x.x; oj[u][1] = x.y; oj[u][2] = x.z; oj[u][3] = x.w;
        } else if constexpr (V == 2) {
          const float2 x = *reinterpret_cast<const float2*>(src);
          oj[u][0] = x.x; oj[u][1] = x.y;
        } else {
          oj[u][0] = *src;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (mj[u] == -INFINITY) continue;   // no visible cell in that split: weight 0
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
  if (wave == 0) {
    float* out = a.out + (size_t)row * D + lane * V;
    float Mt = red_ml[0][0];
#pragma unroll
    for (int w = 1; w < 4; ++w) Mt = fmaxf(Mt, red_ml[w][0]);
    if (Mt == -INFINITY) {                  // no visible cell: zeros
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
#pragma unroll
    for (int e = 0; e < V; ++e) {
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) x = fmaf(f[w], red_o[w][lane * V + e], x);
      x = x / Ls;
      if (gated) x *= 1.0f / (1.0f + __expf(-gt[e]));
      out[e] = x;
    }
  }
}

// Merge after a balanced-partition attention call: row (s, t, h)'s partials
// fill its slots 0 .. n-1, n = flat_n[s] as written by the attention call (0
// for an empty window).  Wave w requests slots w, w+4, .., w+4(U-1)
// together with n, before n is known (slots below P lie inside the
// workspace either way; those at or past n are dropped), so rows of up to
// 4U partials take one round trip.  The host sizes U from the partials a
// sequence of the batch's mean window gets (P / S): one for batches of
// about a piece per sequence, four for sixteen pieces per sequence.
template <int D, int U>
__global__ __launch_bounds__(kThreads) void merge_rows_flat(MergeArgs a) {
  constexpr int V = D / 64;
  __shared__ float red_o[4][D];
  __shared__ float red_ml[4][2];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int row = blockIdx.x;             // ((s * T) + t) * H + h
  const float* ml = a.part_ml + (size_t)row * a.P * 2;
  const float* po = a.part_o + (size_t)row * a.P * D + lane * V;
  float gt[V];
  const bool gated = a.gate != nullptr;
  if (gated && wave == 0) {
    const float* gsrc = a.gate + (size_t)row * a.gate_stride + lane * V;
#pragma unroll
    for (int e = 0; e < V; ++e) gt[e] = gsrc[e];
  }
  auto load = [&](int j, float& mj, float& lj, float (&oj)[V]) {
    mj = ml[2 * j];
    lj = ml[2 * j + 1];
    const float* src = po + (size_t)j * D;
#pragma unroll
    for (int e = 0; e < V; ++e) oj[e] = src[e];
  };
  float m0[U], l0[U], o0[U][V];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    m0[u] = -INFINITY;
    l0[u] = 0.f;
#pragma unroll
    for (int e = 0; e < V; ++e) o0[u][e] = 0.f;
    if (wave + 4 * u < a.P) load(wave + 4 * u, m0[u], l0[u], o0[u]);
  }
  // (P == 0: an empty cache, for which the attention call writes nothing)
  const int n = a.P > 0 ? a.flat_n[row / a.TH] : 0;

  float M = -INFINITY, lsum = 0.f;
  float acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = 0.f;
  auto take = [&](float mj, float lj, const float (&oj)[V]) {
    if (mj == -INFINITY) return;          // no visible cell of the row in that split
    if (mj > M) {
      const float c = (M == -INFINITY) ? 0.f : exp2f(M - mj);
      lsum *= c;
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] *= c;
      M = mj;
    }
    const float w = exp2f(mj - M);
    lsum = fmaf(w, lj, lsum);
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = fmaf(w, oj[e], acc[e]);
  };
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (wave + 4 * u < n) take(m0[u], l0[u], o0[u]);
  for (int j = wave + 4 * U; j < n; j += 4) {
    float mj, lj, oj[V];
    load(j, mj, lj, oj);
    take(mj, lj, oj);
  }
#pragma unroll
  for (int e = 0; e < V; ++e) red_o[wave][lane * V + e] = acc[e];
  if (lane == 0) {
    red_ml[wave][0] = M;
    red_ml[wave][1] = lsum;
  }
  __syncthreads();
  if (wave == 0) {
    float* out = a.out + (size_t)row * D + lane * V;
    float Mt = red_ml[0][0];
#pragma unroll
    for (int w = 1; w < 4; ++w) Mt = fmaxf(Mt, red_ml[w][0]);
    if (Mt == -INFINITY) {                  // no visible cell: zeros
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
#pragma unroll
    for (int e = 0; e < V; ++e) {
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) x = fmaf(f[w], red_o[w][lane * V + e], x);
      x = x / Ls;
      if (gated) x *= 1.0f / (1.0f + __expf(-gt[e]));
      out[e] = x;
    }
  }
}

template <int U>
void launch_merge_flat(const MergeArgs& a, int D, dim3 grid, hipStream_t st) {
  switch (D) {
    case 64: hipLaunchKernelGGL((merge_rows_flat<64, U>), grid, dim3(kThreads), 0, st, a); break;
    case 128: hipLaunchKernelGGL((merge_rows_flat<128, U>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((merge_rows_flat<256, U>), grid, dim3(kThreads), 0, st, a); break;
  }
}

template <int U>
void launch_merge(const MergeArgs& a, int D, dim3 grid, hipStream_t st) {
  switch (D) {
    case 64: hipLaunchKernelGGL((merge_rows<64, U>), grid, dim3(kThreads), 0, st, a); break;
    case 128: hipLaunchKernelGGL((merge_rows<128, U>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((merge_rows<256, U>), grid, dim3(kThreads), 0, st, a); break;
  }
}

}  // namespace

extern "C" {

static int merge_common(const float* part, const int32_t* seq_lens, const int32_t* ids_or_null,
                        const float* gate, int64_t gate_stride, float* out, int S, int T,
                        int Lmax, int B, int H, int D, int chunk, void* stream) {
  if (!part || !seq_lens || !out) return GQA_ERR_NULL;
  const bool ids = ids_or_null != nullptr;
  gqa::Shape sh{S, T, Lmax, ids ? B : 0, H, H, D, ids, false};
  int rc = gqa::check_shape(sh);
  if (rc != GQA_OK) return rc;
  if (chunk == 0 || (chunk < 0 && !gqa::balanced_ok(sh, chunk))) return GQA_ERR_CHUNK;
  if (gate && gate_stride < D) return GQA_ERR_SHAPE;
  const int64_t P = gqa::num_splits(sh, chunk);
  if (P > 0 && gqa::part_bytes(sh, chunk) == 0) return GQA_ERR_SHAPE;   // no workspace could hold it
  MergeArgs a;
  a.part_o = part;
  a.part_ml = part + gqa::part_o_floats(sh, P);
  a.out = out;
  a.gate = gate;
  a.gate_stride = gate_stride;
  a.P = (int)P;
  a.flat = chunk < 0;
  a.flat_n = reinterpret_cast<const int32_t*>(part + gqa::flat_n_offset_floats(sh, P));
  a.TH = T * H;
  const size_t rows = (size_t)S * T * H;
  if (rows > 0x7fffffffu) return GQA_ERR_SHAPE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  dim3 grid((unsigned)rows);
  if (a.flat) {
    // partials of a sequence of the mean window: about P / S
    const int64_t per = (P + S - 1) / S;
    if (per <= 4)
      launch_merge_flat<1>(a, D, grid, st);
    else if (per <= 8)
      launch_merge_flat<2>(a, D, grid, st);
    else
      launch_merge_flat<4>(a, D, grid, st);
  } else if (P <= 16)
    launch_merge<4>(a, D, grid, st);
  else if (P <= 32)
    launch_merge<8>(a, D, grid, st);
  else
    launch_merge<16>(a, D, grid, st);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? GQA_OK : (int)e;
}

int gqa_decode_merge(const float* part, const int32_t* seq_lens, const int32_t* ids_or_null,
                     float* out, int S, int T, int Lmax, int B, int H, int D, int chunk,
                     void* stream) {
  return merge_common(part, seq_lens, ids_or_null, nullptr, 0, out, S, T, Lmax, B, H, D, chunk,
                      stream);
}

int gqa_decode_merge_gated(const float* part, const int32_t* seq_lens, const int32_t* ids_or_null,
                           const float* gate, int64_t gate_stride, float* out, int S, int T,
                           int Lmax, int B, int H, int D, int chunk, void* stream) {
  if (!gate) return GQA_ERR_NULL;
  return merge_common(part, seq_lens, ids_or_null, gate, gate_stride, out, S, T, Lmax, B, H, D,
                      chunk, stream);
}

}  // extern "C"
