// The whole decode step (attention + merge) with its partials in a static
// device buffer owned by the library, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  It runs the same kernels as gqa_decode_attn_f16 /
// gqa_decode_attn_i8 followed by gqa_decode_merge; the only difference is
// where the partials live.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "gqa_decode.h"

// One copy per GPU the library runs on, held until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// host code uses only the address hipGetSymbolAddress returns for the
// current device.
static __device__ __align__(256) float scratch[GQA_STATIC_PART_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_lookup;

// This device's address of `scratch` (looked up once per device, with that
// device current); 0, or a hipError_t, or GQA_ERR_SHAPE for a device index
// past kMaxDevices.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return GQA_ERR_SHAPE;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_lookup);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return (int)e;
      if (!p) return (int)hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return 0;
}

}  // namespace

extern "C" int gqa_decode_step_static(const float* q, const void* k, const void* v,
                                      const uint16_t* k_scales, const uint16_t* v_scales,
                                      const int32_t* ids, const int32_t* seq_lens, float* out,
                                      int S, int T, int Lmax, int B, int H, int Hk, int D,
                                      float scale, int chunk, int kv_kind, void* stream) {
  // the checks the two calls make, before the buffer's address is looked up
  if (kv_kind != 0 && kv_kind != 1) return GQA_ERR_SHAPE;
  if (!q || !out || !seq_lens) return GQA_ERR_NULL;
  if (Lmax > 0 && (!k || !v || (kv_kind == 1 && (!k_scales || !v_scales)))) return GQA_ERR_NULL;
  if (ids && B < 1) return GQA_ERR_BUDGET;
  const int Bx = ids ? B : 0;
  if (chunk == 0) {
    chunk = gqa_decode_auto_chunk(S, T, Lmax, Bx, H, Hk, D, kv_kind);
    if (chunk <= 0) return chunk;
  }
  // Every partial slot the merge reads is written by the attention call of
  // the same step, so nothing left in the buffer by an earlier call is read.
  if (gqa_decode_part_bytes(S, T, Lmax, Bx, H, D, chunk) > GQA_STATIC_PART_BYTES)
    return GQA_ERR_STATIC_LIMIT;
  void* part = nullptr;
  int rc = scratch_address(&part);
  if (rc != 0) return rc;
  float* pf = static_cast<float*>(part);
  rc = kv_kind == 1
           ? gqa_decode_attn_i8(q, static_cast<const int8_t*>(k), static_cast<const int8_t*>(v),
                                k_scales, v_scales, ids, seq_lens, pf, GQA_STATIC_PART_BYTES, S, T,
                                Lmax, B, H, Hk, D, scale, chunk, stream)
           : gqa_decode_attn_f16(q, static_cast<const uint16_t*>(k),
                                 static_cast<const uint16_t*>(v), ids, seq_lens, pf,
                                 GQA_STATIC_PART_BYTES, S, T, Lmax, B, H, Hk, D, scale, chunk,
                                 stream);
  if (rc != GQA_OK) return rc;
  return gqa_decode_merge(pf, seq_lens, ids, out, S, T, Lmax, B, H, D, chunk, stream);
}
