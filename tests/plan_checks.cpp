// Host-side planning and validation (decode_attention_kv_gqa_amd/csrc/plan.cpp)
// over extreme and random shapes, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_plan_sanitized.py.  Every result
// is checked against the same quantity computed here in 128-bit integers, so
// an overflow in the library's arithmetic either trips the sanitizer or
// fails a check.  Exit status 0 = every check passed.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>

#include "gqa_decode.h"
#include "plan.h"

static int failures = 0;
#define CHECK(cond, ...)                          \
  do {                                            \
    if (!(cond)) {                                \
      if (failures < 20) {                        \
        std::fprintf(stderr, "FAIL %s: ", #cond); \
        std::fprintf(stderr, __VA_ARGS__);        \
        std::fprintf(stderr, "\n");               \
      }                                           \
      ++failures;                                 \
    }                                             \
  } while (0)

typedef __int128 i128;

static void check_shape_case(int S, int T, int Lmax, int B, int H, int Hk, int D, bool ids, bool i8) {
  gqa::Shape s{S, T, Lmax, ids ? B : 0, H, Hk, D, ids, i8};
  const int rc = gqa::check_shape(s);
  const bool valid = S >= 1 && T >= 1 && H >= 1 && Hk >= 1 && Lmax >= 0 && H % Hk == 0 &&
                     (D == 64 || D == 128 || D == 256) && (!ids || B >= 1);
  if (!valid) {
    CHECK(rc != GQA_OK, "S=%d T=%d Lmax=%d B=%d H=%d Hk=%d D=%d accepted", S, T, Lmax, B, H, Hk, D);
    return;
  }
  const i128 G = H / Hk, R = ids ? G : G * T;
  const i128 rows_per_block = D <= 128 ? 64 : 32;    // four 16-row blocks up to head_dim 128
  const i128 nrb = (R + rows_per_block - 1) / rows_per_block;
  const i128 units = (i128)S * Hk * nrb * (ids ? T : 1);
  const bool grid_ok = units <= 0x7fffffff && (i128)S * T * H <= 0x7fffffff;
  CHECK((rc == GQA_OK) == grid_ok, "S=%d T=%d H=%d Hk=%d grid check rc=%d", S, T, H, Hk, rc);
  if (rc != GQA_OK) return;
  const int chunk = gqa::auto_chunk(s);
  const i128 mc = gqa::max_chunk(s);
  CHECK(chunk >= 1 && chunk <= mc, "auto_chunk %d outside [1, %lld]", chunk, (long long)mc);
  const i128 W = ids ? (B < Lmax ? B : Lmax) : Lmax;
  for (int c : {1, 7, 32, 64, chunk, (int)(mc < 0x7fffffff ? mc : 0x7fffffff)}) {
    if (c < 1) continue;
    const i128 P = W <= 0 ? 0 : (W + c - 1) / c;
    CHECK(gqa::num_splits(s, c) == (int64_t)P, "num_splits");
    const i128 bytes = (i128)S * T * H * P * (D + 2) * 4;
    const size_t got = gqa::part_bytes(s, c);
    if (bytes < ((i128)1 << 62)) CHECK((i128)got == bytes, "part_bytes %zu vs %lld", got, (long long)bytes);
    const i128 ofl = (i128)S * T * H * P * D;
    if (ofl < ((i128)1 << 62)) CHECK((i128)gqa::part_o_floats(s, P) == ofl, "part_o_floats");
  }
  // balanced partition (negative chunk): dense windows only, at most 65536
  // pieces, S * (Lmax + 1152) below 2^31; P slots per row, then S int32
  // slot counts rounded up to 16 bytes
  for (int c : {-1, -7, -32, -65536, -65537, -2147483647 - 1}) {
    const bool ok = !ids && (i128)-(i128)c <= 65536 && (i128)S * ((i128)Lmax + 1152) < ((i128)1 << 31);
    CHECK(gqa::balanced_ok(s, c) == ok, "balanced_ok S=%d Lmax=%d c=%d ids=%d", S, Lmax, c, (int)ids);
    const size_t got = gqa::part_bytes(s, c);
    if (!ok) {
      CHECK(got == 0, "part_bytes of a refused balanced partition %zu", got);
      continue;
    }
    const i128 P = Lmax <= 0 ? 0 : -(i128)c;
    CHECK(gqa::num_splits(s, c) == (int64_t)P, "balanced num_splits");
    const i128 bytes = (i128)S * T * H * P * (D + 2) * 4 + ((i128)S * 4 + 15) / 16 * 16;
    if (bytes < ((i128)1 << 62)) CHECK((i128)got == bytes, "balanced part_bytes %zu vs %lld", got, (long long)bytes);
    const i128 off = (i128)S * T * H * P * (D + 2);
    if (off < ((i128)1 << 62)) CHECK((i128)gqa::flat_n_offset_floats(s, P) == off, "flat_n_offset_floats");
    const int pad = i8 ? 256 : 65536 / (4 * D);
    CHECK(gqa::flat_pad_cells(s) == (pad + 127) / 128 * 128, "flat_pad_cells");
  }
  CHECK(gqa_decode_part_bytes(S, T, Lmax, ids ? B : 0, H, D, chunk) ==
            gqa::part_bytes(gqa::Shape{S, T, Lmax, ids ? B : 0, H, H, D, ids, false}, chunk),
        "exported part_bytes");
  const int ac = gqa_decode_auto_chunk(S, T, Lmax, ids ? B : 0, H, Hk, D, i8 ? 1 : 0);
  CHECK(ac == chunk, "exported auto_chunk %d vs %d", ac, chunk);
}

int main() {
  const int big[] = {0, 1, 2, 3, 7, 8, 31, 32, 33, 1000, 65536, 1 << 20, 0x3fffffff, 0x7fffffff, -1,
                     -2147483647 - 1};
  for (int S : big)
    for (int T : {1, 8, 0x7fffffff})
      for (int H : {1, 24, 4096, 0x7fffffff})
        for (int Hk : {1, 2, 8})
          for (int Lmax : {0, 1, 32768, 0x7fffffff})
            for (int D : {64, 256, 96})
              for (int ids = 0; ids < 2; ++ids) check_shape_case(S, T, Lmax, 2048, H, Hk, D, ids, ids);
  std::mt19937_64 rng(12345);
  auto pick = [&](int lo, int hi) { return (int)std::uniform_int_distribution<long long>(lo, hi)(rng); };
  const int dims[] = {64, 128, 256};
  for (int i = 0; i < 200000; ++i) {
    const int Hk = pick(1, 64), G = pick(1, 64), ids = pick(0, 1);
    const int H = (int)((long long)Hk * G > 0x7fffffff ? 0x7fffffff : Hk * G);
    check_shape_case(pick(1, 1 << pick(0, 30)), pick(1, 1 << pick(0, 12)), pick(0, 1 << pick(0, 30)),
                     pick(1, 1 << pick(0, 24)), H, Hk, dims[pick(0, 2)], ids, pick(0, 1));
  }
  for (int c = -10; c < 10; ++c) CHECK(gqa_decode_strerror(c) != nullptr && std::strlen(gqa_decode_strerror(c)) > 0, "strerror %d", c);
  std::printf("plan checks: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
