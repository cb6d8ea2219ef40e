// codec_driver.cpp -- test infrastructure: runs the library's host NVFP4
// encoder (flint_nvfp4_quantize_host, nvfp4_bit_projection_amd/csrc/
// codec_host.cpp) on seeded inputs, edge cases and its error paths, so that a
// build with AddressSanitizer + UndefinedBehaviorSanitizer, or with
// ThreadSanitizer (the encoder splits large matrices over threads), can report
// out-of-bounds accesses, undefined arithmetic or data races in it.  Its
// values are pinned bit-exactly against the oracle by the Python tests; the
// checks here are properties that hold for any correct encoder.  Exit status
// 0 when every check holds.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../../include/flint_moe.h"

static int failures = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      failures++;                                                     \
    }                                                                 \
  } while (0)

static uint64_t lcg = 0x2545F4914F6CDD1Dull;
static float uni(float amp) {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return amp * (float)((double)(lcg >> 11) * (2.0 / 9007199254740992.0) - 1.0);
}

struct Packed {
  std::vector<uint8_t> codes, scales;
  float S = -1.0f;
  int32_t rc = -1;
};

static Packed pack(const std::vector<float>& w, int64_t rows, int64_t cols) {
  Packed p;
  p.codes.assign((size_t)(rows * cols / 2), 0xAB);
  p.scales.assign((size_t)(rows * cols / 16), 0xAB);
  p.rc = flint_nvfp4_quantize_host(w.data(), rows, cols, p.codes.data(), p.scales.data(), &p.S);
  return p;
}

int main() {
  // one thread (below 2^20 values) and several (2^21 values): every byte of
  // both outputs written, and equal to the same rows packed on their own when
  // the tensor scale is the same (the largest value sits in the first rows)
  const int64_t C = 2048;
  for (int64_t R : {int64_t(64), int64_t(1024)}) {
    std::vector<float> w((size_t)(R * C));
    for (auto& v : w) v = uni(1.0f);
    w[7] = 4.0f;
    w[9] = -0.0f;
    Packed all = pack(w, R, C);
    CHECK(all.rc == FLINT_OK);
    CHECK(all.S == (float)(4.0 / 2688.0));
    std::vector<float> head(w.begin(), w.begin() + 8 * C);
    Packed first = pack(head, 8, C);
    CHECK(first.rc == FLINT_OK && first.S == all.S);
    CHECK(memcmp(first.codes.data(), all.codes.data(), first.codes.size()) == 0);
    CHECK(memcmp(first.scales.data(), all.scales.data(), first.scales.size()) == 0);
    Packed again = pack(w, R, C);
    CHECK(again.codes == all.codes && again.scales == all.scales);
  }

  // all zero (S = 0, zero codes and scales), negative zeros, one block
  {
    std::vector<float> z(16 * 64, 0.0f);
    Packed p = pack(z, 16, 64);
    CHECK(p.rc == FLINT_OK && p.S == 0.0f);
    for (uint8_t c : p.codes) CHECK(c == 0);
    for (uint8_t s : p.scales) CHECK(s == 0);
    std::vector<float> one(16);
    for (auto& v : one) v = uni(100.0f);
    Packed q = pack(one, 1, 16);
    CHECK(q.rc == FLINT_OK && q.S > 0.0f);
    CHECK(q.scales[0] == 0x7E);  // the largest block lands on E4M3's 448
  }

  // error paths: nothing written
  {
    std::vector<float> w(64, 1.0f);
    uint8_t c[32], s[4];
    float S = -1.0f;
    CHECK(flint_nvfp4_quantize_host(nullptr, 1, 64, c, s, &S) == FLINT_E_NULL);
    CHECK(flint_nvfp4_quantize_host(w.data(), 1, 64, nullptr, s, &S) == FLINT_E_NULL);
    CHECK(flint_nvfp4_quantize_host(w.data(), 1, 64, c, s, nullptr) == FLINT_E_NULL);
    CHECK(flint_nvfp4_quantize_host(w.data(), 0, 64, c, s, &S) == FLINT_E_DIMS);
    CHECK(flint_nvfp4_quantize_host(w.data(), 1, 8, c, s, &S) == FLINT_E_DIMS);
    CHECK(flint_nvfp4_quantize_host(w.data(), 2, 24, c, s, &S) == FLINT_E_DIMS);
    CHECK(flint_nvfp4_quantize_host(w.data(), int64_t(1) << 40, 64, c, s, &S) == FLINT_E_DIMS);
    CHECK(S == -1.0f);
  }

  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("codec driver: all checks passed\n");
  return 0;
}
