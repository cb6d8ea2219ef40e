// codec_host.cpp -- the library's NVFP4 encoder on the host (no GPU needed):
// packs an fp32 matrix into the interchange layout that every decode kernel
// reads.
//
// Format [P3 "Flint: 125 tokens a second is what 2.5B active parameters buy
// at 273 GB/s", "Checking 125 tokens a second": 4-bit values with one 8-bit
// scale per 16 values; P1 "Flint-40B-A2B: AI-Built MoE Coding Model Hits
// 125 tok/s on MacBook Pro", "Quantization with Offline Distillation":
// NVFP4 weights and head].  Element codes are E2M1 (sign, two exponent bits
// with bias 1, one mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), block
// scales OCP E4M3FN (bias 7, three mantissa bits, largest finite 448), and one
// fp32 scale S per tensor.
//
// Recipe (the same reading as the device quantiser): S = fl32(max|w| / 2688),
// i.e. the largest block scale lands on E4M3's 448; block scale = E4M3
// round-to-nearest-even of blockmax / (6 S), saturating at 448; element code =
// E2M1 round-to-nearest-even of w / (d S), saturating at 6, with the sign bit
// of w (also when the magnitude rounds to 0); a block whose scale is 0, and an
// all-zero tensor (S = 0), get zero codes.  Every ratio is formed in double
// precision, where 6 S and d S are exact.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "../../include/flint_moe.h"

namespace {

// OCP E4M3FN code of r >= 0, round to nearest even, saturating at 448 (0x7E).
// Normal codes hold (1 + m/8) 2^(e-7) for e = 1..15; subnormals m 2^-9.
int e4m3_code(double r) {
  if (!(r < 448.0)) return 0x7E;
  if (r < 0.015625) {  // below the smallest normal 2^-6: steps of 2^-9
    const double q = nearbyint(r * 512.0);  // round half to even (default mode)
    return (int)q;                          // q == 8 is the code of 2^-6 itself
  }
  int ex;
  const double f = frexp(r, &ex);           // r = f 2^ex, f in [0.5, 1)
  double m = nearbyint((2.0 * f - 1.0) * 8.0);
  int e = ex - 1 + 7;
  if (m == 8.0) { m = 0.0; ++e; }           // rounded up to the next binade
  const int code = (e << 3) | (int)m;
  return code > 0x7E ? 0x7E : code;
}

double e4m3_decode(int code) {
  const int e = code >> 3, m = code & 7;
  return e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
}

// E2M1 code of v: the magnitude rounded to the nearest of {0, .5, 1, 1.5, 2,
// 3, 4, 6} with ties to the even code (the midpoints .25 .75 1.25 1.75 2.5
// 3.5 5 go to codes 0 2 2 4 4 6 6, i.e. the values 0 1 1 2 2 4 4), saturating
// at 6; bit 3 is the sign of v.
uint8_t e2m1_code(double v) {
  static const double kMid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  const double a = fabs(v);
  int c = 0;
  while (c < 7 && a > kMid[c]) ++c;
  // a equal to a midpoint: the loop stopped below it at code c (even or odd);
  // ties go to the even neighbour of the two codes c and c + 1
  if (c < 7 && a == kMid[c] && (c & 1)) ++c;
  return (uint8_t)(c | (signbit(v) ? 8 : 0));
}

void pack_rows(const float* w, int64_t r0, int64_t r1, int64_t cols, float S, uint8_t* codes, uint8_t* scales) {
  const int64_t nb = cols / 16;
  for (int64_t r = r0; r < r1; ++r) {
    const float* row = w + r * cols;
    for (int64_t b = 0; b < nb; ++b) {
      const float* x = row + 16 * b;
      uint8_t* c = codes + r * (cols / 2) + 8 * b;
      int sc = 0;
      if (S != 0.0f) {
        float bm = 0.0f;
        for (int i = 0; i < 16; ++i) bm = std::max(bm, fabsf(x[i]));
        sc = e4m3_code((double)bm / (6.0 * (double)S));
      }
      scales[r * nb + b] = (uint8_t)sc;
      const double dS = e4m3_decode(sc) * (double)S;
      for (int j = 0; j < 8; ++j) {
        uint8_t lo = 0, hi = 0;
        if (dS != 0.0) {
          lo = e2m1_code((double)x[2 * j] / dS);
          hi = e2m1_code((double)x[2 * j + 1] / dS);
        }
        c[j] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

}  // namespace

extern "C" int32_t flint_nvfp4_quantize_host(const float* w, int64_t rows, int64_t cols, uint8_t* codes,
                                             uint8_t* scales, float* tscale) {
  if (!w || !codes || !scales || !tscale) return FLINT_E_NULL;
  if (rows < 1 || cols < 16 || cols % 16 || rows > ((int64_t)1 << 40) / cols) return FLINT_E_DIMS;
  const int64_t n = rows * cols;
  unsigned nt = std::thread::hardware_concurrency();
  nt = nt == 0 ? 1 : std::min(nt, 32u);
  if (n < ((int64_t)1 << 20)) nt = 1;
  // max |w| (an exact operation: any order gives the same value)
  std::vector<float> part(nt, 0.0f);
  auto amax_range = [&](unsigned i) {
    const int64_t a = n * i / nt, b = n * (i + 1) / nt;
    float m = 0.0f;
    for (int64_t k = a; k < b; ++k) m = std::max(m, fabsf(w[k]));
    part[i] = m;
  };
  std::vector<std::thread> th;
  for (unsigned i = 1; i < nt; ++i) th.emplace_back(amax_range, i);
  amax_range(0);
  for (auto& t : th) t.join();
  th.clear();
  float amax = 0.0f;
  for (float m : part) amax = std::max(amax, m);
  const float S = (float)((double)amax / 2688.0);
  *tscale = S;
  // blocks are independent: rows split over threads, identical results for
  // any thread count
  auto pack = [&](unsigned i) { pack_rows(w, rows * i / nt, rows * (i + 1) / nt, cols, S, codes, scales); };
  for (unsigned i = 1; i < nt; ++i) th.emplace_back(pack, i);
  pack(0);
  for (auto& t : th) t.join();
  return FLINT_OK;
}
