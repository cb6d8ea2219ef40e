/* oracle_driver.c -- test infrastructure: runs every entry point of the
 * oracle (oracle/oracle.c) on small seeded inputs and edge cases, so that a
 * build with AddressSanitizer + UndefinedBehaviorSanitizer, or with
 * ThreadSanitizer, can report out-of-bounds accesses, leaks, undefined
 * arithmetic or data races in it.  The checks here are invariants of the
 * codecs (a decoded value encodes back to itself, all-zero input gives zero
 * codes, routing weights sum to one); the values themselves are pinned by the
 * Python tests.  Exit status 0 when every check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e2m1_value(int code);
double oracle_e4m3_value(int code);
int oracle_e2m1_encode(double v);
int oracle_e4m3_encode(double r);
void oracle_nvfp4_quantize(const float* w, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                           float* tscale, int nthreads);
void oracle_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, float tscale, int64_t rows,
                             int64_t cols, float* out);
void oracle_nvfp4_gemv(const uint8_t* codes, const uint8_t* scales, float tscale, int64_t rows, int64_t cols,
                       const double* x, double* y, int nthreads);
void oracle_f32_gemv(const float* w, int64_t rows, int64_t cols, const double* x, double* y, int nthreads);
void oracle_topk_softmax(const double* logits, int E, int k, int32_t* idx, double* w, double* gap);
void oracle_topk_sigmoid(const double* logits, int E, int k, int32_t* idx, double* w, double* gap);
void oracle_bf16_decode(const uint16_t* b, int64_t n, double* out);
double oracle_rms_inv(const double* h, int64_t n, double eps);
void oracle_swiglu_expert(const uint8_t* gc, const uint8_t* gs, float gS, const uint8_t* uc, const uint8_t* us,
                          float uS, const uint8_t* dc, const uint8_t* ds, float dS, int64_t H, int64_t I,
                          const double* u, double* y, double* h_out, int nthreads);
int64_t oracle_argmax(const double* v, int64_t n, double* gap);
uint16_t oracle_bf16_encode(double v);
void oracle_bf16_round(const double* x, int64_t n, uint16_t* out);
void oracle_head_rmsnorm(double* v, int D, const float* g, double eps);
void oracle_rope(double* v, int D, int64_t pos, double theta);
int oracle_attn_decode(int H, int Hq, int Hkv, int D, int window, int rope, double theta, double eps,
                       const uint8_t* const* codes, const uint8_t* const* scales, const float* tscales,
                       const float* qn, const float* kn, const float* sinks, const double* x, int64_t pos,
                       uint16_t* kc, uint16_t* vc, int64_t cap, double* y, double* o_out, double* qkv_out,
                       int nthreads);
void oracle_int4_quantize(const float* w, int64_t rows, int64_t cols, uint8_t* codes, uint16_t* scales,
                          uint16_t* biases);
void oracle_int4_dequantize(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t rows,
                            int64_t cols, float* out);
void oracle_int4_gemv(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t rows,
                      int64_t cols, const double* x, double* y, int nthreads);
void oracle_nvfp4_gemm(const uint8_t* codes, const uint8_t* scales, float tscale, int64_t N, int64_t K,
                       const double* X, int64_t T, double* Y, int nthreads);
void oracle_nvfp4_gemm_a4(const uint8_t* codes, const uint8_t* scales, float tscale, int64_t N, int64_t K,
                          const float* X, int64_t T, double* Y, int nthreads);

static int failures = 0;
#define CHECK(c)                                                    \
  do {                                                              \
    if (!(c)) {                                                     \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      failures++;                                                   \
    }                                                               \
  } while (0)

/* seeded uniform values in [-1, 1) from a 64-bit LCG (inputs only) */
static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static double uni(void) {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(lcg >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}
static float* fill_f32(int64_t n, double amp) {
  float* p = malloc(sizeof(float) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) p[i] = (float)(amp * uni());
  return p;
}
static double* fill_f64(int64_t n, double amp) {
  double* p = malloc(sizeof(double) * (size_t)n);
  for (int64_t i = 0; i < n; ++i) p[i] = amp * uni();
  return p;
}

typedef struct {
  uint8_t* c;
  uint8_t* s;
  float S;
} nv;

static nv quant(const float* w, int64_t rows, int64_t cols, int nt) {
  nv m;
  m.c = malloc((size_t)(rows * cols / 2));
  m.s = malloc((size_t)(rows * cols / 16));
  oracle_nvfp4_quantize(w, rows, cols, m.c, m.s, &m.S, nt);
  return m;
}
static void nv_free(nv m) {
  free(m.c);
  free(m.s);
}

static void codecs(void) {
  for (int c = 0; c < 16; ++c) CHECK(oracle_e2m1_encode(oracle_e2m1_value(c)) == (c == 8 ? 8 : c));
  for (int c = 0; c < 127; ++c) CHECK(oracle_e4m3_encode(oracle_e4m3_value(c)) == c);
  CHECK(oracle_e4m3_encode(1e9) == 0x7E);

  /* quantise -> decode -> quantise gives the same codes (rows >= 64: threads) */
  const int64_t R = 96, C = 256;
  float* w = fill_f32(R * C, 3.0);
  w[5] = -0.0f;
  for (int k = 16; k < 32; ++k) w[k] = 0.0f; /* an all-zero block */
  nv a = quant(w, R, C, 4);
  float* d = malloc(sizeof(float) * (size_t)(R * C));
  oracle_nvfp4_dequantize(a.c, a.s, a.S, R, C, d);
  nv b = quant(d, R, C, 3);
  CHECK(a.S == b.S);
  CHECK(memcmp(a.c, b.c, (size_t)(R * C / 2)) == 0);
  CHECK(memcmp(a.s, b.s, (size_t)(R * C / 16)) == 0);

  double* x = fill_f64(C, 1.0);
  double* y1 = malloc(sizeof(double) * R);
  double* y2 = malloc(sizeof(double) * R);
  double* yt = malloc(sizeof(double) * 3 * R);
  oracle_nvfp4_gemv(a.c, a.s, a.S, R, C, x, y1, 1);
  oracle_nvfp4_gemv(a.c, a.s, a.S, R, C, x, y2, 5);
  CHECK(memcmp(y1, y2, sizeof(double) * R) == 0);
  oracle_f32_gemv(d, R, C, x, y2, 7);
  for (int64_t r = 0; r < R; ++r) CHECK(fabs(y1[r] - y2[r]) <= 1e-9 * (1.0 + fabs(y1[r])));

  double* X = fill_f64(3 * C, 1.0);
  memcpy(X, x, sizeof(double) * C);
  oracle_nvfp4_gemm(a.c, a.s, a.S, R, C, X, 3, yt, 4);
  CHECK(memcmp(yt, y1, sizeof(double) * R) == 0);
  float* Xf = fill_f32(3 * C, 2.0);
  oracle_nvfp4_gemm_a4(a.c, a.s, a.S, R, C, Xf, 3, yt, 2);
  for (int64_t i = 0; i < 3 * R; ++i) CHECK(isfinite(yt[i]));

  /* all-zero tensor: S = 0 and zero codes */
  float* z = calloc((size_t)(64 * 32), sizeof(float));
  nv zq = quant(z, 64, 32, 2);
  CHECK(zq.S == 0.0f);
  for (int i = 0; i < 64 * 16; ++i) CHECK(zq.c[i] == 0);
  nv_free(zq);
  free(z);

  free(w);
  free(d);
  free(x);
  free(y1);
  free(y2);
  free(yt);
  free(X);
  free(Xf);
  nv_free(a);
  nv_free(b);
}

static void routing(void) {
  for (int E = 6; E <= 256; E = E == 6 ? 32 : E * 8) {
    double* l = fill_f64(E, 4.0);
    if (E > 8) l[3] = l[4]; /* a tie */
    int32_t idx[6];
    double w[6], gap, sum;
    oracle_topk_softmax(l, E, 6, idx, w, &gap);
    sum = 0;
    for (int i = 0; i < 6; ++i) {
      CHECK(idx[i] >= 0 && idx[i] < E);
      sum += w[i];
    }
    CHECK(fabs(sum - 1.0) < 1e-12);
    CHECK(gap >= 0.0);
    oracle_topk_sigmoid(l, E, 6, idx, w, &gap);
    sum = 0;
    for (int i = 0; i < 6; ++i) sum += w[i];
    CHECK(fabs(sum - 1.0) < 1e-12);
    int64_t am = oracle_argmax(l, E, &gap);
    CHECK(am >= 0 && am < E && gap >= 0.0);
    free(l);
  }
}

static void bf16_and_norms(void) {
  uint16_t all[65536];
  double dec[65536];
  for (int i = 0; i < 65536; ++i) all[i] = (uint16_t)i;
  oracle_bf16_decode(all, 65536, dec);
  for (int i = 0; i < 65536; ++i) {
    int ex = (i >> 7) & 0xFF;
    if (ex != 0xFF) CHECK(oracle_bf16_encode(dec[i]) == (uint16_t)i);
  }
  double* h = fill_f64(2048, 1.0);
  uint16_t r[2048];
  oracle_bf16_round(h, 2048, r);
  CHECK(oracle_rms_inv(h, 2048, 1e-6) > 0.0);
  float g[128];
  for (int i = 0; i < 128; ++i) g[i] = 1.0f;
  oracle_head_rmsnorm(h, 128, g, 1e-6);
  oracle_rope(h, 128, 1000, 1e6);
  free(h);
}

static void expert_and_attention(void) {
  const int H = 256, I = 64;
  float* gw = fill_f32((int64_t)I * H, 1.0);
  float* uw = fill_f32((int64_t)I * H, 1.0);
  float* dw = fill_f32((int64_t)H * I, 1.0);
  nv G = quant(gw, I, H, 2), U = quant(uw, I, H, 2), Dn = quant(dw, H, I, 4);
  double* u = fill_f64(H, 1.0);
  double* y = malloc(sizeof(double) * H);
  double* hs = malloc(sizeof(double) * I);
  oracle_swiglu_expert(G.c, G.s, G.S, U.c, U.s, U.S, Dn.c, Dn.s, Dn.S, H, I, u, y, hs, 3);
  oracle_swiglu_expert(G.c, G.s, G.S, U.c, U.s, U.S, Dn.c, Dn.s, Dn.S, H, I, u, y, NULL, 1);

  /* attention: 4 query heads over 2 key/value heads of 32, sliding window 5
   * in a ring of 5 slots, then full context, with and without rotation */
  const int Hq = 4, Hkv = 2, D = 32;
  float* mw[4] = {fill_f32((int64_t)Hq * D * H, 1.0), fill_f32((int64_t)Hkv * D * H, 1.0),
                  fill_f32((int64_t)Hkv * D * H, 1.0), fill_f32((int64_t)H * Hq * D, 1.0)};
  const int64_t rows[4] = {Hq * D, Hkv * D, Hkv * D, H}, cols[4] = {H, H, H, Hq * D};
  nv m[4];
  const uint8_t* codes[4];
  const uint8_t* scales[4];
  float ts[4];
  for (int i = 0; i < 4; ++i) {
    m[i] = quant(mw[i], rows[i], cols[i], 2);
    codes[i] = m[i].c;
    scales[i] = m[i].s;
    ts[i] = m[i].S;
  }
  float qn[32], kn[32], sinks[4];
  for (int i = 0; i < 32; ++i) qn[i] = kn[i] = 1.0f + 0.01f * (float)i;
  for (int i = 0; i < 4; ++i) sinks[i] = 0.5f * (float)i;
  const int64_t cap = 9;
  uint16_t* kc = calloc((size_t)(Hkv * cap * D), sizeof(uint16_t));
  uint16_t* vc = calloc((size_t)(Hkv * cap * D), sizeof(uint16_t));
  double* o = malloc(sizeof(double) * Hq * D);
  double* qkv = malloc(sizeof(double) * (Hq * D + 2 * Hkv * D));
  for (int64_t pos = 0; pos < 12; ++pos) /* the ring wraps past cap */
    CHECK(oracle_attn_decode(H, Hq, Hkv, D, 5, 1, 1e4, 1e-6, codes, scales, ts, qn, kn, sinks, u, pos, kc, vc,
                             cap, y, o, qkv, 2) == 0);
  memset(kc, 0, sizeof(uint16_t) * (size_t)(Hkv * cap * D));
  memset(vc, 0, sizeof(uint16_t) * (size_t)(Hkv * cap * D));
  for (int64_t pos = 0; pos < cap; ++pos)
    CHECK(oracle_attn_decode(H, Hq, Hkv, D, 0, 0, 1e4, 1e-6, codes, scales, ts, qn, kn, sinks, u, pos, kc, vc,
                             cap, y, NULL, NULL, 1) == 0);
  CHECK(oracle_attn_decode(H, Hq, Hkv, D, 0, 0, 1e4, 1e-6, codes, scales, ts, qn, kn, sinks, u, cap, kc, vc,
                           cap, y, NULL, NULL, 1) == -1); /* full context needs cap > pos */
  for (int i = 0; i < 4; ++i) {
    nv_free(m[i]);
    free(mw[i]);
  }
  free(kc);
  free(vc);
  free(o);
  free(qkv);
  nv_free(G);
  nv_free(U);
  nv_free(Dn);
  free(gw);
  free(uw);
  free(dw);
  free(u);
  free(y);
  free(hs);
}

static void int4(void) {
  const int64_t R = 70, C = 192;
  float* w = fill_f32(R * C, 2.0);
  for (int k = 64; k < 128; ++k) w[k] = 0.25f; /* a constant group: scale 0 */
  uint8_t* c = malloc((size_t)(R * C / 2));
  uint16_t* s = malloc(sizeof(uint16_t) * (size_t)(R * C / 64));
  uint16_t* b = malloc(sizeof(uint16_t) * (size_t)(R * C / 64));
  float* d = malloc(sizeof(float) * (size_t)(R * C));
  oracle_int4_quantize(w, R, C, c, s, b);
  oracle_int4_dequantize(c, s, b, R, C, d);
  for (int k = 64; k < 128; ++k) CHECK(d[k] == 0.25f);
  double* x = fill_f64(C, 1.0);
  double* y = malloc(sizeof(double) * R);
  oracle_int4_gemv(c, s, b, R, C, x, y, 3);
  for (int64_t r = 0; r < R; ++r) CHECK(isfinite(y[r]));
  free(w);
  free(c);
  free(s);
  free(b);
  free(d);
  free(x);
  free(y);
}

int main(void) {
  codecs();
  routing();
  bf16_and_norms();
  expert_and_attention();
  int4();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle driver: all checks passed\n");
  return 0;
}
