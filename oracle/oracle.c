/*
 * oracle.c -- plain, slow CPU reference for the NVFP4 sparse-MoE decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no source, header, table or helper with the HIP
 * path.  All arithmetic is double precision over the exactly defined fp32
 * dequantised weights, in the order the definitions below state.
 *
 * Sources (page titles as published; sections named):
 *  [P3] "Flint: 125 tokens a second is what 2.5B active parameters buy at
 *       273 GB/s" -- "The shape, read from the headers" (hidden 2,048; 256
 *       routed experts of width 512, 6 chosen per token, one shared expert of
 *       width 1,024; vocabulary 150,144; three matrices per expert), "Why
 *       active parameters set the speed" (4-bit output head, 1,024 B of codes
 *       per 2,048-wide row) and "Checking 125 tokens a second" (NVFP4 stores
 *       4-bit values with one 8-bit scale per 16 values).
 *  [P2] "Recursive Releases Flint, a 40B MoE Coding Model That Runs Locally at
 *       125 Tokens per Second" -- "How does Flint's architecture work?" (a
 *       router picks 6 of 256 experts, plus one always-active shared expert).
 *  [P1] "Flint-40B-A2B: AI-Built MoE Coding Model Hits 125 tok/s on MacBook
 *       Pro" -- "Quantization with Offline Distillation" (the output layer is
 *       NVFP4 too).
 * Where the pages leave a step open (the value encodings, the per-tensor
 * scale, rounding, the routing weights, the SwiGLU form, the norm) the
 * plainest reading is taken; each one is stated at the function that uses it.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- codec -- */

/* E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit; no Inf/NaN),
 * decoded from its bit fields: e = 0 is subnormal, m * 2^-1; otherwise
 * 2^(e-1) * (1 + m/2). */
double oracle_e2m1_value(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* OCP FP8 E4M3FN (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * Inf; S.1111.111 is NaN).  Normal 2^(e-7) (1 + m/8), subnormal 2^-6 (m/8). */
double oracle_e4m3_value(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* Round-to-nearest-even by exhaustive search over the representable
 * magnitudes: the nearest value wins; of two equally near, the one whose code
 * is even (last mantissa bit 0).  Beyond the largest magnitude the search
 * returns the largest, i.e. saturation. */
int oracle_e2m1_encode(double v) {
  double a = fabs(v);
  if (a >= 6.0) return 7 | (signbit(v) ? 8 : 0); /* saturate (distances to a huge |v| all round equal) */
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c < 8; ++c) {
    double d = fabs(oracle_e2m1_value(c) - a);
    if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) { bd = d; best = c; }
  }
  return best | (signbit(v) ? 8 : 0);
}

/* r >= 0 (a block scale); non-negative finite E4M3 codes 0x00..0x7E. */
int oracle_e4m3_encode(double r) {
  if (r >= 448.0) return 0x7E; /* saturate */
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double d = fabs(oracle_e4m3_value(c) - r);
    if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) { bd = d; best = c; }
  }
  return best;
}

/* ------------------------------------------------------------- quantise -- */

typedef struct {
  const float* w;
  int64_t cols, r0, r1;
  float S;
  uint8_t *codes, *scales;
} quant_job;

static void* quant_rows(void* p) {
  quant_job* j = (quant_job*)p;
  const int64_t cols = j->cols, nb = cols / 16;
  const double S = (double)j->S;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const float* blk = j->w + r * cols + b * 16;
      double bm = 0.0;
      for (int i = 0; i < 16; ++i) {
        double a = fabs((double)blk[i]);
        if (a > bm) bm = a;
      }
      int sc = oracle_e4m3_encode(bm / (6.0 * S));
      j->scales[r * nb + b] = (uint8_t)sc;
      double d = oracle_e4m3_value(sc);
      if (d == 0.0) continue;
      for (int i = 0; i < 16; ++i) {
        int c = oracle_e2m1_encode((double)blk[i] / (d * S));
        int64_t k = b * 16 + i;
        uint8_t* byte = &j->codes[r * (cols / 2) + k / 2];
        *byte |= (uint8_t)((k & 1) ? (c << 4) : c);
      }
    }
  }
  return NULL;
}

/* NVFP4 quantisation of one matrix W [rows][cols] (cols a multiple of 16;
 * blocks of 16 run along cols, the reduction axis) into
 *   codes  [rows][cols/2]  element 2j in the low nibble of byte j,
 *   scales [rows][cols/16] one E4M3 code per block,
 *   tscale               one fp32 per-tensor scale S.
 * [P3 "Checking 125 tokens a second": 4-bit values, one 8-bit scale per 16.]
 * Readings taken here: S = fl32(amax / (6 * 448)), so that the largest block
 * scale lands on E4M3's largest finite value; block scale = E4M3-RNE of
 * blockmax / (6 S); element code = E2M1-RNE of w / (d S); a block whose scale
 * decodes to 0 stores all-zero codes; all ratios in double. */
void oracle_nvfp4_quantize(const float* w, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                           float* tscale, int nthreads) {
  double amax = 0.0;
  for (int64_t i = 0; i < rows * cols; ++i) {
    double a = fabs((double)w[i]);
    if (a > amax) amax = a;
  }
  float S = (float)(amax / 2688.0);
  *tscale = S;
  memset(codes, 0, (size_t)(rows * cols / 2));
  memset(scales, 0, (size_t)(rows * (cols / 16)));
  if (S == 0.0f) return;
  /* rows are independent: splitting them over threads changes nothing */
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (rows < 64) nthreads = 1;
  quant_job jobs[64];
  pthread_t th[64];
  int64_t chunk = (rows + nthreads - 1) / nthreads;
  int used = 0;
  for (int t = 0; t < nthreads; ++t) {
    int64_t r0 = t * chunk, r1 = r0 + chunk < rows ? r0 + chunk : rows;
    if (r0 >= rows) break;
    jobs[t] = (quant_job){w, cols, r0, r1, S, codes, scales};
    used++;
  }
  if (used == 1) { quant_rows(&jobs[0]); return; }
  for (int t = 0; t < used; ++t) pthread_create(&th[t], NULL, quant_rows, &jobs[t]);
  for (int t = 0; t < used; ++t) pthread_join(th[t], NULL);
}

/* w = fl32((e2m1(c) * d) * S): c*d is exact, then one rounding to fp32. */
static inline float deq(const uint8_t* codes, const uint8_t* scales, float S, int64_t cols, int64_t r, int64_t k) {
  uint8_t byte = codes[r * (cols / 2) + k / 2];
  int c = (k & 1) ? (byte >> 4) : (byte & 15);
  double d = oracle_e4m3_value(scales[r * (cols / 16) + k / 16]);
  return (float)((oracle_e2m1_value(c) * d) * (double)S);
}

void oracle_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, float tscale, int64_t rows,
                             int64_t cols, float* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < cols; ++k) out[r * cols + k] = deq(codes, scales, tscale, cols, r, k);
}

/* ------------------------------------------------------------- products -- */

typedef struct {
  const uint8_t* codes;
  const uint8_t* scales;
  float S;
  const float* wf32; /* when non-NULL: an unquantised fp32 matrix */
  int64_t rows, cols, r0, r1;
  const double* x;
  double* y;
} gemv_job;

static void* gemv_rows(void* p) {
  gemv_job* j = (gemv_job*)p;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    double acc = 0.0;
    if (j->wf32) {
      for (int64_t k = 0; k < j->cols; ++k) acc += (double)j->wf32[r * j->cols + k] * j->x[k];
    } else {
      for (int64_t k = 0; k < j->cols; ++k) acc += (double)deq(j->codes, j->scales, j->S, j->cols, r, k) * j->x[k];
    }
    j->y[r] = acc;
  }
  return NULL;
}

static void gemv_any(const uint8_t* codes, const uint8_t* scales, float S, const float* wf32, int64_t rows,
                     int64_t cols, const double* x, double* y, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (rows < 64) nthreads = 1;
  gemv_job jobs[64];
  pthread_t th[64];
  int64_t chunk = (rows + nthreads - 1) / nthreads;
  int used = 0;
  for (int t = 0; t < nthreads; ++t) {
    int64_t r0 = t * chunk, r1 = r0 + chunk < rows ? r0 + chunk : rows;
    if (r0 >= rows) break;
    jobs[t] = (gemv_job){codes, scales, S, wf32, rows, cols, r0, r1, x, y};
    used++;
  }
  if (used == 1) { gemv_rows(&jobs[0]); return; }
  for (int t = 0; t < used; ++t) pthread_create(&th[t], NULL, gemv_rows, &jobs[t]);
  for (int t = 0; t < used; ++t) pthread_join(th[t], NULL);
}

/* y = deq(W) x in double; each row's sum runs k = 0..cols-1 in order, so the
 * result does not depend on the thread count. */
void oracle_nvfp4_gemv(const uint8_t* codes, const uint8_t* scales, float tscale, int64_t rows, int64_t cols,
                       const double* x, double* y, int nthreads) {
  gemv_any(codes, scales, tscale, NULL, rows, cols, x, y, nthreads);
}

/* y = W x for an unquantised fp32 matrix (the router). */
void oracle_f32_gemv(const float* w, int64_t rows, int64_t cols, const double* x, double* y, int nthreads) {
  gemv_any(NULL, NULL, 0.0f, w, rows, cols, x, y, nthreads);
}

/* -------------------------------------------------------------- routing -- */

static const double* g_sort_keys;
static int by_logit_desc_then_index(const void* a, const void* b) {
  int i = *(const int*)a, j = *(const int*)b;
  double li = g_sort_keys[i], lj = g_sort_keys[j];
  if (li > lj) return -1;
  if (li < lj) return 1;
  return (i > j) - (i < j);
}

/* Top-k routing [P2 "How does Flint's architecture work?": the router selects
 * 6 experts per token].  Selection: full sort by (logit descending, index
 * ascending), first k.  Weights (reading): softmax over all E logits, then
 * renormalised over the chosen k.  gap = k-th minus (k+1)-th largest logit
 * (INFINITY when E == k).  Not thread-safe (uses a static sort key). */
void oracle_topk_softmax(const double* logits, int E, int k, int32_t* idx, double* w, double* gap) {
  int* order = (int*)malloc(sizeof(int) * (size_t)E);
  for (int e = 0; e < E; ++e) order[e] = e;
  g_sort_keys = logits;
  qsort(order, (size_t)E, sizeof(int), by_logit_desc_then_index);
  double mx = logits[order[0]];
  double z = 0.0;
  for (int e = 0; e < E; ++e) z += exp(logits[e] - mx);
  double sel = 0.0;
  for (int i = 0; i < k; ++i) sel += exp(logits[order[i]] - mx) / z;
  for (int i = 0; i < k; ++i) {
    idx[i] = order[i];
    w[i] = (exp(logits[order[i]] - mx) / z) / sel;
  }
  *gap = (E > k) ? logits[order[k - 1]] - logits[order[k]] : INFINITY;
  free(order);
}

/* Sigmoid routing [P3 "Flint: 125 tokens a second is what 2.5B active
 * parameters buy at 273 GB/s", "The shape, read from the headers": the router
 * scores experts with a sigmoid, as DeepSeek-V3 does, and has no
 * bias-correction tensor].  Reading: score s_e = 1 / (1 + e^-l_e); the k
 * largest scores are chosen, ties to the lower index; the weights are the
 * chosen scores divided by their sum, with no further scaling factor.
 * gap = k-th minus (k+1)-th largest logit, in the chosen order (INFINITY when
 * E == k).  Not thread-safe (uses a static sort key). */
void oracle_topk_sigmoid(const double* logits, int E, int k, int32_t* idx, double* w, double* gap) {
  double* score = (double*)malloc(sizeof(double) * (size_t)E);
  int* order = (int*)malloc(sizeof(int) * (size_t)E);
  for (int e = 0; e < E; ++e) {
    score[e] = 1.0 / (1.0 + exp(-logits[e]));
    order[e] = e;
  }
  g_sort_keys = score;
  qsort(order, (size_t)E, sizeof(int), by_logit_desc_then_index);
  double sel = 0.0;
  for (int i = 0; i < k; ++i) sel += score[order[i]];
  for (int i = 0; i < k; ++i) {
    idx[i] = order[i];
    w[i] = score[order[i]] / sel;
  }
  *gap = (E > k) ? logits[order[k - 1]] - logits[order[k]] : INFINITY;
  free(order);
  free(score);
}

/* BF16 values [same page and section: the router is stored in BF16].  The
 * format: bit 15 the sign, bits 14..7 a biased exponent (bias 127), bits 6..0
 * the fraction; exponent 0 is subnormal (fraction / 128 * 2^-126).  Exponent
 * 255 (infinities, NaN) is outside the inputs and decodes to NaN. */
void oracle_bf16_decode(const uint16_t* b, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) {
    int sign = b[i] >> 15, ex = (b[i] >> 7) & 0xFF, fr = b[i] & 0x7F;
    double v;
    if (ex == 0)
      v = ldexp(fr / 128.0, -126);
    else if (ex == 255)
      v = NAN;
    else
      v = ldexp(1.0 + fr / 128.0, ex - 127);
    out[i] = sign ? -v : v;
  }
}

/* RMSNorm scale with unit gain (reading: eps inside the root):
 * 1 / sqrt(mean(h^2) + eps). */
double oracle_rms_inv(const double* h, int64_t n, double eps) {
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += h[i] * h[i];
  return 1.0 / sqrt(s / (double)n + eps);
}

/* --------------------------------------------------------------- expert -- */

/* One SwiGLU expert [P3 "The shape, read from the headers": three matrices
 * per expert].  Reading: the first matrix (gate) goes through SiLU, the
 * second (up) is linear, the third (down) maps back to the hidden size:
 *   g = Wg u, a = Wu u, h = g / (1 + e^-g) * a, y = Wd h.
 * Wg, Wu are [I][H]; Wd is [H][I]; all NVFP4. */
void oracle_swiglu_expert(const uint8_t* gc, const uint8_t* gs, float gS, const uint8_t* uc, const uint8_t* us,
                          float uS, const uint8_t* dc, const uint8_t* ds, float dS, int64_t H, int64_t I,
                          const double* u, double* y, double* h_out, int nthreads) {
  double* g = (double*)malloc(sizeof(double) * (size_t)I);
  double* a = (double*)malloc(sizeof(double) * (size_t)I);
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  oracle_nvfp4_gemv(gc, gs, gS, I, H, u, g, nthreads);
  oracle_nvfp4_gemv(uc, us, uS, I, H, u, a, nthreads);
  for (int64_t i = 0; i < I; ++i) h[i] = g[i] / (1.0 + exp(-g[i])) * a[i];
  oracle_nvfp4_gemv(dc, ds, dS, H, I, h, y, nthreads);
  if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)I);
  free(g);
  free(a);
  free(h);
}

/* --------------------------------------------------------------- argmax -- */

/* First index of the largest value; gap = largest minus second largest. */
int64_t oracle_argmax(const double* v, int64_t n, double* gap) {
  int64_t best = 0;
  for (int64_t i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  double second = -INFINITY;
  for (int64_t i = 0; i < n; ++i)
    if (i != best && v[i] > second) second = v[i];
  if (gap) *gap = v[best] - second;
  return best;
}

/* ------------------------------------------------------------ attention -- */

/* BF16 encoding of a finite double: the nearest value with 8 significant
 * bits, ties to the even fraction; below 2^-126 the step is 2^-133
 * (subnormals); values past the largest finite BF16 saturate to infinity.
 * Written from the format (sign, 8-bit exponent with bias 127, 7-bit
 * fraction), one rounding from the exact double. */
uint16_t oracle_bf16_encode(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e); /* a = m * 2^e with m in [0.5, 1) */
  int ex = e - 1; /* a in [2^ex, 2^(ex+1)) */
  if (ex < -126) ex = -126;
  double q = ldexp(1.0, ex - 7); /* spacing of BF16 values near a */
  double n = a / q;              /* exact: a power-of-two division */
  double r = floor(n);
  double f = n - r;
  if (f > 0.5 || (f == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  double val = r * q;
  if (val >= ldexp(1.0, 128)) return sign | 0x7F80;
  int e2;
  frexp(val, &e2);
  if (val < ldexp(1.0, -126)) return sign | (uint16_t)r; /* subnormal: fraction = r */
  int bexp = e2 - 1 + 127;
  uint16_t frac = (uint16_t)(ldexp(val, -(e2 - 1)) * 128.0 - 128.0);
  return sign | (uint16_t)(bexp << 7) | frac;
}

void oracle_bf16_round(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_encode(x[i]);
}

/* Per-head RMSNorm [P3 "The shape, read from the headers": every layer
 * normalises each query and key head].  Reading: over the head's D values,
 * v_i <- v_i * g_i / sqrt(mean(v^2) + eps), one gain vector g of length D
 * shared by the heads of q (and one by the heads of k). */
void oracle_head_rmsnorm(double* v, int D, const float* g, double eps) {
  double s = 0.0;
  for (int i = 0; i < D; ++i) s += v[i] * v[i];
  double r = 1.0 / sqrt(s / D + eps);
  for (int i = 0; i < D; ++i) v[i] = v[i] * r * (double)g[i];
}

/* Rotary position embedding [same section: the sliding-window layers use
 * RoPE].  Reading: the pages give no base or pairing; the rotation pairs
 * element i with element i + D/2 (i < D/2) and turns the pair by the angle
 * pos * theta^(-2i/D):  (a, b) -> (a cos - b sin, a sin + b cos). */
void oracle_rope(double* v, int D, int64_t pos, double theta) {
  int h = D / 2;
  for (int i = 0; i < h; ++i) {
    double ang = (double)pos * pow(theta, -2.0 * i / D);
    double c = cos(ang), s = sin(ang);
    double a = v[i], b = v[i + h];
    v[i] = a * c - b * s;
    v[i + h] = a * s + b * c;
  }
}

/* Attention over the cache for one query head [same section: grouped-query
 * attention, 32 query heads over 4 key/value heads of dimension 128;
 * sliding-window layers see the current token and 512 before it, the other
 * layers the whole context; learned per-head sinks].  Reading of the sink: a
 * logit that joins the softmax's normaliser and carries no value.
 *   s_t = q . K_t / sqrt(D) for t in [first, pos]
 *   M = max(max_t s_t, sink);  Z = sum_t e^(s_t - M) + e^(sink - M)
 *   o = sum_t e^(s_t - M) / Z * V_t
 * K_t and V_t are the BF16 cache rows at slot t mod cap. */
static void attend_head(const double* q, int D, const uint16_t* kc, const uint16_t* vc, int64_t cap, int64_t first,
                        int64_t pos, double sink, double* o) {
  int64_t n = pos - first + 1;
  double* s = (double*)malloc(sizeof(double) * (size_t)n);
  double* row = (double*)malloc(sizeof(double) * (size_t)D);
  double M = sink;
  for (int64_t t = first; t <= pos; ++t) {
    oracle_bf16_decode(kc + (t % cap) * D, D, row);
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += q[d] * row[d];
    s[t - first] = acc / sqrt((double)D);
    if (s[t - first] > M) M = s[t - first];
  }
  double Z = exp(sink - M);
  for (int64_t i = 0; i < n; ++i) Z += exp(s[i] - M);
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  for (int64_t t = first; t <= pos; ++t) {
    double p = exp(s[t - first] - M) / Z;
    oracle_bf16_decode(vc + (t % cap) * D, D, row);
    for (int d = 0; d < D; ++d) o[d] += p * row[d];
  }
  free(row);
  free(s);
}

/* One attention layer for one new token at position pos (no norm before it,
 * no residual after it):
 *   q = Wq x, k = Wk x, v = Wv x           (NVFP4 [Hq*D][H], [Hkv*D][H] x2)
 *   per-head RMSNorm of q and k (gains qn, kn), then RoPE at pos if rope
 *   K[g][pos mod cap] = bf16(k_g), V[g][pos mod cap] = bf16(v_g)
 *   o_h = attention of q_h over kv head g = h / (Hq/Hkv), positions
 *         max(0, pos-window+1)..pos (window > 0) or 0..pos (window == 0)
 *   y = Wo o                                (NVFP4 [H][Hq*D])
 * mats[0..3] = q, k, v, o: codes, scales and tensor scale of each.  The
 * caches are uint16 [Hkv][cap][D] and are updated in place.  cap must be at
 * least `window` (window > 0) or greater than pos (window == 0); returns -1
 * otherwise.  o_out (Hq*D) and qkv_out (Hq*D + 2*Hkv*D: q, k after norm and
 * rotation, then v) are optional. */
int oracle_attn_decode(int H, int Hq, int Hkv, int D, int window, int rope, double theta, double eps,
                       const uint8_t* const* codes, const uint8_t* const* scales, const float* tscales,
                       const float* qn, const float* kn, const float* sinks, const double* x, int64_t pos,
                       uint16_t* kc, uint16_t* vc, int64_t cap, double* y, double* o_out, double* qkv_out,
                       int nthreads) {
  if (Hq % Hkv || D % 2 || pos < 0) return -1;
  if (window > 0 ? cap < window : cap <= pos) return -1;
  int nq = Hq * D, nk = Hkv * D;
  double* q = (double*)malloc(sizeof(double) * (size_t)nq);
  double* k = (double*)malloc(sizeof(double) * (size_t)nk);
  double* v = (double*)malloc(sizeof(double) * (size_t)nk);
  double* o = (double*)malloc(sizeof(double) * (size_t)nq);
  oracle_nvfp4_gemv(codes[0], scales[0], tscales[0], nq, H, x, q, nthreads);
  oracle_nvfp4_gemv(codes[1], scales[1], tscales[1], nk, H, x, k, nthreads);
  oracle_nvfp4_gemv(codes[2], scales[2], tscales[2], nk, H, x, v, nthreads);
  for (int h = 0; h < Hq; ++h) {
    oracle_head_rmsnorm(q + h * D, D, qn, eps);
    if (rope) oracle_rope(q + h * D, D, pos, theta);
  }
  for (int g = 0; g < Hkv; ++g) {
    oracle_head_rmsnorm(k + g * D, D, kn, eps);
    if (rope) oracle_rope(k + g * D, D, pos, theta);
    oracle_bf16_round(k + g * D, D, kc + ((int64_t)g * cap + pos % cap) * D);
    oracle_bf16_round(v + g * D, D, vc + ((int64_t)g * cap + pos % cap) * D);
  }
  int64_t first = (window > 0 && pos - window + 1 > 0) ? pos - window + 1 : 0;
  int group = Hq / Hkv;
  for (int h = 0; h < Hq; ++h) {
    int g = h / group;
    attend_head(q + h * D, D, kc + (int64_t)g * cap * D, vc + (int64_t)g * cap * D, cap, first, pos,
                (double)sinks[h], o + h * D);
  }
  oracle_nvfp4_gemv(codes[3], scales[3], tscales[3], H, nq, o, y, nthreads);
  if (o_out) memcpy(o_out, o, sizeof(double) * (size_t)nq);
  if (qkv_out) {
    memcpy(qkv_out, q, sizeof(double) * (size_t)nq);
    memcpy(qkv_out + nq, k, sizeof(double) * (size_t)nk);
    memcpy(qkv_out + nq + nk, v, sizeof(double) * (size_t)nk);
  }
  free(q);
  free(k);
  free(v);
  free(o);
  return 0;
}

/* ------------------------------------------------------ INT4 affine codec -- */

/* Group-64 affine INT4 [P3 "Why active parameters set the speed": Recursive's
 * Apple build stores each group of 64 weights as 4-bit codes plus a BF16
 * scale and a BF16 offset, 4.5 bits per weight].  Reading (min-max affine
 * quantisation, the pages give no rule): for each group of 64 consecutive
 * values along a row, in fp32 arithmetic,
 *   scale  s = bf16(fl32((max - min) / 15)),  offset b = bf16(min),
 *   code   q = clamp(rint(fl32(fl32(w - b) / s)), 0, 15), or 0 when s == 0,
 * with BF16 rounding to nearest even and rint ties to even.  Codes are packed
 * two per byte, element 2j in the low nibble of byte j.  The decisions are
 * taken in fp32, the precision the device quantiser uses. */
void oracle_int4_quantize(const float* w, int64_t rows, int64_t cols, uint8_t* codes, uint16_t* scales,
                          uint16_t* biases) {
  int64_t groups = cols / 64;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t g = 0; g < groups; ++g) {
      const float* v = w + r * cols + g * 64;
      float lo = v[0], hi = v[0];
      for (int i = 1; i < 64; ++i) {
        if (v[i] < lo) lo = v[i];
        if (v[i] > hi) hi = v[i];
      }
      float range = hi - lo;
      float sf = range / 15.0f;
      uint16_t sb = oracle_bf16_encode((double)sf), bb = oracle_bf16_encode((double)lo);
      double sv, bv;
      oracle_bf16_decode(&sb, 1, &sv);
      oracle_bf16_decode(&bb, 1, &bv);
      scales[r * groups + g] = sb;
      biases[r * groups + g] = bb;
      for (int i = 0; i < 64; ++i) {
        int q = 0;
        if (sv != 0.0) {
          float t = (v[i] - (float)bv) / (float)sv;
          float rq = rintf(t);
          q = rq < 0.0f ? 0 : rq > 15.0f ? 15 : (int)rq;
        }
        int64_t k = g * 64 + i;
        uint8_t* byte = codes + r * (cols / 2) + k / 2;
        if (k % 2 == 0)
          *byte = (uint8_t)((*byte & 0xF0) | q);
        else
          *byte = (uint8_t)((*byte & 0x0F) | (q << 4));
      }
    }
  }
}

/* Dequantised value fl32(s * q + b): s * q is exact, the sum rounds once. */
void oracle_int4_dequantize(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t rows,
                            int64_t cols, float* out) {
  int64_t groups = cols / 64;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t g = 0; g < groups; ++g) {
      double s, b;
      oracle_bf16_decode(&scales[r * groups + g], 1, &s);
      oracle_bf16_decode(&biases[r * groups + g], 1, &b);
      for (int64_t k = g * 64; k < g * 64 + 64; ++k) {
        uint8_t byte = codes[r * (cols / 2) + k / 2];
        int q = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
        out[r * cols + k] = (float)(s * q + b);
      }
    }
}

/* y = W x over the dequantised INT4 matrix, double accumulation. */
void oracle_int4_gemv(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t rows,
                      int64_t cols, const double* x, double* y, int nthreads) {
  float* row = (float*)malloc(sizeof(float) * (size_t)cols);
  (void)nthreads;
  for (int64_t r = 0; r < rows; ++r) {
    oracle_int4_dequantize(codes + r * (cols / 2), scales + r * (cols / 64), biases + r * (cols / 64), 1, cols, row);
    double acc = 0.0;
    for (int64_t k = 0; k < cols; ++k) acc += (double)row[k] * x[k];
    y[r] = acc;
  }
  free(row);
}

/* ------------------------------------------------------- prefill GEMM ---- */

/* Prompt processing [P1 "Flint-40B-A2B: AI-Built MoE Coding Model Hits 125
 * tok/s on MacBook Pro", "Custom Inference Kernels": kernels for prompt
 * processing; P2 "How did the Eureka Machine build Flint?": kernels for
 * low-bit projections and prompt processing].  T tokens at once through one
 * NVFP4 matrix W [N][K]:
 *   Y[t][n] = sum_k deq(W)[n][k] * X[t][k]        (X at full precision),
 * which is the decode GEMV once per token. */
void oracle_nvfp4_gemm(const uint8_t* codes, const uint8_t* scales, float tscale, int64_t N, int64_t K,
                       const double* X, int64_t T, double* Y, int nthreads) {
  for (int64_t t = 0; t < T; ++t) oracle_nvfp4_gemv(codes, scales, tscale, N, K, X + t * K, Y + t * N, nthreads);
}

/* The A4 variant: the activations are quantised with the same NVFP4 codec
 * first (reading: X [T][K] is one tensor, so one fp32 scale over all of it;
 * E4M3 block scales per 16 values along K), then multiplied exactly:
 *   Y[t][n] = sum_k deq(W)[n][k] * deq(Xq)[t][k]. */
void oracle_nvfp4_gemm_a4(const uint8_t* codes, const uint8_t* scales, float tscale, int64_t N, int64_t K,
                          const float* X, int64_t T, double* Y, int nthreads) {
  uint8_t* xc = (uint8_t*)malloc((size_t)(T * K / 2));
  uint8_t* xs = (uint8_t*)malloc((size_t)(T * K / 16));
  float* xd = (float*)malloc(sizeof(float) * (size_t)(T * K));
  double* xv = (double*)malloc(sizeof(double) * (size_t)(T * K));
  float xS;
  oracle_nvfp4_quantize(X, T, K, xc, xs, &xS, nthreads);
  oracle_nvfp4_dequantize(xc, xs, xS, T, K, xd);
  for (int64_t i = 0; i < T * K; ++i) xv[i] = (double)xd[i];
  oracle_nvfp4_gemm(codes, scales, tscale, N, K, xv, T, Y, nthreads);
  free(xc);
  free(xs);
  free(xd);
  free(xv);
}
