/*
 * synth.c -- seeded synthetic inputs shared by the product's tests/benchmark
 * and by the CPU oracle.  It holds none of the NVFP4 method's arithmetic: it
 * only draws Gaussian numbers.
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), a counter-based generator.  Element i
 * of stream (seed, stream) uses counter block (i/4, i>>34 ... ) with key
 * (seed, stream); the four 32-bit words feed two Box-Muller pairs
 * (Box & Muller 1958), so element i is fully determined by (seed, stream, i).
 *
 * Every floating-point step is an IEEE-754 +, -, *, / or sqrt on doubles, built
 * with -ffp-contract=off; the logarithm and the sine/cosine are short series
 * written out here rather than taken from the host libm.  The output is
 * therefore bit-identical on every x86-64 host, whatever its libm or vector
 * width.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>
#include <unistd.h>
#include <math.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += PHILOX_W0; k1 += PHILOX_W1;
  }
}

/* exported for the known-answer test of the generator itself */
void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  philox4x32_10(c, key[0], key[1]);
  memcpy(out, c, sizeof c);
}

/* Branch-free versions of the transforms above over a batch of counter
 * blocks, so that the compiler can vectorise them; same operations, same
 * order, hence the same bits. */
#define NB 16
static void bm_pairs(const uint32_t* ur, const uint32_t* ut, double mean, double sd, float* out);
static void gen_blocks(uint32_t seed, uint32_t stream, uint64_t blk0, double mean, double sd, float* out /*[4*NB]*/) {
  uint32_t c0[NB], c1[NB], c2[NB], c3[NB];
  for (int i = 0; i < NB; ++i) {
    uint64_t b = blk0 + (uint64_t)i;
    c0[i] = (uint32_t)b; c1[i] = (uint32_t)(b >> 32); c2[i] = 0; c3[i] = 0;
  }
  uint32_t k0 = seed, k1 = stream;
  for (int r = 0; r < 10; ++r) {
    for (int i = 0; i < NB; ++i) {
      uint64_t p0 = (uint64_t)PHILOX_M0 * c0[i];
      uint64_t p1 = (uint64_t)PHILOX_M1 * c2[i];
      uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1[i] ^ k0;
      uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3[i] ^ k1;
      c1[i] = (uint32_t)p1; c3[i] = (uint32_t)p0; c0[i] = n0; c2[i] = n2;
    }
    k0 += PHILOX_W0; k1 += PHILOX_W1;
  }
  bm_pairs(c0, c1, mean, sd, out);
  bm_pairs(c2, c3, mean, sd, out + 2);
}

/* Box-Muller on NB (radius word, angle word) pairs; writes out[4*i], out[4*i+1] */
static void bm_pairs(const uint32_t* ur, const uint32_t* ut, double mean, double sd, float* out) {
  {
    for (int i = 0; i < NB; ++i) {
      /* radius: sqrt(-2 ln u), u = m * 2^e, m in [sqrt(1/2), sqrt(2)),
       * ln m = 2 atanh(t), t = (m-1)/(m+1), |t| <= 0.1716 */
      double u = ((double)(int32_t)(ur[i] ^ 0x80000000u) + 2147483648.5) * (1.0 / 4294967296.0);
      union { double d; uint64_t b; } v = {u};
      double e = (double)(int32_t)((v.b >> 52) & 0x7FF) - 1023.0;
      v.b = (v.b & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull;
      double m = v.d;
      double big = (double)(m > 1.4142135623730951);
      m = m * (1.0 - 0.5 * big);
      e = e + big;
      double t = (m - 1.0) / (m + 1.0);
      double t2 = t * t;
      double s = 1.0 / 15.0;
      s = s * t2 + 1.0 / 13.0;
      s = s * t2 + 1.0 / 11.0;
      s = s * t2 + 1.0 / 9.0;
      s = s * t2 + 1.0 / 7.0;
      s = s * t2 + 1.0 / 5.0;
      s = s * t2 + 1.0 / 3.0;
      s = s * t2 + 1.0;
      double ln = e * 0.6931471805599453094 + 2.0 * t * s;
      double rad = sqrt(-2.0 * ln);
      /* angle: cos/sin of 2 pi w, reduced to the nearest quarter turn (the
       * rounding uses the 1.5*2^52 constant, i.e. round-half-even) and
       * Taylor series on |a| <= pi/4 */
      double w = ((double)(int32_t)(ut[i] ^ 0x80000000u) + 2147483648.5) * (1.0 / 4294967296.0);
      w = w - (double)(w >= 0.5);
      double q4 = w * 4.0;
      double qd = (q4 + 6755399441055744.0) - 6755399441055744.0;
      double f = w - qd * 0.25;
      double a = f * 6.283185307179586477;
      double a2 = a * a;
      double sn = a - a * a2 * (1.0 / 6.0 - a2 * (1.0 / 120.0 - a2 * (1.0 / 5040.0 - a2 * (1.0 / 362880.0 - a2 * (1.0 / 39916800.0 - a2 / 6227020800.0)))));
      double cs = 1.0 - a2 * (0.5 - a2 * (1.0 / 24.0 - a2 * (1.0 / 720.0 - a2 * (1.0 / 40320.0 - a2 * (1.0 / 3628800.0 - a2 * (1.0 / 479001600.0 - a2 / 87178291200.0))))));
      /* rotate by qd quarter turns (qd in -2..2); factors are 0 or +-1, so exact */
      double q0 = (double)(qd == 0.0), q1 = (double)(qd == 1.0), qm1 = (double)(qd == -1.0);
      double q2 = 1.0 - q0 - q1 - qm1;
      double co = cs * (q0 - q2) + sn * (qm1 - q1);
      double si = sn * (q0 - q2) + cs * (q1 - qm1);
      out[4 * i] = (float)(mean + sd * (rad * co));
      out[4 * i + 1] = (float)(mean + sd * (rad * si));
    }
  }
}

/* fill out[j] = mean + std * z(offset + j), j in [0, n) */
static void fill_range(uint32_t seed, uint32_t stream, uint64_t offset, int64_t n, double mean, double sd, float* out) {
  float buf[4 * NB];
  int64_t j = 0;
  while (j < n) {
    uint64_t idx = offset + (uint64_t)j;
    uint64_t blk = idx >> 2;
    int lane0 = (int)(idx & 3);
    if (lane0 == 0 && n - j >= 4 * NB) {
      gen_blocks(seed, stream, blk, mean, sd, out + j);
      j += 4 * NB;
      continue;
    }
    gen_blocks(seed, stream, blk, mean, sd, buf);
    for (int l = lane0; l < 4 * NB && j < n; ++l, ++j) out[j] = buf[l];
  }
}

typedef struct {
  uint32_t seed, stream;
  uint64_t offset;
  int64_t n;
  double mean, sd;
  float* out;
} job_t;

static void* worker(void* p) {
  job_t* jb = (job_t*)p;
  fill_range(jb->seed, jb->stream, jb->offset, jb->n, jb->mean, jb->sd, jb->out);
  return NULL;
}

static int pick_threads(int nthreads, int64_t n) {
  if (nthreads <= 0) {
    const char* e = getenv("SYNTH_THREADS");
    nthreads = e ? atoi(e) : (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads > 16) nthreads = 16;
  }
  if (nthreads < 1) nthreads = 1;
  int64_t maxt = n / 65536 + 1;
  if (nthreads > maxt) nthreads = (int)maxt;
  if (nthreads > 64) nthreads = 64;
  return nthreads;
}

/* out[j] = mean + std * N(0,1) element (offset + j) of stream (seed, stream).
 * The result does not depend on nthreads (0 = choose automatically). */
void synth_normal_f32(uint32_t seed, uint32_t stream, uint64_t offset, int64_t n, float mean, float sd,
                      float* out, int nthreads) {
  if (n <= 0) return;
  int t = pick_threads(nthreads, n);
  if (t == 1) { fill_range(seed, stream, offset, n, mean, sd, out); return; }
  pthread_t th[64];
  job_t jobs[64];
  int64_t chunk = (n + t - 1) / t;
  chunk = (chunk + 3) & ~(int64_t)3;
  int used = 0;
  for (int i = 0; i < t; ++i) {
    int64_t b = (int64_t)i * chunk;
    if (b >= n) break;
    int64_t e = b + chunk < n ? b + chunk : n;
    jobs[i] = (job_t){seed, stream, offset + (uint64_t)b, e - b, mean, sd, out + b};
    pthread_create(&th[i], NULL, worker, &jobs[i]);
    used++;
  }
  for (int i = 0; i < used; ++i) pthread_join(th[i], NULL);
}
