// synth_dev.hip -- the generator of synth.c, for filling device buffers.
//
// Same definition, same operations in the same order: Philox4x32-10 counter
// block i/4 keyed by (seed, stream), two Box-Muller pairs with the logarithm
// and sine/cosine written as the same short series, every floating-point
// step an IEEE +, -, *, / or sqrt in double precision, built with
// -ffp-contract=off.  Its output is compared bit-for-bit with the host
// generator by the tests.  Holds none of the NVFP4 method's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

__device__ __forceinline__ void box_muller(uint32_t ur, uint32_t ut, double mean, double sd, float* o) {
  double u = ((double)(int32_t)(ur ^ 0x80000000u) + 2147483648.5) * (1.0 / 4294967296.0);
  uint64_t bits = (uint64_t)__double_as_longlong(u);
  double e = (double)(int32_t)((bits >> 52) & 0x7FF) - 1023.0;
  double m = __longlong_as_double((long long)((bits & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull));
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
  double rad = __builtin_sqrt(-2.0 * ln);
  double w = ((double)(int32_t)(ut ^ 0x80000000u) + 2147483648.5) * (1.0 / 4294967296.0);
  w = w - (double)(w >= 0.5);
  double q4 = w * 4.0;
  double qd = (q4 + 6755399441055744.0) - 6755399441055744.0;
  double f = w - qd * 0.25;
  double a = f * 6.283185307179586477;
  double a2 = a * a;
  double sn = a - a * a2 * (1.0 / 6.0 - a2 * (1.0 / 120.0 - a2 * (1.0 / 5040.0 - a2 * (1.0 / 362880.0 - a2 * (1.0 / 39916800.0 - a2 / 6227020800.0)))));
  double cs = 1.0 - a2 * (0.5 - a2 * (1.0 / 24.0 - a2 * (1.0 / 720.0 - a2 * (1.0 / 40320.0 - a2 * (1.0 / 3628800.0 - a2 * (1.0 / 479001600.0 - a2 / 87178291200.0))))));
  double q0 = (double)(qd == 0.0), q1 = (double)(qd == 1.0), qm1 = (double)(qd == -1.0);
  double q2 = 1.0 - q0 - q1 - qm1;
  double co = cs * (q0 - q2) + sn * (qm1 - q1);
  double si = sn * (q0 - q2) + cs * (q1 - qm1);
  o[0] = (float)(mean + sd * (rad * co));
  o[1] = (float)(mean + sd * (rad * si));
}

// blockIdx.y selects stream `stream + blockIdx.y`, written at out + blockIdx.y * n
__global__ __launch_bounds__(256) void k_synth_normal(uint32_t seed, uint32_t stream0, uint64_t offset, int64_t n,
                                                      double mean, double sd, float* __restrict__ out0) {
  const uint32_t stream = stream0 + blockIdx.y;
  float* out = out0 + (size_t)blockIdx.y * (size_t)n;
  const uint64_t first_blk = offset >> 2;
  const uint64_t nblk = ((offset & 3) + (uint64_t)n + 3) >> 2;
  for (uint64_t t = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nblk; t += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t blk = first_blk + t;
    uint32_t c0 = (uint32_t)blk, c1 = (uint32_t)(blk >> 32), c2 = 0, c3 = 0;
    uint32_t k0 = seed, k1 = stream;
    for (int r = 0; r < 10; ++r) {
      const uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
      const uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
      const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
      const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
      c1 = (uint32_t)p1; c3 = (uint32_t)p0; c0 = n0; c2 = n2;
      k0 += PHILOX_W0; k1 += PHILOX_W1;
    }
    float z[4];
    box_muller(c0, c1, mean, sd, z);
    box_muller(c2, c3, mean, sd, z + 2);
#pragma unroll
    for (int lane = 0; lane < 4; ++lane) {
      const int64_t j = (int64_t)(blk * 4 + lane) - (int64_t)offset;
      if (j >= 0 && j < n) out[j] = z[lane];
    }
  }
}

// n_streams consecutive streams stream, stream+1, ... (e.g. the experts of one
// matrix kind), each n elements from `offset`, stored one after the other.
extern "C" int synth_dev_normal_f32(uint32_t seed, uint32_t stream, uint64_t offset, int64_t n, int32_t n_streams,
                                    float mean, float sd, float* out, void* hip_stream) {
  if (n <= 0 || n_streams <= 0) return 0;
  const uint64_t nblk = ((offset & 3) + (uint64_t)n + 3) >> 2;
  uint64_t g = (nblk + 255) / 256;
  if (g > 16384) g = 16384;
  for (int32_t s0 = 0; s0 < n_streams; s0 += 65535) {
    const int32_t ns = (n_streams - s0) < 65535 ? (n_streams - s0) : 65535;
    k_synth_normal<<<dim3((unsigned)g, (unsigned)ns), 256, 0, (hipStream_t)hip_stream>>>(
        seed, stream + (uint32_t)s0, offset, n, (double)mean, (double)sd, out + (size_t)s0 * (size_t)n);
    int e = (int)hipGetLastError();
    if (e) return e;
  }
  return 0;
}
