// int4.hip -- group-64 affine INT4 (BF16 scale and offset per 64 values) on
// gfx950: quantiser, dequantiser and a GEMV with argmax, the same streaming
// GEMV as the NVFP4 path with another decode.
//
// Format [P3 "Flint: 125 tokens a second is what 2.5B active parameters buy
// at 273 GB/s", "Why active parameters set the speed": 4-bit codes per
// weight plus a BF16 scale and a BF16 offset per group of 64, 4.5 bits per
// weight; the 4-bit output head holds 1,024 code bytes per 2,048-wide row].
// A row of 2,048 values is 1,024 code bytes + 64 scale bytes + 64 offset
// bytes: the same 1,152 bytes as NVFP4, read once per token with 128-bit
// loads.
#include <float.h>
#include <limits.h>

#include "../../include/flint_int4.h"
#include "flint_common.h"
#include "flint_device.h"

namespace flint {
namespace {

constexpr int kChunk = 2048;       // one pass of 64 lanes x 32 values
constexpr int kI4Blocks = 1024;    // GEMV workgroups (argmax partials per token)
constexpr int kI4MaxB = 64;

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {  // finite f
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_value(uint32_t bits) { return __uint_as_float(bits << 16); }

// One thread per group of 64: min, max, BF16 scale and offset, 32 code bytes.
__global__ __launch_bounds__(256) void k_int4_quant(const float* __restrict__ w, long long groups,
                                                    uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                    uint16_t* __restrict__ biases) {
  for (long long gi = blockIdx.x * 256ll + threadIdx.x; gi < groups; gi += (long long)gridDim.x * 256) {
    const float4* v4 = reinterpret_cast<const float4*>(w + gi * 64);
    float v[64];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 t = v4[i];
      v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
    float lo = v[0], hi = v[0];
#pragma unroll
    for (int i = 1; i < 64; ++i) {
      lo = v[i] < lo ? v[i] : lo;
      hi = v[i] > hi ? v[i] : hi;
    }
    const uint32_t sb = bf16_bits_rne(__fdiv_rn(hi - lo, 15.0f)), bb = bf16_bits_rne(lo);
    const float sv = bf16_value(sb), bv = bf16_value(bb);
    uint32_t packed[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t q = 0;
        if (sv != 0.0f) {
          const float r = rintf(__fdiv_rn(v[8 * j + e] - bv, sv));
          q = r < 0.0f ? 0u : r > 15.0f ? 15u : (uint32_t)r;
        }
        word |= q << (4 * e);
      }
      packed[j] = word;
    }
    uint4* c4 = reinterpret_cast<uint4*>(codes + gi * 32);
    c4[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    c4[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    scales[gi] = (uint16_t)sb;
    biases[gi] = (uint16_t)bb;
  }
}

// One thread per code byte: two values fl32(s q + b).
__global__ __launch_bounds__(256) void k_int4_dequant(const uint8_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint16_t* __restrict__ biases, long long nbytes,
                                                      float* __restrict__ out) {
  for (long long i = blockIdx.x * 256ll + threadIdx.x; i < nbytes; i += (long long)gridDim.x * 256) {
    const long long g = i / 32;  // 32 code bytes per group
    const float s = bf16_value(scales[g]), b = bf16_value(biases[g]);
    const uint32_t c = codes[i];
    out[2 * i] = __builtin_fmaf(s, (float)(c & 15u), b);
    out[2 * i + 1] = __builtin_fmaf(s, (float)(c >> 4), b);
  }
}

// sum q_j x_j over the 8 codes of one word (element 2i in the low nibble of
// byte i): the low nibbles are elements 0, 2, 4, 6, the high ones 1, 3, 5, 7
__device__ __forceinline__ float ubyte(uint32_t w, int i) { return (float)((w >> (8 * i)) & 0xFFu); }
__device__ __forceinline__ float int4x8_dot(uint32_t w, const float* x, float acc) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  acc = __builtin_fmaf(ubyte(lo, 0), x[0], acc);
  acc = __builtin_fmaf(ubyte(hi, 0), x[1], acc);
  acc = __builtin_fmaf(ubyte(lo, 1), x[2], acc);
  acc = __builtin_fmaf(ubyte(hi, 1), x[3], acc);
  acc = __builtin_fmaf(ubyte(lo, 2), x[4], acc);
  acc = __builtin_fmaf(ubyte(hi, 2), x[5], acc);
  acc = __builtin_fmaf(ubyte(lo, 3), x[6], acc);
  acc = __builtin_fmaf(ubyte(hi, 3), x[7], acc);
  return acc;
}

struct I4Partial {
  float value;
  int32_t index;
};

// y[b][r] = W[r] . x_b.  Lane l holds x[i*2048 + 32l .. +31] (i < KI) and
// their sum per pass; its 32 values share one group (lanes 2g and 2g+1 read
// group g's scale and offset).  R rows per wave step; waves stride over the
// rows, keeping the best (value, index); with `partials` each workgroup
// writes its best for k_i4_argmax.
template <int KI, int R>
__global__ __launch_bounds__(256) void k_int4_gemv(flint_int4 W, int rows, const float* __restrict__ x,
                                                   float* __restrict__ y, I4Partial* __restrict__ partials) {
  constexpr int K = KI * kChunk;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, b = blockIdx.y;
  float xv[KI * 32], xs[KI];
  const float* xb = x + (size_t)b * K;
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    float t = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(xb + i * kChunk + 32 * lane + 4 * q);
      xv[32 * i + 4 * q + 0] = v.x;
      xv[32 * i + 4 * q + 1] = v.y;
      xv[32 * i + 4 * q + 2] = v.z;
      xv[32 * i + 4 * q + 3] = v.w;
      t += (v.x + v.y) + (v.z + v.w);
    }
    xs[i] = t;
  }
  float* yb = y + (size_t)b * rows;
  float best = -FLT_MAX;
  int besti = INT_MAX;
  const int stride = gridDim.x * 4 * R;
  // the next step's rows are requested before the current step is reduced
  uint4 c[R][KI];
  uint32_t sc[R][KI], bi[R][KI];
  auto load = [&](int r0, uint4 (&cc)[R][KI], uint32_t (&ss)[R][KI], uint32_t (&bb)[R][KI]) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int row = min(r0 + j, rows - 1);
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        cc[j][i] = ld_nt_u4(W.codes + (size_t)row * (K / 2) + i * (kChunk / 2) + 16 * lane);
        ss[j][i] = ld_nt_u16(W.scales + (size_t)row * (K / 64) + i * (kChunk / 64) + (lane >> 1));
        bb[j][i] = ld_nt_u16(W.biases + (size_t)row * (K / 64) + i * (kChunk / 64) + (lane >> 1));
      }
    }
  };
  int r0 = (blockIdx.x * 4 + wv) * R;
  if (r0 < rows) load(r0, c, sc, bi);
  for (; r0 < rows; r0 += stride) {
    uint4 cn[R][KI];
    uint32_t sn[R][KI], bn[R][KI];
    if (r0 + stride < rows) load(r0 + stride, cn, sn, bn);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const float* xi = xv + 32 * i;
        float d = int4x8_dot(c[j][i].x, xi, 0.0f);
        d = int4x8_dot(c[j][i].y, xi + 8, d);
        d = int4x8_dot(c[j][i].z, xi + 16, d);
        d = int4x8_dot(c[j][i].w, xi + 24, d);
        a = __builtin_fmaf(bf16_value(sc[j][i]), d, a);
        a = __builtin_fmaf(bf16_value(bi[j][i]), xs[i], a);
      }
      const float v = wave_sum(a);
      const int row = r0 + j;
      if (row < rows) {
        if (lane == 0) yb[row] = v;
        if (v > best) { best = v; besti = row; }
      }
    }
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        c[j][i] = cn[j][i];
        sc[j][i] = sn[j][i];
        bi[j][i] = bn[j][i];
      }
  }
  if (!partials) return;  // uniform: no argmax requested
  __shared__ float sv[4];
  __shared__ int si[4];
  if (lane == 0) { sv[wv] = best; si[wv] = besti; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float bv = sv[0];
    int bidx = si[0];
    for (int w = 1; w < 4; ++w)
      if (sv[w] > bv || (sv[w] == bv && si[w] < bidx)) { bv = sv[w]; bidx = si[w]; }
    partials[(size_t)b * gridDim.x + blockIdx.x] = I4Partial{bv, bidx};
  }
}

// grid (B), 64 threads: the first index of the largest of n workgroup bests
// (a separate launch: a last-workgroup ticket would need a device-scope
// release fence, an L2 write-back, in every workgroup)
__global__ __launch_bounds__(64) void k_i4_argmax(const I4Partial* __restrict__ partials, int n,
                                                  int32_t* __restrict__ argmax) {
  const int lane = threadIdx.x, b = blockIdx.x;
  float bv = -FLT_MAX;
  int bidx = INT_MAX;
  for (int i = lane; i < n; i += 64) {
    const I4Partial p = partials[(size_t)b * n + i];
    if (p.value > bv || (p.value == bv && p.index < bidx)) { bv = p.value; bidx = p.index; }
  }
  wave_argmax(bv, bidx);
  if (lane == 0) argmax[b] = bidx;
}

template <int KI, int R>
hipError_t i4_launch(const flint_int4& W, int rows, const float* x, int B, float* y, int32_t* am, I4Partial* parts,
                     hipStream_t st) {
  const int waves = (rows + R - 1) / R;
  int blocks = (waves + 3) / 4;
  if (blocks > kI4Blocks) blocks = kI4Blocks;
  k_int4_gemv<KI, R><<<dim3(blocks, B), 256, 0, st>>>(W, rows, x, y, am ? parts : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !am) return e;
  k_i4_argmax<<<B, 64, 0, st>>>(parts, blocks, am);
  return hipGetLastError();
}

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool al2(const void* p) { return ((uintptr_t)p & 1u) == 0; }
size_t al256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace
}  // namespace flint

using namespace flint;

extern "C" {

int32_t flint_int4_quantize(const float* w, int64_t rows, int64_t cols, uint8_t* codes, uint16_t* scales,
                            uint16_t* biases, void* stream) {
  if (!w || !codes || !scales || !biases) return FLINT_E_NULL;
  if (rows < 1 || cols < 64 || cols % 64 || rows > (1ll << 40) / cols) return FLINT_E_DIMS;
  if (!al16(w) || !al16(codes) || !al2(scales) || !al2(biases)) return FLINT_E_ALIGN;
  int32_t st;
  if ((st = api_check_device())) return st;
  const long long groups = rows * (cols / 64);
  long long blocks = (groups + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  k_int4_quant<<<(int)blocks, 256, 0, (hipStream_t)stream>>>(w, groups, codes, scales, biases);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? FLINT_OK : api_hip_fail(e);
}

int32_t flint_int4_dequantize(const flint_int4* q, int64_t rows, int64_t cols, float* out, void* stream) {
  if (!q || !q->codes || !q->scales || !q->biases || !out) return FLINT_E_NULL;
  if (rows < 1 || cols < 64 || cols % 64 || rows > (1ll << 40) / cols) return FLINT_E_DIMS;
  if (!al2(q->scales) || !al2(q->biases) || !al16(out)) return FLINT_E_ALIGN;
  int32_t st;
  if ((st = api_check_device())) return st;
  const long long nbytes = rows * cols / 2;
  long long blocks = (nbytes + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  k_int4_dequant<<<(int)blocks, 256, 0, (hipStream_t)stream>>>(q->codes, q->scales, q->biases, nbytes, out);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? FLINT_OK : api_hip_fail(e);
}

size_t flint_int4_gemv_workspace_bytes(int32_t B) {
  if (B < 1 || B > kI4MaxB) return 0;
  return al256(sizeof(I4Partial) * (size_t)B * kI4Blocks);
}

int32_t flint_int4_gemv(const flint_int4* W, int32_t rows, int32_t cols, const float* x, int32_t B, float* y,
                        int32_t* argmax_opt, void* ws, size_t ws_bytes, void* stream) {
  if (!W || !W->codes || !W->scales || !W->biases || !x || !y || !ws) return FLINT_E_NULL;
  if (rows < 1 || cols < 1 || B < 1) return FLINT_E_DIMS;
  if (cols % kChunk || cols > 4 * kChunk || B > kI4MaxB) return FLINT_E_UNSUPPORTED;
  if (!al16(W->codes) || !al2(W->scales) || !al2(W->biases) || !al16(x) || !al16(y) || !al16(ws) ||
      ((uintptr_t)argmax_opt & 3u))
    return FLINT_E_ALIGN;
  if (ws_bytes < flint_int4_gemv_workspace_bytes(B)) return FLINT_E_WORKSPACE;
  int32_t st;
  if ((st = api_check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  I4Partial* parts = static_cast<I4Partial*>(ws);
  hipError_t e;
  switch (cols / kChunk) {
    case 1: e = i4_launch<1, 4>(*W, rows, x, B, y, argmax_opt, parts, s); break;
    case 2: e = i4_launch<2, 2>(*W, rows, x, B, y, argmax_opt, parts, s); break;
    case 3: e = i4_launch<3, 2>(*W, rows, x, B, y, argmax_opt, parts, s); break;
    default: e = i4_launch<4, 2>(*W, rows, x, B, y, argmax_opt, parts, s); break;
  }
  return e == hipSuccess ? FLINT_OK : api_hip_fail(e);
}

}  // extern "C"
