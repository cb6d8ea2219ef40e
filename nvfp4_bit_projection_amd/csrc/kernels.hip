// kernels.hip -- per-operation HIP kernels for gfx950: router GEMV + wavefront
// top-k, NVFP4 gate/up dequant-GEMV with SwiGLU, NVFP4 down dequant-GEMV with
// the weighted combine, NVFP4 head GEMV with argmax, and the NVFP4 quantiser.
//
// Method [P2 "Recursive Releases Flint, a 40B MoE Coding Model That Runs
// Locally at 125 Tokens per Second", "How does Flint's architecture work?";
// P3 "Flint: 125 tokens a second is what 2.5B active parameters buy at
// 273 GB/s", "The shape, read from the headers", "Why active parameters set
// the speed"]: a router picks the top k of E experts per token, each expert is
// three NVFP4 matrices (SwiGLU), a shared expert is always added, and the
// output head is an NVFP4 GEMV.  Every kernel here is bound by HBM bandwidth
// at batch 1: each weight byte is loaded once with a 128-bit load, decoded in
// registers and used for one multiply-add.
#include <float.h>
#include <limits.h>

#include "flint_device.h"
#include "flint_internal.h"

namespace flint {

// 32 activations of this lane: x[32*lane .. 32*lane+31] of a 2,048-vector,
// optionally scaled by 1/sqrt(mean(x^2) + eps) (RMSNorm with unit gain).
__device__ __forceinline__ void load_x32(const float* __restrict__ x, int lane, float norm_eps, float* xv) {
  const float4* p = reinterpret_cast<const float4*>(x + 32 * lane);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float4 v = p[i];
    xv[4 * i + 0] = v.x; xv[4 * i + 1] = v.y; xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
  }
  if (norm_eps >= 0.0f) {
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) ss = __builtin_fmaf(xv[i], xv[i], ss);
    ss = wave_sum(ss);
    float s = 1.0f / sqrtf(ss * (1.0f / kHidden) + norm_eps);
#pragma unroll
    for (int i = 0; i < 32; ++i) xv[i] *= s;
  }
}

// weight loads stream (non-temporal): each weight byte is read once per call
__device__ __forceinline__ uint4 ld_codes16(const uint8_t* p) { return ld_nt_u4(p); }
__device__ __forceinline__ uint32_t ld_scales2(const uint8_t* p) { return ld_nt_u16(p); }

// ----------------------------------------------------------------- router --
// Dot of one lane's 32 router weights (elements 32*lane .. 32*lane+31 of the
// row) with its 32 activations.  fp32 rows: 8 x 16 B loads; BF16 rows: 4 x
// 16 B loads, each BF16 value widened exactly (its bits are the top half of
// the fp32 pattern).  Same fma order for both.
__device__ __forceinline__ float router_dot32(const float* row, int lane, const float* xv) {
  const float* rw = row + 32 * lane;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = ld_nt_f4(rw + 4 * i);
    acc = __builtin_fmaf(v.x, xv[4 * i + 0], acc);
    acc = __builtin_fmaf(v.y, xv[4 * i + 1], acc);
    acc = __builtin_fmaf(v.z, xv[4 * i + 2], acc);
    acc = __builtin_fmaf(v.w, xv[4 * i + 3], acc);
  }
  return acc;
}
__device__ __forceinline__ float router_dot32(const uint16_t* row, int lane, const float* xv) {
  const uint16_t* rw = row + 32 * lane;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = ld_nt_u4(rw + 8 * i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = __builtin_fmaf(__uint_as_float(w[j] << 16), xv[8 * i + 2 * j + 0], acc);
      acc = __builtin_fmaf(__uint_as_float(w[j] & 0xFFFF0000u), xv[8 * i + 2 * j + 1], acc);
    }
  }
  return acc;
}

// grid (ceil(E/4), B), 256 threads: one router row per wave.  The top k is
// chosen by k_topk (next launch): a last-workgroup ticket would need a
// device-scope release fence in every workgroup, each writing back the XCD's
// L2.
template <typename RT>
__global__ __launch_bounds__(256) void k_route(const RT* __restrict__ router, int E, const float* __restrict__ x,
                                               float norm_eps, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, b = blockIdx.y;
  float xv[32];
  load_x32(x + (size_t)b * kHidden, lane, norm_eps, xv);
  const int e = blockIdx.x * 4 + wv;
  if (e < E) {
    float acc = router_dot32(router + (size_t)e * kHidden, lane, xv);
    acc = wave_sum(acc);
    if (lane == 0) logits[(size_t)b * E + e] = acc;
  }
}

// grid (B), 64 threads: the k largest of E <= 256 logits (4 per lane, k
// rounds of a (value, index) max; ties to the lower index), ordered by logit,
// and their weights: sigmoid == 0, softmax over the chosen logits; sigmoid !=
// 0, the chosen sigmoid scores over their sum.
__global__ __launch_bounds__(64) void k_topk(const float* __restrict__ logits, int E, int k, int sigmoid,
                                             int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  const int lane = threadIdx.x, b = blockIdx.x;
  float v[4];
  int id[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // all four loads in flight (an index past E reads expert E - 1)
    const int e = lane + 64 * j;
    v[j] = logits[(size_t)b * E + (e < E ? e : E - 1)];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    id[j] = lane + 64 * j;
    if (id[j] >= E) {
      v[j] = -FLT_MAX;
      id[j] = INT_MAX;
    }
  }
  float top_v[kMaxTopK];
  int top_i[kMaxTopK];
  for (int r = 0; r < k; ++r) {
    float bv = v[0];
    int bi = id[0];
#pragma unroll
    for (int j = 1; j < 4; ++j)
      if (v[j] > bv || (v[j] == bv && id[j] < bi)) { bv = v[j]; bi = id[j]; }
    wave_argmax(bv, bi);
    top_v[r] = bv;
    top_i[r] = bi;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (id[j] == bi) { v[j] = -FLT_MAX; id[j] = INT_MAX; }
  }
  if (lane == 0) {
    float sc[kMaxTopK];
    float z = 0.0f;
    for (int r = 0; r < k; ++r) {
      sc[r] = sigmoid ? 1.0f / (1.0f + __expf(-top_v[r])) : __expf(top_v[r] - top_v[0]);
      z += sc[r];
    }
    for (int r = 0; r < k; ++r) {
      idx_out[b * k + r] = top_i[r];
      w_out[b * k + r] = sc[r] / z;
    }
  }
}

// ---------------------------------------------------------- expert gate/up --
// Row j of the concatenated hidden layer: j < k*I is row j%I of routed slot
// j/I, otherwise row j-k*I of the shared expert.  One (gate, up) row pair per
// wave: h_j = silu(Sg * gate_j . x) * (Su * up_j . x).
__global__ __launch_bounds__(256) void k_gateup(flint_moe_layer L, int I, int k, int Is, const float* __restrict__ x,
                                                float norm_eps, const int32_t* __restrict__ idx,
                                                float* __restrict__ hact) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, b = blockIdx.y;
  const int nrows = k * I + Is;
  float xv[32];
  load_x32(x + (size_t)b * kHidden, lane, norm_eps, xv);
  const int j = blockIdx.x * 4 + wv;
  if (j >= nrows) return;
  const uint8_t *gc, *gs, *uc, *us;
  float Sg, Su;
  if (j < k * I) {
    const int e = idx[b * k + j / I], r = j % I;
    const size_t row = (size_t)e * I + r;
    gc = L.gate_codes + row * (kHidden / 2);
    gs = L.gate_scales + row * (kHidden / 16);
    uc = L.up_codes + row * (kHidden / 2);
    us = L.up_scales + row * (kHidden / 16);
    Sg = L.expert_tscales[3 * e + 0];
    Su = L.expert_tscales[3 * e + 1];
  } else {
    const size_t r = (size_t)(j - k * I);
    gc = L.shared_gate.codes + r * (kHidden / 2);
    gs = L.shared_gate.scales + r * (kHidden / 16);
    uc = L.shared_up.codes + r * (kHidden / 2);
    us = L.shared_up.scales + r * (kHidden / 16);
    Sg = *L.shared_gate.tscale;
    Su = *L.shared_up.tscale;
  }
  const uint4 cg = ld_codes16(gc + 16 * lane), cu = ld_codes16(uc + 16 * lane);
  const uint32_t sg = ld_scales2(gs + 2 * lane), su = ld_scales2(us + 2 * lane);
  float g = wave_sum(nvfp4_lane_dot32(cg, sg, xv)) * Sg;
  float a = wave_sum(nvfp4_lane_dot32(cu, su, xv)) * Su;
  if (lane == 0) hact[(size_t)b * nrows + j] = silu(g) * a;
}

// ------------------------------------------------------ expert down+combine --
// y[n] = sum_i w_i * Sd(e_i) * (Wd[e_i][n] . h_i) + Ssd * (Wsd[n] . h_s).
// The k routed rows (I wide) and the shared row (Is wide) of output n form
// one concatenated row of K = k*I + Is; each lane owns 32 consecutive
// elements of it per pass (two passes for K = 4096).  Each wave handles
// `kRowsPerWave` output rows; its h slices and per-lane coefficients are
// loaded once.
constexpr int kDownRowsPerWave = 4;
__global__ __launch_bounds__(256) void k_down(flint_moe_layer L, int I, int k, int Is, const int32_t* __restrict__ idx,
                                              const float* __restrict__ wts, const float* __restrict__ hact,
                                              float* __restrict__ y, int add_to_y) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, b = blockIdx.y;
  const int K = k * I + Is, nchunks = K / 32;
  const uint8_t* cbase[2] = {nullptr, nullptr};
  const uint8_t* sbase[2] = {nullptr, nullptr};
  size_t cstride[2] = {0, 0}, sstride[2] = {0, 0};
  float coef[2] = {0.0f, 0.0f};
  float hv[2][32];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int c = p * 64 + lane;
    if (c < nchunks) {
      const int kk = c * 32;
      if (kk < k * I) {
        const int slot = kk / I, off = kk % I, e = idx[b * k + slot];
        cbase[p] = L.down_codes + (size_t)e * kHidden * (I / 2) + off / 2;
        sbase[p] = L.down_scales + (size_t)e * kHidden * (I / 16) + off / 16;
        cstride[p] = I / 2;
        sstride[p] = I / 16;
        coef[p] = wts[b * k + slot] * L.expert_tscales[3 * e + 2];
      } else {
        const int off = kk - k * I;
        cbase[p] = L.shared_down.codes + off / 2;
        sbase[p] = L.shared_down.scales + off / 16;
        cstride[p] = Is / 2;
        sstride[p] = Is / 16;
        coef[p] = *L.shared_down.tscale;
      }
      const float4* hp = reinterpret_cast<const float4*>(hact + (size_t)b * K + kk);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float4 v = hp[i];
        hv[p][4 * i + 0] = v.x; hv[p][4 * i + 1] = v.y; hv[p][4 * i + 2] = v.z; hv[p][4 * i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) hv[p][i] = 0.0f;
    }
  }
  const int n0 = (blockIdx.x * 4 + wv) * kDownRowsPerWave;
#pragma unroll
  for (int r = 0; r < kDownRowsPerWave; ++r) {
    const int n = n0 + r;
    if (n >= kHidden) break;
    float acc = 0.0f;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (cbase[p]) {
        const uint4 c = ld_codes16(cbase[p] + (size_t)n * cstride[p]);
        const uint32_t s = ld_scales2(sbase[p] + (size_t)n * sstride[p]);
        acc += coef[p] * nvfp4_lane_dot32(c, s, hv[p]);
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      float* o = y + (size_t)b * kHidden + n;
      *o = add_to_y ? *o + acc : acc;
    }
  }
}

// -------------------------------------------------------------- lm head --
// grid (kHeadBlocks, B), 256 threads.  Each wave streams rows r0.. r0+R-1,
// then jumps by the total wave count; logits and a running (max, first index)
// per wave; each workgroup writes its best, and k_head_argmax (next launch)
// reduces them.  (A last-workgroup ticket would need a device-scope release
// fence in every workgroup, which writes back the XCD's L2 each time: it cost
// more than the GEMV.)
constexpr int kHeadRows = 4;
__global__ __launch_bounds__(256) void k_lmhead(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                const float* __restrict__ tscale, int vocab,
                                                const float* __restrict__ x, float norm_eps,
                                                float* __restrict__ logits, int32_t* __restrict__ argmax,
                                                HeadPartial* __restrict__ partials) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, b = blockIdx.y;
  float xv[32];
  load_x32(x + (size_t)b * kHidden, lane, norm_eps, xv);
  const float S = *tscale;
  float* lg = logits ? logits + (size_t)b * vocab : nullptr;
  const int nwaves = gridDim.x * 4;
  float best = -FLT_MAX;
  int besti = INT_MAX;
  for (int r0 = (blockIdx.x * 4 + wv) * kHeadRows; r0 < vocab; r0 += nwaves * kHeadRows) {
    uint4 c[kHeadRows];
    uint32_t s[kHeadRows];
#pragma unroll
    for (int j = 0; j < kHeadRows; ++j) {
      const int row = min(r0 + j, vocab - 1);
      c[j] = ld_codes16(codes + (size_t)row * (kHidden / 2) + 16 * lane);
      s[j] = ld_scales2(scales + (size_t)row * (kHidden / 16) + 2 * lane);
    }
#pragma unroll
    for (int j = 0; j < kHeadRows; ++j) {
      const float v = wave_sum(nvfp4_lane_dot32(c[j], s[j], xv)) * S;
      const int row = r0 + j;
      if (row < vocab) {
        if (lane == 0 && lg) lg[row] = v;
        if (v > best) { best = v; besti = row; }
      }
    }
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  if (lane == 0) { sv[wv] = best; si[wv] = besti; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float bv = sv[0];
    int bi = si[0];
    for (int w = 1; w < 4; ++w)
      if (sv[w] > bv || (sv[w] == bv && si[w] < bi)) { bv = sv[w]; bi = si[w]; }
    partials[(size_t)b * gridDim.x + blockIdx.x] = HeadPartial{bv, bi};
  }
}

// grid (B), 64 threads: the first index of the largest of n block maxima
__global__ __launch_bounds__(64) void k_head_argmax(const HeadPartial* __restrict__ partials, int n,
                                                    int32_t* __restrict__ argmax) {
  const int lane = threadIdx.x, b = blockIdx.x;
  float bv = -FLT_MAX;
  int bi = INT_MAX;
  for (int i = lane; i < n; i += 64) {
    const HeadPartial hp = partials[(size_t)b * n + i];
    if (hp.value > bv || (hp.value == bv && hp.index < bi)) { bv = hp.value; bi = hp.index; }
  }
  wave_argmax(bv, bi);
  if (lane == 0) argmax[b] = bi;
}

// ------------------------------------------------------------- quantiser --
// Reading of the NVFP4 recipe: S = fl32(max|w| / (6 * 448)); block scale =
// E4M3 round-to-nearest-even of blockmax / (6 S), saturating at 448; element
// code = E2M1 round-to-nearest-even of w / (d S), saturating at 6, sign kept;
// zero-scale blocks get zero codes.  Ratios in double precision.

__device__ __forceinline__ int e4m3_rne_code(double r) {  // r >= 0
  if (r >= 448.0) return 0x7E;
  if (r < 0.015625) return (int)rint(r * 512.0);  // subnormal step 2^-9; 8 -> 0x08
  int e;
  const double f = frexp(r, &e);                   // r = f 2^e, f in [0.5, 1)
  double mant = rint((2.0 * f - 1.0) * 8.0);       // r = (1 + mant/8) 2^(e-1)
  int E = e - 1 + 7;
  if (mant >= 8.0) { mant = 0.0; E += 1; }
  const int code = (E << 3) | (int)mant;
  return code > 0x7E ? 0x7E : code;
}

__device__ __forceinline__ double e4m3_value(int code) {  // non-negative finite codes
  const int E = code >> 3, m = code & 7;
  return E == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, E - 7);
}

// E2M1 magnitude code by thresholds; ties go to the even code.
__device__ __forceinline__ uint32_t e2m1_rne_code(double v) {
  const double a = fabs(v);
  uint32_t c;
  if (a <= 0.25) c = 0;
  else if (a < 0.75) c = 1;
  else if (a <= 1.25) c = 2;
  else if (a < 1.75) c = 3;
  else if (a <= 2.5) c = 4;
  else if (a < 3.5) c = 5;
  else if (a <= 5.0) c = 6;
  else c = 7;
  return c | (signbit(v) ? 8u : 0u);
}

// amax: each thread keeps four independent 16-byte loads in flight per step
// (per_mat is a multiple of 16 and every matrix 64-byte aligned); the
// workgroup's maximum is reduced in LDS and published with one atomic, so a
// matrix sees one atomic per workgroup (one per wave made the atomics on the
// single word the bottleneck).  The maximum does not depend on the order.
__global__ __launch_bounds__(256) void k_quant_amax(const float* __restrict__ w, int64_t per_mat,
                                                    uint32_t* __restrict__ amax_bits) {
  const int m = blockIdx.y;
  const float4* p = reinterpret_cast<const float4*>(w + (size_t)m * per_mat);
  const int64_t n4 = per_mat / 4, stride = (int64_t)gridDim.x * blockDim.x;
  float mx = 0.0f;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n4; i += 4 * stride) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
  }
  for (; i < n4; i += stride) {
    const float4 v = p[i];
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  mx = wave_max(mx);
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(&amax_bits[m], __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))));
}

__global__ __launch_bounds__(256) void k_quant_pack(const float* __restrict__ w, int64_t rows, int64_t cols,
                                                    const uint32_t* __restrict__ amax_bits,
                                                    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                    float* __restrict__ tscales) {
  const int m = blockIdx.y;
  const int64_t per_mat = rows * cols, nblk = per_mat / 16;
  const double amax = (double)__uint_as_float(amax_bits[m]);
  const float S = (float)(amax / 2688.0);
  if (blockIdx.x == 0 && threadIdx.x == 0) tscales[m] = S;
  const float* wm = w + (size_t)m * per_mat;
  uint8_t* cm = codes + (size_t)m * (per_mat / 2);
  uint8_t* sm = scales + (size_t)m * nblk;
  for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < nblk; blk += (int64_t)gridDim.x * blockDim.x) {
    const float4* p = reinterpret_cast<const float4*>(wm + blk * 16);
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 q = p[i];
      v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
    }
    uint32_t sc = 0, lo = 0, hi = 0;
    if (S != 0.0f) {
      float bm = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) bm = fmaxf(bm, fabsf(v[i]));
      sc = (uint32_t)e4m3_rne_code((double)bm / (6.0 * (double)S));
      const double dS = e4m3_value((int)sc) * (double)S;
      if (dS != 0.0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) lo |= e2m1_rne_code((double)v[i] / dS) << (4 * i);
#pragma unroll
        for (int i = 0; i < 8; ++i) hi |= e2m1_rne_code((double)v[8 + i] / dS) << (4 * i);
      }
    }
    *reinterpret_cast<uint2*>(cm + blk * 8) = make_uint2(lo, hi);
    sm[blk] = (uint8_t)sc;
  }
}

__global__ void k_zero_u32(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

// w = fl32((e2m1(c) * d) * S): the first product is exact in fp32.
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                 const float* __restrict__ tscale, int64_t n_blocks,
                                                 float* __restrict__ out) {
  const float S = *tscale;
  for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < n_blocks;
       blk += (int64_t)gridDim.x * blockDim.x) {
    const float d = e4m3_to_f32(scales[blk]);
    const uint2 c = *reinterpret_cast<const uint2*>(codes + blk * 8);
    float o[16];
    fp4x8_values(c.x, o);
    fp4x8_values(c.y, o + 8);
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = (o[i] * d) * S;
    float4* op = reinterpret_cast<float4*>(out + blk * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) op[i] = make_float4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
  }
}

__global__ void k_copy_f32(const float* __restrict__ s, float* __restrict__ d, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) d[i] = s[i];
}

// --------------------------------------------------------------- launchers --
hipError_t launch_route(const flint_moe_dims& d, const float* router, const float* x, int B, float norm_eps,
                        float* logits, int32_t* idx, float* w, hipStream_t s) {
  dim3 grid((d.n_experts + 3) / 4, B);
  k_route<float><<<grid, 256, 0, s>>>(router, d.n_experts, x, norm_eps, logits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_topk<<<B, 64, 0, s>>>(logits, d.n_experts, d.top_k, 0, idx, w);
  return hipGetLastError();
}

hipError_t launch_route_ex(const flint_moe_dims& d, const void* router, bool bf16, bool sigmoid, const float* x,
                           int B, float* logits, int32_t* idx, float* w, hipStream_t s) {
  dim3 grid((d.n_experts + 3) / 4, B);
  if (bf16)
    k_route<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(router), d.n_experts, x, -1.0f, logits);
  else
    k_route<float><<<grid, 256, 0, s>>>(static_cast<const float*>(router), d.n_experts, x, -1.0f, logits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_topk<<<B, 64, 0, s>>>(logits, d.n_experts, d.top_k, sigmoid ? 1 : 0, idx, w);
  return hipGetLastError();
}

hipError_t launch_gateup(const flint_moe_dims& d, const flint_moe_layer& L, const float* x, int B, float norm_eps,
                         const int32_t* idx, float* hact, hipStream_t s) {
  const int nrows = d.top_k * d.expert_width + d.shared_width;
  dim3 grid((nrows + 3) / 4, B);
  k_gateup<<<grid, 256, 0, s>>>(L, d.expert_width, d.top_k, d.shared_width, x, norm_eps, idx, hact);
  return hipGetLastError();
}

hipError_t launch_down(const flint_moe_dims& d, const flint_moe_layer& L, const int32_t* idx, const float* w,
                       const float* hact, int B, float* y, bool add_to_y, hipStream_t s) {
  dim3 grid(kHidden / (4 * kDownRowsPerWave), B);
  k_down<<<grid, 256, 0, s>>>(L, d.expert_width, d.top_k, d.shared_width, idx, w, hact, y, add_to_y ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_lmhead(const flint_nvfp4& head, int vocab, const float* x, int B, float norm_eps, float* logits,
                         int32_t* argmax, HeadPartial* partials, hipStream_t s) {
  dim3 grid(kHeadBlocks, B);
  k_lmhead<<<grid, 256, 0, s>>>(head.codes, head.scales, head.tscale, vocab, x, norm_eps, logits, argmax, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_head_argmax<<<B, 64, 0, s>>>(partials, kHeadBlocks, argmax);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* w, int64_t n_mats, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, float* tscales, uint32_t* amax_bits, hipStream_t s) {
  const int64_t per_mat = rows * cols;
  int gx = (int)((per_mat + 256 * 64 - 1) / (256 * 64));  // 64 values a thread: fewer workgroups, fewer atomics
  if (gx > 1024) gx = 1024;
  if (gx < 1) gx = 1;
  for (int64_t m0 = 0; m0 < n_mats; m0 += 65535) {
    const int nm = (int)((n_mats - m0) < 65535 ? (n_mats - m0) : 65535);
    k_quant_amax<<<dim3(gx, nm), 256, 0, s>>>(w + m0 * per_mat, per_mat, amax_bits + m0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nblk = per_mat / 16;
    int gp = (int)((nblk + 255) / 256);
    if (gp > 4096) gp = 4096;
    k_quant_pack<<<dim3(gp, nm), 256, 0, s>>>(w + m0 * per_mat, rows, cols, amax_bits + m0, codes + m0 * (per_mat / 2),
                                             scales + m0 * (per_mat / 16), tscales + m0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  k_zero_u32<<<(int)((n_mats + 255) / 256 < 1024 ? (n_mats + 255) / 256 : 1024), 256, 0, s>>>(amax_bits, n_mats);
  return hipGetLastError();
}

hipError_t launch_dequantize(const flint_nvfp4& q, int64_t rows, int64_t cols, float* out, hipStream_t s) {
  const int64_t nblk = rows * cols / 16;
  int g = (int)((nblk + 255) / 256);
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  k_dequant<<<g, 256, 0, s>>>(q.codes, q.scales, q.tscale, nblk, out);
  return hipGetLastError();
}

// Column slicing of a byte matrix for the stack schedule: src [outer][rows][rb]
// -> dst [outer][G][rows][rb/G], 2-byte granules (rb/G even).
__global__ void k_slice_cols(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int64_t outer, int rows,
                             int rb, int G) {
  const int sw = rb / G / 2;  // 2-byte words per slice row
  const int64_t n = outer * (int64_t)G * rows * sw;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int k = (int)(i % sw);
    int64_t r = i / sw;
    const int row = (int)(r % rows);
    r /= rows;
    const int g = (int)(r % G);
    const int64_t o = r / G;
    dst[i] = src[((o * rows + row) * rb + (int64_t)g * (rb / G)) / 2 + k];
  }
}

hipError_t launch_slice_cols(const uint8_t* src, uint8_t* dst, int64_t outer, int rows, int rb, int G,
                             hipStream_t s) {
  const int64_t words = outer * rows * (int64_t)rb / 2;
  const int blocks = (int)((words + 255) / 256 < 4096 ? (words + 255) / 256 : 4096);
  k_slice_cols<<<blocks, 256, 0, s>>>(reinterpret_cast<const uint16_t*>(src), reinterpret_cast<uint16_t*>(dst), outer,
                                      rows, rb, G);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, int n, hipStream_t s) {
  k_copy_f32<<<(n + 255) / 256, 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}

}  // namespace flint
