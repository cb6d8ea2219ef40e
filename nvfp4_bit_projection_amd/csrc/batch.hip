// batch.hip -- small-batch decode step: B tokens (B <= 64) through the layer
// stack and the head together, every weight byte read once per step.
//
// Method [P2 "Recursive Releases Flint, a 40B MoE Coding Model That Runs
// Locally at 125 Tokens per Second", "How does Flint's architecture work?";
// P3 "Flint: 125 tokens a second is what 2.5B active parameters buy at
// 273 GB/s", "The shape, read from the headers"]: each token has its own
// top-6 routing; the B*6 (token, slot) pairs are bucketed by expert, so a
// chosen expert's three matrices are streamed once for all the tokens that
// picked it.  The shared expert, the router and the head are streamed once
// and applied to all B tokens.  Per layer:
//   k_bnorm     u_b = h_b / sqrt(mean(h_b^2) + eps)
//   k_broute    logits[b][e] = router[e] . u_b   (one router row per wave)
//   k_btopk     top-k and renormalised softmax per token (one wave per token)
//   k_bucket    (token, slot) pairs grouped by expert, experts in index
//               order, pairs in (token, slot) order: a histogram, a scan, a
//               scatter in one workgroup
//   k_bgateup   SwiGLU rows: one (gate, up) row pair per wave, applied to
//               every pair of its expert; k_bgateup_shared the same for the
//               shared expert and every token (tokens staged in LDS)
//   k_bdown     down rows per 16/32-lane group, same sharing; k_bdown_shared
//   k_bcombine  h_b += sum_s down[b][s] + shared[b]   (fixed order)
// and at the end k_bnorm + k_bhead (rows streamed once, tokens in LDS) +
// k_bargmax.  All arithmetic fp32; weights NVFP4 decoded in registers.
#include <float.h>
#include <limits.h>

#include "flint_device.h"
#include "flint_internal.h"

namespace flint {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void lane_x32(const float* __restrict__ v, int lane, float* xv) {
  const float4* p = reinterpret_cast<const float4*>(v + 32 * lane);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 a = p[i];
    xv[4 * i] = a.x; xv[4 * i + 1] = a.y; xv[4 * i + 2] = a.z; xv[4 * i + 3] = a.w;
  }
}

// Token vectors staged in LDS for the kernels that apply one weight row to
// every token: rows of 32 values padded to 36, so that the 64 lanes of a
// wave, each reading its own 32 consecutive values with 128-bit loads, hit
// distinct banks.  K = 2048: 12 tokens per pass (110,592 B).
constexpr int kPad = 36;
constexpr int kStageFloats = 12 * (kHidden / 32) * kPad;
template <int K>
constexpr int stage_tokens_per_pass() { return kStageFloats / ((K / 32) * kPad); }

template <int K>
__device__ __forceinline__ void stage_tokens(const float* __restrict__ src, int b0, int nb, float* sh) {
  const int n4 = nb * (K / 4);
  for (int i = threadIdx.x; i < n4; i += kThreads) {
    const int b = i / (K / 4), c = 4 * (i % (K / 4));
    const float4 v = *reinterpret_cast<const float4*>(src + (size_t)(b0 + b) * K + c);
    *reinterpret_cast<float4*>(sh + (b * (K / 32) + c / 32) * kPad + c % 32) = v;
  }
}
// the 32 values of lane chunk j of staged token b
template <int K>
__device__ __forceinline__ void staged_x32(const float* sh, int b, int j, float* xv) {
  const float4* p = reinterpret_cast<const float4*>(sh + (b * (K / 32) + j) * kPad);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 a = p[i];
    xv[4 * i] = a.x; xv[4 * i + 1] = a.y; xv[4 * i + 2] = a.z; xv[4 * i + 3] = a.w;
  }
}

// ---------------------------------------------------------------- norm --
// grid B, 256 threads: u_b = h_b * s_b, s_b = 1/sqrt(mean(h_b^2) + eps)
__global__ __launch_bounds__(kThreads) void k_bnorm(const float* __restrict__ h, float* __restrict__ u, float eps) {
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const float* hb = h + (size_t)b * kHidden;
  float v[kHidden / kThreads];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kHidden / kThreads; ++i) {
    v[i] = hb[t + i * kThreads];
    ss = __builtin_fmaf(v[i], v[i], ss);
  }
  ss = wave_sum(ss);
  __shared__ float red[kThreads / 64];
  if (lane == 0) red[w] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float s = 1.0f / sqrtf(tot * (1.0f / kHidden) + eps);
#pragma unroll
  for (int i = 0; i < kHidden / kThreads; ++i) u[(size_t)b * kHidden + t + i * kThreads] = v[i] * s;
}

// --------------------------------------------------------------- router --
// grid ceil(E/4), 256 threads: router row e = 4 blockIdx.x + wave, read once,
// dotted with every token (tokens staged in LDS, 12 per pass).
__global__ __launch_bounds__(kThreads) void k_broute(const float* __restrict__ router, int E,
                                                     const float* __restrict__ u, int B, float* __restrict__ logits) {
  __shared__ __align__(16) float sh[kStageFloats];
  const int lane = threadIdx.x & 63, e = blockIdx.x * 4 + (threadIdx.x >> 6);
  float wr[32];
  {
    const float* rw = router + (size_t)(e < E ? e : 0) * kHidden + 32 * lane;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 a = ld_nt_f4(rw + 4 * i);
      wr[4 * i] = a.x; wr[4 * i + 1] = a.y; wr[4 * i + 2] = a.z; wr[4 * i + 3] = a.w;
    }
  }
  constexpr int P = stage_tokens_per_pass<kHidden>();
  for (int b0 = 0; b0 < B; b0 += P) {
    const int nb = B - b0 < P ? B - b0 : P;
    __syncthreads();
    stage_tokens<kHidden>(u, b0, nb, sh);
    __syncthreads();
    for (int b = 0; b < nb; ++b) {
      float xv[32];
      staged_x32<kHidden>(sh, b, lane, xv);
      float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; i += 2) {
        a0 = __builtin_fmaf(wr[i], xv[i], a0);
        a1 = __builtin_fmaf(wr[i + 1], xv[i + 1], a1);
      }
      const float acc = wave_sum(a0 + a1);
      if (lane == 0 && e < E) logits[(size_t)(b0 + b) * E + e] = acc;
    }
  }
}

// ----------------------------------------------------------------- top-k --
// grid B, 64 threads: 4 logits per lane kept sorted by (value desc, index
// asc); k rounds: wave maximum of the lanes' heads (DPP), the lane holding it
// by a ballot (on a tie between lanes, the lowest index by a wave minimum),
// pop that head; weights exp(l_i - l_0) / sum.
__global__ __launch_bounds__(64) void k_btopk(const float* __restrict__ logits, int E, int k,
                                              int32_t* __restrict__ idx, float* __restrict__ wts) {
  const int b = blockIdx.x, lane = threadIdx.x;
  int key[4], id[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    id[j] = lane + 64 * j;
    key[j] = id[j] < E ? ord_key(logits[(size_t)b * E + id[j]]) : INT_MIN;
  }
  auto cswap = [&](int a, int c) {
    const bool sw = key[c] > key[a] || (key[c] == key[a] && id[c] < id[a]);
    const int tk = sw ? key[c] : key[a], ti = sw ? id[c] : id[a];
    key[c] = sw ? key[a] : key[c];
    id[c] = sw ? id[a] : id[c];
    key[a] = tk;
    id[a] = ti;
  };
  cswap(0, 1); cswap(2, 3); cswap(0, 2); cswap(1, 3); cswap(1, 2);
  int my_key = INT_MIN, my_id = 0;
  for (int r = 0; r < k; ++r) {
    const int m = wave_max_i32(key[0]);
    const uint64_t at = __builtin_amdgcn_ballot_w64(key[0] == m);
    const int mi = __builtin_popcountll(at) == 1 ? __builtin_amdgcn_readlane(id[0], __builtin_ctzll(at))
                                                 : wave_min_dpp(key[0] == m ? id[0] : INT_MAX);
    if (lane == r) { my_key = m; my_id = mi; }
    if (id[0] == mi) {
      key[0] = key[1]; id[0] = id[1];
      key[1] = key[2]; id[1] = id[2];
      key[2] = key[3]; id[2] = id[3];
      key[3] = INT_MIN; id[3] = INT_MAX;
    }
  }
  const float my_v = ord_key_value(my_key);
  const float first = lane_f32(my_v, 0);
  const float ex = lane < k ? __expf(my_v - first) : 0.0f;
  const float z = lane_f32(row16_sum(ex), 0);
  if (lane < k) {
    idx[b * k + lane] = my_id;
    wts[b * k + lane] = ex / z;
  }
}

// ---------------------------------------------------------------- bucket --
// one workgroup of 256 threads (E <= 256): thread e counts its pairs; an
// exclusive scan gives each expert's start and each chosen expert its rank;
// thread e then writes its pairs in (token, slot) order.
// Output: bk[0] = U (distinct experts), bk[1 .. 1+256) = expert of rank u,
// bk[257 .. 257+257) = start of rank u's pairs (start[U] = B*k), then the
// pair ids b*k + s.
constexpr int kBkExperts = 1, kBkStart = 1 + kMaxExperts, kBkPairs = 1 + kMaxExperts + kMaxExperts + 1;

__device__ __forceinline__ int block_excl_scan(int v, int* sh) {  // 256 threads
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += sh[i];
  __syncthreads();
  return base + x - v;
}

__global__ __launch_bounds__(kThreads) void k_bucket(const int32_t* __restrict__ idx_g, int nb, int E,
                                                     int32_t* __restrict__ bk) {
  const int e = threadIdx.x;
  __shared__ int sh[kThreads / 64];
  __shared__ int idx[kMaxBatch * kMaxTopK];
  for (int p = e; p < nb; p += kThreads) idx[p] = idx_g[p];
  __syncthreads();
  int cnt = 0;
  if (e < E)
    for (int p = 0; p < nb; ++p) cnt += idx[p] == e;
  const int start = block_excl_scan(cnt, sh);
  const int rank = block_excl_scan(cnt > 0 ? 1 : 0, sh);
  if (cnt > 0) {
    bk[kBkExperts + rank] = e;
    bk[kBkStart + rank] = start;
    int o = start;
    for (int p = 0; p < nb; ++p)
      if (idx[p] == e) bk[kBkPairs + o++] = p;
  }
  if (e == kThreads - 1) {
    const int U = rank + (cnt > 0 ? 1 : 0);
    bk[0] = U;
    bk[kBkStart + U] = start + cnt;
  }
}

// -------------------------------------------------------------- gate/up --
// Routed: grid (I/16, Umax), 256 threads; blockIdx.y < U is the rank-u
// expert; each wave takes 4 consecutive rows (all their loads issued at once)
// and applies them to each of the expert's (token, slot) pairs (few per
// expert, so a token vector comes straight from memory and serves 4 rows).
// hr [B*k][I].
constexpr int kRowsPerWave = 4;
__global__ __launch_bounds__(kThreads) void k_bgateup(flint_moe_layer L, int I, int k, const float* __restrict__ u,
                                                      const int32_t* __restrict__ bk, float* __restrict__ hr) {
  const int lane = threadIdx.x & 63, r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kRowsPerWave;
  const int ub = blockIdx.y;
  if (ub >= bk[0] || r0 >= I) return;
  const int e = bk[kBkExperts + ub];
  uint4 cg[kRowsPerWave], cu[kRowsPerWave];
  uint32_t sg[kRowsPerWave], su[kRowsPerWave];
#pragma unroll
  for (int q = 0; q < kRowsPerWave; ++q) {
    const size_t row = (size_t)e * I + r0 + q;
    cg[q] = ld_nt_u4(L.gate_codes + row * (kHidden / 2) + 16 * lane);
    cu[q] = ld_nt_u4(L.up_codes + row * (kHidden / 2) + 16 * lane);
    sg[q] = ld_nt_u16(L.gate_scales + row * (kHidden / 16) + 2 * lane);
    su[q] = ld_nt_u16(L.up_scales + row * (kHidden / 16) + 2 * lane);
  }
  const float Sg = L.expert_tscales[3 * e + 0], Su = L.expert_tscales[3 * e + 1];
  const int p0 = bk[kBkStart + ub], p1 = bk[kBkStart + ub + 1];
  for (int p = p0; p < p1; ++p) {
    const int pid = bk[kBkPairs + p];
    float xv[32];
    lane_x32(u + (size_t)(pid / k) * kHidden, lane, xv);
#pragma unroll 2
    for (int q = 0; q < kRowsPerWave; ++q) {
      const float g = wave_sum(nvfp4_lane_dot32(cg[q], sg[q], xv)) * Sg;
      const float a = wave_sum(nvfp4_lane_dot32(cu[q], su[q], xv)) * Su;
      if (lane == 0) hr[(size_t)pid * I + r0 + q] = silu(g) * a;
    }
  }
}

// Shared: grid Is/4, 256 threads; wave row r, decoded once, applied to every
// token (tokens staged in LDS).  hs [B][Is].
__global__ __launch_bounds__(kThreads) void k_bgateup_shared(flint_moe_layer L, int Is, int B,
                                                             const float* __restrict__ u, float* __restrict__ hs) {
  __shared__ __align__(16) float sh[kStageFloats];
  const int lane = threadIdx.x & 63, r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const uint4 cg = ld_nt_u4(L.shared_gate.codes + (size_t)r * (kHidden / 2) + 16 * lane);
  const uint4 cu = ld_nt_u4(L.shared_up.codes + (size_t)r * (kHidden / 2) + 16 * lane);
  const uint32_t sg = ld_nt_u16(L.shared_gate.scales + (size_t)r * (kHidden / 16) + 2 * lane);
  const uint32_t su = ld_nt_u16(L.shared_up.scales + (size_t)r * (kHidden / 16) + 2 * lane);
  const float Sg = *L.shared_gate.tscale, Su = *L.shared_up.tscale;
  float wg[32], wu[32];
  fp4x8_values(cg.x, wg); fp4x8_values(cg.y, wg + 8); fp4x8_values(cg.z, wg + 16); fp4x8_values(cg.w, wg + 24);
  fp4x8_values(cu.x, wu); fp4x8_values(cu.y, wu + 8); fp4x8_values(cu.z, wu + 16); fp4x8_values(cu.w, wu + 24);
  const float dg0 = e4m3_to_f32(sg & 0xFF), dg1 = e4m3_to_f32(sg >> 8);
  const float du0 = e4m3_to_f32(su & 0xFF), du1 = e4m3_to_f32(su >> 8);
  constexpr int P = stage_tokens_per_pass<kHidden>();
  for (int b0 = 0; b0 < B; b0 += P) {
    const int nb = B - b0 < P ? B - b0 : P;
    __syncthreads();
    stage_tokens<kHidden>(u, b0, nb, sh);
    __syncthreads();
    for (int b = 0; b < nb; ++b) {
      float xv[32];
      staged_x32<kHidden>(sh, b, lane, xv);
      float g0 = 0.0f, g1 = 0.0f, a0 = 0.0f, a1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        g0 = __builtin_fmaf(wg[i], xv[i], g0);
        g1 = __builtin_fmaf(wg[16 + i], xv[16 + i], g1);
        a0 = __builtin_fmaf(wu[i], xv[i], a0);
        a1 = __builtin_fmaf(wu[16 + i], xv[16 + i], a1);
      }
      const float g = wave_sum(dg0 * g0 + dg1 * g1) * Sg;
      const float a = wave_sum(du0 * a0 + du1 * a1) * Su;
      if (lane == 0) hs[(size_t)(b0 + b) * Is + r] = silu(g) * a;
    }
  }
}

// ---------------------------------------------------------------- down --
// Output rows n of a K-wide down matrix (K = I routed, Is shared): a row is
// covered by G = K/32 lanes (16 B of codes each), 64/G rows per wave.
template <int G>
__device__ __forceinline__ float group_reduce(float v) {
  if constexpr (G == 16) return row16_sum(v);
  else return group_sum<G>(v);
}

// Routed: grid (H / (4 * 4 * 64/G), Umax), 256 threads; each wave takes 4
// passes of 64/G rows, all loads issued at once.
// dr[pid][n] = w_pid * Sd_e * (Wd[e][n] . hr[pid]).
template <int G>
__global__ __launch_bounds__(kThreads) void k_bdown(flint_moe_layer L, int I, const int32_t* __restrict__ bk,
                                                    const float* __restrict__ wts, const float* __restrict__ hr,
                                                    float* __restrict__ dr) {
  constexpr int RPW = 64 / G;  // rows per wave pass
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int ub = blockIdx.y;
  if (ub >= bk[0]) return;
  const int j = lane % G, n0 = (blockIdx.x * 4 + wv) * RPW * kRowsPerWave + lane / G;
  const int e = bk[kBkExperts + ub], p0 = bk[kBkStart + ub], p1 = bk[kBkStart + ub + 1];
  uint4 c[kRowsPerWave];
  uint32_t sc[kRowsPerWave];
#pragma unroll
  for (int q = 0; q < kRowsPerWave; ++q) {
    const size_t row = (size_t)e * kHidden + n0 + q * RPW;
    c[q] = ld_nt_u4(L.down_codes + row * (I / 2) + 16 * j);
    sc[q] = ld_nt_u16(L.down_scales + row * (I / 16) + 2 * j);
  }
  const float S = L.expert_tscales[3 * e + 2];
  for (int p = p0; p < p1; ++p) {
    const int pid = bk[kBkPairs + p];
    float hv[32];
    lane_x32(hr + (size_t)pid * I, j, hv);
    const float coef = S * wts[pid];
#pragma unroll 2
    for (int q = 0; q < kRowsPerWave; ++q) {
      const float acc = group_reduce<G>(nvfp4_lane_dot32(c[q], sc[q], hv)) * coef;
      if (j == 0) dr[(size_t)pid * kHidden + n0 + q * RPW] = acc;
    }
  }
}

// Shared: grid H / (4 * 64/G), 256 threads; rows decoded once, applied to
// every token (hidden vectors staged in LDS).  ds[b][n].
template <int G>
__global__ __launch_bounds__(kThreads) void k_bdown_shared(flint_moe_layer L, int B, const float* __restrict__ hs,
                                                           float* __restrict__ ds) {
  constexpr int RPW = 64 / G, K = 32 * G;
  __shared__ __align__(16) float sh[kStageFloats];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int j = lane % G, n = (blockIdx.x * 4 + wv) * RPW + lane / G;
  const uint4 c = ld_nt_u4(L.shared_down.codes + (size_t)n * (K / 2) + 16 * j);
  const uint32_t s = ld_nt_u16(L.shared_down.scales + (size_t)n * (K / 16) + 2 * j);
  const float S = *L.shared_down.tscale;
  float w[32];
  fp4x8_values(c.x, w); fp4x8_values(c.y, w + 8); fp4x8_values(c.z, w + 16); fp4x8_values(c.w, w + 24);
  const float d0 = e4m3_to_f32(s & 0xFF), d1 = e4m3_to_f32(s >> 8);
  constexpr int P = stage_tokens_per_pass<K>();
  for (int b0 = 0; b0 < B; b0 += P) {
    const int nb = B - b0 < P ? B - b0 : P;
    __syncthreads();
    stage_tokens<K>(hs, b0, nb, sh);
    __syncthreads();
    for (int b = 0; b < nb; ++b) {
      float hv[32];
      staged_x32<K>(sh, b, j, hv);
      float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        a0 = __builtin_fmaf(w[i], hv[i], a0);
        a1 = __builtin_fmaf(w[16 + i], hv[16 + i], a1);
      }
      const float acc = group_reduce<G>(d0 * a0 + d1 * a1) * S;
      if (j == 0) ds[(size_t)(b0 + b) * kHidden + n] = acc;
    }
  }
}

// ------------------------------------------------------------- combine --
// grid (H/256, B): h_b[n] += (sum over slots in order of dr) + ds
__global__ __launch_bounds__(kThreads) void k_bcombine(float* __restrict__ h, const float* __restrict__ dr,
                                                       const float* __restrict__ ds, int k) {
  const int b = blockIdx.y, n = blockIdx.x * kThreads + threadIdx.x;
  float y = 0.0f;
  for (int sl = 0; sl < k; ++sl) y += dr[((size_t)b * k + sl) * kHidden + n];
  y += ds[(size_t)b * kHidden + n];
  h[(size_t)b * kHidden + n] += y;
}

// ----------------------------------------------------------------- head --
// grid kBHeadBlocks, 256 threads.  The B normalised hidden vectors sit in
// LDS; each wave decodes a row once and dots it with every token; per token
// a running (max, first index) in LDS; each block writes its per-token
// partials, k_bargmax reduces them.
constexpr int kBHeadBlocks = 1024;
constexpr int kBHeadMaxTok = 16;  // tokens per pass (LDS: 16 x 9 KB, padded rows)

__global__ __launch_bounds__(kThreads) void k_bhead(const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ scales,
                                                    const float* __restrict__ tscale, int vocab,
                                                    const float* __restrict__ z, int b0, int nb,
                                                    float* __restrict__ logits, HeadPartial* __restrict__ partials) {
  __shared__ __align__(16) float zs[kBHeadMaxTok * (kHidden / 32) * kPad];
  __shared__ float bv[4][kBHeadMaxTok];
  __shared__ int bi[4][kBHeadMaxTok];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  stage_tokens<kHidden>(z, b0, nb, zs);
  if (lane < kBHeadMaxTok) { bv[wv][lane] = -FLT_MAX; bi[wv][lane] = INT_MAX; }
  __syncthreads();
  const float S = *tscale;
  const int nwaves = gridDim.x * 4;
  for (int r = blockIdx.x * 4 + wv; r < vocab; r += nwaves) {
    const uint4 c = ld_nt_u4(codes + (size_t)r * (kHidden / 2) + 16 * lane);
    const uint32_t s = ld_nt_u16(scales + (size_t)r * (kHidden / 16) + 2 * lane);
    float w[32];
    fp4x8_values(c.x, w); fp4x8_values(c.y, w + 8); fp4x8_values(c.z, w + 16); fp4x8_values(c.w, w + 24);
    const float d0 = e4m3_to_f32(s & 0xFF), d1 = e4m3_to_f32(s >> 8);
    for (int b = 0; b < nb; ++b) {
      float xv[32];
      staged_x32<kHidden>(zs, b, lane, xv);
      float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        a0 = __builtin_fmaf(w[i], xv[i], a0);
        a1 = __builtin_fmaf(w[16 + i], xv[16 + i], a1);
      }
      const float v = wave_sum(d0 * a0 + d1 * a1) * S;
      if (lane == 0) {
        if (logits) logits[(size_t)(b0 + b) * vocab + r] = v;
        if (v > bv[wv][b]) { bv[wv][b] = v; bi[wv][b] = r; }  // rows rise, so ties keep the first
      }
    }
  }
  __syncthreads();
  if (t < nb) {
    float v = bv[0][t];
    int id = bi[0][t];
    for (int w = 1; w < 4; ++w)
      if (bv[w][t] > v || (bv[w][t] == v && bi[w][t] < id)) { v = bv[w][t]; id = bi[w][t]; }
    partials[(size_t)(b0 + t) * gridDim.x + blockIdx.x] = HeadPartial{v, id};
  }
}

// grid B, 64 threads: argmax over the blocks' partials, ties to the lower index
__global__ __launch_bounds__(64) void k_bargmax(const HeadPartial* __restrict__ partials, int nblocks,
                                                int32_t* __restrict__ argmax) {
  const int b = blockIdx.x, lane = threadIdx.x;
  float v = -FLT_MAX;
  int id = INT_MAX;
  for (int i = lane; i < nblocks; i += 64) {
    const HeadPartial hp = partials[(size_t)b * nblocks + i];
    if (hp.value > v || (hp.value == v && hp.index < id)) { v = hp.value; id = hp.index; }
  }
  wave_argmax(v, id);
  if (lane == 0) argmax[b] = id;
}

template <int G>
hipError_t launch_bdown_routed(const flint_moe_layer& L, int I, int Umax, const int32_t* bk, const float* wts,
                               const float* hr, float* dr, hipStream_t s) {
  k_bdown<G><<<dim3(kHidden / (4 * (64 / G) * kRowsPerWave), Umax), kThreads, 0, s>>>(L, I, bk, wts, hr, dr);
  return hipGetLastError();
}
template <int G>
hipError_t launch_bdown_shared(const flint_moe_layer& L, int B, const float* hs, float* ds, hipStream_t s) {
  k_bdown_shared<G><<<kHidden / (4 * (64 / G)), kThreads, 0, s>>>(L, B, hs, ds);
  return hipGetLastError();
}

}  // namespace

bool batch_supported(const flint_moe_dims& d, int B) {
  auto pow2_lanes = [](int K) { const int G = K / 32; return K % 32 == 0 && G >= 8 && G <= 64 && (G & (G - 1)) == 0; };
  return d.hidden == kHidden && B >= 1 && B <= kMaxBatch && pow2_lanes(d.expert_width) && pow2_lanes(d.shared_width) &&
         d.n_experts <= kMaxExperts && d.top_k <= kMaxTopK;
}

BatchWs::BatchWs(const flint_moe_dims& d, int B, int vocab) {
  (void)vocab;
  const int nb = B * d.top_k;
  size_t o = 0;
  h = o; o = align_up(o + 4 * (size_t)B * kHidden, 256);
  u = o; o = align_up(o + 4 * (size_t)B * kHidden, 256);
  logits = o; o = align_up(o + 4 * (size_t)B * d.n_experts, 256);
  idx = o; o = align_up(o + 4 * (size_t)nb, 256);
  wts = o; o = align_up(o + 4 * (size_t)nb, 256);
  bucket = o; o = align_up(o + 4 * (size_t)(kBkPairs + nb), 256);
  hr = o; o = align_up(o + 4 * (size_t)nb * d.expert_width, 256);
  hs = o; o = align_up(o + 4 * (size_t)B * d.shared_width, 256);
  dr = o; o = align_up(o + 4 * (size_t)nb * kHidden, 256);
  ds = o; o = align_up(o + 4 * (size_t)B * kHidden, 256);
  partials = o; o = align_up(o + sizeof(HeadPartial) * (size_t)B * kBHeadBlocks, 256);
  total = o;
}

hipError_t launch_batch_step(const flint_moe_dims& d, const flint_moe_layer* layers, int L, const flint_nvfp4& head,
                             int vocab, const float* x, int B, float eps, float* logits, int32_t* argmax,
                             int32_t* routes, void* ws, hipStream_t s) {
  const BatchWs w(d, B, vocab);
  char* base = static_cast<char*>(ws);
  float* h = reinterpret_cast<float*>(base + w.h);
  float* u = reinterpret_cast<float*>(base + w.u);
  float* lg = reinterpret_cast<float*>(base + w.logits);
  int32_t* idx = reinterpret_cast<int32_t*>(base + w.idx);
  float* wts = reinterpret_cast<float*>(base + w.wts);
  int32_t* bk = reinterpret_cast<int32_t*>(base + w.bucket);
  float* hr = reinterpret_cast<float*>(base + w.hr);
  float* hs = reinterpret_cast<float*>(base + w.hs);
  float* dr = reinterpret_cast<float*>(base + w.dr);
  float* ds = reinterpret_cast<float*>(base + w.ds);
  HeadPartial* parts = reinterpret_cast<HeadPartial*>(base + w.partials);
  const int k = d.top_k, E = d.n_experts, I = d.expert_width, Is = d.shared_width, nb = B * k;
  const int Umax = nb < E ? nb : E;
  hipError_t e = hipMemcpyAsync(h, x, 4 * (size_t)B * kHidden, hipMemcpyDeviceToDevice, s);
  for (int l = 0; l < L && e == hipSuccess; ++l) {
    const flint_moe_layer& Ly = layers[l];
    k_bnorm<<<B, kThreads, 0, s>>>(h, u, eps);
    k_broute<<<(E + 3) / 4, kThreads, 0, s>>>(Ly.router, E, u, B, lg);
    k_btopk<<<B, 64, 0, s>>>(lg, E, k, idx, wts);
    if (routes) e = hipMemcpyAsync(routes + (size_t)l * nb, idx, 4 * (size_t)nb, hipMemcpyDeviceToDevice, s);
    k_bucket<<<1, kThreads, 0, s>>>(idx, nb, E, bk);
    k_bgateup<<<dim3((I + 4 * kRowsPerWave - 1) / (4 * kRowsPerWave), Umax), kThreads, 0, s>>>(Ly, I, k, u, bk, hr);
    k_bgateup_shared<<<Is / 4, kThreads, 0, s>>>(Ly, Is, B, u, hs);
    switch (I / 32) {
      case 8: e = launch_bdown_routed<8>(Ly, I, Umax, bk, wts, hr, dr, s); break;
      case 16: e = launch_bdown_routed<16>(Ly, I, Umax, bk, wts, hr, dr, s); break;
      case 32: e = launch_bdown_routed<32>(Ly, I, Umax, bk, wts, hr, dr, s); break;
      case 64: e = launch_bdown_routed<64>(Ly, I, Umax, bk, wts, hr, dr, s); break;
      default: e = hipErrorInvalidValue;
    }
    if (e != hipSuccess) break;
    switch (Is / 32) {
      case 8: e = launch_bdown_shared<8>(Ly, B, hs, ds, s); break;
      case 16: e = launch_bdown_shared<16>(Ly, B, hs, ds, s); break;
      case 32: e = launch_bdown_shared<32>(Ly, B, hs, ds, s); break;
      case 64: e = launch_bdown_shared<64>(Ly, B, hs, ds, s); break;
      default: e = hipErrorInvalidValue;
    }
    if (e != hipSuccess) break;
    k_bcombine<<<dim3(kHidden / kThreads, B), kThreads, 0, s>>>(h, dr, ds, k);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  k_bnorm<<<B, kThreads, 0, s>>>(h, u, eps);
  for (int b0 = 0; b0 < B; b0 += kBHeadMaxTok) {
    const int n = B - b0 < kBHeadMaxTok ? B - b0 : kBHeadMaxTok;
    k_bhead<<<kBHeadBlocks, kThreads, 0, s>>>(head.codes, head.scales, head.tscale, vocab, u, b0, n, logits, parts);
  }
  k_bargmax<<<B, 64, 0, s>>>(parts, kBHeadBlocks, argmax);
  return hipGetLastError();
}

}  // namespace flint
