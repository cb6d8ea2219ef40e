// attn.hip -- the rest of a decode step for gfx950: one grouped-query
// attention layer over a BF16 key/value cache, the dense SwiGLU MLP, and the
// generic NVFP4 GEMV both are built from.
//
// Method [P3 "Flint: 125 tokens a second is what 2.5B active parameters buy
// at 273 GB/s", "The shape, read from the headers": 32 query heads over 4
// key/value heads of dimension 128, per-head QK RMSNorm, learned per-head
// sinks, sliding-window (513) layers with RoPE and full-context layers
// without positional encoding; "Why active parameters set the speed": a BF16
// key and value per token and layer; "Built from scratch?": dense MLP layers
// 6,144 wide].
//
// One attention layer at batch 1 is four launches:
//   k_gemv       q, k, v rows of three NVFP4 matrices, K = 2048
//   k_attn       grid: context chunks x key/value heads -- head norms and
//                RoPE of the group's queries, the current key/value written
//                to the cache, flash-decoding over 64-position sub-chunks
//                staged in LDS; one record (max, sum, o) per chunk and head
//   k_attn_merge one workgroup per query head: the chunk records and the sink
//   k_gemv       o rows, K = n_q * 128
// Every stage is bound by HBM bandwidth: weights and cache rows are read
// once per token with 128-bit loads.
#include <float.h>
#include <math.h>

#include "../../include/flint_attn.h"
#include "flint_common.h"
#include "flint_device.h"

namespace flint {
namespace {

constexpr int kHid = 2048;        // the hidden size with kernels
constexpr int kD = 128;           // head dimension
constexpr int kSub = 64;          // positions per sub-chunk: one per lane
constexpr int kMaxChunks = 256;   // context chunks per key/value head
constexpr int kKRow = 65;         // LDS key row stride in dwords: lane t reads bank (t + dp) mod 64
static_assert(kMaxChunks % 64 == 0, "the merge holds kMaxChunks / 64 chunks per lane");
constexpr int kMaxGroup = 8;      // query heads per key/value head
constexpr int kPart = kD + 2;     // chunk record: running max, sum, o[128]
constexpr int kMaxDenseB = 64;

inline size_t al256(size_t v) { return (v + 255) / 256 * 256; }

// --------------------------------------------------------- NVFP4 GEMV ------
struct GemvMat {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tscale;
  int rows;
};
struct GemvSet {
  GemvMat m[3];
};

// y[b][r] = S * (W[r] . x_b) over the rows of up to three matrices stacked
// (all rows of m[0], then m[1], then m[2]); with PAIR the rows of m[0] and
// m[1] are taken together: y[b][r] = silu(S0 W0[r].x_b) * (S1 W1[r].x_b).
// K = KI * 2048: lane l holds x[i*2048 + 32l .. +31] for i < KI in registers
// and reads 16 code bytes and 2 scale bytes per row and i.  A wave takes R
// rows per step (their loads issued together), waves stride over the rows;
// grid.y is the token.
// norm_eps >= 0: x is first scaled by 1 / sqrt(mean(x^2) + norm_eps) (RMSNorm
// with unit gain, every wave over the whole vector); accumulate: y += result.
template <int KI, int R, bool PAIR>
__global__ __launch_bounds__(256) void k_gemv(GemvSet M, int total_rows, const float* __restrict__ x, int ldx,
                                              float* __restrict__ y, int ldy, float norm_eps, int accumulate) {
  constexpr int K = KI * kHid;
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.y;
  float xv[KI * 32];
  const float* xb = x + (size_t)b * ldx;
#pragma unroll
  for (int i = 0; i < KI; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 v = *reinterpret_cast<const float4*>(xb + i * kHid + 32 * lane + 4 * q);
      xv[32 * i + 4 * q + 0] = v.x;
      xv[32 * i + 4 * q + 1] = v.y;
      xv[32 * i + 4 * q + 2] = v.z;
      xv[32 * i + 4 * q + 3] = v.w;
    }
  if (norm_eps >= 0.0f) {
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < KI * 32; ++i) ss = __builtin_fmaf(xv[i], xv[i], ss);
    const float r = 1.0f / sqrtf(wave_sum(ss) * (1.0f / K) + norm_eps);
#pragma unroll
    for (int i = 0; i < KI * 32; ++i) xv[i] *= r;
  }
  const int nwaves = gridDim.x * 4;
  for (int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * R; r0 < total_rows; r0 += nwaves * R) {
    uint4 c[R][KI], c2[PAIR ? R : 1][KI];
    uint32_t s[R][KI], s2[PAIR ? R : 1][KI];
    float S[R], S2[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
      int lr = min(r0 + j, total_rows - 1);
      const uint8_t* cp = M.m[0].codes;
      const uint8_t* sp = M.m[0].scales;
      const float* tp = M.m[0].tscale;
      if (!PAIR && lr >= M.m[0].rows) {
        lr -= M.m[0].rows;
        if (lr >= M.m[1].rows) {
          lr -= M.m[1].rows;
          cp = M.m[2].codes; sp = M.m[2].scales; tp = M.m[2].tscale;
        } else {
          cp = M.m[1].codes; sp = M.m[1].scales; tp = M.m[1].tscale;
        }
      }
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        c[j][i] = ld_nt_u4(cp + (size_t)lr * (K / 2) + i * (kHid / 2) + 16 * lane);
        s[j][i] = ld_nt_u16(sp + (size_t)lr * (K / 16) + i * (kHid / 16) + 2 * lane);
      }
      S[j] = *tp;
      if constexpr (PAIR) {
#pragma unroll
        for (int i = 0; i < KI; ++i) {
          c2[j][i] = ld_nt_u4(M.m[1].codes + (size_t)lr * (K / 2) + i * (kHid / 2) + 16 * lane);
          s2[j][i] = ld_nt_u16(M.m[1].scales + (size_t)lr * (K / 16) + i * (kHid / 16) + 2 * lane);
        }
        S2[j] = *M.m[1].tscale;
      }
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < KI; ++i) a += nvfp4_lane_dot32(c[j][i], s[j][i], xv + 32 * i);
      float v = wave_sum(a) * S[j];
      if constexpr (PAIR) {
        float a2 = 0.0f;
#pragma unroll
        for (int i = 0; i < KI; ++i) a2 += nvfp4_lane_dot32(c2[j][i], s2[j][i], xv + 32 * i);
        v = silu(v) * (wave_sum(a2) * S2[j]);
      }
      if (lane == 0 && r0 + j < total_rows) {
        float* yp = y + (size_t)b * ldy + r0 + j;
        *yp = accumulate ? *yp + v : v;
      }
    }
  }
}

template <int KI, int R, bool PAIR>
hipError_t gemv_launch(const GemvSet& M, int rows, const float* x, int ldx, float* y, int ldy, int B, float norm_eps,
                       bool acc, hipStream_t st) {
  const int waves = (rows + R - 1) / R;
  int blocks = (waves + 3) / 4;
  if (blocks > 2048) blocks = 2048;
  k_gemv<KI, R, PAIR><<<dim3(blocks, B), 256, 0, st>>>(M, rows, x, ldx, y, ldy, norm_eps, acc ? 1 : 0);
  return hipGetLastError();
}

// K in {2048, 4096, 6144, 8192}; PAIR only at K = 2048
hipError_t launch_gemv(const GemvSet& M, int rows, int K, bool pair, const float* x, int ldx, float* y, int ldy,
                       int B, hipStream_t st, float norm_eps = -1.0f, bool acc = false) {
  if (pair) return gemv_launch<1, 2, true>(M, rows, x, ldx, y, ldy, B, norm_eps, acc, st);
  switch (K / kHid) {
    case 1: return gemv_launch<1, 4, false>(M, rows, x, ldx, y, ldy, B, norm_eps, acc, st);
    case 2: return gemv_launch<2, 2, false>(M, rows, x, ldx, y, ldy, B, norm_eps, acc, st);
    case 3: return gemv_launch<3, 2, false>(M, rows, x, ldx, y, ldy, B, norm_eps, acc, st);
    default: return gemv_launch<4, 2, false>(M, rows, x, ldx, y, ldy, B, norm_eps, acc, st);
  }
}

// ------------------------------------------------------------ attention --
__device__ __forceinline__ uint32_t bf16_rne(float f) {  // finite f
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

struct AttnArgs {
  const float* qkv;  // raw q [n_q*D], k [n_kv*D], v [n_kv*D] of this token
  const float* q_norm;
  const float* k_norm;
  const float* sinks;
  uint16_t* kc;  // [n_kv][cap][D]
  uint16_t* vc;
  long long cap, pos, first;
  int n_q, n_kv, group;
  int per;      // sub-chunks per chunk
  int n_sub;    // sub-chunks in first .. pos
  int nchunks;  // chunks per key/value head (= grid.x)
  int rope;
  float eps;
  float rope_cos[kD / 2], rope_sin[kD / 2];  // angle of pair i at pos (host, double)
  float* part;  // [n_kv][kMaxGroup][kMaxChunks][kPart]
};

// The cache rows of sub-chunk s for key/value head g: thread tid loads 16
// bytes (segment tid & 15) of rows (tid >> 4) + 16 j of the keys and of the
// values; rows at or past pos are zero.  Positions fit in 32 bits (pos and
// cap are int32 at the boundary), so the ring slot is a 32-bit remainder;
// every load is issued whatever the row (a masked row reads slot 0) and the
// eight are independent, so they are in flight together.
__device__ __forceinline__ void attn_load_sub(const AttnArgs& A, int g, int tid, int s, uint4 (&kk)[4],
                                              uint4 (&vv)[4]) {
  const uint32_t cap = (uint32_t)A.cap, pos = (uint32_t)A.pos;
  const uint32_t p0 = (uint32_t)A.first + (uint32_t)s * kSub;
  const size_t head = (size_t)g * (size_t)cap;
  const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t t = p0 + (uint32_t)(tid >> 4) + 16u * (uint32_t)j;
    const bool ok = t < pos;
    const size_t off = (head + (ok ? t : 0u) % cap) * kD + (size_t)(tid & 15) * 8;
    const uint4 kr = *reinterpret_cast<const uint4*>(A.kc + off);
    const uint4 vr = *reinterpret_cast<const uint4*>(A.vc + off);
    kk[j] = ok ? kr : zero;
    vv[j] = ok ? vr : zero;
  }
}

// grid (nchunks, n_kv), 256 threads.  Chunk c covers sub-chunks
// [c*per, min((c+1)*per, n_sub)) of 64 positions from `first`; the last chunk
// holds `pos`.  Wave w owns query heads 2w and 2w+1 of the group (a second
// head past the group is computed on a copy of the first and dropped).
__global__ __launch_bounds__(256) void k_attn(AttnArgs A) {
  __shared__ uint32_t sK[kSub * kKRow];  // key BF16 pairs, [position][dim pair], padded rows
  __shared__ uint32_t sV[kSub * 64];     // value BF16 pairs, [position][dim pair]
  __shared__ __align__(16) float sq[kMaxGroup][kD];    // queries: normalised, rotated, / sqrt(D)
  __shared__ __align__(16) float sp[kMaxGroup][kSub];  // probabilities of the current sub-chunk
  __shared__ __align__(16) uint16_t scur[2][kD];       // this token's key and value (BF16)
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g = blockIdx.y, c = blockIdx.x;
  const int nq = A.n_q * kD, nk = A.n_kv * kD;
  const int s_begin = c * A.per;
  const int s_end = min(s_begin + A.per, A.n_sub);
  const bool has_cur = (s_end == A.n_sub);
  const long long cur_slot = A.pos % A.cap;

  // cache rows of one sub-chunk: thread tid loads 16 bytes (segment tid & 15)
  // of rows (tid >> 4) + 16 j; rows at or past pos are zero here
  uint4 kk[4], vv[4];
  attn_load_sub(A, g, tid, s_begin, kk, vv);

  const float cs = A.rope ? A.rope_cos[lane] : 1.0f, sn = A.rope ? A.rope_sin[lane] : 0.0f;
  const float qscale = 0.08838834764831845f;  // 1 / sqrt(128)
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int hh = 2 * wv + k;
    if (hh < A.group) {
      const int h = g * A.group + hh;
      float a = A.qkv[h * kD + lane], b = A.qkv[h * kD + 64 + lane];
      const float r = 1.0f / sqrtf(wave_sum(a * a + b * b) * (1.0f / kD) + A.eps);
      a = a * r * A.q_norm[lane];
      b = b * r * A.q_norm[lane + 64];
      if (A.rope) {
        const float a2 = a * cs - b * sn;
        b = a * sn + b * cs;
        a = a2;
      }
      sq[hh][lane] = a * qscale;
      sq[hh][lane + 64] = b * qscale;
    }
  }
  // this token's key (wave 0) and value (wave 1), rounded to BF16, into the
  // cache slot of pos and into LDS for the last sub-chunk
  if (has_cur && wv < 2) {
    const float* src = A.qkv + nq + (wv == 0 ? 0 : nk) + g * kD;
    float a = src[lane], b = src[lane + 64];
    if (wv == 0) {
      const float r = 1.0f / sqrtf(wave_sum(a * a + b * b) * (1.0f / kD) + A.eps);
      a = a * r * A.k_norm[lane];
      b = b * r * A.k_norm[lane + 64];
      if (A.rope) {
        const float a2 = a * cs - b * sn;
        b = a * sn + b * cs;
        a = a2;
      }
    }
    const uint16_t ba = (uint16_t)bf16_rne(a), bb = (uint16_t)bf16_rne(b);
    uint16_t* dst = (wv == 0 ? A.kc : A.vc) + ((long long)g * A.cap + cur_slot) * kD;
    dst[lane] = ba;
    dst[lane + 64] = bb;
    scur[wv][lane] = ba;
    scur[wv][lane + 64] = bb;
  }

  const int h0 = min(2 * wv, A.group - 1), h1 = min(2 * wv + 1, A.group - 1);
  const bool act = 2 * wv < A.group;  // wave-uniform
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};
  float o_run[2][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}};
  for (int s = s_begin; s < s_end; ++s) {
    const long long p0 = A.first + (long long)s * kSub;
    const int nvalid = (int)min((long long)kSub, A.pos + 1 - p0);
    __syncthreads();  // LDS of the previous sub-chunk consumed; sq, scur written
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = (tid >> 4) + 16 * j, seg = tid & 15;
      uint4 kw = kk[j], vw = vv[j];
      if (p0 + r == A.pos) {
        kw = *reinterpret_cast<const uint4*>(&scur[0][seg * 8]);
        vw = *reinterpret_cast<const uint4*>(&scur[1][seg * 8]);
      }
      *reinterpret_cast<uint4*>(&sV[r * 64 + seg * 4]) = vw;
      sK[r * kKRow + seg * 4 + 0] = kw.x;
      sK[r * kKRow + seg * 4 + 1] = kw.y;
      sK[r * kKRow + seg * 4 + 2] = kw.z;
      sK[r * kKRow + seg * 4 + 3] = kw.w;
    }
    if (s + 1 < s_end) attn_load_sub(A, g, tid, s + 1, kk, vv);
    __syncthreads();
    if (act) {
      // scores of both heads at position t = lane: four independent chains
      float a0 = 0.0f, a1 = 0.0f, b0 = 0.0f, b1 = 0.0f;
      const float2* q0 = reinterpret_cast<const float2*>(sq[h0]);
      const float2* q1 = reinterpret_cast<const float2*>(sq[h1]);
#pragma unroll 16
      for (int dp = 0; dp < 64; ++dp) {
        const uint32_t w = sK[lane * kKRow + dp];
        const float k0 = bf16_lo(w), k1 = bf16_hi(w);
        const float2 qa = q0[dp], qb = q1[dp];
        a0 = __builtin_fmaf(qa.x, k0, a0);
        a1 = __builtin_fmaf(qa.y, k1, a1);
        b0 = __builtin_fmaf(qb.x, k0, b0);
        b1 = __builtin_fmaf(qb.y, k1, b1);
      }
      const float sc[2] = {lane < nvalid ? a0 + a1 : -INFINITY, lane < nvalid ? b0 + b1 : -INFINITY};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float m_new = fmaxf(m_run[k], wave_max(sc[k]));
        const float p = lane < nvalid ? __expf(sc[k] - m_new) : 0.0f;
        const float alpha = (m_run[k] == -INFINITY) ? 0.0f : __expf(m_run[k] - m_new);
        l_run[k] = l_run[k] * alpha + wave_sum(p);
        o_run[k][0] *= alpha;
        o_run[k][1] *= alpha;
        m_run[k] = m_new;
        sp[2 * wv + k][lane] = p;  // rows of this wave only
      }
    }
    __syncthreads();
    if (act) {
      // o += p_t V_t over all 64 rows (p = 0 and V = 0 past the valid ones);
      // lane owns dims 2 lane, 2 lane + 1
      float x0 = 0.0f, x1 = 0.0f, y0 = 0.0f, y1 = 0.0f, z0 = 0.0f, z1 = 0.0f, w0 = 0.0f, w1 = 0.0f;
      const float4* p0v = reinterpret_cast<const float4*>(sp[2 * wv]);
      const float4* p1v = reinterpret_cast<const float4*>(sp[2 * wv + 1]);
#pragma unroll 4
      for (int t4 = 0; t4 < kSub / 4; ++t4) {
        const float4 pa = p0v[t4], pb = p1v[t4];
        const uint32_t v0 = sV[(4 * t4 + 0) * 64 + lane], v1 = sV[(4 * t4 + 1) * 64 + lane];
        const uint32_t v2 = sV[(4 * t4 + 2) * 64 + lane], v3 = sV[(4 * t4 + 3) * 64 + lane];
        x0 = __builtin_fmaf(pa.x, bf16_lo(v0), x0); x1 = __builtin_fmaf(pa.x, bf16_hi(v0), x1);
        y0 = __builtin_fmaf(pa.y, bf16_lo(v1), y0); y1 = __builtin_fmaf(pa.y, bf16_hi(v1), y1);
        x0 = __builtin_fmaf(pa.z, bf16_lo(v2), x0); x1 = __builtin_fmaf(pa.z, bf16_hi(v2), x1);
        y0 = __builtin_fmaf(pa.w, bf16_lo(v3), y0); y1 = __builtin_fmaf(pa.w, bf16_hi(v3), y1);
        z0 = __builtin_fmaf(pb.x, bf16_lo(v0), z0); z1 = __builtin_fmaf(pb.x, bf16_hi(v0), z1);
        w0 = __builtin_fmaf(pb.y, bf16_lo(v1), w0); w1 = __builtin_fmaf(pb.y, bf16_hi(v1), w1);
        z0 = __builtin_fmaf(pb.z, bf16_lo(v2), z0); z1 = __builtin_fmaf(pb.z, bf16_hi(v2), z1);
        w0 = __builtin_fmaf(pb.w, bf16_lo(v3), w0); w1 = __builtin_fmaf(pb.w, bf16_hi(v3), w1);
      }
      o_run[0][0] += x0 + y0;
      o_run[0][1] += x1 + y1;
      o_run[1][0] += z0 + w0;
      o_run[1][1] += z1 + w1;
    }
  }
  // chunk records
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int hh = 2 * wv + k;
    if (hh < A.group) {
      float* P = A.part + (((size_t)g * kMaxGroup + hh) * kMaxChunks + c) * kPart;
      if (lane == 0) {
        P[0] = m_run[k];
        P[1] = l_run[k];
      }
      *reinterpret_cast<float2*>(P + 2 + 2 * lane) = make_float2(o_run[k][0], o_run[k][1]);
    }
  }
}

// grid (n_q), 256 threads: query head h merges its chunk records with the
// sink.  All loads are issued at once: wave w takes chunks w, w+4, ... for
// the dim pair of its lane; lanes over chunks (kMaxChunks / 64 each) give the
// maximum M, the weights f_c = e^(m_c - M) and Z; the four waves' sums meet
// in LDS.
template <int NC>  // NC >= nchunks: 64 or kMaxChunks
__global__ __launch_bounds__(256) void k_attn_merge(const float* __restrict__ part, const float* __restrict__ sinks,
                                                    int group, int nchunks, float* __restrict__ o) {
  constexpr int kPerLane = NC / 64;
  __shared__ float2 sred[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int h = blockIdx.x, g = h / group, hh = h % group;
  const float* P0 = part + ((size_t)g * kMaxGroup + hh) * kMaxChunks * kPart;
  float2 ov[NC / 4];
#pragma unroll
  for (int i = 0; i < NC / 4; ++i) {
    const int cc = wv + 4 * i;
    ov[i] = cc < nchunks ? *reinterpret_cast<const float2*>(P0 + cc * kPart + 2 + 2 * lane) : make_float2(0.f, 0.f);
  }
  float m[kPerLane], l[kPerLane];
  const float sink = sinks[h];
  float M = sink;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int cc = lane + 64 * i;
    m[i] = cc < nchunks ? P0[cc * kPart] : -INFINITY;
    l[i] = cc < nchunks ? P0[cc * kPart + 1] : 0.0f;
    M = fmaxf(M, m[i]);
  }
  M = wave_max(M);
  float f[kPerLane], zl = 0.0f;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    f[i] = (lane + 64 * i) < nchunks ? __expf(m[i] - M) : 0.0f;
    zl = __builtin_fmaf(f[i], l[i], zl);
  }
  const float Z = wave_sum(zl) + __expf(sink - M);
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int i = 0; i < NC / 4; ++i) {
    const int cc = wv + 4 * i;  // wave-uniform
    float fi = f[0];
#pragma unroll
    for (int q = 1; q < kPerLane; ++q)
      if ((cc >> 6) == q) fi = f[q];
    const float fc = lane_f32(fi, cc & 63);
    a0 = __builtin_fmaf(fc, ov[i].x, a0);
    a1 = __builtin_fmaf(fc, ov[i].y, a1);
  }
  sred[wv][lane] = make_float2(a0, a1);
  __syncthreads();
  if (wv == 0) {
    float2 t = sred[0][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      t.x += sred[w][lane].x;
      t.y += sred[w][lane].y;
    }
    *reinterpret_cast<float2*>(o + h * kD + 2 * lane) = make_float2(t.x / Z, t.y / Z);
  }
}

// Short contexts (nchunks <= 16): one wave per query head, every record of
// the head requested at once, no LDS.  Same rule as k_attn_merge.
__global__ __launch_bounds__(64) void k_attn_merge16(const float* __restrict__ part, const float* __restrict__ sinks,
                                                     int group, int nchunks, float* __restrict__ o) {
  const int lane = threadIdx.x, h = blockIdx.x, g = h / group, hh = h % group;
  const float* P0 = part + ((size_t)g * kMaxGroup + hh) * kMaxChunks * kPart;
  float2 ov[16];
#pragma unroll
  for (int cc = 0; cc < 16; ++cc)
    ov[cc] = cc < nchunks ? *reinterpret_cast<const float2*>(P0 + cc * kPart + 2 + 2 * lane) : make_float2(0.f, 0.f);
  const float mc = lane < nchunks ? P0[lane * kPart] : -INFINITY;
  const float lc = lane < nchunks ? P0[lane * kPart + 1] : 0.0f;
  const float sink = sinks[h];
  const float M = wave_max(fmaxf(mc, sink));
  const float f = lane < nchunks ? __expf(mc - M) : 0.0f;
  const float Z = wave_sum(f * lc) + __expf(sink - M);
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int cc = 0; cc < 16; ++cc) {
    const float fc = lane_f32(f, cc);  // 0 past nchunks
    a0 = __builtin_fmaf(fc, ov[cc].x, a0);
    a1 = __builtin_fmaf(fc, ov[cc].y, a1);
  }
  *reinterpret_cast<float2*>(o + h * kD + 2 * lane) = make_float2(a0 / Z, a1 / Z);
}

// --------------------------------------------------------- host helpers --
struct AttnWs {
  size_t qkv, o, part, total;
  explicit AttnWs(const flint_attn_dims& d) {
    const size_t nq = (size_t)d.n_q_heads * kD, nk = (size_t)d.n_kv_heads * kD;
    size_t off = 0;
    qkv = off; off = al256(off + 4 * (nq + 2 * nk));
    o = off; off = al256(off + 4 * nq);
    part = off; off = al256(off + 4 * (size_t)d.n_kv_heads * kMaxGroup * kMaxChunks * kPart);
    total = off;
  }
};

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int32_t check_attn_dims(const flint_attn_dims* d) {
  if (!d) return FLINT_E_NULL;
  if (d->hidden < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 2 || d->head_dim % 2 ||
      d->n_q_heads % d->n_kv_heads || d->window < 0 || (d->rope != 0 && d->rope != 1) || !(d->eps >= 0.0f) ||
      (d->rope && !(d->rope_theta > 0.0f)))
    return FLINT_E_DIMS;
  if (d->hidden != kHid || d->head_dim != kD || d->n_q_heads % 16 || d->n_q_heads > 64 ||
      d->n_q_heads / d->n_kv_heads > kMaxGroup)
    return FLINT_E_UNSUPPORTED;
  return FLINT_OK;
}

int32_t check_mat(const flint_nvfp4* q) {
  if (!q || !q->codes || !q->scales || !q->tscale) return FLINT_E_NULL;
  if (!al16(q->codes) || !al4(q->scales) || !al4(q->tscale)) return FLINT_E_ALIGN;
  return FLINT_OK;
}

GemvMat gm(const flint_nvfp4& q, int rows) { return GemvMat{q.codes, q.scales, q.tscale, rows}; }

}  // namespace
}  // namespace flint

int32_t flint::attn_check(const flint_attn_dims* dims, const flint_attn_layer* layer, int pos, const void* kc,
                          const void* vc, int cap) {
  int32_t st;
  if ((st = check_attn_dims(dims))) return st;
  if (!layer || !kc || !vc) return FLINT_E_NULL;
  if (!layer->q_norm || !layer->k_norm || !layer->sinks) return FLINT_E_NULL;
  if ((st = check_mat(&layer->q)) || (st = check_mat(&layer->k)) || (st = check_mat(&layer->v)) ||
      (st = check_mat(&layer->o)))
    return st;
  if (pos < 0 || cap < 1) return FLINT_E_DIMS;
  if (dims->window > 0 ? cap < dims->window : cap <= pos) return FLINT_E_DIMS;
  if (!al16(kc) || !al16(vc) || !al4(layer->q_norm) || !al4(layer->k_norm) || !al4(layer->sinks))
    return FLINT_E_ALIGN;
  return FLINT_OK;
}

size_t flint::attn_ws_bytes(const flint_attn_dims& d) { return AttnWs(d).total; }
size_t flint::attn_qkv_offset(const flint_attn_dims& d) { return AttnWs(d).qkv; }

hipError_t flint::attn_run(const flint_attn_dims& d, const flint_attn_layer& layer, const float* x, float norm_eps,
                           int pos, uint16_t* k_cache, uint16_t* v_cache, int cap, float* y, bool accumulate, void* ws,
                           hipStream_t s, bool qkv_ready) {
  const AttnWs w(d);
  char* base = static_cast<char*>(ws);
  float* qkv = reinterpret_cast<float*>(base + w.qkv);
  float* o = reinterpret_cast<float*>(base + w.o);
  const int nq = d.n_q_heads * kD, nk = d.n_kv_heads * kD;

  hipError_t e = hipSuccess;
  if (!qkv_ready) {
    GemvSet in{};
    in.m[0] = gm(layer.q, nq);
    in.m[1] = gm(layer.k, nk);
    in.m[2] = gm(layer.v, nk);
    e = launch_gemv(in, nq + 2 * nk, kHid, false, x, 0, qkv, 0, 1, s, norm_eps);
    if (e != hipSuccess) return e;
  }

  AttnArgs A{};
  A.qkv = qkv;
  A.q_norm = layer.q_norm;
  A.k_norm = layer.k_norm;
  A.sinks = layer.sinks;
  A.kc = k_cache;
  A.vc = v_cache;
  A.cap = cap;
  A.pos = pos;
  A.first = (d.window > 0 && pos - d.window + 1 > 0) ? pos - d.window + 1 : 0;
  A.n_q = d.n_q_heads;
  A.n_kv = d.n_kv_heads;
  A.group = d.n_q_heads / d.n_kv_heads;
  const long long n = (long long)pos - A.first + 1;
  A.n_sub = (int)((n + kSub - 1) / kSub);
  A.per = (A.n_sub + kMaxChunks - 1) / kMaxChunks;
  A.nchunks = (A.n_sub + A.per - 1) / A.per;
  A.rope = d.rope;
  A.eps = d.eps;
  for (int i = 0; i < kD / 2; ++i) {
    const double ang = d.rope ? (double)pos * pow((double)d.rope_theta, -2.0 * i / kD) : 0.0;
    A.rope_cos[i] = (float)cos(ang);
    A.rope_sin[i] = (float)sin(ang);
  }
  A.part = reinterpret_cast<float*>(base + w.part);
  k_attn<<<dim3(A.nchunks, d.n_kv_heads), 256, 0, s>>>(A);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (A.nchunks <= 16)
    k_attn_merge16<<<d.n_q_heads, 64, 0, s>>>(A.part, layer.sinks, A.group, A.nchunks, o);
  else if (A.nchunks <= 64)
    k_attn_merge<64><<<d.n_q_heads, 256, 0, s>>>(A.part, layer.sinks, A.group, A.nchunks, o);
  else
    k_attn_merge<kMaxChunks><<<d.n_q_heads, 256, 0, s>>>(A.part, layer.sinks, A.group, A.nchunks, o);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  GemvSet out{};
  out.m[0] = gm(layer.o, kHid);
  return launch_gemv(out, kHid, nq, false, o, 0, y, 0, 1, s, -1.0f, accumulate);
}

int32_t flint::dense_check(const flint_nvfp4* gate, const flint_nvfp4* up, const flint_nvfp4* down, int hidden,
                           int width) {
  int32_t st;
  if ((st = check_mat(gate)) || (st = check_mat(up)) || (st = check_mat(down))) return st;
  if (hidden < 1 || width < 1) return FLINT_E_DIMS;
  if (hidden != kHid || width % kHid || width > 4 * kHid) return FLINT_E_UNSUPPORTED;
  return FLINT_OK;
}

hipError_t flint::dense_run(const flint_nvfp4& gate, const flint_nvfp4& up, const flint_nvfp4& down, int width,
                            const float* x, float norm_eps, float* y, bool accumulate, void* ws, hipStream_t s) {
  float* h = static_cast<float*>(ws);
  GemvSet gu{};
  gu.m[0] = gm(gate, width);
  gu.m[1] = gm(up, width);
  hipError_t e = launch_gemv(gu, width, kHid, true, x, kHid, h, width, 1, s, norm_eps);
  if (e != hipSuccess) return e;
  GemvSet dn{};
  dn.m[0] = gm(down, kHid);
  return launch_gemv(dn, kHid, width, false, h, width, y, kHid, 1, s, -1.0f, accumulate);
}

using namespace flint;

extern "C" {

size_t flint_attn_workspace_bytes(const flint_attn_dims* dims) {
  if (check_attn_dims(dims) != FLINT_OK) return 0;
  return AttnWs(*dims).total;
}

int32_t flint_attn_decode(const flint_attn_dims* dims, const flint_attn_layer* layer, const float* x, int32_t pos,
                          uint16_t* k_cache, uint16_t* v_cache, int32_t cap, float* y, void* ws, size_t ws_bytes,
                          void* stream) {
  int32_t st;
  if ((st = check_attn_dims(dims))) return st;
  if (!x || !y || !ws) return FLINT_E_NULL;
  if ((st = attn_check(dims, layer, pos, k_cache, v_cache, cap))) return st;
  if (!al16(x) || !al16(y) || !al16(ws)) return FLINT_E_ALIGN;
  if (ws_bytes < AttnWs(*dims).total) return FLINT_E_WORKSPACE;
  if ((st = api_check_device())) return st;
  hipError_t e = attn_run(*dims, *layer, x, -1.0f, pos, k_cache, v_cache, cap, y, false, ws, (hipStream_t)stream);
  return e == hipSuccess ? FLINT_OK : api_hip_fail(e);
}

size_t flint_dense_workspace_bytes(int32_t hidden, int32_t width, int32_t B) {
  if (hidden != kHid || width < kHid || width % kHid || width > 4 * kHid || B < 1 || B > kMaxDenseB) return 0;
  return al256(4 * (size_t)B * width);
}

int32_t flint_dense_mlp(const flint_nvfp4* gate, const flint_nvfp4* up, const flint_nvfp4* down, int32_t hidden,
                        int32_t width, const float* x, int32_t B, float* y, void* ws, size_t ws_bytes, void* stream) {
  int32_t st;
  if ((st = check_mat(gate)) || (st = check_mat(up)) || (st = check_mat(down))) return st;
  if (!x || !y || !ws) return FLINT_E_NULL;
  if (hidden < 1 || width < 1 || B < 1) return FLINT_E_DIMS;
  if (hidden != kHid || width % kHid || width > 4 * kHid || B > kMaxDenseB) return FLINT_E_UNSUPPORTED;
  if (!al16(x) || !al16(y) || !al16(ws)) return FLINT_E_ALIGN;
  if (ws_bytes < flint_dense_workspace_bytes(hidden, width, B)) return FLINT_E_WORKSPACE;
  if ((st = api_check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  float* h = static_cast<float*>(ws);
  GemvSet gu{};
  gu.m[0] = gm(*gate, width);
  gu.m[1] = gm(*up, width);
  hipError_t e = launch_gemv(gu, width, kHid, true, x, kHid, h, width, B, s);
  if (e != hipSuccess) return api_hip_fail(e);
  GemvSet dn{};
  dn.m[0] = gm(*down, kHid);
  e = launch_gemv(dn, kHid, width, false, h, width, y, kHid, B, s);
  return e == hipSuccess ? FLINT_OK : api_hip_fail(e);
}

}  // extern "C"
