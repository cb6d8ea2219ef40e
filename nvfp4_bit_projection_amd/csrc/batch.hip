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
//   k_broute     logits[b][e] = router[e] . u_b (one router row per wave, 8
//                tokens per workgroup, fp32)
//   k_btopk      top-k and renormalised softmax per token (one wave per token)
//   k_bucket     (token, slot) pairs grouped by expert, experts in index
//                order, pairs in (token, slot) order
//   k_mm_gateup  h = silu(gate . u) * (up . u) for every chosen expert and its
//                tokens, and for the shared expert and all tokens, on matrix
//                cores (one launch)
//   k_mm_down    the down projections of both, routed outputs weighted by
//                their routing weights (one launch)
//   k_bnorm      h_b += sum over slots (fixed order) + shared, then the next
//                norm u_b = h_b / sqrt(mean(h_b^2) + eps)
// and at the end k_mm_head (rows streamed once for all tokens) + k_bargmax.
// Weights are NVFP4 decoded in registers; results as accurate as fp32.
#include <float.h>
#include <limits.h>

#include <type_traits>

#include "flint_device.h"
#include "flint_common.h"
#include "flint_internal.h"

namespace flint {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint16_t bf16_bits(__bf16 v) { return __builtin_bit_cast(uint16_t, v); }

// x = hi + mid + lo, each bf16 rounded to nearest even (exact for normal x:
// each remainder is exact in fp32 and has 8 fewer significant bits)
__device__ __forceinline__ void split3(float x, uint16_t* o) {
  const __bf16 hi = (__bf16)x;
  const float r1 = x - (float)hi;
  const __bf16 mid = (__bf16)r1;
  const __bf16 lo = (__bf16)(r1 - (float)mid);
  o[0] = bf16_bits(hi);
  o[1] = bf16_bits(mid);
  o[2] = bf16_bits(lo);
}


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

// --------------------------------------------------------------- router --
// grid (ceil(E/4), ceil(B/2)), 256 threads: router row e = 4 blockIdx.x +
// wave, dotted with tokens 2 blockIdx.y, 2 blockIdx.y + 1 (staged in LDS).
// The router is read once per token pair (2 MB, from L2 after the first).
// Two tokens per workgroup measured faster than 4 or 8 (more workgroups,
// less staging each): 6.5% of the step at B = 8, 1% at B = 32.
constexpr int kRouteTok = 2;
__global__ __launch_bounds__(kThreads) void k_broute(const float* __restrict__ router, int E,
                                                     const float* __restrict__ u, int B, float* __restrict__ logits) {
  __shared__ __align__(16) float sh[kRouteTok * (kHidden / 32) * kPad];
  const int lane = threadIdx.x & 63, e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b0 = blockIdx.y * kRouteTok, nb = B - b0 < kRouteTok ? B - b0 : kRouteTok;
  float wr[32];
  {
    const float* rw = router + (size_t)(e < E ? e : 0) * kHidden + 32 * lane;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 a = *reinterpret_cast<const float4*>(rw + 4 * i);
      wr[4 * i] = a.x; wr[4 * i + 1] = a.y; wr[4 * i + 2] = a.z; wr[4 * i + 3] = a.w;
    }
  }
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

// ----------------------------------------------------------------- top-k --
// grid B, 64 threads: 4 logits per lane kept sorted by (value desc, index
// asc); k rounds: wave maximum of the lanes' heads (DPP), the lane holding it
// by a ballot (on a tie between lanes, the lowest index by a wave minimum),
// pop that head; weights exp(l_i - l_0) / sum.
__global__ __launch_bounds__(64) void k_btopk(const float* __restrict__ logits, int E, int k,
                                              int32_t* __restrict__ idx, float* __restrict__ wts) {
  const int b = blockIdx.x, lane = threadIdx.x;
  int key[4], id[4];
  float lv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // all four loads in flight (an index past E reads expert E - 1)
    const int e = lane + 64 * j;
    lv[j] = logits[(size_t)b * E + (e < E ? e : E - 1)];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    id[j] = lane + 64 * j;
    key[j] = id[j] < E ? ord_key(lv[j]) : INT_MIN;
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

// One workgroup of 256 threads (E <= 256, B*k <= 512): per-expert counts by
// LDS atomics (order-free), exclusive scans for each expert's start and each
// chosen expert's rank, then every pair p goes to start[e] + (number of
// earlier pairs with the same expert): pairs in (token, slot) order within
// an expert, experts in index order, independent of timing.
__global__ __launch_bounds__(kThreads) void k_bucket(const int32_t* __restrict__ idx_g, int nb, int E,
                                                     int32_t* __restrict__ bk) {
  const int t = threadIdx.x;
  __shared__ int sh[kThreads / 64];
  __shared__ int idx[kMaxBatch * kMaxTopK];
  __shared__ int cnt[kMaxExperts], start[kMaxExperts];
  cnt[t] = 0;
  for (int p = t; p < nb; p += kThreads) idx[p] = idx_g[p];
  __syncthreads();
  for (int p = t; p < nb; p += kThreads) atomicAdd(&cnt[idx[p]], 1);
  __syncthreads();
  const int c = t < E ? cnt[t] : 0;
  const int st = block_excl_scan(c, sh);
  const int rank = block_excl_scan(c > 0 ? 1 : 0, sh);
  start[t] = st;
  if (c > 0) {
    bk[kBkExperts + rank] = t;
    bk[kBkStart + rank] = st;
  }
  if (t == kThreads - 1) {
    const int U = rank + (c > 0 ? 1 : 0);
    bk[0] = U;
    bk[kBkStart + U] = st + c;
  }
  __syncthreads();
  for (int p = t; p < nb; p += kThreads) {
    const int e = idx[p];
    int before = 0;
    for (int q = 0; q < p; ++q) before += idx[q] == e;
    bk[kBkPairs + start[e] + before] = p;
  }
}

// ------------------------------------------------------ matrix cores --
// The contractions over K run on 16x16x32 matrix-core instructions with
// results as accurate as fp32 arithmetic:
//  - an E2M1 code times its E4M3 block scale has at most 5 significant bits,
//    so every weight is exact in fp16 and in bf16 (decoded in registers; the
//    fp32 tensor scale multiplies the result);
//  - every fp32 activation is split into parts that sum to it, kept as planes
//    [P][rows][K]: two fp16 parts (hi + lo, 22 significant bits) for inputs
//    bounded by an RMSNorm (|u| <= sqrt(H) = 45.3: no fp16 overflow), three
//    bf16 parts (hi + mid + lo, exact for normal values, fp32 range) for the
//    SwiGLU outputs, which have no such bound;
//  - products of two such parts are exact in fp32 and accumulate in fp32.
// A workgroup of 4 waves takes one weight group (a chosen expert, the shared
// expert, or the head) and a range of its rows; each wave takes two 16-row
// tiles; tokens go in passes of 32 (two 16-token tiles).  The pass's
// activation planes are copied into LDS in K segments, gathered by token;
// a lane's weight bytes are requested three 256-wide chunks ahead.
//
// Operand layout (16x16x32, lane l, m = l % 16, q = l / 16): A (tokens x K)
// token m, B (K x rows) row m, each with 8 K values of group q; C (tokens x
// rows) row m, tokens 4q .. 4q+3.  A lane's 32 bytes of codes per chunk hold
// K values 64q .. 64q+63 of the chunk, consumed in 8 steps of 8; the
// activations are staged in the same K order, so the A and B operands of step
// j are K values 64q + 8j .. 64q + 8j + 7.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kMmThreads = 256;
constexpr int kMmWaves = kMmThreads / 64;
constexpr int kMmChunk = 256;                   // K per 32-byte group of a lane's weight codes
constexpr int kMmTok = 32;                      // tokens per pass
constexpr int kMmStage = 8192;                  // values per plane per staged segment (rows x K)
constexpr int kMmGateUpRows = 16 * kMmWaves;    // gate/up row pairs per workgroup
constexpr int kMmRows = 32 * kMmWaves;          // rows per workgroup (down, head)

// The two operand formats.  decode(): the 8 E2M1 codes of a 32-bit word
// (element 2i in the low nibble of byte i) times an E4M3 block scale.
struct FmtF16 {
  static constexpr int P = 2;
  typedef f16x8_t vec;
  struct Scale {
    float p2;     // power-of-two part of the block scale
    _Float16 f;   // the rest: 1 + m/8, or m for a subnormal scale
  };
  static __device__ __forceinline__ Scale scale(uint32_t b) {
    const uint32_t e = (b >> 3) & 15, m = b & 7;
    Scale s;
    s.p2 = __uint_as_float((e ? e + 120u : 118u) << 23);  // 2^(e-7), or 2^-9
    s.f = e ? (_Float16)(1.0f + 0.125f * (float)m) : (_Float16)(float)m;
    return s;
  }
  static __device__ __forceinline__ vec decode(uint32_t w, Scale s) {
    const f16x2_t ff = {s.f, s.f};
    const f16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.p2, 0) * ff;
    const f16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.p2, 1) * ff;
    const f16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.p2, 2) * ff;
    const f16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.p2, 3) * ff;
    return vec{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
  }
  static __device__ __forceinline__ f32x4_t mma(vec a, vec b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // x = hi + lo
  static __device__ __forceinline__ void split(float x, uint16_t* o) {
    const _Float16 hi = (_Float16)x;
    o[0] = __builtin_bit_cast(uint16_t, hi);
    o[1] = __builtin_bit_cast(uint16_t, (_Float16)(x - (float)hi));
  }
};
struct FmtBF16 {
  static constexpr int P = 3;
  typedef bf16x8_t vec;
  typedef float Scale;
  static __device__ __forceinline__ Scale scale(uint32_t b) { return e4m3_to_f32(b); }
  static __device__ __forceinline__ vec decode(uint32_t w, Scale d) {
    const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    vec r;
    r[0] = (__bf16)(v0[0] * d); r[1] = (__bf16)(v0[1] * d);
    r[2] = (__bf16)(v1[0] * d); r[3] = (__bf16)(v1[1] * d);
    r[4] = (__bf16)(v2[0] * d); r[5] = (__bf16)(v2[1] * d);
    r[6] = (__bf16)(v3[0] * d); r[7] = (__bf16)(v3[1] * d);
    return r;
  }
  static __device__ __forceinline__ f32x4_t mma(vec a, vec b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void split(float x, uint16_t* o) { split3(x, o); }
};
template <class F>
constexpr int mm_buf_bytes() { return F::P * kMmStage * 2; }

// One wave's two 16-row weight tiles, in one of two layouts (a type with a
// static load).
// Row-major matrices: c, s point at this lane's first code and scale bytes
// of chunk 0 of each tile; the lane's 32 code bytes of a chunk are contiguous
// (second half 16 bytes on) and chunks are 128 code / 16 scale bytes apart,
// so one address per tile serves every chunk (offsets fit the instruction).
// Tiled copies (flint_stack_batch_tiles): each (16-row tile, chunk) is one
// 2 KB block of codes, lane L = 16 q + m holding bytes 16 L and 1024 + 16 L,
// and one 256-byte block of scales (4 L); the wave's tiles are buffer
// resources rc, rs (16 KB of codes, 2 KB of scales) read at the lane offset
// plus a constant.
struct MmTiles {
  const uint8_t* c[2];
  const uint8_t* s[2];
  rsrc_t rc[2], rs[2];
  uint32_t lane;
};
struct MmRegs {  // a lane's weight bytes of one chunk
  uint4 c[2][2];
  uint32_t s[2];
};
struct MmRowMajor {
  static __device__ __forceinline__ void load(const MmTiles& T, int u, MmRegs& R) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const uint8_t* cp = T.c[rt] + (kMmChunk / 2) * u;
      R.c[rt][0] = ld_nt_u4(cp);
      R.c[rt][1] = ld_nt_u4(cp + 16);
      R.s[rt] = ld_nt_u32(T.s[rt] + (kMmChunk / 16) * u);
    }
  }
};
struct MmTiled {
  static __device__ __forceinline__ void load(const MmTiles& T, int u, MmRegs& R) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      R.c[rt][0] = bload_u4_nt(T.rc[rt], 16 * T.lane + 2048 * u);
      R.c[rt][1] = bload_u4_nt(T.rc[rt], 16 * T.lane + 2048 * u + 1024);
      R.s[rt] = __builtin_amdgcn_raw_buffer_load_b32(T.rs[rt], 4 * T.lane + 256 * u, 0, kAuxNT);
    }
  }
};

// Byte offsets of the down matrices in one layer's tiled copy, after the
// gate/up part: routed codes [E][H/16][I/256][2 KB], shared codes
// [H/16][Is/256][2 KB], routed scales [E][H/16][I/256][256 B], shared scales
// [H/16][Is/256][256 B]; total = the layer's bytes.
struct DownTiles {
  size_t routed_c, shared_c, routed_s, shared_s, total;
  __host__ __device__ DownTiles(int E, int I, int Is) {
    const size_t ntile = (size_t)E * (I / 16) + Is / 16;  // gate/up tiles
    size_t o = 2 * ntile * 16 * (kHidden / 2 + kHidden / 16);
    routed_c = o; o += (size_t)E * kHidden * (I / 2);
    shared_c = o; o += (size_t)kHidden * (Is / 2);
    routed_s = o; o += (size_t)E * kHidden * (I / 16);
    shared_s = o; o += (size_t)kHidden * (Is / 16);
    total = o;
  }
};

// Staged activations: the pass's tokens padded to R rows (a power of two, 4
// .. 32) and a K segment of kseg = min(8192 / R, K) values, P planes, in LDS
// as [plane][row][kseg] 16-bit values; granule g (8 values) of row r sits at
// position g ^ (r % 16), so the rows read in one step hit distinct banks.
// The copy is made of 1 KB buffer-to-LDS loads (64 lanes x 16 B) dealt
// round-robin to the waves; a row without a token reads past the end of the
// planes (zeros, no memory access) and its results are dropped.
__device__ __forceinline__ void mm_stage(rsrc_t rA, int P, int a_rows, int K, const int* srow, int R, int kseg,
                                         int k0, unsigned char* buf, int wv, int lane) {
  const int row_bytes = 2 * kseg, plane_bytes = R * row_bytes, ncopies = P * plane_bytes / 1024;
  for (int cpy = wv; cpy < ncopies; cpy += kMmWaves) {
    const int off = cpy * 1024 + 16 * lane;
    const int p = off / plane_bytes, rem = off % plane_bytes;
    const int r = rem / row_bytes, g = ((rem % row_bytes) >> 4) ^ (r & 15);
    const int tr = srow[r];
    const uint32_t src =
        tr >= 0 ? (uint32_t)((((size_t)p * a_rows + tr) * K + k0 + 8 * g) * 2) : 0xFFFFFFF0u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (__attribute__((address_space(3))) void*)(buf + cpy * 1024), 16, src,
                                             0, 0, 0);
  }
}

// The matrix-core steps of one 256-wide K chunk (chunk c of the staged
// segment): acc[rt][tt] += A(token tile tt) x B(row tile rt) over the planes.
template <class F>
__device__ __forceinline__ void mm_chunk(const MmRegs& R, const unsigned char* buf, int Rrows, int kseg, int c,
                                         int ntt, int lane, f32x4_t (&acc)[2][2]) {
  const int m = lane & 15, q = lane >> 4;
  const int row_bytes = 2 * kseg, plane_bytes = Rrows * row_bytes;
  typename F::Scale d[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) d[rt][i] = F::scale((R.s[rt] >> (8 * i)) & 0xFF);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t w0 = j < 4 ? (&R.c[0][0].x)[j] : (&R.c[0][1].x)[j - 4];
    const uint32_t w1 = j < 4 ? (&R.c[1][0].x)[j] : (&R.c[1][1].x)[j - 4];
    const typename F::vec b0 = F::decode(w0, d[0][j / 2]);
    const typename F::vec b1 = F::decode(w1, d[1][j / 2]);
    const int g = (kMmChunk / 8) * c + 8 * q + j;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (tt < ntt) {
        const int r = (16 * tt + m) & (Rrows - 1);
        const unsigned char* ap = buf + r * row_bytes + ((g ^ (r & 15)) << 4);
#pragma unroll
        for (int p = 0; p < F::P; ++p) {
          const typename F::vec a = *reinterpret_cast<const typename F::vec*>(ap + p * plane_bytes);
          acc[0][tt] = F::mma(a, b0, acc[0][tt]);
          acc[1][tt] = F::mma(a, b1, acc[1][tt]);
        }
      }
    }
  }
}

// One pass: nt (<= 32) tokens whose source rows are in srow, over K = 256
// NCH.  The caller has published srow with a barrier.  The activations are
// staged segment by segment (a barrier pair each); a lane's weight bytes are
// requested AHEAD chunks before they are multiplied (the chunk loop is
// unrolled, so every chunk has its own registers).  From the tiled copy two
// chunks ahead (with the grids sized to each group's rows, better than one
// at B = 32 and than three at B = 8); from row-major weights three are best
// at B = 8 and as good at B = 32.
template <class F, int NCH, class Lay = MmRowMajor, int AHEAD = 2>
__device__ __forceinline__ void mm_pass_n(const MmTiles& T, rsrc_t rA, int a_rows, const int* srow, int nt,
                                          unsigned char* abuf, int wv, int lane, f32x4_t (&acc)[2][2]) {
  constexpr int K = NCH * kMmChunk;
  const int ntt = nt > 16 ? 2 : 1;
  const int Rrows = nt <= 4 ? 4 : nt <= 8 ? 8 : nt <= 16 ? 16 : 32;
  const int kseg = kMmStage / Rrows < K ? kMmStage / Rrows : K, cps = kseg / kMmChunk;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) acc[rt][tt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  MmRegs R[NCH];
#pragma unroll
  for (int u = 0; u < NCH && u < AHEAD; ++u) Lay::load(T, u, R[u]);
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    if (u % cps == 0) {  // next segment: everyone is done with the buffer, then copy
      __syncthreads();
      mm_stage(rA, F::P, a_rows, K, srow, Rrows, kseg, u * kMmChunk, abuf, wv, lane);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies are in
      __syncthreads();
    }
    if (u + AHEAD < NCH) Lay::load(T, u + AHEAD, R[u + AHEAD]);
    mm_chunk<F>(R[u], abuf, Rrows, kseg, u % cps, ntt, lane, acc);
  }
}

// ---------------------------------------------------------------- norm --
// grid B, 1,024 threads.  With dr: the layer's residual update first, h_b +=
// (sum over slots in order of dr) + ds (fixed order).  Then u_b = h_b * s_b,
// s_b = 1/sqrt(mean(h_b^2) + eps), as fp32 (router; skipped when u is null)
// and as two fp16 planes up [2][B][H] (matrix cores; |u| <= sqrt(H), well
// inside the fp16 range).
constexpr int kNormThreads = 1024;  // 2 values per thread: more loads in flight per token
__global__ __launch_bounds__(kNormThreads) void k_bnorm(float* __restrict__ h, const float* __restrict__ dr,
                                                    const float* __restrict__ ds, int k, float* __restrict__ u,
                                                    uint16_t* __restrict__ up, int B, float eps) {
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  float* hb = h + (size_t)b * kHidden;
  float v[kHidden / kNormThreads];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kHidden / kNormThreads; ++i) {
    const int n = t + i * kNormThreads;
    v[i] = hb[n];
  }
  if (dr) {
    // every load issued before the sums (slots unrolled to the maximum k)
    float y[kHidden / kNormThreads][kMaxTopK + 1];
#pragma unroll
    for (int i = 0; i < kHidden / kNormThreads; ++i) {
      const int n = t + i * kNormThreads;
#pragma unroll
      for (int sl = 0; sl < kMaxTopK; ++sl) {  // unconditional loads (slot k - 1 again past k), all in flight
        const float v = dr[((size_t)b * k + (sl < k ? sl : k - 1)) * kHidden + n];
        y[i][sl] = sl < k ? v : 0.0f;
      }
      y[i][kMaxTopK] = ds[(size_t)b * kHidden + n];
    }
#pragma unroll
    for (int i = 0; i < kHidden / kNormThreads; ++i) {
      float acc = 0.0f;
#pragma unroll
      for (int sl = 0; sl < kMaxTopK; ++sl)
        if (sl < k) acc += y[i][sl];
      v[i] += acc + y[i][kMaxTopK];
      hb[t + i * kNormThreads] = v[i];
    }
  }
#pragma unroll
  for (int i = 0; i < kHidden / kNormThreads; ++i) ss = __builtin_fmaf(v[i], v[i], ss);
  ss = wave_sum(ss);
  __shared__ float red[kNormThreads / 64];
  if (lane == 0) red[w] = ss;
  __syncthreads();
  float r4[4];  // fixed order: four sums of four, then their pairs
#pragma unroll
  for (int j = 0; j < 4; ++j) r4[j] = (red[4 * j] + red[4 * j + 1]) + (red[4 * j + 2] + red[4 * j + 3]);
  const float tot = (r4[0] + r4[1]) + (r4[2] + r4[3]);
  const float s = 1.0f / sqrtf(tot * (1.0f / kHidden) + eps);
#pragma unroll
  for (int i = 0; i < kHidden / kNormThreads; ++i) {
    const int c = t + i * kNormThreads;
    const float x = v[i] * s;
    if (u) u[(size_t)b * kHidden + c] = x;
    uint16_t o[2];
    FmtF16::split(x, o);
#pragma unroll
    for (int p = 0; p < 2; ++p) up[((size_t)p * B + b) * kHidden + c] = o[p];
  }
}

// ------------------------------------------------------------ gate / up --
// grid (I / 64, nsh + Umax), 256 threads, nsh = ceil(Is / I).  Grid rows
// 0 .. nsh - 1: the shared expert and all B tokens (workgroup (x, y) takes
// rows 64 (y I/64 + x) ..); row nsh + ub (ub < U): the rank-ub chosen expert
// and its (token, slot) pairs.  Wave w takes gate rows and up rows r0 + 16 w .. + 15 of
// its group (two tiles with the same rows) from the fp16 planes of the
// normalised tokens up [2][B][H], and writes h = silu(gate) * up for each
// token as three bf16 planes: hrp [3][B*k][I] by pair id (routed),
// hsp [3][B][Is] by token (shared).
template <bool TILED, int AHEAD>
__global__ __launch_bounds__(kMmThreads, 3) void k_mm_gateup(flint_moe_layer L, int I, int Is, int k, int B,
                                                             int Umax, const uint16_t* __restrict__ up,
                                                             const int32_t* __restrict__ bk, uint16_t* __restrict__ hrp,
                                                             uint16_t* __restrict__ hsp, int nb,
                                                             const uint8_t* tiles, int E) {
  __shared__ __align__(16) unsigned char abuf[mm_buf_bytes<FmtF16>()];
  __shared__ int srow[kMmTok], orow[kMmTok];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6, m = lane & 15, q = lane >> 4;
  // the first nsh grid rows are the shared expert (all B tokens, the longest
  // workgroups: dispatched first, they overlap the routed experts' rows)
  const int nsh = (Is + I - 1) / I;
  const bool sh = (int)blockIdx.y < nsh;
  const int ub = (int)blockIdx.y - nsh;
  if (!sh && ub >= bk[0]) return;
  const int rows = sh ? Is : I, r0 = ((sh ? (int)blockIdx.y * (int)gridDim.x : 0) + (int)blockIdx.x) * kMmGateUpRows;
  if (r0 >= rows) return;
  int e = 0, p0 = 0, ntok = B;
  if (!sh) {
    e = bk[kBkExperts + ub];
    p0 = bk[kBkStart + ub];
    ntok = bk[kBkStart + ub + 1] - p0;
  }
  const int row = r0 + 16 * wv + m;
  MmTiles T;
  float Sg, Su;
  if (TILED) {
    // this layer's tiled gate and up matrices (routed experts' tiles, then
    // the shared expert's): codes [2][nt][H/256][2 KB], then scales
    // [2][nt][H/256][256 B], nt = E I / 16 + Is / 16
    const size_t ntile = (size_t)E * (I / 16) + Is / 16;
    const size_t mat_c = ntile * 16 * (kHidden / 2), mat_s = ntile * 16 * (kHidden / 16);
    const int wtile = __builtin_amdgcn_readfirstlane((r0 + 16 * wv) / 16);  // the same in every lane
    const size_t tile = (sh ? (size_t)E * (I / 16) : (size_t)e * (I / 16)) + wtile;
    const uint8_t* tc = tiles + tile * (kHidden / kMmChunk) * 2048;
    const uint8_t* ts = tiles + 2 * mat_c + tile * (kHidden / kMmChunk) * 256;
    T.rc[0] = make_rsrc(tc, (kHidden / kMmChunk) * 2048);
    T.rc[1] = make_rsrc(tc + mat_c, (kHidden / kMmChunk) * 2048);
    T.rs[0] = make_rsrc(ts, (kHidden / kMmChunk) * 256);
    T.rs[1] = make_rsrc(ts + mat_s, (kHidden / kMmChunk) * 256);
    T.lane = lane;
  } else if (sh) {
    T.c[0] = L.shared_gate.codes + (size_t)row * (kHidden / 2) + 32 * q;
    T.s[0] = L.shared_gate.scales + (size_t)row * (kHidden / 16) + 4 * q;
    T.c[1] = L.shared_up.codes + (size_t)row * (kHidden / 2) + 32 * q;
    T.s[1] = L.shared_up.scales + (size_t)row * (kHidden / 16) + 4 * q;
  } else {
    const size_t er = (size_t)e * I + row;
    T.c[0] = L.gate_codes + er * (kHidden / 2) + 32 * q;
    T.s[0] = L.gate_scales + er * (kHidden / 16) + 4 * q;
    T.c[1] = L.up_codes + er * (kHidden / 2) + 32 * q;
    T.s[1] = L.up_scales + er * (kHidden / 16) + 4 * q;
  }
  if (sh) {
    Sg = *L.shared_gate.tscale;
    Su = *L.shared_up.tscale;
  } else {
    Sg = L.expert_tscales[3 * e + 0];
    Su = L.expert_tscales[3 * e + 1];
  }
  const rsrc_t rA = make_rsrc(up, (uint64_t)FmtF16::P * B * kHidden * 2);
  uint16_t* outp = sh ? hsp : hrp;
  const int ow = sh ? Is : I, orows = sh ? B : nb;
  for (int t0 = 0; t0 < ntok; t0 += kMmTok) {
    const int nt = ntok - t0 < kMmTok ? ntok - t0 : kMmTok;
    __syncthreads();  // the previous pass is done with srow, orow and the buffers
    if (t < kMmTok) {
      int sr = -1, orr = -1;
      if (t < nt) {
        if (sh) {
          sr = orr = t0 + t;
        } else {
          orr = bk[kBkPairs + p0 + t0 + t];
          sr = orr / k;
        }
      }
      srow[t] = sr;
      orow[t] = orr;
    }
    __syncthreads();
    f32x4_t acc[2][2];
    mm_pass_n<FmtF16, kHidden / kMmChunk, typename std::conditional<TILED, MmTiled, MmRowMajor>::type, AHEAD>(
        T, rA, B, srow, nt, abuf, wv, lane, acc);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * tt + 4 * q + i;
        if (tok < nt) {
          uint16_t o[3];
          FmtBF16::split(silu(acc[0][tt][i] * Sg) * (acc[1][tt][i] * Su), o);
          const int orr = orow[tok];
#pragma unroll
          for (int p = 0; p < 3; ++p) outp[((size_t)p * orows + orr) * ow + row] = o[p];
        }
      }
  }
}

// ----------------------------------------------------------------- down --
// grid (H / 128, Umax + 1), 256 threads; groups as for gate/up.  Wave w takes
// output rows r0 + 32 w .. + 31.  Routed: dr[pid][n] = w_pid * S_e * (Wd[e][n]
// . h_pid) over K = I; shared: ds[b][n] = S * (Wsd[n] . hs_b) over K = Is.
template <bool TILED, int AHEAD>
__global__ __launch_bounds__(kMmThreads, 3) void k_mm_down(flint_moe_layer L, int I, int Is, int B, int Umax,
                                                           const uint16_t* __restrict__ hrp,
                                                           const uint16_t* __restrict__ hsp,
                                                           const int32_t* __restrict__ bk,
                                                           const float* __restrict__ wts, float* __restrict__ dr,
                                                           float* __restrict__ ds, int nb, const uint8_t* dtiles,
                                                           int E) {
  __shared__ __align__(16) unsigned char abuf[mm_buf_bytes<FmtBF16>()];
  __shared__ int srow[kMmTok];
  __shared__ float coef[kMmTok];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6, m = lane & 15, q = lane >> 4;
  // grid row 0 is the shared expert (all B tokens, the longest workgroups:
  // dispatched first, they overlap the routed experts' rows 1 .. U)
  const bool sh = blockIdx.y == 0;
  const int ub = (int)blockIdx.y - 1;
  if (!sh && ub >= bk[0]) return;
  int e = 0, p0 = 0, ntok = B;
  if (!sh) {
    e = bk[kBkExperts + ub];
    p0 = bk[kBkStart + ub];
    ntok = bk[kBkStart + ub + 1] - p0;
  }
  const int K = sh ? Is : I;
  const int rbase = blockIdx.x * kMmRows + 32 * wv;
  MmTiles T;
  if constexpr (TILED) {
    // this layer's tiled down matrices (DownTiles): the routed experts'
    // 16-row tiles, then the shared expert's, each tile's K chunks in a row
    const DownTiles D(E, I, Is);
    const int nch = K / kMmChunk;
    const int t0 = __builtin_amdgcn_readfirstlane(rbase / 16);  // the same in every lane
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      // tile of rows rbase + 16 rt .. + 15: the shared expert's, or expert e's
      const size_t tile = sh ? (size_t)t0 + rt : (size_t)e * (kHidden / 16) + t0 + rt;
      const size_t cb = (sh ? D.shared_c : D.routed_c) + tile * nch * 2048;
      const size_t sb = (sh ? D.shared_s : D.routed_s) + tile * nch * 256;
      T.rc[rt] = make_rsrc(dtiles + cb, (uint64_t)nch * 2048);
      T.rs[rt] = make_rsrc(dtiles + sb, (uint64_t)nch * 256);
    }
    T.lane = lane;
  } else {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int row = rbase + 16 * rt + m;
      if (sh) {
        T.c[rt] = L.shared_down.codes + (size_t)row * (Is / 2) + 32 * q;
        T.s[rt] = L.shared_down.scales + (size_t)row * (Is / 16) + 4 * q;
      } else {
        const size_t er = (size_t)e * kHidden + row;
        T.c[rt] = L.down_codes + er * (I / 2) + 32 * q;
        T.s[rt] = L.down_scales + er * (I / 16) + 4 * q;
      }
    }
  }
  using Lay = typename std::conditional<TILED, MmTiled, MmRowMajor>::type;
  const float S = sh ? *L.shared_down.tscale : L.expert_tscales[3 * e + 2];
  const rsrc_t rA = sh ? make_rsrc(hsp, (uint64_t)3 * B * Is * 2) : make_rsrc(hrp, (uint64_t)3 * nb * I * 2);
  const int a_rows = sh ? B : nb;
  float* out = sh ? ds : dr;
  for (int t0 = 0; t0 < ntok; t0 += kMmTok) {
    const int nt = ntok - t0 < kMmTok ? ntok - t0 : kMmTok;
    __syncthreads();
    if (t < kMmTok) {
      int sr = -1;
      float c = 0.0f;
      if (t < nt) {
        sr = sh ? t0 + t : bk[kBkPairs + p0 + t0 + t];
        c = sh ? S : S * wts[sr];
      }
      srow[t] = sr;
      coef[t] = c;
    }
    __syncthreads();
    f32x4_t acc[2][2];
    if (K == 1024) mm_pass_n<FmtBF16, 4, Lay, AHEAD>(T, rA, a_rows, srow, nt, abuf, wv, lane, acc);
    else if (K == 2048) mm_pass_n<FmtBF16, 8, Lay, AHEAD>(T, rA, a_rows, srow, nt, abuf, wv, lane, acc);
    else mm_pass_n<FmtBF16, 2, Lay, AHEAD>(T, rA, a_rows, srow, nt, abuf, wv, lane, acc);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * tt + 4 * q + i;
        if (tok < nt) {
          const int orr = srow[tok];
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) out[(size_t)orr * kHidden + rbase + 16 * rt + m] = acc[rt][tt][i] * coef[tok];
        }
      }
  }
}

// ----------------------------------------------------------------- head --
// grid ceil(V / 256), 512 threads: rows r0 + 32 w .. + 31 of the head for
// all B tokens (final-norm fp16 planes zp [2][B][H]); logits (optional) and, per
// token, this workgroup's (max, first index) -> partials[b][blockIdx.x].
// (codes and scales are not marked restrict: the rows are read again in
// every token pass, and hoisting those loads out of the pass loop would pin
// all of them in registers)
__global__ __launch_bounds__(kMmThreads, 3) void k_mm_head(const uint8_t* codes, const uint8_t* scales,
                                                           const float* __restrict__ tscale, int vocab,
                                                           const uint16_t* __restrict__ zp, int B,
                                                           float* __restrict__ logits,
                                                           HeadPartial* __restrict__ partials) {
  __shared__ __align__(16) unsigned char abuf[mm_buf_bytes<FmtF16>()];
  __shared__ int srow[kMmTok];
  __shared__ float bv[kMmWaves][kMmTok];
  __shared__ int bi[kMmWaves][kMmTok];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6, m = lane & 15, q = lane >> 4;
  const int rbase = blockIdx.x * kMmRows + 32 * wv;
  MmTiles T;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = min(rbase + 16 * rt + m, vocab - 1);  // rows past the end read the last row; dropped
    T.c[rt] = codes + (size_t)row * (kHidden / 2) + 32 * q;
    T.s[rt] = scales + (size_t)row * (kHidden / 16) + 4 * q;
  }
  const float S = *tscale;
  const rsrc_t rA = make_rsrc(zp, (uint64_t)FmtF16::P * B * kHidden * 2);
  for (int t0 = 0; t0 < B; t0 += kMmTok) {
    const int nt = B - t0 < kMmTok ? B - t0 : kMmTok;
    __syncthreads();
    if (t < kMmTok) srow[t] = t < nt ? t0 + t : -1;
    __syncthreads();
    f32x4_t acc[2][2];
    mm_pass_n<FmtF16, kHidden / kMmChunk>(T, rA, B, srow, nt, abuf, wv, lane, acc);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * tt + 4 * q + i;
        // this lane's two rows, then the best over the 16 lanes of its DPP row
        float v = -FLT_MAX;
        int n = INT_MAX;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const int row = rbase + 16 * rt + m;
          const float x = acc[rt][tt][i] * S;
          if (row < vocab && tok < nt) {
            if (logits) logits[(size_t)(t0 + tok) * vocab + row] = x;
            if (x > v) { v = x; n = row; }  // rt = 0 rows come first
          }
        }
        auto step = [&](float ov, int on) {
          if (ov > v || (ov == v && on < n)) { v = ov; n = on; }
        };
        step(dpp_f32<kDppXor1>(v), dpp_i32<kDppXor1>(n));
        step(dpp_f32<kDppXor2>(v), dpp_i32<kDppXor2>(n));
        step(dpp_f32<kDppHalfMirror>(v), dpp_i32<kDppHalfMirror>(n));
        step(dpp_f32<kDppMirror>(v), dpp_i32<kDppMirror>(n));
        if (m == 0) {
          bv[wv][tok] = v;
          bi[wv][tok] = n;
        }
      }
    __syncthreads();
    if (t < nt) {
      float v = bv[0][t];
      int n = bi[0][t];
      for (int w = 1; w < kMmWaves; ++w)
        if (bv[w][t] > v || (bv[w][t] == v && bi[w][t] < n)) { v = bv[w][t]; n = bi[w][t]; }
      partials[(size_t)(t0 + t) * gridDim.x + blockIdx.x] = HeadPartial{v, n};
    }
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

}  // namespace

bool batch_supported(const flint_moe_dims& d, int B) {
  // the down projection's K loop is instantiated for 2, 4 and 8 chunks of 256
  auto width_ok = [](int K) { return K == 512 || K == 1024 || K == 2048; };
  return d.hidden == kHidden && B >= 1 && B <= kMaxBatch && width_ok(d.expert_width) && width_ok(d.shared_width) &&
         d.n_experts <= kMaxExperts && d.top_k <= kMaxTopK;
}

static int head_blocks(int vocab) { return (vocab + kMmRows - 1) / kMmRows; }

BatchWs::BatchWs(const flint_moe_dims& d, int B, int vocab) {
  const int nb = B * d.top_k;
  size_t o = 0;
  h = o; o = align_up(o + 4 * (size_t)B * kHidden, 256);
  u = o; o = align_up(o + 4 * (size_t)B * kHidden, 256);
  up = o; o = align_up(o + 2 * 2 * (size_t)B * kHidden, 256);
  logits = o; o = align_up(o + 4 * (size_t)B * d.n_experts, 256);
  idx = o; o = align_up(o + 4 * (size_t)nb, 256);
  wts = o; o = align_up(o + 4 * (size_t)nb, 256);
  bucket = o; o = align_up(o + 4 * (size_t)(kBkPairs + nb), 256);
  hr = o; o = align_up(o + 2 * 3 * (size_t)nb * d.expert_width, 256);
  hs = o; o = align_up(o + 2 * 3 * (size_t)B * d.shared_width, 256);
  dr = o; o = align_up(o + 4 * (size_t)nb * kHidden, 256);
  ds = o; o = align_up(o + 4 * (size_t)B * kHidden, 256);
  partials = o; o = align_up(o + sizeof(HeadPartial) * (size_t)B * head_blocks(vocab), 256);
  total = o;
}

// Tiled copy of one layer's gate and up matrices for k_mm_gateup: the routed
// experts' 16-row tiles (expert e, rows 16 j .. 16 j + 15 at tile e I/16 + j),
// then the shared expert's (tile E I/16 + j); codes [2][nt][H/256][2 KB], then
// scales [2][nt][H/256][256 B] (the MmTiled layout).  One thread per (matrix,
// tile, chunk, lane L = 16 q + m): row 16 j + m, K values 64 q .. +63 of the
// chunk.
__global__ __launch_bounds__(kThreads) void k_tile_gateup(flint_moe_layer L, int E, int I, int Is,
                                                          uint8_t* __restrict__ dst) {
  constexpr int nch = kHidden / kMmChunk;
  const size_t nrt = (size_t)E * (I / 16), ntile = nrt + Is / 16;
  const size_t mat_c = ntile * 16 * (kHidden / 2), mat_s = ntile * 16 * (kHidden / 16);
  const size_t per_mat = ntile * nch * 64, total = 2 * per_mat;
  for (size_t i = blockIdx.x * (size_t)kThreads + threadIdx.x; i < total; i += (size_t)gridDim.x * kThreads) {
    const int kind = (int)(i / per_mat);
    size_t r = i % per_mat;
    const int lane = (int)(r % 64);
    r /= 64;
    const int u = (int)(r % nch);
    r /= nch;  // the tile
    const int m = lane & 15, q = lane >> 4;
    const uint8_t *sc, *ss;
    if (r < nrt) {
      const size_t row = r * 16 + m;  // e I + 16 j + m
      sc = (kind ? L.up_codes : L.gate_codes) + row * (kHidden / 2);
      ss = (kind ? L.up_scales : L.gate_scales) + row * (kHidden / 16);
    } else {
      const size_t row = (r - nrt) * 16 + m;
      const flint_nvfp4& W = kind ? L.shared_up : L.shared_gate;
      sc = W.codes + row * (kHidden / 2);
      ss = W.scales + row * (kHidden / 16);
    }
    sc += (kMmChunk / 2) * u + 32 * q;
    ss += (kMmChunk / 16) * u + 4 * q;
    uint8_t* dc = dst + kind * mat_c + (r * nch + u) * 2048 + 16 * lane;
    uint8_t* ds = dst + 2 * mat_c + kind * mat_s + (r * nch + u) * 256 + 4 * lane;
    *reinterpret_cast<uint4*>(dc) = *reinterpret_cast<const uint4*>(sc);
    *reinterpret_cast<uint4*>(dc + 1024) = *reinterpret_cast<const uint4*>(sc + 16);
    *reinterpret_cast<uint32_t*>(ds) = *reinterpret_cast<const uint32_t*>(ss);
  }
}

// Tiled copy of rows x K NVFP4 (row-major codes and scales) for the MmTiled
// layout: [rows/16][K/256][2 KB] codes, [rows/16][K/256][256 B] scales.  One
// thread per (tile, chunk, lane L = 16 q + m).
__global__ __launch_bounds__(kThreads) void k_tile_rows(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales, size_t rows, int K,
                                                        uint8_t* __restrict__ dc, uint8_t* __restrict__ ds) {
  const int nch = K / kMmChunk;
  const size_t total = rows / 16 * nch * 64;
  for (size_t i = blockIdx.x * (size_t)kThreads + threadIdx.x; i < total; i += (size_t)gridDim.x * kThreads) {
    const int lane = (int)(i % 64);
    const size_t r = i / 64;  // tile * nch + chunk
    const int u = (int)(r % nch);
    const size_t tile = r / nch;
    const int m = lane & 15, q = lane >> 4;
    const size_t row = tile * 16 + m;
    const uint8_t* sc = codes + row * (K / 2) + (kMmChunk / 2) * u + 32 * q;
    const uint8_t* ss = scales + row * (K / 16) + (kMmChunk / 16) * u + 4 * q;
    *reinterpret_cast<uint4*>(dc + r * 2048 + 16 * lane) = *reinterpret_cast<const uint4*>(sc);
    *reinterpret_cast<uint4*>(dc + r * 2048 + 1024 + 16 * lane) = *reinterpret_cast<const uint4*>(sc + 16);
    *reinterpret_cast<uint32_t*>(ds + r * 256 + 4 * lane) = *reinterpret_cast<const uint32_t*>(ss);
  }
}

size_t batch_tiles_layer_bytes(const flint_moe_dims& d) {
  return DownTiles(d.n_experts, d.expert_width, d.shared_width).total;
}

hipError_t launch_batch_tiles(const flint_moe_dims& d, const flint_moe_layer* layers, int L, uint8_t* tiles,
                              hipStream_t s) {
  const size_t per = batch_tiles_layer_bytes(d);
  for (int l = 0; l < L; ++l) {
    uint8_t* base = tiles + (size_t)l * per;
    const DownTiles D(d.n_experts, d.expert_width, d.shared_width);
    const flint_moe_layer& Ly = layers[l];
    k_tile_gateup<<<2048, kThreads, 0, s>>>(Ly, d.n_experts, d.expert_width, d.shared_width, base);
    k_tile_rows<<<2048, kThreads, 0, s>>>(Ly.down_codes, Ly.down_scales, (size_t)d.n_experts * kHidden,
                                          d.expert_width, base + D.routed_c, base + D.routed_s);
    k_tile_rows<<<2048, kThreads, 0, s>>>(Ly.shared_down.codes, Ly.shared_down.scales, kHidden, d.shared_width,
                                          base + D.shared_c, base + D.shared_s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// 4-byte word copy (the step uses kernels only, so it can be captured in a
// HIP graph)
__global__ __launch_bounds__(kThreads) void k_copy_words(const uint32_t* __restrict__ src,
                                                         uint32_t* __restrict__ dst, int n) {
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads) dst[i] = src[i];
}

hipError_t launch_batch_step_tiled(const flint_moe_dims& d, const flint_moe_layer* layers, int L,
                                   const flint_nvfp4& head, int vocab, const float* x, int B, float eps, float* logits,
                                   int32_t* argmax, int32_t* routes, void* ws, hipStream_t s, const uint8_t* tiles) {
  const BatchWs w(d, B, vocab);
  char* base = static_cast<char*>(ws);
  float* h = reinterpret_cast<float*>(base + w.h);
  float* u = reinterpret_cast<float*>(base + w.u);
  uint16_t* up = reinterpret_cast<uint16_t*>(base + w.up);
  float* lg = reinterpret_cast<float*>(base + w.logits);
  int32_t* idx = reinterpret_cast<int32_t*>(base + w.idx);
  float* wts = reinterpret_cast<float*>(base + w.wts);
  int32_t* bk = reinterpret_cast<int32_t*>(base + w.bucket);
  uint16_t* hrp = reinterpret_cast<uint16_t*>(base + w.hr);
  uint16_t* hsp = reinterpret_cast<uint16_t*>(base + w.hs);
  float* dr = reinterpret_cast<float*>(base + w.dr);
  float* ds = reinterpret_cast<float*>(base + w.ds);
  HeadPartial* parts = reinterpret_cast<HeadPartial*>(base + w.partials);
  const int k = d.top_k, E = d.n_experts, I = d.expert_width, Is = d.shared_width, nb = B * k;
  const int Umax = nb < E ? nb : E;
  const int gu_x = (I + kMmGateUpRows - 1) / kMmGateUpRows;  // a routed expert's rows; the shared one spans
  const int gu_sh = (Is + I - 1) / I;                        // gu_sh grid rows
  k_copy_words<<<(B * kHidden + kThreads - 1) / kThreads, kThreads, 0, s>>>(
      reinterpret_cast<const uint32_t*>(x), reinterpret_cast<uint32_t*>(h), B * kHidden);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_bnorm<<<B, kNormThreads, 0, s>>>(h, nullptr, nullptr, k, u, up, B, eps);
  for (int l = 0; l < L && e == hipSuccess; ++l) {
    const flint_moe_layer& Ly = layers[l];
    k_broute<<<dim3((E + 3) / 4, (B + kRouteTok - 1) / kRouteTok), kThreads, 0, s>>>(Ly.router, E, u, B, lg);
    k_btopk<<<B, 64, 0, s>>>(lg, E, k, idx, wts);
    if (routes)
      k_copy_words<<<1, kThreads, 0, s>>>(reinterpret_cast<const uint32_t*>(idx),
                                          reinterpret_cast<uint32_t*>(routes + (size_t)l * nb), nb);
    k_bucket<<<1, kThreads, 0, s>>>(idx, nb, E, bk);
    const uint8_t* lt = tiles ? tiles + (size_t)l * batch_tiles_layer_bytes(d) : nullptr;
    const dim3 gg(gu_x, gu_sh + Umax), gd(kHidden / kMmRows, Umax + 1);
    if (tiles) {  // tiled weights: two chunks ahead (with the current grids at every B; three is slower at B = 8)
      k_mm_gateup<true, 2><<<gg, kMmThreads, 0, s>>>(Ly, I, Is, k, B, Umax, up, bk, hrp, hsp, nb, lt, E);
      k_mm_down<true, 2><<<gd, kMmThreads, 0, s>>>(Ly, I, Is, B, Umax, hrp, hsp, bk, wts, dr, ds, nb, lt, E);
    } else {  // row-major weights: longer load latency, three chunks ahead
      k_mm_gateup<false, 3><<<gg, kMmThreads, 0, s>>>(Ly, I, Is, k, B, Umax, up, bk, hrp, hsp, nb, lt, E);
      k_mm_down<false, 3><<<gd, kMmThreads, 0, s>>>(Ly, I, Is, B, Umax, hrp, hsp, bk, wts, dr, ds, nb, lt, E);
    }
    // the residual update and the next norm (after the last layer: the
    // final norm, the head's input)
    k_bnorm<<<B, kNormThreads, 0, s>>>(h, dr, ds, k, l + 1 < L ? u : nullptr, up, B, eps);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  const int hb = head_blocks(vocab);
  k_mm_head<<<hb, kMmThreads, 0, s>>>(head.codes, head.scales, head.tscale, vocab, up, B, logits, parts);
  k_bargmax<<<B, 64, 0, s>>>(parts, hb, argmax);
  return hipGetLastError();
}

hipError_t launch_batch_step(const flint_moe_dims& d, const flint_moe_layer* layers, int L, const flint_nvfp4& head,
                             int vocab, const float* x, int B, float eps, float* logits, int32_t* argmax,
                             int32_t* routes, void* ws, hipStream_t s) {
  return launch_batch_step_tiled(d, layers, L, head, vocab, x, B, eps, logits, argmax, routes, ws, s, nullptr);
}

}  // namespace flint
