// gemm.hip -- prompt processing on gfx950 matrix cores: T tokens through one
// NVFP4 matrix, Y = X W^T, with full-precision activations (A32) or with the
// activations quantised to NVFP4 first (A4).
//
// Method [P1 "Flint-40B-A2B: AI-Built MoE Coding Model Hits 125 tok/s on
// MacBook Pro", "Custom Inference Kernels"; P2 "Recursive Releases Flint, a
// 40B MoE Coding Model That Runs Locally at 125 Tokens per Second", "How did
// the Eureka Machine build Flint?": kernels for low-bit projections and prompt
// processing].  With many tokens the product is a dense contraction, so it
// runs on 16x16x32 fp16 MFMA:
//  - an E2M1 code times its E4M3 block scale has at most 5 significant bits
//    and lies in [2^-10, 2688]: exact in fp16.  It is decoded in registers
//    (the hardware FP4 -> fp16 conversion with the scale's power of two, then
//    a packed fp16 multiply by the rest of the scale); the tensor scale
//    multiplies the fp32 result;
//  - A32: every fp32 activation is split into two fp16 parts (hi = fp16(x),
//    lo = fp16(x - hi): 22 significant bits, |x| < 65504); both parts go
//    through the matrix cores, products are exact in fp32;
//  - A4: the activations are NVFP4 too (one tensor scale over X, quantised
//    on the device by the same codec) and decode like the weights: one part.
// A pre-pass writes the activations once per call as fp16 planes in the
// workspace (A32: hi and lo; A4: code x block scale), which both kernels
// below copy into LDS with buffer-to-LDS loads.
// gfx950's scaled-FP4 MFMA takes one power-of-two scale per 32 values, so it
// cannot carry NVFP4's E4M3 scale per 16 exactly; it is not used.
//
// Narrow kernel (calls with few 256 x 256 tiles): a workgroup (4 waves) owns
// 256 weight rows x 32 tokens; each wave 64 rows (four 16-row tiles) x the
// 32 tokens (two 16-token tiles), so every activation fragment read from LDS
// feeds four products.  K runs in chunks of 256: the chunk's planes are
// copied into LDS (double-buffered; the next chunk's copies are issued
// before the current chunk's products), each lane's weight bytes for the
// next chunk are requested before the current chunk is multiplied and
// decoded in registers.
#include <float.h>

#include <algorithm>

#include "../../include/flint_gemm.h"
#include "flint_common.h"
#include "flint_device.h"
#include "flint_internal.h"

namespace flint {
namespace {

typedef __attribute__((ext_vector_type(8))) _Float16 h8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 h2_t;
typedef __attribute__((ext_vector_type(4))) float f4_t;

constexpr int kRT = 4;        // 16-row weight tiles per wave
constexpr int kGRows = 64 * kRT;  // weight rows per workgroup
constexpr int kGTok = 32;     // tokens per workgroup
constexpr int kGChunk = 256;  // K per stage
constexpr int kGRowBytes = kGChunk * 2;            // one token's fp16 part of a chunk
constexpr int kGPartBytes = kGTok * kGRowBytes;    // 16 KB

// E4M3 block scale as (power of two, fp16 rest): value = p2 * f exactly
struct H16Scale {
  float p2;
  _Float16 f;
};
__device__ __forceinline__ H16Scale h16_scale(uint32_t b) {
  const uint32_t e = (b >> 3) & 15, m = b & 7;
  H16Scale s;
  s.p2 = __uint_as_float((e ? e + 120u : 118u) << 23);  // 2^(e-7), or 2^-9 (subnormal)
  s.f = e ? (_Float16)(1.0f + 0.125f * (float)m) : (_Float16)(float)m;
  return s;
}
// the 8 values of one code word (element 2i in the low nibble of byte i) times
// the block scale, as fp16 (exact)
__device__ __forceinline__ h8_t h16_decode(uint32_t w, H16Scale s) {
  const h2_t ff = {s.f, s.f};
  const h2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.p2, 0) * ff;
  const h2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.p2, 1) * ff;
  const h2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.p2, 2) * ff;
  const h2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s.p2, 3) * ff;
  return h8_t{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

struct GemmArgs {
  const uint8_t* wc;   // W codes [N][K/2]
  const uint8_t* ws;   // W scales [N][K/16]
  const float* wS;     // W tensor scale
  const uint16_t* xp;  // activation planes [P][T][K] fp16 (A32: hi, lo; A4: code x block scale)
  const float* xS;     // A4: X tensor scale (else null)
  float* y;            // Y [T][N]
  int N, K, T;
};

// byte offset of (token row r, 8-value group g) in one part of a staged chunk:
// rows are 512 bytes; groups are XOR-swizzled by the row so that the 16 rows
// a wave reads for one product fall on different banks
__device__ __forceinline__ int stage_off(int r, int g) { return r * kGRowBytes + ((g ^ (r & 15)) << 4); }

// Activation staging: a chunk's P planes (32 token rows x 512 bytes each)
// are copied buffer-to-LDS, 1 KB (two rows) per wave instruction, into the
// swizzled layout above: lane L of copy c writes row 2c + L/32, slot L % 32,
// which holds granule (L % 32) ^ (row % 16).  Rows past T read as zero.
template <int P>
struct PlaneRsrc {  // the activation planes of a token block, one buffer resource each
  rsrc_t r[P];
  __device__ __forceinline__ void copy(int K, int kc, unsigned char* buf, int wv, int lane) const {
    constexpr int kCopies = kGPartBytes / 1024;  // per plane
#pragma unroll
    for (int i = 0; i < P * kCopies / 4; ++i) {
      const int p = 4 * i / kCopies, c = 4 * i % kCopies + wv;  // copy wv + 4 i (kCopies is a multiple of 4)
      const int row = 2 * c + (lane >> 5), g = (lane & 31) ^ (row & 15);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r[p],
                                               (__attribute__((address_space(3))) void*)(buf + p * kGPartBytes + c * 1024),
                                               16, (uint32_t)((row * K + kc + 8 * g) * 2), 0, 0, 0);
    }
  }
};

// a lane's weight bytes of one chunk for its row tiles: 64 values
// (K = kc + 64 q .. +64) of row m of each tile
struct WFrag {
  uint4 c[kRT][2];
  uint32_t s[kRT];
};
__device__ __forceinline__ void wfrag_load(const GemmArgs& A, const int* rows, int kc, int q, WFrag& f) {
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const uint8_t* cp = A.wc + (size_t)rows[rt] * (A.K / 2) + kc / 2 + 32 * q;
    f.c[rt][0] = ld_nt_u4(cp);
    f.c[rt][1] = ld_nt_u4(cp + 16);
    f.s[rt] = ld_nt_u32(A.ws + (size_t)rows[rt] * (A.K / 16) + kc / 16 + 4 * q);
  }
}

// The products of one 256-wide chunk from its staged planes (buf) and this
// lane's weight bytes (f).
template <int P>
__device__ __forceinline__ void narrow_chunk(const WFrag& f, const unsigned char* buf, int m, int q,
                                             f4_t (&acc)[kRT][2]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    h8_t b[kRT];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
      b[rt] = h16_decode((&f.c[rt][j >> 2].x)[j & 3], h16_scale((f.s[rt] >> (8 * (j >> 1))) & 0xFF));
    const int g = 8 * q + j;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int r = 16 * tt + m;
      const unsigned char* ap = buf + stage_off(r, g);
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const h8_t a = *reinterpret_cast<const h8_t*>(ap + p * kGPartBytes);
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt)
          acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[rt], acc[rt][tt], 0, 0, 0);
      }
    }
  }
}

// Iteration c (R = c % 2): chunk c's planes are in sbuf[R] and its weight
// bytes in f[R]; the next chunk's copies and bytes go to sbuf[1 - R] and
// f[1 - R] first.  The requests are made unconditionally (past the end the
// last chunk again, into buffers no one reads any more) and the register
// sets are not copied, so the compiler's waits before this chunk's products
// never include the requests just made.  When the chunk count is odd, the
// second half of the last pair of iterations only makes its requests.
template <int P, int R>
__device__ __forceinline__ void narrow_iter(const GemmArgs& A, const PlaneRsrc<P>& rx, const int (&rows)[kRT], int c,
                                            int nch, unsigned char (&sbuf)[2][P * kGPartBytes], WFrag (&f)[2],
                                            int wv, int lane, f4_t (&acc)[kRT][2]) {
  const int m = lane & 15, q = lane >> 4;
  const int cn = c + 1 < nch ? c + 1 : nch - 1;
  rx.copy(A.K, cn * kGChunk, sbuf[1 - R], wv, lane);
  wfrag_load(A, rows, cn * kGChunk, q, f[1 - R]);
  if (c < nch) narrow_chunk<P>(f[R], sbuf[R], m, q, acc);
  __syncthreads();  // every wave's copies of the next chunk are in (after the last, every copy has landed)
}

template <int P>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs A) {
  __shared__ __align__(16) unsigned char sbuf[2][P * kGPartBytes];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, m = lane & 15, q = lane >> 4;
  const int n0 = blockIdx.x * kGRows + 16 * kRT * wv, t0 = blockIdx.y * kGTok;
  int rows[kRT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) rows[rt] = min(n0 + 16 * rt + m, A.N - 1);
  const int nch = A.K / kGChunk;
  f4_t acc[kRT][2];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) acc[rt][tt] = f4_t{0.f, 0.f, 0.f, 0.f};

  const int toks_here = A.T - t0 < kGTok ? A.T - t0 : kGTok;
  PlaneRsrc<P> rx;
#pragma unroll
  for (int p = 0; p < P; ++p) rx.r[p] = make_rsrc(A.xp + ((size_t)p * A.T + t0) * A.K, (uint64_t)toks_here * A.K * 2);
  WFrag f[2];
  rx.copy(A.K, 0, sbuf[0], wv, lane);
  wfrag_load(A, rows, 0, q, f[0]);
  __syncthreads();  // waits for this wave's copies as well
  for (int c = 0; c < nch; c += 2) {
    narrow_iter<P, 0>(A, rx, rows, c, nch, sbuf, f, wv, lane, acc);
    narrow_iter<P, 1>(A, rx, rows, c + 1, nch, sbuf, f, wv, lane, acc);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the last (unused) requests are in before the workgroup ends
  // lane (m, q) holds tokens 4q .. 4q+3 of each token tile for weight row m
  const float S = *A.wS * (P == 1 && A.xS ? *A.xS : 1.0f);
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    const int n = n0 + 16 * rt + m;
    if (n >= A.N) continue;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * tt + 4 * q + i;
        if (t < A.T) A.y[(size_t)t * A.N + n] = acc[rt][tt][i] * S;
      }
  }
}

// ------------------------------------------------------------ wide tiles --
// Many tokens: a workgroup of 8 waves owns 256 weight rows x 256 tokens;
// wave w takes rows 128 (w & 1) .. + 127 and tokens 64 (w >> 1) .. + 63, as
// 8 x 4 tiles of 16 x 16 (128 fp32 accumulators a lane).  The activations
// arrive as fp16 planes written once by a pre-pass (A32: hi and lo; A4: the
// decoded NVFP4 value, exact in fp16, the tensor scale applied at the end),
// so a K stage of the token tile is a plain buffer-to-LDS copy; the stage's
// weight rows are decoded once per workgroup into LDS by all 512 threads.
// Every product then takes both operands from LDS: a decoded weight serves
// 256 tokens, a staged activation 256 rows, against 32 tokens a decode in
// the narrow kernel above.
// Stages of BK K values run as a pipeline with one barrier a stage: the
// activation copies two stages ahead (three LDS buffers), the weight bytes
// three stages ahead (two register sets), the decode of the next stage's
// weights (two LDS buffers) between the two halves of the current stage's
// products, so its VALU work overlaps the matrix cores.  The barrier is
// s_barrier after a wait that leaves the iteration's own requests in
// flight (__syncthreads() would wait for all of them).  Against one stage
// ahead and decode-then-multiply, 7-9% faster on the 150,144-row head.
// Matrix-core operands: A = weight rows (C rows), B = tokens (C columns), so
// a lane's four accumulators are four consecutive weight rows of one token:
// one 16-byte store of Y.
// LDS rows hold BK fp16 values; granule g (8 values) of row r sits in slot
// g ^ wswz(r): the 8 rows that a 128-bit read serves in one cycle, and the 8
// granules of one decode store, fall in distinct banks.
constexpr int kWRows = 256, kWTok = 256, kWThreads = 512;

template <int BK>
__device__ __forceinline__ int wswz(int r) {
  constexpr int G = BK / 8;  // granules a row
  return (r / (8 / G)) & (G - 1);
}

struct WideArgs {
  const uint8_t* wc;    // W codes [N][K/2]
  const uint8_t* ws;    // W scales [N][K/16]
  const float* wS;      // W tensor scale
  const uint16_t* xp;   // activation planes [P][T][K] fp16
  const float* xS;      // A4: X tensor scale (else null)
  float* y;             // Y [T][N]
  int N, K, T;
};

// One workgroup's stage traffic: the decoding thread's weight bytes (row
// drow, values BK/2 dh .. + BK/2 of a stage) and the activation copies (1 KB
// buffer-to-LDS loads dealt round-robin to the waves).  Rows and tokens past
// the ends of W and X read as zero (buffer bounds).
template <int P, int BK>
struct WideStage {
  static constexpr int RB = 2 * BK, TB = kWTok * RB;
  static constexpr int NW = BK / 16;     // code words a decoding thread holds
  static constexpr int CPP = TB / 1024;  // 1 KB copies a plane
  static_assert(CPP % 8 == 0, "a plane's copies are dealt to the 8 waves evenly");
  static constexpr int OPS_W = 2;            // vector-memory requests a wave makes for a stage's weights
  static constexpr int OPS_T = P * CPP / 8;  // ... and for its activations
  static_assert(2 * OPS_W + OPS_T <= 15, "vmcnt field");
  rsrc_t rc, rs, rx[P];
  // two sets of the decoding thread's weight bytes: stage j in set j % 2
  uint32_t c_off, s_off, wcw[2][NW], wsb[2];
  int drow, dh, K;
  __device__ __forceinline__ void init(const WideArgs& A, int n0, int t0, int tid) {
    const int rows_here = A.N - n0 < kWRows ? A.N - n0 : kWRows;
    const int toks_here = A.T - t0 < kWTok ? A.T - t0 : kWTok;
    rc = make_rsrc(A.wc + (size_t)n0 * (A.K / 2), (uint64_t)rows_here * (A.K / 2));
    rs = make_rsrc(A.ws + (size_t)n0 * (A.K / 16), (uint64_t)rows_here * (A.K / 16));
#pragma unroll
    for (int p = 0; p < P; ++p) rx[p] = make_rsrc(A.xp + ((size_t)p * A.T + t0) * A.K, (uint64_t)toks_here * A.K * 2);
    K = A.K;
    drow = tid >> 1;
    dh = tid & 1;
    c_off = (uint32_t)drow * (K / 2) + dh * (BK / 4);
    s_off = (uint32_t)drow * (K / 16) + dh * (BK / 32);
  }
  template <int R>
  __device__ __forceinline__ void wload(int k0) {
    if constexpr (NW == 4) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rc, c_off + k0 / 2, 0, kAuxNT);
      wcw[R][0] = v[0]; wcw[R][1] = v[1]; wcw[R][2] = v[2]; wcw[R][3] = v[3];
      wsb[R] = (uint32_t)(unsigned short)__builtin_amdgcn_raw_buffer_load_b16(rs, s_off + k0 / 16, 0, kAuxNT);
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rc, c_off + k0 / 2, 0, kAuxNT);
      wcw[R][0] = v[0]; wcw[R][1] = v[1];
      wsb[R] = (uint32_t)(unsigned char)__builtin_amdgcn_raw_buffer_load_b8(rs, s_off + k0 / 16, 0, kAuxNT);
    }
  }
  template <int R>
  __device__ __forceinline__ void wstore(unsigned char* wbuf) const {
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int g = dh * NW + j;
      *reinterpret_cast<h8_t*>(wbuf + drow * RB + ((g ^ wswz<BK>(drow)) << 4)) =
          h16_decode(wcw[R][j], h16_scale((wsb[R] >> (8 * (j >> 1))) & 0xFF));
    }
  }
  __device__ __forceinline__ void tcopy(int k0, unsigned char* tbuf, int wv, int lane) const {
#pragma unroll
    for (int i = 0; i < P * CPP / 8; ++i) {
      const int p = 8 * i / CPP, cc = 8 * i % CPP + wv;  // copy wv + 8 i (CPP is a multiple of 8)
      const int pos = cc * 1024 + 16 * lane, r = pos / RB, g = ((pos % RB) >> 4) ^ wswz<BK>(r);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx[p],
                                               (__attribute__((address_space(3))) void*)(tbuf + p * TB + cc * 1024),
                                               16, (uint32_t)((r * K + k0 + 8 * g) * 2), 0, 0, 0);
    }
  }
};

// The wide kernel's barrier: this wave's LDS stores done and at most N of its
// vector-memory requests (the newest, still landing in the buffer two stages
// ahead) in flight, then s_barrier.  __syncthreads() would wait for every
// request.  The empty asm statements keep the compiler from moving LDS
// accesses across the barrier.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070 | N);  // vmcnt(N) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The products of one stage: A = decoded weight rows (wave rows 128 wr ..),
// B = tokens (wave tokens 64 wt ..), token tiles tt in [T0, T1) of K step KS.
template <int BK>
__device__ __forceinline__ void wide_afrag(const unsigned char* cw, int KS, int wr, int m, int q, h8_t (&a)[8]) {
  constexpr int RB = 2 * BK;
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) {
    const int r = 128 * wr + 16 * rt + m;
    a[rt] = *reinterpret_cast<const h8_t*>(cw + r * RB + (((4 * KS + q) ^ wswz<BK>(r)) << 4));
  }
}
template <int P, int BK, int T0, int T1>
__device__ __forceinline__ void wide_mma(const h8_t (&a)[8], const unsigned char* ct, int KS, int wt, int m, int q,
                                         f4_t (&acc)[8][4]) {
  constexpr int RB = 2 * BK, TB = kWTok * RB;
#pragma unroll
  for (int tt = T0; tt < T1; ++tt) {
    const int r = 64 * wt + 16 * tt + m;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const h8_t b = *reinterpret_cast<const h8_t*>(ct + p * TB + r * RB + (((4 * KS + q) ^ wswz<BK>(r)) << 4));
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) acc[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[rt], b, acc[rt][tt], 0, 0, 0);
    }
  }
}

// Iteration st (register set R = (st + 1) % 2): activation copies for stage
// st + 2, the products of stage st in two halves, and between them the
// decode of stage st + 1 (its VALU work overlaps the first half's matrix
// operations) followed by the request of stage st + 3's weight bytes into
// the set just decoded.  A wave raises its issue priority while it issues a
// half's matrix operations, so the other wave of its SIMD decodes in the
// gaps rather than delaying them (0.6-3% faster with A4).  Every iteration makes the same requests (stages
// past the end re-read the last one: cache hits, never used), so each ends
// with the same wait and the compiler's own waits stay exact.
template <int P, int BK, int R>
__device__ __forceinline__ void wide_iter(WideStage<P, BK>& S, int st, int nst, unsigned char* wbuf,
                                          unsigned char* tbuf, int wv, int lane, f4_t (&acc)[8][4]) {
  constexpr int RB = 2 * BK, WB = kWRows * RB, TB = kWTok * RB;
  const int m = lane & 15, q = lane >> 4, wr = wv & 1, wt = wv >> 1;
  const unsigned char* cw = wbuf + (st & 1) * WB;
  const unsigned char* ct = tbuf + (st % 3) * P * TB;
  const int last = (nst - 1) * BK;
  S.tcopy(min((st + 2) * BK, last), tbuf + ((st + 2) % 3) * P * TB, wv, lane);
  h8_t a[8];
  wide_afrag<BK>(cw, 0, wr, m, q, a);
  __builtin_amdgcn_s_setprio(1);
  if constexpr (BK == 64) wide_mma<P, BK, 0, 4>(a, ct, 0, wt, m, q, acc);
  else wide_mma<P, BK, 0, 2>(a, ct, 0, wt, m, q, acc);
  __builtin_amdgcn_s_setprio(0);
  S.template wstore<R>(wbuf + ((st + 1) & 1) * WB);  // past the end: a buffer no one reads again
  S.template wload<R>(min((st + 3) * BK, last));
  if constexpr (BK == 64) {
    wide_afrag<BK>(cw, 1, wr, m, q, a);
    __builtin_amdgcn_s_setprio(1);
    wide_mma<P, BK, 0, 4>(a, ct, 1, wt, m, q, acc);
    __builtin_amdgcn_s_setprio(0);
  } else {
    __builtin_amdgcn_s_setprio(1);
    wide_mma<P, BK, 2, 4>(a, ct, 0, wt, m, q, acc);
    __builtin_amdgcn_s_setprio(0);
  }
  stage_barrier<WideStage<P, BK>::OPS_W + WideStage<P, BK>::OPS_T>();  // stage st + 1 is in
}

template <int P, int BK>
__global__ __launch_bounds__(kWThreads) void k_gemm_wide(WideArgs A) {
  constexpr int RB = 2 * BK;          // bytes a LDS row
  constexpr int WB = kWRows * RB;     // weight tile bytes a stage
  constexpr int TB = kWTok * RB;      // one plane's token tile bytes a stage
  // two decoded weight buffers, three activation buffers (copies run two
  // stages ahead): 160 KB for (P, BK) = (1, 64), 128 KB for (2, 32)
  __shared__ __align__(16) unsigned char lds[2 * WB + 3 * P * TB];
  unsigned char* const wbuf = lds;
  unsigned char* const tbuf = lds + 2 * WB;

  // tile: workgroups L, L + 8, ... run on one XCD and take consecutive tiles
  // (the token blocks of one row block first), so a weight block is read
  // from memory once per XCD and served from its L2 to the other token
  // blocks.  (Groups of 8 row blocks x 4 token blocks at a time were 3%
  // slower.)
  const int nrb = (A.N + kWRows - 1) / kWRows, ntb = (A.T + kWTok - 1) / kWTok;
  const int per = (int)gridDim.x / 8, L = (int)blockIdx.x;
  const int lt = (L % 8) * per + L / 8;
  if (lt >= nrb * ntb) return;
  const int n0 = (lt / ntb) * kWRows, t0 = (lt % ntb) * kWTok;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, m = lane & 15, q = lane >> 4;
  const int wr = wv & 1, wt = wv >> 1;

  WideStage<P, BK> S;
  S.init(A, n0, t0, tid);
  f4_t acc[8][4];
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[rt][tt] = f4_t{0.f, 0.f, 0.f, 0.f};

  // Stage st: its weight bytes requested in iteration st - 3 into register
  // set st % 2 and decoded into wbuf[st % 2] in iteration st - 1; its
  // activations copied into tbuf[st % 3] from iteration st - 2.  At the end
  // of an iteration a wave waits until only that iteration's requests are in
  // flight (stage st + 1's copies have landed), then the barrier.
  const int nst = A.K / BK;  // a multiple of 4
  S.template wload<0>(0);
  S.tcopy(0, tbuf, wv, lane);
  asm volatile("" ::: "memory");
  S.template wstore<0>(wbuf);
  S.template wload<1>(BK);
  S.tcopy(BK, tbuf + P * TB, wv, lane);
  asm volatile("" ::: "memory");
  S.template wload<0>(2 * BK);
  stage_barrier<2 * WideStage<P, BK>::OPS_W + WideStage<P, BK>::OPS_T>();  // stage 0 is in
  for (int st = 0; st < nst; st += 2) {
    wide_iter<P, BK, 1>(S, st, nst, wbuf, tbuf, wv, lane, acc);
    wide_iter<P, BK, 0>(S, st + 1, nst, wbuf, tbuf, wv, lane, acc);
  }
  // the last requests land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // lane (m, q) of tile (rt, tt): weight rows 4q .. 4q+3 of the tile, token m
  const float sc = *A.wS * (P == 1 && A.xS ? *A.xS : 1.0f);
  const bool vec = (A.N & 3) == 0;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int t = t0 + 64 * wt + 16 * tt + m;
    if (t >= A.T) continue;
    float* yrow = A.y + (size_t)t * A.N;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      const int n = n0 + 128 * wr + 16 * rt + 4 * q;
      const f4_t v = acc[rt][tt] * sc;
      if (vec) {
        if (n < A.N) __builtin_nontemporal_store(v, reinterpret_cast<f4_t*>(yrow + n));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n + i < A.N) yrow[n + i] = v[i];
      }
    }
  }
}

// Activation planes for the wide kernel.  A32: x = hi + lo, [2][T][K] fp16;
// each thread 8 values a step.
__global__ __launch_bounds__(256) void k_gemm_split(const float* __restrict__ x, size_t n,
                                                    uint16_t* __restrict__ planes) {
  for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8; i < n; i += (size_t)gridDim.x * 256 * 8) {
    const float4 u = *reinterpret_cast<const float4*>(x + i), v = *reinterpret_cast<const float4*>(x + i + 4);
    const float f[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
    h8_t hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi[e] = (_Float16)f[e];
      lo[e] = (_Float16)(f[e] - (float)hi[e]);
    }
    *reinterpret_cast<h8_t*>(planes + i) = hi;
    *reinterpret_cast<h8_t*>(planes + n + i) = lo;
  }
}
// A4: the quantised activations decoded (code x block scale, exact in fp16),
// [T][K]; each thread one 16-value block a step.
__global__ __launch_bounds__(256) void k_gemm_deq(const uint8_t* __restrict__ codes,
                                                  const uint8_t* __restrict__ scales, size_t n,
                                                  uint16_t* __restrict__ plane) {
  for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 16; i < n; i += (size_t)gridDim.x * 256 * 16) {
    const uint2 c = *reinterpret_cast<const uint2*>(codes + i / 2);
    const H16Scale s = h16_scale(scales[i / 16]);
    *reinterpret_cast<h8_t*>(plane + i) = h16_decode(c.x, s);
    *reinterpret_cast<h8_t*>(plane + i + 8) = h16_decode(c.y, s);
  }
}

// Workspace: the quantiser's amax counter first (at a fixed offset, so calls
// with different T on one workspace find it zero), then the tensor scale, the
// codes and the block scales of the quantised activations (A4), then the fp16
// activation planes of the wide kernel ([2][T][K] for A32, [T][K] for A4).
struct GemmWs {
  size_t amax, tscale, codes, scales, planes, total;
  GemmWs(int T, int K, int mode) {
    const bool a4 = mode == FLINT_GEMM_A4;
    size_t o = 0;
    amax = o; o = align_up(o + 4, 256);
    tscale = o; o = align_up(o + 4, 256);
    codes = o; o = align_up(o + (a4 ? (size_t)T * K / 2 : 0), 256);
    scales = o; o = align_up(o + (a4 ? (size_t)T * K / 16 : 0), 256);
    planes = o; o = align_up(o + (a4 ? 1 : 2) * (size_t)T * K * 2, 256);
    total = o;
  }
};

// The wide kernel takes calls with at least this many 256 x 256 tiles (half
// a grid of one workgroup per compute unit: a tile of K = 2,048 takes about
// 93 us with A4 and 160 us with A32, about the narrow kernel's time for a
// 6,144 x 2,048 x 2,048 call); below it the narrow kernel (256 rows x 32
// tokens a workgroup) fills more of the chip.
constexpr int kWideMinTiles = 128;

bool a16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool a4b(const void* p) { return ((uintptr_t)p & 3u) == 0; }

}  // namespace
}  // namespace flint

using namespace flint;

extern "C" {

size_t flint_nvfp4_gemm_workspace_bytes(int32_t T, int32_t K, int32_t mode) {
  if (T < 1 || K < kGChunk || K % kGChunk || (mode != FLINT_GEMM_A32 && mode != FLINT_GEMM_A4)) return 0;
  return GemmWs(T, K, mode).total;
}

int32_t flint_nvfp4_gemm(const flint_nvfp4* W, int32_t N, int32_t K, const float* X, int32_t T, int32_t mode,
                         float* Y, void* ws, size_t ws_bytes, void* stream) {
  if (!W || !W->codes || !W->scales || !W->tscale || !X || !Y || !ws) return FLINT_E_NULL;
  if (N < 1 || K < 1 || T < 1 || (mode != FLINT_GEMM_A32 && mode != FLINT_GEMM_A4)) return FLINT_E_DIMS;
  if (K % kGChunk || (int64_t)T * K > (1ll << 40) || K > (1 << 20)) return FLINT_E_UNSUPPORTED;
  if (!a16(W->codes) || !a4b(W->scales) || !a4b(W->tscale) || !a16(X) || !a16(Y) || !a16(ws)) return FLINT_E_ALIGN;
  if (ws_bytes < flint_nvfp4_gemm_workspace_bytes(T, K, mode)) return FLINT_E_WORKSPACE;
  int32_t st;
  if ((st = api_check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  const GemmWs w(T, K, mode);
  char* base = static_cast<char*>(ws);
  hipError_t e = hipSuccess;
  const uint8_t* xc = reinterpret_cast<uint8_t*>(base + w.codes);
  const uint8_t* xs = reinterpret_cast<uint8_t*>(base + w.scales);
  const float* xS = reinterpret_cast<float*>(base + w.tscale);
  if (mode == FLINT_GEMM_A4) {
    e = launch_quantize(X, 1, T, K, const_cast<uint8_t*>(xc), const_cast<uint8_t*>(xs), const_cast<float*>(xS),
                        reinterpret_cast<uint32_t*>(base + w.amax), s);
    if (e != hipSuccess) return api_hip_fail(e);
  }
  // the activations as fp16 planes (both kernels stage them with
  // buffer-to-LDS copies)
  uint16_t* xp = reinterpret_cast<uint16_t*>(base + w.planes);
  const size_t n = (size_t)T * K;
  const int pg = (int)std::min<size_t>((n + 256 * 16 - 1) / (256 * 16), 4096);
  if (mode == FLINT_GEMM_A4) k_gemm_deq<<<pg, 256, 0, s>>>(xc, xs, n, xp);
  else k_gemm_split<<<pg, 256, 0, s>>>(X, n, xp);
  const int64_t tiles = (int64_t)((N + kWRows - 1) / kWRows) * ((T + kWTok - 1) / kWTok);
  if (tiles >= kWideMinTiles) {
    WideArgs A{};
    A.wc = W->codes;
    A.ws = W->scales;
    A.wS = W->tscale;
    A.xp = xp;
    A.xS = mode == FLINT_GEMM_A4 ? xS : nullptr;
    A.y = Y;
    A.N = N;
    A.K = K;
    A.T = T;
    const int grid = (int)((tiles + 7) / 8 * 8);
    if (mode == FLINT_GEMM_A4) k_gemm_wide<1, 64><<<grid, kWThreads, 0, s>>>(A);
    else k_gemm_wide<2, 32><<<grid, kWThreads, 0, s>>>(A);
  } else {
    GemmArgs A{};
    A.wc = W->codes;
    A.ws = W->scales;
    A.wS = W->tscale;
    A.xp = xp;
    A.xS = mode == FLINT_GEMM_A4 ? xS : nullptr;
    A.y = Y;
    A.N = N;
    A.K = K;
    A.T = T;
    const dim3 grid((N + kGRows - 1) / kGRows, (T + kGTok - 1) / kGTok);
    if (mode == FLINT_GEMM_A4) k_gemm<1><<<grid, 256, 0, s>>>(A);
    else k_gemm<2><<<grid, 256, 0, s>>>(A);
  }
  e = hipGetLastError();
  return e == hipSuccess ? FLINT_OK : api_hip_fail(e);
}

}  // extern "C"
