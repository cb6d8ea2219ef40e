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
// gfx950's scaled-FP4 MFMA takes one power-of-two scale per 32 values, so it
// cannot carry NVFP4's E4M3 scale per 16 exactly; it is not used.
//
// Tiling: a workgroup (4 waves) owns 256 weight rows x 32 tokens; each wave
// 64 rows (four 16-row tiles) x the 32 tokens (two 16-token tiles), so every
// activation fragment read from LDS feeds four products.  K runs in
// chunks of 256: the chunk's activations are staged in LDS as fp16 parts
// (double-buffered; the next chunk's global loads are issued before the
// current chunk's products), each lane's weight bytes for the next chunk are
// requested before the current chunk is multiplied.
#include <float.h>

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
  const uint8_t* wc;  // W codes [N][K/2]
  const uint8_t* ws;  // W scales [N][K/16]
  const float* wS;    // W tensor scale
  const float* x;     // A32: X [T][K]
  const uint8_t* xc;  // A4: X codes [T][K/2]
  const uint8_t* xs;  // A4: X scales [T][K/16]
  const float* xS;    // A4: X tensor scale
  float* y;           // Y [T][N]
  int N, K, T;
};

// byte offset of (token row r, 8-value group g) in one part of a staged chunk:
// rows are 512 bytes; groups are XOR-swizzled by the row so that the 16 rows
// a wave reads for one product fall on different banks
__device__ __forceinline__ int stage_off(int r, int g) { return r * kGRowBytes + ((g ^ (r & 15)) << 4); }

// Activation staging, thread t: token row t >> 3, values 32 (t & 7) .. +32 of
// the chunk (groups 4 (t & 7) .. +3).
template <int P>
struct Stage {
  float4 v[8];     // A32
  uint4 c;         // A4 codes
  uint32_t s;      // A4 scale bytes
};

template <int P>
__device__ __forceinline__ void stage_load(const GemmArgs& A, int t0, int kc, int tid, Stage<P>& st) {
  const int r = tid >> 3, seg = tid & 7, tok = t0 + r;
  if constexpr (P == 2) {
    if (tok < A.T) {
      const float4* src = reinterpret_cast<const float4*>(A.x + (size_t)tok * A.K + kc + 32 * seg);
#pragma unroll
      for (int i = 0; i < 8; ++i) st.v[i] = src[i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) st.v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  } else {
    if (tok < A.T) {
      st.c = *reinterpret_cast<const uint4*>(A.xc + (size_t)tok * (A.K / 2) + kc / 2 + 16 * seg);
      st.s = *reinterpret_cast<const uint16_t*>(A.xs + (size_t)tok * (A.K / 16) + kc / 16 + 2 * seg);
    } else {
      st.c = make_uint4(0, 0, 0, 0);
      st.s = 0;
    }
  }
}

template <int P>
__device__ __forceinline__ void stage_store(const Stage<P>& st, unsigned char* buf, int tid) {
  const int r = tid >> 3, seg = tid & 7;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int off = stage_off(r, 4 * seg + u);
    if constexpr (P == 2) {
      const float f[8] = {st.v[2 * u].x, st.v[2 * u].y, st.v[2 * u].z, st.v[2 * u].w,
                          st.v[2 * u + 1].x, st.v[2 * u + 1].y, st.v[2 * u + 1].z, st.v[2 * u + 1].w};
      h8_t hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = (_Float16)f[e];
        lo[e] = (_Float16)(f[e] - (float)hi[e]);
      }
      *reinterpret_cast<h8_t*>(buf + off) = hi;
      *reinterpret_cast<h8_t*>(buf + kGPartBytes + off) = lo;
    } else {
      const uint32_t w = (&st.c.x)[u];
      *reinterpret_cast<h8_t*>(buf + off) = h16_decode(w, h16_scale((st.s >> (8 * (u >> 1))) & 0xFF));
    }
  }
}

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

  Stage<P> st;
  stage_load<P>(A, t0, 0, tid, st);
  WFrag cur;
  wfrag_load(A, rows, 0, q, cur);
  stage_store<P>(st, sbuf[0], tid);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const bool more = c + 1 < nch;
    WFrag nxt;
    if (more) {
      stage_load<P>(A, t0, (c + 1) * kGChunk, tid, st);
      wfrag_load(A, rows, (c + 1) * kGChunk, q, nxt);
    }
    const unsigned char* buf = sbuf[c & 1];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      h8_t b[kRT];
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
        b[rt] = h16_decode((&cur.c[rt][j >> 2].x)[j & 3], h16_scale((cur.s[rt] >> (8 * (j >> 1))) & 0xFF));
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
    if (more) {
      stage_store<P>(st, sbuf[(c + 1) & 1], tid);
      cur = nxt;
    }
    __syncthreads();
  }
  // lane (m, q) holds tokens 4q .. 4q+3 of each token tile for weight row m
  const float S = *A.wS * (P == 1 ? *A.xS : 1.0f);
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

// A4 workspace: the quantiser's amax counter first (at a fixed offset, so
// calls with different T on one workspace find it zero), then the tensor
// scale, the codes and the block scales of the quantised activations.
struct GemmWs {
  size_t amax, tscale, codes, scales, total;
  GemmWs(int T, int K) {
    size_t o = 0;
    amax = o; o = align_up(o + 4, 256);
    tscale = o; o = align_up(o + 4, 256);
    codes = o; o = align_up(o + (size_t)T * K / 2, 256);
    scales = o; o = align_up(o + (size_t)T * K / 16, 256);
    total = o;
  }
};

bool a16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool a4b(const void* p) { return ((uintptr_t)p & 3u) == 0; }

}  // namespace
}  // namespace flint

using namespace flint;

extern "C" {

size_t flint_nvfp4_gemm_workspace_bytes(int32_t T, int32_t K, int32_t mode) {
  if (T < 1 || K < kGChunk || K % kGChunk || (mode != FLINT_GEMM_A32 && mode != FLINT_GEMM_A4)) return 0;
  return mode == FLINT_GEMM_A4 ? GemmWs(T, K).total : 256;
}

int32_t flint_nvfp4_gemm(const flint_nvfp4* W, int32_t N, int32_t K, const float* X, int32_t T, int32_t mode,
                         float* Y, void* ws, size_t ws_bytes, void* stream) {
  if (!W || !W->codes || !W->scales || !W->tscale || !X || !Y || !ws) return FLINT_E_NULL;
  if (N < 1 || K < 1 || T < 1 || (mode != FLINT_GEMM_A32 && mode != FLINT_GEMM_A4)) return FLINT_E_DIMS;
  if (K % kGChunk || (int64_t)T * K > (1ll << 40)) return FLINT_E_UNSUPPORTED;
  if (!a16(W->codes) || !a4b(W->scales) || !a4b(W->tscale) || !a16(X) || !a16(Y) || !a16(ws)) return FLINT_E_ALIGN;
  if (ws_bytes < flint_nvfp4_gemm_workspace_bytes(T, K, mode)) return FLINT_E_WORKSPACE;
  int32_t st;
  if ((st = api_check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  GemmArgs A{};
  A.wc = W->codes;
  A.ws = W->scales;
  A.wS = W->tscale;
  A.x = X;
  A.y = Y;
  A.N = N;
  A.K = K;
  A.T = T;
  const dim3 grid((N + kGRows - 1) / kGRows, (T + kGTok - 1) / kGTok);
  hipError_t e;
  if (mode == FLINT_GEMM_A4) {
    const GemmWs w(T, K);
    char* base = static_cast<char*>(ws);
    A.xc = reinterpret_cast<uint8_t*>(base + w.codes);
    A.xs = reinterpret_cast<uint8_t*>(base + w.scales);
    A.xS = reinterpret_cast<float*>(base + w.tscale);
    e = launch_quantize(X, 1, T, K, const_cast<uint8_t*>(A.xc), const_cast<uint8_t*>(A.xs),
                        const_cast<float*>(A.xS), reinterpret_cast<uint32_t*>(base + w.amax), s);
    if (e != hipSuccess) return api_hip_fail(e);
    k_gemm<1><<<grid, 256, 0, s>>>(A);
  } else {
    k_gemm<2><<<grid, 256, 0, s>>>(A);
  }
  e = hipGetLastError();
  return e == hipSuccess ? FLINT_OK : api_hip_fail(e);
}

}  // extern "C"
