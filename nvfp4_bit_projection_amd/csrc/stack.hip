// stack.hip -- persistent batch-1 decode of the whole MoE layer stack plus the
// NVFP4 head, one launch per call.
//
// Method [P2 "Recursive Releases Flint, a 40B MoE Coding Model That Runs
// Locally at 125 Tokens per Second", "How does Flint's architecture work?":
// 47 MoE layers, router picks 6 experts plus an always-on shared expert; P3
// "Flint: 125 tokens a second is what 2.5B active parameters buy at
// 273 GB/s", "The shape, read from the headers" and "Why active parameters
// set the speed": batch-1 decode reads each touched weight once, so the step
// is bound by weight bytes].  The pages' own answer to per-kernel launch cost
// is one fused kernel for the whole decode pass ("Custom Inference Kernels",
// P1); this is the MI355X form of that idea.
//
// Geometry.  256 workgroups of 512 threads, one per compute unit, all
// resident at once.  Workgroups are dealt to the 8 XCDs
// round-robin, so workgroup b sits on XCD b % 8: group g = b % 8 is the 32
// workgroups of one XCD, and li = b / 8 is the index inside the group.
//
// Work split of one layer (E experts, top-k, width I, shared width Is):
//  A  workgroup b owns router row b (the fp32 router is read once per
//     layer): its logit is (row . h) * s, s the RMSNorm scale of the
//     residual h, both sums formed while h arrived (phase D of the layer
//     before), and goes into the logit exchange of every group; u = s h;
//     each group computes the SwiGLU of its 1/8 slice of the shared
//     expert's rows;
//  B  the first wave of every workgroup gathers the E logits and takes the
//     top k, then the group computes the SwiGLU of its 1/8 slice (I/8 rows)
//     of each chosen expert; the down-projection weights of phase C are
//     loaded here too;
//  C  the group multiplies its slice of the hidden activations by the
//     matching 1/8 column slice of every down matrix (routed, weighted by the
//     routing weights, and shared): a partial output for all H rows;
//  D  the 8 partial outputs are summed (fixed order, across 8 lanes of
//     the polling waves) and added to the residual; the polling threads form
//     the next layer's router and norm sums from the new residual they
//     receive.
// Exchanges.  A -> B logits (across XCDs), B -> C hidden slice (inside a
// group), C -> D partial outputs (across groups) and D -> A the new residual
// (inside a group).  Values travel as 64-bit (value, epoch) pairs; a
// consumer reads them with 128-bit loads until every epoch matches, so no
// separate flag or barrier is needed.  Epochs are unique per (call, token,
// layer, exchange).  Every wait is bounded: on time-out a workgroup raises
// the error flag and all workgroups leave the kernel.
#include <float.h>
#include <limits.h>

#include <atomic>

#include "flint_device.h"
#include "flint_internal.h"

namespace flint {

constexpr int kGroups = 8;
constexpr int kGroupWGs = 32;
constexpr int kStackWGs = kGroups * kGroupWGs;
constexpr int kStackThreads = 512;
constexpr int kStackWaves = kStackThreads / 64;
constexpr int kSliceK = 512;            // k * (I/8) + Is/8: one group's slice of the hidden layer
constexpr int kHeadRowsPerWave = 8;
constexpr int kCommWaves = 4;                      // waves that poll the exchanges
constexpr int kCommThreads = kCommWaves * 64;
static_assert(kStackWaves - kCommWaves == 4 && kCommWaves == 4,
              "four loading waves hold the router row; four polling waves sum its dot product and the norm");
constexpr int kGateUpComm = 2;                     // routed gate/up pairs per communication wave
constexpr int kDownPasses = 2;                     // 4-row down-projection passes of every wave
constexpr uint32_t kSpinLimit = 1u << 22;
#ifndef FLINT_POLL_SLEEP
#define FLINT_POLL_SLEEP 0
#endif
// back-off between polls of data that has not arrived (units of 64 clocks).
// None by default: with the current exchanges every back-off measured
// (1, 2 and 4 sleeps of 64 clocks) made the stack slower
__device__ __forceinline__ void poll_backoff() {
  if (FLINT_POLL_SLEEP > 0) __builtin_amdgcn_s_sleep(FLINT_POLL_SLEEP);
}
// Placement of the logit exchange.  Device-scope traffic to a 4 KB block is
// served from one of the two halves of the chip: on this part the XCDs 0-3
// and 4-7 each reach half of the blocks in about 420 ns and the other half in
// about 615 ns (one way, from ping-pong between XCD pairs), and which half is
// near alternates every 8 KB of address, with a phase fixed for each 2 MB
// page.  The logit copy that XCD g polls sits in blocks near g's half: in a
// 32 KB-aligned area, blocks 4 m + 2 c + {0, 1} are class c, and half h = g / 4
// uses class h ^ phase.  The area lies in one 2 MB page; its phase is measured
// once per workspace (exchange_phase below).  Each of the 16 lines of a copy
// is in a block of its own.
constexpr uint32_t kXchBlock = 4096;
constexpr int kLogitLines = kMaxExperts / 16;                        // 16 (value, epoch) pairs per 128-byte line
constexpr uint32_t kS2Area = kLogitLines * kGroups * kXchBlock;      // 512 KB
constexpr uint32_t kPhaseProbe = 3072;                               // byte of a block the logits never use
// byte offset of pair e of group g's logit copy, parity par: line j = e / 16
// of the copy is block 8 j + gb of the area, parity par at byte 2048 par
__device__ __forceinline__ uint32_t s2_off(int par, int g, int e, int phase) {
  const int q = g & 3, cls = (g >> 2) ^ phase;
  const int gb = (q & 1) + (q >> 1) * 4 + 2 * cls;
  return (uint32_t)((e >> 4) * 8 + gb) * kXchBlock + (uint32_t)par * 2048u + (uint32_t)(e & 15) * 8u;
}
// Activation vectors in LDS are stored in rows of 32 values padded to 36, so
// that the 64 lanes of a wave, each reading its own 32 consecutive values with
// 128-bit loads, hit distinct banks.
constexpr int kRowPad = 36;
__device__ __forceinline__ int padded(int e) { return (e >> 5) * kRowPad + (e & 31); }

struct StackParams {
  const StackTable* table;
  int l0;  // first layer of the table to run
  int L, E, I, k, Is, V, T;
  float eps;
  const float* x;
  float* logits;
  int32_t* argmax;
  int32_t* routes;
  uint32_t* ctrl;  // [0] epoch base, [1] error flag, [2] 1 + the logit area's phase (0: not measured yet)
  uint8_t* s2;     // logit exchange area (kS2Area bytes, 32 KB aligned, in one 2 MB page)
  uint64_t* s3;    // [2][8][512]  hidden slice
  uint64_t* s4a;   // [2][8][2048] partial outputs
  uint64_t* s4b;   // [2][8][2048] residual
  uint64_t* hp;    // [2][256][2]  head (max, index)
  int64_t* trace;  // optional [2][L+1][kTracePoints] phase timestamps of workgroups 0 and 255
  float* h_out;    // k_stack_decode<false> (one token, no head): the final residual [H]
  StackQkv qkv;    // k_stack_decode<false>: rows applied to the final residual's norm (out == nullptr: none)
  uint32_t stress_seed;  // stress instantiation: seed of the injected delays
  uint32_t spin_limit;   // stress instantiation: polls before a wait gives up
};

// In-place use (h_out == x, one launch per layer of a longer model) relies on
// every workgroup storing a partial output of every layer: each workgroup of
// an XCD owns 64 rows of the 2,048-wide partial output, so the residual
// exchange cannot finish before every workgroup has read x.
static_assert(kGroupWGs * 64 == kHidden, "every workgroup owns 64 rows of the partial outputs");

constexpr int kTracePoints = 32;
constexpr int kTraceMaxLayers = kMaxStackLayers;

// Exchange scopes.  Values that cross XCDs are stored with device-scope
// stores (written through to the coherence point beyond the per-XCD L2) and
// polled with device-scope loads.  Values exchanged inside one XCD stay in
// its shared L2: plain stores (the per-CU vector cache is write-through) and
// loads that miss the per-CU cache (SC0) and stream (NT) -- about 30% less
// latency per round trip.  The kernel checks at start that workgroup b runs
// on XCD b % 8, which the in-XCD exchanges rely on.
enum class Scope { kXcd, kDevice };
template <Scope sc>
__device__ __forceinline__ void put_pair(uint64_t* p, float v, uint32_t ep) {
  const uint64_t x = (uint64_t)__float_as_uint(v) | ((uint64_t)ep << 32);
  if constexpr (sc == Scope::kDevice)
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
template <Scope sc>
constexpr int poll_aux() { return sc == Scope::kDevice ? 16 /* SC1 */ : 3 /* SC0 | NT */; }
__device__ __forceinline__ uint32_t xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its global loads and stores (the exchanges carry their
// own epochs, and loads issued ahead of time stay in flight across it).
// The signal fences keep the compiler from moving memory accesses across.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// maximum over the wave of an int, uniform (scalar) result: four fused DPP
// steps leave each row's maximum in every lane of the row, and the scalar
// unit takes the maximum of the four rows
__device__ __forceinline__ int wave_max_i32_s(int v) {
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppXor1, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppXor2, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppHalfMirror, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppMirror, 0xF, 0xF, true));
  const int a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const int c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

struct WaitCtx {
  uint32_t* err;
  int* bad;        // LDS flag
  uint32_t limit;  // polls before a wait gives up
};

// Raise the error flag after a wait timed out (or another workgroup raised it).
__device__ __forceinline__ bool poll_gave_up(uint32_t& spins, const WaitCtx& w) {
  ++spins;
  if (spins > w.limit || ((spins & 1023) == 0 && ld_dev_u32(w.err))) {
    atomicOr(w.err, 1u);
    *w.bad = 1;
    return true;
  }
  poll_backoff();
  return false;
}

// Poll until pairs [0, n) (n even, n <= 8 * kCommThreads) of buf carry epoch
// ep; values -> dst (pair i to dst[i], or to its padded row position).  Called
// by the communication waves only; each thread owns up to four 128-bit
// chunks and keeps all of its outstanding chunks in flight at once.
// Router partial dot product and sum of squares of one (value, value) pair of
// rows 2c, 2c + 1, and the fixed order in which a polling thread adds its
// four pairs' parts; the same arithmetic whether the values come from an
// exchange or from LDS, so that a layer gives the same bits either way.
__device__ __forceinline__ float pair_dot(float2 w, float v0, float v1) { return __builtin_fmaf(w.y, v1, w.x * v0); }
__device__ __forceinline__ float pair_sq(float v0, float v1) { return __builtin_fmaf(v1, v1, v0 * v0); }
__device__ __forceinline__ float sum4(const float* p) { return (p[0] + p[1]) + (p[2] + p[3]); }

// With kDot, once all of the thread's pairs have arrived, each (rows 2c,
// 2c + 1) gives pair_dot(wrow[2c], wrow[2c + 1]; v0, v1) and pair_sq(v0, v1)
// (wrow in LDS), added in a fixed order into dacc and sacc.
template <Scope sc, bool kDot = false>
__device__ __forceinline__ void poll_pairs(const uint64_t* buf, int n, uint32_t ep, float* dst, const WaitCtx& w,
                                           bool pad = false, const float* wrow = nullptr, float* dacc = nullptr,
                                           float* sacc = nullptr) {
  constexpr int kMaxPer = 4;
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t*>(buf), 0, n * 8, 0x00020000);
  const int t = threadIdx.x;
  uint32_t pending = 0;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i)
    if (t + i * kCommThreads < n / 2) pending |= 1u << i;
  uint32_t spins = 0;
  float2 got[kMaxPer];  // kDot: the thread's pairs, kept for the sums after the loop
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) got[i] = make_float2(0.0f, 0.0f);
  while (pending) {
    uint32_t v[kMaxPer][4];
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      if (pending & (1u << i)) {
        auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, (t + i * kCommThreads) * 16, 0, poll_aux<sc>());
        v[i][0] = x[0]; v[i][1] = x[1]; v[i][2] = x[2]; v[i][3] = x[3];
      }
    }
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      if ((pending & (1u << i)) && v[i][1] == ep && v[i][3] == ep) {
        const int c = t + i * kCommThreads;
        const int d = pad ? padded(2 * c) : 2 * c;  // 2c, 2c+1 share a row
        const float v0 = __uint_as_float(v[i][0]), v1 = __uint_as_float(v[i][2]);
        dst[d] = v0;
        dst[d + 1] = v1;
        if constexpr (kDot) got[i] = make_float2(v0, v1);
        pending &= ~(1u << i);
      }
    }
    if (!pending || poll_gave_up(spins, w)) break;
  }
  if constexpr (kDot) {
    static_assert(kMaxPer == 4, "four parts per thread");
    float dp[kMaxPer], sp[kMaxPer];
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int c = t + i * kCommThreads;
      const float2 ww = (t + i * kCommThreads < n / 2) ? *reinterpret_cast<const float2*>(wrow + 2 * c)
                                                        : make_float2(0.0f, 0.0f);
      dp[i] = pair_dot(ww, got[i].x, got[i].y);
      sp[i] = pair_sq(got[i].x, got[i].y);
    }
    *dacc = sum4(dp);
    *sacc = sum4(sp);
  }
}

__device__ __forceinline__ void lds_x32(const float* src, float* xv) {
  const float4* p = reinterpret_cast<const float4*>(src);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float4 v = p[i];
    xv[4 * i] = v.x; xv[4 * i + 1] = v.y; xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
  }
}

// RMSNorm scale s of h (kHidden values) -> u = s * h (padded rows); two
// barriers.  on_scale(s) runs in every wave as soon as s is known, before u
// is written.
template <class F>
__device__ __forceinline__ void rms_to_u(const float* h, float* u, float* red, float eps, F&& on_scale) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  float v[kHidden / kStackThreads];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kHidden / kStackThreads; ++i) {
    v[i] = h[t + i * kStackThreads];
    ss = __builtin_fmaf(v[i], v[i], ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[w] = ss;
  wg_barrier();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kStackWaves; ++i) tot += red[i];
  const float s = 1.0f / sqrtf(tot * (1.0f / kHidden) + eps);
  on_scale(s);
#pragma unroll
  for (int i = 0; i < kHidden / kStackThreads; ++i) u[padded(t + i * kStackThreads)] = v[i] * s;
  wg_barrier();
}
__device__ __forceinline__ void rms_to_u(const float* h, float* u, float* red, float eps) {
  rms_to_u(h, u, red, eps, [](float) {});
}

// The layer table (device pointers) is copied to LDS at the start, so that a
// pointer costs an LDS read rather than a scalar-cache miss on the way to a
// dependent load.  Word indices of one layer's entry:
enum LayerWord {
  kWRouter, kWGateC, kWGateS, kWUpC, kWUpS, kWDownC, kWDownS, kWExpTs,
  kWSgC, kWSgS, kWSgT, kWSuC, kWSuS, kWSuT, kWSdC, kWSdS, kWSdT, kLayerWords
};
static_assert(sizeof(flint_moe_layer) == kLayerWords * sizeof(uint64_t), "layer entry is a pointer array");
static_assert(sizeof(flint_nvfp4) == 3 * sizeof(uint64_t), "head entry is a pointer array");

struct StackLds {
  float h[kHidden];                                  // residual stream
  float u[kHidden / 32 * kRowPad];                   // normalised residual, padded rows
  float hs[kSliceK / 32 * kRowPad];                  // this group's hidden slice, padded rows
  float hp[2 * kStackWGs];                           // head partials (max, index)
  float red[kStackWaves];
  float rp[kCommWaves];                              // router logit: one partial dot per polling wave
  float rq[kCommWaves];                              // sum of squares of the residual: one part per polling wave
  float wr[kHidden];                                 // router row of this workgroup for the next layer
  float w[kMaxTopK];
  int32_t pk[kMaxTopK];                              // picks of phase B: (layer tag << 8) | expert
  float bv[kStackWaves];
  int32_t bi[kStackWaves];
  int32_t bad;
  uint32_t ctl[3];                                   // control words read at the start
  uint64_t tab[kMaxStackLayers * kLayerWords + 3];   // layer table, then the head
  int64_t tr[(kTraceMaxLayers + 1) * kTracePoints];  // phase stamps of the first token
};

// pointer word of the LDS table as a wave-uniform (scalar) pointer
template <class T>
__device__ __forceinline__ T* tab_ptr(const StackLds& S, int word) {
  const uint64_t v = S.tab[word];
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Block and wave coordinates shared by both roles.
struct StackCoord {
  int t, lane, wv, g, li;
  int L, E, I, k, Is, V;
  int Ix, Isx, nroutedx;
  uint32_t base;
  int phase;  // placement phase of the logit area
  bool tracing;
};

// Stress instantiation only: before an exchange store, a wave sleeps for a
// pseudo-random time (a hash of the seed, workgroup, wave, token, layer and
// store site; one store in four, up to 15 x 32 x 64 clocks, about 14 us), so
// that workgroups and waves reach every exchange in arbitrary orders and with
// arbitrary skew.  The results must not change.
template <bool kStress>
__device__ __forceinline__ void stress_delay(const StackParams& P, int tok, int l, int site) {
  if constexpr (kStress) {
    uint32_t h = P.stress_seed * 0x9E3779B1u ^ blockIdx.x * 0x85EBCA77u ^ (uint32_t)(tok * 128 + l) * 0xC2B2AE3Du ^
                 (uint32_t)site * 0x27D4EB2Fu ^ (threadIdx.x >> 6) * 0x165667B1u;
    h ^= h >> 15; h *= 0x2C1B3C6Du; h ^= h >> 12; h *= 0x297A2D39u; h ^= h >> 15;
    h = __builtin_amdgcn_readfirstlane(h);
    if ((h & 3) == 0) {
      const int n = (int)((h >> 2) & 15);
      for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(32);
    }
  }
}

// One role's pass over all tokens.  Both roles execute the same sequence of
// workgroup barriers (marked B1..B5 per layer, H1..H5 per token) and
// leave at the same barrier on error; returns false then.
//
// Communication role (waves 0-3): polls every exchange (the first wave alone
// gathers the logits and takes the top k), computes 2 of the 12 routed
// gate/up pairs per wave and workgroup, and forms the router and norm sums
// from the residual it receives.  A wave's loads complete in issue order, so
// a wave that polls must not have weight loads in flight.
// Loading role (waves 4-7): the shared expert's gate/up (phase A), one
// routed gate/up pair and the down-projection operands (phase B), the
// partial outputs (phase C), and the next layer's router row (a quarter per
// wave, to LDS in phase C) and shared rows, requested behind the down
// operands.  The polling waves also sum the partial outputs of the
// workgroup's residual rows and publish them (end of phase C).
template <bool kComm, bool kHead, bool kStress>
__device__ bool stack_role(const StackParams& P, StackLds& S, const StackCoord& C) {
  const int t = C.t, lane = C.lane, wv = C.wv, g = C.g, li = C.li;
  const int L = C.L, E = C.E, I = C.I, k = C.k, Is = C.Is, V = C.V;
  const int Ix = C.Ix, Isx = C.Isx, nroutedx = C.nroutedx;
  const int lw = wv - kCommWaves;  // loading-wave index (loading role)
  WaitCtx wc{P.ctrl + 1, &S.bad, kStress ? P.spin_limit : kSpinLimit};
#define FLINT_TRACE_AT(tid_, l_, i_)                                                                 \
  do {                                                                                                 \
    if (C.tracing && t == (tid_) && tok == 0) S.tr[(l_) * kTracePoints + (i_)] = wall_clock64();       \
  } while (0)
#define FLINT_TRACE(l_, i_) FLINT_TRACE_AT(0, l_, i_)
#define FLINT_TRACE_LOAD(l_, i_) FLINT_TRACE_AT(kCommThreads, l_, i_)

  // ---- loading role: phase-A operands, requested one layer ahead and held
  // in registers: the first loading wave holds router row blockIdx.x (every
  // router row is read by exactly one workgroup of the chip), every loading
  // wave one pair qa of the shared expert and its tensor scales.
  // Unconditional loads (a wave without a row reads row 0 and ignores it), so
  // that no branch join forces an early wait on the data.
  // router row of this workgroup (if < E); the stress instantiation permutes
  // the roles inside each XCD, and with them the rows
  const int rrow = kStress ? g + kGroups * li : (int)blockIdx.x;
  const int qa = li + kGroupWGs * lw;
  // the loading waves split the router row: wave lw holds columns
  // 512 lw .. 512 lw + 511
  constexpr int kRouterCols = kHidden / (kStackWaves - kCommWaves);
  float4 wr[kRouterCols / 256];
  uint4 cgs = make_uint4(0, 0, 0, 0), cus = make_uint4(0, 0, 0, 0);
  uint32_t sgs = 0, sus = 0;
  float tgs = 0.0f, tus = 0.0f;
  bool have_a = false;  // this layer's phase-A operands were requested earlier
  // Every loading wave issues the same loads, with no branch around them, so
  // that the wait counts for data requested before them are exact (a branch
  // join makes the compiler wait as if the longer path had been taken).
  // live false (no next layer in this call): the buffers get a size of 0, so
  // the loads return zeros and touch no memory.
  auto load_phase_a = [&](int lx, bool live) {
    const int w0 = lx * kLayerWords;
    const rsrc_t rr =
        make_rsrc(tab_ptr<const float>(S, w0 + kWRouter), live && rrow < E ? (uint64_t)E * kHidden * 4 : 0);
    const uint32_t r0 = rrow < E ? (uint32_t)rrow : 0u;
#pragma unroll
    for (int i = 0; i < kRouterCols / 256; ++i)
      wr[i] = bload_f4_nt(rr, (r0 * kHidden + kRouterCols * lw + 256 * i) * 4 + 16 * lane);
    const uint32_t row = (uint32_t)(g * Isx + (qa < Isx ? qa : 0));
    const uint64_t nc = live ? (uint64_t)Is * kHidden / 2 : 0, ns = live ? (uint64_t)Is * kHidden / 16 : 0;
    cgs = bload_u4_nt(make_rsrc(tab_ptr<const uint8_t>(S, w0 + kWSgC), nc), row * (kHidden / 2) + 16 * lane);
    sgs = bload_u16_nt(make_rsrc(tab_ptr<const uint8_t>(S, w0 + kWSgS), ns), row * (kHidden / 16) + 2 * lane);
    cus = bload_u4_nt(make_rsrc(tab_ptr<const uint8_t>(S, w0 + kWSuC), nc), row * (kHidden / 2) + 16 * lane);
    sus = bload_u16_nt(make_rsrc(tab_ptr<const uint8_t>(S, w0 + kWSuS), ns), row * (kHidden / 16) + 2 * lane);
    tgs = sload_f32(tab_ptr<const float>(S, w0 + kWSgT), 0);
    tus = sload_f32(tab_ptr<const float>(S, w0 + kWSuT), 0);
  };
  // SwiGLU of routed gate/up pair p of this group's slice: loads ...
  struct PairOps {
    uint4 cg, cu;
    uint32_t sg, su;
    float Sg, Su;
  };
  // The layer's routed gate/up buffers, set up before the picks are known so
  // that a pick is followed by its loads at once.
  struct PairRs {
    rsrc_t gc, uc, gs, us;
    const float* ts;  // expert tensor scales [E][3] (gate, up, down)
  };
  auto pair_rs = [&](int w0) {
    const uint64_t nc = (uint64_t)E * I * kHidden / 2, ns = (uint64_t)E * I * kHidden / 16;
    PairRs r;
    r.gc = make_rsrc(tab_ptr<const uint8_t>(S, w0 + kWGateC), nc);
    r.uc = make_rsrc(tab_ptr<const uint8_t>(S, w0 + kWUpC), nc);
    r.gs = make_rsrc(tab_ptr<const uint8_t>(S, w0 + kWGateS), ns);
    r.us = make_rsrc(tab_ptr<const uint8_t>(S, w0 + kWUpS), ns);
    r.ts = tab_ptr<const float>(S, w0 + kWExpTs);
    return r;
  };
  // pair p of this group's slice of expert e (the pick of slot p / Ix)
  auto load_pair = [&](const PairRs& R, int p, int e) {
    const int rl = (p < nroutedx ? p : 0) % Ix;
    const uint32_t row = (uint32_t)(e * I + g * Ix + rl);
    PairOps o;
    o.cg = bload_u4_nt(R.gc, row * (kHidden / 2) + 16 * lane);
    o.cu = bload_u4_nt(R.uc, row * (kHidden / 2) + 16 * lane);
    o.sg = bload_u16_nt(R.gs, row * (kHidden / 16) + 2 * lane);
    o.su = bload_u16_nt(R.us, row * (kHidden / 16) + 2 * lane);
    // (vector loads: a scalar load here would make the wave's next LDS wait
    // also wait for it)
    // (vector loads: a scalar load here would make the wave's next LDS wait,
    // such as the next pick or the down operands' expert, wait for it too)
    const rsrc_t rts = make_rsrc(R.ts, (uint64_t)E * 3 * 4);
    o.Sg = bload_f32(rts, (uint32_t)(3 * e + 0) * 4);
    o.Su = bload_f32(rts, (uint32_t)(3 * e + 1) * 4);
    return o;
  };
  // ... and the SwiGLU value g(x) * u(x) with g = silu(gate . x)
  auto pair_value = [&](const PairOps& o, const float* xv) {
    const float gv = wave_sum(nvfp4_lane_dot32(o.cg, o.sg, xv)) * o.Sg;
    const float av = wave_sum(nvfp4_lane_dot32(o.cu, o.su, xv)) * o.Su;
    return silu(gv) * av;
  };

  const rsrc_t rx = make_rsrc(P.x, (uint64_t)P.T * kHidden * 4);
  for (int tok = 0; tok < P.T; ++tok) {
    // residual stream <- x_t
#pragma unroll
    for (int i = 0; i < kHidden / kStackThreads; ++i)
      S.h[t + i * kStackThreads] = bload_f32(rx, (uint32_t)(tok * kHidden + t + i * kStackThreads) * 4);
    wg_barrier();

    for (int l = 0; l < L; ++l) {
      const int w0 = l * kLayerWords;
      const int par = l & 1;
      const uint32_t ep0 = C.base + 1u + (uint32_t)((tok * (L + 1) + l) * 4);
      uint64_t* s3 = P.s3 + ((size_t)par * kGroups + g) * kSliceK;
      uint64_t* s4a = P.s4a + (size_t)par * kGroups * kHidden;
      uint64_t* s4b = P.s4b + ((size_t)par * kGroups + g) * kHidden;

      // ---------------------------------------------------------- phase A
      FLINT_TRACE(l, 0);
      if (!kComm && !have_a) {
        load_phase_a(l, true);
      }
      // router logit rrow = (router row . residual) * the norm's scale,
      // stored into the logit exchange of every group by the first loading
      // wave as soon as the scale is known.
      const bool rwave = !kComm && lw == 0 && rrow < E;  // uniform
      auto publish_logit = [&](float sc) {
        if (rwave) {
          stress_delay<kStress>(P, tok, l, 0);
          const float racc = sum4(S.rp);
          if (lane < kGroups)
            put_pair<Scope::kDevice>(reinterpret_cast<uint64_t*>(P.s2 + s2_off(par, lane, rrow, C.phase)), racc * sc,
                                     ep0);
          FLINT_TRACE_LOAD(l, 8);
        }
      };
      if (l == 0) {
        // a call's or token's first layer: the residual did not come through
        // the exchange, so the polling waves take the same parts of it from
        // LDS (the router row goes there from the loading waves' registers)
        if constexpr (!kComm) {
#pragma unroll
          for (int i = 0; i < kRouterCols / 256; ++i)
            *reinterpret_cast<float4*>(S.wr + kRouterCols * lw + 256 * i + 4 * lane) = wr[i];
        }
        wg_barrier();  // B0: router row in LDS
        if constexpr (kComm) {
          float dp[4], sp[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = t + i * kCommThreads;
            const float2 ww = *reinterpret_cast<const float2*>(S.wr + 2 * c);
            const float2 hv = *reinterpret_cast<const float2*>(S.h + 2 * c);
            dp[i] = pair_dot(ww, hv.x, hv.y);
            sp[i] = pair_sq(hv.x, hv.y);
          }
          const float d = wave_sum(sum4(dp)), q = wave_sum(sum4(sp));
          if (lane == 0) {
            S.rp[wv] = d;
            S.rq[wv] = q;
          }
        }
        wg_barrier();  // B0'
      }
      // The polling waves have the parts of the router dot product and of the
      // sum of squares (summed while the residual arrived, in phase D of the
      // previous layer, or just above): the logit goes out at once, and u =
      // s h needs one barrier.
      {
        const float sc = 1.0f / sqrtf(sum4(S.rq) * (1.0f / kHidden) + P.eps);
        publish_logit(sc);
#pragma unroll
        for (int i = 0; i < kHidden / kStackThreads; ++i)
          S.u[padded(t + i * kStackThreads)] = S.h[t + i * kStackThreads] * sc;
        wg_barrier();  // B1
      }
      FLINT_TRACE(l, 1);
      float xv[32];  // this lane's 32 normalised activations (phases A and B)
      lds_x32(S.u + kRowPad * lane, xv);
      if constexpr (!kComm) {
        stress_delay<kStress>(P, tok, l, 1);
        if (qa < Isx) {
          const float gv = wave_sum(nvfp4_lane_dot32(cgs, sgs, xv)) * tgs;
          const float av = wave_sum(nvfp4_lane_dot32(cus, sus, xv)) * tus;
          if (lane == 0) put_pair<Scope::kXcd>(&s3[nroutedx + qa], silu(gv) * av, ep0 + 1);
        }
        FLINT_TRACE_LOAD(l, 9);
      }
      // ---------------------------------------------------------- phase B
      // The first communication wave gathers the E logits and takes the top
      // k.  It publishes each pick in LDS as soon as its round ends (S.pk[r]:
      // this layer's tag and the expert in one word, written by the lane that
      // held the pick), and every other wave requests the gate/up rows of its
      // pairs as soon as their expert is known, so the routed loads overlap
      // the remaining rounds; the first wave takes the pairs of the last pick.
      // Routed gate/up pairs p = li + 32 q of this group's slice: q = 2 (wv -
      // 1) + {0, 1} for communication waves 1-3, q = 6 + lw for a loading
      // wave, q = 10 + {0, 1} for the first wave.
      // 24-bit tag of this (token, layer), never 0 (0 marks no layer); a slot
      // is rewritten every layer, so a stale word never carries this tag
      const uint32_t tag = ((uint32_t)(tok * L + l) % 0xFFFFFFu) + 1u;
      // expert of pick r once it is published (S.bad and expert 0 on time-out)
      auto wait_pick = [&](int r) {
        uint32_t spins = 0;
        uint32_t v;
        while (((v = (uint32_t)__hip_atomic_load(&S.pk[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) >> 8) !=
               tag) {
          if (++spins > wc.limit) {
            S.bad = 1;
            v = 0;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        return __builtin_amdgcn_readfirstlane((int)(v & 0xFFu));
      };
      const PairRs prs = pair_rs(w0);
      constexpr int kNq = kComm ? kGateUpComm : 1;
      int pq[kNq];
#pragma unroll
      for (int pp = 0; pp < kNq; ++pp)
        pq[pp] = li + kGroupWGs * (!kComm ? 2 * kCommWaves - 2 + lw : wv == 0 ? 10 + pp : 2 * (wv - 1) + pp);
      // Down-projection operands (every wave): output rows n = 64 li + 8 wv
      // + 4 pc + lane/16, 16 lanes per row, lane chunk j = 32 columns of the
      // slice; chunks j < 12 are routed columns, the rest shared ones.  These
      // loads are issued after the wave's gate/up loads, so the gate/up
      // arithmetic does not wait for them, and they arrive well before the
      // hidden slice is complete.
      const int j = lane & 15;
      const bool routed = 32 * j < nroutedx;
      const int dslot = routed ? (32 * j) / Ix : 0;
      uint4 cd[kDownPasses];
      uint32_t sd[kDownPasses];
      float sts = 0.0f;
      // Column-sliced layouts (packed at prepare time, one block per layer in
      // the order routed codes, routed scales, shared codes, shared scales):
      // routed [E][8][H][Ix], shared [8][H][Isx], codes 2 per byte, one scale
      // byte per 16 columns.  One buffer covers the block, so a lane takes
      // its routed or shared chunk with the same two loads per pass.  The
      // routed columns' tensor scale is folded into the routing weights (by
      // the first wave); the shared one is a scalar load.
      auto load_down = [&]() {
        const uint8_t* blk = tab_ptr<const uint8_t>(S, w0 + kWDownC);
        const uint8_t* ss = tab_ptr<const uint8_t>(S, w0 + kWSdS);
        const uint32_t o_rs = (uint32_t)(tab_ptr<const uint8_t>(S, w0 + kWDownS) - blk);
        const uint32_t o_sc = (uint32_t)(tab_ptr<const uint8_t>(S, w0 + kWSdC) - blk);
        const uint32_t o_ss = (uint32_t)(ss - blk);
        const rsrc_t rd = make_rsrc(blk, (uint64_t)o_ss + (uint64_t)kHidden * Is / 16);
        const int de = S.pk[dslot] & 0xFF;
        const int doff = routed ? (32 * j) % Ix : 0;          // column in the expert's slice
        const int scol = routed ? 0 : 32 * j - nroutedx;      // column in the shared slice
        const uint32_t rslice = (uint32_t)((de * kGroups + g) * kHidden);
        const uint32_t sslice = (uint32_t)(g * kHidden);
#pragma unroll
        for (int pc = 0; pc < kDownPasses; ++pc) {
          const uint32_t n = (uint32_t)(64 * li + 8 * wv + 4 * pc + (lane >> 4));
          const uint32_t rr = rslice + n, sr = sslice + n;
          cd[pc] = bload_u4_nt(rd, routed ? rr * (Ix / 2) + doff / 2 : o_sc + sr * (Isx / 2) + scol / 2);
          sd[pc] = bload_u16_nt(rd, routed ? o_rs + rr * (Ix / 16) + doff / 16 : o_ss + sr * (Isx / 16) + scol / 16);
        }
        sts = sload_f32(tab_ptr<const float>(S, w0 + kWSdT), 0);
      };
      PairOps o[kNq];
      if (kComm && wv == 0) {
        // The E logits, four per lane (experts 4 lane .. 4 lane + 3),
        // straight into registers; the top k is taken there.
        __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(P.s2, 0, (int)kS2Area, 0x00020000);
        const uint32_t o2 = s2_off(par, g, 4 * lane, C.phase);
        uint32_t v[8];
        uint32_t spins = 0;
        while (true) {
          const auto a = __builtin_amdgcn_raw_buffer_load_b128(rs, o2, 0, poll_aux<Scope::kDevice>());
          const auto c = __builtin_amdgcn_raw_buffer_load_b128(rs, o2 + 16, 0, poll_aux<Scope::kDevice>());
          v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
          v[4] = c[0]; v[5] = c[1]; v[6] = c[2]; v[7] = c[3];
          bool ok = true;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) ok = ok && (4 * lane + jj >= E || v[2 * jj + 1] == ep0);
          if (__builtin_amdgcn_ballot_w64(!ok) == 0 || poll_gave_up(spins, wc)) break;
        }
        FLINT_TRACE(l, 2);
        // Keys ordered by (logit descending, index ascending) as one signed
        // 64-bit value: the order-preserving integer key of the logit above,
        // 255 - index below.  Experts past E get the smallest key.
        int64_t c4[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int e = 4 * lane + jj;
          const int key = e < E ? ord_key(__uint_as_float(v[2 * jj])) : INT_MIN;
          c4[jj] = (int64_t)(((uint64_t)(uint32_t)key << 32) | (uint32_t)(kMaxExperts - 1 - e));
        }
        // each lane sorts its four keys, largest first
        auto cx = [&](int i0, int i1) {
          const int64_t hi = c4[i0] > c4[i1] ? c4[i0] : c4[i1];
          const int64_t lo = c4[i0] > c4[i1] ? c4[i1] : c4[i0];
          c4[i0] = hi; c4[i1] = lo;
        };
        cx(0, 1); cx(2, 3); cx(0, 2); cx(1, 3); cx(1, 2);
        FLINT_TRACE(l, 16);
        // k rounds: the wave maximum of the lanes' first keys (upper halves)
        // and, by a ballot, the lowest lane holding it; lanes cover the
        // experts in increasing order and each lane's first key is its lowest
        // index among equal logits, so that lane holds the lowest index.  The
        // winning lane publishes its expert (all but the last pick) and drops
        // its first key.  Lane r keeps the r-th key.
        int my_key = INT_MIN;
        int popped = 0;  // expert of the key this lane dropped last
        int lwin = 0;    // winning lane of the last round
        for (int r = 0; r < k; ++r) {
          const int head = (int)(c4[0] >> 32);
          const int m = wave_max_i32_s(head);
          lwin = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(head == m));
          my_key = lane == r ? m : my_key;
          const bool win = lane == lwin;
          const int e = kMaxExperts - 1 - (int)(uint32_t)c4[0];
          if (win && r + 1 < k)
            __hip_atomic_store(&S.pk[r], (int)((tag << 8) | (uint32_t)e), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
          popped = win ? e : popped;
          c4[0] = win ? c4[1] : c4[0];
          c4[1] = win ? c4[2] : c4[1];
          c4[2] = win ? c4[3] : c4[2];
          c4[3] = win ? (int64_t)((uint64_t)(uint32_t)INT_MIN << 32) : c4[3];
          if (r == 0) FLINT_TRACE(l, 17);
        }
        FLINT_TRACE(l, 18);
        // this wave's own pairs (of the last pick), then the last pick is
        // published: the other waves' down-projection requests follow them
        const int elast = __builtin_amdgcn_readlane(popped, lwin);
#pragma unroll
        for (int pp = 0; pp < kNq; ++pp) o[pp] = load_pair(prs, pq[pp], elast);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0)
          __hip_atomic_store(&S.pk[k - 1], (int)((tag << 8) | (uint32_t)elast), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
        // the down tensor scale of the expert of pick r (lane r), requested
        // before the down operands so that it arrives with this wave's pairs
        const float dts = bload_f32(make_rsrc(prs.ts, (uint64_t)E * 3 * 4),
                                    (uint32_t)(3 * (lane < k ? S.pk[lane] & 0xFF : 0) + 2) * 4);
        FLINT_TRACE(l, 3);
        load_down();
        // softmax over the k chosen logits (lane r holds the r-th; the first
        // is the largest), times the down tensor scale of its expert; the
        // weights are read in phase C
        const float my_v = ord_key_value(my_key);
        const float first = lane_f32(my_v, 0);
        const float ex = lane < k ? __expf(my_v - first) : 0.0f;
        const float z = lane_f32(row16_sum(ex), 0);
        if (lane < k) S.w[lane] = ex / z * dts;
        FLINT_TRACE(l, 15);
      } else {
        if constexpr (!kComm) FLINT_TRACE_LOAD(l, 11);
#pragma unroll
        for (int pp = 0; pp < kNq; ++pp) {
          const int e = wait_pick(pq[pp] < nroutedx ? pq[pp] / Ix : 0);
          FLINT_TRACE_AT(64, l, 23 + 2 * pp);
          FLINT_TRACE_LOAD(l, 19);
          o[pp] = load_pair(prs, pq[pp], e);
          FLINT_TRACE_AT(64, l, 24 + 2 * pp);
          FLINT_TRACE_LOAD(l, 20);
        }
        wait_pick(k - 1);
        FLINT_TRACE_LOAD(l, 21);
        if constexpr (!kComm) {
          if (P.routes && blockIdx.x == 0 && t - kCommThreads < k)
            P.routes[((size_t)tok * L + l) * k + (t - kCommThreads)] = S.pk[t - kCommThreads] & 0xFF;
        }
        load_down();
        FLINT_TRACE_LOAD(l, 22);
        if constexpr (!kComm) {
          // the next layer's router and shared rows (the next token's first
          // layer after the last one) do not depend on this token: request
          // them behind this layer's down-projection operands, so that they
          // stream in with the routed weights rather than during the
          // exchanges at the end of the layer (whose polls they would slow)
          have_a = l + 1 < L || tok + 1 < P.T;
          load_phase_a(l + 1 < L ? l + 1 : 0, have_a);
          FLINT_TRACE_LOAD(l, 13);
        }
      }
      stress_delay<kStress>(P, tok, l, 2);
#pragma unroll
      for (int pp = 0; pp < kNq; ++pp) {
        if (pq[pp] < nroutedx) {
          const float hval = pair_value(o[pp], xv);
          if (lane == 0) put_pair<Scope::kXcd>(&s3[pq[pp]], hval, ep0 + 1);
        }
      }
      FLINT_TRACE_AT(64, l, 27);
      if constexpr (kComm) {
        FLINT_TRACE(l, 4);
        poll_pairs<Scope::kXcd>(s3, kSliceK, ep0 + 1, S.hs, wc, true);
      } else {
        FLINT_TRACE_LOAD(l, 12);
      }
      wg_barrier();  // B3: hidden slice in LDS
      if (S.bad) return false;
      FLINT_TRACE(l, 5);

      // ---------------------------------------------------------- phase C
      stress_delay<kStress>(P, tok, l, 3);
      {
        float hv[32];
        lds_x32(S.hs + kRowPad * j, hv);
        const float coef = routed ? S.w[dslot] : sts;
#pragma unroll
        for (int pc = 0; pc < kDownPasses; ++pc) {
          const float acc = row16_sum(coef * nvfp4_lane_dot32(cd[pc], sd[pc], hv));
          const int n = 64 * li + 8 * wv + 4 * pc + (lane >> 4);
          if (j == 0) put_pair<Scope::kDevice>(&s4a[(size_t)g * kHidden + n], acc, ep0 + 2);
        }
      }
      FLINT_TRACE(l, 28);
      FLINT_TRACE_LOAD(l, 29);
      if constexpr (!kComm) {
        // the next layer's router row (requested in phase B) to LDS, where
        // the polling waves apply it to the residual as it arrives
        if (l + 1 < L) {
#pragma unroll
          for (int i = 0; i < kRouterCols / 256; ++i)
            *reinterpret_cast<float4*>(S.wr + kRouterCols * lw + 256 * i + 4 * lane) = wr[i];
        }
      }
      if constexpr (kComm) {
        // rows 64 li .. 64 li + 63: thread t takes group t % 8's partial
        // outputs of rows 64 li + 2 (t / 8) and the next one; the 8 groups'
        // values are summed over 8 neighbouring lanes (fixed butterfly
        // order), added to the residual and published by the group-0 lane
        __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(s4a, 0, kGroups * kHidden * 8, 0x00020000);
        const int gg = t & 7, rp = t >> 3;  // kCommThreads == kGroups * 32 pairs of rows
        const int off = (gg * kHidden + 64 * li + 2 * rp) * 8;
        float y0 = 0.0f, y1 = 0.0f;
        uint32_t spins = 0;
        while (true) {
          auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 16);
          if (v[1] == ep0 + 2 && v[3] == ep0 + 2) {
            y0 = __uint_as_float(v[0]);
            y1 = __uint_as_float(v[2]);
            break;
          }
          if (poll_gave_up(spins, wc)) break;
        }
        y0 += dpp_f32<kDppXor1>(y0);
        y1 += dpp_f32<kDppXor1>(y1);
        y0 += dpp_f32<kDppXor2>(y0);
        y1 += dpp_f32<kDppXor2>(y1);
        y0 += dpp_f32<kDppHalfMirror>(y0);
        y1 += dpp_f32<kDppHalfMirror>(y1);
        stress_delay<kStress>(P, tok, l, 4);
        if (gg == 0) {
          const int n = 64 * li + 2 * rp;
          put_pair<Scope::kXcd>(&s4b[n], S.h[n] + y0, ep0 + 3);
          put_pair<Scope::kXcd>(&s4b[n + 1], S.h[n + 1] + y1, ep0 + 3);
        }
        FLINT_TRACE(l, 14);
      }
      wg_barrier();  // B4: the next layer's router row in LDS (phase D reads it)
      if (S.bad) return false;
      FLINT_TRACE(l, 6);

      // ---------------------------------------------------------- phase D
      // the communication waves collect the group's new residual (the rows
      // this workgroup owns arrive only after they were read above)
      if constexpr (kComm) {
        if (l + 1 < L) {
          float dacc, sacc;
          poll_pairs<Scope::kXcd, true>(s4b, kHidden, ep0 + 3, S.h, wc, false, S.wr, &dacc, &sacc);
          dacc = wave_sum(dacc);
          sacc = wave_sum(sacc);
          if (lane == 0) {
            S.rp[wv] = dacc;
            S.rq[wv] = sacc;
          }
        } else {
          poll_pairs<Scope::kXcd>(s4b, kHidden, ep0 + 3, S.h, wc);
        }
      }
      wg_barrier();  // B5: new residual in LDS
      if (S.bad) return false;
      FLINT_TRACE(l, 7);
    }

    if constexpr (!kHead) {
      // no head (a single token, one or more layers of a longer model): the
      // first XCD's workgroups store their rows of the new residual
      if constexpr (kComm) {
        if (wv == 0 && g == 0) P.h_out[64 * li + lane] = S.h[64 * li + lane];
      }
      if (P.qkv.out) {
        // the following layer's q, k, v rows of the new residual's norm (the
        // norm every workgroup has in LDS): one row per wave and step, all
        // of a wave's rows requested before any is reduced
        rms_to_u(S.h, S.u, S.red, P.eps);  // Q1, Q2
        float xv[32];
        lds_x32(S.u + kRowPad * lane, xv);
        const int n0 = P.qkv.rows[0], n01 = n0 + P.qkv.rows[1], R = n01 + P.qkv.rows[2];
        const int gw = blockIdx.x * kStackWaves + wv, nw = kStackWGs * kStackWaves;
        constexpr int kQ = 3;
        for (int r0 = gw; r0 < R; r0 += kQ * nw) {
          uint4 c[kQ];
          uint32_t sc[kQ];
#pragma unroll
          for (int q = 0; q < kQ; ++q) {
            const int r = r0 + q * nw;  // wave-uniform
            c[q] = make_uint4(0, 0, 0, 0);
            sc[q] = 0;
            if (r < R) {
              const int m = r < n0 ? 0 : r < n01 ? 1 : 2;
              const size_t lr = (size_t)(r - (m == 0 ? 0 : m == 1 ? n0 : n01));
              c[q] = ld_nt_u4(P.qkv.codes[m] + lr * (kHidden / 2) + 16 * lane);
              sc[q] = ld_nt_u16(P.qkv.scales[m] + lr * (kHidden / 16) + 2 * lane);
            }
          }
#pragma unroll
          for (int q = 0; q < kQ; ++q) {
            const int r = r0 + q * nw;
            if (r < R) {
              const int m = r < n0 ? 0 : r < n01 ? 1 : 2;
              const float v = wave_sum(nvfp4_lane_dot32(c[q], sc[q], xv)) * *P.qkv.tscale[m];
              if (lane == 0) P.qkv.out[r] = v;
            }
          }
        }
      }
      continue;
    }

    // -------------------------------------------------------------- head
    FLINT_TRACE(L, 0);
    rms_to_u(S.h, S.u, S.red, P.eps);  // H1, H2
    const uint32_t eph = C.base + 1u + (uint32_t)((tok * (L + 1) + L) * 4);
    {
      float xv[32];
      lds_x32(S.u + kRowPad * lane, xv);
      const int hw = kMaxStackLayers * kLayerWords;
      const float Sh = bload_f32(make_rsrc(tab_ptr<const float>(S, hw + 2), 4), 0);
      const rsrc_t rhc = make_rsrc(tab_ptr<const uint8_t>(S, hw + 0), (uint64_t)V * kHidden / 2);
      const rsrc_t rhs = make_rsrc(tab_ptr<const uint8_t>(S, hw + 1), (uint64_t)V * kHidden / 16);
      float* lg = P.logits ? P.logits + (size_t)tok * V : nullptr;
      const int gw = blockIdx.x * kStackWaves + wv, nw = kStackWGs * kStackWaves;
      float best = -FLT_MAX;
      int besti = INT_MAX;
      for (int r0 = gw * kHeadRowsPerWave; r0 < V; r0 += nw * kHeadRowsPerWave) {
        uint4 c[kHeadRowsPerWave];
        uint32_t s[kHeadRowsPerWave];
#pragma unroll
        for (int q = 0; q < kHeadRowsPerWave; ++q) {
          const int row = min(r0 + q, V - 1);
          c[q] = bload_u4_nt(rhc, (uint32_t)row * (kHidden / 2) + 16 * lane);
          s[q] = bload_u16_nt(rhs, (uint32_t)row * (kHidden / 16) + 2 * lane);
        }
#pragma unroll
        for (int q = 0; q < kHeadRowsPerWave; ++q) {
          const float v = wave_sum(nvfp4_lane_dot32(c[q], s[q], xv)) * Sh;
          const int row = r0 + q;
          if (row < V) {
            if (lane == 0 && lg) lg[row] = v;
            if (v > best) { best = v; besti = row; }
          }
        }
      }
      if (lane == 0) { S.bv[wv] = best; S.bi[wv] = besti; }
      wg_barrier();  // H3
      FLINT_TRACE(L, 1);
      stress_delay<kStress>(P, tok, L, 5);
      if (!kComm && t == kCommThreads) {
        float bv = S.bv[0];
        int bi = S.bi[0];
        for (int w = 1; w < kStackWaves; ++w)
          if (S.bv[w] > bv || (S.bv[w] == bv && S.bi[w] < bi)) { bv = S.bv[w]; bi = S.bi[w]; }
        uint64_t* hp = P.hp + ((size_t)(tok & 1) * kStackWGs + blockIdx.x) * 2;
        put_pair<Scope::kDevice>(hp, bv, eph);
        put_pair<Scope::kDevice>(hp + 1, __int_as_float(bi), eph);
      }
    }
    // every workgroup waits for all head partials: the token boundary
    if constexpr (kComm) poll_pairs<Scope::kDevice>(P.hp + (size_t)(tok & 1) * kStackWGs * 2, 2 * kStackWGs, eph, S.hp, wc);
    wg_barrier();  // H4
    if (S.bad) return false;
    FLINT_TRACE(L, 2);
    if (kComm && wv == 0) {
      float bv = -FLT_MAX;
      int bi = INT_MAX;
      for (int i = lane; i < kStackWGs; i += 64) {
        const float v = S.hp[2 * i];
        const int id = __float_as_int(S.hp[2 * i + 1]);
        if (v > bv || (v == bv && id < bi)) { bv = v; bi = id; }
      }
      wave_argmax(bv, bi);
      if (lane == 0 && blockIdx.x == 0) P.argmax[tok] = bi;
    }
    wg_barrier();  // H5: S.hp and S.h are rewritten by the next token
  }
  return true;
#undef FLINT_TRACE
#undef FLINT_TRACE_LOAD
#undef FLINT_TRACE_AT
}

// kHead false: one token, no head, the final residual to P.h_out.  kStress:
// injected delays, roles permuted inside each XCD, the caller's wait limit
// (a test of the exchange protocol; the results equal the plain kernel's).

// The logit area's phase (which of its 8 KB classes is near XCDs 0-3), kept in
// ctrl[2] of the workspace as 1 + phase.  The first call on a workspace
// measures it: workgroup 0 (XCD 0) times device-scope stores to four blocks
// of each class, each until its home has acknowledged it (best of 8; near
// blocks take about 160-200 ns, far ones 240-320 ns), and publishes the
// result; every workgroup waits for it (bounded).  The phase decides
// placement only, never results.  `cal` is ctrl[2] as this workgroup read it
// (uniform across the workgroup).
__device__ bool exchange_phase(const StackParams& P, StackLds& S, StackCoord& C, uint32_t cal) {
  if (cal == 0) {
    if (blockIdx.x == 0 && C.t == 0) {
      uint32_t near0 = 0, near1 = 0;       // summed times of class 0 and class 1 blocks (10 ns ticks)
#pragma unroll 1
      for (int blk = 0; blk < 8; ++blk) {  // class (blk >> 1) & 1
        uint64_t* p = reinterpret_cast<uint64_t*>(P.s2 + (uint32_t)blk * kXchBlock + kPhaseProbe);
        uint32_t best = UINT_MAX;
#pragma unroll 1
        for (int r = 0; r < 8; ++r) {
          const uint32_t t0 = (uint32_t)wall_clock64();
          __hip_atomic_store(p, (uint64_t)r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the store is acknowledged by its home
          const uint32_t dt = (uint32_t)wall_clock64() - t0;
          best = dt < best ? dt : best;
        }
        if ((blk >> 1) & 1)
          near1 += best;
        else
          near0 += best;
      }
      st_dev_u32(P.ctrl + 2, near0 <= near1 ? 1u : 2u);  // XCD 0 is in half 0: its near class is the phase
    }
    if (C.t == 0) {
      uint32_t spins = 0, v;
      while ((v = ld_dev_u32(P.ctrl + 2)) == 0) {
        if (++spins > kSpinLimit || ((spins & 1023) == 0 && ld_dev_u32(P.ctrl + 1))) {
          atomicOr(P.ctrl + 1, 1u);
          S.bad = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      S.ctl[2] = v;
    }
    wg_barrier();
    if (S.bad) return false;
    cal = S.ctl[2];
  }
  C.phase = (int)((cal - 1u) & 1u);
  return true;
}

template <bool kHead, bool kStress = false>
__global__ __launch_bounds__(kStackThreads, 1) void k_stack_decode(StackParams P,
                                                                  const StackTable* __restrict__ table) {
  __shared__ StackLds S;
  StackCoord C;
  C.t = threadIdx.x;
  C.lane = C.t & 63;
  // the wave index is uniform across a wave: say so, so that the role branch
  // and everything derived from it stay scalar
  C.wv = __builtin_amdgcn_readfirstlane(C.t >> 6);
  C.g = blockIdx.x % kGroups;
  C.li = kStress ? kGroupWGs - 1 - (int)blockIdx.x / kGroups : (int)blockIdx.x / kGroups;
  C.L = P.L; C.E = P.E; C.I = P.I; C.k = P.k; C.Is = P.Is; C.V = P.V;
  C.Ix = C.I / kGroups;
  C.Isx = C.Is / kGroups;
  C.nroutedx = C.k * C.Ix;
  C.tracing = P.trace != nullptr;
  if (C.tracing && C.t == 0) S.tr[C.L * kTracePoints + 3] = wall_clock64();  // kernel entry
  // layer table (and head) to LDS
  {
    const uint64_t* src = reinterpret_cast<const uint64_t*>(table->layers + P.l0);
    for (int i = C.t; i < C.L * kLayerWords; i += kStackThreads) S.tab[i] = src[i];
    const uint64_t* hsrc = reinterpret_cast<const uint64_t*>(&table->head);
    if (C.t < 3) S.tab[kMaxStackLayers * kLayerWords + C.t] = hsrc[C.t];
  }
  if (C.t < kMaxTopK) S.pk[C.t] = 0;  // tag 0: no layer
  if (C.t == 0) {
    S.bad = 0;
    // control words [0] epoch base, [1] error flag, [2] logit-area phase, in
    // one device-scope load
    const auto cw = __builtin_amdgcn_raw_buffer_load_b128(__builtin_amdgcn_make_buffer_rsrc(P.ctrl, 0, 16, 0x00020000),
                                                          0, 0, poll_aux<Scope::kDevice>());
    S.ctl[0] = cw[0]; S.ctl[1] = cw[1]; S.ctl[2] = cw[2];
  }
  wg_barrier();
  if (S.ctl[1]) return;              // an earlier call gave up: do nothing
  if (xcc_id() != (uint32_t)C.g) {   // the in-XCD exchanges need b -> XCD b % 8
    if (C.t == 0) atomicOr(P.ctrl + 1, 2u);
    return;
  }
  C.base = S.ctl[0];
  if (!exchange_phase(P, S, C, S.ctl[2])) return;
  if (C.tracing && C.t == 0) S.tr[C.L * kTracePoints + 4] = wall_clock64();  // set-up done
  const bool ok =
      C.wv < kCommWaves ? stack_role<true, kHead, kStress>(P, S, C) : stack_role<false, kHead, kStress>(P, S, C);
  if (!ok) return;
  if (C.tracing) {
    const int L = C.L, t = C.t;
    if (blockIdx.x == 0 || blockIdx.x == kStackWGs - 1) {
      int64_t* dst = P.trace + (blockIdx.x == 0 ? 0 : (size_t)(L + 1) * kTracePoints);
      for (int i = t; i < (L + 1) * kTracePoints; i += kStackThreads) dst[i] = S.tr[i];
    }
    if (t < kTracePoints)
      P.trace[2 * (size_t)(L + 1) * kTracePoints + (size_t)blockIdx.x * kTracePoints + t] = S.tr[kTracePoints + t];
  }
  if (blockIdx.x == 0 && C.t == 0) st_dev_u32(P.ctrl, C.base + (uint32_t)(P.T * (P.L + 1) * 4) + 4u);
}

bool stack_persistent_supported(const flint_moe_dims& d, int L) {
  return L >= 1 && L <= kMaxStackLayers && d.hidden == kHidden && d.n_experts % 2 == 0 && d.expert_width % 256 == 0 && d.shared_width % 256 == 0 &&
         d.n_experts % 8 == 0 && d.shared_width / kGroups <= 4 * kGroupWGs && d.n_experts <= kStackWaves * kGroupWGs &&
         d.top_k * (d.expert_width / kGroups) + d.shared_width / kGroups == kSliceK &&
         d.top_k * (d.expert_width / kGroups) <= (kGateUpComm * kCommWaves + kStackWaves - kCommWaves) * kGroupWGs &&
         d.shared_width / kGroups <= (kStackWaves - kCommWaves) * kGroupWGs &&
         d.n_experts <= 2 * (kStackWaves - kCommWaves) * kGroupWGs;
}

size_t stack_persistent_ws_bytes() {
  size_t o = 256;                                                  // ctrl
  o += sizeof(uint64_t) * 2 * kGroups * kSliceK;                   // s3
  o += sizeof(uint64_t) * 2 * kGroups * kHidden * 2;               // s4a, s4b
  o += sizeof(uint64_t) * 2 * kStackWGs * 2;                       // hp
  o += 32768 + 2 * (size_t)kS2Area;                                // s2: alignment, one 2 MB page
  return align_up(o, 256);
}

hipError_t launch_stack_persistent(const flint_moe_dims& d, int L, int vocab, const void* table, const float* x,
                                   int T, float eps, float* logits, int32_t* argmax, int32_t* routes, void* ws,
                                   int64_t* trace, hipStream_t s, int l0, float* h_out, const StackQkv* qkv,
                                   uint32_t stress_seed, uint32_t spin_limit) {
  StackParams P;
  P.stress_seed = stress_seed;
  P.spin_limit = spin_limit;
  const bool stress = spin_limit != 0 && vocab > 0;
  P.trace = trace;
  P.qkv = qkv ? *qkv : StackQkv{};
  P.table = static_cast<const StackTable*>(table);
  P.l0 = l0;
  P.h_out = h_out;
  P.L = L; P.E = d.n_experts; P.I = d.expert_width; P.k = d.top_k; P.Is = d.shared_width; P.V = vocab; P.T = T;
  P.eps = eps; P.x = x; P.logits = logits; P.argmax = argmax; P.routes = routes;
  char* w = static_cast<char*>(ws);
  P.ctrl = reinterpret_cast<uint32_t*>(w);
  w += 256;
  P.s3 = reinterpret_cast<uint64_t*>(w); w += sizeof(uint64_t) * 2 * kGroups * kSliceK;
  P.s4a = reinterpret_cast<uint64_t*>(w); w += sizeof(uint64_t) * 2 * kGroups * kHidden;
  P.s4b = reinterpret_cast<uint64_t*>(w); w += sizeof(uint64_t) * 2 * kGroups * kHidden;
  P.hp = reinterpret_cast<uint64_t*>(w); w += sizeof(uint64_t) * 2 * kStackWGs * 2;
  {
    // the logit area: 32 KB aligned, moved to the next 2 MB boundary if it
    // would cross one
    uintptr_t r = (reinterpret_cast<uintptr_t>(w) + 32767) & ~(uintptr_t)32767;
    if ((r >> 21) != ((r + kS2Area - 1) >> 21)) r = (r + ((uintptr_t)1 << 21) - 1) & ~(((uintptr_t)1 << 21) - 1);
    P.s2 = reinterpret_cast<uint8_t*>(r);
  }
  const StackTable* tab = P.table;
  // A plain launch: 256 workgroups of 512 threads, one per compute unit,
  // all resident at once when the device is otherwise idle (checked once per
  // device from the occupancy calculator).  If another queue holds compute
  // units so that some workgroups cannot start, the running ones give up at
  // their wait limit and raise the error flag, the late ones see it and
  // return: a reported error, not a hang.
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::atomic<int> resident[64];
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int r = resident[dev].load();
  if (r == 0) {
    int per_cu = 0, cus = 0;
    int per_cu2 = 0;
    int per_cu3 = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_stack_decode<true>, kStackThreads, 0);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu2, k_stack_decode<false>, kStackThreads, 0);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu3, k_stack_decode<true, true>, kStackThreads, 0);
    per_cu = per_cu < per_cu2 ? per_cu : per_cu2;
    per_cu = per_cu < per_cu3 ? per_cu : per_cu3;
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    r = per_cu * cus >= kStackWGs ? 1 : -1;
    resident[dev].store(r);
  }
  if (r != 1) return hipErrorCooperativeLaunchTooLarge;
  if (stress)
    k_stack_decode<true, true><<<dim3(kStackWGs), dim3(kStackThreads), 0, s>>>(P, tab);
  else if (vocab > 0)
    k_stack_decode<true><<<dim3(kStackWGs), dim3(kStackThreads), 0, s>>>(P, tab);
  else
    k_stack_decode<false><<<dim3(kStackWGs), dim3(kStackThreads), 0, s>>>(P, tab);
  return hipGetLastError();
}

hipError_t read_stack_error(const void* ws, int32_t* out) {
  uint32_t v = 0;
  hipError_t e = hipMemcpy(&v, static_cast<const char*>(ws) + 4, 4, hipMemcpyDeviceToHost);
  *out = (int32_t)v;
  return e;
}

}  // namespace flint
