// stack.hip -- persistent batch-1 decode of the whole MoE layer stack plus the
// NVFP4 head, one cooperative launch per call.
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
// Geometry.  256 workgroups of 512 threads, one per compute unit, launched
// cooperatively so all are resident.  Workgroups are dealt to the 8 XCDs
// round-robin, so workgroup b sits on XCD b % 8: group g = b % 8 is the 32
// workgroups of one XCD, and li = b / 8 is the index inside the group.
//
// Work split of one layer (E experts, top-k, width I, shared width Is):
//  A  every group computes all E router logits (8 rows per workgroup, the fp32
//     router is read once per XCD) and the SwiGLU of its 1/8 slice of the
//     shared expert's rows;
//  B  each workgroup takes the top k of the E logits of its group, then the
//     group computes the SwiGLU of its 1/8 slice (I/8 rows) of each chosen
//     expert; the down-projection weights of phase C are loaded here too;
//  C  the group multiplies its slice of the hidden activations by the
//     matching 1/8 column slice of every down matrix (routed, weighted by the
//     routing weights, and shared): a partial output for all H rows;
//  D  the 8 partial outputs are summed (fixed order) and added to the
//     residual.
// Exchanges.  A -> B logits (inside a group), B -> C hidden slice (inside a
// group), C -> D partial outputs (across groups) and D -> A the new residual
// (inside a group).  Values travel as 64-bit (value, epoch) pairs written
// with device-scope stores; a consumer reads them with device-scope 128-bit
// loads until every epoch matches, so no separate flag or barrier is needed.
// Epochs are unique per (call, token, layer, exchange).  Every wait is
// bounded: on time-out a workgroup raises the error flag and all workgroups
// leave the kernel.
#include <float.h>
#include <limits.h>

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
constexpr int kGateUpPerWave = 3;                  // routed gate/up pairs per communication wave
constexpr int kDownPasses = 4;                     // 4-row passes of a load wave in phase C
constexpr uint32_t kSpinLimit = 1u << 22;
#ifndef FLINT_POLL_SLEEP
#define FLINT_POLL_SLEEP 2
#endif
// back-off between polls of data that has not arrived (units of 64 clocks):
// keeps waiting workgroups from flooding the coherence point
__device__ __forceinline__ void poll_backoff() {
  if (FLINT_POLL_SLEEP > 0) __builtin_amdgcn_s_sleep(FLINT_POLL_SLEEP);
}
// Activation vectors in LDS are stored in rows of 32 values padded to 36, so
// that the 64 lanes of a wave, each reading its own 32 consecutive values with
// 128-bit loads, hit distinct banks.
constexpr int kRowPad = 36;
__device__ __forceinline__ int padded(int e) { return (e >> 5) * kRowPad + (e & 31); }

struct StackParams {
  const StackTable* table;
  int L, E, I, k, Is, V, T;
  float eps;
  const float* x;
  float* logits;
  int32_t* argmax;
  int32_t* routes;
  uint32_t* ctrl;  // [0] epoch base, [1] error flag
  uint64_t* s2;    // [2][8][256]  router logits
  uint64_t* s3;    // [2][8][512]  hidden slice
  uint64_t* s4a;   // [2][8][2048] partial outputs
  uint64_t* s4b;   // [2][8][2048] residual
  uint64_t* hp;    // [2][256][2]  head (max, index)
  int64_t* trace;  // optional [2][L+1][kTracePoints] phase timestamps of workgroups 0 and 255
};

constexpr int kTracePoints = 10;

__device__ __forceinline__ void put_pair(uint64_t* p, float v, uint32_t ep) {
  __hip_atomic_store(p, (uint64_t)__float_as_uint(v) | ((uint64_t)ep << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

struct WaitCtx {
  uint32_t* err;
  int* bad;  // LDS flag
};

// Wait until pairs [0, n) (n even) of buf carry epoch ep; values -> dst.
// Pair i goes to dst[i]; for a strided source use wait_pairs_rows.
__device__ __forceinline__ void wait_pairs(const uint64_t* buf, int n, uint32_t ep, float* dst, const WaitCtx& w,
                                           bool pad = false) {
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t*>(buf), 0, n * 8, 0x00020000);
  for (int c = threadIdx.x; threadIdx.x < kCommThreads && c < n / 2; c += kCommThreads) {
    uint32_t spins = 0;
    while (true) {
      auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, c * 16, 0, 16);
      if (v[1] == ep && v[3] == ep) {
        const int d = pad ? padded(2 * c) : 2 * c;  // 2c, 2c+1 share a row
        dst[d] = __uint_as_float(v[0]);
        dst[d + 1] = __uint_as_float(v[2]);
        break;
      }
      ++spins;
      if (spins > kSpinLimit || ((spins & 1023) == 0 && ld_dev_u32(w.err))) {
        atomicOr(w.err, 1u);
        *w.bad = 1;
        break;
      }
      poll_backoff();
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void lds_x32(const float* src, float* xv) {
  const float4* p = reinterpret_cast<const float4*>(src);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float4 v = p[i];
    xv[4 * i] = v.x; xv[4 * i + 1] = v.y; xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
  }
}

// RMSNorm scale of sh_h (kHidden values) -> sh_u = s * sh_h
__device__ __forceinline__ void rms_to_u(const float* sh_h, float* sh_u, float* sh_red, float eps) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  float v[kHidden / kStackThreads];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kHidden / kStackThreads; ++i) {
    v[i] = sh_h[t + i * kStackThreads];
    ss = __builtin_fmaf(v[i], v[i], ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) sh_red[w] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kStackWaves; ++i) tot += sh_red[i];
  const float s = 1.0f / sqrtf(tot * (1.0f / kHidden) + eps);
#pragma unroll
  for (int i = 0; i < kHidden / kStackThreads; ++i) sh_u[padded(t + i * kStackThreads)] = v[i] * s;
  __syncthreads();
}

__device__ __forceinline__ void load_f32x32(rsrc_t r, uint32_t off, float* v) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 a = bload_f4(r, off + 16 * i);
    v[4 * i] = a.x; v[4 * i + 1] = a.y; v[4 * i + 2] = a.z; v[4 * i + 3] = a.w;
  }
}

__device__ __forceinline__ float dot32(const float* a, const float* b) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) acc = __builtin_fmaf(a[i], b[i], acc);
  return acc;
}

__global__ __launch_bounds__(kStackThreads, 1) void k_stack_decode(StackParams P,
                                                                  const StackTable* __restrict__ table) {
  __shared__ __align__(16) float sh_h[kHidden];
  __shared__ __align__(16) float sh_u[kHidden / 32 * kRowPad];
  __shared__ __align__(16) float sh_logit[kMaxExperts];
  __shared__ __align__(16) float sh_hs[kSliceK / 32 * kRowPad];
  __shared__ __align__(16) float sh_part[kGroups * 64];
  __shared__ __align__(16) float sh_hp[2 * kStackWGs];
  __shared__ float sh_red[kStackWaves];
  __shared__ int32_t sh_idx[kMaxTopK];
  __shared__ float sh_w[kMaxTopK];
  __shared__ float sh_bv[kStackWaves];
  __shared__ int sh_bi[kStackWaves];
  __shared__ int sh_bad;

  // the wave index is uniform across a wave: say so, so that everything
  // derived from it (row choices, buffer resources) stays in scalar registers
  const int t = threadIdx.x, lane = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = blockIdx.x % kGroups, li = blockIdx.x / kGroups;
  const int L = P.L, E = P.E, I = P.I, k = P.k, Is = P.Is, V = P.V;
  const int Ix = I / kGroups, Isx = Is / kGroups;  // this group's slice widths
  const int nroutedx = k * Ix;                     // routed rows of the slice (384)
  // Wave roles.  A wave's loads complete in issue order, so a wave polling
  // for an exchange must not have weight loads in flight: waves 0-3 poll
  // every exchange and compute the routed gate/up rows (whose loads they
  // consume before polling); waves 4-7 compute the router, shared and down
  // rows and hold the loads issued ahead of time.
  const bool comm = wv < kCommWaves;
  const int lw = wv - kCommWaves;
  if (t == 0) sh_bad = 0;
  __syncthreads();
  WaitCtx wc{P.ctrl + 1, &sh_bad};
  if (ld_dev_u32(P.ctrl + 1)) return;  // an earlier call gave up: do nothing
  const uint32_t base = ld_dev_u32(P.ctrl);
  // phase timestamps (first token only) of one workgroup on XCD 0 and one on XCD 7
  // (workgroup-uniform pointers, written by thread 0 only)
  int64_t* trace = nullptr;
  if (P.trace && (blockIdx.x == 0 || blockIdx.x == kStackWGs - 1))
    trace = P.trace + (blockIdx.x == 0 ? 0 : (size_t)(L + 1) * kTracePoints);
  int64_t* trace_all = P.trace ? P.trace + 2 * (size_t)(L + 1) * kTracePoints +
                                     (size_t)blockIdx.x * kTracePoints : nullptr;
#define FLINT_TRACE(l_, i_)                                                                         \
  do {                                                                                               \
    if (trace && t == 0 && tok == 0) trace[(size_t)(l_) * kTracePoints + (i_)] = wall_clock64();     \
    if (trace_all && t == 0 && tok == 0 && (l_) == 1) trace_all[(i_)] = wall_clock64();              \
  } while (0)

  // phase-A operands of a load wave: router rows ra0, ra1 and shared pair qa
  const int ra0 = li + kGroupWGs * (2 * lw), ra1 = li + kGroupWGs * (2 * lw + 1);
  const int qa = li + kGroupWGs * lw;
  float wr0[32], wr1[32];
  uint4 cgs, cus;
  uint32_t sgs = 0, sus = 0;
  bool prefetched = false;
  // unconditional loads (a wave with no row reads row 0 and ignores it), so
  // that no branch join forces an early wait on the data
  auto load_phase_a = [&](const flint_moe_layer& Lx) {
    const rsrc_t rr = make_rsrc(Lx.router, (uint64_t)E * kHidden * 4);
    const uint32_t r0 = ra0 < E ? (uint32_t)ra0 : 0u, r1 = ra1 < E ? (uint32_t)ra1 : 0u;
    load_f32x32(rr, (r0 * kHidden + 32 * lane) * 4, wr0);
    load_f32x32(rr, (r1 * kHidden + 32 * lane) * 4, wr1);
    const uint32_t row = (uint32_t)(g * Isx + (qa < Isx ? qa : 0));
    cgs = bload_u4(make_rsrc(Lx.shared_gate.codes, (uint64_t)Is * kHidden / 2), row * (kHidden / 2) + 16 * lane);
    sgs = bload_u16(make_rsrc(Lx.shared_gate.scales, (uint64_t)Is * kHidden / 16), row * (kHidden / 16) + 2 * lane);
    cus = bload_u4(make_rsrc(Lx.shared_up.codes, (uint64_t)Is * kHidden / 2), row * (kHidden / 2) + 16 * lane);
    sus = bload_u16(make_rsrc(Lx.shared_up.scales, (uint64_t)Is * kHidden / 16), row * (kHidden / 16) + 2 * lane);
  };

  const rsrc_t rx = make_rsrc(P.x, (uint64_t)P.T * kHidden * 4);
  for (int tok = 0; tok < P.T; ++tok) {
    // residual stream <- x_t
#pragma unroll
    for (int i = 0; i < kHidden / kStackThreads; ++i)
      sh_h[t + i * kStackThreads] = bload_f32(rx, (uint32_t)(tok * kHidden + t + i * kStackThreads) * 4);
    __syncthreads();

    for (int l = 0; l < L; ++l) {
      const flint_moe_layer& Lw = table->layers[l];
      const int par = l & 1;
      const uint32_t ep0 = base + 1u + (uint32_t)((tok * (L + 1) + l) * 4);
      uint64_t* s2 = P.s2 + ((size_t)par * kGroups + g) * kMaxExperts;
      uint64_t* s3 = P.s3 + ((size_t)par * kGroups + g) * kSliceK;
      uint64_t* s4b = P.s4b + ((size_t)par * kGroups + g) * kHidden;

      // ---------------------------------------------------------- phase A
      FLINT_TRACE(l, 0);
      if (!comm && !prefetched) load_phase_a(Lw);
      prefetched = false;
      rms_to_u(sh_h, sh_u, sh_red, P.eps);
      FLINT_TRACE(l, 1);
      float xv[32];  // this lane's 32 normalised activations (phases A and B)
      lds_x32(sh_u + kRowPad * lane, xv);
      if (!comm) {
        if (ra0 < E) {
          const float acc = wave_sum(dot32(wr0, xv));
          if (lane == 0) put_pair(&s2[ra0], acc, ep0);
        }
        if (ra1 < E) {
          const float acc = wave_sum(dot32(wr1, xv));
          if (lane == 0) put_pair(&s2[ra1], acc, ep0);
        }
        if (qa < Isx) {
          const float gv = wave_sum(nvfp4_lane_dot32(cgs, sgs, xv)) *
                           bload_f32(make_rsrc(Lw.shared_gate.tscale, 4), 0);
          const float av = wave_sum(nvfp4_lane_dot32(cus, sus, xv)) *
                           bload_f32(make_rsrc(Lw.shared_up.tscale, 4), 0);
          if (lane == 0) put_pair(&s3[nroutedx + qa], silu(gv) * av, ep0 + 1);
        }
      }
      FLINT_TRACE(l, 2);

      // ---------------------------------------------------------- phase B
      wait_pairs(s2, E, ep0, sh_logit, wc);
      if (sh_bad) return;
      FLINT_TRACE(l, 3);
      if (wv == 0) {
        // top-k in one wave: each lane holds 4 logits sorted by (value desc,
        // index asc); k rounds of a wave maximum (DPP), ties to the lowest index
        float v[4];
        int id[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          id[q] = lane + 64 * q;
          v[q] = id[q] < E ? sh_logit[id[q]] : -FLT_MAX;
          if (id[q] >= E) id[q] = INT_MAX;
        }
        auto cswap = [&](int a, int b) {
          const bool sw = v[b] > v[a] || (v[b] == v[a] && id[b] < id[a]);
          const float tv = sw ? v[b] : v[a];
          const int ti = sw ? id[b] : id[a];
          v[b] = sw ? v[a] : v[b];
          id[b] = sw ? id[a] : id[b];
          v[a] = tv;
          id[a] = ti;
        };
        cswap(0, 1); cswap(2, 3); cswap(0, 2); cswap(1, 3); cswap(1, 2);
        float first = 0.0f, z = 0.0f, my_v = 0.0f;
        int my_i = 0;
        for (int r = 0; r < k; ++r) {
          const float m = wave_max_dpp(v[0]);
          const int mi = wave_min_dpp(v[0] == m ? id[0] : INT_MAX);
          if (r == 0) first = m;
          z += __expf(m - first);
          if (lane == r) { my_v = m; my_i = mi; }
          if (id[0] == mi) {
            v[0] = v[1]; id[0] = id[1];
            v[1] = v[2]; id[1] = id[2];
            v[2] = v[3]; id[2] = id[3];
            v[3] = -FLT_MAX; id[3] = INT_MAX;
          }
        }
        if (lane < k) {
          sh_idx[lane] = my_i;
          sh_w[lane] = __expf(my_v - first) / z;
        }
      }
      __syncthreads();
      FLINT_TRACE(l, 4);
      if (P.routes && blockIdx.x == 0 && t < k) P.routes[((size_t)tok * L + l) * k + t] = sh_idx[t];

      // routed gate/up (communication waves): pairs p = li + 32 (wv + 4 pp)
      // down-projection operands (load waves): output rows n = 64 li + 16 lw
      // + 4 pc + lane/16, 16 lanes per row, lane chunk j = 32 columns of the
      // slice; chunks j < 12 are routed columns, the rest shared ones, both
      // loads are issued for every lane and the right one is picked at use
      const int j = lane & 15;
      const bool routed = 32 * j < nroutedx;
      const int dslot = routed ? (32 * j) / Ix : 0;
      uint4 cd[kDownPasses];
      uint32_t sd[kDownPasses];
      float dts = 0.0f, sts = 0.0f, dw = 0.0f;
      if (comm) {
        const rsrc_t rgc = make_rsrc(Lw.gate_codes, (uint64_t)E * I * kHidden / 2);
        const rsrc_t rgs = make_rsrc(Lw.gate_scales, (uint64_t)E * I * kHidden / 16);
        const rsrc_t ruc = make_rsrc(Lw.up_codes, (uint64_t)E * I * kHidden / 2);
        const rsrc_t rus = make_rsrc(Lw.up_scales, (uint64_t)E * I * kHidden / 16);
        const rsrc_t rts = make_rsrc(Lw.expert_tscales, (uint64_t)E * 3 * 4);
        uint4 cg[kGateUpPerWave], cu[kGateUpPerWave];
        uint32_t sg[kGateUpPerWave], su[kGateUpPerWave];
        float Sg[kGateUpPerWave], Su[kGateUpPerWave];
#pragma unroll
        for (int pp = 0; pp < kGateUpPerWave; ++pp) {
          const int p = li + kGroupWGs * (wv + kCommWaves * pp);
          const int p_ = p < nroutedx ? p : 0;
          const int slot = p_ / Ix, rl = p_ % Ix;
          const int e = sh_idx[slot];
          const uint32_t row = (uint32_t)(e * I + g * Ix + rl);
          cg[pp] = bload_u4(rgc, row * (kHidden / 2) + 16 * lane);
          cu[pp] = bload_u4(ruc, row * (kHidden / 2) + 16 * lane);
          sg[pp] = bload_u16(rgs, row * (kHidden / 16) + 2 * lane);
          su[pp] = bload_u16(rus, row * (kHidden / 16) + 2 * lane);
          Sg[pp] = bload_f32(rts, (uint32_t)(3 * e + 0) * 4);
          Su[pp] = bload_f32(rts, (uint32_t)(3 * e + 1) * 4);
        }
#pragma unroll
        for (int pp = 0; pp < kGateUpPerWave; ++pp) {
          const int p = li + kGroupWGs * (wv + kCommWaves * pp);
          if (p < nroutedx) {
            const float gv = wave_sum(nvfp4_lane_dot32(cg[pp], sg[pp], xv)) * Sg[pp];
            const float av = wave_sum(nvfp4_lane_dot32(cu[pp], su[pp], xv)) * Su[pp];
            if (lane == 0) put_pair(&s3[p], silu(gv) * av, ep0 + 1);
          }
        }
      } else {
        const rsrc_t rdc = make_rsrc(Lw.down_codes, (uint64_t)E * kHidden * I / 2);
        const rsrc_t rds = make_rsrc(Lw.down_scales, (uint64_t)E * kHidden * I / 16);
        const rsrc_t rsdc = make_rsrc(Lw.shared_down.codes, (uint64_t)kHidden * Is / 2);
        const rsrc_t rsds = make_rsrc(Lw.shared_down.scales, (uint64_t)kHidden * Is / 16);
        const int doff = routed ? (32 * j) % Ix : 0;
        const int de = sh_idx[dslot];
        const int rcol = g * Ix + doff, scol = routed ? 0 : g * Isx + (32 * j - nroutedx);
#pragma unroll
        for (int pc = 0; pc < kDownPasses; ++pc) {
          const int n = 64 * li + 16 * lw + 4 * pc + (lane >> 4);
          const uint32_t rrow = (uint32_t)(de * kHidden + n);
          // lanes of routed and of shared chunks load into the same registers
          // under their own execution masks
          if (routed) {
            cd[pc] = bload_u4(rdc, rrow * (I / 2) + rcol / 2);
            sd[pc] = bload_u16(rds, rrow * (I / 16) + rcol / 16);
          } else {
            cd[pc] = bload_u4(rsdc, (uint32_t)(n * (Is / 2) + scol / 2));
            sd[pc] = bload_u16(rsds, (uint32_t)(n * (Is / 16) + scol / 16));
          }
        }
        dts = bload_f32(make_rsrc(Lw.expert_tscales, (uint64_t)E * 3 * 4), (uint32_t)(3 * de + 2) * 4);
        sts = bload_f32(make_rsrc(Lw.shared_down.tscale, 4), 0);
        dw = sh_w[dslot];
      }
      FLINT_TRACE(l, 5);

      // ---------------------------------------------------------- phase C
      wait_pairs(s3, kSliceK, ep0 + 1, sh_hs, wc, true);
      if (sh_bad) return;
      FLINT_TRACE(l, 6);
      if (!comm) {
        float hv[32];
        lds_x32(sh_hs + kRowPad * j, hv);
        const float coef = routed ? dw * dts : sts;
#pragma unroll
        for (int pc = 0; pc < kDownPasses; ++pc) {
          const float acc = row16_sum(coef * nvfp4_lane_dot32(cd[pc], sd[pc], hv));
          const int n = 64 * li + 16 * lw + 4 * pc + (lane >> 4);
          if (j == 0) put_pair(&P.s4a[((size_t)par * kGroups + g) * kHidden + n], acc, ep0 + 2);
        }
        // the next layer's router and shared rows do not depend on this
        // token: load them now, while the partial outputs are exchanged
        if (l + 1 < L) {
          __builtin_amdgcn_sched_barrier(0);  // keep these loads after the down rows
          load_phase_a(table->layers[l + 1]);
          prefetched = true;
        }
      }
      FLINT_TRACE(l, 7);

      // ---------------------------------------------------------- phase D
      if (comm) {  // rows 64 li .. 64 li + 63 of every group's partial output
        __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            P.s4a + (size_t)par * kGroups * kHidden, 0, kGroups * kHidden * 8, 0x00020000);
        const int gg = t >> 5, cc = t & 31;  // kCommThreads == kGroups * 32 chunks
        const int off = (gg * kHidden + 64 * li + 2 * cc) * 8;
        uint32_t spins = 0;
        while (true) {
          auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 16);
          if (v[1] == ep0 + 2 && v[3] == ep0 + 2) {
            sh_part[gg * 64 + 2 * cc] = __uint_as_float(v[0]);
            sh_part[gg * 64 + 2 * cc + 1] = __uint_as_float(v[2]);
            break;
          }
          ++spins;
          if (spins > kSpinLimit || ((spins & 1023) == 0 && ld_dev_u32(wc.err))) {
            atomicOr(wc.err, 1u);
            sh_bad = 1;
            break;
          }
          poll_backoff();
        }
      }
      __syncthreads();
      if (sh_bad) return;
      FLINT_TRACE(l, 8);
      if (t < 64) {
        float y = 0.0f;
#pragma unroll
        for (int gg = 0; gg < kGroups; ++gg) y += sh_part[gg * 64 + t];
        put_pair(&s4b[64 * li + t], sh_h[64 * li + t] + y, ep0 + 3);
      }
      __syncthreads();
      wait_pairs(s4b, kHidden, ep0 + 3, sh_h, wc);
      if (sh_bad) return;
      FLINT_TRACE(l, 9);
    }

    // -------------------------------------------------------------- head
    FLINT_TRACE(L, 0);
    rms_to_u(sh_h, sh_u, sh_red, P.eps);
    const uint32_t eph = base + 1u + (uint32_t)((tok * (L + 1) + L) * 4);
    {
      float xv[32];
      lds_x32(sh_u + kRowPad * lane, xv);
      const flint_nvfp4& Hd = table->head;
      const float S = bload_f32(make_rsrc(Hd.tscale, 4), 0);
      const rsrc_t rhc = make_rsrc(Hd.codes, (uint64_t)V * kHidden / 2);
      const rsrc_t rhs = make_rsrc(Hd.scales, (uint64_t)V * kHidden / 16);
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
          c[q] = bload_u4(rhc, (uint32_t)row * (kHidden / 2) + 16 * lane);
          s[q] = bload_u16(rhs, (uint32_t)row * (kHidden / 16) + 2 * lane);
        }
#pragma unroll
        for (int q = 0; q < kHeadRowsPerWave; ++q) {
          const float v = wave_sum(nvfp4_lane_dot32(c[q], s[q], xv)) * S;
          const int row = r0 + q;
          if (row < V) {
            if (lane == 0 && lg) lg[row] = v;
            if (v > best) { best = v; besti = row; }
          }
        }
      }
      if (lane == 0) { sh_bv[wv] = best; sh_bi[wv] = besti; }
      __syncthreads();
      FLINT_TRACE(L, 1);
      if (t == 0) {
        float bv = sh_bv[0];
        int bi = sh_bi[0];
        for (int w = 1; w < kStackWaves; ++w)
          if (sh_bv[w] > bv || (sh_bv[w] == bv && sh_bi[w] < bi)) { bv = sh_bv[w]; bi = sh_bi[w]; }
        uint64_t* hp = P.hp + ((size_t)(tok & 1) * kStackWGs + blockIdx.x) * 2;
        put_pair(hp, bv, eph);
        put_pair(hp + 1, __int_as_float(bi), eph);
      }
    }
    // every workgroup waits for all head partials: the token boundary
    wait_pairs(P.hp + (size_t)(tok & 1) * kStackWGs * 2, 2 * kStackWGs, eph, sh_hp, wc);
    if (sh_bad) return;
    FLINT_TRACE(L, 2);
    if (wv == 0) {
      float bv = -FLT_MAX;
      int bi = INT_MAX;
      for (int i = lane; i < kStackWGs; i += 64) {
        const float v = sh_hp[2 * i];
        const int id = __float_as_int(sh_hp[2 * i + 1]);
        if (v > bv || (v == bv && id < bi)) { bv = v; bi = id; }
      }
      wave_argmax(bv, bi);
      if (lane == 0 && blockIdx.x == 0) P.argmax[tok] = bi;
    }
    __syncthreads();
  }
  if (blockIdx.x == 0 && t == 0)
    st_dev_u32(P.ctrl, base + (uint32_t)(P.T * (P.L + 1) * 4) + 4u);
#undef FLINT_TRACE
}

bool stack_persistent_supported(const flint_moe_dims& d) {
  return d.hidden == kHidden && d.n_experts % 2 == 0 && d.expert_width % 256 == 0 && d.shared_width % 256 == 0 &&
         d.n_experts % 8 == 0 && d.shared_width / kGroups <= 4 * kGroupWGs && d.n_experts <= kStackWaves * kGroupWGs &&
         d.top_k * (d.expert_width / kGroups) + d.shared_width / kGroups == kSliceK &&
         d.top_k * (d.expert_width / kGroups) <= kGateUpPerWave * kCommWaves * kGroupWGs &&
         d.shared_width / kGroups <= (kStackWaves - kCommWaves) * kGroupWGs &&
         d.n_experts <= 2 * (kStackWaves - kCommWaves) * kGroupWGs;
}

size_t stack_persistent_ws_bytes() {
  size_t o = 256;                                                  // ctrl
  o += sizeof(uint64_t) * 2 * kGroups * kMaxExperts;               // s2
  o += sizeof(uint64_t) * 2 * kGroups * kSliceK;                   // s3
  o += sizeof(uint64_t) * 2 * kGroups * kHidden * 2;               // s4a, s4b
  o += sizeof(uint64_t) * 2 * kStackWGs * 2;                       // hp
  return align_up(o, 256);
}

hipError_t launch_stack_persistent(const flint_moe_dims& d, int L, int vocab, const void* table, const float* x,
                                   int T, float eps, float* logits, int32_t* argmax, int32_t* routes, void* ws,
                                   int64_t* trace, hipStream_t s) {
  StackParams P;
  P.trace = trace;
  P.table = static_cast<const StackTable*>(table);
  P.L = L; P.E = d.n_experts; P.I = d.expert_width; P.k = d.top_k; P.Is = d.shared_width; P.V = vocab; P.T = T;
  P.eps = eps; P.x = x; P.logits = logits; P.argmax = argmax; P.routes = routes;
  char* w = static_cast<char*>(ws);
  P.ctrl = reinterpret_cast<uint32_t*>(w);
  w += 256;
  P.s2 = reinterpret_cast<uint64_t*>(w); w += sizeof(uint64_t) * 2 * kGroups * kMaxExperts;
  P.s3 = reinterpret_cast<uint64_t*>(w); w += sizeof(uint64_t) * 2 * kGroups * kSliceK;
  P.s4a = reinterpret_cast<uint64_t*>(w); w += sizeof(uint64_t) * 2 * kGroups * kHidden;
  P.s4b = reinterpret_cast<uint64_t*>(w); w += sizeof(uint64_t) * 2 * kGroups * kHidden;
  P.hp = reinterpret_cast<uint64_t*>(w);
  const StackTable* tab = P.table;
  void* args[] = {&P, &tab};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_stack_decode), dim3(kStackWGs),
                                    dim3(kStackThreads), args, 0, s);
}

hipError_t read_stack_error(const void* ws, int32_t* out) {
  uint32_t v = 0;
  hipError_t e = hipMemcpy(&v, static_cast<const char*>(ws) + 4, 4, hipMemcpyDeviceToHost);
  *out = (int32_t)v;
  return e;
}

}  // namespace flint
