// flint_internal.h -- host-side declarations shared by the C-ABI layer and the
// kernel launchers: dims, workspace layout, launch entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/flint_moe.h"

namespace flint {

constexpr int kHidden = 2048;    // the only hidden size with kernels
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 256;
constexpr int kMaxKdown = 4096;  // top_k * expert_width + shared_width
constexpr int kHeadBlocks = 1024;  // workgroups of the head GEMV (argmax partials)

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// argmax partial of one head workgroup
struct HeadPartial {
  float value;
  int32_t index;
};

// Workspace layouts.  Every section starts on a 256-byte boundary.
struct RouteWs {
  size_t logits, total;
  RouteWs(int E, int B) {
    size_t o = 0;
    logits = o; o = align_up(o + 4 * (size_t)B * E, 256);
    total = o;
  }
};

struct DecodeWs {
  size_t route, idx, wts, hact, total;
  DecodeWs(const flint_moe_dims& d, int B) {
    RouteWs r(d.n_experts, B);
    size_t o = 0;
    route = o; o = align_up(o + r.total, 256);
    idx = o; o = align_up(o + 4 * (size_t)B * d.top_k, 256);
    wts = o; o = align_up(o + 4 * (size_t)B * d.top_k, 256);
    hact = o; o = align_up(o + 4 * (size_t)B * (d.top_k * d.expert_width + d.shared_width), 256);
    total = o;
  }
};

struct HeadWs {
  size_t partials, total;
  explicit HeadWs(int B) {
    size_t o = 0;
    partials = o; o = align_up(o + sizeof(HeadPartial) * (size_t)B * kHeadBlocks, 256);
    total = o;
  }
};

// persistent decode (stack.hip)
constexpr int kMaxStackLayers = 64;  // layers the persistent schedule takes
constexpr int kStackGroups = 8;      // XCDs: column slices of the down projections
// Down projections of one layer repacked for the persistent schedule: the
// columns of each routed expert and of the shared expert cut into 8 slices,
// each slice stored contiguously over all rows, so that the XCD that owns a
// slice reads whole cache lines.
struct PackedDown {
  size_t codes, scales, shared_codes, shared_scales, total;  // byte offsets in one layer's block
  explicit PackedDown(const flint_moe_dims& d) {
    size_t o = 0;
    codes = o; o = align_up(o + (size_t)d.n_experts * d.hidden * d.expert_width / 2, 256);
    scales = o; o = align_up(o + (size_t)d.n_experts * d.hidden * d.expert_width / 16, 256);
    shared_codes = o; o = align_up(o + (size_t)d.hidden * d.shared_width / 2, 256);
    shared_scales = o; o = align_up(o + (size_t)d.hidden * d.shared_width / 16, 256);
    total = o;
  }
};
bool stack_persistent_supported(const flint_moe_dims& d, int L);
size_t stack_persistent_ws_bytes();

// Stack workspace: the persistent kernel's exchange area first (its control
// words at offset 0), then the buffers of the kernel-sequence schedule.
struct StackWs {
  size_t persist, h, decode, head, total;
  StackWs(const flint_moe_dims& d, int vocab) {
    (void)vocab;
    DecodeWs dw(d, 1);
    HeadWs hw(1);
    size_t o = 0;
    persist = o; o = align_up(o + stack_persistent_ws_bytes(), 256);
    h = o; o = align_up(o + 4 * (size_t)d.hidden, 256);
    decode = o; o = align_up(o + dw.total, 256);
    head = o; o = align_up(o + hw.total, 256);
    total = o;
  }
};

// Device-side table of the layer stack: the head, then the layers.
struct StackTable {
  flint_nvfp4 head;
  flint_moe_layer layers[1];  // n_layers entries
};
inline size_t stack_table_bytes(int L) { return sizeof(StackTable) + sizeof(flint_moe_layer) * (size_t)(L > 1 ? L - 1 : 0); }

// batched decode (batch.hip)
constexpr int kMaxBatch = 64;
struct BatchWs {
  size_t h, u, up, logits, idx, wts, bucket, hr, hs, dr, ds, partials, total;
  BatchWs(const flint_moe_dims& d, int B, int vocab);
};
bool batch_supported(const flint_moe_dims& d, int B);
hipError_t launch_batch_step(const flint_moe_dims& d, const flint_moe_layer* layers, int L, const flint_nvfp4& head,
                             int vocab, const float* x, int B, float eps, float* logits, int32_t* argmax,
                             int32_t* routes, void* ws, hipStream_t s);

// ---- kernel launchers (kernels.hip); all return the hipError_t of the launch
hipError_t launch_route(const flint_moe_dims& d, const float* router, const float* x, int B, float norm_eps,
                        float* logits, int32_t* idx, float* w, hipStream_t s);
// router variants: BF16 router rows and/or sigmoid-score weights, no norm
hipError_t launch_route_ex(const flint_moe_dims& d, const void* router, bool bf16, bool sigmoid, const float* x,
                           int B, float* logits, int32_t* idx, float* w, hipStream_t s);
hipError_t launch_gateup(const flint_moe_dims& d, const flint_moe_layer& L, const float* x, int B, float norm_eps,
                         const int32_t* idx, float* hact, hipStream_t s);
hipError_t launch_down(const flint_moe_dims& d, const flint_moe_layer& L, const int32_t* idx, const float* w,
                       const float* hact, int B, float* y, bool add_to_y, hipStream_t s);
hipError_t launch_lmhead(const flint_nvfp4& head, int vocab, const float* x, int B, float norm_eps, float* logits,
                         int32_t* argmax, HeadPartial* partials, hipStream_t s);
hipError_t launch_quantize(const float* w, int64_t n_mats, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, float* tscales, uint32_t* amax_bits, hipStream_t s);
hipError_t launch_dequantize(const flint_nvfp4& q, int64_t rows, int64_t cols, float* out, hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, int n, hipStream_t s);
hipError_t launch_slice_cols(const uint8_t* src, uint8_t* dst, int64_t outer, int rows, int rb, int G,
                             hipStream_t s);
// Rows of up to three NVFP4 matrices with K = hidden (a following attention
// layer's q, k and v) applied to the RMSNorm of the final residual at the end
// of a no-head launch: out[r] for r over rows[0] + rows[1] + rows[2].
struct StackQkv {
  const uint8_t* codes[3];
  const uint8_t* scales[3];
  const float* tscale[3];
  int rows[3];
  float* out;
};
// vocab == 0: no head, T == 1; layers l0 .. l0 + L - 1 of the table, the
// final residual to h_out (which may be x), and with qkv its rows.
// spin_limit != 0 (with a head): the stress instantiation, with delays seeded
// by stress_seed and waits that give up after spin_limit polls.
hipError_t launch_stack_persistent(const flint_moe_dims& d, int L, int vocab, const void* table, const float* x,
                                   int T, float eps, float* logits, int32_t* argmax, int32_t* routes, void* ws,
                                   int64_t* trace, hipStream_t s, int l0 = 0, float* h_out = nullptr,
                                   const StackQkv* qkv = nullptr, uint32_t stress_seed = 0,
                                   uint32_t spin_limit = 0);
hipError_t read_stack_error(const void* ws, int32_t* out);

}  // namespace flint
