// flint_common.h -- host helpers shared by the C-ABI source files: the
// last-HIP-error record and the device check.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/flint_attn.h"

namespace flint {

// records e as the last HIP error and returns FLINT_E_HIP
int32_t api_hip_fail(hipError_t e);
// FLINT_OK when the current device is gfx950 (cached per device)
int32_t api_check_device();

// One MoE layer for one token (kernel sequence), validated by the caller:
// y = MoE(rmsnorm(x)) (norm_eps < 0: no norm), added to y when add is set.
// Workspace api_moe_ws_bytes(d).
int32_t api_moe_check(const flint_moe_dims* d, const flint_moe_layer* L);
size_t api_moe_ws_bytes(const flint_moe_dims& d);
hipError_t api_moe_run(const flint_moe_dims& d, const flint_moe_layer& L, const float* x, float norm_eps, float* y,
                       bool add, void* ws, hipStream_t s);

// One attention layer for one token (attn.hip), validated by attn_check:
// y (+)= Attn(rmsnorm(x)) with the cache update of flint_attn_decode.
int32_t attn_check(const flint_attn_dims* d, const flint_attn_layer* L, int pos, const void* kc, const void* vc,
                   int cap);
size_t attn_ws_bytes(const flint_attn_dims& d);
// Byte offset in the workspace of q, k, v (float [n_q D + 2 n_kv D]).
size_t attn_qkv_offset(const flint_attn_dims& d);
// qkv_ready: q, k, v of rmsnorm(x) are already in the workspace (written by
// the kernel before), so the projection is skipped.
hipError_t attn_run(const flint_attn_dims& d, const flint_attn_layer& L, const float* x, float norm_eps, int pos,
                    uint16_t* kc, uint16_t* vc, int cap, float* y, bool accumulate, void* ws, hipStream_t s,
                    bool qkv_ready = false);

// Dense SwiGLU MLP for one token (attn.hip): y (+)= down(silu(gate u) * up u),
// u = rmsnorm(x); workspace 4 * width bytes.
int32_t dense_check(const flint_nvfp4* g, const flint_nvfp4* u, const flint_nvfp4* d, int hidden, int width);
hipError_t dense_run(const flint_nvfp4& g, const flint_nvfp4& u, const flint_nvfp4& d, int width, const float* x,
                     float norm_eps, float* y, bool accumulate, void* ws, hipStream_t s);

// Batched step with the routed gate/up matrices read from a tiled copy
// (batch.hip); tiles == nullptr reads the row-major weights.
size_t batch_tiles_layer_bytes(const flint_moe_dims& d);
hipError_t launch_batch_tiles(const flint_moe_dims& d, const flint_moe_layer* layers, int L, uint8_t* tiles,
                              hipStream_t s);
hipError_t launch_batch_step_tiled(const flint_moe_dims& d, const flint_moe_layer* layers, int L,
                                   const flint_nvfp4& head, int vocab, const float* x, int B, float eps, float* logits,
                                   int32_t* argmax, int32_t* routes, void* ws, hipStream_t s, const uint8_t* tiles);

}  // namespace flint
