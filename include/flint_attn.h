/*
 * flint_attn.h -- C ABI for the rest of a Flint decode step on MI355X
 * (gfx950): one grouped-query attention layer over a BF16 key/value cache,
 * and the dense SwiGLU MLP layers.  Conventions (device pointers, caller-owned
 * buffers, host-side validation, status codes, zero-filled workspaces,
 * 16-byte alignment, finite inputs) and the NVFP4 layout are those of
 * flint_moe.h.
 *
 * The method follows these pages (titles as published, sections named):
 *  [P3] "Flint: 125 tokens a second is what 2.5B active parameters buy at
 *       273 GB/s" -- "The shape, read from the headers": 32 query heads and 4
 *       key/value heads of dimension 128 on a 2,048-wide stream; 35 layers
 *       attend over a sliding window of 513 tokens (the current one and 512
 *       before it) with RoPE, 14 over the whole context without positional
 *       encoding; every layer normalises each query and key head (RMSNorm)
 *       and has one learned sink per query head; two dense MLP layers.
 *       "Why active parameters set the speed": the cache holds one key and
 *       one value of 4 x 128 BF16 values per token and layer.  "Built from
 *       scratch?": the dense MLP layers are 6,144 wide.
 *  [P2] "Recursive Releases Flint, a 40B MoE Coding Model That Runs Locally
 *       at 125 Tokens per Second" -- "How does Flint's architecture work?":
 *       2 dense layers before the 47 MoE layers; 35 sliding-window and 14
 *       full-attention layers; 32 query and 4 key/value heads.
 */
#ifndef FLINT_ATTN_H
#define FLINT_ATTN_H

#include "flint_moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Shape of one attention layer.  This build supports hidden == 2048,
 * head_dim == 128, n_q_heads a multiple of 16 up to 64, n_kv_heads dividing
 * n_q_heads with at most 8 query heads per key/value head (FLINT_E_UNSUPPORTED
 * otherwise). */
typedef struct {
  int32_t hidden;     /* 2048 */
  int32_t n_q_heads;  /* 32 */
  int32_t n_kv_heads; /* 4 */
  int32_t head_dim;   /* 128 */
  int32_t window;     /* > 0: attend to positions pos-window+1 .. pos (513); 0: to 0 .. pos */
  int32_t rope;       /* 1: rotate q and k by position (RoPE); 0: no positional encoding */
  float rope_theta;   /* RoPE base; the pages give none (10000 in the tests) */
  float eps;          /* head RMSNorm epsilon (1e-6) */
} flint_attn_dims;

/* Weights of one attention layer.
 *   q  NVFP4 [n_q*D][hidden]     k, v NVFP4 [n_kv*D][hidden]
 *   o  NVFP4 [hidden][n_q*D]
 *   q_norm, k_norm float [D]     gains of the per-head RMSNorms (one vector
 *                                shared by all query heads, one by all key heads)
 *   sinks float [n_q]            one learned sink logit per query head */
typedef struct {
  flint_nvfp4 q;
  flint_nvfp4 k;
  flint_nvfp4 v;
  flint_nvfp4 o;
  const float* q_norm;
  const float* k_norm;
  const float* sinks;
} flint_attn_layer;

/* Workspace bytes for flint_attn_decode (0 if dims are invalid or
 * unsupported).  It does not depend on the context length. */
size_t flint_attn_workspace_bytes(const flint_attn_dims* dims /*[host]*/);

/* One attention layer for one new token at position `pos` (no norm before it,
 * no residual after it), x float [hidden] -> y float [hidden]:
 *   q = Wq x, k = Wk x, v = Wv x (fp32 arithmetic on exactly dequantised
 *   weights);
 *   each query head q_h <- q_h * q_norm / sqrt(mean(q_h^2) + eps), each key
 *   head likewise with k_norm;
 *   if rope: element i of a head turns with element i + D/2 by the angle
 *   pos * theta^(-2i/D), (a, b) -> (a cos - b sin, a sin + b cos);
 *   the key and value of every key/value head g, rounded to BF16 (nearest
 *   even), are stored at slot pos mod cap:
 *     k_cache[g][pos mod cap][0..D), v_cache[g][pos mod cap][0..D);
 *   query head h reads key/value head g = h / (n_q/n_kv) over the positions
 *   t = first .. pos (first = max(0, pos-window+1) for window > 0, else 0),
 *   each at slot t mod cap:
 *     s_t = q_h . K_t / sqrt(D),  M = max(max_t s_t, sinks[h]),
 *     Z = sum_t exp(s_t - M) + exp(sinks[h] - M),
 *     o_h = sum_t exp(s_t - M) / Z * V_t       (the sink adds to Z only);
 *   y = Wo o.
 * k_cache, v_cache: uint16 (BF16 bit patterns) [n_kv][cap][D], owned by the
 * caller; slots of earlier positions in the window must hold their keys and
 * values (written by earlier calls or by the caller).  Only the slot of `pos`
 * is written.  cap must be >= window (window > 0; a ring of slots) or > pos
 * (window == 0), else FLINT_E_DIMS; pos >= 0.
 * Workspace: flint_attn_workspace_bytes(dims) (no zero-fill needed); calls
 * that may overlap need distinct workspaces and caches. */
int32_t flint_attn_decode(const flint_attn_dims* dims /*[host]*/, const flint_attn_layer* layer /*[host]*/,
                          const float* x, int32_t pos, uint16_t* k_cache, uint16_t* v_cache, int32_t cap, float* y,
                          void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for flint_dense_mlp at B tokens (0 if invalid). */
size_t flint_dense_workspace_bytes(int32_t hidden, int32_t width, int32_t B);

/* Dense SwiGLU MLP for B tokens (no norm, no residual), x, y float [B][hidden]:
 *   y_b = Wdown (silu(Wgate x_b) * (Wup x_b)),   silu(g) = g / (1 + e^-g),
 * gate, up NVFP4 [width][hidden], down NVFP4 [hidden][width].  This build
 * supports hidden == 2048, width a multiple of 2048 up to 8192 (6144 in
 * Flint), 1 <= B <= 64.  Workspace: flint_dense_workspace_bytes(hidden,
 * width, B) (no zero-fill needed). */
int32_t flint_dense_mlp(const flint_nvfp4* gate /*[host]*/, const flint_nvfp4* up /*[host]*/,
                        const flint_nvfp4* down /*[host]*/, int32_t hidden, int32_t width, const float* x, int32_t B,
                        float* y, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLINT_ATTN_H */
