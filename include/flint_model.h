/*
 * flint_model.h -- C ABI of one whole Flint decode step on MI355X (gfx950):
 * every layer's attention (flint_attn.h) and its dense MLP or MoE layer
 * (flint_attn.h, flint_moe.h), then the NVFP4 output head with argmax, for
 * one token at one position.  Conventions (device pointers, caller-owned
 * buffers, host-side validation, status codes, zero-filled workspaces,
 * 16-byte alignment, finite inputs) are those of flint_moe.h.
 *
 * The layer plan follows [P2 "Recursive Releases Flint, a 40B MoE Coding
 * Model That Runs Locally at 125 Tokens per Second", "How does Flint's
 * architecture work?": 49 layers, the first 2 dense and the other 47 MoE;
 * 35 sliding-window and 14 full-attention layers] and [P3 "Flint: 125 tokens
 * a second is what 2.5B active parameters buy at 273 GB/s", "The shape, read
 * from the headers"].
 */
#ifndef FLINT_MODEL_H
#define FLINT_MODEL_H

#include "flint_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* A model of n_layers layers.  Layer l: h += Attn_l(rmsnorm(h)), then
 * h += F_l(rmsnorm(h)) with F_l the dense SwiGLU MLP for l < n_dense and the
 * MoE layer (flint_moe_decode) otherwise; after the last layer
 * logits = head(rmsnorm(h)) and argmax.  Every rmsnorm here has unit gain:
 * v / sqrt(mean(v^2) + eps).  All arrays are [host] arrays of device
 * pointers or values, read during the call only. */
typedef struct {
  int32_t n_layers;
  int32_t n_dense;                   /* 0 <= n_dense <= n_layers */
  int32_t dense_width;               /* 6144 */
  flint_moe_dims moe;                /* the MoE layers (and hidden size) */
  flint_attn_dims sliding;           /* layers with is_full[l] == 0 */
  flint_attn_dims full;              /* layers with is_full[l] == 1 */
  const int32_t* is_full;            /* [host] [n_layers] */
  const flint_attn_layer* attn;      /* [host] [n_layers] */
  uint16_t* const* k_cache;          /* [host] [n_layers] BF16 caches [n_kv][cap[l]][D] */
  uint16_t* const* v_cache;          /* [host] [n_layers] */
  const int32_t* cap;                /* [host] [n_layers] */
  const flint_nvfp4* dense;          /* [host] [n_dense][3]: gate [W][H], up [W][H], down [H][W] */
  const flint_moe_layer* moe_layers; /* [host] [n_layers - n_dense] */
  flint_nvfp4 head;                  /* [vocab][hidden] */
  int32_t vocab;
  float eps;                         /* block and final norms (1e-6) */
  /* Optional (may be NULL): a plan of the same MoE layers, prepared by
   * flint_stack_prepare with repacked down projections (its head and vocab
   * are not used).  With it every MoE layer runs as one launch of the
   * persistent stack kernel (one layer, no head); without it, as the kernel
   * sequence of flint_moe_decode.  The plan's dims must equal `moe`, its
   * n_layers must be n_layers - n_dense, and the sizes must allow the
   * persistent schedule (FLINT_E_UNSUPPORTED otherwise). */
  const flint_stack_plan* moe_plan;  /* [host] */
} flint_model;

/* Workspace bytes for flint_model_decode (0 if the model is invalid). */
size_t flint_model_workspace_bytes(const flint_model* m /*[host]*/);

/* One token x (float [hidden]) at position pos through the whole model:
 * logits_opt (float [vocab], may be NULL) and argmax (int32 [1]); every
 * layer's cache slot pos mod cap[l] is written as in flint_attn_decode.
 * h_out_opt (float [hidden]) receives the final residual when non-NULL.
 * Workspace: flint_model_workspace_bytes(m), zero-filled before first use;
 * with moe_plan it carries the persistent kernel's epoch counter from call to
 * call (as the stack workspace does) and must not be changed between calls. */
int32_t flint_model_decode(const flint_model* m /*[host]*/, const float* x, int32_t pos, float* logits_opt,
                           int32_t* argmax, float* h_out_opt, void* ws, size_t ws_bytes, void* stream);

/* The watchdog flag of the persistent MoE layers (as flint_stack_error):
 * synchronously copies it to *error [host] (0: none; always 0 without
 * moe_plan).  A set flag makes later calls skip their MoE layers until the
 * workspace is zeroed again. */
int32_t flint_model_error(const flint_model* m /*[host]*/, const void* ws, size_t ws_bytes, int32_t* error);

#ifdef __cplusplus
}
#endif

#endif /* FLINT_MODEL_H */
