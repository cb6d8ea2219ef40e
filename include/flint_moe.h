/*
 * flint_moe.h -- C ABI of the NVFP4 sparse-MoE decode library for AMD MI355X
 * (gfx950): router top-k, NVFP4 expert projections with SwiGLU and weighted
 * combine, the NVFP4 output head with argmax, and the whole layer stack.
 *
 * The method follows these pages (titles as published, sections named):
 *  [P3] "Flint: 125 tokens a second is what 2.5B active parameters buy at
 *       273 GB/s" -- "The shape, read from the headers": hidden size 2,048;
 *       47 MoE layers, each with 256 routed experts of width 512 of which 6
 *       are selected per token, plus a shared expert of width 1,024; three
 *       matrices per expert; untied output head over a 150,144-entry
 *       vocabulary.  "Why active parameters set the speed": batch-1 decode
 *       reads every touched weight once per token, so weight bytes set the
 *       speed; the output head is 4-bit.  "Checking 125 tokens a second":
 *       NVFP4 holds 4-bit values with one 8-bit scale per 16 values.
 *  [P2] "Recursive Releases Flint, a 40B MoE Coding Model That Runs Locally
 *       at 125 Tokens per Second" -- "How does Flint's architecture work?":
 *       the router selects 6 experts per token, plus 1 always-active shared
 *       expert.
 *  [P1] "Flint-40B-A2B: AI-Built MoE Coding Model Hits 125 tok/s on MacBook
 *       Pro" -- "Quantization with Offline Distillation": the output layer is
 *       quantised to NVFP4 as well.
 *
 * Conventions for every call below
 *  - Pointers are DEVICE pointers unless marked [host].  The caller owns every
 *    buffer (weights, activations, outputs, workspace, plan); the library
 *    allocates nothing and keeps no per-call state.
 *  - A call validates its arguments on the host first.  On any non-zero
 *    status nothing has been enqueued and nothing written.  FLINT_OK means
 *    "enqueued on `stream`" (a hipStream_t; NULL is the default stream);
 *    results are ready after the caller synchronises with that stream.
 *  - Workspaces: size from flint_workspace_bytes(); they must be zero-filled
 *    once before first use (e.g. allocated with torch.zeros) and every
 *    completed call leaves them zero-filled again.  Calls that may run at the
 *    same time need distinct workspaces.
 *  - Alignment: weight codes/scales rows and activation vectors must be
 *    16-byte aligned (128-bit loads).
 *  - Inputs must be finite; NaN/Inf inputs give unspecified results.
 *
 * NVFP4 matrix W [rows][cols] (the interchange layout; cols is the reduction
 * axis and a multiple of 32):
 *    codes  uint8 [rows][cols/2]   E2M1 codes, element 2j in the LOW nibble of
 *                                  byte j, element 2j+1 in the high nibble;
 *    scales uint8 [rows][cols/16]  OCP E4M3FN scale of elements 16b..16b+15;
 *    tscale float [1]              per-tensor fp32 scale S.
 *  Dequantised value: fl32((e2m1(code) * e4m3(scale)) * S), the first product
 *  exact.  Each routed expert matrix (gate, up, down of every expert), each
 *  shared-expert matrix and the head is its own tensor with its own S.
 */
#ifndef FLINT_MOE_H
#define FLINT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define FLINT_OK 0
#define FLINT_E_NULL (-1)        /* a required pointer is NULL */
#define FLINT_E_DIMS (-2)        /* a size is out of range */
#define FLINT_E_ALIGN (-3)       /* a pointer is not 16-byte aligned */
#define FLINT_E_WORKSPACE (-4)   /* workspace or plan buffer too small */
#define FLINT_E_DEVICE (-5)      /* current device is not gfx950 */
#define FLINT_E_HIP (-6)         /* a HIP call failed; see flint_last_hip_error() */
#define FLINT_E_INTERNAL (-7)    /* a device-side wait gave up (watchdog) in an earlier call */
#define FLINT_E_UNSUPPORTED (-8) /* valid sizes this build has no kernel for */

/* MoE layer sizes.  Supported: hidden == 2048; 1 <= top_k <= 8;
 * top_k <= n_experts <= 256; expert_width and shared_width multiples of 32,
 * 32..2048 each. */
typedef struct {
  int32_t hidden;       /* H: 2048 */
  int32_t n_experts;    /* E: 256 (32 in the reduced layer) */
  int32_t expert_width; /* I: 512 */
  int32_t top_k;        /* k: 6 */
  int32_t shared_width; /* Is: 1024 */
} flint_moe_dims;

/* one NVFP4 matrix (device pointers; tscale points at one float) */
typedef struct {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tscale;
} flint_nvfp4;

/* one MoE layer.  Routed experts are stacked along the first axis:
 *   router        float [E][H]            unquantised
 *   gate/up codes uint8 [E][I][H/2], scales [E][I][H/16]
 *   down codes    uint8 [E][H][I/2], scales [E][H][I/16]
 *   expert_tscales float [E][3]           S of gate, up, down of each expert
 *   shared_gate/up [Is][H], shared_down [H][Is]                              */
typedef struct {
  const float* router;
  const uint8_t* gate_codes;
  const uint8_t* gate_scales;
  const uint8_t* up_codes;
  const uint8_t* up_scales;
  const uint8_t* down_codes;
  const uint8_t* down_scales;
  const float* expert_tscales;
  flint_nvfp4 shared_gate;
  flint_nvfp4 shared_up;
  flint_nvfp4 shared_down;
} flint_moe_layer;

/* operation ids for flint_workspace_bytes */
#define FLINT_OP_ROUTE 1
#define FLINT_OP_DECODE 2
#define FLINT_OP_LMHEAD 3
#define FLINT_OP_STACK 4
#define FLINT_OP_QUANTIZE 5
#define FLINT_OP_STACK_BATCH 6

/* Bytes of workspace `op` needs for batch B (tokens), vocabulary `vocab`
 * (lmhead/stack) and L layers (stack); 0 if the arguments are invalid. */
size_t flint_workspace_bytes(int32_t op, const flint_moe_dims* dims /*[host], may be NULL for LMHEAD/QUANTIZE*/,
                             int32_t B, int32_t vocab, int32_t L);

/* Router and top-k [P2 "How does Flint's architecture work?"; P3 "The shape,
 * read from the headers"]: for each of B tokens x_b (float [B][H]):
 *   logits_e = sum_k router[e][k] * x_b[k]   (fp32 router, fp32 arithmetic);
 *   topk_idx[b][0..k) = the k largest logits, ordered by (logit descending,
 *                       expert index ascending);
 *   topk_w[b][i] = exp(l_i - l_0) / sum_j exp(l_j - l_0) over the chosen k
 *                  (the softmax over all E renormalised to the chosen set).
 * logits_opt (float [B][E]) receives the logits when non-NULL. */
int32_t flint_moe_route(const flint_moe_dims* dims /*[host]*/, const float* router, const float* x, int32_t B,
                        int32_t* topk_idx, float* topk_w, float* logits_opt, void* ws, size_t ws_bytes,
                        void* stream);

/* Router variants for flint_moe_route_ex. */
#define FLINT_ROUTER_F32 0   /* router is float [E][H] */
#define FLINT_ROUTER_BF16 1  /* router is BF16 bit patterns, uint16 [E][H] */
#define FLINT_SCORE_SOFTMAX 0 /* weights as in flint_moe_route */
#define FLINT_SCORE_SIGMOID 1 /* weights from sigmoid scores, see below */

/* Router and top-k with the variants the pages describe [P3 "Flint: 125
 * tokens a second is what 2.5B active parameters buy at 273 GB/s", "The
 * shape, read from the headers": the router scores with a sigmoid, as
 * DeepSeek-V3 does, without a bias-correction tensor; "Why active parameters
 * set the speed": Recursive's build keeps the router in BF16].
 *   router_dtype FLINT_ROUTER_F32: `router` is float [E][H], as in
 *                flint_moe_route;
 *                FLINT_ROUTER_BF16: `router` is uint16 [E][H] holding BF16
 *                bit patterns, each widened exactly to fp32 (half the router
 *                bytes); the products and sums are fp32.
 *   scoring      FLINT_SCORE_SOFTMAX: weights exactly as flint_moe_route;
 *                FLINT_SCORE_SIGMOID: score s_e = 1 / (1 + exp(-l_e)); the k
 *                largest scores are chosen (the same set and order as the k
 *                largest logits, since the sigmoid is increasing; ties to the
 *                lower index) and topk_w[b][i] = s_i / sum_j s_j over the
 *                chosen k, with no further scaling factor.
 * Every other argument, the workspace (FLINT_OP_ROUTE) and the status codes
 * are as for flint_moe_route; an unknown router_dtype or scoring returns
 * FLINT_E_DIMS.  flint_moe_route(...) equals flint_moe_route_ex(...,
 * FLINT_ROUTER_F32, FLINT_SCORE_SOFTMAX, ...). */
int32_t flint_moe_route_ex(const flint_moe_dims* dims /*[host]*/, const void* router, int32_t router_dtype,
                           int32_t scoring, const float* x, int32_t B, int32_t* topk_idx, float* topk_w,
                           float* logits_opt, void* ws, size_t ws_bytes, void* stream);

/* One MoE layer for B tokens (float [B][H]), no norm and no residual:
 *   y_b = sum_i topk_w[b][i] * E_{topk_idx[b][i]}(x_b) + Shared(x_b),
 * where each expert is SwiGLU: E(x) = Wdown (silu(Wgate x) * (Wup x)), silu
 * on the first (gate) matrix, all three matrices NVFP4 [P3 "The shape, read
 * from the headers": three matrices per expert].  The shared expert has
 * weight 1.  topk_idx_opt / topk_w_opt (int32/float [B][k]) receive the
 * routing when non-NULL.  y is float [B][H]. */
int32_t flint_moe_decode(const flint_moe_dims* dims /*[host]*/, const flint_moe_layer* layer /*[host]*/,
                         const float* x, int32_t B, float* y, int32_t* topk_idx_opt, float* topk_w_opt, void* ws,
                         size_t ws_bytes, void* stream);

/* flint_moe_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same layer, arguments and results (bit-identical), but no
 * workspace argument.  Its scratch is a fixed 1.125 MiB device array inside
 * the library, one per GPU, held until the process ends; the first call on a
 * device looks up that array's address (hipGetSymbolAddress) and keeps it.
 * The call allocates nothing (no hipMalloc, no allocating library routine).
 * Sizes whose flint_workspace_bytes(FLINT_OP_DECODE, dims, B) exceeds the
 * array return FLINT_E_WORKSPACE before anything is enqueued (the Flint
 * layer, E = 256, k = 6, I = 512, Is = 1024, fits up to B = 64).  Every call
 * on one GPU uses the same array and leaves its contents behind: calls that
 * may overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  Nothing needs clearing between calls. */
int32_t flint_moe_decode_noalloc(const flint_moe_dims* dims /*[host]*/, const flint_moe_layer* layer /*[host]*/,
                                 const float* x, int32_t B, float* y, int32_t* topk_idx_opt, float* topk_w_opt,
                                 void* stream);

/* NVFP4 output head [P1 "Quantization with Offline Distillation"; P3 "Why
 * active parameters set the speed"]: logits[b][v] = sum_k Wdeq[v][k] x[b][k]
 * for head W [vocab][hidden], x float [B][hidden]; argmax[b] = first index
 * of the largest logit (int32).  hidden must be 2048; vocab >= 1. */
int32_t flint_lmhead_gemv(const flint_nvfp4* head /*[host]*/, int32_t vocab, int32_t hidden, const float* x, int32_t B,
                          float* logits, int32_t* argmax, void* ws, size_t ws_bytes, void* stream);

/* Decode stack [P2 "How does Flint's architecture work?": 47 MoE layers; P3
 * "The shape, read from the headers": norms in the body].  For each of T
 * tokens, strictly one after the other (batch 1: token t+1 starts after
 * token t has produced its argmax):
 *   h_0 = x_t;  h_{l+1} = h_l + MoE_l(h_l / sqrt(mean(h_l^2) + eps))  (l < L);
 *   logits_t = Head(h_L / sqrt(mean(h_L^2) + eps));  argmax_t.
 *
 * flint_stack_prepare copies the layers' pointer table into `table`, a device
 * buffer of flint_stack_table_bytes(L) bytes, and fills the host-side plan.
 * For the persistent schedule it also repacks every layer's down projections
 * (routed and shared) into `packed`, a device buffer of
 * flint_stack_packed_bytes(dims, L) bytes: the columns of each down matrix
 * cut into 8 slices (one per XCD), each slice contiguous over all rows, same
 * codes and scales.  `packed` may be NULL (then only the kernel-sequence
 * schedule is available); flint_stack_packed_bytes returns 0 when the sizes
 * do not allow the persistent schedule.  Prepare synchronises `stream`.
 * The plan keeps `layers` (the caller's host array), `table` and `packed`;
 * they, and every weight they point at, must stay valid and unchanged while
 * calls that use the plan run.  flint_stack_decode: x float [T][H]; logits float [T][vocab] (may be
 * NULL: only argmax is written); argmax int32 [T]; routes_opt int32
 * [T][L][k] receives every layer's chosen experts (ordered by logit
 * descending) when non-NULL. */
typedef struct {
  flint_moe_dims dims;
  int32_t n_layers;
  int32_t vocab;
  flint_nvfp4 head;
  const flint_moe_layer* layers; /* [host] caller's array of n_layers */
  const void* table;             /* device copy of the layer table */
  int32_t schedule;              /* FLINT_SCHEDULE_*; prepare sets AUTO */
  const void* packed;            /* repacked down projections, or NULL */
} flint_stack_plan;

/* Schedules of flint_stack_decode.  PERSISTENT: one launch (256 workgroups,
 * one per compute unit, all resident) that
 * runs every token, layer and the head (needs expert_width and shared_width
 * multiples of 256, top_k*expert_width/8 + shared_width/8 == 512,
 * shared_width <= 1024, an even n_experts); KERNELS: three kernels per layer
 * and one for the head, any supported sizes; AUTO: PERSISTENT when the sizes
 * allow it and the plan holds packed down projections. */
#define FLINT_SCHEDULE_AUTO 0
#define FLINT_SCHEDULE_KERNELS 1
#define FLINT_SCHEDULE_PERSISTENT 2

size_t flint_stack_table_bytes(int32_t L);
size_t flint_stack_packed_bytes(const flint_moe_dims* dims /*[host]*/, int32_t L);
int32_t flint_stack_prepare(const flint_moe_dims* dims /*[host]*/, const flint_moe_layer* layers /*[host] array of L*/,
                            int32_t L, const flint_nvfp4* head /*[host]*/, int32_t vocab, void* table,
                            size_t table_bytes, void* packed, size_t packed_bytes,
                            flint_stack_plan* plan /*[host], out*/, void* stream);
int32_t flint_stack_decode(const flint_stack_plan* plan /*[host]*/, const float* x, int32_t T, float eps, float* logits,
                           int32_t* argmax, int32_t* routes_opt, void* ws, size_t ws_bytes, void* stream);

/* Profiling variant of flint_stack_decode for the persistent schedule: also
 * writes, for the first token, device wall-clock stamps (100 MHz ticks) of
 * the phase boundaries of two workgroups (one on the first XCD, one on the
 * last) into trace, int64 [2][L+1][32], followed by the stamps of layer 1 of
 * all 256 workgroups, int64 [256][32].  Per layer l, seen by the first
 * polling wave: 0 layer start, 1 norm done, 2 logits arrived, 16 its keys
 * sorted, 17 first pick published, 18 last round done, 3 every pick of the
 * top k published, 4 its routed pairs stored, 5 hidden slice arrived,
 * 28 its partial outputs stored, 14 its residual rows stored (partial
 * outputs arrived and summed), 6 the barrier after them passed, 7 new
 * residual arrived, 15 routing weights computed; seen by the second polling
 * wave: 23 / 25 the pick of its first /
 * second pair known, 24 / 26 that pair requested, 27 its pairs stored; seen
 * by the first loading wave: 8 router logit stored, 9 shared pair stored, 11
 * routed phase started, 19 the pick of its pair known, 20 its pair
 * requested, 21 every pick known, 22 down-projection operands requested, 13
 * the next layer's rows requested, 12 its routed pair stored, 29 its partial
 * outputs stored; 10, 30 and 31 are unused (0).
 * Row L holds the head start, the head rows done, the head partials
 * arrived, the kernel entry and the end of the kernel's set-up.  Returns
 * FLINT_E_UNSUPPORTED for the kernel-sequence schedule and for more than 64
 * layers. */
int32_t flint_stack_decode_traced(const flint_stack_plan* plan /*[host]*/, const float* x, int32_t T, float eps,
                                  float* logits, int32_t* argmax, int32_t* routes_opt, void* ws, size_t ws_bytes,
                                  int64_t* trace, void* stream);

/* Part of the stack for one token, no head [P2 "How does Flint's
 * architecture work?": 47 MoE layers; P3 "The shape, read from the headers"]:
 * h_0 = x (float [H]); for l = l0 .. l0 + n - 1 of the plan's layers,
 * h <- h + MoE_l(h / sqrt(mean(h^2) + eps)); the final h to h_out (float
 * [H]; may be the same buffer as x).  One launch of the persistent schedule
 * (the plan needs packed down projections; FLINT_E_UNSUPPORTED otherwise),
 * for checking single layers against a reference and for models that put
 * other layers between MoE layers.  routes_opt int32 [n][k] receives each
 * layer's chosen experts (by logit descending) when non-NULL.  Workspace and
 * watchdog flag as for flint_stack_decode (the same stack workspace may be
 * used by both, one call after the other).  l0 >= 0, n >= 1,
 * l0 + n <= n_layers. */
int32_t flint_stack_decode_layers(const flint_stack_plan* plan /*[host]*/, int32_t l0, int32_t n, const float* x,
                                  float eps, float* h_out, int32_t* routes_opt, void* ws, size_t ws_bytes,
                                  void* stream);

/* Test hook for the persistent schedule's exchange protocol: the decode of
 * flint_stack_decode (same arguments, workspace and results) by a second
 * instantiation of the persistent kernel that, before every exchange store,
 * sleeps for a pseudo-random time derived from `seed` (up to about 14 us, at
 * one store in four), permutes the roles of the workgroups inside each XCD,
 * and lets every wait give up after `spin_limit` polls (>= 1; the plain
 * kernel's limit is 2^22).  With a generous limit the results are
 * bit-identical to flint_stack_decode's; with a tiny one the waits give up,
 * the watchdog flag is raised (flint_stack_error) and the call's outputs are
 * unspecified.  Needs a plan with packed down projections
 * (FLINT_E_UNSUPPORTED otherwise). */
int32_t flint_stack_decode_stress(const flint_stack_plan* plan /*[host]*/, const float* x, int32_t T, float eps,
                                  float* logits, int32_t* argmax, int32_t* routes_opt, void* ws, size_t ws_bytes,
                                  uint32_t seed, uint32_t spin_limit, void* stream);

/* Small-batch decode step [P2 "How does Flint's architecture work?"; P3
 * "The shape, read from the headers"]: B tokens (1 <= B <= 64) through the
 * same stack and head together, each token with its own top-k routing:
 * for every token b the result is that of flint_stack_decode on x_b alone.
 * Per layer the B*k (token, slot) pairs are grouped by expert, so each
 * chosen expert's matrices are read once for all the tokens that chose it;
 * the router, the shared expert and the head are read once per step.
 * x float [B][H]; logits float [B][vocab] or NULL; argmax int32 [B];
 * routes_opt int32 [L][B][k] (chosen experts per layer, by logit
 * descending).  Workspace: flint_workspace_bytes(FLINT_OP_STACK_BATCH, dims,
 * B, vocab, L); no zero-fill needed.  Uses the plan's host layer array (the
 * canonical layout; `packed` is not needed).  Needs expert_width and
 * shared_width in {512, 1024, 2048} (FLINT_E_UNSUPPORTED otherwise). */
int32_t flint_stack_decode_batch(const flint_stack_plan* plan /*[host]*/, const float* x, int32_t B, float eps,
                                 float* logits, int32_t* argmax, int32_t* routes_opt, void* ws, size_t ws_bytes,
                                 void* stream);

/* Optional tiled copy of every layer's gate, up and down matrices (routed
 * experts and the shared expert) for the batched step: the same codes and
 * scales, reordered so that each 16-row x 256-column block is one contiguous
 * 2 KB run of codes and one 256-byte run of scales, in the order the
 * matrix-core kernels read them (3 (E I + Is) H (1/2 + 1/16) bytes per
 * layer: 456.5 MB per Flint layer, 21.5 GB for the 47).
 * flint_stack_batch_tiles_bytes: size of that copy for L layers (0 if the
 * sizes are not supported by the batched step).  flint_stack_batch_tiles
 * fills `tiles` (device, caller-owned) from the plan's layers; call it again
 * after the weights change.  flint_stack_decode_batch_tiled is
 * flint_stack_decode_batch with the expert weights read from `tiles`
 * (bit-identical results). */
size_t flint_stack_batch_tiles_bytes(const flint_moe_dims* dims /*[host]*/, int32_t L);
int32_t flint_stack_batch_tiles(const flint_stack_plan* plan /*[host]*/, void* tiles, size_t tiles_bytes,
                                void* stream);
int32_t flint_stack_decode_batch_tiled(const flint_stack_plan* plan /*[host]*/, const void* tiles, const float* x,
                                       int32_t B, float eps, float* logits, int32_t* argmax, int32_t* routes_opt,
                                       void* ws, size_t ws_bytes, void* stream);

/* Stack workspace contract: zero-filled before the first call; afterwards it
 * carries the persistent schedule's epoch counter and the placement phase of
 * its logit exchange, and must not be changed between calls.  The first call
 * on a zeroed workspace measures that phase (a few microseconds: one
 * workgroup times device-scope stores to blocks of the exchange area, which
 * the chip serves from its nearer or farther half depending on the address);
 * the phase affects speed only, never results.  Every wait inside the persistent kernel is bounded; if one
 * gives up (a fault elsewhere), the kernel raises a flag in the workspace and
 * returns, and later calls on that workspace do nothing until it is zeroed
 * again.  flint_stack_error synchronously copies that flag to *error [host]
 * (0: none). */
int32_t flint_stack_error(const void* ws, size_t ws_bytes, int32_t* error /*[host]*/);

/* NVFP4 quantiser (device): quantises n_mats independent matrices stacked in
 * w (float [n_mats][rows][cols], cols a multiple of 32) into codes
 * [n_mats][rows][cols/2], scales [n_mats][rows][cols/16] and tscales
 * [n_mats].  Per matrix: S = fl32(max|w| / 2688); block scale = E4M3
 * round-to-nearest-even of blockmax / (6 S), saturating at 448; code = E2M1
 * round-to-nearest-even of w / (d S), saturating at 6, sign kept (also for
 * values that round to zero); a block whose scale is 0 gets all-zero codes;
 * an all-zero matrix gets S = 0.  Ratios are computed in double precision.
 * [P3 "Checking 125 tokens a second": 4-bit values, one 8-bit scale per 16.] */
int32_t flint_nvfp4_quantize(const float* w, int64_t n_mats, int64_t rows, int64_t cols, uint8_t* codes,
                             uint8_t* scales, float* tscales, void* ws, size_t ws_bytes, void* stream);

/* NVFP4 quantiser on the host [P3 "Checking 125 tokens a second": 4-bit
 * values, one 8-bit scale per 16 values; P1 "Quantization with Offline
 * Distillation": NVFP4 weights and output head]: the library's own encoder
 * for weights prepared off the GPU, with the recipe of flint_nvfp4_quantize
 * (bit-identical results) for one matrix w [rows][cols] (all [host]):
 * codes uint8 [rows][cols/2], scales uint8 [rows][cols/16], *tscale = S.
 * cols must be a multiple of 16 (>= 16), rows >= 1.  Needs no GPU and no HIP
 * runtime; runs on up to 32 host threads (the result does not depend on
 * their number); synchronous.  Returns FLINT_E_NULL or FLINT_E_DIMS without
 * writing anything, else FLINT_OK.  Inputs must be finite. */
int32_t flint_nvfp4_quantize_host(const float* w, int64_t rows, int64_t cols, uint8_t* codes, uint8_t* scales,
                                  float* tscale);

/* Dequantise an NVFP4 matrix to float [rows][cols] (the exact values above). */
int32_t flint_nvfp4_dequantize(const flint_nvfp4* w /*[host]*/, int64_t rows, int64_t cols, float* out, void* stream);

/* Measurement aid, not part of the decode path: reads `bytes` bytes of src
 * (device, 16-byte aligned, bytes a multiple of 16) once with 128-bit
 * non-temporal loads, the access pattern of the decode kernels' weight
 * streams, and does nothing else with them (out, one device uint32, is
 * written only on a hash coincidence).  Timed over a buffer much larger than
 * the 256 MB last-level cache it gives the achievable read bandwidth that the
 * decode step's bandwidth (bytes per token x tokens per second [P3 "Checking
 * 125 tokens a second"]) is compared with. */
int32_t flint_stream_read(const void* src, size_t bytes, uint32_t* out, void* stream);

/* Human-readable status; the last hipError_t seen by a failing call (0 if none). */
const char* flint_status_str(int32_t status);
int32_t flint_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FLINT_MOE_H */
