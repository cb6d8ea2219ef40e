/*
 * flint_gemm.h -- C ABI of prompt processing on MI355X (gfx950): T tokens at
 * once through one NVFP4 matrix on the matrix cores, with full-precision
 * activations or with the activations quantised to NVFP4 as well (A4).
 * Conventions (device pointers, caller-owned buffers, host-side validation,
 * status codes, zero-filled workspaces, 16-byte alignment, finite inputs) and
 * the NVFP4 layout are those of flint_moe.h.
 *
 * The method follows [P1 "Flint-40B-A2B: AI-Built MoE Coding Model Hits 125
 * tok/s on MacBook Pro", "Custom Inference Kernels"; P2 "Recursive Releases
 * Flint, a 40B MoE Coding Model That Runs Locally at 125 Tokens per Second",
 * "How did the Eureka Machine build Flint?"]: dedicated kernels for low-bit
 * projections and for prompt processing.
 */
#ifndef FLINT_GEMM_H
#define FLINT_GEMM_H

#include "flint_moe.h"

#ifdef __cplusplus
extern "C" {
#endif

#define FLINT_GEMM_A32 0 /* activations at full precision */
#define FLINT_GEMM_A4 1  /* activations quantised to NVFP4 first */

/* Workspace bytes for flint_nvfp4_gemm (0 if the arguments are invalid). */
size_t flint_nvfp4_gemm_workspace_bytes(int32_t T, int32_t K, int32_t mode);

/* Y [T][N] = X [T][K] . W^T for an NVFP4 matrix W [N][K] (the layout of
 * flint_moe.h), Y and X float, row-major.
 *   FLINT_GEMM_A32: Y[t][n] = S_W * sum_k (e2m1 * e4m3)(W)[n][k] * X[t][k]
 *     on fp16 matrix cores: each activation is split into two fp16 parts
 *     (x = hi + lo to 22 significant bits; requires |x| < 65504), each weight
 *     is exact in fp16, products are exact and accumulate in fp32.
 *   FLINT_GEMM_A4: X is first quantised with the NVFP4 codec of
 *     flint_nvfp4_quantize as one [T][K] tensor (one fp32 tensor scale over
 *     all of X, E4M3 scales per 16 values along K), then
 *     Y = deq(Xq) . deq(W)^T, one fp16 part per operand.
 * Sizes: N >= 1, T >= 1, K a multiple of 256 and at most 2^20
 * (FLINT_E_UNSUPPORTED otherwise).
 * Workspace: flint_nvfp4_gemm_workspace_bytes(T, K, mode), zero-filled before
 * first use; every completed call leaves its counter zero.  A4 keeps the
 * quantised activations there: codes [T][K/2] from byte 512, then the E4M3
 * scales [T][K/16] at the next 256-byte boundary.  After them (both modes)
 * come the activations as fp16 planes for the matrix cores, [2][T][K]
 * (A32: hi, lo) or [T][K] (A4: code x block scale), written by every call. */
int32_t flint_nvfp4_gemm(const flint_nvfp4* W /*[host]*/, int32_t N, int32_t K, const float* X, int32_t T,
                         int32_t mode, float* Y, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLINT_GEMM_H */
