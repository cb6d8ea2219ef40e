/*
 * flint_int4.h -- C ABI of the second 4.5-bit weight codec on MI355X
 * (gfx950): group-64 affine INT4 with a BF16 scale and a BF16 offset per
 * group, its quantiser, and a GEMV with argmax (the output head of a 4-bit
 * build).  Conventions (device pointers, caller-owned buffers, host-side
 * validation, status codes, zero-filled workspaces, 16-byte alignment,
 * finite inputs) are those of flint_moe.h.
 *
 * The format follows [P3 "Flint: 125 tokens a second is what 2.5B active
 * parameters buy at 273 GB/s", "Why active parameters set the speed"]:
 * Recursive's Apple build stores each group of 64 weights as 4-bit codes plus
 * a BF16 scale and a BF16 offset (4.5 bits per weight), and its output head
 * is 4-bit too (1,024 code bytes per 2,048-wide row).
 */
#ifndef FLINT_INT4_H
#define FLINT_INT4_H

#include "flint_moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* An INT4 matrix W [rows][cols] (cols, the reduction axis, a multiple of 64):
 *    codes  uint8  [rows][cols/2]   unsigned 4-bit codes q, element 2j in the
 *                                   LOW nibble of byte j, 2j+1 in the high one;
 *    scales uint16 [rows][cols/64]  BF16 bit patterns: scale s of elements
 *                                   64g .. 64g+63;
 *    biases uint16 [rows][cols/64]  BF16 bit patterns: offset b of the group.
 * Dequantised value fl32(s * q + b) (s * q is exact; one rounding). */
typedef struct {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* biases;
} flint_int4;

/* Quantise float w [rows][cols] (cols a multiple of 64; rows, cols >= 1) into
 * caller buffers, every decision in fp32:
 *   s = bf16(fl32((max - min) / 15)), b = bf16(min) over each group of 64,
 *   q = clamp(rint(fl32(fl32(w - b) / s)), 0, 15), or q = 0 when s == 0,
 * BF16 rounding to nearest even, rint ties to even.  No workspace. */
int32_t flint_int4_quantize(const float* w, int64_t rows, int64_t cols, uint8_t* codes, uint16_t* scales,
                            uint16_t* biases, void* stream);

/* out float [rows][cols] = the dequantised values (test export). */
int32_t flint_int4_dequantize(const flint_int4* w /*[host]*/, int64_t rows, int64_t cols, float* out,
                              void* stream);

/* Workspace bytes for flint_int4_gemv at B tokens (0 if B < 1 or B > 64). */
size_t flint_int4_gemv_workspace_bytes(int32_t B);

/* y_b = W x_b for B tokens (x float [B][cols], y float [B][rows]), fp32
 * arithmetic over the exactly dequantised weights: each lane forms
 * s * sum(q x) + b * sum(x) over its 32 elements.  argmax_opt (int32 [B]),
 * when non-NULL, receives the first index of each token's largest y.  This
 * build supports cols in {2048, 4096, 6144, 8192}, 1 <= rows < 2^31,
 * 1 <= B <= 64.  Workspace: flint_int4_gemv_workspace_bytes(B) (no
 * zero-fill needed). */
int32_t flint_int4_gemv(const flint_int4* w /*[host]*/, int32_t rows, int32_t cols, const float* x, int32_t B,
                        float* y, int32_t* argmax_opt, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLINT_INT4_H */
