// flint_device.h -- gfx950 device building blocks shared by the kernels of this
// library: NVFP4 decode in registers, wave reductions, cross-workgroup stores.
//
// NVFP4 as used here [P3 "Flint: 125 tokens a second is what 2.5B active
// parameters buy at 273 GB/s", "Checking 125 tokens a second": 4-bit values,
// one 8-bit scale per 16 values]: E2M1 element codes, one OCP E4M3FN scale per
// 16 elements along the reduction axis, one fp32 scale per tensor.
//
// Lane layout of every NVFP4 dot product: a lane owns 32 consecutive elements
// of a row, i.e. one 16-byte load of codes (two blocks) and one 2-byte load of
// scales; 64 lanes cover a 2,048-wide row with a single 128-bit load each.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flint {

constexpr int kWave = 64;

// Buffer loads: a uniform resource per matrix plus a per-lane byte offset.
// Unlike generic (flat) loads of pointers read from a device-side table they
// count only against the vector-memory wait counter, so LDS accesses and
// barriers do not wait for weight loads in flight.  Sizes above 2 GiB are not
// used by these kernels.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           (int)(bytes < 0x7FFFFFFFull ? bytes : 0x7FFFFFFFull), 0x00020000);
}
__device__ __forceinline__ uint4 bload_u4(rsrc_t r, uint32_t off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t bload_u16(rsrc_t r, uint32_t off) {
  return (uint32_t)(unsigned short)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ float4 bload_f4(rsrc_t r, uint32_t off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}
__device__ __forceinline__ float bload_f32(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// Scalar load of read-only data at a wave-uniform address (through the
// constant address space, so the compiler emits a scalar-memory load): for
// per-matrix values such as tensor scales, which then take no slot of the
// vector-memory pipeline.  The data must not be written while a kernel that
// reads it runs (the scalar cache is not kept coherent with vector stores).
typedef __attribute__((address_space(4))) const float const_f32;
__device__ __forceinline__ float sload_f32(const float* p, uint32_t i) {
  return ((const_f32*)p)[i];
}
// Streaming variants (non-temporal: the weights are read once per token and
// not kept in the caches), about 10% more HBM bandwidth on long streams.
constexpr int kAuxNT = 2;
__device__ __forceinline__ uint4 bload_u4_nt(rsrc_t r, uint32_t off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxNT);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t bload_u16_nt(rsrc_t r, uint32_t off) {
  return (uint32_t)(unsigned short)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kAuxNT);
}
__device__ __forceinline__ float4 bload_f4_nt(rsrc_t r, uint32_t off) {
  auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxNT);
  return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3]));
}

// Streaming loads through a plain pointer (non-temporal global loads).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt_u4(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_nt_u16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const unsigned short*>(p));
}
__device__ __forceinline__ uint32_t ld_nt_u32(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ float4 ld_nt_f4(const void* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// OCP E4M3FN byte -> float (gfx950 converts OCP FP8 in hardware).
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(byte, 0);
}

// sum_j e2m1(code_j) * x[j] over the 8 codes of one 32-bit word (element 2i in
// the low nibble of byte i).  The hardware conversion takes a power-of-two
// scale; 1.0 leaves the E2M1 values unchanged.
__device__ __forceinline__ float fp4x8_dot(uint32_t w, const float* x, float acc) {
  auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  acc = __builtin_fmaf(v0[0], x[0], acc);
  acc = __builtin_fmaf(v0[1], x[1], acc);
  acc = __builtin_fmaf(v1[0], x[2], acc);
  acc = __builtin_fmaf(v1[1], x[3], acc);
  acc = __builtin_fmaf(v2[0], x[4], acc);
  acc = __builtin_fmaf(v2[1], x[5], acc);
  acc = __builtin_fmaf(v3[0], x[6], acc);
  acc = __builtin_fmaf(v3[1], x[7], acc);
  return acc;
}

// the 8 E2M1 values of one 32-bit word, element order as stored
__device__ __forceinline__ void fp4x8_values(uint32_t w, float* v) {
  auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  v[0] = v0[0]; v[1] = v0[1]; v[2] = v1[0]; v[3] = v1[1];
  v[4] = v2[0]; v[5] = v2[1]; v[6] = v3[0]; v[7] = v3[1];
}

// One lane's share of an NVFP4 row dot product: 32 elements = codes c (two
// 16-element blocks) with block scales sc (low byte = first block) against
// x[0..31].  Returns d0 * dot(block0) + d1 * dot(block1) (tensor scale not
// applied).
__device__ __forceinline__ float nvfp4_lane_dot32(uint4 c, uint32_t sc, const float* x) {
  float a0 = fp4x8_dot(c.x, x + 0, 0.0f);
  a0 = fp4x8_dot(c.y, x + 8, a0);
  float a1 = fp4x8_dot(c.z, x + 16, 0.0f);
  a1 = fp4x8_dot(c.w, x + 24, a1);
  return e4m3_to_f32(sc & 0xFF) * a0 + e4m3_to_f32((sc >> 8) & 0xFF) * a1;
}

// Cross-lane steps with DPP (data-parallel primitives: register-to-register
// moves inside a 16-lane row), a few cycles each, instead of LDS round trips.
// Every lane of the wave must be active.
template <int ctrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}
template <int ctrl>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, ctrl, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

// sum over each row of 16 lanes, result in every lane of the row
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ float lane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Row broadcasts (GFX9 DPP): lane 15 of each row to the next row, and lane
// 31 to rows 2 and 3; rows outside the row mask keep `old`.
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// sum over the wave, result (uniform) in every lane: row sums, then row 1 +=
// row 0 and row 3 += row 2, then row 3 += row 1; lane 63 holds
// (r0 + r1) + (r2 + r3)
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowBcast15, 0xA, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowBcast31, 0xC, 0xF, false));
  return lane_f32(v, 63);
}

// sum over groups of `width` consecutive lanes (width a power of two <= 64)
template <int width>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (width == 16) {
    return row16_sum(v);
  } else {
#pragma unroll
    for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
  }
}

// maximum over the wave, result (uniform) in every lane
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), kDppRowBcast15,
                                                           0xA, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), kDppRowBcast31,
                                                           0xC, 0xF, false)));
  return lane_f32(v, 63);
}

// Order-preserving int32 key of a float (not NaN): flipping the magnitude
// bits of negative values makes signed integer order match float order.  The
// map is its own inverse.
__device__ __forceinline__ int ord_key(float f) {
  const int b = __float_as_int(f + 0.0f);  // -0 -> +0: equal floats, equal keys
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float ord_key_value(int key) { return __int_as_float(key ^ ((key >> 31) & 0x7FFFFFFF)); }

// maximum over the wave of an int, result (uniform) in every lane; every
// step is one fused DPP max
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppXor1, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppXor2, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppHalfMirror, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_mov_dpp(v, kDppMirror, 0xF, 0xF, true));
  v = max(v, __builtin_amdgcn_update_dpp(v, v, kDppRowBcast15, 0xA, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(v, v, kDppRowBcast31, 0xC, 0xF, false));
  return __builtin_amdgcn_readlane(v, 63);
}

// minimum over the wave, result (uniform) in every lane
__device__ __forceinline__ int wave_min_dpp(int v) {
  v = min(v, dpp_i32<kDppXor1>(v));
  v = min(v, dpp_i32<kDppXor2>(v));
  v = min(v, dpp_i32<kDppHalfMirror>(v));
  v = min(v, dpp_i32<kDppMirror>(v));
  v = min(v, __builtin_amdgcn_update_dpp(v, v, kDppRowBcast15, 0xA, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(v, v, kDppRowBcast31, 0xC, 0xF, false));
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// (value, index) maximum with ties to the lower index, over the wave.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, kWave);
    int oi = __shfl_xor(i, o, kWave);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Device-scope (all XCDs) relaxed accesses: the store writes through to the
// coherence point, the load bypasses the non-coherent per-XCD L2.
__device__ __forceinline__ void st_dev_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev_u32(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_f32(float* p, float v) { st_dev_u32(reinterpret_cast<uint32_t*>(p), __float_as_uint(v)); }
__device__ __forceinline__ float ld_dev_f32(const float* p) {
  return __uint_as_float(ld_dev_u32(reinterpret_cast<const uint32_t*>(p)));
}

}  // namespace flint
