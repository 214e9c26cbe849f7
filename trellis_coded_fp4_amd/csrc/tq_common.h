// tq_common.h -- device helpers shared by the libtrellis kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "trellis.h"   // include/ is on the include path (build.py)
#include "tq_decode.h"

namespace tq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- matrix core
//
// v_mfma_scale_f32_16x16x128_f8f6f4 with A = FP4 (E2M1) and B = FP8 (OCP E4M3),
// both block-scaled by UE8M0 bytes. Operand layout on gfx950 (measured with
// an in-bounds probe of the builtin): lane l = 16*g + i.
//   A (16 x 128): lane holds row i, K-block g (k = 32g .. 32g+31) as 32
//                 nibbles in its first 4 registers, low nibble first.
//   B (128 x 16): lane holds column i; bytes 0..15 are k = 16g .. 16g+15 and
//                 bytes 16..31 are k = 64+16g .. 64+16g+15.
//   scale_a / scale_b of lane 16*g + i: UE8M0 of row / column i, K-block g.
//   D (16 x 16): register r of lane l is D[4*(l/16) + r][l % 16].
__device__ __forceinline__ v4f mfma_fp4_fp8(v8i a, v8i b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, sa, 0, sb);
}

// ---------------------------------------------------------------- FP8 E4M3

// Round a float (|v| <= 448) to OCP E4M3, ties to even, subnormals kept:
// gfx950's v_cvt_pk_fp8_f32, which converts to the OCP formats on this chip.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xFFu;
}
// Two at once: a in byte 0, b in byte 1.
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// The value of E4M3 code c (its low byte; exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }

// UE8M0 exponent E such that amax / 2^E lies in [128, 256); 2^E is exact.
__device__ __forceinline__ int block_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127 - 7;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

}  // namespace tq
