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

// Round a float (|v| < 448) to OCP E4M3, ties to even.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  // |v| >= 2^-6: normal E4M3, keep 3 mantissa bits (round half to even),
  // saturate at 448. Below: subnormals, multiples of 2^-9 (0..8; 8 is the
  // smallest normal). Both are computed and selected, without branches.
  const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
  const uint32_t normal = min(r - ((127u - 7u) << 3), 0x7Eu);
  const uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  return sign | (a >= 0x3C800000u ? normal : sub);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * (1.0f / 512.0f);
  return (c & 0x80u) ? -mag : mag;
}

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
