// Device-side helpers shared by the mxattn kernels (gfx950 only).
//
// MXFP4: blocks of 32 elements share one E8M0 scale; elements are FP4 E2M1
// (BitDecoding-FP4 page, "The KV Cache Bottleneck in Long-Context LLM
// Serving").  OCP and UOS scale rules: see include/mxattn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxattn {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Value of element i of a row of bf16/fp16/fp32 data, widened to fp32.
__device__ __forceinline__ float load_elem(const void* base, int64_t i, int dtype) {
  if (dtype == 0) return reinterpret_cast<const float*>(base)[i];
  uint16_t u = reinterpret_cast<const uint16_t*>(base)[i];
  if (dtype == 2) return __uint_as_float(static_cast<uint32_t>(u) << 16);
  return static_cast<float>(__builtin_bit_cast(_Float16, u));
}

// E8M0 byte for a block maximum given as the fp32 bit pattern of |amax|.
// OCP: e = floor(log2 amax) - 2.  UOS: one more when amax / 2^e_ocp > qmax,
// i.e. when the significand 1.m exceeds qmax/4 (qmax in (4, 8)).  Zero and
// subnormal maxima land in the clamp region: byte 0 (e = -127).
__device__ __forceinline__ int e8m0_byte(uint32_t amax_bits, bool uos, float qmax_quarter) {
  int biased = static_cast<int>(amax_bits >> 23);
  if (biased == 0) return 0;
  int inc = 0;
  if (uos) {
    float sig = __uint_as_float(0x3F800000u | (amax_bits & 0x7FFFFFu));
    inc = sig > qmax_quarter ? 1 : 0;
  }
  int b = biased - 2 + inc;
  return b < 0 ? 0 : (b > 254 ? 254 : b);
}

// E2M1 code of fp32 value y in a block with scale byte sb, round to nearest
// even with saturation; the sign bit is kept for values that round to 0.
// |y| / 2^e is formed exactly with ldexp (denormals preserved) and placed
// against the grid midpoints; a midpoint goes to its even neighbour.
__device__ __forceinline__ uint32_t e2m1_code(float y, int sb) {
  uint32_t sign = (__float_as_uint(y) >> 31) << 3;
  float z = __builtin_ldexpf(__builtin_fabsf(y), 127 - sb);
  uint32_t c = (z > 0.25f) + (z >= 0.75f) + (z > 1.25f) + (z >= 1.75f) + (z > 2.5f) +
               (z >= 3.5f) + (z > 5.0f);
  return c | sign;
}

// Exact value of a 4-bit code under scale byte sb: the E2M1 magnitude built
// as fp32 bits (0, 0.5, or 2^(e-1) (1 + m/2) for exponent field e >= 1)
// times 2^(sb-127) through ldexp, which is exact here because subnormal
// results are kept.
__device__ __forceinline__ float e2m1_value(uint32_t code, int sb) {
  const uint32_t c3 = code & 7u;
  const uint32_t bits = c3 == 0 ? 0u : (c3 == 1 ? (126u << 23) : (((126u + (c3 >> 1)) << 23) | ((c3 & 1u) << 22)));
  const float mag = __builtin_ldexpf(__uint_as_float(bits), sb - 127);
  return (code & 8u) ? -mag : mag;
}

// Scaled FP4 x FP4 MFMAs (E2M1 both sides, one E8M0 scale per lane held in
// byte 0 of the scale operand).
__device__ __forceinline__ v16f mfma32_fp4(v4i a, v4i b, v16f c, int sa, int sb) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, sa, 0, sb);
}

// As mfma32_fp4, with the A scale taken from byte `sel` (0..3, a constant
// after inlining) of the 32-bit word sa4 by the instruction's operand select.
__device__ __forceinline__ v16f mfma32_fp4_sel(v4i a, v4i b, v16f c, int sa4, int sel, int sb) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, sa4, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 1, sa4, 0, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 2, sa4, 0, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 3, sa4, 0, sb);
  }
}

__device__ __forceinline__ v4f mfma16_fp4(v4i a, v4i b, v4f c, int sa, int sb) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 4, 4, 0, sa, 0, sb);
}

// Hardware exp2 (v_exp_f32); results below 2^-126 flush to 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^(byte-127) as an fp32 scale for the convert instructions (byte >= 1).
__device__ __forceinline__ float scale_of_byte(int b) { return __uint_as_float(static_cast<uint32_t>(b) << 23); }

// Eight elements to eight packed E2M1 codes (element i in nibble i) under
// scale byte sb.  From byte 3 up the hardware convert does it: it rounds
// y/2^e to nearest even on the E2M1 grid, saturates and keeps the sign, and
// every fp32 subnormal element lands below 0.25 and codes to signed zero
// whatever the convert's denormal handling.  Bytes 0..2 take the
// integer-exact encoder.
__device__ __forceinline__ uint32_t encode8(const float* y, int sb) {
  uint32_t packed = 0;
  if (sb >= 3) {
    const float scl = scale_of_byte(sb);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[0], y[1], scl, 0);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[2], y[3], scl, 1);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[4], y[5], scl, 2);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[6], y[7], scl, 3);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= e2m1_code(y[i], sb) << (4 * i);
  }
  return packed;
}

}  // namespace mxattn
