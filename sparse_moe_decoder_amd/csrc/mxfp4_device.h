// MXFP4 device helpers shared by the 4-bit weight-streaming kernels and the 4-bit
// grouped GEMM: E2M1 codes (element 2i in the low nibble of byte i) with one E8M0
// scale 2^(s - 127) per 32 values (OCP Microscaling Formats specification v1.0).
#pragma once
#include "common.h"

namespace beam {

// 2^(s - 127) as an FP32 multiplier (s = 0 is 2^-127, a subnormal; s = 255, the
// E8M0 NaN, is never produced by the quantiser)
__device__ __forceinline__ float e8m0_scale(uint32_t s) {
  return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

// Eight codes (one dword) times the scale: the BF16 operand fragment, element i in
// half-word i. v_cvt_scalef32_pk_bf16_fp4 converts the code pair of one byte; every
// E2M1 value times a power of two is a BF16 number, so the result is exact.
__device__ __forceinline__ u32x4 fp4x8_to_bf16(uint32_t codes, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
  return r;
}

}  // namespace beam
