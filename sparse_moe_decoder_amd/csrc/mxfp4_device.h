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

// MXFP4 quantisation of one block of 32 BF16 values (v[i] holds elements 8 i .. 8 i + 7,
// element e in half-word e % 8) by the OCP MX v1.0 rule; returns the scale byte X + 127
// and the codes in out (element e in nibble e % 8 of dword e / 8).
//   X = floor(log2 max|v|) - 2, clamped to [-127, 127]: for a BF16 maximum with
//   exponent field ex (0 for zero and subnormals), X = max(ex - 129, -127), so the
//   stored scale is max(ex - 2, 0).
//   q = |v| * 2^-X (exact: a power-of-two scaling, q < 8) is rounded to the nearest
//   E2M1 magnitude with ties to the even code and saturation at 6: the code counts
//   the decision points q passes, strictly past a point where the lower neighbour
//   has the even code (0.25, 1.25, 2.5, 5) and from the point on where the upper one
//   has it (0.75, 1.75, 3.5). The sign bit is the input's.
__device__ __forceinline__ uint32_t mxfp4_quantize32(const u32x4 v[4], u32x4& out) {
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = v[i][j];
      amax = max_u32(amax, max_u32(w & 0x7FFFu, (w >> 16) & 0x7FFFu));
    }
  const int ex = (int)(amax >> 7);                      // BF16 exponent field (< 255: finite)
  const int sbyte = ex > 2 ? ex - 2 : 0;                // X + 127
  const float inv = __uint_as_float((uint32_t)(254 - sbyte) << 23);  // 2^-X
  out = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint32_t bits = hh ? (v[i][j] >> 16) : (v[i][j] & 0xFFFFu);
        const float q = __uint_as_float((bits & 0x7FFFu) << 16) * inv;
        const uint32_t m = (q > 0.25f) + (q >= 0.75f) + (q > 1.25f) + (q >= 1.75f) +
                           (q > 2.5f) + (q >= 3.5f) + (q > 5.0f);
        const uint32_t code = m | ((bits >> 12) & 8u);
        const int e = i * 8 + j * 2 + hh;  // element of the block
        out[e >> 3] |= code << (4 * (e & 7));
      }
  return (uint32_t)sbyte;
}

}  // namespace beam
