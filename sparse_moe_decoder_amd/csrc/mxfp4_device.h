// MXFP4 device helpers shared by the 4-bit weight-streaming kernels and the 4-bit
// grouped GEMM: E2M1 codes (element 2i in the low nibble of byte i) with one E8M0
// scale 2^(s - 127) per 32 values (OCP Microscaling Formats specification v1.0).
#pragma once
#include "common.h"

namespace beam {

// The scale operand of v_cvt_scalef32_pk_bf16_fp4 for E8M0 byte s (2^(s - 127)): the
// byte in the FP32 exponent field. The instruction takes the scale from that field alone,
// so s = 0 (0.0 here) converts as 2^-127 — on gfx950 every code pair converts to the same
// bits with this operand as with the exact multiplier (the subnormal 2^-127 for s = 0),
// for every s in 0 .. 254. s = 255, the E8M0 NaN, is never produced by the quantiser.
// Only for the conversion instructions: not an FP32 multiplier for s = 0.
__device__ __forceinline__ float e8m0_scale(uint32_t s) { return __uint_as_float(s << 23); }

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
// The largest magnitude (BF16 bits without the sign) of eight values
__device__ __forceinline__ uint32_t bf16x8_amax(const u32x4& v) {
  uint32_t amax = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) amax = max_u32(amax, max_u32(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
  return amax;
}

// The scale byte X + 127 of a block whose largest magnitude has BF16 bits amax
__device__ __forceinline__ uint32_t mxfp4_scale_byte(uint32_t amax) {
  const int ex = (int)(amax >> 7);  // BF16 exponent field (< 255: finite)
  return (uint32_t)(ex > 2 ? ex - 2 : 0);
}

// Eight values (half-word e of v is element e) to their codes with scale byte sbyte:
// element e in nibble e. v_cvt_scalef32_pk_fp4_f32 divides two FP32 values by its scale
// operand and rounds each quotient to E2M1 with ties to the even code and saturation at 6,
// the sign kept (the first value in the low nibble of the selected byte, the other bytes
// kept): on gfx950 it gives exactly the codes of the rule above for every finite BF16 value
// and every scale exponent X in [-127, 127] when the operand is 2^X (checked exhaustively,
// 2^-127 passed as the subnormal), so one instruction per pair replaces seven comparisons
// per value. The pairs are unpacked to FP32 explicitly: the packed-BF16 form of the
// instruction, fed from elements of a vector, was compiled with one source register for all
// four byte positions.
__device__ __forceinline__ uint32_t mxfp4_codes8(const u32x4& v, uint32_t sbyte) {
  const float sc = __uint_as_float(sbyte ? (sbyte << 23) : 0x00400000u);  // 2^X exactly
  uint32_t out = 0;
#define BEAM_FP4_PAIR(j)                                                                   \
  out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(v[j] << 16),        \
                                                 __uint_as_float(v[j] & 0xFFFF0000u), sc, j)
  BEAM_FP4_PAIR(0);
  BEAM_FP4_PAIR(1);
  BEAM_FP4_PAIR(2);
  BEAM_FP4_PAIR(3);
#undef BEAM_FP4_PAIR
  return out;
}

__device__ __forceinline__ uint32_t mxfp4_quantize32(const u32x4 v[4], u32x4& out) {
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) amax = max_u32(amax, bf16x8_amax(v[i]));
  const uint32_t sbyte = mxfp4_scale_byte(amax);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = mxfp4_codes8(v[i], sbyte);
  return sbyte;
}

// Block codes in natural order (dword q = K values 8 q ..) -> the order the scaled FP4
// matrix-core kernels read them in ("GEMM order"): dword p holds K values 8 q .. 8 q + 7
// with q = (0, 2, 1, 3)[p]
__device__ __forceinline__ u32x4 gemm_order(u32x4 c) { return u32x4{c[0], c[2], c[1], c[3]}; }

// The exact BF16 values of one block's codes (natural order) and scale byte: v[i] holds
// elements 8 i .. 8 i + 7 (every E2M1 value times a power of two is a BF16 number).
__device__ __forceinline__ void mxfp4_dequantize32(const u32x4& codes, uint32_t sbyte, u32x4 v[4]) {
  const float sc = e8m0_scale(sbyte);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = fp4x8_to_bf16(codes[i], sc);
}

// One block of 32 BF16 values (v, replaced by its round trip when rt is not null) to its
// codes (16 bytes at codes, GEMM order), its scale byte (at scale) and, with rt, its round
// trip (32 BF16 values at rt).
__device__ __forceinline__ void mxfp4_block_out(u32x4 v[4], uint8_t* codes, uint8_t* scale,
                                                uint16_t* rt) {
  u32x4 out;
  const uint32_t sbyte = mxfp4_quantize32(v, out);
  st_u32x4(codes, gemm_order(out));
  *scale = (uint8_t)sbyte;
  if (rt) {
    mxfp4_dequantize32(out, sbyte, v);
#pragma unroll
    for (int i = 0; i < 4; ++i) st_u32x4(rt + i * 8, v[i]);
  }
}

// One block of 32 BF16 values held by four consecutive lanes (lane 4 j + q holds elements
// 8 q .. 8 q + 7 in v): this lane's eight values of the block's round trip; with keep, also
// the block's codes (16 bytes at codes, GEMM order) and scale byte (at scale), which every
// lane of the four passes. The four lanes must be active together.
__device__ __forceinline__ u32x4 mxfp4_block_rt_4lanes(const u32x4& v, uint8_t* codes,
                                                      uint8_t* scale, bool keep) {
  const int q = threadIdx.x & 3;
  uint32_t amax = bf16x8_amax(v);
  amax = max_u32(amax, dpp_u32<0xB1>(amax));  // the four lanes are a DPP quad: quad_perm [1,0,3,2]
  amax = max_u32(amax, dpp_u32<0x4E>(amax));  // quad_perm [2,3,0,1]
  const uint32_t sbyte = mxfp4_scale_byte(amax);
  const uint32_t c = mxfp4_codes8(v, sbyte);
  if (keep) {
    reinterpret_cast<uint32_t*>(codes)[q == 1 ? 2 : q == 2 ? 1 : q] = c;  // GEMM order
    if (q == 0) *scale = (uint8_t)sbyte;
  }
  return fp4x8_to_bf16(c, e8m0_scale(sbyte));
}

// The same block with its codes, scale and round trip (32 BF16 values at rt) written out.
__device__ __forceinline__ void mxfp4_block_out_4lanes(const u32x4& v, uint8_t* codes,
                                                       uint8_t* scale, uint16_t* rt) {
  st_u32x4(rt + 8 * (threadIdx.x & 3), mxfp4_block_rt_4lanes(v, codes, scale, true));
}

}  // namespace beam
