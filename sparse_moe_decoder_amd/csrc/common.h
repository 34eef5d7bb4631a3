// Shared device helpers for the Beam MoE kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kWave = 64;

// BF16 <-> FP32. Widening is exact; narrowing is the hardware round-to-nearest-even
// conversion (v_cvt_pk_bf16_f32), which keeps NaN quiet.
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// Butterfly sum over the 64 lanes. Every step adds the same two values in
// every lane that uses them (a + b and b + a), so all lanes end with the
// bitwise-identical total. Steps 1, 2 use DPP quad permutes, 4 and 8 DPP row
// half-mirror / mirror (lane i <-> 7-i, 15-i within a row), 16 and 32 swizzle.
__device__ __forceinline__ float dpp_quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_half_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = v + dpp_quad_xor1(v);
  v = v + dpp_quad_xor2(v);
  v = v + dpp_half_mirror(v);
  v = v + dpp_mirror(v);
  v = v + __shfl_xor(v, 16, 64);
  v = v + __shfl_xor(v, 32, 64);
  return v;
}

// 64-bit max over the wave, returned wave-uniform. Max is associative and
// commutative, so the reduction order does not matter: DPP moves (quad
// permutes, row half-mirror, row mirror) give every lane its row's maximum, then
// the four row maxima are read into scalar registers and compared there.
// Wave-wide maximum of a uint32, identical in every lane: DPP max within each row
// of 16 lanes, then the four row results through SGPRs.
__device__ __forceinline__ uint32_t max_u32(uint32_t a, uint32_t b) { return a > b ? a : b; }
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max_u32(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max_u32(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max_u32(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = max_u32(v, dpp_u32<0x140>(v));  // row_mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max_u32(max_u32(r0, r1), max_u32(r2, r3));
}

// Lowest lane whose predicate holds (the predicate must hold somewhere).
__device__ __forceinline__ int first_lane(bool pred) {
  return __builtin_ctzll((unsigned long long)__ballot(pred));
}

// Number of lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Order-preserving map of a finite FP32 value to uint32 (larger value -> larger key).
// -0.0 is folded onto +0.0 first so the two compare equal, as in FP compares.
__device__ __forceinline__ uint32_t f32_order_key(float v) {
  v = v + 0.0f;
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ u32x4 ld_u32x4(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void st_u32x4(void* p, u32x4 v) { *(u32x4*)p = v; }

// Streaming 16-byte load: weights are read once per call, so hint the caches
// not to keep them (non-temporal).
__device__ __forceinline__ u32x4 ld_stream_u32x4(const void* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

// Buffer loads: a raw buffer resource over `bytes` bytes from `base` (gfx9-family
// resource word); a 16-byte load at a byte offset at or past `bytes` returns zeros
// without touching memory, so rows that do not exist can issue the same
// instruction as rows that do.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ u32x4 ld_buf_u32x4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16: lane l holds A[l % 32][8*(l/32) .. +7],
// B[8*(l/32) .. +7][l % 32] and D[8*(r/4) + 4*(l/32) + r%4][l % 32] in register r.
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// silu(v) = v / (1 + e^-v) in FP32, with the hardware exp2 (v_exp_f32) and reciprocal
// (v_rcp_f32): a few ulp of FP32, far below the BF16 rounding of silu(g) * u that follows,
// and five instructions where expf and an IEEE division take about twenty-five (the SiLU of
// a grouped-GEMM tile otherwise holds the matrix cores idle for 3-8 % of the gate/up time)
__device__ __forceinline__ float silu(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * -1.4426950408889634f));
}

}  // namespace beam
