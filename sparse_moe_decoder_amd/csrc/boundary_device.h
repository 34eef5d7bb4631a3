// Sublayer boundary arithmetic shared by the boundary kernels and the fused
// single-token routing kernel, so both produce the same bits.
//
// [vLLM "Serving Reflection Beam auf vLLM ab Tag 0", §MoE und Residual-Stream]
//   sandwich norm; the n-th residual add is h <- sqrt((n-1)/n) h + x / sqrt(n).
// [same page, §Agentengetriebene Optimierung, change 1] post-norm, scaled add and
//   next pre-norm as one kernel with FP32 math and BF16 rounding points.
// [SGLang "SGLang 支撑编程模型 Beam 生产部署", §三明治归一化与深度缩放残差]
//   both scaled operands are rounded to BF16 before the add.
#pragma once
#include "common.h"
#include "kernels.h"

namespace beam {

__device__ __forceinline__ float sumsq8(const u32x4& v) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = lo_bf(v[i]), b = hi_bf(v[i]);
    s += a * a;
    s += b * b;
  }
  return s;
}

// (v * r) * w, rounded, for 8 packed values
__device__ __forceinline__ u32x4 norm8(const u32x4& v, float r, const u32x4& w) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = pack_bf2((lo_bf(v[i]) * r) * lo_bf(w[i]), (hi_bf(v[i]) * r) * hi_bf(w[i]));
  return o;
}

// h' = bf16(bf16(c1 h) + bf16(c2 xn)) for 8 packed values; accumulates sum of h'^2
__device__ __forceinline__ u32x4 residual8(const u32x4& h, const u32x4& xn, float c1, float c2,
                                           float& ss) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a0 = bf2f(f2bf(c1 * lo_bf(h[i]))), a1 = bf2f(f2bf(c1 * hi_bf(h[i])));
    float b0 = bf2f(f2bf(c2 * lo_bf(xn[i]))), b1 = bf2f(f2bf(c2 * hi_bf(xn[i])));
    float s0 = bf2f(f2bf(a0 + b0)), s1 = bf2f(f2bf(a1 + b1));
    ss += s0 * s0;
    ss += s1 * s1;
    o[i] = (uint32_t)f2bf(s0) | ((uint32_t)f2bf(s1) << 16);
  }
  return o;
}

__device__ __forceinline__ float rms_scale(float ss, int d, float eps) {
  return 1.0f / sqrtf(ss / (float)d + eps);
}

// One token row of width d <= kBoundaryWgMaxD by a workgroup of FOUR waves, in
// exactly the arithmetic order of boundary_row_wg_kernel (one 16-byte chunk per
// lane, nv = ceil(d / 512) waves): chunk idx = 64 v + lane belongs to that kernel's
// wave v, here handled by wave v % 4 as its (v / 4)-th "virtual wave". Each virtual
// wave forms the same wave sums, and the nv sums are added in wave order, so h' and
// z are bit-identical to that kernel's. Split in two so a caller can put other loads
// in flight between them: boundary_row_4waves_load issues the row's loads (chunk j of
// virtual wave 4 j + wave), boundary_row_4waves_finish forms z into zl (LDS, d values)
// and, when z_out is not null, z_out, leaving the lane's h' chunks in hv.
struct BoundaryRow4 {
  u32x4 xv[4], hv[4], wo[4], wr[4];
};

__device__ __forceinline__ void boundary_row_4waves_load(const BoundaryArgs& a, int64_t t,
                                                         BoundaryRow4& b) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nch = a.d >> 3, nv = (nch + 63) >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int v = wv + 4 * j, idx = 64 * v + lane;
    const int li = idx < nch ? idx : 0;
    if (v < nv) {
      b.xv[j] = ld_u32x4((const u32x4*)(a.x + t * a.d) + li);
      b.hv[j] = ld_u32x4((const u32x4*)(a.h + t * a.d) + li);
      b.wo[j] = ld_u32x4((const u32x4*)a.w_post + li);
      b.wr[j] = ld_u32x4((const u32x4*)a.w_pre + li);
    }
  }
}

// `red` is LDS [2][16]
__device__ __forceinline__ void boundary_row_4waves_finish(const BoundaryArgs& a, int64_t t,
                                                           BoundaryRow4& b, uint16_t* zl,
                                                           uint16_t* z_out, float (*red)[16]) {
  const int lane = threadIdx.x & 63;
  // wave-uniform (scalar branches keep the load counters exact for loads still in flight)
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nch = a.d >> 3, nv = (nch + 63) >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int v = wv + 4 * j, idx = 64 * v + lane;
    if (v < nv) {
      const float s = wave_sum(idx < nch ? sumsq8(b.xv[j]) : 0.0f);
      if (lane == 0) red[0][v] = s;
    }
  }
  __syncthreads();
  float ss = 0.0f;
  for (int w = 0; w < nv; ++w) ss += red[0][w];
  const float r = rms_scale(ss, a.d, a.eps);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int v = wv + 4 * j, idx = 64 * v + lane;
    if (v < nv) {
      float ss2 = 0.0f;
      const u32x4 xn = norm8(b.xv[j], r, b.wo[j]);
      b.hv[j] = residual8(b.hv[j], xn, a.c1, a.c2, ss2);
      const float s = wave_sum(idx < nch ? ss2 : 0.0f);
      if (lane == 0) red[1][v] = s;
    }
  }
  __syncthreads();
  float ss2 = 0.0f;
  for (int w = 0; w < nv; ++w) ss2 += red[1][w];
  const float r2 = rms_scale(ss2, a.d, a.eps);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int v = wv + 4 * j, idx = 64 * v + lane;
    if (v < nv && idx < nch) {
      const u32x4 zc = norm8(b.hv[j], r2, b.wr[j]);
      *((u32x4*)zl + idx) = zc;
      if (z_out) st_u32x4((u32x4*)(z_out + t * a.d) + idx, zc);
    }
  }
  __syncthreads();
}

// The lane's h' chunks (from boundary_row_4waves_finish) to h_out
__device__ __forceinline__ void boundary_row_4waves_store_h(const BoundaryArgs& a, int64_t t,
                                                            const BoundaryRow4& b) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nch = a.d >> 3, nv = (nch + 63) >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int v = wv + 4 * j, idx = 64 * v + lane;
    if (v < nv && idx < nch) st_u32x4((u32x4*)(a.h_out + t * a.d) + idx, b.hv[j]);
  }
}

}  // namespace beam
