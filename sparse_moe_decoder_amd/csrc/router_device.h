// Small-batch FP32 router dot products, shared by the stand-alone router kernel and
// the fused small-batch routing kernel so both sum in the same order.
//
// [vLLM "Serving Reflection Beam auf vLLM ab Tag 0", §MoE und Residual-Stream]
//   router weights (5120 x 256), accumulation and logits are FP32.
#pragma once
#include "common.h"
#include "kernels.h"

namespace beam {

constexpr int kRouterRT = 16;  // tokens per workgroup
static_assert(kFusedRouteMaxT <= kRouterRT, "the fused router covers its batch in one block");

// Per-lane partial logits of expert e for TT token slots (tokens t0 .. t0 + nt - 1,
// nt <= TT): lane walks the 4-float chunks c = lane, lane + 64, ... of its wave's
// quarter of d, in that order, adding the four products of a chunk in index order.
// Loads are issued UNR chunks at a time from valid addresses (slots past nt read
// token t0's row, chunks past the quarter read chunk 0) and only real terms are
// accumulated, so the sums are the plain in-order ones.
template <int TT, int UNR>
__device__ __forceinline__ void router_lane_partials(const RouterArgs& a, int e, int t0, int nt,
                                                     float (&acc)[TT]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nch = a.d >> 2, per = nch >> 2;  // 4-float chunks; d % 256 == 0
  const f32x4* wr = (const f32x4*)(a.W + (int64_t)e * a.d) + wv * per;
  const uint16_t* zq = a.z + (int64_t)t0 * a.d + 4 * wv * per;
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
  const int iters = (per + 63) >> 6;
  for (int i0 = 0; i0 < iters; i0 += UNR) {
    f32x4 w[UNR];
    uint2 zz[UNR][TT];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int c = lane + 64 * (i0 + u);
      const int cc = c < per ? c : 0;
      w[u] = wr[cc];
#pragma unroll
      for (int t = 0; t < TT; ++t)
        zz[u][t] = *(const uint2*)(zq + (int64_t)(t < nt ? t : 0) * a.d + 4 * cc);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      if (lane + 64 * (i0 + u) < per) {
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          if (t < nt) {
            acc[t] += lo_bf(zz[u][t].x) * w[u][0];
            acc[t] += hi_bf(zz[u][t].x) * w[u][1];
            acc[t] += lo_bf(zz[u][t].y) * w[u][2];
            acc[t] += hi_bf(zz[u][t].y) * w[u][3];
          }
        }
      }
    }
  }
}

// Logits of expert e for tokens t0 .. t0 + nt - 1 (nt <= TT) by a workgroup of four
// waves that split d into four contiguous quarters: each lane's in-order partial
// (above) is summed across the wave, and the four quarter sums are added in wave
// order. Returns token t0 + t's logit in lane t of wave 0 (t < nt); other lanes
// return 0. `part` is LDS [3][kRouterRT].
template <int TT, int UNR>
__device__ __forceinline__ float router_small_dot_t(const RouterArgs& a, int e, int t0, int nt,
                                                    float (*part)[kRouterRT]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  float acc[TT];
  router_lane_partials<TT, UNR>(a, e, t0, nt, acc);
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    if (t < nt) {
      const float v = wave_sum(acc[t]);
      if (wv > 0 && lane == 0) part[wv - 1][t] = v;
      acc[t] = v;
    }
  }
  __syncthreads();
  float v = 0.0f;
  if (wv == 0 && lane < nt) {
#pragma unroll
    for (int t = 0; t < TT; ++t)
      if (t == lane) v = acc[t];
    v = ((v + part[0][lane]) + part[1][lane]) + part[2][lane];
  }
  return v;
}

// One token, with the weights already in registers and z in LDS. d <= 8192: each
// wave's quarter has at most 8 chunks per lane. The lane's terms, the wave sum and
// the quarter sums are formed in the order of router_small_dot, so the logit is
// bit-identical to it.
constexpr int kRouterPreChunks = 8;

// Expert e's weight chunks of this lane (chunks past the quarter read chunk 0).
__device__ __forceinline__ void router_load_w(const RouterArgs& a, int e, f32x4 (&w)[kRouterPreChunks]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int per = (a.d >> 2) >> 2;
  const f32x4* wr = (const f32x4*)(a.W + (int64_t)e * a.d) + wv * per;
#pragma unroll
  for (int i = 0; i < kRouterPreChunks; ++i) {
    const int c = lane + 64 * i;
    w[i] = wr[c < per ? c : 0];
  }
}

__device__ __forceinline__ float router_dot_1_lds(const RouterArgs& a, const f32x4 (&w)[kRouterPreChunks],
                                                  const uint16_t* zl, float (*part)[kRouterRT]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int per = (a.d >> 2) >> 2;
  const uint16_t* zq = zl + 4 * wv * per;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < kRouterPreChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < per) {
      const uint2 zz = *(const uint2*)(zq + 4 * c);
      acc += lo_bf(zz.x) * w[i][0];
      acc += hi_bf(zz.x) * w[i][1];
      acc += lo_bf(zz.y) * w[i][2];
      acc += hi_bf(zz.y) * w[i][3];
    }
  }
  float v = wave_sum(acc);
  if (wv > 0 && lane == 0) part[wv - 1][0] = v;
  __syncthreads();
  if (wv == 0 && lane == 0) return ((v + part[0][0]) + part[1][0]) + part[2][0];
  return 0.0f;
}

// nt <= kRouterRT tokens; the token-slot count is the next power of two >= nt.
__device__ __forceinline__ float router_small_dot(const RouterArgs& a, int e, int t0, int nt,
                                                  float (*part)[kRouterRT]) {
  if (nt <= 1) return router_small_dot_t<1, 8>(a, e, t0, nt, part);
  if (nt <= 2) return router_small_dot_t<2, 8>(a, e, t0, nt, part);
  if (nt <= 4) return router_small_dot_t<4, 4>(a, e, t0, nt, part);
  if (nt <= 8) return router_small_dot_t<8, 2>(a, e, t0, nt, part);
  return router_small_dot_t<16, 1>(a, e, t0, nt, part);
}

}  // namespace beam
