// FP32 router logits and grouped top-k routing.
//
// [vLLM "Serving Reflection Beam auf vLLM ab Tag 0", §MoE und Residual-Stream]
//   routing as in DeepSeek-V3: sigmoid scores plus a correction bias select the
//   best 4 of 8 expert groups, then the top 8 experts; renormalised weights are
//   scaled by 2.5. Router weights (5120 x 256), accumulation and logits are FP32.
// [SGLang "SGLang 支撑编程模型 Beam 生产部署", §稠密层与分组 MoE 路由]
//   FP32 logits, grouped top-k over sigmoid scores and the correction bias,
//   FP32 routing coefficients, scale folded into the weights.
#include "common.h"
#include "kernels.h"
#include "topk_device.h"

namespace beam {

// ---------------------------------------------------------------------------------------------
// Router logits, FP32 on the vector ALUs: logits[t, e] = sum_i z[t, i] * W[e, i].
// One wavefront per (expert, block of RT tokens): each lane walks 16-byte chunks
// of W's row (chunk c -> lane c % 64) and keeps one FP32 partial per token; the
// partials are then summed across the wave. W's row is read once per token block.
constexpr int RT = 16;

__global__ __launch_bounds__(256) void router_fp32_kernel(RouterArgs a) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t0 = blockIdx.y * RT;
  if (e >= a.E) return;
  const int nt = min(RT, a.T - t0);
  const int nch = a.d >> 2;  // 4-float chunks
  const f32x4* wr = (const f32x4*)(a.W + (int64_t)e * a.d);
  float acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = 0.0f;
  for (int c = lane; c < nch; c += 64) {
    f32x4 w = *(wr + c);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      if (t < nt) {
        const uint2 zz = *(const uint2*)(a.z + (int64_t)(t0 + t) * a.d + 4 * c);
        acc[t] += lo_bf(zz.x) * w[0];
        acc[t] += hi_bf(zz.x) * w[1];
        acc[t] += lo_bf(zz.y) * w[2];
        acc[t] += hi_bf(zz.y) * w[3];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    if (t < nt) {
      float v = wave_sum(acc[t]);
      if (lane == 0) a.logits[(int64_t)(t0 + t) * a.E + e] = v;
    }
  }
}

// Small batches: one workgroup per (expert, block of RT tokens); its four waves
// split d, so a W row is fetched by 256 lanes at once. Partials from the four
// waves are added in wave order.
__global__ __launch_bounds__(256) void router_fp32_small_kernel(RouterArgs a) {
  __shared__ float part[3][RT];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * RT;
  const int nt = min(RT, a.T - t0);
  const int nch = a.d >> 2, per = nch >> 2;  // 4-float chunks; d % 256 == 0
  const f32x4* wr = (const f32x4*)(a.W + (int64_t)e * a.d) + wv * per;
  float acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = 0.0f;
  for (int c = lane; c < per; c += 64) {
    f32x4 w = *(wr + c);
    const int col = 4 * (wv * per + c);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      if (t < nt) {
        const uint2 zz = *(const uint2*)(a.z + (int64_t)(t0 + t) * a.d + col);
        acc[t] += lo_bf(zz.x) * w[0];
        acc[t] += hi_bf(zz.x) * w[1];
        acc[t] += lo_bf(zz.y) * w[2];
        acc[t] += hi_bf(zz.y) * w[3];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    if (t < nt) {
      float v = wave_sum(acc[t]);
      if (wv > 0 && lane == 0) part[wv - 1][t] = v;
      acc[t] = v;
    }
  }
  __syncthreads();
  if (wv == 0 && lane < nt) {
    float v = 0.0f;
#pragma unroll
    for (int t = 0; t < RT; ++t)
      if (t == lane) v = acc[t];
    v = ((v + part[0][lane]) + part[1][lane]) + part[2][lane];
    a.logits[(int64_t)(t0 + lane) * a.E + e] = v;
  }
}

hipError_t launch_router_fp32(const RouterArgs& a, hipStream_t s) {
  if (a.T <= kStreamMaxT) {
    dim3 grid((unsigned)a.E, (unsigned)((a.T + RT - 1) / RT));
    hipLaunchKernelGGL(router_fp32_small_kernel, grid, dim3(256), 0, s, a);
  } else {
    dim3 grid((unsigned)((a.E + 3) / 4), (unsigned)((a.T + RT - 1) / RT));
    hipLaunchKernelGGL(router_fp32_kernel, grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Grouped top-k: one wavefront per token.
//   s = sigmoid(logit) (double, rounded once to FP32), c = s + bias
//   group score = sum of the two largest c of the group (the c itself if E/G = 1)
//   keep kg groups, then k experts, each by (value desc, index asc)
//   w_j = (s_j / den) * scale, den summed over the slots in order
// Selection uses 64-bit keys (order-preserving value bits << 32 | ~index), so one
// wave max picks the winner and breaks ties toward the lower index.
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  __shared__ float s_lds[4][256];
  __shared__ float c_lds[4][256];
  __shared__ int32_t sel_ids[4][32];
  const int wv = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wv;
  if (t >= a.T) return;
  topk_token(a, t, s_lds[wv], c_lds[wv], sel_ids[wv], threadIdx.x & 63);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace beam
