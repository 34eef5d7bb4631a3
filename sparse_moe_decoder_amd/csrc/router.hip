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

hipError_t launch_router_fp32(const RouterArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.E + 3) / 4), (unsigned)((a.T + RT - 1) / RT));
  hipLaunchKernelGGL(router_fp32_kernel, grid, dim3(256), 0, s, a);
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
__device__ __forceinline__ uint64_t make_key(float v, int idx) {
  return ((uint64_t)f32_order_key(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}

__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  __shared__ float s_lds[4][256];
  __shared__ float c_lds[4][256];
  __shared__ int32_t sel_ids[4][32];
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + wv;
  if (t >= a.T) return;
  const int E = a.E, G = a.G, gs = E / G;
  float* s = s_lds[wv];
  float* c = c_lds[wv];
  for (int e = lane; e < E; e += 64) {
    float l = a.logits[t * E + e];
    float sv = (float)(1.0 / (1.0 + exp(-(double)l)));
    s[e] = sv;
    c[e] = sv + a.bias[e];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // group scores: lane j < G scans its group
  uint64_t gkey = 0;
  if (lane < G) {
    float m1 = -INFINITY, m2 = -INFINITY;
    for (int q = 0; q < gs; ++q) {
      float v = c[lane * gs + q];
      if (v > m1) {
        m2 = m1;
        m1 = v;
      } else if (v > m2) {
        m2 = v;
      }
    }
    gkey = make_key(gs >= 2 ? m1 + m2 : m1, lane);
  }
  // keep the kg best groups
  uint64_t kept = 0;  // bit j set: group j kept
  for (int r = 0; r < a.kg; ++r) {
    uint64_t best = wave_max_u64(gkey);
    int j = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
    kept |= 1ull << j;
    if (lane == j) gkey = 0;
  }
  // candidate keys: each lane owns experts lane, lane + 64, ...
  uint64_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = lane + 64 * i;
    key[i] = (e < E && ((kept >> (e / gs)) & 1)) ? make_key(c[e], e) : 0;
  }
  for (int j = 0; j < a.k; ++j) {
    uint64_t m = key[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) m = key[i] > m ? key[i] : m;
    uint64_t best = wave_max_u64(m);
    int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (key[i] == best) key[i] = 0;
    if (lane == 0) sel_ids[wv][j] = e;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // denominator in slot order (every lane computes the same sequential sum)
  float den = 0.0f;
  for (int j = 0; j < a.k; ++j) {
    float sj = s[sel_ids[wv][j]];
    den = (j == 0) ? sj : den + sj;
  }
  if (lane < a.k) {
    int e = sel_ids[wv][lane];
    float wj = (s[e] / den) * a.scale;
    a.ids[t * a.k + lane] = e;
    a.w[t * a.k + lane] = wj;
    if (a.ids2) a.ids2[t * a.k + lane] = e;
    if (a.w2) a.w2[t * a.k + lane] = wj;
  }
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace beam
