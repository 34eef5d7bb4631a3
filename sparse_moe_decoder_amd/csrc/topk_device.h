// Grouped top-k for one token, executed by one wavefront (device code shared by
// the stand-alone routing kernel and the fused small-batch routing kernel).
//
// [vLLM "Serving Reflection Beam auf vLLM ab Tag 0", §MoE und Residual-Stream]
//   sigmoid scores plus a correction bias select the best 4 of 8 expert groups,
//   then the top 8 experts; the renormalised weights are scaled by 2.5.
// [SGLang "SGLang 支撑编程模型 Beam 生产部署", §稠密层与分组 MoE 路由]
//   FP32 routing coefficients; the scale may be folded into the weights.
//
//   s = sigmoid(logit) (double, rounded once to FP32), c = s + bias
//   group score = sum of the two largest c of the group (the c itself if E/G = 1)
//   keep kg groups, then k experts, each by (value desc, index asc)
//   w_j = (s_j / den) * scale, den summed over the slots in order
// Selection uses 64-bit keys (order-preserving value bits << 32 | ~index), so one
// wave max picks the winner and breaks ties toward the lower index.
#pragma once
#include "common.h"
#include "kernels.h"

namespace beam {

__device__ __forceinline__ uint64_t make_key(float v, int idx) {
  return ((uint64_t)f32_order_key(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// s, c: this wave's E-entry LDS scratch; sel: its k-entry LDS scratch. Writes
// ids/w (and the optional copies) for token t; leaves the selected ids in sel.
__device__ __forceinline__ void topk_token(const TopkArgs& a, int64_t t, float* s, float* c,
                                           int32_t* sel, int lane) {
  const int E = a.E, G = a.G, gs = E / G;
  for (int e = lane; e < E; e += 64) {
    float l = a.logits[t * E + e];
    float sv = (float)(1.0 / (1.0 + exp(-(double)l)));
    s[e] = sv;
    c[e] = sv + a.bias[e];
  }
  wave_lds_sync();
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
    kept |= 1ull << (j & 63);
    if (lane == j) gkey = 0;
  }
  // candidate keys: each lane owns experts lane, lane + 64, lane + 128, lane + 192
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
    if (lane == 0) sel[j] = e;
  }
  wave_lds_sync();
  // denominator in slot order (every lane computes the same sequential sum)
  float den = 0.0f;
  for (int j = 0; j < a.k; ++j) {
    float sj = s[sel[j]];
    den = (j == 0) ? sj : den + sj;
  }
  if (lane < a.k) {
    int e = sel[lane];
    float wj = (s[e] / den) * a.scale;
    a.ids[t * a.k + lane] = e;
    a.w[t * a.k + lane] = wj;
    if (a.ids2) a.ids2[t * a.k + lane] = e;
    if (a.w2) a.w2[t * a.k + lane] = wj;
  }
  wave_lds_sync();
}

}  // namespace beam
