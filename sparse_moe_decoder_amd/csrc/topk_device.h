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

// Token t's grouped top-k by one wavefront, in registers: lane l holds experts
// 4l .. 4l+3 (E <= 256). A group of gs experts spans gs/4 lanes when gs is a
// multiple of 4 and gs/4 a power of two up to 16 (then the group's two largest
// biased scores are merged across its lanes with shuffles); other group sizes go
// through LDS scratch `c_lds` (E floats). Selected ids land in sel[0..k) (LDS) and
// in ids/w (and the optional copies).
__device__ __forceinline__ void top2_merge(float& m1, float& m2, float o1, float o2) {
  const float hi = fmaxf(m1, o1), lo = fminf(m1, o1);
  m2 = fmaxf(lo, fmaxf(m2, o2));
  m1 = hi;
}

// COHERENT: read the logits with device-coherent loads (they were published within
// the same launch by other workgroups' write-through stores).
template <bool COHERENT = false>
__device__ __forceinline__ void topk_token(const TopkArgs& a, int64_t t, float* c_lds, int32_t* sel,
                                           int lane) {
  const int E = a.E, G = a.G, gs = E / G;
  float s[4], c[4];
  const int e0 = 4 * lane;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const float l = COHERENT ? __hip_atomic_load(a.logits + t * E + e, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                               : a.logits[t * E + e];
      s[i] = (float)(1.0 / (1.0 + exp(-(double)l)));
      c[i] = s[i] + a.bias[e];
    } else {
      s[i] = 0.0f;
      c[i] = -INFINITY;
    }
  }
  // group score: sum of the two largest biased scores of the group
  uint64_t gkey = 0;
  const int lpg = gs >> 2;  // lanes per group
  const bool lane_groups = (gs & 3) == 0 && lpg <= 16 && (lpg & (lpg - 1)) == 0;
  if (lane_groups) {
    float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) top2_merge(m1, m2, c[i], -INFINITY);
    for (int off = 1; off < lpg; off <<= 1) {
      const float o1 = __shfl_xor(m1, off, 64), o2 = __shfl_xor(m2, off, 64);
      top2_merge(m1, m2, o1, o2);
    }
    const int j = lane / lpg;
    if (j < G && (lane % lpg) == 0) gkey = make_key(gs >= 2 ? m1 + m2 : m1, j);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e0 + i < E) c_lds[e0 + i] = c[i];
    wave_lds_sync();
    if (lane < G) {
      float m1 = -INFINITY, m2 = -INFINITY;
      for (int q = 0; q < gs; ++q) top2_merge(m1, m2, c_lds[lane * gs + q], -INFINITY);
      gkey = make_key(gs >= 2 ? m1 + m2 : m1, lane);
    }
  }
  // keep the kg best groups
  uint64_t kept = 0;  // bit j set: group j kept
  for (int r = 0; r < a.kg; ++r) {
    const uint64_t best = wave_max_u64(gkey);
    const int j = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
    kept |= 1ull << (j & 63);
    if (gkey == best) gkey = 0;
  }
  uint64_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + i;
    key[i] = (e < E && ((kept >> (e / gs)) & 1)) ? make_key(c[i], e) : 0;
  }
  // k rounds of wave max; the winner's score is read from its owner lane
  float my_s = 0.0f, den = 0.0f;
  int my_e = 0;
  for (int j = 0; j < a.k; ++j) {
    uint64_t m = key[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) m = key[i] > m ? key[i] : m;
    const uint64_t best = wave_max_u64(m);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (key[i] == best) key[i] = 0;
    const int q = e & 3;
    const float sv_local = q == 0 ? s[0] : q == 1 ? s[1] : q == 2 ? s[2] : s[3];
    const float sv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv_local), e >> 2));
    den = (j == 0) ? sv : den + sv;  // slot order
    if (lane == j) {
      my_s = sv;
      my_e = e;
    }
  }
  if (lane < a.k) {
    const float wj = (my_s / den) * a.scale;
    sel[lane] = my_e;
    a.ids[t * a.k + lane] = my_e;
    a.w[t * a.k + lane] = wj;
    if (a.ids2) a.ids2[t * a.k + lane] = my_e;
    if (a.w2) a.w2[t * a.k + lane] = wj;
  }
  wave_lds_sync();
}

}  // namespace beam
