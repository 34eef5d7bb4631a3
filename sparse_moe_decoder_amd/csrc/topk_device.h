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
// Selection: each candidate's value becomes an order-preserving 32-bit key; a
// round takes the wave maximum of the lanes' best keys and the lowest lane that
// holds it. Lane l holds experts 4l .. 4l+3 and prefers its lowest index among
// equal keys, so the winner is the lowest index of the largest value: the order is
// (value desc, index asc) exactly.
#pragma once
#include "common.h"
#include "kernels.h"

namespace beam {

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

// The routing score of a logit: sigmoid in double, rounded once to FP32.
__device__ __forceinline__ float routing_score(float l) {
  return (float)(1.0 / (1.0 + exp(-(double)l)));
}

// SCORES: instead of logits, read each expert's (score s, biased score c) pair from
// `sc` [T, E] (s in the low 32 bits) with device-coherent loads: the pairs were
// published within the same launch by other workgroups' write-through stores.
template <bool SCORES = false>
__device__ __forceinline__ void topk_token(const TopkArgs& a, int64_t t, float* c_lds, int32_t* sel,
                                           int lane, const uint64_t* sc = nullptr) {
  const int E = a.E, G = a.G, gs = E / G;
  float s[4], c[4];
  const int e0 = 4 * lane;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + i;
    if (e < E) {
      if constexpr (SCORES) {
        const uint64_t p = __hip_atomic_load(sc + t * E + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s[i] = __uint_as_float((uint32_t)p);
        c[i] = __uint_as_float((uint32_t)(p >> 32));
      } else {
        s[i] = routing_score(a.logits[t * E + e]);
        c[i] = s[i] + a.bias[e];
      }
    } else {
      s[i] = 0.0f;
      c[i] = -INFINITY;
    }
  }
  // group score: sum of the two largest biased scores of the group; the group's
  // key sits in the lowest lane of the group (groups ascend with lanes)
  uint32_t gkey = 0;
  int gof = 0;  // group held by this lane
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
    gof = lane / lpg;
    if (gof < G && (lane % lpg) == 0) gkey = f32_order_key(gs >= 2 ? m1 + m2 : m1);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e0 + i < E) c_lds[e0 + i] = c[i];
    wave_lds_sync();
    gof = lane;
    if (lane < G) {
      float m1 = -INFINITY, m2 = -INFINITY;
      for (int q = 0; q < gs; ++q) top2_merge(m1, m2, c_lds[lane * gs + q], -INFINITY);
      gkey = f32_order_key(gs >= 2 ? m1 + m2 : m1);
    }
  }
  // keep the kg best groups (ties: lower group)
  uint64_t kept = 0;  // bit j set: group j kept
  for (int r = 0; r < a.kg; ++r) {
    const uint32_t best = wave_max_u32(gkey);
    const int L = first_lane(gkey == best);
    const int j = __builtin_amdgcn_readlane(gof, L);
    kept |= 1ull << (j & 63);
    if (lane == L) gkey = 0;
  }
  uint32_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + i;
    key[i] = (e < E && ((kept >> (e / gs)) & 1)) ? f32_order_key(c[i]) : 0u;
  }
  // k rounds: the lane's best candidate (lowest index among equal keys), the wave's
  // best key, the lowest lane holding it; the winner's score comes from that lane
  float my_s = 0.0f, den = 0.0f;
  int my_e = 0;
  for (int j = 0; j < a.k; ++j) {
    uint32_t lm = key[0];
    int li = 0;
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (key[i] > lm) {
        lm = key[i];
        li = i;
      }
    const uint32_t best = wave_max_u32(lm);
    const int L = first_lane(lm == best);
    const int q = __builtin_amdgcn_readlane(li, L);
    const int e = 4 * L + q;
    const float sl = li == 0 ? s[0] : li == 1 ? s[1] : li == 2 ? s[2] : s[3];
    const float sv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sl), L));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane == L && i == li) key[i] = 0u;
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
