// Weighted combine of one token's expert rows, shared by the combine kernel and the
// fused combine + next-boundary kernel, so both produce the same bits.
//
// [vLLM "Serving Reflection Beam auf vLLM ab Tag 0", §Agentengetriebene Optimierung,
//   change 3] and [SGLang "SGLang 支撑编程模型 Beam 生产部署", kernel-fusion paragraph]:
//   the top-k expert outputs (each already multiplied by its routing weight) are
//   summed once and rounded once.
#pragma once
#include "common.h"

namespace beam {

// Chunk c (8 values) of token t: bf16(sum over slots j in order of yk[t*k + j]), in
// FP32 starting from -0.0 (the exact additive identity); slots with an invalid id
// are skipped. Slots are taken eight at a time: all ids, then all rows in flight,
// then the adds in order.
__device__ __forceinline__ u32x4 combine_chunk(int64_t t, int c, int k, int d, int E,
                                               const int32_t* __restrict__ ids,
                                               const uint16_t* __restrict__ yk) {
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = -0.0f;
  for (int j0 = 0; j0 < k; j0 += 8) {
    bool ok[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = j0 + u < k ? ids[t * k + j0 + u] : -1;
      ok[u] = e >= 0 && e < E;
    }
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = ld_u32x4(yk + ((t * k + (ok[u] ? j0 + u : 0)) * d) + c * 8);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (ok[u]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += lo_bf(v[u][i]);
          acc[2 * i + 1] += hi_bf(v[u][i]);
        }
      }
  }
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf2(acc[2 * i], acc[2 * i + 1]);
  return o;
}

}  // namespace beam
