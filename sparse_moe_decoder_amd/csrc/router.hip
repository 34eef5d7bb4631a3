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
#include "router_device.h"
#include "topk_device.h"

#include <type_traits>

namespace beam {

// ---------------------------------------------------------------------------------------------
// Router logits, FP32 on the vector ALUs: logits[t, e] = sum_i z[t, i] * W[e, i].
// One wavefront per (expert, block of RT tokens): each lane walks 16-byte chunks
// of W's row (chunk c -> lane c % 64) and keeps one FP32 partial per token; the
// partials are then summed across the wave. W's row is read once per token block.
constexpr int RT = kRouterRT;

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
// split d, so a W row is fetched by 256 lanes at once.
__global__ __launch_bounds__(256) void router_fp32_small_kernel(RouterArgs a) {
  __shared__ float part[3][kRouterRT];
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * kRouterRT;
  const int nt = min(kRouterRT, a.T - t0);
  const float v = router_small_dot(a, e, t0, nt, part);
  if (threadIdx.x < nt) a.logits[(int64_t)(t0 + threadIdx.x) * a.E + e] = v;
}

// ---------------------------------------------------------------------------------------------
// Large batches: the FP32 router as three BF16 matrix-core products.
// [SGLang "SGLang 支撑编程模型 Beam 生产部署", overview of kernel optimisations]
//   a dedicated BF16x3 GEMM serves the FP32 router.
// At init W is split exactly into W = hi + mid + lo, each part BF16 (hi = bf16(W),
// mid = bf16(W - hi), lo = W - hi - mid: each residual holds at most the next 8
// significant bits, so no bits are lost). z is BF16, so every product z * part is
// exact in FP32; the matrix cores add all three products of a column into one FP32
// accumulator. Parts are packed like the expert weights: [3][E/16][d/32][64][8].
__global__ void repack_router_kernel(const float* __restrict__ W, uint16_t* __restrict__ out,
                                     int E, int d) {
  const int64_t NT = E / 16, KS = d / 32;
  const int64_t total = NT * KS * 64;  // 16-byte fragments per part
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t lane = q % 64, r = q / 64;
    const int64_t ks = r % KS, nt = r / KS;
    const int64_t row = nt * 16 + (lane & 15), col = ks * 32 + 8 * (lane >> 4);
    u32x4 hi, mid, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t h2 = 0, m2 = 0, l2 = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float w = W[row * d + col + 2 * i + j];
        const uint16_t h = f2bf(w);
        const float r1 = w - bf2f(h);
        const uint16_t m = f2bf(r1);
        const uint16_t l = f2bf(r1 - bf2f(m));
        h2 |= (uint32_t)h << (16 * j);
        m2 |= (uint32_t)m << (16 * j);
        l2 |= (uint32_t)l << (16 * j);
      }
      hi[i] = h2;
      mid[i] = m2;
      lo[i] = l2;
    }
    st_u32x4(out + q * 8, hi);
    st_u32x4(out + (total + q) * 8, mid);
    st_u32x4(out + (2 * total + q) * 8, lo);
  }
}

hipError_t launch_repack_router(const float* W, uint16_t* out, int E, int d, hipStream_t s) {
  hipLaunchKernelGGL(repack_router_kernel, dim3(4096), dim3(256), 0, s, W, out, E, d);
  return hipGetLastError();
}

// Tile: 256 tokens x 64 experts, 4 waves of 64 tokens x 64 experts (2 x 2 tiles of
// 32x32x16, three B fragments per product). K advances 32 at a time through four LDS
// stages filled by direct global-to-LDS loads, three K blocks ahead.
constexpr int RBM = 256, RBN = 64, RBK = 32, RSTAGES = 4;
constexpr int RSTAGE_A = RBM * RBK, RSTAGE_B = 3 * RBN * RBK;  // elements

__device__ __forceinline__ uint32_t lds_addr_r(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_dma16_r(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ int ra_slot(int row, int c) {
  return row * RBK + ((c ^ ((row >> 2) & 3)) << 3);
}

__global__ __launch_bounds__(256) void router_bf16x3_kernel(RouterX3Args a) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[RSTAGES * (RSTAGE_A + RSTAGE_B)];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int t0 = blockIdx.x * RBM;
  const int eb = blockIdx.y;  // 64-expert block
  const int rows = min(RBM, a.T - t0);
  const int KS = a.d / 32, NT = a.E / 16;
  // A: wave wv fills rows [64 wv, 64 wv + 64): 4 instructions of 16 rows
  int aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wv * 64 + i * 16 + (lane >> 2);
    const int rr = r < rows ? r : 0;
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    aoff[i] = (t0 + rr) * a.d + c * 8;
  }
  // B: 12 blocks per stage (part p, 16-expert tile t: block p * 4 + t); wave wv copies 3
  int boff[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int b = wvu * 3 + i, p = b >> 2, t = b & 3;
    boff[i] = ((p * NT + eb * 4 + t) * KS) * 512 + lane * 8;
  }
  auto issue = [&](int kb, int st) {
    const uint32_t A = lds_addr_r(smem + st * RSTAGE_A) + (uint32_t)(wvu * 64 * RBK * 2);
    const uint32_t B = lds_addr_r(smem + RSTAGES * RSTAGE_A + st * RSTAGE_B) +
                       (uint32_t)(wvu * 3 * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_dma16_r(a.z + aoff[i] + kb * RBK, A + i * 16 * RBK * 2);
#pragma unroll
    for (int i = 0; i < 3; ++i) lds_dma16_r(a.wx3 + boff[i] + kb * 512, B + i * 1024);
  };
  const int l32 = lane & 31, lh = lane >> 5;
  int aread[2][2], bread[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) aread[mt][kk] = ra_slot(wv * 64 + mt * 32 + l32, kk * 2 + lh);
#pragma unroll
    for (int nn = 0; nn < 2; ++nn)
      bread[nn][kk] = (nn * 2 + ((lane >> 4) & 1)) * 512 + ((lane & 15) + 16 * (kk * 2 + lh)) * 8;
  }
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nkb = a.d / RBK;
  auto step = [&](int kb, auto S) {
    constexpr int st = decltype(S)::value;
    const int left = nkb - 1 - kb;
    if (left >= 2) asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
    else if (left == 1) asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    const uint16_t* A = smem + st * RSTAGE_A;
    const uint16_t* B = smem + RSTAGES * RSTAGE_A + st * RSTAGE_B;
    u32x4 fa[2][2], fb[2][2][3];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) fa[kk][mt] = ld_u32x4(A + aread[mt][kk]);
#pragma unroll
      for (int nn = 0; nn < 2; ++nn)
#pragma unroll
        for (int p = 0; p < 3; ++p) fb[kk][nn][p] = ld_u32x4(B + p * 4 * 512 + bread[nn][kk]);
    }
    if (kb + RSTAGES - 1 < nkb) issue(kb + RSTAGES - 1, (st + 3) & 3);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nn = 0; nn < 2; ++nn) acc[mt][nn] = mfma32(fa[kk][mt], fb[kk][nn][p], acc[mt][nn]);
  };
  issue(0, 0);
  issue(1, 1);
  issue(2, 2);
  for (int kb = 0; kb < nkb; kb += 4) {
    step(kb, std::integral_constant<int, 0>{});
    step(kb + 1, std::integral_constant<int, 1>{});
    step(kb + 2, std::integral_constant<int, 2>{});
    step(kb + 3, std::integral_constant<int, 3>{});
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nn = 0; nn < 2; ++nn)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wv * 64 + mt * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (row < rows)
          a.logits[(int64_t)(t0 + row) * a.E + eb * 64 + nn * 32 + l32] = acc[mt][nn][r];
      }
}

hipError_t launch_router_bf16x3(const RouterX3Args& a, hipStream_t s) {
  dim3 grid((unsigned)((a.T + RBM - 1) / RBM), (unsigned)(a.E / RBN));
  hipLaunchKernelGGL(router_bf16x3_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
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
// Selection: order-preserving 32-bit keys, a wave max per round and the lowest lane
// (lowest index) holding it (topk_token).
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  __shared__ float c_lds[4][256];
  __shared__ int32_t sel_ids[4][32];
  const int wv = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wv;
  if (t >= a.T) return;
  topk_token(a, t, c_lds[wv], sel_ids[wv], threadIdx.x & 63);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace beam
