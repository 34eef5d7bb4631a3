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

// Tile: 256 tokens x 64 experts per workgroup of 8 waves (two per SIMD): wave w =
// 2 wm + wn holds tokens [64 wm, 64 wm + 64) x experts [32 wn, 32 wn + 32) as 2 x 1
// tiles of 32x32x16, three B fragments (the weight's three parts) per product. K
// advances 32 at a time through NS LDS stages (5 when d / 32 is a multiple of 5,
// else 4) filled by direct global-to-LDS loads NS - 1 K blocks ahead; each wave's
// copies of a block are spread between its MFMA groups.
//   A stage: 256 rows x 32 values (64 B per row), chunk c of row r in slot
//     c ^ ((r / 4) % 4); wave w copies rows [32 w, 32 w + 32).
//   B stage: 12 packed 16x16x32 blocks (part p, 16-expert tile t: block 4 p + t);
//     waves 0-3 copy two blocks each, waves 4-7 one.
constexpr int RBM = 256, RBN = 64, RBK = 32, RMAXST = 5;
constexpr int RSTAGE_A = RBM * RBK, RSTAGE_B = 3 * RBN * RBK;  // elements
static_assert(RMAXST * (RSTAGE_A + RSTAGE_B) * 2 <= 160 * 1024, "LDS");

__device__ __forceinline__ uint32_t lds_addr_r(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Direct global-to-LDS 16-byte copy per lane (to lds + 16 lane), as in the expert GEMM:
// inline assembly that sets m0 itself; the kernel holds no value in m0.
__device__ __forceinline__ void lds_dma16_r(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ int ra_slot(int row, int c) {
  return row * RBK + ((c ^ ((row >> 2) & 3)) << 3);
}
// at most n K blocks of this wave's copies in flight (per block: 4 copies for
// waves 0-3, 3 for waves 4-7)
__device__ __forceinline__ void router_wait_blocks(int n, bool four) {
  if (four) {
    if (n >= 3) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else if (n == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (n == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (n >= 3) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else if (n == 2) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else if (n == 1) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

template <int NS>
__device__ __forceinline__ void router_x3_tile(const RouterX3Args& a, uint16_t* smem) {
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int wm = wvu >> 1, wn = wvu & 1;
  const bool four = wvu < 4;  // this wave copies two B blocks per K block
  const int t0 = blockIdx.x * RBM;
  const int eb = blockIdx.y;  // 64-expert block
  const int rows = min(RBM, a.T - t0);
  const int KS = a.d / 32, NT = a.E / 16;
  const int nkb = a.d / RBK;  // a multiple of NS
  int aoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wv * 32 + i * 16 + (lane >> 2);
    const int rr = r < rows ? r : 0;
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    aoff[i] = (t0 + rr) * a.d + c * 8;
  }
  const int b0 = four ? 2 * wvu : 8 + (wvu - 4);  // first B block of this wave
  int boff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int b = b0 + i, p = b >> 2, t = b & 3;
    boff[i] = ((p * NT + eb * 4 + t) * KS) * 512 + lane * 8;
  }
  auto stage_a = [&](int st) -> uint16_t* { return smem + st * RSTAGE_A; };
  auto stage_b = [&](int st) -> uint16_t* { return smem + NS * RSTAGE_A + st * RSTAGE_B; };
  // copy q of K block kb (0, 1: A rows; 2, 3: B blocks, 3 only for waves 0-3)
  auto issue = [&](int kb, int st, int q) {
    if (q < 2)
      lds_dma16_r(a.z + aoff[q] + kb * RBK,
                  lds_addr_r(stage_a(st)) + (uint32_t)(wvu * 32 * RBK * 2) + q * 16 * RBK * 2);
    else if (q == 2 || four)
      lds_dma16_r(a.wx3 + boff[q - 2] + kb * 512,
                  lds_addr_r(stage_b(st)) + (uint32_t)(b0 * 1024) + (q - 2) * 1024);
  };
  const int l32 = lane & 31, lh = lane >> 5;
  int aread[2][2], bread[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) aread[mt][kk] = ra_slot(wm * 64 + mt * 32 + l32, kk * 2 + lh);
    bread[kk] = (wn * 2 + ((lane >> 4) & 1)) * 512 + ((lane & 15) + 16 * (kk * 2 + lh)) * 8;
  }
  f32x16 acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

  auto step = [&](int kb, auto S) {
    constexpr int st = decltype(S)::value;
    const int later = nkb - 1 - kb;
    router_wait_blocks(later < NS - 2 ? later : NS - 2, four);
    __builtin_amdgcn_s_barrier();
    const uint16_t* A = stage_a(st);
    const uint16_t* B = stage_b(st);
    u32x4 fa[2][2], fb[2][3];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) fa[kk][mt] = ld_u32x4(A + aread[mt][kk]);
#pragma unroll
      for (int p = 0; p < 3; ++p) fb[kk][p] = ld_u32x4(B + p * 4 * 512 + bread[kk]);
    }
    const bool more = kb + NS - 1 < nkb;
    const int kn = kb + NS - 1, sn = (st + NS - 1) % NS;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int p = 0; p < 3; ++p) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[mt] = mfma32(fa[kk][mt], fb[kk][p], acc[mt]);
        const int g = kk * 3 + p;  // six MFMA pairs; a copy after pairs 0, 1, 3, 4
        if (g == 0 || g == 1 || g == 3 || g == 4) {
          __builtin_amdgcn_sched_barrier(0);
          if (more) issue(kn, sn, g < 2 ? g : g - 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
  };
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) issue(j, j, q);
  for (int kb = 0; kb < nkb; kb += NS) {
    step(kb, std::integral_constant<int, 0>{});
    step(kb + 1, std::integral_constant<int, 1>{});
    step(kb + 2, std::integral_constant<int, 2>{});
    step(kb + 3, std::integral_constant<int, 3>{});
    if constexpr (NS == 5) step(kb + 4, std::integral_constant<int, 4>{});
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 64 + mt * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
      if (row < rows) a.logits[(int64_t)(t0 + row) * a.E + eb * 64 + wn * 32 + l32] = acc[mt][r];
    }
}

__global__ __launch_bounds__(512) void router_bf16x3_kernel(RouterX3Args a) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[RMAXST * (RSTAGE_A + RSTAGE_B)];
  if ((a.d / RBK) % 5 == 0)
    router_x3_tile<5>(a, smem);
  else
    router_x3_tile<4>(a, smem);
}

hipError_t launch_router_bf16x3(const RouterX3Args& a, hipStream_t s) {
  dim3 grid((unsigned)((a.T + RBM - 1) / RBM), (unsigned)(a.E / RBN));
  hipLaunchKernelGGL(router_bf16x3_kernel, grid, dim3(512), 0, s, a);
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
