// Routed SwiGLU experts and the weighted combine.
//
// [vLLM "Serving Reflection Beam auf vLLM ab Tag 0", §MoE und Residual-Stream]
//   256 routed SwiGLU experts, d_ff 2560. [same page, §Der fusionierte Graph]
//   two grouped GEMMs (gate/up, then down) carry most of the MoE time.
// [SGLang "SGLang 支撑编程模型 Beam 生产部署", §BF16 MoE 内核优化]
//   gate/up and the activation keep BF16 rounding boundaries; the FP32 routing
//   weight multiplies the down projection before its BF16 rounding; a
//   single-token decode path streams the weights as two GEMV kernels.
// [vLLM §Agentengetriebene Optimierung, change 3; SGLang kernel-fusion
//   paragraph] the top-k outputs are summed, scaled and rounded once.
//
// Matrix cores: v_mfma_f32_16x16x32_bf16. For D = A * B (16 x 32 by 32 x 16):
//   lane l holds A[l % 16][8*(l/16) .. +7], B[8*(l/16) .. +7][l % 16] and
//   D[4*(l/16) .. +3][l % 16].
// Weights are repacked once into that B-operand order, so one 16-byte load per
// lane is one fragment and one wavefront load instruction reads 1 KB of
// contiguous memory:
//   gate/up: [E][f/16][d/32][2 (gate, up)][64 lanes][8]   row q of the tile = output q
//   down:    [E][d/16][f/32][64 lanes][8]
// so fragment (tile n, k-step s) holds W[16n + l%16][32s + 8(l/16) + i].
#include "common.h"
#include "kernels.h"
#include "combine_device.h"
#include "expert_device.h"
#include "mxfp4_device.h"
#include "gemm_device.h"

#include <type_traits>

namespace beam {

// ---------------------------------------------------------------------------------------------
// Repack (init only)

__global__ void repack_gateup_kernel(const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu,
                                     uint16_t* __restrict__ out, int E, int f, int d) {
  const int64_t NJ = f / 16, KS = d / 32;
  const int64_t total = (int64_t)E * NJ * KS * 2 * 64;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    int64_t lane = q % 64, r = q / 64;
    int64_t gu = r % 2;
    r /= 2;
    int64_t ks = r % KS;
    r /= KS;
    int64_t j = r % NJ;
    int64_t e = r / NJ;
    int64_t row = j * 16 + (lane & 15), col = ks * 32 + 8 * (lane >> 4);
    const uint16_t* src = (gu ? wu : wg) + (e * f + row) * d + col;
    st_u32x4(out + q * 8, ld_u32x4(src));
  }
}

__global__ void repack_down_kernel(const uint16_t* __restrict__ wd, uint16_t* __restrict__ out,
                                   int E, int f, int d) {
  const int64_t ND = d / 16, KS = f / 32;
  const int64_t total = (int64_t)E * ND * KS * 64;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    int64_t lane = q % 64, r = q / 64;
    int64_t ks = r % KS;
    r /= KS;
    int64_t nt = r % ND;
    int64_t e = r / ND;
    int64_t row = nt * 16 + (lane & 15), col = ks * 32 + 8 * (lane >> 4);
    st_u32x4(out + q * 8, ld_u32x4(wd + (e * d + row) * f + col));
  }
}

hipError_t launch_repack(const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                         uint16_t* wgu, uint16_t* wdp, int E, int f, int d, hipStream_t s) {
  hipLaunchKernelGGL(repack_gateup_kernel, dim3(65536), dim3(256), 0, s, wg, wu, wgu, E, f, d);
  hipLaunchKernelGGL(repack_down_kernel, dim3(65536), dim3(256), 0, s, wd, wdp, E, f, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Decode path: weight streaming. One workgroup per (active expert, 16 output
// columns); its four waves split the K dimension, each streaming a contiguous
// stretch of the packed weights with 16-byte non-temporal loads, U k-steps in
// flight. Rows of the expert (at most 16*MT per pass) ride along as the MFMA
// A operand, so every weight byte is read once per pass however many rows the
// expert has. Partial sums from the four waves are added in wave order.

template <int MT, int U>
__global__ __launch_bounds__(256) void gateup_stream_kernel(ExpertArgs a) {
  const int NJ = a.f / 16;
  const int j = blockIdx.x % NJ;
  int row0, cnt;
  const int e = expert_of_block(a, blockIdx.x / NJ, row0, cnt);
  if (e < 0) return;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KS = a.d / 32, ksw = KS / 4, ks0 = wv * ksw;
  const uint16_t* bp = a.wgu + ((((int64_t)e * NJ + j) * KS + ks0) * 2) * 512 + lane * 8;
  // the expert's rows are read through a buffer resource: rows past its count read
  // zeros without memory traffic, so every k-step issues the same loads
  const uint32_t zbytes = (uint32_t)a.T * a.d * 2;
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(a.z, zbytes);
  __shared__ f32x4 red[3][2 * MT][64];
  for (int m0 = 0; m0 < cnt; m0 += 16 * MT) {
    f32x4 ag[MT], au[MT];
    // the rows' slots are loaded first and used only after the weight prologue is
    // issued: older than the weight loads, they never make those wait
    int pv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      ag[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      au[mt] = ag[mt];
      const int r = m0 + mt * 16 + (lane & 15);
      pv[mt] = a.perm[row0 + (r < cnt ? r : cnt - 1)];
    }
    __builtin_amdgcn_sched_barrier(0);
    uint32_t xo[MT];  // byte offsets of the rows' fragments in z; past the end for no row
    // ring of U k-steps in flight: slot u is consumed, then refilled with the
    // k-step U ahead, so the stream never drains until its last U steps
    u32x4 bg[U], bu[U], x[MT][U];
    auto load_b = [&](int u, int ks) {
      bg[u] = ld_stream_u32x4(bp + (int64_t)ks * 1024);
      bu[u] = ld_stream_u32x4(bp + (int64_t)ks * 1024 + 512);
    };
    auto load_x = [&](int u, int ks) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) x[mt][u] = ld_buf_u32x4(zr, xo[mt] + ks * 64);
    };
    auto load = [&](int u, int ks) {
      load_b(u, ks);
      load_x(u, ks);
    };
    auto use = [&](int u) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        ag[mt] = mfma16(x[mt][u], bg[u], ag[mt]);
        au[mt] = mfma16(x[mt][u], bu[u], au[mt]);
      }
    };
    // prologue: all U weight k-steps first (their addresses need only the expert),
    // then the rows (which wait for the permutation)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load_b(u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = m0 + mt * 16 + (lane & 15);
      xo[mt] = r < cnt ? 2u * (uint32_t)((pv[mt] / a.k) * a.d + ks0 * 32 + 8 * (lane >> 4)) : zbytes;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load_x(u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int ks = 0; ks < ksw - U; ks += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        use(u);
        load(u, ks + U + u);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads in ring order
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) use(u);
    if (wv > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        red[wv - 1][2 * mt][lane] = ag[mt];
        red[wv - 1][2 * mt + 1][lane] = au[mt];
      }
    }
    __syncthreads();
    if (wv == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 g = ag[mt], u = au[mt];
#pragma unroll
        for (int w = 0; w < 3; ++w) {
          g += red[w][2 * mt][lane];
          u += red[w][2 * mt + 1][lane];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = m0 + mt * 16 + 4 * (lane >> 4) + i;
          if (r < cnt) {
            const float gv = bf2f(f2bf(g[i])), uv = bf2f(f2bf(u[i]));
            a.act[(int64_t)(row0 + r) * a.f + j * 16 + (lane & 15)] = f2bf(silu(gv) * uv);
          }
        }
      }
    }
    __syncthreads();
  }
}

// Down projection for the weight-streaming path: a workgroup covers 4 output
// tiles of 16 columns of one expert, one wave per tile accumulating the full K in
// order (the same per-output accumulation as the single-token kernel, so a token's
// result does not depend on the batch it is in).
template <int MT, int U>
__global__ __launch_bounds__(256) void down_stream_kernel(ExpertArgs a) {
  const int ND = a.d / 16, NB = ND / 4;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nt = (blockIdx.x % NB) * 4 + wv;
  int row0, cnt;
  const int e = expert_of_block(a, blockIdx.x / NB, row0, cnt);
  if (e < 0) return;
  const int KS = a.f / 32;
  const uint16_t* bp = a.wdp + ((int64_t)e * ND + nt) * KS * 512 + lane * 8;
  for (int m0 = 0; m0 < cnt; m0 += 16 * MT) {
    f32x4 acc[MT];
    const uint16_t* ap[MT];
    bool av[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = m0 + mt * 16 + (lane & 15);
      av[mt] = r < cnt;
      ap[mt] = a.act + (int64_t)(row0 + (av[mt] ? r : 0)) * a.f + 8 * (lane >> 4);
    }
    // U k-steps per batch; rows past the count are not loaded (masked lanes move no
    // bytes), which measured faster here than a ring with zero-filling buffer loads
    for (int ks = 0; ks < KS; ks += U) {
      u32x4 b[U], x[MT][U];
#pragma unroll
      for (int u = 0; u < U; ++u) b[u] = ld_stream_u32x4(bp + (int64_t)(ks + u) * 512);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int u = 0; u < U; ++u)
          x[mt][u] = av[mt] ? ld_u32x4(ap[mt] + (ks + u) * 32) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma16(x[mt][u], b[u], acc[mt]);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m0 + mt * 16 + 4 * (lane >> 4) + i;
        if (r < cnt) {
          const int slot = a.perm[row0 + r];
          a.yk[(int64_t)slot * a.d + nt * 16 + (lane & 15)] = f2bf(a.w[slot] * acc[mt][i]);
        }
      }
  }
}

// Down projection for batches of up to 16 tokens, split like gate/up: one
// workgroup per (active expert, 16 output columns); its four waves split K (f) into
// quarters, each streaming its stretch of the packed weights through a ring of U
// k-steps (16-byte non-temporal loads), with the expert's rows (at most 16 per
// pass; rows past the count are not loaded) as the MFMA A operand. The quarters are
// added in wave order, then bf16(w * sum) is written to the row's slot; the combine
// pass sums the slots. Small batches give few experts, so this spreads the weight
// stream over many small workgroups (2560 for one token: ten per CU, evenly) where
// one workgroup per 16 columns and all slots would leave some CUs with twice the
// work of others. Every T served here uses this same order, so a token's result
// does not depend on the batch.
template <int MT, int U>
__global__ __launch_bounds__(256) void down_split_kernel(ExpertArgs a) {
  const int ND = a.d / 16;
  const int nt = blockIdx.x % ND;
  int row0, cnt;
  const int e = expert_of_block(a, blockIdx.x / ND, row0, cnt);
  if (e < 0) return;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KS = a.f / 32, ksw = KS / 4, ks0 = wv * ksw;
  const uint16_t* bp = a.wdp + ((int64_t)e * ND + nt) * KS * 512 + (int64_t)ks0 * 512 + lane * 8;
  const uint32_t abytes = (uint32_t)a.T * a.k * a.f * 2;
  __shared__ f32x4 red[3][MT][64];
  for (int m0 = 0; m0 < cnt; m0 += 16 * MT) {
    f32x4 acc[MT];
    uint32_t xo[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = m0 + mt * 16 + (lane & 15);
      xo[mt] = r < cnt ? 2u * (uint32_t)((row0 + r) * a.f + ks0 * 32 + 8 * (lane >> 4)) : abytes;
    }
    u32x4 b[U], x[MT][U];
    auto load = [&](int u, int ks) {
      b[u] = ld_stream_u32x4(bp + (int64_t)ks * 512);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        x[mt][u] = xo[mt] < abytes ? ld_u32x4((const char*)a.act + xo[mt] + ks * 64)
                                   : u32x4{0u, 0u, 0u, 0u};
    };
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load(u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int ks = 0; ks < ksw - U; ks += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma16(x[mt][u], b[u], acc[mt]);
        load(u, ks + U + u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma16(x[mt][u], b[u], acc[mt]);
    if (wv > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[wv - 1][mt][lane] = acc[mt];
    }
    __syncthreads();
    if (wv == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 v = acc[mt];
#pragma unroll
        for (int w = 0; w < 3; ++w) v += red[w][mt][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = m0 + mt * 16 + 4 * (lane >> 4) + i;
          if (r < cnt) {
            const int slot = a.perm[row0 + r];
            a.yk[(int64_t)slot * a.d + nt * 16 + (lane & 15)] = f2bf(a.w[slot] * v[i]);
          }
        }
      }
    }
    __syncthreads();
  }
}

// Down projection of a dense layer (one expert) for up to 16 tokens: the expert alone
// gives only d/16 column tiles, too few workgroups for the chip, so K (f) is also split
// across P workgroups per tile. Workgroup (tile nt, part p) covers K values
// [p f/P, (p+1) f/P), its four waves a quarter of that each (summed in wave order), and
// writes FP32 partial sums part[p][row][col]; dense_finish_kernel adds the P parts in order
// and rounds once.
template <int U>
__global__ __launch_bounds__(256) void down_splitk_kernel(ExpertArgs a, int P, float* __restrict__ part) {
  const int ND = a.d / 16;
  const int nt = blockIdx.x % ND, pk = blockIdx.x / ND;
  const int cnt = a.T;  // one expert, rows in token order
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KS = a.f / 32, ksp = KS / P, ksw = ksp / 4, ks0 = pk * ksp + wv * ksw;
  const uint16_t* bp = a.wdp + (int64_t)nt * KS * 512 + (int64_t)ks0 * 512 + lane * 8;
  const uint32_t abytes = (uint32_t)a.T * a.f * 2;
  __shared__ f32x4 red[3][64];
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const int r = lane & 15;
  const uint32_t xo = r < cnt ? 2u * (uint32_t)(r * a.f + ks0 * 32 + 8 * (lane >> 4)) : abytes;
  u32x4 b[U], x[U];
  auto load = [&](int u, int ks) {
    b[u] = ld_stream_u32x4(bp + (int64_t)ks * 512);
    x[u] = xo < abytes ? ld_u32x4((const char*)a.act + xo + ks * 64) : u32x4{0u, 0u, 0u, 0u};
  };
#pragma unroll
  for (int u = 0; u < U; ++u) {
    load(u, u);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int ks = 0; ks < ksw - U; ks += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc = mfma16(x[u], b[u], acc);
      load(u, ks + U + u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) acc = mfma16(x[u], b[u], acc);
  if (wv > 0) red[wv - 1][lane] = acc;
  __syncthreads();
  if (wv == 0) {
    f32x4 v = acc;
#pragma unroll
    for (int w = 0; w < 3; ++w) v += red[w][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (lane >> 4) + i;
      if (row < cnt) part[((int64_t)pk * 16 + row) * a.d + nt * 16 + (lane & 15)] = v[i];
    }
  }
}

// y[t][o] = bf16(w[t] * (((part[0] + part[1]) + ...) + part[P-1])), one output per thread
__global__ __launch_bounds__(256) void dense_finish_kernel(int T, int d, int P, const float* __restrict__ part,
                                                           const float* __restrict__ w,
                                                           uint16_t* __restrict__ y) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T * d) return;
  const int t = i / d, o = i % d;
  float v = part[(int64_t)t * d + o];
  for (int p = 1; p < P; ++p) v += part[((int64_t)p * 16 + t) * d + o];
  y[i] = f2bf(w[t] * v);
}

hipError_t launch_down_splitk_dense(const ExpertArgs& a, int P, float* part, hipStream_t s) {
  const int ksw = a.f / 32 / P / 4;
  dim3 g((unsigned)((a.d / 16) * P)), blk(256);
  if (ksw % 10 == 0)
    hipLaunchKernelGGL((down_splitk_kernel<10>), g, blk, 0, s, a, P, part);
  else if (ksw % 8 == 0)
    hipLaunchKernelGGL((down_splitk_kernel<8>), g, blk, 0, s, a, P, part);
  else if (ksw % 4 == 0)
    hipLaunchKernelGGL((down_splitk_kernel<4>), g, blk, 0, s, a, P, part);
  else if (ksw % 2 == 0)
    hipLaunchKernelGGL((down_splitk_kernel<2>), g, blk, 0, s, a, P, part);
  else
    hipLaunchKernelGGL((down_splitk_kernel<1>), g, blk, 0, s, a, P, part);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const int n = a.T * a.d;
  hipLaunchKernelGGL(dense_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.T,
                     a.d, P, (const float*)part, a.w, a.yk);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_gateup_stream_mt(const ExpertArgs& a, int max_active, hipStream_t s) {
  const int ksw = a.d / 32 / 4;
  dim3 g((unsigned)(max_active * (a.f / 16))), blk(256);
  if (ksw % 8 == 0)
    hipLaunchKernelGGL((gateup_stream_kernel<MT, 8>), g, blk, 0, s, a);
  else if (ksw % 4 == 0)
    hipLaunchKernelGGL((gateup_stream_kernel<MT, 4>), g, blk, 0, s, a);
  else
    hipLaunchKernelGGL((gateup_stream_kernel<MT, 2>), g, blk, 0, s, a);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_down_stream_mt(const ExpertArgs& a, int max_active, hipStream_t s) {
  const int ksw = a.f / 32;  // every wave runs the full K
  dim3 g((unsigned)(max_active * (a.d / 64))), blk(256);
  if (ksw % 8 == 0)
    hipLaunchKernelGGL((down_stream_kernel<MT, 8>), g, blk, 0, s, a);
  else if (ksw % 4 == 0)
    hipLaunchKernelGGL((down_stream_kernel<MT, 4>), g, blk, 0, s, a);
  else
    hipLaunchKernelGGL((down_stream_kernel<MT, 2>), g, blk, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_split(const ExpertArgs& a, int max_active, hipStream_t s) {
  const int ksw = a.f / 32 / 4;  // k-steps per wave (f % 256 == 0: a multiple of 2)
  dim3 g((unsigned)(max_active * (a.d / 16))), blk(256);
  if (ksw % 10 == 0)
    hipLaunchKernelGGL((down_split_kernel<1, 10>), g, blk, 0, s, a);
  else if (ksw % 5 == 0)
    hipLaunchKernelGGL((down_split_kernel<1, 5>), g, blk, 0, s, a);
  else
    hipLaunchKernelGGL((down_split_kernel<1, 2>), g, blk, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gateup_stream(const ExpertArgs& a, int max_active, hipStream_t s) {
  return a.T <= 16 ? launch_gateup_stream_mt<1>(a, max_active, s)
                   : launch_gateup_stream_mt<2>(a, max_active, s);
}

hipError_t launch_down_stream(const ExpertArgs& a, int max_active, hipStream_t s) {
  return a.T <= 16 ? launch_down_stream_mt<1>(a, max_active, s)
                   : launch_down_stream_mt<2>(a, max_active, s);
}

// ---------------------------------------------------------------------------------------------
// Prefill path: grouped GEMM on the matrix cores (v_mfma_f32_32x32x16_bf16).
//
// A workgroup (8 waves, two per SIMD) computes up to 256 rows x 256 columns of one
// expert: rows are that expert's assignment rows (gathered through the permutation
// for gate/up: the z rows of their tokens), columns are 128 gate + 128 up outputs
// (gate/up) or 256 outputs (down). Wave w = 4 wm + wn owns the 32-row tiles
// 2 mt + wm (mt < MW) x columns [64 wn, 64 wn + 64) as MW x 2 MFMA tiles; MW =
// ceil(rows / 64). With an odd number of 32-row tiles the wm = 1 waves skip their last
// tile's MFMAs; each SIMD holds one wm = 0 and one wm = 1 wave, so its matrix core does
// the work of the rows rounded up to 32. An expert's rows are cut into ceil(rows / 256)
// tiles of equal size (a multiple of 32), so the tiles that share one weight tile take
// the same time.
//
// K advances 32 at a time through NS LDS stages (NS = 5 when K / 32 is a multiple
// of 5, else 4) filled by direct global-to-LDS 16-byte loads (global_load_lds_dwordx4:
// each lane's 16 bytes land at the stage base + 16 * lane), NS - 1 K blocks ahead of
// the multiply, with one barrier per K block and no staging registers. Loads take
// a few microseconds under this traffic, so the depth of the ring (up to 128 KB in
// flight per CU) sets the speed more than any other choice here. A wave's four
// copies of a K block are spread between its MFMAs, so a full memory queue stalls
// one MFMA group instead of the fragment reads of the whole block.
//   A stage: 256 rows x 32 values, 64 bytes per row; chunk c of row r is stored
//     in slot c ^ ((r / 4) % 4), so the 16 lanes of a fragment read hit 16
//     distinct 16-byte bank groups. A lane loads the logical chunk that belongs
//     in its slot. Rows past the tile's count load row 0 again (L2 hits).
//   B stage: sixteen packed 16x16x32 fragments (1 KB each) copied verbatim; a
//     32x32x16 fragment reads two adjacent blocks, 256 contiguous bytes per 16 lanes.
// For gate/up, wave w's two N tiles are gate[32 wn, 32 wn + 32) and up of the same
// outputs, so g and u of one output sit in the same lane and register and the
// SiLU-mul epilogue needs no data movement. Results are staged through LDS and
// written as 16-byte row chunks.
//
// Tile order: workgroups are dispatched round-robin over the 8 XCDs (block b runs
// on XCD b % 8), so XCD x is given a contiguous range of the tile list, which is
// ordered by expert, then (in blocks of up to 8 m-tiles) by n-tile, then m-tile:
// an expert's m-tiles read each weight tile at about the same time from one L2, and
// consecutive n-tiles share the expert's rows.
constexpr int GBM = kGemmBM, GBN = 256, GBK = 32, GMAXST = 5;
constexpr int GSTAGE_A = GBM * GBK, GSTAGE_B = GBN * GBK;  // elements per stage
constexpr int GSMEM = GMAXST * (GSTAGE_A + GSTAGE_B);      // 160 KB
static_assert(GSMEM * 2 <= 160 * 1024, "LDS");
static_assert(GBM * 256 * 2 + GBM * 8 <= GSMEM * 2, "down epilogue: output tile, weights and slots");

__device__ __forceinline__ int a_slot(int row, int c) { return row * GBK + ((c ^ ((row >> 2) & 3)) << 3); }

// s_waitcnt vmcnt(4 n): at most n K blocks of this wave's copies still in flight
__device__ __forceinline__ void wait_blocks(int n) {
  if (n >= 3) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else if (n == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// s_waitcnt vmcnt(3 n): the same for three copies per K block (4-bit weights)
__device__ __forceinline__ void wait_blocks3(int n) {
  if (n >= 3) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  else if (n == 2) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// 4-bit weights in the grouped GEMM (MXFP4, see experts_mxfp4.hip): per (expert, n-tile of
// 256 stage columns, 32-wide K block) 4096 bytes of codes — stage column c at 16 c, the
// 8-value half h of its 16-wide k-step kk at ((h ^ ((c >> 4) & 1)) * 8 + kk * 4) — and 256
// scale bytes (column c's scale of the block, byte c). Stage columns: gate/up c < 128 gate
// output 128 nb + c, c >= 128 up output 128 nb + c - 128; down output 256 nb + c.
constexpr int GSTAGE_Q = 4096 + 256;  // bytes per 4-bit B stage


// SKIP: this wave's last 32-row tile is empty (an odd number of 32-row tiles leaves wm = 1 one
// tile short), so its MFMAs are left out; the SIMD it shares with a wm = 0 wave then does
// 2 MW - 1 tiles' work. A template parameter, so the K loop has no branch.
template <bool GATEUP, int MW, int NS, bool FP4, bool SKIP>
__device__ __forceinline__ void gemm_tile_body(const ExpertArgs& a, const GemmTile& t,
                                               uint16_t* smem) {
  constexpr int NW = 8;
  static_assert(NS >= 3 && NS <= GMAXST && NS - 2 <= 3, "stages");
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);  // wave-uniform for the LDS base
  const int wm = wvu >> 2, wn = wvu & 3;
  const int K = GATEUP ? a.d : a.f;
  const int KS = K / 32;
  const int nkb = K / GBK;  // a multiple of NS
  const int e = t.e, row0 = t.row0, rows = t.rows, nb = t.nb;

  // A: wave w fills rows [32 w, 32 w + 32) of a stage with 2 instructions of 16
  // rows; lane l covers row 16 i + l / 4, slot l % 4.
  const uint16_t* abase = GATEUP ? a.z : a.act;
  int aoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wv * 32 + i * 16 + (lane >> 2);
    const int rr = r < rows ? r : 0;
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    aoff[i] = (GATEUP ? (a.perm[row0 + rr] / a.k) * a.d : (row0 + rr) * a.f) + c * 8;
  }
  // B: wave w copies blocks 2 w, 2 w + 1 of a stage (block = 64 lanes x 16 B)
  const uint16_t* bbase;
  int boff[2];
  if (GATEUP) {
    const int NJ = a.f / 16;
    bbase = a.wgu + ((int64_t)e * NJ + nb * 8) * KS * 2 * 512;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int b = wv * 2 + i, jj = b >> 1, gu = b & 1;  // stage block b = jj * 2 + gu
      boff[i] = (jj * KS * 2 + gu) * 512 + lane * 8;
    }
  } else {
    const int ND = a.d / 16;
    bbase = a.wdp + ((int64_t)e * ND + nb * 16) * KS * 512;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int b = wv * 2 + i;  // stage block b = n-tile b
      boff[i] = b * KS * 512 + lane * 8;
    }
  }
  const int bstep = GATEUP ? 2 * 512 : 512;  // elements per 32-wide K block
  // 4-bit B: waves 0-3 copy a quarter each of a block's codes, waves 4-7 its scales
  // (lanes 0-15; the same bytes), so every wave issues three copies per K block
  const uint8_t* qsrc = nullptr;
  uint32_t qdst = 0;
  if constexpr (FP4) {
    const int NTL = GATEUP ? a.f / 128 : a.d / 256;
    const int64_t blk0 = ((int64_t)e * NTL + nb) * nkb;  // (expert, n-tile, K block 0)
    qsrc = wv < 4 ? (GATEUP ? a.pqgu : a.pqd) + blk0 * 4096 + wv * 1024 + lane * 16
                  : (GATEUP ? a.psgu : a.psd) + blk0 * 256 + (lane & 15) * 16;
    qdst = wvu < 4 ? (uint32_t)(wvu * 1024) : 4096u;
  }
  // down: thread r < 256 holds row r's slot and routing weight for the epilogue
  // (loaded now, so the loads are long done when the K loop ends)
  int my_slot = 0;
  float my_w = 0.0f;
  if (!GATEUP && tid < GBM && tid < rows) {
    my_slot = a.perm[row0 + tid];
    my_w = a.w[my_slot];
  }

  auto stage_a = [&](int st) -> uint16_t* { return smem + st * GSTAGE_A; };
  auto stage_b = [&](int st) -> uint16_t* {
    if constexpr (FP4) return smem + NS * GSTAGE_A + st * (GSTAGE_Q / 2);
    return smem + NS * GSTAGE_A + st * GSTAGE_B;
  };
  // copy p (0, 1: A rows; 2, 3: B blocks; 4-bit: 2 is the wave's share of the B block)
  // of K block kb into stage st
  auto issue = [&](int kb, int st, int p) {
    if (p < 2) {
      lds_dma16(abase + aoff[p] + kb * GBK,
                lds_addr(stage_a(st)) + (uint32_t)(wvu * 32 * GBK * 2) + p * 16 * GBK * 2);
    } else if constexpr (FP4) {
      const uint16_t* src = (const uint16_t*)(qsrc + (int64_t)kb * (wv < 4 ? 4096 : 256));
      if (wv < 4 || lane < 16) lds_dma16(src, lds_addr(stage_b(st)) + qdst);
    } else {
      lds_dma16(bbase + boff[p - 2] + kb * bstep,
                lds_addr(stage_b(st)) + (uint32_t)(wvu * 2 * 1024) + (p - 2) * 1024);
    }
  };
  constexpr int CP = FP4 ? 3 : 4;  // copies per wave and K block

  const int l32 = lane & 31, lh = lane >> 5;
  int aread[2], bread[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    // (row / 4) % 4 does not change across 32-row tiles: this wave's tile mt (rows
    // 32 (2 mt + wm) ..) is at + mt * 64 * GBK
    aread[kk] = a_slot(wm * 32 + l32, kk * 2 + lh);
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      const int lanep = (lane & 15) + 16 * (kk * 2 + lh);
      const int b = GATEUP ? (2 * wn + ((lane >> 4) & 1)) * 2 + nn : wn * 4 + nn * 2 + ((lane >> 4) & 1);
      bread[nn][kk] = b * 512 + lanep * 8;
    }
  }

  f32x16 acc[MW][2];
#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // fragments of stage st, then the MFMAs with the copies of K block kb + NS - 1, one after
  // each of the first CP groups of two MFMAs (issued early, measured 1-2 % faster than spread
  // over the block at MW = 4). Past the last K block the
  // copies repeat the last block into the stage just freed (block kb - 1's, read by every
  // wave before this step's barrier), so every step issues the same copies with no branch
  // and every wait counts NS - 2 blocks behind the one it waits for.
  auto compute = [&](int st, int kb) {
    const uint16_t* A = stage_a(st);
    const uint16_t* B = stage_b(st);
    u32x4 fa[2][MW], fb[2][2];
    if constexpr (FP4) {
      // stage column of this lane's N tile nn; both k-steps' codes in one 8-byte read
      const uint8_t* Bq = (const uint8_t*)B;
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        const int c = GATEUP ? nn * 128 + 32 * wn + l32 : 64 * wn + 32 * nn + l32;
        const uint2 q = *(const uint2*)(Bq + c * 16 + ((lh ^ ((c >> 4) & 1)) * 8));
        const float sc = e8m0_scale(Bq[4096 + c]);
        fb[0][nn] = fp4x8_to_bf16(q.x, sc);
        fb[1][nn] = fp4x8_to_bf16(q.y, sc);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int mt = 0; mt < MW; ++mt) fa[kk][mt] = ld_u32x4(A + aread[kk] + mt * 64 * GBK);
    } else {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int nn = 0; nn < 2; ++nn) fb[kk][nn] = ld_u32x4(B + bread[nn][kk]);
#pragma unroll
        for (int mt = 0; mt < MW; ++mt) fa[kk][mt] = ld_u32x4(A + aread[kk] + mt * 64 * GBK);
      }
    }
    const int kn = min(kb + NS - 1, nkb - 1), sn = (st + NS - 1) % NS;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int mt = 0; mt < MW; ++mt) {
        if (mt + 1 < MW || !SKIP) {
#pragma unroll
          for (int nn = 0; nn < 2; ++nn) acc[mt][nn] = mfma32(fa[kk][mt], fb[kk][nn], acc[mt][nn]);
        }
        const int q = kk * MW + mt;
        if (q < CP) {
          __builtin_amdgcn_sched_barrier(0);
          issue(kn, sn, q);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    if (MW == 1) {  // two MFMA groups: the remaining copies go after them
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int p = 2; p < CP; ++p) issue(kn, sn, p);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // step kb: blocks kb + 1 .. kb + NS - 2 (or their repeats) are in flight behind block kb
  auto step = [&](int kb, auto S) {
    constexpr int st = decltype(S)::value;
    if constexpr (FP4) wait_blocks3(NS - 2);
    else wait_blocks(NS - 2);
    __builtin_amdgcn_s_barrier();
    compute(st, kb);
  };
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
#pragma unroll
    for (int p = 0; p < CP; ++p) issue(min(j, nkb - 1), j, p);
  for (int kb = 0; kb < nkb; kb += NS) {
    step(kb, std::integral_constant<int, 0>{});
    step(kb + 1, std::integral_constant<int, 1>{});
    step(kb + 2, std::integral_constant<int, 2>{});
    step(kb + 3, std::integral_constant<int, 3 % NS>{});
    if constexpr (NS == 5) step(kb + 4, std::integral_constant<int, 4>{});
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // epilogue through LDS (row quads, quad_store / quad_rows): the stages hold the output tile
  uint16_t* stage = smem;
  const int nq = (rows + 3) >> 2;  // row quads holding rows
  if (GATEUP) {
    // act tile [256 rows][128 q]; wave (wm, wn) holds 32-row tiles 2 mt + wm, q [32 wn, +32)
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float gv = bf2f(f2bf(acc[mt][0][4 * i + j])), uv = bf2f(f2bf(acc[mt][1][4 * i + j]));
          h[j] = f2bf(silu(gv) * uv);
        }
        quad_store<128>(stage, (2 * mt + wm) * 8 + 2 * i + lh, wn * 32 + l32, h[0] | (h[1] << 16),
                        h[2] | (h[3] << 16));
      }
    }
    __syncthreads();
    for (int c = tid; c < nq * 16; c += 64 * NW) {
      const int q = c >> 4, k = c & 15;
      u32x4 v[4];
      quad_rows<128>(stage, q, k, v);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * q + j < rows) st_u32x4(a.act + (int64_t)(row0 + 4 * q + j) * a.f + nb * 128 + k * 8, v[j]);
    }
  } else {
    // output tile [256 rows][256 cols] in the first 128 KB, weighted and rounded;
    // the rows' weights and slots behind it (rows past the count: weight 0)
    float* w_row = reinterpret_cast<float*>(smem + GBM * 256);
    int* slot_row = reinterpret_cast<int*>(w_row + GBM);
    if (tid < GBM) {
      w_row[tid] = my_w;
      slot_row[tid] = my_slot;
    }
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rq = (2 * mt + wm) * 8 + 2 * i + lh;
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(w_row + 4 * rq);
#pragma unroll
        for (int nn = 0; nn < 2; ++nn)
          quad_store<256>(stage, rq, wn * 64 + nn * 32 + l32,
                          pack_bf2(w4[0] * acc[mt][nn][4 * i], w4[1] * acc[mt][nn][4 * i + 1]),
                          pack_bf2(w4[2] * acc[mt][nn][4 * i + 2], w4[3] * acc[mt][nn][4 * i + 3]));
      }
    }
    __syncthreads();
    for (int c = tid; c < nq * 32; c += 64 * NW) {
      const int q = c >> 5, k = c & 31;
      u32x4 v[4];
      quad_rows<256>(stage, q, k, v);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * q + j < rows) st_u32x4(a.yk + (int64_t)slot_row[4 * q + j] * a.d + nb * 256 + k * 8, v[j]);
    }
  }
}

template <bool GATEUP, int MW, int NS, bool FP4>
__device__ __forceinline__ void gemm_tile_skip(const ExpertArgs& a, const GemmTile& t, uint16_t* smem,
                                               bool skip) {
  if (skip) gemm_tile_body<GATEUP, MW, NS, FP4, true>(a, t, smem);
  else gemm_tile_body<GATEUP, MW, NS, FP4, false>(a, t, smem);
}

template <bool GATEUP, int NS, bool FP4 = false>
__device__ __forceinline__ void gemm_tile_mw(const ExpertArgs& a, const GemmTile& t, uint16_t* smem) {
  const int n32 = (t.rows + 31) >> 5;  // 32-row tiles: wm = 0 takes the even ones, wm = 1 the odd
  const int wm = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) >> 2;
  const bool skip = (n32 & 1) && wm == 1;
  switch ((n32 + 1) >> 1) {  // tiles per wave
    case 1: gemm_tile_skip<GATEUP, 1, NS, FP4>(a, t, smem, skip); break;
    case 2: gemm_tile_skip<GATEUP, 2, NS, FP4>(a, t, smem, skip); break;
    case 3: gemm_tile_skip<GATEUP, 3, NS, FP4>(a, t, smem, skip); break;
    default: gemm_tile_skip<GATEUP, 4, NS, FP4>(a, t, smem, skip); break;
  }
}

template <bool GATEUP>
__global__ __launch_bounds__(512) void grouped_gemm_kernel(ExpertArgs a) {
  // the stages, reused as the epilogue's staging tile
  __shared__ __attribute__((aligned(1024))) uint16_t smem[GSMEM];
  const int NT = GATEUP ? a.f / 128 : a.d / 256;  // n-tiles per m-tile
  const int total = a.tile_start[a.E] * NT;        // (expert, n-tile, m-tile) triples
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int R = (total + 7) >> 3;
  const int L = xcd * R + q;
  if (q >= R || L >= total) return;
  const GemmTile t = decode_tile(a, NT, L);
  if (((GATEUP ? a.d : a.f) / GBK) % 5 == 0)
    gemm_tile_mw<GATEUP, 5>(a, t, smem);
  else
    gemm_tile_mw<GATEUP, 4>(a, t, smem);
}

// The same GEMM on 4-bit weights: the B stages hold codes and scales (GSTAGE_Q bytes),
// each lane dequantises its B fragments when it reads them (exact BF16 values), so the
// MFMAs and their order are the BF16 kernel's.
template <bool GATEUP>
__global__ __launch_bounds__(512) void grouped_gemm_fp4_kernel(ExpertArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[GSMEM];
  const int NT = GATEUP ? a.f / 128 : a.d / 256;
  const int total = a.tile_start[a.E] * NT;
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int R = (total + 7) >> 3;
  const int L = xcd * R + q;
  if (q >= R || L >= total) return;
  const GemmTile t = decode_tile(a, NT, L);
  if (((GATEUP ? a.d : a.f) / GBK) % 5 == 0)
    gemm_tile_mw<GATEUP, 5, true>(a, t, smem);
  else
    gemm_tile_mw<GATEUP, 4, true>(a, t, smem);
}
static_assert(GMAXST * (GSTAGE_A * 2 + GSTAGE_Q) <= GSMEM * 2, "4-bit stages");

hipError_t launch_gateup_gemm_fp4(const ExpertArgs& a, int max_tiles, hipStream_t s) {
  const unsigned gx = (unsigned)(8 * ((max_tiles * (a.f / 128) + 7) / 8));
  hipLaunchKernelGGL(grouped_gemm_fp4_kernel<true>, dim3(gx), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_gemm_fp4(const ExpertArgs& a, int max_tiles, hipStream_t s) {
  const unsigned gx = (unsigned)(8 * ((max_tiles * (a.d / 256) + 7) / 8));
  hipLaunchKernelGGL(grouped_gemm_fp4_kernel<false>, dim3(gx), dim3(512), 0, s, a);
  return hipGetLastError();
}

// 1-D grid of 8 * ceil(max_tiles * n-tiles / 8) workgroups (see the tile order above)
hipError_t launch_gateup_gemm(const ExpertArgs& a, int max_tiles, hipStream_t s) {
  const unsigned gx = (unsigned)(8 * ((max_tiles * (a.f / 128) + 7) / 8));
  hipLaunchKernelGGL(grouped_gemm_kernel<true>, dim3(gx), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_gemm(const ExpertArgs& a, int max_tiles, hipStream_t s) {
  const unsigned gx = (unsigned)(8 * ((max_tiles * (a.d / 256) + 7) / 8));
  hipLaunchKernelGGL(grouped_gemm_kernel<false>, dim3(gx), dim3(512), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Combine: y[t] = bf16(sum over slots j in order of yk[t*k+j]) (combine_chunk), one
// 16-byte output chunk per thread.
__global__ __launch_bounds__(256) void combine_kernel(int T, int k, int d, int E,
                                                      const int32_t* __restrict__ ids,
                                                      const uint16_t* __restrict__ yk,
                                                      uint16_t* __restrict__ y) {
  const int nch = d / 8;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= (int64_t)T * nch) return;
  const int64_t t = q / nch;
  const int c = (int)(q % nch);
  st_u32x4(y + t * d + c * 8, combine_chunk(t, c, k, d, E, ids, yk));
}

hipError_t launch_combine(int T, int k, int d, int E, const int32_t* ids, const uint16_t* yk,
                          uint16_t* y, hipStream_t s) {
  const int64_t n = (int64_t)T * (d / 8);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, T, k, d,
                     E, ids, yk, y);
  return hipGetLastError();
}

}  // namespace beam
