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

__device__ __forceinline__ int expert_of_block(const ExpertArgs& a, int slot, int& row0,
                                               int& cnt) {
  if (slot >= *a.n_active) return -1;
  const int e = a.active[slot];
  row0 = a.offsets[e];
  cnt = a.offsets[e + 1] - row0;
  return e;
}

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
  __shared__ f32x4 red[3][2 * MT][64];
  for (int m0 = 0; m0 < cnt; m0 += 16 * MT) {
    f32x4 ag[MT], au[MT];
    const uint16_t* ap[MT];
    bool av[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      ag[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      au[mt] = ag[mt];
      const int r = m0 + mt * 16 + (lane & 15);
      av[mt] = r < cnt;
      const int tok = av[mt] ? a.perm[row0 + r] / a.k : 0;
      ap[mt] = a.z + (int64_t)tok * a.d + ks0 * 32 + 8 * (lane >> 4);
    }
    for (int ks = 0; ks < ksw; ks += U) {
      u32x4 bg[U], bu[U], x[MT][U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bg[u] = ld_stream_u32x4(bp + ((int64_t)(ks + u) * 2 + 0) * 512);
        bu[u] = ld_stream_u32x4(bp + ((int64_t)(ks + u) * 2 + 1) * 512);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int u = 0; u < U; ++u)
          x[mt][u] = av[mt] ? ld_u32x4(ap[mt] + (ks + u) * 32) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          ag[mt] = mfma16(x[mt][u], bg[u], ag[mt]);
          au[mt] = mfma16(x[mt][u], bu[u], au[mt]);
        }
    }
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

template <int MT, int U>
__global__ __launch_bounds__(256) void down_stream_kernel(ExpertArgs a) {
  const int ND = a.d / 16;
  const int nt = blockIdx.x % ND;
  int row0, cnt;
  const int e = expert_of_block(a, blockIdx.x / ND, row0, cnt);
  if (e < 0) return;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KS = a.f / 32, ksw = KS / 4, ks0 = wv * ksw;
  const uint16_t* bp = a.wdp + (((int64_t)e * ND + nt) * KS + ks0) * 512 + lane * 8;
  __shared__ f32x4 red[3][MT][64];
  for (int m0 = 0; m0 < cnt; m0 += 16 * MT) {
    f32x4 acc[MT];
    const uint16_t* ap[MT];
    bool av[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = m0 + mt * 16 + (lane & 15);
      av[mt] = r < cnt;
      ap[mt] = a.act + (int64_t)(row0 + (av[mt] ? r : 0)) * a.f + ks0 * 32 + 8 * (lane >> 4);
    }
    for (int ks = 0; ks < ksw; ks += U) {
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
    if (wv > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[wv - 1][mt][lane] = acc[mt];
    }
    __syncthreads();
    if (wv == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 c = acc[mt];
#pragma unroll
        for (int w = 0; w < 3; ++w) c += red[w][mt][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = m0 + mt * 16 + 4 * (lane >> 4) + i;
          if (r < cnt) {
            const int slot = a.perm[row0 + r];
            a.yk[(int64_t)slot * a.d + nt * 16 + (lane & 15)] = f2bf(a.w[slot] * c[i]);
          }
        }
      }
    }
    __syncthreads();
  }
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
  const int ksw = a.f / 32 / 4;
  dim3 g((unsigned)(max_active * (a.d / 16))), blk(256);
  if (ksw % 8 == 0)
    hipLaunchKernelGGL((down_stream_kernel<MT, 8>), g, blk, 0, s, a);
  else if (ksw % 4 == 0)
    hipLaunchKernelGGL((down_stream_kernel<MT, 4>), g, blk, 0, s, a);
  else
    hipLaunchKernelGGL((down_stream_kernel<MT, 2>), g, blk, 0, s, a);
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
// Prefill path: grouped GEMM on the matrix cores. A workgroup computes a
// 128-row x 128-column tile of one expert: rows are that expert's assignment
// rows (gathered through the permutation for gate/up), columns are 4 gate/up
// tile pairs (gate/up) or 8 output tiles (down). K advances 64 at a time through
// LDS; the next K block is fetched into registers while the current one is
// multiplied. The four waves each own a 64 x 64 quarter (4 x 4 MFMA tiles).
constexpr int GBM = kGemmBM, GBK = 64, GLDA = GBK + 8;

template <bool GATEUP>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(ExpertArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[GBM * GLDA];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2 * 8 * 512];
  const int g = blockIdx.x;
  const int nb = blockIdx.y;
  if (g >= a.tile_start[a.E]) return;
  int lo = 0, hi = a.E;  // largest e with tile_start[e] <= g
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (a.tile_start[mid] <= g) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int row0 = a.offsets[e];
  const int m0 = (g - a.tile_start[e]) * GBM;
  const int rows = min(GBM, a.offsets[e + 1] - row0 - m0);
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int wm = wv >> 1, wn = wv & 1;
  const int K = GATEUP ? a.d : a.f;
  const int KS = K / 32;

  // global sources for this thread's 4 A chunks and 4 B chunks
  const uint16_t* asrc[4];
  int adst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i, r = q >> 3, kc = q & 7;
    adst[i] = r * GLDA + kc * 8;
    if (r < rows) {
      if (GATEUP) {
        const int tok = a.perm[row0 + m0 + r] / a.k;
        asrc[i] = a.z + (int64_t)tok * a.d + kc * 8;
      } else {
        asrc[i] = a.act + (int64_t)(row0 + m0 + r) * a.f + kc * 8;
      }
    } else {
      asrc[i] = nullptr;
    }
  }
  const uint16_t* bsrc[4];
  int64_t bstep;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i, blk = q >> 6, ln = q & 63;
    const int ksl = blk >> 3, bb = blk & 7;
    if (GATEUP) {
      const int NJ = a.f / 16, jj = bb >> 1, gu = bb & 1;
      bsrc[i] = a.wgu + ((((int64_t)e * NJ + nb * 4 + jj) * KS + ksl) * 2 + gu) * 512 + ln * 8;
    } else {
      const int ND = a.d / 16;
      bsrc[i] = a.wdp + (((int64_t)e * ND + nb * 8 + bb) * KS + ksl) * 512 + ln * 8;
    }
  }
  bstep = GATEUP ? 4 * 512 : 2 * 512;  // elements per 64-wide K block

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[4], rb[4];
  auto fetch = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = asrc[i] ? ld_u32x4(asrc[i] + kb * GBK) : u32x4{0u, 0u, 0u, 0u};
      rb[i] = ld_u32x4(bsrc[i] + (int64_t)kb * bstep);
    }
  };
  const int nkb = K / GBK;
  fetch(0);
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      st_u32x4(As + adst[i], ra[i]);
      st_u32x4(Bs + (tid + 256 * i) * 8, rb[i]);
    }
    __syncthreads();
    if (kb + 1 < nkb) fetch(kb + 1);
#pragma unroll
    for (int ksl = 0; ksl < 2; ++ksl) {
      u32x4 fa[4], fb[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        fa[mt] = ld_u32x4(As + (wm * 64 + mt * 16 + (lane & 15)) * GLDA + ksl * 32 + 8 * (lane >> 4));
#pragma unroll
      for (int nn = 0; nn < 4; ++nn) {
        const int blk = GATEUP ? ksl * 8 + (2 * wn + (nn >> 1)) * 2 + (nn & 1) : ksl * 8 + wn * 4 + nn;
        fb[nn] = ld_u32x4(Bs + blk * 512 + lane * 8);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) acc[mt][nn] = mfma16(fa[mt], fb[nn], acc[mt][nn]);
    }
  }

  // epilogue
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + mt * 16 + 4 * (lane >> 4) + i;
      if (r >= rows) continue;
      const int row = row0 + m0 + r;
      if (GATEUP) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const float gv = bf2f(f2bf(acc[mt][2 * jj][i])), uv = bf2f(f2bf(acc[mt][2 * jj + 1][i]));
          const int col = (nb * 4 + 2 * wn + jj) * 16 + (lane & 15);
          a.act[(int64_t)row * a.f + col] = f2bf(silu(gv) * uv);
        }
      } else {
        const int slot = a.perm[row];
        const float wt = a.w[slot];
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) {
          const int col = (nb * 8 + wn * 4 + nn) * 16 + (lane & 15);
          a.yk[(int64_t)slot * a.d + col] = f2bf(wt * acc[mt][nn][i]);
        }
      }
    }
  }
}

hipError_t launch_gateup_gemm(const ExpertArgs& a, int max_tiles, hipStream_t s) {
  hipLaunchKernelGGL(grouped_gemm_kernel<true>, dim3((unsigned)max_tiles, (unsigned)(a.f / 64)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_gemm(const ExpertArgs& a, int max_tiles, hipStream_t s) {
  hipLaunchKernelGGL(grouped_gemm_kernel<false>, dim3((unsigned)max_tiles, (unsigned)(a.d / 128)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Combine: y[t] = bf16(sum over slots j in order of yk[t*k+j]), FP32, starting
// from -0.0 (the exact additive identity); slots with an invalid id are skipped.
__global__ __launch_bounds__(256) void combine_kernel(int T, int k, int d, int E,
                                                      const int32_t* __restrict__ ids,
                                                      const uint16_t* __restrict__ yk,
                                                      uint16_t* __restrict__ y) {
  const int nch = d / 8;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= (int64_t)T * nch) return;
  const int64_t t = q / nch;
  const int c = (int)(q % nch);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = -0.0f;
  for (int j = 0; j < k; ++j) {
    const int e = ids[t * k + j];
    if (e < 0 || e >= E) continue;
    const u32x4 v = ld_u32x4(yk + ((t * k + j) * d) + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += lo_bf(v[i]);
      acc[2 * i + 1] += hi_bf(v[i]);
    }
  }
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf2(acc[2 * i], acc[2 * i + 1]);
  st_u32x4(y + t * d + c * 8, o);
}

hipError_t launch_combine(int T, int k, int d, int E, const int32_t* ids, const uint16_t* yk,
                          uint16_t* y, hipStream_t s) {
  const int64_t n = (int64_t)T * (d / 8);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, T, k, d,
                     E, ids, yk, y);
  return hipGetLastError();
}

}  // namespace beam
