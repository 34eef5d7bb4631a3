// Routed SwiGLU experts with 4-bit (MXFP4) weights: quantisation, the decode-layout
// repack, and the weight-streaming gate/up and down kernels.
//
// [vLLM "Serving Reflection Beam auf vLLM ab Tag 0", §Modellarchitektur] the routed
//   experts are served with 4-bit floating-point weights (NVFP4 on the pages'
//   hardware). [SGLang "SGLang 支撑编程模型 Beam 生产部署", §BF16、NVFP4 和 FP8 模型支持]
//   BF16, NVFP4 and FP8 checkpoints.
// The 4-bit format here is MXFP4 (OCP Microscaling Formats specification v1.0):
// E2M1 codes (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 = sign), one E8M0 scale
// 2^(s - 127) per 32 consecutive values along K, element 2i in the low nibble of
// byte i. gfx950 converts a code pair and a scale to two BF16 values in one
// instruction (v_cvt_scalef32_pk_bf16_fp4); every E2M1 value times a power of two
// is a BF16 number, so the dequantised weights are exact and the kernels below run
// the BF16 decode kernels' arithmetic (same K split, same MFMA order) on them.
//
// Decode layout (repacked at init). A "k-quad" is 128 consecutive K values = four
// 32-wide MFMA k-steps; lane l of a 16-row output tile holds row l % 16 and, for
// each k-step s of the quad, K values 32 s + 8 (l / 16) .. +7 as one dword (8
// codes), so one 16-byte load per lane brings four B fragments:
//   gate/up codes:  [E][f/16][d/128][gate|up][64 lanes][16 B]
//   gate/up scales: [E][f/16][d/128][gate|up][16 rows][4 k-steps]   (1 B each)
//   down codes:     [E][d/16][f/128][64 lanes][16 B]
//   down scales:    [E][d/16][f/128][16 rows][4 k-steps]
// A lane's four scales of one quad are one dword at row * 4.
#include "common.h"
#include "kernels.h"
#include "expert_device.h"
#include "mxfp4_device.h"

namespace beam {

__device__ __forceinline__ uint32_t ld_stream_u32(const void* p) {
  return __builtin_nontemporal_load((const uint32_t*)p);
}

// ---------------------------------------------------------------------------------------------
// Quantisation: one thread per block of 32 values of a row (mxfp4_quantize32).
__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(int64_t nblocks, const uint16_t* __restrict__ src,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks;
       b += (int64_t)gridDim.x * blockDim.x) {
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ld_u32x4(src + b * 32 + i * 8);
    u32x4 out;
    const uint32_t sbyte = mxfp4_quantize32(v, out);
    st_u32x4(codes + b * 16, out);
    scales[b] = (uint8_t)sbyte;
  }
}

hipError_t launch_mxfp4_quantize(int64_t nblocks, const uint16_t* src, uint8_t* codes,
                                 uint8_t* scales, hipStream_t s) {
  int64_t g = (nblocks + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(mxfp4_quantize_kernel, dim3((unsigned)g), dim3(256), 0, s, nblocks, src,
                     codes, scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Repack (init only): row-major codes [E][N][K/2] and scales [E][N][K/32] of NMAT
// matrices (gate, up: NMAT = 2, interleaved per quad; down: NMAT = 1) into the
// decode layout above.
__global__ void repack_mxfp4_kernel(const uint8_t* __restrict__ c0, const uint8_t* __restrict__ s0,
                                    const uint8_t* __restrict__ c1, const uint8_t* __restrict__ s1,
                                    int nmat, int E, int N, int K, uint8_t* __restrict__ qout,
                                    uint8_t* __restrict__ sout) {
  const int64_t NT = N / 16, KQ = K / 128;
  const int64_t total = (int64_t)E * NT * KQ * nmat * 64;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t lane = q % 64;
    int64_t r = q / 64;
    const int64_t m = r % nmat;
    r /= nmat;
    const int64_t kq = r % KQ;
    r /= KQ;
    const int64_t t = r % NT;
    const int64_t e = r / NT;
    const int64_t row = t * 16 + (lane & 15);
    const uint8_t* cs = (m ? c1 : c0) + (e * N + row) * (K / 2);
    const uint8_t* ss = (m ? s1 : s0) + (e * N + row) * (K / 32);
    u32x4 o;
#pragma unroll
    for (int s = 0; s < 4; ++s)  // k-step s: K values 128 kq + 32 s + 8 (lane / 16) .. +7
      o[s] = *(const uint32_t*)(cs + (128 * kq + 32 * s + 8 * (lane >> 4)) / 2);
    st_u32x4(qout + q * 16, o);
    if (lane < 16) {
      uint32_t sc = 0;
#pragma unroll
      for (int s = 0; s < 4; ++s) sc |= (uint32_t)ss[4 * kq + s] << (8 * s);
      const int64_t quad = q / 64;  // (e, t, kq, m)
      *(uint32_t*)(sout + quad * 64 + lane * 4) = sc;
    }
  }
}

hipError_t launch_repack_mxfp4(const uint8_t* gq, const uint8_t* gs, const uint8_t* uq,
                               const uint8_t* us, const uint8_t* dq, const uint8_t* ds, int E,
                               int f, int d, uint8_t* qgu, uint8_t* sgu, uint8_t* qd, uint8_t* sd,
                               hipStream_t s) {
  hipLaunchKernelGGL(repack_mxfp4_kernel, dim3(16384), dim3(256), 0, s, gq, gs, uq, us, 2, E, f, d,
                     qgu, sgu);
  hipLaunchKernelGGL(repack_mxfp4_kernel, dim3(16384), dim3(256), 0, s, dq, ds, dq, ds, 1, E, d, f,
                     qd, sd);
  return hipGetLastError();
}

// Repack (init only) into the grouped-GEMM layout of experts.hip: per (expert, n-tile of
// 256 stage columns, 32-wide K block) 4096 bytes of codes (column c at 16 c; the 8-value
// half h of k-step kk at ((h ^ ((c >> 4) & 1)) * 8 + kk * 4)) and 256 scale bytes. Stage
// columns: gate/up (gateup = 1) c < 128 gate row 128 nt + c, c >= 128 up row 128 nt + c -
// 128; down row 256 nt + c. One thread per (expert, n-tile, K block, column).
__global__ void repack_mxfp4_gemm_kernel(const uint8_t* __restrict__ c0, const uint8_t* __restrict__ s0,
                                         const uint8_t* __restrict__ c1, const uint8_t* __restrict__ s1,
                                         int gateup, int E, int N, int K, uint8_t* __restrict__ qout,
                                         uint8_t* __restrict__ sout) {
  const int64_t NT = gateup ? N / 128 : N / 256, KB = K / 32;
  const int64_t total = (int64_t)E * NT * KB * 256;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(q % 256);
    const int64_t blk = q / 256;  // (e, nt, kb)
    const int64_t kb = blk % KB, r = blk / KB;
    const int64_t nt = r % NT, e = r / NT;
    const bool up = gateup && c >= 128;
    const int64_t row = gateup ? nt * 128 + (c & 127) : nt * 256 + c;
    const uint8_t* rc = (up ? c1 : c0) + (e * N + row) * (K / 2) + kb * 16;
    // dword j of the block's 16 code bytes holds K values 8 j .. 8 j + 7 = k-step j / 2, half j % 2
    const int sw = (c >> 4) & 1;
    uint32_t dw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) dw[j] = *(const uint32_t*)(rc + 4 * j);
    uint32_t* dst = (uint32_t*)(qout + blk * 4096 + c * 16);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) dst[(h ^ sw) * 2 + kk] = dw[kk * 2 + h];
    sout[blk * 256 + c] = (up ? s1 : s0)[(e * N + row) * (K / 32) + kb];
  }
}

hipError_t launch_repack_mxfp4_gemm(const uint8_t* gq, const uint8_t* gs, const uint8_t* uq,
                                    const uint8_t* us, const uint8_t* dq, const uint8_t* ds,
                                    int E, int f, int d, uint8_t* pqgu, uint8_t* psgu,
                                    uint8_t* pqd, uint8_t* psd, hipStream_t s) {
  hipLaunchKernelGGL(repack_mxfp4_gemm_kernel, dim3(16384), dim3(256), 0, s, gq, gs, uq, us, 1, E,
                     f, d, pqgu, psgu);
  hipLaunchKernelGGL(repack_mxfp4_gemm_kernel, dim3(16384), dim3(256), 0, s, dq, ds, dq, ds, 0, E,
                     d, f, pqd, psd);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Gate/up: one workgroup per (active expert, NTW tiles of 16 outputs); the four
// waves split K into quarters (d/512 quads each) in wave order, each with a ring of
// U quads of code and scale loads in flight (slot u consumed, then refilled U quads
// ahead) for its NTW tiles, which share one activation fragment per k-step; the
// expert's rows (at most 16 MT per pass) ride along as the MFMA A operand through a
// buffer resource (rows past the count read zeros with no traffic). Per k-step:
// dequantise the gate and up fragments, then the MFMAs. Each output accumulates its
// k-steps in the BF16 kernel's order and the quarters are added in wave order, so
// the result equals the BF16 kernel's on the dequantised weights.
template <int MT, int U, int NTW>
__global__ __launch_bounds__(256) void gateup_fp4_kernel(ExpertArgs a) {
  const int NJ = a.f / 16, NB = NJ / NTW;
  const int j0 = (blockIdx.x % NB) * NTW;
  int row0, cnt;
  const int e = expert_of_block(a, blockIdx.x / NB, row0, cnt);
  if (e < 0) return;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KQ = a.d / 128, kqw = KQ / 4, kq0 = wv * kqw;
  const int64_t quad0 = ((int64_t)e * NJ + j0) * KQ + kq0;  // (expert, tile, quad) of this wave
  const int64_t tstride = (int64_t)KQ * 2;                 // quads of one tile (gate and up)
  const uint8_t* cp = a.qgu + quad0 * 2 * 1024 + lane * 16;
  const uint8_t* sp = a.sgu + quad0 * 2 * 64 + (lane & 15) * 4;
  const uint32_t zbytes = (uint32_t)a.T * a.d * 2;
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(a.z, zbytes);
  __shared__ f32x4 red[3][2 * MT * NTW][64];
  for (int m0 = 0; m0 < cnt; m0 += 16 * MT) {
    f32x4 ag[NTW][MT], au[NTW][MT];
    int pv[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        ag[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        au[t][mt] = ag[t][mt];
      }
      const int r = m0 + mt * 16 + (lane & 15);
      pv[mt] = a.perm[row0 + (r < cnt ? r : cnt - 1)];
    }
    __builtin_amdgcn_sched_barrier(0);
    uint32_t xo[MT];
    u32x4 cg[U][NTW], cu[U][NTW], x[MT][U][4];
    uint32_t sg[U][NTW], su[U][NTW];
    auto load_w = [&](int u, int kq) {
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int64_t q = t * tstride + kq * 2;
        cg[u][t] = ld_stream_u32x4(cp + q * 1024);
        cu[u][t] = ld_stream_u32x4(cp + q * 1024 + 1024);
        sg[u][t] = ld_stream_u32(sp + q * 64);
        su[u][t] = ld_stream_u32(sp + q * 64 + 64);
      }
    };
    auto load_x = [&](int u, int kq) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s) x[mt][u][s] = ld_buf_u32x4(zr, xo[mt] + (kq * 4 + s) * 64);
    };
    auto use = [&](int u) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const u32x4 bg = fp4x8_to_bf16(cg[u][t][s], e8m0_scale((sg[u][t] >> (8 * s)) & 255u));
          const u32x4 bu = fp4x8_to_bf16(cu[u][t][s], e8m0_scale((su[u][t] >> (8 * s)) & 255u));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            ag[t][mt] = mfma16(x[mt][u][s], bg, ag[t][mt]);
            au[t][mt] = mfma16(x[mt][u][s], bu, au[t][mt]);
          }
        }
    };
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load_w(u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = m0 + mt * 16 + (lane & 15);
      xo[mt] = r < cnt ? 2u * (uint32_t)((pv[mt] / a.k) * a.d + kq0 * 128 + 8 * (lane >> 4)) : zbytes;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load_x(u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int kq = 0; kq < kqw - U; kq += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        use(u);
        load_w(u, kq + U + u);
        load_x(u, kq + U + u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) use(u);
    if (wv > 0) {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          red[wv - 1][(t * MT + mt) * 2][lane] = ag[t][mt];
          red[wv - 1][(t * MT + mt) * 2 + 1][lane] = au[t][mt];
        }
    }
    __syncthreads();
    if (wv == 0) {
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4 g = ag[t][mt], u = au[t][mt];
#pragma unroll
          for (int w = 0; w < 3; ++w) {
            g += red[w][(t * MT + mt) * 2][lane];
            u += red[w][(t * MT + mt) * 2 + 1][lane];
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = m0 + mt * 16 + 4 * (lane >> 4) + i;
            if (r < cnt) {
              const float gv = bf2f(f2bf(g[i])), uv = bf2f(f2bf(u[i]));
              a.act[(int64_t)(row0 + r) * a.f + (j0 + t) * 16 + (lane & 15)] = f2bf(silu(gv) * uv);
            }
          }
        }
    }
    __syncthreads();
  }
}

// Single-token gate/up (T = 1, d / 4 <= 2048): gateup_fp4_kernel<1, U, 1>'s grid, split,
// k-step order and reduction, with the token row staged in LDS (one_row_load) so the
// register ring of U quads holds codes and scales only. Every row an expert holds at
// T = 1 is the one token, so the result is written to each of them. Same results bit
// for bit.
template <int U>
__global__ __launch_bounds__(256) void gateup_fp4_one_kernel(ExpertArgs a) {
  const int NJ = a.f / 16;
  const int j0 = blockIdx.x % NJ;
  const int e = active_expert(a, blockIdx.x / NJ);
  if (e < 0) return;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int KQ = a.d / 128, kqw = KQ / 4, kq0 = wv * kqw;
  const int64_t quad0 = ((int64_t)e * NJ + j0) * KQ + kq0;
  const uint8_t* cp = a.qgu + quad0 * 2 * 1024 + lane * 16;
  const uint8_t* sp = a.sgu + quad0 * 2 * 64 + (lane & 15) * 4;
  __shared__ u32x4 xs[4][kOneRowChunks * 64];
  __shared__ f32x4 red[3][2][64];
  one_row_load(xs[wv], a.z + kq0 * 128, kqw * 16, lane);  // the token is row 0 of z
  __builtin_amdgcn_sched_barrier(0);
  u32x4 cg[U], cu[U];
  uint32_t sg[U], su[U];
  auto load = [&](int u, int kq) {
    const int64_t q = (int64_t)kq * 2;
    cg[u] = ld_stream_u32x4(cp + q * 1024);
    cu[u] = ld_stream_u32x4(cp + q * 1024 + 1024);
    sg[u] = ld_stream_u32(sp + q * 64);
    su[u] = ld_stream_u32(sp + q * 64 + 64);
  };
#pragma unroll
  for (int u = 0; u < U; ++u) {
    load(u, u);
    __builtin_amdgcn_sched_barrier(0);
  }
  one_row_wait<4 * U>();
  const u32x4* xp = xs[wv] + (lane >> 4);
  f32x4 ag = f32x4{0.f, 0.f, 0.f, 0.f}, au = ag;
  auto use = [&](int u, int kq) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 x = xp[(kq * 4 + s) * 4];
      const u32x4 bg = fp4x8_to_bf16(cg[u][s], e8m0_scale((sg[u] >> (8 * s)) & 255u));
      const u32x4 bu = fp4x8_to_bf16(cu[u][s], e8m0_scale((su[u] >> (8 * s)) & 255u));
      ag = mfma16(x, bg, ag);
      au = mfma16(x, bu, au);
    }
  };
  for (int kq = 0; kq < kqw - U; kq += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      use(u, kq + u);
      load(u, kq + U + u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) use(u, kqw - U + u);
  if (wv > 0) {
    red[wv - 1][0][lane] = ag;
    red[wv - 1][1][lane] = au;
  }
  __syncthreads();
  if (wv == 0 && lane < 16) {  // output row 0 (lanes 0..15, element 0)
    int row0, cnt;
    expert_rows(a, e, row0, cnt);
    float g = ag[0], u = au[0];
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      g += red[w][0][lane][0];
      u += red[w][1][lane][0];
    }
    const float gv = bf2f(f2bf(g)), uv = bf2f(f2bf(u));
    const uint16_t v = f2bf(silu(gv) * uv);
    for (int r = 0; r < cnt; ++r) a.act[(int64_t)(row0 + r) * a.f + j0 * 16 + lane] = v;
  }
}

// Single-token down (T = 1, f / 4 <= 2048): down_split_fp4_kernel's K split and order over
// NTW 16-column tiles per wave (one at one token: twice the workgroups of the split kernel,
// measured faster), with the expert's activation row staged in LDS before the weights' first
// U quads are issued, and each row's slot written from the one sum.
// RT (4-bit activations): the row staged in LDS is the expert's BF16 activation row, and
// each wave replaces its quarter there by the MXFP4 round trip (OCP MX blocks of 32 along f)
// before the MFMAs, while its first weight quads are in flight; every workgroup of the expert
// computes the same values, and the one with column tile 0 also writes the row's codes
// (GEMM order) and scales to a.aq / a.aqs, as the separate round-trip pass does for more
// tokens.
template <int U, int NTW, bool RT>
__global__ __launch_bounds__(256) void down_fp4_one_kernel(ExpertArgs a) {
  const int ND = a.d / 16, NB = ND / NTW;
  const int nt0 = (blockIdx.x % NB) * NTW;
  const int e = active_expert(a, blockIdx.x / NB);
  if (e < 0) return;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int KQ = a.f / 128, kqw = KQ / 4, kq0 = wv * kqw;
  const int64_t quad0 = ((int64_t)e * ND + nt0) * KQ + kq0;
  const uint8_t* cp = a.qd + quad0 * 1024 + lane * 16;
  const uint8_t* sp = a.sd + quad0 * 64 + (lane & 15) * 4;
  __shared__ u32x4 xs[4][kOneRowChunks * 64];
  __shared__ f32x4 red[3][NTW][64];
  u32x4 c[U][NTW];
  uint32_t sc[U][NTW];
  auto load = [&](int u, int kq) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      c[u][t] = ld_stream_u32x4(cp + ((int64_t)t * KQ + kq) * 1024);
      sc[u][t] = ld_stream_u32(sp + ((int64_t)t * KQ + kq) * 64);
    }
  };
  // the row first (its address needs the expert's offset, a scalar load), then the weight
  // ring, which stays in flight while the row is waited for (and, with RT, rounded)
  int row0, cnt;
  expert_rows(a, e, row0, cnt);
  one_row_load(xs[wv], a.act + (int64_t)row0 * a.f + kq0 * 128, kqw * 16, lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    load(u, u);
    __builtin_amdgcn_sched_barrier(0);
  }
  one_row_wait<2 * NTW * U>();
  if constexpr (RT) {
    // chunk ch (values 8 ch .. of the quarter) by lane ch % 64: lanes 4 j .. 4 j + 3 hold a
    // block; the quarter's 16 kqw chunks are whole blocks, so each block's four lanes are
    // active together
    // (a token that names the expert more than once, under replayed routing, gives it
    // identical rows: each gets the codes)
    const bool keep = nt0 == 0;
    for (int ch = lane; ch < kqw * 16; ch += 64) {
      const int blk = kq0 * 4 + (ch >> 2);  // block of the row
      const u32x4 v = xs[wv][ch];
      xs[wv][ch] = mxfp4_block_rt_4lanes(v, a.aq + (int64_t)row0 * (a.f / 2) + blk * 16,
                                         a.aqs + (int64_t)row0 * (a.f / 32) + blk, keep);
      for (int r = 1; keep && r < cnt; ++r)
        (void)mxfp4_block_rt_4lanes(v, a.aq + (int64_t)(row0 + r) * (a.f / 2) + blk * 16,
                                    a.aqs + (int64_t)(row0 + r) * (a.f / 32) + blk, true);
    }
  }
  const u32x4* xp = xs[wv] + (lane >> 4);
  f32x4 acc[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto use = [&](int u, int kq) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 x = xp[(kq * 4 + s) * 4];
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        acc[t] = mfma16(x, fp4x8_to_bf16(c[u][t][s], e8m0_scale((sc[u][t] >> (8 * s)) & 255u)),
                        acc[t]);
    }
  };
  for (int kq = 0; kq < kqw - U; kq += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      use(u, kq + u);
      load(u, kq + U + u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) use(u, kqw - U + u);
  if (wv > 0) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) red[wv - 1][t][lane] = acc[t];
  }
  __syncthreads();
  if (wv == 0 && lane < 16) {
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      float v = acc[t][0];
#pragma unroll
      for (int w = 0; w < 3; ++w) v += red[w][t][lane][0];
      for (int r = 0; r < cnt; ++r) {
        const int slot = a.perm[row0 + r];
        a.yk[(int64_t)slot * a.d + (nt0 + t) * 16 + lane] = f2bf(a.w[slot] * v);
      }
    }
  }
}

// Down for batches up to 16 tokens: one workgroup per (active expert, NTW tiles of
// 16 output columns), the four waves split K (f) into quarters with a ring of U
// quads each; the quarters are added in wave order and bf16(w * sum) goes to the
// row's slot (the BF16 split kernel's order).
template <int U, int NTW>
__global__ __launch_bounds__(256) void down_split_fp4_kernel(ExpertArgs a) {
  const int ND = a.d / 16, NB = ND / NTW;
  const int nt0 = (blockIdx.x % NB) * NTW;
  int row0, cnt;
  const int e = expert_of_block(a, blockIdx.x / NB, row0, cnt);
  if (e < 0) return;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int KQ = a.f / 128, kqw = KQ / 4, kq0 = wv * kqw;
  const int64_t quad0 = ((int64_t)e * ND + nt0) * KQ + kq0;
  const uint8_t* cp = a.qd + quad0 * 1024 + lane * 16;
  const uint8_t* sp = a.sd + quad0 * 64 + (lane & 15) * 4;
  const uint32_t abytes = (uint32_t)a.T * a.k * a.f * 2;
  __shared__ f32x4 red[3][NTW][64];
  for (int m0 = 0; m0 < cnt; m0 += 16) {
    f32x4 acc[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int r = m0 + (lane & 15);
    const uint32_t xo = r < cnt ? 2u * (uint32_t)((row0 + r) * a.f + kq0 * 128 + 8 * (lane >> 4)) : abytes;
    u32x4 c[U][NTW], x[U][4];
    uint32_t sc[U][NTW];
    auto load = [&](int u, int kq) {
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        c[u][t] = ld_stream_u32x4(cp + ((int64_t)t * KQ + kq) * 1024);
        sc[u][t] = ld_stream_u32(sp + ((int64_t)t * KQ + kq) * 64);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
        x[u][s] = xo < abytes ? ld_u32x4((const char*)a.act + xo + (kq * 4 + s) * 64)
                              : u32x4{0u, 0u, 0u, 0u};
    };
    auto use = [&](int u) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int t = 0; t < NTW; ++t)
          acc[t] = mfma16(x[u][s], fp4x8_to_bf16(c[u][t][s], e8m0_scale((sc[u][t] >> (8 * s)) & 255u)),
                          acc[t]);
    };
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load(u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int kq = 0; kq < kqw - U; kq += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        use(u);
        load(u, kq + U + u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) use(u);
    if (wv > 0) {
#pragma unroll
      for (int t = 0; t < NTW; ++t) red[wv - 1][t][lane] = acc[t];
    }
    __syncthreads();
    if (wv == 0) {
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        f32x4 v = acc[t];
#pragma unroll
        for (int w = 0; w < 3; ++w) v += red[w][t][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = m0 + 4 * (lane >> 4) + i;
          if (rr < cnt) {
            const int slot = a.perm[row0 + rr];
            a.yk[(int64_t)slot * a.d + (nt0 + t) * 16 + (lane & 15)] = f2bf(a.w[slot] * v[i]);
          }
        }
      }
    }
    __syncthreads();
  }
}

// Down for 17..128 tokens: a workgroup covers 4 NTW output tiles of 16 columns of
// one expert, each wave NTW tiles accumulating the full K in order (the BF16
// streaming kernel's order) through a ring of U quads.
template <int MT, int U, int NTW>
__global__ __launch_bounds__(256) void down_stream_fp4_kernel(ExpertArgs a) {
  const int ND = a.d / 16, NB = ND / (4 * NTW);
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nt0 = (blockIdx.x % NB) * 4 * NTW + wv * NTW;
  int row0, cnt;
  const int e = expert_of_block(a, blockIdx.x / NB, row0, cnt);
  if (e < 0) return;
  const int KQ = a.f / 128;
  const int64_t quad0 = ((int64_t)e * ND + nt0) * KQ;
  const uint8_t* cp = a.qd + quad0 * 1024 + lane * 16;
  const uint8_t* sp = a.sd + quad0 * 64 + (lane & 15) * 4;
  for (int m0 = 0; m0 < cnt; m0 += 16 * MT) {
    f32x4 acc[NTW][MT];
    const uint16_t* ap[MT];
    bool av[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int t = 0; t < NTW; ++t) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = m0 + mt * 16 + (lane & 15);
      av[mt] = r < cnt;
      ap[mt] = a.act + (int64_t)(row0 + (av[mt] ? r : 0)) * a.f + 8 * (lane >> 4);
    }
    u32x4 c[U][NTW], x[MT][U][4];
    uint32_t sc[U][NTW];
    auto load = [&](int u, int kq) {
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        c[u][t] = ld_stream_u32x4(cp + ((int64_t)t * KQ + kq) * 1024);
        sc[u][t] = ld_stream_u32(sp + ((int64_t)t * KQ + kq) * 64);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          x[mt][u][s] = av[mt] ? ld_u32x4(ap[mt] + (kq * 4 + s) * 32) : u32x4{0u, 0u, 0u, 0u};
    };
    auto use = [&](int u) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const u32x4 b = fp4x8_to_bf16(c[u][t][s], e8m0_scale((sc[u][t] >> (8 * s)) & 255u));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[t][mt] = mfma16(x[mt][u][s], b, acc[t][mt]);
        }
    };
#pragma unroll
    for (int u = 0; u < U; ++u) {
      load(u, u);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int kq = 0; kq < KQ - U; kq += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        use(u);
        load(u, kq + U + u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) use(u);
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = m0 + mt * 16 + 4 * (lane >> 4) + i;
          if (r < cnt) {
            const int slot = a.perm[row0 + r];
            a.yk[(int64_t)slot * a.d + (nt0 + t) * 16 + (lane & 15)] = f2bf(a.w[slot] * acc[t][mt][i]);
          }
        }
  }
}

// Launches: the grids are sized for the largest possible number of active experts;
// workgroups past the active count exit at once. Needs d % 512 == 0 and f % 512 == 0
// (whole quads per wave quarter; tile counts divisible by the tiles per workgroup).
// Every pass uses 16-row MFMA blocks: rows do not interact in an MFMA, so the block
// height changes no result, and most experts hold few rows at these batch sizes.
// Tiles per wave and ring depths (measured on Beam's shapes): gate/up one tile per
// wave up to 16 tokens (more workgroups for the few experts), two above; down two
// tiles per wave up to 16 tokens, four above with a ring of two quads. One token takes
// the single-token kernels (row in LDS) with rings of five quads (half of a gate/up
// wave's quarter, all of a down wave's) and one down tile per wave: with the row out
// of the ring, deeper rings keep the occupancy that rows in registers cost.
hipError_t launch_gateup_fp4(const ExpertArgs& a, int max_active, hipStream_t s) {
  const int kqw = a.d / 128 / 4;  // >= 1; U = 2 when it divides
  if (a.T == 1 && kqw * 16 <= kOneRowChunks * 64) {
    dim3 g((unsigned)(max_active * (a.f / 16))), blk(256);
    if (kqw % 5 == 0)
      hipLaunchKernelGGL((gateup_fp4_one_kernel<5>), g, blk, 0, s, a);
    else if (kqw % 2 == 0)
      hipLaunchKernelGGL((gateup_fp4_one_kernel<2>), g, blk, 0, s, a);
    else
      hipLaunchKernelGGL((gateup_fp4_one_kernel<1>), g, blk, 0, s, a);
  } else if (a.T <= 16) {
    dim3 g((unsigned)(max_active * (a.f / 16))), blk(256);
    if (kqw % 2 == 0)
      hipLaunchKernelGGL((gateup_fp4_kernel<1, 2, 1>), g, blk, 0, s, a);
    else
      hipLaunchKernelGGL((gateup_fp4_kernel<1, 1, 1>), g, blk, 0, s, a);
  } else {
    dim3 g((unsigned)(max_active * (a.f / 32))), blk(256);
    if (kqw % 2 == 0)
      hipLaunchKernelGGL((gateup_fp4_kernel<1, 2, 2>), g, blk, 0, s, a);
    else
      hipLaunchKernelGGL((gateup_fp4_kernel<1, 1, 2>), g, blk, 0, s, a);
  }
  return hipGetLastError();
}

bool down_fp4_rounds_act(const ExpertArgs& a) {
  return a.aq != nullptr && a.T == 1 && (a.f / 128 / 4) * 16 <= kOneRowChunks * 64;
}

template <bool RT>
static void launch_down_fp4_one(const ExpertArgs& a, int max_active, hipStream_t s) {
  const int kqw = a.f / 128 / 4;
  dim3 g((unsigned)(max_active * (a.d / 16))), blk(256);
  if (kqw % 5 == 0)
    hipLaunchKernelGGL((down_fp4_one_kernel<5, 1, RT>), g, blk, 0, s, a);
  else if (kqw % 2 == 0)
    hipLaunchKernelGGL((down_fp4_one_kernel<2, 1, RT>), g, blk, 0, s, a);
  else
    hipLaunchKernelGGL((down_fp4_one_kernel<1, 1, RT>), g, blk, 0, s, a);
}

hipError_t launch_down_fp4(const ExpertArgs& a, int max_active, hipStream_t s) {
  const int kqw = a.f / 128 / 4;
  if (a.T == 1 && kqw * 16 <= kOneRowChunks * 64) {
    if (down_fp4_rounds_act(a)) launch_down_fp4_one<true>(a, max_active, s);
    else launch_down_fp4_one<false>(a, max_active, s);
  } else if (a.T <= kSplitDownMaxT) {
    dim3 g((unsigned)(max_active * (a.d / 32))), blk(256);
    hipLaunchKernelGGL((down_split_fp4_kernel<1, 2>), g, blk, 0, s, a);
  } else {
    const int KQ = a.f / 128;
    dim3 g((unsigned)(max_active * (a.d / 256))), blk(256);
    if (KQ % 2 == 0)
      hipLaunchKernelGGL((down_stream_fp4_kernel<1, 2, 4>), g, blk, 0, s, a);
    else
      hipLaunchKernelGGL((down_stream_fp4_kernel<1, 1, 4>), g, blk, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace beam
