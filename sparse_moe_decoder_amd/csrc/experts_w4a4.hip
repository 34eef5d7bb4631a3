// Routed SwiGLU experts with 4-bit weights AND 4-bit activations (W4A4) on the scaled
// FP4 matrix cores of gfx950.
//
// [vLLM "Serving Reflection Beam auf vLLM ab Tag 0", §Der fusionierte Graph] the 4-bit
//   MoE path quantises the activations, then runs the two grouped GEMMs on the 4-bit
//   experts; [§Modellarchitektur] the routed experts are 4-bit.
// Both GEMM inputs an expert multiplies by its weights are MXFP4 (OCP Microscaling
// Formats v1.0: E2M1 codes, one E8M0 scale per 32 consecutive K values): the token rows z
// (quantised along d before gate/up) and the activations act (quantised along f in the
// gate/up epilogue, the down GEMM's input). v_mfma_scale_f32_32x32x64_f8f6f4 multiplies
// such operands directly: lane l holds row (A) or column (B) l % 32 and the 32 K values
// 32 (l / 32) .. +31 of the 64-wide K step as 16 code bytes, plus that block's scale byte;
// every product of two E2M1 values times the two scales is exact, so each 32-value block
// contributes its exact dot product and only the FP32 accumulation rounds.
//
// Code byte order inside a block's 16 bytes ("GEMM order", gemm_order in mxfp4_device.h):
// dword p holds K values 8 q .. 8 q + 7 with q = (0, 2, 1, 3)[p] — the order the 4-bit
// weights of the grouped-GEMM layout (experts.hip) have once a lane undoes their half swap,
// so A and B lanes agree.
//
// The GEMM is the BF16 engine's (experts.hip) with a 128-wide K block per LDS stage
// instead of 32: 256 x 256 tiles per 8-wave workgroup, wave w = 4 wm + wn owning 32-row
// tiles 2 mt + wm (mt < MW) x two 32-column tiles, two 64-wide MFMA K steps per stage.
// Stage (34 KB; four stages): A codes 256 rows x 64 B (chunk c of row r in slot
// c ^ ((r / 4) % 4)), A scales 256 rows x 4 B (the row's four block scales), B codes 4 K
// blocks x 4 KB and B scales 4 x 256 B copied verbatim from the weight layout. Each wave
// issues five direct-to-LDS copies per stage: two of A codes, two of B codes, and one of
// 4 bytes per lane holding A scales (waves 0-3) or B scales (waves 4-7). The K loop has no
// branch: past the last K block the copies repeat it into the stage just freed.
#include "common.h"
#include "kernels.h"
#include "gemm_device.h"
#include "mxfp4_device.h"

#include <type_traits>

namespace beam {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

// ---------------------------------------------------------------------------------------------
// Token-row quantisation: z [T, d] BF16 -> codes [T, d/2] (GEMM order) and scales [T, d/32];
// with rt, also the rows' exact round trip (the dequantised codes) as BF16 [T, d]. One thread
// per block of 32 values.
__global__ __launch_bounds__(256) void quantize_rows_a4_kernel(int64_t nblocks, const uint16_t* __restrict__ src,
                                                               uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales,
                                                               uint16_t* __restrict__ rt) {
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks;
       b += (int64_t)gridDim.x * blockDim.x) {
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ld_u32x4(src + b * 32 + i * 8);
    mxfp4_block_out(v, codes + b * 16, scales + b, rt ? rt + b * 32 : nullptr);
  }
}

hipError_t launch_quantize_rows_a4(int64_t nblocks, const uint16_t* src, uint8_t* codes,
                                   uint8_t* scales, uint16_t* rt, hipStream_t s) {
  int64_t g = (nblocks + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(quantize_rows_a4_kernel, dim3((unsigned)g), dim3(256), 0, s, nblocks, src,
                     codes, scales, rt);
  return hipGetLastError();
}

// The activations of the weight-streaming passes (T <= 128), quantised in place: each valid
// row of act [rows, f] BF16 (expert-grouped order; *nvalid rows are valid) is replaced by its
// MXFP4 round trip, and its codes (GEMM order) and scales are kept in codes / scales — the
// values and codes the W4A4 GEMM epilogue produces from the same BF16 activations.
__global__ __launch_bounds__(256) void act_round_trip_a4_kernel(int64_t nblocks, int f,
                                                                const int32_t* __restrict__ nvalid,
                                                                uint16_t* __restrict__ act,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales) {
  const int64_t bpr = f / 32;
  const int64_t nb = (int64_t)(*nvalid) * bpr;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks && b < nb;
       b += (int64_t)gridDim.x * blockDim.x) {
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ld_u32x4(act + b * 32 + i * 8);
    mxfp4_block_out(v, codes + b * 16, scales + b, act + b * 32);
  }
}

hipError_t launch_act_round_trip_a4(int64_t rows, int f, const int32_t* nvalid, uint16_t* act,
                                    uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t nblocks = rows * (f / 32);
  int64_t g = (nblocks + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(act_round_trip_a4_kernel, dim3((unsigned)g), dim3(256), 0, s, nblocks, f,
                     nvalid, act, codes, scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// The W4A4 grouped GEMM

constexpr int QBM = kGemmBM, QBK = 128, QNS = 4;
constexpr int QA = QBM * 64, QAS = QBM * 4, QB = 4 * 4096, QBS = 4 * 256;
constexpr int QSTAGE = QA + QAS + QB + QBS;  // 34 KB
static_assert(QNS * QSTAGE <= 160 * 1024, "LDS");
static_assert(QBM * 256 * 2 + QBM * 8 <= QNS * QSTAGE, "down epilogue staging");

// s_waitcnt vmcnt(5 n): at most n K blocks of this wave's copies (five each) in flight
__device__ __forceinline__ void wait_blocks5(int n) {
  if (n >= 2) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ f32x16 mfma_fp4(const u32x4& a, uint32_t sa, const u32x4& b,
                                           uint32_t sb, f32x16 c) {
  const i32x8 A = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const i32x8 B = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// SKIP: this wave's last 32-row tile is empty (an odd number of 32-row tiles leaves wm = 1 one
// tile short), so its MFMAs are left out.
template <bool GATEUP, int MW, bool SKIP>
__device__ __forceinline__ void gemm_a4_tile_body(const ExpertArgs& a, const GemmTile& t,
                                                  uint8_t* smem) {
  constexpr int NW = 8;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int wm = wvu >> 2, wn = wvu & 3;
  const int K = GATEUP ? a.d : a.f;
  const int nkb = K / QBK;  // any count: the loop is not unrolled by stages
  const int e = t.e, row0 = t.row0, rows = t.rows, nb = t.nb;

  // A codes: wave w fills rows [32 w, 32 w + 32) with 2 copies of 16 rows; lane l covers
  // row 16 i + l / 4, slot l % 4, which holds chunk (l % 4) ^ ((r / 4) % 4) of the row
  const uint8_t* abase = GATEUP ? a.zq : a.aq;
  const uint8_t* asbase = GATEUP ? a.zqs : a.aqs;
  const int arow_b = K / 2, arow_s = K / 32;  // bytes per row: codes, scales
  int64_t aoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = wv * 32 + i * 16 + (lane >> 2);
    const int rr = r < rows ? r : 0;
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    const int64_t src_row = GATEUP ? (int64_t)(a.perm[row0 + rr] / a.k) : (int64_t)(row0 + rr);
    aoff[i] = src_row * arow_b + c * 16;
  }
  // B: the weight layout's (expert, n-tile, 32-wide K block) blocks, four per stage
  const int NTL = GATEUP ? a.f / 128 : a.d / 256;
  const int64_t blk0 = ((int64_t)e * NTL + nb) * (K / 32);
  const uint8_t* bq = (GATEUP ? a.pqgu : a.pqd) + blk0 * 4096 + wv * 2048 + lane * 16;
  // scales, 4 bytes per lane and stage: waves 0-3 A's (lane l: row 64 w + l, its four block
  // scales of the stage, sc_step bytes per stage), waves 4-7 B's (scale block w - 4 of the
  // stage's four, 1024 bytes per stage)
  const uint8_t* sc_src;
  int sc_step;
  uint32_t sc_dst;
  if (wvu < 4) {
    const int r = wv * 64 + lane;
    const int rr = r < rows ? r : 0;
    const int64_t src_row = GATEUP ? (int64_t)(a.perm[row0 + rr] / a.k) : (int64_t)(row0 + rr);
    sc_src = asbase + src_row * arow_s;
    sc_step = 4;
    sc_dst = QA + wvu * 256;
  } else {
    sc_src = (GATEUP ? a.psgu : a.psd) + blk0 * 256 + (wvu - 4) * 256 + lane * 4;
    sc_step = 4 * 256;
    sc_dst = QA + QAS + QB + (wvu - 4) * 256;
  }

  // down: thread r < 256 holds row r's slot and routing weight for the epilogue
  int my_slot = 0;
  float my_w = 0.0f;
  if (!GATEUP && tid < QBM && tid < rows) {
    my_slot = a.perm[row0 + tid];
    my_w = a.w[my_slot];
  }

  auto st_base = [&](int st) -> uint8_t* { return smem + st * QSTAGE; };
  // copy p of K block kb into stage st: 0, 1 A codes; 2, 3 B codes; 4 A or B scales
  auto issue = [&](int kb, int st, int p) {
    uint8_t* S = st_base(st);
    if (p < 2) {
      lds_dma16((const uint16_t*)(abase + aoff[p] + kb * 64),
                lds_addr(S) + (uint32_t)(wvu * 32 * 64) + p * 16 * 64);
    } else if (p < 4) {
      lds_dma16((const uint16_t*)(bq + (int64_t)kb * 4 * 4096 + (p - 2) * 1024),
                lds_addr(S + QA + QAS) + (uint32_t)(wvu * 2048) + (p - 2) * 1024);
    } else {
      lds_dma4(sc_src + (int64_t)kb * sc_step, lds_addr(S) + sc_dst);
    }
  };

  const int l32 = lane & 31, lh = lane >> 5;
  // fragment read offsets: A row m = (2 mt + wm) 32 + l32 (mt added per tile), chunk 2 s + lh
  int ar[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int m = wm * 32 + l32;
    ar[s] = m * 64 + (((2 * s + lh) ^ ((m >> 2) & 3)) << 4);
  }
  // B column of this lane's N tile nn (gate/up: 128 gate then 128 up stage columns). The
  // weight layout swaps the 8-byte halves of columns with bit 4 set; the fragment is read as
  // two 8-byte halves from swapped offsets, which puts them back in order and keeps each
  // read free of bank conflicts (the swap exists for that).
  int bc[2], blo[2], bhi[2];
#pragma unroll
  for (int nn = 0; nn < 2; ++nn) {
    bc[nn] = GATEUP ? nn * 128 + 32 * wn + l32 : 64 * wn + 32 * nn + l32;
    const int sw = ((bc[nn] >> 4) & 1) * 8;
    blo[nn] = bc[nn] * 16 + sw;
    bhi[nn] = bc[nn] * 16 + 8 - sw;
  }

  f32x16 acc[MW][2];
#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  constexpr int CP = 5;
  auto compute = [&](int st, int kb) {
    const uint8_t* S = st_base(st);
    const uint8_t* SA = S;
    const uint8_t* SAS = S + QA;
    const uint8_t* SB = S + QA + QAS;
    const uint8_t* SBS = S + QA + QAS + QB;
    const int kn = min(kb + QNS - 1, nkb - 1), sn = (st + QNS - 1) % QNS;
    int q = 0;  // MFMA groups done, for placing the next block's copies
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int b = 2 * s + lh;  // this lane's 32-wide block of the stage
      u32x4 fb[2];
      uint32_t sb[2];
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) {
        const uint2 lo = *(const uint2*)(SB + b * 4096 + blo[nn]);
        const uint2 hi = *(const uint2*)(SB + b * 4096 + bhi[nn]);
        fb[nn] = u32x4{lo.x, lo.y, hi.x, hi.y};
        sb[nn] = SBS[b * 256 + bc[nn]];
      }
      u32x4 fa[MW];
      uint32_t sa[MW];
#pragma unroll
      for (int mt = 0; mt < MW; ++mt) {
        fa[mt] = ld_u32x4(SA + ar[s] + mt * 64 * 64);
        const int m = (2 * mt + wm) * 32 + l32;
        sa[mt] = (*(const uint32_t*)(SAS + m * 4) >> (8 * b)) & 0xFFu;
      }
#pragma unroll
      for (int mt = 0; mt < MW; ++mt) {
        if (mt + 1 < MW || !SKIP) {
#pragma unroll
          for (int nn = 0; nn < 2; ++nn)
            acc[mt][nn] = mfma_fp4(fa[mt], sa[mt], fb[nn], sb[nn], acc[mt][nn]);
        }
        if (q < CP) {
          __builtin_amdgcn_sched_barrier(0);
          issue(kn, sn, q);
          __builtin_amdgcn_sched_barrier(0);
          ++q;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (; q < CP; ++q) issue(kn, sn, q);
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: stages 0 .. QNS - 2 (blocks past the last repeat it)
#pragma unroll
  for (int j = 0; j < QNS - 1; ++j)
#pragma unroll
    for (int p = 0; p < CP; ++p) issue(min(j, nkb - 1), j, p);
  for (int kb = 0; kb < nkb; ++kb) {
    wait_blocks5(QNS - 2);  // blocks kb + 1 .. kb + QNS - 2 (or repeats) stay in flight
    __builtin_amdgcn_s_barrier();
    compute(kb % QNS, kb);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // epilogue through LDS
  if (GATEUP) {
    // act tile [256 rows][128 q] BF16, row-major (the quantiser reads whole 32-value row
    // blocks, one per thread); wave (wm, wn) holds 32-row tiles 2 mt + wm, q [32 wn, +32)
    uint16_t* stage = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (2 * mt + wm) * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int qq = wn * 32 + l32;
        const float gv = bf2f(f2bf(acc[mt][0][r])), uv = bf2f(f2bf(acc[mt][1][r]));
        stage[row * 128 + qq] = f2bf(silu(gv) * uv);
      }
    }
    __syncthreads();
    // quantise each row's four 32-value blocks of this tile (MXFP4, GEMM order)
    for (int u = tid; u < rows * 4; u += 64 * NW) {
      const int r = u >> 2, j = u & 3;
      u32x4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = ld_u32x4(&stage[r * 128 + j * 32 + i * 8]);
      u32x4 out;
      const uint32_t sbyte = mxfp4_quantize32(v, out);
      const int64_t row = row0 + r;
      st_u32x4(a.aq + row * (a.f / 2) + nb * 64 + j * 16, gemm_order(out));
      a.aqs[row * (a.f / 32) + nb * 4 + j] = (uint8_t)sbyte;
    }
  } else {
    // output tile [256 rows][256 cols] BF16, weighted; the rows' weights and slots behind it
    uint16_t* stage = reinterpret_cast<uint16_t*>(smem);
    float* w_row = reinterpret_cast<float*>(stage + QBM * 256);
    int* slot_row = reinterpret_cast<int*>(w_row + QBM);
    if (tid < QBM) {
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
    // copy-out through row quads (quad_store / quad_rows in gemm_device.h)
    const int nq = (rows + 3) >> 2;
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

template <bool GATEUP, int MW>
__device__ __forceinline__ void gemm_a4_tile_skip(const ExpertArgs& a, const GemmTile& t, uint8_t* smem,
                                                  bool skip) {
  if (skip) gemm_a4_tile_body<GATEUP, MW, true>(a, t, smem);
  else gemm_a4_tile_body<GATEUP, MW, false>(a, t, smem);
}

template <bool GATEUP>
__global__ __launch_bounds__(512) void grouped_gemm_a4_kernel(ExpertArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[QNS * QSTAGE];
  const int NT = GATEUP ? a.f / 128 : a.d / 256;
  const int total = a.tile_start[a.E] * NT;
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int R = (total + 7) >> 3;
  const int L = xcd * R + q;
  if (q >= R || L >= total) return;
  const GemmTile t = decode_tile(a, NT, L);
  const int n32 = (t.rows + 31) >> 5;  // 32-row tiles: wm = 0 takes the even ones, wm = 1 the odd
  const int wm = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) >> 2;
  const bool skip = (n32 & 1) && wm == 1;
  switch ((n32 + 1) >> 1) {
    case 1: gemm_a4_tile_skip<GATEUP, 1>(a, t, smem, skip); break;
    case 2: gemm_a4_tile_skip<GATEUP, 2>(a, t, smem, skip); break;
    case 3: gemm_a4_tile_skip<GATEUP, 3>(a, t, smem, skip); break;
    default: gemm_a4_tile_skip<GATEUP, 4>(a, t, smem, skip); break;
  }
}

hipError_t launch_gateup_gemm_a4(const ExpertArgs& a, int max_tiles, hipStream_t s) {
  const unsigned gx = (unsigned)(8 * ((max_tiles * (a.f / 128) + 7) / 8));
  hipLaunchKernelGGL(grouped_gemm_a4_kernel<true>, dim3(gx), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_gemm_a4(const ExpertArgs& a, int max_tiles, hipStream_t s) {
  const unsigned gx = (unsigned)(8 * ((max_tiles * (a.d / 256) + 7) / 8));
  hipLaunchKernelGGL(grouped_gemm_a4_kernel<false>, dim3(gx), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace beam
