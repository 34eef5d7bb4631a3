// Device helpers shared by the grouped GEMMs (BF16 and 4-bit weights in experts.hip, 4-bit
// activations in experts_w4a4.hip): direct global-to-LDS copies, the tile list and its
// decoding.
#pragma once
#include "common.h"
#include "kernels.h"

namespace beam {

// Direct global-to-LDS load of 16 bytes per lane: lane l's bytes land at LDS byte
// address lds + 16 l (lds must be wave-uniform). Issued as inline assembly so the
// compiler does not add its own conservative waits on the stage buffers; the
// kernel waits explicitly (vmcnt) before a stage is read. The asm sets m0 (the LDS
// base of the copy) and lists it as clobbered; the compiler warns that it does not
// save m0 around the asm, which is safe here because on gfx950 these kernels hold
// no value in m0 (LDS reads and writes do not use it; nothing else here does).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_dma16(const uint16_t* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}

// 4 bytes per lane, global to LDS: lane l's dword lands at LDS byte address lds + 4 l.
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}

// Epilogue staging of a GEMM output tile in row quads. A 32x32 MFMA result holds, in lane l
// and register 4 i + j, row 8 i + 4 (l / 32) + j and column l % 32 of its tile: four
// consecutive rows of one column. The tile (NC columns) is staged with element (row, col) at
// half-word ((row / 4) NC + col) 4 + row % 4, so those four values are one 8-byte LDS write
// (a quarter of the write instructions of a row-major tile), and a 4-row x 8-column block is
// 64 contiguous bytes, which quad_rows regroups into the four rows' 16-byte chunks.
template <int NC>
__device__ __forceinline__ void quad_store(uint16_t* stage, int rq, int col, uint32_t rows01,
                                           uint32_t rows23) {
  *reinterpret_cast<uint2*>(stage + ((rq * NC) + col) * 4) = make_uint2(rows01, rows23);
}

// Rows 4 q .. 4 q + 3, columns 8 k .. 8 k + 7 of a row-quad tile: out[j] is row 4 q + j's
// 16-byte chunk (column 8 k + c in half-word c). Column m of the block sits in dwords 2 m and
// 2 m + 1 (rows 0-1, 2-3); v_perm_b32 takes one half-word from each of two such dwords.
template <int NC>
__device__ __forceinline__ void quad_rows(const uint16_t* stage, int q, int k, u32x4 out[4]) {
  const u32x4* src = reinterpret_cast<const u32x4*>(stage + (q * NC + k * 8) * 4);
  const u32x4 b[4] = {src[0], src[1], src[2], src[3]};
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int p = 0; p < 4; ++p)  // columns 2 p (low half-word) and 2 p + 1
      out[j][p] = __builtin_amdgcn_perm(b[p][2 + (j >> 1)], b[p][j >> 1],
                                        (j & 1) ? 0x07060302u : 0x05040100u);
}

// One tile of a grouped GEMM: expert e, its rows [row0, row0 + rows) in the expert-grouped
// order, column tile nb.
struct GemmTile {
  int e, row0, rows, nb;
};

// An XCD runs 32 workgroups at a time; blocks of 8 m-tiles put about 8 m-tiles x 4
// n-tiles in flight for an expert with many rows, so its row tiles and weight
// tiles are each re-read from L2 by several concurrent tiles (measured on a skewed
// 32K-token batch: -4 % gate/up, -15 % down against n-tile-major order).
constexpr int kGemmMBlock = 8;

// Tile number L of the list above
__device__ __forceinline__ GemmTile decode_tile(const ExpertArgs& a, int NT, int L) {
  // expert: largest e with tile_start[e] * NT <= L
  int lo = 0, hi = a.E;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (a.tile_start[mid] * NT <= L) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int mtiles = a.tile_start[e + 1] - a.tile_start[e];
  const int within = L - a.tile_start[e] * NT;
  const int cnt = a.offsets[e + 1] - a.offsets[e];
  // equal tiles, a multiple of 32 rows each (at most GBM; the last one is not empty)
  const int per = (((cnt + mtiles - 1) / mtiles) + 31) & ~31;
  // an expert's tiles in blocks of up to kGemmMBlock m-tiles: block by block, each
  // n-tile with the block's m-tiles (an expert of at most kGemmMBlock m-tiles is one
  // block: n-tile by n-tile, all its m-tiles)
  int mi, ni;
  const int nfull = mtiles / kGemmMBlock;
  if (within < nfull * NT * kGemmMBlock) {
    const int mb = within / (NT * kGemmMBlock), r = within % (NT * kGemmMBlock);
    ni = r / kGemmMBlock;
    mi = mb * kGemmMBlock + r % kGemmMBlock;
  } else {
    const int rem = mtiles - nfull * kGemmMBlock, r = within - nfull * NT * kGemmMBlock;
    ni = r / rem;
    mi = nfull * kGemmMBlock + r % rem;
  }
  GemmTile t;
  t.e = e;
  t.nb = ni;
  t.row0 = a.offsets[e] + mi * per;
  t.rows = min(per, a.offsets[e + 1] - t.row0);
  return t;
}

}  // namespace beam
