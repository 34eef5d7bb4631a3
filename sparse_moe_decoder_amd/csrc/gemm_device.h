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
