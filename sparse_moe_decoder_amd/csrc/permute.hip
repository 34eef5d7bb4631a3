// Expert histogram, offsets and the stable expert-grouped permutation.
//
// [vLLM "Serving Reflection Beam auf vLLM ab Tag 0", §Der fusionierte Graph]
//   the MoE path runs routing kernels ahead of two grouped GEMMs, i.e. the
//   T*k token assignments ("slots" t*k+j) are grouped by expert. The layout is
//   this library's own: rows ordered by expert ascending, then slot ascending.
//
// Determinism: the position of every slot follows from counts alone — per-block
// histograms (LDS atomics only count, they do not order), a block-ordered scan,
// and in-block ranks from wavefront ballots — so the permutation is the same on
// every run.
#include "common.h"
#include "kernels.h"

namespace beam {

__device__ __forceinline__ bool valid_id(int e, int E) { return e >= 0 && e < E; }

// LDS-atomic histogram of one chunk
__device__ void chunk_hist(const PermArgs& a, int b, int* cnt) {
  for (int e = threadIdx.x; e < 256; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int s0 = b * kPermChunk;
  for (int q = threadIdx.x; q < kPermChunk; q += blockDim.x) {
    int s = s0 + q;
    if (s < a.n) {
      int e = a.ids[s];
      if (valid_id(e, a.E)) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void perm_hist_kernel(PermArgs a) {
  __shared__ int cnt[256];
  chunk_hist(a, blockIdx.x, cnt);
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) a.block_cnt[blockIdx.x * a.E + e] = cnt[e];
}

// One block: per-expert running sums over blocks, offsets, active list, tile table.
__device__ void scan_all(const PermArgs& a) {
  __shared__ int tot[257];
  __shared__ int excl[257];
  const int e = threadIdx.x;
  int run = 0;
  if (e < a.E) {
    for (int b = 0; b < a.nb; ++b) {
      int c = a.block_cnt[b * a.E + e];
      a.block_base[b * a.E + e] = run;
      run += c;
    }
    a.counts[e] = run;
  }
  tot[e] = (e < a.E) ? run : 0;
  __syncthreads();
  if (e == 0) {
    int acc = 0, na = 0, tiles = 0;
    for (int x = 0; x < a.E; ++x) {
      excl[x] = acc;
      a.offsets[x] = acc;
      if (a.offsets2) a.offsets2[x] = acc;
      a.tile_start[x] = tiles;
      if (tot[x] > 0) a.active[na++] = x;
      acc += tot[x];
      tiles += (tot[x] + a.bm - 1) / a.bm;
    }
    excl[a.E] = acc;
    a.offsets[a.E] = acc;
    if (a.offsets2) a.offsets2[a.E] = acc;
    a.tile_start[a.E] = tiles;
    *a.n_active = na;
  }
  __syncthreads();
  if (e < a.E)
    for (int b = 0; b < a.nb; ++b) a.block_base[b * a.E + e] += excl[e];
  // rows past the valid ones (slots with invalid ids) read as -1
  for (int r = excl[a.E] + threadIdx.x; r < a.n; r += blockDim.x) {
    a.perm[r] = -1;
    if (a.perm2) a.perm2[r] = -1;
  }
}

__global__ __launch_bounds__(256) void perm_scan_kernel(PermArgs a) { scan_all(a); }

// Stable scatter of one chunk: slots are taken 256 at a time in order; within a
// wave, a slot's rank among earlier lanes with the same expert comes from a
// ballot-built match mask; waves are ordered through per-wave counts in LDS.
__device__ void chunk_scatter(const PermArgs& a, int b) {
  __shared__ int wave_cnt[4][256];
  __shared__ int running[256];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  for (int e = tid; e < 256; e += 256) {
    running[e] = 0;
    for (int w = 0; w < 4; ++w) wave_cnt[w][e] = 0;
  }
  __syncthreads();
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int round = 0; round < kPermChunk / 256; ++round) {
    const int s = b * kPermChunk + round * 256 + tid;
    const int e = (s < a.n) ? a.ids[s] : -1;
    const bool v = valid_id(e, a.E);
    uint64_t match = __ballot(v);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      uint64_t bb = __ballot(v && ((e >> bit) & 1));
      match &= ((e >> bit) & 1) ? bb : ~bb;
    }
    const int rank = __popcll(match & lt_mask);
    if (v && rank == 0) wave_cnt[wv][e] = __popcll(match);
    __syncthreads();
    if (v) {
      int pre = running[e];
      for (int w = 0; w < wv; ++w) pre += wave_cnt[w][e];
      int pos = a.block_base[b * a.E + e] + pre + rank;
      a.perm[pos] = s;
      if (a.perm2) a.perm2[pos] = s;
    }
    __syncthreads();
    {
      int e2 = tid;
      int add = wave_cnt[0][e2] + wave_cnt[1][e2] + wave_cnt[2][e2] + wave_cnt[3][e2];
      running[e2] += add;
      for (int w = 0; w < 4; ++w) wave_cnt[w][e2] = 0;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(PermArgs a) {
  chunk_scatter(a, blockIdx.x);
}

// Small case (a single chunk): histogram, scan and scatter in one block.
__global__ __launch_bounds__(256) void perm_single_kernel(PermArgs a) {
  __shared__ int cnt[256];
  chunk_hist(a, 0, cnt);
  for (int e = threadIdx.x; e < a.E; e += blockDim.x) a.block_cnt[e] = cnt[e];
  __syncthreads();
  scan_all(a);
  __syncthreads();
  chunk_scatter(a, 0);
}

hipError_t launch_permute(const PermArgs& a, hipStream_t s) {
  if (a.nb <= 1) {
    hipLaunchKernelGGL(perm_single_kernel, dim3(1), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(perm_hist_kernel, dim3((unsigned)a.nb), dim3(256), 0, s, a);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(256), 0, s, a);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)a.nb), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace beam
