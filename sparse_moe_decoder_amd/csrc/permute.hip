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
#include "boundary_device.h"
#include "router_device.h"
#include "topk_device.h"
#include "mxfp4_device.h"

#include <type_traits>

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

// Exclusive scan of three per-expert quantities over up to 256 experts, by the
// first four waves of the block (shuffle scan per wave, then wave totals).
// q0 = row counts, q1 = 1 if the expert has rows, q2 = grouped-GEMM tiles.
// Thread e < 256 receives its exclusive prefixes; totals go to tot[3].
__device__ void scan256x3(int e, int v0, int v1, int v2, int& x0, int& x1, int& x2, int* tot) {
  __shared__ int wsum[3][4];
  const int lane = e & 63, wv = e >> 6;
  int i0 = v0, i1 = v1, i2 = v2;
  if (e < 256) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int a0 = __shfl_up(i0, off, 64), a1 = __shfl_up(i1, off, 64), a2 = __shfl_up(i2, off, 64);
      if (lane >= off) {
        i0 += a0;
        i1 += a1;
        i2 += a2;
      }
    }
    if (lane == 63) {
      wsum[0][wv] = i0;
      wsum[1][wv] = i1;
      wsum[2][wv] = i2;
    }
  }
  __syncthreads();
  if (e < 256) {
    int p0 = 0, p1 = 0, p2 = 0;
    for (int w = 0; w < wv; ++w) {
      p0 += wsum[0][w];
      p1 += wsum[1][w];
      p2 += wsum[2][w];
    }
    x0 = p0 + i0 - v0;
    x1 = p1 + i1 - v1;
    x2 = p2 + i2 - v2;
    if (e == 255) {
      tot[0] = x0 + v0;
      tot[1] = x1 + v1;
      tot[2] = x2 + v2;
    }
  }
  __syncthreads();
}

// Offsets, counts, active list and tile table from per-expert totals held by
// threads e < E (others pass 0). Returns the valid row count to every thread.
__device__ int publish_offsets(const PermArgs& a, int e, int cnt, int* excl_lds) {
  __shared__ int tot[3];
  const bool has = e < a.E;
  int x0 = 0, x1 = 0, x2 = 0;
  scan256x3(e, has ? cnt : 0, (has && cnt > 0) ? 1 : 0, has ? (cnt + a.bm - 1) / a.bm : 0, x0,
            x1, x2, tot);
  if (has) {
    excl_lds[e] = x0;
    a.counts[e] = cnt;
    a.offsets[e] = x0;
    if (a.offsets2) a.offsets2[e] = x0;
    a.tile_start[e] = x2;
    if (cnt > 0) a.active[x1] = e;
  }
  if (e == 0) {
    a.offsets[a.E] = tot[0];
    if (a.offsets2) a.offsets2[a.E] = tot[0];
    a.tile_start[a.E] = tot[2];
    *a.n_active = tot[1];
  }
  __syncthreads();
  return tot[0];
}

// One block: per-expert totals over the histogram blocks, the offsets, then each
// block's base (the expert's offset plus the counts of the blocks before it). Thread
// e walks expert e's column 16 blocks at a time, all 16 loads in flight together.
constexpr int kScanBatch = 16;

__device__ void scan_all(const PermArgs& a) {
  __shared__ int excl_s[256];
  const int e = threadIdx.x;
  const bool mine = e < a.E;
  int run = 0;
  if (mine) {
    for (int b0 = 0; b0 < a.nb; b0 += kScanBatch) {
      int cv[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u)
        cv[u] = b0 + u < a.nb ? a.block_cnt[(b0 + u) * a.E + e] : 0;
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) run += cv[u];
    }
  }
  const int total = publish_offsets(a, e, run, excl_s);
  if (mine) {
    int base = excl_s[e];
    for (int b0 = 0; b0 < a.nb; b0 += kScanBatch) {
      int cv[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u)
        cv[u] = b0 + u < a.nb ? a.block_cnt[(b0 + u) * a.E + e] : 0;
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) {
        if (b0 + u < a.nb) a.block_base[(b0 + u) * a.E + e] = base;
        base += cv[u];
      }
    }
  }
  // rows past the valid ones (slots with invalid ids) read as -1
  for (int r = total + threadIdx.x; r < a.n; r += blockDim.x) {
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

// Small batches (T*k <= 1024): grouped top-k for every token (16 waves, one
// token per wave at a time), then the histogram, offsets and stable scatter from
// LDS, all in one launch.
__global__ __launch_bounds__(1024) void route_permute_small_kernel(TopkArgs ta, PermArgs a) {
  __shared__ __attribute__((aligned(16))) float c_lds[16][256];
  __shared__ int32_t sel[16][32];
  __shared__ int32_t ids_lds[1024];
  __shared__ int cnt[256];
  __shared__ int excl[256];
  __shared__ int wave_cnt[16][256];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  for (int e = tid; e < 256; e += 1024) cnt[e] = 0;
  for (int i = tid; i < 16 * 256; i += 1024) (&wave_cnt[0][0])[i] = 0;
  for (int64_t t = wv; t < ta.T; t += 16) {
    topk_token(ta, t, c_lds[wv], sel[wv], lane);
    if (lane < ta.k) ids_lds[t * ta.k + lane] = sel[wv][lane];
  }
  __syncthreads();
  const int n = a.n;
  const int e_mine = tid < n ? ids_lds[tid] : -1;
  const bool v = valid_id(e_mine, a.E);
  if (v) atomicAdd(&cnt[e_mine], 1);
  __syncthreads();
  const int total = publish_offsets(a, tid, (tid < a.E) ? cnt[tid] : 0, excl);
  // stable scatter: rank among earlier lanes with the same expert, then earlier waves
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  uint64_t match = __ballot(v);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    uint64_t bb = __ballot(v && ((e_mine >> bit) & 1));
    match &= ((e_mine >> bit) & 1) ? bb : ~bb;
  }
  const int rank = __popcll(match & lt_mask);
  if (v && rank == 0) wave_cnt[wv][e_mine] = __popcll(match);
  __syncthreads();
  if (v) {
    int pos = excl[e_mine] + rank;
    for (int w = 0; w < wv; ++w) pos += wave_cnt[w][e_mine];
    a.perm[pos] = tid;
    if (a.perm2) a.perm2[pos] = tid;
  }
  for (int r = total + tid; r < n; r += 1024) {
    a.perm[r] = -1;
    if (a.perm2) a.perm2[r] = -1;
  }
}

// Grouping of at most 64 slots by one wave, from the slot ids in LDS (one slot per
// lane). Lane l owns experts 4l .. 4l+3 for counts, offsets, the active list and
// the tile table. The counts come from an LDS histogram (cnt, 256 ints of LDS
// scratch; LDS atomics only count); the exclusive prefixes over experts from
// lane-local sums and ballot bit-plane scans across the lanes; a slot's row is its
// expert's offset (off, 256 ints of LDS scratch) plus the number of earlier slots
// with the same expert (a ballot match mask over the id's bit planes): the rows
// follow (expert, slot) order exactly. At most 64 slots means at most one
// grouped-GEMM tile per expert.
static_assert(kGemmBM >= 64, "the one-wave grouping assumes at most one tile per expert");
__device__ __forceinline__ void group_slots_wave(const PermArgs& a, const int32_t* ids_lds,
                                                 int lane, int* cnt, int* off) {
  const int n = a.n, E = a.E;
  const int e_mine = lane < n ? ids_lds[lane] : -1;
  const bool v = valid_id(e_mine, E);
  *(int4*)(cnt + 4 * lane) = make_int4(0, 0, 0, 0);
  wave_lds_sync();
  if (v) atomicAdd(&cnt[e_mine], 1);
  wave_lds_sync();
  const int4 c = *(const int4*)(cnt + 4 * lane);
  const int c4[4] = {c.x, c.y, c.z, c.w};
  // exclusive prefixes across lanes of: the lane's slot total (< 128: 7 bit planes),
  // its active experts and tiles (<= 4: 3 bit planes; one tile per active expert)
  const int tot = c4[0] + c4[1] + c4[2] + c4[3];
  int act4 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) act4 += c4[i] > 0 ? 1 : 0;
  int base = 0, nvalid = 0, aidx = 0, n_act = 0;
#pragma unroll
  for (int b = 0; b < 7; ++b) {
    const uint64_t bb = __ballot((tot >> b) & 1);
    base += lanes_below(bb) << b;
    nvalid += __popcll(bb) << b;
  }
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const uint64_t ba = __ballot((act4 >> b) & 1);
    aidx += lanes_below(ba) << b;
    n_act += __popcll(ba) << b;
  }
  int below4[4];
  below4[0] = base;
#pragma unroll
  for (int i = 1; i < 4; ++i) below4[i] = below4[i - 1] + c4[i - 1];
  *(int4*)(off + 4 * lane) = make_int4(below4[0], below4[1], below4[2], below4[3]);
  int tidx = aidx;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    if (e < E) {
      a.counts[e] = c4[i];
      a.offsets[e] = below4[i];
      if (a.offsets2) a.offsets2[e] = below4[i];
      a.tile_start[e] = tidx;
      if (c4[i] > 0) {
        a.active[tidx] = e;
        ++tidx;
      }
    }
  }
  if (lane == 0) {
    a.offsets[E] = nvalid;
    if (a.offsets2) a.offsets2[E] = nvalid;
    a.tile_start[E] = n_act;
    *a.n_active = n_act;
  }
  // the slot's row: earlier lanes with the same (valid) id, plus its expert's offset
  uint64_t match = __ballot(v);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const uint64_t bb = __ballot(v && ((e_mine >> bit) & 1));
    match &= ((e_mine >> bit) & 1) ? bb : ~bb;
  }
  wave_lds_sync();
  if (v) {
    const int pos = off[e_mine] + lanes_below(match);
    a.perm[pos] = lane;
    if (a.perm2) a.perm2[pos] = lane;
  }
  if (lane >= nvalid && lane < n) {
    a.perm[lane] = -1;
    if (a.perm2) a.perm2[lane] = -1;
  }
}

// Tiny batches (T*k <= 64): the waves route one token each, then wave 0 groups.
__global__ __launch_bounds__(1024) void route_permute_tiny_kernel(TopkArgs ta, PermArgs a) {
  __shared__ __attribute__((aligned(16))) float c_lds[16][256];
  __shared__ int32_t sel[16][32];
  __shared__ int32_t ids_lds[64];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int nw = blockDim.x >> 6;
  for (int64_t t = wv; t < ta.T; t += nw) {
    topk_token(ta, t, c_lds[wv], sel[wv], lane);
    if (lane < ta.k) ids_lds[t * ta.k + lane] = sel[wv][lane];
  }
  __syncthreads();
  if (wv != 0) return;
  group_slots_wave(a, ids_lds, lane, reinterpret_cast<int*>(c_lds[0]), reinterpret_cast<int*>(c_lds[1]));
}

// Arrival count of the fused routing in two levels: workgroup b counts itself on
// sub-counter b % kRouteSub, the last arrival there counts that sub-counter on the top
// counter, and each counter's last arrival resets it for the next launch. Atomics on one
// address are serialised where they meet, so spreading the E arrivals over sub-counters
// shortens the wait of the last one. Thread 0 calls it after its workgroup's stores have
// completed; it returns true in exactly one workgroup, the last of all nb.
__device__ __forceinline__ bool count_arrival(uint32_t* done, int b, int nb) {
  const int j = b % kRouteSub;
  const uint32_t nj = (uint32_t)((nb - j + kRouteSub - 1) / kRouteSub);
  uint32_t* sub = done + (1 + j) * kRouteCounterStride;
  if (__hip_atomic_fetch_add(sub, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != nj - 1)
    return false;
  __hip_atomic_store(sub, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t nsub = (uint32_t)(nb < kRouteSub ? nb : kRouteSub);
  if (__hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != nsub - 1)
    return false;
  __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Whether one token's top-k and grouping can run on a whole workgroup, one thread per
// expert: E <= 256, power-of-two groups of 2 to 64 experts, kg * k <= 256.
__device__ __forceinline__ bool one_token_wg_ok(const TopkArgs& a) {
  const int gs = a.E / a.G;
  return a.T == 1 && a.E <= 256 && gs >= 2 && gs <= 64 && (gs & (gs - 1)) == 0 &&
         a.kg * a.k <= 256;
}

struct OneTokenLds {
  uint64_t key[256];   // expert e: order key of its biased score, then ~e
  uint64_t gkey[128];  // group g: order key of its score, then ~g
  uint64_t skey[256];  // survivors of the kept groups, at (group rank) * k + (rank in group)
  float s[64];         // slot j: the selected expert's score
  int32_t id[64];      //   and its index
};

// (The counting loops are unrolled so that their LDS reads are in flight together.)
// One token's grouped top-k and grouping by the 256 threads of a workgroup, thread e
// holding expert e. The selection and the weights are topk_token's, found by counting
// instead of in rounds: an entry's rank is the number of entries ahead of it in (value
// desc, index asc) order, which the 64-bit keys (order key, then the inverted index)
// compare directly. The groups' ranks keep kg groups. An expert among the top k of the
// kept experts is among the top k of its own group, so each expert's rank within its
// group leaves at most k survivors per kept group, and the survivors' ranks among
// themselves are the slots. The grouping of the k slots (k distinct experts, one row
// each) follows in the same pass: a selected expert's row is the number of selected
// experts below it, and so is every expert's offset.
__device__ void route_one_token_wg(const TopkArgs& ta, const PermArgs& pa, const uint64_t* sc,
                                   OneTokenLds& L) {
  const int tid = threadIdx.x, E = ta.E, G = ta.G, gs = E / G, k = ta.k, kg = ta.kg;
  const int nsk = kg * k;
  const bool valid = tid < E;
  float s = 0.0f, c = -INFINITY;
  if (valid) {
    const uint64_t p = __hip_atomic_load(sc + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s = __uint_as_float((uint32_t)p);
    c = __uint_as_float((uint32_t)(p >> 32));
  }
  if (tid < nsk) L.skey[tid] = 0;
  const uint64_t key = valid ? ((uint64_t)f32_order_key(c) << 32) | (uint32_t)~tid : 0;
  L.key[tid] = key;
  // group score: the sum of the group's two largest biased scores (a group's threads are
  // adjacent lanes of one wave). Each step merges the top two of two disjoint lane sets of
  // the group, so every lane ends with the group's pair: the quad permutations, the half-row
  // and row mirrors (within 8 and 16 lanes) by DPP, then shuffles across rows.
  float m1 = c, m2 = -INFINITY;
  auto merge_dpp = [&](auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    top2_merge(m1, m2, __uint_as_float(dpp_u32<C>(__float_as_uint(m1))),
               __uint_as_float(dpp_u32<C>(__float_as_uint(m2))));
  };
  if (gs >= 2) merge_dpp(std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  if (gs >= 4) merge_dpp(std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  if (gs >= 8) merge_dpp(std::integral_constant<int, 0x141>{});  // row_half_mirror
  if (gs >= 16) merge_dpp(std::integral_constant<int, 0x140>{}); // row_mirror
  for (int off = 16; off < gs; off <<= 1)
    top2_merge(m1, m2, __shfl_xor(m1, off, 64), __shfl_xor(m2, off, 64));
  const int g = tid / gs;
  if (valid && tid % gs == 0)
    L.gkey[g] = ((uint64_t)f32_order_key(m1 + m2) << 32) | (uint32_t)~g;
  __syncthreads();
  int rg = kg;
  if (valid) {
    const uint64_t mine = L.gkey[g];
    rg = 0;
#pragma unroll 8
    for (int q = 0; q < G; ++q) rg += L.gkey[q] > mine ? 1 : 0;
  }
  bool surv = false;
  int ri = 0;
  if (rg < kg) {
    const uint64_t* gk = L.key + g * gs;
#pragma unroll 8
    for (int q = 0; q < gs; ++q) ri += gk[q] > key ? 1 : 0;
    surv = ri < k;
    if (surv) L.skey[rg * k + ri] = key;
  }
  __syncthreads();
  int slot = -1;
  if (surv) {
    int r = 0;
#pragma unroll 8
    for (int q = 0; q < nsk; ++q) r += L.skey[q] > key ? 1 : 0;
    if (r < k) {
      slot = r;
      L.s[r] = s;
      L.id[r] = tid;
    }
  }
  __syncthreads();
  if (tid < k) {
    float den = L.s[0];
#pragma unroll 8
    for (int j = 1; j < k; ++j) den = den + L.s[j];  // slot order
    const float wj = (L.s[tid] / den) * ta.scale;
    const int e = L.id[tid];
    ta.ids[tid] = e;
    ta.w[tid] = wj;
    if (ta.ids2) ta.ids2[tid] = e;
    if (ta.w2) ta.w2[tid] = wj;
  }
  if (valid) {
    int off = 0;
#pragma unroll 8
    for (int j = 0; j < k; ++j) off += L.id[j] < tid ? 1 : 0;
    pa.counts[tid] = slot >= 0 ? 1 : 0;
    pa.offsets[tid] = off;
    if (pa.offsets2) pa.offsets2[tid] = off;
    pa.tile_start[tid] = off;  // one tile per selected expert
    if (slot >= 0) {
      pa.active[off] = tid;
      pa.perm[off] = slot;
      if (pa.perm2) pa.perm2[off] = slot;
    }
  }
  if (tid == 0) {
    pa.offsets[E] = k;
    if (pa.offsets2) pa.offsets2[E] = k;
    pa.tile_start[E] = k;
    *pa.n_active = k;
  }
}

// The row loads of boundary_row_4waves_load for one token (t = 0) with x the weighted combine
// of the token's k expert rows of the previous MoE (cb), in combine_chunk's arithmetic: every
// slot's row chunk and the slot ids are loaded together (slot j's row is in bounds whatever
// its id), then the FP32 adds in slot order from -0.0 skip the invalid ids, and one rounding.
// after_loads() issues the caller's own loads behind the rows. k <= 8 (kChainMaxK).
template <class AfterLoads>
__device__ __forceinline__ void boundary_row_4waves_load_combine(const BoundaryArgs& a,
                                                                 const CombineArgs& cb,
                                                                 BoundaryRow4& b,
                                                                 AfterLoads after_loads) {
  const int lane = threadIdx.x & 63;
  const int wvu = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // uniform branches
  const int nch = a.d >> 3, nv = (nch + 63) >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int vv = wvu + 4 * j, idx = 64 * vv + lane;
    const int li = idx < nch ? idx : 0;
    if (vv < nv) {
      b.hv[j] = ld_u32x4((const u32x4*)a.h + li);
      b.wo[j] = ld_u32x4((const u32x4*)a.w_post + li);
      b.wr[j] = ld_u32x4((const u32x4*)a.w_pre + li);
    }
  }
  float acc[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = -0.0f;
  // slots j0 .. j0 + 7: ids and rows loaded together, then the adds in slot order
  auto slots8 = [&](int j0) {
    int e8[8];
    u32x4 v[4][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int slot = j0 + u < cb.k ? j0 + u : j0;  // past k: a valid row, not added
      e8[u] = j0 + u < cb.k ? cb.ids[slot] : -1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int vv = wvu + 4 * j, idx = 64 * vv + lane;
        if (vv < nv)
          v[j][u] = ld_u32x4((const u32x4*)(cb.yk + (int64_t)slot * a.d) + (idx < nch ? idx : 0));
      }
    }
    if (j0 == 0) {  // the caller's loads go out behind the first rows
      __builtin_amdgcn_sched_barrier(0);
      after_loads();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = e8[u] >= 0 && e8[u] < cb.E;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (wvu + 4 * j < nv) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {  // an invalid slot leaves the sum as it is (even -0.0)
            const float s0 = acc[j][2 * i] + lo_bf(v[j][u][i]);
            const float s1 = acc[j][2 * i + 1] + hi_bf(v[j][u][i]);
            acc[j][2 * i] = ok ? s0 : acc[j][2 * i];
            acc[j][2 * i + 1] = ok ? s1 : acc[j][2 * i + 1];
          }
        }
    }
  };
  slots8(0);  // k <= 8: straight-line code, so the load counters stay exact
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) b.xv[j][i] = pack_bf2(acc[j][2 * i], acc[j][2 * i + 1]);
}

// Router, grouped top-k and grouping of a small batch (T <= 16 tokens, T * k <= 64
// slots) in one launch: one workgroup per expert computes its logits exactly as the
// stand-alone small-batch router does, writes them out, and publishes each token's
// (score, biased score) pair for its expert (computed as the top-k computes them)
// with device-coherent (write-through) stores; it waits for those stores to
// complete, then counts itself done (count_arrival). The workgroup that counts last
// (every other one has published) runs the top-k (coherent loads of the pairs; one
// wave per token, or the whole workgroup for one token) and the grouping. No
// workgroup waits on another.
// BOUNDARY (one token): the sublayer boundary runs inside the same launch. Each
// workgroup forms the token's z from h and x itself, in the boundary kernel's exact
// order (see boundary_row_4waves_finish), into LDS, with its router weights in
// flight; workgroup 0 writes z out, and the last workgroup writes h' (by then every
// workgroup has read h, so h_out may alias h).
// QUANT (4-bit activations, rq): the workgroups also share out the rows' 32-value blocks,
// four lanes to a block, and write each block's MXFP4 codes, scale and round trip next to
// their logits (the rows are at hand; the stores complete before the workgroup counts
// itself).
// COMBINE (with BOUNDARY): the boundary's x is the weighted combine of the previous MoE's
// expert rows (cb; every workgroup combines the row itself; workgroup 0 writes it to cb.y
// when that is not null): the combine, the next sublayer boundary and that sublayer's
// routing in one launch. Every workgroup has read cb.ids before it counts itself, so the
// last one may overwrite them (the same handle routing its next call).
template <bool BOUNDARY, bool QUANT, bool COMBINE>
__global__ __launch_bounds__(256) void route_fused_tiny_kernel(RouterArgs ra, TopkArgs ta,
                                                               PermArgs pa, uint32_t* done,
                                                               uint64_t* sc, BoundaryArgs ba,
                                                               RowQuantArgs rq, CombineArgs cb) {
  __shared__ float part[3][kRouterRT];
  __shared__ __attribute__((aligned(16))) float c_lds[4][256];
  __shared__ int32_t sel[4][32];
  __shared__ int32_t ids_lds[64];
  __shared__ OneTokenLds one;
  __shared__ int is_last;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int e = blockIdx.x;
  const float bias = ta.bias[e];
  // QUANT: this workgroup's blocks [q0, q1) of the rows' T * d / 32; thread 4 i + p holds
  // part p of block q0 + i (+ 64 per round), the first round's values prefetched
  const int nbq = QUANT ? ra.T * (ra.d >> 5) : 0;
  const int qper = (nbq + (int)gridDim.x - 1) / (int)gridDim.x;
  const int q0 = e * qper, q1 = q0 + qper < nbq ? q0 + qper : nbq;
  const int qb = q0 + (tid >> 2), qp = tid & 3;
  const bool doq = qb < q1;
  auto quant_out = [&](int b, const u32x4& qv) {
    mxfp4_block_out_4lanes(qv, rq.zq + (int64_t)b * 16, rq.zqs + b, rq.zr + (int64_t)b * 32);
  };
  float v;
  BoundaryRow4 brow;  // BOUNDARY: the token row; its h' is stored by the last workgroup
  if constexpr (BOUNDARY) {
    // one token: the row's loads (L2 hits after the first workgroup) go out first,
    // then this expert's router weights (HBM); loads complete in order, so the
    // boundary arithmetic runs while the weights are in flight. Every workgroup forms
    // z itself (workgroup 0 writes it out).
    __shared__ float red[2][16];
    __shared__ __attribute__((aligned(16))) uint16_t zl[kBoundaryWgMaxD];
    f32x4 w[kRouterPreChunks];
    if constexpr (COMBINE) {
      // as below: the rows' loads (the expert rows and h; L2 or cache hits) first, the router
      // weights (HBM) after them, so the combine and the boundary run while they are in flight
      boundary_row_4waves_load_combine(ba, cb, brow, [&] { router_load_w(ra, e, w); });
      if (e == 0 && cb.y) {
        const int nch = ba.d >> 3, nv = (nch + 63) >> 6;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int vv = wv + 4 * j, idx = 64 * vv + lane;
          if (vv < nv && idx < nch) st_u32x4((u32x4*)cb.y + idx, brow.xv[j]);
        }
      }
    } else {
      boundary_row_4waves_load(ba, 0, brow);
      __builtin_amdgcn_sched_barrier(0);
      router_load_w(ra, e, w);
    }
    __builtin_amdgcn_sched_barrier(0);
    boundary_row_4waves_finish(ba, 0, brow, zl, e == 0 ? ba.z_out : nullptr, red);
    v = router_dot_1_lds(ra, w, zl, part);
    if constexpr (QUANT) {
      for (int b = qb; b < q1; b += 64) quant_out(b, *(const u32x4*)(zl + b * 32 + qp * 8));
    }
  } else {
    u32x4 qv;
    if (QUANT && doq) qv = ld_u32x4(ra.z + (int64_t)qb * 32 + qp * 8);
    v = router_small_dot(ra, e, 0, ra.T, part);
    if constexpr (QUANT) {
      if (doq) quant_out(qb, qv);
      for (int b = qb + 64; b < q1; b += 64) quant_out(b, ld_u32x4(ra.z + (int64_t)b * 32 + qp * 8));
    }
  }
  if (tid < ra.T) {
    ra.logits[(int64_t)tid * ra.E + e] = v;
    const float sv = routing_score(v), cv = sv + bias;
    __hip_atomic_store(sc + (int64_t)tid * ra.E + e,
                       (uint64_t)__float_as_uint(sv) | ((uint64_t)__float_as_uint(cv) << 32),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this workgroup's stores are complete
  __syncthreads();
  if (tid == 0) is_last = count_arrival(done, blockIdx.x, gridDim.x);
  __syncthreads();
  if (!is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // every workgroup has read h by now, so h_out may be h itself
  if constexpr (BOUNDARY) boundary_row_4waves_store_h(ba, 0, brow);
  if (one_token_wg_ok(ta)) {
    route_one_token_wg(ta, pa, sc, one);
    return;
  }
  for (int t = wv; t < ta.T; t += 4) {
    topk_token<true>(ta, t, c_lds[wv], sel[wv], lane, sc);
    if (lane < ta.k) ids_lds[t * ta.k + lane] = sel[wv][lane];
  }
  __syncthreads();
  if (wv == 0)
    group_slots_wave(pa, ids_lds, lane, reinterpret_cast<int*>(c_lds[0]), reinterpret_cast<int*>(c_lds[1]));
}

// Dense layer plan (see launch_dense_plan): one expert, every row in token order.
__global__ __launch_bounds__(256) void dense_plan_kernel(int T, int max_tokens, int init, PermArgs a,
                                                         float* w) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (init) {
    for (int r = i; r < max_tokens; r += gridDim.x * blockDim.x) {
      a.perm[r] = r;
      w[r] = 1.0f;
    }
  }
  if (i == 0) {
    a.counts[0] = T;
    a.offsets[0] = 0;
    a.offsets[1] = T;
    a.active[0] = 0;
    *a.n_active = T > 0 ? 1 : 0;
    a.tile_start[0] = 0;
    a.tile_start[1] = (T + a.bm - 1) / a.bm;
  }
}

hipError_t launch_dense_plan(int T, int max_tokens, bool init, const PermArgs& a, float* w,
                             hipStream_t s) {
  const unsigned g = init ? (unsigned)((max_tokens + 255) / 256) : 1u;
  hipLaunchKernelGGL(dense_plan_kernel, dim3(g), dim3(init ? 256 : 64), 0, s, T, max_tokens,
                     init ? 1 : 0, a, w);
  return hipGetLastError();
}

hipError_t launch_route_fused_tiny(const RouterArgs& r, const TopkArgs& t, const PermArgs& a,
                                   uint32_t* done, uint64_t* sc, const RowQuantArgs& q,
                                   hipStream_t s) {
  if (q.zq)
    hipLaunchKernelGGL((route_fused_tiny_kernel<false, true, false>), dim3((unsigned)r.E), dim3(256),
                       0, s, r, t, a, done, sc, BoundaryArgs{}, q, CombineArgs{});
  else
    hipLaunchKernelGGL((route_fused_tiny_kernel<false, false, false>), dim3((unsigned)r.E),
                       dim3(256), 0, s, r, t, a, done, sc, BoundaryArgs{}, q, CombineArgs{});
  return hipGetLastError();
}

hipError_t launch_boundary_route_fused(const BoundaryArgs& b, const RouterArgs& r, const TopkArgs& t,
                                       const PermArgs& a, uint32_t* done, uint64_t* sc,
                                       const RowQuantArgs& q, const CombineArgs* cb, hipStream_t s) {
  const dim3 g((unsigned)r.E), blk(256);
  if (cb) {
    if (q.zq)
      hipLaunchKernelGGL((route_fused_tiny_kernel<true, true, true>), g, blk, 0, s, r, t, a, done,
                         sc, b, q, *cb);
    else
      hipLaunchKernelGGL((route_fused_tiny_kernel<true, false, true>), g, blk, 0, s, r, t, a, done,
                         sc, b, q, *cb);
  } else if (q.zq) {
    hipLaunchKernelGGL((route_fused_tiny_kernel<true, true, false>), g, blk, 0, s, r, t, a, done, sc,
                       b, q, CombineArgs{});
  } else {
    hipLaunchKernelGGL((route_fused_tiny_kernel<true, false, false>), g, blk, 0, s, r, t, a, done,
                       sc, b, q, CombineArgs{});
  }
  return hipGetLastError();
}

hipError_t launch_route_permute_small(const TopkArgs& t, const PermArgs& a, hipStream_t s) {
  if (a.n <= 64) {
    const int waves = t.T < 16 ? t.T : 16;
    hipLaunchKernelGGL(route_permute_tiny_kernel, dim3(1), dim3(64 * waves), 0, s, t, a);
  } else {
    hipLaunchKernelGGL(route_permute_small_kernel, dim3(1), dim3(1024), 0, s, t, a);
  }
  return hipGetLastError();
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
