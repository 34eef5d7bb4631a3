// Kernel argument blocks and launchers shared between the kernels and the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace beam {

constexpr int kPermChunk = 1024;  // slots per permutation block (256 threads x 4 rounds)
constexpr int kGemmBM = 256;      // rows per grouped-GEMM tile
constexpr int kStreamMaxT = 128;  // largest T served by the weight-streaming expert path
constexpr int kSplitDownMaxT = 16;  // largest T whose down pass splits K over four waves
constexpr int kDenseSplitK = 4;     // dense layers, T <= 16: workgroups per down column tile
constexpr int kFusedRouteMaxT = 16;     // router + top-k + grouping in one launch up to this T
constexpr int kFusedRouteMaxSlots = 64;  // ... and up to this many slots (T * k)
constexpr int kRoutePermuteSmallMaxT = 16;  // top-k + grouping in one workgroup (16 waves)
// its arrival count: a top counter and kRouteSub sub-counters, kRouteCounterStride words apart
constexpr int kRouteSub = 16;
constexpr int kRouteCounterStride = 64;
constexpr int kRouteDoneWords = (1 + kRouteSub) * kRouteCounterStride;
constexpr int kBoundaryWgMaxD = 8192;   // boundary rows up to this width: a workgroup per row
constexpr int kChainMaxK = 8;  // combine + boundary + next routing in one launch up to this k

struct BoundaryArgs {
  int T, d;
  const uint16_t* h;
  const uint16_t* x;
  const uint16_t* w_post;
  const uint16_t* w_pre;
  uint16_t* h_out;  // may equal h
  uint16_t* z_out;
  float c1, c2, eps;
};

// The combine feeding a fused boundary: the token's k expert rows yk [T*k, d] with
// their ids [T, k] (invalid ids contribute nothing); y [T, d] receives the combined
// rows when not null.
struct CombineArgs {
  int k, E;
  const int32_t* ids;
  const uint16_t* yk;
  uint16_t* y;
};

struct RouterArgs {
  int T, d, E;
  const uint16_t* z;  // [T, d] BF16
  const float* W;     // [E, d] FP32
  float* logits;      // [T, E]
};

// 4-bit activations: the token rows' MXFP4 codes [T, d/2] (GEMM order), scales [T, d/32]
// and round trip [T, d] BF16, written by the routing launch that reads the rows anyway;
// zq null: none
struct RowQuantArgs {
  uint8_t* zq;
  uint8_t* zqs;
  uint16_t* zr;
};

struct RouterX3Args {
  int T, d, E;            // E % 64 == 0, d % 128 == 0
  const uint16_t* z;      // [T, d] BF16
  const uint16_t* wx3;    // router weight as 3 BF16 parts, packed fragments
  float* logits;          // [T, E]
};

struct TopkArgs {
  int T, E, G, kg, k;
  float scale;
  const float* logits;  // [T, E]
  const float* bias;    // [E]
  int32_t* ids;         // [T, k]
  float* w;             // [T, k]
  int32_t* ids2;        // optional copy for the caller, or null
  float* w2;
};

struct PermArgs {
  int n;   // T * k slots
  int E;
  int nb;  // blocks = ceil(n / kPermChunk)
  int bm;  // rows per grouped-GEMM tile (for the tile table)
  const int32_t* ids;
  int32_t* counts;      // [E]
  int32_t* offsets;     // [E + 1]
  int32_t* perm;        // [n]: row -> slot, -1 past the valid rows
  int32_t* block_cnt;   // [nb * E]
  int32_t* block_base;  // [nb * E]
  int32_t* active;      // [E]: experts with rows, ascending
  int32_t* n_active;    // [1]
  int32_t* tile_start;  // [E + 1]: exclusive prefix of ceil(count / bm)
  int32_t* perm2;       // optional copies for the caller, or null
  int32_t* offsets2;
};

struct ExpertArgs {
  int T, k, d, f, E;
  const uint16_t* z;          // [T, d]
  const uint16_t* wgu;        // packed gate/up
  const uint16_t* wdp;        // packed down
  const int32_t* perm;        // [T*k] row -> slot
  const int32_t* offsets;     // [E + 1]
  const int32_t* active;      // [E]
  const int32_t* n_active;    // [1]
  const int32_t* tile_start;  // [E + 1]
  const float* w;             // [T*k] routing weight by slot
  uint16_t* act;              // [T*k, f] by row (expert-grouped order)
  uint16_t* yk;               // [T*k, d] by slot t*k+j
  // MXFP4 experts (decode layout of experts_mxfp4.hip); null for BF16 experts
  const uint8_t* qgu = nullptr;  // gate/up codes
  const uint8_t* sgu = nullptr;  // gate/up scales
  const uint8_t* qd = nullptr;   // down codes
  const uint8_t* sd = nullptr;   // down scales
  // MXFP4 experts, grouped-GEMM layout (experts.hip); null unless the handle serves T > 128
  const uint8_t* pqgu = nullptr;
  const uint8_t* psgu = nullptr;
  const uint8_t* pqd = nullptr;
  const uint8_t* psd = nullptr;
  // 4-bit activations (experts_w4a4.hip): token-row codes [T, d/2] and scales [T, d/32];
  // activation codes [T*k, f/2] and scales [T*k, f/32] by row (expert-grouped order)
  const uint8_t* zq = nullptr;
  const uint8_t* zqs = nullptr;
  uint8_t* aq = nullptr;
  uint8_t* aqs = nullptr;
};

hipError_t launch_boundary(const BoundaryArgs& a, hipStream_t s);
// MXFP4 experts: block quantisation of BF16 rows (nblocks blocks of 32 values), the
// init-time repack of row-major codes/scales into the decode layout, and the
// weight-streaming expert passes (T <= kStreamMaxT; d, f multiples of 512)
hipError_t launch_mxfp4_quantize(int64_t nblocks, const uint16_t* src, uint8_t* codes,
                                 uint8_t* scales, hipStream_t s);
hipError_t launch_repack_mxfp4(const uint8_t* gq, const uint8_t* gs, const uint8_t* uq,
                               const uint8_t* us, const uint8_t* dq, const uint8_t* ds, int E,
                               int f, int d, uint8_t* qgu, uint8_t* sgu, uint8_t* qd, uint8_t* sd,
                               hipStream_t s);
hipError_t launch_gateup_fp4(const ExpertArgs& a, int max_active, hipStream_t s);
hipError_t launch_gateup_gemm_fp4(const ExpertArgs& a, int max_tiles, hipStream_t s);
hipError_t launch_down_gemm_fp4(const ExpertArgs& a, int max_tiles, hipStream_t s);
// row-major codes/scales of gate and up (gateup) or down into the grouped-GEMM layout
hipError_t launch_repack_mxfp4_gemm(const uint8_t* gq, const uint8_t* gs, const uint8_t* uq,
                                    const uint8_t* us, const uint8_t* dq, const uint8_t* ds,
                                    int E, int f, int d, uint8_t* pqgu, uint8_t* psgu,
                                    uint8_t* pqd, uint8_t* psd, hipStream_t s);
// dense layer down pass for T <= 16 with K split over P workgroups per column tile
// (FP32 partials in part [P][16][d], then the finishing pass writes a.yk = y);
// needs (f / 32) % (4 P) == 0
hipError_t launch_down_splitk_dense(const ExpertArgs& a, int P, float* part, hipStream_t s);
// Dense SwiGLU layer as one expert taking every token with weight 1: with init, rows
// 0..max_tokens-1 get the identity order and weight 1; always, the counts, offsets,
// active list and tile table of a T-token call (one expert, tiles of bm rows)
hipError_t launch_dense_plan(int T, int max_tokens, bool init, const PermArgs& a, float* w,
                             hipStream_t s);
hipError_t launch_down_fp4(const ExpertArgs& a, int max_active, hipStream_t s);
// whether launch_down_fp4 rounds the activations through MXFP4 itself (one token with 4-bit
// activations: a.aq set), so the separate round-trip pass is left out
bool down_fp4_rounds_act(const ExpertArgs& a);
// the boundary with x = the combine of c (b.x unused); b.d <= kBoundaryWgMaxD
hipError_t launch_combine_boundary(const BoundaryArgs& b, const CombineArgs& c, hipStream_t s);
hipError_t launch_router_fp32(const RouterArgs& a, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
hipError_t launch_repack_router(const float* W, uint16_t* out, int E, int d, hipStream_t s);
hipError_t launch_router_bf16x3(const RouterX3Args& a, hipStream_t s);
hipError_t launch_permute(const PermArgs& a, hipStream_t s);
// grouped top-k + permutation in one launch; needs T * k <= kPermChunk
hipError_t launch_route_permute_small(const TopkArgs& t, const PermArgs& a, hipStream_t s);
// Router + grouped top-k + grouping in one launch for T <= 16 and T * k <= 64 (E
// workgroups; `done` is caller-owned, zeroed device memory of kRouteDoneWords words, left
// zeroed; `sc` is caller-owned scratch of T * E 64-bit words for the published scores).
// q: the rows' 4-bit quantisation in the same launch (q.zq null: none).
hipError_t launch_route_fused_tiny(const RouterArgs& r, const TopkArgs& t, const PermArgs& a,
                                   uint32_t* done, uint64_t* sc, const RowQuantArgs& q,
                                   hipStream_t s);
// one token (d <= 8192): the boundary of that token inside the same launch; z goes to
// b.z_out and the router reads it, h' to b.h_out (which may be b.h). cb not null: the
// boundary's x is the combine of the previous MoE's expert rows (b.x unused; the combined
// row goes to cb->y when that is not null).
hipError_t launch_boundary_route_fused(const BoundaryArgs& b, const RouterArgs& r, const TopkArgs& t,
                                       const PermArgs& a, uint32_t* done, uint64_t* sc,
                                       const RowQuantArgs& q, const CombineArgs* cb,
                                       hipStream_t s);
hipError_t launch_repack(const uint16_t* wg, const uint16_t* wu, const uint16_t* wd,
                         uint16_t* wgu, uint16_t* wdp, int E, int f, int d, hipStream_t s);
hipError_t launch_gateup_stream(const ExpertArgs& a, int max_active, hipStream_t s);
// down for T <= kSplitDownMaxT with K split over four waves (then launch_combine)
hipError_t launch_down_split(const ExpertArgs& a, int max_active, hipStream_t s);
hipError_t launch_down_stream(const ExpertArgs& a, int max_active, hipStream_t s);
hipError_t launch_gateup_gemm(const ExpertArgs& a, int max_tiles, hipStream_t s);
hipError_t launch_down_gemm(const ExpertArgs& a, int max_tiles, hipStream_t s);
hipError_t launch_combine(int T, int k, int d, int E, const int32_t* ids, const uint16_t* yk,
                          uint16_t* y, hipStream_t s);
// 4-bit activations: MXFP4 quantisation of token rows (nblocks blocks of 32) into the codes
// and scales the W4A4 GEMM reads, and the W4A4 grouped GEMMs (d, f multiples of 512)
hipError_t launch_quantize_rows_a4(int64_t nblocks, const uint16_t* src, uint8_t* codes,
                                   uint8_t* scales, uint16_t* rt, hipStream_t s);
// the weight-streaming passes' activations [rows, f] replaced by their MXFP4 round trip (the
// first *nvalid rows), codes and scales kept
hipError_t launch_act_round_trip_a4(int64_t rows, int f, const int32_t* nvalid, uint16_t* act,
                                    uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_gateup_gemm_a4(const ExpertArgs& a, int max_tiles, hipStream_t s);
hipError_t launch_down_gemm_a4(const ExpertArgs& a, int max_tiles, hipStream_t s);

}  // namespace beam
