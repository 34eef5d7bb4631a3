// C ABI of the Beam MoE sublayer library: host-side validation, the handle and
// its workspace, and the launch sequence of each entry point. Every check runs
// before the first HIP call, so a rejected call has no side effects.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <type_traits>
#include <vector>

#include "../../include/beam_moe.h"
#include "kernels.h"

using namespace beam;

// ---------------------------------------------------------------------------------------------
// Kernel timing (measurement tools only)

namespace {

enum KernelId {
  K_BOUNDARY = 0,
  K_ROUTER,
  K_TOPK,
  K_PERMUTE,
  K_GATEUP,
  K_DOWN,
  K_COMBINE,
  K_QUANT,          // 4-bit activations: the token rows' and activations' quantisation
  K_COMBINE_ROUTE,  // one token: combine, next boundary and the next layer's routing
  K_COUNT
};
const char* const kKernelNames[K_COUNT] = {"boundary", "router",  "topk",     "permute",
                                           "gate_up",  "down",    "combine",  "quantize",
                                           "combine_route"};

struct ProfRecord {
  int id;
  hipEvent_t start, stop;
};

struct Profiler {
  std::mutex mu;
  bool enabled = false;
  std::vector<ProfRecord> records;
  std::vector<hipEvent_t> pool;
};
Profiler& prof() {
  static Profiler p;
  return p;
}

hipEvent_t take_event(Profiler& p) {
  if (!p.pool.empty()) {
    hipEvent_t e = p.pool.back();
    p.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one launch with events when timing is on.
struct ProfScope {
  int id;
  hipStream_t s;
  hipEvent_t a = nullptr, b = nullptr;
  ProfScope(int id_, hipStream_t s_) : id(id_), s(s_) {
    Profiler& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    if (!p.enabled) return;
    a = take_event(p);
    b = take_event(p);
    if (a && b) (void)hipEventRecord(a, s);
  }
  ~ProfScope() {
    if (!(a && b)) return;
    (void)hipEventRecord(b, s);
    Profiler& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    p.records.push_back({id, a, b});
  }
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? BEAM_OK : BEAM_ERR_HIP; }

}  // namespace

// ---------------------------------------------------------------------------------------------
// Handle

// Per-call device buffers of the MoE forward for T tokens (slots = T * k). A handle owns
// one set sized for max_tokens; the allocation-free entry point carves one out of the
// library's static scratch area instead.
struct Workspace {
  float* logits = nullptr;     // [T, E]
  int32_t* ids = nullptr;      // [T, k]
  float* w = nullptr;          // [T, k]
  int32_t* counts = nullptr;   // [E]
  int32_t* offsets = nullptr;  // [E + 1]
  int32_t* active = nullptr;   // [E]
  int32_t* n_active = nullptr; // [1]
  int32_t* tile_start = nullptr;  // [E + 1]
  int32_t* perm = nullptr;        // [T * k]
  uint32_t* route_done = nullptr;  // [kRouteDoneWords] arrival counters of the fused routing:
                                   // zero before its first launch, left zero by every launch
  uint64_t* route_sc = nullptr;    // [16 * E] its published (score, biased score) pairs
  int32_t* block_cnt = nullptr;   // [nb * E], nb = ceil(slots / kPermChunk)
  int32_t* block_base = nullptr;  // [nb * E]
  uint16_t* act = nullptr;        // [T * k, f]
  uint16_t* yk = nullptr;         // [T * k, d]
  uint8_t* zq = nullptr;          // 4-bit activations: token-row codes [T, d/2]
  uint8_t* zqs = nullptr;         //   and scales [T, d/32]
  uint8_t* aq = nullptr;          // 4-bit activations: activation codes [T * k, f/2]
  uint8_t* aqs = nullptr;         //   and scales [T * k, f/32]
  uint16_t* zr = nullptr;         // 4-bit activations, T <= kStreamMaxT: the token rows' MXFP4
                                  //   round trip [T, d] BF16 (the weight streams' input)
};

struct beam_moe_ctx {
  beam_moe_config cfg;
  int device = 0;
  // weights (owned)
  float* router_w = nullptr;  // [E, d]
  uint16_t* router_x3 = nullptr;  // [3][E/16][d/32][64][8]: W = hi + mid + lo, BF16 parts
  float* bias = nullptr;      // [E]
  uint16_t* wgu = nullptr;    // packed gate/up (BF16 experts)
  uint16_t* wdp = nullptr;    // packed down (BF16 experts)
  bool mxfp4 = false;         // 4-bit experts: the four arrays below instead of wgu, wdp
  bool act_mx = false;        // 4-bit experts with 4-bit activations (the W4A4 GEMMs)
  // routing left in the workspace by beam_moe_forward_boundary_route (the previous layer's
  // call) for the call on routed_z with routed_T tokens; 0: none
  int routed_T = 0;
  const void* routed_z = nullptr;
  bool routed_quant = false;  // ... with the rows' 4-bit quantisation done in that launch
  bool dense = false;         // a dense SwiGLU layer (beam_dense_init): one expert, no routing
  uint8_t* qgu = nullptr;     // gate/up codes, decode layout
  uint8_t* sgu = nullptr;     // gate/up scales
  uint8_t* qd = nullptr;      // down codes
  uint8_t* sd = nullptr;      // down scales
  uint8_t* pqgu = nullptr;    // grouped-GEMM layout of the 4-bit weights (max_tokens > 128)
  uint8_t* psgu = nullptr;
  uint8_t* pqd = nullptr;
  uint8_t* psd = nullptr;
  float* dense_part = nullptr;  // dense layers: FP32 partials of the split-K down pass [4][16][d]
  Workspace ws;                 // owned, sized for max_tokens
  std::vector<void*> allocations;
};

// ---------------------------------------------------------------------------------------------
// Static scratch area for beam_moe_forward_noalloc (callers that cannot allocate device
// memory). Every GPU the library runs on holds one copy, for the life of the process; every
// such call on that GPU shares it. Host code never passes the array's name to a kernel or a
// copy (on the host it only names the symbol): it uses the device address looked up once per
// device by hipGetSymbolAddress while that device is current.
//   bytes [0, kScratchCounterBytes): the fused small-batch routing's arrival counters (zeroed
//                   when the address is looked up; every launch that uses them leaves them zero)
//   bytes [kScratchCounterBytes, kScratchBytes): the per-call workspace of one forward
//                   (carve_scratch)
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr size_t kScratchCounterBytes = (kRouteDoneWords * 4 + 255) & ~(size_t)255;
constexpr int kScratchMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchMaxDevices] = {};

// Look up (once per device) the device address of `scratch` on the current device and zero
// its counter on stream s. Returns the address, or null on failure.
void* scratch_setup(int device, hipStream_t s) {
  if (device < 0 || device >= kScratchMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_ptr[device]) return g_scratch_ptr[device];
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (hipMemsetAsync(ptr, 0, kScratchCounterBytes, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_scratch_ptr[device] = ptr;
  return ptr;
}

void* scratch_of(int device) {
  if (device < 0 || device >= kScratchMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  return g_scratch_ptr[device];
}

// Lay out the workspace of a T-token forward in the scratch area at `base` (256-byte
// aligned pieces after the counters). Returns the bytes used (base may be null to size it).
size_t carve_scratch(const beam_moe_config& c, bool mx, int T, char* base, Workspace* ws) {
  const size_t E = c.n_experts, d = c.hidden, f = c.d_ff, slots = (size_t)T * c.topk;
  const size_t nb = (slots + kPermChunk - 1) / kPermChunk;
  size_t off = kScratchCounterBytes;
  auto take = [&](auto** p, size_t bytes) {
    if (base) *p = reinterpret_cast<std::remove_pointer_t<decltype(p)>>(base + off);
    off += (bytes + 255) & ~(size_t)255;
  };
  Workspace w;
  if (base) w.route_done = reinterpret_cast<uint32_t*>(base);
  take(&w.logits, (size_t)T * E * 4);
  take(&w.ids, slots * 4);
  take(&w.w, slots * 4);
  take(&w.counts, E * 4);
  take(&w.offsets, (E + 1) * 4);
  take(&w.active, E * 4);
  take(&w.n_active, 4);
  take(&w.tile_start, (E + 1) * 4);
  take(&w.perm, slots * 4);
  take(&w.route_sc, (size_t)kFusedRouteMaxT * E * 8);
  take(&w.block_cnt, nb * E * 4);
  take(&w.block_base, nb * E * 4);
  take(&w.act, slots * f * 2);
  take(&w.yk, slots * d * 2);
  if (mx) {
    take(&w.zq, (size_t)T * d / 2);
    take(&w.zqs, (size_t)T * d / 32);
    take(&w.aq, slots * f / 2);
    take(&w.aqs, slots * f / 32);
    if (T <= kStreamMaxT) take(&w.zr, (size_t)T * d * 2);
  }
  if (ws) *ws = w;
  return off;
}

}  // namespace

namespace {

int validate_config(const beam_moe_config* c) {
  if (!c) return BEAM_ERR_INVALID_ARG;
  if (c->hidden <= 0 || c->n_experts <= 0 || c->n_groups <= 0 || c->topk_groups <= 0 ||
      c->topk <= 0 || c->d_ff <= 0 || c->max_tokens <= 0 || !isfinite(c->routed_scale))
    return BEAM_ERR_INVALID_ARG;
  if (c->n_experts % c->n_groups != 0 || c->topk_groups > c->n_groups) return BEAM_ERR_INVALID_ARG;
  const int gs = c->n_experts / c->n_groups;
  if (c->topk > c->topk_groups * gs) return BEAM_ERR_INVALID_ARG;
  if ((int64_t)c->max_tokens * c->topk >= (1ll << 31)) return BEAM_ERR_INVALID_ARG;
  // 32-bit element offsets into activations: T * k * max(d, f) < 2^31
  const int64_t wide = c->hidden > c->d_ff ? c->hidden : c->d_ff;
  if ((int64_t)c->max_tokens * c->topk * wide >= (1ll << 31)) return BEAM_ERR_UNSUPPORTED;
  if (c->hidden % 256 != 0 || c->hidden > 16384) return BEAM_ERR_UNSUPPORTED;
  if (c->d_ff % 256 != 0 || c->d_ff > 32768) return BEAM_ERR_UNSUPPORTED;
  if (c->n_experts > 256 || c->n_groups > 64 || c->topk > 32) return BEAM_ERR_UNSUPPORTED;
  return BEAM_OK;
}

template <class T>
bool dev_alloc(beam_moe_ctx* h, T** p, size_t count) {
  void* q = nullptr;
  if (count == 0) count = 1;
  if (hipMalloc(&q, count * sizeof(T)) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  h->allocations.push_back(q);
  *p = (T*)q;
  return true;
}

void free_all(beam_moe_ctx* h) {
  for (void* p : h->allocations) (void)hipFree(p);
  h->allocations.clear();
}

// Small batches read the FP32 router weight once on the vector ALUs (the bytes are
// the bound); large batches use the exact three-part BF16 split on the matrix cores.
int run_router(beam_moe_ctx* h, int T, const uint16_t* z, float* logits, hipStream_t s) {
  const beam_moe_config& c = h->cfg;
  ProfScope ps(K_ROUTER, s);
  if (T > kStreamMaxT && c.n_experts % 64 == 0) {
    RouterX3Args ra{T, c.hidden, c.n_experts, z, h->router_x3, logits};
    return hip_status(launch_router_bf16x3(ra, s));
  }
  RouterArgs ra{T, c.hidden, c.n_experts, z, h->router_w, logits};
  return hip_status(launch_router_fp32(ra, s));
}

TopkArgs topk_args(beam_moe_ctx* h, const Workspace& ws, int T, const float* logits,
                   int32_t* ids_copy, float* w_copy) {
  const beam_moe_config& c = h->cfg;
  return TopkArgs{T, c.n_experts, c.n_groups, c.topk_groups, c.topk, c.routed_scale,
                  logits, h->bias, ws.ids, ws.w, ids_copy, w_copy};
}

int route(beam_moe_ctx* h, const Workspace& ws, int T, const uint16_t* z, float* logits,
          int32_t* ids_copy, float* w_copy, hipStream_t s) {
  int st = run_router(h, T, z, logits, s);
  if (st != BEAM_OK) return st;
  ProfScope ps(K_TOPK, s);
  return hip_status(launch_topk(topk_args(h, ws, T, logits, ids_copy, w_copy), s));
}

bool overlaps(const void* a, const void* b, int64_t bytes) {
  return (const char*)a < (const char*)b + bytes && (const char*)b < (const char*)a + bytes;
}

// Any call that rewrites a handle's workspace (or changes what its routing launch does)
// drops the routing a previous layer's beam_moe_forward_boundary_route left in it.
void clear_routed(beam_moe_ctx* h) {
  h->routed_T = 0;
  h->routed_z = nullptr;
  h->routed_quant = false;
}

// Computed routing of T rows z (router, grouped top-k, grouping) into ws. bnd (T = 1, d <=
// kBoundaryWgMaxD, k <= kFusedRouteMaxSlots only): the boundary of the token runs inside the
// routing launch and writes z (= bnd->z_out, the z routed) and h'; cb (with bnd): that
// boundary's x is the combine of a previous MoE's rows. With 4-bit activations, the one-launch
// routings also quantise the rows (*quantised is set then).
int route_impl(beam_moe_ctx* h, const Workspace& ws, int T, const uint16_t* z, float* logits_out,
               int32_t* ids_out, float* w_out, int32_t* perm_out, int32_t* offsets_out,
               hipStream_t s, const BoundaryArgs* bnd, const CombineArgs* cb, bool* quantised) {
  const beam_moe_config& c = h->cfg;
  const int k = c.topk, E = c.n_experts;
  const int slots = T * k;
  const bool fused_route = bnd || (T <= kFusedRouteMaxT && slots <= kFusedRouteMaxSlots);
  const RowQuantArgs rq = h->act_mx && T <= kStreamMaxT && fused_route
                              ? RowQuantArgs{ws.zq, ws.zqs, ws.zr}
                              : RowQuantArgs{nullptr, nullptr, nullptr};
  *quantised = rq.zq != nullptr;
  PermArgs pa{slots, E, (slots + kPermChunk - 1) / kPermChunk, kGemmBM, ws.ids, ws.counts,
              ws.offsets, ws.perm, ws.block_cnt, ws.block_base, ws.active, ws.n_active,
              ws.tile_start, perm_out, offsets_out};
  float* lg = logits_out ? logits_out : ws.logits;
  TopkArgs ta = topk_args(h, ws, T, lg, ids_out, w_out);
  if (bnd) {
    ProfScope ps(cb ? K_COMBINE_ROUTE : K_ROUTER, s);  // [combine,] boundary, routing: one launch
    RouterArgs ra{T, c.hidden, E, z, h->router_w, lg};
    return hip_status(
        launch_boundary_route_fused(*bnd, ra, ta, pa, ws.route_done, ws.route_sc, rq, cb, s));
  }
  if (fused_route) {
    ProfScope ps(K_ROUTER, s);  // router, top-k and grouping in one launch
    RouterArgs ra{T, c.hidden, E, z, h->router_w, lg};
    return hip_status(launch_route_fused_tiny(ra, ta, pa, ws.route_done, ws.route_sc, rq, s));
  }
  int st = run_router(h, T, z, lg, s);
  if (st != BEAM_OK) return st;
  // routing and grouping in one workgroup while each of its 16 waves routes at most one
  // token; beyond that the tokens go one per wave over many workgroups (topk_kernel, the
  // same selection) and the grouping follows (one workgroup up to kPermChunk slots)
  if (slots <= kPermChunk && T <= kRoutePermuteSmallMaxT) {
    ProfScope ps(K_PERMUTE, s);
    return hip_status(launch_route_permute_small(ta, pa, s));
  }
  {
    ProfScope ps(K_TOPK, s);
    if (launch_topk(ta, s) != hipSuccess) return BEAM_ERR_HIP;
  }
  ProfScope ps(K_PERMUTE, s);
  return hip_status(launch_permute(pa, s));
}

// The MoE forward after validation. Routing: replayed (ids_in), left by the previous layer's
// call (pre_routed; pre_quantised: with the rows' 4-bit quantisation) or computed here (bnd:
// see route_impl). Tail: the combine into y_out; post: the next sublayer's boundary with x =
// the MoE output, in the combine launch (d <= kBoundaryWgMaxD; y_out may then be null) or
// after it (wider rows, through y_out); next (with post): then the next layer's routing of
// post->z_out into next's workspace — for one token in the same launch as the combine and
// the boundary.
int forward_impl(beam_moe_ctx* h, const Workspace& ws, int T, const uint16_t* z, uint16_t* y_out,
                 const int32_t* ids_in, const float* w_in, float* logits_out, int32_t* ids_out,
                 float* w_out, int32_t* perm_out, int32_t* offsets_out, hipStream_t s,
                 const BoundaryArgs* bnd, const BoundaryArgs* post, bool pre_routed = false,
                 bool pre_quantised = false, beam_moe_ctx* next = nullptr) {
  const beam_moe_config& c = h->cfg;
  const int k = c.topk, E = c.n_experts;
  const int slots = T * k;

  const int32_t* ids = ids_in ? ids_in : ws.ids;
  const float* w = w_in ? w_in : ws.w;
  bool rows_quantised = pre_quantised;
  if (ids_in) {
    if (ids_out &&
        hipMemcpyAsync(ids_out, ids_in, (size_t)slots * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
      return BEAM_ERR_HIP;
    if (w_out &&
        hipMemcpyAsync(w_out, w_in, (size_t)slots * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
      return BEAM_ERR_HIP;
    PermArgs pa{slots, E, (slots + kPermChunk - 1) / kPermChunk, kGemmBM, ids, ws.counts,
                ws.offsets, ws.perm, ws.block_cnt, ws.block_base, ws.active, ws.n_active,
                ws.tile_start, perm_out, offsets_out};
    ProfScope ps(K_PERMUTE, s);
    if (launch_permute(pa, s) != hipSuccess) return BEAM_ERR_HIP;
  } else if (!pre_routed) {
    const int st = route_impl(h, ws, T, z, logits_out, ids_out, w_out, perm_out, offsets_out, s,
                              bnd, nullptr, &rows_quantised);
    if (st != BEAM_OK) return st;
  }
  const bool a4_stream = h->act_mx && T <= kStreamMaxT;
  ExpertArgs ea{T, k, c.hidden, c.d_ff, E, z, h->wgu, h->wdp, ws.perm, ws.offsets, ws.active,
                ws.n_active, ws.tile_start, w, ws.act, ws.yk, h->qgu, h->sgu, h->qd, h->sd,
                h->pqgu, h->psgu, h->pqd, h->psd};
  if (h->act_mx) {  // 4-bit activations: quantise the token rows, then the W4A4 GEMMs
    ea.zq = ws.zq;
    ea.zqs = ws.zqs;
    ea.aq = ws.aq;
    ea.aqs = ws.aqs;
    const bool stream = a4_stream;
    if (!rows_quantised) {
      ProfScope ps(K_QUANT, s);
      if (launch_quantize_rows_a4((int64_t)T * (c.hidden / 32), z, ws.zq, ws.zqs,
                                  stream ? ws.zr : nullptr, s) != hipSuccess)
        return BEAM_ERR_HIP;
    }
    if (stream) {
      // the 4-bit weight streams on the rows' round trip, the activations' round trip between
      // them: the same values the W4A4 GEMMs multiply
      const int max_active = slots < E ? slots : E;
      ExpertArgs es = ea;
      es.z = ws.zr;
      {
        ProfScope ps(K_GATEUP, s);
        if (launch_gateup_fp4(es, max_active, s) != hipSuccess) return BEAM_ERR_HIP;
      }
      if (!down_fp4_rounds_act(es)) {  // one token: the down pass rounds its row itself
        ProfScope ps(K_QUANT, s);
        if (launch_act_round_trip_a4(slots, c.d_ff, ws.offsets + E, ws.act, ws.aq, ws.aqs, s) !=
            hipSuccess)
          return BEAM_ERR_HIP;
      }
      ProfScope ps(K_DOWN, s);
      if (launch_down_fp4(es, max_active, s) != hipSuccess) return BEAM_ERR_HIP;
    } else {
      const int max_tiles = (slots + kGemmBM - 1) / kGemmBM + (slots < E ? slots : E);
      {
        ProfScope ps(K_GATEUP, s);
        if (launch_gateup_gemm_a4(ea, max_tiles, s) != hipSuccess) return BEAM_ERR_HIP;
      }
      ProfScope ps(K_DOWN, s);
      if (launch_down_gemm_a4(ea, max_tiles, s) != hipSuccess) return BEAM_ERR_HIP;
    }
  } else if (h->mxfp4 && T > kStreamMaxT) {  // 4-bit grouped GEMMs
    const int max_tiles = (slots + kGemmBM - 1) / kGemmBM + (slots < E ? slots : E);
    {
      ProfScope ps(K_GATEUP, s);
      if (launch_gateup_gemm_fp4(ea, max_tiles, s) != hipSuccess) return BEAM_ERR_HIP;
    }
    ProfScope ps(K_DOWN, s);
    if (launch_down_gemm_fp4(ea, max_tiles, s) != hipSuccess) return BEAM_ERR_HIP;
  } else if (h->mxfp4) {  // 4-bit weight-streaming passes
    const int max_active = slots < E ? slots : E;
    {
      ProfScope ps(K_GATEUP, s);
      if (launch_gateup_fp4(ea, max_active, s) != hipSuccess) return BEAM_ERR_HIP;
    }
    ProfScope ps(K_DOWN, s);
    if (launch_down_fp4(ea, max_active, s) != hipSuccess) return BEAM_ERR_HIP;
  } else if (T <= kStreamMaxT) {
    const int max_active = slots < E ? slots : E;
    {
      ProfScope ps(K_GATEUP, s);
      if (launch_gateup_stream(ea, max_active, s) != hipSuccess) return BEAM_ERR_HIP;
    }
    ProfScope ps(K_DOWN, s);
    if (T <= kSplitDownMaxT) {
      if (launch_down_split(ea, max_active, s) != hipSuccess) return BEAM_ERR_HIP;
    } else if (launch_down_stream(ea, max_active, s) != hipSuccess) {
      return BEAM_ERR_HIP;
    }
  } else {
    const int max_tiles = (slots + kGemmBM - 1) / kGemmBM + (slots < E ? slots : E);
    {
      ProfScope ps(K_GATEUP, s);
      if (launch_gateup_gemm(ea, max_tiles, s) != hipSuccess) return BEAM_ERR_HIP;
    }
    {
      ProfScope ps(K_DOWN, s);
      if (launch_down_gemm(ea, max_tiles, s) != hipSuccess) return BEAM_ERR_HIP;
    }
  }
  if (next && T == 1 && c.hidden <= kBoundaryWgMaxD && k <= kChainMaxK &&
      next->cfg.topk <= kFusedRouteMaxSlots) {
    // combine, next boundary and the next layer's routing in one launch
    const CombineArgs cb{k, E, ids, ws.yk, y_out};
    bool q = false;
    const int st = route_impl(next, next->ws, T, post->z_out, nullptr, nullptr, nullptr, nullptr,
                              nullptr, s, post, &cb, &q);
    if (st == BEAM_OK) {
      next->routed_T = T;
      next->routed_z = post->z_out;
      next->routed_quant = q;
    }
    return st;
  }
  {
    ProfScope ps(K_COMBINE, s);
    if (!post) return hip_status(launch_combine(T, k, c.hidden, E, ids, ws.yk, y_out, s));
    if (c.hidden <= kBoundaryWgMaxD) {
      if (launch_combine_boundary(*post, CombineArgs{k, E, ids, ws.yk, y_out}, s) != hipSuccess)
        return BEAM_ERR_HIP;
    } else {
      if (launch_combine(T, k, c.hidden, E, ids, ws.yk, y_out, s) != hipSuccess)
        return BEAM_ERR_HIP;
      BoundaryArgs pb = *post;
      pb.x = y_out;
      if (launch_boundary(pb, s) != hipSuccess) return BEAM_ERR_HIP;
    }
  }
  if (!next) return BEAM_OK;
  bool q = false;
  const int st = route_impl(next, next->ws, T, post->z_out, nullptr, nullptr, nullptr, nullptr,
                            nullptr, s, nullptr, nullptr, &q);
  if (st == BEAM_OK) {
    next->routed_T = T;
    next->routed_z = post->z_out;
    next->routed_quant = q;
  }
  return st;
}


}  // namespace

extern "C" {

const char* beam_status_string(int status) {
  switch (status) {
    case BEAM_OK: return "ok";
    case BEAM_ERR_INVALID_ARG: return "invalid argument";
    case BEAM_ERR_UNSUPPORTED: return "unsupported shape";
    case BEAM_ERR_OOM: return "out of device memory";
    case BEAM_ERR_HIP: return "HIP runtime error";
    case BEAM_ERR_CAPACITY: return "T exceeds the handle's max_tokens";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// Shared part of the two init entry points: the handle, the router copies and all
// workspace; `experts` allocates and fills the expert weights on stream s.
template <class Experts>
int init_handle(const beam_moe_config* cfg, const float* router_w, const float* router_bias,
                void* stream, beam_moe_handle* out, Experts experts) {
  beam_moe_ctx* h = new (std::nothrow) beam_moe_ctx();
  if (!h) return BEAM_ERR_OOM;
  h->cfg = *cfg;
  const beam_moe_config& c = h->cfg;
  hipStream_t s = (hipStream_t)stream;
  if (hipGetDevice(&h->device) != hipSuccess) {
    delete h;
    return BEAM_ERR_HIP;
  }
  // the allocation-free forward's scratch address on this device (its own failure only
  // makes that entry point return BEAM_ERR_HIP)
  (void)scratch_setup(h->device, s);
  const size_t E = c.n_experts, d = c.hidden, f = c.d_ff, k = c.topk, T = c.max_tokens;
  const size_t slots = T * k;
  const size_t nb = (slots + kPermChunk - 1) / kPermChunk;
  bool ok = dev_alloc(h, &h->router_w, E * d) && dev_alloc(h, &h->router_x3, 3 * E * d) &&
            dev_alloc(h, &h->bias, E) &&
            dev_alloc(h, &h->ws.logits, T * E) && dev_alloc(h, &h->ws.ids, slots) &&
            dev_alloc(h, &h->ws.w, slots) && dev_alloc(h, &h->ws.counts, E) &&
            dev_alloc(h, &h->ws.offsets, E + 1) && dev_alloc(h, &h->ws.active, E) &&
            dev_alloc(h, &h->ws.n_active, 1) && dev_alloc(h, &h->ws.tile_start, E + 1) &&
            dev_alloc(h, &h->ws.perm, slots) && dev_alloc(h, &h->ws.route_done, kRouteDoneWords) &&
            dev_alloc(h, &h->ws.route_sc, (size_t)kFusedRouteMaxT * E) &&
            dev_alloc(h, &h->ws.block_cnt, nb * E) &&
            dev_alloc(h, &h->ws.block_base, nb * E) && dev_alloc(h, &h->ws.act, slots * f) &&
            dev_alloc(h, &h->ws.yk, slots * d);
  hipError_t e = hipSuccess;
  if (ok) {
    const int st = experts(h, s);
    if (st == BEAM_ERR_OOM) ok = false;
    else if (st != BEAM_OK) e = hipErrorUnknown;
  }
  if (!ok) {
    free_all(h);
    delete h;
    return BEAM_ERR_OOM;
  }
  if (e == hipSuccess)
    e = router_w ? hipMemcpyAsync(h->router_w, router_w, E * d * sizeof(float),
                                  hipMemcpyDeviceToDevice, s)
                 : hipMemsetAsync(h->router_w, 0, E * d * sizeof(float), s);
  if (e == hipSuccess)
    e = router_bias ? hipMemcpyAsync(h->bias, router_bias, E * sizeof(float),
                                     hipMemcpyDeviceToDevice, s)
                    : hipMemsetAsync(h->bias, 0, E * sizeof(float), s);
  if (e == hipSuccess) e = hipMemsetAsync(h->ws.route_done, 0, kRouteDoneWords * sizeof(uint32_t), s);
  if (e == hipSuccess && E % 64 == 0 && router_w)
    e = launch_repack_router(router_w, h->router_x3, (int)E, (int)d, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    free_all(h);
    delete h;
    return BEAM_ERR_HIP;
  }
  *out = h;
  return BEAM_OK;
}

}  // namespace

extern "C" {

int beam_moe_init(const beam_moe_config* cfg, const float* router_w, const float* router_bias,
                  const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                  void* stream, beam_moe_handle* out) {
  int st = validate_config(cfg);
  if (st != BEAM_OK) return st;
  if (!out || !router_w || !router_bias || !w_gate || !w_up || !w_down) return BEAM_ERR_INVALID_ARG;
  if (!aligned16(router_w) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      ((uintptr_t)router_bias & 3u))
    return BEAM_ERR_INVALID_ARG;
  return init_handle(cfg, router_w, router_bias, stream, out, [&](beam_moe_ctx* h, hipStream_t s) -> int {
    const size_t E = cfg->n_experts, d = cfg->hidden, f = cfg->d_ff;
    if (!dev_alloc(h, &h->wgu, E * 2 * f * d) || !dev_alloc(h, &h->wdp, E * d * f))
      return BEAM_ERR_OOM;
    return hip_status(launch_repack(w_gate, w_up, w_down, h->wgu, h->wdp, (int)E, (int)f, (int)d, s));
  });
}

int beam_moe_init_mxfp4(const beam_moe_config* cfg, const float* router_w,
                        const float* router_bias, const uint8_t* gate_codes,
                        const uint8_t* gate_scales, const uint8_t* up_codes,
                        const uint8_t* up_scales, const uint8_t* down_codes,
                        const uint8_t* down_scales, void* stream, beam_moe_handle* out) {
  int st = validate_config(cfg);
  if (st != BEAM_OK) return st;
  if (cfg->hidden % 512 != 0 || cfg->d_ff % 512 != 0) return BEAM_ERR_UNSUPPORTED;
  if (!out || !router_w || !router_bias || !gate_codes || !gate_scales || !up_codes ||
      !up_scales || !down_codes || !down_scales)
    return BEAM_ERR_INVALID_ARG;
  if (!aligned16(router_w) || ((uintptr_t)router_bias & 3u) || ((uintptr_t)gate_codes & 3u) ||
      ((uintptr_t)up_codes & 3u) || ((uintptr_t)down_codes & 3u))
    return BEAM_ERR_INVALID_ARG;
  return init_handle(cfg, router_w, router_bias, stream, out, [&](beam_moe_ctx* h, hipStream_t s) -> int {
    const size_t E = cfg->n_experts, d = cfg->hidden, f = cfg->d_ff;
    h->mxfp4 = true;
    if (!dev_alloc(h, &h->qgu, E * 2 * f * d / 2) || !dev_alloc(h, &h->sgu, E * 2 * f * d / 32) ||
        !dev_alloc(h, &h->qd, E * d * f / 2) || !dev_alloc(h, &h->sd, E * d * f / 32))
      return BEAM_ERR_OOM;
    if (launch_repack_mxfp4(gate_codes, gate_scales, up_codes, up_scales, down_codes, down_scales,
                            (int)E, (int)f, (int)d, h->qgu, h->sgu, h->qd, h->sd, s) != hipSuccess)
      return BEAM_ERR_HIP;
    const size_t T = cfg->max_tokens;
    const size_t S = T * cfg->topk, Ts = T < (size_t)kStreamMaxT ? T : (size_t)kStreamMaxT;
    if (!dev_alloc(h, &h->ws.zq, T * d / 2) || !dev_alloc(h, &h->ws.zqs, T * d / 32) ||
        !dev_alloc(h, &h->ws.aq, S * f / 2) || !dev_alloc(h, &h->ws.aqs, S * f / 32) ||
        !dev_alloc(h, &h->ws.zr, Ts * d))
      return BEAM_ERR_OOM;
    if (!dev_alloc(h, &h->pqgu, E * 2 * f * d / 2) || !dev_alloc(h, &h->psgu, E * 2 * f * d / 32) ||
        !dev_alloc(h, &h->pqd, E * d * f / 2) || !dev_alloc(h, &h->psd, E * d * f / 32))
      return BEAM_ERR_OOM;
    return hip_status(launch_repack_mxfp4_gemm(gate_codes, gate_scales, up_codes, up_scales,
                                               down_codes, down_scales, (int)E, (int)f, (int)d,
                                               h->pqgu, h->psgu, h->pqd, h->psd, s));
  });
}

int beam_mxfp4_quantize(int64_t rows, int32_t K, const uint16_t* src, uint8_t* codes_out,
                        uint8_t* scales_out, void* stream) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return BEAM_ERR_INVALID_ARG;
  if (rows > ((int64_t)1 << 40) / K) return BEAM_ERR_UNSUPPORTED;
  if (rows == 0) return BEAM_OK;
  if (!src || !codes_out || !scales_out || !aligned16(src) || !aligned16(codes_out))
    return BEAM_ERR_INVALID_ARG;
  return hip_status(launch_mxfp4_quantize(rows * (K / 32), src, codes_out, scales_out,
                                          (hipStream_t)stream));
}

int beam_moe_set_activation_format(beam_moe_handle h, int32_t format) {
  if (!h || h->dense || (format != BEAM_ACT_BF16 && format != BEAM_ACT_MXFP4))
    return BEAM_ERR_INVALID_ARG;
  if (format == BEAM_ACT_MXFP4 && !h->mxfp4) return BEAM_ERR_UNSUPPORTED;
  h->act_mx = format == BEAM_ACT_MXFP4;
  clear_routed(h);
  return BEAM_OK;
}

int beam_moe_inspect(beam_moe_handle h, int32_t what, const void** ptr) {
  if (!h || !ptr) return BEAM_ERR_INVALID_ARG;
  const Workspace& ws = h->ws;
  switch (what) {
    case BEAM_INSPECT_ACT: *ptr = ws.act; break;
    case BEAM_INSPECT_ACT_CODES: *ptr = h->act_mx ? (const void*)ws.aq : nullptr; break;
    case BEAM_INSPECT_ACT_SCALES: *ptr = h->act_mx ? (const void*)ws.aqs : nullptr; break;
    case BEAM_INSPECT_Z_CODES: *ptr = ws.zq; break;
    case BEAM_INSPECT_Z_SCALES: *ptr = ws.zqs; break;
    default: return BEAM_ERR_INVALID_ARG;
  }
  return *ptr ? BEAM_OK : BEAM_ERR_UNSUPPORTED;
}

int beam_dense_init(int32_t hidden, int32_t d_ff, int32_t max_tokens, const uint16_t* w_gate,
                    const uint16_t* w_up, const uint16_t* w_down, void* stream,
                    beam_moe_handle* out) {
  beam_moe_config cfg{hidden, 1, 1, 1, 1, d_ff, max_tokens, 1.0f};
  int st = validate_config(&cfg);
  if (st != BEAM_OK) return st;
  if (!out || !w_gate || !w_up || !w_down) return BEAM_ERR_INVALID_ARG;
  if (!aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down)) return BEAM_ERR_INVALID_ARG;
  return init_handle(&cfg, nullptr, nullptr, stream, out, [&](beam_moe_ctx* h, hipStream_t s) -> int {
    const size_t d = hidden, f = d_ff;
    h->dense = true;
    if (!dev_alloc(h, &h->wgu, 2 * f * d) || !dev_alloc(h, &h->wdp, d * f) ||
        !dev_alloc(h, &h->dense_part, (size_t)kDenseSplitK * 16 * d))
      return BEAM_ERR_OOM;
    if (launch_repack(w_gate, w_up, w_down, h->wgu, h->wdp, 1, (int)f, (int)d, s) != hipSuccess)
      return BEAM_ERR_HIP;
    const Workspace& ws = h->ws;
    PermArgs pa{max_tokens, 1, 1, kGemmBM, nullptr, ws.counts, ws.offsets, ws.perm, nullptr,
                nullptr, ws.active, ws.n_active, ws.tile_start, nullptr, nullptr};
    return hip_status(launch_dense_plan(0, max_tokens, true, pa, ws.w, s));
  });
}

int beam_dense_forward(beam_moe_handle h, int32_t T, const uint16_t* z, uint16_t* y_out,
                       void* stream) {
  if (!h || !h->dense || T < 0) return BEAM_ERR_INVALID_ARG;
  if (T > h->cfg.max_tokens) return BEAM_ERR_CAPACITY;
  if (T == 0) return BEAM_OK;
  const beam_moe_config& c = h->cfg;
  if (!z || !y_out || !aligned16(z) || !aligned16(y_out) ||
      overlaps(z, y_out, (int64_t)T * c.hidden * 2))
    return BEAM_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const Workspace& ws = h->ws;
  PermArgs pa{T, 1, 1, kGemmBM, nullptr, ws.counts, ws.offsets, ws.perm, nullptr, nullptr,
              ws.active, ws.n_active, ws.tile_start, nullptr, nullptr};
  {
    ProfScope ps(K_PERMUTE, s);
    if (launch_dense_plan(T, c.max_tokens, false, pa, ws.w, s) != hipSuccess) return BEAM_ERR_HIP;
  }
  // the down pass writes each row's bf16(1 * sum) straight to y (one slot per token)
  ExpertArgs ea{T, 1, c.hidden, c.d_ff, 1, z, h->wgu, h->wdp, ws.perm, ws.offsets, ws.active,
                ws.n_active, ws.tile_start, ws.w, ws.act, y_out};
  if (T <= kStreamMaxT) {
    {
      ProfScope ps(K_GATEUP, s);
      if (launch_gateup_stream(ea, 1, s) != hipSuccess) return BEAM_ERR_HIP;
    }
    ProfScope ps(K_DOWN, s);
    if (T <= kSplitDownMaxT && (c.d_ff / 32) % (4 * kDenseSplitK) == 0)
      return hip_status(launch_down_splitk_dense(ea, kDenseSplitK, h->dense_part, s));
    return hip_status(T <= kSplitDownMaxT ? launch_down_split(ea, 1, s) : launch_down_stream(ea, 1, s));
  }
  const int max_tiles = (T + kGemmBM - 1) / kGemmBM + 1;
  {
    ProfScope ps(K_GATEUP, s);
    if (launch_gateup_gemm(ea, max_tiles, s) != hipSuccess) return BEAM_ERR_HIP;
  }
  ProfScope ps(K_DOWN, s);
  return hip_status(launch_down_gemm(ea, max_tiles, s));
}

int beam_moe_destroy(beam_moe_handle h) {
  if (!h) return BEAM_OK;
  int st = hip_status(hipDeviceSynchronize());
  free_all(h);
  delete h;
  return st;
}

int beam_sublayer_norm_residual(int32_t T, int32_t d, const uint16_t* h_in, const uint16_t* x,
                                const uint16_t* w_post, const uint16_t* w_pre, int32_t n,
                                float eps, uint16_t* h_out, uint16_t* z_out, void* stream) {
  if (T < 0 || d <= 0 || (d % 8) != 0 || n < 1 || !(eps >= 0.0f) || !isfinite(eps))
    return BEAM_ERR_INVALID_ARG;
  if (d > 65536) return BEAM_ERR_UNSUPPORTED;
  if (T == 0) return BEAM_OK;
  if (!h_in || !x || !w_post || !w_pre || !h_out || !z_out) return BEAM_ERR_INVALID_ARG;
  if (!aligned16(h_in) || !aligned16(x) || !aligned16(w_post) || !aligned16(w_pre) ||
      !aligned16(h_out) || !aligned16(z_out))
    return BEAM_ERR_INVALID_ARG;
  const float c1 = (float)sqrt((double)(n - 1) / (double)n);
  const float c2 = (float)(1.0 / sqrt((double)n));
  hipStream_t s = (hipStream_t)stream;
  ProfScope ps(K_BOUNDARY, s);
  BoundaryArgs a{T, d, h_in, x, w_post, w_pre, h_out, z_out, c1, c2, eps};
  return hip_status(launch_boundary(a, s));
}

int beam_router_topk(beam_moe_handle h, int32_t T, const uint16_t* z, float* logits_out,
                     int32_t* ids_out, float* w_out, void* stream) {
  if (!h || h->dense || T < 0) return BEAM_ERR_INVALID_ARG;
  if (T > h->cfg.max_tokens) return BEAM_ERR_CAPACITY;
  if (T == 0) return BEAM_OK;
  if (!z || !ids_out || !w_out || !aligned16(z) || ((uintptr_t)ids_out & 3u) ||
      ((uintptr_t)w_out & 3u) || (logits_out && ((uintptr_t)logits_out & 3u)))
    return BEAM_ERR_INVALID_ARG;
  clear_routed(h);
  return route(h, h->ws, T, z, logits_out ? logits_out : h->ws.logits, ids_out, w_out,
               (hipStream_t)stream);
}

int beam_grouped_topk(beam_moe_handle h, int32_t T, const float* logits, int32_t* ids_out,
                      float* w_out, void* stream) {
  if (!h || h->dense || T < 0) return BEAM_ERR_INVALID_ARG;
  if (T > h->cfg.max_tokens) return BEAM_ERR_CAPACITY;
  if (T == 0) return BEAM_OK;
  if (!logits || !ids_out || !w_out || ((uintptr_t)logits & 3u) || ((uintptr_t)ids_out & 3u) ||
      ((uintptr_t)w_out & 3u))
    return BEAM_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  clear_routed(h);
  ProfScope ps(K_TOPK, s);
  TopkArgs ta = topk_args(h, h->ws, T, logits, nullptr, nullptr);
  ta.ids = ids_out;
  ta.w = w_out;
  return hip_status(launch_topk(ta, s));
}

int beam_moe_forward(beam_moe_handle h, int32_t T, const uint16_t* z, uint16_t* y_out,
                     const int32_t* ids_in, const float* w_in, float* logits_out,
                     int32_t* ids_out, float* w_out, int32_t* perm_out, int32_t* offsets_out,
                     void* stream) {
  if (!h || h->dense || T < 0) return BEAM_ERR_INVALID_ARG;
  if (T > h->cfg.max_tokens) return BEAM_ERR_CAPACITY;
  if (T == 0) return BEAM_OK;
  if (!z || !y_out || !aligned16(z) || !aligned16(y_out)) return BEAM_ERR_INVALID_ARG;
  if ((ids_in == nullptr) != (w_in == nullptr)) return BEAM_ERR_INVALID_ARG;
  if (ids_in && logits_out) return BEAM_ERR_INVALID_ARG;
  const void* ptrs4[] = {ids_in, w_in, logits_out, ids_out, w_out, perm_out, offsets_out};
  for (const void* p : ptrs4)
    if (p && ((uintptr_t)p & 3u)) return BEAM_ERR_INVALID_ARG;
  const beam_moe_config& c = h->cfg;
  if (overlaps(y_out, z, (int64_t)T * c.hidden * 2)) return BEAM_ERR_INVALID_ARG;
  clear_routed(h);
  return forward_impl(h, h->ws, T, z, y_out, ids_in, w_in, logits_out, ids_out, w_out, perm_out,
                      offsets_out, (hipStream_t)stream, nullptr, nullptr);
}

int beam_moe_forward_noalloc(beam_moe_handle h, int32_t T, const uint16_t* z, uint16_t* y_out,
                             const int32_t* ids_in, const float* w_in, float* logits_out,
                             int32_t* ids_out, float* w_out, int32_t* perm_out,
                             int32_t* offsets_out, void* stream) {
  if (!h || h->dense || T < 0) return BEAM_ERR_INVALID_ARG;
  if (T > h->cfg.max_tokens) return BEAM_ERR_CAPACITY;
  if (T == 0) return BEAM_OK;
  if (carve_scratch(h->cfg, h->mxfp4, T, nullptr, nullptr) > kScratchBytes) return BEAM_ERR_CAPACITY;
  if (!z || !y_out || !aligned16(z) || !aligned16(y_out)) return BEAM_ERR_INVALID_ARG;
  if ((ids_in == nullptr) != (w_in == nullptr)) return BEAM_ERR_INVALID_ARG;
  if (ids_in && logits_out) return BEAM_ERR_INVALID_ARG;
  const void* ptrs4[] = {ids_in, w_in, logits_out, ids_out, w_out, perm_out, offsets_out};
  for (const void* p : ptrs4)
    if (p && ((uintptr_t)p & 3u)) return BEAM_ERR_INVALID_ARG;
  const beam_moe_config& c = h->cfg;
  if (overlaps(y_out, z, (int64_t)T * c.hidden * 2)) return BEAM_ERR_INVALID_ARG;
  char* base = static_cast<char*>(scratch_of(h->device));
  if (!base) return BEAM_ERR_HIP;
  Workspace ws;
  carve_scratch(c, h->mxfp4, T, base, &ws);
  return forward_impl(h, ws, T, z, y_out, ids_in, w_in, logits_out, ids_out, w_out, perm_out,
                      offsets_out, (hipStream_t)stream, nullptr, nullptr);
}

int beam_moe_forward_boundary(beam_moe_handle h, int32_t T, const uint16_t* z,
                              const uint16_t* h_in, const uint16_t* w_post, const uint16_t* w_pre,
                              int32_t n, float eps, uint16_t* h_out, uint16_t* z_out,
                              uint16_t* y_out, const int32_t* ids_in, const float* w_in,
                              float* logits_out, int32_t* ids_out, float* w_out, void* stream) {
  if (!h || h->dense || T < 0) return BEAM_ERR_INVALID_ARG;
  if (T > h->cfg.max_tokens) return BEAM_ERR_CAPACITY;
  if (T == 0) return BEAM_OK;
  const beam_moe_config& c = h->cfg;
  const int d = c.hidden;
  if (n < 1 || !(eps >= 0.0f) || !isfinite(eps)) return BEAM_ERR_INVALID_ARG;
  if (!z || !h_in || !w_post || !w_pre || !h_out || !z_out) return BEAM_ERR_INVALID_ARG;
  if (!aligned16(z) || !aligned16(h_in) || !aligned16(w_post) || !aligned16(w_pre) ||
      !aligned16(h_out) || !aligned16(z_out) || (y_out && !aligned16(y_out)))
    return BEAM_ERR_INVALID_ARG;
  if ((ids_in == nullptr) != (w_in == nullptr)) return BEAM_ERR_INVALID_ARG;
  if (ids_in && logits_out) return BEAM_ERR_INVALID_ARG;
  const void* ptrs4[] = {ids_in, w_in, logits_out, ids_out, w_out};
  for (const void* p : ptrs4)
    if (p && ((uintptr_t)p & 3u)) return BEAM_ERR_INVALID_ARG;
  if (d > kBoundaryWgMaxD && !y_out) return BEAM_ERR_UNSUPPORTED;
  const int64_t bytes = (int64_t)T * d * 2;
  // the boundary reads h_in row by row before writing that row's h_out (so h_out may
  // be h_in) and z_out; z is consumed by the expert launches before it runs (so z_out
  // may be z)
  if ((h_out != h_in && overlaps(h_out, h_in, bytes)) || overlaps(h_out, z_out, bytes) ||
      overlaps(z_out, h_in, bytes) || (z_out != z && overlaps(z_out, z, bytes)) ||
      overlaps(h_out, z, bytes))
    return BEAM_ERR_INVALID_ARG;
  if (y_out) {
    const void* others[] = {z, h_in, h_out, z_out};
    for (const void* p : others)
      if (overlaps(y_out, p, bytes)) return BEAM_ERR_INVALID_ARG;
  }
  const float c1 = (float)sqrt((double)(n - 1) / (double)n);
  const float c2 = (float)(1.0 / sqrt((double)n));
  BoundaryArgs post{T, d, h_in, nullptr, w_post, w_pre, h_out, z_out, c1, c2, eps};
  clear_routed(h);
  return forward_impl(h, h->ws, T, z, y_out, ids_in, w_in, logits_out, ids_out, w_out, nullptr,
                      nullptr, (hipStream_t)stream, nullptr, &post);
}

int beam_moe_forward_boundary_route(beam_moe_handle h, beam_moe_handle next, int32_t T,
                                    const uint16_t* z, const uint16_t* h_in,
                                    const uint16_t* w_post, const uint16_t* w_pre, int32_t n,
                                    float eps, uint16_t* h_out, uint16_t* z_out, uint16_t* y_out,
                                    int32_t routed, void* stream) {
  if (!h || !next || h->dense || next->dense || T < 0) return BEAM_ERR_INVALID_ARG;
  if (next->cfg.hidden != h->cfg.hidden) return BEAM_ERR_INVALID_ARG;
  if (T > h->cfg.max_tokens || T > next->cfg.max_tokens) return BEAM_ERR_CAPACITY;
  if (T == 0) return BEAM_OK;
  const int d = h->cfg.hidden;
  if (n < 1 || !(eps >= 0.0f) || !isfinite(eps)) return BEAM_ERR_INVALID_ARG;
  if (!z || !h_in || !w_post || !w_pre || !h_out || !z_out) return BEAM_ERR_INVALID_ARG;
  if (!aligned16(z) || !aligned16(h_in) || !aligned16(w_post) || !aligned16(w_pre) ||
      !aligned16(h_out) || !aligned16(z_out) || (y_out && !aligned16(y_out)))
    return BEAM_ERR_INVALID_ARG;
  if (d > kBoundaryWgMaxD && !y_out) return BEAM_ERR_UNSUPPORTED;
  const int64_t bytes = (int64_t)T * d * 2;
  // as beam_moe_forward_boundary: h_out may be h_in and z_out may be z
  if ((h_out != h_in && overlaps(h_out, h_in, bytes)) || overlaps(h_out, z_out, bytes) ||
      overlaps(z_out, h_in, bytes) || (z_out != z && overlaps(z_out, z, bytes)) ||
      overlaps(h_out, z, bytes))
    return BEAM_ERR_INVALID_ARG;
  if (y_out) {
    const void* others[] = {z, h_in, h_out, z_out};
    for (const void* p : others)
      if (overlaps(y_out, p, bytes)) return BEAM_ERR_INVALID_ARG;
  }
  if (routed && (h->routed_T != T || h->routed_z != z)) return BEAM_ERR_INVALID_ARG;
  const bool pre_quantised = routed && h->routed_quant;
  clear_routed(h);
  clear_routed(next);
  const float c1 = (float)sqrt((double)(n - 1) / (double)n);
  const float c2 = (float)(1.0 / sqrt((double)n));
  BoundaryArgs post{T, d, h_in, nullptr, w_post, w_pre, h_out, z_out, c1, c2, eps};
  return forward_impl(h, h->ws, T, z, y_out, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                      nullptr, (hipStream_t)stream, nullptr, &post, routed != 0, pre_quantised,
                      next);
}

int beam_sublayer_forward(beam_moe_handle h, int32_t T, const uint16_t* h_in, const uint16_t* x,
                          const uint16_t* w_post, const uint16_t* w_pre, int32_t n, float eps,
                          uint16_t* h_out, uint16_t* z_out, uint16_t* y_out, float* logits_out,
                          int32_t* ids_out, float* w_out, void* stream) {
  if (!h || h->dense || T < 0) return BEAM_ERR_INVALID_ARG;
  if (T > h->cfg.max_tokens) return BEAM_ERR_CAPACITY;
  if (T == 0) return BEAM_OK;
  const beam_moe_config& c = h->cfg;
  const int d = c.hidden;
  if (n < 1 || !(eps >= 0.0f) || !isfinite(eps)) return BEAM_ERR_INVALID_ARG;
  if (!h_in || !x || !w_post || !w_pre || !h_out || !z_out || !y_out) return BEAM_ERR_INVALID_ARG;
  if (!aligned16(h_in) || !aligned16(x) || !aligned16(w_post) || !aligned16(w_pre) ||
      !aligned16(h_out) || !aligned16(z_out) || !aligned16(y_out))
    return BEAM_ERR_INVALID_ARG;
  const void* ptrs4[] = {logits_out, ids_out, w_out};
  for (const void* p : ptrs4)
    if (p && ((uintptr_t)p & 3u)) return BEAM_ERR_INVALID_ARG;
  const int64_t bytes = (int64_t)T * d * 2;
  // z_out and y_out are written while the inputs are still read; only h_out may be h_in
  const void* ins[] = {h_in, x};
  for (const void* p : ins)
    if (overlaps(p, z_out, bytes) || overlaps(p, y_out, bytes)) return BEAM_ERR_INVALID_ARG;
  if (overlaps(z_out, y_out, bytes) || overlaps(h_out, z_out, bytes) ||
      overlaps(h_out, y_out, bytes) || (h_out != h_in && overlaps(h_out, h_in, bytes)) ||
      overlaps(h_out, x, bytes))
    return BEAM_ERR_INVALID_ARG;
  const float c1 = (float)sqrt((double)(n - 1) / (double)n);
  const float c2 = (float)(1.0 / sqrt((double)n));
  hipStream_t s = (hipStream_t)stream;
  clear_routed(h);
  BoundaryArgs ba{T, d, h_in, x, w_post, w_pre, h_out, z_out, c1, c2, eps};
  if (T == 1 && d <= kBoundaryWgMaxD && c.topk <= kFusedRouteMaxSlots)
    return forward_impl(h, h->ws, T, z_out, y_out, nullptr, nullptr, logits_out, ids_out, w_out,
                        nullptr, nullptr, s, &ba, nullptr);
  {
    ProfScope ps(K_BOUNDARY, s);
    if (launch_boundary(ba, s) != hipSuccess) return BEAM_ERR_HIP;
  }
  return forward_impl(h, h->ws, T, z_out, y_out, nullptr, nullptr, logits_out, ids_out, w_out,
                      nullptr, nullptr, s, nullptr, nullptr);
}

int beam_profile_enable(int enable) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.enabled = enable != 0;
  return BEAM_OK;
}

int beam_profile_reset(void) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  for (auto& r : p.records) {
    (void)hipEventSynchronize(r.stop);
    p.pool.push_back(r.start);
    p.pool.push_back(r.stop);
  }
  p.records.clear();
  return BEAM_OK;
}

int beam_profile_read(int32_t kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= K_COUNT || !total_ms || !launches) return BEAM_ERR_INVALID_ARG;
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  double sum = 0.0;
  int64_t n = 0;
  for (auto& r : p.records) {
    if (r.id != kernel) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return BEAM_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return BEAM_ERR_HIP;
    sum += ms;
    ++n;
  }
  *total_ms = sum;
  *launches = n;
  return BEAM_OK;
}

int32_t beam_kernel_count(void) { return K_COUNT; }

const char* beam_kernel_name(int32_t kernel) {
  return (kernel >= 0 && kernel < K_COUNT) ? kKernelNames[kernel] : nullptr;
}

}  // extern "C"
