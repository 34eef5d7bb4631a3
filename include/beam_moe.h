/*
 * beam_moe.h — C ABI of the Beam sparse-decoder MoE sublayer for MI355X (gfx950).
 *
 * One library, libbeam_moe.so, built from hand-written HIP kernels. It computes
 * one sublayer boundary (post-RMSNorm -> depth-scaled residual -> next
 * pre-RMSNorm) and the routed MoE FFN that follows it (FP32 router, sigmoid
 * scores + correction bias, grouped top-k, BF16 SwiGLU experts, FP32 weighted
 * combine), on one GPU.
 *
 * Sources, cited by page title and section:
 *   [vLLM]   "Serving Reflection Beam auf vLLM ab Tag 0"
 *   [SGLang] "SGLang 支撑编程模型 Beam 生产部署" (SGLang powers Beam in production)
 *
 * Conventions shared by every entry point:
 *   - BF16 tensors are passed as uint16_t* holding bit patterns; FP32 as float*.
 *   - Every array argument is DEVICE memory owned by the caller, row-major and
 *     contiguous, 16-byte aligned. The library never frees caller memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Compute calls only enqueue work on it and return; BEAM_OK means
 *     "validated and enqueued". Device-side faults surface at the caller's next
 *     synchronisation. beam_moe_init and beam_moe_destroy synchronise.
 *   - All arguments are validated on the host before any HIP call; a call that
 *     returns an error has enqueued nothing and written nothing.
 *   - Non-finite inputs give unspecified (but in-bounds) results.
 *   - Compute calls allocate nothing, so they can be captured in a HIP graph.
 *   - A handle must not be used by two streams at the same time (its
 *     workspace is shared by its calls). A dense-layer handle (beam_dense_init)
 *     serves beam_dense_forward only; the MoE compute calls reject it.
 *   - No exception or signal crosses the ABI.
 */
#ifndef BEAM_MOE_H
#define BEAM_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum {
  BEAM_OK = 0,
  BEAM_ERR_INVALID_ARG = -1, /* null/misaligned pointer, negative size, bad scalar */
  BEAM_ERR_UNSUPPORTED = -2, /* a shape the library does not implement */
  BEAM_ERR_OOM = -3,         /* device allocation failed (init only) */
  BEAM_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  BEAM_ERR_CAPACITY = -5     /* T larger than the handle's max_tokens */
};

/* Layer shape, fixed at init.
 * [vLLM §MoE und Residual-Stream]: Beam uses hidden 5120, 256 routed experts
 * in 8 groups, best 4 groups then top 8 experts, d_ff 2560, scale 2.5.
 * Supported here: hidden % 256 == 0 and hidden <= 16384; d_ff % 256 == 0 and
 * d_ff <= 32768; n_experts <= 256 and a multiple of n_groups; n_groups <= 64;
 * 1 <= topk_groups <= n_groups; 1 <= topk <= min(32, topk_groups * E/G);
 * 1 <= max_tokens and max_tokens * topk < 2^31; routed_scale finite. Activations are
 * addressed with 32-bit element offsets, so max_tokens * topk * max(hidden, d_ff) < 2^31
 * (about 52K tokens at Beam's shape), else BEAM_ERR_UNSUPPORTED. */
typedef struct {
  int32_t hidden;      /* d */
  int32_t n_experts;   /* E */
  int32_t n_groups;    /* G */
  int32_t topk_groups; /* kg: groups kept per token */
  int32_t topk;        /* k: experts per token */
  int32_t d_ff;        /* f: expert intermediate size */
  int32_t max_tokens;  /* largest T any compute call on this handle may use */
  float routed_scale;  /* multiplies the renormalised routing weights */
} beam_moe_config;

typedef struct beam_moe_ctx* beam_moe_handle;

/*
 * beam_moe_init — create a handle for one MoE layer.
 * Inputs (device memory, read during the call only):
 *   router_w    [E, d] FP32   router weight, row e = expert e's logit weights
 *   router_bias [E]    FP32   per-expert correction bias (selection only)
 *   w_gate, w_up [E, f, d] BF16   expert gate / up projections (row q = output q)
 *   w_down      [E, d, f] BF16    expert down projections (row o = output o)
 * The weights are copied and repacked into handle-owned device memory laid out
 * for the kernels (about the same size again), and all workspace for
 * max_tokens is allocated here. The caller may free its copies after return.
 * [vLLM §MoE und Residual-Stream]: router weights, accumulation and logits
 * are FP32. Returns BEAM_ERR_UNSUPPORTED for shapes outside the list above,
 * BEAM_ERR_OOM if device memory runs out. *out is set only on BEAM_OK.
 */
int beam_moe_init(const beam_moe_config* cfg, const float* router_w, const float* router_bias,
                  const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                  void* stream, beam_moe_handle* out);

/*
 * beam_mxfp4_quantize — 4-bit block quantisation of BF16 rows (MXFP4).
 * [vLLM §Modellarchitektur]: the routed experts are served with 4-bit floating-point
 * weights; [SGLang §BF16、NVFP4 和 FP8 模型支持]: 4-bit expert checkpoints. The format here
 * is MXFP4 of the OCP Microscaling Formats specification v1.0, which gfx950 converts
 * natively: E2M1 codes (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 = sign) sharing one
 * E8M0 scale 2^(s-127) per 32 consecutive values of a row. Per block:
 *   X = floor(log2 max|v|) - 2, clamped to [-127, 127] (-127 for an all-zero block);
 *   code = v / 2^X rounded to the nearest E2M1 value, ties to the even code, |.| > 6
 *          saturating to 6, sign kept (also when the magnitude rounds to zero).
 * Arguments: src [rows, K] BF16, K % 32 == 0 (16-byte aligned). Outputs codes_out
 * [rows, K/2] (element 2i in the low nibble of byte i; 16-byte aligned) and scales_out
 * [rows, K/32] (the byte X + 127). Stateless; rows == 0 is a no-op. Non-finite inputs
 * give unspecified codes.
 */
int beam_mxfp4_quantize(int64_t rows, int32_t K, const uint16_t* src, uint8_t* codes_out,
                        uint8_t* scales_out, void* stream);

/*
 * beam_moe_init_mxfp4 — a handle like beam_moe_init's whose experts hold MXFP4
 * weights (the layout beam_mxfp4_quantize writes):
 *   gate_codes, up_codes [E, f, d/2] and gate_scales, up_scales [E, f, d/32];
 *   down_codes [E, d, f/2] and down_scales [E, d, f/32].
 * The codes are dequantised exactly (every E2M1 value times a power of two is a BF16
 * number) inside the expert kernels, with BF16 activations, so the forward computes
 * what a beam_moe_init handle computes on the dequantised weights, bit for bit, while
 * reading about 0.53 bytes per weight instead of 2 (the decode path is bound by the
 * weight stream). Every compute entry point takes either kind of handle.
 * Supported: the beam_moe_init shapes with hidden % 512 == 0 and d_ff % 512 == 0;
 * others give BEAM_ERR_UNSUPPORTED. Code arrays must be 4-byte aligned. The weights are
 * copied and repacked into handle-owned memory (one layout for the weight-streaming
 * passes of T <= 128, and, when max_tokens > 128, a second one for the grouped GEMMs:
 * about 0.53 and 1.06 bytes per weight); the caller may free its copies after return.
 */
int beam_moe_init_mxfp4(const beam_moe_config* cfg, const float* router_w,
                        const float* router_bias, const uint8_t* gate_codes,
                        const uint8_t* gate_scales, const uint8_t* up_codes,
                        const uint8_t* up_scales, const uint8_t* down_codes,
                        const uint8_t* down_scales, void* stream, beam_moe_handle* out);

/* Activation formats of the expert GEMMs (beam_moe_set_activation_format). */
enum { BEAM_ACT_BF16 = 0, BEAM_ACT_MXFP4 = 1 };

/*
 * beam_moe_set_activation_format — choose what the expert GEMMs of a handle multiply its
 * weights with. BEAM_ACT_BF16 (the default): BF16 activations. BEAM_ACT_MXFP4 (handles from
 * beam_moe_init_mxfp4 only): 4-bit activations as well as 4-bit weights (W4A4), the pages'
 * 4-bit MoE path ([vLLM §Der fusionierte Graph]: an activation quantisation ahead of the
 * two grouped GEMMs on the 4-bit experts). Every MoE compute call then quantises each
 * token row z to MXFP4 (blocks of 32 along d, the rule of beam_mxfp4_quantize) and the
 * activation act = bf16(silu(g) * u) to MXFP4 (blocks of 32 along f), and the grouped GEMMs
 * multiply the 4-bit operands on the scaled FP4 matrix cores (each 32-value block's
 * products are exact; FP32 accumulation); g, u, the routing weight, the BF16 rounding of
 * each expert row and the combine are as in beam_moe_forward. The format applies to every
 * T; for T <= 128 the same values are multiplied on the 4-bit weight-streaming passes (the
 * round trips of z and act, which are BF16 numbers, times the exactly dequantised weights),
 * since there the weight stream, not the arithmetic, bounds the step. Takes effect for calls
 * made after it returns; allocates and enqueues nothing.
 * Returns BEAM_ERR_UNSUPPORTED for BEAM_ACT_MXFP4 on a BF16-weight handle and
 * BEAM_ERR_INVALID_ARG for a dense handle or another format.
 */
int beam_moe_set_activation_format(beam_moe_handle h, int32_t format);

/* Intermediate buffers of the last compute call (beam_moe_inspect). */
enum {
  BEAM_INSPECT_ACT = 0,        /* BF16 activations [T*k, f], rows in the expert-grouped order */
  BEAM_INSPECT_ACT_CODES = 1,  /* 4-bit activations: codes [T*k, f/2] (see below) */
  BEAM_INSPECT_ACT_SCALES = 2, /* 4-bit activations: E8M0 scales [T*k, f/32] */
  BEAM_INSPECT_Z_CODES = 3,    /* 4-bit activations: token-row codes [T, d/2] */
  BEAM_INSPECT_Z_SCALES = 4    /* 4-bit activations: token-row scales [T, d/32] */
};

/*
 * beam_moe_inspect — the device address of one of a handle's intermediate buffers, for
 * tests and tools that check the expert stages separately. The contents are those of the
 * last compute call on the handle (rows 0 .. T*k-1 or T-1 of it) once that call has
 * completed on its stream. 4-bit codes are stored per 32-value block as 16 bytes whose
 * dword p holds block elements 8 q .. 8 q + 7, q = (0, 2, 1, 3)[p] (element 2i of a dword's
 * eight in its low nibble). BEAM_INSPECT_ACT holds BF16 activations only after BF16-
 * activation calls. Returns BEAM_ERR_UNSUPPORTED when the handle has no such buffer (4-bit
 * codes of an activation-BF16 handle), BEAM_ERR_INVALID_ARG for an unknown `what`. The
 * buffer is owned by the handle; the caller only reads it.
 */
int beam_moe_inspect(beam_moe_handle h, int32_t what, const void** ptr);

/*
 * beam_dense_init — a handle for one dense SwiGLU MLP layer.
 * [vLLM §Modellarchitektur]: Beam's layers 0-2 use a dense SwiGLU MLP (d_ff 20480)
 * instead of the routed experts. Computed per token row with the experts' rounding
 * points (FP32 accumulation; gate, up and the activation rounded to BF16):
 *   g = bf16(z . Wg^T), u = bf16(z . Wu^T), act = bf16(silu(g) * u), y = bf16(act . Wd^T)
 * Arguments: hidden (d), d_ff (f) and max_tokens as in beam_moe_config (the same
 * shape limits); w_gate, w_up [f, d] BF16 and w_down [d, f] BF16 (device memory,
 * read during the call only; copied and repacked into the handle). The handle runs
 * the expert kernels as one expert that every token takes with weight 1 (exactly the
 * dense result), and serves only beam_dense_forward; the MoE entry points reject it
 * with BEAM_ERR_INVALID_ARG. Synchronises; *out is set only on BEAM_OK.
 */
int beam_dense_init(int32_t hidden, int32_t d_ff, int32_t max_tokens, const uint16_t* w_gate,
                    const uint16_t* w_up, const uint16_t* w_down, void* stream,
                    beam_moe_handle* out);

/*
 * beam_dense_forward — y [T, d] BF16 = the dense SwiGLU layer of beam_dense_init on
 * z [T, d] BF16 (T <= max_tokens, else BEAM_ERR_CAPACITY; T == 0 is a no-op). y_out
 * must not overlap z. A handle from beam_moe_init gives BEAM_ERR_INVALID_ARG.
 */
int beam_dense_forward(beam_moe_handle h, int32_t T, const uint16_t* z, uint16_t* y_out,
                       void* stream);

/* beam_moe_destroy — synchronise and free everything the handle owns. NULL is a no-op. */
int beam_moe_destroy(beam_moe_handle h);

/*
 * beam_sublayer_norm_residual — the fused sublayer boundary, per token row:
 *   xn = bf16(RMSNorm(x) * w_post)                 post-norm of the branch x
 *   h' = bf16(bf16(c1 * h) + bf16(c2 * xn))         depth-scaled residual,
 *        c1 = sqrt((n-1)/n), c2 = 1/sqrt(n)         both operands rounded first
 *   z  = bf16(RMSNorm(h') * w_pre)                  next sublayer's pre-norm
 * with RMSNorm(v) = v / sqrt(mean(v^2) + eps), FP32 math throughout.
 * [vLLM §MoE und Residual-Stream] sandwich norm and the depth-scaled residual;
 * [vLLM §Agentengetriebene Optimierung, change 1] one fused kernel, FP32 math,
 * BF16 rounding points; [SGLang §三明治归一化与深度缩放残差] both scaled operands
 * are rounded to BF16 before the add.
 * Arguments: h_in, x [T, d] BF16; w_post, w_pre [d] BF16; n >= 1 is the 1-based
 * index of this residual add; eps >= 0. Outputs h_out, z_out [T, d] BF16.
 * h_out may equal h_in (in place); no other overlap is allowed.
 * Needs d % 8 == 0 and d <= 65536. T == 0 is a no-op.
 */
int beam_sublayer_norm_residual(int32_t T, int32_t d, const uint16_t* h_in, const uint16_t* x,
                                const uint16_t* w_post, const uint16_t* w_pre, int32_t n,
                                float eps, uint16_t* h_out, uint16_t* z_out, void* stream);

/*
 * beam_router_topk — FP32 router logits and grouped top-k for T tokens.
 *   logits[t, e] = sum_i z[t, i] * W[e, i]          FP32
 *   s = sigmoid(logits), c = s + bias
 *   group score = sum of the two largest c in the group (one if E/G == 1)
 *   keep the topk_groups best groups, then the topk best experts in them by c
 *   (every order: value descending, then index ascending)
 *   w[t, j] = s[ids[t, j]] / sum_j s[ids[t, j]] * routed_scale   (sum in slot order)
 * [vLLM §MoE und Residual-Stream]: DeepSeek-V3-style routing, sigmoid scores
 * plus correction bias, 4 of 8 groups, top 8, renormalised x 2.5, FP32 router.
 * [SGLang §稠密层与分组 MoE 路由]: FP32 logits and routing coefficients.
 * Arguments: z [T, d] BF16 (the MoE input). Outputs: logits_out [T, E] FP32 or
 * NULL; ids_out [T, k] int32 in selection order; w_out [T, k] FP32.
 * T <= max_tokens.
 */
int beam_router_topk(beam_moe_handle h, int32_t T, const uint16_t* z, float* logits_out,
                     int32_t* ids_out, float* w_out, void* stream);

/*
 * beam_grouped_topk — the routing step of beam_router_topk on caller-supplied
 * FP32 logits [T, E] (same rules, same handle bias and scale). Outputs ids_out
 * [T, k] and w_out [T, k]. For callers with their own router, and for
 * checking the selection on fixed logits.
 */
int beam_grouped_topk(beam_moe_handle h, int32_t T, const float* logits, int32_t* ids_out,
                      float* w_out, void* stream);

/*
 * beam_moe_forward — the routed MoE FFN for T tokens of z [T, d] BF16:
 *   route (unless replayed), group the T*k assignments by expert (stable:
 *   expert ascending, then slot t*k+j ascending), run each expert's SwiGLU on
 *   its rows, and combine:
 *     g = bf16(z . Wg[e]^T), u = bf16(z . Wu[e]^T)  FP32 accumulation
 *     act = bf16(silu(g) * u)
 *     y_j = bf16(w[t, j] * (act . Wd[e]^T))         weight applied before rounding
 *     y[t] = bf16(y_0 + y_1 + ... + y_{k-1})         FP32 sum in slot order
 * [SGLang §BF16 MoE 内核优化]: BF16 boundaries at gate/up and the activation;
 * the FP32 routing weight is applied before the down output is rounded.
 * [vLLM §Agentengetriebene Optimierung, change 3] and [SGLang, kernel-fusion
 * paragraph]: the top-k outputs are summed, scaled and rounded once.
 * Routing replay: if ids_in != NULL, ids_in [T, k] and w_in [T, k] (FP32) are
 * used instead of routing ([SGLang §在 Miles 中进行强化学习] records and
 * replays the selected experts); a slot whose id is outside [0, E) contributes
 * nothing. Otherwise w_in must be NULL.
 * Optional outputs (NULL to skip): logits_out [T, E] FP32 (computed routing
 * only); ids_out [T, k]; w_out [T, k]; perm_out [T*k] int32 (row r of the
 * expert-grouped order holds slot t*k+j; rows past the valid count are -1);
 * offsets_out [E+1] int32 (exclusive prefix of per-expert row counts).
 * Output y_out [T, d] BF16 must not overlap z.
 */
int beam_moe_forward(beam_moe_handle h, int32_t T, const uint16_t* z, uint16_t* y_out,
                     const int32_t* ids_in, const float* w_in, float* logits_out,
                     int32_t* ids_out, float* w_out, int32_t* perm_out, int32_t* offsets_out,
                     void* stream);

/*
 * beam_moe_forward_noalloc — beam_moe_forward for callers that cannot allocate device
 * memory at all (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation), including the handle's per-call workspace: the logits, routing, grouping
 * tables, activations and expert rows of the call live in a static scratch area of the
 * library (32 MiB per GPU, held by every GPU the library runs on until the process ends)
 * instead of the handle's workspace. Same arguments, results (bit for bit) and errors as
 * beam_moe_forward; additionally BEAM_ERR_CAPACITY when the call's workspace does not fit
 * the scratch area: T * k * 2 * (d_ff + hidden) bytes plus T * E * 4 and small tables,
 * i.e. up to 256 tokens at Beam's shape (hidden 5120, d_ff 2560, k 8, E 256), and
 * BEAM_ERR_HIP if the area's device address could not be looked up when the handle was
 * created. Allocates nothing and synchronises nothing. Every such call on one GPU uses the
 * same area, which keeps the last call's contents: calls that overlap in time on one GPU
 * (two streams, or two host threads) race and must not be issued.
 */
int beam_moe_forward_noalloc(beam_moe_handle h, int32_t T, const uint16_t* z, uint16_t* y_out,
                             const int32_t* ids_in, const float* w_in, float* logits_out,
                             int32_t* ids_out, float* w_out, int32_t* perm_out,
                             int32_t* offsets_out, void* stream);

/*
 * beam_moe_forward_boundary — beam_moe_forward on z, then the NEXT sublayer's
 * boundary with the MoE output as its branch: the result is bit-identical to
 *   beam_moe_forward(h, T, z, y, ids_in, w_in, logits_out, ids_out, w_out, ...)
 *   beam_sublayer_norm_residual(T, d, h_in, y, w_post, w_pre, n, eps, h_out, z_out)
 * but the combine of the top-k expert rows and the boundary run as one kernel, so
 * y does not pass through HBM ([vLLM §Agentengetriebene Optimierung, changes 1 and
 * 3]: after the MoE, the post-norm kernel of the boundary also combines the top-8
 * expert outputs).
 * Arguments: z [T, d] BF16 (the MoE input); h_in [T, d] the residual stream; w_post,
 * w_pre [d]; n >= 1; eps >= 0; outputs h_out, z_out [T, d] (the next sublayer's
 * residual and input). y_out [T, d] or NULL (required when d > 8192). Routing replay
 * (ids_in, w_in) and the optional routing outputs as in beam_moe_forward.
 * Aliasing: h_out may be h_in; z_out may be z (the experts have read z before the
 * boundary writes); nothing else may overlap.
 */
int beam_moe_forward_boundary(beam_moe_handle h, int32_t T, const uint16_t* z,
                              const uint16_t* h_in, const uint16_t* w_post, const uint16_t* w_pre,
                              int32_t n, float eps, uint16_t* h_out, uint16_t* z_out,
                              uint16_t* y_out, const int32_t* ids_in, const float* w_in,
                              float* logits_out, int32_t* ids_out, float* w_out, void* stream);

/*
 * beam_moe_forward_boundary_route — beam_moe_forward_boundary for a loop over MoE layers
 * (decode): the MoE of handle h on z, then the weighted combine, the NEXT sublayer's
 * boundary (h_out, z_out) and the NEXT layer's routing of z_out with handle `next` (router,
 * grouped top-k and grouping into next's workspace; with 4-bit activations also the rows'
 * quantisation), for one token (T = 1, hidden <= 8192, topk <= 8) all in ONE launch —
 * the pages' fused graph ([vLLM §Der fusionierte Graph; §Agentengetriebene Optimierung,
 * changes 1 and 3]: the post-MoE norm combines the top-8 outputs, and the boundary feeds the
 * router) carried one step further. Other T run the same steps as separate launches.
 * The call on the next layer passes routed = 1 to use that routing: it must name the same T
 * and, as z, the z_out of this call (the handle records both; a mismatch returns
 * BEAM_ERR_INVALID_ARG, as does routed = 1 on a handle with no such routing). Any other
 * compute call on `next`, or beam_moe_set_activation_format, drops the recorded routing.
 * With routed = 0 the call routes z itself. next may be h.
 * Arguments and aliasing as beam_moe_forward_boundary (no routing replay or routing
 * outputs); next must have the same hidden size; T <= both handles' max_tokens, else
 * BEAM_ERR_CAPACITY. Results equal, bit for bit,
 *   beam_moe_forward_boundary(h, T, z, h_in, w_post, w_pre, n, eps, h_out, z_out, y_out, ...)
 *   followed by the routing of z_out that beam_moe_forward(next, T, z_out, ...) computes.
 */
int beam_moe_forward_boundary_route(beam_moe_handle h, beam_moe_handle next, int32_t T,
                                    const uint16_t* z, const uint16_t* h_in,
                                    const uint16_t* w_post, const uint16_t* w_pre, int32_t n,
                                    float eps, uint16_t* h_out, uint16_t* z_out, uint16_t* y_out,
                                    int32_t routed, void* stream);

/*
 * beam_sublayer_forward — one sublayer step: the boundary of beam_sublayer_norm_residual
 * on (h_in, x) writing h_out and z_out, then beam_moe_forward on z_out with computed
 * routing writing y_out. The results are bit-identical to those two calls in sequence.
 * For one token (d <= 8192, k <= 64) the boundary runs inside the routing launch —
 * every routing workgroup forms z itself while its router weights load, which saves
 * the boundary's launch — as [vLLM §Agentengetriebene Optimierung, change 1] fuses the
 * boundary into its neighbours and [vLLM §Der fusionierte Graph] runs the routing
 * kernels right after it.
 * Arguments as in those calls: h_in, x [T, d] BF16; w_post, w_pre [d] BF16; n >= 1;
 * eps >= 0. h_out may be h_in itself; z_out and y_out must not overlap each other or
 * any input. Optional outputs (NULL to skip): logits_out [T, E] FP32, ids_out [T, k],
 * w_out [T, k]. T <= max_tokens.
 */
int beam_sublayer_forward(beam_moe_handle h, int32_t T, const uint16_t* h_in, const uint16_t* x,
                          const uint16_t* w_post, const uint16_t* w_pre, int32_t n, float eps,
                          uint16_t* h_out, uint16_t* z_out, uint16_t* y_out, float* logits_out,
                          int32_t* ids_out, float* w_out, void* stream);

/* beam_status_string — a static description of a status code. */
const char* beam_status_string(int status);

/*
 * Kernel timing, for measurement tools. While enabled, every kernel the
 * library launches is bracketed by two HIP events on its stream.
 * beam_profile_read synchronises the recorded events and returns, for kernel
 * id `kernel` (0 <= kernel < beam_kernel_count()), the summed duration in
 * milliseconds and the number of launches since the last reset. Not for use
 * during graph capture. beam_kernel_name returns a static name or NULL.
 */
int beam_profile_enable(int enable);
int beam_profile_reset(void);
int beam_profile_read(int32_t kernel, double* total_ms, int64_t* launches);
int32_t beam_kernel_count(void);
const char* beam_kernel_name(int32_t kernel);

#ifdef __cplusplus
}
#endif

#endif /* BEAM_MOE_H */
