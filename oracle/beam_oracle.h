/*
 * CPU oracle for one Beam sparse-decoder sublayer boundary plus its routed MoE
 * FFN. TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
 * CPU-baseline leg are the only callers. The product path never links or calls it.
 *
 * Plain, slow, single-threaded C: loops run in ascending index order, FP32
 * accumulations are sequential, BF16 rounding is round-to-nearest-even by bit
 * manipulation. Built with -ffp-contract=off so every product and sum rounds
 * separately as written.
 *
 * Sources (cited by page title and section):
 *   [vLLM]   "Serving Reflection Beam auf vLLM ab Tag 0"
 *   [SGLang] "SGLang 支撑编程模型 Beam 生产部署" (SGLang powers Beam in production)
 *
 * BF16 values travel as uint16_t bit patterns. All arrays are row-major and
 * owned by the caller. Functions return 0 on success, negative on bad input.
 */
#ifndef BEAM_ORACLE_H
#define BEAM_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* float -> BF16, round to nearest even (quiet NaN kept) */
uint16_t oracle_bf16(float v);
/* BF16 -> float (exact) */
float oracle_f32(uint16_t b);
/* sigmoid in double, rounded once to FP32 */
float oracle_sigmoid(float logit);
/* SiLU in FP32: v / (1 + expf(-v)) */
float oracle_silu(float v);

/* O1: post-RMSNorm -> depth-scaled residual -> next pre-RMSNorm, per token row.
 * h, x: [T, d] BF16 (x = the sublayer's raw output). w_post, w_pre: [d] BF16.
 * n >= 1: the 1-based index of this residual add. h_out, z_out: [T, d] BF16. */
int oracle_boundary(int64_t T, int64_t d, const uint16_t* h, const uint16_t* x,
                    const uint16_t* w_post, const uint16_t* w_pre, int64_t n, float eps,
                    uint16_t* h_out, uint16_t* z_out);

/* O2: FP32 router. z: [T, d] BF16; W: [E, d] FP32; logits: [T, E] FP32. */
int oracle_router(int64_t T, int64_t d, int64_t E, const uint16_t* z, const float* W,
                  float* logits);

/* O3: sigmoid scores + correction bias, grouped top-k, renormalise x scale.
 * logits: [T, E]; bias: [E]. ids: [T, k] int32 (slot order = selection rank);
 * w: [T, k] FP32. ggap, egap: [T] near-tie gaps (may be NULL). */
int oracle_topk(int64_t T, int64_t E, int64_t G, int64_t kg, int64_t k, float scale,
                const float* logits, const float* bias, int32_t* ids, float* w, float* ggap,
                float* egap);

/* O4: expert histogram + stable permutation. ids: [T, k]; counts: [E];
 * offsets: [E+1]; perm: [T*k] (row r holds t*k+j); inv: [T*k] (slot -> row).
 * Slots whose id is outside [0, E) are skipped (inv = -1) and leave the tail of
 * perm at -1. */
int oracle_permute(int64_t T, int64_t k, int64_t E, const int32_t* ids, int32_t* counts,
                   int32_t* offsets, int32_t* perm, int32_t* inv);

/* O5: one expert's weighted SwiGLU rows.
 * zrows: [R, d] BF16; Wg, Wu: [f, d] BF16; Wd: [d, f] BF16; wrow: [R] FP32.
 * yk: [R, d] BF16 = bf16(wrow[r] * (act_r . Wd^T)). */
int oracle_expert_rows(int64_t R, int64_t d, int64_t f, const uint16_t* zrows,
                       const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd,
                       const float* wrow, uint16_t* yk);

/* O6: combine. yk: [T, k, d] BF16 (slot order); ids: [T, k] (slots with an id
 * outside [0, E) are skipped; ids may be NULL = all valid); y: [T, d] BF16. */
int oracle_combine(int64_t T, int64_t k, int64_t d, int64_t E, const int32_t* ids,
                   const uint16_t* yk, uint16_t* y);

/* O7: MXFP4 (OCP MX v1.0: E2M1 elements, one E8M0 scale per 32 values along K).
 * v: [rows, K] BF16, K % 32 == 0. codes: [rows, K/2] (element 2i in the low
 * nibble of byte i); scales: [rows, K/32] (X + 127). Non-finite input: -1. */
int oracle_mxfp4_quantize(int64_t rows, int64_t K, const uint16_t* v, uint8_t* codes,
                          uint8_t* scales);
/* Exact inverse image: out [rows, K] BF16 = sign * E2M1 value * 2^(scale - 127). */
int oracle_mxfp4_dequantize(int64_t rows, int64_t K, const uint8_t* codes, const uint8_t* scales,
                            uint16_t* out);

/* O8: O5 with 4-bit activations: each token row z and each activation row act is
 * MXFP4-quantised (O7, blocks of 32 along its K) and used at its dequantised value.
 * Arguments as in O5 (the weights are the experts' dequantised 4-bit weights). */
int oracle_expert_rows_mx(int64_t R, int64_t d, int64_t f, const uint16_t* zrows,
                          const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd,
                          const float* wrow, uint16_t* yk);

/* O5's halves: act [R, f] BF16 from z rows (gate/up, SiLU * up), and yk [R, d] from act
 * rows (down, routing weight, one rounding). down(act(z)) is O5. */
int oracle_expert_act(int64_t R, int64_t d, int64_t f, const uint16_t* zrows, const uint16_t* Wg,
                      const uint16_t* Wu, uint16_t* act);
int oracle_expert_down(int64_t R, int64_t d, int64_t f, const uint16_t* act, const uint16_t* Wd,
                       const float* wrow, uint16_t* yk);

#ifdef __cplusplus
}
#endif
#endif
