/*
 * CPU oracle for the Beam MoE sublayer. TEST INFRASTRUCTURE ONLY (see
 * beam_oracle.h): plain, slow, single-threaded, obviously correct. Shares no
 * code with the GPU library.
 *
 * Readings of points the pages leave open are marked "reading:" and are the
 * same ones the GPU path implements.
 */
#include "beam_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

uint16_t oracle_bf16(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) /* inf or nan */
    return (uint16_t)((u >> 16) | ((u & 0x007FFFFFu) ? 0x0040u : 0u));
  /* round to nearest, ties to even, on the 16 bits that are dropped */
  uint32_t lsb = (u >> 16) & 1u;
  u = u + 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

float oracle_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float v;
  memcpy(&v, &u, 4);
  return v;
}

/* [vLLM §MoE und Residual-Stream; SGLang §稠密层与分组 MoE 路由 (grouped MoE routing)]
 * Scores are sigmoid(logit). Reading: evaluated in double and rounded once to
 * FP32, which is the correctly rounded FP32 sigmoid for all practical inputs. */
float oracle_sigmoid(float logit) {
  return (float)(1.0 / (1.0 + exp(-(double)logit)));
}

/* SwiGLU's activation: silu(v) = v * sigmoid(v), written v / (1 + e^-v), FP32. */
float oracle_silu(float v) {
  return v / (1.0f + expf(-v));
}

/*
 * O1 — the sublayer boundary.
 * [vLLM §MoE und Residual-Stream]: sandwich norm (an RMSNorm before and after
 *   every sublayer) and the depth-scaled residual: the n-th residual add is
 *   h <- sqrt((n-1)/n) * h + x / sqrt(n).
 * [vLLM §Agentengetriebene Optimierung, change 1]: post-norm, scaled residual
 *   add and next pre-norm fused, FP32 math, the reference's BF16 rounding points.
 * [SGLang §三明治归一化与深度缩放残差 (sandwich norm and depth-scaled residual)]:
 *   both scaled operands are rounded to the activation dtype before the add;
 *   the unfused path writes the normalised branch and reads it back for the
 *   residual, so the post-norm output is itself a BF16 tensor.
 * Readings: textbook RMSNorm y = x * 1/sqrt(mean(x^2) + eps) * w with eps
 *   inside the root and one BF16 rounding of (x*r)*w; the coefficients are
 *   computed in double and rounded once to FP32; x/sqrt(n) is a multiply by
 *   the FP32 coefficient 1/sqrt(n).
 */
static void rmsnorm_row(int64_t d, const uint16_t* v, const uint16_t* w, float eps,
                        uint16_t* out) {
  float ss = 0.0f;
  for (int64_t i = 0; i < d; ++i) {
    float a = oracle_f32(v[i]);
    ss = ss + a * a;
  }
  float r = 1.0f / sqrtf(ss / (float)d + eps);
  for (int64_t i = 0; i < d; ++i)
    out[i] = oracle_bf16((oracle_f32(v[i]) * r) * oracle_f32(w[i]));
}

int oracle_boundary(int64_t T, int64_t d, const uint16_t* h, const uint16_t* x,
                    const uint16_t* w_post, const uint16_t* w_pre, int64_t n, float eps,
                    uint16_t* h_out, uint16_t* z_out) {
  if (T < 0 || d <= 0 || n < 1 || !(eps >= 0.0f)) return -1;
  const float c1 = (float)sqrt((double)(n - 1) / (double)n); /* scales the residual h */
  const float c2 = (float)(1.0 / sqrt((double)n));           /* scales the branch */
  uint16_t* xn = (uint16_t*)malloc((size_t)d * sizeof(uint16_t));
  if (!xn) return -3;
  for (int64_t t = 0; t < T; ++t) {
    const uint16_t* hr = h + t * d;
    const uint16_t* xr = x + t * d;
    uint16_t* ho = h_out + t * d;
    uint16_t* zo = z_out + t * d;
    rmsnorm_row(d, xr, w_post, eps, xn); /* post-norm of the branch, rounded */
    for (int64_t i = 0; i < d; ++i) {
      uint16_t a = oracle_bf16(c1 * oracle_f32(hr[i])); /* scaled residual, rounded */
      uint16_t b = oracle_bf16(c2 * oracle_f32(xn[i])); /* scaled branch, rounded */
      ho[i] = oracle_bf16(oracle_f32(a) + oracle_f32(b));
    }
    rmsnorm_row(d, ho, w_pre, eps, zo); /* next sublayer's pre-norm */
  }
  free(xn);
  return 0;
}

/*
 * O2 — the FP32 router.
 * [vLLM §MoE und Residual-Stream]: router weights (5120 x 256), accumulation
 *   and logits are all FP32.
 * Readings: the router reads the MoE sublayer's pre-normed input z; W is
 *   stored [E, d] (output features by input features).
 */
int oracle_router(int64_t T, int64_t d, int64_t E, const uint16_t* z, const float* W,
                  float* logits) {
  if (T < 0 || d <= 0 || E <= 0) return -1;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int64_t i = 0; i < d; ++i) acc = acc + oracle_f32(z[t * d + i]) * W[e * d + i];
      logits[t * E + e] = acc;
    }
  return 0;
}

/*
 * O3 — grouped top-k.
 * [vLLM §MoE und Residual-Stream]: routed as in DeepSeek-V3: sigmoid scores
 *   plus a correction bias pick the best 4 of 8 expert groups, then the top 8
 *   experts; the renormalised weights are scaled by 2.5; no shared expert.
 * [SGLang §稠密层与分组 MoE 路由]: FP32 logits; grouped top-k over sigmoid
 *   scores and the expert correction bias; FP32 routing coefficients; the
 *   routing scale may be folded into the routing weights.
 * Readings: a group's score is the sum of its two largest biased scores
 *   (DeepSeek-V3's rule; one expert per group -> that expert's score); the bias
 *   enters selection only, the weights use the unbiased scores; every order is
 *   (value descending, index ascending), so the selection is unique; the k
 *   outputs are in that order; the denominator is summed in slot order; the
 *   scale is applied to each weight.
 */
static int better(float va, int64_t ia, float vb, int64_t ib) {
  return va > vb || (va == vb && ia < ib);
}

/* insertion sort of idx[0..m) by (val desc, idx asc) */
static void sort_desc(int64_t m, int64_t* idx, const float* val) {
  for (int64_t a = 1; a < m; ++a) {
    int64_t cur = idx[a];
    int64_t b = a - 1;
    while (b >= 0 && better(val[cur], cur, val[idx[b]], idx[b])) {
      idx[b + 1] = idx[b];
      --b;
    }
    idx[b + 1] = cur;
  }
}

int oracle_topk(int64_t T, int64_t E, int64_t G, int64_t kg, int64_t k, float scale,
                const float* logits, const float* bias, int32_t* ids, float* w, float* ggap,
                float* egap) {
  if (T < 0 || E <= 0 || G <= 0 || E % G != 0 || kg < 1 || kg > G || k < 1) return -1;
  const int64_t gs = E / G;
  if (k > kg * gs) return -1;
  float* s = (float*)malloc((size_t)E * sizeof(float));
  float* c = (float*)malloc((size_t)E * sizeof(float));
  float* g = (float*)malloc((size_t)G * sizeof(float));
  int64_t* gi = (int64_t*)malloc((size_t)G * sizeof(int64_t));
  int64_t* cand = (int64_t*)malloc((size_t)E * sizeof(int64_t));
  if (!s || !c || !g || !gi || !cand) {
    free(s); free(c); free(g); free(gi); free(cand);
    return -3;
  }
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    for (int64_t e = 0; e < E; ++e) {
      s[e] = oracle_sigmoid(l[e]);
      c[e] = s[e] + bias[e];
    }
    /* group scores: sum of the two largest biased scores in the group */
    for (int64_t j = 0; j < G; ++j) {
      float m1 = -INFINITY, m2 = -INFINITY;
      for (int64_t q = 0; q < gs; ++q) {
        float v = c[j * gs + q];
        if (v > m1) {
          m2 = m1;
          m1 = v;
        } else if (v > m2) {
          m2 = v;
        }
      }
      g[j] = (gs >= 2) ? m1 + m2 : m1;
      gi[j] = j;
    }
    sort_desc(G, gi, g);
    /* candidates: every expert of the kept groups */
    int64_t m = 0;
    for (int64_t a = 0; a < kg; ++a)
      for (int64_t q = 0; q < gs; ++q) cand[m++] = gi[a] * gs + q;
    sort_desc(m, cand, c);
    float den = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
      ids[t * k + j] = (int32_t)cand[j];
      den = (j == 0) ? s[cand[0]] : den + s[cand[j]];
    }
    for (int64_t j = 0; j < k; ++j) w[t * k + j] = (s[cand[j]] / den) * scale;
    if (ggap) ggap[t] = (kg < G) ? g[gi[kg - 1]] - g[gi[kg]] : INFINITY;
    if (egap) {
      float mg = INFINITY;
      for (int64_t j = 0; j < k && j + 1 < m; ++j) {
        float gap = c[cand[j]] - c[cand[j + 1]];
        if (gap < mg) mg = gap;
      }
      egap[t] = mg;
    }
  }
  free(s); free(c); free(g); free(gi); free(cand);
  return 0;
}

/*
 * O4 — expert histogram and stable permutation.
 * [vLLM §Der fusionierte Graph]: the MoE path runs routing kernels ahead of
 *   two grouped GEMMs, i.e. the token assignments are grouped by expert. The
 *   pages do not describe the layout. Reading: rows ordered by expert
 *   ascending, then by slot index t*k+j ascending (a counting sort).
 */
int oracle_permute(int64_t T, int64_t k, int64_t E, const int32_t* ids, int32_t* counts,
                   int32_t* offsets, int32_t* perm, int32_t* inv) {
  if (T < 0 || k < 1 || E <= 0) return -1;
  const int64_t n = T * k;
  for (int64_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t a = 0; a < n; ++a)
    if (ids[a] >= 0 && ids[a] < E) counts[ids[a]] += 1;
  offsets[0] = 0;
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int64_t* cursor = (int64_t*)malloc((size_t)E * sizeof(int64_t));
  if (!cursor) return -3;
  for (int64_t e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int64_t a = 0; a < n; ++a) perm[a] = -1;
  for (int64_t a = 0; a < n; ++a) {
    int32_t e = ids[a];
    if (e < 0 || e >= E) {
      inv[a] = -1;
      continue;
    }
    int64_t r = cursor[e]++;
    perm[r] = (int32_t)a;
    inv[a] = (int32_t)r;
  }
  free(cursor);
  return 0;
}

/*
 * O5 — one routed SwiGLU expert, weighted.
 * [vLLM §MoE und Residual-Stream]: 256 routed SwiGLU experts, d_ff 2560.
 * [SGLang §BF16 MoE 内核优化 (BF16 MoE kernel optimisation)]: the decode path
 *   keeps BF16 rounding boundaries for the gate/up projections and the
 *   activation, and applies the FP32 routing weight to the down projection's
 *   output before it is rounded to BF16.
 * Reading: g and u are each rounded to BF16; act = bf16(silu(g) * u); the down
 *   projection accumulates in FP32, is multiplied by the FP32 weight, and is
 *   rounded once.
 */
int oracle_expert_rows(int64_t R, int64_t d, int64_t f, const uint16_t* zrows,
                       const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd,
                       const float* wrow, uint16_t* yk) {
  if (R < 0 || d <= 0 || f <= 0) return -1;
  uint16_t* act = (uint16_t*)malloc((size_t)f * sizeof(uint16_t));
  if (!act) return -3;
  for (int64_t r = 0; r < R; ++r) {
    const uint16_t* z = zrows + r * d;
    for (int64_t q = 0; q < f; ++q) {
      float ag = 0.0f, au = 0.0f;
      for (int64_t i = 0; i < d; ++i) {
        float zi = oracle_f32(z[i]);
        ag = ag + zi * oracle_f32(Wg[q * d + i]);
        au = au + zi * oracle_f32(Wu[q * d + i]);
      }
      float gq = oracle_f32(oracle_bf16(ag));
      float uq = oracle_f32(oracle_bf16(au));
      act[q] = oracle_bf16(oracle_silu(gq) * uq);
    }
    for (int64_t o = 0; o < d; ++o) {
      float acc = 0.0f;
      for (int64_t q = 0; q < f; ++q) acc = acc + oracle_f32(act[q]) * oracle_f32(Wd[o * f + q]);
      yk[r * d + o] = oracle_bf16(wrow[r] * acc);
    }
  }
  free(act);
  return 0;
}

/*
 * O6 — the weighted top-k combine.
 * [vLLM §Agentengetriebene Optimierung, change 3]: after the MoE, the norm
 *   kernel also combines the top-8 expert outputs.
 * [SGLang, kernel-fusion paragraph]: the BF16 MoE path merges the local expert
 *   sum, the routing scale and the BF16 rounding.
 * Reading: per token, an FP32 sum of the k BF16 expert rows in slot order,
 *   rounded once. The sum starts from -0.0, the exact additive identity.
 */
int oracle_combine(int64_t T, int64_t k, int64_t d, int64_t E, const int32_t* ids,
                   const uint16_t* yk, uint16_t* y) {
  if (T < 0 || k < 1 || d <= 0) return -1;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t o = 0; o < d; ++o) {
      float acc = -0.0f;
      for (int64_t j = 0; j < k; ++j) {
        if (ids && (ids[t * k + j] < 0 || ids[t * k + j] >= E)) continue;
        acc = acc + oracle_f32(yk[(t * k + j) * d + o]);
      }
      y[t * d + o] = oracle_bf16(acc);
    }
  return 0;
}

/*
 * O7 — 4-bit expert weights.
 * [vLLM §Modellarchitektur]: the 256 routed experts are stored in a 4-bit
 *   floating-point format (NVFP4 there); [SGLang §BF16、NVFP4 和 FP8 模型支持]: the
 *   serving path takes BF16, NVFP4 and FP8 checkpoints.
 * Reading: the 4-bit format here is MXFP4 as the OCP Microscaling Formats (MX)
 *   specification v1.0 defines it, the block-scaled 4-bit format gfx950 converts
 *   natively: FP4 E2M1 elements (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 of a
 *   code is the sign) that share one E8M0 scale 2^X (stored as X + 127) per block of
 *   32 consecutive values along K. Quantising a block follows the specification's
 *   conversion: X = floor(log2(max |v|)) - 2, where 2 is the exponent of the largest
 *   E2M1 normal, clamped to [-127, 127] (an all-zero block takes X = -127); each
 *   element is v / 2^X rounded to the nearest E2M1 value, ties to the even code,
 *   magnitudes beyond 6 saturating to 6, with the sign kept even when the magnitude
 *   rounds to zero. Element 2i of a row is the low nibble of byte i.
 *   Every E2M1 value times 2^X is a BF16 number, so dequantisation is exact, and the
 *   experts then compute exactly as in O5 on the dequantised weights (activations
 *   stay BF16: the decode path is bound by the weight stream, not by arithmetic).
 */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

int oracle_mxfp4_quantize(int64_t rows, int64_t K, const uint16_t* v, uint8_t* codes,
                          uint8_t* scales) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return -1;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < K / 32; ++b) {
      const uint16_t* blk = v + r * K + b * 32;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) {
        const double a = fabs((double)oracle_f32(blk[i]));
        if (!(a <= 3.4e38)) return -1; /* inf or nan */
        if (a > amax) amax = a;
      }
      int X = -127;
      if (amax > 0.0) {
        int e;
        frexp(amax, &e); /* amax = m * 2^e, 0.5 <= m < 1: floor(log2(amax)) = e - 1 */
        X = (e - 1) - 2;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
      }
      scales[r * (K / 32) + b] = (uint8_t)(X + 127);
      for (int i = 0; i < 32; ++i) {
        const float vi = oracle_f32(blk[i]);
        const double q = ldexp(fabs((double)vi), -X);
        int best = 0;
        for (int j = 1; j < 8; ++j) {
          const double dj = fabs(q - kE2M1[j]), db = fabs(q - kE2M1[best]);
          if (dj < db || (dj == db && (j & 1) == 0)) best = j;
        }
        const int code = best | (signbit(vi) ? 8 : 0);
        uint8_t* byte = codes + r * (K / 2) + b * 16 + i / 2;
        if (i % 2 == 0) *byte = (uint8_t)code;
        else *byte = (uint8_t)(*byte | (code << 4));
      }
    }
  return 0;
}

int oracle_mxfp4_dequantize(int64_t rows, int64_t K, const uint8_t* codes, const uint8_t* scales,
                            uint16_t* out) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return -1;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < K; ++i) {
      const int s = scales[r * (K / 32) + i / 32];
      if (s == 255) return -1; /* the E8M0 NaN encoding */
      const uint8_t byte = codes[r * (K / 2) + i / 2];
      const int code = (i % 2 == 0) ? (byte & 15) : (byte >> 4);
      const double mag = ldexp(kE2M1[code & 7], s - 127);
      const double val = (code & 8) ? -mag : mag;
      out[r * K + i] = oracle_bf16((float)val); /* exact: val is a BF16 number */
    }
  return 0;
}

/*
 * O8 — experts with 4-bit activations.
 * [vLLM §Der fusionierte Graph]: the 4-bit MoE path at batch-1 decode is an activation
 *   quantisation, two routing kernels and two grouped GEMMs, i.e. the GEMMs multiply
 *   quantised activations by the 4-bit experts; [SGLang §BF16、NVFP4 和 FP8 模型支持]: the
 *   4-bit checkpoints are served on that path.
 * Reading: both GEMM inputs an expert multiplies by its weights are MXFP4-quantised by O7's
 *   rule, blocks of 32 consecutive values along the contraction: the token row z (blocks
 *   along d) before gate/up, and the activation row act (blocks along f) before down. They
 *   enter at their exact dequantised values; everything else is O5: g and u rounded to
 *   BF16, act = bf16(silu(g) * u), FP32 accumulation, the FP32 routing weight on the
 *   FP32 down sum, one rounding.
 */
int oracle_expert_rows_mx(int64_t R, int64_t d, int64_t f, const uint16_t* zrows,
                          const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd,
                          const float* wrow, uint16_t* yk) {
  if (R < 0 || d <= 0 || f <= 0 || d % 32 != 0 || f % 32 != 0) return -1;
  const int64_t big = d > f ? d : f;
  uint16_t* zq = (uint16_t*)malloc((size_t)d * sizeof(uint16_t));
  uint16_t* act = (uint16_t*)malloc((size_t)f * sizeof(uint16_t));
  uint16_t* actq = (uint16_t*)malloc((size_t)f * sizeof(uint16_t));
  uint8_t* codes = (uint8_t*)malloc((size_t)big / 2);
  uint8_t* scales = (uint8_t*)malloc((size_t)big / 32);
  int rc = 0;
  if (!zq || !act || !actq || !codes || !scales) rc = -3;
  for (int64_t r = 0; r < R && rc == 0; ++r) {
    /* the token row, quantised along d */
    if (oracle_mxfp4_quantize(1, d, zrows + r * d, codes, scales) != 0 ||
        oracle_mxfp4_dequantize(1, d, codes, scales, zq) != 0) {
      rc = -1;
      break;
    }
    for (int64_t q = 0; q < f; ++q) {
      float ag = 0.0f, au = 0.0f;
      for (int64_t i = 0; i < d; ++i) {
        float zi = oracle_f32(zq[i]);
        ag = ag + zi * oracle_f32(Wg[q * d + i]);
        au = au + zi * oracle_f32(Wu[q * d + i]);
      }
      float gq = oracle_f32(oracle_bf16(ag));
      float uq = oracle_f32(oracle_bf16(au));
      act[q] = oracle_bf16(oracle_silu(gq) * uq);
    }
    /* the activation row, quantised along f */
    if (oracle_mxfp4_quantize(1, f, act, codes, scales) != 0 ||
        oracle_mxfp4_dequantize(1, f, codes, scales, actq) != 0) {
      rc = -1;
      break;
    }
    for (int64_t o = 0; o < d; ++o) {
      float acc = 0.0f;
      for (int64_t q = 0; q < f; ++q) acc = acc + oracle_f32(actq[q]) * oracle_f32(Wd[o * f + q]);
      yk[r * d + o] = oracle_bf16(wrow[r] * acc);
    }
  }
  free(zq);
  free(act);
  free(actq);
  free(codes);
  free(scales);
  return rc;
}

/*
 * O5 in two halves, so a GPU path whose activation leaves one kernel for the next can be
 * checked stage by stage on identical inputs (the halves compose to O5, and with the two
 * MXFP4 round trips between them to O8; pinned by those identities):
 *   oracle_expert_act:  act[r] = bf16(silu(bf16(z_r . Wg^T)) * bf16(z_r . Wu^T))
 *   oracle_expert_down: yk[r]  = bf16(wrow[r] * (act_r . Wd^T))
 */
int oracle_expert_act(int64_t R, int64_t d, int64_t f, const uint16_t* zrows, const uint16_t* Wg,
                      const uint16_t* Wu, uint16_t* act) {
  if (R < 0 || d <= 0 || f <= 0) return -1;
  for (int64_t r = 0; r < R; ++r) {
    const uint16_t* z = zrows + r * d;
    for (int64_t q = 0; q < f; ++q) {
      float ag = 0.0f, au = 0.0f;
      for (int64_t i = 0; i < d; ++i) {
        float zi = oracle_f32(z[i]);
        ag = ag + zi * oracle_f32(Wg[q * d + i]);
        au = au + zi * oracle_f32(Wu[q * d + i]);
      }
      float gq = oracle_f32(oracle_bf16(ag));
      float uq = oracle_f32(oracle_bf16(au));
      act[r * f + q] = oracle_bf16(oracle_silu(gq) * uq);
    }
  }
  return 0;
}

int oracle_expert_down(int64_t R, int64_t d, int64_t f, const uint16_t* act, const uint16_t* Wd,
                       const float* wrow, uint16_t* yk) {
  if (R < 0 || d <= 0 || f <= 0) return -1;
  for (int64_t r = 0; r < R; ++r)
    for (int64_t o = 0; o < d; ++o) {
      float acc = 0.0f;
      for (int64_t q = 0; q < f; ++q)
        acc = acc + oracle_f32(act[r * f + q]) * oracle_f32(Wd[o * f + q]);
      yk[r * d + o] = oracle_bf16(wrow[r] * acc);
    }
  return 0;
}
