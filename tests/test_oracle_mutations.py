"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that the
pins in test_oracle_pins.py catch every one of them."""
import inspect
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

MUTATIONS = [
    ("swap residual coefficients", "uint16_t a = oracle_bf16(c1 *", "uint16_t a = oracle_bf16(c2 *"),
    ("coefficient without root", "(float)sqrt((double)(n - 1) / (double)n)", "(float)((double)(n - 1) / (double)n)"),
    ("eps outside the root", "1.0f / sqrtf(ss / (float)d + eps)", "1.0f / (sqrtf(ss / (float)d) + eps)"),
    ("sum instead of mean", "1.0f / sqrtf(ss / (float)d + eps)", "1.0f / sqrtf(ss + eps)"),
    ("norm weight dropped", "* oracle_f32(w[i]));", ");"),
    ("operands not rounded", "ho[i] = oracle_bf16(oracle_f32(a) + oracle_f32(b));",
     "ho[i] = oracle_bf16(c1 * oracle_f32(hr[i]) + c2 * oracle_f32(xn[i]));"),
    ("router transposed", "* W[e * d + i]", "* W[(i % E) * d + (i / E) % d]"),
    ("router in bf16", "acc = acc + oracle_f32(z[t * d + i]) * W[e * d + i];",
     "acc = oracle_f32(oracle_bf16(acc + oracle_f32(z[t * d + i]) * W[e * d + i]));"),
    ("sigmoid sign", "exp(-(double)logit)", "exp((double)logit)"),
    ("group score = max", "g[j] = (gs >= 2) ? m1 + m2 : m1;", "g[j] = m1;"),
    ("bias enters weights", "w[t * k + j] = (s[cand[j]] / den) * scale;",
     "w[t * k + j] = (c[cand[j]] / den) * scale;"),
    ("tie-break upward", "(va == vb && ia < ib)", "(va == vb && ia > ib)"),
    ("scale dropped", "w[t * k + j] = (s[cand[j]] / den) * scale;", "w[t * k + j] = (s[cand[j]] / den);"),
    ("permutation unstable", "for (int64_t a = 0; a < n; ++a) {\n    int32_t e = ids[a];",
     "for (int64_t a = n - 1; a >= 0; --a) {\n    int32_t e = ids[a];"),
    ("down weight transposed", "Wd[o * f + q]", "Wd[(q % d) * f + (o % f)]"),
    ("gate and up swapped", "oracle_silu(gq) * uq", "oracle_silu(uq) * gq"),
    ("weight after rounding", "yk[r * d + o] = oracle_bf16(wrow[r] * acc);",
     "yk[r * d + o] = oracle_bf16(wrow[r] * oracle_f32(oracle_bf16(acc)));"),
    ("mx scale rounds up", "X = (e - 1) - 2;", "X = e - 2;"),
    ("mx element exponent 3", "X = (e - 1) - 2;", "X = (e - 1) - 3;"),
    ("mx ties to the larger", "(dj == db && (j & 1) == 0)", "(dj == db && j > best)"),
    ("mx zero loses its sign", "best | (signbit(vi) ? 8 : 0)", "best | (vi < 0.0f ? 8 : 0)"),
    ("mx nibbles swapped", "if (i % 2 == 0) *byte = (uint8_t)code;", "if (i % 2 == 1) *byte = (uint8_t)code;"),
    ("mx dequant scale off by one", "ldexp(kE2M1[code & 7], s - 127)", "ldexp(kE2M1[code & 7], s - 126)"),
    ("mx no clamp of tiny scales", "if (X < -127) X = -127;", ""),
    ("combine rounds each add", "acc = acc + oracle_f32(yk[(t * k + j) * d + o]);",
     "acc = oracle_f32(oracle_bf16(acc + oracle_f32(yk[(t * k + j) * d + o])));"),
    ("sigmoid in FP32", "(float)(1.0 / (1.0 + exp(-(double)logit)))",
     "1.0f / (1.0f + expf(-logit))"),
    ("mx token row not quantised", "float zi = oracle_f32(zq[i]);",
     "float zi = oracle_f32(zrows[r * d + i]);"),
    ("mx activation not quantised", "acc = acc + oracle_f32(actq[q]) * oracle_f32(Wd[o * f + q]);",
     "acc = acc + oracle_f32(act[q]) * oracle_f32(Wd[o * f + q]);"),
    ("mx gate quantised instead of the activation", [
        ("float gq = oracle_f32(oracle_bf16(ag));\n      float uq = oracle_f32(oracle_bf16(au));\n"
         "      act[q] = oracle_bf16(oracle_silu(gq) * uq);\n    }\n    /* the activation row",
         "float gq = oracle_f32(oracle_bf16(ag));\n      float uq = oracle_f32(oracle_bf16(au));\n"
         "      act[q] = oracle_bf16(gq);\n      actq[q] = oracle_bf16(uq);\n    }\n"
         "    if (oracle_mxfp4_quantize(1, f, act, codes, scales) != 0 ||\n"
         "        oracle_mxfp4_dequantize(1, f, codes, scales, act) != 0) { rc = -1; break; }\n"
         "    for (int64_t q = 0; q < f; ++q)\n"
         "      act[q] = oracle_bf16(oracle_silu(oracle_f32(act[q])) * oracle_f32(actq[q]));\n"
         "    /* the activation row"),
        ("oracle_mxfp4_dequantize(1, f, codes, scales, actq) != 0) {\n      rc = -1;",
         "0) {\n      rc = -1;"),
        ("acc = acc + oracle_f32(actq[q]) * oracle_f32(Wd[o * f + q]);",
         "acc = acc + oracle_f32(act[q]) * oracle_f32(Wd[o * f + q]);"),
    ]),
    # the branch scaled from the unrounded post-norm output (norm factor recomputed per row)
    ("post-norm output not rounded", [
        ("rmsnorm_row(d, xr, w_post, eps, xn); /* post-norm of the branch, rounded */",
         "rmsnorm_row(d, xr, w_post, eps, xn); /* post-norm of the branch, rounded */\n"
         "    float rr_ = 0.0f;\n"
         "    for (int64_t q = 0; q < d; ++q) rr_ = rr_ + oracle_f32(xr[q]) * oracle_f32(xr[q]);\n"
         "    rr_ = 1.0f / sqrtf(rr_ / (float)d + eps);"),
        ("uint16_t b = oracle_bf16(c2 * oracle_f32(xn[i]));",
         "uint16_t b = oracle_bf16(c2 * ((oracle_f32(xr[i]) * rr_) * oracle_f32(w_post[i])));"),
    ]),
]

PIN_TESTS = [(name, fn) for name, fn in inspect.getmembers(pins, inspect.isfunction)
             if name.startswith("test_")]


def _run_pins(golden):
    failed = []
    for name, fn in PIN_TESTS:
        params = inspect.signature(fn).parameters
        kwargs = {}
        if "golden" in params:
            kwargs["golden"] = golden
        if "E" in params:  # the parametrised brute-force test: use one size
            kwargs["E"] = 8
        try:
            fn(**kwargs)
        except Exception:  # AssertionError or an error raised by a mutant
            failed.append(name)
    return failed


def _edits(m):
    """A mutation is (label, old, new) or (label, [(old, new), ...])."""
    return m[1] if len(m) == 2 else [(m[1], m[2])]


@pytest.mark.parametrize("label,edits", [(m[0], _edits(m)) for m in MUTATIONS],
                         ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(label, edits, tmp_path, golden):
    src = open(oracle.SRC_PATH).read()
    mutated = src
    for old, new in edits:
        assert mutated.count(old) >= 1, label
        mutated = mutated.replace(old, new)
    c_path = tmp_path / "mut.c"
    c_path.write_text(mutated)
    hdr = os.path.join(os.path.dirname(oracle.SRC_PATH), "beam_oracle.h")
    (tmp_path / "beam_oracle.h").write_text(open(hdr).read())
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                           str(c_path), "-o", str(so), "-lm"])
    saved_lib, saved_path = oracle._lib, oracle.LIB_PATH
    try:
        oracle._lib = None
        oracle.LIB_PATH = str(so)
        failed = _run_pins(golden)
    finally:
        oracle._lib, oracle.LIB_PATH = saved_lib, saved_path
    assert failed, f"no pin caught the mutation '{label}'"


def test_unmutated_oracle_passes_all_pins(golden):
    assert _run_pins(golden) == []
