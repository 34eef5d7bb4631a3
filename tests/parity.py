"""Comparison helpers for the GPU-vs-oracle parity tests (test-side only)."""
from __future__ import annotations

import numpy as np

import oracle

F = oracle.bf16_to_f32

# floating-point bars
REL_L2_MAX = 2e-3      # BF16 outputs, relative L2 over the compared set
ABS_MAX = 3e-2         # per element; an element over it that is within one BF16 ulp of the
                       # larger of the two magnitudes is counted as a final-rounding flip
LOGIT_REL_MAX = 1e-5   # per token row, relative L2
NEAR_TIE = 1e-6        # selection-score gap under which a token is reported as a near tie


def bits(t) -> np.ndarray:
    """BF16 torch tensor -> numpy uint16 bit patterns (host)."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev(a: np.ndarray, dtype=None):
    """numpy -> device tensor. uint16 arrays become BF16 tensors with the same bits."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    t = torch.from_numpy(a).cuda()
    return t if dtype is None else t.to(dtype)


def compare_bf16(got: np.ndarray, want: np.ndarray, rel_max=REL_L2_MAX, abs_max=ABS_MAX,
                 two_ulp=None):
    """Reading of the max-abs bar (3e-2): one BF16 ulp at |v| in [4, 8) is 0.03125, so a
    single final-rounding flip there exceeds it whatever the FP32 summation order. An
    element over the bar that is within one ulp of the larger of the two magnitudes is
    counted as such a flip; anything else over the bar fails; rel-L2 stays strict.
    two_ulp: optional mask of elements whose input already differs by a final
    rounding flip upstream (z where h' differs: z = bf16(h' r w), so a one-ulp h'
    difference carries into z before z's own rounding); there the allowance is two
    ulps of the larger magnitude (the inherited one plus this rounding)."""
    g = F(got).astype(np.float64)
    w = F(want).astype(np.float64)
    diff = np.abs(g - w)
    rel = float(np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-30))
    over = diff > abs_max
    big = np.maximum(np.abs(g), np.abs(w))
    # BF16 ulp of the larger magnitude: 2^(exponent - 7) for normal values
    ulp = np.exp2(np.floor(np.log2(np.maximum(big, 2.0 ** -126))) - 7)
    allow = ulp if two_ulp is None else np.where(two_ulp, 2 * ulp, ulp)
    one_ulp = over & (diff <= allow)
    fails = int(np.count_nonzero(over & ~one_ulp))
    stats = dict(rel_l2=rel, max_abs=float(diff.max()) if diff.size else 0.0,
                 ulp_flips=int(np.count_nonzero(one_ulp)), fails=fails,
                 exact=float(np.mean(got == want)) if got.size else 1.0, n=int(got.size))
    ok = rel <= rel_max and fails == 0
    return ok, stats


def assert_bf16_close(got, want, what, **kw):
    ok, st = compare_bf16(got, want, **kw)
    print(f"[parity] {what}: {st}", flush=True)
    assert ok, f"{what}: {st}"
    return st


def logit_rel_rows(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    g = got.astype(np.float64)
    w = want.astype(np.float64)
    return np.linalg.norm(g - w, axis=1) / np.maximum(np.linalg.norm(w, axis=1), 1e-30)


def check_routing(g_ids, g_w, o_ids, o_w, ggap, egap, g_logits, o_logits, what):
    """Compare the GPU's routing (from its own logits) with the oracle's.

    Expert ids and slot order must match exactly, except on tokens whose oracle
    selection gap is within what the logit difference between the two sides can
    move (scores are sigmoid(logit), slope <= 1/4; a group score sums two scores):
    those are counted as near-tie flips. Weights of matching tokens must agree to
    1e-5 relative plus what the logit difference explains (w = s / sum(s) * scale,
    so |dw|/w <= 2 max|ds| / min(s)). Returns (mask of matching tokens, stats)."""
    T = g_ids.shape[0]
    dl = np.max(np.abs(g_logits.astype(np.float64) - o_logits.astype(np.float64)), axis=1)
    tol = 4 * 0.25 * dl + NEAR_TIE
    gap = np.minimum(ggap.astype(np.float64), egap.astype(np.float64))
    same = np.all(g_ids == o_ids, axis=1)
    flips = ~same
    bad = flips & (gap > tol)
    near = int(np.count_nonzero(gap < NEAR_TIE))
    stats = dict(tokens=T, flips=int(np.count_nonzero(flips)), near_ties=near,
                 unexplained=int(np.count_nonzero(bad)), max_dlogit=float(dl.max()))
    wbad = 0
    if np.any(same):
        s_sel = 1.0 / (1.0 + np.exp(-np.take_along_axis(o_logits.astype(np.float64),
                                                          o_ids.astype(np.int64), axis=1)))
        wrel = np.abs(g_w.astype(np.float64) - o_w) / np.abs(o_w)
        wtol = 1e-5 + 2 * 0.25 * dl[:, None] / s_sel.min(axis=1, keepdims=True)
        wbad = int(np.count_nonzero((wrel > wtol)[same]))
        stats["w_max_rel"] = float(wrel[same].max())
        stats["w_bad"] = wbad
    print(f"[parity] {what} routing: {stats}", flush=True)
    assert stats["unexplained"] == 0, f"{what}: routing differs beyond near ties: {stats}"
    assert wbad == 0, f"{what}: routing weights differ beyond the logit difference: {stats}"
    return same, stats


def check_permutation_valid(ids: np.ndarray, perm: np.ndarray, offsets: np.ndarray, E: int):
    """Properties of the expert-grouped order that hold at any size: counts and
    offsets agree with ids, every valid slot appears once, rows are grouped by
    expert ascending and slots ascend within an expert."""
    flat = ids.ravel()
    n = flat.size
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    assert np.array_equal(np.diff(offsets), counts)
    assert offsets[0] == 0 and offsets[-1] == np.count_nonzero(valid)
    nv = int(offsets[-1])
    rows = perm[:nv]
    assert np.all(perm[nv:] == -1)
    assert np.array_equal(np.sort(rows), np.nonzero(valid)[0])
    e_of_row = flat[rows]
    assert np.all(np.diff(e_of_row) >= 0)
    same_e = np.diff(e_of_row) == 0
    assert np.all(np.diff(rows)[same_e] > 0)
