"""Pins for the CPU oracle: what the pages and plain mathematics fix, checked
without re-typing the oracle's formulas.

Each oracle step is pinned by closed forms on special inputs, invariants the
pages state, brute-force enumeration on tiny sizes, or error bounds against an
FP64 computation, chosen so that a dropped term, a wrong sign or index, a swapped
coefficient or a transposed operand fails at least one test (the "mutation"
test at the bottom plants such mistakes in a copy of the oracle and checks that
the pins catch them).
"""
import itertools
import math

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

F = oracle.bf16_to_f32


def to_bf16(a):
    """numpy RNE float32 -> bf16 bits (test-side helper for building inputs)."""
    a = np.asarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


# ---------------------------------------------------------------------------------------------
# scalar pieces

def test_bf16_rne_golden(golden):
    for case in golden["bf16_rne"]["cases"]:
        f = np.array([int(case["f32_bits"], 16)], dtype=np.uint32).view(np.float32)[0]
        assert oracle.bf16(float(f)) == int(case["bf16_bits"], 16), case


def test_bf16_widen_exact():
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    for b in bits[finite][:2000]:
        assert oracle.bf16(oracle.f32(int(b))) == int(b)


def test_sigmoid_golden(golden):
    for case in golden["sigmoid"]["cases"]:
        s = oracle.sigmoid(np.float32(case["logit"]))
        ulp = np.spacing(np.float32(case["score"]))
        assert abs(s - case["score"]) <= case["ulps"] * ulp + 0.0, case


def _f32_nearest(v):
    """The FP32 number nearest to the Decimal v (ties to even): the double nearest to v,
    narrowed, then its FP32 neighbours compared with v exactly."""
    from decimal import Decimal
    f = np.float32(float(v))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    errs = [abs(Decimal(float(c)) - v) for c in cands]
    best = min(errs)
    picks = [c for c, e in zip(cands, errs) if e == best]
    if len(picks) > 1:  # a tie: the even significand
        picks = [c for c in picks if (int(np.float32(c).view(np.uint32)) & 1) == 0]
    return picks[0]


def test_sigmoid_correctly_rounded():
    """Scores are sigmoid(logit) in FP32 ([vLLM page, MoE und Residual-Stream]; reading:
    the FP32 value nearest to the exact sigmoid). Checked against 1 / (1 + e^-v) evaluated
    with 50 significant digits (Python's decimal module) and rounded to the nearest FP32
    number, over logits spanning the router's range and the saturating tails."""
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    rng = np.random.default_rng(43)
    xs = np.concatenate([rng.standard_normal(2500) * 2.0, rng.uniform(-20.0, 20.0, 1000),
                         np.array([-88.0, -30.0, -17.5, -1e-6, 1e-6, 15.9, 17.0, 40.0])])
    xs = xs.astype(np.float32)
    bad = []
    for v in xs:
        exact = Decimal(1) / (Decimal(1) + (-Decimal(float(v))).exp())
        want = _f32_nearest(exact)
        got = np.float32(oracle.sigmoid(v))
        if got != want:
            bad.append((float(v), float(got), float(want)))
    assert not bad, bad[:5]


def test_sigmoid_symmetry_and_range():
    xs = np.linspace(-30, 30, 2001, dtype=np.float32)
    s = np.array([oracle.sigmoid(v) for v in xs])
    sm = np.array([oracle.sigmoid(-v) for v in xs])
    assert np.all(np.diff(s) >= 0)
    assert np.all((s >= 0) & (s <= 1))
    assert np.max(np.abs(s + sm - 1.0)) <= 2 * 2.0 ** -24


def test_silu_identities():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(40.0) == 40.0
    for v in np.linspace(-8, 8, 161, dtype=np.float32):
        # silu(-v) = silu(v) - v and silu(v) = v * sigmoid(v)
        assert abs(oracle.silu(-v) - (oracle.silu(v) - v)) <= 4e-6 * max(1.0, abs(v))
        assert abs(oracle.silu(v) - v * oracle.sigmoid(v)) <= 4e-6 * max(1.0, abs(v))


# ---------------------------------------------------------------------------------------------
# O1 boundary

def _rows(T, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return to_bf16(rng.standard_normal((T, d)).astype(np.float32) * scale)


def test_boundary_n1_is_postnorm(golden):
    """n = 1: sqrt(0) * h + x / 1 -> h' is the post-normed branch and ignores h."""
    d = 256
    x = _rows(4, d, 1)
    w = to_bf16(np.linspace(0.9, 1.1, d))
    h1 = _rows(4, d, 2)
    h2 = _rows(4, d, 3)
    a, za = oracle.boundary(h1, x, w, w, 1, 1e-6)
    b, zb = oracle.boundary(h2, x, w, w, 1, 1e-6)
    assert np.array_equal(a, b) and np.array_equal(za, zb)
    # and h' = xn: post-norm of x with w -> check against the constant-row closed form below
    xc = np.full((1, d), to_bf16(np.float32(1.5)), dtype=np.uint16)
    hc, _ = oracle.boundary(np.zeros_like(xc), xc, w, w, 1, 0.0)
    assert np.array_equal(hc[0], w)


def test_boundary_constant_row_closed_form():
    """A constant branch row c with eps = 0 normalises to sign(c) * w_post exactly."""
    d = 512
    w_post = to_bf16(np.random.default_rng(0).uniform(0.9, 1.1, d))
    w_pre = to_bf16(np.random.default_rng(1).uniform(0.9, 1.1, d))
    ones = to_bf16(np.ones(d))
    for c in (1.5, -1.5, 3.0, 0.75):
        x = np.full((1, d), to_bf16(np.float32(c)), dtype=np.uint16)
        # n = 4: c2 = 1/2 exactly; h = 0 -> h' = bf16(0.5 * xn) = 0.5 * sign(c) * w_post (exact)
        hp, z = oracle.boundary(np.zeros((1, d), np.uint16), x, w_post, w_pre, 4, 0.0)
        assert np.array_equal(F(hp[0]), np.float32(0.5) * np.sign(c) * F(w_post))
        # with w_post = 1 the next norm sees a constant row +-0.5 -> z = sign(c) * w_pre
        hp, z = oracle.boundary(np.zeros((1, d), np.uint16), x, ones, w_pre, 4, 0.0)
        assert np.array_equal(F(z[0]), np.sign(c) * F(w_pre))


def test_boundary_coefficients_golden(golden):
    """x = 0 isolates the residual scale: h' = bf16(c1 * h); h = 0 isolates the branch scale."""
    d = 64
    h = to_bf16(np.linspace(-4, 4, d)).reshape(1, d)
    ones = to_bf16(np.ones(d))
    for case in golden["depth_scaled_residual"]["cases"]:
        n, c1, c2 = case["n"], case["c1"], case["c2"]
        assert abs(c1 * c1 + c2 * c2 - 1.0) < 1e-11  # the unit-variance identity
        hp, _ = oracle.boundary(h, np.zeros((1, d), np.uint16), ones, ones, n, 1e-6)
        # the oracle multiplies by FP32(c1) and rounds twice (operand, then sum with +0)
        want = F(to_bf16(np.float32(c1) * F(h[0])))
        assert np.array_equal(F(hp[0]), want), n
        # branch scale: constant x row of 1.5 normalises to exactly w (= 1) with eps = 0
        x = np.full((1, d), to_bf16(np.float32(1.5)), dtype=np.uint16)
        hp, _ = oracle.boundary(np.zeros((1, d), np.uint16), x, ones, ones, n, 0.0)
        assert np.all(F(hp[0]) == F(to_bf16(np.float32(c2)))), n


def test_boundary_eps_inside_root():
    """A tiny constant row v with eps: xn = w * v / sqrt(v^2 + eps) (eps inside the root)."""
    d = 128
    v = float(F(to_bf16(np.float32(1e-3))))
    x = np.full((1, d), to_bf16(np.float32(v)), dtype=np.uint16)
    ones = to_bf16(np.ones(d))
    hp, _ = oracle.boundary(np.zeros((1, d), np.uint16), x, ones, ones, 1, 1e-6)
    want = v / math.sqrt(v * v + 1e-6)
    assert abs(F(hp[0])[0] - want) <= 2.0 ** -8 * want


def test_boundary_scale_invariance():
    """Doubling the branch (eps = 0) changes nothing; doubling w_pre doubles z exactly."""
    d = 256
    x = _rows(6, d, 4)
    h = _rows(6, d, 5)
    w = to_bf16(np.random.default_rng(2).uniform(0.9, 1.1, d))
    a, za = oracle.boundary(h, x, w, w, 20, 0.0)
    x2 = to_bf16(F(x) * 2)
    b, zb = oracle.boundary(h, x2, w, w, 20, 0.0)
    assert np.array_equal(a, b) and np.array_equal(za, zb)
    w2 = to_bf16(F(w) * 2)
    c, zc = oracle.boundary(h, x, w, w2, 20, 0.0)
    assert np.array_equal(c, a) and np.array_equal(F(zc), 2 * F(za))


def test_boundary_unit_variance_invariant():
    """With unit-variance h and x, and unit norm weights, h' keeps unit variance."""
    T, d = 1024, 1024
    h = _rows(T, d, 6)
    x = _rows(T, d, 7)
    ones = to_bf16(np.ones(d))
    for n in (2, 20):
        hp, z = oracle.boundary(h, x, ones, ones, n, 1e-6)
        v = float(np.mean(F(hp).astype(np.float64) ** 2))
        N = T * d
        assert abs(v - 1.0) < 5 * math.sqrt(2.0 / N) + 2e-3, (n, v)
        # the next pre-norm makes every row's mean square 1 (up to BF16 rounding)
        ms = np.mean(F(z).astype(np.float64) ** 2, axis=1)
        assert np.all(np.abs(ms - 1.0) < 4e-3)


def test_boundary_rejects_bad_args():
    d = 8
    h = np.zeros((1, d), np.uint16)
    with pytest.raises(ValueError):
        oracle.boundary(h, h, h[0], h[0], 0, 1e-6)


# ---------------------------------------------------------------------------------------------
# O2 router

def test_router_one_hot_rows_pick_entries():
    """W[e] = one-hot at pi(e) -> logits[:, e] = z[:, pi(e)] exactly (catches a transpose)."""
    T, d, E = 5, 96, 40
    z = _rows(T, d, 8)
    pi = np.random.default_rng(3).permutation(d)[:E]
    W = np.zeros((E, d), np.float32)
    W[np.arange(E), pi] = 1.0
    lg = oracle.router(z, W)
    assert np.array_equal(lg, F(z)[:, pi])


def test_router_exact_small_integers():
    T, d, E = 7, 128, 24
    rng = np.random.default_rng(9)
    zi = rng.integers(-8, 9, (T, d))
    Wi = rng.integers(-16, 17, (E, d))
    lg = oracle.router(to_bf16(zi.astype(np.float32)), Wi.astype(np.float32))
    assert np.array_equal(lg.astype(np.int64), zi @ Wi.T)


def test_router_fp32_error_bound():
    """Sequential FP32 accumulation: |l - exact| <= gamma_d * sum |z W| (Higham 3.1)."""
    T, d, E = 4, 5120, 16
    z = _rows(T, d, 10)
    W = (np.random.default_rng(11).standard_normal((E, d)) / math.sqrt(d)).astype(np.float32)
    lg = oracle.router(z, W)
    zf = F(z).astype(np.float64)
    exact = zf @ W.astype(np.float64).T
    mag = np.abs(zf) @ np.abs(W.astype(np.float64)).T
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    assert np.all(np.abs(lg - exact) <= gamma * mag)
    # and it is FP32, not a lower precision: typical error far below a BF16 rounding
    assert np.max(np.abs(lg - exact)) < 1e-4


# ---------------------------------------------------------------------------------------------
# O3 grouped top-k

def _brute_topk(logit_row, bias, G, kg, k, scale):
    """Enumerate every kept-group subset and expert subset; keep the one that
    dominates under (value desc, index asc). Independent of the oracle's sort."""
    E = len(logit_row)
    gs = E // G
    s = np.array([oracle.sigmoid(v) for v in logit_row], dtype=np.float32)
    c = (s + bias).astype(np.float32)

    def beats(va, ia, vb, ib):
        return va > vb or (va == vb and ia < ib)

    g = []
    for j in range(G):
        mem = c[j * gs:(j + 1) * gs]
        if gs == 1:
            g.append(np.float32(mem[0]))
        else:  # best pair sum = sum of the two largest
            g.append(max(np.float32(mem[a] + mem[b]) for a in range(gs) for b in range(gs) if a != b))
    good_groups = []
    for S in itertools.combinations(range(G), kg):
        rest = [j for j in range(G) if j not in S]
        if all(beats(g[a], a, g[b], b) for a in S for b in rest):
            good_groups.append(S)
    assert len(good_groups) == 1
    cand = [j * gs + q for j in good_groups[0] for q in range(gs)]
    good = []
    for K in itertools.combinations(cand, k):
        rest = [e for e in cand if e not in K]
        if all(beats(c[a], a, c[b], b) for a in K for b in rest):
            good.append(K)
    assert len(good) == 1
    ids = sorted(good[0], key=lambda e: (-float(c[e]), e))
    den = np.float32(0)
    for j, e in enumerate(ids):
        den = s[e] if j == 0 else np.float32(den + s[e])
    w = [np.float32(np.float32(s[e] / den) * np.float32(scale)) for e in ids]
    return np.array(ids, np.int32), np.array(w, np.float32)


@pytest.mark.parametrize("E", [4, 6, 8, 12])
def test_topk_brute_force(E):
    rng = np.random.default_rng(E)
    for G in [g for g in range(1, E + 1) if E % g == 0]:
        gs = E // G
        for kg in range(1, G + 1):
            for k in range(1, min(kg * gs, 6) + 1):
                for trial in range(2):
                    lg = rng.standard_normal((1, E)).astype(np.float32)
                    if trial == 1:  # forced ties: quantised logits, zero bias
                        lg = np.round(lg * 2) / 2
                        bias = np.zeros(E, np.float32)
                    else:
                        bias = rng.uniform(-0.01, 0.01, E).astype(np.float32)
                    ids, w, _, _ = oracle.topk(lg, bias, G, kg, k, 2.5)
                    bi, bw = _brute_topk(lg[0], bias, G, kg, k, 2.5)
                    assert np.array_equal(ids[0], bi), (E, G, kg, k, trial)
                    assert np.array_equal(w[0], bw), (E, G, kg, k, trial)


def test_topk_weights_sum_to_scale():
    E, G, kg, k = 256, 8, 4, 8
    rng = np.random.default_rng(12)
    lg = rng.standard_normal((500, E)).astype(np.float32)
    bias = rng.uniform(-0.01, 0.01, E).astype(np.float32)
    ids, w, _, _ = oracle.topk(lg, bias, G, kg, k, 2.5)
    sums = w.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(sums - 2.5) <= 4 * np.spacing(np.float32(2.5)))
    # distinct ids, each row's ids from at most kg groups
    for row in ids:
        assert len(set(row.tolist())) == k
        assert len(set((row // (E // G)).tolist())) <= kg


def test_topk_single_group_is_plain_topk():
    E, k = 64, 8
    rng = np.random.default_rng(13)
    lg = rng.standard_normal((50, E)).astype(np.float32)
    bias = rng.uniform(-0.01, 0.01, E).astype(np.float32)
    ids, _, _, _ = oracle.topk(lg, bias, 1, 1, k, 2.5)
    for t in range(50):
        s = np.array([oracle.sigmoid(v) for v in lg[t]], np.float32)
        c = (s + bias).astype(np.float32)
        order = np.lexsort((np.arange(E), -c.astype(np.float64)))
        assert np.array_equal(ids[t], order[:k])


def test_topk_all_experts_is_dense_softmax_free_mixture():
    """kg = G, k = E: every expert selected; w = s / sum(s) * scale in c order."""
    E, G = 16, 4
    rng = np.random.default_rng(14)
    lg = rng.standard_normal((3, E)).astype(np.float32)
    bias = np.zeros(E, np.float32)
    ids, w, _, _ = oracle.topk(lg, bias, G, G, E, 2.5)
    for t in range(3):
        assert sorted(ids[t].tolist()) == list(range(E))
        s = np.array([oracle.sigmoid(v) for v in lg[t]], np.float64)
        assert np.allclose(w[t], s[ids[t]] / s.sum() * 2.5, rtol=1e-6)


def test_topk_bias_selects_but_does_not_weight():
    """A large bias forces a low-score expert in; its weight still uses its unbiased score."""
    E, G, kg, k = 8, 1, 1, 2
    lg = np.array([[3.0, 2.0, 1.0, 0.0, -1.0, -2.0, -3.0, -4.0]], np.float32)
    bias = np.zeros(E, np.float32)
    bias[7] = 1.0
    ids, w, _, _ = oracle.topk(lg, bias, G, kg, k, 2.5)
    assert ids[0].tolist() == [7, 0]  # c7 = sigmoid(-4) + 1 = 1.018 > c0 = 0.953
    s7, s0 = oracle.sigmoid(-4.0), oracle.sigmoid(3.0)
    assert abs(w[0][0] - s7 / (s7 + s0) * 2.5) < 1e-6
    assert abs(w[0][1] - s0 / (s7 + s0) * 2.5) < 1e-6


def test_topk_group_score_is_top2_sum():
    """Group A: one strong expert; group B: two good ones. Top-2 sum prefers B,
    a max rule would prefer A, a sum over the whole group would prefer C."""
    # 3 groups of 4 experts, keep 1 group, pick 1 expert
    E, G = 12, 3
    s_target = {0: 0.95, 1: 0.10, 2: 0.10, 3: 0.10,   # A: max 0.95, top2 1.05, all 1.25
                4: 0.60, 5: 0.58, 6: 0.05, 7: 0.05,   # B: max 0.60, top2 1.18, all 1.28
                8: 0.40, 9: 0.40, 10: 0.40, 11: 0.40}  # C: max 0.40, top2 0.80, all 1.60
    lg = np.array([[math.log(p / (1 - p)) for p in (s_target[e] for e in range(E))]], np.float32)
    ids, _, _, _ = oracle.topk(lg, np.zeros(E, np.float32), G, 1, 1, 2.5)
    assert ids[0].tolist() == [4]


def test_topk_gaps_report_near_ties():
    E, G, kg, k = 16, 4, 2, 3
    lg = np.zeros((1, E), np.float32)  # all equal: every gap is zero
    ids, w, ggap, egap = oracle.topk(lg, np.zeros(E, np.float32), G, kg, k, 2.5)
    assert ggap[0] == 0 and egap[0] == 0
    assert ids[0].tolist() == [0, 1, 2]  # lower index wins every tie
    # w = (s / den) * scale with each step rounded to FP32: (0.5 / 1.5) * 2.5
    assert np.all(w[0] == np.float32(np.float32(np.float32(0.5) / np.float32(1.5)) * np.float32(2.5)))


# ---------------------------------------------------------------------------------------------
# O4 permutation

def test_permute_matches_brute_force_sort():
    rng = np.random.default_rng(15)
    for T, k, E in [(1, 8, 256), (37, 8, 32), (200, 4, 16), (3, 2, 5)]:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        counts, offsets, perm, inv = oracle.permute(ids, E)
        pairs = sorted((int(ids.ravel()[a]), a) for a in range(T * k))
        assert perm.tolist() == [a for _, a in pairs]
        assert counts.tolist() == np.bincount(ids.ravel(), minlength=E).tolist()
        assert offsets[0] == 0 and offsets[-1] == T * k and np.all(np.diff(offsets) >= 0)
        assert np.array_equal(inv[perm], np.arange(T * k))


def test_permute_skips_invalid_ids():
    ids = np.array([[0, 5, -1], [2, 9, 0]], np.int32)  # E = 6: -1 and 9 are invalid
    counts, offsets, perm, inv = oracle.permute(ids, 6)
    assert counts.tolist() == [2, 0, 1, 0, 0, 1]
    assert perm.tolist() == [0, 5, 3, 1, -1, -1]
    assert inv.tolist() == [0, 3, -1, 2, -1, 1]


# ---------------------------------------------------------------------------------------------
# O5 / O6 experts and combine

def _perm_matrix(rows, cols, pi, val):
    M = np.zeros((rows, cols), np.float32)
    M[np.arange(rows), pi] = val
    return to_bf16(M)


def test_expert_permutation_closed_form():
    """Wg = 2 P_g, Wu = 0.5 P_u, Wd = P_d (one-hot rows): every sum has one
    non-zero term, so y_o = bf16(w * act[pd(o)]) with
    act_q = bf16(silu(2 z[pg(q)]) * 0.5 z[pu(q)]). A transposed operand reads
    the inverse permutation and fails."""
    d = f = 64
    rng = np.random.default_rng(16)
    pg, pu, pd = rng.permutation(f), rng.permutation(f), rng.permutation(d)
    Wg = _perm_matrix(f, d, pg, 2.0)
    Wu = _perm_matrix(f, d, pu, 0.5)
    Wd = _perm_matrix(d, f, pd, 1.0)
    z = _rows(3, d, 17)
    wrow = np.array([2.5, 0.75, 1.0], np.float32)
    yk = oracle.expert_rows(z, Wg, Wu, Wd, wrow)
    zf = F(z).astype(np.float64)
    for r in range(3):
        g = 2.0 * zf[r, pg]
        u = 0.5 * zf[r, pu]
        act = F(to_bf16((g / (1.0 + np.exp(-g)) * u).astype(np.float32)))
        want = F(to_bf16((wrow[r] * act[pd]).astype(np.float32)))
        got = F(yk[r])
        # silu differs from the FP64 form only at FP32 rounding -> at most one BF16 step
        step = np.spacing(np.maximum(np.abs(want), 1e-30).astype(np.float32)) * 65536
        assert np.all(np.abs(got - want) <= step), r
        assert np.mean(got == want) > 0.97


def _mx_round_trip(v):
    """O7 quantise-dequantise of BF16 rows (blocks of 32 along the row); O7 itself is pinned
    by the hand-derived blocks below."""
    return oracle.mxfp4_dequantize(*oracle.mxfp4_quantize(v))


def test_mx_activations_permutation_closed_form():
    """O8 ([vLLM page, Der fusionierte Graph]: the 4-bit MoE path quantises the activations
    before its grouped GEMMs). With one-hot weight rows every GEMM sum has one term, so
      g_q = zq[pg(q)], u_q = zq[pu(q)], act = bf16(silu(g) * u), y_o = bf16(w * actq[pd(o)])
    where zq and actq are the MXFP4 round trips of the token row and the activation row,
    blocks of 32 along each row. The rows differ in magnitude by 2^10 and 2^-10, so blocks
    that straddle rows, a skipped quantisation, or quantising g, u or y instead fail."""
    d = f = 64
    rng = np.random.default_rng(46)
    pg, pu, pd = rng.permutation(f), rng.permutation(f), rng.permutation(d)
    Wg = _perm_matrix(f, d, pg, 1.0)
    Wu = _perm_matrix(f, d, pu, 1.0)
    Wd = _perm_matrix(d, f, pd, 1.0)
    z = to_bf16(rng.standard_normal((3, d)).astype(np.float32) *
                np.array([[1.0], [1024.0], [1.0 / 1024]], np.float32))
    wrow = np.array([2.5, 0.75, 1.25], np.float32)
    yk = oracle.expert_rows_mx(z, Wg, Wu, Wd, wrow)
    zq = F(_mx_round_trip(z))
    g, u = zq[:, pg], zq[:, pu]
    act = to_bf16(np.array([[oracle.silu(a) for a in row] for row in g], np.float32) * u)
    actq = F(_mx_round_trip(act))
    want = to_bf16(wrow[:, None] * actq[:, pd])
    # values (the FP32 sums start at +0, so a -0 term leaves +0: compare as numbers)
    assert np.array_equal(F(yk), F(want))
    # the case tells the readings apart: both quantisations change many outputs
    no_act_q = to_bf16(wrow[:, None] * F(act)[:, pd])
    assert np.mean(no_act_q != want) > 0.5
    assert np.mean(zq != F(z)) > 0.5


def test_mx_activations_half_step_bound():
    """Random layer: O8 differs from O5 (BF16 activations) by about the MXFP4 quantisation
    noise of the activations, far more than rounding and far less than the signal."""
    d, f, R = 128, 96, 8
    rng = np.random.default_rng(47)
    z = _rows(R, d, 48)
    Wg = to_bf16(rng.standard_normal((f, d)) * 0.1)
    Wu = to_bf16(rng.standard_normal((f, d)) * 0.1)
    Wd = to_bf16(rng.standard_normal((d, f)) * 0.1)
    w = np.ones(R, np.float32)
    a = F(oracle.expert_rows_mx(z, Wg, Wu, Wd, w)).astype(np.float64)
    b = F(oracle.expert_rows(z, Wg, Wu, Wd, w)).astype(np.float64)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert 0.02 < rel < 0.5, rel


def test_expert_halves_compose_to_o5_and_o8():
    """The stage functions used to check GPU kernels one stage at a time: down(act(z)) is O5
    bit for bit, and with MXFP4 round trips of z and act between them, O8; act alone is O5's
    output through an identity down projection with weight 1."""
    d, f, R = 128, 96, 5
    rng = np.random.default_rng(49)
    z = _rows(R, d, 50)
    Wg = to_bf16(rng.standard_normal((f, d)) * 0.1)
    Wu = to_bf16(rng.standard_normal((f, d)) * 0.1)
    Wd = to_bf16(rng.standard_normal((d, f)) * 0.1)
    w = np.array([2.5, 0.5, 1.0, 0.25, 1.75], np.float32)
    act = oracle.expert_act(z, Wg, Wu)
    assert np.array_equal(oracle.expert_down(act, Wd, w), oracle.expert_rows(z, Wg, Wu, Wd, w))
    act_mx = oracle.expert_act(_mx_round_trip(z), Wg, Wu)
    assert np.array_equal(oracle.expert_down(_mx_round_trip(act_mx), Wd, w),
                          oracle.expert_rows_mx(z, Wg, Wu, Wd, w))
    # d = f: an identity down projection with weight 1 passes act through unchanged
    zs = z[:, :f].copy()
    Wg2, Wu2 = Wg[:, :f].copy(), Wu[:, :f].copy()
    ident = to_bf16(np.eye(f, dtype=np.float32))
    assert np.array_equal(F(oracle.expert_rows(zs, Wg2, Wu2, ident, np.ones(R, np.float32))),
                          F(oracle.expert_act(zs, Wg2, Wu2)))


def _dense_swiglu_fp64(z, Wg, Wu, Wd, w):
    """Independent FP64 dense SwiGLU with the BF16 rounding points (test-side)."""
    zf = F(z).astype(np.float64)
    g = F(to_bf16((zf @ F(Wg).astype(np.float64).T).astype(np.float32)))
    u = F(to_bf16((zf @ F(Wu).astype(np.float64).T).astype(np.float32)))
    gd = g.astype(np.float64)
    act = F(to_bf16((gd / (1.0 + np.exp(-gd)) * u).astype(np.float32)))
    dn = act.astype(np.float64) @ F(Wd).astype(np.float64).T
    return F(to_bf16((w[:, None] * dn).astype(np.float32)))


def test_one_expert_is_dense_swiglu_times_scale():
    """E = G = k = 1: the weight is s/s * 2.5 = 2.5 exactly, the output a dense SwiGLU x 2.5."""
    d, f, T = 128, 96, 6
    rng = np.random.default_rng(18)
    z = _rows(T, d, 19)
    Wg = to_bf16(rng.standard_normal((f, d)) * 0.1)
    Wu = to_bf16(rng.standard_normal((f, d)) * 0.1)
    Wd = to_bf16(rng.standard_normal((d, f)) * 0.1)
    lg = rng.standard_normal((T, 1)).astype(np.float32)
    ids, w, _, _ = oracle.topk(lg, np.zeros(1, np.float32), 1, 1, 1, 2.5)
    assert np.all(ids == 0) and np.all(w == np.float32(2.5))
    y, _ = oracle.moe_experts(z, ids, w, 1, lambda e: (Wg, Wu, Wd))
    want = _dense_swiglu_fp64(z, Wg, Wu, Wd, np.full(T, 2.5))
    got = F(y)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel < 2e-3
    assert np.mean(got == want) > 0.95  # identical except rare FP32-vs-FP64 rounding flips


def test_all_experts_is_dense_mixture():
    """k = E: y = bf16(sum_e bf16(w_e * D_e(z))) in selection order."""
    d, f, E, G, T = 64, 64, 4, 2, 3
    rng = np.random.default_rng(20)
    Ws = [(to_bf16(rng.standard_normal((f, d)) * 0.1), to_bf16(rng.standard_normal((f, d)) * 0.1),
           to_bf16(rng.standard_normal((d, f)) * 0.1)) for _ in range(E)]
    z = _rows(T, d, 21)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    ids, w, _, _ = oracle.topk(lg, np.zeros(E, np.float32), G, G, E, 2.5)
    y, _ = oracle.moe_experts(z, ids, w, E, lambda e: Ws[e])
    for t in range(T):
        acc = np.float32(-0.0)
        for j in range(E):
            e = ids[t, j]
            part = _dense_swiglu_fp64(z[t:t + 1], *Ws[e], np.array([w[t, j]], np.float64))[0]
            acc = (acc + part).astype(np.float32)
        want = F(to_bf16(acc))
        got = F(y[t])
        assert np.linalg.norm(got - want) / np.linalg.norm(want) < 2e-3
        assert np.mean(got == want) > 0.9


def test_combine_slot_order_and_invalid_slots():
    """FP32 sum in slot order, one rounding; invalid slots are skipped."""
    big, small = 256.0, 1.0  # 256 + 1 is exact in FP32; rounding only at the end
    yk = to_bf16(np.array([[[big], [small], [small], [-big]]], np.float32))
    y = oracle.combine(yk)
    assert F(y)[0, 0] == 2.0
    ids = np.array([[0, 1, 9, 2]], np.int32)  # slot 2 invalid for E = 4
    y2 = oracle.combine(yk, ids, 4)
    assert F(y2)[0, 0] == 1.0
    # all-negative-zero rows stay -0 (the sum starts from -0.0)
    yz = np.full((1, 3, 1), 0x8000, np.uint16)
    assert oracle.combine(yz)[0, 0] == 0x8000


def test_boundary_operands_rounded_before_add():
    """[SGLang, sandwich norm section] both scaled operands are rounded to BF16
    before the add. Pick h where bf16(c1*h) + b rounds differently from
    c1*h + b, so an implementation that adds unrounded operands fails."""
    n = 20
    c1 = np.float32(math.sqrt(19 / 20))
    d = 64
    # x row constant 1.5 with eps = 0 -> xn = w_post exactly; w_post = 1 -> b = bf16(c2)
    ones = to_bf16(np.ones(d))
    x = np.full((1, d), to_bf16(np.float32(1.5)), dtype=np.uint16)
    b = F(to_bf16(np.float32(1.0 / math.sqrt(20))))
    cand = to_bf16(np.linspace(0.5, 8.0, 20000).astype(np.float32))
    hv = F(cand)
    rounded = F(to_bf16(F(to_bf16(c1 * hv)) + b))
    unrounded = F(to_bf16((c1 * hv).astype(np.float32) + b))
    pick = np.nonzero(rounded != unrounded)[0]
    assert len(pick) >= d
    h = cand[pick[:d]].reshape(1, d)
    hp, _ = oracle.boundary(h, x, ones, ones, n, 0.0)
    assert np.array_equal(F(hp[0]), rounded[pick[:d]])


def power_of_four_rows(T, seed):
    """Branch rows of 64 small odd integers (twenty 5s, thirty 3s, nine 1s, five 7s, random
    signs and order) whose squares sum to 1024 = 64 * 16: the mean square is exactly 16 in
    any summation order, so with eps = 0 the RMSNorm factor is exactly 1/4, and each
    x * (1/4) * w (at most 3 + 8 significant bits) is exact in FP32 but usually not a
    BF16 number."""
    base = np.array([5.0] * 20 + [3.0] * 30 + [1.0] * 9 + [7.0] * 5, np.float32)
    assert float(np.sum(base.astype(np.float64) ** 2)) == 1024.0
    rng = np.random.default_rng(seed)
    rows = np.stack([rng.permutation(base) * rng.choice([-1.0, 1.0], 64) for _ in range(T)])
    return to_bf16(rows.astype(np.float32))


def test_boundary_postnorm_output_rounded(golden):
    """[SGLang, sandwich norm section] the unfused boundary writes the post-normed branch
    and reads it back for the residual: the post-norm output is a BF16 tensor before it is
    scaled by 1/sqrt(n). On rows with an exact norm factor (h = 0, eps = 0) the result is
    h' = bf16(c2 * bf16(x * w / 4)); scaling the unrounded x * w / 4 instead gives a
    different h' on some elements, which this case checks it has."""
    d, n = 64, 20
    c2 = np.float32([c["c2"] for c in golden["depth_scaled_residual"]["cases"]
                     if c["n"] == n][0])
    x = power_of_four_rows(8, 41)
    w_post = to_bf16(np.random.default_rng(42).uniform(0.9, 1.1, d))
    ones = to_bf16(np.ones(d))
    xn = (F(x) * np.float32(0.25)) * F(w_post)  # exact in FP32
    with_r1 = F(to_bf16(c2 * F(to_bf16(xn))))
    without_r1 = F(to_bf16(c2 * xn))
    assert np.count_nonzero(with_r1 != without_r1) >= 16  # the case can tell them apart
    hp, _ = oracle.boundary(np.zeros_like(x), x, w_post, ones, n, 0.0)
    assert np.array_equal(F(hp), with_r1)


def test_expert_weight_applied_before_rounding():
    """[SGLang, BF16 MoE kernel section] the FP32 routing weight multiplies the
    down projection's FP32 output before its BF16 rounding. Two-term down sums
    make the difference visible: y = bf16(w * (act_a + act_b)), exact in FP32."""
    d = f = 32
    rng = np.random.default_rng(22)
    pg, pu = rng.permutation(f), rng.permutation(f)
    Wg = _perm_matrix(f, d, pg, 1.0)
    Wu = _perm_matrix(f, d, pu, 1.0)
    Wd = np.zeros((d, f), np.float32)
    a_idx, b_idx = rng.permutation(f), rng.permutation(f)
    b_idx = np.where(b_idx == a_idx, (b_idx + 1) % f, b_idx)
    Wd[np.arange(d), a_idx] = 1.0
    Wd[np.arange(d), b_idx] = 1.0
    Wd = to_bf16(Wd)
    z = _rows(2, d, 23)
    wrow = np.array([2.5, 1.25], np.float32)
    yk = oracle.expert_rows(z, Wg, Wu, Wd, wrow)
    for r in range(2):
        g = F(z[r])[pg].astype(np.float32)
        u = F(z[r])[pu].astype(np.float32)
        act = np.array([oracle.f32(oracle.bf16(oracle.silu(gv) * uv)) for gv, uv in zip(g, u)],
                       np.float32)
        s = (act[a_idx] + act[b_idx]).astype(np.float32)  # exact: both BF16 of similar size
        want = F(to_bf16((np.float32(wrow[r]) * s).astype(np.float32)))
        alt = F(to_bf16((np.float32(wrow[r]) * F(to_bf16(s))).astype(np.float32)))
        assert np.array_equal(F(yk[r]), want)
        assert not np.array_equal(want, alt)  # the case does tell the two readings apart


# ---- O7: MXFP4 expert weights ------------------------------------------------------------------

_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _golden_value(v):
    """A fixture value: a decimal, "-0.0", or "a*2^b" / "2^b" (exact binary fractions)."""
    if isinstance(v, str):
        if v == "-0.0":
            return -0.0
        mant, _, exp = v.rpartition("2^")
        m = float(mant.rstrip("*")) if mant else 1.0
        return math.ldexp(m, int(exp))
    return float(v)


def _to_bf16_exact(vals):
    f = np.asarray(vals, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "fixture value is not exactly BF16"
    return (bits >> 16).astype(np.uint16)


def _nibbles(codes):
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = c & 15
    out[..., 1::2] = c >> 4
    return out


def test_mxfp4_golden_blocks():
    """Hand-derived blocks (tests/golden/mxfp4.json): the scale rule, every rounding tie,
    saturation, signed zero, the clamped scale of tiny and the largest blocks."""
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "mxfp4.json")
    blocks = json.load(open(path))["blocks"]
    for blk in blocks:
        vals = [0.0] * 32
        for i, v in blk["inputs"]:
            vals[i] = _golden_value(v)
        want = [0] * 32
        for i, c in blk["codes"]:
            want[i] = c
        codes, scales = oracle.mxfp4_quantize(_to_bf16_exact(vals)[None, :])
        assert int(scales[0, 0]) == blk["scale"], blk["note"]
        assert _nibbles(codes)[0].tolist() == want, blk["note"]
        # the dequantised block is the E2M1 grid value times the scale, exactly
        deq = oracle.bf16_to_f32(oracle.mxfp4_dequantize(codes, scales))[0].astype(np.float64)
        for i, c in enumerate(want):
            m = math.ldexp(_E2M1[c & 7], blk["scale"] - 127)
            assert deq[i] == (-m if c & 8 else m) and math.copysign(1, deq[i]) == (-1 if c & 8 else 1)


def test_mxfp4_round_trip_of_representable_blocks():
    """A block whose values are E2M1 values times 2^X, with one magnitude 4 or 6 so that
    floor(log2 max) - 2 = X, quantises to exactly those codes and dequantises to itself."""
    rng = np.random.default_rng(7)
    for trial in range(200):
        X = int(rng.integers(-120, 121))
        codes = rng.integers(0, 16, size=32)
        codes[int(rng.integers(0, 32))] = int(rng.choice([6, 7, 14, 15]))
        vals = np.array([(-1.0 if c & 8 else 1.0) * math.ldexp(_E2M1[c & 7], X) for c in codes])
        q, s = oracle.mxfp4_quantize(_to_bf16_exact(vals)[None, :])
        assert int(s[0, 0]) == X + 127
        assert _nibbles(q)[0].tolist() == codes.tolist()
        back = oracle.mxfp4_dequantize(q, s)[0]
        assert back.tolist() == _to_bf16_exact(vals).tolist()


def test_mxfp4_scale_rule_and_half_step_bound():
    """Random BF16 blocks: scale byte = floor(log2 max|v|) - 2 + 127 (from frexp), and each
    element lands on the grid point nearest v / 2^X (within half the local grid step),
    saturating at 6; the sign of the code is the sign of v."""
    rng = np.random.default_rng(11)
    for std in (0.02, 1.0, 300.0):
        v32 = (rng.standard_normal((64, 128)) * std).astype(np.float32)
        vb = (v32.view(np.uint32) >> 16).astype(np.uint16)  # truncation: exact BF16 inputs
        q, s = oracle.mxfp4_quantize(vb)
        codes = _nibbles(q)
        vals = oracle.bf16_to_f32(vb).astype(np.float64)
        for r in range(vals.shape[0]):
            for b in range(vals.shape[1] // 32):
                blk = vals[r, 32 * b:32 * b + 32]
                _, e = math.frexp(float(np.max(np.abs(blk))))
                X = max(-127, min(127, (e - 1) - 2))
                assert int(s[r, b]) == X + 127
                for i in range(32):
                    c = int(codes[r, 32 * b + i])
                    qv = abs(blk[i]) / 2.0 ** X
                    g = _E2M1[c & 7]
                    assert bool(c & 8) == (math.copysign(1.0, blk[i]) < 0)
                    if qv >= 6.0:
                        assert g == 6.0
                    else:
                        step = 0.5 if qv < 2.0 else (1.0 if qv < 4.0 else 2.0)
                        assert abs(qv - g) <= step / 2, (qv, g)
                        assert all(abs(qv - g) <= abs(qv - o) for o in _E2M1)


def test_mxfp4_sign_symmetry():
    rng = np.random.default_rng(3)
    v32 = (rng.standard_normal((8, 64)) * 0.05).astype(np.float32)
    vb = (v32.view(np.uint32) >> 16).astype(np.uint16)
    q1, s1 = oracle.mxfp4_quantize(vb)
    q2, s2 = oracle.mxfp4_quantize(vb ^ np.uint16(0x8000))
    assert np.array_equal(s1, s2)
    assert np.array_equal(q1 ^ np.uint8(0x88), q2)
