"""GPU parity at Beam's shapes (d 5120, 256 experts in 8 groups, top 4 groups /
top 8, d_ff 2560, ~20 GB of BF16 experts) for the decode batches (T = 1, 32, 128:
every element compared) and the prefill workloads (16384 tokens with near-uniform
routing; 32768 tokens with 16 hot experts): h', z and routing for every token,
the permutation's invariants for the whole batch, and the MoE output on a sample
of tokens (the oracle computes them one by one). All calls go through the C ABI."""
import os
import threading

import numpy as np
import pytest

import oracle
import synth
from tests import parity as P

pytestmark = pytest.mark.gpu

BASE = synth.WORKLOADS["decode1"]
THREADS = max(1, min(16, os.cpu_count() or 1))


class ExpertCache:
    """Host expert weights drawn from the input generator, kept for the session."""

    def __init__(self, wl):
        self.wl, self.store, self.lock = wl, {}, threading.Lock()

    def prefetch(self, experts):
        need = [e for e in sorted(set(int(e) for e in experts)) if e not in self.store]
        if need:
            print(f"[beam] drawing {len(need)} experts on the host", flush=True)
        for e in need:
            self.store[e] = synth.expert_weights(self.wl, e)

    def __call__(self, e):
        with self.lock:
            if e not in self.store:
                self.store[e] = synth.expert_weights(self.wl, e)
            return self.store[e]


@pytest.fixture(scope="module")
def beam_gpu():
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    print("[beam] drawing device weights (20 GB) and creating handles", flush=True)
    d = {}
    d["wpost"], d["wpre"] = sd.norm_weights(BASE)
    W, b = sd.router(BASE)
    wg, wu, wd = sd.experts(BASE)
    d["moe"] = beam.BeamMoE(sd.moe_config(BASE, max_tokens=32768), W, b, wg, wu, wd)
    for key in ("skew32k", "skew32k_half"):
        skew = synth.WORKLOADS[key]
        _, b_skew = sd.router(skew)
        d[key] = beam.BeamMoE(sd.moe_config(skew, max_tokens=32768), W, b_skew, wg, wu, wd)
    del wg, wu, wd
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    yield d
    for key in ("moe", "skew32k", "skew32k_half"):
        d[key].close()


@pytest.fixture(scope="module")
def experts():
    return ExpertCache(BASE)


def host_front(wl, T):
    """Oracle boundary, router and routing for tokens 0..T-1."""
    hh = synth.token_rows(wl, range(T), "h")
    xx = synth.token_rows(wl, range(T), "x")
    h_out, z = oracle.boundary(hh, xx, synth.norm_weight(wl, "post"), synth.norm_weight(wl, "pre"),
                               wl.n, wl.eps)
    logits = oracle.router_threaded(z, synth.router_weight(wl), THREADS)
    ids, w, ggap, egap = oracle.topk(logits, synth.router_bias(wl), wl.G, wl.kg, wl.k, wl.scale)
    return dict(h_out=h_out, z=z, logits=logits, ids=ids, w=w, ggap=ggap, egap=egap)


def gpu_run(d, moe, wl, T, ref_z):
    """The boundary on device inputs, the MoE forward on the oracle's z (identical
    inputs for the stage comparison), and the composed chain (MoE on the GPU's own
    z) for the end-to-end report."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    h, x = sd.tokens(wl, "h", T=T), sd.tokens(wl, "x", T=T)
    h_out, z = beam.beam_sublayer_norm_residual(h, x, d["wpost"], d["wpre"], wl.n, wl.eps)
    out = {"h_out": P.bits(h_out), "z": P.bits(z)}
    del h, x, h_out
    y_chain, rc = moe.forward(z, want_routing=True)
    out["y_chain"] = P.bits(y_chain)
    out["ids_chain"] = rc["ids_out"].cpu().numpy()
    del z, y_chain, rc
    zo = P.to_dev(ref_z)
    y, r = moe.forward(zo, want_routing=True)
    torch.cuda.synchronize()
    out.update({k: v.cpu().numpy() for k, v in r.items()})
    out["y"] = P.bits(y)
    del zo, y, r
    return out


def compare_front(g, ref, wl, what):
    """Boundary outputs, then routing and grouping on identical z."""
    P.assert_bf16_close(g["h_out"], ref["h_out"], f"{what} h'")
    P.assert_bf16_close(g["z"], ref["z"], f"{what} z", two_ulp=g["h_out"] != ref["h_out"])
    rel = P.logit_rel_rows(g["logits_out"], ref["logits"])
    print(f"[parity] {what} logits max row rel-L2 {rel.max():.3e}", flush=True)
    assert rel.max() <= P.LOGIT_REL_MAX
    same, st = P.check_routing(g["ids_out"], g["w_out"], ref["ids"], ref["w"], ref["ggap"],
                               ref["egap"], g["logits_out"], ref["logits"], what)
    P.check_permutation_valid(g["ids_out"], g["perm_out"], g["offsets_out"], wl.E)
    if np.all(same):
        _, o_off, o_perm, _ = oracle.permute(ref["ids"], wl.E)
        assert np.array_equal(g["perm_out"], o_perm)
        assert np.array_equal(g["offsets_out"], o_off)
    return same


def oracle_y(ref, g, rows, same, wl, experts):
    """The oracle's MoE output for tokens `rows` on the oracle's z: with the oracle's own
    routing where the two sides selected the same experts, and with the GPU's routing
    replayed where a near tie flipped the selection (the GPU's y of such a token was
    computed with its own routing, so the experts' arithmetic is still compared)."""
    keep = same[rows][:, None]
    ids = np.where(keep, ref["ids"][rows], g["ids_out"][rows])
    w = np.where(keep, ref["w"][rows], g["w_out"][rows])
    experts.prefetch(ids.ravel())
    y, _ = oracle.moe_experts(ref["z"][rows], ids, w, wl.E, experts, threads=THREADS)
    return y


def report_chain(g, ref, y_ref, rows, what):
    """Composed chain (each side from its own z) on tokens `rows` (y_ref: the oracle's
    output for them): reported; asserted only against gross error, since one-ulp z
    differences legitimately move logits, weights and final roundings downstream. A
    token whose chain routing (from the GPU's own z) selects other experts than the
    oracle's is counted, not compared: its output is a different mixture."""
    keep = np.all(g["ids_chain"][rows] == ref["ids"][rows], axis=1)
    keep &= np.all(g["ids_out"][rows] == ref["ids"][rows], axis=1)  # y_ref used these ids
    ok, st = P.compare_bf16(g["y_chain"][rows][keep], y_ref[keep])
    st["routing_flips_from_own_z"] = int(np.count_nonzero(~keep))
    print(f"[parity] {what} composed chain (own z each side): {st}", flush=True)
    assert st["rel_l2"] < 1e-2


@pytest.mark.parametrize("T", [1, 32, 128])
def test_decode_full(beam_gpu, experts, T):
    wl = BASE.with_tokens(T)
    print(f"[beam] decode T={T}", flush=True)
    ref = host_front(wl, T)
    g = gpu_run(beam_gpu, beam_gpu["moe"], wl, T, ref["z"])
    same = compare_front(g, ref, wl, f"decode T={T}")
    rows = np.arange(T)
    y = oracle_y(ref, g, rows, same, wl, experts)
    n_exp = len(set(ref["ids"].ravel().tolist()))
    print(f"[beam] decode T={T}: {n_exp} distinct experts, {int(np.sum(~same))} replayed",
          flush=True)
    P.assert_bf16_close(g["y"], y, f"decode T={T} y")
    report_chain(g, ref, y, rows, f"decode T={T} y")


def test_sublayer_forward_decode1(beam_gpu):
    """Beam shapes, one token (boundary inside the routing launch, d = 5120): the one-call
    path equals the boundary call followed by the MoE forward bit for bit, over several
    token sets and with h updated in place."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    moe = beam_gpu["moe"]
    E, k = BASE.E, BASE.k
    for s in range(4):
        print(f"[beam] sublayer forward token set {s}", flush=True)
        h, x = sd.tokens(BASE, "h", T=1, token_set=s), sd.tokens(BASE, "x", T=1, token_set=s)
        h_ref, z_ref = beam.beam_sublayer_norm_residual(h, x, beam_gpu["wpost"], beam_gpu["wpre"],
                                                        BASE.n, BASE.eps)
        y_ref = torch.empty_like(h)
        lg_ref = torch.empty((1, E), dtype=torch.float32, device="cuda")
        ids_ref = torch.empty((1, k), dtype=torch.int32, device="cuda")
        beam.beam_moe_forward(moe.handle, z_ref, y_ref, logits_out=lg_ref, ids_out=ids_ref)
        hh = h.clone()
        y = torch.empty_like(h)
        lg = torch.empty_like(lg_ref)
        ids = torch.empty_like(ids_ref)
        _, z = beam.beam_sublayer_forward(moe.handle, hh, x, beam_gpu["wpost"], beam_gpu["wpre"],
                                          BASE.n, BASE.eps, y, h_out=hh, logits_out=lg, ids_out=ids)
        assert torch.equal(hh.view(torch.int16), h_ref.view(torch.int16))
        assert torch.equal(z.view(torch.int16), z_ref.view(torch.int16))
        assert torch.equal(lg.view(torch.int32), lg_ref.view(torch.int32))
        assert torch.equal(ids, ids_ref)
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))


@pytest.mark.parametrize("T", [1, 32, 300])
def test_forward_boundary_beam(beam_gpu, T):
    """Beam shapes (d = 5120: ten waves per row): the MoE forward with the next
    boundary fused into its combine equals the forward then the boundary call, bit
    for bit, with h and z updated in place."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    moe = beam_gpu["moe"]
    wl = BASE.with_tokens(T)
    print(f"[beam] forward+boundary T={T}", flush=True)
    z, h = sd.tokens(wl, "x", T=T), sd.tokens(wl, "h", T=T)
    y_ref = torch.empty_like(z)
    beam.beam_moe_forward(moe.handle, z, y_ref)
    h_ref, z_ref = beam.beam_sublayer_norm_residual(h, y_ref, beam_gpu["wpost"], beam_gpu["wpre"],
                                                    wl.n, wl.eps)
    hh, zz, y = h.clone(), z.clone(), torch.empty_like(z)
    beam.beam_moe_forward_boundary(moe.handle, zz, hh, beam_gpu["wpost"], beam_gpu["wpre"], wl.n,
                                   wl.eps, h_out=hh, z_out=zz, y_out=y)
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    assert torch.equal(hh.view(torch.int16), h_ref.view(torch.int16))
    assert torch.equal(zz.view(torch.int16), z_ref.view(torch.int16))


def sampled_tokens(offsets, perm, k, T, n_rand=32, seed=0):
    """Tokens whose outputs are checked: the first and last 8, n_rand random ones, and one
    row of every row tile of the grouped GEMMs (an expert's rows in the expert-grouped
    order are cut into ceil(rows / 256) equal tiles of a multiple of 64 rows; every tile
    of both GEMMs then has a checked row in every column tile). The row is random within
    the tile, except in an expert's last tile, where it is the last row (the ragged tail)."""
    rng = np.random.default_rng(seed)
    pick = set(range(8)) | set(range(T - 8, T)) | set(rng.choice(T, n_rand, replace=False).tolist())
    tiles = 0
    for e in range(len(offsets) - 1):
        cnt = int(offsets[e + 1] - offsets[e])
        if cnt == 0:
            continue
        mt = -(-cnt // 256)
        per = ((-(-cnt // mt)) + 63) // 64 * 64
        for i in range(mt):
            lo, hi = i * per, min(cnt, (i + 1) * per)
            r = hi - 1 if i == mt - 1 else lo + int(rng.integers(hi - lo))
            pick.add(int(perm[offsets[e] + r]) // k)
            tiles += 1
    return np.array(sorted(pick)), tiles


@pytest.mark.parametrize("name", ["prefill16k", "skew32k", "skew32k_half"])
def test_prefill_sampled(beam_gpu, experts, name):
    wl = synth.WORKLOADS[name]
    T = wl.T
    moe = beam_gpu[name] if wl.hot_experts else beam_gpu["moe"]
    print(f"[beam] {name}: oracle boundary/router/routing for all {T} tokens", flush=True)
    ref = host_front(wl, T)
    print(f"[beam] {name}: GPU run T={T}", flush=True)
    g = gpu_run(beam_gpu, moe, wl, T, ref["z"])
    same = compare_front(g, ref, wl, name)
    counts = np.bincount(g["ids_out"].ravel(), minlength=wl.E)
    hot_share = counts[list(wl.hot_experts)].sum() / counts.sum() if wl.hot_experts else 0.0
    print(f"[beam] {name}: rows per expert min {counts.min()} max {counts.max()}, "
          f"hot share {hot_share:.3f}", flush=True)
    rows, tiles = sampled_tokens(g["offsets_out"], g["perm_out"], wl.k, T)
    print(f"[beam] {name}: {len(rows)} sampled tokens cover {tiles} row tiles, "
          f"{int(np.sum(~same[rows]))} with replayed routing", flush=True)
    y = oracle_y(ref, g, rows, same, wl, experts)
    P.assert_bf16_close(g["y"][rows], y, f"{name} y ({len(rows)} sampled tokens)")
    report_chain(g, ref, y, rows, f"{name} y ({len(rows)} sampled tokens)")


@pytest.mark.parametrize("T", [1, 32, 300])
def test_forward_boundary_beam_oracle(beam_gpu, experts, T):
    """beam_moe_forward_boundary (the step bench.py times by default) against the oracle
    at Beam's shapes: the MoE on the oracle's z with the GPU's routing checked as the
    oracle's top-k of the GPU's logits, then the next boundary (residual = another seeded
    stream) with the oracle's MoE output as its branch. Every element of y, h' and z."""
    import torch
    import sparse_moe_decoder_amd as beam
    wl = BASE.with_tokens(T)
    print(f"[beam] forward+boundary vs oracle T={T}", flush=True)
    ref = host_front(wl, T)
    h_next = synth.token_rows(wl, range(T), "h", token_set=2)
    moe = beam_gpu["moe"]
    zz, hh = P.to_dev(ref["z"]), P.to_dev(h_next)
    y = torch.empty_like(zz)
    lg = torch.empty((T, wl.E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, wl.k), dtype=torch.float32, device="cuda")
    h_out, z_out = beam.beam_moe_forward_boundary(moe.handle, zz, hh, beam_gpu["wpost"],
                                                  beam_gpu["wpre"], wl.n, wl.eps, y_out=y,
                                                  logits_out=lg, ids_out=ids, w_out=w)
    torch.cuda.synchronize()
    g_lg, g_ids, g_w = lg.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
    assert P.logit_rel_rows(g_lg, ref["logits"]).max() <= P.LOGIT_REL_MAX
    o_ids, o_w, _, _ = oracle.topk(g_lg, synth.router_bias(wl), wl.G, wl.kg, wl.k, wl.scale)
    assert np.array_equal(g_ids, o_ids)
    assert np.max(np.abs(g_w.view(np.int32).astype(np.int64) - o_w.view(np.int32))) <= 1
    experts.prefetch(o_ids.ravel())
    o_y, _ = oracle.moe_experts(ref["z"], o_ids, o_w, wl.E, experts, threads=THREADS)
    o_h, o_z = oracle.boundary(h_next, o_y, synth.norm_weight(wl, "post"),
                               synth.norm_weight(wl, "pre"), wl.n, wl.eps)
    g_h = P.bits(h_out)
    P.assert_bf16_close(P.bits(y), o_y, f"fused T={T} y")
    P.assert_bf16_close(g_h, o_h, f"fused T={T} h'")
    P.assert_bf16_close(P.bits(z_out), o_z, f"fused T={T} z", two_ulp=g_h != o_h)


@pytest.mark.parametrize("T", [1, 32, 300])
def test_sublayer_forward_beam_oracle(beam_gpu, experts, T):
    """beam_sublayer_forward at Beam's shapes against the oracle, stage by stage: h' and z
    from the seeded h, x; logits from the GPU's z; ids bit-exact with the oracle's top-k of
    the GPU's logits; y = the oracle's experts on the GPU's z and that routing."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    wl = BASE.with_tokens(T)
    print(f"[beam] sublayer forward vs oracle T={T}", flush=True)
    hh = synth.token_rows(wl, range(T), "h", token_set=3)
    xx = synth.token_rows(wl, range(T), "x", token_set=3)
    o_h, o_z = oracle.boundary(hh, xx, synth.norm_weight(wl, "post"),
                               synth.norm_weight(wl, "pre"), wl.n, wl.eps)
    moe = beam_gpu["moe"]
    y = torch.empty((T, wl.d), dtype=torch.bfloat16, device="cuda")
    lg = torch.empty((T, wl.E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, wl.k), dtype=torch.float32, device="cuda")
    h_out, z = beam.beam_sublayer_forward(moe.handle, P.to_dev(hh), P.to_dev(xx),
                                          beam_gpu["wpost"], beam_gpu["wpre"], wl.n, wl.eps, y,
                                          logits_out=lg, ids_out=ids, w_out=w)
    torch.cuda.synchronize()
    g_h, g_z = P.bits(h_out), P.bits(z)
    P.assert_bf16_close(g_h, o_h, f"one-call T={T} h'")
    P.assert_bf16_close(g_z, o_z, f"one-call T={T} z", two_ulp=g_h != o_h)
    g_lg = lg.cpu().numpy()
    assert P.logit_rel_rows(g_lg, oracle.router_threaded(g_z, synth.router_weight(wl),
                                                         THREADS)).max() <= P.LOGIT_REL_MAX
    o_ids, o_w, _, _ = oracle.topk(g_lg, synth.router_bias(wl), wl.G, wl.kg, wl.k, wl.scale)
    assert np.array_equal(ids.cpu().numpy(), o_ids)
    experts.prefetch(o_ids.ravel())
    o_y, _ = oracle.moe_experts(g_z, o_ids, o_w, wl.E, experts, threads=THREADS)
    P.assert_bf16_close(P.bits(y), o_y, f"one-call T={T} y")


def test_routing_identical_across_batch_paths(beam_gpu, experts):
    """A token's logits, experts and weights are the same bits whether it is routed alone
    (the one-launch small-batch routing), in a batch of 16 (the same launch with 16 tokens)
    or in a batch of 128 (the separate FP32 router and top-k): all three use one dot-product
    order. Its MoE output differs at most by final-rounding flips between the expert paths
    (T <= 16 and 17..128 sum K in different orders), and each matches the oracle."""
    import torch
    wl = BASE.with_tokens(128)
    ref = host_front(wl, 128)
    moe = beam_gpu["moe"]
    z = P.to_dev(ref["z"])
    outs = {}
    for T in (1, 16, 128):
        y, r = moe.forward(z[:T].contiguous(), want_routing=True)
        torch.cuda.synchronize()
        outs[T] = (P.bits(y), {k: v.cpu().numpy() for k, v in r.items()})
    for key in ("logits_out", "ids_out", "w_out"):
        for T in (16, 128):
            assert np.array_equal(outs[T][1][key][:1].view(np.uint32),
                                  outs[1][1][key][:1].view(np.uint32)), (T, key)
        assert np.array_equal(outs[128][1][key][:16].view(np.uint32),
                              outs[16][1][key].view(np.uint32)), key
    experts.prefetch(outs[1][1]["ids_out"].ravel())
    o_y, _ = oracle.moe_experts(ref["z"][:1], outs[1][1]["ids_out"], outs[1][1]["w_out"], wl.E,
                                experts)
    for T in (1, 16, 128):
        P.assert_bf16_close(outs[T][0][:1], o_y, f"token 0 of T={T}")
