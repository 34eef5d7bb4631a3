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
    skew = synth.WORKLOADS["skew32k"]
    _, b_skew = sd.router(skew)
    d["moe_skew"] = beam.BeamMoE(sd.moe_config(skew, max_tokens=32768), W, b_skew, wg, wu, wd)
    del wg, wu, wd
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    yield d
    d["moe"].close()
    d["moe_skew"].close()


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
    y_chain = moe.forward(z)
    out["y_chain"] = P.bits(y_chain)
    del z, y_chain
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


def report_chain(g_chain, y_ref, what):
    """Composed chain (each side from its own z): reported; asserted only against
    gross error, since one-ulp z differences legitimately move logits, weights and
    final roundings downstream."""
    ok, st = P.compare_bf16(g_chain, y_ref)
    print(f"[parity] {what} composed chain (own z each side): {st}", flush=True)
    assert st["rel_l2"] < 1e-2


@pytest.mark.parametrize("T", [1, 32, 128])
def test_decode_full(beam_gpu, experts, T):
    wl = BASE.with_tokens(T)
    print(f"[beam] decode T={T}", flush=True)
    ref = host_front(wl, T)
    g = gpu_run(beam_gpu, beam_gpu["moe"], wl, T, ref["z"])
    same = compare_front(g, ref, wl, f"decode T={T}")
    experts.prefetch(ref["ids"].ravel())
    y, _ = oracle.moe_experts(ref["z"], ref["ids"], ref["w"], wl.E, experts, threads=THREADS)
    n_exp = len(set(ref["ids"].ravel().tolist()))
    print(f"[beam] decode T={T}: {n_exp} distinct experts", flush=True)
    P.assert_bf16_close(g["y"][same], y[same], f"decode T={T} y")
    report_chain(g["y_chain"][same], y[same], f"decode T={T} y")


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


def sampled_tokens(ids, T, hot=(), n_rand=32, seed=0):
    rng = np.random.default_rng(seed)
    pick = set(range(8)) | set(range(T - 8, T)) | set(rng.choice(T, n_rand, replace=False).tolist())
    for e in hot:  # at least one token routed to each hot expert
        rows = np.nonzero(np.any(ids == e, axis=1))[0]
        if len(rows):
            pick.add(int(rows[0]))
    return np.array(sorted(pick))


@pytest.mark.parametrize("name", ["prefill16k", "skew32k"])
def test_prefill_sampled(beam_gpu, experts, name):
    wl = synth.WORKLOADS[name]
    T = wl.T
    moe = beam_gpu["moe_skew"] if wl.hot_experts else beam_gpu["moe"]
    print(f"[beam] {name}: oracle boundary/router/routing for all {T} tokens", flush=True)
    ref = host_front(wl, T)
    print(f"[beam] {name}: GPU run T={T}", flush=True)
    g = gpu_run(beam_gpu, moe, wl, T, ref["z"])
    same = compare_front(g, ref, wl, name)
    counts = np.bincount(g["ids_out"].ravel(), minlength=wl.E)
    hot_share = counts[list(wl.hot_experts)].sum() / counts.sum() if wl.hot_experts else 0.0
    print(f"[beam] {name}: rows per expert min {counts.min()} max {counts.max()}, "
          f"hot share {hot_share:.3f}", flush=True)
    rows = sampled_tokens(ref["ids"], T, wl.hot_experts)
    rows = rows[same[rows]]
    experts.prefetch(ref["ids"][rows].ravel())
    y, _ = oracle.moe_experts(ref["z"][rows], ref["ids"][rows], ref["w"][rows], wl.E, experts,
                              threads=THREADS)
    P.assert_bf16_close(g["y"][rows], y, f"{name} y ({len(rows)} sampled tokens)")
    report_chain(g["y_chain"][rows], y, f"{name} y ({len(rows)} sampled tokens)")
