"""GPU parity on the tiny sublayer (T 8, d 512, 32 experts in 8 groups of 4, d_ff 256),
every element compared with the CPU oracle, plus routing on fixed logits, replay,
determinism, batch invariance and edge cases. All calls go through the C ABI."""
import numpy as np
import pytest

import oracle
import synth
from tests import parity as P

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS["tiny"]


@pytest.fixture(scope="module")
def gpu():
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    assert torch.cuda.is_available()
    print(f"[tiny] building device inputs {WL}", flush=True)
    d = dict(h=sd.tokens(WL, "h"), x=sd.tokens(WL, "x"))
    d["wpost"], d["wpre"] = sd.norm_weights(WL)
    d["W"], d["b"] = sd.router(WL)
    d["wg"], d["wu"], d["wd"] = sd.experts(WL)
    d["moe"] = beam.BeamMoE(sd.moe_config(WL, max_tokens=64), d["W"], d["b"], d["wg"], d["wu"],
                            d["wd"])
    torch.cuda.synchronize()
    yield d
    d["moe"].close()


@pytest.fixture(scope="module")
def host():
    hh = synth.token_rows(WL, range(WL.T), "h")
    xx = synth.token_rows(WL, range(WL.T), "x")
    experts = {e: synth.expert_weights(WL, e) for e in range(WL.E)}
    ref = oracle.sublayer(hh, xx, synth.norm_weight(WL, "post"), synth.norm_weight(WL, "pre"),
                          WL.n, WL.eps, synth.router_weight(WL), synth.router_bias(WL), WL.G,
                          WL.kg, WL.k, WL.scale, experts.__getitem__)
    ref["h"], ref["x"], ref["experts"] = hh, xx, experts
    return ref


def test_device_generator_matches_host(gpu):
    """The device input generator draws the same bits as the host one."""
    assert np.array_equal(P.bits(gpu["h"]), synth.token_rows(WL, range(WL.T), "h"))
    assert np.array_equal(P.bits(gpu["x"]), synth.token_rows(WL, range(WL.T), "x"))
    assert np.array_equal(P.bits(gpu["wpost"]), synth.norm_weight(WL, "post"))
    assert np.array_equal(P.bits(gpu["wpre"]), synth.norm_weight(WL, "pre"))
    assert np.array_equal(gpu["W"].cpu().numpy(), synth.router_weight(WL))
    assert np.array_equal(gpu["b"].cpu().numpy(), synth.router_bias(WL))
    for e in (0, 7, WL.E - 1):
        wg, wu, wd = synth.expert_weights(WL, e)
        assert np.array_equal(P.bits(gpu["wg"][e]), wg)
        assert np.array_equal(P.bits(gpu["wu"][e]), wu)
        assert np.array_equal(P.bits(gpu["wd"][e]), wd)


def test_boundary(gpu, host):
    import sparse_moe_decoder_amd as beam
    h_out, z = beam.beam_sublayer_norm_residual(gpu["h"], gpu["x"], gpu["wpost"], gpu["wpre"],
                                                WL.n, WL.eps)
    P.assert_bf16_close(P.bits(h_out), host["h_out"], "tiny h'")
    P.assert_bf16_close(P.bits(z), host["z"], "tiny z")


def test_boundary_in_place_and_n1(gpu):
    """h_out may alias h; n = 1 makes h' the post-normed branch (oracle closed form)."""
    import sparse_moe_decoder_amd as beam
    h = gpu["h"].clone()
    _, z1 = beam.beam_sublayer_norm_residual(gpu["h"], gpu["x"], gpu["wpost"], gpu["wpre"], 20,
                                            1e-6)
    h_ref = P.bits(beam.beam_sublayer_norm_residual(gpu["h"], gpu["x"], gpu["wpost"],
                                                    gpu["wpre"], 20, 1e-6)[0])
    _, z2 = beam.beam_sublayer_norm_residual(h, gpu["x"], gpu["wpost"], gpu["wpre"], 20, 1e-6,
                                            h_out=h)
    assert np.array_equal(P.bits(h), h_ref)
    assert np.array_equal(P.bits(z1), P.bits(z2))
    hn1, _ = beam.beam_sublayer_norm_residual(gpu["h"], gpu["x"], gpu["wpost"], gpu["wpre"], 1,
                                              1e-6)
    o_h, _ = oracle.boundary(P.bits(gpu["h"]), P.bits(gpu["x"]), P.bits(gpu["wpost"]),
                             P.bits(gpu["wpre"]), 1, 1e-6)
    P.assert_bf16_close(P.bits(hn1), o_h, "tiny h' at n=1")


def test_router_logits_and_routing(gpu, host):
    z = P.to_dev(host["z"])
    logits, ids, w = gpu["moe"].router_topk(z)
    lg = logits.cpu().numpy()
    rel = P.logit_rel_rows(lg, host["logits"])
    print(f"[parity] tiny logits max row rel-L2 {rel.max():.3e}", flush=True)
    assert rel.max() <= P.LOGIT_REL_MAX
    P.check_routing(ids.cpu().numpy(), w.cpu().numpy(), host["ids"], host["w"], host["ggap"],
                    host["egap"], lg, host["logits"], "tiny")


@pytest.mark.parametrize("kind", ["normal", "ties", "wide"])
def test_routing_bit_exact_on_identical_logits(gpu, kind):
    """Same FP32 logits on both sides -> expert ids bit-exact, weights bit-exact."""
    import torch
    T = 64
    lg = synth.synthetic_logits(WL, T, seed=3, std=1.0 if kind != "wide" else 6.0)
    if kind == "ties":
        lg = (np.round(lg * 2) / 2).astype(np.float32)  # many exact ties
    bias = synth.router_bias(WL)
    o_ids, o_w, _, _ = oracle.topk(lg, bias, WL.G, WL.kg, WL.k, WL.scale)
    ids, w = gpu["moe"].grouped_topk(torch.from_numpy(lg).cuda())
    assert np.array_equal(ids.cpu().numpy(), o_ids)
    ulps = np.abs(w.cpu().numpy().view(np.int32).astype(np.int64) - o_w.view(np.int32))
    print(f"[parity] tiny routing on identical logits ({kind}): max weight ulps {ulps.max()}",
          flush=True)
    assert ulps.max() <= 1 and np.mean(ulps == 0) > 0.999


def test_forward_matches_oracle(gpu, host):
    z = P.to_dev(host["z"])
    y, r = gpu["moe"].forward(z, want_routing=True)
    g_ids = r["ids_out"].cpu().numpy()
    same, _ = P.check_routing(g_ids, r["w_out"].cpu().numpy(), host["ids"], host["w"],
                              host["ggap"], host["egap"], r["logits_out"].cpu().numpy(),
                              host["logits"], "tiny forward")
    perm, offs = r["perm_out"].cpu().numpy(), r["offsets_out"].cpu().numpy()
    P.check_permutation_valid(g_ids, perm, offs, WL.E)
    if np.all(same):
        _, o_off, o_perm, _ = oracle.permute(host["ids"], WL.E)
        assert np.array_equal(perm, o_perm) and np.array_equal(offs, o_off)
    P.assert_bf16_close(P.bits(y)[same], host["y"][same], "tiny y")


def test_replay_matches_oracle(gpu, host):
    """Caller-supplied routing (replay): permutation bit-exact, output vs oracle."""
    import torch
    z = P.to_dev(host["z"])
    ids = torch.from_numpy(host["ids"]).cuda()
    w = torch.from_numpy(host["w"]).cuda()
    y, r = gpu["moe"].forward(z, ids_in=ids, w_in=w, want_routing=True)
    _, o_off, o_perm, _ = oracle.permute(host["ids"], WL.E)
    assert np.array_equal(r["perm_out"].cpu().numpy(), o_perm)
    assert np.array_equal(r["offsets_out"].cpu().numpy(), o_off)
    assert np.array_equal(r["ids_out"].cpu().numpy(), host["ids"])
    P.assert_bf16_close(P.bits(y), host["y"], "tiny y (replay)")


def test_replay_invalid_and_all_experts(gpu, host):
    """Invalid ids contribute nothing; a token may use every expert (k = E style)."""
    import torch
    z = P.to_dev(host["z"])
    ids = host["ids"].copy()
    ids[0, 3] = -1
    ids[2, 0] = WL.E + 5
    w = host["w"].copy()
    y, r = gpu["moe"].forward(z, ids_in=torch.from_numpy(ids).cuda(),
                              w_in=torch.from_numpy(w).cuda(), want_routing=True)
    o_y, _ = oracle.moe_experts(host["z"], ids, w, WL.E, host["experts"].__getitem__)
    P.assert_bf16_close(P.bits(y), o_y, "tiny y (replay, invalid slots)")
    P.check_permutation_valid(ids, r["perm_out"].cpu().numpy(), r["offsets_out"].cpu().numpy(),
                              WL.E)


def test_replay_one_token_repeated_expert(gpu, host):
    """One token whose replayed routing names one expert three times (and has an invalid
    slot): that expert holds three rows of the same token, each slot scaled by its own
    weight, as the oracle's per-slot experts give."""
    import torch
    z1 = host["z"][:1].copy()
    ids = host["ids"][:1].copy()
    ids[0, 1] = ids[0, 0]
    ids[0, 5] = ids[0, 0]
    ids[0, 3] = -1
    w = host["w"][:1].copy()
    y, r = gpu["moe"].forward(P.to_dev(z1), ids_in=torch.from_numpy(ids).cuda(),
                              w_in=torch.from_numpy(w).cuda(), want_routing=True)
    o_y, _ = oracle.moe_experts(z1, ids, w, WL.E, host["experts"].__getitem__)
    P.assert_bf16_close(P.bits(y), o_y, "tiny y (one token, repeated expert)")
    P.check_permutation_valid(ids, r["perm_out"].cpu().numpy(), r["offsets_out"].cpu().numpy(),
                              WL.E)


def test_deterministic(gpu, host):
    z = P.to_dev(host["z"])
    a = P.bits(gpu["moe"].forward(z))
    b = P.bits(gpu["moe"].forward(z))
    assert np.array_equal(a, b)


def test_batch_invariance(gpu, host):
    """A token's routing and output do not depend on the other tokens in the batch."""
    z = P.to_dev(host["z"])
    full = P.bits(gpu["moe"].forward(z))
    for t in (0, 5):
        one = P.bits(gpu["moe"].forward(z[t:t + 1].contiguous()))
        assert np.array_equal(one[0], full[t])


def test_single_token_paths_agree(gpu, host):
    """One token alone equals the same token inside a batch (routing replayed, so
    both see the same ids and weights), over repeated calls; the grouping tables
    of a single-token call are valid."""
    import torch
    import sparse_moe_decoder_amd as beam
    moe = gpu["moe"]
    z = P.to_dev(host["z"])
    T = z.shape[0]
    _, ids, w = moe.router_topk(z, want_logits=False)
    full = P.bits(moe.forward(z, ids_in=ids, w_in=w))
    for rep in range(3):
        for t in range(T):
            one = P.bits(moe.forward(z[t:t + 1].contiguous(), ids_in=ids[t:t + 1].contiguous(),
                                     w_in=w[t:t + 1].contiguous()))
            assert np.array_equal(one[0], full[t]), (rep, t)
    k = ids.shape[1]
    y1 = torch.empty((1, z.shape[1]), dtype=torch.bfloat16, device="cuda")
    perm = torch.full((k,), -7, dtype=torch.int32, device="cuda")
    offs = torch.full((WL.E + 1,), -7, dtype=torch.int32, device="cuda")
    beam.beam_moe_forward(moe.handle, z[:1].contiguous(), y1, perm_out=perm, offsets_out=offs)
    P.check_permutation_valid(ids[:1].cpu().numpy(), perm.cpu().numpy(), offs.cpu().numpy(), WL.E)


def _two_calls(moe, h, x, wpost, wpre, n, eps):
    """The reference sequence: boundary, then the MoE forward on its z."""
    import torch
    import sparse_moe_decoder_amd as beam
    T, d = h.shape
    E, k = moe.cfg["n_experts"], moe.cfg["topk"]
    h_out, z = beam.beam_sublayer_norm_residual(h, x, wpost, wpre, n, eps)
    y = torch.empty_like(z)
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    beam.beam_moe_forward(moe.handle, z, y, logits_out=lg, ids_out=ids, w_out=w)
    return [P.bits(h_out), P.bits(z), P.bits(y), lg.cpu().numpy(), ids.cpu().numpy(),
            w.cpu().numpy()]


def _one_call(moe, h, x, wpost, wpre, n, eps, in_place=False):
    import torch
    import sparse_moe_decoder_amd as beam
    T, d = h.shape
    E, k = moe.cfg["n_experts"], moe.cfg["topk"]
    y = torch.empty_like(h)
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    hh = h.clone() if in_place else h
    h_out, z = beam.beam_sublayer_forward(moe.handle, hh, x, wpost, wpre, n, eps, y,
                                          h_out=hh if in_place else None, logits_out=lg,
                                          ids_out=ids, w_out=w)
    return [P.bits(h_out), P.bits(z), P.bits(y), lg.cpu().numpy(), ids.cpu().numpy(),
            w.cpu().numpy()]


@pytest.mark.parametrize("T", [1, 3, 8])
@pytest.mark.parametrize("in_place", [False, True])
def test_sublayer_forward_equals_two_calls(gpu, T, in_place):
    """beam_sublayer_forward (boundary inside the routing launch at T = 1) gives the
    same h', z, y, logits, ids and weights bit for bit as the boundary call followed
    by the MoE forward; h_out may be h itself. Repeated, so the launch's counter
    reset is exercised."""
    print(f"[tiny] sublayer forward T={T} in_place={in_place}", flush=True)
    h, x = gpu["h"][:T].contiguous(), gpu["x"][:T].contiguous()
    ref = _two_calls(gpu["moe"], h, x, gpu["wpost"], gpu["wpre"], WL.n, WL.eps)
    names = ["h'", "z", "y", "logits", "ids", "w"]
    for rep in range(3):
        got = _one_call(gpu["moe"], h, x, gpu["wpost"], gpu["wpre"], WL.n, WL.eps, in_place)
        for nm, a, b in zip(names, got, ref):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (nm, rep)


def test_sublayer_forward_matches_oracle(gpu, host):
    """Single token through the one-call path against the oracle's sublayer."""
    got = _one_call(gpu["moe"], gpu["h"][:1].contiguous(), gpu["x"][:1].contiguous(),
                    gpu["wpost"], gpu["wpre"], WL.n, WL.eps)
    P.assert_bf16_close(got[0], host["h_out"][:1], "tiny h' (one call)")
    P.assert_bf16_close(got[1], host["z"][:1], "tiny z (one call)")
    rel = P.logit_rel_rows(got[3], host["logits"][:1])
    assert rel.max() <= P.LOGIT_REL_MAX
    o_ids, o_w, _, _ = oracle.topk(got[3], synth.router_bias(WL), WL.G, WL.kg, WL.k, WL.scale)
    assert np.array_equal(got[4], o_ids)
    o_y, _ = oracle.moe_experts(got[1], o_ids, o_w, WL.E, host["experts"].__getitem__)
    P.assert_bf16_close(got[2], o_y, "tiny y (one call)")


def _forward_then_boundary(moe, z, h, wpost, wpre, n, eps, ids_in=None, w_in=None):
    """Reference sequence: the MoE forward, then the boundary with its output as x."""
    import torch
    import sparse_moe_decoder_amd as beam
    T = z.shape[0]
    E, k = moe.cfg["n_experts"], moe.cfg["topk"]
    y = torch.empty_like(z)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lg = None if ids_in is not None else torch.empty((T, E), dtype=torch.float32, device="cuda")
    beam.beam_moe_forward(moe.handle, z, y, ids_in=ids_in, w_in=w_in, logits_out=lg, ids_out=ids,
                          w_out=w)
    h_out, z_out = beam.beam_sublayer_norm_residual(h, y, wpost, wpre, n, eps)
    out = dict(h=P.bits(h_out), z=P.bits(z_out), y=P.bits(y), ids=ids.cpu().numpy(),
               w=w.cpu().numpy())
    if lg is not None:
        out["logits"] = lg.cpu().numpy()
    return out


def _forward_boundary(moe, z, h, wpost, wpre, n, eps, ids_in=None, w_in=None, want_y=True,
                      h_in_place=False, z_in_place=False):
    import torch
    import sparse_moe_decoder_amd as beam
    T = z.shape[0]
    E, k = moe.cfg["n_experts"], moe.cfg["topk"]
    zz = z.clone() if z_in_place else z
    hh = h.clone() if h_in_place else h
    y = torch.empty_like(z) if want_y else None
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lg = None if ids_in is not None else torch.empty((T, E), dtype=torch.float32, device="cuda")
    h_out, z_out = beam.beam_moe_forward_boundary(
        moe.handle, zz, hh, wpost, wpre, n, eps, h_out=hh if h_in_place else None,
        z_out=zz if z_in_place else None, y_out=y, ids_in=ids_in, w_in=w_in, logits_out=lg,
        ids_out=ids, w_out=w)
    out = dict(h=P.bits(h_out), z=P.bits(z_out), ids=ids.cpu().numpy(), w=w.cpu().numpy())
    if want_y:
        out["y"] = P.bits(y)
    if lg is not None:
        out["logits"] = lg.cpu().numpy()
    return out


def _same(a, b, what):
    for key, v in a.items():
        assert np.array_equal(v.view(np.uint8), b[key].view(np.uint8)), (what, key)


@pytest.mark.parametrize("T", [1, 8, 40])
@pytest.mark.parametrize("replay", [False, True])
def test_forward_boundary_equals_two_calls(gpu, host, T, replay):
    """The MoE forward with the next boundary fused into its combine equals the
    forward followed by the boundary call, bit for bit: h', z, y, routing; with
    h_out = h, z_out = z and without y_out as well."""
    import torch
    print(f"[tiny] forward+boundary T={T} replay={replay}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(T)
    z = torch.randn((T, WL.d), generator=g).to(torch.bfloat16).cuda()
    h = torch.randn((T, WL.d), generator=g).to(torch.bfloat16).cuda()
    ids_in = w_in = None
    if replay:
        _, ids_in, w_in = gpu["moe"].router_topk(z, want_logits=False)
        ids_in[0, 0] = WL.E + 3  # an invalid id contributes nothing, on both sides
    ref = _forward_then_boundary(gpu["moe"], z, h, gpu["wpost"], gpu["wpre"], WL.n, WL.eps,
                                 ids_in, w_in)
    for kw in (dict(), dict(want_y=False), dict(h_in_place=True, z_in_place=True)):
        got = _forward_boundary(gpu["moe"], z, h, gpu["wpost"], gpu["wpre"], WL.n, WL.eps,
                                ids_in, w_in, **kw)
        _same(got, ref, f"T={T} {kw}")


def test_forward_boundary_wide_rows():
    """Rows wider than one workgroup's chunks (d = 8448): the combine goes through
    y_out and the wave-per-row boundary; the same bits as the two calls. Without
    y_out such a width is rejected."""
    import sparse_moe_decoder_amd as beam
    from synth import Workload
    from synth import device as sd
    wl = Workload("wide", T=3, d=8448, E=16, G=4, kg=2, k=4, f=256)
    print(f"[tiny] wide rows {wl}", flush=True)
    W, b = sd.router(wl)
    wg, wu, wd = sd.experts(wl)
    wpost, wpre = sd.norm_weights(wl)
    moe = beam.BeamMoE(sd.moe_config(wl, max_tokens=8), W, b, wg, wu, wd)
    try:
        z = sd.tokens(wl, "x")
        h = sd.tokens(wl, "h")
        ref = _forward_then_boundary(moe, z, h, wpost, wpre, wl.n, wl.eps)
        got = _forward_boundary(moe, z, h, wpost, wpre, wl.n, wl.eps)
        _same(got, ref, "wide")
        with pytest.raises(beam.BeamError) as ei:
            _forward_boundary(moe, z, h, wpost, wpre, wl.n, wl.eps, want_y=False)
        assert ei.value.status == -2
    finally:
        moe.close()


def test_single_token_routing_ties():
    """One token through the one-launch routing with
    exact ties: experts 2i and 2i+1 share their router row and bias, so their scores
    are equal bit for bit and the lower index must come first. Ids exact and weights
    within one ulp of the oracle's top-k on the GPU's own logits, over several tokens."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    wl = WL
    W, b = sd.router(wl)
    W = W.clone()
    b = b.clone()
    W[1::2] = W[0::2]
    b[1::2] = b[0::2]
    wg, wu, wd = sd.experts(wl)
    moe = beam.BeamMoE(sd.moe_config(wl, max_tokens=4), W, b, wg, wu, wd)
    try:
        bias = b.cpu().numpy()
        for t in range(6):
            z = (torch.randn((1, wl.d), generator=torch.Generator().manual_seed(100 + t))
                 .to(torch.bfloat16).cuda())
            _, r = moe.forward(z, want_routing=True)
            lg = r["logits_out"].cpu().numpy()
            assert np.array_equal(lg[:, 0::2].view(np.uint32), lg[:, 1::2].view(np.uint32))
            o_ids, o_w, _, _ = oracle.topk(lg, bias, wl.G, wl.kg, wl.k, wl.scale)
            assert np.array_equal(r["ids_out"].cpu().numpy(), o_ids), t
            ulps = np.abs(r["w_out"].cpu().numpy().view(np.int32).astype(np.int64) - o_w.view(np.int32))
            assert ulps.max() <= 1
    finally:
        moe.close()


def test_edge_sizes(gpu, host):
    """T = 0 is a no-op; T = max_tokens works; T > max_tokens is rejected up front."""
    import torch
    import sparse_moe_decoder_amd as beam
    moe = gpu["moe"]
    z0 = torch.empty((0, WL.d), dtype=torch.bfloat16, device="cuda")
    y0 = torch.empty_like(z0)
    beam.beam_moe_forward(moe.handle, z0, y0)
    zmax = torch.randn((64, WL.d), device="cuda").to(torch.bfloat16)
    ymax = moe.forward(zmax)
    assert torch.isfinite(ymax.float()).all()
    with pytest.raises(beam.BeamError) as ei:
        moe.forward(torch.zeros((65, WL.d), dtype=torch.bfloat16, device="cuda"))
    assert ei.value.status == -5
    # the 64-token batch matches the oracle on its first rows
    zb = P.bits(zmax)
    ref = oracle.router(zb[:4], synth.router_weight(WL))
    ids, w, _, _ = oracle.topk(ref, synth.router_bias(WL), WL.G, WL.kg, WL.k, WL.scale)
    o_y, _ = oracle.moe_experts(zb[:4], ids, w, WL.E, host["experts"].__getitem__)
    P.assert_bf16_close(P.bits(ymax)[:4], o_y, "tiny y at T = max_tokens (first rows)")


def test_prefill_path_ragged_tiles():
    """T above the weight-streaming range takes the grouped-GEMM path: expert row
    counts that span several 128-row tiles and ragged tails, checked in full."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    T = 1536
    wl = WL.with_tokens(T)
    h, x = sd.tokens(wl, "h"), sd.tokens(wl, "x")
    wpost, wpre = sd.norm_weights(wl)
    W, b = sd.router(wl)
    wg, wu, wd = sd.experts(wl)
    moe = beam.BeamMoE(sd.moe_config(wl, max_tokens=T), W, b, wg, wu, wd)
    try:
        _, z = beam.beam_sublayer_norm_residual(h, x, wpost, wpre, wl.n, wl.eps)
        y = moe.forward(z)
        torch.cuda.synchronize()
        hh = synth.token_rows(wl, range(T), "h")
        xx = synth.token_rows(wl, range(T), "x")
        experts = {e: synth.expert_weights(wl, e) for e in range(wl.E)}
        ref = oracle.sublayer(hh, xx, synth.norm_weight(wl, "post"), synth.norm_weight(wl, "pre"),
                              wl.n, wl.eps, synth.router_weight(wl), synth.router_bias(wl), wl.G,
                              wl.kg, wl.k, wl.scale, experts.__getitem__, threads=8)
        P.assert_bf16_close(P.bits(z), ref["z"], "tiny@1536 z")
        y_chain = P.bits(y)
        # the MoE stage on identical inputs (the oracle's z)
        y, r = moe.forward(P.to_dev(ref["z"]), want_routing=True)
        rel = P.logit_rel_rows(r["logits_out"].cpu().numpy(), ref["logits"])
        print(f"[parity] tiny@1536 logits max row rel-L2 {rel.max():.3e}", flush=True)
        assert rel.max() <= P.LOGIT_REL_MAX
        g_ids = r["ids_out"].cpu().numpy()
        counts = np.bincount(g_ids.ravel(), minlength=wl.E)
        print(f"[parity] tiny@1536 rows per expert: min {counts.min()} max {counts.max()}",
              flush=True)
        assert counts.min() > 256  # every expert spans two 256-row tiles, ragged tails
        same, _ = P.check_routing(g_ids, r["w_out"].cpu().numpy(), ref["ids"], ref["w"],
                                  ref["ggap"], ref["egap"], r["logits_out"].cpu().numpy(),
                                  ref["logits"], "tiny@1536")
        P.check_permutation_valid(g_ids, r["perm_out"].cpu().numpy(),
                                  r["offsets_out"].cpu().numpy(), wl.E)
        P.assert_bf16_close(P.bits(y)[same], ref["y"][same], "tiny@1536 y")
        ok, st = P.compare_bf16(y_chain[same], ref["y"][same])
        print(f"[parity] tiny@1536 y composed chain (own z each side): {st}", flush=True)
        assert st["rel_l2"] < 1e-2
        # replay with the oracle's routing on the oracle's z: the expert path alone
        y2 = moe.forward(P.to_dev(ref["z"]), ids_in=torch.from_numpy(ref["ids"]).cuda(),
                         w_in=torch.from_numpy(ref["w"]).cuda())
        P.assert_bf16_close(P.bits(y2), ref["y"], "tiny@1536 y (replay)")
    finally:
        moe.close()


def _front(T, token_set=0):
    """Oracle boundary of seeded tokens 0..T-1: (h, x, h', z) as BF16 bits."""
    hh = synth.token_rows(WL, range(T), "h", token_set=token_set)
    xx = synth.token_rows(WL, range(T), "x", token_set=token_set)
    h_out, z = oracle.boundary(hh, xx, synth.norm_weight(WL, "post"), synth.norm_weight(WL, "pre"),
                               WL.n, WL.eps)
    return hh, xx, h_out, z


@pytest.mark.parametrize("T", [1, 8, 40])
@pytest.mark.parametrize("replay", [False, True])
def test_forward_boundary_matches_oracle(gpu, host, T, replay):
    """beam_moe_forward_boundary against the oracle: the MoE on z (routing from the GPU's
    logits must be the oracle's top-k of those logits, bit for bit; replayed routing with an
    invalid slot contributes nothing), then the next boundary with the MoE output as its
    branch: oracle.moe_experts followed by oracle.boundary on the same inputs."""
    import torch
    print(f"[tiny] forward+boundary vs oracle T={T} replay={replay}", flush=True)
    _, _, h_next, z = _front(T)          # z: the MoE input; h_next: the residual stream
    ids_in = w_in = None
    if replay:
        ids, w, _, _ = oracle.topk(oracle.router(z, synth.router_weight(WL)),
                                   synth.router_bias(WL), WL.G, WL.kg, WL.k, WL.scale)
        ids[T // 2, 1] = -1
        ids_in, w_in = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    got = _forward_boundary(gpu["moe"], P.to_dev(z), P.to_dev(h_next), gpu["wpost"], gpu["wpre"],
                            WL.n, WL.eps, ids_in, w_in)
    if replay:
        o_ids, o_w = ids, w
        assert np.array_equal(got["ids"], o_ids)
    else:
        rel = P.logit_rel_rows(got["logits"], oracle.router(z, synth.router_weight(WL)))
        assert rel.max() <= P.LOGIT_REL_MAX
        o_ids, o_w, _, _ = oracle.topk(got["logits"], synth.router_bias(WL), WL.G, WL.kg, WL.k,
                                       WL.scale)
        assert np.array_equal(got["ids"], o_ids)
        assert np.max(np.abs(got["w"].view(np.int32).astype(np.int64) - o_w.view(np.int32))) <= 1
    o_y, _ = oracle.moe_experts(z, o_ids, o_w, WL.E, host["experts"].__getitem__)
    o_h, o_z = oracle.boundary(h_next, o_y, synth.norm_weight(WL, "post"),
                               synth.norm_weight(WL, "pre"), WL.n, WL.eps)
    P.assert_bf16_close(got["y"], o_y, f"tiny fused y T={T}")
    P.assert_bf16_close(got["h"], o_h, f"tiny fused h' T={T}")
    P.assert_bf16_close(got["z"], o_z, f"tiny fused z T={T}", two_ulp=got["h"] != o_h)


@pytest.mark.parametrize("T", [1, 8, 40])
def test_sublayer_forward_stages_match_oracle(gpu, host, T):
    """beam_sublayer_forward against the oracle stage by stage: h' and z from the seeded
    h, x; logits from the GPU's z; ids = the oracle's top-k of the GPU's logits (bit-exact);
    y = the oracle's experts on the GPU's z and routing."""
    print(f"[tiny] sublayer forward vs oracle T={T}", flush=True)
    hh, xx, o_h, o_z = _front(T, token_set=1)
    got = _one_call(gpu["moe"], P.to_dev(hh), P.to_dev(xx), gpu["wpost"], gpu["wpre"], WL.n,
                    WL.eps)
    g_h, g_z, g_y, g_lg, g_ids, g_w = got
    P.assert_bf16_close(g_h, o_h, f"tiny one-call h' T={T}")
    P.assert_bf16_close(g_z, o_z, f"tiny one-call z T={T}", two_ulp=g_h != o_h)
    rel = P.logit_rel_rows(g_lg, oracle.router(g_z, synth.router_weight(WL)))
    assert rel.max() <= P.LOGIT_REL_MAX
    o_ids, o_w, _, _ = oracle.topk(g_lg, synth.router_bias(WL), WL.G, WL.kg, WL.k, WL.scale)
    assert np.array_equal(g_ids, o_ids)
    o_y, _ = oracle.moe_experts(g_z, o_ids, o_w, WL.E, host["experts"].__getitem__)
    P.assert_bf16_close(g_y, o_y, f"tiny one-call y T={T}")


def test_boundary_closed_forms_bit_exact(gpu):
    """Rows whose norm factors are exact (eps = 0): branch rows of small odd integers with
    mean square 16 (factor 1/4, so the post-norm output x w / 4 is exact before its BF16
    rounding) and constant rows. Every sum of squares is exact in any order, so the GPU's
    h' must equal the closed form bf16(c2 * bf16(x w / 4)) bit for bit (h = 0, n = 20), and
    a constant branch row c gives sign(c) * w_post / 2 at n = 4."""
    import sparse_moe_decoder_amd as beam
    from tests.test_oracle_pins import power_of_four_rows, to_bf16
    d = WL.d
    x = np.concatenate([power_of_four_rows(6, 41 + j) for j in range(d // 64)], axis=1)
    rng = np.random.default_rng(44)
    w_post = to_bf16(rng.uniform(0.9, 1.1, d))
    ones = to_bf16(np.ones(d))
    c2 = np.float32(1.0 / np.sqrt(20.0))
    want = P.F(to_bf16(c2 * P.F(to_bf16((P.F(x) * np.float32(0.25)) * P.F(w_post)))))
    zero = np.zeros_like(x)
    hp, _ = beam.beam_sublayer_norm_residual(P.to_dev(zero), P.to_dev(x), P.to_dev(w_post),
                                             P.to_dev(ones), 20, 0.0)
    assert np.array_equal(P.F(P.bits(hp)), want)
    o_h, _ = oracle.boundary(zero, x, w_post, ones, 20, 0.0)
    assert np.array_equal(P.bits(hp), o_h)
    for c in (1.5, -3.0):
        xc = np.full((2, d), to_bf16(np.float32(c)), np.uint16)
        hp, _ = beam.beam_sublayer_norm_residual(P.to_dev(np.zeros_like(xc)), P.to_dev(xc),
                                                 P.to_dev(w_post), P.to_dev(ones), 4, 0.0)
        want_c = np.float32(0.5 * np.sign(c)) * P.F(w_post)
        assert np.array_equal(P.F(P.bits(hp)), np.broadcast_to(want_c, (2, d)))
