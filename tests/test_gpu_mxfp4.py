"""GPU parity of the 4-bit (MXFP4) expert path, every call through the C ABI:

- the GPU quantiser against the oracle's codes and scales, bit for bit, on seeded
  normals at many magnitudes and on every rounding decision point with its BF16
  neighbours, signed zeros, subnormals and the largest finite values;
- an MXFP4 layer against a BF16 layer built from the oracle's dequantised weights,
  bit for bit (the 4-bit kernels run the BF16 kernels' arithmetic on exactly those
  values), at T = 1, 8 and 40 (both weight-streaming down passes) and 129, 300 and 2048
  (the grouped GEMMs, up to 512 rows per expert: every tile height), computed and
  replayed routing, and the fused boundary entry points;
- end to end against the oracle (MoE on the oracle's z; routing exact), at a small
  shape (d 512, 32 experts, d_ff 512), at Beam's decode shapes and at 4096 tokens.
"""
import dataclasses
import os

import numpy as np
import pytest

import oracle
import synth
from tests import parity as P

pytestmark = pytest.mark.gpu

WL = dataclasses.replace(synth.WORKLOADS["tiny"], f=512, name="tiny_f512")
BEAM = synth.WORKLOADS["decode1"]
THREADS = max(1, min(16, os.cpu_count() or 1))
TIES = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.5]  # decision points, saturation


def _exact_bf16(vals):
    f = np.asarray(vals, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def quantiser_inputs():
    """[rows, 256] BF16 bit patterns (seeded) covering the quantiser's cases."""
    rng = np.random.default_rng(2024)
    rows = []
    for std in (1e-30, 1e-6, 0.02, 1.0, 1e4, 1e30):
        v = (rng.standard_normal(8 * 256) * std).astype(np.float32)
        rows.append((v.view(np.uint32) >> 16).astype(np.uint16).reshape(8, 256))
    tie_rows = []
    for X in (-127, -126, -20, -7, 0, 5, 120, 125):
        pts = _exact_bf16([np.ldexp(np.float32(t), X) for t in TIES])
        block = [pts[-1]]  # 7.5 * 2^X: the block maximum, scale X
        for p in pts[:7]:  # each decision point, its BF16 neighbours and its negative
            block += [p, p + 1, p - 1, p | 0x8000]
        block += [pts[7], pts[8] | 0x8000, 0x8000]  # 6, -7.5 (saturates), -0
        assert len(block) == 32
        tie_rows.append(np.array(block * 8, dtype=np.uint16))
    rows.append(np.stack(tie_rows))
    special = np.zeros((4, 256), dtype=np.uint16)
    special[1] = 0x8000                                   # all negative zero
    special[2] = rng.integers(1, 0x80, 256)               # BF16 subnormals
    special[3] = rng.choice([0x7F7F, 0xFF7F, 0x7F00, 0x3F80], 256)  # largest finite
    rows.append(special)
    return np.concatenate(rows, axis=0)


def test_quantise_matches_oracle_bits():
    import sparse_moe_decoder_amd as beam
    src = quantiser_inputs()
    print(f"[mxfp4] quantiser on {src.shape[0]} rows of 256", flush=True)
    codes, scales = beam.beam_mxfp4_quantize(P.to_dev(src))
    o_codes, o_scales = oracle.mxfp4_quantize(src)
    assert np.array_equal(scales.cpu().numpy(), o_scales)
    assert np.array_equal(codes.cpu().numpy(), o_codes)


def test_quantise_expert_weights_match_oracle_bits():
    """The generator's expert weights (N(0, 0.02)), all matrices of the small layer."""
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    wg, wu, wd = sd.experts(WL)
    for name, t, e_host in (("gate", wg, 0), ("up", wu, 1), ("down", wd, 2)):
        codes, scales = beam.beam_mxfp4_quantize(t)
        for e in (0, 13, WL.E - 1):
            oc, os_ = oracle.mxfp4_quantize(synth.expert_weights(WL, e)[e_host])
            assert np.array_equal(codes[e].cpu().numpy(), oc), (name, e)
            assert np.array_equal(scales[e].cpu().numpy(), os_), (name, e)


def quantised_experts(wl, experts):
    """Oracle codes, scales and dequantised BF16 weights of the given experts."""
    q, deq = {}, {}
    for e in experts:
        mats = synth.expert_weights(wl, e)
        q[e] = [oracle.mxfp4_quantize(m) for m in mats]
        deq[e] = tuple(oracle.mxfp4_dequantize(c, s) for c, s in q[e])
    return q, deq


@pytest.fixture(scope="module")
def layer():
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    print(f"[mxfp4] small layer {WL}", flush=True)
    q, deq = quantised_experts(WL, range(WL.E))
    stack = lambda m, i: np.stack([q[e][m][i] for e in range(WL.E)])  # noqa: E731
    fp4 = tuple(P.to_dev(stack(m, i)) for m in range(3) for i in range(2))
    W, b = sd.router(WL)
    cfg = sd.moe_config(WL, max_tokens=2048)
    d = dict(deq=deq)
    d["wpost"], d["wpre"] = sd.norm_weights(WL)
    d["moe4"] = beam.BeamMoE(cfg, W, b, None, None, None, mxfp4=fp4)
    d["moe_deq"] = beam.BeamMoE(cfg, W, b, *[P.to_dev(np.stack([deq[e][m] for e in range(WL.E)]))
                                            for m in range(3)])
    torch.cuda.synchronize()
    yield d
    d["moe4"].close()
    d["moe_deq"].close()


@pytest.mark.parametrize("T", [1, 8, 40, 129, 300, 2048])
def test_mxfp4_equals_bf16_on_dequantised(layer, T):
    import torch
    from synth import device as sd
    z = sd.tokens(WL, "h", T=T)
    y4, r4 = layer["moe4"].forward(z, want_routing=True)
    yd, rd = layer["moe_deq"].forward(z, want_routing=True)
    torch.cuda.synchronize()
    assert np.array_equal(r4["ids_out"].cpu().numpy(), rd["ids_out"].cpu().numpy())
    assert np.array_equal(P.bits(y4), P.bits(yd)), f"T={T}"
    # replayed routing (a slot pointing at no expert, one naming an expert twice)
    ids = r4["ids_out"].clone()
    ids[0, 1] = -1
    ids[0, 2] = ids[0, 0]
    w = r4["w_out"].clone()
    y4r = layer["moe4"].forward(z, ids_in=ids, w_in=w)
    ydr = layer["moe_deq"].forward(z, ids_in=ids, w_in=w)
    assert np.array_equal(P.bits(y4r), P.bits(ydr)), f"T={T} replay"


@pytest.mark.parametrize("d", [8192, 8704])
def test_mxfp4_one_token_wide_rows(d):
    """One token on rows at the single-token passes' limit (hidden 8192: a wave's quarter of
    the row fills its LDS area) and past it (8704: the generic passes), with computed routing
    and with replayed routing that names an expert twice: the 4-bit handle equals the BF16
    handle on the oracle's dequantised weights bit for bit."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    wl = synth.Workload(f"wide{d}", T=1, d=d, E=8, G=2, kg=1, k=2, f=512)
    print(f"[mxfp4] wide layer {wl}", flush=True)
    q, deq = quantised_experts(wl, range(wl.E))
    stack = lambda m, i: np.stack([q[e][m][i] for e in range(wl.E)])  # noqa: E731
    W, b = sd.router(wl)
    cfg = sd.moe_config(wl, max_tokens=4)
    moe4 = beam.BeamMoE(cfg, W, b, None, None, None,
                        mxfp4=tuple(P.to_dev(stack(m, i)) for m in range(3) for i in range(2)))
    moed = beam.BeamMoE(cfg, W, b, *[P.to_dev(np.stack([deq[e][m] for e in range(wl.E)]))
                                     for m in range(3)])
    try:
        z = sd.tokens(wl, "h", T=1)
        y4, r4 = moe4.forward(z, want_routing=True)
        yd, rd = moed.forward(z, want_routing=True)
        torch.cuda.synchronize()
        assert np.array_equal(r4["ids_out"].cpu().numpy(), rd["ids_out"].cpu().numpy())
        assert np.array_equal(P.bits(y4), P.bits(yd)), f"d={d}"
        ids = r4["ids_out"].clone()
        ids[0, 1] = ids[0, 0]
        w = r4["w_out"].clone()
        y4r = moe4.forward(z, ids_in=ids, w_in=w)
        ydr = moed.forward(z, ids_in=ids, w_in=w)
        assert np.array_equal(P.bits(y4r), P.bits(ydr)), f"d={d} replay"
    finally:
        moe4.close()
        moed.close()


@pytest.mark.parametrize("T", [1, 8])
def test_mxfp4_fused_entry_points(layer, T):
    """beam_sublayer_forward and beam_moe_forward_boundary on an MXFP4 handle equal the
    same calls on the BF16 handle of the dequantised weights, bit for bit."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    h, x = sd.tokens(WL, "h", T=T), sd.tokens(WL, "x", T=T)
    outs = []
    for moe in (layer["moe4"], layer["moe_deq"]):
        y = torch.empty_like(h)
        h1, z1 = beam.beam_sublayer_forward(moe.handle, h, x, layer["wpost"], layer["wpre"],
                                            WL.n, WL.eps, y)
        h2, z2 = beam.beam_moe_forward_boundary(moe.handle, z1, h1, layer["wpost"],
                                                layer["wpre"], WL.n + 1, WL.eps)
        torch.cuda.synchronize()
        outs.append([P.bits(t) for t in (h1, z1, y, h2, z2)])
    for a, b_ in zip(*outs):
        assert np.array_equal(a, b_)


def test_mxfp4_matches_oracle(layer):
    """The small layer end to end against the oracle on its own z: routing exact,
    outputs to the BF16 bar."""
    import torch
    hh = synth.token_rows(WL, range(WL.T), "h")
    xx = synth.token_rows(WL, range(WL.T), "x")
    ref = oracle.sublayer(hh, xx, synth.norm_weight(WL, "post"), synth.norm_weight(WL, "pre"),
                          WL.n, WL.eps, synth.router_weight(WL), synth.router_bias(WL), WL.G,
                          WL.kg, WL.k, WL.scale, layer["deq"].__getitem__)
    y, r = layer["moe4"].forward(P.to_dev(ref["z"]), want_routing=True)
    torch.cuda.synchronize()
    same, _ = P.check_routing(r["ids_out"].cpu().numpy(), r["w_out"].cpu().numpy(), ref["ids"],
                              ref["w"], ref["ggap"], ref["egap"], r["logits_out"].cpu().numpy(),
                              ref["logits"], "mxfp4 small")
    P.assert_bf16_close(P.bits(y)[same], ref["y"][same], "mxfp4 small y")


@pytest.fixture(scope="module")
def beam4():
    """Beam's layer with MXFP4 experts quantised on the device from the generator's
    BF16 weights (the quantiser is checked against the oracle separately)."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    print("[mxfp4] drawing Beam's BF16 experts on the device and quantising", flush=True)
    W, b = sd.router(BEAM)
    fp4 = []
    for t in sd.experts(BEAM):
        fp4 += list(beam.beam_mxfp4_quantize(t))
        del t
    torch.cuda.synchronize()
    moe = beam.BeamMoE(sd.moe_config(BEAM, max_tokens=128), W, b, None, None, None,
                       mxfp4=tuple(fp4))
    d = dict(moe=moe, codes=fp4)
    yield d
    moe.close()


@pytest.mark.parametrize("T,sample", [(1, 1), (32, 4)])
def test_mxfp4_beam_decode(beam4, T, sample):
    """Beam shapes: routing for every token; the MoE output of the first `sample`
    tokens against the oracle (which quantises their experts itself); the device codes
    of one touched expert against the oracle's, bit for bit."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    wl = BEAM.with_tokens(T)
    hh = synth.token_rows(wl, range(T), "h")
    xx = synth.token_rows(wl, range(T), "x")
    _, z = oracle.boundary(hh, xx, synth.norm_weight(wl, "post"), synth.norm_weight(wl, "pre"),
                           wl.n, wl.eps)
    logits = oracle.router_threaded(z, synth.router_weight(wl), THREADS)
    ids, w, ggap, egap = oracle.topk(logits, synth.router_bias(wl), wl.G, wl.kg, wl.k, wl.scale)
    y, r = beam4["moe"].forward(P.to_dev(z), want_routing=True)
    torch.cuda.synchronize()
    same, _ = P.check_routing(r["ids_out"].cpu().numpy(), r["w_out"].cpu().numpy(), ids, w, ggap,
                              egap, r["logits_out"].cpu().numpy(), logits, f"mxfp4 beam T={T}")
    need = sorted(set(int(e) for e in ids[:sample].ravel()))
    print(f"[mxfp4] oracle quantises {len(need)} Beam experts", flush=True)
    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(lambda e: quantised_experts(wl, [e]), need))
    q = {e: p[0][e] for e, p in zip(need, parts)}
    deq = {e: p[1][e] for e, p in zip(need, parts)}
    e0 = need[0]
    for m in range(3):
        assert np.array_equal(beam4["codes"][2 * m][e0].cpu().numpy(), q[e0][m][0])
        assert np.array_equal(beam4["codes"][2 * m + 1][e0].cpu().numpy(), q[e0][m][1])
    y_ref, _ = oracle.moe_experts(z[:sample], ids[:sample], w[:sample], wl.E, deq.__getitem__,
                                  threads=THREADS)
    keep = same[:sample]
    P.assert_bf16_close(P.bits(y)[:sample][keep], y_ref[keep], f"mxfp4 beam T={T} y")


def test_mxfp4_beam_prefill_sampled(beam4):
    """Beam shapes at 4096 tokens (the 4-bit grouped GEMMs): routing for every token
    against the oracle, the permutation's invariants, and the MoE output of sampled
    tokens against the oracle (which quantises their experts itself)."""
    import torch
    import sparse_moe_decoder_amd as beam
    from concurrent.futures import ThreadPoolExecutor
    from synth import device as sd
    T = 4096
    wl = BEAM.with_tokens(T)
    W, b = sd.router(BEAM)
    moe = beam.BeamMoE(sd.moe_config(BEAM, max_tokens=T), W, b, None, None, None,
                       mxfp4=tuple(beam4["codes"]))
    hh = synth.token_rows(wl, range(T), "h")
    xx = synth.token_rows(wl, range(T), "x")
    _, z = oracle.boundary(hh, xx, synth.norm_weight(wl, "post"), synth.norm_weight(wl, "pre"),
                           wl.n, wl.eps)
    logits = oracle.router_threaded(z, synth.router_weight(wl), THREADS)
    ids, w, ggap, egap = oracle.topk(logits, synth.router_bias(wl), wl.G, wl.kg, wl.k, wl.scale)
    y, r = moe.forward(P.to_dev(z), want_routing=True)
    torch.cuda.synchronize()
    g_ids = r["ids_out"].cpu().numpy()
    same, _ = P.check_routing(g_ids, r["w_out"].cpu().numpy(), ids, w, ggap, egap,
                              r["logits_out"].cpu().numpy(), logits, "mxfp4 beam T=4096")
    P.check_permutation_valid(g_ids, r["perm_out"].cpu().numpy(), r["offsets_out"].cpu().numpy(),
                              wl.E)
    rows = [0, 1, 1000, 2047, 2048, 4095]
    need = sorted(set(int(e) for e in ids[rows].ravel()))
    print(f"[mxfp4] prefill: oracle quantises {len(need)} Beam experts", flush=True)
    with ThreadPoolExecutor(THREADS) as ex:
        parts = list(ex.map(lambda e: quantised_experts(wl, [e]), need))
    deq = {e: p[1][e] for e, p in zip(need, parts)}
    y_ref, _ = oracle.moe_experts(z[rows], ids[rows], w[rows], wl.E, deq.__getitem__,
                                  threads=THREADS)
    keep = same[rows]
    P.assert_bf16_close(P.bits(y)[rows][keep], y_ref[keep], "mxfp4 beam T=4096 y (sampled)")
    moe.close()
