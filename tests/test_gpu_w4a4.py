"""GPU parity of the W4A4 expert path (4-bit weights and 4-bit activations, the scaled FP4
matrix cores) against oracle O8, stage by stage on identical inputs:
  1. token-row quantisation: the GPU's z codes and scales equal the oracle's MXFP4 (O7)
     bit for bit;
  2. gate/up + SiLU-mul + activation quantisation: the GPU's activation codes equal O7 of
     the oracle's activation (O5's first half on the same 4-bit z and weights) except where
     a final BF16 rounding of g, u or act flipped between the two FP32 summation orders and
     moved a value across an E2M1 decision point: at most 1e-3 of the codes, each within one
     grid step of the oracle's;
  3. down + weight + combine: the GPU's y equals the oracle's down half and combine on the
     GPU's own activation codes, to the BF16 bar (rel-L2 <= 2e-3, max-abs rule);
and the composed O8 (oracle from z alone) reported, asserted only against gross error.
T <= 128 runs on the 4-bit weight-streaming passes (with the round trips of z and act), larger
T on the W4A4 GEMMs; both are checked the same way. All calls go through the C ABI."""
import numpy as np
import pytest

import oracle
import synth
from synth import Workload
from tests import parity as P

pytestmark = pytest.mark.gpu

WL = Workload("w4a4", T=1536, d=512, E=32, G=8, kg=4, k=8, f=512)
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


@pytest.fixture(scope="module")
def layer():
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    print(f"[w4a4] layer {WL}", flush=True)
    W, b = sd.router(WL)
    wg, wu, wd = sd.experts(WL)
    fp4 = []
    for t in (wg, wu, wd):
        fp4 += list(beam.beam_mxfp4_quantize(t))
    moe = beam.BeamMoE(sd.moe_config(WL, max_tokens=WL.T), W, b, None, None, None,
                       mxfp4=tuple(fp4))
    moe.set_activation_format(beam.ACT_MXFP4)
    torch.cuda.synchronize()
    # the oracle's own 4-bit weights (O7), dequantised
    host = {}
    for e in range(WL.E):
        host[e] = tuple(oracle.mxfp4_dequantize(*oracle.mxfp4_quantize(m))
                        for m in synth.expert_weights(WL, e))
    yield moe, host
    moe.close()


def natural_order(codes, K):
    """GEMM-order block codes [rows, K/2] -> natural order (O7's layout)."""
    c = codes.reshape(-1, K // 32, 4, 4)[:, :, [0, 2, 1, 3], :]
    return c.reshape(-1, K // 2)


def dequant(codes, scales):
    return P.F(oracle.mxfp4_dequantize(codes, scales)).astype(np.float64)


def run(moe, z, ids_in=None, w_in=None, wl=WL):
    import torch
    T = z.shape[0]
    y, r = moe.forward(P.to_dev(z), ids_in=ids_in, w_in=w_in, want_routing=True)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in r.items()}
    g["y"] = P.bits(y)
    S = T * wl.k
    g["zq"] = moe.inspect("z_codes", T * wl.d // 2).cpu().numpy().reshape(T, wl.d // 2)
    g["zs"] = moe.inspect("z_scales", T * wl.d // 32).cpu().numpy().reshape(T, wl.d // 32)
    g["aq"] = moe.inspect("act_codes", S * wl.f // 2).cpu().numpy().reshape(S, wl.f // 2)
    g["as"] = moe.inspect("act_scales", S * wl.f // 32).cpu().numpy().reshape(S, wl.f // 32)
    return g


def check_stages(g, z, ids, w, host, what, wl=WL):
    T, k = ids.shape
    WL = wl  # noqa: N806 (the stage checks below read the workload's shapes)
    # 1. token rows
    o_zq, o_zs = oracle.mxfp4_quantize(z)
    assert np.array_equal(natural_order(g["zq"], WL.d), o_zq), what
    assert np.array_equal(g["zs"], o_zs), what
    zq = oracle.mxfp4_dequantize(o_zq, o_zs)
    # 2. activations, rows in the expert-grouped order
    nv = int(g["offsets_out"][-1])
    perm = g["perm_out"][:nv]
    tok, slot_j = perm // k, perm % k
    eid = ids.ravel()[perm]
    o_act = np.empty((nv, WL.f), np.uint16)
    for e in np.unique(eid):
        rows = np.nonzero(eid == e)[0]
        o_act[rows] = oracle.expert_act(zq[tok[rows]], host[e][0], host[e][1])
    o_aq, o_as = oracle.mxfp4_quantize(o_act)
    g_aq = natural_order(g["aq"][:nv], WL.f)
    g_as = g["as"][:nv]
    code_diff = np.mean(g_aq != o_aq)
    scale_diff = np.mean(g_as != o_as)
    dg, do = dequant(g_aq, g_as), dequant(o_aq, o_as)
    step = 2.0 * np.exp2(np.maximum(g_as, o_as).astype(np.float64) - 127.0)
    step = np.repeat(step, 32, axis=1)
    far = int(np.count_nonzero(np.abs(dg - do) > step))
    print(f"[parity] {what} act codes: differ {code_diff:.2e}, scales differ {scale_diff:.2e}, "
          f"beyond one grid step {far}", flush=True)
    assert code_diff <= 1e-3 and scale_diff <= 1e-3 and far == 0, what
    # 3. down, weight and combine on the GPU's activation codes
    g_act = oracle.mxfp4_dequantize(g_aq, g_as)
    yk = np.zeros((T, k, WL.d), np.uint16)
    for e in np.unique(eid):
        rows = np.nonzero(eid == e)[0]
        yk[tok[rows], slot_j[rows]] = oracle.expert_down(g_act[rows], host[e][2],
                                                         w[tok[rows], slot_j[rows]])
    y_stage = oracle.combine(yk, ids, WL.E)
    P.assert_bf16_close(g["y"], y_stage, f"{what} y (down stage on the GPU's codes)")
    # composed O8 from z alone (act code flips included): gross error only
    y_o8, _ = oracle.moe_experts(z, ids, w, WL.E, host.__getitem__, threads=8, mx_act=True)
    ok, st = P.compare_bf16(g["y"], y_o8)
    print(f"[parity] {what} y vs composed O8: {st}", flush=True)
    assert st["rel_l2"] < 1e-2, what


def host_z(T, token_set=0):
    hh = synth.token_rows(WL, range(T), "h", token_set=token_set)
    xx = synth.token_rows(WL, range(T), "x", token_set=token_set)
    _, z = oracle.boundary(hh, xx, synth.norm_weight(WL, "post"), synth.norm_weight(WL, "pre"),
                           WL.n, WL.eps)
    return z


@pytest.mark.parametrize("T", [1, 8, 40, 300, 1536])
def test_w4a4_stages(layer, T):
    """Computed routing (the router is unchanged: ids = the oracle's top-k of the GPU's
    logits), then every stage of the W4A4 experts; T = 1536 gives every expert several
    row tiles and ragged tails."""
    moe, host = layer
    print(f"[w4a4] T={T}", flush=True)
    z = host_z(T)
    g = run(moe, z)
    o_ids, o_w, _, _ = oracle.topk(g["logits_out"], synth.router_bias(WL), WL.G, WL.kg, WL.k,
                                   WL.scale)
    assert np.array_equal(g["ids_out"], o_ids)
    check_stages(g, z, o_ids, g["w_out"], host, f"w4a4 T={T}")


def test_w4a4_replay_and_format_switch(layer):
    """Replayed routing with an invalid slot; switching back to BF16 activations gives the
    4-bit-weight path's result again, bit for bit, and differs from the W4A4 result."""
    import torch
    import sparse_moe_decoder_amd as beam
    moe, host = layer
    T = 40
    z = host_z(T, token_set=1)
    ids, w, _, _ = oracle.topk(oracle.router(z, synth.router_weight(WL)), synth.router_bias(WL),
                               WL.G, WL.kg, WL.k, WL.scale)
    ids[3, 2] = -1
    g = run(moe, z, torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda())
    check_stages(g, z, ids, w, host, "w4a4 replay")
    zd = P.to_dev(z)
    moe.set_activation_format(beam.ACT_BF16)
    try:
        a = P.bits(moe.forward(zd))
        b = P.bits(moe.forward(zd))
    finally:
        moe.set_activation_format(beam.ACT_MXFP4)
    c = P.bits(moe.forward(zd))
    assert np.array_equal(a, b)
    assert np.mean(a != c) > 0.5
    moe.set_activation_format(beam.ACT_BF16)
    try:
        assert np.array_equal(P.bits(moe.forward(zd)), a)
    finally:
        moe.set_activation_format(beam.ACT_MXFP4)


@pytest.mark.parametrize("T", [1, 8])
def test_w4a4_fused_entry_points(layer, T):
    """Up to 16 tokens the routing launch quantises the token rows itself (for one token
    inside the boundary + routing launch of beam_sublayer_forward, from its LDS copy of z):
    the z codes equal the oracle's MXFP4 of the GPU's z bit for bit, and the output equals,
    bit for bit, that of beam_moe_forward on the same z with computed routing and with that
    routing replayed (rows then quantised by the stand-alone quantiser)."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    moe, host = layer
    print(f"[w4a4] fused entry points T={T}", flush=True)
    wpost, wpre = sd.norm_weights(WL)
    h, x = sd.tokens(WL, "h", T=T), sd.tokens(WL, "x", T=T)
    y1 = torch.empty_like(h)
    h1, z1 = beam.beam_sublayer_forward(moe.handle, h, x, wpost, wpre, WL.n, WL.eps, y1)
    torch.cuda.synchronize()
    zq = moe.inspect("z_codes", T * WL.d // 2).cpu().numpy().reshape(T, WL.d // 2)
    zs = moe.inspect("z_scales", T * WL.d // 32).cpu().numpy().reshape(T, WL.d // 32)
    o_zq, o_zs = oracle.mxfp4_quantize(P.bits(z1))
    assert np.array_equal(natural_order(zq, WL.d), o_zq)
    assert np.array_equal(zs, o_zs)
    y2, r = moe.forward(z1, want_routing=True)
    y3 = moe.forward(z1, ids_in=r["ids_out"], w_in=r["w_out"])
    torch.cuda.synchronize()
    assert np.array_equal(P.bits(y2), P.bits(y1))
    assert np.array_equal(P.bits(y3), P.bits(y1))


WL_ROW = Workload("w4a4_row", T=1, d=5120, E=16, G=4, kg=2, k=4, f=2560)


@pytest.mark.parametrize("repeat", [False, True])
def test_w4a4_one_token_beam_rows(repeat):
    """One token at Beam's hidden size and d_ff: the single-token down pass rounds the
    activation row through MXFP4 itself (80 chunks of the row per wave, two passes of 64
    lanes, the five-deep weight ring). Every stage is checked as in the decode tests: the
    activation codes and scales against the oracle's MXFP4 of the oracle's activations, y
    against the oracle's down + combine on the GPU's codes. With replayed routing that names
    one expert twice, that expert's two rows both carry the codes."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    wl = WL_ROW
    print(f"[w4a4] one token, Beam rows, repeat={repeat}", flush=True)
    W, b = sd.router(wl)
    fp4 = []
    for t in sd.experts(wl):
        fp4 += list(beam.beam_mxfp4_quantize(t))
        del t
    moe = beam.BeamMoE(sd.moe_config(wl, max_tokens=1), W, b, None, None, None, mxfp4=tuple(fp4))
    del fp4
    try:
        moe.set_activation_format(beam.ACT_MXFP4)
        torch.cuda.synchronize()

        class Host(dict):  # the oracle's dequantised 4-bit weights, per expert on first use
            def __missing__(self, e):
                self[e] = tuple(oracle.mxfp4_dequantize(*oracle.mxfp4_quantize(m))
                                for m in synth.expert_weights(wl, e))
                return self[e]

        host = Host()
        z = synth.token_rows(wl, range(1), "x")
        g = run(moe, z, wl=wl)
        ids, w = g["ids_out"].reshape(1, wl.k), g["w_out"].reshape(1, wl.k)
        if repeat:
            ids = ids.copy()
            ids[0, 1] = ids[0, 0]
            g = run(moe, z, ids_in=P.to_dev(ids), w_in=P.to_dev(w), wl=wl)
            nv = int(g["offsets_out"][-1])
            e0 = int(ids[0, 0])
            rows = np.nonzero(ids.ravel()[g["perm_out"][:nv]] == e0)[0]
            assert rows.size == 2
            assert np.array_equal(g["aq"][rows[0]], g["aq"][rows[1]])
            assert np.array_equal(g["as"][rows[0]], g["as"][rows[1]])
        check_stages(g, z, ids, w, host, f"one token, Beam rows, repeat={repeat}", wl=wl)
    finally:
        moe.close()


WL_FEW = Workload("w4a4_few", T=8, d=4096, E=8, G=2, kg=1, k=2, f=512)


@pytest.mark.parametrize("T", [1, 8])
def test_w4a4_routing_quantiser_rounds(T):
    """Eight experts and rows of 4096: the routing launch's eight workgroups each quantise up
    to 128 of the rows' blocks (two rounds of 64 per workgroup). z codes equal the oracle's
    MXFP4 bit for bit; the output equals the replayed-routing output (stand-alone quantiser)
    bit for bit."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    print(f"[w4a4] few experts T={T}", flush=True)
    W, b = sd.router(WL_FEW)
    fp4 = []
    for t in sd.experts(WL_FEW):
        fp4 += list(beam.beam_mxfp4_quantize(t))
    moe = beam.BeamMoE(sd.moe_config(WL_FEW, max_tokens=WL_FEW.T), W, b, None, None, None,
                       mxfp4=tuple(fp4))
    try:
        moe.set_activation_format(beam.ACT_MXFP4)
        z = P.to_dev(synth.token_rows(WL_FEW, range(T), "x"))
        y1, r = moe.forward(z, want_routing=True)
        torch.cuda.synchronize()
        zq = moe.inspect("z_codes", T * WL_FEW.d // 2).cpu().numpy().reshape(T, WL_FEW.d // 2)
        zs = moe.inspect("z_scales", T * WL_FEW.d // 32).cpu().numpy().reshape(T, WL_FEW.d // 32)
        o_zq, o_zs = oracle.mxfp4_quantize(P.bits(z))
        assert np.array_equal(natural_order(zq, WL_FEW.d), o_zq)
        assert np.array_equal(zs, o_zs)
        y2 = moe.forward(z, ids_in=r["ids_out"], w_in=r["w_out"])
        torch.cuda.synchronize()
        assert np.array_equal(P.bits(y2), P.bits(y1))
    finally:
        moe.close()


def test_w4a4_format_rejected_for_bf16_weights():
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    W, b = sd.router(WL)
    wg, wu, wd = sd.experts(WL)
    moe = beam.BeamMoE(sd.moe_config(WL, max_tokens=8), W, b, wg, wu, wd)
    try:
        with pytest.raises(beam.BeamError) as ei:
            moe.set_activation_format(beam.ACT_MXFP4)
        assert ei.value.status == -2
        with pytest.raises(beam.BeamError):
            moe.set_activation_format(7)
        moe.set_activation_format(beam.ACT_BF16)
    finally:
        moe.close()
