"""GPU tests of beam_moe_forward_boundary_route (a loop over MoE layers: each call runs its
layer's MoE, then the combine, the next boundary and the NEXT layer's routing, for one token
in one launch). A chain of calls must equal, bit for bit, the same layers run one by one with
beam_moe_forward_boundary (each layer routing its own z), which the other test files check
against the oracle; plus the routing record's checks. All calls go through the C ABI."""
import dataclasses

import numpy as np
import pytest

import synth
from tests import parity as P

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny"]
LAYERS = [TINY, dataclasses.replace(TINY, seed=1, name="tiny_seed1"),
          dataclasses.replace(TINY, seed=2, name="tiny_seed2")]


def _handle(wl, max_tokens, mx_act=False):
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    W, b = sd.router(wl)
    if mx_act:
        fp4 = []
        for t in sd.experts(wl):
            fp4 += list(beam.beam_mxfp4_quantize(t))
        m = beam.BeamMoE(sd.moe_config(wl, max_tokens=max_tokens), W, b, None, None, None,
                         mxfp4=tuple(fp4))
        m.set_activation_format(beam.ACT_MXFP4)
        return m
    wg, wu, wd = sd.experts(wl)
    return beam.BeamMoE(sd.moe_config(wl, max_tokens=max_tokens), W, b, wg, wu, wd)


def _chain_vs_reference(handles, wl, T, steps, token_set=0):
    """`steps` layers (handle i % len(handles)) from the same start, chained and one by one."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    wpost, wpre = sd.norm_weights(wl)
    h0 = sd.tokens(wl, "h", token_set=token_set, T=T)
    z0 = sd.tokens(wl, "x", token_set=token_set, T=T)  # any BF16 rows serve as the first z
    # one by one: each layer routes its own z
    ref = []
    h, z = h0.clone(), z0.clone()
    for i in range(steps):
        moe = handles[i % len(handles)]
        y = torch.empty_like(h)
        h, z = beam.beam_moe_forward_boundary(moe.handle, z, h, wpost, wpre, wl.n, wl.eps,
                                              y_out=y)
        torch.cuda.synchronize()
        ref.append([P.bits(t) for t in (h, z, y)])
    # chained: layer i routes layer i + 1's z in its last launch
    h, z = h0.clone(), z0.clone()
    for i in range(steps):
        moe, nxt = handles[i % len(handles)], handles[(i + 1) % len(handles)]
        y = torch.empty_like(h)
        h, z = beam.beam_moe_forward_boundary_route(moe.handle, nxt.handle, z, h, wpost, wpre,
                                                    wl.n, wl.eps, y_out=y, routed=i > 0)
        torch.cuda.synchronize()
        got = [P.bits(t) for t in (h, z, y)]
        for name, a, b in zip(("h'", "z'", "y"), got, ref[i]):
            assert np.array_equal(a, b), f"T={T} layer {i}: {name} differs"
    print(f"[chain] T={T}: {steps} chained layers equal the one-by-one layers bit for bit",
          flush=True)


@pytest.fixture(scope="module")
def tiny_layers():
    import torch
    hs = [_handle(wl, 64) for wl in LAYERS]
    torch.cuda.synchronize()
    yield hs
    for m in hs:
        m.close()


@pytest.mark.parametrize("T", [1, 8])
def test_chain_three_layers(tiny_layers, T):
    """Three layers with their own routers and experts, cycled over seven steps: T = 1 runs the
    combine, boundary and next routing in one launch; T = 8 as separate launches."""
    _chain_vs_reference(tiny_layers, TINY, T, 7)


def test_chain_same_handle(tiny_layers):
    """A handle routing its own next call (the last launch overwrites the routing the combine
    in the same launch reads)."""
    _chain_vs_reference(tiny_layers[:1], TINY, 1, 5, token_set=1)


def test_chain_routing_record(tiny_layers):
    """routed = 1 needs the routing the previous call left for this T and this z: a different
    z, a different T, an intervening call on the handle, or no previous call are rejected."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    a, b = tiny_layers[0], tiny_layers[1]
    wpost, wpre = sd.norm_weights(TINY)
    h = sd.tokens(TINY, "h", T=1)
    z = sd.tokens(TINY, "x", T=1)

    def call(m, nxt, zz, routed):
        return beam.beam_moe_forward_boundary_route(m.handle, nxt.handle, zz, h, wpost, wpre,
                                                    TINY.n, TINY.eps, routed=routed)
    b.forward(z)  # drops whatever the earlier tests left recorded on b
    with pytest.raises(beam.BeamError):
        call(b, a, z, True)  # nothing recorded for b
    h1, z1 = call(a, b, z, False)
    with pytest.raises(beam.BeamError):
        call(b, a, z, True)  # not the z routed for b
    b.forward(z1)  # another call on b drops the record
    with pytest.raises(beam.BeamError):
        call(b, a, z1, True)
    h1, z1 = call(a, b, z, False)
    call(b, a, z1, True)  # accepted
    torch.cuda.synchronize()


def test_chain_beam_decode():
    """Beam's shape at one token (the decode step bench.py times), one handle chained."""
    import torch
    wl = synth.WORKLOADS["decode1"]
    m = _handle(wl, 1)
    torch.cuda.synchronize()
    try:
        _chain_vs_reference([m], wl, 1, 4)
    finally:
        m.close()


def test_chain_w4a4():
    """4-bit weights and activations: the last launch also quantises the next layer's rows."""
    import torch
    wl = dataclasses.replace(TINY, f=512, name="tiny_f512")
    hs = [_handle(wl, 64, mx_act=True), _handle(dataclasses.replace(wl, seed=3), 64, mx_act=True)]
    torch.cuda.synchronize()
    try:
        _chain_vs_reference(hs, wl, 1, 5)
        _chain_vs_reference(hs, wl, 8, 3)
    finally:
        for m in hs:
            m.close()
