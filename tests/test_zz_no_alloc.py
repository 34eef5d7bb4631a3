"""GPU test of beam_moe_forward_noalloc (the allocation-free MoE forward, whose per-call
workspace lives in the library's static scratch area) against beam_moe_forward on the same
handle: the same outputs bit for bit over consecutive calls of decreasing size that take
every routing and expert path (grouped GEMMs, weight streams, the one-launch routing whose
counters live in the scratch area), computed and replayed routing, the size limit, and a
4-bit handle with 4-bit activations (its extra buffers: token-row and activation codes and
scales, and the rows' round trip that the weight streams read). Both entry points are called
through the C ABI."""
import numpy as np
import pytest

import synth
from tests import parity as P

pytestmark = pytest.mark.gpu

WL = synth.WORKLOADS["tiny"]


@pytest.fixture(scope="module")
def moe():
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    print(f"[noalloc] building the tiny layer {WL}", flush=True)
    W, b = sd.router(WL)
    wg, wu, wd = sd.experts(WL)
    m = beam.BeamMoE(sd.moe_config(WL, max_tokens=8192), W, b, wg, wu, wd)
    torch.cuda.synchronize()
    yield m
    m.close()


def _outputs(fn, moe, z, ids_in=None, w_in=None):
    import torch
    T, k, E = z.shape[0], moe.cfg["topk"], moe.cfg["n_experts"]
    dev = z.device
    y = torch.full_like(z, 7.0)
    o = dict(ids_out=torch.full((T, k), -9, dtype=torch.int32, device=dev),
             w_out=torch.full((T, k), -9.0, dtype=torch.float32, device=dev),
             perm_out=torch.full((T * k,), -9, dtype=torch.int32, device=dev),
             offsets_out=torch.full((E + 1,), -9, dtype=torch.int32, device=dev))
    if ids_in is None:
        o["logits_out"] = torch.full((T, E), -9.0, dtype=torch.float32, device=dev)
    fn(moe.handle, z, y, ids_in=ids_in, w_in=w_in, **o)
    torch.cuda.synchronize()
    out = {key: v.cpu().numpy() for key, v in o.items()}
    out["y"] = P.bits(y)
    return out


@pytest.mark.parametrize("replay", [False, True])
def test_noalloc_equals_forward(moe, replay):
    """Calls of 1500 tokens (grouped GEMMs), 40 (weight streams) and 1 (one-launch routing)
    in a row, each compared with beam_moe_forward bit for bit; the scratch area keeps the
    previous call's contents, so each smaller call runs over a larger call's leftovers."""
    import torch
    import sparse_moe_decoder_amd as beam
    g = torch.Generator(device="cpu").manual_seed(11 + replay)
    for T in (1500, 40, 1):
        print(f"[noalloc] T={T} replay={replay}", flush=True)
        z = torch.randn((T, WL.d), generator=g).to(torch.bfloat16).cuda()
        ids_in = w_in = None
        if replay:
            _, ids_in, w_in = moe.router_topk(z, want_logits=False)
            ids_in[0, 0] = WL.E + 1  # an invalid slot contributes nothing on both paths
        ref = _outputs(beam.beam_moe_forward, moe, z, ids_in, w_in)
        for rep in range(2):
            got = _outputs(beam.beam_moe_forward_noalloc, moe, z, ids_in, w_in)
            for key, v in ref.items():
                assert np.array_equal(got[key].view(np.uint8), v.view(np.uint8)), (T, rep, key)


def test_noalloc_limits(moe):
    """A call whose workspace does not fit the 32 MiB scratch area (8192 tokens of this
    layer: about 100 MB) and one above max_tokens are rejected before any work; T = 0 is
    a no-op; the largest batch tried that fits (2048 tokens, about 26 MB) runs."""
    import torch
    import sparse_moe_decoder_amd as beam
    z = torch.zeros((8192, WL.d), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(z)
    with pytest.raises(beam.BeamError) as ei:
        beam.beam_moe_forward_noalloc(moe.handle, z, y)
    assert ei.value.status == -5
    z2 = torch.zeros((8193, WL.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(beam.BeamError) as ei:
        beam.beam_moe_forward_noalloc(moe.handle, z2, torch.empty_like(z2))
    assert ei.value.status == -5
    beam.beam_moe_forward_noalloc(moe.handle, z[:0], y[:0])
    # the largest batch that fits still runs and equals the handle-workspace result
    zf = torch.randn((2048, WL.d), device="cuda").to(torch.bfloat16)
    a = _outputs(beam.beam_moe_forward, moe, zf)
    b = _outputs(beam.beam_moe_forward_noalloc, moe, zf)
    for key, v in a.items():
        assert np.array_equal(b[key].view(np.uint8), v.view(np.uint8)), key


W4 = synth.Workload("noalloc_w4a4", T=1500, d=512, E=32, G=8, kg=4, k=8, f=512)


def test_noalloc_w4a4_equals_forward():
    """A 4-bit-weight handle set to 4-bit activations: 1500 tokens (W4A4 grouped GEMMs), 40
    (weight streams, rows quantised by the stand-alone quantiser) and 1 (weight streams, rows
    quantised inside the one-launch routing) in a row, each equal to beam_moe_forward bit for
    bit, twice."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    print(f"[noalloc] building the 4-bit layer {W4}", flush=True)
    W, b = sd.router(W4)
    fp4 = []
    for t in sd.experts(W4):
        fp4 += list(beam.beam_mxfp4_quantize(t))
    m = beam.BeamMoE(sd.moe_config(W4, max_tokens=W4.T), W, b, None, None, None, mxfp4=tuple(fp4))
    try:
        m.set_activation_format(beam.ACT_MXFP4)
        g = torch.Generator(device="cpu").manual_seed(23)
        for T in (1500, 40, 1):
            print(f"[noalloc] w4a4 T={T}", flush=True)
            z = torch.randn((T, W4.d), generator=g).to(torch.bfloat16).cuda()
            ref = _outputs(beam.beam_moe_forward, m, z)
            for rep in range(2):
                got = _outputs(beam.beam_moe_forward_noalloc, m, z)
                for key, v in ref.items():
                    assert np.array_equal(got[key].view(np.uint8), v.view(np.uint8)), (T, rep, key)
    finally:
        m.close()
