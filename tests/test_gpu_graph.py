"""HIP-graph capture of the compute entry points (a call only enqueues kernels: it allocates
nothing and never synchronises). Each case is captured once and replayed several times with
the program's own eager work and synchronisations in between; every replay must equal the
eager result bit for bit. Covers the single-token fused routing, the small-batch and the
grouped-GEMM expert paths, the fused boundary entry points, 4-bit experts (with BF16 and with
4-bit activations) and the dense layer;
all calls go through the C ABI."""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from tests import parity as P

pytestmark = pytest.mark.gpu

TINY = synth.WORKLOADS["tiny"]
SMALL4 = dataclasses.replace(TINY, f=512, name="tiny_f512")
DENSE = dataclasses.replace(synth.WORKLOADS["dense1"], d=512, f=2048, name="dense_small")


def _host(o):
    import torch
    return P.bits(o).copy() if o.dtype == torch.bfloat16 else o.cpu().numpy().copy()


def check_graph(fn, outs, what, reps=3):
    """fn() enqueues work that writes the tensors `outs`; the eager result against replays."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    fn()
    torch.cuda.synchronize()
    want = [_host(o) for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for r in range(reps):
        for o in outs:
            o.zero_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            assert np.array_equal(_host(o), w), f"{what}: replay {r}, output {i}"
    print(f"[graph] {what}: {reps} replays equal the eager result", flush=True)


@pytest.fixture(scope="module")
def tiny():
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    d = {}
    d["wpost"], d["wpre"] = sd.norm_weights(TINY)
    W, b = sd.router(TINY)
    wg, wu, wd = sd.experts(TINY)
    d["moe"] = beam.BeamMoE(sd.moe_config(TINY, max_tokens=512), W, b, wg, wu, wd)
    torch.cuda.synchronize()
    yield d
    d["moe"].close()


@pytest.mark.parametrize("T", [1, 8, 40, 300])
def test_graph_moe_forward(tiny, T):
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    z = sd.tokens(TINY, "h", T=T)
    y = torch.empty_like(z)
    check_graph(lambda: beam.beam_moe_forward(tiny["moe"].handle, z, y), [y], f"moe T={T}")


@pytest.mark.parametrize("T", [1, 8])
def test_graph_fused_boundary_calls(tiny, T):
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    h, x = sd.tokens(TINY, "h", T=T), sd.tokens(TINY, "x", T=T)
    h1, z1, y = torch.empty_like(h), torch.empty_like(h), torch.empty_like(h)
    h2, z2 = torch.empty_like(h), torch.empty_like(h)
    n, eps, m = TINY.n, TINY.eps, tiny["moe"].handle

    def run():
        beam.beam_sublayer_forward(m, h, x, tiny["wpost"], tiny["wpre"], n, eps, y, h_out=h1,
                                   z_out=z1)
        beam.beam_moe_forward_boundary(m, z1, h1, tiny["wpost"], tiny["wpre"], n + 1, eps,
                                       h_out=h2, z_out=z2)

    check_graph(run, [h1, z1, y, h2, z2], f"sublayer + forward_boundary T={T}")


def test_graph_mxfp4():
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    q = {e: [oracle.mxfp4_quantize(m) for m in synth.expert_weights(SMALL4, e)]
         for e in range(SMALL4.E)}
    fp4 = tuple(P.to_dev(np.stack([q[e][m][i] for e in range(SMALL4.E)]))
                for m in range(3) for i in range(2))
    W, b = sd.router(SMALL4)
    moe = beam.BeamMoE(sd.moe_config(SMALL4, max_tokens=512), W, b, None, None, None, mxfp4=fp4)
    for T in (1, 40, 300):
        z = sd.tokens(SMALL4, "h", T=T)
        y = torch.empty_like(z)
        check_graph(lambda: beam.beam_moe_forward(moe.handle, z, y), [y], f"mxfp4 T={T}")
    # 4-bit activations: the rows quantised inside the routing launch (T = 1), by the
    # stand-alone quantiser with the activations' round-trip pass (T = 40), the W4A4 GEMMs (300)
    moe.set_activation_format(beam.ACT_MXFP4)
    for T in (1, 40, 300):
        z = sd.tokens(SMALL4, "h", T=T)
        y = torch.empty_like(z)
        check_graph(lambda: beam.beam_moe_forward(moe.handle, z, y), [y], f"w4a4 T={T}")
    moe.close()


def test_graph_dense():
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    wg, wu, wd = sd.experts(DENSE)
    h = beam.beam_dense_init(DENSE.d, DENSE.f, 512, wg[0], wu[0], wd[0])
    for T in (1, 20, 300):
        z = sd.tokens(DENSE, "h", T=T)
        y = torch.empty_like(z)
        check_graph(lambda: beam.beam_dense_forward(h, z, y), [y], f"dense T={T}")
    beam.beam_moe_destroy(h)


def test_edge_calls_new_entry_points():
    """T = 0 is a no-op; T beyond max_tokens is rejected on the host; an MXFP4 handle with
    every slot replayed to no expert returns zeros (the combine of nothing)."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    wg, wu, wd = sd.experts(DENSE)
    h = beam.beam_dense_init(DENSE.d, DENSE.f, 4, wg[0], wu[0], wd[0])
    z0 = torch.empty((0, DENSE.d), dtype=torch.bfloat16, device="cuda")
    beam.beam_dense_forward(h, z0)
    with pytest.raises(beam.BeamError):
        beam.beam_dense_forward(h, sd.tokens(DENSE, "h", T=5))
    beam.beam_moe_destroy(h)
    codes, scales = beam.beam_mxfp4_quantize(torch.empty((0, 64), dtype=torch.bfloat16,
                                                         device="cuda"))
    assert codes.shape == (0, 32) and scales.shape == (0, 2)
    q = [beam.beam_mxfp4_quantize(t) for t in sd.experts(SMALL4)]
    W, b = sd.router(SMALL4)
    moe = beam.BeamMoE(sd.moe_config(SMALL4, max_tokens=8), W, b, None, None, None,
                       mxfp4=tuple(a for pair in q for a in pair))
    z = sd.tokens(SMALL4, "h", T=3)
    ids = torch.full((3, SMALL4.k), -1, dtype=torch.int32, device="cuda")
    w = torch.ones((3, SMALL4.k), dtype=torch.float32, device="cuda")
    y = moe.forward(z, ids_in=ids, w_in=w)
    torch.cuda.synchronize()
    assert np.array_equal(P.bits(y), np.full((3, SMALL4.d), 0x8000, dtype=np.uint16))
    with pytest.raises(beam.BeamError):
        moe.forward(sd.tokens(SMALL4, "h", T=9))
    moe.close()
