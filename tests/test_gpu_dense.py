"""GPU parity of the dense SwiGLU layer (beam_dense_init / beam_dense_forward) against the
oracle, every call through the C ABI:

- a small layer (d 512, d_ff 2048) at T = 1, 8, 20, 40 and 300: every row compared; this takes
  both weight-streaming down passes and the grouped GEMM with a ragged last tile;
- Beam's dense layer (d 5120, d_ff 20480) at T = 1 and 20 (every element) and at 16384 tokens
  (sampled rows, first and last rows of tiles included);
- the two handle kinds reject each other's entry points.
"""
import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
import synth
from tests import parity as P

pytestmark = pytest.mark.gpu

SMALL = dataclasses.replace(synth.WORKLOADS["dense1"], d=512, f=2048, name="dense_small")
BEAM = synth.WORKLOADS["dense1"]
THREADS = max(1, min(16, os.cpu_count() or 1))


def make_layer(wl, max_tokens):
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    wg, wu, wd = sd.experts(wl)
    h = beam.beam_dense_init(wl.d, wl.f, max_tokens, wg[0], wu[0], wd[0])
    torch.cuda.synchronize()
    return h


def oracle_rows(wl, rows, W):
    """The oracle's dense layer on the generator's token rows `rows` (threaded by row)."""
    z = synth.token_rows(wl, rows, "h")
    parts = np.array_split(np.arange(len(rows)), min(THREADS, len(rows)))
    with ThreadPoolExecutor(len(parts)) as ex:
        outs = list(ex.map(lambda p: oracle.dense_swiglu(z[p], *W), parts))
    return np.concatenate(outs, axis=0)


@pytest.fixture(scope="module")
def small():
    import sparse_moe_decoder_amd as beam
    h = make_layer(SMALL, 512)
    yield h, synth.expert_weights(SMALL, 0)
    beam.beam_moe_destroy(h)


@pytest.mark.parametrize("T", [1, 8, 20, 40, 300])
def test_dense_small(small, T):
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    h, W = small
    y = beam.beam_dense_forward(h, sd.tokens(SMALL, "h", T=T))
    torch.cuda.synchronize()
    P.assert_bf16_close(P.bits(y), oracle_rows(SMALL, range(T), W), f"dense small T={T}")


def test_handle_kinds(small):
    """MoE entry points reject a dense handle; beam_dense_forward rejects an MoE handle."""
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    h, _ = small
    z = sd.tokens(SMALL, "h", T=2)
    ids = torch.zeros((2, 1), dtype=torch.int32, device="cuda")
    w = torch.ones((2, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(beam.BeamError):
        beam.beam_moe_forward(h, z, torch.empty_like(z))
    with pytest.raises(beam.BeamError):
        beam.beam_router_topk(h, z, ids, w)
    tiny = synth.WORKLOADS["tiny"]
    W, b = sd.router(tiny)
    wg, wu, wd = sd.experts(tiny)
    moe = beam.BeamMoE(sd.moe_config(tiny), W, b, wg, wu, wd)
    with pytest.raises(beam.BeamError):
        beam.beam_dense_forward(moe.handle, sd.tokens(tiny, "h", T=2))
    moe.close()


@pytest.fixture(scope="module")
def beam_dense():
    import sparse_moe_decoder_amd as beam
    print("[dense] Beam's dense layer: drawing 0.63 GB of weights", flush=True)
    h = make_layer(BEAM, 16384)
    yield h, synth.expert_weights(BEAM, 0)
    beam.beam_moe_destroy(h)


@pytest.mark.parametrize("T", [1, 20])
def test_dense_beam_decode(beam_dense, T):
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    h, W = beam_dense
    y = beam.beam_dense_forward(h, sd.tokens(BEAM, "h", T=T))
    torch.cuda.synchronize()
    P.assert_bf16_close(P.bits(y), oracle_rows(BEAM, range(T), W), f"dense Beam T={T}")


def test_dense_beam_prefill_sampled(beam_dense):
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    h, W = beam_dense
    T = 16384
    y = beam.beam_dense_forward(h, sd.tokens(BEAM, "h", T=T))
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    rows = sorted(set([0, 1, 255, 256, 8191, T - 1] + rng.integers(0, T, 10).tolist()))
    got = P.bits(y)[rows]
    print(f"[dense] prefill: oracle on {len(rows)} sampled rows", flush=True)
    P.assert_bf16_close(got, oracle_rows(BEAM, rows, W), "dense Beam T=16384 (sampled)")
