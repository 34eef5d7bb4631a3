"""GPU parity across layer shapes that take the other code paths.

- group sizes that do not map onto lanes (group scores through LDS): 12 experts per
  group, and one expert per group;
- a single group of 64 experts (16 lanes per group), 64 groups of 4, the largest k (32);
- E not a multiple of 64 (the FP32 router serves every batch size);
- the one-token routing by a whole workgroup (power-of-two groups of 2 to 64 experts) with
  its two-level arrival count: sub-counters with unequal arrivals (24 experts), and fewer
  experts than sub-counters (8);
- batch sizes that take each routing, grouping and expert path: the one-launch
  small-batch routing (T <= 16 and T*k <= 64), routing and grouping in one workgroup
  (T <= 16), the one-wave-per-token top-k before the one-workgroup grouping (from 17
  tokens; 16 and 17 sit on either side), the multi-block grouping, the split and the
  streaming down passes, the grouped GEMMs.

Routing is compared bit for bit with the oracle on identical logits (the GPU's own);
the logits to 1e-5 per row; the permutation exactly; the output element by element
with the oracle running the experts on the same routing. All calls go through the
C ABI."""
import numpy as np
import pytest

import oracle
import synth
from synth import Workload
from tests import parity as P

pytestmark = pytest.mark.gpu

CONFIGS = [
    Workload("e48g4", T=1, d=256, E=48, G=4, kg=2, k=6, f=256),      # 12 per group: LDS
    Workload("e16g16", T=1, d=256, E=16, G=16, kg=4, k=4, f=256),    # 1 per group: LDS
    Workload("e64g1", T=1, d=512, E=64, G=1, kg=1, k=8, f=256),      # one group, 16 lanes
    Workload("e256g64", T=1, d=256, E=256, G=64, kg=16, k=32, f=256),  # k = 32
    Workload("e128g4", T=1, d=768, E=128, G=4, kg=2, k=8, f=512),    # 8 lanes per group
    Workload("e24g3", T=1, d=256, E=24, G=3, kg=2, k=3, f=256),      # uneven arrival counts
    Workload("e8g2", T=1, d=256, E=8, G=2, kg=1, k=2, f=256),        # fewer experts than counters
]
MAX_T = 300
T_FORWARD = (1, 7, 16, 17, 40, MAX_T)


@pytest.fixture(scope="module", params=CONFIGS, ids=[c.name for c in CONFIGS])
def cfg(request):
    import torch
    import sparse_moe_decoder_amd as beam
    from synth import device as sd
    wl = request.param
    print(f"[configs] {wl}", flush=True)
    W, b = sd.router(wl)
    wg, wu, wd = sd.experts(wl)
    moe = beam.BeamMoE(sd.moe_config(wl, max_tokens=MAX_T), W, b, wg, wu, wd)
    del wg, wu, wd
    torch.cuda.synchronize()
    experts = {e: synth.expert_weights(wl, e) for e in range(wl.E)}
    yield dict(wl=wl, moe=moe, experts=experts, W=synth.router_weight(wl),
               bias=synth.router_bias(wl))
    moe.close()


@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_routing_bit_exact(cfg, kind):
    import torch
    wl = cfg["wl"]
    lg = synth.synthetic_logits(wl, 64, seed=5, std=1.0)
    if kind == "ties":
        lg = (np.round(lg * 2) / 2).astype(np.float32)
    o_ids, o_w, _, _ = oracle.topk(lg, cfg["bias"], wl.G, wl.kg, wl.k, wl.scale)
    ids, w = cfg["moe"].grouped_topk(torch.from_numpy(lg).cuda())
    assert np.array_equal(ids.cpu().numpy(), o_ids), wl.name
    ulps = np.abs(w.cpu().numpy().view(np.int32).astype(np.int64) - o_w.view(np.int32))
    print(f"[configs] {wl.name} routing ({kind}): max weight ulps {ulps.max()}", flush=True)
    assert ulps.max() <= 1


@pytest.mark.parametrize("T", T_FORWARD)
def test_forward(cfg, T):
    wl = cfg["wl"].with_tokens(T)
    print(f"[configs] {wl.name} forward", flush=True)
    zb = synth.token_rows(wl, range(T), "x")
    y, r = cfg["moe"].forward(P.to_dev(zb), want_routing=True)
    g_lg = r["logits_out"].cpu().numpy()
    g_ids, g_w = r["ids_out"].cpu().numpy(), r["w_out"].cpu().numpy()
    # logits against the oracle's router on the same z
    o_lg = oracle.router(zb, cfg["W"])
    rel = P.logit_rel_rows(g_lg, o_lg)
    print(f"[parity] {wl.name} logits max row rel-L2 {rel.max():.3e}", flush=True)
    assert rel.max() <= P.LOGIT_REL_MAX
    # routing bit for bit on the GPU's own logits
    o_ids, o_w, _, _ = oracle.topk(g_lg, cfg["bias"], wl.G, wl.kg, wl.k, wl.scale)
    assert np.array_equal(g_ids, o_ids)
    ulps = np.abs(g_w.view(np.int32).astype(np.int64) - o_w.view(np.int32))
    assert ulps.max() <= 1
    # grouping exactly
    _, o_off, o_perm, _ = oracle.permute(g_ids, wl.E)
    assert np.array_equal(r["perm_out"].cpu().numpy(), o_perm)
    assert np.array_equal(r["offsets_out"].cpu().numpy(), o_off)
    # experts and combine on the same routing
    o_y, _ = oracle.moe_experts(zb, g_ids, g_w, wl.E, cfg["experts"].__getitem__, threads=8)
    P.assert_bf16_close(P.bits(y), o_y, f"{wl.name} y")
