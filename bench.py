"""Benchmark: one Beam MoE sublayer step (fused boundary + routed MoE FFN) on one MI355X.

A step is one pass of the whole path over one batch of T tokens: the MoE FFN
(FP32 router, grouped top-k, expert grouping, BF16 SwiGLU experts, weighted
combine) and one sublayer boundary (post-norm, depth-scaled residual, pre-norm).
By default (--step boundary-last) it is beam_moe_forward_boundary: the MoE on z,
then the next sublayer's boundary fused into the combine, as a decode loop runs
it; --step boundary-first times beam_sublayer_forward (the boundary, then the MoE
on its z). Both are bit-identical to the separate calls. Inputs are seeded synthetic tensors already resident
in HBM when the timed region starts; decode steps rotate over distinct token sets
so the experts touched change from step to step.

Prints one JSON line. `value` is tokens per second for the whole job;
`roofline` reports the dominant kernel (expert gate/up) against HBM (decode) or
BF16 matrix-core (prefill) peak, from HIP events recorded around that kernel on
its own stream during a timed region; `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense BF16 matrix cores
METRIC = "MoE-layer tokens/s (decode T=1/32/128, prefill 16K) + % HBM/MFMA peak"


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="decode1",
                   choices=["decode1", "decode32", "decode128", "prefill16k", "skew32k",
                            "skew32k_half", "tiny", "dense1", "dense16k"],
                   help="dense1 / dense16k: Beam's dense SwiGLU layer (d_ff 20480) instead of "
                        "the MoE; a step is that layer, then the next boundary on its output")
    p.add_argument("--rotations", type=int, default=None, help="distinct token sets")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--step", choices=("boundary-first", "boundary-last"), default="boundary-last",
                   help="boundary-first: beam_sublayer_forward (the boundary, then the MoE on its z); "
                        "boundary-last: beam_moe_forward_boundary (the MoE on a z computed before the "
                        "timed region, then the next sublayer's boundary fused into the combine)")
    p.add_argument("--cpu-sample", type=int, default=None, help="tokens in the CPU sample")
    p.add_argument("--experts", choices=("bf16", "mxfp4"), default="bf16",
                   help="expert weight format: BF16, or MXFP4 (4-bit E2M1 codes with one E8M0 "
                        "scale per 32 values, quantised on the device from the BF16 weights; "
                        "BF16 activations)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run plain device-to-device copies of BYTES (for scaling HBM "
                        "counter readings) and exit")
    return p.parse_args()


def copy_calibration(nbytes: int, reps: int = 5):
    """Plain device copies of a known size: what FETCH_SIZE / WRITE_SIZE read per
    dispatch for nbytes read + nbytes written gives the counters' scale."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_moe_decoder_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None if
    there is none for this kernel and workload or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha") != src_hash:
        return None
    try:
        fetch = float(vals["FETCH_SIZE_KiB_per_dispatch"]) * 1024 * float(vals["fetch_scale"])
        write = float(vals["WRITE_SIZE_KiB_per_dispatch"]) * 1024 * float(vals["write_scale"])
        return fetch + write
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has "
              "no multi-GPU path; the per-GPU kernels are what one GPU shows.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    from synth import device as sd
    import sparse_moe_decoder_amd as beam

    wl = synth.WORKLOADS[args.workload]
    T = wl.T
    decode = T <= 128
    steps = args.steps or (200 if decode else 10)
    warmup = args.warmup if args.warmup is not None else (20 if decode else 3)
    R = args.rotations or (32 if decode else 1)
    torch.cuda.set_device(0)
    dev = torch.cuda.current_device()
    log(f"workload {wl.name}: T={T} d={wl.d} E={wl.E} f={wl.f}; steps {steps} warmup {warmup} "
        f"rotations {R}")

    t0 = time.time()
    wpost, wpre = sd.norm_weights(wl)
    W, b = sd.router(wl)
    wg, wu, wd = sd.experts(wl)
    mx = args.experts == "mxfp4"
    dense = wl.name.startswith("dense")
    if mx and dense:
        print("--experts mxfp4 applies to the MoE workloads", file=sys.stderr)
        sys.exit(2)
    if dense:
        moe = None
        dense_h = beam.beam_dense_init(wl.d, wl.f, T, wg[0], wu[0], wd[0])
    elif mx:
        fp4 = []
        for t in (wg, wu, wd):
            fp4 += list(beam.beam_mxfp4_quantize(t))
        moe = beam.BeamMoE(sd.moe_config(wl, max_tokens=T), W, b, None, None, None,
                           mxfp4=tuple(fp4))
        del fp4
    else:
        moe = beam.BeamMoE(sd.moe_config(wl, max_tokens=T), W, b, wg, wu, wd)
    del wg, wu, wd
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    hs = [sd.tokens(wl, "h", token_set=s) for s in range(R)]
    xs = [sd.tokens(wl, "x", token_set=s) for s in range(R)]
    h_out = torch.empty((T, wl.d), dtype=torch.bfloat16, device="cuda")
    z = torch.empty_like(h_out)
    y = torch.empty_like(h_out)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t0:.1f}s")

    if dense:
        # each token set's z from its boundary, before the timed region; a step is the dense
        # layer on it, then the next boundary with its output as the branch
        z_in = [beam.beam_sublayer_norm_residual(hs[s], xs[s], wpost, wpre, wl.n, wl.eps)[1]
                for s in range(R)]

        def step(i):
            s = i % R
            beam.beam_dense_forward(dense_h, z_in[s], y)
            beam.beam_sublayer_norm_residual(hs[s], y, wpost, wpre, wl.n, wl.eps, h_out=h_out,
                                             z_out=z)
    elif args.step == "boundary-first":
        def step(i):
            s = i % R
            beam.beam_sublayer_forward(moe.handle, hs[s], xs[s], wpost, wpre, wl.n, wl.eps, y,
                                       h_out=h_out, z_out=z)
    else:
        # each token set's z from its boundary, before the timed region; a step is the MoE on
        # it and the next boundary (x = the MoE output), whose outputs are h_out and z
        z_in = []
        for s in range(R):
            z_in.append(beam.beam_sublayer_norm_residual(hs[s], xs[s], wpost, wpre, wl.n,
                                                         wl.eps)[1])

        def step(i):
            s = i % R
            beam.beam_moe_forward_boundary(moe.handle, z_in[s], hs[s], wpost, wpre, wl.n, wl.eps,
                                           h_out=h_out, z_out=z)

    # distinct experts per token set (for the algorithmic byte count)
    distinct = []
    ids_buf = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
    w_buf = torch.empty((T, wl.k), dtype=torch.float32, device="cuda")
    for s in range(R if not dense else 0):
        beam.beam_sublayer_norm_residual(hs[s], xs[s], wpost, wpre, wl.n, wl.eps, h_out=h_out,
                                         z_out=z)
        beam.beam_router_topk(moe.handle, z, ids_buf, w_buf)
        distinct.append(len(np.unique(ids_buf.cpu().numpy())))
    if dense:
        distinct = [1]
    mean_distinct = float(np.mean(distinct))

    def timed(fn, n):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # 1) eager
    for i in range(warmup):
        step(i)
    ms_eager = timed(step, steps)
    log(f"eager: {ms_eager * 1e3:.1f} us/step")

    # 2) HIP graph of one step per token set (no allocation, no host sync inside)
    ms_graph = None
    if not args.no_graph:
        try:
            graphs = []
            cs = torch.cuda.Stream()
            cs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cs):
                for s in range(R):
                    step(s)  # warm on the capture stream
            torch.cuda.current_stream().wait_stream(cs)
            torch.cuda.synchronize()
            for s in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step(s)
                graphs.append(g)
            for i in range(warmup):
                graphs[i % R].replay()
            ms_graph = timed(lambda i: graphs[i % R].replay(), steps)
            log(f"graph: {ms_graph * 1e3:.1f} us/step")
            # graph result equals the eager result
            step(0)
            out = y if (args.step == "boundary-first" and not dense) else z  # last output
            out_eager = out.clone()
            graphs[0].replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), out_eager.view(torch.int16)), "graph != eager"
        except Exception as exc:  # report, fall back to the eager number
            log(f"graph capture unavailable: {exc!r}")
            ms_graph = None

    # per-step spread: events around each eager step (a separate pass; the value above is
    # the whole timed region divided by the step count)
    per = []
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(steps, 200))]
    torch.cuda.synchronize()
    for i, (a, b_) in enumerate(ev):
        a.record()
        step(i)
        b_.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b_) for a, b_ in ev)
    pct = {f"p{q}": round(float(np.percentile(per, q)), 5) for q in (10, 50, 90)}
    log(f"per-step ms: {pct}")

    # 3) per-kernel durations from HIP events around each launch, over a timed region
    beam.profile_reset()
    beam.profile_enable(True)
    ms_prof = timed(step, steps)
    beam.profile_enable(False)
    kern = beam.profile_read()
    beam.profile_reset()
    kernel_us = {k: (v[0] / v[1] * 1e3 if v[1] else None) for k, v in kern.items()}
    log("kernel avg us: " + ", ".join(f"{k} {v:.1f}" for k, v in kernel_us.items() if v))

    best_ms = ms_eager if ms_graph is None else min(ms_eager, ms_graph)
    mode = "hipgraph" if (ms_graph is not None and ms_graph <= ms_eager) else "eager"
    value = T / (best_ms / 1e3)

    # roofline of the dominant kernel (expert gate/up)
    gu_us = kernel_us.get("gate_up")
    # the sources of the gate/up kernels (4-bit: streams in experts_mxfp4.hip, GEMM in experts.hip)
    src = source_hash(*(("experts.hip", "experts_mxfp4.hip", "common.h") if mx
                        else ("experts.hip", "common.h")))
    wbytes = (0.5 + 1.0 / 32) if mx else 2.0  # bytes per expert weight (codes + scales)
    if decode:
        # algorithmic bytes per launch: each touched expert's gate+up weights once, the
        # token rows in, the activations out
        bytes_gu = mean_distinct * 2 * wl.f * wl.d * wbytes + T * wl.d * 2 + T * wl.k * wl.f * 2
        achieved = bytes_gu / (gu_us * 1e-6) / 1e9
        roof = dict(kernel="gate_up", bound="hbm", achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4))
        traffic = read_traffic("gate_up_mxfp4" if mx else "gate_up", wl.name, src)
        roof["traffic"] = traffic
        step_bytes = (mean_distinct * 3 * wl.f * wl.d * wbytes + (0 if dense else wl.E * wl.d * 4)
                      + T * wl.d * 2 * 6 + T * wl.k * (wl.f * 4 + wl.d * 4))
        whole = dict(algorithmic_bytes=round(step_bytes), hbm_frac=round(
            step_bytes / (best_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    else:
        flops_gu = 2.0 * T * wl.k * (2 * wl.f) * wl.d
        achieved = flops_gu / (gu_us * 1e-6) / 1e12
        roof = dict(kernel="gate_up", bound="mfma", achieved=round(achieved, 1),
                    peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / BF16_PEAK_TFLOPS, 4))
        roof["traffic"] = read_traffic("gate_up", wl.name, src)
        step_flops = 2.0 * T * wl.k * 3 * wl.f * wl.d
        whole = dict(expert_flops=step_flops, mfma_frac=round(
            step_flops / (best_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_sample, mxfp4=mx)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(best_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if not mx else "bf16 (mxfp4 expert weights)",
        "data": "synthetic (seeded counter-based generator; random-init weights of Beam's MoE layer)",
        "config": {
            "workload": wl.name, "tokens": T, "hidden": wl.d, "experts": wl.E,
            "groups": wl.G, "groups_kept": wl.kg, "topk": wl.k, "d_ff": wl.f,
            "experts_format": args.experts,
            "token_sets": R, "distinct_experts_per_step": round(mean_distinct, 1),
            "step": args.step, "mode": mode, "ms_eager": round(ms_eager, 5),
            "ms_graph": None if ms_graph is None else round(ms_graph, 5),
            "ms_profiled": round(ms_prof, 5),
            "ms_per_step_eager_percentiles": pct,
            "kernel_us": {k: (None if v is None else round(v, 2)) for k, v in kernel_us.items()},
            "whole_step": whole,
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    if dense:
        beam.beam_moe_destroy(dense_h)
    else:
        moe.close()


def cpu_baseline(wl, sample=None, mxfp4=False):
    """The CPU oracle, as it is, on a bounded sample of the same workload: each
    sampled token goes through boundary, router, routing, its experts and the
    combine, single-threaded per token; tokens run in a thread pool. With mxfp4 the
    experts' weights are the oracle's MXFP4 quantisation, dequantised (not timed)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import synth

    threads = max(1, min(16, os.cpu_count() or 1))
    n = sample or (threads if (mxfp4 or wl.name.startswith("dense")) else 2 * threads)
    rows = list(range(min(n, wl.T))) if wl.T >= n else list(range(wl.T))
    if len(rows) < n:  # decode: also take tokens of the rotation sets
        extra = n - len(rows)
        rot = [(s, t) for s in range(1, 1 + (extra + wl.T - 1) // wl.T) for t in range(wl.T)]
        rot = rot[:extra]
    else:
        rot = []
    hh = [synth.token_rows(wl, [t], "h") for t in rows] + \
         [synth.token_rows(wl, [t], "h", token_set=s) for s, t in rot]
    xx = [synth.token_rows(wl, [t], "x") for t in rows] + \
         [synth.token_rows(wl, [t], "x", token_set=s) for s, t in rot]
    wpost, wpre = synth.norm_weight(wl, "post"), synth.norm_weight(wl, "pre")
    Wr, bias = synth.router_weight(wl), synth.router_bias(wl)
    if wl.name.startswith("dense"):
        W = synth.expert_weights(wl, 0)

        def one_dense(i):
            _, z = oracle.boundary(hh[i], xx[i], wpost, wpre, wl.n, wl.eps)
            return oracle.dense_swiglu(z, *W)

        t0 = time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one_dense, range(len(hh))))
        dt = time.perf_counter() - t0
        log(f"cpu baseline: {len(hh)} tokens in {dt:.2f}s on {threads} threads")
        return dict(value=round(len(hh) / dt, 3), unit="tokens/s", cores=threads, kind="oracle",
                    sample=f"{len(hh)} tokens of {wl.name}, each through the boundary and the "
                           f"dense SwiGLU layer single-threaded, {threads} tokens at a time; "
                           f"{dt:.1f} s wall")
    # routing first (cheap) to know which experts to draw; drawing inputs is not timed
    zs, routes = [], []
    for h, x in zip(hh, xx):
        _, z = oracle.boundary(h, x, wpost, wpre, wl.n, wl.eps)
        ids, w, _, _ = oracle.topk(oracle.router(z, Wr), bias, wl.G, wl.kg, wl.k, wl.scale)
        zs.append(z)
        routes.append(ids)
    need = sorted(set(int(e) for r in routes for e in r.ravel()))
    log(f"cpu baseline: drawing {len(need)} experts for {len(hh)} tokens")
    weights = {e: synth.expert_weights(wl, e) for e in need}  # each draw is threaded
    if mxfp4:
        def quant(e):
            return e, tuple(oracle.mxfp4_dequantize(*oracle.mxfp4_quantize(m)) for m in weights[e])
        with ThreadPoolExecutor(threads) as ex:
            for i, (e, ws) in enumerate(ex.map(quant, need)):
                weights[e] = ws
                if i % 16 == 15 or i + 1 == len(need):
                    log(f"cpu baseline: quantised {i + 1} of {len(need)} experts")

    def one(i):
        out = oracle.sublayer(hh[i], xx[i], wpost, wpre, wl.n, wl.eps, Wr, bias, wl.G, wl.kg,
                              wl.k, wl.scale, weights.__getitem__)
        return out["y"]

    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(len(hh))))
    dt = time.perf_counter() - t0
    log(f"cpu baseline: {len(hh)} tokens in {dt:.2f}s on {threads} threads")
    return dict(value=round(len(hh) / dt, 3), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{len(hh)} tokens of {wl.name}{' (mxfp4 experts)' if mxfp4 else ''}, "
                       f"each through the whole path "
                       f"(boundary, FP32 router, grouped top-k, {wl.k} SwiGLU experts, combine) "
                       f"single-threaded, {threads} tokens at a time; {dt:.1f} s wall")


if __name__ == "__main__":
    main()
