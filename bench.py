"""Benchmark: the Beam MoE sublayer (routed MoE FFN + one sublayer boundary) on one MI355X.

A step is one pass of the whole path over one batch of T tokens: the MoE FFN
(FP32 router, grouped top-k, expert grouping, BF16 SwiGLU experts, weighted
combine) and one sublayer boundary (post-norm, depth-scaled residual, pre-norm).
By default (--step boundary-last) it is beam_moe_forward_boundary: the MoE on z,
then the next sublayer's boundary fused into the combine, as a decode loop runs
it; --step boundary-first times beam_sublayer_forward (the boundary, then the MoE
on its z). Both are bit-identical to the separate calls. Inputs are seeded
synthetic tensors already resident in HBM when the timed region starts; decode
steps rotate over distinct token sets so the experts touched change from step to
step.

Without --workload the run measures every configuration of the metric in one
process — batch-1 decode (the headline `value`), decode batches of 32 and 128,
the 8 x 2048-token prefill and the skewed 32K-token prefill — on two layer
handles (the uniform and the skewed router bias) built once from the same
weights; each gets an entry under config.workloads. --workload X measures X
alone (what the rocprofv3 traces run).

Prints one JSON line. `value` is tokens per second for the whole job;
`roofline` reports the dominant kernel (expert gate/up) against HBM (decode) or
BF16 matrix-core (prefill) peak, from HIP events recorded around that kernel on
its own stream during a timed region; `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense BF16 matrix cores
FP4_PEAK_TFLOPS = 10100.0    # MI355X dense FP4 matrix cores
STREAM_MAX_T = 128           # largest batch the library serves with its weight-streaming passes
METRIC = "MoE-layer tokens/s (decode T=1/32/128, prefill 16K) + % HBM/MFMA peak"
SUITE = ("decode1", "decode32", "decode128", "prefill16k", "skew32k")


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default=None,
                   choices=["decode1", "decode32", "decode128", "prefill16k", "skew32k",
                            "skew32k_half", "tiny", "dense1", "dense16k"],
                   help="measure one workload only (default: every configuration of the "
                        "metric). dense1 / dense16k: Beam's dense SwiGLU layer (d_ff 20480) "
                        "instead of the MoE; a step is that layer, then the next boundary")
    p.add_argument("--rotations", type=int, default=None, help="distinct token sets")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--step", choices=("boundary-first", "boundary-last", "chain"),
                   default="boundary-last",
                   help="boundary-first: beam_sublayer_forward (the boundary, then the MoE on its z); "
                        "boundary-last: beam_moe_forward_boundary (the MoE on a z computed before the "
                        "timed region, then the next sublayer's boundary fused into the combine); "
                        "chain: beam_moe_forward_boundary_route in a decode loop (each step's h', z' "
                        "feed the next step, whose routing the step computes after its boundary)")
    p.add_argument("--cpu-sample", type=int, default=None, help="tokens in the CPU sample")
    p.add_argument("--experts", choices=("bf16", "mxfp4"), default="bf16",
                   help="expert weight format: BF16, or MXFP4 (4-bit E2M1 codes with one E8M0 "
                        "scale per 32 values, quantised on the device from the BF16 weights; "
                        "BF16 activations)")
    p.add_argument("--act", choices=("bf16", "mxfp4"), default="bf16",
                   help="activation format of the expert GEMMs: BF16, or MXFP4 (4-bit activations "
                        "on the FP4 matrix cores; needs --experts mxfp4)")
    p.add_argument("--no-peaks", action="store_true",
                   help="skip measuring the copy and vendor-GEMM references on this GPU")
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


def measured_peaks(reps: int = 5):
    """What this GPU itself reaches, reported beside the published peaks: a plain
    device-to-device copy of 1 GiB (bytes read + bytes written per second) and the vendor
    BF16 GEMM (torch.matmul, hipBLASLt) on 8192 x 8192 x 8192 random operands; each the
    fastest of `reps` timed runs after one untimed run."""
    import torch

    def best_ms(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return min(ts)

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    copy_gbs = 2 * n / (best_ms(lambda: dst.copy_(src)) * 1e-3) / 1e9
    del src, dst
    m = 8192
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn((m, m), device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn((m, m), device="cuda", dtype=torch.bfloat16, generator=g)
    gemm_tf = 2.0 * m ** 3 / (best_ms(lambda: torch.matmul(a, b)) * 1e-3) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"hbm_copy_GBps": round(copy_gbs, 1), "bf16_gemm_TFLOPs": round(gemm_tf, 1),
            "what": "1 GiB device copy (read + write bytes); torch.matmul BF16 8192^3 (hipBLASLt)"}


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed (the sources hold no
    string literal with a comment marker inside)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(unit):
    """Hash of the code (comments and layout aside) of a kernel source file and every local
    header it includes (transitively): a committed counter summary applies only while this
    is unchanged."""
    csrc = os.path.join(ROOT, "sparse_moe_decoder_amd", "csrc")
    seen, todo = [], [unit]
    while todo:
        n = todo.pop(0)
        if n in seen:
            continue
        seen.append(n)
        with open(os.path.join(csrc, n)) as fh:
            for line in fh:
                m = re.match(r'\s*#include\s+"([^"]+)"', line)
                if m and os.path.exists(os.path.join(csrc, m.group(1))):
                    todo.append(m.group(1))
    h = hashlib.sha256()
    for n in sorted(seen):
        with open(os.path.join(csrc, n)) as fh:
            h.update(n.encode() + b"\0" + _code_only(fh.read()).encode())
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


class GraphMismatch(RuntimeError):
    pass


def timed(step, n):
    """Mean ms per call of step(i), i < n, between two events on the current stream."""
    import torch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def measure(wl, moe, dense_h, args, mx):
    """Time one workload on an existing handle; returns its entry (dict)."""
    import numpy as np
    import torch

    import sparse_moe_decoder_amd as beam
    from synth import device as sd

    T = wl.T
    decode = T <= STREAM_MAX_T
    dense = dense_h is not None
    steps = args.steps or (200 if decode else 10)
    warmup = args.warmup if args.warmup is not None else (20 if decode else 3)
    R = args.rotations or (32 if decode else 1)
    log(f"workload {wl.name}: T={T} d={wl.d} E={wl.E} f={wl.f}; steps {steps} warmup {warmup} "
        f"rotations {R}")
    wpost, wpre = sd.norm_weights(wl)
    hs = [sd.tokens(wl, "h", token_set=s) for s in range(R)]
    xs = [sd.tokens(wl, "x", token_set=s) for s in range(R)]
    h_out = torch.empty((T, wl.d), dtype=torch.bfloat16, device="cuda")
    z = torch.empty_like(h_out)
    y = torch.empty_like(h_out)
    # each token set's z from its boundary, before the timed region
    z_in = [beam.beam_sublayer_norm_residual(hs[s], xs[s], wpost, wpre, wl.n, wl.eps)[1]
            for s in range(R)]

    if dense:
        def step(i):  # the dense layer, then the next boundary with its output as the branch
            s = i % R
            beam.beam_dense_forward(dense_h, z_in[s], y)
            beam.beam_sublayer_norm_residual(hs[s], y, wpost, wpre, wl.n, wl.eps, h_out=h_out,
                                             z_out=z)
    elif args.step == "chain":
        # a decode loop: h and z are updated in place; each step runs the MoE on z with the
        # routing the previous step left, then the combine, the boundary and the next routing
        hc, zc = hs[0].clone(), z_in[0].clone()

        def chain_call(routed):
            beam.beam_moe_forward_boundary_route(moe.handle, moe.handle, zc, hc, wpost, wpre,
                                                 wl.n, wl.eps, h_out=hc, z_out=zc, routed=routed)

        def step(i):
            chain_call(True)
    elif args.step == "boundary-first":
        def step(i):
            s = i % R
            beam.beam_sublayer_forward(moe.handle, hs[s], xs[s], wpost, wpre, wl.n, wl.eps, y,
                                       h_out=h_out, z_out=z)
    else:
        def step(i):  # the MoE on z, then the next boundary (x = the MoE output)
            s = i % R
            beam.beam_moe_forward_boundary(moe.handle, z_in[s], hs[s], wpost, wpre, wl.n, wl.eps,
                                           h_out=h_out, z_out=z)
    last_out = (y if (args.step == "boundary-first" and not dense)
                else zc if (args.step == "chain" and not dense) else z)

    # distinct experts per token set (for the algorithmic byte count) and rows per expert
    distinct, max_rows, hot_share = [1], None, None
    if not dense:
        distinct = []
        ids_buf = torch.empty((T, wl.k), dtype=torch.int32, device="cuda")
        w_buf = torch.empty((T, wl.k), dtype=torch.float32, device="cuda")
        for s in range(R):
            beam.beam_router_topk(moe.handle, z_in[s], ids_buf, w_buf)
            ids_np = ids_buf.cpu().numpy()
            distinct.append(len(np.unique(ids_np)))
        counts = np.bincount(ids_np.ravel(), minlength=wl.E)
        max_rows = int(counts.max())
        if wl.hot_experts:
            hot_share = round(float(counts[list(wl.hot_experts)].sum() / counts.sum()), 4)
    mean_distinct = float(np.mean(distinct))

    # 1) eager
    if args.step == "chain" and not dense:
        chain_call(False)  # the first step routes its own z (and leaves the next routing)
    for i in range(warmup):
        step(i)
    ms_eager = timed(step, steps)
    log(f"{wl.name} eager: {ms_eager * 1e3:.1f} us/step")

    # 2) HIP graph of one step per token set (no allocation, no host sync inside); its
    # result must equal the eager result bit for bit
    ms_graph, graph_ok = None, None
    if not args.no_graph:
        graphs = []
        try:
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
        except Exception as exc:  # capture not available: report the eager number
            log(f"{wl.name}: graph capture unavailable: {exc!r}")
            graphs = []
        if graphs:
            for i in range(warmup):
                graphs[i % R].replay()
            ms_graph = timed(lambda i: graphs[i % R].replay(), steps)
            log(f"{wl.name} graph: {ms_graph * 1e3:.1f} us/step")
            if args.step == "chain" and not dense:
                # from one saved state: the eager steps and (after the same priming step) a replay
                h_save, z_save = hc.clone(), zc.clone()
                chain_call(False)
                step(0)
                torch.cuda.synchronize()
                out_eager = last_out.clone()
                hc.copy_(h_save)
                zc.copy_(z_save)
                chain_call(False)
                graphs[0].replay()
            else:
                step(0)
                torch.cuda.synchronize()
                out_eager = last_out.clone()
                last_out.zero_()
                graphs[0].replay()
            torch.cuda.synchronize()
            graph_ok = bool(torch.equal(last_out.view(torch.int16), out_eager.view(torch.int16)))
            if not graph_ok:
                raise GraphMismatch(f"{wl.name}: graph replay differs from the eager step")
            del graphs

    # per-step spread: events around each eager step (a separate pass)
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

    # 3) per-kernel durations from HIP events around each launch, over a timed region
    beam.profile_reset()
    beam.profile_enable(True)
    ms_prof = timed(step, steps)
    beam.profile_enable(False)
    kern = beam.profile_read()
    beam.profile_reset()
    kernel_us = {k: (v[0] / v[1] * 1e3 if v[1] else None) for k, v in kern.items()}
    log(f"{wl.name} kernel avg us: " + ", ".join(f"{k} {v:.1f}" for k, v in kernel_us.items() if v))

    best_ms = ms_eager if ms_graph is None else min(ms_eager, ms_graph)
    mode = "hipgraph" if (ms_graph is not None and ms_graph <= ms_eager) else "eager"

    # roofline of the dominant kernel (expert gate/up)
    gu_us = kernel_us.get("gate_up")
    a4 = args.act == "mxfp4"
    a4_gemm = a4 and T > STREAM_MAX_T  # up to 128 tokens W4A4 runs on the 4-bit weight streams
    # the gate/up kernel's source file: W4A4 GEMMs, 4-bit weight streams, else experts.hip
    # (BF16 streams and grouped GEMMs, and the 4-bit-weight grouped GEMM)
    src = source_hash("experts_w4a4.hip" if a4_gemm
                      else "experts_mxfp4.hip" if (mx and T <= STREAM_MAX_T)
                      else "experts.hip")
    ctr_name = "gate_up_w4a4" if a4_gemm else "gate_up_mxfp4" if mx else "gate_up"
    wbytes = (0.5 + 1.0 / 32) if mx else 2.0  # bytes per expert weight (codes + scales)
    if decode:
        # algorithmic bytes per launch: each touched expert's gate+up weights once, the
        # token rows in, the activations out
        bytes_gu = mean_distinct * 2 * wl.f * wl.d * wbytes + T * wl.d * 2 + T * wl.k * wl.f * 2
        achieved = bytes_gu / (gu_us * 1e-6) / 1e9
        roof = dict(kernel="gate_up", bound="hbm", achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                    algorithmic_bytes=round(bytes_gu))
        roof["traffic"] = read_traffic(ctr_name, wl.name, src)
        step_bytes = (mean_distinct * 3 * wl.f * wl.d * wbytes + (0 if dense else wl.E * wl.d * 4)
                      + T * wl.d * 2 * 6 + T * wl.k * (wl.f * 4 + wl.d * 4))
        whole = dict(algorithmic_bytes=round(step_bytes), hbm_frac=round(
            step_bytes / (best_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))
    else:
        kk = 1 if dense else wl.k
        flops_gu = 2.0 * T * kk * (2 * wl.f) * wl.d
        achieved = flops_gu / (gu_us * 1e-6) / 1e12
        peak = FP4_PEAK_TFLOPS if a4_gemm else BF16_PEAK_TFLOPS  # the contraction's own dtype
        roof = dict(kernel="gate_up", bound="mfma", achieved=round(achieved, 1),
                    peak=peak, unit="TFLOP/s",
                    frac=round(achieved / peak, 4), algorithmic_flops=flops_gu)
        roof["traffic"] = read_traffic(ctr_name, wl.name, src)
        step_flops = 2.0 * T * kk * 3 * wl.f * wl.d
        gemm_us = gu_us + (kernel_us.get("down") or 0.0)
        whole = dict(expert_flops=step_flops,
                     mfma_frac=round(step_flops / (best_ms * 1e-3) / 1e12 / peak, 4),
                     expert_gemms_mfma_frac=round(
                         step_flops / (gemm_us * 1e-6) / 1e12 / peak, 4))
    entry = {
        "tokens": T, "ms_per_step": round(best_ms, 5), "tokens_per_s": round(T / (best_ms / 1e3), 2),
        "mode": mode, "ms_eager": round(ms_eager, 5),
        "ms_graph": None if ms_graph is None else round(ms_graph, 5),
        "graph_matches_eager": graph_ok, "ms_profiled": round(ms_prof, 5),
        "ms_per_step_eager_percentiles": pct, "steps": steps, "warmup": warmup,
        "token_sets": R, "distinct_experts_per_step": round(mean_distinct, 1),
        "kernel_us": {k: (None if v is None else round(v, 2)) for k, v in kernel_us.items()},
        "roofline": roof, "whole_step": whole,
    }
    if max_rows is not None:
        entry["max_rows_per_expert"] = max_rows
    if hot_share is not None:
        entry["hot_share"] = hot_share
    del hs, xs, z_in, h_out, z, y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return entry


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has "
              "no multi-GPU path; the per-GPU kernels are what one GPU shows.", file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    from synth import device as sd
    import sparse_moe_decoder_amd as beam

    torch.cuda.set_device(0)
    mx = args.experts == "mxfp4"
    if args.act == "mxfp4" and not mx:
        print("--act mxfp4 needs --experts mxfp4", file=sys.stderr)
        sys.exit(2)
    names = [args.workload] if args.workload else list(SUITE)
    wls = [synth.WORKLOADS[n] for n in names]
    dense = names[0].startswith("dense")
    if mx and dense:
        print("--experts mxfp4 applies to the MoE workloads", file=sys.stderr)
        sys.exit(2)
    head = wls[0]
    t0 = time.time()

    # one handle per router bias, each sized for the largest batch that uses it
    W, _ = sd.router(head)
    wg, wu, wd = sd.experts(head)
    fp4 = None
    if mx:
        fp4 = []
        for t in (wg, wu, wd):
            fp4 += list(beam.beam_mxfp4_quantize(t))
        fp4 = tuple(fp4)
    handles, dense_h = {}, None
    if dense:
        dense_h = beam.beam_dense_init(head.d, head.f, head.T, wg[0], wu[0], wd[0])
    else:
        for wl in wls:
            key = wl.hot_bias if wl.hot_experts else 0.0
            need = max(w.T for w in wls if (w.hot_bias if w.hot_experts else 0.0) == key)
            if key in handles:
                continue
            _, b = sd.router(wl)
            cfg = sd.moe_config(wl, max_tokens=need)
            handles[key] = (beam.BeamMoE(cfg, W, b, None, None, None, mxfp4=fp4) if mx
                            else beam.BeamMoE(cfg, W, b, wg, wu, wd))
            if args.act == "mxfp4":
                handles[key].set_activation_format(beam.ACT_MXFP4)
    del wg, wu, wd, fp4
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"setup {time.time() - t0:.1f}s ({len(handles) or 1} handle(s))")

    entries = {}
    try:
        for wl in wls:
            moe = None if dense else handles[wl.hot_bias if wl.hot_experts else 0.0]
            entries[wl.name] = measure(wl, moe, dense_h, args, mx)
    except GraphMismatch as exc:
        log(f"FAILED: {exc}")
        sys.exit(3)
    finally:
        for h in handles.values():
            h.close()
        if dense_h is not None:
            beam.beam_moe_destroy(dense_h)

    peaks = None
    if not args.no_peaks:
        peaks = measured_peaks()
        log(f"measured on this GPU: {peaks}")
        for ent in entries.values():
            r = ent["roofline"]
            ref = (peaks["hbm_copy_GBps"] if r["bound"] == "hbm"
                   else peaks["bf16_gemm_TFLOPs"] if r["peak"] == BF16_PEAK_TFLOPS else None)
            r["frac_of_measured"] = round(r["achieved"] / ref, 4) if ref else None
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(head, args.cpu_sample, mxfp4=mx, act4=args.act == "mxfp4")

    e = entries[head.name]
    config = {
        "workload": head.name, "tokens": head.T, "hidden": head.d, "experts": head.E,
        "groups": head.G, "groups_kept": head.kg, "topk": head.k, "d_ff": head.f,
        "experts_format": args.experts, "activations_format": args.act, "step": args.step,
    }
    config.update({k: v for k, v in e.items() if k != "roofline"})
    if len(entries) > 1:
        config["workloads"] = entries
    out = {
        "metric": METRIC,
        "value": e["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": e["steps"],
        "warmup": e["warmup"],
        "ms_per_step": e["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp4 (4-bit activations and weights, FP32 accumulation)" if args.act == "mxfp4"
                  else "bf16 (mxfp4 expert weights)" if mx else "bf16"),
        "data": "synthetic (seeded counter-based generator; random-init weights of Beam's MoE layer)",
        "config": config,
        "roofline": e["roofline"],
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(wl, sample=None, mxfp4=False, act4=False):
    """The CPU oracle, as it is, on a bounded sample of the same workload: each
    sampled token goes through boundary, router, routing, its experts and the
    combine, single-threaded per token; tokens run in a thread pool of the host's CPU
    share, and a few tokens also run alone on one thread (the single-core figure).
    With mxfp4 the experts' weights are the oracle's MXFP4 quantisation, dequantised
    (not timed)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import synth

    threads = max(1, min(16, os.cpu_count() or 1))
    light = mxfp4 or wl.name.startswith("dense")
    n = sample or (2 * threads if light else 16 * threads)
    n1 = max(2, n // (2 * threads))  # tokens timed on one thread
    rows = list(range(min(n, wl.T)))
    rot = []
    if len(rows) < n:  # decode: also take tokens of the rotation sets
        extra = n - len(rows)
        rot = [(s, t) for s in range(1, 1 + (extra + wl.T - 1) // wl.T) for t in range(wl.T)]
        rot = rot[:extra]
    hh = [synth.token_rows(wl, [t], "h") for t in rows] + \
         [synth.token_rows(wl, [t], "h", token_set=s) for s, t in rot]
    xx = [synth.token_rows(wl, [t], "x") for t in rows] + \
         [synth.token_rows(wl, [t], "x", token_set=s) for s, t in rot]
    wpost, wpre = synth.norm_weight(wl, "post"), synth.norm_weight(wl, "pre")
    Wr, bias = synth.router_weight(wl), synth.router_bias(wl)
    if wl.name.startswith("dense"):
        W = synth.expert_weights(wl, 0)

        def one(i):
            _, z = oracle.boundary(hh[i], xx[i], wpost, wpre, wl.n, wl.eps)
            return oracle.dense_swiglu(z, *W)
        what = "the boundary and the dense SwiGLU layer"
    else:
        # routing first (cheap) to know which experts to draw; drawing inputs is not timed
        routes = []
        for h, x in zip(hh, xx):
            _, z = oracle.boundary(h, x, wpost, wpre, wl.n, wl.eps)
            ids, w, _, _ = oracle.topk(oracle.router(z, Wr), bias, wl.G, wl.kg, wl.k, wl.scale)
            routes.append(ids)
        need = sorted(set(int(e) for r in routes for e in r.ravel()))
        log(f"cpu baseline: drawing {len(need)} experts for {len(hh)} tokens")
        weights = {e: synth.expert_weights(wl, e) for e in need}  # each draw is threaded
        if mxfp4:
            def quant(e):
                return e, tuple(oracle.mxfp4_dequantize(*oracle.mxfp4_quantize(m))
                                for m in weights[e])
            with ThreadPoolExecutor(threads) as ex:
                for i, (e, ws) in enumerate(ex.map(quant, need)):
                    weights[e] = ws
                    if i % 16 == 15 or i + 1 == len(need):
                        log(f"cpu baseline: quantised {i + 1} of {len(need)} experts")

        def one(i):
            _, z = oracle.boundary(hh[i], xx[i], wpost, wpre, wl.n, wl.eps)
            ids, w, _, _ = oracle.topk(oracle.router(z, Wr), bias, wl.G, wl.kg, wl.k, wl.scale)
            return oracle.moe_experts(z, ids, w, wl.E, weights.__getitem__, mx_act=act4)[0]
        what = (f"the whole path (boundary, FP32 router, grouped top-k, {wl.k} SwiGLU experts, "
                f"combine)")

    t0 = time.perf_counter()
    for i in range(n1):
        one(i)
    dt1 = time.perf_counter() - t0
    log(f"cpu baseline: {n1} tokens in {dt1:.2f}s on one thread")
    t0 = time.perf_counter()
    done = 0
    with ThreadPoolExecutor(threads) as ex:
        for _ in ex.map(one, range(len(hh))):
            done += 1
            if done % (4 * threads) == 0:
                log(f"cpu baseline: {done} of {len(hh)} tokens")
    dt = time.perf_counter() - t0
    log(f"cpu baseline: {len(hh)} tokens in {dt:.2f}s on {threads} threads")
    fmt = " (mxfp4 activations and experts)" if act4 else " (mxfp4 experts)" if mxfp4 else ""
    return dict(value=round(len(hh) / dt, 3), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{len(hh)} tokens of {wl.name}{fmt}, each through {what} "
                       f"single-threaded, {threads} tokens at a time; {dt:.1f} s wall",
                single_core=dict(value=round(n1 / dt1, 3), unit="tokens/s", cores=1,
                                 sample=f"{n1} tokens of {wl.name}{fmt} one after another on "
                                        f"one thread; {dt1:.1f} s"))


if __name__ == "__main__":
    main()
