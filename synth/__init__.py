"""Seeded synthetic inputs for the Beam MoE sublayer (input plumbing only).

This module holds no arithmetic of the method. It defines the workload table and
draws every input tensor from one counter-based generator (SplitMix64 streams,
Box-Muller normals; the definition is in ``synth.c``), with a host
implementation (``libbeam_synth.so``, built from ``synth.c`` by gcc) and a device
twin (``libbeam_synth_gpu.so``, built from ``synth_gpu.hip``). Both the CPU
oracle and the GPU path take their inputs from here; neither one's code is used.

Distributions follow the workload descriptions: h, x ~ N(0, 1) in BF16; RMSNorm
weights 1 + U(-0.1, 0.1) in BF16; router W ~ N(0, std 1/sqrt(d)) in FP32;
correction bias U(-0.01, 0.01) in FP32 (hot experts of the skewed workload get
a fixed bias instead); expert weights ~ N(0, std 0.02) in BF16.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
CPU_LIB_PATH = os.path.join(_HERE, "libbeam_synth.so")
GPU_LIB_PATH = os.path.join(_HERE, "libbeam_synth_gpu.so")

# tensor ids of the counter-based streams
T_H, T_X, T_WPOST, T_WPRE, T_WR, T_BIAS, T_WG, T_WU, T_WD = 1, 2, 3, 4, 5, 6, 7, 8, 9
T_H_ROT, T_X_ROT = 10, 11  # extra decode token sets (rotation), set s >= 1
T_LOGITS = 12  # synthetic router logits for routing-only tests


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    G: int
    kg: int
    k: int
    f: int
    n: int = 20
    eps: float = 1e-6
    scale: float = 2.5
    seed: int = 0
    hot_experts: tuple = ()
    hot_bias: float = 0.0
    note: str = ""

    @property
    def gs(self) -> int:
        return self.E // self.G

    def with_tokens(self, T: int) -> "Workload":
        return replace(self, T=T, name=f"{self.name}@T{T}")


def _beam(name, T, **kw):
    return Workload(name=name, T=T, d=5120, E=256, G=8, kg=4, k=8, f=2560, **kw)


def _dense(name, T, **kw):
    # a dense SwiGLU layer (Beam's layers 0-2) as one expert that every token takes
    return Workload(name=name, T=T, d=5120, E=1, G=1, kg=1, k=1, f=20480, scale=1.0, **kw)


HOT16 = tuple(range(0, 256, 16))  # two per group of 32: balanced across groups

WORKLOADS = {
    "tiny": Workload("tiny", T=8, d=512, E=32, G=8, kg=4, k=8, f=256,
                     note="tiny sublayer: 8 tokens, d 512, 32 experts in 8 groups of 4, d_ff 256"),
    "decode1": _beam("decode1", 1, note="batch-1 decode"),
    "decode32": _beam("decode32", 32, note="decode batch of 32 tokens"),
    "decode128": _beam("decode128", 128, note="decode batch of 128 tokens"),
    "prefill16k": _beam("prefill16k", 16384, note="prefill 8 x 2048 tokens"),
    "skew32k": _beam("skew32k", 32768, hot_experts=HOT16, hot_bias=0.5,
                     note="skewed long prefill: 16 hot experts at bias +0.5"),
    "dense1": _dense("dense1", 1, note="dense SwiGLU layer (d_ff 20480), batch-1 decode"),
    "dense16k": _dense("dense16k", 16384, note="dense SwiGLU layer (d_ff 20480), prefill 8 x 2048"),
    "skew32k_half": _beam("skew32k_half", 32768, hot_experts=HOT16, hot_bias=0.255,
                          note="skewed long prefill: bias +0.255 (about half the assignments hot)"),
}

# ---------------------------------------------------------------------------------------------
# host generator


_cpu_lib = None


def cpu_lib():
    global _cpu_lib
    if _cpu_lib is None:
        if not os.path.exists(CPU_LIB_PATH):
            build_cpu()
        lib = ctypes.CDLL(CPU_LIB_PATH)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        for name in ("synth_normal_f32", "synth_normal_bf16", "synth_uniform_f32",
                     "synth_uniform_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [u64, u64, u64, i64, dbl, dbl, vp]
            fn.restype = None
        lib.synth_raw_u64.argtypes = [u64, u64, u64, i64, vp]
        lib.synth_raw_u64.restype = None
        _cpu_lib = lib
    return _cpu_lib


def build_cpu() -> str:
    import subprocess
    src = os.path.join(_HERE, "synth.c")
    tmp = CPU_LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", src, "-o", tmp,
                           "-lm"])
    os.replace(tmp, CPU_LIB_PATH)
    return CPU_LIB_PATH


def build_gpu() -> str:
    import subprocess
    src = os.path.join(_HERE, "synth_gpu.hip")
    tmp = GPU_LIB_PATH + ".tmp"
    subprocess.check_call(["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           src, "-o", tmp])
    os.replace(tmp, GPU_LIB_PATH)
    return GPU_LIB_PATH


_POOL_THREADS = max(1, min(16, os.cpu_count() or 1))


def _fill(fn_name, dtype, seed, tensor, start, n, a, b, threads=None):
    out = np.empty(int(n), dtype=dtype)
    fn = getattr(cpu_lib(), fn_name)
    threads = threads or _POOL_THREADS
    chunk = 1 << 22
    if n <= chunk or threads == 1:
        fn(seed, tensor, start, n, a, b, out.ctypes.data)
        return out
    # every element is drawn on its own, so chunks are independent
    starts = list(range(0, int(n), chunk))

    def run(s):
        m = min(chunk, int(n) - s)
        fn(seed, tensor, start + s, m, a, b, out.ctypes.data + s * out.itemsize)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, starts))
    return out


def normal_bf16(seed, tensor, start, n, std=1.0, mean=0.0):
    return _fill("synth_normal_bf16", np.uint16, seed, tensor, start, n, mean, std)


def normal_f32(seed, tensor, start, n, std=1.0, mean=0.0):
    return _fill("synth_normal_f32", np.float32, seed, tensor, start, n, mean, std)


def uniform_bf16(seed, tensor, start, n, lo, hi):
    return _fill("synth_uniform_bf16", np.uint16, seed, tensor, start, n, lo, hi)


def uniform_f32(seed, tensor, start, n, lo, hi):
    return _fill("synth_uniform_f32", np.float32, seed, tensor, start, n, lo, hi)


def raw_u64(seed, tensor, start, n):
    out = np.empty(int(n), dtype=np.uint64)
    cpu_lib().synth_raw_u64(seed, tensor, start, n, out.ctypes.data)
    return out


# ----- per-tensor recipes (host) -----------------------------------------------------------------

def token_rows(wl: Workload, rows, which: str, token_set: int = 0) -> np.ndarray:
    """Rows of h ('h') or x ('x') as BF16 bits [len(rows), d]; token_set > 0 draws a rotation set."""
    rows = np.asarray(rows, dtype=np.int64)
    d = wl.d
    if token_set == 0:
        tid, base_row = (T_H if which == "h" else T_X), 0
    else:
        tid, base_row = (T_H_ROT if which == "h" else T_X_ROT), (token_set - 1) * wl.T
    out = np.empty((len(rows), d), dtype=np.uint16)
    if len(rows) and np.all(np.diff(rows) == 1):
        out[:] = normal_bf16(wl.seed, tid, (base_row + int(rows[0])) * d, len(rows) * d).reshape(-1, d)
        return out
    for i, t in enumerate(rows):
        out[i] = normal_bf16(wl.seed, tid, (base_row + int(t)) * d, d)
    return out


def norm_weight(wl: Workload, which: str) -> np.ndarray:
    tid = T_WPOST if which == "post" else T_WPRE
    return uniform_bf16(wl.seed, tid, 0, wl.d, 0.9, 1.1)


def router_weight(wl: Workload) -> np.ndarray:
    """[E, d] FP32, N(0, std 1/sqrt(d))."""
    return normal_f32(wl.seed, T_WR, 0, wl.E * wl.d, std=1.0 / np.sqrt(wl.d)).reshape(wl.E, wl.d)


def router_bias(wl: Workload) -> np.ndarray:
    b = uniform_f32(wl.seed, T_BIAS, 0, wl.E, -0.01, 0.01)
    for e in wl.hot_experts:
        b[e] = np.float32(wl.hot_bias)
    return b


def expert_weights(wl: Workload, e: int):
    """(Wg [f, d], Wu [f, d], Wd [d, f]) BF16 bits for expert e."""
    fd = wl.f * wl.d
    wg = normal_bf16(wl.seed, T_WG, e * fd, fd, std=0.02).reshape(wl.f, wl.d)
    wu = normal_bf16(wl.seed, T_WU, e * fd, fd, std=0.02).reshape(wl.f, wl.d)
    wd = normal_bf16(wl.seed, T_WD, e * fd, fd, std=0.02).reshape(wl.d, wl.f)
    return wg, wu, wd


def synthetic_logits(wl: Workload, T: int, seed: int = 0, std: float = 1.0) -> np.ndarray:
    """FP32 router logits drawn directly (routing-only tests), [T, E]."""
    return normal_f32(seed, T_LOGITS, 0, T * wl.E, std=std).reshape(T, wl.E)


# ---------------------------------------------------------------------------------------------
# device generator (raw device pointers; the caller owns the memory)

_gpu_lib = None


def gpu_lib():
    global _gpu_lib
    if _gpu_lib is None:
        if not os.path.exists(GPU_LIB_PATH):
            raise RuntimeError(f"{GPU_LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(GPU_LIB_PATH)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        for name in ("synth_gpu_normal_f32", "synth_gpu_normal_bf16", "synth_gpu_uniform_f32",
                     "synth_gpu_uniform_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, u64, u64, u64, i64, dbl, dbl, vp]
            fn.restype = ctypes.c_int
        _gpu_lib = lib
    return _gpu_lib


def _gpu_call(name, ptr, seed, tensor, start, n, a, b, stream):
    rc = getattr(gpu_lib(), name)(ptr, seed, tensor, start, n, a, b, stream)
    if rc != 0:
        raise RuntimeError(f"{name} failed with {rc}")


def gpu_normal_bf16(ptr, seed, tensor, start, n, std=1.0, mean=0.0, stream=None):
    _gpu_call("synth_gpu_normal_bf16", ptr, seed, tensor, start, n, mean, std, stream)


def gpu_normal_f32(ptr, seed, tensor, start, n, std=1.0, mean=0.0, stream=None):
    _gpu_call("synth_gpu_normal_f32", ptr, seed, tensor, start, n, mean, std, stream)


def gpu_uniform_bf16(ptr, seed, tensor, start, n, lo, hi, stream=None):
    _gpu_call("synth_gpu_uniform_bf16", ptr, seed, tensor, start, n, lo, hi, stream)


def gpu_uniform_f32(ptr, seed, tensor, start, n, lo, hi, stream=None):
    _gpu_call("synth_gpu_uniform_f32", ptr, seed, tensor, start, n, lo, hi, stream)
