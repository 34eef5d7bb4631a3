"""CPU oracle for the Beam MoE sublayer — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It wraps ``liboracle.so`` (built by gcc
from ``beam_oracle.c``, a plain single-threaded C implementation) with numpy
marshalling. It shares no code with the GPU library and imports nothing from it.

BF16 tensors are numpy ``uint16`` arrays holding the bit patterns.

Parity status of each step (how it is pinned is listed in ``tests/test_oracle_pins.py``):
  O1 boundary ........ pinned (closed forms, n = 1 identity, unit-variance invariant; the
                        BF16 post-norm output on rows with an exact norm factor)
  O2 router .......... pinned (one-hot rows, exact small-integer sums, FP64 error bound)
  O3 grouped top-k ... pinned (brute-force enumeration, forced ties, sum of weights; the
                        sigmoid equals the FP32 rounding of a 50-digit evaluation)
  O4 permutation ..... pinned (brute-force sort of (expert, slot) pairs)
  O5/O6 experts ...... pinned (permutation-matrix closed forms, one-expert dense SwiGLU x 2.5,
                        all-experts dense mixture, FP64 error bound)
  O7 MXFP4 weights ... pinned (hand-derived blocks from the OCP MX v1.0 definitions: scale
                        rule, every rounding tie, saturation, signed zero; exact round trip
                        of representable blocks; the half-step error bound; sign symmetry)
  O8 4-bit act. ...... pinned (permutation-matrix closed forms over hand-derived MXFP4
                        blocks: z and act quantised per row along their contraction, not
                        g, u or y; identity on representable rows; the half-step bound)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "beam_oracle.c")


def build() -> str:
    """Compile the oracle with gcc (strict FP: no contraction, no fast-math)."""
    tmp = LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           "-Wall", "-fPIC", "-shared", SRC_PATH, "-o", tmp, "-lm"])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
        L.oracle_bf16.argtypes = [f32]
        L.oracle_bf16.restype = ctypes.c_uint16
        L.oracle_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f32.restype = f32
        L.oracle_sigmoid.argtypes = [f32]
        L.oracle_sigmoid.restype = f32
        L.oracle_silu.argtypes = [f32]
        L.oracle_silu.restype = f32
        L.oracle_boundary.argtypes = [i64, i64, vp, vp, vp, vp, i64, f32, vp, vp]
        L.oracle_router.argtypes = [i64, i64, i64, vp, vp, vp]
        L.oracle_topk.argtypes = [i64, i64, i64, i64, i64, f32, vp, vp, vp, vp, vp, vp]
        L.oracle_permute.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp]
        L.oracle_expert_rows.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.oracle_combine.argtypes = [i64, i64, i64, i64, vp, vp, vp]
        L.oracle_mxfp4_quantize.argtypes = [i64, i64, vp, vp, vp]
        L.oracle_mxfp4_dequantize.argtypes = [i64, i64, vp, vp, vp]
        L.oracle_expert_rows_mx.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp]
        L.oracle_expert_act.argtypes = [i64, i64, i64, vp, vp, vp, vp]
        L.oracle_expert_down.argtypes = [i64, i64, i64, vp, vp, vp, vp]
        for name in ("oracle_boundary", "oracle_router", "oracle_topk", "oracle_permute",
                     "oracle_expert_rows", "oracle_combine", "oracle_mxfp4_quantize",
                     "oracle_mxfp4_dequantize", "oracle_expert_rows_mx", "oracle_expert_act",
                     "oracle_expert_down"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} returned {rc}")


# ---- scalar helpers (for pins) -------------------------------------------------------------------

def bf16(v: float) -> int:
    return int(lib().oracle_bf16(float(v)))


def f32(b: int) -> float:
    return float(lib().oracle_f32(int(b)))


def sigmoid(v: float) -> float:
    return float(lib().oracle_sigmoid(float(v)))


def silu(v: float) -> float:
    return float(lib().oracle_silu(float(v)))


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns (numpy, for test comparisons)."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---- O1..O6 ------------------------------------------------------------------------------------

def boundary(h, x, w_post, w_pre, n, eps):
    h, x = _c(h, np.uint16), _c(x, np.uint16)
    T, d = h.shape
    ho = np.empty_like(h)
    zo = np.empty_like(h)
    _check(lib().oracle_boundary(T, d, _p(h), _p(x), _p(_c(w_post, np.uint16)),
                                 _p(_c(w_pre, np.uint16)), int(n), float(eps), _p(ho), _p(zo)),
           "oracle_boundary")
    return ho, zo


def router(z, W):
    z, W = _c(z, np.uint16), _c(W, np.float32)
    T, d = z.shape
    E = W.shape[0]
    assert W.shape[1] == d
    out = np.empty((T, E), dtype=np.float32)
    _check(lib().oracle_router(T, d, E, _p(z), _p(W), _p(out)), "oracle_router")
    return out


def router_threaded(z, W, threads=8):
    """Same arithmetic per row as router(); rows split across threads."""
    z = _c(z, np.uint16)
    T = z.shape[0]
    if T <= 1 or threads <= 1:
        return router(z, W)
    chunks = np.array_split(np.arange(T), min(threads, T))
    with ThreadPoolExecutor(len(chunks)) as ex:
        parts = list(ex.map(lambda c: router(z[c[0]:c[-1] + 1], W), chunks))
    return np.concatenate(parts, axis=0)


def topk(logits, bias, G, kg, k, scale):
    logits, bias = _c(logits, np.float32), _c(bias, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    ggap = np.empty(T, dtype=np.float32)
    egap = np.empty(T, dtype=np.float32)
    _check(lib().oracle_topk(T, E, G, kg, k, float(scale), _p(logits), _p(bias), _p(ids), _p(w),
                             _p(ggap), _p(egap)), "oracle_topk")
    return ids, w, ggap, egap


def permute(ids, E):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(T * k, dtype=np.int32)
    inv = np.empty(T * k, dtype=np.int32)
    _check(lib().oracle_permute(T, k, E, _p(ids), _p(counts), _p(offsets), _p(perm), _p(inv)),
           "oracle_permute")
    return counts, offsets, perm, inv


def expert_rows(zrows, Wg, Wu, Wd, wrow):
    zrows = _c(zrows, np.uint16)
    R, d = zrows.shape
    f = Wg.shape[0]
    assert Wg.shape == (f, d) and Wu.shape == (f, d) and Wd.shape == (d, f)
    out = np.empty((R, d), dtype=np.uint16)
    _check(lib().oracle_expert_rows(R, d, f, _p(zrows), _p(_c(Wg, np.uint16)),
                                    _p(_c(Wu, np.uint16)), _p(_c(Wd, np.uint16)),
                                    _p(_c(wrow, np.float32)), _p(out)), "oracle_expert_rows")
    return out


def expert_rows_mx(zrows, Wg, Wu, Wd, wrow):
    """O8: O5 with the token rows and the activation rows MXFP4-quantised (O7, blocks of 32
    along each GEMM's contraction) and used at their dequantised values."""
    zrows = _c(zrows, np.uint16)
    R, d = zrows.shape
    f = Wg.shape[0]
    assert Wg.shape == (f, d) and Wu.shape == (f, d) and Wd.shape == (d, f)
    out = np.empty((R, d), dtype=np.uint16)
    _check(lib().oracle_expert_rows_mx(R, d, f, _p(zrows), _p(_c(Wg, np.uint16)),
                                       _p(_c(Wu, np.uint16)), _p(_c(Wd, np.uint16)),
                                       _p(_c(wrow, np.float32)), _p(out)), "oracle_expert_rows_mx")
    return out


def expert_act(zrows, Wg, Wu):
    """O5's first half: act [R, f] = bf16(silu(bf16(z Wg^T)) * bf16(z Wu^T))."""
    zrows = _c(zrows, np.uint16)
    R, d = zrows.shape
    f = Wg.shape[0]
    assert Wg.shape == (f, d) and Wu.shape == (f, d)
    out = np.empty((R, f), dtype=np.uint16)
    _check(lib().oracle_expert_act(R, d, f, _p(zrows), _p(_c(Wg, np.uint16)),
                                   _p(_c(Wu, np.uint16)), _p(out)), "oracle_expert_act")
    return out


def expert_down(act, Wd, wrow):
    """O5's second half: yk [R, d] = bf16(wrow * (act Wd^T))."""
    act = _c(act, np.uint16)
    R, f = act.shape
    d = Wd.shape[0]
    assert Wd.shape == (d, f)
    out = np.empty((R, d), dtype=np.uint16)
    _check(lib().oracle_expert_down(R, d, f, _p(act), _p(_c(Wd, np.uint16)),
                                    _p(_c(wrow, np.float32)), _p(out)), "oracle_expert_down")
    return out


def dense_swiglu(z, Wg, Wu, Wd):
    """A dense SwiGLU MLP layer ([vLLM page, §Modellarchitektur]: Beam's layers 0-2, d_ff
    20480) on rows z [T, d]: O5 with routing weight 1, i.e. g = bf16(z.Wg^T), u = bf16(z.Wu^T),
    act = bf16(silu(g) * u), y = bf16(act.Wd^T) (1 * acc is exact). Reading: the dense layer
    keeps the experts' rounding points."""
    z = _c(z, np.uint16)
    return expert_rows(z, Wg, Wu, Wd, np.ones(z.shape[0], dtype=np.float32))


def combine(yk, ids=None, E=None):
    yk = _c(yk, np.uint16)
    T, k, d = yk.shape
    y = np.empty((T, d), dtype=np.uint16)
    if ids is not None:
        ids = _c(ids, np.int32)
    _check(lib().oracle_combine(T, k, d, int(E if E is not None else 1 << 30), _p(ids), _p(yk),
                                _p(y)), "oracle_combine")
    return y


def mxfp4_quantize(v):
    """O7: BF16 [rows, K] -> (codes uint8 [rows, K/2], scales uint8 [rows, K/32])."""
    v = _c(v, np.uint16)
    shape = v.shape
    K = shape[-1]
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    codes = np.empty(shape[:-1] + (K // 2,), dtype=np.uint8)
    scales = np.empty(shape[:-1] + (K // 32,), dtype=np.uint8)
    _check(lib().oracle_mxfp4_quantize(rows, K, _p(v), _p(codes), _p(scales)),
           "oracle_mxfp4_quantize")
    return codes, scales


def mxfp4_dequantize(codes, scales):
    """O7: exact BF16 values of MXFP4 codes [rows, K/2] with scales [rows, K/32]."""
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    K = codes.shape[-1] * 2
    rows = int(np.prod(codes.shape[:-1])) if codes.ndim > 1 else 1
    assert scales.shape[-1] * 32 == K
    out = np.empty(codes.shape[:-1] + (K,), dtype=np.uint16)
    _check(lib().oracle_mxfp4_dequantize(rows, K, _p(codes), _p(scales), _p(out)),
           "oracle_mxfp4_dequantize")
    return out


# ---- composition -------------------------------------------------------------------------------

def moe_experts(z, ids, w, E, get_expert, threads=1, mx_act=False):
    """O5 + O6 for tokens z [T, d] with routing (ids [T, k], w [T, k]).

    get_expert(e) -> (Wg [f, d], Wu [f, d], Wd [d, f]) as BF16 bits. The loop is
    expert-major (each expert's rows computed by O5 with its own per-element
    sequential arithmetic), so the result does not depend on `threads`.
    Slots with an id outside [0, E) contribute nothing. mx_act: O8 (4-bit activations)
    instead of O5.
    """
    z = _c(z, np.uint16)
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    T, k = ids.shape
    d = z.shape[1]
    yk = np.zeros((T, k, d), dtype=np.uint16)
    experts = sorted(set(int(e) for e in ids.ravel() if 0 <= e < E))

    def run(e):
        tt, jj = np.nonzero(ids == e)
        wg, wu, wd = get_expert(e)
        rows = (expert_rows_mx if mx_act else expert_rows)(z[tt], wg, wu, wd, w[tt, jj])
        return tt, jj, rows

    if threads > 1 and len(experts) > 1:
        with ThreadPoolExecutor(threads) as ex:
            results = list(ex.map(run, experts))
    else:
        results = [run(e) for e in experts]
    for tt, jj, rows in results:
        yk[tt, jj] = rows
    return combine(yk, ids, E), yk


def sublayer(h, x, w_post, w_pre, n, eps, W_r, bias, G, kg, k, scale, get_expert, threads=1):
    """The whole path O1..O6 on the given tokens."""
    E = W_r.shape[0]
    h_out, z = boundary(h, x, w_post, w_pre, n, eps)
    logits = router_threaded(z, W_r, threads) if threads > 1 else router(z, W_r)
    ids, w, ggap, egap = topk(logits, bias, G, kg, k, scale)
    y, _ = moe_experts(z, ids, w, E, get_expert, threads)
    return dict(h_out=h_out, z=z, logits=logits, ids=ids, w=w, ggap=ggap, egap=egap, y=y)
