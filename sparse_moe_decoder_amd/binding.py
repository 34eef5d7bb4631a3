"""ctypes binding of include/beam_moe.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbeam_moe.so")

BEAM_OK = 0
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape", -3: "out of device memory",
          -4: "HIP runtime error", -5: "T exceeds the handle's max_tokens"}


class BeamError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status})")


class beam_moe_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("routed_scale", ctypes.c_float)]


_lib = None


def lib():
    """Load libbeam_moe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        L.beam_moe_init.argtypes = [ctypes.POINTER(beam_moe_config), vp, vp, vp, vp, vp, vp,
                                    ctypes.POINTER(vp)]
        L.beam_moe_init_mxfp4.argtypes = [ctypes.POINTER(beam_moe_config), vp, vp, vp, vp, vp,
                                          vp, vp, vp, vp, ctypes.POINTER(vp)]
        L.beam_mxfp4_quantize.argtypes = [ctypes.c_int64, i32, vp, vp, vp, vp]
        L.beam_dense_init.argtypes = [i32, i32, i32, vp, vp, vp, vp, ctypes.POINTER(vp)]
        L.beam_dense_forward.argtypes = [vp, i32, vp, vp, vp]
        L.beam_moe_destroy.argtypes = [vp]
        L.beam_sublayer_norm_residual.argtypes = [i32, i32, vp, vp, vp, vp, i32, f32, vp, vp, vp]
        L.beam_router_topk.argtypes = [vp, i32, vp, vp, vp, vp, vp]
        L.beam_grouped_topk.argtypes = [vp, i32, vp, vp, vp, vp]
        L.beam_moe_forward.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.beam_moe_forward_noalloc.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.beam_moe_set_activation_format.argtypes = [vp, i32]
        L.beam_moe_inspect.argtypes = [vp, i32, ctypes.POINTER(vp)]
        L.beam_sublayer_forward.argtypes = [vp, i32, vp, vp, vp, vp, i32, f32, vp, vp, vp, vp, vp,
                                            vp, vp]
        L.beam_moe_forward_boundary.argtypes = [vp, i32, vp, vp, vp, vp, i32, f32, vp, vp, vp, vp,
                                                vp, vp, vp, vp, vp]
        L.beam_moe_forward_boundary_route.argtypes = [vp, vp, i32, vp, vp, vp, vp, i32, f32, vp,
                                                      vp, vp, i32, vp]
        L.beam_status_string.argtypes = [ctypes.c_int]
        L.beam_status_string.restype = ctypes.c_char_p
        L.beam_profile_enable.argtypes = [ctypes.c_int]
        L.beam_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64)]
        L.beam_kernel_count.restype = i32
        L.beam_kernel_name.argtypes = [i32]
        L.beam_kernel_name.restype = ctypes.c_char_p
        for name in ("beam_moe_init", "beam_moe_init_mxfp4", "beam_mxfp4_quantize",
                     "beam_dense_init", "beam_dense_forward",
                     "beam_moe_destroy", "beam_sublayer_norm_residual",
                     "beam_router_topk", "beam_grouped_topk", "beam_moe_forward",
                     "beam_moe_forward_noalloc", "beam_moe_set_activation_format",
                     "beam_moe_inspect",
                     "beam_sublayer_forward", "beam_moe_forward_boundary",
                     "beam_moe_forward_boundary_route",
                     "beam_profile_enable", "beam_profile_reset", "beam_profile_read"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn, st):
    if st != BEAM_OK:
        raise BeamError(fn, st)


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t, dtype=None, shape=None, name="tensor"):
    """Device pointer of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


# ---- the C entry points under their own names ----------------------------------------------

def beam_moe_init(cfg: dict, router_w, router_bias, w_gate, w_up, w_down, stream=None):
    import torch
    c = beam_moe_config(cfg["hidden"], cfg["n_experts"], cfg["n_groups"], cfg["topk_groups"],
                        cfg["topk"], cfg["d_ff"], cfg["max_tokens"], cfg["routed_scale"])
    E, d, f = cfg["n_experts"], cfg["hidden"], cfg["d_ff"]
    h = ctypes.c_void_p()
    _check("beam_moe_init", lib().beam_moe_init(
        ctypes.byref(c), _ptr(router_w, torch.float32, (E, d), "router_w"),
        _ptr(router_bias, torch.float32, (E,), "router_bias"),
        _ptr(w_gate, torch.bfloat16, (E, f, d), "w_gate"),
        _ptr(w_up, torch.bfloat16, (E, f, d), "w_up"),
        _ptr(w_down, torch.bfloat16, (E, d, f), "w_down"), _stream(stream), ctypes.byref(h)))
    return h


def beam_mxfp4_quantize(src, codes_out=None, scales_out=None, stream=None):
    """MXFP4 codes [..., K/2] (uint8) and scales [..., K/32] (uint8) of BF16 rows [..., K]."""
    import torch
    K = src.shape[-1]
    rows = src.numel() // K if K else 0
    lead = tuple(src.shape[:-1])
    if codes_out is None:
        codes_out = torch.empty(lead + (K // 2,), dtype=torch.uint8, device=src.device)
    if scales_out is None:
        scales_out = torch.empty(lead + (K // 32,), dtype=torch.uint8, device=src.device)
    _check("beam_mxfp4_quantize", lib().beam_mxfp4_quantize(
        rows, K, _ptr(src, torch.bfloat16, name="src"),
        _ptr(codes_out, torch.uint8, lead + (K // 2,), "codes_out"),
        _ptr(scales_out, torch.uint8, lead + (K // 32,), "scales_out"), _stream(stream)))
    return codes_out, scales_out


def beam_moe_init_mxfp4(cfg: dict, router_w, router_bias, gate_codes, gate_scales, up_codes,
                        up_scales, down_codes, down_scales, stream=None):
    import torch
    c = beam_moe_config(cfg["hidden"], cfg["n_experts"], cfg["n_groups"], cfg["topk_groups"],
                        cfg["topk"], cfg["d_ff"], cfg["max_tokens"], cfg["routed_scale"])
    E, d, f = cfg["n_experts"], cfg["hidden"], cfg["d_ff"]
    u8 = torch.uint8
    h = ctypes.c_void_p()
    _check("beam_moe_init_mxfp4", lib().beam_moe_init_mxfp4(
        ctypes.byref(c), _ptr(router_w, torch.float32, (E, d), "router_w"),
        _ptr(router_bias, torch.float32, (E,), "router_bias"),
        _ptr(gate_codes, u8, (E, f, d // 2), "gate_codes"),
        _ptr(gate_scales, u8, (E, f, d // 32), "gate_scales"),
        _ptr(up_codes, u8, (E, f, d // 2), "up_codes"),
        _ptr(up_scales, u8, (E, f, d // 32), "up_scales"),
        _ptr(down_codes, u8, (E, d, f // 2), "down_codes"),
        _ptr(down_scales, u8, (E, d, f // 32), "down_scales"), _stream(stream), ctypes.byref(h)))
    return h


def beam_dense_init(hidden, d_ff, max_tokens, w_gate, w_up, w_down, stream=None):
    import torch
    bf, f, d = torch.bfloat16, d_ff, hidden
    h = ctypes.c_void_p()
    _check("beam_dense_init", lib().beam_dense_init(
        int(hidden), int(d_ff), int(max_tokens), _ptr(w_gate, bf, (f, d), "w_gate"),
        _ptr(w_up, bf, (f, d), "w_up"), _ptr(w_down, bf, (d, f), "w_down"), _stream(stream),
        ctypes.byref(h)))
    return h


def beam_dense_forward(handle, z, y_out=None, stream=None):
    """Dense SwiGLU layer on z [T, d]; returns y [T, d]."""
    import torch
    T, d = z.shape
    if y_out is None:
        y_out = torch.empty_like(z)
    bf = torch.bfloat16
    _check("beam_dense_forward", lib().beam_dense_forward(
        handle, T, _ptr(z, bf, (T, d), "z"), _ptr(y_out, bf, (T, d), "y_out"), _stream(stream)))
    return y_out


def beam_moe_destroy(handle):
    _check("beam_moe_destroy", lib().beam_moe_destroy(handle))


def beam_sublayer_norm_residual(h, x, w_post, w_pre, n, eps, h_out=None, z_out=None,
                                stream=None):
    """Returns (h_out, z_out); h_out may be h itself (in place)."""
    import torch
    T, d = h.shape
    if h_out is None:
        h_out = torch.empty_like(h)
    if z_out is None:
        z_out = torch.empty_like(h)
    bf = torch.bfloat16
    _check("beam_sublayer_norm_residual", lib().beam_sublayer_norm_residual(
        T, d, _ptr(h, bf, (T, d), "h"), _ptr(x, bf, (T, d), "x"),
        _ptr(w_post, bf, (d,), "w_post"), _ptr(w_pre, bf, (d,), "w_pre"), int(n), float(eps),
        _ptr(h_out, bf, (T, d), "h_out"), _ptr(z_out, bf, (T, d), "z_out"), _stream(stream)))
    return h_out, z_out


def beam_router_topk(handle, z, ids_out, w_out, logits_out=None, stream=None):
    T = z.shape[0]
    _check("beam_router_topk", lib().beam_router_topk(
        handle, T, _ptr(z, name="z"), _ptr(logits_out, name="logits_out"),
        _ptr(ids_out, name="ids_out"), _ptr(w_out, name="w_out"), _stream(stream)))


def beam_grouped_topk(handle, logits, ids_out, w_out, stream=None):
    T = logits.shape[0]
    _check("beam_grouped_topk", lib().beam_grouped_topk(
        handle, T, _ptr(logits, name="logits"), _ptr(ids_out, name="ids_out"),
        _ptr(w_out, name="w_out"), _stream(stream)))


def beam_moe_forward(handle, z, y_out, ids_in=None, w_in=None, logits_out=None, ids_out=None,
                     w_out=None, perm_out=None, offsets_out=None, stream=None):
    T = z.shape[0]
    _check("beam_moe_forward", lib().beam_moe_forward(
        handle, T, _ptr(z, name="z"), _ptr(y_out, name="y_out"), _ptr(ids_in, name="ids_in"),
        _ptr(w_in, name="w_in"), _ptr(logits_out, name="logits_out"),
        _ptr(ids_out, name="ids_out"), _ptr(w_out, name="w_out"),
        _ptr(perm_out, name="perm_out"), _ptr(offsets_out, name="offsets_out"),
        _stream(stream)))


ACT_BF16, ACT_MXFP4 = 0, 1
INSPECT = {"act": 0, "act_codes": 1, "act_scales": 2, "z_codes": 3, "z_scales": 4}


def beam_moe_set_activation_format(handle, fmt):
    _check("beam_moe_set_activation_format", lib().beam_moe_set_activation_format(handle, fmt))


def beam_moe_inspect(handle, what):
    """Device address (int) of one of the handle's intermediate buffers (see beam_moe.h)."""
    p = ctypes.c_void_p()
    _check("beam_moe_inspect", lib().beam_moe_inspect(handle, INSPECT[what], ctypes.byref(p)))
    return p.value


def beam_moe_forward_noalloc(handle, z, y_out, ids_in=None, w_in=None, logits_out=None,
                             ids_out=None, w_out=None, perm_out=None, offsets_out=None,
                             stream=None):
    T = z.shape[0]
    _check("beam_moe_forward_noalloc", lib().beam_moe_forward_noalloc(
        handle, T, _ptr(z, name="z"), _ptr(y_out, name="y_out"), _ptr(ids_in, name="ids_in"),
        _ptr(w_in, name="w_in"), _ptr(logits_out, name="logits_out"),
        _ptr(ids_out, name="ids_out"), _ptr(w_out, name="w_out"),
        _ptr(perm_out, name="perm_out"), _ptr(offsets_out, name="offsets_out"),
        _stream(stream)))


def beam_sublayer_forward(handle, h, x, w_post, w_pre, n, eps, y_out, h_out=None, z_out=None,
                          logits_out=None, ids_out=None, w_out=None, stream=None):
    """Boundary then MoE in one call; returns (h_out, z_out). h_out may be h itself."""
    import torch
    T, d = h.shape
    if h_out is None:
        h_out = torch.empty_like(h)
    if z_out is None:
        z_out = torch.empty_like(h)
    bf = torch.bfloat16
    _check("beam_sublayer_forward", lib().beam_sublayer_forward(
        handle, T, _ptr(h, bf, (T, d), "h"), _ptr(x, bf, (T, d), "x"),
        _ptr(w_post, bf, (d,), "w_post"), _ptr(w_pre, bf, (d,), "w_pre"), int(n), float(eps),
        _ptr(h_out, bf, (T, d), "h_out"), _ptr(z_out, bf, (T, d), "z_out"),
        _ptr(y_out, bf, (T, d), "y_out"), _ptr(logits_out, name="logits_out"),
        _ptr(ids_out, name="ids_out"), _ptr(w_out, name="w_out"), _stream(stream)))
    return h_out, z_out


def beam_moe_forward_boundary(handle, z, h, w_post, w_pre, n, eps, h_out=None, z_out=None,
                              y_out=None, ids_in=None, w_in=None, logits_out=None, ids_out=None,
                              w_out=None, stream=None):
    """MoE forward on z, then the next boundary with its output; returns (h_out, z_out).
    h_out may be h and z_out may be z; y_out (optional) receives the MoE output."""
    import torch
    T, d = h.shape
    if h_out is None:
        h_out = torch.empty_like(h)
    if z_out is None:
        z_out = torch.empty_like(h)
    bf = torch.bfloat16
    _check("beam_moe_forward_boundary", lib().beam_moe_forward_boundary(
        handle, T, _ptr(z, bf, (T, d), "z"), _ptr(h, bf, (T, d), "h"),
        _ptr(w_post, bf, (d,), "w_post"), _ptr(w_pre, bf, (d,), "w_pre"), int(n), float(eps),
        _ptr(h_out, bf, (T, d), "h_out"), _ptr(z_out, bf, (T, d), "z_out"),
        _ptr(y_out, bf, (T, d), "y_out"), _ptr(ids_in, name="ids_in"), _ptr(w_in, name="w_in"),
        _ptr(logits_out, name="logits_out"), _ptr(ids_out, name="ids_out"),
        _ptr(w_out, name="w_out"), _stream(stream)))
    return h_out, z_out


def beam_moe_forward_boundary_route(handle, next_handle, z, h, w_post, w_pre, n, eps,
                                    h_out=None, z_out=None, y_out=None, routed=False,
                                    stream=None):
    """MoE forward of `handle` on z (routed: its routing of z was left by the previous layer's
    call), then the combine, the next boundary and `next_handle`'s routing of z_out; returns
    (h_out, z_out). h_out may be h and z_out may be z; y_out (optional) receives the MoE
    output."""
    import torch
    T, d = h.shape
    if h_out is None:
        h_out = torch.empty_like(h)
    if z_out is None:
        z_out = torch.empty_like(h)
    bf = torch.bfloat16
    _check("beam_moe_forward_boundary_route", lib().beam_moe_forward_boundary_route(
        handle, next_handle, T, _ptr(z, bf, (T, d), "z"), _ptr(h, bf, (T, d), "h"),
        _ptr(w_post, bf, (d,), "w_post"), _ptr(w_pre, bf, (d,), "w_pre"), int(n), float(eps),
        _ptr(h_out, bf, (T, d), "h_out"), _ptr(z_out, bf, (T, d), "z_out"),
        _ptr(y_out, bf, (T, d), "y_out"), 1 if routed else 0, _stream(stream)))
    return h_out, z_out


# ---- measurement hooks ------------------------------------------------------------------

def kernel_names():
    L = lib()
    return [L.beam_kernel_name(i).decode() for i in range(L.beam_kernel_count())]


def profile_enable(on=True):
    _check("beam_profile_enable", lib().beam_profile_enable(1 if on else 0))


def profile_reset():
    _check("beam_profile_reset", lib().beam_profile_reset())


def profile_read():
    """{kernel name: (total ms, launches)} since the last reset."""
    out = {}
    for i, name in enumerate(kernel_names()):
        ms, n = ctypes.c_double(), ctypes.c_int64()
        _check("beam_profile_read", lib().beam_profile_read(i, ctypes.byref(ms), ctypes.byref(n)))
        out[name] = (ms.value, n.value)
    return out


def lib_copy(dst, src, nbytes):
    """Device-to-device copy of nbytes (plain HIP copy through torch's runtime)."""
    import torch
    # a view of the source address: torch copies between two device tensors
    from torch.cuda import current_stream  # noqa: F401
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    torch.cuda.synchronize()
    rc = hip.hipMemcpy(ctypes.c_void_p(dst), ctypes.c_void_p(src), nbytes, 3)
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed: {rc}")


# ---- convenience object ----------------------------------------------------------------

class BeamMoE:
    """One MoE layer handle with torch-allocated outputs."""

    def __init__(self, cfg: dict, router_w, router_bias, w_gate, w_up, w_down, stream=None,
                 mxfp4=None):
        """BF16 experts from (w_gate, w_up, w_down); or, with mxfp4 = (gate_codes,
        gate_scales, up_codes, up_scales, down_codes, down_scales) and the three BF16
        weights None, 4-bit experts (see beam_moe_init_mxfp4)."""
        self.cfg = dict(cfg)
        self.handle = None
        if mxfp4 is not None:
            self.handle = beam_moe_init_mxfp4(cfg, router_w, router_bias, *mxfp4, stream=stream)
        else:
            self.handle = beam_moe_init(cfg, router_w, router_bias, w_gate, w_up, w_down, stream)

    def set_activation_format(self, fmt):
        beam_moe_set_activation_format(self.handle, fmt)

    def inspect(self, what, nbytes):
        """Copy nbytes of an intermediate buffer to a new uint8 device tensor."""
        import torch
        src = beam_moe_inspect(self.handle, what)
        out = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        lib_copy(out.data_ptr(), src, nbytes)
        return out

    def close(self):
        if self.handle is not None and self.handle.value:
            beam_moe_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def router_topk(self, z, want_logits=True, stream=None):
        import torch
        T, k, E = z.shape[0], self.cfg["topk"], self.cfg["n_experts"]
        ids = torch.empty((T, k), dtype=torch.int32, device=z.device)
        w = torch.empty((T, k), dtype=torch.float32, device=z.device)
        logits = torch.empty((T, E), dtype=torch.float32, device=z.device) if want_logits else None
        beam_router_topk(self.handle, z, ids, w, logits, stream)
        return logits, ids, w

    def grouped_topk(self, logits, stream=None):
        import torch
        T, k = logits.shape[0], self.cfg["topk"]
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
        w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
        beam_grouped_topk(self.handle, logits, ids, w, stream)
        return ids, w

    def forward(self, z, y=None, ids_in=None, w_in=None, want_routing=False, stream=None):
        import torch
        T, k, E = z.shape[0], self.cfg["topk"], self.cfg["n_experts"]
        if y is None:
            y = torch.empty_like(z)
        extra = {}
        if want_routing:
            dev = z.device
            extra = dict(ids_out=torch.empty((T, k), dtype=torch.int32, device=dev),
                         w_out=torch.empty((T, k), dtype=torch.float32, device=dev),
                         perm_out=torch.empty((T * k,), dtype=torch.int32, device=dev),
                         offsets_out=torch.empty((E + 1,), dtype=torch.int32, device=dev))
            if ids_in is None:
                extra["logits_out"] = torch.empty((T, E), dtype=torch.float32, device=dev)
        beam_moe_forward(self.handle, z, y, ids_in=ids_in, w_in=w_in, stream=stream, **extra)
        return (y, extra) if want_routing else y
