"""The C ABI library (CPU side): it loads, exports every entry point its header
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "beam_moe.h")


@pytest.fixture(scope="module")
def L():
    import sparse_moe_decoder_amd as beam
    return beam.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(beam_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"beam_moe_init", "beam_sublayer_norm_residual", "beam_router_topk",
            "beam_moe_forward"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert L.beam_status_string(0) == b"ok"
    assert L.beam_status_string(-5).startswith(b"T exceeds")
    assert L.beam_status_string(123) == b"unknown status"


def _cfg(**kw):
    from sparse_moe_decoder_amd.binding import beam_moe_config
    c = dict(hidden=5120, n_experts=256, n_groups=8, topk_groups=4, topk=8, d_ff=2560,
             max_tokens=128, routed_scale=2.5)
    c.update(kw)
    return beam_moe_config(**c)


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=5000), -2),          # not a multiple of 256
    (dict(d_ff=2600), -2),
    (dict(n_experts=512, n_groups=8), -2),
    (dict(topk=33, topk_groups=8), -2),
    (dict(n_groups=7), -1),           # E % G != 0
    (dict(topk_groups=9), -1),
    (dict(topk=200), -1),             # more than kg * E/G
    (dict(max_tokens=0), -1),
    (dict(routed_scale=float("inf")), -1),
    (dict(hidden=-256), -1),
])
def test_init_rejects_bad_config(L, kw, status):
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    st = L.beam_moe_init(ctypes.byref(_cfg(**kw)), fake, fake, fake, fake, fake, None,
                         ctypes.byref(h))
    assert st == status
    assert not h.value


def test_init_rejects_null_and_misaligned(L):
    h = ctypes.c_void_p()
    ok = ctypes.c_void_p(0x1000)
    assert L.beam_moe_init(ctypes.byref(_cfg()), None, ok, ok, ok, ok, None, ctypes.byref(h)) == -1
    bad = ctypes.c_void_p(0x1008)
    assert L.beam_moe_init(ctypes.byref(_cfg()), ok, ok, bad, ok, ok, None, ctypes.byref(h)) == -1
    assert L.beam_moe_init(None, ok, ok, ok, ok, ok, None, ctypes.byref(h)) == -1


def test_boundary_validation(L):
    p = ctypes.c_void_p(0x1000)
    f = L.beam_sublayer_norm_residual
    assert f(-1, 512, p, p, p, p, 20, 1e-6, p, p, None) == -1      # negative T
    assert f(4, 500, p, p, p, p, 20, 1e-6, p, p, None) == -1       # d % 8 != 0
    assert f(4, 512, p, p, p, p, 0, 1e-6, p, p, None) == -1        # n < 1
    assert f(4, 512, p, p, p, p, 20, -1.0, p, p, None) == -1       # eps < 0
    assert f(4, 512, p, p, p, p, 20, float("nan"), p, p, None) == -1
    assert f(4, 512, None, p, p, p, 20, 1e-6, p, p, None) == -1    # null
    assert f(4, 512, ctypes.c_void_p(0x1004), p, p, p, 20, 1e-6, p, p, None) == -1
    assert f(4, 70000, p, p, p, p, 20, 1e-6, p, p, None) == -2     # too wide
    assert f(0, 512, None, None, None, None, 20, 1e-6, None, None, None) == 0  # T = 0: no-op


def test_handle_calls_reject_null_handle(L):
    p = ctypes.c_void_p(0x1000)
    assert L.beam_router_topk(None, 1, p, None, p, p, None) == -1
    assert L.beam_grouped_topk(None, 1, p, p, p, None) == -1
    assert L.beam_moe_forward(None, 1, p, p, None, None, None, None, None, None, None, None) == -1
    assert L.beam_moe_forward_noalloc(None, 1, p, p, None, None, None, None, None, None, None,
                                      None) == -1
    assert L.beam_sublayer_forward(None, 1, p, p, p, p, 20, 1e-6, p, p, p, None, None, None,
                                   None) == -1
    assert L.beam_moe_forward_boundary(None, 1, p, p, p, p, 20, 1e-6, p, p, None, None, None,
                                       None, None, None, None) == -1
    assert L.beam_moe_forward_boundary_route(None, None, 1, p, p, p, p, 20, 1e-6, p, p, None, 0,
                                             None) == -1
    assert L.beam_moe_destroy(None) == 0


def test_profile_api_without_records(L):
    assert L.beam_kernel_count() == 9
    assert L.beam_kernel_name(4) == b"gate_up"
    assert L.beam_kernel_name(99) is None
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert L.beam_profile_read(0, ctypes.byref(ms), ctypes.byref(n)) == 0 and n.value == 0
    assert L.beam_profile_read(99, ctypes.byref(ms), ctypes.byref(n)) == -1


def test_product_path_has_no_oracle_or_fallback():
    """The package never imports the oracle, and the binding has no CPU fallback."""
    pkg = os.path.join(ROOT, "sparse_moe_decoder_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, fn), encoding="utf-8").read()
                assert "import oracle" not in src and "from oracle" not in src, fn
                assert "beam_oracle" not in src and "liboracle" not in src, fn


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=768), -2),            # hidden % 512 != 0
    (dict(d_ff=2816), -2),             # d_ff % 512 != 0
    (dict(n_groups=7), -1),            # the shared checks still come first
])
def test_init_mxfp4_rejects_bad_config(L, kw, status):
    h = ctypes.c_void_p()
    p = ctypes.c_void_p(0x1000)
    st = L.beam_moe_init_mxfp4(ctypes.byref(_cfg(**kw)), p, p, p, p, p, p, p, p, None,
                               ctypes.byref(h))
    assert st == status
    assert not h.value


def test_init_mxfp4_rejects_null_and_misaligned(L):
    h = ctypes.c_void_p()
    p = ctypes.c_void_p(0x1000)
    f = L.beam_moe_init_mxfp4
    assert f(ctypes.byref(_cfg()), p, p, None, p, p, p, p, p, None, ctypes.byref(h)) == -1
    assert f(ctypes.byref(_cfg()), p, p, p, p, p, p, p, None, None, ctypes.byref(h)) == -1
    assert f(ctypes.byref(_cfg()), p, p, ctypes.c_void_p(0x1002), p, p, p, p, p, None,
             ctypes.byref(h)) == -1
    assert not h.value


def test_mxfp4_quantize_validation(L):
    p = ctypes.c_void_p(0x1000)
    f = L.beam_mxfp4_quantize
    assert f(4, 48, p, p, p, None) == -1          # K % 32 != 0
    assert f(-1, 64, p, p, p, None) == -1         # negative rows
    assert f(4, 0, p, p, p, None) == -1
    assert f(4, 64, None, p, p, None) == -1       # null
    assert f(4, 64, ctypes.c_void_p(0x1008), p, p, None) == -1  # misaligned source
    assert f(0, 64, None, None, None, None) == 0  # rows = 0: no-op


def test_dense_validation(L):
    h = ctypes.c_void_p()
    p = ctypes.c_void_p(0x1000)
    f = L.beam_dense_init
    assert f(5000, 20480, 16, p, p, p, None, ctypes.byref(h)) == -2    # hidden % 256 != 0
    assert f(5120, 40960, 16, p, p, p, None, ctypes.byref(h)) == -2    # d_ff above 32768
    assert f(5120, 20480, 0, p, p, p, None, ctypes.byref(h)) == -1     # max_tokens
    assert f(5120, 20480, 16, None, p, p, None, ctypes.byref(h)) == -1
    assert f(5120, 20480, 16, p, ctypes.c_void_p(0x1008), p, None, ctypes.byref(h)) == -1
    assert not h.value
    assert L.beam_dense_forward(None, 1, p, p, None) == -1
