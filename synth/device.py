"""Device-resident seeded inputs (torch tensors filled by the device generator).

Same recipes as the host functions in synth/__init__.py; values are bitwise equal
to the host draws (checked by the GPU tests).
"""
from __future__ import annotations

import numpy as np

from . import (T_BIAS, T_H, T_H_ROT, T_WD, T_WG, T_WPOST, T_WPRE, T_WR, T_WU, T_X, T_X_ROT,
               Workload, gpu_normal_bf16, gpu_normal_f32, gpu_uniform_bf16, gpu_uniform_f32)


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def tokens(wl: Workload, which: str, token_set: int = 0, T: int | None = None, device="cuda"):
    """h ('h') or x ('x') as a [T, d] BF16 device tensor."""
    import torch
    T = wl.T if T is None else T
    out = torch.empty((T, wl.d), dtype=torch.bfloat16, device=device)
    if token_set == 0:
        tid, row0 = (T_H if which == "h" else T_X), 0
    else:
        tid, row0 = (T_H_ROT if which == "h" else T_X_ROT), (token_set - 1) * wl.T
    gpu_normal_bf16(out.data_ptr(), wl.seed, tid, row0 * wl.d, T * wl.d, stream=_stream())
    return out


def norm_weights(wl: Workload, device="cuda"):
    import torch
    wpost = torch.empty((wl.d,), dtype=torch.bfloat16, device=device)
    wpre = torch.empty((wl.d,), dtype=torch.bfloat16, device=device)
    gpu_uniform_bf16(wpost.data_ptr(), wl.seed, T_WPOST, 0, wl.d, 0.9, 1.1, stream=_stream())
    gpu_uniform_bf16(wpre.data_ptr(), wl.seed, T_WPRE, 0, wl.d, 0.9, 1.1, stream=_stream())
    return wpost, wpre


def router(wl: Workload, device="cuda"):
    """(router_w [E, d] FP32, bias [E] FP32)."""
    import torch
    W = torch.empty((wl.E, wl.d), dtype=torch.float32, device=device)
    b = torch.empty((wl.E,), dtype=torch.float32, device=device)
    gpu_normal_f32(W.data_ptr(), wl.seed, T_WR, 0, wl.E * wl.d, std=1.0 / np.sqrt(wl.d),
                   stream=_stream())
    gpu_uniform_f32(b.data_ptr(), wl.seed, T_BIAS, 0, wl.E, -0.01, 0.01, stream=_stream())
    if wl.hot_experts:
        b[list(wl.hot_experts)] = float(np.float32(wl.hot_bias))
    return W, b


def experts(wl: Workload, device="cuda"):
    """(w_gate [E, f, d], w_up [E, f, d], w_down [E, d, f]) BF16 device tensors."""
    import torch
    n = wl.E * wl.f * wl.d
    wg = torch.empty((wl.E, wl.f, wl.d), dtype=torch.bfloat16, device=device)
    wu = torch.empty((wl.E, wl.f, wl.d), dtype=torch.bfloat16, device=device)
    wd = torch.empty((wl.E, wl.d, wl.f), dtype=torch.bfloat16, device=device)
    gpu_normal_bf16(wg.data_ptr(), wl.seed, T_WG, 0, n, std=0.02, stream=_stream())
    gpu_normal_bf16(wu.data_ptr(), wl.seed, T_WU, 0, n, std=0.02, stream=_stream())
    gpu_normal_bf16(wd.data_ptr(), wl.seed, T_WD, 0, n, std=0.02, stream=_stream())
    return wg, wu, wd


def moe_config(wl: Workload, max_tokens: int | None = None) -> dict:
    return dict(hidden=wl.d, n_experts=wl.E, n_groups=wl.G, topk_groups=wl.kg, topk=wl.k,
                d_ff=wl.f, max_tokens=max_tokens or wl.T, routed_scale=wl.scale)
