"""Device-side fill of seeded synthetic inputs (bit-identical to synth.inputs).

Writes into caller-provided torch bf16 tensors on the GPU through
``synth/libsynth.so``.  Input plumbing only; none of the layer's arithmetic.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import inputs as S

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth.so")
_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is missing: build with `python -m sparse_moe_router_amd.build`")
        L = ctypes.CDLL(_PATH)
        L.synth_fill_normal_bf16.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                             ctypes.c_float, ctypes.c_void_p]
        L.synth_fill_normal_bf16.restype = ctypes.c_int
        _lib = L
    return _lib


def fill(t: torch.Tensor, key: int, start: int, sigma: float, stream=None) -> torch.Tensor:
    """t.view(-1)[j] = bf16 element start+j of stream `key` scaled to sigma."""
    assert t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous()
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rc = _L().synth_fill_normal_bf16(t.data_ptr(), key & S.MASK64, start, t.numel(),
                                     ctypes.c_float(float(S.scale_f32(sigma))), s)
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal_bf16 failed: hipError {rc}")
    return t


def layer_tensors(w: S.Workload, layer: int = 0, device="cuda", x_rows: int = None, x_row0: int = 0):
    """x [rows,H], router [E,H], experts [E, 3IH], shared [3 I_s H] (or None) on the device."""
    rows = w.M if x_rows is None else x_rows
    x = torch.empty(rows, w.H, dtype=torch.bfloat16, device=device)
    fill(x, S.x_key(w, layer), x_row0 * w.H, w.x_sigma)
    r = torch.empty(w.E, w.H, dtype=torch.bfloat16, device=device)
    fill(r, S.router_key(w, layer), 0, w.router_sigma)
    ex = torch.empty(w.E, w.expert_elems(), dtype=torch.bfloat16, device=device)
    for e in range(w.E):
        fill(ex[e], S.expert_key(w, layer, e), 0, w.w_sigma)
    sh = None
    if w.I_shared:
        sh = torch.empty(w.shared_elems(), dtype=torch.bfloat16, device=device)
        fill(sh, S.shared_key(w, layer), 0, w.w_sigma)
    return x, r, ex, sh
