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
        L.synth_fill_q4_codes.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]
        L.synth_fill_q4_codes.restype = ctypes.c_int
        L.synth_fill_q4_scale_bias.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_float,
                                               ctypes.c_void_p]
        L.synth_fill_q4_scale_bias.restype = ctypes.c_int
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


def fill_q4(codes: torch.Tensor, sb: torch.Tensor, code_key: int, sb_key: int, sigma: float, stream=None):
    """4-bit expert block: codes (uint8, nbytes % 8 == 0) and scale/bias words (int32 view of uint32)."""
    assert codes.is_cuda and codes.dtype == torch.uint8 and codes.is_contiguous()
    assert sb.is_cuda and sb.dtype == torch.int32 and sb.is_contiguous()
    s = (stream or torch.cuda.current_stream()).cuda_stream
    rc = _L().synth_fill_q4_codes(codes.data_ptr(), code_key & S.MASK64, codes.numel(), s)
    if rc == 0:
        rc = _L().synth_fill_q4_scale_bias(sb.data_ptr(), sb_key & S.MASK64, sb.numel(),
                                           ctypes.c_float(float(S.q4_s0(sigma))), s)
    if rc != 0:
        raise RuntimeError(f"synth q4 fill failed: hipError {rc}")


def layer_tensors_q4(w: S.Workload, layer: int = 0, device="cuda", x_rows: int = None, x_row0: int = 0):
    """x [rows,H], router [E,H] (bf16); expert codes [E, 3IH/2] uint8 and scale/bias [E, 3IH/64]
    int32; shared codes / scale-bias (or None) on the device."""
    rows = w.M if x_rows is None else x_rows
    x = torch.empty(rows, w.H, dtype=torch.bfloat16, device=device)
    fill(x, S.x_key(w, layer), x_row0 * w.H, w.x_sigma)
    r = torch.empty(w.E, w.H, dtype=torch.bfloat16, device=device)
    fill(r, S.router_key(w, layer), 0, w.router_sigma)
    n = w.expert_elems()
    eq = torch.empty(w.E, n // 2, dtype=torch.uint8, device=device)
    esb = torch.empty(w.E, n // S.Q4_GROUP, dtype=torch.int32, device=device)
    for e in range(w.E):
        fill_q4(eq[e], esb[e], S.q4_expert_key(w, layer, e, False), S.q4_expert_key(w, layer, e, True), w.w_sigma)
    sq = ssb = None
    if w.I_shared:
        ns = w.shared_elems()
        sq = torch.empty(ns // 2, dtype=torch.uint8, device=device)
        ssb = torch.empty(ns // S.Q4_GROUP, dtype=torch.int32, device=device)
        fill_q4(sq, ssb, S.q4_shared_key(w, layer, False), S.q4_shared_key(w, layer, True), w.w_sigma)
    return x, r, eq, esb, sq, ssb
