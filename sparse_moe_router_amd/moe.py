"""Thin Python binding of the C ABI in ``include/moe_layer.h``.

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the layer runs in the library's HIP
kernels.  There is no fallback: if the library is not built, or a tensor is
not a contiguous bf16/fp32/int32 tensor on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # noqa: F401  (loads torch's HIP runtime before the library)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_layer.so")

FLAG_FORCE_GEMV = 0x1
FLAG_FORCE_GEMM = 0x2
FLAG_TILED_WEIGHTS = 0x4
FLAG_WAIT_PROBE = 0x8  # test hook: the two-launch decode path's in-launch wait takes its give-up path
FLAG_DECODE_TWO_LAUNCH = 0x10  # decode path in two launches (opt-in; three launches are faster on MI355X)

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED_SHAPE",
          3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_MISALIGNED", 5: "MOE_ERR_HIP"}

EXPORTS = ("moe_workspace_size", "moe_block_map_capacity", "moe_layer_forward", "moe_route", "moe_layer_forward_traced",
           "moe_layer_forward_q4", "moe_tile_weights", "moe_tile_weights_q4", "moe_layer_forward_noalloc",
           "moe_status_string",
           "moe_last_hip_error")
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES

# moe_kernel_t
KERNELS = {1: "router_scores", 2: "topk", 3: "route_scan", 4: "route_scatter", 5: "gemm_gateup",
           6: "gemm_down", 7: "combine", 8: "dec_router", 9: "dec_gateup", 10: "dec_down",
           11: "sm_router", 12: "sm_topk", 13: "sm_gateup", 14: "sm_down", 15: "dec_route", 16: "dec_experts",
           17: "shared_down_combine", 18: "route_scan_scatter"}


class MoeDesc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("I", ctypes.c_int32), ("I_shared", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("router_bias", ctypes.c_void_p)]


class MoeRouting(ctypes.Structure):
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("logits", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p), ("perm", ctypes.c_void_p),
                ("tiles", ctypes.c_void_p), ("num_tiles", ctypes.c_void_p), ("wait_status", ctypes.c_void_p)]


class MoeTrace(ctypes.Structure):
    _fields_ = [("begin", ctypes.POINTER(ctypes.c_void_p)), ("end", ctypes.POINTER(ctypes.c_void_p)),
                ("kernel", ctypes.POINTER(ctypes.c_int32)), ("capacity", ctypes.c_int32),
                ("count", ctypes.c_int32)]


class MoeQ4(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scale_bias", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_moe_router_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.moe_workspace_size.argtypes = [ctypes.POINTER(MoeDesc), ctypes.c_int]
        L.moe_workspace_size.restype = sz
        L.moe_block_map_capacity.argtypes = [ctypes.POINTER(MoeDesc), ctypes.c_int]
        L.moe_block_map_capacity.restype = ctypes.c_int64
        L.moe_layer_forward.argtypes = [ctypes.POINTER(MoeDesc), vp, vp, vp, vp, ctypes.c_int, vp, vp, sz, vp,
                                        ctypes.POINTER(MoeRouting)]
        L.moe_layer_forward.restype = ctypes.c_int
        L.moe_layer_forward_traced.argtypes = L.moe_layer_forward.argtypes + [ctypes.POINTER(MoeTrace)]
        L.moe_layer_forward_traced.restype = ctypes.c_int
        L.moe_layer_forward_q4.argtypes = [ctypes.POINTER(MoeDesc), vp, vp, ctypes.POINTER(MoeQ4),
                                           ctypes.POINTER(MoeQ4), ctypes.c_int, vp, vp, sz, vp,
                                           ctypes.POINTER(MoeRouting), ctypes.POINTER(MoeTrace)]
        L.moe_layer_forward_q4.restype = ctypes.c_int
        L.moe_layer_forward_noalloc.argtypes = [ctypes.POINTER(MoeDesc), vp, vp, vp, vp, ctypes.c_int, vp, vp,
                                                ctypes.POINTER(MoeRouting)]
        L.moe_layer_forward_noalloc.restype = ctypes.c_int
        L.moe_route.argtypes = [ctypes.POINTER(MoeDesc), vp, vp, ctypes.c_int, vp, sz, vp,
                                ctypes.POINTER(MoeRouting)]
        L.moe_route.restype = ctypes.c_int
        L.moe_tile_weights.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, vp, vp]
        L.moe_tile_weights.restype = ctypes.c_int
        L.moe_tile_weights_q4.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp, vp]
        L.moe_tile_weights_q4.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_hip_error.argtypes = []
        L.moe_last_hip_error.restype = ctypes.c_int
        _lib = L
    return _lib


def make_desc(M, H, E, I, I_shared, flags=0, router_bias=None) -> MoeDesc:
    return MoeDesc(int(M), int(H), int(E), int(I), int(I_shared), int(flags),
                   None if router_bias is None else _ptr(router_bias, torch.float32, "router_bias"))


def workspace_size(M, H, E, I, I_shared, top_k, flags=0, with_bias=False) -> int:
    d = make_desc(M, H, E, I, I_shared, flags)
    return int(lib().moe_workspace_size(ctypes.byref(d), int(top_k)))


def block_map_capacity(M, H, E, I, I_shared, top_k, flags=0) -> int:
    """Tiles the routing output ``tiles`` ([capacity, 4] int32) must hold."""
    d = make_desc(M, H, E, I, I_shared, flags)
    return int(lib().moe_block_map_capacity(ctypes.byref(d), int(top_k)))


def _ptr(t: torch.Tensor, dtype, name) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_ws_cache: dict = {}


def _workspace(nbytes: int, device, stream) -> torch.Tensor:
    """A cached workspace for calls that pass none: one buffer per (device, stream), so calls on
    different streams never share one (calls sharing a workspace must be ordered, and calls on one
    stream are).  The buffer is allocated on `stream`; when it grows, the old buffer goes back to
    torch's caching allocator, which reuses it only after the work queued on that stream so far."""
    key = (device.type, device.index, stream.cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.stream(stream):
            buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def _routing_struct(routing: Optional[dict]) -> Optional[MoeRouting]:
    if not routing:
        return None
    spec = {"topk_ids": torch.int32, "topk_w": torch.float32, "logits": torch.float32,
            "counts": torch.int32, "offsets": torch.int32, "perm": torch.int32, "tiles": torch.int32,
            "num_tiles": torch.int32, "wait_status": torch.int32}
    r = MoeRouting()
    for k, v in routing.items():
        if k not in spec:
            raise KeyError(f"unknown routing output {k}")
        setattr(r, k, _ptr(v, spec[k], k))
    return r


def _stream_obj(stream, device):
    return torch.cuda.current_stream(device) if stream is None else stream


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(st: int, what: str):
    if st != 0:
        if st == 5:
            raise MoeError(st, f"{what} (hipError {lib().moe_last_hip_error()})")
        raise MoeError(st, what)


def forward(x: torch.Tensor, router_w: torch.Tensor, expert_w: torch.Tensor,
            shared_w: Optional[torch.Tensor], top_k: int, out: Optional[torch.Tensor] = None,
            router_bias: Optional[torch.Tensor] = None, routing: Optional[dict] = None,
            flags: int = 0, workspace: Optional[torch.Tensor] = None, stream=None,
            trace: Optional[MoeTrace] = None) -> torch.Tensor:
    """moe_layer_forward (moe_layer_forward_traced when a trace is given).  x [M,H] bf16; router_w [E,H] bf16; expert_w [E, 3*I*H] bf16
    (gate [I,H], up [I,H], down [H,I] per expert); shared_w [3*I_s*H] bf16 or None."""
    _ptr(x, torch.bfloat16, "x")  # a CPU tensor fails here, before any stream or workspace is touched
    M, H = x.shape
    E = router_w.shape[0]
    I = expert_w.numel() // (3 * E * H)
    I_s = 0 if shared_w is None else shared_w.numel() // (3 * H)
    if out is None:
        out = torch.empty_like(x)
    d = make_desc(M, H, E, I, I_s, flags, router_bias)
    need = lib().moe_workspace_size(ctypes.byref(d), int(top_k))
    if need == 0 and M > 0:
        raise MoeError(2, "moe_workspace_size rejected the shapes")
    ws = workspace if workspace is not None else _workspace(need, x.device, _stream_obj(stream, x.device))
    r = _routing_struct(routing)
    args = (ctypes.byref(d), _ptr(x, torch.bfloat16, "x"), _ptr(router_w, torch.bfloat16, "router_w"),
            _ptr(expert_w, torch.bfloat16, "expert_w"),
            None if shared_w is None else _ptr(shared_w, torch.bfloat16, "shared_w"), int(top_k),
            _ptr(out, torch.bfloat16, "out"), _ptr(ws, torch.uint8, "workspace"), ws.numel(), _stream(stream),
            None if r is None else ctypes.byref(r))
    if trace is None:
        st = lib().moe_layer_forward(*args)
    else:
        st = lib().moe_layer_forward_traced(*args, ctypes.byref(trace))
    _check(st, "moe_layer_forward")
    return out


def forward_noalloc(x: torch.Tensor, router_w: torch.Tensor, expert_w: torch.Tensor,
                    shared_w: Optional[torch.Tensor], top_k: int, out: torch.Tensor,
                    router_bias: Optional[torch.Tensor] = None, routing: Optional[dict] = None, flags: int = 0,
                    stream=None) -> torch.Tensor:
    """moe_layer_forward_noalloc: the layer with the library's static per-device scratch as its
    workspace.  ``out`` must be given (nothing is allocated here either); the current device must
    be the tensors' device."""
    _ptr(x, torch.bfloat16, "x")
    M, H = x.shape
    E = router_w.shape[0]
    I = expert_w.numel() // (3 * E * H)
    I_s = 0 if shared_w is None else shared_w.numel() // (3 * H)
    d = make_desc(M, H, E, I, I_s, flags, router_bias)
    r = _routing_struct(routing)
    st = lib().moe_layer_forward_noalloc(ctypes.byref(d), _ptr(x, torch.bfloat16, "x"),
                                         _ptr(router_w, torch.bfloat16, "router_w"),
                                         _ptr(expert_w, torch.bfloat16, "expert_w"),
                                         None if shared_w is None else _ptr(shared_w, torch.bfloat16, "shared_w"),
                                         int(top_k), _ptr(out, torch.bfloat16, "out"), _stream(stream),
                                         None if r is None else ctypes.byref(r))
    _check(st, "moe_layer_forward_noalloc")
    return out


def forward_q4(x: torch.Tensor, router_w: torch.Tensor, codes: torch.Tensor, scale_bias: torch.Tensor,
               shared_codes: Optional[torch.Tensor], shared_scale_bias: Optional[torch.Tensor], top_k: int,
               out: Optional[torch.Tensor] = None, router_bias: Optional[torch.Tensor] = None,
               routing: Optional[dict] = None, flags: int = 0, workspace: Optional[torch.Tensor] = None,
               stream=None, trace: Optional[MoeTrace] = None) -> torch.Tensor:
    """moe_layer_forward_q4.  codes uint8 [E, 3*I*H/2] (two 4-bit codes per byte, low nibble first);
    scale_bias int32 [E, 3*I*H/64] (bf16 scale in the low half, bf16 bias in the high half of each
    word); shared_codes / shared_scale_bias the same for the shared expert (E = 1), or None."""
    _ptr(x, torch.bfloat16, "x")  # a CPU tensor fails here, before any stream or workspace is touched
    M, H = x.shape
    E = router_w.shape[0]
    I = codes.numel() * 2 // (3 * E * H)
    I_s = 0 if shared_codes is None else shared_codes.numel() * 2 // (3 * H)
    if scale_bias.numel() * 64 != codes.numel() * 2:
        raise ValueError("scale_bias must hold one word per 64 codes")
    if shared_codes is not None and (shared_scale_bias is None or shared_scale_bias.numel() * 64 != shared_codes.numel() * 2):
        raise ValueError("shared_scale_bias must hold one word per 64 shared codes")
    if out is None:
        out = torch.empty_like(x)
    d = make_desc(M, H, E, I, I_s, flags, router_bias)
    need = lib().moe_workspace_size(ctypes.byref(d), int(top_k))
    if need == 0 and M > 0:
        raise MoeError(2, "moe_workspace_size rejected the shapes")
    ws = workspace if workspace is not None else _workspace(need, x.device, _stream_obj(stream, x.device))
    r = _routing_struct(routing)
    ex = MoeQ4(_ptr(codes, torch.uint8, "codes"), _ptr(scale_bias, torch.int32, "scale_bias"))
    sh = None if shared_codes is None else MoeQ4(_ptr(shared_codes, torch.uint8, "shared_codes"),
                                                  _ptr(shared_scale_bias, torch.int32, "shared_scale_bias"))
    st = lib().moe_layer_forward_q4(ctypes.byref(d), _ptr(x, torch.bfloat16, "x"),
                                    _ptr(router_w, torch.bfloat16, "router_w"), ctypes.byref(ex),
                                    None if sh is None else ctypes.byref(sh), int(top_k),
                                    _ptr(out, torch.bfloat16, "out"), _ptr(ws, torch.uint8, "workspace"), ws.numel(),
                                    _stream(stream), None if r is None else ctypes.byref(r),
                                    None if trace is None else ctypes.byref(trace))
    _check(st, "moe_layer_forward_q4")
    return out


def tile_weights(w: torch.Tensor, H: int, I: int, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_tile_weights: bf16 expert blocks (w.numel() // (3*I*H) of them, row-major packing) rewritten
    into the tiled layout read with FLAG_TILED_WEIGHTS; returns a tensor of w's shape."""
    n = w.numel() // (3 * I * H)
    if n * 3 * I * H != w.numel():
        raise ValueError("w must hold whole expert blocks of 3*I*H elements")
    if out is None:
        out = torch.empty_like(w)
    st = lib().moe_tile_weights(n, int(H), int(I), _ptr(w, torch.bfloat16, "w"), _ptr(out, torch.bfloat16, "out"),
                                _stream(stream))
    _check(st, "moe_tile_weights")
    return out


def tile_weights_q4(codes: torch.Tensor, scale_bias: torch.Tensor, H: int, I: int, stream=None):
    """moe_tile_weights_q4: 4-bit expert blocks (codes uint8, 3*I*H/2 bytes per block; scale_bias int32,
    3*I*H/64 words per block) rewritten into the tiled order read with FLAG_TILED_WEIGHTS by
    forward_q4; returns (codes, scale_bias) tensors of the inputs' shapes."""
    n = codes.numel() * 2 // (3 * I * H)
    if n * 3 * I * H != codes.numel() * 2 or n * 3 * I * H != scale_bias.numel() * 64:
        raise ValueError("codes and scale_bias must hold the same whole expert blocks")
    c_out, g_out = torch.empty_like(codes), torch.empty_like(scale_bias)
    st = lib().moe_tile_weights_q4(n, int(H), int(I), _ptr(codes, torch.uint8, "codes"),
                                   _ptr(scale_bias, torch.int32, "scale_bias"), _ptr(c_out, torch.uint8, "codes_out"),
                                   _ptr(g_out, torch.int32, "scale_bias_out"), _stream(stream))
    _check(st, "moe_tile_weights_q4")
    return c_out, g_out


def route(x: torch.Tensor, router_w: torch.Tensor, top_k: int, routing: dict,
          router_bias: Optional[torch.Tensor] = None, flags: int = 0, I: int = 64, I_shared: int = 0,
          workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """moe_route: routing decisions only, written into the tensors of ``routing``."""
    _ptr(x, torch.bfloat16, "x")  # a CPU tensor fails here, before any stream or workspace is touched
    M, H = x.shape
    E = router_w.shape[0]
    d = make_desc(M, H, E, I, I_shared, flags, router_bias)
    need = lib().moe_workspace_size(ctypes.byref(d), int(top_k))
    if need == 0 and M > 0:
        raise MoeError(2, "moe_workspace_size rejected the shapes")
    ws = workspace if workspace is not None else _workspace(need, x.device, _stream_obj(stream, x.device))
    r = _routing_struct(routing)
    st = lib().moe_route(ctypes.byref(d), _ptr(x, torch.bfloat16, "x"), _ptr(router_w, torch.bfloat16, "router_w"),
                         int(top_k), _ptr(ws, torch.uint8, "workspace"), ws.numel(), _stream(stream),
                         None if r is None else ctypes.byref(r))
    _check(st, "moe_route")
    return routing
