"""The C-ABI library loads, exports every declared symbol, and rejects invalid
arguments with the documented status before launching anything (CPU only:
no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

from sparse_moe_router_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_layer.h")

OK, INVALID, SHAPE, WS, MISALIGNED = 0, 1, 2, 3, 4


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = moe.lib()
    names = declared_functions()
    assert set(names) == set(moe.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = moe.lib()
    for code in range(6):
        s = L.moe_status_string(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert L.moe_status_string(0) == b"ok"
    assert L.moe_last_hip_error() == 0


def _desc(M=64, H=256, E=16, I=128, Is=128, flags=0, bias=None):
    return moe.MoeDesc(M, H, E, I, Is, flags, bias)


def ws_size(d, k):
    return moe.lib().moe_workspace_size(ctypes.byref(d), k)


def test_workspace_size_valid_and_invalid():
    assert ws_size(_desc(), 2) > 0
    big = ws_size(_desc(M=4096, H=2048, E=256, I=512, Is=512), 8)
    # y_r alone is M*k*H bf16
    assert big > 4096 * 8 * 2048 * 2
    gemv = ws_size(_desc(M=1, H=2048, E=256, I=512, Is=512), 8)
    gemm = ws_size(_desc(M=1, H=2048, E=256, I=512, Is=512, flags=moe.FLAG_FORCE_GEMM), 8)
    assert 0 < gemv < gemm  # the decode path needs no permutation tables or y rows
    for bad in [_desc(H=100), _desc(I=96), _desc(E=0), _desc(E=2000), _desc(Is=32), _desc(M=-1),
                _desc(flags=3), _desc(flags=0x20)]:
        assert ws_size(bad, 2) == 0
    assert ws_size(_desc(), 0) == 0
    assert ws_size(_desc(), 17) == 0  # top_k > E
    assert ws_size(_desc(E=64), 33) == 0  # top_k > 32
    assert ws_size(_desc(M=1 << 28), 8) == 0  # M*k >= 2^31
    assert ws_size(_desc(M=65, flags=moe.FLAG_FORCE_GEMV), 2) == 0  # matrix-vector paths take M <= 64
    small = ws_size(_desc(M=5, flags=moe.FLAG_FORCE_GEMV), 2)
    assert small > ws_size(_desc(M=1, flags=moe.FLAG_FORCE_GEMV), 2) > 0


FAKE = 0x7F0000000000  # never dereferenced: every call below fails its checks first


def fwd(d, k=2, x=FAKE, r=FAKE + (1 << 24), ex=FAKE + (2 << 24), sh=FAKE + (3 << 24), out=FAKE + (4 << 24),
        ws=FAKE + (5 << 24), wsb=1 << 40, routing=None):
    # x, router, experts, shared, out and workspace 16 MiB apart (each smaller at _desc's shapes)
    return moe.lib().moe_layer_forward(ctypes.byref(d), x, r, ex, sh, k, out, ws, wsb, None,
                                       None if routing is None else ctypes.byref(routing))


def test_forward_rejects_bad_arguments():
    d = _desc()
    assert fwd(d, x=None) == INVALID
    assert fwd(d, r=None) == INVALID
    assert fwd(d, ex=None) == INVALID
    assert fwd(d, out=None) == INVALID
    assert fwd(d, sh=None) == INVALID  # I_shared > 0 needs shared weights
    assert fwd(_desc(Is=0)) == INVALID  # shared weights given but I_shared == 0
    assert fwd(d, ws=None) == INVALID
    assert fwd(d, out=FAKE) == INVALID  # out aliases x
    assert fwd(d, ws=FAKE + 1024) == INVALID  # workspace overlaps x
    assert fwd(d, x=FAKE + 2) == MISALIGNED
    assert fwd(d, ex=FAKE + (2 << 24) + 8) == MISALIGNED
    assert fwd(d, ws=FAKE + (5 << 24) + 16) == MISALIGNED
    assert fwd(d, wsb=ws_size(d, 2) - 1) == WS
    assert fwd(_desc(H=100)) == SHAPE
    assert fwd(d, k=0) == SHAPE
    assert fwd(d, k=17) == SHAPE
    assert fwd(_desc(M=65, flags=moe.FLAG_FORCE_GEMV)) == SHAPE
    assert fwd(_desc(flags=3)) == INVALID
    bad_bias = _desc(bias=FAKE + (6 << 24) + 4)
    assert fwd(bad_bias) == MISALIGNED
    r = moe.MoeRouting(FAKE + (7 << 24) + 2, None, None, None, None, None)
    assert fwd(d, routing=r) == MISALIGNED
    assert moe.lib().moe_layer_forward(None, FAKE, FAKE, FAKE, FAKE, 2, FAKE, FAKE, 0, None, None) == INVALID


def test_forward_empty_batch_is_noop():
    # M == 0: nothing to compute, returns OK without touching memory
    assert fwd(_desc(M=0), ws=None, wsb=0) == OK


def test_route_rejects_bad_arguments():
    L = moe.lib()
    d = _desc()
    r = moe.MoeRouting(None, None, None, None, None, None)
    assert L.moe_route(ctypes.byref(d), FAKE, FAKE + (1 << 24), 2, FAKE + (5 << 24), 1 << 40, None, None) == INVALID
    assert L.moe_route(ctypes.byref(d), None, FAKE + (1 << 24), 2, FAKE + (5 << 24), 1 << 40, None,
                       ctypes.byref(r)) == INVALID
    assert L.moe_route(ctypes.byref(d), FAKE + 8, FAKE + (1 << 24), 2, FAKE + (5 << 24), 1 << 40, None,
                       ctypes.byref(r)) == MISALIGNED
    assert L.moe_route(ctypes.byref(d), FAKE, FAKE + (1 << 24), 2, FAKE + (5 << 24), 16, None,
                       ctypes.byref(r)) == WS


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    r = torch.zeros(16, 256, dtype=torch.bfloat16)
    ex = torch.zeros(16, 3 * 128 * 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        moe.forward(x, r, ex, None, 2)


def fwd_q4(d, k=2, x=FAKE, r=FAKE + (1 << 24), codes=FAKE + (2 << 24), sb=FAKE + (8 << 24),
           sh_codes=FAKE + (3 << 24), sh_sb=FAKE + (9 << 24), out=FAKE + (4 << 24), ws=FAKE + (5 << 24),
           wsb=1 << 40, experts=True, shared=True):
    ex = moe.MoeQ4(codes, sb)
    sh = moe.MoeQ4(sh_codes, sh_sb)
    return moe.lib().moe_layer_forward_q4(ctypes.byref(d), x, r, ctypes.byref(ex) if experts else None,
                                          ctypes.byref(sh) if shared else None, k, out, ws, wsb, None, None, None)


def test_forward_q4_rejects_bad_arguments():
    d = _desc()
    assert fwd_q4(d, experts=False) == INVALID
    assert fwd_q4(d, codes=None) == INVALID
    assert fwd_q4(d, sb=None) == INVALID
    assert fwd_q4(d, shared=False) == INVALID  # I_shared > 0 needs shared weights
    assert fwd_q4(d, sh_sb=None) == INVALID  # half a shared weight set
    assert fwd_q4(_desc(Is=0)) == INVALID  # shared weights given but I_shared == 0
    assert fwd_q4(d, x=None) == INVALID
    assert fwd_q4(d, out=FAKE) == INVALID
    assert fwd_q4(d, codes=FAKE + (2 << 24) + 4) == MISALIGNED
    assert fwd_q4(d, sb=FAKE + (8 << 24) + 4) == MISALIGNED
    assert fwd_q4(d, sh_codes=FAKE + (3 << 24) + 8) == MISALIGNED
    assert fwd_q4(d, wsb=ws_size(d, 2) - 1) == WS
    assert fwd_q4(_desc(I=96)) == SHAPE
    assert fwd_q4(d, k=17) == SHAPE
    assert fwd_q4(_desc(M=0), ws=None, wsb=0) == OK


def test_tiled_flag_and_tile_weights_arguments():
    L = moe.lib()
    # the 4-bit entry point takes the flag too (weights from moe_tile_weights_q4); its other checks still apply
    assert fwd_q4(_desc(flags=moe.FLAG_TILED_WEIGHTS), k=17) == SHAPE
    assert fwd_q4(_desc(flags=moe.FLAG_TILED_WEIGHTS), wsb=ws_size(_desc(), 2) - 1) == WS
    assert ws_size(_desc(flags=moe.FLAG_TILED_WEIGHTS), 2) == ws_size(_desc(), 2)
    assert ws_size(_desc(flags=moe.FLAG_TILED_WEIGHTS | moe.FLAG_FORCE_GEMM), 2) > 0
    dst = FAKE + (1 << 28)
    tw = L.moe_tile_weights
    assert tw(-1, 256, 128, FAKE, dst, None) == INVALID
    assert tw(2, 256, 128, None, dst, None) == INVALID
    assert tw(2, 256, 128, FAKE, None, None) == INVALID
    assert tw(2, 100, 128, FAKE, dst, None) == SHAPE
    assert tw(2, 256, 96, FAKE, dst, None) == SHAPE
    assert tw(2, 256, 32768, FAKE, dst, None) == SHAPE
    assert tw(2, 256, 128, FAKE + 8, dst, None) == MISALIGNED
    assert tw(2, 256, 128, FAKE, dst + 4, None) == MISALIGNED
    assert tw(2, 256, 128, FAKE, FAKE + 1024, None) == INVALID  # dst overlaps src
    assert tw(0, 256, 128, FAKE, dst, None) == OK  # no blocks: nothing enqueued
    # 4-bit: codes (3*I*H/2 bytes per block) and group words (3*I*H/16 bytes per block), four pointers
    tq = L.moe_tile_weights_q4
    cb, gb = 3 * 128 * 256 // 2 * 2, 3 * 128 * 256 // 16 * 2  # two blocks at H=256, I=128
    c, g, cd, gd = FAKE, FAKE + (1 << 24), FAKE + (2 << 24), FAKE + (3 << 24)
    assert tq(-1, 256, 128, c, g, cd, gd, None) == INVALID
    for i in range(4):
        args = [c, g, cd, gd]
        args[i] = None
        assert tq(2, 256, 128, *args, None) == INVALID
    assert tq(2, 100, 128, c, g, cd, gd, None) == SHAPE
    assert tq(2, 256, 96, c, g, cd, gd, None) == SHAPE
    assert tq(2, 256, 128, c + 8, g, cd, gd, None) == MISALIGNED
    assert tq(2, 256, 128, c, g, cd, gd + 4, None) == MISALIGNED
    assert tq(2, 256, 128, c, g, c + cb - 256, gd, None) == INVALID  # codes out overlaps codes in
    assert tq(2, 256, 128, c, g, cd, g + gb - 256, None) == INVALID  # groups out overlaps groups in
    assert tq(2, 256, 128, c, g, cd, cd + cb - 256, None) == INVALID  # the two outputs overlap
    assert tq(2, 256, 128, c, g, g, gd, None) == INVALID  # codes out is the groups input
    assert tq(0, 256, 128, c, g, cd, gd, None) == OK


def _routing(**kw):
    r = moe.MoeRouting()
    for k, v in kw.items():
        setattr(r, k, v)
    return r


def test_outputs_must_not_overlap_inputs_or_each_other():
    """moe_layer.h: out, the workspace and the routing buffers are disjoint from every input
    (x, router, experts, shared expert, router bias) and from each other."""
    d = _desc()
    bias = FAKE + (6 << 24)
    db = _desc(bias=bias)
    # out over each input
    assert fwd(d, out=FAKE + (1 << 24)) == INVALID            # router
    assert fwd(d, out=FAKE + (2 << 24) + 4096) == INVALID     # inside the expert weights
    assert fwd(d, out=FAKE + (3 << 24) + 256) == INVALID      # shared expert
    assert fwd(db, out=bias - 64) == INVALID                  # router bias
    # workspace over each input
    assert fwd(d, ws=FAKE + (1 << 24)) == INVALID
    assert fwd(d, ws=FAKE + (2 << 24) + (1 << 20)) == INVALID
    assert fwd(d, ws=FAKE + (3 << 24)) == INVALID
    # workspace over out
    assert fwd(d, ws=FAKE + (4 << 24) + 256) == INVALID
    # routing buffers over inputs, out, the workspace, each other
    assert fwd(d, routing=_routing(topk_ids=FAKE + 64)) == INVALID
    assert fwd(d, routing=_routing(logits=FAKE + (2 << 24))) == INVALID
    assert fwd(d, routing=_routing(perm=FAKE + (4 << 24))) == INVALID
    assert fwd(d, routing=_routing(counts=FAKE + (5 << 24) + 1024)) == INVALID
    assert fwd(db, routing=_routing(topk_w=bias)) == INVALID
    assert fwd(d, routing=_routing(topk_ids=FAKE + (7 << 24), topk_w=FAKE + (7 << 24) + 64)) == INVALID
    assert fwd(d, routing=_routing(tiles=FAKE + (7 << 24), num_tiles=FAKE + (7 << 24) + 16)) == INVALID
    # 4-bit weights: out over the codes or the group words
    assert fwd_q4(d, out=FAKE + (2 << 24) + 512) == INVALID
    assert fwd_q4(d, out=FAKE + (8 << 24)) == INVALID
    assert fwd_q4(d, out=FAKE + (9 << 24)) == INVALID
    # routing only: outputs over x or the router
    L = moe.lib()
    for r in (_routing(topk_ids=FAKE), _routing(logits=FAKE + (1 << 24) + 128)):
        assert L.moe_route(ctypes.byref(d), FAKE, FAKE + (1 << 24), 2, FAKE + (5 << 24), 1 << 40, None,
                           ctypes.byref(r)) == INVALID
    assert L.moe_route(ctypes.byref(d), FAKE, FAKE + (1 << 24), 2, FAKE + 4096, 1 << 40, None,
                       ctypes.byref(_routing(topk_ids=FAKE + (7 << 24)))) == INVALID  # workspace over x


def test_block_map_capacity():
    L = moe.lib()
    cap = lambda d, k: L.moe_block_map_capacity(ctypes.byref(d), k)
    # ceil(M*k / 256) + E (+ ceil(M / 256) with a shared expert), whatever path the shapes select
    assert cap(_desc(M=4096, H=2048, E=256, I=512, Is=512), 8) == 128 + 256 + 16
    assert cap(_desc(M=300, E=16, Is=0), 4) == 5 + 16
    assert cap(_desc(M=1, E=16), 2) == 1 + 16 + 1
    assert cap(_desc(H=100), 2) == 0 and cap(_desc(), 0) == 0


def test_header_compiles_as_c_and_with_hip():
    """The header is plain C11 (no HIP include needed) and agrees with HIP's own declaration of
    hipStream_t when both are included."""
    import shutil
    import subprocess
    import tempfile
    gcc, gxx = shutil.which("gcc"), shutil.which("g++")
    if not gcc or not gxx:
        pytest.skip("no host compiler")
    inc = os.path.join(ROOT, "include")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "use.c")
        with open(c, "w") as f:
            f.write('#include "moe_layer.h"\nint main(void) { moe_desc_t d = {0}; hipStream_t s = 0;\n'
                    '  return (int)moe_workspace_size(&d, 1) + (s != 0); }\n')
        subprocess.run([gcc, "-std=c11", "-Wall", "-Werror", "-I", inc, "-c", c, "-o", c + ".o"], check=True)
        cc = os.path.join(d, "use.cc")
        with open(cc, "w") as f:
            f.write('#include <hip/hip_runtime_api.h>\n#include "moe_layer.h"\n'
                    'int main() { hipStream_t s = nullptr; return s != nullptr; }\n')
        subprocess.run([gxx, "-std=c++17", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                        "-I", inc, "-c", cc, "-o", cc + ".o"], check=True)


def test_noalloc_rejects_before_touching_the_device():
    """moe_layer_forward_noalloc checks every argument, and that the call's workspace fits the
    64 MiB static scratch, before it looks up the device's scratch (none of these calls reach it)."""
    L = moe.lib()

    def na(d, k=2, x=FAKE, r=FAKE + (1 << 24), ex=FAKE + (2 << 24), sh=FAKE + (3 << 24), out=FAKE + (4 << 24)):
        return L.moe_layer_forward_noalloc(ctypes.byref(d), x, r, ex, sh, k, out, None, None)

    big = _desc(M=4096, H=2048, E=256, I=512, Is=512)
    assert ws_size(big, 8) > moe.NOALLOC_SCRATCH_BYTES
    assert na(big, k=8, r=FAKE + (1 << 30), ex=FAKE + (2 << 30), sh=FAKE + (8 << 30), out=FAKE + (9 << 30)) == WS
    d = _desc()
    assert ws_size(d, 2) <= moe.NOALLOC_SCRATCH_BYTES
    assert na(d, x=None) == INVALID
    assert na(d, out=FAKE) == INVALID  # out over x
    assert na(d, x=FAKE + 2) == MISALIGNED
    assert na(_desc(H=100)) == SHAPE
    assert na(_desc(M=0)) == OK  # nothing to do
