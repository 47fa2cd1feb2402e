"""GPU tests of the call contract in moe_layer.h: calls are asynchronous on
the caller's stream, keep no state between calls, and calls on distinct
workspaces are independent.

  - a call captured in a HIP graph replays to the same bits as the eager
    call, also after the input buffer is refilled between replays and with
    other work on the device in between (decode, small-batch and grouped
    paths; bf16, tiled bf16 and 4-bit weights);
  - calls on two streams with two workspaces, interleaved, give the bits of
    the same calls made one after another;
  - a traced call (per-kernel events) gives the bits of the untraced one and
    records its path's kernels in launch order, up to the trace's capacity."""
import numpy as np
import pytest
import torch

from gpu_util import moe, rand_case, upload
from synth import device as SD
from synth import inputs as S

pytestmark = pytest.mark.gpu

H, E, K, I, IS = 256, 32, 4, 128, 128


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    moe.lib()
    yield


def _weights(kind, seed=3):
    _, r, ex, sh, _ = rand_case(1, H, E, K, I, IS, seed=seed)
    r, ex, sh = upload(r), upload(ex), upload(sh)
    if kind == "tiled":
        return r, (moe.tile_weights(ex, H, I), moe.tile_weights(sh, H, IS)), moe.FLAG_TILED_WEIGHTS
    if kind == "q4":
        w = S.reduced(S.TINY, H=H, E=E, k=K, I=I, I_shared=IS)
        _, _, ec, esb, sc, ssb = SD.layer_tensors_q4(w, x_rows=1)
        return r, (ec, esb, sc, ssb), 0
    return r, (ex, sh), 0


def _call(x, r, wts, flags, out, ws, stream=None):
    if len(wts) == 4:
        return moe.forward_q4(x, r, *wts, K, out=out, flags=flags, workspace=ws, stream=stream)
    return moe.forward(x, r, wts[0], wts[1], K, out=out, flags=flags, workspace=ws, stream=stream)


@pytest.mark.parametrize("kind", ["bf16", "tiled", "q4"])
@pytest.mark.parametrize("M", [1, 8, 300])
def test_graph_replay_matches_eager(kind, M):
    r, wts, flags = _weights(kind)
    g0 = torch.Generator().manual_seed(M)
    xs = [upload(np.random.default_rng(M + i).standard_normal((M, H)).astype(np.float32)) for i in range(3)]
    x = xs[0].clone()
    out = torch.empty_like(x)
    ws = torch.empty(moe.workspace_size(M, H, E, I, IS, K, flags=flags), dtype=torch.uint8, device="cuda")
    eager = []
    for xi in xs:
        x.copy_(xi)
        _call(x, r, wts, flags, out, ws)
        torch.cuda.synchronize()
        eager.append(out.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _call(x, r, wts, flags, out, ws)
    torch.cuda.synchronize()
    other = torch.randn(1 << 20, generator=g0).cuda()
    for rep in range(2):
        for i, xi in enumerate(xs):
            x.copy_(xi)
            out.zero_()
            other.mul_(1.0001)  # unrelated device work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eager[i].view(torch.int16)), f"replay {rep}, input {i}"


@pytest.mark.parametrize("M", [1, 8, 300])
def test_two_streams_two_workspaces(M):
    r, wts, flags = _weights("bf16", seed=5)
    xa = upload(np.random.default_rng(10 + M).standard_normal((M, H)).astype(np.float32))
    xb = upload(np.random.default_rng(20 + M).standard_normal((M, H)).astype(np.float32))
    n = moe.workspace_size(M, H, E, I, IS, K)
    wa = torch.empty(n, dtype=torch.uint8, device="cuda")
    wb = torch.empty(n, dtype=torch.uint8, device="cuda")
    ref_a = _call(xa, r, wts, flags, torch.empty_like(xa), wa).clone()
    ref_b = _call(xb, r, wts, flags, torch.empty_like(xb), wb).clone()
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a = [torch.empty_like(xa) for _ in range(4)]
    outs_b = [torch.empty_like(xb) for _ in range(4)]
    for i in range(4):  # interleaved enqueues; each stream's calls share its own workspace
        _call(xa, r, wts, flags, outs_a[i], wa, stream=sa)
        _call(xb, r, wts, flags, outs_b[i], wb, stream=sb)
    torch.cuda.synchronize()
    for i in range(4):
        assert torch.equal(outs_a[i].view(torch.int16), ref_a.view(torch.int16)), f"stream a call {i}"
        assert torch.equal(outs_b[i].view(torch.int16), ref_b.view(torch.int16)), f"stream b call {i}"


PATH_KERNELS = {1: [8, 9, 10], 8: [11, 12, 13, 14], 300: [1, 2, 3, 4, 5, 6, 7]}  # moe_kernel_t ids


@pytest.mark.parametrize("kind", ["bf16", "q4"])
@pytest.mark.parametrize("M", [1, 8, 300])
def test_traced_call_matches_and_records_kernels(kind, M):
    """With a trace the call gives the bits of the untraced call and records each kernel of its
    path once, in launch order, with a finite duration; with a trace shorter than the path the
    rest of the kernels run untimed and unrecorded (count stops at capacity)."""
    import ctypes
    import bench
    hip = bench.Hip()
    r, wts, flags = _weights(kind, seed=7)
    x = upload(np.random.default_rng(30 + M).standard_normal((M, H)).astype(np.float32))
    ws = torch.empty(moe.workspace_size(M, H, E, I, IS, K, flags=flags), dtype=torch.uint8, device="cuda")
    ref = _call(x, r, wts, flags, torch.empty_like(x), ws).clone()
    torch.cuda.synchronize()
    want = PATH_KERNELS[M]
    for cap in (16, 2):
        begin, end = hip.events(16), hip.events(16)
        kid = (ctypes.c_int32 * 16)(*([-1] * 16))
        tr = moe.MoeTrace(ctypes.cast(begin, ctypes.POINTER(ctypes.c_void_p)),
                          ctypes.cast(end, ctypes.POINTER(ctypes.c_void_p)), kid, cap, 0)
        out = torch.empty_like(x)
        if kind == "q4":
            moe.forward_q4(x, r, *wts, K, out=out, flags=flags, workspace=ws, trace=tr)
        else:
            moe.forward(x, r, wts[0], wts[1], K, out=out, flags=flags, workspace=ws, trace=tr)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"capacity {cap}"
        n = min(len(want), cap)
        assert tr.count == n and list(kid[:16]) == want[:n] + [-1] * (16 - n), f"capacity {cap}"
        for i in range(n):
            assert 0.0 <= hip.elapsed_ms(begin[i], end[i]) < 1000.0
        hip.destroy(begin)
        hip.destroy(end)


def test_two_streams_cached_workspaces():
    """Calls that pass no workspace take the binding's cached one, one per (device, stream): calls
    interleaved on two streams, some of them growing their stream's buffer, give the bits of the
    same calls made one after another with their own workspaces."""
    r, wts, flags = _weights("bf16", seed=6)
    Ms = [8, 300, 40, 700, 1]
    xs = [upload(np.random.default_rng(40 + i).standard_normal((M, H)).astype(np.float32)) for i, M in enumerate(Ms)]
    refs = []
    for x in xs:
        ws = torch.empty(moe.workspace_size(x.shape[0], H, E, I, IS, K), dtype=torch.uint8, device="cuda")
        refs.append(_call(x, r, wts, flags, torch.empty_like(x), ws).clone())
    torch.cuda.synchronize()
    moe._ws_cache.clear()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for i, x in enumerate(xs):
        for s in (sa, sb):
            out = torch.empty_like(x)
            _call(x, r, wts, flags, out, None, stream=s)
            outs.append((i, out))
    torch.cuda.synchronize()
    for i, out in outs:
        assert torch.equal(out.view(torch.int16), refs[i].view(torch.int16)), f"call {i}"
    keys = [kk for kk in moe._ws_cache if kk[2] in (sa.cuda_stream, sb.cuda_stream)]
    assert len(keys) == 2, keys
