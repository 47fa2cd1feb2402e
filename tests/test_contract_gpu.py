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
@pytest.mark.parametrize("M", [1, 3, 8, 300, 8200, -1])  # -1: one row on the two-launch decode path
def test_graph_replay_matches_eager(kind, M):
    r, wts, flags = _weights(kind)
    if M == -1:
        M, flags = 1, flags | TWO
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


# moe_kernel_t ids; calls of up to 5 rows (8 with 4-bit experts) run the decode kernels; grouped
# calls of more than 8192 tokens scan and scatter in two launches
PATH_KERNELS = {1: [8, 9, 10], 3: [8, 9, 10], 8: [11, 12, 13, 14], 300: [1, 2, 18, 5, 6, 17],
                8200: [1, 2, 3, 4, 5, 6, 17], -1: [15, 16]}


def path_kernels(kind, M):
    return [8, 9, 10] if kind == "q4" and M == 8 else PATH_KERNELS[M]
TWO = moe.FLAG_DECODE_TWO_LAUNCH


@pytest.mark.parametrize("kind", ["bf16", "q4"])
@pytest.mark.parametrize("M", [1, 3, 8, 300, 8200, -1])  # -1: one row on the two-launch decode path
def test_traced_call_matches_and_records_kernels(kind, M):
    """With a trace the call gives the bits of the untraced call and records each kernel of its
    path once, in launch order, with a finite duration; with a trace shorter than the path the
    rest of the kernels run untimed and unrecorded (count stops at capacity)."""
    import ctypes
    import bench
    hip = bench.Hip()
    r, wts, flags = _weights(kind, seed=7)
    want = path_kernels(kind, M)
    if M == -1:
        M, flags = 1, flags | TWO
    x = upload(np.random.default_rng(30 + M).standard_normal((M, H)).astype(np.float32))
    ws = torch.empty(moe.workspace_size(M, H, E, I, IS, K, flags=flags), dtype=torch.uint8, device="cuda")
    ref = _call(x, r, wts, flags, torch.empty_like(x), ws).clone()
    torch.cuda.synchronize()
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


@pytest.mark.parametrize("kind", ["bf16", "q4"])
def test_decode_wait_status_and_give_up(kind):
    """The two-launch decode path's second launch waits inside the kernel for the routed experts'
    gated activations.  A normal call reports wait_status 0 (so do the paths without such a wait); with
    the test hook MOE_FLAG_WAIT_PROBE the wait is for a condition that never occurs, bounded to a
    few polls: it gives up, every output row is NaN and wait_status is 1, and the next normal call
    on the same workspace is exact again."""
    r, wts, flags = _weights(kind, seed=8)
    x = upload(np.random.default_rng(77).standard_normal((1, H)).astype(np.float32))
    ws = torch.empty(moe.workspace_size(1, H, E, I, IS, K, flags=flags), dtype=torch.uint8, device="cuda")
    flags |= TWO

    def run(extra, M_x=x, extra_off=0):
        st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        out = torch.empty_like(M_x)
        rb = {"wait_status": st}
        f = (flags | extra) & ~extra_off
        if len(wts) == 4:
            moe.forward_q4(M_x, r, *wts, K, out=out, flags=f, workspace=ws, routing=rb)
        else:
            moe.forward(M_x, r, wts[0], wts[1], K, out=out, flags=f, workspace=ws, routing=rb)
        torch.cuda.synchronize()
        return out, int(st.item())

    ref, st0 = run(0)
    assert st0 == 0 and torch.isfinite(ref.float()).all()
    bad, st1 = run(moe.FLAG_WAIT_PROBE)
    assert st1 == 1 and torch.isnan(bad.float()).all()
    again, st2 = run(0)
    assert st2 == 0 and torch.equal(again.view(torch.int16), ref.view(torch.int16))
    # paths without an in-kernel wait write 0 (the three-launch decode path too)
    three, st3 = run(0, extra_off=TWO)
    assert st3 == 0 and torch.equal(three.view(torch.int16), ref.view(torch.int16))
    for M in (8, 300):
        xm = upload(np.random.default_rng(M).standard_normal((M, H)).astype(np.float32))
        wsm = torch.empty(moe.workspace_size(M, H, E, I, IS, K, flags=flags), dtype=torch.uint8, device="cuda")
        st = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        f = flags & ~TWO
        if len(wts) == 4:
            moe.forward_q4(xm, r, *wts, K, flags=f, workspace=wsm, routing={"wait_status": st})
        else:
            moe.forward(xm, r, wts[0], wts[1], K, flags=f, workspace=wsm, routing={"wait_status": st})
        torch.cuda.synchronize()
        assert int(st.item()) == 0, M
