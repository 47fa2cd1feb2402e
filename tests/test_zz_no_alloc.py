"""moe_layer_forward_noalloc: the layer with the library's static per-device scratch as its
workspace gives the bits of moe_layer_forward with a caller workspace, on every path, for two
calls in a row (the second with a smaller input, so it runs over what the first left in the
scratch), and rejects a call whose workspace exceeds the scratch."""
import numpy as np
import pytest
import torch

from gpu_util import device_layer, moe, rand_case, upload, S

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    moe.lib()
    yield


def _pair(x, r, ex, sh, k, flags=0, bias=None, routing=True):
    """(noalloc output, routing) and (workspace output, routing) for one input."""
    M, E = x.shape[0], r.shape[0]
    outs = []
    for fn in ("noalloc", "ws"):
        out = torch.full_like(x, float("nan"))
        rb = {"topk_ids": torch.full((M, k), -1, dtype=torch.int32, device="cuda")} if routing else None
        if fn == "noalloc":
            moe.forward_noalloc(x, r, ex, sh, k, out, router_bias=bias, routing=rb, flags=flags)
        else:
            moe.forward(x, r, ex, sh, k, out=out, router_bias=bias, routing=rb, flags=flags)
        torch.cuda.synchronize()
        outs.append((out.clone(), None if rb is None else rb["topk_ids"].clone()))
    return outs


@pytest.mark.parametrize("Ms,flags", [((1, 1), 0), ((8, 3), moe.FLAG_FORCE_GEMV), ((700, 300), 0),
                                       ((64, 2), moe.FLAG_FORCE_GEMM)])
def test_noalloc_matches_workspace_calls(Ms, flags):
    H, E, k, I, Is = 256, 32, 4, 128, 128
    _, r, ex, sh, _ = rand_case(1, H, E, k, I, Is, seed=sum(Ms))
    r, ex, sh = upload(r), upload(ex), upload(sh)
    for i, M in enumerate(Ms):
        x = upload(np.random.default_rng(100 * i + M).standard_normal((M, H)).astype(np.float32))
        (a, ia), (b, ib) = _pair(x, r, ex, sh, k, flags)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"call {i} (M={M}) output"
        assert torch.equal(ia, ib), f"call {i} (M={M}) ids"


def test_noalloc_full_shapes_and_limit():
    """At the configs' shapes: a decode row, then a 1,000-row grouped call (46 MB of workspace), then
    a 3-row small batch, each against the workspace call; M = 4096 exceeds the scratch."""
    w = S.PREFILL
    x, r, ex, sh = device_layer(w, x_rows=1000)
    ext, sht = moe.tile_weights(ex, w.H, w.I), moe.tile_weights(sh, w.H, w.I_shared)
    for xs, flags in ((x[:1], moe.FLAG_TILED_WEIGHTS), (x, moe.FLAG_TILED_WEIGHTS), (x[:3], 0)):
        xs = xs.contiguous()
        e, s = (ext, sht) if flags else (ex, sh)
        (a, ia), (b, ib) = _pair(xs, r, e, s, w.k, flags)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"M={xs.shape[0]}"
        assert torch.equal(ia, ib)
    big = torch.zeros(4096, w.H, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(big)
    with pytest.raises(moe.MoeError) as ei:
        moe.forward_noalloc(big, r, ex, sh, w.k, out)
    assert ei.value.status == 3  # MOE_ERR_WORKSPACE_TOO_SMALL
