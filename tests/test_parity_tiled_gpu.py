"""GPU tests of the tiled weight layout (moe_tile_weights, MOE_FLAG_TILED_WEIGHTS).

The tiling kernel is checked against the layout's definition in moe_layer.h,
written out on the host.  The layer on tiled weights is checked against the
same call on row-major weights, bit for bit, on every path (decode, small
batch, grouped), at partial panels and at the full prefill and decode
shapes: the layout changes where each weight is read from, never the
arithmetic or its order.  One case also goes against the oracle."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from gpu_util import (check, device_layer, grouped_path, moe, rand_case, routing_buffers, upload, S)

pytestmark = pytest.mark.gpu
TILED = moe.FLAG_TILED_WEIGHTS


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    moe.lib()
    yield


def host_tile(blocks: np.ndarray, H: int, I: int) -> np.ndarray:
    """The tiled layout of moe_layer.h applied to row-major blocks [n, 3*I*H] (any dtype)."""
    n = blocks.shape[0]
    dst = np.empty_like(blocks)
    k = np.arange(H)
    for m in range(2):  # gate, up: row i -> panel i // 128, tile row 64 c + 32 m + l
        for i in range(I):
            p, j = divmod(i, 128)
            rows_p = min(128, I - 128 * p)
            R = 64 * (j // 32) + 32 * m + j % 32
            pos = 256 * p * H + (k // 64) * (2 * rows_p * 64) + 64 * R + 8 * (((k // 8) % 8) ^ ((R // 2) % 8)) + k % 8
            dst[:, pos] = blocks[:, (m * I + i) * H + k]
    k = np.arange(I)
    for c in range(H):  # down: row c -> panel c // 256, tile row c % 256
        p, R = divmod(c, 256)
        rows_p = min(256, H - 256 * p)
        pos = 2 * I * H + 256 * p * I + (k // 64) * (rows_p * 64) + 64 * R + 8 * (((k // 8) % 8) ^ ((R // 2) % 8)) + k % 8
        dst[:, pos] = blocks[:, 2 * I * H + c * I + k]
    return dst


@pytest.mark.parametrize("H,I,n", [(192, 64, 2), (256, 192, 3), (192, 320, 1), (2048, 512, 2)])
def test_tile_weights_matches_layout_definition(H, I, n):
    rng = np.random.default_rng(H + I)
    bits = rng.integers(0, 1 << 16, size=(n, 3 * I * H), dtype=np.uint16)
    src = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    got = moe.tile_weights(src, H, I)
    torch.cuda.synchronize()
    want = host_tile(bits, H, I)
    assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), want)


def _both(x, r, ex, sh, k, flags=0, bias=None):
    """The layer on row-major and on tiled weights: (outputs, routing) pairs."""
    M, H = x.shape
    E = r.shape[0]
    I = ex.numel() // (3 * E * H)
    Is = 0 if sh is None else sh.numel() // (3 * H)
    ext = moe.tile_weights(ex, H, I)
    sht = None if sh is None else moe.tile_weights(sh, H, Is)
    res = []
    for e_w, s_w, f in ((ex, sh, flags), (ext, sht, flags | TILED)):
        rb = routing_buffers(M, E, k, grouped=grouped_path(M, k, E, flags))
        out = moe.forward(x, r, e_w, s_w, k, routing=rb, flags=f, router_bias=bias)
        torch.cuda.synchronize()
        res.append((out.view(torch.int16).cpu().numpy(), {n: t.cpu().numpy() for n, t in rb.items()}))
    return res


def _assert_same(res, label):
    (o1, r1), (o2, r2) = res
    assert np.array_equal(o1, o2), f"{label}: outputs differ on {(o1 != o2).sum()} elements"
    for n in r1:
        assert np.array_equal(r1[n], r2[n]), f"{label}: routing output {n} differs"


# partial panels: I % 128 != 0 (gate/up), H % 256 != 0 (down), shared I different from routed
SHAPES = [(256, 32, 4, 128, 128), (192, 16, 2, 64, 192), (256, 16, 2, 192, 64), (192, 24, 4, 320, 0),
          (512, 64, 8, 256, 128)]


@pytest.mark.parametrize("H,E,k,I,Is", SHAPES)
@pytest.mark.parametrize("M,flags", [(1, 0), (5, 0), (40, moe.FLAG_FORCE_GEMV), (1, moe.FLAG_FORCE_GEMM),
                                     (300, 0)])
def test_tiled_bitwise_equal_to_row_major(H, E, k, I, Is, M, flags):
    x, r, ex, sh, bias = rand_case(M, H, E, k, I, Is, seed=M + H + I)
    res = _both(upload(x), upload(r), upload(ex), None if sh is None else upload(sh), k, flags=flags)
    _assert_same(res, f"M={M} H={H} E={E} k={k} I={I} Is={Is} flags={flags}")


def test_tiled_against_oracle():
    M, H, E, k, I, Is = 70, 192, 16, 2, 192, 64
    x, r, ex, sh, bias = rand_case(M, H, E, k, I, Is, seed=9)
    ext = moe.tile_weights(upload(ex), H, I)
    sht = moe.tile_weights(upload(sh), H, Is)
    rb = routing_buffers(M, E, k)
    out = moe.forward(upload(x), upload(r), ext, sht, k, routing=rb, flags=TILED)
    torch.cuda.synchronize()
    g = {n: t.cpu().numpy() for n, t in rb.items()}
    g["out"] = out.float().cpu().numpy()

    def fn(force):
        return O.moe_forward(x, r, ex, sh, k, I, force_ids=force, I_shared=Is)
    check(g, fn, k, E, label="tiled M=70")


def test_tiled_full_prefill_and_decode_shapes():
    """H=2048, 256 experts top-8 + shared, I=512: M=4096 (grouped), 16 rows (small batch), 1 row."""
    w = S.PREFILL
    x, r, ex, sh = device_layer(w)
    for M, label in ((w.M, "prefill M=4096"), (16, "small M=16"), (1, "decode M=1")):
        _assert_same(_both(x[:M].contiguous(), r, ex, sh, w.k), label)


def test_tiled_skewed_prefill():
    w = S.SKEW
    x, r, ex, sh = device_layer(w)
    bias = torch.from_numpy(S.zipf_router_bias(w)).cuda()
    _assert_same(_both(x, r, ex, sh, w.k, bias=bias), "skew M=4096")


def test_tiled_long_prompt_chunk():
    """An 8192-token chunk of the long prompt (groups of ~288 rows: two tiles each)."""
    w = S.LONG
    x, r, ex, sh = device_layer(w, x_row0=3 * w.M)
    _assert_same(_both(x, r, ex, sh, w.k), "long chunk M=8192")
