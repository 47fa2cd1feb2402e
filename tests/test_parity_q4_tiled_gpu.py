"""GPU tests of the tiled layout of 4-bit experts (moe_tile_weights_q4,
MOE_FLAG_TILED_WEIGHTS on moe_layer_forward_q4).

The tiling kernel is checked against the layout's definition in moe_layer.h,
written out on the host at the level of single codes (nibbles) and group
words.  The layer on tiled 4-bit weights is checked against the same call on
row-major 4-bit weights, bit for bit, on every path (decode, small batch,
grouped), at partial panels and at the full prefill and decode shapes: the
layout changes where each code and group word is read from, never the
arithmetic or its order (the row-major 4-bit path is itself checked against
the oracle in test_parity_q4_gpu.py)."""
import numpy as np
import pytest
import torch

from gpu_util import grouped_path, moe, routing_buffers, S, SD

pytestmark = pytest.mark.gpu
TILED = moe.FLAG_TILED_WEIGHTS


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    moe.lib()
    yield


def tiled_order(H: int, I: int) -> np.ndarray:
    """src[e] = the row-major element stored at element e of a tiled block (moe_layer.h: panels of
    gate/up rows and of down rows, 64-element K-steps, tile rows in order, no chunk swizzle)."""
    src = np.empty(3 * I * H, dtype=np.int64)
    k = np.arange(H)
    for m in range(2):  # gate, up: row i -> panel i // 128, tile row 64 c + 32 m + l
        for i in range(I):
            p, j = divmod(i, 128)
            rows_p = min(128, I - 128 * p)
            R = 64 * (j // 32) + 32 * m + j % 32
            src[256 * p * H + (k // 64) * (2 * rows_p * 64) + 64 * R + k % 64] = (m * I + i) * H + k
    k = np.arange(I)
    for c in range(H):  # down: row c -> panel c // 256, tile row c % 256
        p, R = divmod(c, 256)
        rows_p = min(256, H - 256 * p)
        src[2 * I * H + 256 * p * I + (k // 64) * (rows_p * 64) + 64 * R + k % 64] = 2 * I * H + c * I + k
    return src


def host_tile_q4(codes: np.ndarray, words: np.ndarray, H: int, I: int):
    """The tiled 4-bit layout applied to row-major blocks: codes uint8 [n, 3IH/2] (low nibble first),
    group words [n, 3IH/64]."""
    src = tiled_order(H, I)
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)  # [n, 3IH] codes
    t = nib[:, src]
    tcodes = (t[:, 0::2] | (t[:, 1::2] << 4)).astype(np.uint8)
    twords = words[:, src[::64] // 64]
    return tcodes, twords


def _q4_random(E, n, rng, sigma=0.02):
    codes = rng.integers(0, 256, size=(E, n // 2), dtype=np.uint8)
    words = np.stack([S.q4_scale_bias(int(rng.integers(1 << 62)), n // 64, sigma) for _ in range(E)])
    return codes, words


def _dev_words(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).cuda()


@pytest.mark.parametrize("H,I,n", [(192, 64, 2), (256, 192, 3), (192, 320, 1), (2048, 512, 2)])
def test_tile_weights_q4_matches_layout_definition(H, I, n):
    rng = np.random.default_rng(H + I)
    codes, words = _q4_random(n, 3 * I * H, rng)
    gc, gw = moe.tile_weights_q4(torch.from_numpy(codes).cuda(), _dev_words(words), H, I)
    torch.cuda.synchronize()
    wc, ww = host_tile_q4(codes, words, H, I)
    assert np.array_equal(gc.cpu().numpy(), wc)
    assert np.array_equal(gw.cpu().numpy().view(np.uint32), ww.view(np.uint32))


def _both(x, r, codes, sb, sc, ssb, k, H, I, Is, flags=0, bias=None):
    """The layer on row-major and on tiled 4-bit weights: (outputs, routing) pairs."""
    M, E = x.shape[0], r.shape[0]
    tc, tsb = moe.tile_weights_q4(codes, sb, H, I)
    tsc, tssb = (None, None) if sc is None else moe.tile_weights_q4(sc, ssb, H, Is)
    res = []
    for w, f in (((codes, sb, sc, ssb), flags), ((tc, tsb, tsc, tssb), flags | TILED)):
        rb = routing_buffers(M, E, k, grouped=grouped_path(M, k, E, flags))
        out = moe.forward_q4(x, r, *w, k, routing=rb, flags=f, router_bias=bias)
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
def test_q4_tiled_bitwise_equal_to_row_major(H, E, k, I, Is, M, flags):
    rng = np.random.default_rng(M + H + I)
    q = lambda a: torch.from_numpy(S.bf16_bits_to_f32(S.f32_to_bf16_bits(a.astype(np.float32)))).to(
        torch.bfloat16).cuda()
    x, r = q(rng.standard_normal((M, H))), q(rng.standard_normal((E, H)) * 0.02)
    codes, words = _q4_random(E, 3 * I * H, rng)
    sc = ssb = None
    if Is:
        c1, w1 = _q4_random(1, 3 * Is * H, rng)
        sc, ssb = torch.from_numpy(c1[0]).cuda(), _dev_words(w1[0])
    res = _both(x, r, torch.from_numpy(codes).cuda(), _dev_words(words), sc, ssb, k, H, I, Is, flags=flags)
    _assert_same(res, f"M={M} H={H} E={E} k={k} I={I} Is={Is} flags={flags}")


@pytest.mark.parametrize("name,M", [("PREFILL", 4096), ("SKEW", 4096), ("DECODE", 1), ("DECODE", 16)])
def test_q4_tiled_full_shapes(name, M):
    """The configs' shapes: the grouped path at M=4096 (near-uniform and skewed routing), one decode
    row and a 16-row small batch."""
    w = getattr(S, name)
    x, r, codes, sb, sc, ssb = SD.layer_tensors_q4(w, x_rows=M)
    bias = None if not w.zipf_s else torch.from_numpy(S.zipf_router_bias(w)).cuda()
    res = _both(x, r, codes, sb, sc, ssb, w.k, w.H, w.I, w.I_shared, bias=bias)
    _assert_same(res, f"{name} M={M}")
