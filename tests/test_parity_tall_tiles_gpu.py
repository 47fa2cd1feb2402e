"""GPU parity of the grouped GEMMs' tall last tiles.

A routed group whose row count lies 1..32 rows past a multiple of 256 keeps
those rows in its last tile (up to 288 rows, nine 32-row blocks), so the
group's weights are streamed once fewer.  The ninth block has its own
staging and, in the gate/up GEMM, an exchange of up values between the row
groups of a workgroup; these cases put one expert (a router bias of 100 on
expert 5) at such counts: a group of 257..288 rows (one tile, first rows of
the group), 256 + 257..288 (the tall tile second), exactly 288 and 289, and
2 * 256 + 288, at full and partial weight panels, with and without a shared
expert.  bf16 and 4-bit experts, each row-major against the oracle and tiled
against row-major bit for bit."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from gpu_util import check, edge_case, grouped_path, moe, rand_case, routing_buffers, upload, S

pytestmark = pytest.mark.gpu
TILED = moe.FLAG_TILED_WEIGHTS
HOT = 5


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    moe.lib()
    yield


# (M, H, E, k, I, Is): expert 5 receives all M tokens
CASES = [(280, 256, 16, 4, 128, 128), (288, 256, 16, 4, 128, 128), (289, 256, 16, 4, 128, 128),
         (536, 320, 8, 2, 192, 64), (281, 192, 8, 1, 320, 0), (800, 2048, 64, 8, 512, 512),
         (270, 2048, 32, 8, 512, 0)]


def _bias(E):
    b = np.zeros(E, np.float32)
    b[HOT] = 100.0
    return b


def _run(x, r, w, k, bias, flags, q4):
    M, E = x.shape[0], r.shape[0]
    rb = routing_buffers(M, E, k, grouped=grouped_path(M, k, E, flags))
    b = torch.from_numpy(bias).cuda()
    if q4:
        out = moe.forward_q4(x, r, *w, k, routing=rb, flags=flags, router_bias=b)
    else:
        out = moe.forward(x, r, *w, k, routing=rb, flags=flags, router_bias=b)
    torch.cuda.synchronize()
    res = {n: t.cpu().numpy() for n, t in rb.items()}
    res["out"] = out.float().cpu().numpy()
    res["bits"] = out.view(torch.int16).cpu().numpy()
    return res


def _same(a, b, label):
    for n in a:
        assert np.array_equal(a[n], b[n]), f"{label}: tiled and row-major differ in {n}"


@pytest.mark.parametrize("M,H,E,k,I,Is", CASES)
def test_tall_tiles_bf16(M, H, E, k, I, Is):
    label = f"bf16 M={M} H={H} E={E} k={k} I={I} Is={Is}"
    g, _ = edge_case(M, H, E, k, I, Is, seed=M + H, hot=HOT)
    assert g["counts"][HOT] == M
    # the same inputs again: row-major through this file's call, then tiled, the same bits
    x, r, ex, sh, bias = rand_case(M, H, E, k, I, Is, seed=M + H, hot=HOT)
    xd, rd, exd = upload(x), upload(r), upload(ex)
    shd = None if sh is None else upload(sh)
    row = _run(xd, rd, (exd, shd), k, bias, 0, False)
    assert np.array_equal(row["out"], g["out"]), label
    ext = moe.tile_weights(exd, H, I)
    sht = None if shd is None else moe.tile_weights(shd, H, Is)
    _same(row, _run(xd, rd, (ext, sht), k, bias, TILED, False), label)


def _q4_random(E, n, rng, sigma=0.02):
    codes = rng.integers(0, 256, size=(E, n // 2), dtype=np.uint8)
    words = np.stack([S.q4_scale_bias(int(rng.integers(1 << 62)), n // 64, sigma) for _ in range(E)])
    return codes, words


@pytest.mark.parametrize("M,H,E,k,I,Is", CASES)
def test_tall_tiles_q4(M, H, E, k, I, Is):
    label = f"q4 M={M} H={H} E={E} k={k} I={I} Is={Is}"
    rng = np.random.default_rng(M + H + 1)
    q = lambda a: S.bf16_bits_to_f32(S.f32_to_bf16_bits(a.astype(np.float32)))
    x = q(rng.standard_normal((M, H)))
    r = q(rng.standard_normal((E, H)) * 0.02)
    codes, words = _q4_random(E, 3 * I * H, rng)
    sc = sw = None
    if Is:
        sc, sw = _q4_random(1, 3 * Is * H, rng)
    bias = _bias(E)
    dev_w = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).cuda()
    cd, wd = torch.from_numpy(codes).cuda(), dev_w(words)
    scd = None if sc is None else torch.from_numpy(sc[0]).cuda()
    swd = None if sw is None else dev_w(sw[0])
    xd, rd = upload(x), upload(r)
    g = _run(xd, rd, (cd, wd, scd, swd), k, bias, 0, True)
    assert g["counts"][HOT] == M
    experts = lambda e: O.unpack_expert(O.dequant_q4(codes[e], words[e]), I, H)
    shared = None if sc is None else O.dequant_q4(sc[0], sw[0])

    def fn(force):
        return O.moe_forward(x, r, experts, shared, k, I, bias=bias, force_ids=force, I_shared=Is)
    check(g, fn, k, E, grouped=True, label=label)
    tc, tw = moe.tile_weights_q4(cd, wd, H, I)
    tsc, tsw = (None, None) if scd is None else moe.tile_weights_q4(scd, swd, H, Is)
    _same(g, _run(xd, rd, (tc, tw, tsc, tsw), k, bias, TILED, True), label)
