"""GPU parity of the small-batch path (MOE_FLAG_FORCE_GEMV with 2 <= M <= 64:
matrix-vector products over the union of the experts the rows select)
against the oracle, on the decode workload's shapes and on edge cases, plus
properties that pin the union bookkeeping: the result per row equals the
batch-1 decode path's, bit for bit, and does not depend on the batch's
composition."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from gpu_util import (HostLayer, bits_to_dev, check, device_layer, edge_case, moe, oracle_fn, run_gpu, S)

pytestmark = pytest.mark.gpu
GEMV = moe.FLAG_FORCE_GEMV


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    moe.lib()
    yield


@pytest.mark.parametrize("M", [2, 3, 16, 64])
def test_small_tiny(M):
    w = S.TINY
    hl = HostLayer(w)
    x, r, ex, sh = device_layer(w)
    g = run_gpu(x[:M].contiguous(), r, ex, sh, w.k, flags=GEMV)
    check(g, oracle_fn(hl, hl.x(0, M)), w.k, w.E, grouped=False, label=f"tiny small M={M}")


@pytest.mark.parametrize("M", [2, 5, 16])
def test_small_decode_shape(M):
    """H=2048, 256 experts top-8 + shared, I=512; every row checked."""
    w = S.DECODE
    layer = 3
    hl = HostLayer(w, layer)
    xb = S.x_rows(w, 10, M, layer)
    _, r, ex, sh = device_layer(w, layer, x_rows=1)
    g = run_gpu(bits_to_dev(xb), r, ex, sh, w.k, flags=GEMV)
    del ex
    hl.prefetch(g["topk_ids"].ravel())
    st = check(g, oracle_fn(hl, hl.x(10, M)), w.k, w.E, grouped=False, label=f"decode-shape small M={M}")
    print(M, st, "union", len(np.unique(g["topk_ids"])))


def test_small_matches_decode_rows_bitwise():
    """Each row of a small batch equals the batch-1 decode path on that row alone."""
    w = S.reduced(S.DECODE, E=64, k=8)
    x, r, ex, sh = device_layer(w, 0, x_rows=12)
    batch = moe.forward(x, r, ex, sh, w.k, flags=GEMV).clone()
    for t in range(x.shape[0]):
        one = moe.forward(x[t:t + 1].contiguous(), r, ex, sh, w.k)
        assert torch.equal(one.view(torch.int16), batch[t:t + 1].view(torch.int16)), f"row {t}"


def test_small_batch_composition_invariant():
    """Permuting or splitting the batch changes no output bit (union lists differ)."""
    w = S.reduced(S.DECODE, E=64, k=8)
    x, r, ex, sh = device_layer(w, 1, x_rows=40)
    a = moe.forward(x, r, ex, sh, w.k, flags=GEMV).clone()
    p = torch.randperm(40, generator=torch.Generator().manual_seed(1)).cuda()
    b = moe.forward(x[p].contiguous(), r, ex, sh, w.k, flags=GEMV)
    assert torch.equal(b.view(torch.int16), a[p].view(torch.int16))
    c1 = moe.forward(x[:7].contiguous(), r, ex, sh, w.k, flags=GEMV).clone()
    c2 = moe.forward(x[7:].contiguous(), r, ex, sh, w.k, flags=GEMV)
    assert torch.equal(torch.cat([c1, c2]).view(torch.int16), a.view(torch.int16))


def test_small_against_grouped_path():
    """Both multi-row paths on the same inputs: identical routing, outputs within the bar."""
    w = S.reduced(S.DECODE, E=64, k=8)
    x, r, ex, sh = device_layer(w, 2, x_rows=24)
    gs = run_gpu(x, r, ex, sh, w.k, flags=GEMV)
    gg = run_gpu(x, r, ex, sh, w.k, flags=moe.FLAG_FORCE_GEMM)
    assert np.array_equal(gs["topk_ids"], gg["topk_ids"])
    assert np.abs(gs["topk_w"] - gg["topk_w"]).max() <= 1e-6
    assert O.rel_err_per_token(gs["out"], gg["out"]).max() <= 1e-2


# ------------------------------------------------------------------ edge cases (every output checked)

@pytest.mark.parametrize("M", [2, 17, 64])
def test_small_ragged(M):
    edge_case(M, 256, 32, 4, 128, 128, flags=GEMV, seed=200 + M)


def test_small_no_shared_and_shapes():
    edge_case(9, 256, 16, 2, 128, 0, flags=GEMV, seed=1)
    edge_case(6, 192, 16, 2, 64, 256, flags=GEMV, seed=2)
    edge_case(6, 256, 16, 2, 256, 64, flags=GEMV, seed=3)
    edge_case(4, 4096, 16, 2, 64, 64, flags=GEMV, seed=4)  # H past one 2048-element load batch


def test_small_one_expert_all_rows():
    """E = 1: the union is one expert whose list holds every row (more than one register batch)."""
    g, _ = edge_case(23, 128, 1, 1, 64, 64, flags=GEMV, seed=5)
    assert (g["topk_ids"] == 0).all()


def test_small_hot_expert_and_ties():
    g, _ = edge_case(30, 256, 32, 4, 64, 64, flags=GEMV, hot=5, seed=6)
    assert (g["topk_ids"][:, 0] == 5).all()
    g, _ = edge_case(12, 256, 16, 4, 64, 64, flags=GEMV, zero_router=True)
    assert (g["topk_ids"] == np.arange(4)[None, :]).all()


@pytest.mark.parametrize("E,k", [(300, 8), (1000, 8), (64, 32)])
def test_small_expert_counts_and_top32(E, k):
    edge_case(20, 128, E, k, 64, 64, flags=GEMV, seed=E + k)


def test_small_route_matches_forward():
    w = S.reduced(S.DECODE, E=64, k=8)
    x, r, ex, sh = device_layer(w, 0, x_rows=10)
    g = run_gpu(x, r, ex, sh, w.k, flags=GEMV)
    rb = {k: torch.empty_like(torch.from_numpy(v)).cuda() for k, v in g.items() if k != "out"}
    moe.route(x, r, w.k, rb, flags=GEMV, I=w.I, I_shared=w.I_shared)
    torch.cuda.synchronize()
    for k, v in rb.items():
        assert np.array_equal(v.cpu().numpy(), g[k]), k


# ------------------------------------------------------------------ batches of 2 to 4 rows

def test_few_row_pieces_match_larger_batch_bitwise():
    """A 3-row and a 4-row batch equal the same rows of a 16-row batch bit for bit, and each of
    the 4 rows equals the one-row decode path on it."""
    w = S.reduced(S.DECODE, E=64, k=8)
    x, r, ex, sh = device_layer(w, 3, x_rows=16)
    a = moe.forward(x, r, ex, sh, w.k, flags=GEMV).clone()
    b3 = moe.forward(x[:3].contiguous(), r, ex, sh, w.k, flags=GEMV).clone()
    b4 = moe.forward(x[3:7].contiguous(), r, ex, sh, w.k, flags=GEMV).clone()
    assert torch.equal(b3.view(torch.int16), a[:3].view(torch.int16))
    assert torch.equal(b4.view(torch.int16), a[3:7].view(torch.int16))
    for t in range(3, 7):
        one = moe.forward(x[t:t + 1].contiguous(), r, ex, sh, w.k)
        assert torch.equal(one.view(torch.int16), b4[t - 3:t - 2].view(torch.int16)), f"row {t}"


@pytest.mark.parametrize("M,E,k", [(4, 1000, 8), (4, 64, 32), (3, 1, 1), (2, 300, 8)])
def test_few_rows_expert_counts_and_top32(M, E, k):
    """The widest selections (E up to 1000, k = 32) and the smallest union (one expert) on a few rows."""
    edge_case(M, 128, E, k, 64, 64, flags=GEMV, seed=7 * M + E + k)


def test_few_rows_hot_expert_and_ties():
    g, _ = edge_case(4, 256, 32, 4, 64, 64, flags=GEMV, hot=5, seed=8)
    assert (g["topk_ids"][:, 0] == 5).all()
    g, _ = edge_case(3, 256, 16, 4, 64, 0, flags=GEMV, zero_router=True)
    assert (g["topk_ids"] == np.arange(4)[None, :]).all()


def test_few_rows_route_matches_forward():
    w = S.reduced(S.DECODE, E=64, k=8)
    x, r, ex, sh = device_layer(w, 0, x_rows=3)
    g = run_gpu(x, r, ex, sh, w.k, flags=GEMV)
    rb = {k: torch.empty_like(torch.from_numpy(v)).cuda() for k, v in g.items() if k != "out"}
    moe.route(x, r, w.k, rb, flags=GEMV, I=w.I, I_shared=w.I_shared)
    torch.cuda.synchronize()
    for k, v in rb.items():
        assert np.array_equal(v.cpu().numpy(), g[k]), k
