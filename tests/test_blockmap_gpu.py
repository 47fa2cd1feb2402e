"""The grouped GEMMs' block map, read back through the routing outputs.

"Optimizing on-device inference for Apple Silicon", section "Keep expert
routing on the GPU": after the histogram, prefix scan and scatter, a block
map lists the fixed-size blocks of rows the grouped matrix multiplication
works on.  Here a routed group of c rows is one tile when c <= 288, else
ceil((c - 32) / 256) tiles, all of 256 rows but the last, which takes the
rest (up to 288 rows: a group's last 1..32 rows past a multiple of 256 ride
with the tile before, so its weights are streamed once fewer); routed groups
come in expert order, then the shared expert's tokens in order in tiles of
256 rows but the last; every row of every group lies in exactly one tile."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from gpu_util import HostLayer, device_layer, moe, rand_case, routing_buffers, upload, S

pytestmark = pytest.mark.gpu
TILE = 256
LAST = TILE + 32  # the largest last tile of a routed group


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    moe.lib()
    yield


def expected_tiles(counts, offsets, M, shared):
    E = len(counts)
    want = []
    for g in range(E):
        c = int(counts[g])
        r0 = 0
        while c - r0 > LAST:  # full tiles while more than a last tile's worth is left
            want.append((g, r0, TILE, int(offsets[g]) + r0))
            r0 += TILE
        if c > r0:
            want.append((g, r0, c - r0, int(offsets[g]) + r0))
    if shared:
        for r0 in range(0, M, TILE):
            want.append((E, r0, min(TILE, M - r0), r0))
    return np.array(want, dtype=np.int64).reshape(-1, 4)


def run_blockmap(x, r, ex, sh, k, bias=None, I=None, Is=None):
    """One grouped-path call that exports the block map.  Its workspace is filled with 0x7F bytes
    first: the grouped GEMMs must take the block map from the exported buffers the scan wrote (a
    tile list read from this workspace would point far outside every buffer).  The output is
    compared bit for bit with the same call exporting nothing."""
    M, H = x.shape
    E = r.shape[0]
    f = moe.FLAG_FORCE_GEMM
    cap = moe.block_map_capacity(M, H, E, I, Is, k, flags=f)
    rb = routing_buffers(M, E, k)
    rb["tiles"] = torch.full((cap, 4), -1, dtype=torch.int32, device="cuda")
    rb["num_tiles"] = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    ws = torch.full((moe.workspace_size(M, H, E, I, Is, k, flags=f),), 0x7F, dtype=torch.uint8, device="cuda")
    out = moe.forward(x, r, ex, sh, k, routing=rb, router_bias=bias, flags=f, workspace=ws)
    ref = moe.forward(x, r, ex, sh, k, router_bias=bias, flags=f)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "exporting the block map changed the output"
    res = {n: t.cpu().numpy() for n, t in rb.items()}
    res["out"] = out.float().cpu().numpy()
    return res, cap


def check_blockmap(g, cap, M, k, shared):
    counts, offsets = g["counts"], g["offsets"]
    E = len(counts)
    assert counts.sum() == M * k and offsets[E] == M * k
    n = int(g["num_tiles"][0])
    want = expected_tiles(counts, offsets, M, shared)
    nt = np.where(counts <= LAST, (counts > 0).astype(np.int64), -(-(counts.astype(np.int64) - 32) // TILE))
    assert n == len(want) == int(nt.sum()) + (-(-M // TILE) if shared else 0)
    assert n <= cap
    got = g["tiles"][:n].astype(np.int64)
    assert np.array_equal(got, want), "block map differs"
    # every row of every group in exactly one tile
    cover = np.zeros(M * k + (M if shared else 0), dtype=np.int64)
    for gg, r0, rows, pos0 in got:
        assert 0 < rows <= (LAST if gg < E else TILE)
        base = 0 if gg < E else M * k
        cover[base + pos0: base + pos0 + rows] += 1
    assert (cover == 1).all()
    return n


def test_block_map_uniform_prefill():
    w = S.PREFILL
    x, r, ex, sh = device_layer(w)
    g, cap = run_blockmap(x, r, ex, sh, w.k, I=w.I, Is=w.I_shared)
    n = check_blockmap(g, cap, w.M, w.k, True)
    print("uniform: tiles", n, "groups", (g["counts"] > 0).sum())


def test_block_map_skewed_prefill():
    w = S.SKEW
    hl = HostLayer(w)
    x, r, ex, sh = device_layer(w)
    g, cap = run_blockmap(x, r, ex, sh, w.k, bias=torch.from_numpy(hl.bias).cuda(), I=w.I, Is=w.I_shared)
    assert g["counts"].max() > 1000
    n = check_blockmap(g, cap, w.M, w.k, True)
    # the routing the block map was built from is the oracle's (counts bit-exact; near-ties aside)
    ids = O.topk_ids(O.selection_logits(O.router_logits(hl.x(0, w.M), hl.router, hl.bias)), w.k)
    flagged = O.near_tie_flags(O.selection_logits(O.router_logits(hl.x(0, w.M), hl.router, hl.bias)), w.k)
    if not flagged.any():
        assert np.array_equal(g["counts"], O.route_tables(ids, w.E)[0])
    print("skew: tiles", n, "max group", g["counts"].max())


@pytest.mark.parametrize("M,E,k,shared", [(520, 32, 4, True), (600, 1, 1, False), (1, 16, 2, True),
                                          (257, 8, 8, True), (4100, 4, 2, False), (288, 4, 4, True),
                                          (289, 2, 2, False), (544, 1, 1, True), (545, 1, 1, False),
                                          (800, 1, 1, True)])
def test_block_map_hot_and_edge(M, E, k, shared):
    """A bias that sends every token to expert 5 first (or a single expert), one row, k = E, groups
    just over a multiple of the tile height and at the edges of the last tile's 288 rows (288 and
    289, 544 = 256 + 288 and 545, 800 = 2 * 256 + 288)."""
    Is = 64 if shared else 0
    x, r, ex, s, bias = rand_case(M, 128, E, k, 64, Is, seed=M, hot=5 if E > 5 else None)
    g, cap = run_blockmap(upload(x), upload(r), upload(ex), upload(s) if shared else None, k,
                          bias=None if bias is None else torch.from_numpy(bias).cuda(), I=64, Is=Is)
    check_blockmap(g, cap, M, k, shared)
    if E > 5:
        assert g["counts"][5] == M
    orc = O.moe_forward(x, r, ex, s, k, 64, bias=bias, I_shared=Is)
    rel = O.rel_err_per_token(g["out"], orc["out"])
    assert rel.max() <= 1e-2, rel.max()


@pytest.mark.parametrize("M,E,k,shared", [(8192, 16, 2, True), (8193, 16, 2, False), (8256, 8, 3, True),
                                          (4097, 256, 8, False)])
def test_routing_tables_both_scan_forms(M, E, k, shared):
    """Calls of up to 8192 tokens scan, build the block map and scatter in one launch (one
    workgroup per 64-token chunk), longer ones in two (one workgroup scans, then a scatter):
    on each side of that boundary, with a ragged last chunk, the counts, offsets, permutation
    and block map equal the oracle's routing tables (ids bit-exact, near-ties aside)."""
    Is = 64 if shared else 0
    x, r, ex, s, _ = rand_case(M, 128, E, k, 64, Is, seed=M + E)
    g, cap = run_blockmap(upload(x), upload(r), upload(ex), upload(s) if shared else None, k, I=64, Is=Is)
    check_blockmap(g, cap, M, k, shared)
    L32 = O.selection_logits(O.router_logits(x, r))
    ids = O.topk_ids(L32, k)
    flagged = O.near_tie_flags(L32, k)
    assert np.array_equal(g["topk_ids"][~flagged], ids[~flagged])
    if not flagged.any():
        counts, offsets, perm, _ = O.route_tables(ids, E)
        assert np.array_equal(g["counts"], counts) and np.array_equal(g["offsets"], offsets)
        assert np.array_equal(g["perm"], perm)
