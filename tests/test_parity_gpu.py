"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the
seeded synthetic workloads (every output row at full size, except the
131,072-token single call, which is checked bit for bit against its 16
chunks and on sampled rows) and on the layer's edge and degenerate cases."""
import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from gpu_util import (HostLayer, bits_to_dev, check, device_layer, edge_case as _edge, moe, oracle_fn,
                      routing_buffers, run_gpu, S, SD, f32)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    moe.lib()
    yield


# ------------------------------------------------------------------ generator

def test_device_generator_matches_host():
    for key, start, n, sigma in [(S.stream_key(1, 2, 3, 4), 0, 100_003, 0.02), (12345, 777, 4096, 1.0),
                                 (S.x_key(S.PREFILL), 4095 * 2048, 2048, 1.0)]:
        t = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        SD.fill(t, key, start, sigma)
        got = t.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, S.normal_bf16(key, start, n, sigma))


# ------------------------------------------------------------------ tiny workload

def test_tiny_grouped_all_tokens():
    w = S.TINY
    hl = HostLayer(w)
    x, r, ex, sh = device_layer(w)
    g = run_gpu(x, r, ex, sh, w.k)
    check(g, oracle_fn(hl, hl.x(0, w.M)), w.k, w.E, label="tiny")


@pytest.mark.parametrize("flags", [0, moe.FLAG_FORCE_GEMM])
def test_tiny_single_rows(flags):
    w = S.TINY
    hl = HostLayer(w)
    _, r, ex, sh = device_layer(w)
    for t in [0, 1, 17, 63]:
        x1 = bits_to_dev(S.x_rows(w, t, 1))
        g = run_gpu(x1, r, ex, sh, w.k, flags=flags)
        check(g, oracle_fn(hl, hl.x(t, 1)), w.k, w.E, grouped=bool(flags), label=f"tiny row {t} flags {flags}")


# ------------------------------------------------------------------ full-size workloads

def _full_case(w, layer=0, x_row0=0):
    """One full-size call; every token's routing and output checked against the oracle."""
    hl = HostLayer(w, layer)
    xh = hl.x(x_row0, w.M)
    x, r, ex, sh = device_layer(w, layer, x_row0=x_row0)
    bias = None if hl.bias is None else torch.from_numpy(hl.bias).cuda()
    g = run_gpu(x, r, ex, sh, w.k, bias=bias)
    del ex
    ids_o = O.topk_ids(O.selection_logits(O.router_logits(xh, hl.router, hl.bias)), w.k)
    hl.prefetch(np.union1d(ids_o.ravel(), g["topk_ids"].ravel()))
    stats = check(g, oracle_fn(hl, xh), w.k, w.E, label=w.name)
    return g, stats


def test_prefill_full():
    g, st = _full_case(S.PREFILL)
    assert g["counts"].sum() == S.PREFILL.M * S.PREFILL.k
    print("prefill, all tokens", st)


def test_skew_full():
    g, st = _full_case(S.SKEW)
    counts = g["counts"]
    assert counts.max() > 1000 and (counts == 0).sum() > 50, "skewed routing expected"
    print("skew, all tokens", st, "max group", counts.max(), "empty", (counts == 0).sum())


def test_long_prefill_chunk():
    w = S.LONG
    g, st = _full_case(w, x_row0=5 * w.M)
    print("long chunk 5, all tokens", st)


def _route_all_tokens(hl, M, step, k):
    """The oracle's routing steps over all M token rows (scores in pieces of `step` rows)."""
    L = np.concatenate([O.router_logits(hl.x(t, min(step, M - t)), hl.router, hl.bias)
                        for t in range(0, M, step)])
    L32 = O.selection_logits(L)
    return L, L32, O.topk_ids(L32, k), O.near_tie_flags(L32, k)


def test_long_prompt_single_call():
    """The 131,072-token prompt in one call (the largest configuration): bit-identical to the
    same rows in 16 calls of 8,192; every token's scores, selection, weights and the
    histogram / offsets / permutation against the oracle; sampled tokens' outputs against it."""
    w = S.LONG
    big = S.reduced(w, M=w.tokens, chunks=1)
    x, r, ex, sh = device_layer(big)
    rb = routing_buffers(big.M, w.E, w.k, grouped=True)
    one = moe.forward(x, r, ex, sh, w.k, routing=rb)
    chunked = torch.empty_like(x)
    for c in range(w.chunks):
        moe.forward(x[c * w.M:(c + 1) * w.M], r, ex, sh, w.k, out=chunked[c * w.M:(c + 1) * w.M])
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), chunked.view(torch.int16)), "one call != 16 chunks"
    del ex, chunked
    hl = HostLayer(big)
    # routing of all 131,072 tokens: the same rules as check(), over the whole call
    L, L32, ids_o, flagged = _route_all_tokens(hl, big.M, w.M, w.k)
    ids_g = rb["topk_ids"].cpu().numpy().astype(np.int64)
    diff = (ids_g != ids_o).any(axis=1)
    assert not (diff & ~flagged).any(), f"ids differ on {(diff & ~flagged).sum()} unflagged tokens"
    assert O.valid_topk(L32[diff], ids_g[diff]).all(), "invalid top-k at flagged tokens"
    assert np.abs(rb["logits"].cpu().numpy().astype(np.float64) - L).max() < 1e-4, "router scores"
    werr = np.abs(rb["topk_w"].cpu().numpy().astype(np.float64) - O.topk_weights(L, ids_g)).max()
    assert werr <= 1e-5, f"routing weights differ by {werr}"
    counts, offsets, perm, _ = O.route_tables(ids_g, w.E)
    for name, want in (("counts", counts), ("offsets", offsets), ("perm", perm)):
        assert np.array_equal(rb[name].cpu().numpy(), want), name
    print("long prompt one call, routing of all tokens: flagged", int(flagged.sum()), "swapped",
          int(diff.sum()), "max group", int(counts.max()), "w err", werr)
    del L, L32
    rng = np.random.default_rng(17)
    sample = sorted(set(rng.choice(big.M, 6, replace=False).tolist()) | {0, big.M - 1})
    xs = np.concatenate([hl.x(t, 1) for t in sample])
    g = {n: rb[n][sample].cpu().numpy() for n in ("topk_ids", "topk_w", "logits")}
    g["out"] = one[sample].float().cpu().numpy()
    hl.prefetch(g["topk_ids"].ravel())
    st = check(g, oracle_fn(hl, xs), w.k, w.E, grouped=False, label="long prompt, one call")
    print("long prompt one call", st)


DECODE_ROWS = (0, 9, 18, 27, 36, 45, 54, 63)


def test_decode_full_shape():
    """Batch-1 decode at full shape: 8 token rows (one call each) through every one of the 40
    layers, every output against the oracle."""
    w = S.DECODE
    worst = 0.0
    for layer in range(w.layers):
        hl = HostLayer(w, layer)
        _, r, ex, sh = device_layer(w, layer, x_rows=1)
        xs = [bits_to_dev(S.x_rows(w, row, 1, layer)) for row in DECODE_ROWS]
        gs = [run_gpu(x1, r, ex, sh, w.k) for x1 in xs]
        # the two-launch decode path gives the same bits
        for x1, g1 in zip(xs, gs):
            two = moe.forward(x1, r, ex, sh, w.k, flags=moe.FLAG_DECODE_TWO_LAUNCH)
            assert np.array_equal(two.float().cpu().numpy(), g1["out"]), f"two launches, layer {layer}"
        del ex, r, sh
        g = {n: np.concatenate([one[n] for one in gs]) for n in gs[0]}
        xh = np.concatenate([hl.x(row, 1) for row in DECODE_ROWS])
        hl.prefetch(g["topk_ids"].ravel())
        st = check(g, oracle_fn(hl, xh), w.k, w.E, grouped=False, label=f"decode layer {layer}")
        worst = max(worst, st["max_rel"])
    print(f"decode: {len(DECODE_ROWS)} rows x {w.layers} layers, worst rel err {worst:.3e}")


# ------------------------------------------------------------------ edge cases (every output checked)

@pytest.mark.parametrize("M", [1, 2, 63, 64, 65, 257, 700])
def test_ragged_token_counts(M):
    # grouped path at every M (small M would default to the matrix-vector paths)
    _edge(M, 256, 32, 4, 128, 128, flags=moe.FLAG_FORCE_GEMM if M <= 64 else 0, seed=M)


def test_no_shared_expert():
    _edge(130, 256, 16, 2, 128, 0, seed=1)
    _edge(1, 256, 16, 2, 128, 0, seed=2)


@pytest.mark.parametrize("k", [1, 16])
def test_top1_and_all_experts(k):
    _edge(96, 256, 16, k, 64, 64, seed=k)


def test_single_expert_many_tiles():
    g, _ = _edge(600, 128, 1, 1, 64, 64, seed=3)
    assert g["counts"][0] == 600


def test_zero_router_exact_ties():
    g, _ = _edge(100, 256, 16, 4, 64, 64, zero_router=True)
    assert (g["topk_ids"] == np.arange(4)[None, :]).all()
    assert np.allclose(g["topk_w"], 0.25, rtol=0, atol=1e-7)


@pytest.mark.parametrize("M", [1, 5, 70])
@pytest.mark.parametrize("cluster", [40, 100])
def test_clustered_scores_select_exactly(M, cluster):
    """Scores set by a router bias (zero router weights): `cluster` experts on 16 levels within
    2^-8 of 1.0 (many exact ties), the rest near -4.  With 40 such experts the selection's
    prefilter keeps them all as candidates and ranks them; with 100 (more than a wave's 64 lanes)
    its full radix select takes over.  On the decode, small-batch and grouped paths the ids must be
    exactly the first k of (score descending, expert index ascending)."""
    E, k = 256, 8
    rng = np.random.default_rng(cluster + M)
    bias = (rng.standard_normal(E) - 4.0).astype(np.float32)
    members = rng.choice(E, cluster, replace=False)
    bias[members] = (1.0 + rng.integers(0, 16, cluster) * 2.0 ** -12).astype(np.float32)
    g, _ = _edge(M, 128, E, k, 64, 64, zero_router=True, bias=bias, seed=cluster)
    want = np.lexsort((np.arange(E), -bias.astype(np.float64)))[:k]
    assert (g["topk_ids"] == want[None, :]).all()


def test_hot_expert_bias():
    g, _ = _edge(520, 256, 32, 4, 64, 64, hot=5)
    assert (g["topk_ids"][:, 0] == 5).all() and g["counts"][5] == 520


@pytest.mark.parametrize("E", [100, 300, 1000])
def test_expert_counts(E):
    _edge(80, 128, E, 8, 64, 64, seed=E)
    _edge(1, 128, E, 8, 64, 64, seed=E + 1)


@pytest.mark.parametrize("M", [1, 4, 80])
def test_max_experts(M):
    """E at the supported maximum (1024, sixteen scores per lane in the top-k) on the decode,
    small-batch and grouped paths."""
    _edge(M, 128, 1024, 8, 64, 64, seed=1024 + M)


def test_shared_size_differs():
    _edge(90, 256, 16, 2, 128, 256, seed=5)
    _edge(90, 256, 16, 2, 256, 64, seed=6)
    _edge(1, 256, 16, 2, 128, 256, seed=7)


def test_hidden_not_multiple_of_128():
    _edge(70, 192, 16, 2, 64, 64, seed=8)
    _edge(1, 192, 16, 2, 64, 64, seed=9)


@pytest.mark.parametrize("M,flags", [(1, 0), (5, moe.FLAG_FORCE_GEMV), (70, 0)])
def test_largest_dimensions(M, flags):
    """H and I at the supported maximum (16384) on every path: 256 K-steps in the grouped GEMMs
    and the router scores, 16384-element rows in the matrix-vector kernels."""
    _edge(M, 16384, 4, 2, 64, 64, flags=flags, seed=M)      # H = 16384
    _edge(M, 64, 2, 1, 16384, 0, flags=flags, seed=M + 1)  # I = 16384 (down K), no shared expert
    _edge(M, 64, 2, 1, 64, 16384, flags=flags, seed=M + 2)  # shared I = 16384


def test_decode_topk_32():
    _edge(1, 128, 64, 32, 64, 64, seed=10)
    _edge(40, 128, 64, 32, 64, 64, seed=11)


# ------------------------------------------------------------------ properties (bit-exact)

def test_determinism_chunking_and_permutation():
    w = S.reduced(S.PREFILL, M=512, E=64)
    x, r, ex, sh = device_layer(w)
    a = moe.forward(x, r, ex, sh, w.k).clone()
    b = moe.forward(x, r, ex, sh, w.k).clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "run-to-run bits differ"
    c1 = moe.forward(x[:200].contiguous(), r, ex, sh, w.k).clone()
    c2 = moe.forward(x[200:].contiguous(), r, ex, sh, w.k).clone()
    assert torch.equal(torch.cat([c1, c2]).view(torch.int16), a.view(torch.int16)), "chunking changed bits"
    p = torch.randperm(w.M, generator=torch.Generator().manual_seed(0)).cuda()
    d = moe.forward(x[p].contiguous(), r, ex, sh, w.k)
    assert torch.equal(d.view(torch.int16), a[p].view(torch.int16)), "token permutation changed bits"


def test_route_matches_forward_routing():
    w = S.reduced(S.SKEW, M=300)
    hl = HostLayer(w)
    x, r, ex, sh = device_layer(w)
    bias = torch.from_numpy(hl.bias).cuda()
    g = run_gpu(x, r, ex, sh, w.k, bias=bias)
    rb = {k: torch.empty_like(torch.from_numpy(v)).cuda() for k, v in g.items() if k != "out"}
    moe.route(x, r, w.k, rb, router_bias=bias, I=w.I, I_shared=w.I_shared)
    torch.cuda.synchronize()
    for k, v in rb.items():
        assert np.array_equal(v.cpu().numpy(), g[k]), k


@pytest.mark.parametrize("H,E,k,I,Is", [(4096, 64, 8, 512, 512), (4096, 64, 16, 512, 512), (4160, 64, 8, 512, 512),
                                        (2048, 64, 32, 512, 512), (256, 16, 2, 576, 64), (192, 16, 2, 64, 0),
                                        (256, 300, 8, 128, 256)])
def test_decode_two_launch_limits(H, E, k, I, Is):
    """Batch-1 decode with MOE_FLAG_DECODE_TWO_LAUNCH at the edges of the two-launch path (H = 4096:
    256 down workgroups; top-16; no shared expert; E = 300) and just past them (H = 4160, h of 33
    slots beyond 64 KB, I = 576), where the three launches run: every output against the oracle."""
    _edge(1, H, E, k, I, Is, flags=moe.FLAG_DECODE_TWO_LAUNCH, seed=H + k + I)
