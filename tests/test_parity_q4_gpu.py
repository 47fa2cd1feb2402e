"""GPU parity of the 4-bit expert-weight path (moe_layer_forward_q4) against
the oracle: the oracle rebuilds every weight from its code and its group's
scale and bias (dequant_q4) and runs the same layer in float64, on the
seeded synthetic workloads (4-bit variant) and on the edge shapes."""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from gpu_util import check, grouped_path, moe, routing_buffers, S, SD, f32

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    moe.lib()
    yield


class HostLayerQ4:
    """Oracle-side copy of one layer with 4-bit experts, regenerated on the host."""

    def __init__(self, w, layer=0):
        self.w, self.layer = w, layer
        self.router = f32(S.router_weight(w, layer))
        self.bias = S.zipf_router_bias(w, layer)
        self.shared = None
        if w.I_shared:
            c, g = S.q4_shared(w, layer)
            self.shared = O.dequant_q4(c, g)
        self._experts = {}

    def x(self, row0, n):
        return f32(S.x_rows(self.w, row0, n, self.layer))

    def _gen(self, e):
        c, g = S.q4_expert(self.w, self.layer, e)
        return O.unpack_expert(O.dequant_q4(c, g), self.w.I, self.w.H)

    def prefetch(self, experts):
        todo = sorted(set(int(e) for e in experts) - set(self._experts))
        with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4)) as ex:
            for e, v in zip(todo, ex.map(self._gen, todo)):
                self._experts[e] = v

    def expert(self, e):
        if e not in self._experts:
            self._experts[e] = self._gen(e)
        return self._experts[e]

    def oracle(self, x_host, tokens=None):
        def fn(force):
            return O.moe_forward(x_host, self.router, self.expert, self.shared, self.w.k, self.w.I, bias=self.bias,
                                 force_ids=force, tokens=tokens, I_shared=self.w.I_shared)
        return fn


def run_q4(x, r, codes, sb, sc, ssb, k, bias=None, flags=0):
    M, E = x.shape[0], r.shape[0]
    grouped = grouped_path(M, k, E, flags)
    rb = routing_buffers(M, E, k, grouped=grouped)
    out = moe.forward_q4(x, r, codes, sb, sc, ssb, k, routing=rb, flags=flags, router_bias=bias)
    torch.cuda.synchronize()
    res = {name: t.cpu().numpy() for name, t in rb.items()}
    res["out"] = out.float().cpu().numpy()
    return res


def bits_to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def test_device_q4_generator_matches_host():
    w = S.TINY
    codes = torch.empty(w.expert_elems() // 2, dtype=torch.uint8, device="cuda")
    sb = torch.empty(w.expert_elems() // 64, dtype=torch.int32, device="cuda")
    ck, gk = S.q4_expert_key(w, 0, 5, False), S.q4_expert_key(w, 0, 5, True)
    SD.fill_q4(codes, sb, ck, gk, w.w_sigma)
    hc, hg = S.q4_expert(w, 0, 5)
    assert np.array_equal(codes.cpu().numpy(), hc)
    assert np.array_equal(sb.cpu().numpy().view(np.uint32), hg)


def test_q4_tiny_grouped_all_tokens():
    w = S.TINY
    hl = HostLayerQ4(w)
    x, r, ex, esb, sh, ssb = SD.layer_tensors_q4(w)
    g = run_q4(x, r, ex, esb, sh, ssb, w.k)
    check(g, hl.oracle(hl.x(0, w.M)), w.k, w.E, label="q4 tiny")


@pytest.mark.parametrize("flags", [0, moe.FLAG_FORCE_GEMM])
def test_q4_tiny_single_rows(flags):
    w = S.TINY
    hl = HostLayerQ4(w)
    _, r, ex, esb, sh, ssb = SD.layer_tensors_q4(w)
    for t in [0, 9, 63]:
        x1 = bits_to_dev(S.x_rows(w, t, 1))
        g = run_q4(x1, r, ex, esb, sh, ssb, w.k, flags=flags)
        check(g, hl.oracle(hl.x(t, 1)), w.k, w.E, grouped=bool(flags), label=f"q4 tiny row {t} flags {flags}")


def test_q4_decode_full_shape():
    """4-bit decode at full shape: 8 token rows (one call each) through all 40 layers."""
    w = S.DECODE
    rows = (0, 9, 18, 27, 36, 45, 54, 63)
    for layer in range(w.layers):
        hl = HostLayerQ4(w, layer)
        _, r, ex, esb, sh, ssb = SD.layer_tensors_q4(w, layer, x_rows=1)
        xs = [bits_to_dev(S.x_rows(w, row, 1, layer)) for row in rows]
        gs = [run_q4(x1, r, ex, esb, sh, ssb, w.k) for x1 in xs]
        for x1, g1 in zip(xs, gs):  # the two-launch decode path gives the same bits
            two = moe.forward_q4(x1, r, ex, esb, sh, ssb, w.k, flags=moe.FLAG_DECODE_TWO_LAUNCH)
            assert np.array_equal(two.float().cpu().numpy(), g1["out"]), f"two launches, layer {layer}"
        del ex, esb
        g = {n: np.concatenate([one[n] for one in gs]) for n in gs[0]}
        hl.prefetch(g["topk_ids"].ravel())
        xh = np.concatenate([hl.x(row, 1) for row in rows])
        check(g, hl.oracle(xh), w.k, w.E, grouped=False, label=f"q4 decode layer {layer}")


@pytest.mark.parametrize("name", ["PREFILL", "SKEW"])
def test_q4_prefill_full(name):
    """Full-size 4-bit prefill: every token's routing and output against the oracle."""
    w = getattr(S, name)
    hl = HostLayerQ4(w)
    x, r, ex, esb, sh, ssb = SD.layer_tensors_q4(w)
    bias = None if hl.bias is None else torch.from_numpy(hl.bias).cuda()
    g = run_q4(x, r, ex, esb, sh, ssb, w.k, bias=bias)
    del ex, esb
    xh = hl.x(0, w.M)
    ids_o = O.topk_ids(O.selection_logits(O.router_logits(xh, hl.router, hl.bias)), w.k)
    hl.prefetch(np.union1d(ids_o.ravel(), g["topk_ids"].ravel()))
    st = check(g, hl.oracle(xh), w.k, w.E, label=f"q4 {name}")
    assert g["counts"].sum() == w.M * w.k
    print(name, "all tokens", st)


def _q4_random(E, n, rng, sigma=0.02):
    """Random 4-bit blocks: codes uint8 [E, n/2], words uint32 [E, n/64] (host), from the generator's recipe."""
    codes = rng.integers(0, 256, size=(E, n // 2), dtype=np.uint8)
    words = np.stack([S.q4_scale_bias(int(rng.integers(1 << 62)), n // 64, sigma) for _ in range(E)])
    return codes, words


def _edge_q4(M, H, E, k, I, Is, flags=0, seed=0):
    rng = np.random.default_rng(seed)
    q = lambda a: S.bf16_bits_to_f32(S.f32_to_bf16_bits(a.astype(np.float32)))
    x = q(rng.standard_normal((M, H)))
    r = q(rng.standard_normal((E, H)) * 0.02)
    codes, words = _q4_random(E, 3 * I * H, rng)
    sc = sw = None
    if Is:
        sc, sw = _q4_random(1, 3 * Is * H, rng)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).cuda()
    dev_w = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).cuda()
    g = run_q4(up(x), up(r), torch.from_numpy(codes).cuda(), dev_w(words),
               None if sc is None else torch.from_numpy(sc[0]).cuda(), None if sw is None else dev_w(sw[0]),
               k, flags=flags)
    experts = lambda e: O.unpack_expert(O.dequant_q4(codes[e], words[e]), I, H)
    shared = None if sc is None else O.dequant_q4(sc[0], sw[0])

    def fn(force):
        return O.moe_forward(x, r, experts, shared, k, I, force_ids=force, I_shared=Is)
    grouped = grouped_path(M, k, E, flags)
    return check(g, fn, k, E, grouped=grouped, label=f"q4 M={M} H={H} E={E} k={k} I={I} Is={Is}")


@pytest.mark.parametrize("M", [1, 2, 65, 257])
def test_q4_ragged_token_counts(M):
    _edge_q4(M, 256, 32, 4, 128, 128, seed=M)  # M = 2: the small-batch path
    if M <= 64:
        _edge_q4(M, 256, 32, 4, 128, 128, flags=moe.FLAG_FORCE_GEMM, seed=100 + M)


def test_q4_no_shared_expert_and_shapes():
    _edge_q4(70, 256, 16, 2, 128, 0, seed=1)
    _edge_q4(1, 256, 16, 2, 128, 0, seed=2)
    _edge_q4(60, 192, 16, 2, 64, 256, seed=3)
    _edge_q4(1, 192, 16, 2, 64, 256, seed=4)


def test_q4_many_experts_and_top32():
    _edge_q4(40, 128, 300, 8, 64, 64, flags=moe.FLAG_FORCE_GEMM, seed=5)
    _edge_q4(1, 128, 300, 8, 64, 64, seed=6)
    _edge_q4(1, 128, 64, 32, 64, 64, seed=7)
    _edge_q4(20, 128, 64, 32, 64, 64, seed=8)


@pytest.mark.parametrize("M", [3, 6, 8])
def test_q4_few_rows_route_matches_forward(M):
    """4-bit calls of up to eight rows run the decode kernels (a grid row per token row); their
    scores, selections and weights equal, bit for bit, those of the routing-only call, which takes
    the small-batch router and selection above four rows, and each row equals a one-row call."""
    w = S.reduced(S.DECODE, E=64, k=8)
    x, r, ec, esb, sc, ssb = SD.layer_tensors_q4(w, 2, x_rows=M)
    g = run_q4(x, r, ec, esb, sc, ssb, w.k, flags=moe.FLAG_FORCE_GEMV)
    rb = {k: torch.empty_like(torch.from_numpy(v)).cuda() for k, v in g.items() if k != "out"}
    moe.route(x, r, w.k, rb, flags=moe.FLAG_FORCE_GEMV, I=w.I, I_shared=w.I_shared)
    torch.cuda.synchronize()
    for name, v in rb.items():
        assert np.array_equal(v.cpu().numpy(), g[name]), name
    for t in (0, M - 1):
        one = run_q4(x[t:t + 1].contiguous(), r, ec, esb, sc, ssb, w.k)
        assert np.array_equal(one["out"], g["out"][t:t + 1]), f"row {t}"


@pytest.mark.parametrize("M", [1, 4, 80])
def test_q4_max_experts(M):
    """E at the supported maximum (1024) on the decode, small-batch and grouped paths."""
    _edge_q4(M, 128, 1024, 8, 64, 64, seed=2048 + M)


# ------------------------------------------------------------------ small-batch path (4-bit experts)

def test_q4_small_decode_shape():
    w = S.DECODE
    M, layer = 8, 2
    hl = HostLayerQ4(w, layer)
    _, r, ex, esb, sh, ssb = SD.layer_tensors_q4(w, layer, x_rows=1)
    g = run_q4(bits_to_dev(S.x_rows(w, 20, M, layer)), r, ex, esb, sh, ssb, w.k, flags=moe.FLAG_FORCE_GEMV)
    del ex, esb
    check(g, hl.oracle(hl.x(20, M)), w.k, w.E, grouped=False, label=f"q4 small decode-shape M={M}")


@pytest.mark.parametrize("M", [2, 16, 64])
def test_q4_small_edges(M):
    _edge_q4(M, 256, 32, 4, 128, 128, flags=moe.FLAG_FORCE_GEMV, seed=300 + M)


def test_q4_small_shapes():
    _edge_q4(7, 256, 16, 2, 128, 0, flags=moe.FLAG_FORCE_GEMV, seed=9)
    _edge_q4(7, 192, 16, 2, 64, 256, flags=moe.FLAG_FORCE_GEMV, seed=10)
    _edge_q4(20, 128, 64, 32, 64, 64, flags=moe.FLAG_FORCE_GEMV, seed=11)
