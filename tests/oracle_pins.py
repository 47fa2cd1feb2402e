"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``check_*`` takes the oracle module (or a deliberately broken copy of it)
and raises AssertionError when the oracle disagrees with: a closed form, a
brute-force evaluation on tiny inputs, a library routine (torch / scipy) with
a documented convention, an invariant, or a figure printed in the pages
(``tests/golden``).  ``test_oracle.py`` runs them on the real oracle and
``test_oracle_mutants.py`` runs them on mutants with one planted mistake each.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

from synth import inputs as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tiny_bf16():
    w = S.TINY
    x = S.bf16_bits_to_f32(S.x_rows(w, 0, w.M)).astype(np.float64)
    r = S.bf16_bits_to_f32(S.router_weight(w)).astype(np.float64)
    ex = S.bf16_bits_to_f32(S.all_expert_weights(w)).astype(np.float64)
    sh = S.bf16_bits_to_f32(S.shared_weight(w)).astype(np.float64)
    return w, x, r, ex, sh


def _torch_ffn(X, Wg, Wu, Wd):
    """SwiGLU FFN through torch's own layers (nn.Linear convention: weight [out, in])."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    X, Wg, Wu, Wd = map(t, (X, Wg, Wu, Wd))
    return F.linear(F.silu(F.linear(X, Wg)) * F.linear(X, Wu), Wd).numpy()


# ------------------------------------------------------------------ selection

def check_topk_bruteforce(O):
    """Top-k ids equal a pure-Python selection loop (max, ties -> lower index)."""
    rng = np.random.default_rng(1)
    for E, k in [(8, 3), (16, 2), (16, 16), (5, 1), (32, 8)]:
        # few distinct levels so exact ties are common
        L32 = rng.integers(-3, 4, size=(40, E)).astype(np.float32) * np.float32(0.25)
        ids = O.topk_ids(L32, k)
        for t in range(L32.shape[0]):
            left = list(range(E))
            want = []
            for _ in range(k):
                best = left[0]
                for e in left[1:]:
                    if L32[t, e] > L32[t, best]:
                        best = e
                want.append(best)
                left.remove(best)
            assert list(ids[t]) == want, (E, k, t, list(ids[t]), want)


def check_zero_router(O):
    """Wr = 0: every score ties, so ids = 0..k-1, w = 1/k, groups 0..k-1 hold all tokens."""
    M, H, E, k, I = 12, 64, 8, 3, 64
    rng = np.random.default_rng(2)
    x = rng.standard_normal((M, H))
    Wr = np.zeros((E, H))
    ex = rng.standard_normal((E, 3 * I * H)) * 0.02
    r = O.moe_forward(x, Wr, ex, None, k, I)
    assert (r["ids"] == np.arange(k)[None, :]).all()
    assert np.allclose(r["w"], 1.0 / k, rtol=0, atol=1e-15)
    want_counts = np.array([M] * k + [0] * (E - k))
    assert (r["counts"] == want_counts).all()
    for e in range(k):
        grp = r["perm"][r["offsets"][e]:r["offsets"][e + 1]]
        assert (grp == np.arange(M) * k + e).all()


def check_planted_router(O):
    """One-hot tokens and an integer router with a known ranking: ids and weights in closed form.

    Token t is the unit vector of column h = t mod H; Wr[e, h] = (7e + 3h) mod 16,
    a bijection e -> score for each h (7 is invertible mod 16 with inverse 7).
    So slot j holds e = 7 (15 - j - 3h) mod 16 with score 15 - j, and the
    renormalised weights are exp(-j) / sum_{i<k} exp(-i).
    """
    E, H, k, I = 16, 16, 4, 64
    M = 32
    x = np.zeros((M, H))
    x[np.arange(M), np.arange(M) % H] = 1.0
    Wr = np.array([[(7 * e + 3 * h) % 16 for h in range(H)] for e in range(E)], dtype=np.float64)
    rng = np.random.default_rng(3)
    ex = rng.standard_normal((E, 3 * I * H)) * 0.02
    r = O.moe_forward(x, Wr, ex, None, k, I)
    for t in range(M):
        h = t % H
        want = [(7 * (15 - j - 3 * h)) % 16 for j in range(k)]
        assert list(r["ids"][t]) == want, (t, list(r["ids"][t]), want)
    z = sum(math.exp(-i) for i in range(k))
    wj = np.array([math.exp(-j) / z for j in range(k)])
    assert np.allclose(r["w"], wj[None, :], rtol=1e-14, atol=0)
    assert not r["flagged"].any()


def check_router_bias(O):
    """A zero router plus a per-expert bias: the ranking is the bias's ranking and
    the weights are the softmax of the selected bias values (scipy)."""
    E, H, k, I, M = 10, 32, 3, 32, 6
    rng = np.random.default_rng(13)
    bias = np.array([0.5, -1.0, 2.0, 0.25, 1.5, -3.0, 0.0, 1.0, -0.5, 0.75], dtype=np.float32)
    x = rng.standard_normal((M, H))
    ex = rng.standard_normal((E, 3 * I * H)) * 0.02
    r = O.moe_forward(x, np.zeros((E, H)), ex, None, k, I, bias=bias)
    assert (r["ids"] == np.array([2, 4, 7])[None, :]).all()
    ref = scipy.special.softmax(bias[[2, 4, 7]].astype(np.float64))
    assert np.allclose(r["w"], ref[None, :], rtol=1e-14, atol=0)


def check_k_equals_E_is_softmax(O):
    """k = E: the renormalised weights are the full softmax (scipy), in rank order."""
    rng = np.random.default_rng(4)
    L = rng.standard_normal((20, 9)) * 2
    ids = O.topk_ids(O.selection_logits(L), 9)
    w = O.topk_weights(L, ids)
    ref = np.take_along_axis(scipy.special.softmax(L, axis=1), ids.astype(np.int64), axis=1)
    assert np.allclose(w, ref, rtol=1e-13, atol=0)
    assert (np.diff(np.take_along_axis(L, ids.astype(np.int64), 1), axis=1) <= 0).all()


def check_k1_weight_one(O):
    rng = np.random.default_rng(5)
    L = rng.standard_normal((30, 7))
    ids = O.topk_ids(O.selection_logits(L), 1)
    assert (ids[:, 0] == np.argmax(L, axis=1)).all()
    assert np.allclose(O.topk_weights(L, ids), 1.0, rtol=0, atol=1e-15)


def check_weights_closed_form(O):
    """w_j = exp(L_j - L_0) / sum_i exp(L_i - L_0) over the selected experts (softmax
    over the selected scores, equal to renormalised full-softmax probabilities),
    and sum_j w_j = 1."""
    rng = np.random.default_rng(6)
    L = rng.standard_normal((50, 32)) * 3
    k = 5
    ids = O.topk_ids(O.selection_logits(L), k)
    w = O.topk_weights(L, ids)
    sel = np.take_along_axis(L, ids.astype(np.int64), axis=1)
    ref = scipy.special.softmax(sel, axis=1)
    assert np.allclose(w, ref, rtol=1e-13, atol=0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=4e-16 * k)


def check_near_tie_rules(O):
    L = np.array([[3.0, 1.0, 1.0 + 5e-6, -2.0, 0.5],
                  [3.0, 1.0, 2.0, -2.0, 0.5]])
    L32 = O.selection_logits(L)
    fl = O.near_tie_flags(L32, 2)
    assert fl[0] and not fl[1]
    # token 0: picking expert 1 or 2 in slot 1 are both acceptable; expert 4 is not
    assert O.valid_topk(L32[:1], [[0, 2]])[0]
    assert O.valid_topk(L32[:1], [[0, 1]])[0]
    assert not O.valid_topk(L32[:1], [[0, 4]])[0]
    assert not O.valid_topk(L32[1:], [[0, 1]])[0]
    assert not O.valid_topk(L32[1:], [[2, 0]])[0]


# ------------------------------------------------------------------ routing tables

def check_route_invariants(O):
    """Histogram / scan / scatter invariants on a random routing."""
    rng = np.random.default_rng(7)
    M, E, k = 300, 24, 4
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(M)]).astype(np.int32)
    counts, offsets, perm, inv = O.route_tables(ids, E)
    assert counts.sum() == M * k
    assert (counts == np.array([(ids == e).sum() for e in range(E)])).all()
    assert offsets[0] == 0 and offsets[E] == M * k
    assert (offsets[1:] == np.cumsum(counts)).all()
    assert sorted(perm.tolist()) == list(range(M * k))
    assert (inv[perm] == np.arange(M * k)).all()
    for e in range(E):
        grp = perm[offsets[e]:offsets[e + 1]]
        assert (ids.ravel()[grp] == e).all()
        assert (np.diff(grp // k) > 0).all()  # ascending tokens, each at most once
    per_token = np.bincount(perm // k, minlength=M)
    assert (per_token == k).all()


def check_pages_assignment_arithmetic(O):
    """The pages' worked figure: 2K tokens routed to 8 of 256 experts give
    16,384 assignments, 64 rows per expert on average (tests/golden)."""
    g = _golden("p1_routing_arithmetic.json")
    M, E, k = g["tokens"], g["experts"], g["top_k"]
    rng = np.random.default_rng(8)
    H = 32
    x = rng.standard_normal((M, H))
    Wr = rng.standard_normal((E, H))
    L = O.router_logits(x, Wr)
    ids = O.topk_ids(O.selection_logits(L), k)
    counts, offsets, perm, inv = O.route_tables(ids, E)
    assert int(counts.sum()) == g["assignments"]
    assert int(offsets[E]) == g["assignments"]
    assert counts.mean() == g["mean_rows_per_expert"]
    assert counts.std() > 0  # uneven groups


# ------------------------------------------------------------------ expert FFN and layer

def check_ffn_matches_torch(O):
    """The expert FFN equals torch's Linear/SiLU composition (weights [out, in])."""
    rng = np.random.default_rng(9)
    H, I = 48, 32
    X = rng.standard_normal((10, H))
    Wg, Wu = rng.standard_normal((I, H)) * 0.3, rng.standard_normal((I, H)) * 0.3
    Wd = rng.standard_normal((H, I)) * 0.3
    assert np.allclose(O.swiglu_ffn(X, Wg, Wu, Wd), _torch_ffn(X, Wg, Wu, Wd), rtol=1e-12, atol=1e-12)
    z = np.array([0.0, -50.0, 50.0, 1.5, -0.3])
    assert np.allclose(O.silu(z), F.silu(torch.from_numpy(z)).numpy(), rtol=1e-15, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0


def check_single_expert_layer(O):
    """E = 1, k = 1: the layer is two dense SwiGLU FFNs added (routed + shared), via torch."""
    rng = np.random.default_rng(10)
    M, H, I = 9, 64, 64
    x = rng.standard_normal((M, H))
    Wr = rng.standard_normal((1, H))
    blk = rng.standard_normal((1, 3 * I * H)) * 0.1
    sh = rng.standard_normal(3 * I * H) * 0.1
    r = O.moe_forward(x, Wr, blk, sh, 1, I)
    n = I * H
    ref = _torch_ffn(x, blk[0, :n].reshape(I, H), blk[0, n:2 * n].reshape(I, H), blk[0, 2 * n:].reshape(H, I))
    ref = ref + _torch_ffn(x, sh[:n].reshape(I, H), sh[n:2 * n].reshape(I, H), sh[2 * n:].reshape(H, I))
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


def check_identical_experts(O):
    """All routed experts equal F: out = S(x) + F(x) whatever the routing (weights sum to 1)."""
    rng = np.random.default_rng(11)
    M, H, E, k, I = 20, 64, 12, 3, 32
    x = rng.standard_normal((M, H))
    Wr = rng.standard_normal((E, H))
    one = rng.standard_normal(3 * I * H) * 0.1
    sh = rng.standard_normal(3 * I * H) * 0.1
    ex = np.tile(one, (E, 1))
    r = O.moe_forward(x, Wr, ex, sh, k, I)
    n = I * H
    ref = _torch_ffn(x, one[:n].reshape(I, H), one[n:2 * n].reshape(I, H), one[2 * n:].reshape(H, I))
    ref = ref + _torch_ffn(x, sh[:n].reshape(I, H), sh[n:2 * n].reshape(I, H), sh[2 * n:].reshape(H, I))
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


def check_planted_combine(O):
    """Experts that output known constants: out = sum_j w_j * c_{ids[t,j]} exactly.

    Expert e has gate/up weights that make SiLU(g)*u a fixed nonzero vector
    independent of x (x has a constant-1 column) and a down projection that
    maps it to c_e * ones; the planted router fixes ids and weights.
    """
    E, H, k, I = 16, 16, 3, 4
    M = 16
    x = np.zeros((M, H))
    x[np.arange(M), np.arange(M) % (H - 1)] = 1.0
    x[:, H - 1] = 1.0  # constant feature
    Wr = np.array([[(7 * e + 3 * h) % 16 if h < H - 1 else 0 for h in range(H)] for e in range(E)], dtype=np.float64)
    ex = np.zeros((E, 3 * I * H))
    n = I * H
    c = np.arange(1, E + 1, dtype=np.float64) * 10.0
    for e in range(E):
        g = np.zeros((I, H)); g[:, H - 1] = 1.0   # gate = 1
        u = np.zeros((I, H)); u[:, H - 1] = 1.0   # up = 1
        d = np.zeros((H, I)); d[:, 0] = c[e] * (1.0 + math.exp(-1.0))  # 1 / silu(1)
        ex[e, :n], ex[e, n:2 * n], ex[e, 2 * n:] = g.ravel(), u.ravel(), d.ravel()
    r = O.moe_forward(x, Wr, ex, None, k, I)
    z = sum(math.exp(-i) for i in range(k))
    for t in range(M):
        h = t % (H - 1)
        ids = [(7 * (15 - j - 3 * h)) % 16 for j in range(k)]
        want = sum(math.exp(-j) / z * c[ids[j]] for j in range(k))
        assert np.allclose(r["out"][t], want, rtol=1e-12, atol=0), (t, r["out"][t, 0], want)


def check_dense_equals_grouped(O):
    """Grouped (permute/compute/combine) equals brute force dense-then-masked on the tiny workload."""
    w, x, r, ex, sh = _tiny_bf16()
    a = O.moe_forward(x, r, ex, sh, w.k, w.I)["out"]
    b = O.dense_forward(x, r, ex, sh, w.k, w.I)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)
    xf, rf, exf, shf = S.tiny_f32()
    a = O.moe_forward(xf, rf, exf, shf, w.k, w.I)["out"]
    b = O.dense_forward(xf, rf, exf, shf, w.k, w.I)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


def check_token_permutation(O):
    """Permuting tokens permutes outputs and selections (the layer is per token)."""
    w, x, r, ex, sh = _tiny_bf16()
    rng = np.random.default_rng(12)
    p = rng.permutation(w.M)
    a = O.moe_forward(x, r, ex, sh, w.k, w.I)
    b = O.moe_forward(x[p], r, ex, sh, w.k, w.I)
    assert (b["ids"] == a["ids"][p]).all()
    assert np.allclose(b["out"], a["out"][p], rtol=1e-13, atol=1e-14)


def check_chunk_invariance(O):
    """Splitting the tokens into chunks does not change any token's output."""
    w, x, r, ex, sh = _tiny_bf16()
    a = O.moe_forward(x, r, ex, sh, w.k, w.I)["out"]
    h = w.M // 2 + 5
    b1 = O.moe_forward(x[:h], r, ex, sh, w.k, w.I)["out"]
    b2 = O.moe_forward(x[h:], r, ex, sh, w.k, w.I)["out"]
    assert np.allclose(np.vstack([b1, b2]), a, rtol=1e-13, atol=1e-14)


def check_down_linearity(O):
    """Doubling every down projection doubles the output exactly (power-of-two scaling)."""
    w, x, r, ex, sh = _tiny_bf16()
    n = w.I * w.H
    ex2 = ex.copy(); ex2[:, 2 * n:] *= 2.0
    sh2 = sh.copy(); sh2[2 * n:] *= 2.0
    a = O.moe_forward(x, r, ex, sh, w.k, w.I)["out"]
    b = O.moe_forward(x, r, ex2, sh2, w.k, w.I)["out"]
    assert (b == 2.0 * a).all()


def check_subset_tokens(O):
    """Computing only some tokens' outputs gives the same rows as the full evaluation."""
    w, x, r, ex, sh = _tiny_bf16()
    a = O.moe_forward(x, r, ex, sh, w.k, w.I)
    sel = [0, 5, 17, 63]
    b = O.moe_forward(x, r, ex, sh, w.k, w.I, tokens=sel)
    assert np.allclose(b["out"][sel], a["out"][sel], rtol=1e-13, atol=1e-14)
    assert np.isnan(b["out"][1]).all()
    assert (b["perm"] == a["perm"]).all()


def check_forced_routing(O):
    """Forced selections recompute weights/groups/outputs for that selection."""
    w, x, r, ex, sh = _tiny_bf16()
    a = O.moe_forward(x, r, ex, sh, w.k, w.I)
    ids = a["ids"].copy()
    ids[:, [0, 1]] = ids[:, [1, 0]]  # swap slots: same set, other order
    b = O.moe_forward(x, r, ex, sh, w.k, w.I, force_ids=ids)
    assert np.allclose(b["out"], a["out"], rtol=1e-13, atol=1e-14)
    assert np.allclose(b["w"][:, [1, 0]], a["w"][:, [0, 1]], rtol=1e-14, atol=0)


# ------------------------------------------------------------------ 4-bit weights

def _bf16_bits(v):
    """bf16 bit pattern of an exactly representable value."""
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0] >> 16)


def check_q4_hand_example(O):
    """Hand-decoded group: bytes 0x21, 0xF0 hold codes 1, 2, 0, 15 (low nibble first);
    scale 0.5 and bias -1 give 1*0.5-1, 2*0.5-1, -1, 15*0.5-1; the rest (code 0) -1."""
    codes = np.zeros(32, np.uint8)
    codes[0], codes[1] = 0x21, 0xF0
    word = _bf16_bits(0.5) | (_bf16_bits(-1.0) << 16)
    w = O.dequant_q4(codes, np.array([word], np.uint32))
    want = np.full(64, -1.0)
    want[:4] = [-0.5, 0.0, -1.0, 6.5]
    assert w.shape == (64,) and np.array_equal(w, want), w[:6]


def check_q4_groups_and_affinity(O):
    """Each 64-value group uses its own (scale, bias); within a group the
    values are exactly affine in the code: w(q) - w(0) = q * s."""
    rng = np.random.default_rng(7)
    ngroups = 5
    scales = [0.25, -0.125, 2.0, 0.0078125, 1.5]
    biases = [1.0, -3.0, 0.5, -0.0625, 0.0]
    words = np.array([_bf16_bits(a) | (_bf16_bits(b) << 16) for a, b in zip(scales, biases)], np.uint32)
    q = rng.integers(0, 16, size=64 * ngroups).astype(np.uint8)
    packed = (q[0::2] | (q[1::2] << 4)).astype(np.uint8)
    w = O.dequant_q4(packed, words)
    for g in range(ngroups):
        seg = slice(64 * g, 64 * (g + 1))
        assert np.array_equal(w[seg], q[seg] * scales[g] + biases[g]), g


def check_q4_bf16_decoding(O):
    """bf16 patterns decode to their values (sign, exponent, zero, subnormal)."""
    pats = {0x3F80: 1.0, 0xC000: -2.0, 0x0000: 0.0, 0x8000: -0.0, 0x3E80: 0.25, 0x4120: 10.0,
            0x0001: 2.0 ** -133, 0x7F7F: float(np.finfo(np.float32).max) // 2 ** 104 * 2 ** 104}
    for bits, v in pats.items():
        got = O.bf16_value(np.array([bits], np.uint32))[0]
        if bits == 0x7F7F:
            assert got == float(np.uint32(0x7F7F0000).view(np.float32)), got
        else:
            assert got == v and np.signbit(got) == np.signbit(v), (hex(bits), got)


def check_q4_layer_is_dense_on_dequantised(O):
    """The layer on 4-bit experts equals, for E = 1 and k = 1, two dense SwiGLU
    FFNs (torch) on weights rebuilt by hand from the codes."""
    rng = np.random.default_rng(8)
    H, I, M = 64, 64, 5
    n = 3 * I * H
    q = rng.integers(0, 16, size=n).astype(np.uint8)
    packed = (q[0::2] | (q[1::2] << 4)).astype(np.uint8)
    s = rng.choice([2.0 ** -7, 2.0 ** -6, 3 * 2.0 ** -8], size=n // 64)
    b = -8 * s
    words = np.array([_bf16_bits(a) | (_bf16_bits(c) << 16) for a, c in zip(s, b)], np.uint32)
    wts = (q.astype(np.float64) - 8.0) * np.repeat(s, 64)  # by hand: s * q + (-8 s)
    x = rng.standard_normal((M, H))
    router = np.zeros((1, H))
    got = O.moe_forward(x, router, lambda e: O.unpack_expert(O.dequant_q4(packed, words), I, H),
                        O.dequant_q4(packed, words), 1, I)["out"]
    Wg, Wu, Wd = wts[:I * H].reshape(I, H), wts[I * H:2 * I * H].reshape(I, H), wts[2 * I * H:].reshape(H, I)
    want = 2 * _torch_ffn(x, Wg, Wu, Wd)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ the parity metric

def check_rel_err_per_token(O):
    """The per-token error metric used by every output comparison, on values computed by hand:
    max over a row of |y - ref| divided by max over the same row of |ref|.

    Row 0 is negative-dominant: its largest |ref| is 10 at a negative entry, while its
    largest ref is 4; |y - ref| = (0.5, 1, 3), so the value is 3 / 10.  Row 1:
    |y - ref| = (0, 0.25, 0) over max |ref| = 1.  Row 2 is all zeros on both sides and
    must give 0, not NaN.  A per-column reduction, a mean for the max, a dropped absolute
    value or the denominator taken from y each change one of these numbers (or the shape).
    """
    ref = np.array([[2.0, -10.0, 4.0], [1.0, 0.5, -0.25], [0.0, 0.0, 0.0]])
    y = np.array([[2.5, -9.0, 1.0], [1.0, 0.25, -0.25], [0.0, 0.0, 0.0]])
    got = O.rel_err_per_token(y, ref)
    assert got.shape == (3,), got.shape
    assert got[0] == 3.0 / 10.0 and got[1] == 0.25 and got[2] == 0.0, got
    # invariant: scaling both sides by a power of two leaves every row's value unchanged
    assert np.array_equal(O.rel_err_per_token(8.0 * y, 8.0 * ref), got)


ALL_CHECKS = [
    check_topk_bruteforce, check_zero_router, check_planted_router, check_router_bias,
    check_k_equals_E_is_softmax, check_k1_weight_one, check_weights_closed_form,
    check_near_tie_rules, check_route_invariants, check_pages_assignment_arithmetic,
    check_ffn_matches_torch, check_single_expert_layer, check_identical_experts,
    check_planted_combine, check_dense_equals_grouped, check_token_permutation,
    check_chunk_invariance, check_down_linearity, check_subset_tokens, check_forced_routing,
    check_q4_hand_example, check_q4_groups_and_affinity, check_q4_bf16_decoding,
    check_q4_layer_is_dense_on_dequantised, check_rel_err_per_token,
]
