"""CPU oracle of the sparse mixture-of-experts FFN layer.

TEST INFRASTRUCTURE ONLY.  This module is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``,
and by nothing else.  The GPU library never imports, links or calls it, and
it shares no code with the GPU library: it depends on NumPy alone.

What it computes is the plain layer, step by step, in the order the sources
give, in float64 (NumPy; matrix products go to BLAS dgemm):

1. router logits, one score per routed expert ........ ``router_logits``
2. softmax over all experts, the top k by score, the
   k selected probabilities renormalised to sum 1 .... ``topk_ids``, ``topk_weights``
3. histogram of assignments per expert, exclusive
   prefix scan to group offsets, scatter of the
   assignments into expert groups .................... ``route_tables``
4. per group: two input projections, gated (SiLU)
   activation, output projection ..................... ``swiglu_ffn``
5. the always-on shared expert on every token ........ ``swiglu_ffn``
6. weighted combine of the k expert outputs plus the
   shared expert's output ............................ ``moe_forward``
7. (4-bit experts) weights rebuilt from 4-bit codes
   and a scale and bias per group of 64 .............. ``dequant_q4``

Sources (page title, then section):
- "Optimizing on-device inference for Apple Silicon" (Perplexity, 2026),
  section "Qwen creates three distinct workload shapes": the router scores
  256 experts, picks 8, and one shared expert serves every token.
- same page, "Keep expert routing on the GPU": histogram -> prefix scan ->
  scatter into expert groups -> block map for the grouped GEMM.
- same page, "Match tile size to expert load": 2K tokens x 8 of 256 experts
  = 16,384 assignments, 64 rows per expert on average.
- same page, "Reduce intermediate and state traffic": the two input
  projections go with their gated activation; the output projection goes
  with its routing score and the shared expert's result.
- same page, "Dequantize weights during matrix multiplication": fp32
  accumulation, bf16 output (the GPU kernels' precision; the oracle is fp64);
  each weight a 4-bit integer code, each group of 64 weights sharing one
  bf16 scale and one bf16 bias from which its values are rebuilt.

The pages give the structure but no formulas; where they are silent the
reading used is stated at the function (softmax scoring, renormalisation,
tie-break, SiLU(gate)*up, unit-weight shared expert, no capacity limit).

Precision and decisions: all arithmetic is float64.  The top-k selection is
an integer decision taken from floating point; it is taken, as in the GPU
kernel, on fp32 logits: the float64 logit rounded once to fp32.  Tokens whose
fp32 logits have an adjacent gap <= 1e-5 among ranks 0..k are flagged as
near-ties (``near_tie_flags``); there either choice is correct and
``valid_topk`` decides whether a given choice is one.
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence, Union

import numpy as np

NEAR_TIE_EPS = 1e-5

ExpertSource = Union[np.ndarray, Callable[[int], tuple]]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- 1. router

def router_logits(x, router_w, bias=None) -> np.ndarray:
    """Router scores L[t, e] = x[t] . Wr[e] (+ bias[e]), float64 [M, E].

    Follows "Qwen creates three distinct workload shapes" (the router scores
    every routed expert for every token).  Scores are a linear map of the
    token row; the optional per-expert bias is added to the score.
    """
    L = _f64(x) @ _f64(router_w).T
    if bias is not None:
        L = L + _f64(bias)[None, :]
    return L


def selection_logits(L) -> np.ndarray:
    """The fp32 values the top-k decision is taken on (one rounding of the fp64 logit)."""
    return np.asarray(L, dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------- 2. top-k

def topk_ids(L32, k: int) -> np.ndarray:
    """The k experts with the largest scores, int32 [M, k], slot j = rank j.

    Follows "Qwen creates three distinct workload shapes" (8 of 256 chosen).
    Reading: experts are ranked by descending score; equal scores rank the
    lower expert index first (a stable sort on the negated score).
    """
    L32 = np.asarray(L32)
    order = np.argsort(-L32, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def softmax(L) -> np.ndarray:
    """Row-wise softmax over all experts, max-subtracted, float64."""
    L = _f64(L)
    z = np.exp(L - L.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def topk_weights(L, ids) -> np.ndarray:
    """Routing weights w[t, j] = p[t, ids[t, j]] / sum_j' p[t, ids[t, j']], float64.

    p = softmax of the scores over all experts; the k selected probabilities
    are renormalised to sum to 1 (reading: the pages name no normalisation;
    this is the usual one for top-k routing with a softmax router).
    """
    p = softmax(L)
    sel = np.take_along_axis(p, np.asarray(ids, dtype=np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def near_tie_flags(L32, k: int, eps: float = NEAR_TIE_EPS) -> np.ndarray:
    """True for tokens whose sorted fp32 scores have a gap <= eps among ranks 0..k.

    Such a token's selection (or slot order) can legitimately differ between
    two correct fp32 evaluations that sum in different orders.
    """
    s = -np.sort(-np.asarray(L32, dtype=np.float64), axis=1)
    s = s[:, :min(k + 1, s.shape[1])]
    if s.shape[1] < 2:
        return np.zeros(s.shape[0], dtype=bool)
    return ((s[:, :-1] - s[:, 1:]) <= eps).any(axis=1)


def valid_topk(L32, ids, eps: float = NEAR_TIE_EPS) -> np.ndarray:
    """Per token: is ``ids`` a correct top-k (distinct, slot order and selection
    consistent with the fp32 scores up to eps)?  bool [M]."""
    L32 = np.asarray(L32, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    M, E = L32.shape
    k = ids.shape[1]
    ok = np.ones(M, dtype=bool)
    for t in range(M):
        row = ids[t]
        if row.min() < 0 or row.max() >= E or len(set(row.tolist())) != k:
            ok[t] = False
            continue
        v = L32[t, row]
        if np.any(v[:-1] < v[1:] - eps):
            ok[t] = False
            continue
        rest = np.ones(E, dtype=bool)
        rest[row] = False
        if rest.any() and L32[t, rest].max() > v.min() + eps:
            ok[t] = False
    return ok


# ---------------------------------------------------------------- 3. routing tables

def route_tables(ids, E: int):
    """Histogram, exclusive prefix scan and scatter of the assignments.

    Follows "Keep expert routing on the GPU": the histogram counts the
    assignments that went to each expert, the prefix scan turns the counts
    into start offsets, and the scatter places each assignment in its
    expert's group.  Assignment (t, j) has flat index a = t*k + j.

    Returns counts [E], offsets [E+1] (offsets[E] = M*k), perm [M*k] with
    perm[p] = the assignment stored at group position p, and inv [M*k] with
    inv[a] = p.  Reading: inside a group, assignments are in ascending token
    order (the pages leave the order open; a stable sort by expert gives it).
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int64)
    return counts, offsets, perm, inv


# ---------------------------------------------------------------- 4/5. expert FFN

def silu(z) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)), float64."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(X, Wg, Wu, Wd) -> np.ndarray:
    """One expert on a block of token rows: (SiLU(X Wg^T) * (X Wu^T)) Wd^T.

    Follows "Reduce intermediate and state traffic" (two input projections
    with their gated activation, then the output projection).  Reading: the
    gate projection goes through SiLU and multiplies the up projection.
    Layouts: Wg, Wu are [I, H], Wd is [H, I] (row = output feature).
    """
    X = _f64(X)
    G = X @ _f64(Wg).T
    U = X @ _f64(Wu).T
    return (silu(G) * U) @ _f64(Wd).T


def unpack_expert(blk, I: int, H: int):
    """(gate [I,H], up [I,H], down [H,I]) from a packed expert block of 3*I*H values."""
    blk = np.asarray(blk).ravel()
    n = I * H
    return blk[:n].reshape(I, H), blk[n:2 * n].reshape(I, H), blk[2 * n:3 * n].reshape(H, I)


def _expert_getter(experts: ExpertSource, I: int, H: int):
    if callable(experts):
        return experts
    arr = np.asarray(experts)
    return lambda e: unpack_expert(arr[e], I, H)


# ---------------------------------------------------------------- 6. the layer

def moe_forward(x, router_w, experts: ExpertSource, shared, k: int, I: int,
                bias=None, force_ids=None, tokens: Optional[Sequence[int]] = None,
                I_shared: Optional[int] = None) -> dict:
    """The whole layer.  out[t] = S(x_t) + sum_j w[t,j] * F_{ids[t,j]}(x_t).

    Follows "Reduce intermediate and state traffic" (the output projection is
    combined with its routing score and with the shared expert's result) and
    "Qwen creates three distinct workload shapes" (one shared expert on every
    token).  Reading: the shared expert's output is added with weight 1; no
    capacity limit, no token is dropped.

    experts: array [E, 3*I*H] of packed blocks, or a callable e -> (Wg, Wu, Wd).
    shared:  packed block [3*I_shared*H], or (Wg, Wu, Wd), or None.
    force_ids: take the selection from here instead of the scores (steps
             2-6 are then recomputed for that selection).
    tokens:  compute outputs only for these token rows (routing tables are
             always for all tokens); other rows of ``out`` are NaN.
    """
    x = _f64(x)
    M, H = x.shape
    E = np.asarray(router_w).shape[0]
    get = _expert_getter(experts, I, H)

    L = router_logits(x, router_w, bias)
    L32 = selection_logits(L)
    ids = topk_ids(L32, k) if force_ids is None else np.asarray(force_ids, dtype=np.int32)
    w = topk_weights(L, ids)
    counts, offsets, perm, inv = route_tables(ids, E)

    want = np.ones(M, dtype=bool) if tokens is None else np.isin(np.arange(M), np.asarray(tokens))
    y_perm = np.full((M * k, H), np.nan)
    for e in range(E):
        pos = np.arange(offsets[e], offsets[e + 1])
        if pos.size == 0:
            continue
        tok = perm[pos] // k
        keep = want[tok]
        if not keep.any():
            continue
        Wg, Wu, Wd = get(e)
        y_perm[pos[keep]] = swiglu_ffn(x[tok[keep]], Wg, Wu, Wd)

    out = np.full((M, H), np.nan)
    rows = np.nonzero(want)[0]
    if shared is not None:
        if isinstance(shared, tuple):
            Sg, Su, Sd = shared
        else:
            Is = I if I_shared is None else I_shared
            Sg, Su, Sd = unpack_expert(shared, Is, H)
        out[rows] = swiglu_ffn(x[rows], Sg, Su, Sd)
    else:
        out[rows] = 0.0
    for t in rows:
        for j in range(k):
            out[t] += w[t, j] * y_perm[inv[t * k + j]]

    return dict(out=out, logits=L, logits32=L32, ids=ids, w=w, counts=counts,
                offsets=offsets, perm=perm, inv=inv,
                flagged=near_tie_flags(L32, k))


def dense_forward(x, router_w, experts: ExpertSource, shared, k: int, I: int,
                  bias=None, I_shared: Optional[int] = None) -> np.ndarray:
    """Brute force: every expert on every token, then masked by the routing weights.

    out = S(x) + sum_e Gm[:, e] * F_e(x), Gm[t, e] = w[t, j] if e = ids[t, j]
    else 0.  No permutation, no groups: a cross-check of the grouped
    evaluation in ``moe_forward``.
    """
    x = _f64(x)
    M, H = x.shape
    E = np.asarray(router_w).shape[0]
    get = _expert_getter(experts, I, H)
    L = router_logits(x, router_w, bias)
    ids = topk_ids(selection_logits(L), k)
    w = topk_weights(L, ids)
    Gm = np.zeros((M, E))
    np.put_along_axis(Gm, ids.astype(np.int64), w, axis=1)
    if shared is None:
        out = np.zeros((M, H))
    else:
        Is = I if I_shared is None else I_shared
        Sg, Su, Sd = shared if isinstance(shared, tuple) else unpack_expert(shared, Is, H)
        out = swiglu_ffn(x, Sg, Su, Sd)
    for e in range(E):
        out = out + Gm[:, e:e + 1] * swiglu_ffn(x, *get(e))
    return out


# ---------------------------------------------------- 7. 4-bit group-affine weights
#
# "Dequantize weights during matrix multiplication": every weight is stored
# as a 4-bit integer code and every group of 64 weights shares a bf16 scale
# and a bf16 bias used to rebuild the weights.  Reading: the rebuilt weight
# is the affine value w = s * q + b with q the unsigned code 0..15, groups of
# 64 consecutive weights along a row's reduction dimension, and no further
# rounding (the GPU matrix kernels round w to bf16 for their operands, as
# they take x in bf16).  Storage (this library's layout): two codes per byte,
# low nibble first; one 32-bit word per group, scale in the low 16 bits,
# bias in the high 16 bits.

Q4_GROUP = 64


def bf16_value(bits) -> np.ndarray:
    """Values of bfloat16 bit patterns (the high half of an IEEE binary32), float64."""
    hi = (np.asarray(bits, dtype=np.uint64) & np.uint64(0xFFFF)).astype(np.uint32) << np.uint32(16)
    return hi.view(np.float32).astype(np.float64)


def q4_codes(packed) -> np.ndarray:
    """Unsigned 4-bit codes, two per byte, low nibble first (uint8, length 2 * bytes)."""
    b = np.asarray(packed, dtype=np.uint8).ravel()
    q = np.empty(2 * b.size, dtype=np.uint8)
    q[0::2] = b & np.uint8(0x0F)
    q[1::2] = b >> np.uint8(4)
    return q


def dequant_q4(packed, scale_bias) -> np.ndarray:
    """Weights of a 4-bit block, float64: w[i] = s[g] * q[i] + b[g] with g = i // 64.

    packed: the codes (bytes); scale_bias: one uint32 word per group of 64.
    Applied to a packed expert block (gate [I][H], up [I][H], down [H][I],
    rows of a multiple of 64 values) it gives the packed fp64 expert block.
    """
    q = q4_codes(packed).astype(np.float64)
    words = np.asarray(scale_bias, dtype=np.uint64).ravel()
    if q.size != words.size * Q4_GROUP:
        raise ValueError("4-bit block: codes and scale/bias groups do not match")
    s = bf16_value(words)
    b = bf16_value(words >> np.uint64(16))
    return q * np.repeat(s, Q4_GROUP) + np.repeat(b, Q4_GROUP)


def rel_err_per_token(y, ref) -> np.ndarray:
    """max_c |y[t,c] - ref[t,c]| / max_c |ref[t,c]| for each token row t.

    The comparison every output check uses.  Reading: the bound on the
    layer's outputs is a maximum relative error without a stated norm; it is
    taken per token in the max norm (an elementwise relative error is
    ill-posed at outputs near zero).  A row whose reference is all zero
    divides by the smallest normal double, so equal zero rows give 0.
    """
    y = _f64(y)
    ref = _f64(ref)
    num = np.abs(y - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    return num / np.maximum(den, np.finfo(np.float64).tiny)
