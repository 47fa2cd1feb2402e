"""Each mutant is the oracle with one planted, plausible mistake; at least one pin
must reject it.  This shows the pins constrain every step of the oracle."""
import inspect
import types

import pytest

import oracle.moe_oracle as O
from oracle_pins import ALL_CHECKS

SRC = inspect.getsource(O)

# (name, original text, replacement)
MUTANTS = [
    ("tie_to_higher_index",
     'order = np.argsort(-L32, axis=1, kind="stable")',
     'order = (L32.shape[1] - 1) - np.argsort(-L32[:, ::-1], axis=1, kind="stable")'),
    ("ascending_selection", 'np.argsort(-L32, axis=1', 'np.argsort(L32, axis=1'),
    ("no_renormalisation", "return sel / sel.sum(axis=1, keepdims=True)", "return sel"),
    ("softmax_wrong_axis", "z / z.sum(axis=1, keepdims=True)", "z / z.sum(axis=0, keepdims=True)"),
    ("swiglu_orientation", "(silu(G) * U)", "(G * silu(U))"),
    ("silu_sign", "1.0 + np.exp(-z)", "1.0 + np.exp(z)"),
    ("no_shared_expert", "out[rows] = swiglu_ffn(x[rows], Sg, Su, Sd)", "out[rows] = 0.0"),
    ("descending_tokens_in_group",
     'perm = np.argsort(flat, kind="stable").astype(np.int64)',
     'perm = (flat.size - 1 - np.argsort(flat[::-1], kind="stable")).astype(np.int64)'),
    ("scan_off_by_one", "offsets[1:] = np.cumsum(counts)", "offsets[1:] = np.cumsum(counts) - counts"),
    ("combine_wrong_slot_weight", "out[t] += w[t, j] * y_perm[inv[t * k + j]]",
     "out[t] += w[t, k - 1 - j] * y_perm[inv[t * k + j]]"),
    ("combine_uniform_weight", "out[t] += w[t, j] * y_perm[inv[t * k + j]]",
     "out[t] += y_perm[inv[t * k + j]] / k"),
    ("down_not_transposed", "return (silu(G) * U) @ _f64(Wd).T", "return (silu(G) * U) @ _f64(Wd).reshape(-1, Wd.shape[0])"),
    ("bias_dropped", "L = L + _f64(bias)[None, :]", "L = L"),
    ("bias_subtracted", "L = L + _f64(bias)[None, :]", "L = L - _f64(bias)[None, :]"),
    ("wrong_expert_for_group", "Wg, Wu, Wd = get(e)\n", "Wg, Wu, Wd = get((e + 1) % E)\n"),
    ("gate_up_swapped_in_unpack",
     "return blk[:n].reshape(I, H), blk[n:2 * n].reshape(I, H), blk[2 * n:3 * n].reshape(H, I)",
     "return blk[n:2 * n].reshape(I, H), blk[:n].reshape(I, H), blk[2 * n:3 * n].reshape(H, I)"),
    ("weights_from_selected_only_wrong_index",
     "sel = np.take_along_axis(p, np.asarray(ids, dtype=np.int64), axis=1)",
     "sel = np.take_along_axis(p, np.sort(np.asarray(ids, dtype=np.int64), axis=1), axis=1)"),
    ("near_tie_wrong_direction", "((s[:, :-1] - s[:, 1:]) <= eps)", "((s[:, :-1] - s[:, 1:]) >= eps)"),
    ("token_row_gather_wrong", "tok = perm[pos] // k", "tok = perm[pos] % k"),
    ("q4_high_nibble_first", "q[0::2] = b & np.uint8(0x0F)\n    q[1::2] = b >> np.uint8(4)",
     "q[1::2] = b & np.uint8(0x0F)\n    q[0::2] = b >> np.uint8(4)"),
    ("q4_scale_bias_halves_swapped", "s = bf16_value(words)\n    b = bf16_value(words >> np.uint64(16))",
     "b = bf16_value(words)\n    s = bf16_value(words >> np.uint64(16))"),
    ("q4_group_of_32", "np.repeat(s, Q4_GROUP) + np.repeat(b, Q4_GROUP)",
     "np.repeat(np.repeat(s, 2)[:s.size], Q4_GROUP) + np.repeat(np.repeat(b, 2)[:b.size], Q4_GROUP)"),
    ("q4_bias_subtracted", "np.repeat(s, Q4_GROUP) + np.repeat(b, Q4_GROUP)",
     "np.repeat(s, Q4_GROUP) - np.repeat(b, Q4_GROUP)"),
    ("q4_signed_codes", "q = q4_codes(packed).astype(np.float64)",
     "q = q4_codes(packed).astype(np.int8).astype(np.float64) - 8.0 * (q4_codes(packed) > 7)"),
    ("q4_bf16_low_bits", "hi = (np.asarray(bits, dtype=np.uint64) & np.uint64(0xFFFF)).astype(np.uint32) << np.uint32(16)",
     "hi = (np.asarray(bits, dtype=np.uint64) & np.uint64(0xFFFF)).astype(np.uint32) << np.uint32(15)"),
    ("rel_err_per_column", "num = np.abs(y - ref).max(axis=1)", "num = np.abs(y - ref).max(axis=0)"),
    ("rel_err_mean_for_max", "num = np.abs(y - ref).max(axis=1)", "num = np.abs(y - ref).mean(axis=1)"),
    ("rel_err_no_abs_numerator", "num = np.abs(y - ref).max(axis=1)", "num = (y - ref).max(axis=1)"),
    ("rel_err_no_abs_denominator", "den = np.abs(ref).max(axis=1)", "den = ref.max(axis=1)"),
    ("rel_err_denominator_from_y", "den = np.abs(ref).max(axis=1)", "den = np.abs(y).max(axis=1)"),
    ("drop_last_group_row", "pos = np.arange(offsets[e], offsets[e + 1])", "pos = np.arange(offsets[e], max(offsets[e], offsets[e + 1] - 1))"),
]


def _mutant(orig, repl):
    assert SRC.count(orig) >= 1, f"mutation anchor not found: {orig!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(orig, repl), "<mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,orig,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, orig, repl):
    M = _mutant(orig, repl)
    caught = []
    for check in ALL_CHECKS:
        try:
            check(M)
        except Exception as e:  # AssertionError, or a crash on a shape mistake
            caught.append((check.__name__, type(e).__name__))
    assert caught, f"mutant {name} passed every pin"
