"""The seeded input generator (host side): published SplitMix64 outputs, bf16
rounding against torch's own conversion, slicing consistency, moments."""
import math

import numpy as np
import torch

from synth import inputs as S


def test_splitmix64_published_outputs():
    # First outputs of SplitMix64 seeded with 0 (Steele, Lea & Flood 2014;
    # the values every reference implementation reproduces).
    got = [int(v) for v in S.splitmix64_outputs(0, 1, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    assert S.mix64_int(0x9E3779B97F4A7C15) == 0xE220A8397B1DCDAF


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = (rng.standard_normal(200_000) * np.exp(rng.uniform(-20, 20, 200_000))).astype(np.float32)
    # exact halfway cases: ties go to even
    one = np.float32(1.0)
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130 * 3], dtype=np.float32)
    a = np.concatenate([a, ties, [one, -one, np.float32(0.0), np.float32(-0.0)]])
    ours = S.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(S.bf16_bits_to_f32(ours), torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_slices_are_consistent():
    key = S.stream_key(5, 1, 2, 3)
    full = S.normal_f32(key, 0, 1000, 0.02)
    assert np.array_equal(S.normal_f32(key, 300, 200, 0.02), full[300:500])
    assert np.array_equal(S.x_rows(S.TINY, 10, 5), S.x_rows(S.TINY, 0, 20)[10:15])


def test_moments_and_bounds():
    v = S.normal_f32(S.stream_key(1, 0, 0, 0), 0, 2_000_000, 1.0).astype(np.float64)
    assert abs(v.mean()) < 3e-3
    assert abs(v.std() - 1.0) < 3e-3
    kurt = ((v - v.mean()) ** 4).mean() / v.var() ** 2
    assert abs(kurt - (3 - 1.2 / 8)) < 0.02  # Irwin-Hall(8)
    assert np.abs(v).max() <= S.IH_MEAN / S.IH_STD + 1e-6


def test_keys_distinct():
    keys = {S.stream_key(s, l, t, e) for s in range(3) for l in range(3) for t in range(5) for e in range(20)}
    assert len(keys) == 3 * 3 * 5 * 20


def test_zipf_bias():
    b = S.zipf_router_bias(S.SKEW).astype(np.float64)
    ranks = np.rint(np.exp(-b / 1.2)).astype(int)
    assert sorted(ranks.tolist()) == list(range(1, 257))
    assert np.allclose(b, -1.2 * np.log(ranks), rtol=0, atol=1e-6)
    assert S.zipf_router_bias(S.PREFILL) is None


def test_workload_shapes():
    assert S.PREFILL.M * S.PREFILL.k == 32768
    assert S.LONG.tokens == 131072
    assert S.DECODE.layers * S.DECODE.E * S.DECODE.expert_elems() * 2 > 64e9


def test_q4_generator():
    """4-bit experts: code bytes are the stream's outputs, scale/bias words
    follow their recipe exactly, and the rebuilt weights have mean ~0 and
    standard deviation ~sigma."""
    key = S.stream_key(3, 0, S.T_Q4_CODES, 1)
    b = S.q4_codes(key, 40)
    assert np.array_equal(b[:16], S.splitmix64_outputs(key, 1, 2).view(np.uint8))
    assert np.array_equal(S.q4_codes(key, 64)[:40], b)
    sb = S.q4_scale_bias(S.stream_key(3, 0, S.T_Q4_SB, 1), 4096, 0.02)
    s = S.bf16_bits_to_f32((sb & 0xFFFF).astype(np.uint16)).astype(np.float64)
    off = S.bf16_bits_to_f32((sb >> 16).astype(np.uint16)).astype(np.float64)
    s0 = 0.02 / S.Q4_STD
    assert np.all(s >= 0.49 * s0) and np.all(s <= 1.51 * s0)
    assert np.all(-off / s >= 6.9) and np.all(-off / s <= 8.1)
    codes, words = S.q4_expert(S.TINY, 0, 3)
    q = np.empty(2 * codes.size)
    q[0::2], q[1::2] = codes & 15, codes >> 4
    sv = S.bf16_bits_to_f32((words & 0xFFFF).astype(np.uint16)).astype(np.float64)
    bv = S.bf16_bits_to_f32((words >> 16).astype(np.uint16)).astype(np.float64)
    wts = q * np.repeat(sv, S.Q4_GROUP) + np.repeat(bv, S.Q4_GROUP)
    assert codes.size * 2 == S.TINY.expert_elems() and words.size * 64 == S.TINY.expert_elems()
    assert abs(wts.mean()) < 0.1 * S.TINY.w_sigma
    assert abs(wts.std() / S.TINY.w_sigma - 1) < 0.1


def test_host_c_twin_matches_numpy():
    """The C twin of the generator (used when built) gives the NumPy definition's bits."""
    if S._host_lib() is None:
        import pytest
        pytest.skip("synth/libsynth_host.so not built")
    for key, start, n, sigma in [(S.stream_key(1, 2, 3, 4), 0, 100_003, 0.02), (12345, 777, 4096, 1.0),
                                 (S.x_key(S.PREFILL), 4095 * 2048, 2048, 1.0), (2 ** 64 - 1, 2 ** 40, 999, 0.5)]:
        assert np.array_equal(S.normal_bf16(key, start, n, sigma), S.normal_bf16_np(key, start, n, sigma))
