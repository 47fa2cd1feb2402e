"""Seeded synthetic inputs for the sparse MoE FFN layer.

This module is shared by the CPU oracle and the GPU path.  It holds none of
the layer's arithmetic: it only draws tensors of the shapes and value
distributions of the workloads, bit-exactly identical on the host (NumPy,
here) and on the device (``synth/csrc/synth_fill.hip``).

Generator
---------
Counter-based SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; the 64-bit finaliser is Stafford's "Mix13").
A stream is a 64-bit key ``s``; its n-th output (n >= 1) is
``mix64(s + n * GAMMA)`` with wrapping 64-bit arithmetic.

Element ``i`` of a stream takes outputs ``2i+1`` and ``2i+2`` (128 bits),
splits them into eight 16-bit uniforms and sums them (Irwin-Hall with n=8,
an integer approximation of a normal variate: mean and variance exact,
kurtosis 2.85, support +-4.9 sigma).  The centred integer sum is exact in
fp32, is multiplied by one fp32 scale (a single IEEE multiply, so host and
device round identically) and rounded to bfloat16 with round-to-nearest-even.
The float32 value before that last rounding is available for the tiny
workload's fp32 variant.

Keys are derived per (seed, layer, tensor, expert) so that any expert's
weights can be regenerated alone, which lets the oracle rebuild just the
experts a token selected at full size.

4-bit group-affine experts
--------------------------
The 4-bit variant stores each weight as an unsigned 4-bit code q and each
group of 64 consecutive weights of a row (along the reduction dimension)
with one bf16 scale s and bias b.  Codes are the bytes of a stream's
outputs (output n gives bytes 8(n-1) .. 8n-1, little-endian), two codes per
byte, low nibble first.  Group g takes output g+1 of a second stream: with
u = (bits 9..31) / 2^23 and v = (bits 43..63) / 2^21,
s = bf16(S0 * (0.5 + u)) and b = bf16(-(s * (7 + v))), where S0 is the fp32
constant sigma / 4.61 (every fp32 step is exact or a single IEEE rounding,
so host and device agree).  The affine weights s*q + b then have standard
deviation close to sigma.  The pair is stored as one 32-bit word, s in the
low half.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX_M1 = 0xBF58476D1CE4E5B9
MIX_M2 = 0x94D049BB133111EB

IH_N = 8  # uniforms summed per variate
IH_MEAN = IH_N * 65535 // 2  # 262140 (the true mean 262140.0 is an integer for n=8)
IH_STD = math.sqrt(IH_N * (65536.0 * 65536.0 - 1.0) / 12.0)

# tensor ids for key derivation
T_X = 0
T_ROUTER = 1
T_EXPERT = 2
T_SHARED = 3
T_PERM = 4
T_Q4_CODES = 5
T_Q4_SB = 6
T_Q4_SHARED_CODES = 7
T_Q4_SHARED_SB = 8

Q4_GROUP = 64  # weights per scale/bias group
Q4_STD = 4.61  # standard deviation of q - 7.5 for q uniform on 0..15 (sqrt(255/12))


def mix64_int(z: int) -> int:
    """SplitMix64 finaliser on a Python int (reference for tests and keys)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX_M1) & MASK64
    z = ((z ^ (z >> 27)) * MIX_M2) & MASK64
    return z ^ (z >> 31)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= np.uint64(MIX_M1)
    z ^= z >> np.uint64(27)
    z *= np.uint64(MIX_M2)
    z ^= z >> np.uint64(31)
    return z


def splitmix64_outputs(key: int, first: int, count: int) -> np.ndarray:
    """Outputs ``first .. first+count-1`` (1-based) of the SplitMix64 stream ``key``."""
    n = np.arange(first, first + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(key & MASK64) + n * np.uint64(GAMMA)
    return _mix64_np(z)


def stream_key(seed: int, layer: int, tensor: int, expert: int) -> int:
    """64-bit stream key for one tensor slice."""
    z = mix64_int(seed + GAMMA)
    z = mix64_int(z + layer + 1)
    z = mix64_int(z + tensor + 1)
    return mix64_int(z + expert + 1)


def scale_f32(sigma: float) -> np.float32:
    """The fp32 scale that maps a centred Irwin-Hall sum to standard deviation sigma."""
    return np.float32(sigma / IH_STD)


def normal_f32(key: int, start: int, n: int, sigma: float) -> np.ndarray:
    """Elements ``start .. start+n-1`` of stream ``key`` as fp32 (before bf16 rounding)."""
    if n == 0:
        return np.zeros(0, np.float32)
    raw = splitmix64_outputs(key, 2 * start + 1, 2 * n)
    # the eight 16-bit fields of the element's two outputs (summation order is immaterial)
    s = raw.view(np.uint16).reshape(n, 8).sum(axis=1, dtype=np.int32)
    centred = (s - IH_MEAN).astype(np.float32)  # exact: |s - mean| < 2**24
    return centred * scale_f32(sigma)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 bits, round-to-nearest-even (inputs are finite)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16_np(key: int, start: int, n: int, sigma: float) -> np.ndarray:
    """Elements of stream ``key`` rounded to bfloat16 (uint16 bits): the NumPy definition."""
    return f32_to_bf16_bits(normal_f32(key, start, n, sigma))


_HOST_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth_host.so")
_host = None


def _host_lib():
    """The C twin of ``normal_bf16_np`` (``synth/csrc/synth_host.c``), or None if not built."""
    global _host
    if _host is None:
        if not os.path.exists(_HOST_LIB):
            return None
        L = ctypes.CDLL(_HOST_LIB)
        L.synth_host_normal_bf16.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                             ctypes.c_float]
        L.synth_host_normal_bf16.restype = None
        _host = L
    return _host


def normal_bf16(key: int, start: int, n: int, sigma: float) -> np.ndarray:
    """Elements of stream ``key`` rounded to bfloat16 (returned as uint16 bits).

    Computed by the C twin when it is built (bit-identical, about 100x faster;
    ctypes releases the GIL, so threads run it in parallel), else by NumPy."""
    L = _host_lib()
    if L is None or n == 0:
        return normal_bf16_np(key, start, n, sigma)
    out = np.empty(n, dtype=np.uint16)
    L.synth_host_normal_bf16(out.ctypes.data, key & MASK64, start, n, ctypes.c_float(float(scale_f32(sigma))))
    return out


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes and distributions of one synthetic MoE-layer workload."""

    name: str
    M: int  # tokens per forward call
    H: int
    E: int
    k: int
    I: int
    I_shared: int
    layers: int = 1
    chunks: int = 1  # long prefill: M tokens per call, `chunks` calls
    w_sigma: float = 0.02
    router_sigma: float = 0.02
    x_sigma: float = 1.0
    zipf_s: Optional[float] = None  # per-expert log-Zipf router bias
    seed: int = 0
    x_pool: int = 0  # decode: rows in the rotating input pool

    @property
    def tokens(self) -> int:
        return self.M * self.chunks

    def expert_elems(self) -> int:
        return 3 * self.I * self.H

    def shared_elems(self) -> int:
        return 3 * self.I_shared * self.H

    def describe(self) -> str:
        s = (f"M={self.M} H={self.H} E={self.E} top-{self.k}"
             f"{' + 1 shared' if self.I_shared else ''} I={self.I}")
        if self.layers > 1:
            s += f" x {self.layers} layers"
        if self.chunks > 1:
            s += f" x {self.chunks} chunks ({self.tokens} tokens)"
        if self.zipf_s:
            s += f" zipf_s={self.zipf_s}"
        return s


TINY = Workload("tiny", M=64, H=256, E=16, k=2, I=128, I_shared=128, seed=11)
DECODE = Workload("decode", M=1, H=2048, E=256, k=8, I=512, I_shared=512,
                  layers=40, x_pool=64, seed=21)
PREFILL = Workload("prefill", M=4096, H=2048, E=256, k=8, I=512, I_shared=512, seed=31)
SKEW = Workload("skew", M=4096, H=2048, E=256, k=8, I=512, I_shared=512,
                zipf_s=1.2, seed=41)
LONG = Workload("long", M=8192, H=2048, E=256, k=8, I=512, I_shared=512,
                chunks=16, seed=51)

WORKLOADS = {w.name: w for w in (TINY, DECODE, PREFILL, SKEW, LONG)}


def reduced(w: Workload, **kw) -> Workload:
    """A copy of ``w`` with some shape fields changed (same seed and distributions)."""
    return dataclasses.replace(w, **kw)


# ----------------------------------------------------------------------------
# Host-side tensor builders (bf16 bits as uint16 arrays)
# ----------------------------------------------------------------------------


def x_key(w: Workload, layer: int = 0) -> int:
    return stream_key(w.seed, layer, T_X, 0)


def router_key(w: Workload, layer: int = 0) -> int:
    return stream_key(w.seed, layer, T_ROUTER, 0)


def expert_key(w: Workload, layer: int, e: int) -> int:
    return stream_key(w.seed, layer, T_EXPERT, e)


def shared_key(w: Workload, layer: int = 0) -> int:
    return stream_key(w.seed, layer, T_SHARED, 0)


def x_rows(w: Workload, row0: int, nrows: int, layer: int = 0) -> np.ndarray:
    """Token rows ``row0 .. row0+nrows-1`` of the input, bf16 bits [nrows, H]."""
    return normal_bf16(x_key(w, layer), row0 * w.H, nrows * w.H, w.x_sigma).reshape(nrows, w.H)


def router_weight(w: Workload, layer: int = 0) -> np.ndarray:
    """Router weight [E, H], bf16 bits."""
    return normal_bf16(router_key(w, layer), 0, w.E * w.H, w.router_sigma).reshape(w.E, w.H)


def expert_weight(w: Workload, layer: int, e: int) -> np.ndarray:
    """One routed expert's packed weights, bf16 bits [3*I*H]: gate [I,H], up [I,H], down [H,I]."""
    return normal_bf16(expert_key(w, layer, e), 0, w.expert_elems(), w.w_sigma)


def shared_weight(w: Workload, layer: int = 0) -> np.ndarray:
    """The shared expert's packed weights, bf16 bits [3*I_shared*H] (same packing)."""
    return normal_bf16(shared_key(w, layer), 0, w.shared_elems(), w.w_sigma)


def all_expert_weights(w: Workload, layer: int = 0) -> np.ndarray:
    """All routed experts, bf16 bits [E, 3*I*H] (for small workloads)."""
    return np.stack([expert_weight(w, layer, e) for e in range(w.E)])


def unpack_expert(blk: np.ndarray, I: int, H: int):
    """Split one packed expert block into (gate [I,H], up [I,H], down [H,I]) views."""
    n = I * H
    return blk[:n].reshape(I, H), blk[n:2 * n].reshape(I, H), blk[2 * n:3 * n].reshape(H, I)


def zipf_router_bias(w: Workload, layer: int = 0) -> Optional[np.ndarray]:
    """Per-expert router bias for the skewed workload, fp32 [E], or None.

    A seeded permutation pi of the experts gives each expert a rank
    r_e = pi(e) + 1; the bias is the log of the unnormalised Zipf pmf,
    -s * ln(r_e), so the router's probabilities are multiplied by r_e**-s.
    """
    if not w.zipf_s:
        return None
    draws = splitmix64_outputs(stream_key(w.seed, layer, T_PERM, 0), 1, w.E)
    order = np.argsort(draws, kind="stable")  # order[r] = expert with rank r+1
    rank = np.empty(w.E, dtype=np.int64)
    rank[order] = np.arange(1, w.E + 1)
    return np.array([-w.zipf_s * math.log(r) for r in rank], dtype=np.float64).astype(np.float32)


# ----------------------------------------------------------------------------
# 4-bit group-affine experts
# ----------------------------------------------------------------------------


def q4_codes(key: int, nbytes: int) -> np.ndarray:
    """Bytes 0 .. nbytes-1 of code stream ``key`` (two 4-bit codes per byte, low nibble first)."""
    nout = (nbytes + 7) // 8
    return splitmix64_outputs(key, 1, nout).view(np.uint8)[:nbytes].copy()


def q4_s0(sigma: float) -> np.float32:
    return np.float32(sigma / Q4_STD)


def q4_scale_bias(key: int, ngroups: int, sigma: float) -> np.ndarray:
    """uint32 [ngroups]: bf16 scale (low half) and bias (high half) of each group."""
    raw = splitmix64_outputs(key, 1, ngroups)
    u = ((raw >> np.uint64(9)) & np.uint64(0x7FFFFF)).astype(np.float32) * np.float32(2.0 ** -23)
    v = (raw >> np.uint64(43)).astype(np.float32) * np.float32(2.0 ** -21)
    s_bits = f32_to_bf16_bits(q4_s0(sigma) * (np.float32(0.5) + u))
    s_val = bf16_bits_to_f32(s_bits)
    b_bits = f32_to_bf16_bits(-(s_val * (np.float32(7.0) + v)))
    return s_bits.astype(np.uint32) | (b_bits.astype(np.uint32) << np.uint32(16))


def q4_expert_key(w: "Workload", layer: int, e: int, sb: bool) -> int:
    return stream_key(w.seed, layer, T_Q4_SB if sb else T_Q4_CODES, e)


def q4_shared_key(w: "Workload", layer: int, sb: bool) -> int:
    return stream_key(w.seed, layer, T_Q4_SHARED_SB if sb else T_Q4_SHARED_CODES, 0)


def q4_expert(w: "Workload", layer: int, e: int):
    """One routed expert in 4-bit form: (codes uint8 [3*I*H/2], scale/bias uint32 [3*I*H/64]),
    blocks gate [I][H], up [I][H], down [H][I] as in the bf16 packing."""
    n = w.expert_elems()
    return (q4_codes(q4_expert_key(w, layer, e, False), n // 2),
            q4_scale_bias(q4_expert_key(w, layer, e, True), n // Q4_GROUP, w.w_sigma))


def q4_shared(w: "Workload", layer: int = 0):
    """The shared expert in 4-bit form (same packing)."""
    n = w.shared_elems()
    return (q4_codes(q4_shared_key(w, layer, False), n // 2),
            q4_scale_bias(q4_shared_key(w, layer, True), n // Q4_GROUP, w.w_sigma))


def tiny_f32(w: Workload = TINY):
    """The tiny workload's tensors before bf16 rounding (fp32): x, router, experts, shared."""
    x = normal_f32(x_key(w), 0, w.M * w.H, w.x_sigma).reshape(w.M, w.H)
    r = normal_f32(router_key(w), 0, w.E * w.H, w.router_sigma).reshape(w.E, w.H)
    ex = np.stack([normal_f32(expert_key(w, 0, e), 0, w.expert_elems(), w.w_sigma) for e in range(w.E)])
    sh = normal_f32(shared_key(w), 0, w.shared_elems(), w.w_sigma)
    return x, r, ex, sh
