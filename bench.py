"""Benchmark of the sparse MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

Headline workload: batch-1 decode, one token row through 40 MoE layers with
distinct weights (H=2048, 256 experts top-8 + 1 shared, I=512, bf16; 64.7 GB
of weights, so every layer streams from HBM).  One step = one token through
all 40 layers, replayed from a captured HIP graph; the input row rotates
through a pool of 64 rows.  Alongside: prefill of M=4096 tokens through one
layer (same shapes; near-uniform and Zipf-skewed routing), one step = one
layer call; and a long prompt of 131,072 tokens through one layer as 16
calls of 8,192 rows with one reused workspace, one step = all 16 calls.

Timing: every leg runs its steps in 5 rounds, each bracketed by a device
synchronisation and timed with events; the reported time per step is the
median over the rounds (the headline leg times exactly K steps in all).
The CPU oracle's rounds run between the GPU rounds of the same leg, in the
same process.  Rooflines count algorithmic bytes and FLOPs only (the
weights of the experts that received rows, the router, x and out; no
intermediates, no padding) and are given against the datasheet peaks and
against the rates the measurement kernels of include/moe_peaks.h sustain.

Inputs are seeded synthetic tensors generated on the device before timing.
Printed: one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, datasheet
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, datasheet
METRIC = "MoE-layer tokens/s: prefill M=4096 & decode M=1; % of MFMA / HBM roofline"
ROUNDS = 5


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-q4", action="store_true", help="skip the 4-bit expert-weight runs")
    ap.add_argument("--no-long", action="store_true", help="skip the chunked long-prefill run")
    ap.add_argument("--no-small", action="store_true", help="skip the small-batch runs")
    ap.add_argument("--layout", choices=("tiled", "row"), default="tiled",
                    help="bf16 expert weights: tiled once by moe_tile_weights before timing (default), or "
                         "row-major as generated")
    ap.add_argument("--layers", type=int, default=40, help=argparse.SUPPRESS)
    ap.add_argument("--trace-steps", type=int, default=10)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy three times (the reference "
                         "kernel of known size for scaling HBM byte counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


# source files each kernel is built from (traffic figures taken from other sources are stale)
KERNEL_SOURCES = {
    "k_dec": ("decode.hip", "wave_topk.h", "weights.h", "moe_internal.h", "tiling.hip"),
    "k_sm": ("smallm.hip", "wave_topk.h", "weights.h", "moe_internal.h", "tiling.hip"),
    "k_grouped_gemm": ("grouped_gemm.hip", "moe_internal.h", "tiling.hip"),
    "k_combine": ("grouped_gemm.hip", "moe_internal.h"),
    "k_router_logits": ("route.hip", "moe_internal.h"),
    "k_topk": ("route.hip", "wave_topk.h", "moe_internal.h"),
    "k_route": ("route.hip", "moe_internal.h"),
}


def kernel_source_hash(kernel: str):
    """Hash of the sources of `kernel` (its name or name prefix), or None if unknown."""
    import hashlib
    files = next((v for k, v in KERNEL_SOURCES.items() if kernel.startswith(k)), None)
    if files is None:
        return None
    h = hashlib.sha256()
    d = os.path.join(ROOT, "sparse_moe_router_amd", "csrc")
    for f in files:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def traffic_for(key: str):
    """HBM bytes per launch of the kernel under `key` in the committed counter summary (FETCH_SIZE
    and WRITE_SIZE scaled by the copy-kernel calibration), or None if absent or if the kernel's
    sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get(key)
    if k is None or k.get("source_hash") != kernel_source_hash(key):
        return None
    return round(k["fetch_kib"] * 1024 * t["fetch_scale"] + k["write_kib"] * 1024 * t["write_scale"])


class Hip:
    """hipEvent helpers through the HIP runtime torch already loaded."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so.7")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            assert self.L.hipEventCreate(ctypes.byref(ev)) == 0
            arr[i] = ev
        return arr

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.L.hipEventElapsedTime(ctypes.byref(ms), a, b)
        assert rc == 0, rc
        return ms.value

    def destroy(self, arr):
        for e in arr:
            self.L.hipEventDestroy(e)


class LayerCall:
    """Pre-marshalled moe_layer_forward (bf16 experts) or moe_layer_forward_q4 arguments for one
    layer.  ex / sh: bf16 tensors, or (codes, scale_bias) pairs for 4-bit experts."""

    def __init__(self, moe, x, r, ex, sh, k, out, ws, bias=None, routing=None, flags=0):
        import torch
        M, H = x.shape
        E = r.shape[0]
        self.q4 = isinstance(ex, tuple)
        if self.q4:
            I = ex[0].numel() * 2 // (3 * E * H)
            Is = 0 if sh is None else sh[0].numel() * 2 // (3 * H)
            self.ex_q4 = moe.MoeQ4(ex[0].data_ptr(), ex[1].data_ptr())
            self.sh_q4 = None if sh is None else moe.MoeQ4(sh[0].data_ptr(), sh[1].data_ptr())
            wargs = [ctypes.byref(self.ex_q4), None if sh is None else ctypes.byref(self.sh_q4)]
        else:
            I = ex.numel() // (3 * E * H)
            Is = 0 if sh is None else sh.numel() // (3 * H)
            wargs = [ex.data_ptr(), None if sh is None else sh.data_ptr()]
        self.lib = moe.lib()
        self.desc = moe.make_desc(M, H, E, I, Is, flags, bias)
        self.routing = moe._routing_struct(routing)
        self.args = [ctypes.byref(self.desc), x.data_ptr(), r.data_ptr(), *wargs, k, out.data_ptr(), ws.data_ptr(),
                     ws.numel(), None, None if self.routing is None else ctypes.byref(self.routing)]
        self.torch = torch

    def __call__(self, trace=None):
        self.args[9] = self.torch.cuda.current_stream().cuda_stream
        if self.q4:
            st = self.lib.moe_layer_forward_q4(*self.args, None if trace is None else ctypes.byref(trace))
        elif trace is None:
            st = self.lib.moe_layer_forward(*self.args)
        else:
            st = self.lib.moe_layer_forward_traced(*self.args, ctypes.byref(trace))
        if st != 0:
            raise RuntimeError(f"moe_layer_forward failed with status {st}")


def layout_flag(args, moe, q4, q4_tiled=False):
    """MOE_FLAG_TILED_WEIGHTS when the expert weights were tiled: bf16 weights with --layout tiled
    (moe_tile_weights), 4-bit weights only in the legs that ask for it (moe_tile_weights_q4: faster
    grouped GEMMs, slower matrix-vector paths, so the 4-bit decode and small-batch legs keep the
    row-major packing)."""
    if q4:
        return moe.FLAG_TILED_WEIGHTS if q4_tiled else 0
    return moe.FLAG_TILED_WEIGHTS if args.layout == "tiled" else 0


def layout_name(args, q4, q4_tiled=False):
    if q4:
        return ("4-bit codes + scale/bias words, tiled (moe_tile_weights_q4, once before timing)"
                if q4_tiled else "4-bit codes + scale/bias words, row-major")
    return "tiled (moe_tile_weights, once before timing)" if args.layout == "tiled" else "row-major"


def kernel_times(hip, moe, calls_fn, n_calls_per_step, steps, kernels_per_call):
    """Run `steps` eager steps with per-kernel events; returns {kernel name: [ms per launch]}."""
    import torch
    cap = steps * n_calls_per_step * kernels_per_call
    begin, end = hip.events(cap), hip.events(cap)
    kid = (ctypes.c_int32 * cap)()
    tr = moe.MoeTrace(ctypes.cast(begin, ctypes.POINTER(ctypes.c_void_p)),
                      ctypes.cast(end, ctypes.POINTER(ctypes.c_void_p)), kid, cap, 0)
    for s in range(steps):
        calls_fn(s, tr)
    torch.cuda.synchronize()
    res = {}
    for i in range(tr.count):
        res.setdefault(moe.KERNELS[kid[i]], []).append(hip.elapsed_ms(begin[i], end[i]))
    hip.destroy(begin)
    hip.destroy(end)
    return res


def kernels_us(kt):
    return {n: round(1000.0 * sum(v) / len(v), 3) for n, v in kt.items()}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return os.cpu_count() or 1


def round_sizes(total: int, rounds: int = ROUNDS):
    """`total` steps split into at most `rounds` rounds of (nearly) equal size."""
    r = max(1, min(rounds, total))
    return [total // r + (1 if i < total % r else 0) for i in range(r)]


REWARM_MS = 25.0  # untimed device work after each CPU oracle arm (at least REWARM_MIN calls)
REWARM_MIN = 3


def rewarm(step, sync, ms=REWARM_MS):
    """Untimed calls of step(0) until `ms` of wall time (synchronised every 8 calls, so that it
    tracks device time) and at least REWARM_MIN calls have passed."""
    t0 = time.perf_counter()
    n = 0
    while n < REWARM_MIN or (time.perf_counter() - t0) * 1e3 < ms:
        step(0)
        n += 1
        if n % 8 == 0:
            sync()
    sync()
    return n


def timed_rounds(step, total, between=None, rounds=ROUNDS, sync=None, event=None, rewarm_ms=REWARM_MS):
    """Times exactly `total` calls of step(i) in rounds, each bracketed by a device synchronisation
    and timed with events on the current stream; between(r) runs after round r, untimed (the CPU
    oracle's arm of the same leg), and is followed by untimed calls of step(0) for rewarm_ms: a
    second or more of host work lets the device drop its clocks, and the ramp back would otherwise
    be charged to the next round (and to whatever the caller times after the last one).  Returns
    the per-round milliseconds per call."""
    import torch
    sync = sync or torch.cuda.synchronize
    event = event or (lambda: torch.cuda.Event(enable_timing=True))
    per = []
    i = 0
    for r, n in enumerate(round_sizes(total, rounds)):
        e0, e1 = event(), event()
        sync()
        e0.record()
        for _ in range(n):
            step(i)
            i += 1
        e1.record()
        sync()
        per.append(e0.elapsed_time(e1) / n)
        if between is not None:
            between(r)
            rewarm(step, sync, rewarm_ms)
    return per


def spread(per):
    return {"median": round(statistics.median(per), 5), "min": round(min(per), 5), "max": round(max(per), 5),
            "rounds": len(per)}


def roofline_obj(kernel, avg_ms, nbytes, flops, peaks, traffic=None, layer=None):
    """Roofline position of one kernel from its algorithmic bytes / FLOPs per launch and its average
    launch duration: the bound is the resource that work needs longer on at datasheet peaks."""
    gbs = nbytes / (avg_ms * 1e-3) / 1e9
    tfs = flops / (avg_ms * 1e-3) / 1e12 if flops else 0.0
    mfma_bound = flops and flops / BF16_PEAK_TFLOPS / 1e12 > nbytes / HBM_PEAK_GBS / 1e9
    if mfma_bound:
        r = dict(bound="mfma", achieved=round(tfs, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                 frac=round(tfs / BF16_PEAK_TFLOPS, 4), traffic=traffic,
                 peak_measured=peaks.get("mfma_tflops"), hbm_frac=round(gbs / HBM_PEAK_GBS, 4))
        if peaks.get("mfma_tflops"):
            r["frac_measured"] = round(tfs / peaks["mfma_tflops"], 4)
    else:
        r = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                 frac=round(gbs / HBM_PEAK_GBS, 4), traffic=traffic,
                 peak_measured=peaks.get("hbm_gbs"), mfma_frac=round(tfs / BF16_PEAK_TFLOPS, 4))
        if peaks.get("hbm_gbs"):
            r["frac_measured"] = round(gbs / peaks["hbm_gbs"], 4)
    r.update(kernel=kernel, bytes_per_launch=int(nbytes), flops_per_launch=int(flops), avg_us=round(avg_ms * 1e3, 3))
    if layer is not None:
        r["layer"] = layer
    return r


def layer_fracs(nbytes, flops, ms, peaks):
    """Both roofline fractions of a whole layer (or step) from its algorithmic bytes and FLOPs."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    tfs = flops / (ms * 1e-3) / 1e12
    d = dict(achieved_gbs=round(gbs, 1), hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
             achieved_tflops=round(tfs, 1), mfma_frac=round(tfs / BF16_PEAK_TFLOPS, 4),
             bound="mfma" if flops / BF16_PEAK_TFLOPS / 1e12 > nbytes / HBM_PEAK_GBS / 1e9 else "hbm")
    if peaks.get("hbm_gbs"):
        d["hbm_frac_measured"] = round(gbs / peaks["hbm_gbs"], 4)
    if peaks.get("mfma_tflops"):
        d["mfma_frac_measured"] = round(tfs / peaks["mfma_tflops"], 4)
    return d


# ------------------------------------------------------------------ measured peaks

def measure_peaks():
    """Sustainable rates from the two kernels of include/moe_peaks.h: a 4 GiB streaming read (16 times
    the last-level cache) and a loop of independent bf16 MFMAs on every SIMD; median of 5 rounds."""
    import torch
    path = os.path.join(ROOT, "sparse_moe_router_amd", "libmoe_peaks.so")
    L = ctypes.CDLL(path)
    L.moe_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    L.moe_peak_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    sink = torch.empty(L.moe_peak_stream_blocks(), dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    fsink = torch.empty(cus * 8, dtype=torch.float32, device="cuda")
    iters = 4096
    flops = cus * 8 * iters * 8 * 32 * 32 * 16 * 2

    def read(_):
        s = torch.cuda.current_stream().cuda_stream
        assert L.moe_peak_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), s) == 0

    def mfma(_):
        s = torch.cuda.current_stream().cuda_stream
        assert L.moe_peak_mfma_loop(cus, iters, fsink.data_ptr(), s) == 0

    for f in (read, mfma):
        f(0)
    r_ms = statistics.median(timed_rounds(read, 15))
    m_ms = statistics.median(timed_rounds(mfma, 15))
    del buf
    torch.cuda.empty_cache()
    return dict(hbm_gbs=round(nbytes / (r_ms * 1e-3) / 1e9, 1), mfma_tflops=round(flops / (m_ms * 1e-3) / 1e12, 1),
                stream_read={"bytes": nbytes, "us": round(r_ms * 1e3, 2)},
                mfma_loop={"flops": flops, "us": round(m_ms * 1e3, 2), "cus": cus})


# ------------------------------------------------------------------ decode

def q4_layer(SD, S, w, l, dev="cuda"):
    """One layer's 4-bit experts on the device: ((codes, scale_bias), (shared codes, shared scale_bias))."""
    import torch
    n = w.expert_elems()
    codes = torch.empty(w.E, n // 2, dtype=torch.uint8, device=dev)
    sb = torch.empty(w.E, n // S.Q4_GROUP, dtype=torch.int32, device=dev)
    for e in range(w.E):
        SD.fill_q4(codes[e], sb[e], S.q4_expert_key(w, l, e, False), S.q4_expert_key(w, l, e, True), w.w_sigma)
    ns = w.shared_elems()
    sc = torch.empty(ns // 2, dtype=torch.uint8, device=dev)
    ssb = torch.empty(ns // S.Q4_GROUP, dtype=torch.int32, device=dev)
    SD.fill_q4(sc, ssb, S.q4_shared_key(w, l, False), S.q4_shared_key(w, l, True), w.w_sigma)
    return (codes, sb), (sc, ssb)


class CpuDecode:
    """The oracle's arm of the decode leg: per round, `rows` single-token (M=1) calls through one
    layer (layer r of the 40), the selected experts' weights regenerated on the host before the
    timed part.  tok/s = 1 / (mean time per token-layer x layers)."""

    def __init__(self, S, O, rows=24):
        self.S, self.O, self.rows = S, O, rows
        self.t = []

    def __call__(self, r):
        import concurrent.futures as cf
        S, O, w = self.S, self.O, self.S.DECODE
        f = S.bf16_bits_to_f32
        xs = f(S.x_rows(w, r * self.rows, self.rows, 0))
        rw = f(S.router_weight(w, r))
        sh = f(S.shared_weight(w, r))
        ids = O.topk_ids(O.selection_logits(O.router_logits(xs, rw)), w.k)
        need = sorted(set(int(e) for e in ids.ravel()))
        with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4)) as ex:
            cache = dict(zip(need, ex.map(lambda e: O.unpack_expert(f(S.expert_weight(w, r, e)), w.I, w.H), need)))
        t = time.perf_counter()
        for i in range(self.rows):
            O.moe_forward(xs[i:i + 1], rw, lambda e: cache[e], sh, w.k, w.I)
        self.t.append((time.perf_counter() - t) / self.rows)

    def result(self, layers):
        per = statistics.median(self.t)
        return dict(value=round(1.0 / (per * layers), 4), unit="tok/s", cores=blas_threads(), kind="oracle",
                    sample=f"{len(self.t)} rounds interleaved with the GPU rounds, each {self.rows} single-token "
                           f"calls through one of the {layers} layers (float64 NumPy oracle; the selected experts' "
                           f"weights regenerated outside the timing); tok/s = 1 / (median time per token-layer "
                           f"x {layers})",
                    seconds=round(sum(self.t) * self.rows, 3))


def bench_decode(args, hip, moe, SD, S, peaks, q4=False, cpu=None):
    import torch
    w = S.DECODE
    L = args.layers
    dev = "cuda"
    H, E, I, k = w.H, w.E, w.I, w.k
    t0 = time.time()
    xpool = torch.empty(w.x_pool, H, dtype=torch.bfloat16, device=dev)
    SD.fill(xpool, S.x_key(w, 0), 0, w.x_sigma)
    layers = []
    for l in range(L):
        r = torch.empty(E, H, dtype=torch.bfloat16, device=dev)
        SD.fill(r, S.router_key(w, l), 0, w.router_sigma)
        if q4:
            ex, sh = q4_layer(SD, S, w, l, dev)
        else:
            ex = torch.empty(E, w.expert_elems(), dtype=torch.bfloat16, device=dev)
            for e in range(E):
                SD.fill(ex[e], S.expert_key(w, l, e), 0, w.w_sigma)
            sh = torch.empty(w.shared_elems(), dtype=torch.bfloat16, device=dev)
            SD.fill(sh, S.shared_key(w, l), 0, w.w_sigma)
            if args.layout == "tiled":
                ex, sh = moe.tile_weights(ex, H, I), moe.tile_weights(sh, H, w.I_shared)
        layers.append((r, ex, sh))
    out = torch.empty(L, H, dtype=torch.bfloat16, device=dev)
    wsn = moe.workspace_size(1, H, E, I, w.I_shared, k)
    ws = torch.empty(wsn, dtype=torch.uint8, device=dev)  # layers run in stream order: one workspace
    torch.cuda.synchronize()
    gen_s = time.time() - t0

    xs = [xpool[i:i + 1] for i in range(w.x_pool)]
    lay = layout_flag(args, moe, q4)
    calls = [[LayerCall(moe, xs[i], r, ex, sh, k, out[l:l + 1], ws, flags=lay) for l, (r, ex, sh) in enumerate(layers)]
             for i in range(w.x_pool)]

    # eager reference for row 0, then one captured graph per pool row
    for c in calls[0]:
        c()
    torch.cuda.synchronize()
    eager0 = out.clone()
    graphs = []
    cap_stream = torch.cuda.Stream()
    for i in range(w.x_pool):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap_stream):
            for c in calls[i]:
                c()
        graphs.append(g)
    for rep in range(3):  # replays must reproduce the eager result bit for bit
        out.zero_()
        graphs[0].replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager0.view(torch.int16)), "graph replay differs from eager"

    for s in range(args.warmup):
        graphs[s % w.x_pool].replay()
    per = timed_rounds(lambda i: graphs[i % w.x_pool].replay(), args.steps, between=cpu)
    ms = statistics.median(per)

    # per-kernel durations (eager, traced)
    def step(s, tr):
        for c in calls[s % w.x_pool]:
            c(tr)
    kt = kernel_times(hip, moe, step, L, args.trace_steps, 3)

    # algorithmic bytes (weights: 2 bytes per element in bf16; 4-bit: half a byte per code plus a
    # 4-byte scale/bias word per 64 elements = 0.5625 bytes per element)
    wb = 0.5625 if q4 else 2
    layer_bytes = int((k + 1) * w.expert_elems() * wb) + E * H * 2 + 2 * H * 2
    layer_flops = 2 * H * E + (k + 1) * 3 * 2 * H * I
    Is = w.I_shared
    if "dec_experts" in kt:
        # two launches: the second streams the selected experts' gate/up rows and every down row
        # (selected and shared), reads x and writes out
        dom, kname = "dec_experts", "k_dec_experts"
        dom_bytes = int((k * 2 * I * H + (k * I + Is) * H) * wb) + 2 * H * 2
        dom_flops = 2 * H * (k * 2 * I + k * I + Is)
    else:
        # three launches: the gate/up kernel streams the selected and shared experts' gate/up rows and x
        dom, kname = "dec_gateup", "k_dec_gateup"
        dom_bytes = int((k * I + Is) * 2 * H * wb) + H * 2
        dom_flops = (k * I + Is) * 2 * 2 * H
    avg_ms = sum(kt[dom]) / len(kt[dom])
    lay_f = layer_fracs(layer_bytes * L, layer_flops * L, ms, peaks)
    res = dict(
        value=1000.0 / ms, ms_per_step=ms, ms_rounds=spread(per), gen_s=gen_s,
        layer_us=ms * 1000.0 / L, layer_bytes=layer_bytes, layer=lay_f,
        kernels_us=kernels_us(kt),
        roofline=roofline_obj(kname + ("<q4>" if q4 else ""), avg_ms, dom_bytes, dom_flops, peaks,
                              traffic=traffic_for(kname + ("<q4>" if q4 else "")),
                              layer={"hbm_frac": lay_f["hbm_frac"], "frac_measured": lay_f.get("hbm_frac_measured"),
                                     "us_per_layer": round(ms * 1000.0 / L, 3), "bytes_per_layer": layer_bytes}),
    )
    return res, (layers, xpool)


def bench_small(args, hip, moe, S, layers, xpool, Ms=(2, 4, 8, 16, 32, 64)):
    """Small batches of M token rows through the decode workload's layers: the matrix-vector
    paths (FORCE_GEMV: the decode kernels for up to 5 rows (8 with 4-bit experts), the
    small-batch kernels over the union of the selected experts above) beside the grouped path (FORCE_GEMM), both HIP-graph
    replayed.  Bytes = the union's expert weights + the shared expert + router + activations,
    from the routing the call itself produced (the minimum any path must read)."""
    import torch
    w = S.DECODE
    H, E, I, k, Is = w.H, w.E, w.I, w.k, w.I_shared
    L = len(layers)
    q4 = isinstance(layers[0][1], tuple)
    wb = 0.5625 if q4 else 2
    cap_stream = torch.cuda.Stream()
    steps = max(5, args.steps // 10)
    res = {}
    for M in Ms:
        x = xpool[:M]
        entry = {}
        for name, flags in (("small", moe.FLAG_FORCE_GEMV), ("grouped", moe.FLAG_FORCE_GEMM)):
            out = torch.empty(L, M, H, dtype=torch.bfloat16, device="cuda")
            ids = torch.empty(L, M, k, dtype=torch.int32, device="cuda")
            ws = torch.empty(moe.workspace_size(M, H, E, I, Is, k, flags=flags), dtype=torch.uint8, device="cuda")
            calls = [LayerCall(moe, x, r, ex, sh, k, out[l], ws, routing={"topk_ids": ids[l]},
                               flags=flags | layout_flag(args, moe, q4))
                     for l, (r, ex, sh) in enumerate(layers)]
            for c in calls:
                c()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap_stream):
                for c in calls:
                    c()
            for _ in range(2):
                g.replay()
            per = timed_rounds(lambda i: g.replay(), steps)
            ms = statistics.median(per)
            union = sum(len(torch.unique(ids[l]).tolist()) for l in range(L)) / L
            layer_bytes = (union + 1) * w.expert_elems() * wb + E * H * 2 + 2 * M * H * 2
            kt = kernel_times(hip, moe, lambda s, tr: [c(tr) for c in calls], L, 3, 7)
            entry[name] = {"tok_s": round(M * 1000.0 / ms, 1), "us_per_layer": round(ms * 1000.0 / L, 3),
                           "hbm_frac": round(layer_bytes * L / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "kernels_us": kernels_us(kt)}
            entry["union_experts"] = round(union, 2)
            if name == "small":
                small_out = out.clone()
            else:
                d = (out.float() - small_out.float()).abs().amax(dim=-1) / small_out.float().abs().amax(dim=-1)
                entry["paths_max_rel_diff"] = round(float(d.max()), 5)
            del calls, ws
        res[str(M)] = entry
    return res


# ------------------------------------------------------------------ prefill

def gateup_roofline(kt, w, M, nonempty, q4, peaks=None, q4_tiled=False):
    """Roofline position of the gate/up grouped GEMM (k_grouped_gemm<0>) for M rows: algorithmic
    bytes (the gate/up weights of the routed experts that received rows, x read once; no
    intermediates) and FLOPs (2 * 2*I*H per assignment) per launch over its average event-timed
    duration; the bound is the resource that work needs longer on at datasheet peaks.  The
    shared expert's gate/up tiles run in the down launch, so they count there, not here."""
    H, I, k = w.H, w.I, w.k
    wb = 0.5625 if q4 else 2  # weight bytes per element
    gu_bytes = int(nonempty * 2 * I * H * wb) + M * H * 2
    gu_flops = M * k * 2 * I * H * 2
    avg = sum(kt["gemm_gateup"]) / len(kt["gemm_gateup"])
    tag = ("<0,q4t>" if q4_tiled else "<0,q4>") if q4 else "<0>"
    kname = {"<0>": "k_grouped_gemm<0>", "<0,q4>": "k_grouped_gemm<0, q4>",
             "<0,q4t>": "k_grouped_gemm<0, q4> on tiled 4-bit weights"}[tag] + " (gate/up + SwiGLU)"
    traffic = traffic_for(f"k_grouped_gemm{tag}@{w.name}")
    return roofline_obj(kname, avg, gu_bytes, gu_flops, peaks or {}, traffic=traffic)


class CpuPrefill:
    """The oracle's arm of a prefill leg: per round, all tokens of the layer (or the first
    m_sample); every selected expert's weights regenerated on the host once, before the first
    round."""

    def __init__(self, S, O, w, m_sample=None):
        import concurrent.futures as cf
        self.S, self.O, self.w = S, O, w
        self.m = m_sample or w.M
        f = S.bf16_bits_to_f32
        self.x = f(S.x_rows(w, 0, self.m))
        self.r = f(S.router_weight(w))
        self.sh = f(S.shared_weight(w))
        self.bias = S.zipf_router_bias(w)
        ids = O.topk_ids(O.selection_logits(O.router_logits(self.x, self.r, self.bias)), w.k)
        self.need = sorted(set(int(e) for e in ids.ravel()))
        with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4)) as ex:
            self.blocks = dict(zip(self.need, ex.map(
                lambda e: O.unpack_expert(f(S.expert_weight(w, 0, e)), w.I, w.H), self.need)))
        self.t = []

    def __call__(self, r):
        w = self.w
        t = time.perf_counter()
        self.O.moe_forward(self.x, self.r, lambda e: self.blocks[e], self.sh, w.k, w.I, bias=self.bias)
        self.t.append(time.perf_counter() - t)

    def result(self):
        dt = statistics.median(self.t)
        w = self.w
        return dict(value=round(self.m / dt, 2), unit="tok/s", cores=blas_threads(), kind="oracle",
                    sample=(f"first {self.m} of the {w.M} tokens" if self.m < w.M else f"all {w.M} tokens") +
                           f" through the layer per round, {len(self.t)} rounds interleaved with the GPU rounds "
                           f"(float64 NumPy oracle; {len(self.need)} experts' weights regenerated outside the "
                           f"timing); tok/s from the median round",
                    seconds=round(sum(self.t), 3))


def bench_prefill(args, hip, moe, SD, S, w, peaks, q4=False, cpu=None, q4_tiled=False):
    import torch
    if q4:
        x, r, ec, esb, sc, ssb = SD.layer_tensors_q4(w)
        ex, sh = (ec, esb), (sc, ssb)
        if q4_tiled:
            ex, sh = moe.tile_weights_q4(*ex, w.H, w.I), moe.tile_weights_q4(*sh, w.H, w.I_shared)
    else:
        x, r, ex, sh = SD.layer_tensors(w)
        if args.layout == "tiled":
            ex, sh = moe.tile_weights(ex, w.H, w.I), moe.tile_weights(sh, w.H, w.I_shared)
    bias = None
    if w.zipf_s:
        bias = torch.from_numpy(S.zipf_router_bias(w)).cuda()
    out = torch.empty_like(x)
    ws = torch.empty(moe.workspace_size(w.M, w.H, w.E, w.I, w.I_shared, w.k), dtype=torch.uint8, device="cuda")
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    call = LayerCall(moe, x, r, ex, sh, w.k, out, ws, bias=bias, routing={"counts": counts},
                     flags=layout_flag(args, moe, q4, q4_tiled))
    for _ in range(args.warmup):
        call()
    per_round = max(20, args.steps // ROUNDS)
    per = timed_rounds(lambda i: call(), per_round * ROUNDS, between=cpu)
    ms = statistics.median(per)
    kt = kernel_times(hip, moe, lambda s, tr: call(tr), 1, args.trace_steps, 8)
    c = counts.cpu()
    nonempty = int((c > 0).sum())
    M, H, E, I, k = w.M, w.H, w.E, w.I, w.k
    wb = 0.5625 if q4 else 2  # weight bytes per element
    layer_bytes = int((nonempty + 1) * w.expert_elems() * wb) + E * H * 2 + 2 * M * H * 2
    flops = M * (2 * H * E + (k + 1) * 3 * 2 * H * I)
    lay_f = layer_fracs(layer_bytes, flops, ms, peaks)
    roof = gateup_roofline(kt, w, M, nonempty, q4, peaks, q4_tiled)
    roof["layer"] = {"hbm_frac": lay_f["hbm_frac"], "mfma_frac": lay_f["mfma_frac"], "bound": lay_f["bound"]}
    res = dict(
        value=M / (ms * 1e-3), unit="tok/s", ms_per_step=ms, steps=per_round * ROUNDS, ms_rounds=spread(per),
        config=dict(workload=f"{w.name}: {w.describe()}, {'4-bit group-affine' if q4 else 'bf16'} experts",
                    weights_layout=layout_name(args, q4, q4_tiled),
                    nonempty_experts=nonempty,
                    max_group=int(c.max()), empty_groups=int((c == 0).sum())),
        layer_bytes=layer_bytes, layer_flops=flops, layer=lay_f,
        hbm_frac=lay_f["hbm_frac"], mfma_frac=lay_f["mfma_frac"],
        kernels_us=kernels_us(kt),
        roofline=roof,
    )
    del x, r, ex, sh, ws
    return res


def bench_long(args, hip, moe, SD, S, w, peaks):
    """Long prefill: w.tokens token rows through one layer as w.chunks calls of w.M rows on
    consecutive slices of one input, with one workspace sized for a chunk and reused.  One pass =
    all chunks; reports the sustained rates over whole passes and the spread over chunks."""
    import torch
    x, r, ex, sh = SD.layer_tensors(w, x_rows=w.tokens)
    if args.layout == "tiled":
        ex, sh = moe.tile_weights(ex, w.H, w.I), moe.tile_weights(sh, w.H, w.I_shared)
    out = torch.empty_like(x)
    ws = torch.empty(moe.workspace_size(w.M, w.H, w.E, w.I, w.I_shared, w.k), dtype=torch.uint8, device="cuda")
    counts = torch.empty(w.chunks, w.E, dtype=torch.int32, device="cuda")
    M = w.M
    calls = [LayerCall(moe, x[c * M:(c + 1) * M], r, ex, sh, w.k, out[c * M:(c + 1) * M], ws,
                       routing={"counts": counts[c]}, flags=layout_flag(args, moe, False)) for c in range(w.chunks)]

    def one_pass(_=None):
        for call in calls:
            call()

    one_pass()
    passes_per_round = 2  # 32 chunk calls per round
    per = timed_rounds(one_pass, passes_per_round * ROUNDS)
    ms = statistics.median(per)
    # one more pass with an event between chunks: the per-chunk spread
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(w.chunks + 1)]
    ev[0].record()
    for c, call in enumerate(calls):
        call()
        ev[c + 1].record()
    torch.cuda.synchronize()
    chunk_ms = [ev[c].elapsed_time(ev[c + 1]) for c in range(w.chunks)]
    kt = kernel_times(hip, moe, lambda s, tr: calls[s % w.chunks](tr), 1, max(args.trace_steps, w.chunks), 8)
    c = counts.cpu()
    nonempty = (c > 0).sum(dim=1)
    H, E, I, k = w.H, w.E, w.I, w.k
    flops = w.tokens * (2 * H * E + (k + 1) * 3 * 2 * H * I)
    layer_bytes = sum(int((int(n) + 1) * w.expert_elems() * 2) + E * H * 2 + 2 * M * H * 2 for n in nonempty)
    lay_f = layer_fracs(layer_bytes, flops, ms, peaks)
    res = dict(
        value=w.tokens / (ms * 1e-3), unit="tok/s", ms_per_pass=ms, passes=passes_per_round * ROUNDS,
        ms_rounds=spread(per),
        config=dict(workload=f"{w.name}: {w.describe()}, bf16 experts, one workspace reused",
                    weights_layout=layout_name(args, False),
                    nonempty_experts_min=int(nonempty.min()), max_group=int(c.max()),
                    empty_groups_max=int((c == 0).sum(dim=1).max())),
        layer=lay_f, mfma_frac=lay_f["mfma_frac"], hbm_frac=lay_f["hbm_frac"],
        chunk_us={"mean": round(1000.0 * sum(chunk_ms) / len(chunk_ms), 1),
                  "min": round(1000.0 * min(chunk_ms), 1), "max": round(1000.0 * max(chunk_ms), 1)},
        kernels_us=kernels_us(kt),
        roofline=gateup_roofline(kt, w, M, int(nonempty.float().mean().round()), False, peaks),
    )
    del x, out, r, ex, sh, ws
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the layer's multi-GPU sharding is a design, not a build)", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_moe_router_amd import moe
    from synth import device as SD
    from synth import inputs as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moe.lib()  # fails loudly when the library is not built
    hip = Hip()
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    peaks = measure_peaks()
    O = None
    if not args.no_cpu:
        import oracle.moe_oracle as O  # the oracle's arms only (CPU baseline)
    cpu_d = None if O is None else CpuDecode(S, O)
    dec, keep = bench_decode(args, hip, moe, SD, S, peaks, cpu=cpu_d)
    small = None if args.no_small else bench_small(args, hip, moe, S, *keep)
    del keep
    torch.cuda.empty_cache()
    cpu_p = None if O is None else CpuPrefill(S, O, S.PREFILL)
    pre = bench_prefill(args, hip, moe, SD, S, S.PREFILL, peaks, cpu=cpu_p)
    if cpu_p is not None:
        pre["cpu_baseline"] = cpu_p.result()
        del cpu_p
    skew = bench_prefill(args, hip, moe, SD, S, S.SKEW, peaks)
    long = None if args.no_long else bench_long(args, hip, moe, SD, S, S.LONG, peaks)
    torch.cuda.empty_cache()
    dec_q4 = pre_q4 = pre_q4t = small_q4 = None
    if not args.no_q4:
        dq, keep = bench_decode(args, hip, moe, SD, S, peaks, q4=True)
        small_q4 = None if args.no_small else bench_small(args, hip, moe, S, *keep, Ms=(2, 8, 16))
        del keep
        torch.cuda.empty_cache()
        dec_q4 = {"value": round(dq["value"], 2), "unit": "tok/s", "ms_per_step": round(dq["ms_per_step"], 4),
                  "ms_rounds": dq["ms_rounds"], "us_per_layer": round(dq["layer_us"], 3), "layer": dq["layer"],
                  "kernels_us": dq["kernels_us"], "roofline": dq["roofline"],
                  "config": {"workload": f"decode batch-1, {args.layers} layers, 4-bit group-affine experts "
                                         f"(g=64, bf16 scale+bias), bf16 router/x/out"}}
        pre_q4 = bench_prefill(args, hip, moe, SD, S, S.PREFILL, peaks, q4=True)
        torch.cuda.empty_cache()
        pre_q4t = bench_prefill(args, hip, moe, SD, S, S.PREFILL, peaks, q4=True, q4_tiled=True)
    w = S.DECODE
    line = {
        "metric": METRIC, "value": round(dec["value"], 2), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(dec["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; weights ~N(0,0.02), x ~N(0,1), generated on device)",
        "config": {"workload": f"decode batch-1: 1 token row x {args.layers} MoE layers, "
                               f"H={w.H} E={w.E} top-{w.k} + 1 shared, I={w.I}, bf16 weights "
                               f"({args.layers * (w.E + 1) * w.expert_elems() * 2 / 1e9:.1f} GB), "
                               f"HIP-graph replay", "layers": args.layers,
                   "weights_layout": layout_name(args, False),
                   "timing": f"{args.steps} steps in {len(round_sizes(args.steps))} rounds, median round"},
        "roofline": dec["roofline"],
        "cpu_baseline": None if cpu_d is None else cpu_d.result(args.layers),
        "peaks_measured": peaks,
        "decode_layer": {"us_per_layer": round(dec["layer_us"], 3), "layer": dec["layer"],
                         "ms_rounds": dec["ms_rounds"], "kernels_us": dec["kernels_us"]},
        "prefill": pre,
        "prefill_skew": skew,
        "prefill_long": long,
        "decode_q4": dec_q4,
        "prefill_q4": pre_q4,
        "prefill_q4_tiled": pre_q4t,
        "small_batch": None if args.no_small else {
            "config": {"workload": f"M token rows x {args.layers} decode layers (same weights), "
                                   f"matrix-vector path over the union of selected experts vs grouped path"},
            "bf16": small, "q4": small_q4},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
