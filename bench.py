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

Inputs are seeded synthetic tensors generated on the device before timing.
Printed: one JSON line with throughput, the dominant kernel's roofline
position (per-launch algorithmic bytes over its event-timed duration), and
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, datasheet
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, datasheet
METRIC = "MoE-layer tokens/s: prefill M=4096 & decode M=1; % of MFMA / HBM roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-q4", action="store_true", help="skip the 4-bit expert-weight runs")
    ap.add_argument("--no-long", action="store_true", help="skip the chunked long-prefill run")
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


def layout_flag(args, moe, q4):
    """MOE_FLAG_TILED_WEIGHTS when the bf16 expert weights were tiled (4-bit weights stay as they are)."""
    return moe.FLAG_TILED_WEIGHTS if args.layout == "tiled" and not q4 else 0


def layout_name(args, q4):
    if q4:
        return "4-bit codes + scale/bias words, row-major"
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


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return os.cpu_count() or 1


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


def bench_decode(args, hip, moe, SD, S, q4=False):
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
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(args.steps):
        graphs[s % w.x_pool].replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # per-kernel durations (eager, traced)
    def step(s, tr):
        for c in calls[s % w.x_pool]:
            c(tr)
    kt = kernel_times(hip, moe, step, L, args.trace_steps, 3)

    # algorithmic bytes (weights: 2 bytes per element in bf16; 4-bit: half a byte per code plus a
    # 4-byte scale/bias word per 64 elements = 0.5625 bytes per element)
    wb = 0.5625 if q4 else 2
    layer_bytes = int((k + 1) * w.expert_elems() * wb) + E * H * 2 + 2 * H * 2
    # the gate/up kernel streams the selected experts' and the shared expert's gate/up rows
    gateup_bytes = int((k * I + w.I_shared) * 2 * H * wb) + H * 2 + E * 4 + (k * I + w.I_shared) * 4
    dom = "dec_gateup"
    avg_ms = sum(kt[dom]) / len(kt[dom])
    achieved = gateup_bytes / (avg_ms * 1e-3) / 1e9
    res = dict(
        value=1000.0 / ms, ms_per_step=ms, gen_s=gen_s,
        layer_us=ms * 1000.0 / L,
        layer_hbm_frac=layer_bytes * L / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        kernels_us={n: round(1000.0 * sum(v) / len(v), 3) for n, v in kt.items()},
        roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic_for("k_dec_gateup<q4>" if q4 else "k_dec_gateup"),
                      kernel="k_dec_gateup" + ("<q4>" if q4 else ""),
                      bytes_per_launch=gateup_bytes, avg_us=round(avg_ms * 1000, 3)),
    )
    return res, (layers, xpool)


def bench_small(args, hip, moe, S, layers, xpool, Ms=(2, 4, 8, 16, 32, 64)):
    """Small batches of M token rows through the decode workload's layers: the matrix-vector
    path over the union of the selected experts (FORCE_GEMV) beside the grouped path
    (FORCE_GEMM), both HIP-graph replayed.  Bytes = the union's expert weights + the shared
    expert + router + activations, from the routing the call itself produced."""
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
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            union = sum(len(torch.unique(ids[l]).tolist()) for l in range(L)) / L
            layer_bytes = (union + 1) * w.expert_elems() * wb + E * H * 2 + 2 * M * H * 2
            kt = kernel_times(hip, moe, lambda s, tr: [c(tr) for c in calls], L, 3, 7)
            entry[name] = {"tok_s": round(M * 1000.0 / ms, 1), "us_per_layer": round(ms * 1000.0 / L, 3),
                           "hbm_frac": round(layer_bytes * L / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "kernels_us": {n: round(1000.0 * sum(v) / len(v), 3) for n, v in kt.items()}}
            entry["union_experts"] = round(union, 2)
            if name == "small":
                small_out = out.clone()
            else:
                d = (out.float() - small_out.float()).abs().amax(dim=-1) / small_out.float().abs().amax(dim=-1)
                entry["paths_max_rel_diff"] = round(float(d.max()), 5)
            del calls, ws
        res[str(M)] = entry
    return res


def cpu_decode(S, O, layers_sample=2, rows=128):
    """Oracle on a bounded sample of the decode workload: `rows` single-token (M=1)
    calls through each of `layers_sample` layers; the selected experts' weights are
    regenerated on the host outside the timing."""
    import concurrent.futures as cf
    w = S.DECODE
    f = S.bf16_bits_to_f32
    xs = f(S.x_rows(w, 0, rows, 0))
    t_total = 0.0
    for l in range(layers_sample):
        r = f(S.router_weight(w, l))
        sh = f(S.shared_weight(w, l))
        ids = O.topk_ids(O.selection_logits(O.router_logits(xs, r)), w.k)
        need = sorted(set(int(e) for e in ids.ravel()))
        with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4)) as ex:
            cache = dict(zip(need, ex.map(lambda e: O.unpack_expert(f(S.expert_weight(w, l, e)), w.I, w.H), need)))
        t = time.perf_counter()
        for i in range(rows):
            O.moe_forward(xs[i:i + 1], r, lambda e: cache[e], sh, w.k, w.I)
        t_total += time.perf_counter() - t
    per_layer = t_total / (layers_sample * rows)
    return dict(value=1.0 / (per_layer * w.layers), unit="tok/s", cores=blas_threads(), kind="oracle",
                sample=f"{rows} single-token calls through each of {layers_sample} of the {w.layers} layers "
                       f"(fp64 NumPy oracle; selected experts regenerated outside the timing); "
                       f"tok/s = 1 / (mean time per token-layer x {w.layers})",
                seconds=round(t_total, 3))


# ------------------------------------------------------------------ prefill

def gateup_roofline(kt, w, M, nonempty, q4):
    """Roofline position of the gate/up grouped GEMM (k_grouped_gemm<0>) for M rows: algorithmic
    bytes (weights of the experts that received rows + the shared expert, x once, h written) or
    flops per launch over its average event-timed duration; the bound is the resource that work
    needs longer on at peak."""
    H, I, k = w.H, w.I, w.k
    wb = 0.5625 if q4 else 2  # weight bytes per element
    gu_bytes = int((nonempty + 1) * 2 * I * H * wb) + M * H * 2 + (M * k + M) * I * 2
    gu_flops = (M * k + M) * 2 * I * H * 2
    avg = sum(kt["gemm_gateup"]) / len(kt["gemm_gateup"])
    ach = gu_bytes / (avg * 1e-3) / 1e9
    ach_tf = gu_flops / (avg * 1e-3) / 1e12
    mfma_bound = gu_flops / BF16_PEAK_TFLOPS / 1e12 > gu_bytes / HBM_PEAK_GBS / 1e9
    kname = "k_grouped_gemm<0, q4> (gate/up + SwiGLU)" if q4 else "k_grouped_gemm<0> (gate/up + SwiGLU)"
    traffic = traffic_for(f"k_grouped_gemm<0,q4>@{w.name}" if q4 else f"k_grouped_gemm<0>@{w.name}")
    if mfma_bound:
        return dict(bound="mfma", achieved=round(ach_tf, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(ach_tf / BF16_PEAK_TFLOPS, 4), traffic=traffic, kernel=kname,
                    flops_per_launch=gu_flops, bytes_per_launch=gu_bytes, avg_us=round(avg * 1000, 2),
                    hbm_frac=round(ach / HBM_PEAK_GBS, 4))
    return dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(ach / HBM_PEAK_GBS, 4), traffic=traffic, kernel=kname,
                bytes_per_launch=gu_bytes, avg_us=round(avg * 1000, 2),
                mfma_frac=round(ach_tf / BF16_PEAK_TFLOPS, 4))


def bench_prefill(args, hip, moe, SD, S, w, q4=False):
    import torch
    if q4:
        x, r, ec, esb, sc, ssb = SD.layer_tensors_q4(w)
        ex, sh = (ec, esb), (sc, ssb)
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
                     flags=layout_flag(args, moe, q4))
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    steps = max(10, args.steps // 4)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    kt = kernel_times(hip, moe, lambda s, tr: call(tr), 1, args.trace_steps, 7)
    c = counts.cpu()
    nonempty = int((c > 0).sum())
    M, H, E, I, k = w.M, w.H, w.E, w.I, w.k
    wb = 0.5625 if q4 else 2  # weight bytes per element
    layer_bytes = int((nonempty + 1) * w.expert_elems() * wb) + E * H * 2 + 2 * M * H * 2
    flops = M * (2 * H * E + (k + 1) * 3 * 2 * H * I)
    roof = gateup_roofline(kt, w, M, nonempty, q4)
    res = dict(
        value=M / (ms * 1e-3), unit="tok/s", ms_per_step=ms, steps=steps,
        config=dict(workload=f"{w.name}: {w.describe()}, {'4-bit group-affine' if q4 else 'bf16'} experts",
                    weights_layout=layout_name(args, q4),
                    nonempty_experts=nonempty,
                    max_group=int(c.max()), empty_groups=int((c == 0).sum())),
        hbm_frac=layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        mfma_frac=flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        kernels_us={n: round(1000.0 * sum(v) / len(v), 2) for n, v in kt.items()},
        roofline=roof,
    )
    del x, r, ex, sh, ws
    return res


def bench_long(args, hip, moe, SD, S, w):
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

    def one_pass():
        for call in calls:
            call()

    one_pass()
    torch.cuda.synchronize()
    passes = max(2, args.steps // 50)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(passes):
        one_pass()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / passes
    # one more pass with an event between chunks: the per-chunk spread
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(w.chunks + 1)]
    ev[0].record()
    for c, call in enumerate(calls):
        call()
        ev[c + 1].record()
    torch.cuda.synchronize()
    chunk_ms = [ev[c].elapsed_time(ev[c + 1]) for c in range(w.chunks)]
    kt = kernel_times(hip, moe, lambda s, tr: calls[s % w.chunks](tr), 1, max(args.trace_steps, w.chunks), 7)
    c = counts.cpu()
    nonempty = (c > 0).sum(dim=1)
    H, E, I, k = w.H, w.E, w.I, w.k
    flops = w.tokens * (2 * H * E + (k + 1) * 3 * 2 * H * I)
    layer_bytes = sum(int((int(n) + 1) * w.expert_elems() * 2) + E * H * 2 + 2 * M * H * 2 for n in nonempty)
    res = dict(
        value=w.tokens / (ms * 1e-3), unit="tok/s", ms_per_pass=ms, passes=passes,
        config=dict(workload=f"{w.name}: {w.describe()}, bf16 experts, one workspace reused",
                    weights_layout=layout_name(args, False),
                    nonempty_experts_min=int(nonempty.min()), max_group=int(c.max()),
                    empty_groups_max=int((c == 0).sum(dim=1).max())),
        mfma_frac=flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        hbm_frac=layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        chunk_us={"mean": round(1000.0 * sum(chunk_ms) / len(chunk_ms), 1),
                  "min": round(1000.0 * min(chunk_ms), 1), "max": round(1000.0 * max(chunk_ms), 1)},
        kernels_us={n: round(1000.0 * sum(v) / len(v), 2) for n, v in kt.items()},
        roofline=gateup_roofline(kt, w, M, int(nonempty.float().mean().round()), False),
    )
    del x, out, r, ex, sh, ws
    return res


def cpu_prefill(S, O, w, m_sample=None):
    """Oracle on the first m_sample tokens (default: all) of the workload through the layer."""
    import concurrent.futures as cf
    m_sample = m_sample or w.M
    f = S.bf16_bits_to_f32
    x = f(S.x_rows(w, 0, m_sample))
    r = f(S.router_weight(w))
    sh = f(S.shared_weight(w))
    bias = S.zipf_router_bias(w)
    ids = O.topk_ids(O.selection_logits(O.router_logits(x, r, bias)), w.k)
    need = sorted(set(int(e) for e in ids.ravel()))
    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4)) as ex:
        blocks = dict(zip(need, ex.map(lambda e: O.unpack_expert(f(S.expert_weight(w, 0, e)), w.I, w.H), need)))
    t = time.perf_counter()
    O.moe_forward(x, r, lambda e: blocks[e], sh, w.k, w.I, bias=bias)
    dt = time.perf_counter() - t
    return dict(value=m_sample / dt, unit="tok/s", cores=blas_threads(), kind="oracle",
                sample=(f"first {m_sample} of the {w.M} tokens" if m_sample < w.M else f"all {w.M} tokens") +
                       f" through the layer (fp64 NumPy oracle; {len(need)} experts' weights regenerated "
                       f"outside the timing)",
                seconds=round(dt, 3))


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
    hip = Hip()
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    dec, keep = bench_decode(args, hip, moe, SD, S)
    small = bench_small(args, hip, moe, S, *keep)
    del keep
    torch.cuda.empty_cache()
    pre = bench_prefill(args, hip, moe, SD, S, S.PREFILL)
    skew = bench_prefill(args, hip, moe, SD, S, S.SKEW)
    long = None if args.no_long else bench_long(args, hip, moe, SD, S, S.LONG)
    torch.cuda.empty_cache()
    dec_q4 = pre_q4 = small_q4 = None
    if not args.no_q4:
        dq, keep = bench_decode(args, hip, moe, SD, S, q4=True)
        small_q4 = bench_small(args, hip, moe, S, *keep, Ms=(2, 8, 16))
        del keep
        torch.cuda.empty_cache()
        dec_q4 = {"value": round(dq["value"], 2), "unit": "tok/s", "ms_per_step": round(dq["ms_per_step"], 4),
                  "us_per_layer": round(dq["layer_us"], 3), "hbm_frac": round(dq["layer_hbm_frac"], 4),
                  "kernels_us": dq["kernels_us"], "roofline": dq["roofline"],
                  "config": {"workload": f"decode batch-1, {args.layers} layers, 4-bit group-affine experts "
                                         f"(g=64, bf16 scale+bias), bf16 router/x/out"}}
        pre_q4 = bench_prefill(args, hip, moe, SD, S, S.PREFILL, q4=True)
    cpu_d = cpu_p = None
    if not args.no_cpu:
        import oracle.moe_oracle as O
        cpu_d = cpu_decode(S, O)
        cpu_p = cpu_prefill(S, O, S.PREFILL)
        pre["cpu_baseline"] = cpu_p
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
                   "weights_layout": layout_name(args, False)},
        "roofline": dec["roofline"],
        "cpu_baseline": cpu_d,
        "decode_layer": {"us_per_layer": round(dec["layer_us"], 3), "hbm_frac": round(dec["layer_hbm_frac"], 4),
                         "kernels_us": dec["kernels_us"]},
        "prefill": pre,
        "prefill_skew": skew,
        "prefill_long": long,
        "decode_q4": dec_q4,
        "prefill_q4": pre_q4,
        "small_batch": {"config": {"workload": f"M token rows x {args.layers} decode layers (same weights), "
                                               f"matrix-vector path over the union of selected experts "
                                               f"vs grouped path"}, "bf16": small, "q4": small_q4},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
