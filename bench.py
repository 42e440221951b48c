"""Benchmark of the W4A16 weight-only GEMM hot path on one MI355X.

A step is one pass of the hot path over one batch: the four projections of one
27B-class layer (qkv 5120x7168, o 6144x5120, gate+up 5120x34816, down
17408x5120, group 128) at M activation rows, one w4a16_gemm_grouped call through
the C ABI (--separate: four w4a16_gemm calls). Weights are packed once per layer
and kept in HBM; successive steps cycle through --layers distinct layer sets
(1.39 GB at the default 8) so that no step finds its weights in the 256 MB
last-level cache. Inputs are resident on the device before the timed region
starts. The default warmup is long enough (3000 steps) for the clocks to reach
their sustained level before timing.

  python bench.py --sweep   the full-step sweep over a 64-layer stack at
                            M = 1 .. 1024 with the step-time model fitted to it

The headline line reports the decode layer set (M = 1) in HBM TB/s over
algorithmic bytes (packed weights + scales + activations + outputs, counted once
per call). Extra entries report the verify block (M = 16, TB/s), the batched
step (M = 1024, TFLOP/s) and the W4A8 step at M = 256 and 1024 (each
projection's activations quantized to int8, then the int8 MFMA GEMM; TOP/s
against the int8 MFMA peak).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L] [--graph]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, vendor figure
INT8_PEAK_TOPS = 5000.0       # MI355X dense int8 MFMA, vendor figure
GROUP = 128


def algorithmic_bytes(M: int, N: int, K: int, group: int) -> int:
    """Bytes a W4A16 GEMM must move at least once: packed int4 weights, fp16
    scales, bf16 activations in and bf16 outputs out."""
    return K * N // 2 + 2 * N * (K // group) + 2 * M * K + 2 * M * N


def flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def ceiling_tokens_per_s(bandwidth_gbs: float, bytes_per_token_gb: float) -> float:
    """Memory-bound decode ceiling: bandwidth over bytes read per token (the
    bandwidth-ceiling equation of the throughput page's "One weight read" section)."""
    return bandwidth_gbs / bytes_per_token_gb


# ---------------------------------------------------------------------------
# Step-time model: the t_step(B) equation of the throughput page's "One weight
# read, shared by every stream" section, with the per-stream terms of its
# "What one more stream costs on this model" section. Units: bytes, seconds,
# bytes/s, FLOP, FLOP/s.

GIB = 1 << 30
MIB = 1 << 20
KIB = 1 << 10


def kv_bytes_per_token(attn_layers: int, kv_heads: int, head_dim: int, elem_bytes: float) -> float:
    """KV cache per token of context: K and V of every attention layer."""
    return attn_layers * 2 * kv_heads * head_dim * elem_bytes


def state_bytes(layers: int, heads: int, key_dim: int, value_dim: int, elem_bytes: float) -> float:
    """Recurrent state of one stream: one key_dim x value_dim matrix per head per layer."""
    return layers * heads * key_dim * value_dim * elem_bytes


def step_time(B: float, W: float, BW: float, eta: float = 1.0, S: float = 0.0, kappa: float = 0.0,
              L: float = 0.0, r: float = 1.0, F: float = 0.0, P: float = float("inf")) -> float:
    """t_step(B) = max((W + B (2S + kappa L)) / (eta BW), B r F / P): the step
    reads the weights once and each stream's state (read and written) and KV
    cache, or is bound by the arithmetic of B r positions, whichever is longer."""
    memory = (W + B * (2.0 * S + kappa * L)) / (eta * BW)
    compute = B * r * F / P
    return max(memory, compute)


def aggregate_tokens_per_s(B: float, tau: float, t_step_s: float) -> float:
    """Aggregate decode rate: B streams keep tau tokens each per step."""
    return B * tau / t_step_s


def per_stream_tokens_per_s(tau: float, t_step_s: float) -> float:
    return tau / t_step_s


def crossover_streams(W: float, BW: float, F: float, P: float, eta: float = 1.0, S: float = 0.0,
                      kappa: float = 0.0, L: float = 0.0, r: float = 1.0) -> float:
    """Stream count where the two terms of t_step meet (the bend):
    (W + B a) / (eta BW) = B r F / P with a = 2S + kappa L."""
    a = 2.0 * S + kappa * L
    per_stream_compute = r * F / P
    per_stream_memory = a / (eta * BW)
    if per_stream_compute <= per_stream_memory:
        return float("inf")
    return (W / (eta * BW)) / (per_stream_compute - per_stream_memory)


def fit_step_model(rows, step_s, W: float, per_row_bytes: float, flops_per_row: float,
                   BW: float):
    """Fit the two machine parameters of t_step to measured step times of a
    GEMM sweep (rows[i] activation rows take step_s[i] seconds): eta is the
    best bandwidth fraction seen on the memory line (W + rows * per_row_bytes
    per step), P the best arithmetic rate seen (rows * flops_per_row per step).
    Both are the best values seen, so the fitted t_step is an optimistic
    envelope: it is at most every measured time (a lower bound on the step
    time), never above one. Returns (eta, P, bend rows)."""
    eta = max((W + m * per_row_bytes) / (BW * t) for m, t in zip(rows, step_s))
    P = max(m * flops_per_row / t for m, t in zip(rows, step_s))
    bend = crossover_streams(W, BW, flops_per_row, P, eta=eta, S=per_row_bytes / 2.0)
    return eta, P, bend


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4a16_weight_only_gemm_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM traffic per launch from committed rocprofv3 PMC results, or None when
    absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    entry = data.get(f"{kernel}|{workload}")
    if not entry or entry.get("kernel_source_digest") != kernel_source_digest():
        return None
    return entry.get("hbm_bytes_per_launch")


class LayerStore:
    """Packed weights and scales of L layer sets, resident on the device."""

    def __init__(self, layers: int):
        import numpy as np
        import torch

        import synth
        import w4a16_weight_only_gemm_amd as w4
        self.projs = synth.LAYER_PROJECTIONS
        self.layers = []
        for layer in range(layers):
            entry = []
            for pi, p in enumerate(self.projs):
                q = synth.gen_q(synth.tensor_id(synth.KIND_Q, layer, pi), p.N, p.K)
                s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, layer, pi), p.N,
                                     p.K // GROUP)
                qw, sp = w4.w4a16_pack(q, s, GROUP)
                entry.append((torch.from_numpy(qw.view(np.int32)).to("cuda"),
                              torch.from_numpy(sp.view(np.int16)).to("cuda")))
                del q, s, qw, sp
            self.layers.append(entry)
        torch.cuda.synchronize()

    @property
    def weight_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for e in self.layers for pair in e for t in pair)


class Workload:
    """Activations, outputs and launch arguments at M rows for every layer set."""

    def __init__(self, store: LayerStore, M: int, grouped: bool):
        import ctypes

        import numpy as np
        import torch

        import synth
        import w4a16_weight_only_gemm_amd as w4
        self.M = M
        self.store = store
        self.grouped = grouped
        self.x, self.y = [], []
        for layer in range(len(store.layers)):
            xs, ys = [], []
            for pi, p in enumerate(store.projs):
                xb = synth.gen_x(synth.tensor_id(synth.KIND_X, layer, pi, M), M, p.K)
                xs.append(torch.from_numpy(xb.view(np.int16)).to("cuda").view(torch.bfloat16))
                ys.append(torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda"))
            self.x.append(xs)
            self.y.append(ys)
        cols = sum(p.N for p in store.projs)
        self.ws_bytes = w4.w4a16_workspace_bytes(M, cols)
        self.ws = torch.zeros(max(1, self.ws_bytes // 4), dtype=torch.int32, device="cuda")
        # raw launch arguments, so the timed loop does no Python-side checking
        self.args, self.problems = [], []
        for layer in range(len(store.layers)):
            la, entries = [], []
            for pi, p in enumerate(store.projs):
                qw, sp = store.layers[layer][pi]
                la.append((self.x[layer][pi].data_ptr(), qw.data_ptr(), sp.data_ptr(),
                           self.y[layer][pi].data_ptr(), M, p.N, p.K, GROUP))
                entries.append((self.x[layer][pi], qw, sp, self.y[layer][pi], p.N, p.K))
            self.args.append(la)
            arr = w4.make_problems(entries)
            self.problems.append((arr, ctypes.cast(arr, ctypes.c_void_p).value))

    def step_bytes(self) -> int:
        return sum(algorithmic_bytes(self.M, p.N, p.K, GROUP) for p in self.store.projs)

    def step_flops(self) -> int:
        return sum(flops(self.M, p.N, p.K) for p in self.store.projs)


def run_steps(wl: Workload, lib, stream: int, first: int, count: int, only=None):
    """Launch `count` steps starting at step index `first`. Grouped steps are one
    launch (all four projections); otherwise four. With `only`, each step
    launches just projection `only` (to time the dominant launch by itself)."""
    L = len(wl.args)
    for s in range(first, first + count):
        if wl.grouped:
            rc = lib.w4a16_gemm_grouped(wl.problems[s % L][1], 4, wl.M, GROUP,
                                        wl.ws.data_ptr(), wl.ws_bytes, stream)
            if rc != 0:
                raise RuntimeError(f"w4a16_gemm_grouped failed with status {rc}")
            continue
        la = wl.args[s % L]
        for pi, a in enumerate(la):
            if only is not None and pi != only:
                continue
            rc = lib.w4a16_gemm(*a, stream)
            if rc != 0:
                raise RuntimeError(f"w4a16_gemm failed with status {rc}")


def timed(fn, stream_obj) -> float:
    """Milliseconds between HIP events recorded on `stream_obj` around fn()."""
    import torch
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream_obj)
    fn()
    t1.record(stream_obj)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


def time_workload(wl: Workload, steps: int, warmup: int, use_graph: bool, dom: int = 2):
    """(ms per step, mean dominant-launch duration in ms, steps timed).

    The dominant launch (the grouped launch, or projection `dom` otherwise) is
    timed by itself: `steps` back-to-back launches between two events on the
    stream they are launched on, divided by `steps`."""
    import torch

    import w4a16_weight_only_gemm_amd as w4
    lib = w4._lib
    cur = torch.cuda.current_stream()
    stream = cur.cuda_stream
    L = len(wl.args)

    run_steps(wl, lib, stream, 0, warmup)
    torch.cuda.synchronize()
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(cur)
        with torch.cuda.stream(s):
            run_steps(wl, lib, s.cuda_stream, 0, L)  # warm the capture stream
        cur.wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            run_steps(wl, lib, torch.cuda.current_stream().cuda_stream, 0, L)
        for _ in range(max(1, warmup // L)):
            graph.replay()
        reps = max(1, steps // L)
        torch.cuda.synchronize()

        def replay():
            for _ in range(reps):
                graph.replay()
        step_ms, nsteps = timed(replay, cur) / (reps * L), reps * L
    else:
        step_ms, nsteps = timed(lambda: run_steps(wl, lib, stream, 0, steps), cur) / steps, steps

    only = None if wl.grouped else dom
    run_steps(wl, lib, stream, 0, warmup, only=only)
    torch.cuda.synchronize()
    dom_ms = timed(lambda: run_steps(wl, lib, stream, 0, steps, only=only), cur) / steps
    return step_ms, dom_ms, nsteps


def check_parity(wl: Workload, layer: int, cols: int = 64):
    """Sampled parity of the last outputs of one layer against the oracle:
    max over sampled elements of |y - y_ref| / (1e-2 (1 + |y_ref|))."""
    import numpy as np
    import torch

    import oracle
    import synth
    worst = 0.0
    for pi, p in enumerate(wl.store.projs):
        rng = np.random.default_rng(pi)
        c = np.sort(rng.choice(p.N, cols, replace=False))
        rows = min(wl.M, 64)
        q = synth.gen_q(synth.tensor_id(synth.KIND_Q, layer, pi), p.N, p.K)[c]
        s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, layer, pi), p.N, p.K // GROUP)[c]
        x = synth.gen_x(synth.tensor_id(synth.KIND_X, layer, pi, wl.M), wl.M, p.K, rows=(0, rows))
        ref = oracle.gemm(x, q, s, GROUP, threads=synth.default_threads())
        y = wl.y[layer][pi][:rows].view(torch.int16).cpu().numpy().view(np.uint16)[:, c]
        yv = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        worst = max(worst, float(np.max(np.abs(yv - ref) / (1e-2 * (1 + np.abs(ref))))))
    return worst


def time_w4a8(wl: Workload, steps: int, warmup: int):
    """The W4A8 step at wl.M rows: one w4a8_quantize_grouped launch over the
    four projections' activations, then one w4a8_gemm_grouped launch. Returns
    (ms per step, ms per grouped GEMM launch alone, sampled parity ratio
    against the oracle's W4A8 chain)."""
    import ctypes

    import numpy as np
    import torch

    import oracle
    import synth
    import w4a16_weight_only_gemm_amd as w4
    lib = w4._lib
    cur = torch.cuda.current_stream()
    stream = cur.cuda_stream
    M = wl.M
    L = len(wl.args)
    steps_args, keep = [], []
    for layer in range(L):
        qents, gents = [], []
        for pi, p in enumerate(wl.store.projs):
            xq = torch.empty((M, p.K), dtype=torch.int8, device="cuda")
            sx = torch.empty((M,), dtype=torch.float32, device="cuda")
            x, qw, sp, y = wl.args[layer][pi][:4]
            qents.append((x, xq.data_ptr(), sx.data_ptr(), p.K))
            gents.append((xq.data_ptr(), sx.data_ptr(), qw, sp, y, p.N, p.K))
            keep += [xq, sx]
        qa = w4.make_w4a8_quantize_problems(qents)
        ga = w4.make_w4a8_problems(gents)
        keep += [qa, ga]
        steps_args.append((ctypes.cast(qa, ctypes.c_void_p).value, len(qents),
                           ctypes.cast(ga, ctypes.c_void_p).value, len(gents)))

    def run(first, count, gemm_only=False):
        for s_ in range(first, first + count):
            qa, nq, ga, ng = steps_args[s_ % L]
            if not gemm_only:
                rc = lib.w4a8_quantize_grouped(qa, nq, M, stream)
                if rc != 0:
                    raise RuntimeError(f"w4a8_quantize_grouped failed with status {rc}")
            rc = lib.w4a8_gemm_grouped(ga, ng, M, GROUP, stream)
            if rc != 0:
                raise RuntimeError(f"w4a8_gemm_grouped failed with status {rc}")

    run(0, warmup)
    torch.cuda.synchronize()
    step_ms = timed(lambda: run(0, steps), cur) / steps
    dom_ms = timed(lambda: run(0, steps, gemm_only=True), cur) / steps
    run(0, L)  # every layer's outputs from the full chain
    torch.cuda.synchronize()
    worst = 0.0
    for pi, p in enumerate(wl.store.projs):
        rng = np.random.default_rng(10 + pi)
        c = np.sort(rng.choice(p.N, 64, replace=False))
        rows = min(M, 16)
        q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 0, pi), p.N, p.K)[c]
        s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 0, pi), p.N, p.K // GROUP)[c]
        x = synth.gen_x(synth.tensor_id(synth.KIND_X, 0, pi, M), M, p.K, rows=(0, rows))
        xq, sx = oracle.quantize_rows(x)
        ref = oracle.gemm_w4a8(xq, sx, q, s, GROUP)
        y = wl.y[0][pi][:rows].view(torch.int16).cpu().numpy().view(np.uint16)[:, c]
        yv = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        worst = max(worst, float(np.max(np.abs(yv - ref) / (1e-2 * (1 + np.abs(ref))))))
    return step_ms, dom_ms, worst


def read_ceiling(nbytes: int, buffers: int = 8, steps: int = 500, warmup: int = 1000):
    """Practical read ceiling: GB/s of w4a16_read_probe reading `nbytes` once per
    launch (the weight-stream access pattern and nothing else), cycling through
    `buffers` distinct buffers so that no launch finds its bytes in the
    last-level cache. Mean over `steps` back-to-back launches between events
    on the launch stream."""
    import torch

    import w4a16_weight_only_gemm_amd as w4
    nbytes -= nbytes % 16
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(buffers)]
    sink = torch.zeros(w4.READ_PROBE_SINK_BYTES // 4, dtype=torch.int32, device="cuda")
    cur = torch.cuda.current_stream()
    lib, stream = w4._lib, cur.cuda_stream
    ptrs = [b.data_ptr() for b in bufs]

    def run(count):
        for i in range(count):
            rc = lib.w4a16_read_probe(ptrs[i % buffers], nbytes, sink.data_ptr(),
                                      w4.READ_PROBE_SINK_BYTES, stream)
            if rc != 0:
                raise RuntimeError(f"w4a16_read_probe failed with status {rc}")

    run(warmup)
    torch.cuda.synchronize()
    ms = timed(lambda: run(steps), cur) / steps
    del bufs
    return nbytes / (ms * 1e-3) / 1e9, ms


def cpu_baseline(seconds_target: float = 15.0, single_seconds: float = 5.0):
    """The oracle, as it stands, on the host cores: decode layer sets (M = 1),
    projection after projection, layer after layer, until about
    `seconds_target` seconds of CPU work on all host threads, then about
    `single_seconds` on one thread; throughput in the metric's unit."""
    import synth
    import oracle

    def run(threads, seconds):
        done_bytes, t_total, count, layer = 0, 0.0, 0, 0
        while t_total < seconds:
            for pi, p in enumerate(synth.LAYER_PROJECTIONS):
                x, q, s = synth.layer_inputs(layer % 64, pi, 1)
                t0 = time.perf_counter()
                oracle.gemm(x, q, s, GROUP, threads=threads)
                t_total += time.perf_counter() - t0
                done_bytes += algorithmic_bytes(1, p.N, p.K, GROUP)
                count += 1
                if threads == 1 and t_total >= seconds:
                    break
            layer += 1
        return done_bytes / t_total / 1e12, count, layer, t_total

    threads = synth.default_threads()
    value, count, layers, t_total = run(threads, seconds_target)
    single, count1, _, t1 = run(1, single_seconds)
    return {"value": value, "unit": "TB/s", "cores": threads, "kind": "oracle",
            "single_thread_value": single,
            "sample": f"{count} projection GEMMs (decode layer sets M=1, {layers} layers, "
                      f"group {GROUP}), fp64 oracle, {t_total:.1f} s on {threads} threads; "
                      f"single thread: {count1} projection GEMMs, {t1:.1f} s"}


COPY_BYTES = 512 << 20  # calibration kernels: 512 MiB written (fill), 512 MiB read (sum)


def copy_calibration(reps: int = 3):
    """Launch kernels of known traffic a few times -- a fill that writes
    COPY_BYTES and a float32 sum that reads them once (float32, so that no
    widening copy comes first) -- so that a PMC run of this script also
    measures what WRITE_SIZE / FETCH_SIZE report for them."""
    import torch
    buf = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(reps):
        buf.fill_(1.0)
        buf.sum()
    torch.cuda.synchronize()


def traffic_from_pmc(fetch_csv: str, write_csv: str, kernel_substr: str, key: str):
    """HBM bytes per launch of the kernel whose name contains `kernel_substr`,
    from rocprofv3 --pmc counter collections of FETCH_SIZE and of WRITE_SIZE
    (KiB per dispatch), each scaled by (known bytes / counter) of the
    calibration copy in the same run. Writes profiles/traffic.json."""
    import csv
    import statistics

    def per_kernel(path, counter, calib_substr):
        vals, calib = [], []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                v = float(r["Counter_Value"]) * 1024.0
                name = r.get("Kernel_Name", "")
                if kernel_substr in name:
                    vals.append(v)
                elif calib_substr in name:
                    calib.append(v)
        return vals, calib

    fv, fc = per_kernel(fetch_csv, "FETCH_SIZE", "reduce_kernel")   # the sum reads COPY_BYTES
    wv, wc = per_kernel(write_csv, "WRITE_SIZE", "FillFunctor")     # the fill writes COPY_BYTES
    f_scale = COPY_BYTES / statistics.median(fc) if fc else 1.0
    w_scale = COPY_BYTES / statistics.median(wc) if wc else 1.0
    fetch = statistics.median(fv) * f_scale
    write = statistics.median(wv) * w_scale
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[key] = {"kernel_source_digest": kernel_source_digest(),
                 "hbm_bytes_per_launch": fetch + write,
                 "fetch_bytes": fetch, "write_bytes": write,
                 "fetch_scale": f_scale, "write_scale": w_scale,
                 "fetch_samples": len(fv), "write_samples": len(wv)}
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    return data[key]


SWEEP_ROWS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024)


def run_sweep(layers: int, passes: int, rows=SWEEP_ROWS):
    """The full-step sweep: a stack of `layers` layer sets (64 by default, the
    27B-class depth), each step one pass over every layer's four projections
    at M rows; per-M step time, then the step-time model fitted to it."""
    import torch

    import w4a16_weight_only_gemm_amd as w4
    lib = w4._lib
    store = LayerStore(layers)
    projs = store.projs
    W = store.weight_bytes
    per_row = layers * sum(2 * (p.K + p.N) for p in projs)          # x in, y out per row
    flops_row = layers * sum(2 * p.K * p.N for p in projs)
    cur = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    out = []
    for M in rows:
        # activations ~N(0, 1) in bf16, one set per layer and projection
        xs = [[torch.randn((M, p.K), generator=gen, device="cuda").to(torch.bfloat16) for p in projs]
              for _ in range(layers)]
        ys = [[torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda") for p in projs]
              for _ in range(layers)]
        grouped = True
        cols = sum(p.N for p in projs)
        ws_bytes = w4.w4a16_workspace_bytes(M, cols)
        ws = torch.zeros(max(1, ws_bytes // 4), dtype=torch.int32, device="cuda")
        launches = []
        for layer in range(layers):
            entries = [(xs[layer][i], store.layers[layer][i][0], store.layers[layer][i][1],
                        ys[layer][i], p.N, p.K) for i, p in enumerate(projs)]
            if grouped:
                arr = w4.make_problems(entries)
                launches.append(("g", arr))
            else:
                launches.append(("s", [(e[0].data_ptr(), e[1].data_ptr(), e[2].data_ptr(),
                                        e[3].data_ptr(), M, e[4], e[5], GROUP) for e in entries]))
        import ctypes
        stream = cur.cuda_stream

        def one_pass():
            for kind, a in launches:
                if kind == "g":
                    rc = lib.w4a16_gemm_grouped(ctypes.cast(a, ctypes.c_void_p).value, len(projs), M,
                                                GROUP, ws.data_ptr(), ws_bytes, stream)
                    if rc != 0:
                        raise RuntimeError(f"w4a16_gemm_grouped failed with status {rc}")
                else:
                    for args in a:
                        rc = lib.w4a16_gemm(*args, stream)
                        if rc != 0:
                            raise RuntimeError(f"w4a16_gemm failed with status {rc}")

        # warm up for 300 ms (at least two passes): clocks reach their
        # sustained level only after a few thousand launches
        import time
        t_end = time.time() + 0.3
        n_warm = 0
        while n_warm < 2 or time.time() < t_end:
            one_pass()
            n_warm += 1
            torch.cuda.synchronize()

        def timed_passes():
            for _ in range(passes):
                one_pass()
        ms = timed(timed_passes, cur) / passes
        b = W + M * per_row
        f = M * flops_row
        row = {"M": M, "ms_per_step": ms, "tbps": b / (ms * 1e-3) / 1e12,
               "tflops": f / (ms * 1e-3) / 1e12, "positions_per_s": M / (ms * 1e-3),
               "hbm_frac": b / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
               "mfma_frac": f / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)}
        out.append(row)
        print(f"# sweep M={M}: {ms:.3f} ms/step, {row['tbps']:.2f} TB/s, {row['tflops']:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        del xs, ys, ws, launches
        torch.cuda.empty_cache()
    eta, P, bend = fit_step_model([r["M"] for r in out], [r["ms_per_step"] * 1e-3 for r in out],
                                  W, per_row, flops_row, HBM_PEAK_GBS * 1e9)
    return {"workload": f"{layers}-layer stack of the decode layer set (qkv, o, gate_up, down), group "
                        f"{GROUP}; one step = every layer's four projections at M rows, one grouped "
                        f"launch per layer",
            "weight_bytes": W, "rows": out,
            "model": {"eta": eta, "P_tflops": P / 1e12, "bend_rows": bend,
                      "bw_gbs": HBM_PEAK_GBS, "per_row_bytes": per_row, "flops_per_row": flops_row,
                      "note": "t_step(M) = max((W + M a) / (eta BW), M F / P), eta and P the "
                              "best fractions seen over the sweep"}}


HEAD_N, HEAD_K = 248320, 5120
HEAD_ROWS = (1, 2, 4, 8, 16)


def run_head(steps: int, warmup: int, rows=HEAD_ROWS):
    """The output-head workload: one projection of N = 248,320 rows over K = 5120
    (635 MB of packed weights, larger than the last-level cache), at M rows,
    through the workspace entry point; one step = one call."""
    import numpy as np
    import torch

    import synth
    import w4a16_weight_only_gemm_amd as w4
    lib = w4._lib
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 0, 4), HEAD_N, HEAD_K)
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 0, 4), HEAD_N, HEAD_K // GROUP)
    qw, sp = w4.w4a16_pack(q, s, GROUP)
    del q, s
    qw = torch.from_numpy(qw.view(np.int32)).to("cuda")
    sp = torch.from_numpy(sp.view(np.int16)).to("cuda")
    cur = torch.cuda.current_stream()
    out = []
    for M in rows:
        x = torch.from_numpy(synth.gen_x(synth.tensor_id(synth.KIND_X, 0, 4, M), M, HEAD_K)
                             .view(np.int16)).to("cuda")
        y = torch.empty((M, HEAD_N), dtype=torch.int16, device="cuda")
        nb = w4.w4a16_workspace_bytes(M, HEAD_N)
        ws = torch.zeros(max(1, nb // 4), dtype=torch.int32, device="cuda")
        args = (x.data_ptr(), qw.data_ptr(), sp.data_ptr(), y.data_ptr(), M, HEAD_N, HEAD_K, GROUP,
                ws.data_ptr(), nb, cur.cuda_stream)

        def calls(n):
            for _ in range(n):
                rc = lib.w4a16_gemm_ws(*args)
                if rc != 0:
                    raise RuntimeError(f"w4a16_gemm_ws failed with status {rc}")
        calls(warmup)
        torch.cuda.synchronize()
        ms = timed(lambda: calls(steps), cur) / steps
        b = algorithmic_bytes(M, HEAD_N, HEAD_K, GROUP)
        out.append({"M": M, "ms_per_call": ms, "tbps": b / (ms * 1e-3) / 1e12,
                    "hbm_frac": b / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9)})
        print(f"# head M={M}: {ms * 1e3:.1f} us/call, {out[-1]['tbps']:.2f} TB/s", file=sys.stderr,
              flush=True)
    return {"workload": f"output head N={HEAD_N} K={HEAD_K}, group {GROUP}, w4a16_gemm_ws",
            "rows": out}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=3000)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--graph", action="store_true",
                    help="replay the steps from a captured HIP graph (no host launch cost)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--m-list", default="1,16,1024")
    ap.add_argument("--w4a8-m-list", default="256,1024",
                    help="row counts of the W4A8 batched step (empty: none)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain copy of known size (for PMC byte calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="compute profiles/traffic.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--traffic-key", default="streamk_grouped|M=1")
    ap.add_argument("--traffic-kernel", default="::streamk_kernel<")
    ap.add_argument("--separate", action="store_true",
                    help="four launches per step at every M (no grouped streaming launch)")
    ap.add_argument("--sweep", action="store_true",
                    help="full-step sweep over a layer stack at M = 1..1024 and the step-time "
                         "model fitted to it (one JSON object), instead of the headline line")
    ap.add_argument("--sweep-layers", type=int, default=64)
    ap.add_argument("--sweep-passes", type=int, default=5)
    ap.add_argument("--head", action="store_true",
                    help="output-head workload (N = 248,320, K = 5120) at M = 1..16 (one JSON "
                         "object), instead of the headline line")
    args = ap.parse_args(argv)
    if args.traffic_from:
        print(json.dumps(traffic_from_pmc(args.traffic_from[0], args.traffic_from[1],
                                          args.traffic_kernel, args.traffic_key), indent=1))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the GEMM is not sharded across GPUs in this build)", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    import w4a16_weight_only_gemm_amd  # noqa: F401  (fails loudly without the library)
    if args.sweep:
        print(json.dumps(run_sweep(args.sweep_layers, args.sweep_passes)))
        return 0
    if args.head:
        print(json.dumps(run_head(args.steps, min(args.warmup, 1000))))
        return 0

    t0 = time.time()
    store = LayerStore(args.layers)
    print(f"# packed {args.layers} layer sets, {store.weight_bytes / 1e9:.3f} GB resident, "
          f"{time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    results = {}
    for M in [int(v) for v in args.m_list.split(",")]:
        wl = Workload(store, M, grouped=not args.separate)
        ms, dom_ms, nsteps = time_workload(wl, args.steps, args.warmup, args.graph)
        parity = check_parity(wl, 0)
        results[M] = (wl, ms, dom_ms, parity, nsteps)
        print(f"# M={M}: {ms * 1e3:.2f} us/step, dominant launch {dom_ms * 1e3:.2f} us, "
              f"parity ratio {parity:.3f}", file=sys.stderr, flush=True)
        del wl

    M0 = int(args.m_list.split(",")[0])
    wl, ms, dom_ms, parity, nsteps = results[M0]
    step_bytes = wl.step_bytes()
    value = step_bytes / (ms * 1e-3) / 1e12
    gu = store.projs[2]
    if wl.grouped:
        dom_name = "grouped stream-K launch (qkv+o+gate_up+down) at M=%d" % M0
        dom_key = "streamk_grouped"
        dom_bytes = step_bytes
    else:
        dom_name = "gate_up projection (5120x34816) at M=%d" % M0
        dom_key = "gate_up"
        dom_bytes = algorithmic_bytes(M0, gu.N, gu.K, GROUP)
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    workload = (f"decode layer set M={M0}: qkv 5120x7168, o 6144x5120, gate_up 5120x34816, "
                f"down 17408x5120; int4 weights, group {GROUP}, fp16 scales, bf16 activations")
    traffic = load_traffic(dom_key, f"M={M0}")
    extra = []
    for M, (wl2, ms2, dom2, par2, _) in results.items():
        if M == M0:
            continue
        b, f = wl2.step_bytes(), wl2.step_flops()
        e = {"M": M, "ms_per_step": ms2, "tbps": b / (ms2 * 1e-3) / 1e12,
             "tflops": f / (ms2 * 1e-3) / 1e12, "positions_per_s": M / (ms2 * 1e-3),
             "parity_ratio": par2}
        if M >= 256:
            e["roofline"] = {"bound": "mfma", "achieved": e["tflops"], "peak": BF16_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": e["tflops"] / BF16_PEAK_TFLOPS}
        else:
            e["roofline"] = {"bound": "hbm", "achieved": e["tbps"] * 1e3, "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": e["tbps"] * 1e3 / HBM_PEAK_GBS}
        extra.append(e)
    for M in [int(v) for v in args.w4a8_m_list.split(",") if v]:
        wl8 = Workload(store, M, grouped=False)
        ms8, dom8, par8 = time_w4a8(wl8, args.steps, min(args.warmup, 1000))
        f = wl8.step_flops()
        e = {"path": "w4a8", "M": M, "ms_per_step": ms8, "tops": f / (ms8 * 1e-3) / 1e12,
             "positions_per_s": M / (ms8 * 1e-3), "parity_ratio": par8,
             "note": "one w4a8_quantize_grouped launch (bf16 activations of the four "
                     "projections to int8) and one w4a8_gemm_grouped launch; parity against "
                     "the oracle's quantize + W4A8 GEMM"}
        e["roofline"] = {"bound": "mfma", "achieved": f / (dom8 * 1e-3) / 1e12,
                         "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                         "frac": f / (dom8 * 1e-3) / 1e12 / INT8_PEAK_TOPS,
                         "kernel": "w4a8_gemm_grouped launch (qkv+o+gate_up+down) at M=%d" % M}
        if M in results:
            e["speedup_vs_w4a16_step"] = results[M][1] / ms8
        print(f"# W4A8 M={M}: {ms8 * 1e3:.2f} us/step, {e['tops']:.1f} TOP/s, grouped GEMM "
              f"{dom8 * 1e3:.2f} us, parity ratio {par8:.3f}", file=sys.stderr, flush=True)
        extra.append(e)
        del wl8

    line = {
        "metric": "W4A16 GEMM achieved HBM TB/s (M=1,16) and TFLOP/s (M>=256) vs MI355X peak",
        "value": value,
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": nsteps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "M": M0, "group": GROUP, "layers_rotated": args.layers,
                   "graph": bool(args.graph), "positions_per_s": M0 / (ms * 1e-3),
                   "parity_ratio": parity},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": dom_name},
        "extra": extra,
    }
    ceil_gbs, ceil_ms = read_ceiling(step_bytes)
    line["practical_ceiling"] = {
        "value": ceil_gbs, "unit": "GB/s", "frac_of_peak": ceil_gbs / HBM_PEAK_GBS,
        "m1_frac_of_ceiling": achieved / ceil_gbs,
        "kernel": "w4a16_read_probe: one read of the layer set's %d bytes per launch in the "
                  "weight-stream access pattern, 8 rotating buffers, %.2f us per launch"
                  % (step_bytes - step_bytes % 16, ceil_ms * 1e3)}
    print(f"# practical read ceiling: {ceil_gbs:.0f} GB/s ({ceil_ms * 1e3:.2f} us per "
          f"{step_bytes / 1e6:.2f} MB); the M={M0} launch reaches {achieved / ceil_gbs:.1%} of it",
          file=sys.stderr, flush=True)
    if args.copy_calibration:
        copy_calibration()
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
