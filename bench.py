"""Benchmark of the W4A16 weight-only GEMM hot path on one MI355X.

A step is one pass of the hot path over one batch: the four projections of one
27B-class layer (qkv 5120x7168, o 6144x5120, gate+up 5120x34816, down
17408x5120, group 128) at M activation rows. The headline step is one
w4a16_gemm_grouped launch of the four projections as independent GEMMs (with a
caller workspace); next to it, at every M, the same step as four w4a16_gemm
calls (no workspace). Weights of --layers distinct layer sets (the 64-layer
stack by default, 11.07 GB) are packed once and kept in HBM; successive steps
cycle through them, and through 8 activation/output sets, so no step finds its
operands in the 256 MB last-level cache. Inputs are resident on the device
before any timed region.

Timing: a time-based clock warm-up (--clock-warmup seconds of back-to-back
launches, declared in the line), then per M and step kind --warmup untimed
steps, exactly --steps timed back-to-back steps (ms_per_step), and --reps (at
least 50) individually timed steps for the median and p10/p90; the plain calls
also per projection. GPU clocks and power are sampled once a second with
amd-smi. Extra entries: every M of --m-list both ways, config 0 (tiny GEMV)
latency, the full step over all layer sets as one planned launch
(w4a16_gemm_planned) next to one grouped launch per layer, the W4A8 step, the
practical read ceiling and the CPU oracle baseline at M = 1, 16 and 64.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L]
  python bench.py --sweep   the full-step sweep over a 64-layer stack at
                            M = 1 .. 1024 with the step-time model fitted to it
  python bench.py --head    the output-head workload (N = 248,320)
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


# The sources the streaming kernel (streamk_kernel, the one whose traffic is
# measured) is compiled from: its own file, the shared device helpers and the
# launch and boundary headers. A change to any of them voids stored counters.
STREAMK_SOURCES = ("w4a16_weight_only_gemm_amd/csrc/w4a16_skinny.hip",
                   "w4a16_weight_only_gemm_amd/csrc/w4a16_device.h",
                   "w4a16_weight_only_gemm_amd/csrc/w4a16_launch.h",
                   "include/w4a16.h")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for name in STREAMK_SOURCES:
        with open(os.path.join(ROOT, name), "rb") as f:
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
    """Packed weights and scales of L layer sets, resident on the device (packing
    runs in host threads: the generator and the packer release the GIL)."""

    def __init__(self, layers: int, projs=None, proj_base: int = 0):
        from concurrent.futures import ThreadPoolExecutor

        import numpy as np
        import torch

        import synth
        import w4a16_weight_only_gemm_amd as w4
        # the full layer's projections, or another set (the tensor-parallel
        # shard) whose tensors take projection slots proj_base + index
        self.projs = projs or synth.LAYER_PROJECTIONS
        self.proj_base = proj_base

        def pack(job):
            layer, pi = job
            p = self.projs[pi]
            slot = proj_base + pi
            q = synth.gen_q(synth.tensor_id(synth.KIND_Q, layer, slot), p.N, p.K, threads=2)
            s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, layer, slot), p.N, p.K // GROUP,
                                 threads=2)
            return w4.w4a16_pack(q, s, GROUP)

        jobs = [(layer, pi) for layer in range(layers) for pi in range(len(self.projs))]
        self.layers = [[None] * len(self.projs) for _ in range(layers)]
        with ThreadPoolExecutor(max_workers=max(1, synth.default_threads() // 2)) as ex:
            for (layer, pi), (qw, sp) in zip(jobs, ex.map(pack, jobs)):
                self.layers[layer][pi] = (torch.from_numpy(qw.view(np.int32)).to("cuda"),
                                          torch.from_numpy(sp.view(np.int16)).to("cuda"))
        torch.cuda.synchronize()

    @property
    def weight_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for e in self.layers for pair in e for t in pair)


class ClockSampler:
    """GPU clocks and socket power sampled once a second with amd-smi in a
    background thread, as the throughput page does next to every run ("Update,
    12 November"): the mean over the XCDs' current gfx clocks, and the socket
    power. summary(t0, t1) reports the samples taken in [t0, t1]."""

    def __init__(self, period: float = 1.0):
        import threading
        self.period = period
        self.samples = []   # (time, mean gfx MHz, min gfx MHz, socket W)
        self.error = None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _sample(self):
        import subprocess
        out = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"],
                             capture_output=True, text=True, timeout=10)
        data = json.loads(out.stdout)
        gpu = data["gpu_data"][0] if isinstance(data, dict) else data[0]
        clocks = [v["clk"]["value"] for k, v in gpu["clock"].items()
                  if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)
                  and isinstance(v["clk"].get("value"), (int, float))]
        power = gpu["power"]["socket_power"]["value"]
        if clocks:
            self.samples.append((time.time(), sum(clocks) / len(clocks), min(clocks), float(power)))

    def _run(self):
        while not self._stop.is_set():
            try:
                self._sample()
            except Exception as e:  # no amd-smi, or output it cannot parse: no samples
                self.error = f"{type(e).__name__}: {e}"[:200]
                return
            self._stop.wait(self.period)

    def start(self):
        self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        self._thread.join(timeout=15)

    def summary(self, t0: float, t1: float):
        import statistics
        s = [x for x in self.samples if t0 <= x[0] <= t1]
        if not s:
            return {"samples": 0, "note": self.error or "no sample fell in this interval"}
        return {"samples": len(s), "sclk_mhz_median": statistics.median(x[1] for x in s),
                "sclk_mhz_min": min(x[2] for x in s),
                "power_w_median": statistics.median(x[3] for x in s)}


def stats_ms(values):
    """median, p10 and p90 (ms) of a list of durations in ms."""
    import numpy as np
    a = np.asarray(values, dtype=np.float64)
    return {"reps": int(a.size), "median_ms": float(np.median(a)),
            "p10_ms": float(np.percentile(a, 10)), "p90_ms": float(np.percentile(a, 90))}


class Workload:
    """Activations, outputs and launch arguments of one layer-set step at M rows.
    Steps cycle through the store's layer sets (weights) and through `xsets`
    activation and output sets, so no step finds its operands in the cache
    from the step before."""

    def __init__(self, store: LayerStore, M: int, xsets: int = 8):
        import ctypes

        import numpy as np
        import torch

        import synth
        import w4a16_weight_only_gemm_amd as w4
        self.M, self.store = M, store
        self.L, self.X = len(store.layers), xsets
        self.x, self.y = [], []
        for i in range(xsets):
            xs, ys = [], []
            for pi, p in enumerate(store.projs):
                xb = synth.gen_x(synth.tensor_id(synth.KIND_X, i, store.proj_base + pi, M), M, p.K)
                xs.append(torch.from_numpy(xb.view(np.int16)).to("cuda").view(torch.bfloat16))
                ys.append(torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda"))
            self.x.append(xs)
            self.y.append(ys)
        cols = sum(p.N for p in store.projs)
        self.ws_bytes = w4.w4a16_workspace_bytes(M, cols)
        self.ws = torch.zeros(max(1, self.ws_bytes // 4), dtype=torch.int32, device="cuda")
        # raw launch arguments per step kind, so the timed loops do no Python checking
        self.plain, self.problems, self._keep = [], [], []
        for layer in range(self.L):
            xi = layer % xsets
            la, entries = [], []
            for pi, p in enumerate(store.projs):
                qw, sp = store.layers[layer][pi]
                la.append((self.x[xi][pi].data_ptr(), qw.data_ptr(), sp.data_ptr(),
                           self.y[xi][pi].data_ptr(), M, p.N, p.K, GROUP))
                entries.append((self.x[xi][pi], qw, sp, self.y[xi][pi], p.N, p.K))
            self.plain.append(la)
            arr = w4.make_problems(entries)
            self._keep.append(arr)
            self.problems.append(ctypes.cast(arr, ctypes.c_void_p).value)

    def step_bytes(self, only=None) -> int:
        return sum(algorithmic_bytes(self.M, p.N, p.K, GROUP)
                   for i, p in enumerate(self.store.projs) if only is None or i == only)

    def step_flops(self, only=None) -> int:
        return sum(flops(self.M, p.N, p.K)
                   for i, p in enumerate(self.store.projs) if only is None or i == only)

    # one step (grouped: one w4a16_gemm_grouped launch; plain: four w4a16_gemm calls)
    def grouped_step(self, lib, stream, s: int):
        rc = lib.w4a16_gemm_grouped(self.problems[s % self.L], len(self.store.projs), self.M, GROUP,
                                    self.ws.data_ptr(), self.ws_bytes, stream)
        if rc != 0:
            raise RuntimeError(f"w4a16_gemm_grouped failed with status {rc}")

    def plain_call(self, lib, stream, s: int, pi: int):
        rc = lib.w4a16_gemm(*self.plain[s % self.L][pi], stream)
        if rc != 0:
            raise RuntimeError(f"w4a16_gemm failed with status {rc}")

    def plain_step(self, lib, stream, s: int):
        for pi in range(len(self.store.projs)):
            self.plain_call(lib, stream, s, pi)


def timed(fn, stream_obj) -> float:
    """Milliseconds between HIP events recorded on `stream_obj` around fn()."""
    import torch
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream_obj)
    fn()
    t1.record(stream_obj)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


def event_durations(fns, reps: int, stream_obj):
    """Durations (ms) of `reps` rounds of the launches fns[0](r), fns[1](r), ...,
    issued back to back, from HIP events recorded on the launch stream between
    consecutive launches: result[r][i] is launch i of round r."""
    import torch
    n = len(fns)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps * n + 1)]
    evs[0].record(stream_obj)
    k = 1
    for r in range(reps):
        for f in fns:
            f(r)
            evs[k].record(stream_obj)
            k += 1
    torch.cuda.synchronize()
    return [[evs[r * n + i].elapsed_time(evs[r * n + i + 1]) for i in range(n)] for r in range(reps)]


def clock_warmup(fn, seconds: float):
    """Launch fn() back to back for about `seconds` of wall time (a time-based
    warm-up: the clocks reach their sustained level only after a few thousand
    launches, whatever --warmup says)."""
    import torch
    t_end = time.time() + seconds
    n = 0
    while n < 2 or time.time() < t_end:
        for _ in range(16):
            fn()
        n += 16
        torch.cuda.synchronize()
    return n


def window_stats(fn, reps: int, per: int, stream_obj):
    """Per-call durations (ms) from `reps` windows of `per` back-to-back calls
    fn(r * per + i), each window bracketed by HIP events on the launch stream
    (no event between the calls of a window, which would add a gap); median and
    p10/p90 over the windows' means."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    evs[0].record(stream_obj)
    for r in range(reps):
        for i in range(per):
            fn(r * per + i)
        evs[r + 1].record(stream_obj)
    torch.cuda.synchronize()
    st = stats_ms([evs[r].elapsed_time(evs[r + 1]) / per for r in range(reps)])
    st["calls_per_rep"] = per
    return st


def measure(wl: Workload, kind: str, steps: int, warmup: int, reps: int, warm_s: float = 0.3):
    """One step kind at wl.M: a time-based warm-up of this very step (warm_s
    seconds: the clocks settle differently for different M), `warmup` untimed
    steps, the mean ms per step over exactly `steps` back-to-back steps, then
    the median and p10/p90 over `reps` windows of 10 back-to-back steps (and,
    for the plain calls, of each projection's call alone)."""
    import torch

    import w4a16_weight_only_gemm_amd as w4
    lib = w4._lib
    cur = torch.cuda.current_stream()
    stream = cur.cuda_stream
    step = wl.grouped_step if kind == "grouped" else wl.plain_step
    clock_warmup(lambda: step(lib, stream, 0), warm_s)
    for s in range(warmup):
        step(lib, stream, s)
    torch.cuda.synchronize()
    ms = timed(lambda: [step(lib, stream, s) for s in range(steps)], cur) / steps
    out = {"ms_per_step": ms, "warmup_s": warm_s}
    out["step"] = window_stats(lambda s: step(lib, stream, s), reps, 10, cur)
    if kind == "plain":
        out["per_projection"] = {}
        for pi, p in enumerate(wl.store.projs):
            st = window_stats(lambda s, pi=pi: wl.plain_call(lib, stream, s, pi), reps, 10, cur)
            st["tbps_at_median"] = wl.step_bytes(pi) / (st["median_ms"] * 1e-3) / 1e12
            st["tflops_at_median"] = wl.step_flops(pi) / (st["median_ms"] * 1e-3) / 1e12
            out["per_projection"][p.name] = st
    return out


def check_parity(wl: Workload, kind: str, cols: int = 64):
    """One step on layer set 0 with activation set 0, then sampled parity of its
    outputs against the oracle: max over sampled elements of
    |y - y_ref| / (1e-2 (1 + |y_ref|)) (all columns of the sample, up to 64 rows)."""
    import numpy as np
    import torch

    import oracle
    import synth
    import w4a16_weight_only_gemm_amd as w4
    stream = torch.cuda.current_stream().cuda_stream
    (wl.grouped_step if kind == "grouped" else wl.plain_step)(w4._lib, stream, 0)
    torch.cuda.synchronize()
    worst = 0.0
    for pi, p in enumerate(wl.store.projs):
        rng = np.random.default_rng(pi)
        c = np.sort(rng.choice(p.N, cols, replace=False))
        rows = min(wl.M, 64)
        q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 0, wl.store.proj_base + pi), p.N, p.K)[c]
        s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 0, wl.store.proj_base + pi), p.N,
                             p.K // GROUP)[c]
        x = synth.gen_x(synth.tensor_id(synth.KIND_X, 0, wl.store.proj_base + pi, wl.M), wl.M, p.K,
                        rows=(0, rows))
        ref = oracle.gemm(x, q, s, GROUP, threads=synth.default_threads())
        y = wl.y[0][pi][:rows].view(torch.int16).cpu().numpy().view(np.uint16)[:, c]
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
    L = wl.L
    steps_args, keep = [], []
    xq_sets = {}
    for layer in range(L):
        xi = layer % wl.X
        if xi not in xq_sets:
            xq_sets[xi] = [(torch.empty((M, p.K), dtype=torch.int8, device="cuda"),
                            torch.empty((M,), dtype=torch.float32, device="cuda"))
                           for p in wl.store.projs]
        qents, gents = [], []
        for pi, p in enumerate(wl.store.projs):
            xq, sx = xq_sets[xi][pi]
            x, qw, sp, y = wl.plain[layer][pi][:4]
            qents.append((x, xq.data_ptr(), sx.data_ptr(), p.K))
            gents.append((xq.data_ptr(), sx.data_ptr(), qw, sp, y, p.N, p.K))
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

    clock_warmup(lambda: run(0, 1), 0.3)
    run(0, warmup)
    torch.cuda.synchronize()
    step_ms = timed(lambda: run(0, steps), cur) / steps
    dom_ms = timed(lambda: run(0, steps, gemm_only=True), cur) / steps
    run(0, 1)  # layer set 0, activation set 0, through the full chain
    torch.cuda.synchronize()
    worst = 0.0
    for pi, p in enumerate(wl.store.projs):
        rng = np.random.default_rng(10 + pi)
        c = np.sort(rng.choice(p.N, 64, replace=False))
        rows = min(M, 16)
        q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 0, wl.store.proj_base + pi), p.N, p.K)[c]
        s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 0, wl.store.proj_base + pi), p.N,
                             p.K // GROUP)[c]
        x = synth.gen_x(synth.tensor_id(synth.KIND_X, 0, pi, M), M, p.K, rows=(0, rows))
        xq, sx = oracle.quantize_rows(x)
        ref = oracle.gemm_w4a8(xq, sx, q, s, GROUP)
        y = wl.y[0][pi][:rows].view(torch.int16).cpu().numpy().view(np.uint16)[:, c]
        yv = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        worst = max(worst, float(np.max(np.abs(yv - ref) / (1e-2 * (1 + np.abs(ref))))))
    return step_ms, dom_ms, worst


def tiny_latency(reps: int = 200):
    """Config 0 (M = 1, K = 256, N = 512, group 64) through w4a16_gemm: per-call
    latency from events between back-to-back calls (cache-resident; latency
    only), and its parity ratio against the oracle."""
    import numpy as np
    import torch

    import oracle
    import synth
    import w4a16_weight_only_gemm_amd as w4
    t = synth.TINY
    M, N, K, g = t["M"], t["N"], t["K"], t["group"]
    x, q, s = synth.tiny_inputs()
    qw, sp = w4.w4a16_pack(q, s, g)
    dx = torch.from_numpy(x.view(np.int16)).to("cuda")
    dq = torch.from_numpy(qw.view(np.int32)).to("cuda")
    ds = torch.from_numpy(sp.view(np.int16)).to("cuda")
    dy = torch.empty((M, N), dtype=torch.int16, device="cuda")
    cur = torch.cuda.current_stream()
    args = (dx.data_ptr(), dq.data_ptr(), ds.data_ptr(), dy.data_ptr(), M, N, K, g, cur.cuda_stream)

    def call(_r):
        rc = w4._lib.w4a16_gemm(*args)
        if rc != 0:
            raise RuntimeError(f"w4a16_gemm failed with status {rc}")
    for r in range(100):
        call(r)
    d = event_durations([call], reps, cur)
    y = (dy.cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = oracle.gemm(x, q, s, g)
    parity = float(np.max(np.abs(y - ref) / (1e-2 * (1 + np.abs(ref)))))
    t0 = time.perf_counter()
    n_cpu = 0
    while time.perf_counter() - t0 < 0.5:
        oracle.gemm(x, q, s, g)
        n_cpu += 1
    cpu_us = (time.perf_counter() - t0) / n_cpu * 1e6
    st = stats_ms([v[0] for v in d])
    return {"workload": f"tiny GEMV M={M} K={K} N={N} group {g}, one w4a16_gemm call "
                        f"(cache-resident: latency only)",
            "latency_us_median": st["median_ms"] * 1e3, "latency_us_p10": st["p10_ms"] * 1e3,
            "latency_us_p90": st["p90_ms"] * 1e3, "reps": st["reps"], "parity_ratio": parity,
            "oracle_us_one_thread": cpu_us}


def stack_steps(store: LayerStore, rows, sampler=None, passes: int = 10, xsets: int = 8,
                plain: bool = False, label: str = "stack"):
    """The full-step workload (every layer of the store, four projections each)
    at each M in `rows`: one planned launch over all of the step's GEMMs, one
    grouped launch per layer and (with plain) four w4a16_gemm calls per layer,
    each timed over `passes` steps after a 300 ms warm-up. Activations from the
    seeded generator, one set per (layer % xsets, projection); outputs per
    layer."""
    import ctypes

    import numpy as np
    import torch

    import synth
    import w4a16_weight_only_gemm_amd as w4
    lib = w4._lib
    cur = torch.cuda.current_stream()
    stream = cur.cuda_stream
    projs = store.projs
    L = len(store.layers)
    W = store.weight_bytes
    per_row = L * sum(2 * (p.K + p.N) for p in projs)
    flops_row = L * sum(2 * p.K * p.N for p in projs)
    out = []
    for M in rows:
        t_begin = time.time()
        X = min(xsets, L)
        xs = [[torch.from_numpy(synth.gen_x(synth.tensor_id(synth.KIND_X, i, store.proj_base + pi, M),
                                            M, p.K)
                                .view(np.int16)).to("cuda").view(torch.bfloat16)
               for pi, p in enumerate(projs)] for i in range(X)]
        ys = [[torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda") for p in projs]
              for _ in range(L)]
        entries = [(xs[l % X][i], store.layers[l][i][0], store.layers[l][i][1], ys[l][i], p.N, p.K)
                   for l in range(L) for i, p in enumerate(projs)]
        plan = w4.w4a16_plan_build(entries, M, GROUP)
        plan_dev = torch.from_numpy(plan).to("cuda")
        pws_bytes = w4.w4a16_plan_workspace_bytes(plan)
        pws = torch.zeros(max(1, pws_bytes // 4), dtype=torch.int32, device="cuda")
        cols = sum(p.N for p in projs)
        gws_bytes = w4.w4a16_workspace_bytes(M, cols)
        gws = torch.zeros(max(1, gws_bytes // 4), dtype=torch.int32, device="cuda")
        arrs = [w4.make_problems(entries[4 * l:4 * l + 4]) for l in range(L)]
        ptrs = [ctypes.cast(a, ctypes.c_void_p).value for a in arrs]

        def planned():
            rc = lib.w4a16_gemm_planned(plan.ctypes.data, plan_dev.data_ptr(), pws.data_ptr(),
                                        pws_bytes, stream)
            if rc != 0:
                raise RuntimeError(f"w4a16_gemm_planned failed with status {rc}")

        def grouped():
            for ptr in ptrs:
                rc = lib.w4a16_gemm_grouped(ptr, len(projs), M, GROUP, gws.data_ptr(), gws_bytes,
                                            stream)
                if rc != 0:
                    raise RuntimeError(f"w4a16_gemm_grouped failed with status {rc}")

        def plain_calls():
            for (x, qw, sp, y, N, K) in entries:
                rc = lib.w4a16_gemm(x.data_ptr(), qw.data_ptr(), sp.data_ptr(), y.data_ptr(), M, N,
                                    K, GROUP, stream)
                if rc != 0:
                    raise RuntimeError(f"w4a16_gemm failed with status {rc}")

        b = W + M * per_row
        f = M * flops_row
        row = {"M": M}
        kinds = [("planned", planned), ("grouped_per_layer", grouped)]
        if plain:
            kinds.append(("plain_calls", plain_calls))
        for name, fn in kinds:
            clock_warmup(fn, 0.3)
            st = window_stats(lambda r: fn(), passes, 1, cur)
            ms = st["median_ms"]
            row[name] = {"ms_per_step_median": ms, "p10_ms": st["p10_ms"], "p90_ms": st["p90_ms"],
                         "tbps": b / (ms * 1e-3) / 1e12, "tflops": f / (ms * 1e-3) / 1e12,
                         "positions_per_s": M / (ms * 1e-3),
                         "hbm_frac": b / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                         "mfma_frac": f / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)}
        if sampler is not None:
            row["clock"] = sampler.summary(t_begin, time.time())
        out.append(row)
        pl = row["planned"]
        print(f"# {label} M={M}: planned {pl['ms_per_step_median']:.3f} ms/step ({pl['tbps']:.2f} TB/s,"
              f" {pl['tflops']:.1f} TFLOP/s); grouped per layer "
              f"{row['grouped_per_layer']['ms_per_step_median']:.3f} ms", file=sys.stderr, flush=True)
        del xs, ys, pws, gws, plan_dev, arrs
        torch.cuda.empty_cache()
    return {"W": W, "per_row": per_row, "flops_row": flops_row, "rows": out}


def cpu_baseline(seconds_target: float = 15.0, single_seconds: float = 5.0,
                 other_rows=(16, 64, 1024), other_seconds: float = 5.0):
    """The oracle, as it stands, on the host cores, in the metric's unit:
    decode layer sets (M = 1), projection after projection, layer after layer,
    for about `seconds_target` seconds on all host threads, then about
    `single_seconds` on one thread; then the layer sets at each M of
    `other_rows` for about `other_seconds` each on all threads (at M = 1024
    one projection GEMM alone takes a few seconds: the sample is the first
    projections of layer set 0)."""
    import synth
    import oracle

    def run(M, threads, seconds):
        done_bytes, done_flops, t_total, count, layer = 0, 0, 0.0, 0, 0
        while t_total < seconds:
            for pi, p in enumerate(synth.LAYER_PROJECTIONS):
                x, q, s = synth.layer_inputs(layer % 64, pi, M)
                t0 = time.perf_counter()
                oracle.gemm(x, q, s, GROUP, threads=threads)
                t_total += time.perf_counter() - t0
                done_bytes += algorithmic_bytes(M, p.N, p.K, GROUP)
                done_flops += flops(M, p.N, p.K)
                count += 1
                if t_total >= seconds:
                    break
            layer += 1
        return done_bytes / t_total / 1e12, done_flops / t_total / 1e12, count, t_total

    threads = synth.default_threads()
    value, _, count, t_total = run(1, threads, seconds_target)
    single, _, count1, t1 = run(1, 1, single_seconds)
    out = {"value": value, "unit": "TB/s", "cores": threads, "kind": "oracle",
           "single_thread_value": single,
           "sample": f"{count} projection GEMMs of decode layer sets (M=1, group {GROUP}), fp64 "
                     f"oracle, {t_total:.1f} s on {threads} threads; single thread: {count1} "
                     f"projection GEMMs, {t1:.1f} s", "by_M": {}}
    for M in other_rows:
        tb, tf, c, tt = run(M, threads, other_seconds)
        out["by_M"][str(M)] = {"tbps": tb, "tflops": tf, "cores": threads,
                               "sample": f"{c} projection GEMMs of layer sets at M={M}, {tt:.1f} s"}
    return out


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


def run_sweep(layers: int, passes: int, rows=SWEEP_ROWS, plain: bool = True):
    """The full-step sweep: a stack of `layers` layer sets (64 by default, the
    27B-class depth), each step one pass over every layer's four projections
    at M rows; per-M step time of one planned launch (the primary figure), of
    one grouped launch per layer and of four plain calls per layer, then the
    step-time model fitted to the planned times."""
    store = LayerStore(layers)
    res = stack_steps(store, rows, passes=passes, plain=plain)
    W, per_row, flops_row = res["W"], res["per_row"], res["flops_row"]
    out = res["rows"]
    eta, P, bend = fit_step_model([r["M"] for r in out],
                                  [r["planned"]["ms_per_step_median"] * 1e-3 for r in out],
                                  W, per_row, flops_row, HBM_PEAK_GBS * 1e9)
    return {"workload": f"{layers}-layer stack of the decode layer set (qkv, o, gate_up, down), group "
                        f"{GROUP}; one step = every layer's four projections at M rows, "
                        f"independent GEMMs: one planned launch over all of them (primary), one "
                        f"grouped launch per layer, or four w4a16_gemm calls per layer",
            "weight_bytes": W, "rows": out,
            "model": {"eta": eta, "P_tflops": P / 1e12, "bend_rows": bend,
                      "bw_gbs": HBM_PEAK_GBS, "per_row_bytes": per_row, "flops_per_row": flops_row,
                      "fitted_to": "planned launch",
                      "note": "t_step(M) = max((W + M a) / (eta BW), M F / P), eta and P the "
                              "best fractions seen over the sweep (an optimistic envelope)"}}


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


PATH_ROWS = (17, 32, 48, 64, 96, 128, 160, 192, 256, 320, 512, 1024)


def run_paths(layers: int, rows=PATH_ROWS, reps: int = 50):
    """The M-dispatch of w4a16_gemm checked against its two alternatives: for
    every projection of the decode layer set and of its tensor-parallel shard,
    at each M, the median time of one call forced onto the small-M kernel
    (W4A16_PATH_SKINNY: the plain_kernel form its model ranks first), forced
    onto the tile engine (W4A16_PATH_LARGE: the tile height its model ranks
    first), and left to choose (W4A16_PATH_AUTO), with the workgroup tile
    w4a16_select_form reports. Above 320 rows the automatic choice is always
    the tile engine. One JSON object."""
    import ctypes

    import torch

    import synth
    import w4a16_weight_only_gemm_amd as w4
    lib = w4._lib
    cur = torch.cuda.current_stream()
    out = []
    # enough layer sets cycled that no call finds its weights in the 256 MB
    # last-level cache: 8 of the layer set (1.4 GB), 16 of the shard (346 MB)
    for label, projs, base, nl in (("layer set", synth.LAYER_PROJECTIONS, 0, layers),
                                   ("tp8 shard", synth.TP8_SHARD_PROJECTIONS, synth.SHARD_PROJ_BASE,
                                    2 * layers)):
        store = LayerStore(nl, projs, base)
        for M in rows:
            wl = Workload(store, M)
            for pi, p in enumerate(projs):
                rec = {"set": label, "proj": p.name, "M": M, "N": p.N, "K": p.K,
                       "form": w4.w4a16_select_form(M, p.N, p.K, GROUP)}
                for name, path in (("skinny", w4.W4A16_PATH_SKINNY), ("large", w4.W4A16_PATH_LARGE),
                                   ("auto", w4.W4A16_PATH_AUTO)):
                    def call(s, path=path):
                        a = wl.plain[s % wl.L][pi]
                        rc = lib.w4a16_gemm_ex(*a, path, ctypes.c_void_p(cur.cuda_stream))
                        if rc != 0:
                            raise RuntimeError(f"w4a16_gemm_ex failed with status {rc}")
                    clock_warmup(lambda: call(0), 0.05)
                    rec[name + "_us"] = window_stats(call, reps, 10, cur)["median_ms"] * 1e3
                best = min(rec["skinny_us"], rec["large_us"])
                rec["auto_over_best"] = rec["auto_us"] / best
                out.append(rec)
                print(f"# {label} {p.name} M={M}: skinny {rec['skinny_us']:.1f} large "
                      f"{rec['large_us']:.1f} auto {rec['auto_us']:.1f} us, form {rec['form']}",
                      file=sys.stderr, flush=True)
            del wl
        del store
        torch.cuda.empty_cache()
    return {"workload": "w4a16_gemm_ex per projection, forced paths and the automatic choice",
            "rows": out}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=3000)
    ap.add_argument("--layers", type=int, default=64,
                    help="layer sets kept resident and cycled through (64: the 27B-class stack)")
    ap.add_argument("--clock-warmup", type=float, default=2.0,
                    help="seconds of back-to-back launches before any timing, whatever --warmup "
                         "says (declared in the line)")
    ap.add_argument("--reps", type=int, default=100,
                    help="individually timed steps behind each median and p10/p90 (>= 50)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--m-list", default="1,16,64,1024")
    ap.add_argument("--stack-m-list", default="1,16,64,1024",
                    help="row counts of the full-step (all layers) planned launch; empty: none")
    ap.add_argument("--shard-m-list", default="1,16,64",
                    help="row counts of the tensor-parallel (8-way) shard step; empty to skip")
    ap.add_argument("--w4a8-m-list", default="256,1024",
                    help="row counts of the W4A8 batched step (empty: none)")
    ap.add_argument("--no-smi", action="store_true", help="do not sample clocks with amd-smi")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain copy of known size (for PMC byte calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="compute profiles/traffic.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--traffic-key", default="streamk_grouped|M=1")
    ap.add_argument("--traffic-kernel", default="::streamk_kernel<")
    ap.add_argument("--only", choices=["grouped", "plain"],
                    help="time only this step kind at each M of --m-list (for profiling)")
    ap.add_argument("--sweep", action="store_true",
                    help="full-step sweep over a layer stack at M = 1..1024 and the step-time "
                         "model fitted to it (one JSON object), instead of the headline line")
    ap.add_argument("--sweep-layers", type=int, default=64)
    ap.add_argument("--sweep-passes", type=int, default=10)
    ap.add_argument("--paths", action="store_true",
                    help="w4a16_gemm's automatic path against both forced paths per projection "
                         "at M = 17..1024 (one JSON object), instead of the headline line")
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
    import w4a16_weight_only_gemm_amd as w4  # fails loudly without the library
    if args.sweep:
        print(json.dumps(run_sweep(args.sweep_layers, args.sweep_passes)))
        return 0
    if args.head:
        print(json.dumps(run_head(args.steps, min(args.warmup, 1000))))
        return 0
    if args.paths:
        print(json.dumps(run_paths(min(args.layers, 8))))
        return 0

    sampler = None if args.no_smi else ClockSampler().start()
    t0 = time.time()
    store = LayerStore(args.layers)
    print(f"# packed {args.layers} layer sets, {store.weight_bytes / 1e9:.3f} GB resident, "
          f"{time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    lib = w4._lib
    cur = torch.cuda.current_stream()
    stream = cur.cuda_stream
    ms_list = [int(v) for v in args.m_list.split(",")]
    kinds = [args.only] if args.only else ["grouped", "plain"]
    reps = max(50, args.reps)

    # time-based clock warm-up on the headline step
    wl0 = Workload(store, ms_list[0])
    t_w = time.time()
    n_w = clock_warmup(lambda: wl0.grouped_step(lib, stream, 0), args.clock_warmup)
    warm = {"seconds": args.clock_warmup, "launches": n_w}
    if sampler is not None:
        warm["clock"] = sampler.summary(t_w, time.time())
    del wl0

    results = {}
    for M in ms_list:
        wl = Workload(store, M)
        entry = {}
        for kind in kinds:
            t_k = time.time()
            r = measure(wl, kind, args.steps, args.warmup, reps)
            r["parity_ratio"] = check_parity(wl, kind)
            b, f = wl.step_bytes(), wl.step_flops()
            ms = r["ms_per_step"]
            r.update({"tbps": b / (ms * 1e-3) / 1e12, "tflops": f / (ms * 1e-3) / 1e12,
                      "positions_per_s": M / (ms * 1e-3)})
            if sampler is not None:
                r["clock"] = sampler.summary(t_k, time.time())
            entry[kind] = r
            print(f"# M={M} {kind}: {ms * 1e3:.2f} us/step (median {r['step']['median_ms'] * 1e3:.2f},"
                  f" p10 {r['step']['p10_ms'] * 1e3:.2f}, p90 {r['step']['p90_ms'] * 1e3:.2f}), "
                  f"{r['tbps']:.3f} TB/s, {r['tflops']:.1f} TFLOP/s, parity ratio "
                  f"{r['parity_ratio']:.3f}", file=sys.stderr, flush=True)
        results[M] = (wl.step_bytes(), wl.step_flops(), entry)
        del wl
        torch.cuda.empty_cache()
    if args.only:
        if args.copy_calibration:
            copy_calibration()
        print(json.dumps({str(M): e for M, (_, _, e) in results.items()}))
        return 0

    M0 = ms_list[0]
    b0, f0, e0 = results[M0]
    head = e0["grouped"]
    ms = head["ms_per_step"]
    value = b0 / (ms * 1e-3) / 1e12
    # dominant kernel: the grouped stream-K launch itself (one launch per step),
    # its mean duration over the timed steps
    achieved = b0 / (ms * 1e-3) / 1e9
    traffic = load_traffic("streamk_grouped", f"M={M0}")
    workload = (f"decode layer set M={M0} as ONE w4a16_gemm_grouped launch of its four "
                f"independent projections (qkv 5120x7168, o 6144x5120, gate_up 5120x34816, down "
                f"17408x5120), caller workspace; int4 weights, group {GROUP}, fp16 scales, bf16 "
                f"activations; {args.layers} layer sets cycled")
    extra = []
    for M, (b, f, e) in results.items():
        for kind, r in e.items():
            if M == M0 and kind == "grouped":
                continue
            x = {"M": M, "call": ("one w4a16_gemm_grouped launch (four independent projections)"
                                  if kind == "grouped" else
                                  "four w4a16_gemm calls (no workspace), one per projection"),
                 **{k: v for k, v in r.items()}}
            if M >= 256:
                x["roofline"] = {"bound": "mfma", "achieved": r["tflops"], "peak": BF16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": r["tflops"] / BF16_PEAK_TFLOPS}
            else:
                x["roofline"] = {"bound": "hbm", "achieved": r["tbps"] * 1e3, "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": r["tbps"] * 1e3 / HBM_PEAK_GBS}
            extra.append(x)
    extra.append({"config0": tiny_latency()})
    print(f"# config 0 latency: {extra[-1]['config0']['latency_us_median']:.2f} us median",
          file=sys.stderr, flush=True)
    stack_rows = [int(v) for v in args.stack_m_list.split(",") if v]
    if stack_rows:
        st = stack_steps(store, stack_rows, sampler=sampler)
        extra.append({"stack": {
            "workload": f"full step: all {args.layers} layer sets x four projections as independent "
                        f"GEMMs ({st['W'] / 1e9:.3f} GB of packed weights and scales): one "
                        f"w4a16_gemm_planned launch per step, next to one grouped launch per layer",
            "rows": st["rows"]}})
    shard_rows = [int(v) for v in args.shard_m_list.split(",") if v]
    if shard_rows:
        import synth
        sst = LayerStore(args.layers, synth.TP8_SHARD_PROJECTIONS, synth.SHARD_PROJ_BASE)
        sh = stack_steps(sst, shard_rows, sampler=sampler, plain=True, label="tp8 shard")
        extra.append({"tp8_shard": {
            "workload": f"one GPU's share of the full step under 8-way tensor parallelism: all "
                        f"{args.layers} layers x (qkv 5120x896, o 768x5120, gate_up 5120x4352, down "
                        f"2176x5120; qkv and gate_up split by columns, o and down by K) "
                        f"({sh['W'] / 1e9:.3f} GB): one planned launch per step, one grouped "
                        f"launch per layer, or four w4a16_gemm calls per layer (the all-reduce "
                        f"of o and down not included)",
            "rows": sh["rows"]}})
        del sst
        torch.cuda.empty_cache()
    for M in [int(v) for v in args.w4a8_m_list.split(",") if v]:
        wl8 = Workload(store, M)
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
            e["speedup_vs_w4a16_step"] = results[M][2]["grouped"]["ms_per_step"] / ms8
        print(f"# W4A8 M={M}: {ms8 * 1e3:.2f} us/step, {e['tops']:.1f} TOP/s, grouped GEMM "
              f"{dom8 * 1e3:.2f} us, parity ratio {par8:.3f}", file=sys.stderr, flush=True)
        extra.append(e)
        del wl8

    line = {
        "metric": "W4A16 GEMM achieved HBM TB/s (M=1,16) and TFLOP/s (M>=256) vs MI355X peak",
        "value": value,
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "M": M0, "group": GROUP, "layers_rotated": args.layers,
                   "positions_per_s": M0 / (ms * 1e-3), "parity_ratio": head["parity_ratio"],
                   "clock_warmup": warm, "step": head["step"], "clock": head.get("clock")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "streamk_kernel: the grouped launch (qkv+o+gate_up+down) at M=%d, "
                               "mean over the %d timed steps (one launch each)" % (M0, args.steps)},
        "extra": extra,
    }
    ceil_gbs, ceil_ms = read_ceiling(b0)
    line["practical_ceiling"] = {
        "value": ceil_gbs, "unit": "GB/s", "frac_of_peak": ceil_gbs / HBM_PEAK_GBS,
        "m1_frac_of_ceiling": achieved / ceil_gbs,
        "kernel": "w4a16_read_probe: one read of the layer set's %d bytes per launch in the "
                  "weight-stream access pattern, 8 rotating buffers, %.2f us per launch"
                  % (b0 - b0 % 16, ceil_ms * 1e3)}
    print(f"# practical read ceiling: {ceil_gbs:.0f} GB/s ({ceil_ms * 1e3:.2f} us per "
          f"{b0 / 1e6:.2f} MB); the M={M0} launch reaches {achieved / ceil_gbs:.1%} of it",
          file=sys.stderr, flush=True)
    if args.copy_calibration:
        copy_calibration()
    if sampler is not None:
        sampler.stop()
        line["clock_samples"] = {"count": len(sampler.samples), "error": sampler.error}
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
