"""Parity of the tensor-parallel shard shapes: one GPU's share of the decode layer
under 8-way tensor parallelism (qkv 5120x896 and gate_up 5120x4352 split by
columns, o 768x5120 and down 2176x5120 split by K), the shapes the benchmark's
shard step times. Three layers of the four projections at M = 1, 2, 16, 64 and
1024, each run three ways -- one planned launch over all twelve GEMMs, one
grouped launch per layer, and one w4a16_gemm call per GEMM -- and checked
against the oracle, |y - y_ref| <= 1e-2 (1 + |y_ref|): every output at M <= 64,
64 sampled rows (the first, the last, and 62 at random) at M = 1024."""
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_util import tolerance_ratio

pytestmark = pytest.mark.gpu

PROJS = synth.TP8_SHARD_PROJECTIONS
BASE = synth.SHARD_PROJ_BASE
G = synth.GROUP
LAYERS = 3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import w4a16_weight_only_gemm_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def _inputs(layer, pi, M):
    p = PROJS[pi]
    q = synth.gen_q(synth.tensor_id(synth.KIND_Q, layer, BASE + pi), p.N, p.K)
    s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, layer, BASE + pi), p.N, p.K // G)
    x = synth.gen_x(synth.tensor_id(synth.KIND_X, layer, BASE + pi, M), M, p.K)
    return x, q, s


@pytest.mark.parametrize("M", [1, 2, 16, 64, 1024])
def test_tp8_shard_layers_three_ways(M):
    import ctypes

    import torch

    import w4a16_weight_only_gemm_amd as w4
    from gpu_util import dev_u16, dev_u32
    host, dev = [], []
    for layer in range(LAYERS):
        for pi, p in enumerate(PROJS):
            x, q, s = _inputs(layer, pi, M)
            qw, sp = w4.w4a16_pack(q, s, G)
            host.append((x, q, s))
            dev.append((dev_u16(x).view(torch.bfloat16), dev_u32(qw), dev_u16(sp), p.N, p.K))
    outs = {k: [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for (_, _, _, N, _) in dev]
            for k in ("planned", "grouped", "plain")}
    stream = torch.cuda.current_stream().cuda_stream
    # one planned launch over all the GEMMs
    entries = [(x, qw, sp, y, N, K) for (x, qw, sp, N, K), y in zip(dev, outs["planned"])]
    plan = w4.w4a16_plan_build(entries, M, G)
    plan_dev = torch.from_numpy(plan).to("cuda")
    nb = w4.w4a16_plan_workspace_bytes(plan)
    ws = torch.zeros(max(1, (nb + 3) // 4), dtype=torch.int32, device="cuda")
    w4.w4a16_gemm_planned(plan, plan_dev, ws if nb else None)
    # one grouped launch per layer
    cols = sum(p.N for p in PROJS)
    gnb = w4.w4a16_workspace_bytes(M, cols)
    gws = torch.zeros((gnb + 3) // 4, dtype=torch.int32, device="cuda")
    for layer in range(LAYERS):
        sl = slice(4 * layer, 4 * layer + 4)
        w4.w4a16_gemm_grouped([(x, qw, sp, y, N, K) for (x, qw, sp, N, K), y
                               in zip(dev[sl], outs["grouped"][sl])], M, G, gws)
    # one plain call per GEMM
    for (x, qw, sp, N, K), y in zip(dev, outs["plain"]):
        rc = w4._lib.w4a16_gemm(x.data_ptr(), qw.data_ptr(), sp.data_ptr(), y.data_ptr(), M, N, K,
                                G, ctypes.c_void_p(stream))
        assert rc == 0, w4.w4a16_status_string(rc)
    torch.cuda.synchronize()
    if M <= 64:
        rows = np.arange(M)
    else:
        rng = np.random.default_rng(M)
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 62, replace=False)]))
    worst = 0.0
    for i, (x, q, s) in enumerate(host):
        ref = oracle.gemm(x[rows], q, s, G, threads=synth.default_threads())
        for how, ys in outs.items():
            y = ys[i][torch.from_numpy(rows).to("cuda")].view(torch.int16).cpu().numpy()
            r = tolerance_ratio(y.view(np.uint16), ref)
            assert r <= 1.0, f"M={M} GEMM {i} ({PROJS[i % 4].name}) {how}: ratio {r}"
            worst = max(worst, r)
    log(f"tp8 shard M={M}: {len(host)} GEMMs three ways, worst ratio {worst:.3f}")
