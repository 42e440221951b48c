"""Parity of the full-step sweep workload: the 64-layer stack of the decode layer
set (qkv 5120x7168, o 6144x5120, gate_up 5120x34816, down 17408x5120, group
128; 10.7 GB of packed weights), run at M = 1, 2, 4, ..., 1024 both ways the
benchmark times it -- one planned launch over all 256 GEMMs of a step, and 256
plain w4a16_gemm calls -- with every input drawn from the seeded generator, so
the oracle regenerates any slice of it.

Checked against the oracle, |y - y_ref| <= 1e-2 (1 + |y_ref|):
  * every row of 32 random columns of every (layer, projection, M), both ways;
  * every output of layers 0 and 63 at M = 1, 16 and 1024, both ways.
"""
import functools
import sys

import numpy as np
import pytest

import oracle
import synth
from gpu_util import tolerance_ratio

pytestmark = pytest.mark.gpu

LAYERS = synth.N_LAYERS
G = synth.GROUP
PROJS = synth.LAYER_PROJECTIONS
SWEEP_ROWS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024)
FULL_ROWS = (1, 16, 1024)
FULL_LAYERS = (0, LAYERS - 1)
SAMPLED_COLUMNS = 32


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import w4a16_weight_only_gemm_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


@functools.lru_cache(maxsize=1)
def stack():
    import bench
    log(f"packing the {LAYERS}-layer stack")
    return bench.LayerStore(LAYERS)


@functools.lru_cache(maxsize=1)
def run_stack(M):
    """Both ways of running one step at M rows; returns (host activations,
    planned outputs, plain-call outputs), the outputs as device tensors."""
    import ctypes

    import torch

    import w4a16_weight_only_gemm_amd as w4
    st = stack()
    log(f"stack M={M}: activations")
    xh = [[synth.gen_x(synth.tensor_id(synth.KIND_X, layer, pi, M), M, p.K)
           for pi, p in enumerate(PROJS)] for layer in range(LAYERS)]
    xd = [[torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16) for a in row]
          for row in xh]
    yp = [[torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda") for p in PROJS]
          for _ in range(LAYERS)]
    ys = [[torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda") for p in PROJS]
          for _ in range(LAYERS)]
    entries = [(xd[l][i], st.layers[l][i][0], st.layers[l][i][1], yp[l][i], p.N, p.K)
               for l in range(LAYERS) for i, p in enumerate(PROJS)]
    log(f"stack M={M}: one planned launch over {len(entries)} GEMMs")
    plan = w4.w4a16_plan_build(entries, M, G)
    plan_dev = torch.from_numpy(plan).to("cuda")
    nb = w4.w4a16_plan_workspace_bytes(plan)
    ws = torch.zeros((nb + 3) // 4, dtype=torch.int32, device="cuda")
    w4.w4a16_gemm_planned(plan, plan_dev, ws)
    log(f"stack M={M}: {len(entries)} plain calls")
    lib, stream = w4._lib, torch.cuda.current_stream().cuda_stream
    for l in range(LAYERS):
        for i, p in enumerate(PROJS):
            rc = lib.w4a16_gemm(xd[l][i].data_ptr(), st.layers[l][i][0].data_ptr(),
                                st.layers[l][i][1].data_ptr(), ys[l][i].data_ptr(), M, p.N, p.K,
                                G, ctypes.c_void_p(stream))
            assert rc == 0, w4.w4a16_status_string(rc)
    torch.cuda.synchronize()
    del xd, ws, plan_dev
    return xh, yp, ys


def _columns(t, cols):
    import torch
    idx = torch.from_numpy(cols).to("cuda")
    return t.index_select(1, idx).view(torch.int16).cpu().numpy().view(np.uint16)


def _weights(layer, pi, cols):
    p = PROJS[pi]
    q = np.concatenate([synth.gen_q(synth.tensor_id(synth.KIND_Q, layer, pi), p.N, p.K,
                                    rows=(c, c + 1), threads=1) for c in cols])
    s = np.concatenate([synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, layer, pi), p.N,
                                         p.K // G, rows=(c, c + 1), threads=1) for c in cols])
    return q, s


@pytest.mark.parametrize("M", SWEEP_ROWS)
def test_stack_sampled_columns(M):
    xh, yp, ys = run_stack(M)
    worst = 0.0
    for layer in range(LAYERS):
        for pi, p in enumerate(PROJS):
            rng = np.random.default_rng(1000 * M + 4 * layer + pi)
            cols = np.sort(rng.choice(p.N, SAMPLED_COLUMNS, replace=False))
            q, s = _weights(layer, pi, cols)
            ref = oracle.gemm(xh[layer][pi], q, s, G, threads=synth.default_threads())
            for how, y in (("planned", yp[layer][pi]), ("plain", ys[layer][pi])):
                r = tolerance_ratio(_columns(y, cols), ref)
                assert r <= 1.0, f"M={M} layer {layer} {p.name} {how}: ratio {r}"
                worst = max(worst, r)
    log(f"stack M={M}: sampled columns of {LAYERS * len(PROJS)} GEMMs, worst ratio {worst:.3f}")


@pytest.mark.parametrize("layer", FULL_LAYERS)
@pytest.mark.parametrize("M", FULL_ROWS)
def test_stack_full_layer(M, layer):
    import torch
    xh, yp, ys = run_stack(M)
    for pi, p in enumerate(PROJS):
        q = synth.gen_q(synth.tensor_id(synth.KIND_Q, layer, pi), p.N, p.K)
        s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, layer, pi), p.N, p.K // G)
        ref = oracle.gemm(xh[layer][pi], q, s, G, threads=synth.default_threads())
        for how, y in (("planned", yp[layer][pi]), ("plain", ys[layer][pi])):
            yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
            r = tolerance_ratio(yb, ref)
            log(f"stack M={M} layer {layer} {p.name} {how}: every output, ratio {r:.3f}")
            assert r <= 1.0
