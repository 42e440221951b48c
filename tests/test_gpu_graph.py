"""The entry points under HIP graph capture: plain w4a16_gemm calls, a grouped
launch, a planned launch and the no-allocation call are each captured once into
a graph (torch.cuda.CUDAGraph on torch's capture stream, which the library gets
as its stream) and replayed several times. Between replays the program does its
own eager work: the outputs are overwritten with a sentinel, the activations
are redrawn, and an eager call of the same entry point runs on the new inputs.
Every replay must give the same bits as that eager call (the kernels keep no
state between calls except a workspace they leave at zero, and record no
memset node). Shapes: the tensor-parallel shard projections (qkv 5120x896, o
768x5120, gate_up 5120x4352, down 2176x5120), at M = 1 (activations staged in
LDS), 16 (wide units), 64 and 300 (MFMA tile engine; plain calls at 300 take
the one-workgroup-per-tile kernel)."""
import ctypes
import sys

import numpy as np
import pytest

import synth
from gpu_util import dev_u16, dev_u32

pytestmark = pytest.mark.gpu

PROJS = synth.TP8_SHARD_PROJECTIONS
BASE = synth.SHARD_PROJ_BASE
G = synth.GROUP
REPLAYS = 3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import w4a16_weight_only_gemm_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


class Layer:
    """The four shard projections of layer 0 at M rows: packed weights, device
    activations and outputs, and a way to redraw the activations in place."""

    def __init__(self, M):
        import torch

        import w4a16_weight_only_gemm_amd as w4
        self.M = M
        self.w, self.x, self.y = [], [], []
        for pi, p in enumerate(PROJS):
            q = synth.gen_q(synth.tensor_id(synth.KIND_Q, 0, BASE + pi), p.N, p.K)
            s = synth.gen_scales(synth.tensor_id(synth.KIND_SCALES, 0, BASE + pi), p.N, p.K // G)
            qw, sp = w4.w4a16_pack(q, s, G)
            self.w.append((dev_u32(qw), dev_u16(sp)))
            self.x.append(torch.empty((M, p.K), dtype=torch.bfloat16, device="cuda"))
            self.y.append(torch.empty((M, p.N), dtype=torch.bfloat16, device="cuda"))

    def draw(self, seed):
        """New activations in the same buffers (eager copies)."""
        import torch
        for pi, p in enumerate(PROJS):
            xb = synth.gen_x(synth.tensor_id(synth.KIND_X, seed, BASE + pi, self.M), self.M, p.K)
            self.x[pi].view(torch.int16).copy_(torch.from_numpy(xb.view(np.int16)))

    def entries(self):
        return [(x, qw, sp, y, p.N, p.K) for x, (qw, sp), y, p in zip(self.x, self.w, self.y, PROJS)]

    def outputs(self):
        import torch
        torch.cuda.synchronize()
        return [y.view(torch.int16).cpu().numpy().copy() for y in self.y]

    def poison(self):
        for y in self.y:
            y.fill_(float("nan"))


def _callers(layer):
    """Each entry point as a function of the stream handle, with everything it
    needs allocated up front (nothing is allocated during capture)."""
    import torch

    import w4a16_weight_only_gemm_amd as w4
    lib = w4._lib
    M = layer.M
    ents = layer.entries()
    cols = sum(p.N for p in PROJS)
    gnb = w4.w4a16_workspace_bytes(M, cols)
    gws = torch.zeros((gnb + 3) // 4, dtype=torch.int32, device="cuda")
    probs = w4.make_problems(ents)
    pptr = ctypes.cast(probs, ctypes.c_void_p).value
    plan = w4.w4a16_plan_build(ents, M, G)
    plan_dev = torch.from_numpy(plan).to("cuda")
    pnb = w4.w4a16_plan_workspace_bytes(plan)
    pws = torch.zeros(max(1, (pnb + 3) // 4), dtype=torch.int32, device="cuda")

    def plain(stream):
        for (x, qw, sp, y, N, K) in ents:
            rc = lib.w4a16_gemm(x.data_ptr(), qw.data_ptr(), sp.data_ptr(), y.data_ptr(), M, N, K,
                                G, ctypes.c_void_p(stream))
            assert rc == 0, w4.w4a16_status_string(rc)

    def grouped(stream):
        rc = lib.w4a16_gemm_grouped(pptr, len(ents), M, G, gws.data_ptr(), gnb,
                                    ctypes.c_void_p(stream))
        assert rc == 0, w4.w4a16_status_string(rc)

    def planned(stream):
        rc = lib.w4a16_gemm_planned(plan.ctypes.data, plan_dev.data_ptr(), pws.data_ptr(), pnb,
                                    ctypes.c_void_p(stream))
        assert rc == 0, w4.w4a16_status_string(rc)

    def noalloc(stream):
        for (x, qw, sp, y, N, K) in ents:
            rc = lib.w4a16_gemm_noalloc(x.data_ptr(), qw.data_ptr(), sp.data_ptr(), y.data_ptr(), M,
                                        N, K, G, ctypes.c_void_p(stream))
            assert rc == 0, w4.w4a16_status_string(rc)

    keep = (gws, probs, plan, plan_dev, pws)
    return {"plain": plain, "grouped": grouped, "planned": planned, "noalloc": noalloc}, keep


@pytest.mark.parametrize("M", [1, 16, 64, 300])
@pytest.mark.parametrize("kind", ["plain", "grouped", "planned", "noalloc"])
def test_graph_replays_match_eager(kind, M):
    import torch
    layer = Layer(M)
    callers, keep = _callers(layer)
    call = callers[kind]
    layer.draw(100)
    call(torch.cuda.current_stream().cuda_stream)  # eager warm-up (sets up the static scratch)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        layer.draw(101 + r)
        layer.poison()
        call(torch.cuda.current_stream().cuda_stream)  # eager, on the new activations
        eager = layer.outputs()
        layer.poison()
        graph.replay()
        replayed = layer.outputs()
        for pi, (a, b) in enumerate(zip(eager, replayed)):
            assert np.array_equal(a, b), \
                f"{kind} M={M} replay {r}: projection {PROJS[pi].name} differs"
    log(f"graph {kind} M={M}: {REPLAYS} replays bit-identical to eager calls")
    del graph, keep
