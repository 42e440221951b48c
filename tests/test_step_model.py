"""The step-time calculator in bench.py (the t_step(B) equation of the
throughput page's "One weight read, shared by every stream" section) against
the worked numbers the pages print (tests/golden/step_model_pins.json), plus
the fit of its two machine parameters to a sweep."""
import json
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "step_model_pins.json")
PINS = json.load(open(GOLDEN))["pins"]
GB = 1e9


def evaluate(fn, a, model=bench.step_time):
    """The quantity a pin names, computed only through the calculator."""
    if fn == "ceiling":
        return bench.ceiling_tokens_per_s(a["bw_gbs"], a["weights_gb"])
    if fn == "fraction":
        return a["measured"] / bench.ceiling_tokens_per_s(a["bw_gbs"], a["weights_gb"])
    if fn == "gib_to_gb":
        return a["gib"] * bench.GIB / GB
    if fn == "kv_bytes":
        return bench.kv_bytes_per_token(a["attn_layers"], a["kv_heads"], a["head_dim"], a["elem_bytes"])
    if fn == "kv_bytes_kib":
        return bench.kv_bytes_per_token(a["attn_layers"], a["kv_heads"], a["head_dim"],
                                        a["elem_bytes"]) / bench.KIB
    if fn == "state_bytes":
        return bench.state_bytes(a["layers"], a["heads"], a["key_dim"], a["value_dim"], a["elem_bytes"])
    if fn == "state_mib":
        return bench.state_bytes(a["layers"], a["heads"], a["key_dim"], a["value_dim"],
                                 a["elem_bytes"]) / bench.MIB
    if fn == "pool_gib":
        return a["streams"] * a["mib_each"] * bench.MIB / bench.GIB
    if fn == "pool_gib_kib":
        return a["streams"] * a["tokens"] * a["kib_each"] * bench.KIB / bench.GIB
    if fn == "weight_ms":
        return model(0, a["weights_gb"] * GB, a["bw_gbs"] * GB) * 1e3
    if fn == "state_ms":
        # one stream's state traffic alone: the step time of B = 1 with no weights
        return model(1, 0.0, a["bw_gbs"] * GB, S=a["state_mib"] * bench.MIB) * 1e3
    if fn == "compute_ms":
        return model(1, 0.0, 1.0, F=a["gflop"] * GB, P=a["tflops"] * 1e12) * 1e3
    if fn == "compute_rows_ms":
        return model(a["rows"], 0.0, 1.0, F=a["gflop"] * GB, P=a["tflops"] * 1e12) * 1e3
    if fn == "tflop":
        return a["rows"] * a["gflop"] / 1e3
    if fn == "bend":
        # smallest stream count whose step is set by arithmetic, found on the
        # model itself by bisection
        kw = dict(eta=a["eta"], S=a["state_mib"] * bench.MIB, F=a["gflop"] * GB, P=a["tflops"] * 1e12)
        W, BW = a["weights_gb"] * GB, a["bw_gbs"] * GB
        lo, hi = 1e-3, 1e5
        for _ in range(200):
            mid = 0.5 * (lo + hi)
            memory_bound = model(mid, W, BW, **kw) > model(mid, W, BW, **{**kw, "F": 0.0})
            lo, hi = (lo, mid) if memory_bound else (mid, hi)
        return hi
    if fn == "aggregate":
        t = model(a["B"], a["weights_gb"] * GB, a["bw_gbs"] * GB, eta=a["eta"],
                  S=a["state_mib"] * bench.MIB, F=a["gflop"] * GB, P=a["tflops"] * 1e12)
        return bench.aggregate_tokens_per_s(a["B"], 1.0, t)
    if fn == "aggregate_gib":
        t = model(a["B"], a["weights_gib"] * bench.GIB, a["bw_gbs"] * GB, eta=a["eta"],
                  S=a["state_mib"] * bench.MIB)
        return bench.aggregate_tokens_per_s(a["B"], 1.0, t)
    if fn == "per_stream":
        return bench.per_stream_tokens_per_s(1.0, a["tpot_ms"] * 1e-3)
    if fn == "step_fraction":
        return (bench.per_stream_tokens_per_s(1.0, a["step_ms"] * 1e-3)
                / bench.ceiling_tokens_per_s(a["bw_gbs"], a["weights_gb"]))
    raise KeyError(fn)


@pytest.mark.parametrize("pin", PINS, ids=[p["id"] for p in PINS])
def test_printed_numbers(pin):
    got = evaluate(pin["fn"], pin["args"])
    assert abs(got - pin["printed"]) <= pin["tol"], (pin["id"], got, pin["printed"])


def _pins_fail(model):
    for pin in PINS:
        try:
            if abs(evaluate(pin["fn"], pin["args"], model) - pin["printed"]) > pin["tol"]:
                return True
        except ZeroDivisionError:
            return True
    return False


# Planted mistakes in the equation; each must fail at least one printed number.
def _state_once(B, W, BW, eta=1.0, S=0.0, kappa=0.0, L=0.0, r=1.0, F=0.0, P=float("inf")):
    return max((W + B * (S + kappa * L)) / (eta * BW), B * r * F / P)


def _eta_on_compute(B, W, BW, eta=1.0, S=0.0, kappa=0.0, L=0.0, r=1.0, F=0.0, P=float("inf")):
    return max((W + B * (2 * S + kappa * L)) / (eta * BW), B * r * F / (eta * P))


def _sum_not_max(B, W, BW, eta=1.0, S=0.0, kappa=0.0, L=0.0, r=1.0, F=0.0, P=float("inf")):
    return (W + B * (2 * S + kappa * L)) / (eta * BW) + B * r * F / P


def _weights_per_stream(B, W, BW, eta=1.0, S=0.0, kappa=0.0, L=0.0, r=1.0, F=0.0, P=float("inf")):
    return max(B * (W + 2 * S + kappa * L) / (eta * BW), B * r * F / P)


@pytest.mark.parametrize("mutant", [_state_once, _eta_on_compute, _sum_not_max, _weights_per_stream],
                         ids=lambda f: f.__name__)
def test_planted_model_mistake_is_caught(mutant):
    assert _pins_fail(mutant), mutant.__name__


def test_terms_and_limits():
    W, BW, F, P = 10e9, 5e12, 2e9, 1e15
    # memory-bound at one stream, compute-bound far past the bend
    assert bench.step_time(1, W, BW, F=F, P=P) == pytest.approx(W / BW)
    assert bench.step_time(1e6, W, BW, F=F, P=P) == pytest.approx(1e6 * F / P)
    b = bench.crossover_streams(W, BW, F, P)
    assert b == pytest.approx(evaluate("bend", dict(weights_gb=W / GB, bw_gbs=BW / GB, state_mib=0,
                                                     gflop=F / GB, tflops=P / 1e12, eta=1.0)))
    assert bench.step_time(b, W, BW, F=F, P=P) == pytest.approx(b * F / P)
    assert bench.step_time(b, W, BW, F=F, P=P) == pytest.approx(W / BW)
    # KV traffic grows the memory term linearly in context
    t1 = bench.step_time(4, W, BW, kappa=1e5, L=1000)
    t2 = bench.step_time(4, W, BW, kappa=1e5, L=2000)
    assert t2 - t1 == pytest.approx(4 * 1e5 * 1000 / BW)
    # speculation: r positions per stream cost arithmetic, tau tokens are kept
    assert bench.step_time(8, 0, BW, r=16, F=F, P=P) == pytest.approx(8 * 16 * F / P)
    assert bench.aggregate_tokens_per_s(8, 4.0, 0.05) == pytest.approx(640.0)
    # a per-stream term at least as costly as its arithmetic never bends
    assert bench.crossover_streams(W, BW, 1.0, 1e15, S=1e9) == float("inf")


def test_fit_recovers_a_known_machine():
    W, BW, a, F = 11e9, 8e12, 2 * 52224 * 64 * 2 / 2, 2 * 335.5e6 * 64
    eta, P = 0.72, 1.3e15
    rows = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024]
    times = [bench.step_time(m, W, BW, eta=eta, S=a / 2, F=F, P=P) for m in rows]
    e, p, bend = bench.fit_step_model(rows, times, W, a, F, BW)
    assert e == pytest.approx(eta) and p == pytest.approx(P)
    assert bench.step_time(bend, W, BW, eta=e, S=a / 2, F=F, P=p) == pytest.approx(bend * F / p)
    # every fitted prediction is at or below the measurement it came from
    for m, t in zip(rows, times):
        assert bench.step_time(m, W, BW, eta=e, S=a / 2, F=F, P=p) <= t * (1 + 1e-12)
