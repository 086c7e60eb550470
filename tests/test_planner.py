"""The residency planner (CPU only).

The plain planner in oracle/planner.py is pinned to the numbers the pages
print (tests/golden/planner_anchors.json: the binding-bandwidth table, the
tolerable spill as the target drop rises, the bounded-win example, the T5
verdict) and to properties that follow from its definitions (a spill of T*
bytes drops exactly the target; budgets, slot and tile limits hold; a cache
that fits stays resident; a tail inside the free zone is hidden).  Planted
mistakes in a copy of it fail a pin.  The library's rkv_plan_residency (host
code, no GPU) must then give the same plan: integers equal, reals within
1e-12 relative.
"""
import json
import math
import os
import types

import numpy as np
import pytest

import position_split_kv_amd as P
from oracle import planner as OP

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "planner_anchors.json")
GB, MiB = 1e9, 1024.0 * 1024.0


def anchors():
    with open(GOLDEN) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- pins of the plain planner

def pin_bw_eff_table(op):
    for row in anchors()["bw_eff"]["rows"]:
        bw, binding = op.binding_bandwidth(row["link_GBps"] * GB, row["host_ram_GBps"] * GB)
        assert bw == row["bw_eff_GBps"] * GB
        assert binding == (op.HOST_RAM_BOUND if row["binding"] == "host_ram" else op.LINK_BOUND)
    assert op.binding_bandwidth(5 * GB, 0.0) == (5 * GB, op.LINK_BOUND)  # unknown host rate


def pin_drop_response(op):
    """T*(d) is affine in the target drop: fit t_resident and c_engage on the
    page's 0.30 and 0.70 points (solidPC link), then 0.02 gives no spill and
    0.99 the printed 235 MiB within the tolerance."""
    a = anchors()["drop_response"]
    bw = a["link_GBps"] * GB
    d1, d2 = a["target_drops"][1], a["target_drops"][2]
    t1, t2 = a["t_star_MiB"][1] * MiB, a["t_star_MiB"][2] * MiB
    t_res = (t2 - t1) / (d2 - d1) / bw
    c = (d1 * t_res * bw - t1) / bw
    assert c > 0 and t_res > 0
    for d, want in zip(a["target_drops"], a["t_star_MiB"]):
        got = op.t_star_bytes(d, t_res, c, bw)
        if want == 0:
            assert got <= 0  # c_engage > d * t_resident: never spill
        else:
            assert abs(got / MiB - want) <= a["tolerance_rel"] * want, (d, got / MiB, want)


def pin_bounded_win(op):
    """Free zone ~90 MiB and a 236 MiB tail taking max(14, DMA) ms, about 28
    tokens/s (not the sum, 14 + DMA)."""
    a = anchors()["bounded_win"]
    bw, comp = a["link_GBps"] * GB, a["step_compute_ms"] * 1e-3
    tail = a["tail_MiB"] * MiB
    tol = a["tolerance_rel"]
    p = op.plan(1, 1 << 20, 4096, 1 << 31, 0, 1e12, bw, 0.0, 0.0, comp, 0.2, 0.8)
    assert abs(p["free_zone"] / MiB - a["free_zone_MiB"]) <= tol * a["free_zone_MiB"]
    step_ms = op.bounded_step(comp, tail, bw, 0.0) * 1e3
    assert abs(step_ms - a["step_ms"]) <= tol * a["step_ms"], step_ms
    assert abs(1e3 / step_ms - a["tps"]) <= tol * a["tps"]
    assert op.hidden_fraction(comp, tail, bw) < 1.0
    # inside the free zone the tail is hidden and the step is the compute
    assert op.hidden_fraction(comp, 0.5 * p["free_zone"], bw) == 1.0
    assert op.bounded_step(comp, 0.5 * p["free_zone"], bw, 0.0) == comp


def pin_t5_verdict(op):
    """A 1630 MiB spill against T* = 14 MiB (bw_eff 10.3 GB/s, c_engage ~1 ms,
    target 0.20) is rejected: the smaller cache type is chosen, and its drop
    is far above the target."""
    a = anchors()["t5_verdict"]
    bw, c = a["bw_eff_GBps"] * GB, a["c_engage_ms"] * 1e-3
    t_res = (a["t_star_MiB"] * MiB / bw + c) / a["target_drop"]
    assert abs(op.t_star_bytes(a["target_drop"], t_res, c, bw) / MiB - a["t_star_MiB"]) < 1e-9
    bpk, L = 1 << 16, 48
    spill = a["spill_MiB"] * MiB
    n_kv = 4096
    budget = L * n_kv * bpk - int(spill)
    kv_total = L * n_kv * bpk
    p = op.plan(L, n_kv, bpk, budget, 0, kv_total / t_res, bw, 0.0, c, 1e-4, a["target_drop"], 0.8)
    assert p["tactic"] == op.QUANTIZE and p["drop"] > a["target_drop"]
    assert abs(p["t_star"] / MiB - a["t_star_MiB"]) < 1e-6


CASES = [
    # n_layers, n_kv, bytes_per_key, budget, weights, vram_bw, link_bw, host_ram_bw, c_engage, compute, drop, safety
    (48, 131072, 1664, 48 * 65536 * 1664 + 3 * 8192 * 1664, 0, 8e12, 57.2e9, 0.0, 17e-6, 227e-6, 0.2, 0.8),
    (48, 65536, 4096, 48 * 65536 * 4096, 28 << 30, 8e12, 57e9, 30e9, 1e-5, 5e-5, 0.2, 0.8),
    (48, 65536, 4096, 40 * 65536 * 4096, 28 << 30, 8e12, 57e9, 30e9, 1e-5, 5e-5, 0.2, 0.8),
    (64, 262144, 2176, 10 << 30, 4 << 30, 5e12, 25e9, 50e9, 2e-4, 1e-4, 0.3, 0.5),
    (1, 1000, 100, 20000, 0, 1e12, 1e9, 0.0, 0.0, 1e-3, 0.2, 0.8),
    (10, 100000, 64, 10 * 99000 * 64, 0, 1e12, 6.7e9, 11.5e9, 8e-4, 2e-6, 0.2, 0.8),
    (2, 5000, 256, 2 * 256, 0, 1e12, 1e9, 0.0, 0.0, 1e-6, 0.2, 0.8),  # two slots of one position
]


def _infeasible(L, n, bpk, budget):
    """No tile fits: even the largest tile two slots of which fit the budget
    is below what a tail of at most 63 tiles per layer needs."""
    t = budget // (2 * bpk)
    if t < 1:
        return True
    w = max(0, min(n, (budget - 2 * t * bpk) // (L * bpk)))
    return math.ceil((n - w) / 63) > t


def pin_plan_invariants(op):
    rng = np.random.default_rng(3)
    cases = list(CASES)
    for _ in range(300):
        L = int(rng.integers(1, 96))
        n = int(rng.integers(1, 1 << 20))
        bpk = int(rng.choice([64, 208, 1088, 1664, 4096]))
        total = L * n * bpk
        budget = int(total * rng.uniform(0.0, 1.3)) + 2 * bpk
        cases.append((L, n, bpk, budget, int(rng.integers(0, 1 << 34)), float(rng.uniform(1e12, 8e12)),
                      float(rng.uniform(5e9, 60e9)), float(rng.choice([0.0, rng.uniform(5e9, 60e9)])),
                      float(rng.uniform(0, 2e-3)), float(rng.uniform(1e-6, 1e-3)), float(rng.uniform(0.01, 1.0)),
                      float(rng.uniform(0.3, 1.0))))
    feasible = 0
    for (L, n, bpk, budget, w, vbw, lbw, hbw, c, comp, drop, safety) in cases:
        try:
            p = op.plan(L, n, bpk, budget, w, vbw, lbw, hbw, c, comp, drop, safety)
        except ValueError:
            assert _infeasible(L, n, bpk, budget)
            continue
        assert not _infeasible(L, n, bpk, budget)
        feasible += 1
        assert p["bw_eff"] == min(lbw, hbw) if hbw > 0 else p["bw_eff"] == lbw
        assert p["window"] + p["tail"] == n
        if L * n * bpk <= budget:
            assert p["tactic"] == op.RESIDENT and p["tail"] == 0 and p["hidden"] == 1.0
            continue
        assert p["tail"] >= 1 and 1 <= p["tile"] <= p["tail"]
        assert 2 <= p["slots"] <= 4
        assert L * p["window"] * bpk + 2 * p["tile"] * bpk <= budget  # window + two slots fit
        if p["slots"] > 2:
            assert L * p["window"] * bpk + p["slots"] * p["tile"] * bpk <= budget
        assert math.ceil(p["tail"] / p["tile"]) <= op.MAX_TILES_PER_LAYER
        # a spill of exactly T* bytes drops exactly the target
        if p["t_star"] > 0:
            assert abs(op.drop_of(p["t_star"], c, p["bw_eff"], p["t_resident"]) - drop) <= 1e-12 * max(1, drop)
        tail_bytes = L * p["tail"] * bpk
        assert (p["tactic"] == op.STREAM) == (tail_bytes <= p["t_star"])
        # bounded win: hidden in the free zone, max not sum
        assert (p["hidden"] == 1.0) == (tail_bytes <= p["free_zone"])
        assert abs(p["step"] - (max(L * comp, tail_bytes / p["bw_eff"]) + c)) <= 1e-12 * p["step"]
    assert feasible >= 200
    # a larger budget never shrinks the window
    L, n, bpk = 48, 65536, 1664
    prev = -1
    for frac in np.linspace(0.05, 1.1, 40):
        p = op.plan(L, n, bpk, int(L * n * bpk * frac), 0, 8e12, 57e9, 0.0, 1e-5, 2e-4)
        assert p["window"] >= prev
        prev = p["window"]


def pin_weights_term(op):
    """The weights term of t_resident ("T*-aware auto rolling-KV spill", T*
    section: t_resident = (W_active + KV_resident) / vram_bw, the per-token
    time with the cache resident).  The pages print no worked value of it, so
    it is pinned by what the definition fixes: T* is affine in the weights
    with slope target_drop * bw_eff / vram_bw (adding dW bytes of weights
    raises T* by exactly that times dW); at a fixed tail the drop falls as the
    weights grow, in the ratio t_resident(W1) / t_resident(W2); a step whose
    weights alone already make 0.20 t_resident exceed c_engage may spill where
    the same cache without weights may not (the page's short-context gate:
    a tiny t_resident means T* <= 0)."""
    L, n, bpk = 48, 16384, 4096
    kv_total = L * n * bpk
    vbw, lbw, c, comp = 1.8e12, 51.2e9, 8.2e-4, 5e-5
    budget = kv_total // 2
    base = op.plan(L, n, bpk, budget, 0, vbw, lbw, 0.0, c, comp, 0.2, 0.8)
    for w in (1 << 30, 15 << 30, 60 << 30):
        p = op.plan(L, n, bpk, budget, w, vbw, lbw, 0.0, c, comp, 0.2, 0.8)
        assert abs(p["t_resident"] - (w + kv_total) / vbw) <= 1e-12 * p["t_resident"]
        slope = (p["t_star"] - base["t_star"]) / w
        assert abs(slope - 0.2 * lbw / vbw) <= 1e-9 * (0.2 * lbw / vbw), (w, slope)
        assert p["drop"] < base["drop"]
        assert abs(p["drop"] / base["drop"] - base["t_resident"] / p["t_resident"]) <= 1e-12
    # short context: no weights -> T* <= 0 (quantize); 15 GiB of weights -> a spill is tolerable
    small = op.plan(L, 256, bpk, L * 128 * bpk, 0, vbw, lbw, 0.0, c, comp, 0.2, 0.8)
    heavy = op.plan(L, 256, bpk, L * 128 * bpk, 15 << 30, vbw, lbw, 0.0, c, comp, 0.2, 0.8)
    assert small["t_star"] <= 0 and small["tactic"] == op.QUANTIZE
    assert heavy["t_star"] > 0


PINS = [pin_bw_eff_table, pin_drop_response, pin_bounded_win, pin_t5_verdict, pin_plan_invariants,
        pin_weights_term]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_planner_pin(pin):
    pin(OP)


PLANNER_MUTANTS = {
    "bw_max": ("if host_ram_bw > 0 and host_ram_bw < link_bw:", "if host_ram_bw > 0 and host_ram_bw > link_bw:"),
    "t_star_no_engage": ("return (target_drop * t_resident - c_engage) * bw_eff",
                         "return (target_drop * t_resident) * bw_eff"),
    "drop_no_engage": ("return (c_engage + tail_bytes / bw_eff) / t_resident", "return (tail_bytes / bw_eff) / t_resident"),
    "one_slot_reserve": ("window = (kv_budget - 2 * tile * bytes_per_key)", "window = (kv_budget - tile * bytes_per_key)"),
    "slots_clamp_8": ("slots = max(2, min(4, left // (tile * bytes_per_key)))",
                      "slots = max(2, min(8, left // (tile * bytes_per_key)))"),
    "step_sum": ("return max(step_compute, dma) + (c_engage", "return (step_compute + dma) + (c_engage"),
    "no_tile_cap": ("        if tile >= need:\n            break", "        if True:\n            break"),
    "stream_wrong_side": ("tactic=STREAM if tail_bytes <= out[\"t_star\"] else QUANTIZE",
                          "tactic=STREAM if tail_bytes >= out[\"t_star\"] else QUANTIZE"),
    "resident_strict": ("if kv_total <= kv_budget:", "if kv_total < kv_budget:"),
    "hidden_inverted": ("return min(step_compute, dma) / dma", "return min(step_compute, dma) / step_compute"),
    "t_resident_no_weights": ("t_resident = (weights_bytes + kv_total) / vram_bw", "t_resident = kv_total / vram_bw"),
    "t_resident_weights_twice": ("t_resident = (weights_bytes + kv_total) / vram_bw",
                                 "t_resident = (2 * weights_bytes + kv_total) / vram_bw"),
}


@pytest.mark.parametrize("name", sorted(PLANNER_MUTANTS))
def test_planner_mutant_is_caught(name):
    old, new = PLANNER_MUTANTS[name]
    src = open(OP.__file__).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    mod = types.ModuleType(f"planner_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    caught = False
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, ZeroDivisionError):
            caught = True
            break
    assert caught, f"mutant {name} passed every pin"


# ----------------------------------------------------------------------------- the library against the oracle

def _library_cases():
    rng = np.random.default_rng(11)
    cases = list(CASES)
    for _ in range(400):
        L = int(rng.integers(1, 96))
        n = int(rng.integers(1, 1 << 20))
        bpk = int(rng.choice([64, 208, 544, 1088, 1664, 4096]))
        total = L * n * bpk
        cases.append((L, n, bpk, int(total * rng.uniform(0.0, 1.3)) + 2 * bpk, int(rng.integers(0, 1 << 34)),
                      float(rng.uniform(1e12, 8e12)), float(rng.uniform(5e9, 60e9)),
                      float(rng.choice([0.0, rng.uniform(5e9, 60e9)])), float(rng.uniform(0, 2e-3)),
                      float(rng.uniform(1e-6, 1e-3)), float(rng.uniform(0.01, 1.0)), float(rng.uniform(0.3, 1.0))))
    return cases


def test_library_plan_equals_oracle():
    keys = [("tactic", "tactic"), ("binding", "binding"), ("window_keys", "window"), ("tail_keys", "tail"),
            ("tile_keys", "tile"), ("n_slots", "slots")]
    reals = [("bw_eff", "bw_eff"), ("t_resident_s", "t_resident"), ("t_star_bytes", "t_star"), ("drop", "drop"),
             ("free_zone_bytes", "free_zone"), ("predicted_step_s", "step"), ("predicted_hidden", "hidden")]
    for case in _library_cases():
        try:
            want = OP.plan(*case)
        except ValueError:
            with pytest.raises(P.RkvError) as e:
                P.rkv_plan_residency(*case)
            assert e.value.code == P.RKV_E_INVAL
            continue
        got = P.rkv_plan_residency(*case)
        for a, b in keys:
            assert got[a] == want[b], (case, a, got[a], want[b])
        for a, b in reals:
            assert abs(got[a] - want[b]) <= 1e-12 * max(1.0, abs(want[b])), (case, a, got[a], want[b])


def test_library_plan_errors():
    good = dict(n_layers=4, n_kv=1000, bytes_per_key=100, kv_budget_bytes=10000, weights_bytes=0, vram_bw=1e12,
                link_bw=1e9, host_ram_bw=0.0, c_engage_s=0.0, compute_s_per_layer=1e-4)
    P.rkv_plan_residency(**good)
    for k, v in [("n_layers", 0), ("n_kv", 0), ("bytes_per_key", 0), ("vram_bw", 0.0), ("link_bw", -1.0),
                 ("compute_s_per_layer", float("inf")), ("c_engage_s", -1.0), ("kv_budget_bytes", 150)]:
        with pytest.raises(P.RkvError) as e:
            P.rkv_plan_residency(**dict(good, **{k: v}))
        assert e.value.code == P.RKV_E_INVAL, k
    with pytest.raises(P.RkvError):
        P.rkv_plan_residency(**good, safety=1.5)
