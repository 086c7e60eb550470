"""Plain residency planner: which positions stay in device memory, how the
tail is tiled and how many ring slots it gets, and what the spill costs.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): the test-suite and
the CPU-baseline leg of ``bench.py`` may use it; the product path never
imports it.  The library's ``rkv_plan_residency`` is checked against it.

Written from the pages, step by step, in binary64:

1. Binding bandwidth ("T*-aware auto rolling-KV spill", T* section and the
   validation table): bw_eff = min(link, host RAM read); the host RAM binds
   when it is the smaller.  An unknown host rate (0) leaves the link alone.
2. Everything fits: the whole cache stays resident ("F5 M7 -- Rolling KV",
   runtime tactic table: a layer that fits is kept hot, zero DMA).
3. Tile size ("F5 M7 -- Rolling KV", section "Slot pool"):
   tile_bytes_max = compute time of one layer x bw_eff x safety 0.8, so a
   tile's copy fits under one layer's compute; here in whole positions.
4. Window: the positions per layer that fit the budget after two slots (the
   ping-pong minimum of the same section); the tail is the rest.  A tail may
   be cut into at most 63 tiles per layer (one combine merges the window and
   at most 63 tiles), so the tile grows until it does, and the window is
   sized again.
5. Slots: n_slots = clamp(budget left / tile bytes, 2, 4) (same section).
6. Drop model (T* section): t_resident = (weights + whole KV) / device memory
   bandwidth; drop(tail) = (c_engage + tail_bytes / bw_eff) / t_resident;
   T* = (target_drop * t_resident - c_engage) * bw_eff, no spill when <= 0.
   A tail within T* is streamed; a larger one is rejected in favour of a
   smaller cache type ("quantize").
7. Bounded win ("Rolling-KV: step/graph-level tail prefetch (design)",
   section "Bounded win (be honest)"): with perfect
   overlap a step takes max(step compute, tail DMA) instead of their sum;
   the free zone is step compute x bandwidth; the hidden fraction of the tail
   DMA is min(step compute, DMA) / DMA.  The fixed engagement cost c_engage
   is added to a step with a tail (the measured first-spill step).

The pages print no worked value of the weights term of t_resident; it is
pinned by what the definition fixes (T* is affine in the weights with slope
target_drop * bw_eff / vram_bw, and the drop falls with the weights in the
ratio of the t_resident values), not by a printed number.
"""
from __future__ import annotations

import math

RESIDENT, STREAM, QUANTIZE = 0, 1, 2
LINK_BOUND, HOST_RAM_BOUND = 0, 1
MAX_TILES_PER_LAYER = 63


def binding_bandwidth(link_bw, host_ram_bw):
    """(bw_eff, binding) of step 1."""
    if host_ram_bw > 0 and host_ram_bw < link_bw:
        return host_ram_bw, HOST_RAM_BOUND
    return link_bw, LINK_BOUND


def t_star_bytes(target_drop, t_resident, c_engage, bw_eff):
    """Tolerable tail bytes of step 6 (<= 0: never spill)."""
    return (target_drop * t_resident - c_engage) * bw_eff


def drop_of(tail_bytes, c_engage, bw_eff, t_resident):
    """Throughput drop of step 6 for a tail of tail_bytes."""
    return (c_engage + tail_bytes / bw_eff) / t_resident


def bounded_step(step_compute, tail_bytes, bw_eff, c_engage):
    """Step time of step 7: max(step compute, tail DMA), plus c_engage when
    there is a tail."""
    dma = tail_bytes / bw_eff
    return max(step_compute, dma) + (c_engage if tail_bytes > 0 else 0.0)


def hidden_fraction(step_compute, tail_bytes, bw_eff):
    """Fraction of the tail DMA hidden under compute (step 7)."""
    dma = tail_bytes / bw_eff
    return min(step_compute, dma) / dma


def plan(n_layers, n_kv, bytes_per_key, kv_budget, weights_bytes, vram_bw, link_bw, host_ram_bw, c_engage,
         compute_per_layer, target_drop=0.20, safety=0.8):
    """The plan as a dict (see the module docstring for the steps)."""
    bw_eff, binding = binding_bandwidth(link_bw, host_ram_bw)
    kv_total = n_layers * n_kv * bytes_per_key
    t_resident = (weights_bytes + kv_total) / vram_bw
    step_compute = n_layers * compute_per_layer
    out = dict(bw_eff=bw_eff, binding=binding, t_resident=t_resident,
               t_star=t_star_bytes(target_drop, t_resident, c_engage, bw_eff),
               free_zone=step_compute * bw_eff)
    if kv_total <= kv_budget:
        out.update(tactic=RESIDENT, window=n_kv, tail=0, tile=0, slots=0, drop=0.0, step=step_compute,
                   hidden=1.0)
        return out
    # step 3: tile of whole positions, at least one
    tile = max(1, int(math.floor(compute_per_layer * bw_eff * safety / bytes_per_key)))
    tile = min(tile, n_kv)
    # step 4: window after two slots; at most 63 tiles per layer (the tile
    # only grows, the window only shrinks: a budget that cannot hold two
    # slots of the tile the tail needs is infeasible)
    if 2 * tile * bytes_per_key > kv_budget:
        tile = kv_budget // (2 * bytes_per_key)
        if tile < 1:
            raise ValueError("budget below two slots of one position")
    while True:
        window = (kv_budget - 2 * tile * bytes_per_key) // (n_layers * bytes_per_key)
        window = max(0, min(n_kv, window))
        tail = n_kv - window
        need = -(-tail // MAX_TILES_PER_LAYER)
        if tile >= need:
            break
        tile = need
        if 2 * tile * bytes_per_key > kv_budget:
            raise ValueError("budget below two slots of the tile the tail needs")
    tile = min(tile, tail)
    # step 5: slots
    left = kv_budget - n_layers * window * bytes_per_key
    slots = max(2, min(4, left // (tile * bytes_per_key)))
    # steps 6 and 7
    tail_bytes = n_layers * tail * bytes_per_key
    out.update(window=window, tail=tail, tile=tile, slots=slots,
               drop=drop_of(tail_bytes, c_engage, bw_eff, t_resident),
               tactic=STREAM if tail_bytes <= out["t_star"] else QUANTIZE,
               step=bounded_step(step_compute, tail_bytes, bw_eff, c_engage),
               hidden=hidden_fraction(step_compute, tail_bytes, bw_eff))
    return out
