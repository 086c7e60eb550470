// plan.hip -- the residency planner (host code only): how many positions of
// each layer stay in device memory, how the tail is tiled for the ring and
// how many slots the ring gets, and what streaming the tail costs.
//
// Steps, in binary64 (the pages' terms):
//  - bw_eff = min(link, host RAM read) ("T*-aware auto rolling-KV spill", T*
//    section and the validation table of measured terms); host_ram_bw <= 0 =
//    unknown, the link alone.
//  - A cache that fits the budget stays resident ("F5 M7 -- Rolling KV",
//    runtime tactic table).
//  - Tile = one layer's compute time x bw_eff x safety, in whole positions
//    (same page, section "Slot pool"); the window takes what the budget holds
//    after two slots (the ping-pong minimum); a layer's tail is cut into at
//    most 63 tiles (one combine merges the window and the tiles), the tile
//    growing until it is; slots = clamp(budget left / tile, 2, 4).
//  - t_resident = (weights + KV) / device bandwidth; drop = (c_engage +
//    tail bytes / bw_eff) / t_resident; T* = (target drop x t_resident -
//    c_engage) x bw_eff; a tail within T* is streamed, a larger one calls for
//    a smaller cache type ("T*-aware auto rolling-KV spill", T* section).
//  - Step time with perfect overlap max(step compute, tail DMA) + c_engage,
//    free zone step compute x bw_eff, hidden fraction min(compute, DMA) / DMA
//    ("Rolling-KV: step/graph-level tail prefetch (design)", section
//    "Bounded win (be honest)").
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "common.h"

namespace {

thread_local std::string g_plan_err;

int plan_fail(const char *msg)
{
    g_plan_err = msg;
    return RKV_E_INVAL;
}

bool pos_finite(double x) { return x > 0.0 && x < INFINITY; }

}  // namespace

extern "C" const char *rkv_plan_last_error(void) { return g_plan_err.c_str(); }

extern "C" int rkv_plan_residency(const rkv_residency_in *in, rkv_residency_plan *out)
{
    if (!in || !out) return plan_fail("NULL argument");
    if (in->n_layers < 1 || in->n_kv < 1 || in->bytes_per_key < 1 || in->kv_budget_bytes < 0 ||
        in->weights_bytes < 0)
        return plan_fail("n_layers, n_kv, bytes_per_key must be >= 1; budget and weights >= 0");
    if (!pos_finite(in->vram_bw) || !pos_finite(in->link_bw) || !(in->host_ram_bw < INFINITY) ||
        !(in->c_engage_s >= 0.0 && in->c_engage_s < INFINITY) || !pos_finite(in->compute_s_per_layer) ||
        !(in->target_drop >= 0.0 && in->target_drop < INFINITY) || !(in->safety > 0.0 && in->safety <= 1.0))
        return plan_fail("bandwidths and compute time must be positive and finite, c_engage and target_drop "
                         ">= 0, safety in (0, 1]");
    const int64_t L = in->n_layers, n = in->n_kv, bpk = in->bytes_per_key, budget = in->kv_budget_bytes;
    if (n > ((int64_t)1 << 40) || bpk > ((int64_t)1 << 30) || L > (1 << 20) || (double)L * n * bpk > 9.0e18)
        return plan_fail("sizes too large");
    rkv_residency_plan p;
    memset(&p, 0, sizeof p);
    const bool ram_binds = in->host_ram_bw > 0.0 && in->host_ram_bw < in->link_bw;
    p.bw_eff = ram_binds ? in->host_ram_bw : in->link_bw;
    p.binding = ram_binds ? RKV_HOST_RAM_BOUND : RKV_LINK_BOUND;
    const int64_t kv_total = L * n * bpk;
    p.t_resident_s = ((double)in->weights_bytes + (double)kv_total) / in->vram_bw;
    p.t_star_bytes = (in->target_drop * p.t_resident_s - in->c_engage_s) * p.bw_eff;
    const double step_compute = (double)L * in->compute_s_per_layer;
    p.free_zone_bytes = step_compute * p.bw_eff;
    if (kv_total <= budget) {
        p.tactic = RKV_RESIDENT;
        p.window_keys = n;
        p.predicted_step_s = step_compute;
        p.predicted_hidden = 1.0;
        *out = p;
        return RKV_OK;
    }
    const double tk = floor(in->compute_s_per_layer * p.bw_eff * in->safety / (double)bpk);
    int64_t tile = tk >= (double)n ? n : (tk < 1.0 ? 1 : (int64_t)tk);
    // the tile only grows and the window only shrinks: a budget that cannot
    // hold two slots of the tile the tail needs is infeasible
    if (2 * tile * bpk > budget) {
        tile = budget / (2 * bpk);
        if (tile < 1) return plan_fail("budget below two ring slots of one position");
    }
    int64_t window = 0, tail = 0;
    for (;;) {
        window = (budget - 2 * tile * bpk) / (L * bpk);
        window = window < 0 ? 0 : window > n ? n : window;
        tail = n - window;
        const int64_t need = (tail + rkv::kMaxParts - 2) / (rkv::kMaxParts - 1);  // tiles per layer <= 63
        if (tile >= need) break;
        tile = need;
        if (2 * tile * bpk > budget) return plan_fail("budget below two ring slots of the tile the tail needs");
    }
    if (tile > tail) tile = tail;
    const int64_t left = (budget - L * window * bpk) / (tile * bpk);
    p.n_slots = (int32_t)(left < 2 ? 2 : left > 4 ? 4 : left);
    p.window_keys = window;
    p.tail_keys = tail;
    p.tile_keys = tile;
    const double tail_bytes = (double)(L * tail * bpk);
    const double dma = tail_bytes / p.bw_eff;
    p.drop = (in->c_engage_s + tail_bytes / p.bw_eff) / p.t_resident_s;
    p.tactic = tail_bytes <= p.t_star_bytes ? RKV_STREAM : RKV_QUANTIZE;
    p.predicted_step_s = (step_compute > dma ? step_compute : dma) + in->c_engage_s;
    p.predicted_hidden = (step_compute < dma ? step_compute : dma) / dma;
    *out = p;
    return RKV_OK;
}
