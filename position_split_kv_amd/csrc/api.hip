// api.hip -- the C ABI (rkv.h): validation, work planning, and the
// streamed-tail ring.  Every entry point validates its arguments on the host
// before enqueuing anything and reports errors through status codes and a
// thread-local message; nothing here aborts.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <condition_variable>
#include <deque>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "common.h"

using namespace rkv;

// The TBQ3 tier's constants ("F5 M6 -- PolyKV", "S2 -- TurboQuant tier
// family"; the choices are stated in rkv.h).  The codebook: the 8-level
// minimum-MSE quantiser of a unit Gaussian is symmetric, so its positive
// half c_0 < .. < c_3 is the fixed point of Lloyd's two conditions, each
// level the mean of the Gaussian over its cell and each cell boundary the
// midpoint of its two levels; iterated in double from an even spread until
// the levels stop changing.  The signs: bits of splitmix64 (seed 42).
const Tbq3Consts &rkv::tbq3_consts()
{
    static const Tbq3Consts c = [] {
        Tbq3Consts k{};
        auto pdf = [](double x) { return std::isinf(x) ? 0.0 : exp(-0.5 * x * x) * 0.39894228040143267794; };
        auto tail = [](double x) { return std::isinf(x) ? 0.0 : 0.5 * erfc(x * 0.70710678118654752440); };
        double lv[4] = {0.5, 1.0, 1.5, 2.0};
        for (int it = 0; it < 100000; ++it) {
            double edge[5] = {0.0, 0.5 * (lv[0] + lv[1]), 0.5 * (lv[1] + lv[2]), 0.5 * (lv[2] + lv[3]), INFINITY};
            bool same = true;
            double next[4];
            for (int j = 0; j < 4; ++j) {
                next[j] = (pdf(edge[j]) - pdf(edge[j + 1])) / (tail(edge[j]) - tail(edge[j + 1]));
                same = same && next[j] == lv[j];
            }
            for (int j = 0; j < 4; ++j) lv[j] = next[j];
            if (same) break;
        }
        for (int j = 0; j < 4; ++j) k.lv[j] = (float)lv[j];
        uint64_t state = 42, out[4];
        for (int i = 0; i < 4; ++i) {
            state += 0x9e3779b97f4a7c15ull;
            uint64_t z = state;
            z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
            z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
            out[i] = z ^ (z >> 31);
        }
        for (int w = 0; w < 4; ++w) {
            k.s1[w] = (uint32_t)(out[w >> 1] >> (32 * (w & 1)));
            k.s2[w] = (uint32_t)(out[2 + (w >> 1)] >> (32 * (w & 1)));
        }
        return k;
    }();
    return c;
}

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(RKV_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define RKV_HIP(call)                                  \
    do {                                               \
        hipError_t e_ = (call);                        \
        if (e_ != hipSuccess) return hip_fail(e_, #call); \
    } while (0)

// Memory kind of a pointer: 2 device, 1 pinned host, 0 unknown / pageable.
int mem_kind(const void *p)
{
    hipPointerAttribute_t a;
    memset(&a, 0, sizeof a);
    const hipError_t e = hipPointerGetAttributes(&a, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    if (a.type == hipMemoryTypeDevice || a.isManaged) return 2;
    if (a.type == hipMemoryTypeHost) return 1;
    return 0;
}

bool valid_type(int t) { return t >= RKV_F32 && t <= RKV_Q4_0; }   // K, and values
bool valid_v_type(int t) { return valid_type(t) || t == RKV_TBQ3; }  // values only
bool valid_d(int d) { return d == 64 || d == 128 || d == 256 || d == 512; }

int check_desc(const rkv_attn_desc *d)
{
    if (!d) return fail(RKV_E_INVAL, "desc is NULL");
    if (d->n_seq < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1)
        return fail(RKV_E_INVAL, "n_seq, n_q_heads, n_kv_heads must be >= 1");
    if (!valid_d(d->head_dim)) return fail(RKV_E_UNSUPPORTED, "head_dim %d not in {64,128,256,512}", d->head_dim);
    if (d->n_q_heads > 256 || d->n_kv_heads > kMaxKvHeads)
        return fail(RKV_E_UNSUPPORTED, "n_q_heads <= 256 and n_kv_heads <= %d", kMaxKvHeads);
    if ((int64_t)d->n_seq * d->n_q_heads > 65535) return fail(RKV_E_UNSUPPORTED, "n_seq * n_q_heads > 65535");
    if (!(d->scale == d->scale) || !(d->softcap >= 0.f) || d->softcap == INFINITY)
        return fail(RKV_E_INVAL, "scale must be a number and softcap finite >= 0");
    if (d->q_pos && d->n_seq > kMaxMaskSeqs)
        return fail(RKV_E_UNSUPPORTED, "query positions for at most %d sequences", kMaxMaskSeqs);
    if (d->q_to_kv) {
        for (int h = 0; h < d->n_q_heads; ++h)
            if (d->q_to_kv[h] < 0 || d->q_to_kv[h] >= d->n_kv_heads)
                return fail(RKV_E_INVAL, "q_to_kv[%d] = %d out of range", h, d->q_to_kv[h]);
    } else if (d->n_q_heads % d->n_kv_heads) {
        return fail(RKV_E_INVAL, "n_q_heads %% n_kv_heads != 0 needs an explicit q_to_kv");
    }
    return RKV_OK;
}

int kv_of(const rkv_attn_desc *d, int h)
{
    return d->q_to_kv ? d->q_to_kv[h] : h / (d->n_q_heads / d->n_kv_heads);
}

// Host-side checks of a view's fields (no pointer-kind checks).
int check_view_fields(const rkv_attn_desc *d, const rkv_kv_view *v)
{
    if (!v) return fail(RKV_E_INVAL, "view is NULL");
    if (v->k_type == RKV_TBQ3) return fail(RKV_E_UNSUPPORTED, "TBQ3 is a value type (K must be f32, f16, q8_0 or q4_0)");
    if (!valid_type(v->k_type) || !valid_v_type(v->v_type)) return fail(RKV_E_INVAL, "bad K/V type");
    if (v->v_type == RKV_TBQ3 && d->head_dim % 128)
        return fail(RKV_E_UNSUPPORTED, "TBQ3 values need head_dim %% 128 == 0");
    if (v->n_keys < 0) return fail(RKV_E_INVAL, "n_keys < 0");
    if (v->n_keys > ((int64_t)1 << 40)) return fail(RKV_E_UNSUPPORTED, "n_keys too large");
    if (v->pos0 < 0 || v->pos0 > ((int64_t)1 << 40)) return fail(RKV_E_INVAL, "pos0 must be in [0, 2^40]");
    if (v->n_keys == 0) return RKV_OK;
    if (!v->k || !v->v) return fail(RKV_E_INVAL, "K or V pointer is NULL");
    const int D = d->head_dim;
    const int64_t rbk = row_bytes_of(v->k_type, D), rbv = row_bytes_of(v->v_type, D);
    const int64_t wk = load_width_of(v->k_type, D), wv = load_width_of(v->v_type, D);
    if (v->k_pos_stride <= 0 || v->v_pos_stride <= 0 || v->k_head_stride < 0 || v->v_head_stride < 0 ||
        v->k_seq_stride < 0 || v->v_seq_stride < 0)
        return fail(RKV_E_INVAL, "strides must be non-negative (position strides positive)");
    if (v->k_pos_stride > (1 << 24) || v->v_pos_stride > (1 << 24))
        return fail(RKV_E_UNSUPPORTED, "position strides above 16 MiB");
    if ((uintptr_t)v->k % wk || v->k_pos_stride % wk || v->k_head_stride % wk || v->k_seq_stride % wk)
        return fail(RKV_E_INVAL, "K pointer/strides must be multiples of %lld bytes", (long long)wk);
    if ((uintptr_t)v->v % wv || v->v_pos_stride % wv || v->v_head_stride % wv || v->v_seq_stride % wv)
        return fail(RKV_E_INVAL, "V pointer/strides must be multiples of %lld bytes", (long long)wv);
    if (d->n_kv_heads > 1 && (v->k_head_stride < rbk || v->v_head_stride < rbv))
        return fail(RKV_E_INVAL, "head stride smaller than a row");
    const bool k_shared = v->k_seq_stride == 0, v_shared = v->v_seq_stride == 0;
    if (d->n_seq > 1 && k_shared != v_shared)
        return fail(RKV_E_INVAL, "K and V must both be shared (seq stride 0) or both per sequence");
    return RKV_OK;
}

const int kRtSet[] = {1, 2, 4, 5, 8, 16};

// Cut a launch over n segments (same K and V types) into workgroups: row
// groups per KV head, and key splits over all segments together.
int make_plan(const rkv_attn_desc *d, int n, const rkv_kv_view *const *v, SplitPlan *pl, SplitParams *prm)
{
    const int S = d->n_seq, Hq = d->n_q_heads, Hkv = d->n_kv_heads, D = d->head_dim;
    const int kt = v[0]->k_type, vt = v[0]->v_type;
    bool shared = true;
    for (int i = 0; i < n; ++i)
        if (v[i]->n_keys > 0 && (v[i]->k_seq_stride != 0 || v[i]->v_seq_stride != 0)) shared = false;
    shared = shared || S == 1;
    std::vector<std::vector<int>> rows(Hkv);
    for (int b = 0; b < (shared ? S : 1); ++b)
        for (int h = 0; h < Hq; ++h) rows[kv_of(d, h)].push_back(b * Hq + h);
    int rmax = 0;
    for (auto &r : rows) rmax = std::max(rmax, (int)r.size());
    if ((int64_t)rmax * Hkv > kMaxRowTable)
        return fail(RKV_E_UNSUPPORTED, "rows per KV head x KV heads = %d > %d", rmax * Hkv, kMaxRowTable);
    int rt = 16;
    for (int c : kRtSet)
        if (c >= rmax) {
            rt = c;
            break;
        }
    pl->rt = rt;
    pl->n_rg = (rmax + rt - 1) / rt;
    pl->rows_per_g = rmax;
    pl->z = shared ? 1 : S;
    pl->n_rows_total = (int64_t)S * Hq;
    // One round of workgroups: as many as the kernel's occupancy lets every
    // compute unit hold at once (measured on the current device; 2 per unit
    // on 256 units when no device answers, e.g. for a size query on a host
    // without a GPU).  Every segment is cut into splits of the same number of
    // 64-key tiles, a multiple of the waves per KV head.  A workgroup takes
    // as many KV heads (a power of two) as it has waves, so that it reads whole
    // spans of each position's heads; the rest of its waves split the tiles.
    if (d->q_pos)
        for (int i = 0; i < n; ++i)
            if (v[i]->n_keys >= ((int64_t)1 << 30))
                return fail(RKV_E_UNSUPPORTED, "a masked call takes segments of fewer than 2^30 keys");
    int64_t tiles_total = 0;
    for (int i = 0; i < n; ++i) tiles_total += (v[i]->n_keys + kTile - 1) / kTile;
    // With dim slices a head slot is one (KV head, slice) and every wave of a
    // workgroup takes a slot (the slices of a head meet at barriers).
    const int ds = split_dim_slices(kt, vt, D);
    // Several 16-row groups per KV head over block-type K and q4_0 V at
    // head_dim 128: the shared-decode kernel, whose workgroups hold 2 KV heads
    // x 4 row groups that decode each tile once (n_rg then counts blocks of 4
    // row groups).
    pl->shd = ds == 1 && D == 128 && rt == 16 && pl->n_rg >= 2 && split_shd_supported(kt, vt);
    // The same over f16 K and V: the staged-tile kernel, whose workgroups hold
    // one KV head x 4 row groups and stage each tile in LDS once for them.
    pl->rgs = ds == 1 && D == 128 && rt == 16 && pl->n_rg >= 2 && kt == kF16 && vt == kF16;
    const int nw = (pl->shd || pl->rgs) ? 4 : std::max(1, split_waves(kt, vt, D, rt));
    const int slots = Hkv * ds;
    int hpw = 1;
    if (ds > 1 && nw < ds) return fail(RKV_E_UNSUPPORTED, "too few waves per workgroup for %d dim slices", ds);
    // Several row groups of a KV head on the matrix-core path (head_dim 128,
    // no f32 operand): the waves of a head take its row groups, each over all
    // the split's keys, so that one workgroup reads a tile for all of them
    // at once (the copies after the first come from the compute unit's
    // caches) rather than one workgroup per row group each reading it.
    const bool rgw = !pl->shd && !pl->rgs && ds == 1 && D == 128 && kt != kF32 && vt != kF32 && pl->n_rg > 1 && nw >= 2;
    int rg_per_wg = 1;
    if (rgw)
        while (rg_per_wg < pl->n_rg && 2 * rg_per_wg <= nw) rg_per_wg *= 2;
    if (pl->shd || pl->rgs)
        hpw = 1;
    else if (ds > 1)
        hpw = nw;
    else
        while (2 * hpw <= nw / rg_per_wg && 2 * hpw <= slots) hpw *= 2;
    if (pl->shd || pl->rgs) pl->n_rg = (pl->n_rg + 3) / 4;
    if (rgw) pl->n_rg = (pl->n_rg + nw / hpw - 1) / (nw / hpw);
    pl->nw = nw;
    pl->hpw = hpw;
    pl->n_hg = (slots + hpw - 1) / hpw;
    const int64_t wph = (pl->shd || pl->rgs) ? 1 : nw / hpw;
    const int64_t units = (int64_t)pl->n_hg * pl->n_rg * pl->z;
    int occ = pl->shd ? split_shd_occupancy(kt, vt) : pl->rgs ? split_rgs_occupancy() : split_occupancy(kt, vt, D, rt);
    int cus = compute_units();
    if (occ <= 0) occ = 2;
    if (cus <= 0) cus = 256;
    const int64_t want_groups = std::max<int64_t>(1, (int64_t)occ * cus / units);
    int64_t tps = std::max<int64_t>(1, (tiles_total + want_groups - 1) / want_groups);
    if (!rgw) tps = (tps + wph - 1) / wph * wph;  // (row-group waves each walk every tile)
    if (tps * kTile > (1 << 30)) tps = (1 << 30) / kTile;
    int64_t n_splits = 0;
    if (prm) memset(prm, 0, sizeof *prm);
    int ns = 0;
    for (int i = 0; i < n; ++i) {
        const int64_t tiles = (v[i]->n_keys + kTile - 1) / kTile;
        if (tiles == 0) continue;
        if (prm) {
            SegParams &sp = prm->seg[ns];
            sp.k = (const uint8_t *)v[i]->k;
            sp.v = (const uint8_t *)v[i]->v;
            sp.k_pos = v[i]->k_pos_stride;
            sp.v_pos = v[i]->v_pos_stride;
            sp.k_head = v[i]->k_head_stride;
            sp.v_head = v[i]->v_head_stride;
            sp.k_seq = shared ? 0 : v[i]->k_seq_stride;
            sp.v_seq = shared ? 0 : v[i]->v_seq_stride;
            sp.n_keys = v[i]->n_keys;
            sp.pos0 = v[i]->pos0;
            sp.keys_per_split = (int32_t)(tps * kTile);
            sp.split_base = (int32_t)n_splits;
        }
        ++ns;
        n_splits += (tiles + tps - 1) / tps;
    }
    if (n_splits > 65535) return fail(RKV_E_UNSUPPORTED, "segments too long for one launch");
    pl->n_splits = (int)n_splits;
    pl->acc_bytes = n_splits > 1 ? ((size_t)n_splits * pl->n_rows_total * D * sizeof(float) + 255) & ~(size_t)255 : 0;
    pl->ml_bytes = n_splits > 1 ? (size_t)n_splits * pl->n_rows_total * sizeof(float2) : 0;
    pl->ws_bytes = pl->acc_bytes + pl->ml_bytes;
    if (prm) {
        prm->n_segs = ns;
        prm->n_splits = pl->n_splits;
        prm->split_off = 0;
        prm->n_splits_all = pl->n_splits;
        prm->direct = pl->n_splits == 1;
        prm->n_rg = pl->n_rg;
        prm->rows_per_g = rmax;
        prm->n_rows_total = (int32_t)pl->n_rows_total;
        prm->z_row_step = shared ? 0 : Hq;
        prm->scale = d->scale;
        prm->scale_log2 = d->scale * 1.4426950408889634f;
        prm->softcap = d->softcap;
        for (int j = 0; j < 4; ++j) prm->tbq_lv[j] = tbq3_consts().lv[j];
        prm->n_kv_heads = Hkv;
        int hl = 0, wl = 0;
        while ((1 << hl) < hpw) ++hl;
        while ((1 << wl) < wph) ++wl;
        prm->hpw_log2 = hl;
        prm->wph_log2 = wl;
        prm->n_q_heads = Hq;
        prm->masked = d->q_pos != nullptr;
        prm->stream_once = pl->n_rg == 1 && !rgw;  // (with shd / rgs: one block of row groups per head)
        prm->rg_waves = rgw;
        if (d->q_pos)
            for (int b = 0; b < S; ++b)  // (clamped so that position differences stay far from overflow)
                prm->qpos[b] = std::min<int64_t>(std::max<int64_t>(d->q_pos[b], -1), (int64_t)1 << 42);
        for (int g = 0; g < Hkv; ++g) {
            prm->rowcnt[g] = (uint16_t)rows[g].size();
            for (size_t i = 0; i < rows[g].size(); ++i) prm->rowtab[g * rmax + i] = (uint16_t)rows[g][i];
        }
    }
    return RKV_OK;
}

// The non-empty segments of a call, grouped by what one launch of the split
// kernel takes: the same K and V types and the same sequence sharing (kept
// in the caller's order, groups in order of first appearance).
struct SegGroups {
    int n = 0;
    int size[kMaxSegs] = {};
    const rkv_kv_view *v[kMaxSegs][kMaxSegs] = {};
};

void group_segs(const rkv_attn_desc *d, int n, const rkv_kv_view *const *v, SegGroups *g)
{
    bool shared[kMaxSegs];
    for (int i = 0; i < n; ++i) {
        if (v[i]->n_keys == 0) continue;
        const bool sh = d->n_seq == 1 || v[i]->k_seq_stride == 0;
        int j = 0;
        while (j < g->n && !(g->v[j][0]->k_type == v[i]->k_type && g->v[j][0]->v_type == v[i]->v_type &&
                             shared[j] == sh))
            ++j;
        if (j == g->n) shared[g->n++] = sh;
        g->v[j][g->size[j]++] = v[i];
    }
}

// Plans of every launch of a call and the partial workspace they share:
// launch j writes its splits at split_off[j] among n_splits_all partials,
// which one merge reduces.
struct CallPlan {
    SegGroups g;
    SplitPlan pl[kMaxSegs];
    int n_splits_all = 0;
    size_t acc_bytes = 0, ml_bytes = 0, ws_bytes = 0;
};

int make_call_plan(const rkv_attn_desc *d, int n, const rkv_kv_view *const *v, CallPlan *cp, SplitParams *prm)
{
    group_segs(d, n, v, &cp->g);
    int off = 0;
    for (int j = 0; j < cp->g.n; ++j) {
        int rc = make_plan(d, cp->g.size[j], cp->g.v[j], &cp->pl[j], prm ? &prm[j] : nullptr);
        if (rc) return rc;
        if (prm) prm[j].split_off = off;
        off += cp->pl[j].n_splits;
    }
    if (off > 65535) return fail(RKV_E_UNSUPPORTED, "segments too long for one call");
    cp->n_splits_all = off;
    if (prm)
        for (int j = 0; j < cp->g.n; ++j) {
            prm[j].n_splits_all = off;
            prm[j].direct = off == 1;
        }
    const int64_t rows = (int64_t)d->n_seq * d->n_q_heads;
    cp->acc_bytes = off > 1 ? ((size_t)off * rows * d->head_dim * sizeof(float) + 255) & ~(size_t)255 : 0;
    cp->ml_bytes = off > 1 ? (size_t)off * rows * sizeof(float2) : 0;
    cp->ws_bytes = cp->acc_bytes + cp->ml_bytes;
    return RKV_OK;
}

// The split-kernel launches of a call plan (one per group of segments).
int launch_plan(const CallPlan &cp, const SplitParams *prm, const rkv_attn_desc *d, const float *q, float *part_acc,
                float2 *part_ml, float *o, float *lse, hipStream_t stream)
{
    for (int j = 0; j < cp.g.n; ++j) {
        const SplitPlan &pl = cp.pl[j];
        if (!split_supported(cp.g.v[j][0]->k_type, cp.g.v[j][0]->v_type, d->head_dim, pl.rt))
            return fail(RKV_E_UNSUPPORTED, "no kernel for this (type, head_dim, rows)");
        const dim3 grid((unsigned)pl.n_splits, (unsigned)(pl.n_hg * pl.n_rg), (unsigned)pl.z);
        if (pl.rgs)
            RKV_HIP(launch_split_rgs(grid, q, part_acc, part_ml, o, lse, prm[j], stream));
        else if (pl.shd)
            RKV_HIP(launch_split_shd(cp.g.v[j][0]->k_type, cp.g.v[j][0]->v_type, grid, q, part_acc, part_ml, o, lse,
                                     prm[j], stream));
        else
            RKV_HIP(launch_split(cp.g.v[j][0]->k_type, cp.g.v[j][0]->v_type, d->head_dim, pl.rt, grid, q, part_acc,
                                 part_ml, o, lse, prm[j], stream));
    }
    return RKV_OK;
}

// Enqueue the work of one call over up to kMaxSegs segments (arguments already
// validated): one split-kernel launch per group of segments (same K / V types
// and sequence sharing), all writing into one set of per-split partials, then
// one fixed-order merge.  All segments empty: o = 0, lse = -inf.
// phase: 0 the whole call; 1 the split kernels alone (partials in ws, or o /
// lse directly when the call has one split or no keys); 2 the merge alone.
int attend_impl(const rkv_attn_desc *d, const float *q, int n, const rkv_kv_view *const *v, float *o, float *lse,
                void *ws, size_t ws_bytes, hipStream_t stream, int phase = 0)
{
    const int64_t n_rows = (int64_t)d->n_seq * d->n_q_heads;
    int64_t keys = 0;
    for (int i = 0; i < n; ++i) keys += v[i]->n_keys;
    if (keys == 0) {
        if (phase != 2) RKV_HIP(launch_fill_empty(d->head_dim, n_rows, o, lse, stream));
        return RKV_OK;
    }
    CallPlan cp;
    SplitParams prm[kMaxSegs];
    int rc = make_call_plan(d, n, v, &cp, prm);
    if (rc) return rc;
    if (cp.ws_bytes && (ws_bytes < cp.ws_bytes || !ws))
        return fail(RKV_E_INVAL, "workspace too small: %zu < %zu", ws_bytes, cp.ws_bytes);
    for (int j = 0; j < cp.g.n; ++j)
        if (!split_supported(cp.g.v[j][0]->k_type, cp.g.v[j][0]->v_type, d->head_dim, cp.pl[j].rt))
            return fail(RKV_E_UNSUPPORTED, "no kernel for this (type, head_dim, rows)");
    float *part_acc = (float *)ws;
    float2 *part_ml = (float2 *)((char *)ws + cp.acc_bytes);
    // TBQ3 values (then in every segment with keys): the output is summed in
    // the rotated space and turned back by the inverse rotation once final
    bool t3 = false;
    for (int i = 0; i < n; ++i) t3 = t3 || (v[i]->n_keys > 0 && v[i]->v_type == RKV_TBQ3);
    if (phase != 2 && (rc = launch_plan(cp, prm, d, q, part_acc, part_ml, o, lse, stream))) return rc;
    if (cp.n_splits_all == 1) {
        if (t3 && phase != 2) RKV_HIP(launch_unrotate(o, n_rows, d->head_dim, tbq3_consts(), stream));
        return RKV_OK;
    }
    if (phase == 1) return RKV_OK;
    RKV_HIP(launch_reduce(d->head_dim, n_rows, cp.n_splits_all, part_acc, part_ml, o, lse, stream));
    if (t3) RKV_HIP(launch_unrotate(o, n_rows, d->head_dim, tbq3_consts(), stream));
    return RKV_OK;
}

int check_out_args(const float *q, float *o, float *lse)
{
    if (!q || !o || !lse) return fail(RKV_E_INVAL, "q, o and lse must not be NULL");
    if ((uintptr_t)q % 16 || (uintptr_t)o % 16 || (uintptr_t)lse % 4)
        return fail(RKV_E_INVAL, "q and o must be 16-byte aligned, lse 4-byte aligned");
    return RKV_OK;
}

int check_device(const void *p, const char *name)
{
    if (mem_kind(p) != 2) return fail(RKV_E_INVAL, "%s is not device memory", name);
    return RKV_OK;
}

// The segments of one call: each view valid (segments of different types or
// sharing are grouped into separate launches).
int check_segs(const rkv_attn_desc *d, int n, const rkv_kv_view *segs)
{
    if (n < 1 || n > kMaxSegs) return fail(RKV_E_INVAL, "n_segments must be in [1, %d]", kMaxSegs);
    if (!segs) return fail(RKV_E_INVAL, "segments is NULL");
    int rc;
    int n_t3 = 0, n_other = 0;
    for (int i = 0; i < n; ++i) {
        if ((rc = check_view_fields(d, &segs[i]))) return rc;
        if (segs[i].n_keys > 0) (segs[i].v_type == RKV_TBQ3 ? n_t3 : n_other)++;
    }
    // partials over TBQ3 values are in the rotated space, the others are not
    if (n_t3 && n_other)
        return fail(RKV_E_UNSUPPORTED, "TBQ3 values in some segments of a call and not in others");
    return RKV_OK;
}

}  // namespace

extern "C" {

const char *rkv_status_string(int s)
{
    switch (s) {
    case RKV_OK: return "RKV_OK";
    case RKV_E_INVAL: return "RKV_E_INVAL";
    case RKV_E_UNSUPPORTED: return "RKV_E_UNSUPPORTED";
    case RKV_E_HIP: return "RKV_E_HIP";
    case RKV_E_NOMEM: return "RKV_E_NOMEM";
    case RKV_E_STATE: return "RKV_E_STATE";
    default: return "RKV_E_UNKNOWN";
    }
}

const char *rkv_last_error(void) { return g_err.c_str(); }

int64_t rkv_row_bytes(int32_t dtype, int32_t head_dim)
{
    if (!valid_v_type(dtype) || head_dim <= 0) return 0;
    if ((dtype == RKV_Q8_0 || dtype == RKV_Q4_0) && head_dim % 32) return 0;
    if (dtype == RKV_TBQ3 && head_dim % 128) return 0;
    return row_bytes_of(dtype, head_dim);
}

int rkv_attend_split_workspace_bytes(const rkv_attn_desc *desc, int n_segments, const rkv_kv_view *segs,
                                     size_t *bytes)
{
    if (!bytes) return fail(RKV_E_INVAL, "bytes is NULL");
    int rc = check_desc(desc);
    if (rc) return rc;
    if ((rc = check_segs(desc, n_segments, segs))) return rc;
    const rkv_kv_view *vp[kMaxSegs];
    int64_t keys = 0;
    for (int i = 0; i < n_segments; ++i) {
        vp[i] = &segs[i];
        keys += segs[i].n_keys;
    }
    if (keys == 0) {
        *bytes = 0;
        return RKV_OK;
    }
    CallPlan cp;
    rc = make_call_plan(desc, n_segments, vp, &cp, nullptr);
    if (rc) return rc;
    *bytes = cp.ws_bytes;
    return RKV_OK;
}

// rkv_attend_split and its two phases: validation, then the launch (phase as
// for attend_impl; the merge phase reads no query).
static int attend_split_phase(const rkv_attn_desc *desc, const float *q, int n_segments, const rkv_kv_view *segs,
                              float *o, float *lse, void *ws, size_t ws_bytes, hipStream_t stream, int phase)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    if ((rc = check_segs(desc, n_segments, segs))) return rc;
    static const float kDummy[4] __attribute__((aligned(16))) = {};
    if ((rc = check_out_args(phase == 2 ? kDummy : q, o, lse))) return rc;
    if ((phase != 2 && (rc = check_device(q, "q"))) || (rc = check_device(o, "o")) || (rc = check_device(lse, "lse")))
        return rc;
    for (int i = 0; i < n_segments; ++i)
        if (segs[i].n_keys > 0 && ((rc = check_device(segs[i].k, "K")) || (rc = check_device(segs[i].v, "V"))))
            return rc;
    if (ws && (rc = check_device(ws, "workspace"))) return rc;
    const rkv_kv_view *vp[kMaxSegs];
    for (int i = 0; i < n_segments; ++i) vp[i] = &segs[i];
    return attend_impl(desc, q, n_segments, vp, o, lse, ws, ws_bytes, stream, phase);
}

int rkv_attend_split(const rkv_attn_desc *desc, const float *q, int n_segments, const rkv_kv_view *segs, float *o,
                     float *lse, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return attend_split_phase(desc, q, n_segments, segs, o, lse, ws, ws_bytes, stream, 0);
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free attention
//
// rkv_attend_split_noalloc keeps the per-split partials in this fixed device
// array instead of a caller's workspace.  Every GPU the library runs on holds
// its own copy (from module load until the process ends).  In host code the
// name is only a stand-in: the device address of a GPU's copy comes from
// hipGetSymbolAddress with that GPU current, taken once per device and kept.
namespace {
constexpr size_t kScratchBytes = RKV_NOALLOC_MAX_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");
constexpr int kScratchDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
std::atomic<void *> g_scratch_addr[kScratchDevices];

// Device address of the current device's scratch array (looked up once per device).
int scratch_of_current_device(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kScratchDevices) return fail(RKV_E_UNSUPPORTED, "device %d beyond %d", dev, kScratchDevices);
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (scratch)");
            if (!p) return fail(RKV_E_HIP, "hipGetSymbolAddress (scratch) gave NULL");
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return RKV_OK;
}

}  // namespace

extern "C" {

int rkv_attend_split_noalloc(const rkv_attn_desc *desc, const float *q, int n_segments, const rkv_kv_view *segs,
                             float *o, float *lse, hipStream_t stream)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    if ((rc = check_segs(desc, n_segments, segs))) return rc;
    if ((rc = check_out_args(q, o, lse))) return rc;
    if ((rc = check_device(q, "q")) || (rc = check_device(o, "o")) || (rc = check_device(lse, "lse"))) return rc;
    const rkv_kv_view *vp[kMaxSegs];
    int64_t keys = 0;
    for (int i = 0; i < n_segments; ++i) {
        if (segs[i].n_keys > 0 && ((rc = check_device(segs[i].k, "K")) || (rc = check_device(segs[i].v, "V"))))
            return rc;
        vp[i] = &segs[i];
        keys += segs[i].n_keys;
    }
    void *ws = nullptr;
    if (keys > 0) {
        CallPlan cp;
        if ((rc = make_call_plan(desc, n_segments, vp, &cp, nullptr))) return rc;
        if (cp.ws_bytes > kScratchBytes)
            return fail(RKV_E_UNSUPPORTED, "the call needs %zu bytes of partials; the scratch array holds %zu",
                        cp.ws_bytes, kScratchBytes);
        if (cp.ws_bytes > 0 && (rc = scratch_of_current_device(&ws))) return rc;
    }
    return attend_impl(desc, q, n_segments, vp, o, lse, ws, kScratchBytes, stream);
}

int rkv_attend_split_partials(const rkv_attn_desc *desc, const float *q, int n_segments, const rkv_kv_view *segs,
                              float *o, float *lse, void *ws, size_t ws_bytes, hipStream_t stream)
{
    return attend_split_phase(desc, q, n_segments, segs, o, lse, ws, ws_bytes, stream, 1);
}

int rkv_attend_split_merge(const rkv_attn_desc *desc, int n_segments, const rkv_kv_view *segs, float *o, float *lse,
                           void *ws, size_t ws_bytes, hipStream_t stream)
{
    return attend_split_phase(desc, nullptr, n_segments, segs, o, lse, ws, ws_bytes, stream, 2);
}

int rkv_attend_workspace_bytes(const rkv_attn_desc *desc, const rkv_kv_view *seg, size_t *bytes)
{
    return rkv_attend_split_workspace_bytes(desc, 1, seg, bytes);
}

int rkv_attend_segment(const rkv_attn_desc *desc, const float *q, const rkv_kv_view *seg, float *o, float *lse,
                       void *ws, size_t ws_bytes, hipStream_t stream)
{
    return rkv_attend_split(desc, q, 1, seg, o, lse, ws, ws_bytes, stream);
}

int rkv_lse_combine(int n_parts, const float *const *o_parts, const float *const *lse_parts, int64_t n_rows,
                    int32_t head_dim, float *o_out, float *lse_out, hipStream_t stream)
{
    if (n_parts < 1 || n_parts > kMaxParts) return fail(RKV_E_INVAL, "n_parts must be in [1, %d]", kMaxParts);
    if (!o_parts || !lse_parts || !o_out || !lse_out) return fail(RKV_E_INVAL, "NULL argument");
    if (n_rows < 0 || n_rows > 0x7fffffff) return fail(RKV_E_INVAL, "bad n_rows");
    if (head_dim < 1 || head_dim > 4096) return fail(RKV_E_INVAL, "bad head_dim");
    CombineParts parts;
    memset(&parts, 0, sizeof parts);
    for (int t = 0; t < n_parts; ++t) {
        if (!o_parts[t] || !lse_parts[t]) return fail(RKV_E_INVAL, "part %d is NULL", t);
        parts.o[t] = o_parts[t];
        parts.lse[t] = lse_parts[t];
    }
    if (n_rows == 0) return RKV_OK;
    int rc;
    for (int t = 0; t < n_parts; ++t)
        if ((rc = check_device(parts.o[t], "o_parts[t]")) || (rc = check_device(parts.lse[t], "lse_parts[t]")))
            return rc;
    if ((rc = check_device(o_out, "o_out")) || (rc = check_device(lse_out, "lse_out"))) return rc;
    RKV_HIP(launch_combine(n_parts, parts, n_rows, head_dim, o_out, lse_out, stream));
    return RKV_OK;
}

static int dequant_common(const void *blocks, int64_t n, float *out)
{
    if (n < 0 || n % 32) return fail(RKV_E_INVAL, "n_values must be a non-negative multiple of 32");
    if (n == 0) return RKV_OK;
    if (!blocks || !out) return fail(RKV_E_INVAL, "NULL argument");
    int rc;
    if ((rc = check_device(blocks, "blocks")) || (rc = check_device(out, "out"))) return rc;
    return RKV_OK;
}

int rkv_dequant_q8_0(const void *blocks, int64_t n_values, float *out, hipStream_t stream)
{
    int rc = dequant_common(blocks, n_values, out);
    if (rc || n_values == 0) return rc;
    RKV_HIP(launch_dequant_q8_0(blocks, n_values, out, stream));
    return RKV_OK;
}

int rkv_dequant_q4_0(const void *blocks, int64_t n_values, float *out, hipStream_t stream)
{
    int rc = dequant_common(blocks, n_values, out);
    if (rc || n_values == 0) return rc;
    RKV_HIP(launch_dequant_q4_0(blocks, n_values, out, stream));
    return RKV_OK;
}

int rkv_dequant_tbq3(const void *blocks, int64_t n_values, float *out, hipStream_t stream)
{
    if (n_values < 0 || n_values % 128) return fail(RKV_E_INVAL, "n_values must be a non-negative multiple of 128");
    int rc = dequant_common(blocks, n_values, out);
    if (rc || n_values == 0) return rc;
    if (n_values / 128 > 0x7fffffff) return fail(RKV_E_UNSUPPORTED, "too many blocks");
    RKV_HIP(launch_dequant_tbq3(blocks, n_values, out, tbq3_consts(), stream));
    return RKV_OK;
}

// ---------------------------------------------------------------- ring

int64_t rkv_ring_schedule(int n_layers, const int64_t *tiles_per_layer, int n_slots, int64_t max_items,
                          int32_t *layer_of, int64_t *tile_of, int32_t *slot_of, int64_t *waits_on)
{
    if (n_layers < 0 || (n_layers > 0 && !tiles_per_layer)) return fail(RKV_E_INVAL, "bad layers");
    if (n_slots < 2 || n_slots > 16) return fail(RKV_E_INVAL, "n_slots must be in [2, 16]");
    int64_t j = 0;
    for (int l = 0; l < n_layers; ++l) {
        if (tiles_per_layer[l] < 0) return fail(RKV_E_INVAL, "negative tile count");
        for (int64_t t = 0; t < tiles_per_layer[l]; ++t, ++j) {
            if (j >= max_items) continue;
            if (layer_of) layer_of[j] = l;
            if (tile_of) tile_of[j] = t;
            if (slot_of) slot_of[j] = (int32_t)(j % n_slots);
            if (waits_on) waits_on[j] = j >= n_slots ? j - n_slots : -1;
        }
    }
    return j;
}

}  // extern "C"

struct rkv_ring {
    int B = 0;
    int device = 0;
    size_t slot_k = 0, slot_v = 0;
    void *sk[16] = {}, *sv[16] = {};
    hipStream_t copy = nullptr;
    bool own_copy = false;
    hipEvent_t copy_done[16] = {};
    // Slot release: the kernel after a tile's attention kernel (the layer's
    // next tile or its merge; it starts only once the tile's kernel has read
    // the slot) writes the tile's sequence number + 1 to progress[slot],
    // pinned and coherent host memory.  A slot's
    // tiles run one after another (each waits for its copy, which waits for
    // the previous tile of the slot), so each word only grows, whatever
    // streams the tiles run on.  last_user[s]: sequence number of the tile that
    // last read slot s (-1: none); written by the caller's thread under mu.
    uint64_t *progress = nullptr;
    int64_t last_user[16];
    // Rows appended to a layer's tail by rkv_append_kv naming this ring: a
    // kernel after the append writes the layer's append count to
    // written[layer] (pinned, coherent host memory) once the rows are stored,
    // and the copies of that layer in steps begun later wait for it.
    // appends[layer]: appends issued so far (the caller's thread).
    uint64_t *written = nullptr;
    int64_t appends[kRingMaxLayers] = {};
    // plan of the current step
    bool in_step = false;
    std::vector<rkv_kv_view> tails;
    std::vector<char> inplace;  // per layer: the tail is in device memory and is attended where it is
    int64_t tile_keys = 0;
    struct Item {
        int layer;
        int64_t k0, nk;
        int64_t need_w;  // written[layer] must reach this before the copy (appends issued before the step)
    };
    std::vector<Item> items;
    std::vector<int64_t> first_item;  // per layer, plus end
    int next_layer = 0;
    int64_t base = 0;  // sequence number of the step's item 0 (items of all steps are numbered in order)
    // The copier thread: for each requested item it waits on the host for the
    // compute that last read the item's slot, then enqueues the slot's copy
    // and its copy_done record (see enqueue_copy).
    std::thread copier;
    std::mutex mu;
    std::condition_variable cv_req, cv_done;
    std::deque<std::pair<int64_t, int64_t>> req;  // (item index in the step, sequence number the slot must reach)
    int64_t enq[16];               // sequence number of the item whose copy slot s holds or receives
    bool busy = false, stop = false;
    hipError_t err = hipSuccess;   // first failure of the copier
    const char *err_what = "";
};

namespace {

// Wait on the host until a host-visible word written by a kernel reaches
// need (spin briefly, since a tile takes tens of microseconds, then yield).
// false after 60 s.
bool wait_word(const uint64_t *w, int64_t need)
{
    if (need <= 0 || __atomic_load_n(w, __ATOMIC_ACQUIRE) >= (uint64_t)need) return true;
    const auto t0 = std::chrono::steady_clock::now();
    unsigned spins = 0;
    while (__atomic_load_n(w, __ATOMIC_ACQUIRE) < (uint64_t)need) {
        if (++spins < 4096)
            __builtin_ia32_pause();
        else
            std::this_thread::yield();
        if (spins % 1024 == 0 && std::chrono::steady_clock::now() - t0 > std::chrono::seconds(60)) return false;
    }
    return true;
}

// Enqueue the copy of item j (index in the step) into its slot, on the copy
// stream, once the compute that last read the slot has finished: the copier
// waits for that on the host, watching the ring's progress word (the kernel
// after that tile's attention kernel writes it).  A DMA-engine copy made to
// wait on a compute-queue event on the GPU costs tens of microseconds per copy
// even when the event has long completed, and an event record on the compute
// queue costs it a few microseconds per tile; this way the copy goes out with
// no GPU-side dependency and the compute queue records nothing.
hipError_t enqueue_copy(rkv_ring *r, int64_t j, int64_t need, const char **what)
{
    const rkv_ring::Item &it = r->items[j];
    const rkv_kv_view &t = r->tails[it.layer];
    const int s = (int)(j % r->B);
    const size_t kb = (size_t)(it.nk * t.k_pos_stride), vb = (size_t)(it.nk * t.v_pos_stride);
    hipError_t e;
    if (!wait_word(r->progress + s, need)) {
        *what = "slot release: the compute that last read the slot did not finish within 60 s";
        return hipErrorLaunchTimeOut;
    }
    if (!wait_word(r->written + it.layer, it.need_w)) {
        *what = "tail rows: an append to the layer's tail did not finish within 60 s";
        return hipErrorLaunchTimeOut;
    }
    *what = "hipMemcpyAsync (tile K)";
    if ((e = hipMemcpyAsync(r->sk[s], (const char *)t.k + it.k0 * t.k_pos_stride, kb, hipMemcpyHostToDevice,
                            r->copy)) != hipSuccess)
        return e;
    *what = "hipMemcpyAsync (tile V)";
    if ((e = hipMemcpyAsync(r->sv[s], (const char *)t.v + it.k0 * t.v_pos_stride, vb, hipMemcpyHostToDevice,
                            r->copy)) != hipSuccess)
        return e;
    *what = "hipEventRecord (copy_done)";
    return hipEventRecord(r->copy_done[s], r->copy);
}

void copier_main(rkv_ring *r)
{
    (void)hipSetDevice(r->device);
    std::unique_lock<std::mutex> lk(r->mu);
    for (;;) {
        r->cv_req.wait(lk, [r] { return r->stop || !r->req.empty(); });
        if (r->stop) return;
        const int64_t j = r->req.front().first, need = r->req.front().second;
        r->req.pop_front();
        r->busy = true;
        lk.unlock();
        const char *what = "";
        hipError_t e = r->err == hipSuccess ? enqueue_copy(r, j, need, &what) : hipSuccess;
        lk.lock();
        if (e != hipSuccess && r->err == hipSuccess) {
            r->err = e;
            r->err_what = what;
        }
        r->enq[j % r->B] = r->base + j;  // also on failure: the waiter then sees the error
        r->busy = false;
        r->cv_done.notify_all();
    }
}

// Hand item j (index in the step) to the copier; its copy waits until the
// tile that last read its slot has finished (progress > that tile's number).
void request_copy(rkv_ring *r, int64_t j)
{
    {
        std::lock_guard<std::mutex> lk(r->mu);
        r->req.emplace_back(j, r->last_user[j % r->B] + 1);
    }
    r->cv_req.notify_one();
}

// Wait (on the host) until the copy of item j and its copy_done record are
// enqueued.  Returns the copier's failure, if any.
int wait_enqueued(rkv_ring *r, int64_t j)
{
    std::unique_lock<std::mutex> lk(r->mu);
    r->cv_done.wait(lk, [r, j] { return r->err != hipSuccess || r->enq[j % r->B] == r->base + j; });
    if (r->err != hipSuccess) return hip_fail(r->err, r->err_what);
    return RKV_OK;
}

void copier_stop(rkv_ring *r)
{
    if (!r->copier.joinable()) return;
    {
        std::lock_guard<std::mutex> lk(r->mu);
        r->stop = true;
    }
    r->cv_req.notify_all();
    r->copier.join();
}

void ring_free(rkv_ring *r)
{
    copier_stop(r);
    for (int i = 0; i < 16; ++i) {
        if (r->sk[i]) (void)hipFree(r->sk[i]);
        if (r->sv[i]) (void)hipFree(r->sv[i]);
        if (r->copy_done[i]) (void)hipEventDestroy(r->copy_done[i]);
    }
    if (r->progress) (void)hipHostFree(r->progress);
    if (r->written) (void)hipHostFree(r->written);
    if (r->own_copy && r->copy) (void)hipStreamDestroy(r->copy);
    delete r;
}

// The tiles of a layer's tail in the current step: how many, and tile t's
// view -- the ring slot it is copied into (streamed tails; planning only
// needs the sizes, so slot 0 stands in for a slot not yet known) or the tail
// itself at the tile's keys (a tail in device memory, attended in place).
// The sequence strides are 0: a tail is shared by all sequences or n_seq == 1.
int64_t layer_tiles(const rkv_ring *r, int layer)
{
    if (r->inplace[layer]) return (r->tails[layer].n_keys + r->tile_keys - 1) / r->tile_keys;
    return r->first_item[layer + 1] - r->first_item[layer];
}

rkv_kv_view tile_view(const rkv_ring *r, int layer, int64_t t, int slot)
{
    const rkv_kv_view &tail = r->tails[layer];
    rkv_kv_view v = tail;
    const int64_t k0 = t * r->tile_keys;
    v.n_keys = std::min(r->tile_keys, tail.n_keys - k0);
    v.pos0 = tail.pos0 + k0;
    if (r->inplace[layer]) {
        v.k = (const char *)tail.k + k0 * tail.k_pos_stride;
        v.v = (const char *)tail.v + k0 * tail.v_pos_stride;
    } else {
        v.k = r->sk[slot];
        v.v = r->sv[slot];
    }
    v.k_seq_stride = 0;
    v.v_seq_stride = 0;
    return v;
}

// Partials of a layer's tail: every tile's key splits, one set of per-split
// partials for the whole layer (tile t's splits at offset off[t]); total
// splits, and the workspace bytes they take.
int layer_tail_plan(const rkv_ring *r, int layer, const rkv_attn_desc *d, std::vector<int> *off, int *total,
                    size_t *acc_bytes, size_t *bytes)
{
    const int64_t nt = layer_tiles(r, layer);
    off->assign((size_t)nt + 1, 0);
    int64_t tot = 0;
    for (int64_t t = 0; t < nt; ++t) {
        const rkv_kv_view v = tile_view(r, layer, t, 0);
        const rkv_kv_view *vp = &v;
        CallPlan cp;
        int rc = make_call_plan(d, 1, &vp, &cp, nullptr);
        if (rc) return rc;
        (*off)[t] = (int)tot;
        tot += cp.n_splits_all;
        if (tot > 65535) return fail(RKV_E_UNSUPPORTED, "layer %d: tail tiles need more than 65535 splits", layer);
    }
    (*off)[nt] = (int)tot;
    const int64_t rows = (int64_t)d->n_seq * d->n_q_heads;
    *total = (int)tot;
    *acc_bytes = ((size_t)tot * rows * d->head_dim * sizeof(float) + 255) & ~(size_t)255;
    *bytes = *acc_bytes + (size_t)tot * rows * sizeof(float2);
    return RKV_OK;
}

}  // namespace

extern "C" {

int rkv_ring_create(int n_slots, size_t slot_k_bytes, size_t slot_v_bytes, hipStream_t copy_stream, rkv_ring **out)
{
    if (!out) return fail(RKV_E_INVAL, "out is NULL");
    *out = nullptr;
    if (n_slots < 2 || n_slots > 16) return fail(RKV_E_INVAL, "n_slots must be in [2, 16]");
    if (slot_k_bytes == 0 || slot_v_bytes == 0) return fail(RKV_E_INVAL, "slot sizes must be > 0");
    rkv_ring *r = new (std::nothrow) rkv_ring;
    if (!r) return fail(RKV_E_NOMEM, "host allocation failed");
    r->B = n_slots;
    r->slot_k = slot_k_bytes;
    r->slot_v = slot_v_bytes;
    hipError_t e = hipGetDevice(&r->device);
    if (e != hipSuccess) {
        ring_free(r);
        return hip_fail(e, "hipGetDevice");
    }
    for (int i = 0; i < n_slots; ++i) {
        if (hipMalloc(&r->sk[i], slot_k_bytes) != hipSuccess || hipMalloc(&r->sv[i], slot_v_bytes) != hipSuccess) {
            (void)hipGetLastError();
            ring_free(r);
            return fail(RKV_E_NOMEM, "slot allocation failed");
        }
        if ((e = hipEventCreateWithFlags(&r->copy_done[i], hipEventDisableTiming)) != hipSuccess) {
            ring_free(r);
            return hip_fail(e, "hipEventCreateWithFlags");
        }
    }
    if ((e = hipHostMalloc((void **)&r->progress, 16 * sizeof(uint64_t), hipHostMallocCoherent)) != hipSuccess) {
        r->progress = nullptr;
        ring_free(r);
        return hip_fail(e, "hipHostMalloc (progress)");
    }
    if ((e = hipHostMalloc((void **)&r->written, kRingMaxLayers * sizeof(uint64_t), hipHostMallocCoherent)) !=
        hipSuccess) {
        r->written = nullptr;
        ring_free(r);
        return hip_fail(e, "hipHostMalloc (written)");
    }
    for (int i = 0; i < kRingMaxLayers; ++i) __atomic_store_n(r->written + i, (uint64_t)0, __ATOMIC_RELEASE);
    for (int i = 0; i < 16; ++i) {
        __atomic_store_n(r->progress + i, (uint64_t)0, __ATOMIC_RELEASE);
        r->last_user[i] = -1;
    }
    if (copy_stream) {
        r->copy = copy_stream;
    } else {
        if ((e = hipStreamCreateWithFlags(&r->copy, hipStreamNonBlocking)) != hipSuccess) {
            r->copy = nullptr;
            ring_free(r);
            return hip_fail(e, "hipStreamCreateWithFlags");
        }
        r->own_copy = true;
    }
    for (int i = 0; i < 16; ++i) r->enq[i] = -1;
    try {
        r->copier = std::thread(copier_main, r);
    } catch (...) {
        ring_free(r);
        return fail(RKV_E_NOMEM, "could not start the copier thread");
    }
    *out = r;
    return RKV_OK;
}

int rkv_ring_destroy(rkv_ring *r)
{
    if (!r) return RKV_OK;
    copier_stop(r);
    hipError_t e = hipStreamSynchronize(r->copy);
    // the slots are freed only after the last tile of each has been read
    const auto t0 = std::chrono::steady_clock::now();
    // (and the signals of appends that name the ring have been written: they
    // write into the ring's memory)
    auto reached = [&](const uint64_t *w, int64_t need) {
        while (__atomic_load_n(w, __ATOMIC_ACQUIRE) < (uint64_t)need) {
            std::this_thread::sleep_for(std::chrono::microseconds(50));
            if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(60)) return false;
        }
        return true;
    };
    for (int i = 0; i < r->B && e == hipSuccess; ++i)
        if (!reached(r->progress + i, r->last_user[i] + 1)) e = hipErrorLaunchTimeOut;
    for (int l = 0; l < kRingMaxLayers && e == hipSuccess; ++l)
        if (!reached(r->written + l, r->appends[l])) e = hipErrorLaunchTimeOut;
    ring_free(r);
    if (e != hipSuccess) return hip_fail(e, "ring destroy synchronisation");
    return RKV_OK;
}

int rkv_ring_begin_step(rkv_ring *r, int n_layers, const rkv_kv_view *tails, int64_t tile_keys)
{
    if (!r) return fail(RKV_E_INVAL, "ring is NULL");
    if (r->in_step) return fail(RKV_E_STATE, "previous step not ended");
    if (n_layers < 0 || (n_layers > 0 && !tails)) return fail(RKV_E_INVAL, "bad layers");
    if (n_layers > kRingMaxLayers) return fail(RKV_E_UNSUPPORTED, "more than %d layers", kRingMaxLayers);
    if (tile_keys < 1) return fail(RKV_E_INVAL, "tile_keys must be >= 1");
    std::vector<rkv_ring::Item> items;
    std::vector<int64_t> first(n_layers + 1, 0);
    std::vector<char> inplace(n_layers, 0);
    for (int l = 0; l < n_layers; ++l) {
        const rkv_kv_view &t = tails[l];
        first[l] = (int64_t)items.size();
        if (t.n_keys < 0) return fail(RKV_E_INVAL, "tail %d: n_keys < 0", l);
        if (t.n_keys == 0) continue;
        if (!t.k || !t.v || t.k_pos_stride <= 0 || t.v_pos_stride <= 0)
            return fail(RKV_E_INVAL, "tail %d: bad pointers or strides", l);
        // (its partials would be in the rotated space, the window's result is not)
        if (t.v_type == RKV_TBQ3) return fail(RKV_E_UNSUPPORTED, "tail %d: TBQ3 values cannot be streamed", l);
        if ((t.n_keys + tile_keys - 1) / tile_keys > kMaxParts - 1)
            return fail(RKV_E_UNSUPPORTED, "tail %d: more than %d tiles", l, kMaxParts - 1);
        const int mk = mem_kind(t.k), mv = mem_kind(t.v);
        if (mk == 2 && mv == 2) {  // device memory: attended in place, no copies
            inplace[l] = 1;
            continue;
        }
        if (mk != 1 || mv != 1)
            return fail(RKV_E_INVAL, "tail %d must be pinned host memory (or device memory, attended in place)", l);
        if ((size_t)(std::min(tile_keys, t.n_keys) * t.k_pos_stride) > r->slot_k ||
            (size_t)(std::min(tile_keys, t.n_keys) * t.v_pos_stride) > r->slot_v)
            return fail(RKV_E_INVAL, "tail %d: a tile does not fit a slot", l);
        for (int64_t k0 = 0; k0 < t.n_keys; k0 += tile_keys)
            items.push_back({l, k0, std::min(tile_keys, t.n_keys - k0), r->appends[l]});
    }
    first[n_layers] = (int64_t)items.size();
    {
        // the copier is idle between steps (every item of a finished step had
        // its copy enqueued before it was consumed; an aborted step's requests
        // drain here)
        std::unique_lock<std::mutex> lk(r->mu);
        r->cv_done.wait(lk, [r] { return r->req.empty() && !r->busy; });
        if (r->err != hipSuccess) return hip_fail(r->err, r->err_what);
        r->base += (int64_t)r->items.size();
        r->tails.assign(tails, tails + n_layers);
        r->inplace.swap(inplace);
        r->items.swap(items);
        r->first_item.swap(first);
    }
    r->tile_keys = tile_keys;
    r->next_layer = 0;
    r->in_step = true;
    const int64_t n = std::min<int64_t>(r->B, (int64_t)r->items.size());
    for (int64_t j = 0; j < n; ++j) request_copy(r, j);
    return RKV_OK;
}

int rkv_stream_tail_workspace_bytes(const rkv_ring *r, int layer, const rkv_attn_desc *desc, size_t *bytes)
{
    if (!r || !bytes) return fail(RKV_E_INVAL, "NULL argument");
    if (!r->in_step) return fail(RKV_E_STATE, "no step begun");
    if (layer < 0 || layer >= (int)r->tails.size()) return fail(RKV_E_INVAL, "layer out of range");
    int rc = check_desc(desc);
    if (rc) return rc;
    if (layer_tiles(r, layer) > 0) {
        if ((rc = check_view_fields(desc, &r->tails[layer]))) return rc;
    }
    std::vector<int> off;
    int total = 0;
    size_t acc = 0;
    return layer_tail_plan(r, layer, desc, &off, &total, &acc, bytes);
}

int rkv_stream_tail(rkv_ring *r, int layer, const rkv_attn_desc *desc, const float *q, const float *o_window,
                    const float *lse_window, float *o, float *lse, void *ws, size_t ws_bytes, hipStream_t cs)
{
    if (!r) return fail(RKV_E_INVAL, "ring is NULL");
    if (!r->in_step) return fail(RKV_E_STATE, "no step begun");
    if (layer != r->next_layer) return fail(RKV_E_STATE, "layer %d consumed out of order (next is %d)", layer, r->next_layer);
    int rc = check_desc(desc);
    if (rc) return rc;
    if (!q || !o || !lse) return fail(RKV_E_INVAL, "q, o and lse must not be NULL");
    if (lse_window && !o_window) return fail(RKV_E_INVAL, "o_window is NULL");
    const int D = desc->head_dim;
    const int64_t n_rows = (int64_t)desc->n_seq * desc->n_q_heads;
    const int64_t j0 = r->first_item[layer];
    const int64_t n_tiles = layer_tiles(r, layer);
    const rkv_kv_view &tail = r->tails[layer];
    if (n_tiles > 0) {
        if (desc->n_seq > 1 && (tail.k_seq_stride != 0 || tail.v_seq_stride != 0))
            return fail(RKV_E_UNSUPPORTED, "a streamed tail must be shared by all sequences or n_seq == 1");
        const int64_t rbk = row_bytes_of(tail.k_type, D), rbv = row_bytes_of(tail.v_type, D);
        if ((desc->n_kv_heads - 1) * tail.k_head_stride + rbk > tail.k_pos_stride ||
            (desc->n_kv_heads - 1) * tail.v_head_stride + rbv > tail.v_pos_stride)
            return fail(RKV_E_INVAL, "tail rows of one position must fit in its position stride");
    }
    size_t need = 0;
    if ((rc = rkv_stream_tail_workspace_bytes(r, layer, desc, &need))) return rc;
    if (!ws || ws_bytes < need) return fail(RKV_E_INVAL, "workspace too small: %zu < %zu", ws_bytes, need);
    if ((rc = check_device(q, "q")) || (rc = check_device(o, "o")) || (rc = check_device(lse, "lse")) ||
        (rc = check_device(ws, "workspace")))
        return rc;
    if (lse_window && ((rc = check_device(o_window, "o_window")) || (rc = check_device(lse_window, "lse_window"))))
        return rc;

    // Every tile's key splits write into one set of per-split partials for
    // the layer (tile t at offset off[t]); one merge then takes the window's
    // result and all of them, in that order.
    std::vector<int> off;
    int total = 0;
    size_t acc_bytes = 0, plan_bytes = 0;
    if ((rc = layer_tail_plan(r, layer, desc, &off, &total, &acc_bytes, &plan_bytes))) return rc;
    float *part_acc = (float *)ws;
    float2 *part_ml = (float2 *)((char *)ws + acc_bytes);
    const bool inplace = r->inplace[layer] != 0;
    // Slot release of the last streamed tile launched: written by the next
    // kernel on the stream, the layer's next tile or its merge, when it
    // starts (the tile's kernel has then finished reading the slot).
    uint64_t *rel = nullptr;
    uint64_t rel_value = 0;
    // On a failure after a tile's launch: let the launched work finish, then
    // release that tile's slot from the host (nothing on the GPU will), so no
    // copy waits for a release that never comes; the step is aborted (later
    // calls: RKV_E_STATE).
    auto abort_step = [&](int code) {
        if (rel) {
            (void)hipStreamSynchronize(cs);
            __atomic_store_n(rel, rel_value, __ATOMIC_RELEASE);
        }
        r->in_step = false;
        return code;
    };
    for (int64_t t = 0; t < n_tiles; ++t) {
        const int64_t j = j0 + t;
        const int s = inplace ? 0 : (int)(j % r->B);
        const rkv_kv_view v = tile_view(r, layer, t, s);
        if ((rc = check_view_fields(desc, &v)) || (!inplace && (rc = wait_enqueued(r, j)))) return abort_step(rc);
        if (!inplace) {
            hipError_t e = hipStreamWaitEvent(cs, r->copy_done[s], 0);
            if (e != hipSuccess) return abort_step(hip_fail(e, "hipStreamWaitEvent (copy_done)"));
        }
        const rkv_kv_view *vp = &v;
        CallPlan cp;
        SplitParams prm[kMaxSegs];
        rc = make_call_plan(desc, 1, &vp, &cp, prm);
        if (!rc && (cp.g.n != 1 || cp.n_splits_all != off[t + 1] - off[t]))
            rc = fail(RKV_E_STATE, "tile plan changed between the workspace query and the launch");
        if (rc) return abort_step(rc);
        prm[0].split_off = off[t];
        prm[0].n_splits_all = total;
        prm[0].direct = 0;
        prm[0].release = rel;
        prm[0].release_value = rel_value;
        if ((rc = launch_plan(cp, prm, desc, q, part_acc, part_ml, o, lse, cs))) return abort_step(rc);
        rel = nullptr;
        if (!inplace) {
            const int64_t g = r->base + j;
            rel = r->progress + s;
            rel_value = (uint64_t)(g + 1);
            {
                std::lock_guard<std::mutex> lk(r->mu);
                r->last_user[s] = g;
            }
            if (j + r->B < (int64_t)r->items.size()) request_copy(r, j + r->B);
        }
    }
    if (total > 0) {
        hipError_t e = launch_reduce(D, n_rows, total, part_acc, part_ml, o, lse, cs, rel, rel_value,
                                     lse_window ? o_window : nullptr, lse_window);
        if (e != hipSuccess) return abort_step(hip_fail(e, "merge launch"));
    } else if (lse_window) {
        CombineParts parts;
        memset(&parts, 0, sizeof parts);
        parts.o[0] = o_window;
        parts.lse[0] = lse_window;
        RKV_HIP(launch_combine(1, parts, n_rows, D, o, lse, cs));  // a single part: copied bit for bit
    } else {
        RKV_HIP(launch_fill_empty(D, n_rows, o, lse, cs));
    }
    r->next_layer++;
    return RKV_OK;
}

int rkv_append_kv(int n_kv_heads, int head_dim, int n_tokens, int64_t pos0, int seq, const float *k_new,
                  const float *v_new, const rkv_kv_view *window, const rkv_kv_view *tail, const rkv_kv_view *fresh,
                  rkv_ring *ring, int layer, hipStream_t stream)
{
    if (n_kv_heads < 1 || n_kv_heads > 65535) return fail(RKV_E_INVAL, "n_kv_heads must be in [1, 65535]");
    if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512)
        return fail(RKV_E_UNSUPPORTED, "head_dim must be 64, 128, 256 or 512");
    if (n_tokens < 0) return fail(RKV_E_INVAL, "n_tokens < 0");
    if (pos0 < 0 || seq < 0) return fail(RKV_E_INVAL, "pos0 and seq must be >= 0");
    if (ring && (layer < 0 || layer >= kRingMaxLayers))
        return fail(RKV_E_INVAL, "layer must be in [0, %d)", kRingMaxLayers);
    const int64_t wc = window ? window->n_keys : 0, tc = tail ? tail->n_keys : 0;
    if (wc < 0 || tc < 0) return fail(RKV_E_INVAL, "capacities (n_keys) must be >= 0");
    if (pos0 + n_tokens > wc + tc)
        return fail(RKV_E_INVAL, "positions [%lld, %lld) exceed window %lld + tail %lld", (long long)pos0,
                    (long long)(pos0 + n_tokens), (long long)wc, (long long)tc);
    if (n_tokens == 0) return RKV_OK;
    if (n_tokens > (1 << 30) || (int64_t)n_tokens * n_kv_heads > 0x7fff0000)
        return fail(RKV_E_UNSUPPORTED, "n_tokens x n_kv_heads too large");
    int rc;
    if ((rc = check_device(k_new, "k_new")) || (rc = check_device(v_new, "v_new"))) return rc;
    if ((uintptr_t)k_new % 4 || (uintptr_t)v_new % 4) return fail(RKV_E_INVAL, "k_new / v_new must be 4-byte aligned");
    // tokens [0, nw) go to the window, [nw, n_tokens) to the tail
    const int nw = (int)std::max<int64_t>(0, std::min<int64_t>(n_tokens, wc - pos0));
    const int nt = n_tokens - nw;
    AppendParams p;
    memset(&p, 0, sizeof p);
    p.n_kv_heads = n_kv_heads;
    // One destination: validate the region and fill p.dst[p.n_dst].  kinds:
    // bit 1 device memory allowed, bit 0 pinned host memory allowed.
    auto add = [&](const rkv_kv_view *v, const char *name, int first, int count, int64_t row0, int kinds) -> int {
        if (count == 0) return RKV_OK;
        if (v->k_type == RKV_TBQ3 || v->v_type == RKV_TBQ3)
            return fail(RKV_E_UNSUPPORTED, "%s: appending to TBQ3 storage is not supported", name);
        if (!valid_type(v->k_type) || !valid_type(v->v_type)) return fail(RKV_E_INVAL, "%s: bad K/V type", name);
        if (!v->k || !v->v) return fail(RKV_E_INVAL, "%s: K or V pointer is NULL", name);
        const int64_t rbk = row_bytes_of(v->k_type, head_dim), rbv = row_bytes_of(v->v_type, head_dim);
        if (v->k_pos_stride <= 0 || v->v_pos_stride <= 0 || v->k_head_stride < 0 || v->v_head_stride < 0 ||
            v->k_seq_stride < 0 || v->v_seq_stride < 0)
            return fail(RKV_E_INVAL, "%s: strides must be non-negative (position strides positive)", name);
        if ((uintptr_t)v->k % 2 || (uintptr_t)v->v % 2 || v->k_pos_stride % 2 || v->v_pos_stride % 2 ||
            v->k_head_stride % 2 || v->v_head_stride % 2 || v->k_seq_stride % 2 || v->v_seq_stride % 2)
            return fail(RKV_E_INVAL, "%s: pointers and strides must be even", name);
        if (n_kv_heads > 1 && (v->k_head_stride < rbk || v->v_head_stride < rbv))
            return fail(RKV_E_INVAL, "%s: head stride smaller than a row", name);
        if ((n_kv_heads - 1) * v->k_head_stride + rbk > v->k_pos_stride ||
            (n_kv_heads - 1) * v->v_head_stride + rbv > v->v_pos_stride)
            return fail(RKV_E_INVAL, "%s: the rows of one position must fit in its position stride", name);
        auto allowed = [kinds](int m) { return (m == 2 && (kinds & 2)) || (m == 1 && (kinds & 1)); };
        const int mk = mem_kind(v->k), mv = mem_kind(v->v);
        if (!allowed(mk) || !allowed(mv))
            return fail(RKV_E_INVAL, "%s: must be %s", name,
                        kinds == 2 ? "device memory" : "device memory or pinned host memory");
        if (mk == 1 || mv == 1) p.sys_fence = 1;
        AppendDst &d = p.dst[p.n_dst++];
        d.k = (uint8_t *)v->k + (int64_t)seq * v->k_seq_stride;
        d.v = (uint8_t *)v->v + (int64_t)seq * v->v_seq_stride;
        d.k_pos = v->k_pos_stride;
        d.v_pos = v->v_pos_stride;
        d.k_head = v->k_head_stride;
        d.v_head = v->v_head_stride;
        d.k_type = v->k_type;
        d.v_type = v->v_type;
        d.first_tok = first;
        d.n_tok = count;
        d.row0 = row0;
        return RKV_OK;
    };
    if ((rc = add(window, "window", 0, nw, pos0, 2))) return rc;
    if ((rc = add(tail, "tail", nw, nt, pos0 + nw - wc, 3))) return rc;
    if (fresh && nt > 0) {
        if (fresh->n_keys < nt) return fail(RKV_E_INVAL, "fresh holds %lld rows, %d needed", (long long)fresh->n_keys, nt);
        if ((rc = add(fresh, "fresh", nw, nt, 0, 2))) return rc;
    }
    RKV_HIP(launch_append(head_dim, n_tokens, n_kv_heads, k_new, v_new, p, stream));
    if (ring && nt > 0) {
        RKV_HIP(launch_signal(ring->written + layer, (uint64_t)(ring->appends[layer] + 1), stream));
        ring->appends[layer]++;
    }
    return RKV_OK;
}

int rkv_ring_end_step(rkv_ring *r)
{
    if (!r) return fail(RKV_E_INVAL, "ring is NULL");
    if (!r->in_step) return fail(RKV_E_STATE, "no step begun");
    r->in_step = false;
    if (r->next_layer != (int)r->tails.size())
        return fail(RKV_E_STATE, "step ended after %d of %d layers", r->next_layer, (int)r->tails.size());
    return RKV_OK;
}

}  // extern "C"
