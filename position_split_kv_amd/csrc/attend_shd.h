// attend_shd.h -- the split kernel for many query rows per KV head over
// block-type K (q8_0 / q4_0) and q4_0 V at head_dim 128, with the block
// decode shared by the row groups of a head.
//
// With more than 16 query rows per KV head (sequences sharing one prefix, the
// rows of a verify step or a prefill chunk), the general split kernel runs
// each 16-row group of a head in its own workgroup, and every group decodes
// the same key tiles.  Here a workgroup holds one KV head x 4 row groups
// (4 waves, one 16-row group each; two workgroups share a compute unit).
// Per 64-key tile, the head's K and V rows go global -> LDS once (the tile's
// direct-to-LDS loads shared out evenly over the four waves); each of the
// head's four waves decodes a quarter of them into the exact binary16
// matrix-core operands -- K codes of one 32-dim block (with its scales), and
// d * code of one key pair per 8-key group split into high and low binary16
// parts -- in LDS; after a workgroup barrier every wave runs its scores,
// softmax and P.V from those operands.  A second barrier per tile (at the
// next tile's top) keeps the operands until every wave has used them.  The
// arithmetic per row is that of the general kernel (the same MFMA shapes,
// binary16 operands and accumulation orders); only where the operands are
// made differs.
#pragma once

#include "attend_kernel.h"

namespace rkv {

constexpr int kShdRG = 4;                     // row groups of 16 rows per KV head in a workgroup
constexpr int kShdHeads = 1;                  // KV heads per workgroup (two workgroups share a compute unit)
constexpr int kShdWaves = kShdRG * kShdHeads;  // waves per workgroup

template <int KT, int VT>
struct ShdShape {
    using Sh = Shape<KT, VT, 128>;
    static constexpr int LSK = Sh::LSK, LSV = Sh::LSV;
    static constexpr int RAW_DW = kTile * (LSK + LSV) + 8;  // a head's raw K and V tiles (+ read slack)
    static constexpr int BK_DW = 4 * 4 * 64 * 4;             // K operands [kb 4][kk 4][lane 64] x 16 bytes
    static constexpr int DK_DW = 4 * 4 * 16;                 // K block scales [kb][kk][key 16]
    static constexpr int BV_DW = 2 * 8 * 64 * 4;             // V operands [kb 2][c 8][lane 64] x 16 bytes
    static constexpr int HEAD_DW = RAW_DW + BK_DW + DK_DW + 2 * BV_DW;  // (V: high and low parts)
    static constexpr int SP_DW = 16 * kTile;                 // one wave's score rows
    static constexpr int LDS_DW = kShdHeads * HEAD_DW + kShdWaves * SP_DW;
    static constexpr bool OK = (KT == kQ8 || KT == kQ4) && VT == kQ4 && 4 * LDS_DW <= 160 * 1024;
};

template <int KT, int VT>
__global__ void __launch_bounds__(64 * kShdWaves, 2)
rkv_split_shd_kernel(const float *__restrict__ q, float *__restrict__ part_acc, float2 *__restrict__ part_ml,
                     float *__restrict__ o_out, float *__restrict__ lse_out, const SplitParams p)
{
    using SS = ShdShape<KT, VT>;
    using Sh = typename SS::Sh;
    static_assert(SS::OK, "instance outside the shared-decode kernel's LDS budget");
    constexpr int D = 128, RT = 16;
    constexpr int LSK = SS::LSK, LSV = SS::LSV;
    __shared__ __attribute__((aligned(16))) uint32_t lds[SS::LDS_DW];

    if (p.release && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0)
        __hip_atomic_store(p.release, p.release_value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hs = w / kShdRG, rgl = w - hs * kShdRG;  // head slot, row group within the head
    const int hg = blockIdx.y / p.n_rg, rgb = blockIdx.y - hg * p.n_rg;
    const int g = hg * kShdHeads + hs;
    const int rg = rgb * kShdRG + rgl;
    const int cnt = g < p.n_kv_heads ? u16_at(p.rowcnt, g) - rg * RT : 0;
    const int nr = cnt <= 0 ? 0 : cnt < RT ? cnt : RT;  // a wave with no rows still decodes and joins the barriers
    const int z = blockIdx.z;

    uint32_t *const rawK = lds + hs * SS::HEAD_DW;
    uint32_t *const rawV = rawK + kTile * LSK;
    uint32_t *const bK = rawK + SS::RAW_DW;
    float *const dK = (float *)(bK + SS::BK_DW);
    uint32_t *const bVh = (uint32_t *)(dK + SS::DK_DW);
    uint32_t *const bVl = bVh + SS::BV_DW;
    float *const sPw = (float *)(lds + kShdHeads * SS::HEAD_DW + w * SS::SP_DW);

    SegParams sg = p.seg[0];
#pragma unroll
    for (int si = 1; si < kMaxSegs; ++si)
        if (si < p.n_segs && (int)blockIdx.x >= p.seg[si].split_base) sg = p.seg[si];
    const int64_t kbeg = (int64_t)((int)blockIdx.x - sg.split_base) * sg.keys_per_split;
    // every wave of the workgroup walks every tile of the split (barriers)
    const int64_t kend = kbeg + sg.keys_per_split < sg.n_keys ? kbeg + sg.keys_per_split : sg.n_keys;
    const int gr = g < p.n_kv_heads ? g : p.n_kv_heads - 1;
    const uint8_t *kg = sg.k + z * sg.k_seq + gr * sg.k_head;
    const uint8_t *vg = sg.v + z * sg.v_seq + gr * sg.v_head;

    // output row of the wave's row r (-1 past nr); read again after the tile
    // loop rather than held in scalar registers through it
    auto table_row = [&](int r, int nrx) {
        const int ti = g * p.rows_per_g + rg * RT + r;
        const int v = u16_at(p.rowtab, ti < kMaxRowTable ? ti : kMaxRowTable - 1);
        return r < nrx ? z * p.z_row_step + v : -1;
    };
    int tabrow[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) tabrow[r] = table_row(r, nr);
    // causal mask: row r sees the segment's keys with index <= lim[r]
    constexpr int kSeeAll = 1 << 30;
    int limv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * (lane >> 4) + i;
        int x = kSeeAll;
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            if (p.masked && row == r && tabrow[r] >= 0) {
                const int64_t rel = p.qpos[tabrow[r] / p.n_q_heads] - sg.pos0;
                x = rel < -1 ? -1 : rel > kSeeAll ? kSeeAll : (int)rel;
            }
        }
        limv[i] = x;
    }
    // the earliest limit of the wave's rows: tiles that end at or before it
    // need no mask
    int lim_min = kSeeAll;
    if (p.masked) {
#pragma unroll
        for (int r = 0; r < RT; ++r)
            if (tabrow[r] >= 0) {
                const int64_t rel = p.qpos[tabrow[r] / p.n_q_heads] - sg.pos0;
                const int x = rel < -1 ? -1 : rel > kSeeAll ? kSeeAll : (int)rel;
                lim_min = x < lim_min ? x : lim_min;
            }
    }

    // raw tile DMA: the tile's K rows by the slot plan (LSK loads) and its V
    // rows by the whole-row copy (NLV loads, several rows per load), one
    // sequence of loads shared out in quarters over the four waves: wave w
    // issues loads [w * NQ, (w + 1) * NQ) of K's then V's
    static_assert(LSK > 0 && LSV > 0, "block K and V rows are staged in LDS");
    using VRow = RowDma<Sh::RBV / 4, LSV>;
    static_assert(VRow::R >= 2, "several V rows per load");
    constexpr int NLV = VRow::NL, NQ = (LSK + NLV + 3) / 4;
    const uint64_t kwrap = dma_wraps<LSK>(lane);
    const bool kfull_ok = sg.k_pos >= 4 * LSK && sg.k_pos < (1 << 23);
    const bool vfull_ok = sg.v_pos >= 4 * LSV && sg.v_pos < (1 << 23);
    // loads [S0, S1) of the sequence for wave W: K's [K0, K1), V's [V0, V1)
    auto wave_range = [](auto wc) {
        constexpr int W = decltype(wc)::value;
        constexpr int S0 = W * NQ, S1 = (W + 1) * NQ < LSK + NLV ? (W + 1) * NQ : LSK + NLV;
        struct R {
            int k0, k1, v0, v1;
        };
        return R{S0 < LSK ? S0 : LSK, S1 < LSK ? S1 : LSK, S0 > LSK ? S0 - LSK : 0, S1 > LSK ? S1 - LSK : 0};
    };
    // this wave's K load offsets, planned once (no per-load arithmetic), and
    // the V rows' lane offset
    uint32_t koffs[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) koffs[j] = 0;
    auto plan_wave = [&](auto wc) {
        constexpr auto r = wave_range(wc);
        if constexpr (r.k0 < r.k1)
            if (kfull_ok) dma_plan_grp<LSK, r.k0, r.k1>((int)sg.k_pos, kwrap, lane, koffs);
    };
    if (rgl == 0)
        plan_wave(std::integral_constant<int, 0>{});
    else if (rgl == 1)
        plan_wave(std::integral_constant<int, 1>{});
    else if (rgl == 2)
        plan_wave(std::integral_constant<int, 2>{});
    else
        plan_wave(std::integral_constant<int, 3>{});
    const uint32_t voffr = row_dma_voff<LSV>((int)sg.v_pos, lane);
    auto nk_at = [&](int64_t t) { return (int)(kend - t < kTile ? kend - t : kTile); };
    auto dma_raw = [&](int64_t t) {
        const int nkk = nk_at(t);
        const bool whole = nkk == kTile && t + kTile < sg.n_keys;
        int kps = (int)sg.k_pos, vps = (int)sg.v_pos;
        asm volatile("" : "+s"(kps), "+s"(vps));
        waitcnt_lgkm0();
        const uint8_t *ks = kg + t * sg.k_pos, *vs = vg + t * sg.v_pos;
        const uint32_t kbase = lds_addr(rawK), vbase = lds_addr(rawV);
        auto wave_loads = [&](auto wc) {
            constexpr auto r = wave_range(wc);
            constexpr int K0 = r.k0, K1 = r.k1, V0 = r.v0, V1 = r.v1;
            if constexpr (K0 < K1) {
                if (kfull_ok && whole) {
                    dma_issue_grp<K0, K1 - K0>(buffer_rsrc(ks), koffs, kbase);
                } else {
                    dma_rows4<Sh::RBK / 4, LSK, K0, K1>(ks, kps, nkk, kbase, lane);
                }
            }
            if constexpr (V0 < V1) {
                if (vfull_ok && whole) {
                    dma_rows_whole<Sh::RBV / 4, LSV, V0, V1>(buffer_rsrc(vs), voffr, vps,
                                                             (uint32_t)VRow::R * (uint32_t)(vps - 4 * LSV), vbase);
                } else {
                    // the clamped copy in the slot plan's units: the V loads
                    // of this wave's share, scaled to LSV
                    constexpr int C0 = V0 * LSV / NLV, C1 = V1 == NLV ? LSV : V1 * LSV / NLV;
                    dma_rows4<Sh::RBV / 4, LSV, C0, C1>(vs, vps, nkk, vbase, lane);
                }
            }
        };
        if (rgl == 0)
            wave_loads(std::integral_constant<int, 0>{});
        else if (rgl == 1)
            wave_loads(std::integral_constant<int, 1>{});
        else if (rgl == 2)
            wave_loads(std::integral_constant<int, 2>{});
        else
            wave_loads(std::integral_constant<int, 3>{});
    };

    float qraw[D / 32][8];
    {
        const int qr = lane & 15;
        int rowi = 0;
#pragma unroll
        for (int r = 0; r < RT; ++r) rowi = (qr == r && tabrow[r] >= 0) ? tabrow[r] : rowi;
        mfma_q_load<D>(q + (int64_t)rowi * D, lane, qraw);
    }
    int64_t t0 = kbeg;
    if (t0 < kend) dma_raw(t0);
    rkv_half8 qhi[D / 32], qlo[D / 32];
    pin_v<8 * (D / 32)>(&qraw[0][0]);
    int oex[4];  // query-row exponents of the lane's MFMA output rows
    const int qex = mfma_q_split<D>(qraw, (lane & 15) < nr, p.scale_log2, qhi, qlo);
    mfma_out_row_exps(qex, lane, oex);
    const bool qscaled = __builtin_amdgcn_ballot_w64(qex != 0) != 0;  // some row has one (wave-uniform)
    float mrow[4], lrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        mrow[i] = -INFINITY;
        lrow[i] = 0.f;
    }
    rkv_float4v oc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) oc[c] = rkv_float4v{0.f, 0.f, 0.f, 0.f};
    const float cap = p.softcap;
    constexpr float kLog2e = 1.4426950408889634f;
    const float capl = cap * kLog2e;
    const float two_over_cap = cap > 0.f ? 2.f / cap : 0.f;
    const int qi = lane & 15, gq = lane >> 4;
    // LDS layouts free of bank conflicts.  V operands: wave rgl's key pair
    // sits in dword (rgl + gq) mod 4 of a lane's 16-byte operand, so the four
    // lane groups of one store hit different banks; the matrix core pairs A
    // and B element by element within a lane group, so the probabilities of
    // a group take the same rotated key order: 32-key block b, element
    // 2 ((s + g) mod 4) + e of group g holds key 32 b + 8 s + 4 e + g.
    // Probability rows: column c of row r is stored at c ^ swz(r), swz(r) =
    // 4 ((2 (r / 4) + r) mod 4) + 16 (r / 4 mod 4), which keeps 4-column
    // groups whole for the 16-byte reads and spreads both the stores and the
    // reads over all banks.
    const int vslot = (rgl + gq) & 3;
    auto swz = [](int r) { return 4 * ((2 * (r >> 2) + r) & 3) + 16 * ((r >> 2) & 3); };
    int pcol[4];  // rotated column of key 16 kb + qi
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const int key = 16 * kb + qi, g = key & 3, e = (key >> 2) & 1, sk = (key >> 3) & 3;
        pcol[kb] = 16 * g + 8 * (key >> 5) + 2 * ((sk + g) & 3) + e;
    }
    const int swr = swz(qi);

    for (; t0 < kend; t0 += kTile) {
        const int nk = nk_at(t0);
        waitcnt_vm<0>();  // this wave's share of the raw tile DMA has landed
        __syncthreads();  // the head's raw tiles are in LDS; every wave is done with the last tile's operands

        // A tile with a V block scale large enough for d * code to overflow
        // the binary16 operands (rare): every wave multiplies P.V out in
        // binary32 from the raw V tile instead, which then stays in LDS until
        // P.V is done (the next tile's DMA waits).  Every wave scans the whole
        // tile, so all four take the same decision.
        const bool vbig =
            __builtin_amdgcn_ballot_w64(v_row_scale_max<VT, D / 32>(rawV + lane * LSV) >= v_scale_limit<VT>()) != 0;

        // ---- decode this wave's quarter of the head's operands
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            float dsc;
            const rkv_half8 b = block_codes_f16<KT, false>(rawK + (16 * kb + qi) * LSK, rgl, gq, dsc);  // (kk = the wave's row group)
            *(rkv_half8 *)(bK + ((kb * 4 + rgl) * 64 + lane) * 4) = b;
            if (lane < 16) dK[(kb * 4 + rgl) * 16 + lane] = dsc;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            uint32_t ca[4], cb[4], da, db;
            v_group_codes_f16<VT>(rawV + (4 * (8 * kb + 2 * rgl) + gq) * LSV, qi, ca, da);
            v_group_codes_f16<VT>(rawV + (4 * (8 * kb + 2 * rgl + 1) + gq) * LSV, qi, cb, db);
            const rkv_half2 d2 = __builtin_bit_cast(rkv_half2, da | (db << 16));
#pragma unroll
            for (int p2 = 0; p2 < 4; ++p2) {
                const rkv_half2 x0 = __builtin_bit_cast(rkv_half2, __builtin_amdgcn_perm(cb[p2], ca[p2], 0x05040100u));
                const rkv_half2 x1 = __builtin_bit_cast(rkv_half2, __builtin_amdgcn_perm(cb[p2], ca[p2], 0x07060302u));
                const rkv_half2 h0 = d2 * x0, h1 = d2 * x1;
                const rkv_half2 l0 = __builtin_elementwise_fma(d2, x0, -h0);
                const rkv_half2 l1 = __builtin_elementwise_fma(d2, x1, -h1);
                const int i0 = ((kb * 8 + 2 * p2) * 64 + lane) * 4 + vslot, i1 = i0 + 64 * 4;
                bVh[i0] = __builtin_bit_cast(uint32_t, h0);
                bVh[i1] = __builtin_bit_cast(uint32_t, h1);
                bVl[i0] = __builtin_bit_cast(uint32_t, l0);
                bVl[i1] = __builtin_bit_cast(uint32_t, l1);
            }
        }
        __syncthreads();  // the operands are in LDS; the raw tiles are free
        if (!vbig && t0 + kTile < kend) dma_raw(t0 + kTile);

        // ---- scores on the matrix cores from the shared K operands
        float sv[4][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[kb][i] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            // (the four key blocks' operands together, then the high-part
            // products, then the low-part ones: consecutive MFMAs use
            // different accumulators)
            rkv_half8 b[4];
            float dsc[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                b[kb] = *(const rkv_half8 *)(bK + ((kb * 4 + kk) * 64 + lane) * 4);
                dsc[kb] = dK[(kb * 4 + kk) * 16 + qi];
            }
            rkv_float4v acc[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qhi[kk], b[kb], rkv_float4v{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qlo[kk], b[kb], acc[kb], 0, 0, 0);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[kb][i] = fmaf(dsc[kb], acc[kb][i], sv[kb][i]);
        }
        if (qscaled) unscale_rows(sv, oex);
        // ---- mask, cap, online softmax (as the general kernel)
        const bool tile_masked = p.masked && t0 + nk - 1 > lim_min;
        int kmx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tl = limv[i] - (int)t0;
            kmx[i] = tile_masked ? (tl < nk - 1 ? (tl < -1 ? -1 : tl) : nk - 1) : nk - 1;
        }
        if (tile_masked || nk < kTile) {
            if (cap > 0.f)
                cap_mask_tile<true, true>(sv, kmx, qi, capl, two_over_cap);
            else
                cap_mask_tile<false, true>(sv, kmx, qi, capl, two_over_cap);
        } else if (cap > 0.f) {
            cap_mask_tile<true, false>(sv, kmx, qi, capl, two_over_cap);
        }
        float al[4], mex[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float mx = fmaxf(fmaxf(sv[0][i], sv[1][i]), fmaxf(sv[2][i], sv[3][i]));
            mx = row16_max(mx);
            const float mn = fmaxf(mrow[i], mx);
            mex[i] = mn == -INFINITY ? 0.f : mn;
            al[i] = __builtin_amdgcn_exp2f(mrow[i] - mex[i]);
            lrow[i] *= al[i];
            mrow[i] = mn;
        }
        // (skipped when no row's maximum moved: al = 2^0 = 1 exactly)
        if (__builtin_amdgcn_ballot_w64(al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f)) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) oc[c][i] *= al[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * (lane >> 4) + i;
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const float pv = __builtin_amdgcn_exp2f(sv[kb][i] - mex[i]);
                ps += pv;
                sPw[row * kTile + (pcol[kb] ^ swz(row))] = pv;
            }
            lrow[i] += ps;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();

        if (vbig) {
            // ---- P.V in binary32 from the raw V tile (probability of row r,
            // key k at its rotated, swizzled column), then the next tile's DMA
            // once every wave is done with the raw tile
            pv_valu_tile<VT, LSV>(
                rawV,
                [&](int r, int k) {
                    const int kg4 = k & 3;
                    const int col = 16 * kg4 + 8 * (k >> 5) + 2 * ((((k >> 3) & 3) + kg4) & 3) + ((k >> 2) & 1);
                    return sPw[r * kTile + (col ^ swz(r))];
                },
                RT, lane, oc);
            __syncthreads();
            if (t0 + kTile < kend) dma_raw(t0 + kTile);
            continue;
        }
        // ---- P.V on the matrix cores from the shared V operands
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            rkv_half8 ph, pl;
            {
                const float4 a = *(const float4 *)&sPw[qi * kTile + ((gq * 16 + 8 * kb) ^ swr)];
                const float4 b = *(const float4 *)&sPw[qi * kTile + ((gq * 16 + 8 * kb + 4) ^ swr)];
                const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const _Float16 h = (_Float16)x[e];
                    ph[e] = h;
                    pl[e] = (_Float16)(x[e] - (float)h);
                }
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const rkv_half8 bh = *(const rkv_half8 *)(bVh + ((kb * 8 + c) * 64 + lane) * 4);
                const rkv_half8 bl = *(const rkv_half8 *)(bVl + ((kb * 8 + c) * 64 + lane) * 4);
                oc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, bh, oc[c], 0, 0, 0);
                oc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, bl, oc[c], 0, 0, 0);
                oc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, bh, oc[c], 0, 0, 0);
            }
        }
    }

    // ---- each wave owns its rows: write them from the MFMA output layout
    float m[RT], l[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const float t = row16_sum(lrow[r & 3]);
        l[r] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, t), 16 * (r >> 2)));
        m[r] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mrow[r & 3]), 16 * (r >> 2)));
    }
    const bool single = p.direct != 0;
    const int64_t pbase = (int64_t)(p.split_off + (int)blockIdx.x) * p.n_rows_total;
    int orow[RT];
    int nr_e = nr;
    asm volatile("" : "+s"(nr_e));  // (not the loop-spanning copies of r < nr)
#pragma unroll
    for (int r = 0; r < RT; ++r) orow[r] = table_row(r, nr_e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * (lane >> 4) + i;
        int rr = -1;
        float lr = 1.f;
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            rr = row == r ? orow[r] : rr;
            lr = row == r ? l[r] : lr;
        }
        if (rr < 0) continue;
        float v[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = single ? (lr > 0.f ? oc[c][i] / lr : 0.f) : oc[c][i];
        float *dst = single ? o_out + (int64_t)rr * D : part_acc + (pbase + rr) * D;
        *(float4 *)(dst + 8 * qi) = make_float4(v[0], v[1], v[2], v[3]);
        *(float4 *)(dst + 8 * qi + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
    if (lane < RT) {
        int rr = -1;
        float mr = 0.f, lr = 1.f;
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            rr = lane == r ? orow[r] : rr;
            mr = lane == r ? m[r] : mr;
            lr = lane == r ? l[r] : lr;
        }
        if (rr >= 0) {
            if (single) lse_out[rr] = (mr + log2f(lr)) * 0.69314718055994531f;
            else part_ml[(int64_t)rr * p.n_splits_all + p.split_off + blockIdx.x] = make_float2(mr, lr);
        }
    }
}

}  // namespace rkv
