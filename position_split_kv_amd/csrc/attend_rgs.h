// attend_rgs.h -- the split kernel for more than 16 query rows per KV head
// over f16 K and V at head_dim 128, with each key tile staged once per head.
//
// The rows of a verify step or a prefill chunk (n_q > 1 rows of one sequence
// under the causal mask) or of sequences sharing one cache give a KV head
// several 16-row groups.  In the general kernel each row group's wave loads
// its own copy of every tile, right after its previous tile's P.V, and waits
// a whole load latency per tile.  Here a workgroup holds one KV head x 4 row
// groups (4 waves of 16 rows; two workgroups share a compute unit).  The
// head's K and V rows of a 64-key tile go global -> LDS once, by 16-byte
// direct loads (a quarter of them per wave), into one of two stages: the next
// tile's loads are issued as soon as the current tile is in LDS and stay in
// flight through all of its compute.  One workgroup barrier per tile hands
// the stages over.  Every wave runs its scores from the K stage (16-byte
// chunks swizzled as in the general kernel), its softmax, and P.V from the V
// stage (16-byte row reads into the operand layout of the general kernel's
// register-held V).  The arithmetic per row is the general kernel's: the
// same binary16 high / low query and probability parts, MFMA shapes and
// accumulation orders.
#pragma once

#include "attend_kernel.h"

namespace rkv {

constexpr int kRgsRG = 4;  // row groups of 16 rows per workgroup (one KV head)

struct RgsShape {
    static constexpr int D = 128, RB = 256;           // head_dim, bytes of an f16 row
    static constexpr int TILE_DW = kTile * RB / 4;    // one 64-key tile of K or V rows
    static constexpr int HALF_P = 32;                 // keys of one probability half-tile
    static constexpr int SP_DW = 16 * HALF_P;         // a wave's probability rows (16 x 32 keys)
    static constexpr int LDS_DW = 4 * TILE_DW + kRgsRG * SP_DW;  // K and V, two stages each
    static_assert(4 * LDS_DW <= 80 * 1024, "two workgroups per compute unit");
};

__global__ void __launch_bounds__(64 * kRgsRG, 2)
rkv_split_rgs_kernel(const float *__restrict__ q, float *__restrict__ part_acc, float2 *__restrict__ part_ml,
                     float *__restrict__ o_out, float *__restrict__ lse_out, const SplitParams p)
{
    using RS = RgsShape;
    constexpr int D = RS::D, RT = 16, RB = RS::RB;
    __shared__ __attribute__((aligned(16))) uint32_t lds[RS::LDS_DW];

    if (p.release && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0)
        __hip_atomic_store(p.release, p.release_value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const int lane = threadIdx.x & 63;
    const int rgl = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // row group within the workgroup
    const int g = blockIdx.y / p.n_rg, rgb = blockIdx.y - g * p.n_rg;
    const int rg = rgb * kRgsRG + rgl;
    const int cnt = g < p.n_kv_heads ? u16_at(p.rowcnt, g) - rg * RT : 0;
    const int nr = cnt <= 0 ? 0 : cnt < RT ? cnt : RT;  // a wave with no rows still loads and joins the barriers
    const int z = blockIdx.z;

    uint32_t *const stK = lds;                      // [stage 2][64 rows][64 dwords], chunks swizzled
    uint32_t *const stV = lds + 2 * RS::TILE_DW;    // [stage 2][64 rows][64 dwords]
    float *const sPw = (float *)(lds + 4 * RS::TILE_DW + rgl * RS::SP_DW);

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

    int tabrow[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int ti = g * p.rows_per_g + rg * RT + r;
        const int v = u16_at(p.rowtab, ti < kMaxRowTable ? ti : kMaxRowTable - 1);
        tabrow[r] = r < nr ? z * p.z_row_step + v : -1;
    }
    // causal mask: row r sees the segment's keys with index <= its limit
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

    // ---- tile DMA: K and V are 16 loads of 1 KB each (4 rows of 256 bytes);
    // wave rgl issues loads 4 rgl .. 4 rgl + 3 of both.  Load i of K puts the
    // 16-byte chunk (lane & 15) ^ kswz(row) of row 4 i + lane / 16 at LDS
    // slot lane (row-major rows, swizzled chunks); load i of V chunk lane & 15
    // unswizzled.
    const int lg = lane >> 4, lc = lane & 15;
    auto nk_at = [&](int64_t t) { return (int)(kend - t < kTile ? kend - t : kTile); };
    auto dma_tile = [&](int64_t t, int stage) {
        const int nkk = nk_at(t);
        int kps = (int)sg.k_pos, vps = (int)sg.v_pos;
        asm volatile("" : "+s"(kps), "+s"(vps));
        const uint8_t *kt = kg + t * sg.k_pos, *vt = vg + t * sg.v_pos;
        const uint32_t kb = lds_addr(stK + stage * RS::TILE_DW), vb = lds_addr(stV + stage * RS::TILE_DW);
        auto issue = [&](auto policy) {
            constexpr bool NT = decltype(policy)::value;
            if (nkk == kTile) {
                // one group of four buffer loads each for K and V, starting
                // at row 16 rgl (load j at row 4 (4 rgl + j) and LDS byte
                // 1024 (4 rgl + j)); the K chunk swizzle of rows 4i .. 4i+3 is
                // kswz(4i + lg) = (4i mod 16) | lg = 4 j | lg
                uint32_t ko[4], vo[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ko[j] = (uint32_t)lg * (uint32_t)kps + 16u * (uint32_t)(lc ^ (4 * j) ^ lg);
                    vo[j] = (uint32_t)lg * (uint32_t)vps + 16u * (uint32_t)lc;
                }
                lds_dma16_grp<4, NT>(buffer_rsrc(kt), ko, 16u * (uint32_t)rgl * (uint32_t)kps, 4u * (uint32_t)kps - 1024u,
                                     kb + 4096u * (uint32_t)rgl);
                lds_dma16_grp<4, NT>(buffer_rsrc(vt), vo, 16u * (uint32_t)rgl * (uint32_t)vps, 4u * (uint32_t)vps - 1024u,
                                     vb + 4096u * (uint32_t)rgl);
                return;
            }
            // the segment's last, short tile: rows past nkk repeat row nkk - 1
            static_for<0, 4>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                const int i = 4 * rgl + j;
                const int row = 4 * i + lg;
                const int rc = row < nkk ? row : nkk - 1;
                lds_dma16<NT, 1024u * j>(kt + (uint32_t)(rc * kps + 16 * (lc ^ kswz<RB>(row))), kb + 4096u * (uint32_t)rgl);
                lds_dma16<NT, 1024u * j>(vt + (uint32_t)(rc * vps + 16 * lc), vb + 4096u * (uint32_t)rgl);
            });
        };
        if (p.stream_once)
            issue(std::integral_constant<bool, true>{});
        else
            issue(std::integral_constant<bool, false>{});
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
    int stage = 0;
    if (t0 < kend) dma_tile(t0, 0);
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
    // Probability half-tiles: key k of half h (k - 32 h in 0..31) of row r at
    // column (k & 3) * 8 + ((k >> 2) & 7), so that the A operand of P.V step
    // h (row qi, keys 32 h + 4 e + gq, e = 0..7) is 8 consecutive floats; the
    // 4-float chunks of row r are permuted by chunk ^ ((r >> 1) & 7), which
    // puts the 16 rows of a 16-byte read on 16 distinct bank groups.
    auto pswz = [](int r) { return 4 * ((r >> 1) & 7); };
    const int swr = pswz(qi);

    for (; t0 < kend; t0 += kTile, stage ^= 1) {
        const int nk = nk_at(t0);
        waitcnt_vm<0>();  // this wave's share of the tile's DMA has landed
        __syncthreads();  // the whole tile is in LDS; every wave is done with the other stage
        if (t0 + kTile < kend) dma_tile(t0 + kTile, stage ^ 1);
        if (nr == 0) continue;
        const uint32_t *const sK = stK + stage * RS::TILE_DW;
        const uint32_t *const sV = stV + stage * RS::TILE_DW;

        // ---- scores on the matrix cores
        float sv[4][4];
        mfma_scores<D, RB>(sK, qhi, qlo, lane, sv);
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
        float pv[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                pv[kb][i] = __builtin_amdgcn_exp2f(sv[kb][i] - mex[i]);
                ps += pv[kb][i];
            }
            lrow[i] += ps;
        }

        // ---- P.V on the matrix cores, one 32-key half at a time: the half's
        // probabilities go to LDS, then its A operands come back in the
        // matrix-core layout; B operands are 16-byte V row reads (lane (gq,
        // qi) holds dims 8 qi .. 8 qi + 7 of key 4 s + gq, s = 0..15)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * (lane >> 4) + i;
#pragma unroll
                for (int kb = 2 * h; kb < 2 * h + 2; ++kb) {
                    const int kk = 16 * (kb & 1) + qi;  // key within the half
                    sPw[row * RS::HALF_P + (((kk & 3) * 8 + (kk >> 2)) ^ pswz(row))] = pv[kb][i];
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            rkv_half8 ph, pl;
            {
                const float4 a = *(const float4 *)&sPw[qi * RS::HALF_P + ((gq * 8) ^ swr)];
                const float4 b = *(const float4 *)&sPw[qi * RS::HALF_P + ((gq * 8 + 4) ^ swr)];
                const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const _Float16 hh = (_Float16)x[e];
                    ph[e] = hh;
                    pl[e] = (_Float16)(x[e] - (float)hh);
                }
            }
            uint32_t vr[8][4];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const uint4 x = *(const uint4 *)(sV + (4 * (8 * h + s) + gq) * (RB / 4) + 4 * qi);
                vr[s][0] = x.x;
                vr[s][1] = x.y;
                vr[s][2] = x.z;
                vr[s][3] = x.w;
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                uint32_t bw[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2)
                    bw[e2] = __builtin_amdgcn_perm(vr[2 * e2 + 1][c >> 1], vr[2 * e2][c >> 1],
                                                   (c & 1) ? 0x07060302u : 0x05040100u);
                const rkv_half8 bv = __builtin_bit_cast(rkv_half8, bw);
                oc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, bv, oc[c], 0, 0, 0);
                oc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, bv, oc[c], 0, 0, 0);
            }
            // (the second half's stores wait for this half's reads: same wave, LDS order)
            __builtin_amdgcn_sched_barrier(0);
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
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * (lane >> 4) + i;
        int rr = -1;
        float lr = 1.f;
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            rr = row == r ? tabrow[r] : rr;
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
            rr = lane == r ? tabrow[r] : rr;
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
