// attend_kernel.h -- split-K flash-decode kernel for one segment of the cache.
//
// One wave (64 lanes) = one work item: a KV head g, a group of RT query rows
// that attend g (all GQA rows of g, and for a segment shared by every
// sequence, those rows of every sequence), and a contiguous range of the
// segment's keys.  The wave walks its range in tiles of 64 keys:
//
//   1. the K rows of the tile (and V rows when they are block-quantised or
//      wide) are copied with coalesced vector loads into LDS, row by row, at
//      an odd dword stride so that one-row-per-lane reads hit distinct banks;
//      f16 V rows of up to 128 values go straight to registers instead;
//   2. scores, one key per lane: each lane reads its key's row from LDS,
//      dequantises it in registers (f32 / f16 / q8_0 / q4_0; the q8_0 / q4_0
//      block scale is applied once per 32-value partial dot) and takes the
//      dot product with the RT query rows, whose values are wave-uniform and
//      live in scalar registers; then scale and the optional softcap;
//   3. online softmax over the tile: wave max per row, rescale of the running
//      state, p = 2^(s - m) (scores are kept in log2 units);
//   4. P.V: lanes are (key-in-step, 8-dim group); each lane accumulates its 8
//      dims for every row over the tile's keys.
//
// At the end of its range the wave writes its partial (m, l, acc[D]) per row;
// a second, fixed-order pass merges the partials of all ranges (the same
// LSE arithmetic as the segment combine), so results are deterministic.
//
// This is the in-register reading of window and tail at their own types that
// "F5 M7 -- Rolling KV" ships (section "2026-07-12 -- #582-P2 SHIPPED"), with
// the running max and denominator carried in F32 across tiles ("Architecture",
// "CUDA stream graph": flash attention's exact math over rotating key chunks).
#pragma once

#include "common.h"

namespace rkv {

__host__ __device__ constexpr int odd_dwords(int n) { return (n & 1) ? n : n + 1; }

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// (hi:lo) >> (8 * sh), low 32 bits.
__device__ __forceinline__ uint32_t funnel(uint32_t lo, uint32_t hi, uint32_t sh)
{
    return __builtin_amdgcn_alignbyte(hi, lo, sh);
}

__device__ __forceinline__ float h2f(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
}

__device__ __forceinline__ float sbyte(uint32_t w, int k) { return (float)(int)(int8_t)(uint8_t)(w >> (8 * k)); }

__device__ __forceinline__ float nib(uint32_t w, int shift) { return (float)((int)((w >> shift) & 0xfu) - 8); }

// Copy the rows of a tile (row i of RB bytes at src + i*pos_stride) into LDS
// at a stride of LS dwords, with VW-byte loads, in rounds of at most 32 loads
// per lane that are all in flight before the round's LDS stores.  Rows past
// nk repeat row nk-1 (their results are masked), so no load is predicated:
// predicated loads would keep one exec mask per load live in scalar registers.
template <int RB, int VW, int LS>
__device__ __forceinline__ void stage_rows(const uint8_t *__restrict__ src, int pos_stride, int nk,
                                           uint32_t *lds, int lane)
{
    // the stride passes through an empty asm so that the per-iteration row
    // offsets are recomputed here instead of being hoisted out of the key loop
    asm volatile("" : "+s"(pos_stride));
    constexpr int CPR = RB / VW;
    constexpr int NCH = kTile * CPR;  // a multiple of 64
    constexpr int NW = VW / 4;
    constexpr int IT = NCH / 64;
    constexpr int ROUND = IT < 32 ? IT : 32;
    static_assert(NCH % 64 == 0, "tile chunks must fill whole waves");
#pragma unroll
    for (int it0 = 0; it0 < IT; it0 += ROUND) {
        uint32_t buf[ROUND][NW];
#pragma unroll
        for (int i = 0; i < ROUND; ++i) {
            const int c = lane + 64 * (it0 + i);
            const int row = c / CPR, col = c - (c / CPR) * CPR;
            const int rowc = row < nk ? row : nk - 1;
            if (it0 + i < IT) {
                const uint8_t *p = src + (uint32_t)(rowc * pos_stride + col * VW);
                if constexpr (NW == 4) {
                    uint4 x = *(const uint4 *)p;
                    buf[i][0] = x.x; buf[i][1] = x.y; buf[i][2] = x.z; buf[i][3] = x.w;
                } else if constexpr (NW == 2) {
                    uint2 x = *(const uint2 *)p;
                    buf[i][0] = x.x; buf[i][1] = x.y;
                } else {
                    buf[i][0] = *(const uint32_t *)p;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < ROUND; ++i) {
            const int c = lane + 64 * (it0 + i);
            const int row = c / CPR, col = c - (c / CPR) * CPR;
            if (it0 + i < IT) {
#pragma unroll
                for (int e = 0; e < NW; ++e) lds[row * LS + col * NW + e] = buf[i][e];
            }
        }
    }
}

// QC consecutive dims [d0, d0 + QC) of this lane's K row in LDS as floats
// (block types: the codes, without the block scale).  QC is 1, 2, 4 or 8 and
// d0 a multiple of QC, so a chunk never straddles a 32-value block.
template <int KT, int QC>
__device__ __forceinline__ void k_chunk(const uint32_t *row, int d0, float *k)
{
    if constexpr (KT == kF32) {
#pragma unroll
        for (int e = 0; e < QC; ++e) k[e] = __builtin_bit_cast(float, row[d0 + e]);
    } else if constexpr (KT == kF16) {
        if constexpr (QC == 1) {
            const uint32_t w = row[d0 / 2];
            k[0] = (d0 & 1) ? h2f(w >> 16) : h2f(w);
        } else {
#pragma unroll
            for (int e = 0; e < QC / 2; ++e) {
                const uint32_t w = row[d0 / 2 + e];
                k[2 * e] = h2f(w);
                k[2 * e + 1] = h2f(w >> 16);
            }
        }
    } else {
        // q8_0: element c of block bb is byte 34*bb + 2 + c.
        // q4_0: element c of block bb is the low (c < 16) or high nibble of byte 18*bb + 2 + (c & 15).
        constexpr int ND = QC >= 4 ? QC / 4 : 1;  // dwords of codes
        const int bb = d0 >> 5, c = d0 & 31;
        const int o = KT == kQ8 ? 34 * bb + 2 + c : 18 * bb + 2 + (c & 15);
        const int w0 = o >> 2;
        const uint32_t sh = o & 3;
        uint32_t A[ND + 1];
#pragma unroll
        for (int i = 0; i <= ND; ++i) A[i] = row[w0 + i];
#pragma unroll
        for (int j = 0; j < ND; ++j) {
            const uint32_t w = funnel(A[j], A[j + 1], sh);
#pragma unroll
            for (int b = 0; b < (QC < 4 ? QC : 4); ++b)
                k[4 * j + b] = KT == kQ8 ? sbyte(w, b) : nib(w, 8 * b + ((c >> 4) << 2));
        }
    }
}

// The binary16 scale of block bb of a q8_0 / q4_0 row in LDS.
template <int KT>
__device__ __forceinline__ float k_scale(const uint32_t *row, int bb)
{
    const int o = (KT == kQ8 ? 34 : 18) * bb;
    const uint32_t w = row[o >> 2];
    return h2f((o & 2) ? (w >> 16) : w);
}

// QC query values of every row, dims [d0, d0 + QC), into scalar registers.
// The offset passes through an empty asm so that the compiler treats each
// chunk's loads as new: without it, the loads of all RT * head_dim values are
// hoisted out of the key loop and spill.
template <int RT, int QC>
__device__ __forceinline__ void q_chunk(const float *q, const int *qoff, int d0, float (*qv)[QC])
{
    int o = d0;
    asm volatile("" : "+s"(o));
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int e = 0; e < QC; ++e) qv[r][e] = q[qoff[r] + o + e];
}

// Empty asm statements that pin values in place: the compiler may not move a
// memory access across them, and a value passed through one is defined there.
template <int N>
__device__ __forceinline__ void pin_s(float *v)
{
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+s"(v[i]));
}
template <int N>
__device__ __forceinline__ void pin_v(float *v)
{
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

// Scores of one key (this lane's row in LDS) against RT query rows:
// s[r] = sum_d q[r][d] * k[d] (unscaled).  Query values are wave-uniform and
// stream through scalar registers QC dims at a time, software pipelined: the
// loads of chunk i+1 are issued before the multiply-adds of chunk i, and the
// pins keep at most two chunks (2 * RT * QC scalar registers) live.  Block
// types apply their scale once per 32-value partial dot.
template <int KT, int D, int RT>
__device__ __forceinline__ void key_dots(const uint32_t *row, const float *q, const int *qoff, float *s)
{
    constexpr int QC = RT >= 16 ? 1 : RT >= 8 ? 2 : RT >= 4 ? 4 : 8;
    constexpr int CPB = 32 / QC;  // chunks per 32-value block
    constexpr int NB = D / 32;
    constexpr int UNR = NB <= 4 ? NB : 2;
    constexpr bool BLOCKS = KT == kQ8 || KT == kQ4;
#pragma unroll
    for (int r = 0; r < RT; ++r) s[r] = 0.f;
#pragma unroll UNR
    for (int bb = 0; bb < NB; ++bb) {
        float qa[RT][QC], qb[RT][QC], ka[QC], kb[QC], t[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) t[r] = 0.f;
        q_chunk<RT, QC>(q, qoff, 32 * bb, qa);
        k_chunk<KT, QC>(row, 32 * bb, ka);
#pragma unroll
        for (int ci = 0; ci < CPB; ++ci) {
            if (ci + 1 < CPB) {
                q_chunk<RT, QC>(q, qoff, 32 * bb + QC * (ci + 1), qb);
                k_chunk<KT, QC>(row, 32 * bb + QC * (ci + 1), kb);
            }
            pin_s<RT * QC>(&qa[0][0]);
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int e = 0; e < QC; ++e) t[r] = fmaf(qa[r][e], ka[e], t[r]);
            pin_v<RT>(t);
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int e = 0; e < QC; ++e) qa[r][e] = qb[r][e];
#pragma unroll
            for (int e = 0; e < QC; ++e) ka[e] = kb[e];
        }
        if constexpr (BLOCKS) {
            const float dsc = k_scale<KT>(row, bb);
#pragma unroll
            for (int r = 0; r < RT; ++r) s[r] = fmaf(dsc, t[r], s[r]);
        } else {
#pragma unroll
            for (int r = 0; r < RT; ++r) s[r] += t[r];
        }
    }
}

// 8 consecutive values (dims 8*dg .. 8*dg+7) of a V row held in LDS, as
// floats, plus the block scale they must be multiplied by (1 for f32/f16).
template <int VT, int D>
__device__ __forceinline__ float v_group_lds(const uint32_t *row, int dg, float *x)
{
    if constexpr (VT == kF32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = __builtin_bit_cast(float, row[8 * dg + e]);
        return 1.f;
    } else if constexpr (VT == kF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t w = row[4 * dg + e];
            x[2 * e] = h2f(w);
            x[2 * e + 1] = h2f(w >> 16);
        }
        return 1.f;
    } else if constexpr (VT == kQ8) {
        const int bb = dg >> 2, h = dg & 3;
        const int os = 34 * bb;
        const uint32_t sw = row[os >> 2];
        const float dsc = h2f((os & 2) ? (sw >> 16) : sw);
        const int o = os + 2 + 8 * h;
        const uint32_t sh = o & 3;
        const uint32_t A = row[o >> 2], B = row[(o >> 2) + 1], C = row[(o >> 2) + 2];
        const uint32_t w0 = funnel(A, B, sh), w1 = funnel(B, C, sh);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[k] = sbyte(w0, k);
            x[4 + k] = sbyte(w1, k);
        }
        return dsc;
    } else {  // kQ4: dims 8h..8h+7 of the block = low (h < 2) or high nibbles of bytes 8(h&1) ..
        const int bb = dg >> 2, h = dg & 3;
        const int os = 18 * bb;
        const uint32_t sw = row[os >> 2];
        const float dsc = h2f((os & 2) ? (sw >> 16) : sw);
        const int o = os + 2 + 8 * (h & 1);
        const uint32_t sh = o & 3;
        const uint32_t A = row[o >> 2], B = row[(o >> 2) + 1], C = row[(o >> 2) + 2];
        const uint32_t w0 = funnel(A, B, sh), w1 = funnel(B, C, sh);
        const int base = (h >> 1) * 4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[k] = nib(w0, 8 * k + base);
            x[4 + k] = nib(w1, 8 * k + base);
        }
        return dsc;
    }
}

template <int KT, int VT, int D, int RT>
__global__ void __launch_bounds__(64)
rkv_split_kernel(const float *__restrict__ q, const uint8_t *__restrict__ kbase, const uint8_t *__restrict__ vbase,
                 float *__restrict__ part_acc, float2 *__restrict__ part_ml, const SplitParams p)
{
    constexpr int RBK = row_bytes_of(KT, D);
    constexpr int RBV = row_bytes_of(VT, D);
    constexpr int VWK = load_width_of(KT, D);
    constexpr int VWV = load_width_of(VT, D);
    constexpr int LSK = odd_dwords(RBK / 4);
    constexpr int LPR = D / 8;      // lanes per V row in the P.V phase
    constexpr int KPS = 64 / LPR;   // keys per P.V step
    constexpr int NSTEP = kTile / KPS;
    constexpr bool V_REG = (VT == kF16 && D <= 128) || (VT == kF32 && D <= 64);
    constexpr int LSV = V_REG ? 1 : odd_dwords(RBV / 4);
    constexpr int VRW = VT == kF32 ? 8 : 4;  // dwords of one lane's 8 values, register path

    __shared__ uint32_t sK[kTile * LSK + 4];
    __shared__ uint32_t sV[V_REG ? 1 : kTile * LSV + 4];
    __shared__ float sP[RT * kTile];

    const int lane = threadIdx.x;
    const int g = blockIdx.y / p.n_rg;
    const int rg = blockIdx.y - g * p.n_rg;
    const int cnt = (int)p.rowcnt[g] - rg * RT;
    if (cnt <= 0) return;
    const int nr = cnt < RT ? cnt : RT;
    const int z = blockIdx.z;
    const int64_t kbeg = (int64_t)blockIdx.x * p.keys_per_split;
    const int64_t kend = kbeg + p.keys_per_split < p.n_keys ? kbeg + p.keys_per_split : p.n_keys;

    const uint8_t *kg = kbase + z * p.k_seq + g * p.k_head;
    const uint8_t *vg = vbase + z * p.v_seq + g * p.v_head;

    int rid[RT], qoff[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int rr = r < nr ? r : nr - 1;  // padding rows repeat the last row; never written
        rid[r] = z * p.z_row_step + p.rowtab[g * p.rows_per_g + rg * RT + rr];
        qoff[r] = rid[r] * D;
    }

    float m[RT], l[RT], acc[RT][8];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
    }

    const int ks = lane / LPR;
    const int dg = lane - ks * LPR;
    const float sl2 = p.scale_log2;
    const float cap = p.softcap;
    constexpr float kLog2e = 1.4426950408889634f;

    for (int64_t t0 = kbeg; t0 < kend; t0 += kTile) {
        const int nk = (int)(kend - t0 < kTile ? kend - t0 : kTile);

        uint32_t vreg[V_REG ? NSTEP : 1][V_REG ? VRW : 1];
        if constexpr (V_REG) {
            int vps = (int)p.v_pos;
            asm volatile("" : "+s"(vps));
            const uint8_t *vt = vg + t0 * p.v_pos;
#pragma unroll
            for (int st = 0; st < NSTEP; ++st) {
                const int key = st * KPS + ks;
                const int keyc = key < nk ? key : nk - 1;  // masked in P.V
                const uint8_t *pv = vt + (uint32_t)(keyc * vps + dg * (VRW * 4));
                const uint4 a = *(const uint4 *)pv;
                vreg[st][0] = a.x; vreg[st][1] = a.y; vreg[st][2] = a.z; vreg[st][3] = a.w;
                if constexpr (VRW == 8) {
                    const uint4 b = *(const uint4 *)(pv + 16);
                    vreg[st][4] = b.x; vreg[st][5] = b.y; vreg[st][6] = b.z; vreg[st][7] = b.w;
                }
            }
        }
        stage_rows<RBK, VWK, LSK>(kg + t0 * p.k_pos, (int)p.k_pos, nk, sK, lane);
        if constexpr (!V_REG) stage_rows<RBV, VWV, LSV>(vg + t0 * p.v_pos, (int)p.v_pos, nk, sV, lane);
        __syncthreads();

        // ---- scores, one key per lane
        float s[RT];
        key_dots<KT, D, RT>(sK + lane * LSK, q, qoff, s);
        const bool valid = lane < nk;
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            float x;
            if (cap > 0.f)
                x = cap * tanhf(s[r] * p.scale / cap) * kLog2e;
            else
                x = s[r] * sl2;
            s[r] = valid ? x : -INFINITY;
        }

        // ---- online softmax update
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const float mt = wave_max(s[r]);
            const float mn = fmaxf(m[r], mt);
            const float alpha = exp2f(m[r] - mn);
            const float pr = exp2f(s[r] - mn);
            l[r] = l[r] * alpha + pr;
            m[r] = mn;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
            sP[r * kTile + lane] = pr;
        }
        __syncthreads();

        // ---- P.V (fully unrolled when V sits in registers: vreg is indexed by st)
#pragma unroll V_REG ? NSTEP : 4
        for (int st = 0; st < NSTEP; ++st) {
            const int key = st * KPS + ks;
            const bool kv = key < nk;
            float x[8];
            float dsc;
            if constexpr (V_REG) {
                if constexpr (VT == kF16) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[2 * e] = h2f(vreg[st][e]);
                        x[2 * e + 1] = h2f(vreg[st][e] >> 16);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = __builtin_bit_cast(float, vreg[st][e]);
                }
                dsc = 1.f;
            } else {
                dsc = v_group_lds<VT, D>(sV + key * LSV, dg, x);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = kv ? x[e] : 0.f;
            dsc = kv ? dsc : 0.f;
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const float pw = sP[r * kTile + key] * dsc;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(pw, x[e], acc[r][e]);
            }
        }
        __syncthreads();
    }

    // ---- partial of this key range
#pragma unroll
    for (int r = 0; r < RT; ++r) l[r] = wave_sum(l[r]);
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[r][e] += __shfl_xor(acc[r][e], off);
    }
    const int64_t base = (int64_t)blockIdx.x * p.n_rows_total;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        if (r < nr) {
            if (ks == 0) {
                float4 *dst = (float4 *)(part_acc + (base + rid[r]) * D + dg * 8);
                dst[0] = make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
                dst[1] = make_float4(acc[r][4], acc[r][5], acc[r][6], acc[r][7]);
            }
            if (lane == 0) part_ml[base + rid[r]] = make_float2(m[r], l[r]);
        }
    }
}

}  // namespace rkv
