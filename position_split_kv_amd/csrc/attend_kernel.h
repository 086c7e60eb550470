// attend_kernel.h -- split-K flash-decode kernel for one segment of the cache.
//
// A workgroup of NW waves owns a key range of a segment and HPW KV heads
// (HPW a power of two, chosen at launch; NW / HPW = WPH waves per head).  For
// its head g each wave owns a group of RT query rows that attend g (all GQA
// rows of g, and for a segment shared by every sequence, those rows of every
// sequence).  The waves of a head walk tiles ws, ws+WPH, ws+2WPH, ... of the
// range (ws = the wave's index among them), 64 keys per tile.  With HPW > 1
// the waves of one workgroup read neighbouring heads' rows of the same
// positions at the same time, so each position is read as one contiguous
// span: that is what lets the position-major cache stream at the HBM rate
// (reading one head's slice of every position from separate workgroups runs
// about a third slower).  Per tile:
//
//   1. the K rows of the tile (and V rows when they are block-quantised or
//      wide) are copied with coalesced vector loads into the wave's LDS area,
//      row by row, at a padded stride so that one-row-per-lane reads do not
//      collide in LDS banks; f16 V rows of up to 128 values go straight to
//      registers instead;
//   2. scores, one key per lane: each lane reads its key's row from LDS,
//      dequantises it in registers (f32 / f16 / q8_0 / q4_0; the q8_0 / q4_0
//      block scale is applied once per 32-value partial dot) and takes the
//      dot product with the RT query rows, whose values are wave-uniform and
//      stream through scalar registers; then scale and the optional softcap;
//   3. online softmax over the tile: wave max per row (DPP), rescale of the
//      running state only when the max moved, p = 2^(s - m) (scores are kept
//      in log2 units);
//   4. P.V: lanes are (key-in-step, 8-dim group); each lane accumulates its 8
//      dims for every row over the tile's keys.
//
// At the end the waves of each head merge their (m, l, acc) in LDS.  A launch
// that is one workgroup per work item writes its normalised output and LSE
// directly; otherwise each workgroup writes a partial and a second,
// fixed-order kernel merges them (the same LSE arithmetic as the segment
// combine), so the results are deterministic.  (A merge by the last
// workgroup to finish was measured slower: handing partials between
// workgroups inside a kernel needs device-scope release fences, which write
// back the L2 of each XCD.)
//
// This is the in-register reading of window and tail at their own types that
// "F5 M7 -- Rolling KV" ships (section "2026-07-12 -- #582-P2 SHIPPED"), with
// the running max and denominator carried in F32 across tiles ("Architecture",
// "CUDA stream graph": flash attention's exact math over rotating key chunks).
#pragma once

#include <type_traits>

#include "common.h"

namespace rkv {

__host__ __device__ constexpr int odd_dwords(int n) { return (n & 1) ? n : n + 1; }

// LDS row stride (dwords) of a staged row of rb bytes: rows that are a
// multiple of 16 bytes keep 16-byte alignment and get 16 bytes of padding
// (b128 reads by 16 consecutive lanes then hit distinct banks); other rows get
// an odd dword count (b32 reads by consecutive lanes hit distinct banks).
__host__ __device__ constexpr int lds_row_dwords(int rb) { return rb % 16 == 0 ? rb / 4 + 4 : odd_dwords(rb / 4); }

__host__ __device__ constexpr bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

template <int KT, int VT, int D>
struct Shape {
    static constexpr int RBK = row_bytes_of(KT, D);
    static constexpr int RBV = row_bytes_of(VT, D);
    // f32 / f16 K rows of 128..512 bytes go global -> LDS directly (no staging
    // registers), packed at RBK bytes with their 16-byte chunks swizzled.
    static constexpr bool KDMA = (KT == kF32 || KT == kF16) && RBK >= 128 && RBK <= 512 && is_pow2(RBK / 16);
    static constexpr int LSK = KDMA ? RBK / 4 : lds_row_dwords(RBK);
    static constexpr bool V_REG = (VT == kF16 && D <= 128) || (VT == kF32 && D <= 64);
    // q4_0 V rows at 128 dims: 22 dwords instead of 19, so that the P.V
    // operand reads (a block scale and three code words per lane, 16 lanes
    // on each of two rows per half-wave) meet no bank twice.  (With q4_0 K
    // the wider rows would cost workgroups per compute unit; kept at 19.)
    static constexpr int LSV = V_REG                                      ? 0
                               : (VT == kQ4 && D == 128 && KT != kQ4) ? 22
                                                                          : lds_row_dwords(RBV);
    static constexpr int STAGE_DW = kTile * (LSK + LSV) + 8;  // per wave: K (+ V) rows plus read slack
    // With K rows by DMA and V rows in registers, a wave's K tile is not
    // needed between its scores and the next tile's DMA (issued after P.V),
    // so the score rows P of the tile live there (up to 16 rows of 64 keys).
    static constexpr bool P_IN_K = KDMA && V_REG;
    static_assert(!P_IN_K || LSK >= 16, "the K tile holds 16 score rows");
    // LDS bytes of a workgroup of nw waves with rt rows each: the staging
    // areas (reused for the final merge) and the score rows
    static constexpr int lds_bytes(int nw, int rt)
    {
        return 4 * (nw * STAGE_DW > nw * rt * (D + 2) ? nw * STAGE_DW : nw * rt * (D + 2)) +
               (P_IN_K ? 0 : 4 * nw * rt * kTile) + (VT == kT3 ? 512 : 0);
    }
    // waves per workgroup: as many (up to 8) as fit 160 KiB of LDS
    static constexpr int waves(int rt)
    {
        return lds_bytes(8, rt) <= 160 * 1024 ? 8 : lds_bytes(4, rt) <= 160 * 1024 ? 4 : lds_bytes(2, rt) <= 160 * 1024 ? 2 : 1;
    }
};

// ---------------------------------------------------------------- small helpers

// (hi:lo) >> (8 * sh), low 32 bits.
__device__ __forceinline__ uint32_t funnel(uint32_t lo, uint32_t hi, uint32_t sh)
{
    return __builtin_amdgcn_alignbyte(hi, lo, sh);
}

__device__ __forceinline__ float h2f(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
}

// tanh(y) from the identity tanh(y) = 1 - 2 / (e^(2y) + 1), given
// two_y_log2 = 2y log2(e): one hardware exp2, one reciprocal, no branches.
// e^(2y) overflowing to +inf gives 1, underflowing to 0 gives -1.  The
// absolute error is a few units of 2^-24 (the softcap scales it by the cap).
__device__ __forceinline__ float tanh_from_exp2(float two_y_log2)
{
    const float t = __builtin_amdgcn_exp2f(two_y_log2);
    return fmaf(-2.f, __builtin_amdgcn_rcpf(t + 1.f), 1.f);
}

// Softcap (CAP) and mask (MASK) of NKB 16-key blocks of a score tile in the
// matrix-core output layout: sv[kb][i] holds tile key key0 + 16 kb of the
// lane's output row i (scores in log2 units); with MASK, keys past kmx[i]
// become -inf.  Both are template arguments: the caller branches once per
// tile on the uniform cap and on whether the tile needs a mask (a causal
// mask, or a tile shorter than kTile), so that a whole unmasked tile without
// a cap costs nothing here.
template <bool CAP, bool MASK, int NKB>
__device__ __forceinline__ void cap_mask_tile(float (&sv)[NKB][4], const int (&kmx)[4], int key0, float capl,
                                              float two_over_cap)
{
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        const int key = key0 + 16 * kb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x = sv[kb][i];
            // (s/c = x/capl, and 2 (s/c) log2 e = x * 2/c)
            if constexpr (CAP) x = capl * tanh_from_exp2(x * two_over_cap);
            if constexpr (MASK) x = key <= kmx[i] ? x : -INFINITY;
            sv[kb][i] = x;
        }
    }
}

__device__ __forceinline__ float sbyte(uint32_t w, int k) { return (float)(int)(int8_t)(uint8_t)(w >> (8 * k)); }

__device__ __forceinline__ float nib(uint32_t w, int shift) { return (float)((int)((w >> shift) & 0xfu) - 8); }

// One step of a DPP butterfly: x = op(x, x from the lane the control selects),
// only in the rows of row_mask (other rows keep x).  The s_nop covers the
// VALU-write-then-DPP-read hazard of the value just computed.
#define RKV_DPP_MAX(x, ctrl, rmask) \
    asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 " ctrl " row_mask:" rmask " bank_mask:0xf" : "+v"(x))
#define RKV_DPP_ADD(x, ctrl, rmask) \
    asm("s_nop 1\n\tv_add_f32_dpp %0, %0, %0 " ctrl " row_mask:" rmask " bank_mask:0xf" : "+v"(x))

// Maximum over the 64 lanes, returned wave-uniform.
__device__ __forceinline__ float wave_max(float x)
{
    RKV_DPP_MAX(x, "quad_perm:[1,0,3,2]", "0xf");
    RKV_DPP_MAX(x, "quad_perm:[2,3,0,1]", "0xf");
    RKV_DPP_MAX(x, "row_half_mirror", "0xf");
    RKV_DPP_MAX(x, "row_mirror", "0xf");
    RKV_DPP_MAX(x, "row_bcast:15", "0xa");
    RKV_DPP_MAX(x, "row_bcast:31", "0xc");
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Sum over the 64 lanes, returned wave-uniform.
__device__ __forceinline__ float wave_sum(float x)
{
    RKV_DPP_ADD(x, "quad_perm:[1,0,3,2]", "0xf");
    RKV_DPP_ADD(x, "quad_perm:[2,3,0,1]", "0xf");
    RKV_DPP_ADD(x, "row_half_mirror", "0xf");
    RKV_DPP_ADD(x, "row_mirror", "0xf");
    RKV_DPP_ADD(x, "row_bcast:15", "0xa");
    RKV_DPP_ADD(x, "row_bcast:31", "0xc");
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// ---------------------------------------------------------------- staging

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
    constexpr int NWD = VW / 4;
    constexpr int IT = NCH / 64;
    constexpr int ROUND = IT < 32 ? IT : 32;
    static_assert(NCH % 64 == 0, "tile chunks must fill whole waves");
#pragma unroll
    for (int it0 = 0; it0 < IT; it0 += ROUND) {
        uint32_t buf[ROUND][NWD];
#pragma unroll
        for (int i = 0; i < ROUND; ++i) {
            const int c = lane + 64 * (it0 + i);
            const int row = c / CPR, col = c - (c / CPR) * CPR;
            const int rowc = row < nk ? row : nk - 1;
            if (it0 + i < IT) {
                const uint8_t *p = src + (uint32_t)(rowc * pos_stride + col * VW);
                if constexpr (NWD == 4) {
                    uint4 x = *(const uint4 *)p;
                    buf[i][0] = x.x; buf[i][1] = x.y; buf[i][2] = x.z; buf[i][3] = x.w;
                } else if constexpr (NWD == 2) {
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
                uint32_t *dst = lds + row * LS + col * NWD;
                if constexpr (NWD == 4 && LS % 4 == 0) {
                    *(uint4 *)dst = make_uint4(buf[i][0], buf[i][1], buf[i][2], buf[i][3]);
                } else {
#pragma unroll
                    for (int e = 0; e < NWD; ++e) dst[e] = buf[i][e];
                }
            }
        }
    }
}

// The raw bytes of a tile's rows held in registers between their global
// loads and their LDS stores: chunk c = lane + 64*i of VW bytes, row c / CPR.
template <int RB, int VW>
struct RowRegs {
    static constexpr int CPR = RB / VW, NWD = VW / 4, IT = kTile * CPR / 64;
    uint32_t d[IT][NWD];
};

// Issue the loads of a tile's rows (rows past nk repeat row nk-1, so no load
// is predicated).
template <int RB, int VW>
__device__ __forceinline__ void load_rows(RowRegs<RB, VW> &R, const uint8_t *__restrict__ src, int pos_stride,
                                          int nk, int lane)
{
    using T = RowRegs<RB, VW>;
    asm volatile("" : "+s"(pos_stride));
#pragma unroll
    for (int i = 0; i < T::IT; ++i) {
        const int c = lane + 64 * i;
        const int row = c / T::CPR, col = c - (c / T::CPR) * T::CPR;
        const int rowc = row < nk ? row : nk - 1;
        const uint8_t *ptr = src + (uint32_t)(rowc * pos_stride + col * VW);
        if constexpr (T::NWD == 4) {
            const uint4 x = *(const uint4 *)ptr;
            R.d[i][0] = x.x; R.d[i][1] = x.y; R.d[i][2] = x.z; R.d[i][3] = x.w;
        } else if constexpr (T::NWD == 2) {
            const uint2 x = *(const uint2 *)ptr;
            R.d[i][0] = x.x; R.d[i][1] = x.y;
        } else {
            R.d[i][0] = *(const uint32_t *)ptr;
        }
    }
}

// Store loaded rows to LDS at a stride of LS dwords.
template <int RB, int VW, int LS>
__device__ __forceinline__ void store_rows(const RowRegs<RB, VW> &R, uint32_t *lds, int lane)
{
    using T = RowRegs<RB, VW>;
#pragma unroll
    for (int i = 0; i < T::IT; ++i) {
        const int c = lane + 64 * i;
        const int row = c / T::CPR, col = c - (c / T::CPR) * T::CPR;
        uint32_t *dst = lds + row * LS + col * T::NWD;
        if constexpr (T::NWD == 4 && LS % 4 == 0) {
            *(uint4 *)dst = make_uint4(R.d[i][0], R.d[i][1], R.d[i][2], R.d[i][3]);
        } else {
#pragma unroll
            for (int e = 0; e < T::NWD; ++e) dst[e] = R.d[i][e];
        }
    }
}

// Chunk swizzle of a DMA-staged K row: chunk c of row j sits in slot
// c ^ kswz(j).  It makes the 16-byte reads of one chunk by 16 consecutive
// lanes (one row each) hit 16 distinct 4-bank groups.
template <int RB>
__device__ __forceinline__ int kswz(int j)
{
    return RB == 128 ? ((j >> 1) & 7) : (j & 15);
}

// ---------------------------------------------------------------- dma k rows

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// One direct global -> LDS load: the 16 bytes at g (per lane) land at LDS
// address lds + OFF + 16 * lane (the constant OFF is added to M0 inside the
// asm, so that no per-load LDS address is held in a scalar register across a
// tile loop).  Written as asm so that the compiler neither
// inserts its own (conservative or missing) waits for it nor reorders memory
// accesses across it; callers wait with waitcnt_vm() before reading the data
// and wait for their LDS reads (lgkmcnt) before overwriting a buffer.  M0 is
// saved and restored around the load.  When each 16-byte chunk is read
// exactly once by the launch (one row group per KV head), every load takes
// whole cache lines and carries the non-temporal cache policy (NT): on the
// 48-layer f16 step 2.5 % less time than the default policy.  When several
// row groups read the same tile, the default policy keeps it in L2 for the
// others (a verify step of 40 rows per head: 106 -> 94 us).  (The 4-byte
// loads below touch each line from several loads and keep the default: with
// nt they were up to 15 % slower.)
template <bool NT, uint32_t OFF = 0>
__device__ __forceinline__ void lds_dma16(const void *g, uint32_t lds)
{
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t saved;
    if constexpr (NT)
        asm volatile("s_mov_b32 %0, m0\n\ts_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
                     : "=&s"(saved)
                     : "v"(g), "s"(lds), "i"(OFF)
                     : "memory");
    else
        asm volatile("s_mov_b32 %0, m0\n\ts_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                     : "=&s"(saved)
                     : "v"(g), "s"(lds), "i"(OFF)
                     : "memory");
#else
    (void)g;
    (void)lds;
#endif
}

// f(std::integral_constant<int, i>) for i = I .. N-1 (an unrolled loop whose
// index is a compile-time constant)
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Groups of G (1, 2 or 4) sixteen-byte direct-to-LDS buffer loads under one
// M0 setting: load j of a group reads at voff[j] + so_j + 1024 j and lands at
// LDS m0 + 1024 j + 16 lane (the immediate offset advances both addresses),
// with so_0 = so and so_(j+1) = so_j + st (one scalar add per load).  The
// per-load LDS addresses are immediates inside the asm, so none of them is
// held in a scalar register across a loop.
#define RKV_X4_GRP(NTS, BODY)                                                                                        \
    asm volatile("s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[ml]\n\ts_nop 0\n\t"                                        \
                 "buffer_load_dwordx4 %[v0], %[rs], %[so] offen" NTS " lds\n\t" BODY "s_mov_b32 m0, %[sv]"         \
                 : [sv] "=&s"(saved), [so] "+&s"(so)                                                                 \
                 : [v0] "v"(voff[0]), [v1] "v"(voff[G > 1 ? 1 : 0]), [v2] "v"(voff[G > 2 ? 2 : 0]),                \
                   [v3] "v"(voff[G > 3 ? 3 : 0]), [rs] "s"(rs), [ml] "s"(m0v), [st] "s"(st), [o1] "i"(1024),       \
                   [o2] "i"(2048), [o3] "i"(3072)                                                                    \
                 : "memory")
#define RKV_X4_LD(j, NTS) "s_add_u32 %[so], %[so], %[st]\n\tbuffer_load_dwordx4 %[v" #j "], %[rs], %[so] offen offset:%[o" #j "]" NTS " lds\n\t"
template <int G, bool NT>
__device__ __forceinline__ void lds_dma16_grp(__amdgpu_buffer_rsrc_t rs, const uint32_t *voff, uint32_t so, uint32_t st,
                                              uint32_t m0v)
{
    static_assert(G == 1 || G == 2 || G == 4, "group size");
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t saved;
    if constexpr (NT) {
        if constexpr (G == 1)
            RKV_X4_GRP(" nt", "");
        else if constexpr (G == 2)
            RKV_X4_GRP(" nt", RKV_X4_LD(1, " nt"));
        else
            RKV_X4_GRP(" nt", RKV_X4_LD(1, " nt") RKV_X4_LD(2, " nt") RKV_X4_LD(3, " nt"));
    } else {
        if constexpr (G == 1)
            RKV_X4_GRP("", "");
        else if constexpr (G == 2)
            RKV_X4_GRP("", RKV_X4_LD(1, ""));
        else
            RKV_X4_GRP("", RKV_X4_LD(1, "") RKV_X4_LD(2, "") RKV_X4_LD(3, ""));
    }
#else
    (void)rs;
    (void)voff;
    (void)so;
    (void)st;
    (void)m0v;
#endif
}
#undef RKV_X4_LD
#undef RKV_X4_GRP
// Loads [J, N) of a tile copy by lds_dma16_grp: load i reads at
// i * rstep + voff[i] and lands at LDS lds_base + 1024 i.
template <bool NT, int N, int J = 0>
__device__ __forceinline__ void dma16_groups(__amdgpu_buffer_rsrc_t rs, const uint32_t *voff, uint32_t rstep,
                                             uint32_t lds_base)
{
    if constexpr (J < N) {
        constexpr int G = N - J >= 4 ? 4 : N - J >= 2 ? 2 : 1;
        lds_dma16_grp<G, NT>(rs, voff + J, (uint32_t)J * rstep, rstep - 1024u, lds_base + 1024u * J);
        dma16_groups<NT, N, J + G>(rs, voff, rstep, lds_base);
    }
}

// A raw buffer resource for loads at byte offsets (vector + scalar) from a
// uniform base: no stride, no range limit (the offsets are the caller's to
// keep inside the buffer), the data-format word of this GPU family.
typedef uint32_t rkv_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, -1, 0x00020000);
}

// The same for 4 bytes per lane: the dword lands at lds + OFF + 4 * lane.
// The constant OFF is added to M0 inside the asm, so that the compiler does
// not keep one precomputed LDS address per load of a tile in scalar
// registers across the tile loop.
template <uint32_t OFF>
__device__ __forceinline__ void lds_dma4(const void *g, uint32_t lds)
{
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(g), "s"(lds), "i"(OFF)
                 : "memory");
#else
    (void)g;
    (void)lds;
#endif
}

// Direct global -> LDS copy of a tile's kTile rows of RBD dwords (rows past
// nkk repeat row nkk-1) to rows of LS >= RBD dwords: slot s = i*64 + lane of
// load i is dword s % LS of row s / LS (padding slots repeat the row's last
// dword), so the tile takes exactly LS loads.  [I0, I1) selects a range of
// those loads, so that several waves can share one tile's copy.
// (The lane index passes through an empty asm so that the per-slot row and
// column are recomputed here, by an add-and-carry recurrence, instead of being
// hoisted out of the tile loop into registers.)
template <int RBD, int LS, int I, int I1>
__device__ __forceinline__ void dma_rows4_from(const uint8_t *src, int pos_stride, int nkk, uint32_t lds_base, int j,
                                               int c)
{
    if constexpr (I < I1) {
        constexpr int DJ = 64 / LS, DC = 64 % LS;  // slot advance of 64 per load
        const int cc = c < RBD ? c : RBD - 1;
        const int jc = j < nkk ? j : nkk - 1;
        lds_dma4<256u * I>(src + (uint32_t)(jc * pos_stride + 4 * cc), lds_base);
        j += DJ;
        c += DC;
        if (c >= LS) {
            c -= LS;
            ++j;
        }
        dma_rows4_from<RBD, LS, I + 1, I1>(src, pos_stride, nkk, lds_base, j, c);
    }
}
template <int RBD, int LS, int I0 = 0, int I1 = LS>
__device__ __forceinline__ void dma_rows4(const uint8_t *src, int pos_stride, int nkk, uint32_t lds_base, int lane)
{
    static_assert(LS <= 64, "one row per load at least");
    static_assert(0 <= I0 && I0 <= I1 && I1 <= LS, "load range");
    asm volatile("" : "+v"(lane));
    const int s0 = I0 * 64 + lane;
    dma_rows4_from<RBD, LS, I0, I1>(src, pos_stride, nkk, lds_base, s0 / LS, s0 - (s0 / LS) * LS);  // slot of load I0
}

// Slot plan of a whole tile for rows of LS dwords: slot s = i*64 + lane of
// load i sits at byte (s / LS) * P + 4 * (s % LS) of the tile.  From load i to
// i+1 that offset grows by DJ*P + 4*DC (uniform) plus P - 4*LS when the slot
// wraps past a row end; bit i of wrap holds that wrap for the lane, so that
// offset_i = i*(DJ*P + 4*DC) + 4*lane + (lane/LS + wraps before i)*(P - 4*LS).
// Bit i of the plan is set iff (lane mod LS + i * DC) mod LS >= LS - DC.
// Stepping i through every load costs a few VALU per load at the kernel's
// start; when DC has an inverse modulo LS the loads whose column lands on a
// given residue r are i = (r - lane mod LS) * DC^-1 mod LS, so only the
// residues of the smaller class (the DC wrapping ones, or the LS - DC others)
// are visited, each at one add and one conditional subtract.
__host__ __device__ constexpr uint64_t dma_wraps_stepped(int LS, int lane)
{
    const int DC = 64 % LS;
    int c = lane % LS;
    uint64_t wrap = 0;
    for (int i = 0; i + 1 < LS; ++i) {
        if (c >= LS - DC) wrap |= 1ull << i;
        c += DC;
        if (c >= LS) c -= LS;
    }
    return wrap;
}
__host__ __device__ constexpr int dma_wrap_inverse(int LS)
{
    const int DC = 64 % LS;
    for (int x = 1; x < LS; ++x)
        if (DC * x % LS == 1) return x;
    return 0;
}
template <int LS>
__host__ __device__ constexpr uint64_t dma_wraps_by_residue(int lane)
{
    constexpr int DC = 64 % LS, INV = dma_wrap_inverse(LS);
    constexpr bool OTHERS = 2 * DC > LS;  // visit the non-wrapping residues and complement
    constexpr int R0 = OTHERS ? 0 : LS - DC, NR = OTHERS ? LS - DC : DC;
    const int c0 = lane % LS;
    int i = (R0 - c0 + LS) % LS * INV % LS;  // load of residue R0
    uint64_t m = 0;
    for (int k = 0; k < NR; ++k) {
        if (i < LS - 1) m |= 1ull << i;
        i += INV;
        if (i >= LS) i -= LS;
    }
    return OTHERS ? ~m & ((1ull << (LS - 1)) - 1) : m;
}
template <int LS>
constexpr bool dma_wraps_agree()
{
    for (int lane = 0; lane < 64; ++lane)
        if (dma_wraps_by_residue<LS>(lane) != dma_wraps_stepped(LS, lane)) return false;
    return true;
}
template <int LS>
__device__ __forceinline__ uint64_t dma_wraps(int lane)
{
    if constexpr (64 % LS != 0 && dma_wrap_inverse(LS) != 0) {
        static_assert(dma_wraps_agree<LS>(), "the residue form of the wrap plan equals the stepped one for every lane");
        return dma_wraps_by_residue<LS>(lane);
    } else {
        return dma_wraps_stepped(LS, lane);
    }
}

// Whole-row direct global -> LDS copy of a full tile (kTile rows of RBD
// dwords, position stride P bytes) into LDS rows of LS >= RBD dwords.  One
// load carries R = 64 / LS whole rows: lane l holds dword l % LS of the
// load's row l / LS, and the lanes past a row's RBD dwords or past R rows are
// switched off (EXEC), so nothing outside the tile's rows is read and the
// padding slots are not written.  A lane's offset inside its load is the same
// for every load, (l / LS) * P + 4 * (l % LS); load n starts at row R * n in
// memory and at LDS dword R * n * LS.  The loads go out in groups under one
// M0 / EXEC setting as buffer loads: the instruction's immediate offset
// advances the LDS address and the memory address together by 4 * R * LS per
// load, and the scalar offset, stepped by R * (P - 4 * LS) with one scalar
// add per load, makes up the memory side's difference.  No per-lane
// arithmetic per load.
template <int RBD, int LS>
struct RowDma {
    static_assert(RBD <= LS && LS <= 64, "one row per load at least");
    static constexpr int R = 64 / LS;                    // rows per load
    static constexpr int NL = (kTile + R - 1) / R;       // loads per tile
    static constexpr int STEP = 4 * R * LS;              // bytes per load (LDS side)
    static constexpr int LAST_ROWS = kTile - R * (NL - 1);  // rows of the last load
    static constexpr int GMAX = 4095 / STEP + 1 < 16 ? 4095 / STEP + 1 : 16;  // immediate offsets <= 4095
    static constexpr uint64_t lanes(int rows)
    {
        uint64_t m = 0;
        for (int l = 0; l < rows * LS; ++l)
            if (l % LS < RBD) m |= 1ull << l;
        return m;
    }
    static constexpr uint64_t MASK = lanes(R), MASK_LAST = lanes(LAST_ROWS);
};

// One group of G loads (G = 1, 2, 4, 8 or 16) of the whole-row copy: M0 and
// EXEC are set, the loads issued and both restored inside one asm statement,
// so that no other instruction runs under the reduced EXEC.
#define RKV_ROW_LD(j) "s_add_u32 %[so], %[so], %[st]\n\tbuffer_load_dword %[v], %[rs], %[so] offen offset:%[o" #j "] lds\n\t"
#define RKV_ROW_LD2 RKV_ROW_LD(1)
#define RKV_ROW_LD4 RKV_ROW_LD2 RKV_ROW_LD(2) RKV_ROW_LD(3)
#define RKV_ROW_LD8 RKV_ROW_LD4 RKV_ROW_LD(4) RKV_ROW_LD(5) RKV_ROW_LD(6) RKV_ROW_LD(7)
#define RKV_ROW_LD16 \
    RKV_ROW_LD8 RKV_ROW_LD(8) RKV_ROW_LD(9) RKV_ROW_LD(10) RKV_ROW_LD(11) RKV_ROW_LD(12) RKV_ROW_LD(13) RKV_ROW_LD(14) RKV_ROW_LD(15)
#define RKV_ROW_GRP(BODY)                                                                                              \
    asm volatile("s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[ml]\n\ts_mov_b64 %[se], exec\n\ts_mov_b64 exec, %[mk]\n\t" \
                 "s_nop 0\n\tbuffer_load_dword %[v], %[rs], %[so] offen lds\n\t" BODY                                  \
                 "s_mov_b64 exec, %[se]\n\ts_mov_b32 m0, %[sv]"                                                        \
                 : [sv] "=&s"(saved), [se] "=&s"(sexec), [so] "+&s"(so)                                                \
                 : [v] "v"(voff), [rs] "s"(rs), [mk] "s"(mask), [ml] "s"(m0v), [st] "s"(st), [o1] "i"(S),              \
                   [o2] "i"(2 * S), [o3] "i"(3 * S), [o4] "i"(4 * S), [o5] "i"(5 * S), [o6] "i"(6 * S),             \
                   [o7] "i"(7 * S), [o8] "i"(8 * S), [o9] "i"(9 * S), [o10] "i"(10 * S), [o11] "i"(11 * S),        \
                   [o12] "i"(12 * S), [o13] "i"(13 * S), [o14] "i"(14 * S), [o15] "i"(15 * S)                      \
                 : "memory")
template <int G, int S>
__device__ __forceinline__ void lds_rows_grp(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t so, uint32_t st,
                                             uint64_t mask, uint32_t m0v)
{
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
    static_assert((G - 1) * S <= 4095, "immediate offset range");
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t saved;
    uint64_t sexec;
    if constexpr (G == 1)
        RKV_ROW_GRP("");
    else if constexpr (G == 2)
        RKV_ROW_GRP(RKV_ROW_LD2);
    else if constexpr (G == 4)
        RKV_ROW_GRP(RKV_ROW_LD4);
    else if constexpr (G == 8)
        RKV_ROW_GRP(RKV_ROW_LD8);
    else
        RKV_ROW_GRP(RKV_ROW_LD16);
#else
    (void)rs;
    (void)voff;
    (void)so;
    (void)st;
    (void)mask;
    (void)m0v;
#endif
}
#undef RKV_ROW_GRP
#undef RKV_ROW_LD16
#undef RKV_ROW_LD8
#undef RKV_ROW_LD4
#undef RKV_ROW_LD2
#undef RKV_ROW_LD

__host__ __device__ constexpr int row_grp_size(int n, int gmax)
{
    const int m = n < gmax ? n : gmax;
    return m >= 16 ? 16 : m >= 8 ? 8 : m >= 4 ? 4 : m >= 2 ? 2 : 1;
}

// Loads [N0, N1) of the whole-row copy of a tile.  rs addresses the tile's
// first row; voff = RowDma::voff(P, lane); st = R * (P - 4 * LS).
template <int RBD, int LS, int N0, int N1>
__device__ __forceinline__ void dma_rows_whole(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int P, uint32_t st,
                                               uint32_t lds_base)
{
    using RD = RowDma<RBD, LS>;
    static_assert(0 <= N0 && N0 <= N1 && N1 <= RD::NL, "load range");
    if constexpr (N0 < N1) {
        // the tile's last load (fewer rows when R does not divide the tile)
        // goes on its own with its own lane mask
        constexpr bool LASTG = N1 == RD::NL && RD::MASK_LAST != RD::MASK;
        constexpr int NE = LASTG ? N1 - 1 : N1;
        if constexpr (N0 < NE) {
            constexpr int G = row_grp_size(NE - N0, RD::GMAX);
            lds_rows_grp<G, RD::STEP>(rs, voff, (uint32_t)(N0 * RD::R) * (uint32_t)P, st, RD::MASK,
                                      lds_base + (uint32_t)(RD::STEP * N0));
            dma_rows_whole<RBD, LS, N0 + G, N1>(rs, voff, P, st, lds_base);
        } else {
            lds_rows_grp<1, RD::STEP>(rs, voff, (uint32_t)(N0 * RD::R) * (uint32_t)P, st, RD::MASK_LAST,
                                      lds_base + (uint32_t)(RD::STEP * N0));
        }
    }
}
template <int LS>
__device__ __forceinline__ uint32_t row_dma_voff(int P, int lane)
{
    return (uint32_t)(lane / LS) * (uint32_t)P + 4u * (uint32_t)(lane % LS);
}

// The slot plan of a whole tile (kTile rows followed by at least one more
// position of the segment, P >= 4 * LS: a row's padding slots read the dwords
// after the row, inside the next row or position, never used), issued as
// buffer loads in groups under one M0 setting, with no clamps.
// Load i of the plan reads at i * db + voff_i (db = DJ * P + 4 * DC,
// voff_i the lane's offset, which grows by xd = P - 4 * LS after each load
// whose slot wraps past a row end) and lands at LDS lds_base + 256 * i.  In a
// group starting at load i0 the immediate offset 256 * (i - i0) advances both
// addresses; the scalar offset starts at i0 * db and steps by db - 256 =
// DJ * xd per load, and the lane's wrap is added in the asm between loads
// (bit i of the plan, one bit extract and one 24-bit multiply-add).  All 64
// lanes load, so EXEC is untouched.
#define RKV_WRP_LD(j, jb)                                                                                     \
    "v_bfe_u32 %[t], %[wg], " #jb ", 1\n\tv_mad_u32_u24 %[vo], %[t], %[xd], %[vo]\n\ts_add_u32 %[so], %[so], %[st]\n\t" \
    "buffer_load_dword %[vo], %[rs], %[so] offen offset:%[o" #j "] lds\n\t"
#define RKV_WRP_LD2 RKV_WRP_LD(1, 0)
#define RKV_WRP_LD4 RKV_WRP_LD2 RKV_WRP_LD(2, 1) RKV_WRP_LD(3, 2)
#define RKV_WRP_LD8 RKV_WRP_LD4 RKV_WRP_LD(4, 3) RKV_WRP_LD(5, 4) RKV_WRP_LD(6, 5) RKV_WRP_LD(7, 6)
#define RKV_WRP_LD16                                                                                                 \
    RKV_WRP_LD8 RKV_WRP_LD(8, 7) RKV_WRP_LD(9, 8) RKV_WRP_LD(10, 9) RKV_WRP_LD(11, 10) RKV_WRP_LD(12, 11) RKV_WRP_LD(13, 12) \
        RKV_WRP_LD(14, 13) RKV_WRP_LD(15, 14)
#define RKV_WRP_GRP(BODY)                                                                                          \
    asm volatile("s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[ml]\n\ts_nop 0\n\t"                                        \
                 "buffer_load_dword %[vo], %[rs], %[so] offen lds\n\t" BODY "s_mov_b32 m0, %[sv]"                   \
                 : [sv] "=&s"(saved), [so] "+&s"(so), [vo] "+&v"(voff), [t] "=&v"(tmp)                              \
                 : [wg] "v"(wg), [xd] "s"(xd), [rs] "s"(rs), [ml] "s"(m0v), [st] "s"(st), [o1] "i"(256),            \
                   [o2] "i"(512), [o3] "i"(768), [o4] "i"(1024), [o5] "i"(1280), [o6] "i"(1536), [o7] "i"(1792),    \
                   [o8] "i"(2048), [o9] "i"(2304), [o10] "i"(2560), [o11] "i"(2816), [o12] "i"(3072),              \
                   [o13] "i"(3328), [o14] "i"(3584), [o15] "i"(3840)                                               \
                 : "memory")
template <int G>
__device__ __forceinline__ void lds_wrap_grp(__amdgpu_buffer_rsrc_t rs, uint32_t &voff, uint32_t wg, uint32_t xd,
                                             uint32_t so, uint32_t st, uint32_t m0v)
{
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t saved, tmp;
    if constexpr (G == 1)
        RKV_WRP_GRP("");
    else if constexpr (G == 2)
        RKV_WRP_GRP(RKV_WRP_LD2);
    else if constexpr (G == 4)
        RKV_WRP_GRP(RKV_WRP_LD4);
    else if constexpr (G == 8)
        RKV_WRP_GRP(RKV_WRP_LD8);
    else
        RKV_WRP_GRP(RKV_WRP_LD16);
    (void)tmp;
#else
    (void)rs;
    (void)voff;
    (void)wg;
    (void)xd;
    (void)so;
    (void)st;
    (void)m0v;
#endif
}
#undef RKV_WRP_GRP
#undef RKV_WRP_LD16
#undef RKV_WRP_LD8
#undef RKV_WRP_LD4
#undef RKV_WRP_LD2
#undef RKV_WRP_LD

// The same loads from per-lane offsets planned once (dma_plan_grp below):
// load j of a group reads at off[j] + 256 * j and lands at LDS m0 + 256 * j,
// with no arithmetic between the loads.
#define RKV_PLN_LD(j) "buffer_load_dword %[v" #j "], %[rs], %[so] offen offset:%[o" #j "] lds\n\t"
#define RKV_PLN_LD2 RKV_PLN_LD(1)
#define RKV_PLN_LD4 RKV_PLN_LD2 RKV_PLN_LD(2) RKV_PLN_LD(3)
#define RKV_PLN_LD8 RKV_PLN_LD4 RKV_PLN_LD(4) RKV_PLN_LD(5) RKV_PLN_LD(6) RKV_PLN_LD(7)
#define RKV_PLN_LD16 \
    RKV_PLN_LD8 RKV_PLN_LD(8) RKV_PLN_LD(9) RKV_PLN_LD(10) RKV_PLN_LD(11) RKV_PLN_LD(12) RKV_PLN_LD(13) RKV_PLN_LD(14) RKV_PLN_LD(15)
#define RKV_PLN_GRP(BODY)                                                                                           \
    asm volatile("s_mov_b32 %[sv], m0\n\ts_mov_b32 m0, %[ml]\n\ts_nop 0\n\t"                                         \
                 "buffer_load_dword %[v0], %[rs], %[so] offen lds\n\t" BODY "s_mov_b32 m0, %[sv]"                    \
                 : [sv] "=&s"(saved)                                                                                 \
                 : [v0] "v"(off[0]), [v1] "v"(off[G > 1 ? 1 : 0]), [v2] "v"(off[G > 2 ? 2 : 0]),                   \
                   [v3] "v"(off[G > 3 ? 3 : 0]), [v4] "v"(off[G > 4 ? 4 : 0]), [v5] "v"(off[G > 5 ? 5 : 0]),       \
                   [v6] "v"(off[G > 6 ? 6 : 0]), [v7] "v"(off[G > 7 ? 7 : 0]), [v8] "v"(off[G > 8 ? 8 : 0]),       \
                   [v9] "v"(off[G > 9 ? 9 : 0]), [v10] "v"(off[G > 10 ? 10 : 0]), [v11] "v"(off[G > 11 ? 11 : 0]), \
                   [v12] "v"(off[G > 12 ? 12 : 0]), [v13] "v"(off[G > 13 ? 13 : 0]),                                \
                   [v14] "v"(off[G > 14 ? 14 : 0]), [v15] "v"(off[G > 15 ? 15 : 0]), [so] "s"(0u), [rs] "s"(rs),    \
                   [ml] "s"(m0v), [o1] "i"(256), [o2] "i"(512), [o3] "i"(768), [o4] "i"(1024), [o5] "i"(1280),      \
                   [o6] "i"(1536), [o7] "i"(1792), [o8] "i"(2048), [o9] "i"(2304), [o10] "i"(2560),                \
                   [o11] "i"(2816), [o12] "i"(3072), [o13] "i"(3328), [o14] "i"(3584), [o15] "i"(3840)             \
                 : "memory")
template <int G>
__device__ __forceinline__ void lds_plan_grp(__amdgpu_buffer_rsrc_t rs, const uint32_t *off, uint32_t m0v)
{
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t saved;
    if constexpr (G == 1)
        RKV_PLN_GRP("");
    else if constexpr (G == 2)
        RKV_PLN_GRP(RKV_PLN_LD2);
    else if constexpr (G == 4)
        RKV_PLN_GRP(RKV_PLN_LD4);
    else if constexpr (G == 8)
        RKV_PLN_GRP(RKV_PLN_LD8);
    else
        RKV_PLN_GRP(RKV_PLN_LD16);
#else
    (void)rs;
    (void)off;
    (void)m0v;
#endif
}
#undef RKV_PLN_GRP
#undef RKV_PLN_LD16
#undef RKV_PLN_LD8
#undef RKV_PLN_LD4
#undef RKV_PLN_LD2
#undef RKV_PLN_LD

// The per-lane offsets of loads [I0, I1) of the slot plan of a whole tile,
// computed once for the groups dma_issue_grp issues: off[i - I0] = i * db +
// 4 * lane + (lane / LS + wraps before i) * xd - 256 * (position of load i in
// its group).
template <int LS, int I0, int I1>
__device__ __forceinline__ void dma_plan_grp(int P, uint64_t wrap, int lane, uint32_t *off)
{
    static_assert(0 <= I0 && I0 <= I1 && I1 <= LS, "load range");
    constexpr int DJ = 64 / LS, DC = 64 % LS;
    const uint32_t db = (uint32_t)(DJ * P + 4 * DC), xd = (uint32_t)(P - 4 * LS);
    uint32_t wr0 = 0;
    if constexpr (I0 > 0) wr0 = (uint32_t)__builtin_popcountll(wrap & ((1ull << I0) - 1ull));
    uint32_t v = ((uint32_t)(lane / LS) + wr0) * xd + 4u * (uint32_t)lane + (uint32_t)I0 * db;
    int g0 = I0, gl = row_grp_size(I1 - I0, 16);  // current group's first load and size
#pragma unroll
    for (int i = I0; i < I1; ++i) {
        if (i == g0 + gl) {
            g0 = i;
            gl = row_grp_size(I1 - i, 16);
        }
        off[i - I0] = v - 256u * (uint32_t)(i - g0);
        v += db + (uint32_t)((wrap >> i) & 1ull) * xd;
    }
}
template <int I0, int N, int J = 0>
__device__ __forceinline__ void dma_issue_grp(__amdgpu_buffer_rsrc_t rs, const uint32_t *off, uint32_t lds_base)
{
    if constexpr (J < N) {
        constexpr int G = row_grp_size(N - J, 16);
        lds_plan_grp<G>(rs, off + J, lds_base + 256u * (I0 + J));
        dma_issue_grp<I0, N, J + G>(rs, off, lds_base);
    }
}

// Loads [I0, I1) of the slot plan of a whole tile; voff is the lane's offset
// for load I0 (it leaves holding the offset for load I1), rs addresses the
// tile's first row.  The wrap after the group's last load is added here.
template <int LS, int I0, int I1>
__device__ __forceinline__ void dma_rows4_grp(__amdgpu_buffer_rsrc_t rs, uint32_t &voff, uint64_t wrap, int P,
                                              uint32_t lds_base)
{
    static_assert(0 <= I0 && I0 <= I1 && I1 <= LS, "load range");
    if constexpr (I0 < I1) {
        constexpr int DJ = 64 / LS, DC = 64 % LS;
        constexpr int G = row_grp_size(I1 - I0, 16);
        const uint32_t db = (uint32_t)(DJ * P + 4 * DC), xd = (uint32_t)(P - 4 * LS);
        const uint32_t wg = (uint32_t)(wrap >> I0);
        lds_wrap_grp<G>(rs, voff, wg, xd, (uint32_t)I0 * db, (uint32_t)DJ * xd, lds_base + 256u * I0);
        if constexpr (I0 + G < LS) voff += ((wg >> (G - 1)) & 1u) * xd;  // the wrap after the group's last load
        dma_rows4_grp<LS, I0 + G, I1>(rs, voff, wrap, P, lds_base);
    }
}

// s_waitcnt vmcnt(n) (0 <= n <= 63), other counters untouched.
template <int N>
__device__ __forceinline__ void waitcnt_vm()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void waitcnt_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }



// QC dims [d0, d0 + QC) of row j of a DMA-staged f32 / f16 K tile.
template <int KT, int RB, int QC>
__device__ __forceinline__ void k_chunk_dma(const uint32_t *tile, int j, int sw, int d0, float *k)
{
    constexpr int EPC = KT == kF16 ? 8 : 4;  // elements per 16-byte chunk
    const uint32_t *row = tile + j * (RB / 4);
    if constexpr (QC >= EPC) {
#pragma unroll
        for (int cc = 0; cc < QC / EPC; ++cc) {
            const uint4 w = *(const uint4 *)(row + 4 * (((d0 / EPC) + cc) ^ sw));
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
            if constexpr (KT == kF16) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    k[cc * 8 + 2 * e] = h2f(ww[e]);
                    k[cc * 8 + 2 * e + 1] = h2f(ww[e] >> 16);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) k[cc * 4 + e] = __builtin_bit_cast(float, ww[e]);
            }
        }
    } else {
        // part of one chunk: the dword offset inside it
        const int inner = (d0 % EPC) / (KT == kF16 ? 2 : 1);
        const uint32_t *cp = row + 4 * ((d0 / EPC) ^ sw) + inner;
        if constexpr (KT == kF16) {
            if constexpr (QC == 4) {
                const uint2 w = *(const uint2 *)cp;
                k[0] = h2f(w.x); k[1] = h2f(w.x >> 16); k[2] = h2f(w.y); k[3] = h2f(w.y >> 16);
            } else if constexpr (QC == 2) {
                const uint32_t w = *cp;
                k[0] = h2f(w); k[1] = h2f(w >> 16);
            } else {
                const uint32_t w = *cp;
                k[0] = (d0 & 1) ? h2f(w >> 16) : h2f(w);
            }
        } else {
#pragma unroll
            for (int e = 0; e < QC; ++e) k[e] = __builtin_bit_cast(float, cp[e]);
        }
    }
}

// ---------------------------------------------------------------- scores

// QC consecutive dims [d0, d0 + QC) of this lane's K row in LDS as floats
// (block types: the codes, without the block scale).  QC is 1, 2, 4 or 8 and
// d0 a multiple of QC, so a chunk never straddles a 32-value block.  Rows of
// f32 / f16 start 16-byte aligned in LDS.
template <int KT, int QC>
__device__ __forceinline__ void k_chunk(const uint32_t *row, int d0, float *k)
{
    if constexpr (KT == kF32) {
        if constexpr (QC % 4 == 0) {
#pragma unroll
            for (int j = 0; j < QC / 4; ++j) {
                const uint4 w = *(const uint4 *)(row + d0 + 4 * j);
                k[4 * j] = __builtin_bit_cast(float, w.x);
                k[4 * j + 1] = __builtin_bit_cast(float, w.y);
                k[4 * j + 2] = __builtin_bit_cast(float, w.z);
                k[4 * j + 3] = __builtin_bit_cast(float, w.w);
            }
        } else {
#pragma unroll
            for (int e = 0; e < QC; ++e) k[e] = __builtin_bit_cast(float, row[d0 + e]);
        }
    } else if constexpr (KT == kF16) {
        if constexpr (QC == 8) {
            const uint4 w = *(const uint4 *)(row + d0 / 2);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                k[2 * e] = h2f(ww[e]);
                k[2 * e + 1] = h2f(ww[e] >> 16);
            }
        } else if constexpr (QC == 4) {
            const uint2 w = *(const uint2 *)(row + d0 / 2);
            k[0] = h2f(w.x);
            k[1] = h2f(w.x >> 16);
            k[2] = h2f(w.y);
            k[3] = h2f(w.y >> 16);
        } else if constexpr (QC == 2) {
            const uint32_t w = row[d0 / 2];
            k[0] = h2f(w);
            k[1] = h2f(w >> 16);
        } else {
            const uint32_t w = row[d0 / 2];
            k[0] = (d0 & 1) ? h2f(w >> 16) : h2f(w);
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
// The byte offset passes through an empty asm so that the compiler treats each
// chunk's loads as new: without it, the loads of all RT * head_dim values are
// hoisted out of the key loop and spill.  (Laundering the row pointers
// instead would hide that they point at read-only kernel-argument memory,
// and the loads would no longer be scalar.)
template <int RT, int QC>
__device__ __forceinline__ void q_chunk(const float *const *qp, int d0, float (*qv)[QC])
{
    uint32_t ob = 4u * (uint32_t)d0;
    asm volatile("" : "+s"(ob));
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int e = 0; e < QC; ++e) qv[r][e] = *(const float *)((const char *)qp[r] + ob + 4 * e);
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
template <int KT, int D, int RT, bool KDMA = false>
__device__ __forceinline__ void key_dots(const uint32_t *row, const float *const *qp, float *s, int j = 0, int sw = 0)
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
        q_chunk<RT, QC>(qp, 32 * bb, qa);
        if constexpr (KDMA) k_chunk_dma<KT, row_bytes_of(KT, D), QC>(row, j, sw, 32 * bb, ka);
        else k_chunk<KT, QC>(row, 32 * bb, ka);
#pragma unroll
        for (int ci = 0; ci < CPB; ++ci) {
            if (ci + 1 < CPB) {
                q_chunk<RT, QC>(qp, 32 * bb + QC * (ci + 1), qb);
                if constexpr (KDMA) k_chunk_dma<KT, row_bytes_of(KT, D), QC>(row, j, sw, 32 * bb + QC * (ci + 1), kb);
                else k_chunk<KT, QC>(row, 32 * bb + QC * (ci + 1), kb);
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

// ---------------------------------------------------------------- MFMA scores

typedef _Float16 rkv_half8 __attribute__((ext_vector_type(8)));
typedef float rkv_float4v __attribute__((ext_vector_type(4)));

// Maximum / sum over each group of 16 lanes (a DPP row), in every lane of it.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float x)
{
    x = fmaxf(x, dpp_mov<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_mov<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_mov<0x141>(x));  // row_half_mirror
    return fmaxf(x, dpp_mov<0x140>(x));  // row_mirror
}
__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp_mov<0xB1>(x);
    x += dpp_mov<0x4E>(x);
    x += dpp_mov<0x141>(x);
    return x + dpp_mov<0x140>(x);
}

// The query rows of a wave as the A operand of v_mfma_f32_16x16x32_f16: lane
// l holds row l % 16, dims 32*kk + 8*(l / 16) .. +7 of chunk kk, each value
// pre-multiplied by scale * log2(e) and split into binary16 high and low
// parts (hi + lo keeps about 22 significant bits, so the products, exact in
// the f32 accumulator, carry the f32 query).  Rows >= nr are zero.
// A row whose largest magnitude lies outside [2^-2, 2^15) is first
// multiplied by a power of two 2^ex that puts it in [2^14, 2^15): binary16
// then neither overflows (a query of any binary32 size) nor loses the low
// part to its subnormal range (a tiny query); the scores of such a row come
// out multiplied by 2^ex, which unscale_rows takes off exactly.  Inside
// [2^-2, 2^15) ex = 0: the high part of the largest values is normal and
// their low part too, and a smaller value's error stays below 2^-24 of the
// row's largest.  ex is returned per lane (the exponent of the lane's
// A-operand row).
// Loads (mfma_q_load, issued early) and conversion (mfma_q_split).
// (Unpredicated loads: a lane without a row reads a valid row and its values
// are replaced by zero in mfma_q_split.)
template <int D>
__device__ __forceinline__ void mfma_q_load(const float *qrow, int lane, float (*x)[8])
{
    const int kq = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        const float4 a = *(const float4 *)(qrow + 32 * kk + 8 * kq);
        const float4 b = *(const float4 *)(qrow + 32 * kk + 8 * kq + 4);
        x[kk][0] = a.x; x[kk][1] = a.y; x[kk][2] = a.z; x[kk][3] = a.w;
        x[kk][4] = b.x; x[kk][5] = b.y; x[kk][6] = b.z; x[kk][7] = b.w;
    }
}
template <int D>
__device__ __forceinline__ int mfma_q_split(const float (*x)[8], bool has, float sl2, rkv_half8 *qhi, rkv_half8 *qlo)
{
    float y[D / 32][8];
    float mx = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            y[kk][e] = has ? x[kk][e] * sl2 : 0.f;
            mx = fmaxf(mx, fabsf(y[kk][e]));
        }
    // the row's values sit in lanes l, l ^ 16, l ^ 32, l ^ 48
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // mx = f 2^e with f in [0.5, 1): mx 2^(15 - e) is in [2^14, 2^15)
    const int e = __builtin_amdgcn_frexp_expf(mx);
    const int ex = (mx == 0.f || (e >= -1 && e <= 15)) ? 0 : 15 - e;
    // (the scaling pass only when some row of the wave needs it)
    if (__builtin_amdgcn_ballot_w64(ex != 0)) {
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) y[kk][e] = __builtin_amdgcn_ldexpf(y[kk][e], ex);
    }
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const _Float16 h = (_Float16)y[kk][e];
            qhi[kk][e] = h;
            qlo[kk][e] = (_Float16)(y[kk][e] - (float)h);
        }
    return ex;
}

// The query-row exponents of a lane's four MFMA output rows (rows
// 4*(lane/16) + i), from the lanes that hold those rows' A operands.
__device__ __forceinline__ void mfma_out_row_exps(int ex, int lane, int (&oex)[4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) oex[i] = __shfl(ex, 4 * (lane >> 4) + i, 64);
}

// Take the query rows' power-of-two factors off a score tile (exact).
template <int NKB>
__device__ __forceinline__ void unscale_rows(float (&sv)[NKB][4], const int (&oex)[4])
{
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[kb][i] = __builtin_amdgcn_ldexpf(sv[kb][i], -oex[i]);
}

// Block-type V on the matrix cores takes d * code as a binary16 operand,
// which overflows once |d * code| > 65504: q8_0 codes reach -128, so any
// |d| >= 512 (binary16 exponent field >= 24) can; q4_0 codes reach -8, so
// |d| >= 8192 (field >= 28).  The largest scale magnitude (bits without the
// sign) of the blocks of this lane's key row in a staged V tile (row = lane,
// NB blocks); keys past the segment's end repeat a real row.
template <int VT, int NB>
__device__ __forceinline__ uint32_t v_row_scale_max(const uint32_t *row)
{
    constexpr int BB = VT == kQ8 ? 34 : 18;
    uint32_t m = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int o = BB * b;
        const uint32_t w = row[o >> 2];
        m = max(m, ((o & 2) ? (w >> 16) : w) & 0x7fffu);
    }
    return m;
}
template <int VT>
__device__ __forceinline__ constexpr uint32_t v_scale_limit() { return VT == kQ8 ? 0x6000u : 0x7000u; }



// Scores (log2 units) of the 64 keys of a DMA-staged f16 K tile against the
// wave's query rows: sv[kb][i] = score of row 4*(lane/16) + i and key
// 16*kb + lane % 16.  The B operand of chunk kk for key row j is the 16-byte
// chunk 4*kk + lane/16 of that row (swizzled slot in LDS).
template <int D, int RB>
__device__ __forceinline__ void mfma_scores(const uint32_t *tile, const rkv_half8 *qhi, const rkv_half8 *qlo, int lane,
                                            float (*sv)[4])
{
    rkv_float4v acc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) acc[kb] = rkv_float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        // the four B operands of the chunk are read together (one LDS wait per
        // chunk), and the high-part products of the four key blocks go before
        // the low-part ones, so consecutive MFMAs use different accumulators
        rkv_half8 b[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int j = 16 * kb + (lane & 15);
            const int c = 4 * kk + (lane >> 4);
            b[kb] = *(const rkv_half8 *)(tile + j * (RB / 4) + 4 * (c ^ kswz<RB>(j)));
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qhi[kk], b[kb], acc[kb], 0, 0, 0);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qlo[kk], b[kb], acc[kb], 0, 0, 0);
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[kb][i] = acc[kb][i];
}

// Block-type K on the matrix cores.  The codes of one 32-value block are
// exact in binary16 (q8_0: -127..127, q4_0: -8..7), and one block is one
// k-step of v_mfma_f32_16x16x32_f16, so each step's product is multiplied by
// the key's block scale afterwards: s = sum_kk d[key][kk] * (q_kk . code_kk).
// Codes become f16 by placing each (biased) byte under the exponent byte 0x64
// (value 1024 + byte) and subtracting the bias with one packed f16 add.
typedef _Float16 rkv_half2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f16pair_of_bytes(uint32_t x, uint32_t sel, _Float16 bias)
{
    const uint32_t w = __builtin_amdgcn_perm(0x64646464u, x, sel);
    const rkv_half2 h = __builtin_bit_cast(rkv_half2, w) - rkv_half2{bias, bias};
    return __builtin_bit_cast(uint32_t, h);
}

// Signed byte B of x as an exact binary16 in the low half of a fresh dword
// (upper half zero), and signed byte B of y into the high half of r (low
// half kept): one sub-dword-addressed conversion each, no shifts or bias.
template <int B>
__device__ __forceinline__ uint32_t i8_f16_lo(uint32_t x)
{
    uint32_t r;
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (B == 0)
        asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(x));
    else if constexpr (B == 1)
        asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(x));
    else if constexpr (B == 2)
        asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(x));
    else
        asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(x));
#else
    r = x;
#endif
    return r;
}
template <int B>
__device__ __forceinline__ uint32_t i8_f16_hi(uint32_t r, uint32_t y)
{
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (B == 0)
        asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_0" : "+v"(r) : "v"(y));
    else if constexpr (B == 1)
        asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_1" : "+v"(r) : "v"(y));
    else if constexpr (B == 2)
        asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_2" : "+v"(r) : "v"(y));
    else
        asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_3" : "+v"(r) : "v"(y));
#else
    (void)y;
#endif
    return r;
}
// (signed byte BA of x, signed byte BB of y) as a binary16 pair
template <int BA, int BB>
__device__ __forceinline__ uint32_t i8_f16_pair(uint32_t x, uint32_t y)
{
    return i8_f16_hi<BB>(i8_f16_lo<BA>(x), y);
}

// 8 codes of a q8_0 / q4_0 row in LDS (row = dword pointer) for dims
// 32*kk + 8*g .. +7, as the f16 B operand; and the block scale of block kk.
// (q8_0 with SDWA: the codes start 2 bytes into a dword when kk is even and
// on a dword boundary when it is odd, so each pair is converted straight from
// the dwords that hold it -- for a kk known at compile time after unrolling;
// otherwise the codes are aligned by a funnel shift, biased into the
// exponent-0x64 binade and the bias subtracted.)
template <int KT, bool SDWA = true>
__device__ __forceinline__ rkv_half8 block_codes_f16(const uint32_t *row, int kk, int g, float &dsc)
{
    const int os = (KT == kQ8 ? 34 : 18) * kk;
    const uint32_t s0 = row[os >> 2];
    dsc = h2f((os & 2) ? (s0 >> 16) : s0);
    const int o = KT == kQ8 ? os + 2 + 8 * g : os + 2 + 8 * (g & 1);
    uint32_t out[4];
    if constexpr (KT == kQ8 && SDWA) {
        const uint32_t *w = row + (o >> 2);
        if ((kk & 1) == 0) {  // codes at bytes 2, 3 of w[0], then w[1], then bytes 0, 1 of w[2]
            const uint32_t A = w[0], B = w[1], C = w[2];
            out[0] = i8_f16_pair<2, 3>(A, A);
            out[1] = i8_f16_pair<0, 1>(B, B);
            out[2] = i8_f16_pair<2, 3>(B, B);
            out[3] = i8_f16_pair<0, 1>(C, C);
        } else {  // codes at w[0], w[1]
            const uint32_t A = w[0], B = w[1];
            out[0] = i8_f16_pair<0, 1>(A, A);
            out[1] = i8_f16_pair<2, 3>(A, A);
            out[2] = i8_f16_pair<0, 1>(B, B);
            out[3] = i8_f16_pair<2, 3>(B, B);
        }
    } else {
        const uint32_t sh = o & 3;
        const uint32_t A = row[o >> 2], B = row[(o >> 2) + 1], C = row[(o >> 2) + 2];
        uint32_t w0 = funnel(A, B, sh), w1 = funnel(B, C, sh);
        if constexpr (KT == kQ8) {
            w0 ^= 0x80808080u;
            w1 ^= 0x80808080u;
            out[0] = f16pair_of_bytes(w0, 0x04010400u, (_Float16)1152.f);
            out[1] = f16pair_of_bytes(w0, 0x04030402u, (_Float16)1152.f);
            out[2] = f16pair_of_bytes(w1, 0x04010400u, (_Float16)1152.f);
            out[3] = f16pair_of_bytes(w1, 0x04030402u, (_Float16)1152.f);
        } else {
            const int shn = (g >> 1) * 4;  // dims 0..15 of the block: low nibbles; 16..31: high
            w0 = (w0 >> shn) & 0x0f0f0f0fu;
            w1 = (w1 >> shn) & 0x0f0f0f0fu;
            out[0] = f16pair_of_bytes(w0, 0x04010400u, (_Float16)1032.f);
            out[1] = f16pair_of_bytes(w0, 0x04030402u, (_Float16)1032.f);
            out[2] = f16pair_of_bytes(w1, 0x04010400u, (_Float16)1032.f);
            out[3] = f16pair_of_bytes(w1, 0x04030402u, (_Float16)1032.f);
        }
    }
    return __builtin_bit_cast(rkv_half8, out);
}

// The 8 code bytes of dims 8*dg .. 8*dg+7 of a q8_0 row in LDS as two
// dwords (dim 8*dg + j in byte j % 4 of w[j / 4]), and the block's binary16
// scale bits.
__device__ __forceinline__ void v_group_bytes_q8(const uint32_t *row, int dg, uint32_t *w, uint32_t &dbits)
{
    const int bb = dg >> 2, h = dg & 3;
    const int os = 34 * bb;
    const uint32_t s0 = row[os >> 2];
    dbits = (os & 2) ? (s0 >> 16) : (s0 & 0xffffu);
    const int o = os + 2 + 8 * h;
    const uint32_t sh = o & 3;
    const uint32_t A = row[o >> 2], B = row[(o >> 2) + 1], C = row[(o >> 2) + 2];
    w[0] = funnel(A, B, sh);
    w[1] = funnel(B, C, sh);
}

// The 8 codes of dims 8*dg .. 8*dg+7 of a q8_0 / q4_0 row in LDS as four
// packed binary16 pairs (exact), and the block's binary16 scale bits.
template <int VT>
__device__ __forceinline__ void v_group_codes_f16(const uint32_t *row, int dg, uint32_t *c2, uint32_t &dbits)
{
    const int bb = dg >> 2, h = dg & 3;
    const int os = (VT == kQ8 ? 34 : 18) * bb;
    const uint32_t s0 = row[os >> 2];
    dbits = (os & 2) ? (s0 >> 16) : (s0 & 0xffffu);
    const int o = VT == kQ8 ? os + 2 + 8 * h : os + 2 + 8 * (h & 1);
    const uint32_t sh = o & 3;
    const uint32_t A = row[o >> 2], B = row[(o >> 2) + 1], C = row[(o >> 2) + 2];
    uint32_t w0 = funnel(A, B, sh), w1 = funnel(B, C, sh);
    if constexpr (VT == kQ8) {
        w0 ^= 0x80808080u;
        w1 ^= 0x80808080u;
        c2[0] = f16pair_of_bytes(w0, 0x04010400u, (_Float16)1152.f);
        c2[1] = f16pair_of_bytes(w0, 0x04030402u, (_Float16)1152.f);
        c2[2] = f16pair_of_bytes(w1, 0x04010400u, (_Float16)1152.f);
        c2[3] = f16pair_of_bytes(w1, 0x04030402u, (_Float16)1152.f);
    } else {
        const int shn = (h >> 1) * 4;
        w0 = (w0 >> shn) & 0x0f0f0f0fu;
        w1 = (w1 >> shn) & 0x0f0f0f0fu;
        c2[0] = f16pair_of_bytes(w0, 0x04010400u, (_Float16)1032.f);
        c2[1] = f16pair_of_bytes(w0, 0x04030402u, (_Float16)1032.f);
        c2[2] = f16pair_of_bytes(w1, 0x04010400u, (_Float16)1032.f);
        c2[3] = f16pair_of_bytes(w1, 0x04030402u, (_Float16)1032.f);
    }
}

// Scores (log2 units) of the 64 keys of a staged q8_0 / q4_0 K tile (row
// stride LS dwords) against the wave's query rows, in the layout of
// mfma_scores.
template <int KT, int D, int LS>
__device__ __forceinline__ void mfma_scores_blk(const uint32_t *tile, const rkv_half8 *qhi, const rkv_half8 *qlo,
                                                int lane, float (*sv)[4])
{
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[kb][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        // the four key blocks' operands of the chunk first, then the
        // high-part products of all four, then the low-part ones
        // (consecutive MFMAs use different accumulators)
        rkv_half8 b[4];
        float dsc[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            b[kb] = block_codes_f16<KT>(tile + (16 * kb + (lane & 15)) * LS, kk, lane >> 4, dsc[kb]);
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
        // one block of 32 dims at a time: keeps the code reads of later blocks
        // from being hoisted (and held in registers) ahead of this one
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---------------------------------------------------------------- values

// 8 consecutive values (dims 8*dg .. 8*dg+7) of a V row held in LDS, as
// floats, plus the block scale they must be multiplied by (1 for f32/f16).
// A TBQ3 level by index m (0..3) from the four positive levels.
__device__ __forceinline__ float tbq3_level(const float *lv, uint32_t m)
{
    const float lo = (m & 1u) ? lv[1] : lv[0], hi = (m & 1u) ? lv[3] : lv[2];
    return (m & 2u) ? hi : lo;
}

template <int VT, int D>
__device__ __forceinline__ float v_group_lds(const uint32_t *row, int dg, float *x, const float *lv = nullptr)
{
    if constexpr (VT == kF32) {
        const uint4 a = *(const uint4 *)(row + 8 * dg), b = *(const uint4 *)(row + 8 * dg + 4);
        x[0] = __builtin_bit_cast(float, a.x); x[1] = __builtin_bit_cast(float, a.y);
        x[2] = __builtin_bit_cast(float, a.z); x[3] = __builtin_bit_cast(float, a.w);
        x[4] = __builtin_bit_cast(float, b.x); x[5] = __builtin_bit_cast(float, b.y);
        x[6] = __builtin_bit_cast(float, b.z); x[7] = __builtin_bit_cast(float, b.w);
        return 1.f;
    } else if constexpr (VT == kF16) {
        const uint4 w = *(const uint4 *)(row + 4 * dg);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = h2f(ww[e]);
            x[2 * e + 1] = h2f(ww[e] >> 16);
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
    } else if constexpr (VT == kT3) {
        // TBQ3: rotated values of dims 8n..8n+7 of block b (13 dwords per
        // block: norm, 16 bits of magnitude indices at dword 1 + n/2, 8 sign
        // bits at dword 9 + n/4); the block's n / sqrt(128) is the scale
        const int b = dg >> 4, n = dg & 15;
        const uint32_t *blk = row + 13 * b;
        const uint32_t q16 = blk[1 + (n >> 1)] >> (16 * (n & 1));
        const uint32_t s8 = blk[9 + (n >> 2)] >> (8 * (n & 3));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float c = tbq3_level(lv, (q16 >> (2 * e)) & 3u);
            x[e] = ((s8 >> e) & 1u) ? -c : c;
        }
        return h2f(blk[0]) * 0.088388347648318440550f;
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

// P.V of one staged block-type V tile (64 keys, head_dim 128) in binary32 on
// the VALU, accumulated into the matrix-core output layout (lane (g, n):
// oc[c][i] = O[4g + i][8n + c]): the path for tiles whose scales would make
// d * code overflow the binary16 operands.  Each product p * (d * code) is
// one binary32 rounding (d * code is exact).  prob(r, k) is the probability
// of row r and key k of the tile; rows >= rt are skipped.
template <int VT, int LSV, typename ProbFn>
__device__ __forceinline__ void pv_valu_tile(const uint32_t *sv_tile, ProbFn prob, int rt, int lane,
                                             rkv_float4v (&oc)[8])
{
    const int g = lane >> 4, n = lane & 15;
    for (int k = 0; k < kTile; ++k) {
        float x[8];
        const float dsc = v_group_lds<VT, 128>(sv_tile + k * LSV, n, x);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            const float pw = r < rt ? prob(r, k) : 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) oc[c][i] = fmaf(pw, dsc * x[c], oc[c][i]);
        }
    }
}

// Entry i of a 16-bit table in the kernel arguments, read as the aligned
// 32-bit word that holds it: with a wave-uniform index that is a scalar load
// (there are no 16-bit scalar loads), so its wait does not involve the vector
// memory counter.
__device__ __forceinline__ int u16_at(const uint16_t *tab, int i)
{
    const uint32_t v = ((const uint32_t *)tab)[i >> 1];
    return (int)((i & 1) ? (v >> 16) : (v & 0xffffu));
}

// ---------------------------------------------------------------- the kernel

// Rows of a wave's score buffer: RT, or with dim slices (DS > 1) the rows of
// the lanes that hold real rows in the MFMA layout (a multiple of 4), since
// the buffer also carries the partial scores between the slices of a head.
__host__ __device__ constexpr int sp_rows(int rt, int ds) { return ds > 1 ? (rt + 3) / 4 * 4 : rt; }

// D is the head_dim a wave works on.  DS > 1 (block-type K and V at head_dim
// DS*D): every KV head is cut into DS slices of D dims, one wave each, in the
// same workgroup; a slice's partial scores (q . k over its D dims) are summed
// with those of the head's other slices through LDS, in slice order, so that
// all DS waves hold the same scores and softmax, and each then accumulates
// P.V for its own D dims of V.
template <int KT, int VT, int D, int RT, int DS = 1>
__global__ void __launch_bounds__((64 * Shape<KT, VT, D>::waves(sp_rows(RT, DS))))
rkv_split_kernel(const float *__restrict__ q, float *__restrict__ part_acc, float2 *__restrict__ part_ml,
                 float *__restrict__ o_out, float *__restrict__ lse_out, const SplitParams p)
{
    using Sh = Shape<KT, VT, D>;
    constexpr int RTX = sp_rows(RT, DS);
    constexpr int NW = Sh::waves(RTX);
    constexpr int DF = D * DS;  // head_dim of q, o and the partials
    constexpr int LSK = Sh::LSK, LSV = Sh::LSV;
    constexpr bool V_REG = Sh::V_REG;
    constexpr int VWK = load_width_of(KT, D);
    constexpr int VWV = load_width_of(VT, D);
    constexpr int LPR = D / 8;      // lanes per V row in the P.V phase
    constexpr int KPS = 64 / LPR;   // keys per P.V step
    constexpr int NSTEP = kTile / KPS;
    constexpr int VRW = VT == kF32 ? 8 : 4;  // dwords of one lane's 8 values, register path
    constexpr int MERGE_DW = NW * RT * (D + 2);
    constexpr int SMEM_DW1 = NW * Sh::STAGE_DW > MERGE_DW ? NW * Sh::STAGE_DW : MERGE_DW;
    // Block-type K and V rows by DMA at head_dim 128 without dim slices (the
    // BDMA path below): a second V buffer per wave (VDB) wherever it fits the
    // compute unit's LDS without lowering the number of workgroups it holds.
    // Tile i+1's V rows then go out together with its K rows once tile i's
    // scores are done, instead of after tile i's P.V, and have the rest of
    // tile i (softmax, P.V) and tile i+1's scores to land.
    constexpr bool BDMA_SHAPE = (KT == kQ8 || KT == kQ4) && (VT == kQ8 || VT == kQ4 || VT == kT3) && D == 128 &&
                                RT <= 16 && DS == 1 && Sh::RBK % 4 == 0 && Sh::RBV % 4 == 0 && LSK + LSV <= 63;
    constexpr int LDS_REST = 4 * NW * (Sh::P_IN_K ? 4 : RTX * kTile) + 4 * NW * RT + (VT == kT3 ? 512 : 8);
    constexpr int SMEM_DW2 = NW * Sh::STAGE_DW + NW * kTile * LSV > MERGE_DW ? NW * Sh::STAGE_DW + NW * kTile * LSV
                                                                             : MERGE_DW;
    constexpr int LDS1 = 4 * SMEM_DW1 + LDS_REST, LDS2 = 4 * SMEM_DW2 + LDS_REST;
    constexpr bool VDB = BDMA_SHAPE && LDS2 <= 160 * 1024 && (160 * 1024) / LDS2 == (160 * 1024) / LDS1;
    constexpr int SMEM_DW = VDB ? SMEM_DW2 : SMEM_DW1;
    static_assert(4 * SMEM_DW + LDS_REST <= 160 * 1024, "a workgroup's LDS fits one compute unit");

    __shared__ __attribute__((aligned(16))) uint32_t smem[SMEM_DW];
    __shared__ __attribute__((aligned(16))) float sP[NW][Sh::P_IN_K ? 4 : RTX * kTile];
    __shared__ int sRow[NW][RT];  // output row of each wave's rows (-1: none), for the epilogue
    // TBQ3 values: entry m_a | m_b << 2 | sign_a << 4 | sign_b << 5 of
    // two consecutive values, as the binary16 high parts (x) and low parts
    // (y) of the two signed levels, packed as matrix-core operand pairs
    __shared__ uint2 sT3[VT == kT3 ? 64 : 1];

    if (p.release && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0)
        __hip_atomic_store(p.release, p.release_value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if constexpr (VT == kT3) {
        if (threadIdx.x < 64) {
            const int e = threadIdx.x;
            const float va = ((e >> 4) & 1) ? -tbq3_level(p.tbq_lv, e & 3) : tbq3_level(p.tbq_lv, e & 3);
            const float vb = ((e >> 5) & 1) ? -tbq3_level(p.tbq_lv, (e >> 2) & 3) : tbq3_level(p.tbq_lv, (e >> 2) & 3);
            const _Float16 ha = (_Float16)va, hb = (_Float16)vb;
            const _Float16 la = (_Float16)(va - (float)ha), lb = (_Float16)(vb - (float)hb);
            sT3[e] = make_uint2((uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16),
                                (uint32_t)__builtin_bit_cast(uint16_t, la) | ((uint32_t)__builtin_bit_cast(uint16_t, lb) << 16));
        }
        __syncthreads();
    }
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, uniform in the wave
    uint32_t *sK = smem + w * Sh::STAGE_DW;
    uint32_t *sV = sK + kTile * LSK;  // this tile's V rows (block-type V)
    // the next tile's V rows with VDB (the buffers swap after each tile)
    uint32_t *sVn = VDB ? smem + NW * Sh::STAGE_DW + w * kTile * LSV : sV;
    // this wave's score rows P [row][key] (in its K tile when that is free)
    float *const sPw = Sh::P_IN_K ? (float *)sK : &sP[w][0];

    // this wave's head slot hs and its index ws among the head's waves; the
    // waves of a head split its key tiles, or (rg_waves) each takes one of
    // its row groups over all of them
    const int hg = blockIdx.y / p.n_rg;
    const int wph = 1 << p.wph_log2;
    const int hs = w >> p.wph_log2;
    const int ws = w - hs * wph;
    const int rg = p.rg_waves ? (blockIdx.y - hg * p.n_rg) * wph + ws : blockIdx.y - hg * p.n_rg;
    // head slot -> KV head g and dim slice js (js = 0 and g the slot when DS = 1)
    const int vh = (hg << p.hpw_log2) + hs;
    const int g = vh / DS, js = vh - (vh / DS) * DS;
    const int cnt = g < p.n_kv_heads ? u16_at(p.rowcnt, g) - rg * RT : 0;
    const int nr = cnt <= 0 ? 0 : cnt < RT ? cnt : RT;  // 0: a wave with no rows (it still joins the barriers)
    const int z = blockIdx.z;

    // the segment this workgroup's key split belongs to
    SegParams sg = p.seg[0];
#pragma unroll
    for (int si = 1; si < kMaxSegs; ++si)
        if (si < p.n_segs && (int)blockIdx.x >= p.seg[si].split_base) sg = p.seg[si];
    const int64_t kbeg = (int64_t)((int)blockIdx.x - sg.split_base) * sg.keys_per_split;
    // (with dim slices every wave walks the same tiles, rows or not: the slices
    // meet at a barrier per tile)
    int64_t kend = (nr == 0 && DS == 1) ? kbeg
                   : kbeg + sg.keys_per_split < sg.n_keys ? kbeg + sg.keys_per_split : sg.n_keys;
    const int64_t tstep = (p.rg_waves ? 1 : (int64_t)wph) * kTile;  // tile stride of this wave

    const int gr = g < p.n_kv_heads ? g : p.n_kv_heads - 1;  // a slot past the heads reads a real one
    const uint8_t *kg = sg.k + z * sg.k_seq + gr * sg.k_head + js * Sh::RBK;
    const uint8_t *vg = sg.v + z * sg.v_seq + gr * sg.v_head + js * Sh::RBV;

    // Output rows of the wave's RT rows (-1 past nr).  The table is read at
    // a clamped index whatever nr is, so these reads do not wait for the
    // row count (one level of dependent loads fewer before the first tile).
    int tabrow[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int ti = g * p.rows_per_g + rg * RT + r;
        const int v = u16_at(p.rowtab, ti < kMaxRowTable ? ti : kMaxRowTable - 1);
        tabrow[r] = r < nr ? z * p.z_row_step + v : -1;
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < RT; ++r) sRow[w][r] = tabrow[r];
    }
    int rid[RT];
    const float *qp[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        const int rr = r < nr ? r : nr - 1;  // padding rows repeat the last row; never written
        rid[r] = nr == 0 ? 0 : tabrow[rr];
        qp[r] = q + rid[r] * DF + js * D;
    }
    // Causal mask (masked launches): row r sees the keys of the segment with
    // index <= lim[r] (its sequence's query position minus the segment's
    // first position); without a mask every key.  A wave (without dim slices)
    // walks no tile that none of its rows sees.
    // (32-bit: a masked launch has segments of fewer than 2^30 keys, and the
    // limits are clamped to [-1, 2^30])
    constexpr int kSeeAll = 1 << 30;
    int lim[RT];
    int lim_max = -1, lim_min = kSeeAll;  // over the wave's real rows
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        int x = kSeeAll;
        if (p.masked) {
            const int64_t rel = p.qpos[rid[r] / p.n_q_heads] - sg.pos0;
            x = rel < -1 ? -1 : rel > kSeeAll ? kSeeAll : (int)rel;
        }
        lim[r] = x;
        if (r < nr) {
            lim_max = x > lim_max ? x : lim_max;
            lim_min = x < lim_min ? x : lim_min;
        }
    }
    // (limits, kbeg and kend all count keys from the segment's first one)
    if (DS == 1 && p.masked && kend > (int64_t)lim_max + 1) kend = (int64_t)lim_max + 1 > kbeg ? (int64_t)lim_max + 1 : kbeg;

    float m[RT], l[RT], acc[RT][8];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
    }
    rkv_float4v oc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) oc[c] = rkv_float4v{0.f, 0.f, 0.f, 0.f};

    const int ks = lane / LPR;
    const int dg = lane - ks * LPR;
    const float sl2 = p.scale_log2;
    const float cap = p.softcap;
    constexpr float kLog2e = 1.4426950408889634f;
    const float scale_over_cap = cap > 0.f ? p.scale / cap : 0.f;

    // Scores on the matrix cores: f16 K tiles staged by DMA, up to 16 query
    // rows per wave as the 16-row A operand.  Running max and denominator are
    // then kept per lane for the rows 4*(lane/16) .. +3 (mrow / lrow) and the
    // wave-uniform m[] follows them.
    constexpr bool MFMA_S = ((KT == kF16 && Sh::KDMA) || KT == kQ8 || KT == kQ4) && D <= 128 && RT <= 16;
    // P.V on the matrix cores as well, for f16 V rows of 128 values held in
    // registers: lane (g = lane/16, n = lane%16) holds, for step st, the 8
    // values of key 4*st + g at dims 8n .. 8n+7.  Taking as contraction index
    // k = 8g + e the key 4*(8*kb + e) + g, and as output column n the dim
    // 8n + c, every B-operand value a lane needs (element c of steps
    // 8*kb .. 8*kb+7) is already in its own registers; P is stored in LDS as
    // [row][key % 4][key / 4] so that the A operand (row lane%16, keys
    // 4*(8*kb + e) + lane/16) is 8 consecutive floats.  O then lives in the
    // MFMA output layout: oc[c][i] = O[4g + i][8n + c].
    constexpr bool MFMA_PV = MFMA_S && VT == kF16 && Sh::V_REG && D == 128;
    // Block-type V rows in LDS at head_dim 128: P.V on the matrix cores with
    // the same lane layout, lane (g, n) decoding dims 8n .. 8n+7 of key
    // 4*st + g; the dequantised values d * code (exact in f32) are split into
    // binary16 high and low parts and three MFMAs (Ph.Bh, Ph.Bl, Pl.Bh) keep
    // about 22 bits.  The MFMA cost does not depend on the row count (rows are
    // padded to 16), while the VALU form decodes and multiplies every value
    // once per row: even at 1 row the matrix cores leave the VALU far less.
    constexpr bool MFMA_PVB = MFMA_S && (VT == kQ8 || VT == kQ4 || VT == kT3) && !Sh::V_REG && D == 128;
    constexpr bool MFMA_O = MFMA_PV || MFMA_PVB;  // O held in the MFMA output layout
    static_assert(DS == 1 || MFMA_PVB, "dim slices need block-type K and V on the matrix cores");
    constexpr int NKQ = MFMA_S ? D / 32 : 1;
    rkv_half8 qhi[NKQ], qlo[NKQ];
    int oex[4] = {0, 0, 0, 0};  // query-row exponents of the lane's MFMA output rows
    bool qscaled = false;         // some row of the wave has one (wave-uniform)
    float mrow[4], lrow[4];
    const float capl = cap * kLog2e;                  // cap in log2 units
    const float two_over_cap = cap > 0.f ? 2.f / cap : 0.f;

    // Software pipelining of the tile stream: when the raw rows of a tile fit
    // in registers, the loads of tile i+1's K (and block-type V) rows are
    // issued once tile i's scores are done (its K rows in LDS are no longer
    // needed after the next store), and the loads of tile i+1's register-held
    // V rows right after tile i's P.V, so a wave keeps its next tile in
    // flight while it computes, with at most one tile of raw rows in registers
    // beside the P.V working set.
    using KRegs = RowRegs<Sh::RBK, VWK>;
    using VRegs = RowRegs<Sh::RBV, VWV>;
    constexpr int RAW_DW = KRegs::IT * KRegs::NWD + (V_REG ? NSTEP * VRW : VRegs::IT * VRegs::NWD);
    constexpr bool PIPE = !Sh::KDMA && RAW_DW <= 64 && !MFMA_S;  // MFMA operands need those registers
    // Block-type K and V with the matrix-core scores: both tiles go global ->
    // LDS by dword DMA (no staging registers); a tile's K rows go out once
    // the previous tile's scores are done, its V rows after the previous P.V,
    // and the wait for K leaves V's loads in flight.
    constexpr bool BDMA = MFMA_S && (KT == kQ8 || KT == kQ4) && (VT == kQ8 || VT == kQ4 || VT == kT3) && Sh::RBK % 4 == 0 &&
                          Sh::RBV % 4 == 0 && LSK <= 64 && LSV <= 64;
    constexpr int NVD = LSV < 63 ? LSV : 63;  // V loads a wait for K may leave outstanding
    static_assert(!VDB || BDMA, "the second V buffer belongs to the block-type DMA path");
    KRegs kr;
    VRegs vr;
    uint32_t vreg[V_REG ? NSTEP : 1][VRW];
    int vps = (int)sg.v_pos;
    asm volatile("" : "+s"(vps));
    // (whole tiles: lane offset ks * vps + dg * 4 VRW, computed once; the
    // step's uniform part st * KPS * vps goes into the scalar base)
    const uint32_t voff_lane = (uint32_t)ks * (uint32_t)vps + (uint32_t)(dg * (VRW * 4));
    auto load_v_into = [&](uint32_t (&dst)[V_REG ? NSTEP : 1][VRW], int64_t t, int nkk) {
        if constexpr (!V_REG) return;
        const uint8_t *vt = vg + t * sg.v_pos;
        if (nkk == kTile) {
            // buffer loads: the tile base in a scalar resource, the step in
            // the scalar offset, the lane's offset in one vector register;
            // non-temporal like the K tile's DMA when each byte is read once
            // by the launch (whole lines: on the 48-layer f16 step 4.5 % less
            // time for the attention kernel than the default cache policy),
            // the default policy when other row groups read the tile too
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(vt);
            auto issue = [&](auto policy) {
                constexpr int kAux = decltype(policy)::value;  // cache-policy bits: 2 = nt
#pragma unroll
                for (int st = 0; st < NSTEP; ++st) {
                    const rkv_u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, voff_lane, st * KPS * vps, kAux);
                    uint32_t *vr8 = &dst[st][0];
                    vr8[0] = a.x; vr8[1] = a.y; vr8[2] = a.z; vr8[3] = a.w;
                    if constexpr (VRW == 8) {
                        const rkv_u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rs, voff_lane + 16u, st * KPS * vps, kAux);
                        vr8[4] = b.x; vr8[5] = b.y; vr8[6] = b.z; vr8[7] = b.w;
                    }
                }
            };
            if (p.stream_once)
                issue(std::integral_constant<int, 2>{});
            else
                issue(std::integral_constant<int, 0>{});
            return;
        }
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            const int key = st * KPS + ks;
            const int keyc = key < nkk ? key : nkk - 1;  // weight 0 in P.V, finite data
            const uint8_t *pv = vt + (uint32_t)(keyc * vps + dg * (VRW * 4));
            const uint4 a = *(const uint4 *)pv;
            uint32_t *vr8 = &dst[st][0];
            vr8[0] = a.x; vr8[1] = a.y; vr8[2] = a.z; vr8[3] = a.w;
            if constexpr (VRW == 8) {
                const uint4 b = *(const uint4 *)(pv + 16);
                vr8[4] = b.x; vr8[5] = b.y; vr8[6] = b.z; vr8[7] = b.w;
            }
        }
    };
    auto load_vreg = [&](int64_t t, int nkk) { load_v_into(vreg, t, nkk); };
    auto nk_at = [&](int64_t t) { return (int)(kend - t < kTile ? kend - t : kTile); };

    constexpr bool KDMA = Sh::KDMA;
    // Whole-tile K DMA offsets: load i covers rows R i + g (R = 64 / CPR,
    // g = lane / CPR), chunk slot lane % CPR, whose chunk is swizzled by
    // kswz(R i + g) = kswz(g) ^ kswz(R i) (no carries for these row counts),
    // so the lane's offset is its row part plus (its chunk of load 0) ^ a
    // constant of i; the rest of the address is uniform.
    constexpr int KCPR = KDMA ? Sh::RBK / 16 : 16;
    uint32_t krow = 0, kchunk = 0;
    if constexpr (KDMA) {
        static_assert(64 % KCPR == 0, "whole-tile DMA plan");
        krow = (uint32_t)(lane / KCPR) * (uint32_t)sg.k_pos;
        kchunk = 16u * (uint32_t)((lane % KCPR) ^ kswz<Sh::RBK>(lane / KCPR));
    }
    // Issue the direct global -> LDS loads of a tile's K rows (rows past nkk
    // repeat row nkk-1).  Lane l of load i fills slot i*64 + l of the tile.
    auto dma_k = [&](int64_t t, int nkk) {
        if constexpr (KDMA) {
            constexpr int CPR = Sh::RBK / 16;
            constexpr int NI = kTile * Sh::RBK / 1024;
            int kps = (int)sg.k_pos;
            asm volatile("" : "+s"(kps));
            const uint8_t *kt = kg + t * sg.k_pos;
            const uint32_t base = lds_addr(smem + w * Sh::STAGE_DW);
            waitcnt_lgkm0();  // this wave's earlier LDS reads of the buffer are done
            auto issue = [&](auto policy) {
                constexpr bool NT = decltype(policy)::value;
                if (nkk == kTile) {
                    // grouped buffer loads: load i at i * (64 / CPR) rows plus
                    // the lane's swizzled chunk of its row
                    uint32_t vo[NI];
#pragma unroll
                    for (int i = 0; i < NI; ++i) vo[i] = krow + (kchunk ^ (16u * (uint32_t)kswz<Sh::RBK>(i * (64 / CPR))));
                    dma16_groups<NT, NI>(buffer_rsrc(kt), vo, (uint32_t)(64 / CPR) * (uint32_t)kps, base);
                    return;
                }
                static_for<0, NI>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    const int slot = i * 64 + lane;
                    const int j = slot / CPR, cs = slot % CPR;
                    const int c = cs ^ kswz<Sh::RBK>(j);
                    const int jc = j < nkk ? j : nkk - 1;
                    lds_dma16<NT, 1024u * i>(kt + (uint32_t)(jc * kps + 16 * c), base);
                });
            };
            if (p.stream_once)
                issue(std::integral_constant<bool, true>{});
            else
                issue(std::integral_constant<bool, false>{});
        }
    };
    // Block-type K and V tiles by dword DMA, issued separately: a tile's K
    // rows once the previous tile's scores have read theirs, its V rows once
    // the previous tile's P.V has read theirs.
    // A whole tile followed by another position of the segment, with
    // position strides of at least a padded row and below 2^23 bytes, takes
    // the clamp-free form; the segment's last tile the clamped one.
    constexpr int LSK1 = LSK > 0 ? LSK : 1, LSV1 = LSV > 0 ? LSV : 1;
    const uint64_t kwrap = BDMA ? dma_wraps<LSK1>(lane) : 0, vwrap = BDMA ? dma_wraps<LSV1>(lane) : 0;
    const bool kfull_ok = sg.k_pos >= 4 * LSK && sg.k_pos < (1 << 23);
    const bool vfull_ok = sg.v_pos >= 4 * LSV && sg.v_pos < (1 << 23);
    // V rows short enough for several whole rows per load take the whole-row
    // copy (no per-lane arithmetic per load); the others the slot plan.
    // Either issues at least LSV loads, the count the waits below assume.
    constexpr int LSVR = BDMA ? LSV1 : 1;  // (a placeholder shape off the DMA path)
    constexpr int RBDV = BDMA ? Sh::RBV / 4 : 1;
    using VRow = RowDma<RBDV, LSVR>;
    constexpr bool V_ROWS = BDMA && VRow::R >= 2;
    static_assert(!V_ROWS || VRow::NL >= LSV, "the whole-row V copy issues at least as many loads as the slot plan");
    // lane offsets of load 0 of the slot plans (no wraps before it)
    const uint32_t koff0 = BDMA ? (uint32_t)(lane / LSK1) * (uint32_t)(sg.k_pos - 4 * LSK1) + 4u * (uint32_t)lane : 0u;
    const uint32_t voff0 = !BDMA ? 0u
                           : V_ROWS ? row_dma_voff<LSV1>((int)sg.v_pos, lane)
                                    : (uint32_t)(lane / LSV1) * (uint32_t)(sg.v_pos - 4 * LSV1) + 4u * (uint32_t)lane;
    auto dma_kb = [&](int64_t t, int nkk) {
        if constexpr (BDMA) {
            int kps = (int)sg.k_pos;
            asm volatile("" : "+s"(kps));
            waitcnt_lgkm0();  // this wave's earlier LDS reads of the K buffer are done
            const uint32_t base = lds_addr(smem + w * Sh::STAGE_DW);
            if (kfull_ok && nkk == kTile && t + kTile < sg.n_keys) {
                uint32_t vo = koff0;
                dma_rows4_grp<LSK1, 0, LSK1>(buffer_rsrc(kg + t * sg.k_pos), vo, kwrap, kps, base);
            } else {
                dma_rows4<Sh::RBK / 4, LSK>(kg + t * sg.k_pos, kps, nkk, base, lane);
            }
        }
    };
    // V rows of a whole tile can go out in two parts: the loads that touch rows
    // 0..31 only (part 1: loads [0, LSV / 2) of the slot plan, [0, 32 / R) of
    // the whole-row copy), once the first half of P.V has read those rows, and
    // the rest (part 2) after P.V; part 0 is all of them.  vfull(t, nkk): the
    // tile takes the whole-tile copy (a tile that does not goes out whole).
    constexpr int VH1 = V_ROWS ? 32 / VRow::R : LSV1 / 2;
    auto vfull = [&](int64_t t, int nkk) { return vfull_ok && nkk == kTile && t + kTile < sg.n_keys; };
    uint32_t vo_part = 0;  // the slot plan's lane offset between the two parts
    auto dma_vb = [&](int64_t t, int nkk, const uint32_t *dst, auto partc) {
        if constexpr (BDMA) {
            constexpr int PART = decltype(partc)::value;
            int vps2 = (int)sg.v_pos;
            asm volatile("" : "+s"(vps2));
            waitcnt_lgkm0();  // this wave's earlier LDS reads of the V buffer are done
            const uint32_t base = lds_addr(dst);
            if (vfull(t, nkk)) {
                const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(vg + t * sg.v_pos);
                if constexpr (V_ROWS) {
                    constexpr int I0 = PART == 2 ? VH1 : 0, I1 = PART == 1 ? VH1 : VRow::NL;
                    dma_rows_whole<RBDV, LSVR, I0, I1>(rs, voff0, vps2, (uint32_t)VRow::R * (uint32_t)(vps2 - 4 * LSVR),
                                                       base);
                } else {
                    constexpr int I0 = PART == 2 ? VH1 : 0, I1 = PART == 1 ? VH1 : LSV1;
                    if constexpr (PART != 2) vo_part = voff0;
                    dma_rows4_grp<LSV1, I0, I1>(rs, vo_part, vwrap, vps2, base);
                }
            } else if constexpr (PART != 1) {
                dma_rows4<Sh::RBV / 4, LSV>(vg + t * sg.v_pos, vps2, nkk, base, lane);
            }
        }
    };
    // VMEM instructions one load_v_into issues (outstanding loads a wait may leave)
    constexpr int NV = V_REG ? NSTEP * (VRW / 4) : 0;
    static_assert(2 * NV <= 63, "vmcnt range");
    const int sw = kswz<Sh::RBK>(lane);

    // P.V of this wave's staged block-type V tile on the matrix cores
    // (MFMA_PVB), for tiles whose block scales keep d * code inside binary16.
    // mid() runs once the first 32-key half's products are issued (its V rows
    // 0..31 are then no longer read by this tile).
    auto pv_blk = [&](auto &&mid) {
        const int qi = lane & 15, gq = lane >> 4;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            rkv_half8 ph, pl;
            if (qi < RT) {
                const float4 a = *(const float4 *)&sPw[qi * kTile + gq * 16 + 8 * kb];
                const float4 b = *(const float4 *)&sPw[qi * kTile + gq * 16 + 8 * kb + 4];
                const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const _Float16 h = (_Float16)x[e];
                    ph[e] = h;
                    pl[e] = (_Float16)(x[e] - (float)h);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    ph[e] = (_Float16)0.f;
                    pl[e] = (_Float16)0.f;
                }
            }
            // B operands built two keys at a time: element e of bh[c] / bl[c]
            // is d * code of dim 8n + c of key 4*(8kb + e) + g.  The codes are
            // exact in binary16; hi = d * code rounded once (packed f16
            // multiply) and lo = d * code - hi (packed f16 fma, exact while
            // |d * code| <= 65504, which the scale test guarantees).
            // TBQ3: element e is the signed level of dim 8n + c of that key
            // (the key's n / sqrt(128) is in P), high and low parts from the
            // table, two values per lookup.
            uint32_t hw[8][4], lw[8][4];
            if constexpr (VT == kT3) {
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const uint32_t *ra = sV + (4 * (8 * kb + 2 * e2) + gq) * LSV, *rb = ra + 4 * LSV;
                    const uint32_t qa = ra[1 + (qi >> 1)] >> (16 * (qi & 1)), qb = rb[1 + (qi >> 1)] >> (16 * (qi & 1));
                    const uint32_t sa = ra[9 + (qi >> 2)] >> (8 * (qi & 3)), sb = rb[9 + (qi >> 2)] >> (8 * (qi & 3));
#pragma unroll
                    for (int p2 = 0; p2 < 4; ++p2) {
                        const uint2 ta = sT3[((qa >> (4 * p2)) & 15u) | (((sa >> (2 * p2)) & 3u) << 4)];
                        const uint2 tb = sT3[((qb >> (4 * p2)) & 15u) | (((sb >> (2 * p2)) & 3u) << 4)];
                        hw[2 * p2][e2] = __builtin_amdgcn_perm(tb.x, ta.x, 0x05040100u);
                        hw[2 * p2 + 1][e2] = __builtin_amdgcn_perm(tb.x, ta.x, 0x07060302u);
                        lw[2 * p2][e2] = __builtin_amdgcn_perm(tb.y, ta.y, 0x05040100u);
                        lw[2 * p2 + 1][e2] = __builtin_amdgcn_perm(tb.y, ta.y, 0x07060302u);
                    }
                }
            } else if constexpr (VT == kQ8) {
                // (key a, key b) pairs of each dim converted straight from
                // the two keys' code bytes
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    uint32_t wa[2], wb[2], da, db;
                    v_group_bytes_q8(sV + (4 * (8 * kb + 2 * e2) + gq) * LSV, qi, wa, da);
                    v_group_bytes_q8(sV + (4 * (8 * kb + 2 * e2 + 1) + gq) * LSV, qi, wb, db);
                    const rkv_half2 d2 = __builtin_bit_cast(rkv_half2, da | (db << 16));
                    rkv_half2 x[8];
                    x[0] = __builtin_bit_cast(rkv_half2, i8_f16_pair<0, 0>(wa[0], wb[0]));
                    x[1] = __builtin_bit_cast(rkv_half2, i8_f16_pair<1, 1>(wa[0], wb[0]));
                    x[2] = __builtin_bit_cast(rkv_half2, i8_f16_pair<2, 2>(wa[0], wb[0]));
                    x[3] = __builtin_bit_cast(rkv_half2, i8_f16_pair<3, 3>(wa[0], wb[0]));
                    x[4] = __builtin_bit_cast(rkv_half2, i8_f16_pair<0, 0>(wa[1], wb[1]));
                    x[5] = __builtin_bit_cast(rkv_half2, i8_f16_pair<1, 1>(wa[1], wb[1]));
                    x[6] = __builtin_bit_cast(rkv_half2, i8_f16_pair<2, 2>(wa[1], wb[1]));
                    x[7] = __builtin_bit_cast(rkv_half2, i8_f16_pair<3, 3>(wa[1], wb[1]));
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const rkv_half2 h = d2 * x[c];
                        const rkv_half2 l = __builtin_elementwise_fma(d2, x[c], -h);
                        hw[c][e2] = __builtin_bit_cast(uint32_t, h);
                        lw[c][e2] = __builtin_bit_cast(uint32_t, l);
                    }
                }
            } else {
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                uint32_t ca[4], cb[4], da, db;
                v_group_codes_f16<VT>(sV + (4 * (8 * kb + 2 * e2) + gq) * LSV, qi, ca, da);
                v_group_codes_f16<VT>(sV + (4 * (8 * kb + 2 * e2 + 1) + gq) * LSV, qi, cb, db);
                const rkv_half2 d2 = __builtin_bit_cast(rkv_half2, da | (db << 16));
#pragma unroll
                for (int p2 = 0; p2 < 4; ++p2) {
                    // (key a, key b) of dims 2*p2 and 2*p2 + 1
                    const rkv_half2 x0 = __builtin_bit_cast(rkv_half2, __builtin_amdgcn_perm(cb[p2], ca[p2], 0x05040100u));
                    const rkv_half2 x1 = __builtin_bit_cast(rkv_half2, __builtin_amdgcn_perm(cb[p2], ca[p2], 0x07060302u));
                    const rkv_half2 h0 = d2 * x0, h1 = d2 * x1;
                    const rkv_half2 l0 = __builtin_elementwise_fma(d2, x0, -h0);
                    const rkv_half2 l1 = __builtin_elementwise_fma(d2, x1, -h1);
                    hw[2 * p2][e2] = __builtin_bit_cast(uint32_t, h0);
                    hw[2 * p2 + 1][e2] = __builtin_bit_cast(uint32_t, h1);
                    lw[2 * p2][e2] = __builtin_bit_cast(uint32_t, l0);
                    lw[2 * p2 + 1][e2] = __builtin_bit_cast(uint32_t, l1);
                }
            }
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const rkv_half8 bh = __builtin_bit_cast(rkv_half8, hw[c]);
                const rkv_half8 bl = __builtin_bit_cast(rkv_half8, lw[c]);
                oc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, bh, oc[c], 0, 0, 0);
                oc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, bl, oc[c], 0, 0, 0);
                oc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, bh, oc[c], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (kb == 0) mid();
        }
    };

    // Query rows of the matrix-core path, loaded before the first tile's K / V
    // loads are issued.  The row of lane l is row l % 16 of the wave's group:
    // the row table is read with wave-uniform (scalar) loads and picked per
    // lane, since a per-lane read of it would be a vector load whose wait
    // would also wait for the tile loads.
    float qraw[NKQ][8];
    if constexpr (MFMA_S) {
        const int qr = lane & 15;
        int rowi = 0;
#pragma unroll
        for (int r = 0; r < RT; ++r) rowi = (qr == r && tabrow[r] >= 0) ? tabrow[r] : rowi;
        mfma_q_load<D>(q + (int64_t)rowi * DF + js * D, lane, qraw);
    }

    int64_t t0 = kbeg + (p.rg_waves ? 0 : (int64_t)ws * kTile);
    // VMEM loads issued after the K rows' DMA that may stay outstanding when
    // the scores start: 0 or NV.
    //
    // Order of a tile's loads with K by DMA and V in registers: both are
    // issued together, right after the previous tile's P.V (and, for the
    // first tile, before the query rows are loaded), so that a wave waits
    // for one load latency per tile.  The DMA is invisible to the compiler's
    // wait counting: a DMA issued before P.V would be waited for by the
    // compiler's wait on the V registers, so none is in flight there.
    int v_after_dma = 0;
    if constexpr (BDMA) {
        if (t0 < kend) {
            dma_kb(t0, nk_at(t0));
            dma_vb(t0, nk_at(t0), sV, std::integral_constant<int, 0>{});
        }
    } else if constexpr (KDMA) {
        if (t0 < kend) {
            dma_k(t0, nk_at(t0));
            if constexpr (V_REG) {
                load_vreg(t0, nk_at(t0));
                v_after_dma = NV;
            }
        }
    } else if constexpr (PIPE) {
        if (t0 < kend) {
            load_rows(kr, kg + t0 * sg.k_pos, (int)sg.k_pos, nk_at(t0), lane);
            if constexpr (V_REG) load_vreg(t0, nk_at(t0));
            else load_rows(vr, vg + t0 * sg.v_pos, (int)sg.v_pos, nk_at(t0), lane);
        }
    }
    if constexpr (MFMA_S) {
        // the pin keeps the conversion (and the waits for the query loads)
        // after the first tile's loads have been issued
        pin_v<8 * NKQ>(&qraw[0][0]);
        const int qex = mfma_q_split<D>(qraw, (lane & 15) < nr, sl2, qhi, qlo);
        mfma_out_row_exps(qex, lane, oex);
        qscaled = __builtin_amdgcn_ballot_w64(qex != 0) != 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mrow[i] = -INFINITY;
            lrow[i] = 0.f;
        }
    }
    // limit of the row of each of the lane's MFMA outputs (rows 4*(lane/16) + i)
    int limv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * (lane >> 4) + i;
        int x = kSeeAll;
#pragma unroll
        for (int r = 0; r < RT; ++r) x = row == r ? lim[r] : x;
        limv[i] = x;
    }
    for (; t0 < kend; t0 += tstep) {
        const int nk = nk_at(t0);
        const int64_t tn = t0 + tstep;
        bool v_mid = false;  // the first part of the next tile's V rows went out during P.V
        if constexpr (BDMA) {
            // K went out before the previous tile's P.V and V after it (with
            // VDB right after K): once at most V's loads are outstanding this
            // tile's K rows have landed
            waitcnt_vm<NVD>();
        } else if constexpr (KDMA) {
            // K rows arrive by DMA issued one tile ahead (V rows in registers
            // were issued with them; block-type V rows are staged now).
            if constexpr (!V_REG) {
                stage_rows<Sh::RBV, VWV, LSV>(vg + t0 * sg.v_pos, (int)sg.v_pos, nk, sV, lane);
                v_after_dma = 0;
            }
            // this tile's K rows (DMA) have landed; its V loads may still fly
            if (v_after_dma == NV) waitcnt_vm<NV>();
            else waitcnt_vm<0>();
        } else if constexpr (PIPE) {
            store_rows<Sh::RBK, VWK, LSK>(kr, sK, lane);
            if constexpr (!V_REG) store_rows<Sh::RBV, VWV, LSV>(vr, sV, lane);
        } else {
            if constexpr (V_REG) load_vreg(t0, nk);
            stage_rows<Sh::RBK, VWK, LSK>(kg + t0 * sg.k_pos, (int)sg.k_pos, nk, sK, lane);
            if constexpr (!V_REG) stage_rows<Sh::RBV, VWV, LSV>(vg + t0 * sg.v_pos, (int)sg.v_pos, nk, sV, lane);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS stores are done
        __builtin_amdgcn_wave_barrier();

        if constexpr (MFMA_S) {
            // ---- scores on the matrix cores
            float sv[4][4];
            if constexpr (KT == kQ8 || KT == kQ4) mfma_scores_blk<KT, D, LSK>(sK, qhi, qlo, lane, sv);
            else mfma_scores<D, Sh::RBK>(sK, qhi, qlo, lane, sv);
            // (before the slices exchange their partial scores: each slice
            // scaled its query rows by its own power of two)
            if (qscaled) unscale_rows(sv, oex);
            if constexpr (VDB) {
                // the next tile's K rows (its V rows into the other buffer)
                // load through the rest of this tile; then this tile's V rows,
                // issued before them, have landed once at most their loads
                // are outstanding
                __builtin_amdgcn_wave_barrier();
                if (tn < kend) {
                    dma_kb(tn, nk_at(tn));
                    dma_vb(tn, nk_at(tn), sVn, std::integral_constant<int, 0>{});
                    waitcnt_vm<LSK + LSV>();
                } else {
                    waitcnt_vm<0>();
                }
                __builtin_amdgcn_wave_barrier();
            } else if constexpr (BDMA) {
                // this tile's V rows have landed (nothing else is in flight), so
                // the next tile's K rows can load through the rest of the tile
                waitcnt_vm<0>();
                __builtin_amdgcn_wave_barrier();
                if (tn < kend) dma_kb(tn, nk_at(tn));
            }
            if constexpr (DS > 1) {
                // The head's slices exchange their partial scores: lane l holds
                // rows 4*(l/16) .. +3 of keys 16*kb + l%16, so lanes below 4*RTX
                // carry every real row; each slice sums the DS partials in slice
                // order (the same sums, bit for bit, in all DS waves).
                constexpr int XL = 4 * RTX;
                float4 *xs = (float4 *)&sP[w][0];
                if (lane < XL) {
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) xs[kb * XL + lane] = make_float4(sv[kb][0], sv[kb][1], sv[kb][2], sv[kb][3]);
                }
                __syncthreads();
                if (lane < XL) {
                    float4 a4[4];
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) a4[kb] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                    for (int j = 0; j < DS; ++j) {
                        const float4 *xo = (const float4 *)&sP[w - js + j][0];
#pragma unroll
                        for (int kb = 0; kb < 4; ++kb) {
                            const float4 x = xo[kb * XL + lane];
                            a4[kb].x += x.x;
                            a4[kb].y += x.y;
                            a4[kb].z += x.z;
                            a4[kb].w += x.w;
                        }
                    }
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) {
                        sv[kb][0] = a4[kb].x;
                        sv[kb][1] = a4[kb].y;
                        sv[kb][2] = a4[kb].z;
                        sv[kb][3] = a4[kb].w;
                    }
                }
                __syncthreads();  // every slice has read the partials before P overwrites them
            }
            // last key of the tile each output row sees; a masked launch
            // masks only the tiles that reach past some row's last key
            const bool tile_masked = p.masked && t0 + nk - 1 > lim_min;
            int kmx[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) kmx[i] = nk - 1;
            if (tile_masked) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tl = limv[i] - (int)t0;
                    kmx[i] = tl < nk - 1 ? (tl < -1 ? -1 : tl) : nk - 1;
                }
            }
            if (tile_masked || nk < kTile) {
                if (cap > 0.f)
                    cap_mask_tile<true, true>(sv, kmx, lane & 15, capl, two_over_cap);
                else
                    cap_mask_tile<false, true>(sv, kmx, lane & 15, capl, two_over_cap);
            } else if (cap > 0.f) {
                cap_mask_tile<true, false>(sv, kmx, lane & 15, capl, two_over_cap);
            }
            // ---- online softmax: per-lane rows, then the wave-uniform rescale
            // (a row that has seen no key yet keeps m = -inf, l = 0: its
            // exponents are taken against 0 so that they give 0, not NaN)
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
            if constexpr (MFMA_O) {
                // (a row whose maximum did not move has al = 2^0 = 1 exactly:
                // the rescale is skipped when no row of the wave moved)
                if (__builtin_amdgcn_ballot_w64(al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f)) {
#pragma unroll
                    for (int c = 0; c < 8; ++c)
#pragma unroll
                        for (int i = 0; i < 4; ++i) oc[c][i] *= al[i];
                }
            } else {
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    const float mu = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mrow[r & 3]), 16 * (r >> 2)));
                    if (mu > m[r]) {
                        const float alpha = __builtin_amdgcn_exp2f(m[r] - mu);
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
                        m[r] = mu;
                    }
                }
            }
            // TBQ3 values: P is stored times the key's n / sqrt(128) (the
            // value scale; the denominator takes P itself)
            float vs[4] = {1.f, 1.f, 1.f, 1.f};
            if constexpr (VT == kT3) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) vs[kb] = h2f(sV[(16 * kb + (lane & 15)) * LSV]) * 0.088388347648318440550f;
            }
            // (the probabilities first, then the stores of the lanes that
            // hold real rows under as few lane tests as RT allows: one when
            // every lane group holds whole rows)
            float pvs[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float ps = 0.f;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    pvs[kb][i] = __builtin_amdgcn_exp2f(sv[kb][i] - mex[i]);
                    ps += pvs[kb][i];
                }
                lrow[i] += ps;
            }
            auto store_row = [&](int i) {
                const int row = 4 * (lane >> 4) + i;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const int key = 16 * kb + (lane & 15);
                    const int at = MFMA_O ? (key & 3) * 16 + (key >> 2) : key;
                    sPw[row * kTile + at] = VT == kT3 ? pvs[kb][i] * vs[kb] : pvs[kb][i];
                }
            };
            if constexpr (RT % 4 == 0) {
                if (4 * (lane >> 4) < RT) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) store_row(i);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * (lane >> 4) + i < RT) store_row(i);
            }
        } else {
        // ---- scores, one key per lane
        float s[RT];
        if constexpr (KDMA) key_dots<KT, D, RT, true>(sK, qp, s, lane, sw);
        else key_dots<KT, D, RT>(sK + lane * LSK, qp, s);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            float x;
            if (cap > 0.f)
                x = cap * tanh_from_exp2(s[r] * scale_over_cap * (2.f * kLog2e)) * kLog2e;
            else
                x = s[r] * sl2;
            // last key of the tile row r sees (wave-uniform)
            const int tl = lim[r] - (int)t0;
            const int kmr = tl < nk - 1 ? (tl < -1 ? -1 : tl) : nk - 1;
            s[r] = lane <= kmr ? x : -INFINITY;
        }

        // ---- online softmax update (rescale only when a row's max moved)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const float mn = fmaxf(m[r], wave_max(s[r]));
            if (mn > m[r]) {
                const float alpha = __builtin_amdgcn_exp2f(m[r] - mn);
                l[r] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r][e] *= alpha;
                m[r] = mn;
            }
            // (a row that has seen no key yet has m = -inf and gets 0)
            const float pr = m[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s[r] - m[r]);
            l[r] += pr;
            sPw[r * kTile + lane] = pr;
        }
        }
        // the next tile's K (and block-type V) rows load during this tile's P.V
        // (with V in registers they load after it, see above)
        if constexpr (KDMA) {
            if constexpr (!V_REG) {
                if (tn < kend) dma_k(tn, nk_at(tn));
            }
        } else if constexpr (PIPE) {
            if (tn < kend) {
                load_rows(kr, kg + tn * sg.k_pos, (int)sg.k_pos, nk_at(tn), lane);
                if constexpr (!V_REG) load_rows(vr, vg + tn * sg.v_pos, (int)sg.v_pos, nk_at(tn), lane);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();

        if constexpr (MFMA_PVB) {
            // ---- P.V on the matrix cores, block-type V (see where MFMA_PVB is set)
            // A tile with a block scale large enough for d * code to overflow
            // binary16 (rare) is multiplied out in binary32 on the VALU.
            // (TBQ3: levels below 2.2, P times n / sqrt(128) below 5800)
            // (one buffer per wave: the next tile's V rows 0..31 go out once
            // the first half of P.V has read them)
            auto mid = [&]() {
                if constexpr (BDMA && !VDB) {
                    if (tn < kend) {
                        dma_vb(tn, nk_at(tn), sV, std::integral_constant<int, 1>{});
                        v_mid = true;
                    }
                }
            };
            if constexpr (VT == kT3) {
                pv_blk(mid);
            } else {
                const uint32_t vmx = v_row_scale_max<VT, D / 32>(sV + lane * LSV);
                if (__builtin_amdgcn_ballot_w64(vmx >= v_scale_limit<VT>()) == 0)
                    pv_blk(mid);
                else
                    pv_valu_tile<VT, LSV>(
                        sV, [&](int r, int k) { return sPw[r * kTile + (k & 3) * 16 + (k >> 2)]; }, RT, lane, oc);
            }
        } else if constexpr (MFMA_PV) {
            // ---- P.V on the matrix cores (layout described where MFMA_PV is set)
            const int qi = lane & 15, gq = lane >> 4;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                rkv_half8 ph, pl;
                if (qi < RT) {
                    const float4 a = *(const float4 *)&sPw[qi * kTile + gq * 16 + 8 * kb];
                    const float4 b = *(const float4 *)&sPw[qi * kTile + gq * 16 + 8 * kb + 4];
                    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const _Float16 h = (_Float16)x[e];
                        ph[e] = h;
                        pl[e] = (_Float16)(x[e] - (float)h);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        ph[e] = (_Float16)0.f;
                        pl[e] = (_Float16)0.f;
                    }
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    uint32_t bw[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const uint32_t lo = vreg[8 * kb + 2 * e2][c >> 1], hi = vreg[8 * kb + 2 * e2 + 1][c >> 1];
                        bw[e2] = __builtin_amdgcn_perm(hi, lo, (c & 1) ? 0x07060302u : 0x05040100u);
                    }
                    const rkv_half8 bv = __builtin_bit_cast(rkv_half8, bw);
                    oc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, bv, oc[c], 0, 0, 0);
                    oc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, bv, oc[c], 0, 0, 0);
                }
            }
        } else {
        // ---- P.V (fully unrolled when V sits in registers: vreg is indexed by st).
        // Keys past nk have weight 0 and finite (repeated) data.
#pragma unroll V_REG ? NSTEP : MFMA_S ? 2 : 4
        for (int st = 0; st < NSTEP; ++st) {
            const int key = st * KPS + ks;
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
                dsc = v_group_lds<VT, D>(sV + key * LSV, dg, x, p.tbq_lv);
            }
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                const float pw = (VT == kQ8 || VT == kQ4 || VT == kT3) ? sPw[r * kTile + key] * dsc : sPw[r * kTile + key];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(pw, x[e], acc[r][e]);
            }
        }
        }
        if constexpr (PIPE && V_REG) {
            if (tn < kend) load_vreg(tn, nk_at(tn));
        }
        if constexpr (VDB) {
            uint32_t *const sx = sV;
            sV = sVn;
            sVn = sx;
        } else if constexpr (BDMA) {
            if (tn < kend) {
                if (v_mid)
                    dma_vb(tn, nk_at(tn), sV, std::integral_constant<int, 2>{});
                else
                    dma_vb(tn, nk_at(tn), sV, std::integral_constant<int, 0>{});
            }
        }
        if constexpr (KDMA && V_REG) {
            v_after_dma = 0;
            if (tn < kend) {
                dma_k(tn, nk_at(tn));
                load_vreg(tn, nk_at(tn));
                v_after_dma = NV;
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
    }

    // ---- merge the waves of the workgroup in LDS.  Per wave and row: m, l,
    // and acc[D] summed over the wave's key-in-step lane groups.
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        if constexpr (MFMA_S) {
            // per-lane partial sums of row r live in the 16 lanes of its group
            const float t = row16_sum(lrow[r & 3]);
            l[r] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, t), 16 * (r >> 2)));
            if constexpr (MFMA_O)
                m[r] = __builtin_bit_cast(float,
                                          __builtin_amdgcn_readlane(__builtin_bit_cast(int, mrow[r & 3]), 16 * (r >> 2)));
        } else {
            l[r] = wave_sum(l[r]);
        }
    }
    if constexpr (MFMA_O) {
        if (DS > 1 || wph == 1 || p.rg_waves) {
            // One wave per KV head (or dim slice, or row group over all the
            // split's keys): nothing to merge inside the workgroup, so
            // the wave writes its rows straight from the MFMA output layout
            // (lane (g, n) holds dims 8n .. 8n+7 of rows 4g .. 4g+3).  The
            // values are those the LDS merge would produce for one wave.
            // (output rows from the wave's copy of the row table in LDS, so
            // that the table does not hold scalar registers through the loop)
            const bool single = p.direct != 0;
            const int64_t pbase = (int64_t)(p.split_off + (int)blockIdx.x) * p.n_rows_total;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * (lane >> 4) + i;
                const int rr = row < RT ? sRow[w][row] : -1;
                float lr = 1.f;
#pragma unroll
                for (int r = 0; r < RT; ++r) lr = row == r ? l[r] : lr;
                if (rr < 0) continue;
                float v[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) v[c] = single ? (lr > 0.f ? oc[c][i] / lr : 0.f) : oc[c][i];
                float *dst = (single ? o_out + (int64_t)rr * DF : part_acc + (pbase + rr) * DF) + js * D;
                *(float4 *)(dst + 8 * (lane & 15)) = make_float4(v[0], v[1], v[2], v[3]);
                *(float4 *)(dst + 8 * (lane & 15) + 4) = make_float4(v[4], v[5], v[6], v[7]);
            }
            if (js == 0 && lane < RT) {
                const int rr = sRow[w][lane];
                float mr = 0.f, lr = 1.f;
#pragma unroll
                for (int r = 0; r < RT; ++r) {
                    mr = lane == r ? m[r] : mr;
                    lr = lane == r ? l[r] : lr;
                }
                if (rr >= 0) {
                    if (single) lse_out[rr] = (mr + log2f(lr)) * 0.69314718055994531f;
                    else part_ml[(int64_t)rr * p.n_splits_all + p.split_off + blockIdx.x] = make_float2(mr, lr);
                }
            }
            return;
        }
    }
    __syncthreads();  // every wave is done with its staging area
    float *mA = (float *)smem;                  // [NW][RT][D]
    float *mML = mA + NW * RT * D;              // [NW][RT][2]
    if constexpr (MFMA_O) {
        // oc[c][i] = O[4g + i][8n + c]: every element once
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 4 * (lane >> 4) + i;
            if (row < RT) {
#pragma unroll
                for (int c = 0; c < 8; ++c) mA[(w * RT + row) * D + 8 * (lane & 15) + c] = oc[c][i];
            }
        }
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            if (lane == 0) {
                mML[(w * RT + r) * 2] = m[r];
                mML[(w * RT + r) * 2 + 1] = l[r];
            }
        }
        __syncthreads();
    } else {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        if (ks == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) mA[(w * RT + r) * D + dg * 8 + e] = acc[r][e];
        }
        if (lane == 0) {
            mML[(w * RT + r) * 2] = m[r];
            mML[(w * RT + r) * 2 + 1] = l[r];
        }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 1; kk < KPS; ++kk) {
        if (ks == kk) {
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) mA[(w * RT + r) * D + dg * 8 + e] += acc[r][e];
        }
        __syncthreads();
    }
    }
    // Thread t finalises (head slot, row, dim) triples, merging the waves of
    // the head slot; a wave with no keys has m = -inf and weight 0.
    const bool single = p.direct != 0;
    const int64_t pbase = (int64_t)(p.split_off + (int)blockIdx.x) * p.n_rows_total;
    const int hpw = 1 << p.hpw_log2;
    for (int i = threadIdx.x; i < hpw * RT * D; i += 64 * NW) {
        const int h = i / (RT * D);
        const int r = (i - h * RT * D) / D, d = i - (h * RT + r) * D;
        const int w0 = h * wph;
        const int rr = sRow[w0][r];  // the head's waves share their rows
        if (rr < 0) continue;
        float M = -INFINITY;
        for (int ww = w0; ww < w0 + wph; ++ww) M = fmaxf(M, mML[(ww * RT + r) * 2]);
        float L = 0.f, A = 0.f;
        for (int ww = w0; ww < w0 + wph; ++ww) {
            const float mw = mML[(ww * RT + r) * 2];
            const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
            L = fmaf(mML[(ww * RT + r) * 2 + 1], f, L);
            A = fmaf(mA[(ww * RT + r) * D + d], f, A);
        }
        if (single) {
            o_out[(int64_t)rr * D + d] = L > 0.f ? A / L : 0.f;  // a row that saw no key: o = 0, lse = -inf
            if (d == 0) lse_out[rr] = (M + log2f(L)) * 0.69314718055994531f;
        } else {
            part_acc[(pbase + rr) * D + d] = A;
            if (d == 0) part_ml[(int64_t)rr * p.n_splits_all + p.split_off + blockIdx.x] = make_float2(M, L);
        }
    }
}

}  // namespace rkv
