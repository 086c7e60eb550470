// common.h -- internal declarations shared by the HIP translation units of
// librkv.so (kernels, launchers and the C-ABI layer).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rkv.h"

namespace rkv {

constexpr int kF32 = RKV_F32, kF16 = RKV_F16, kQ8 = RKV_Q8_0, kQ4 = RKV_Q4_0, kT3 = RKV_TBQ3;

__host__ __device__ constexpr int row_bytes_of(int t, int d)
{
    return t == kF32 ? 4 * d : t == kF16 ? 2 * d : t == kQ8 ? (d / 32) * 34 : t == kQ4 ? (d / 32) * 18
         : t == kT3 ? (d % 128 ? 0 : (d / 128) * 52) : 0;
}

// The TBQ3 tier's constants, computed once on the host (api.hip): the
// positive Lloyd-Max levels of N(0,1) and the rotation's sign masks (bit i
// of s1 / s2 set: the sign of value i is -1).
struct Tbq3Consts {
    float lv[4];
    uint32_t s1[4], s2[4];
};
const Tbq3Consts &tbq3_consts();

// Width in bytes of the vector loads that stage a row: the largest of 16, 8, 4
// dividing the row size.
__host__ __device__ constexpr int load_width_of(int t, int d)
{
    return row_bytes_of(t, d) % 16 == 0 ? 16 : row_bytes_of(t, d) % 8 == 0 ? 8 : 4;
}

constexpr int kTile = 64;           // keys per wave tile (one key per lane in the score phase)
constexpr int kMaxRowTable = 1024;  // entries of the per-KV-head row table
constexpr int kMaxKvHeads = 64;
constexpr int kMaxParts = 64;

constexpr int kMaxSegs = 4;         // segments one launch can attend
constexpr int kMaxMaskSeqs = 64;    // sequences (query rows) of a call with query positions
constexpr int kRingMaxLayers = 1024;  // layers a tail ring can plan

// One segment of a launch: its K/V base pointers and byte strides, its keys,
// and the range of workgroups (key splits) that cover it.
struct SegParams {
    const uint8_t *k, *v;
    int64_t k_pos, v_pos, k_head, v_head, k_seq, v_seq;
    int64_t n_keys;
    int64_t pos0;        // absolute position of the segment's first key (masked launches)
    int32_t keys_per_split;
    int32_t split_base;  // first grid x index of this segment
};

// Launch parameters of the split attention kernel.
struct SplitParams {
    SegParams seg[kMaxSegs];
    int32_t n_segs;
    int32_t n_splits;      // total key splits over all segments (grid x)
    int32_t split_off;     // index of this launch's first split among all partials of the call
    int32_t n_splits_all;  // partials of the call (all its launches)
    int32_t direct;        // 1: the launch is the call's only split and writes o / lse directly
    int32_t n_rg;          // row groups per KV head
    int32_t rows_per_g;    // stride of rowtab between KV heads
    int32_t n_rows_total;  // n_seq * n_q_heads
    int32_t z_row_step;    // row offset per blockIdx.z (n_q_heads when sequences have their own keys, else 0)
    float scale;           // score scale
    float scale_log2;      // scale * log2(e)
    float softcap;         // natural units, 0 = off
    int32_t n_kv_heads;
    int32_t hpw_log2;      // log2 of the KV heads per workgroup
    int32_t wph_log2;      // log2 of the waves per KV head (waves per workgroup / heads per workgroup)
    int32_t n_q_heads;     // sequence of output row r: r / n_q_heads
    int32_t masked;        // qpos holds the absolute query position of each sequence
    int32_t stream_once;   // every K / V byte is read once by the launch (one row group per KV head)
    int32_t rg_waves;      // the waves of a head slot take its row groups (n_rg counts blocks of them), all tiles each
    // Optional slot release: workgroup (0, 0, 0) writes release_value to
    // *release (host-visible memory, system scope) when the kernel starts,
    // i.e. once the kernel before it on the stream has finished.
    uint64_t *release;
    uint64_t release_value;
    float tbq_lv[4];       // TBQ3 values: the codebook's positive levels
    int64_t qpos[kMaxMaskSeqs];
    uint16_t rowcnt[kMaxKvHeads];
    uint16_t rowtab[kMaxRowTable];
};

// The kernel reads the two 16-bit tables as aligned 32-bit words.
static_assert(offsetof(SplitParams, rowcnt) % 4 == 0 && offsetof(SplitParams, rowtab) % 4 == 0, "table alignment");
static_assert(kMaxKvHeads % 2 == 0 && kMaxRowTable % 2 == 0, "table sizes");

// How a launch is cut into work: shared by the workspace query and the launch.
struct SplitPlan {
    int rt;          // rows per wave (template instance)
    int nw;          // waves per workgroup of that instance
    int hpw;         // KV heads per workgroup
    int n_hg;        // head groups (grid y = n_hg * n_rg)
    int n_rg;        // row groups per KV head
    int rows_per_g;  // max rows of a KV head
    int z;           // grid z (sequences with own keys, or 1)
    int n_splits;    // grid x
    bool shd;        // the shared-decode kernel (n_rg then counts blocks of its row groups)
    bool rgs;        // the staged-tile f16 kernel (n_rg then counts blocks of its row groups)
    int64_t n_rows_total;
    size_t acc_bytes, ml_bytes;
    size_t ws_bytes;
};

// Kernel launchers (attend.hip / combine.hip / dequant.hip).  They enqueue on
// `stream` and return the hipError_t of the launch.
// One launch of the split kernel.  With one split in all (p.n_splits == 1) it
// writes o / lse directly; otherwise every workgroup writes its partial and
// launch_reduce merges them.
hipError_t launch_split(int kt, int vt, int d, int rt, dim3 grid, const float *q, float *part_acc,
                        float2 *part_ml, float *o, float *lse, const SplitParams &p, hipStream_t stream);
// done (optional): host-visible memory that receives done_value once the split
// kernel before the merge has finished (a progress signal for the tail ring).
// o_x / lse_x (optional): one more, already normalised part (an O and its
// LSE, natural log) merged before the splits, e.g. a window's result.
hipError_t launch_reduce(int d, int64_t n_rows, int n_splits, const float *part_acc, const float2 *part_ml,
                         float *o, float *lse, hipStream_t stream, uint64_t *done = nullptr, uint64_t done_value = 0,
                         const float *o_x = nullptr, const float *lse_x = nullptr);
// Write done_value to done (system scope) once the work before it on the stream has finished.
hipError_t launch_signal(uint64_t *done, uint64_t done_value, hipStream_t stream);
bool split_supported(int kt, int vt, int d, int rt);
// Dim slices per KV head the split kernel uses for a (K type, V type,
// head_dim): block-type K and V at head_dim 256 / 512 run as 2 / 4 slices of
// 128 dims, one wave each, all of a head's slices in one workgroup; else 1.
int split_dim_slices(int kt, int vt, int d);
// Waves per workgroup of the split kernel for a (K type, V type, head_dim).
int split_waves(int kt, int vt, int d, int rt);
// Workgroups of a split-kernel instance resident per compute unit on the
// current device, and the device's compute units (0 when no device answers).
int split_occupancy(int kt, int vt, int d, int rt);
int compute_units();
// The shared-decode split kernel (attend_shd.h): many rows per KV head over
// block-type K and q4_0 V at head_dim 128 (16 rows per wave, 4 row groups x
// 2 KV heads per workgroup, grid y = head pairs x row-group blocks).
bool split_shd_supported(int kt, int vt);
int split_shd_occupancy(int kt, int vt);
hipError_t launch_split_shd(int kt, int vt, dim3 grid, const float *q, float *part_acc, float2 *part_ml, float *o,
                            float *lse, const SplitParams &p, hipStream_t stream);
// The staged-tile split kernel (attend_rgs.h): many rows per KV head over f16
// K and V at head_dim 128 (16 rows per wave, 4 row groups of one KV head per
// workgroup, each tile staged once in LDS; grid y = KV heads x row-group blocks).
int split_rgs_occupancy();
hipError_t launch_split_rgs(dim3 grid, const float *q, float *part_acc, float2 *part_ml, float *o, float *lse,
                            const SplitParams &p, hipStream_t stream);
hipError_t launch_fill_empty(int d, int64_t n_rows, float *o, float *lse, hipStream_t stream);

struct CombineParts {
    const float *o[kMaxParts];
    const float *lse[kMaxParts];
};
hipError_t launch_combine(int n_parts, const CombineParts &parts, int64_t n_rows, int d, float *o_out,
                          float *lse_out, hipStream_t stream);

// One destination range of an append: tokens [first_tok, first_tok + n_tok)
// of the call go to rows row0, row0 + 1, ... of a region (k / v already
// offset to the call's sequence).
struct AppendDst {
    uint8_t *k, *v;
    int64_t k_pos, v_pos, k_head, v_head;
    int64_t row0;
    int32_t k_type, v_type;
    int32_t first_tok, n_tok;
};

struct AppendParams {
    AppendDst dst[3];  // window, tail, device copy of the tail rows (unused entries have n_tok = 0)
    int32_t n_dst;
    int32_t n_kv_heads;
    int32_t sys_fence;  // a destination is host memory: make the rows visible system-wide before the end
};

// One launch of the append kernel (append.hip): n_tokens x n_kv_heads
// workgroups; k_new / v_new binary32 [n_tokens][n_kv_heads][d].
hipError_t launch_append(int d, int n_tokens, int n_kv_heads, const float *k_new, const float *v_new,
                         const AppendParams &p, hipStream_t stream);

hipError_t launch_dequant_q8_0(const void *blocks, int64_t n_values, float *out, hipStream_t stream);
hipError_t launch_dequant_tbq3(const void *blocks, int64_t n_values, float *out, const Tbq3Consts &c,
                               hipStream_t stream);
// o [n_rows][d] (d % 128 == 0) in place: each 128-value block y -> R^T y, the
// TBQ3 tier's inverse rotation (the output of attention over TBQ3 values).
hipError_t launch_unrotate(float *o, int64_t n_rows, int d, const Tbq3Consts &c, hipStream_t stream);
hipError_t launch_dequant_q4_0(const void *blocks, int64_t n_values, float *out, hipStream_t stream);

}  // namespace rkv
