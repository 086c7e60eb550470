/*
 * rkv.h -- C ABI of the position-split decode-attention library (librkv.so).
 *
 * The method ("F5 M7 -- Rolling KV: position-windowed KV residency", header
 * note): one layer's KV cache is divided by KEY POSITION into a
 * device-resident window [0, wc) and a tail [wc, n_kv).  Each part is
 * attended on its own with flash attention that also emits the per-head
 * log-sum-exp, and an online-softmax combine merges the parts into exactly
 * the attention of the unsplit cache ("Implementation decomposition,
 * refined", S2: lse_t = m_t + log d_t; O = sum_t O_t e^{lse_t - M} /
 * sum_t e^{lse_t - M}, M = max_t lse_t, in F32).  Quantised K/V blocks are
 * read in registers inside the attention loop (section "2026-07-12 -- #582-P2
 * SHIPPED: position-axis mixed KV": window and tail each read in-register at
 * its own type, no whole-cache f16 materialise).  A tail held in
 * pinned host memory is streamed through a B-slot device ring on a copy
 * stream; a slot's refill waits for the compute that read it, a tile's
 * compute waits for its slot's copy ("Architecture",
 * "CUDA stream graph"; and the page "Rolling-KV: step/graph-level tail
 * prefetch (design)", section "The fix: a persistent, step-spanning
 * tail-prefetch ring").
 *
 * Conventions for every entry point:
 *  - The return value is a status code (RKV_OK = 0, negative on error).  No
 *    call aborts the process.  Arguments are validated on the host before
 *    anything is enqueued; on an error nothing is enqueued and
 *    rkv_last_error() gives a thread-local message.  A fault inside a kernel
 *    is asynchronous and surfaces at the caller's next synchronisation.
 *  - Device buffers are owned by the caller.  The compute entry points
 *    allocate nothing and create no events or streams, so they may be
 *    enqueued on any stream, including under stream capture.
 *  - Work is enqueued on the stream argument (NULL = the legacy default
 *    stream); calls return without waiting for it.
 *  - Floating-point outputs are IEEE binary32.  LSE values are natural-log.
 */
#ifndef RKV_H
#define RKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

/* ---- status ------------------------------------------------------------ */
enum {
    RKV_OK = 0,
    RKV_E_INVAL = -1,       /* bad argument: null pointer, bad size, stride, host pointer where device memory is needed */
    RKV_E_UNSUPPORTED = -2, /* valid but not implemented: (type, head_dim) pair, too many heads / parts */
    RKV_E_HIP = -3,         /* a HIP runtime call failed (message has the HIP error string) */
    RKV_E_NOMEM = -4,       /* device or host allocation failed (ring creation only) */
    RKV_E_STATE = -5        /* ring call out of order: layer not next in the plan, step not begun / not finished */
};

/* Static name of a status code. */
const char *rkv_status_string(int status);
/* Message of the last failing call on this thread ("" if none). */
const char *rkv_last_error(void);

/* ---- cache storage types ------------------------------------------------
 * Blocks follow "F5 M6 -- PolyKV", section "S0 -- Bootstrap" and the
 * tier-family table (1.062 and 0.562 bytes per value): 32 consecutive values
 * along head_dim share one binary16 scale d.
 *   RKV_Q8_0: 34 bytes = d, then 32 signed bytes q_i;           x_i = d * q_i
 *   RKV_Q4_0: 18 bytes = d, then 16 bytes of 4-bit codes n_i;   x_i = d * (n_i - 8)
 *             element i < 16 is the low nibble of byte i, element i >= 16
 *             the high nibble of byte i - 16.
 * Block types need head_dim % 32 == 0; a row of head_dim values is
 * head_dim/32 blocks back to back.
 *   RKV_TBQ3 (values only): the 3-bit tier of "F5 M6 -- PolyKV", section
 *             "S2 -- TurboQuant tier family (TBQ8_0 / TBQ4_0 / TBQ3_0)": a
 *             128-value block is rotated by a seeded fast Walsh-Hadamard
 *             transform and each rotated value stored as the nearest level
 *             of the 8-level Lloyd-Max codebook of N(0,1), with the block's
 *             binary16 norm, 2-bit indices and one sign bit per value (the
 *             fields that page lists).  52 bytes per block:
 *               bytes 0-1  n, the block's L2 norm (binary16); bytes 2-3 zero;
 *               bytes 4-35 magnitude index m_i of value i at bits 2(i%4) of
 *                          byte 4 + i/4;
 *               bytes 36-51 sign bit of value i at bit i%8 of byte 36 + i/8.
 *             Rotated value y_i = (-1)^sign c_{m_i} n / sqrt(128), with
 *             c_0..c_3 the positive levels of the codebook (about 0.2451,
 *             0.7560, 1.3439, 2.1519); the value is x = R^T y with
 *             R = S2 H S1 / sqrt(128), H the 128 x 128 Sylvester Hadamard
 *             matrix, S1 / S2 diagonal signs from bits 0..127 of the first
 *             two / next two outputs of splitmix64 seeded with 42 (bit set:
 *             -1).  The pages print neither the levels, the signs nor the
 *             byte order; these are this library's.  head_dim % 128 == 0.
 *             Attention over TBQ3 values sums P.y in the rotated space and
 *             applies R^T once to the output ("S2 perf-path Level B": the O
 *             inverse rotation, exact by Parseval).  Limits: V only; a call
 *             whose segments hold keys must have TBQ3 values in all of them
 *             or in none (RKV_E_UNSUPPORTED), since partials of the two
 *             spaces are not merged; not accepted as a streamed tail or as
 *             an append destination (RKV_E_UNSUPPORTED). */
typedef enum rkv_dtype { RKV_F32 = 0, RKV_F16 = 1, RKV_Q8_0 = 2, RKV_Q4_0 = 3, RKV_TBQ3 = 4 } rkv_dtype;

/* Bytes of one row of head_dim values of a type (0 if invalid). */
int64_t rkv_row_bytes(int32_t dtype, int32_t head_dim);

/* ---- a segment of the KV cache -------------------------------------------
 * One view is one segment: a window, a tail, a tile of the tail, a shared
 * prefix or a private suffix.  Its positions [0, n_keys) are relative to the
 * view.  Row (position p, KV head g, sequence b) of K starts at byte
 *     k + b * k_seq_stride + p * k_pos_stride + g * k_head_stride
 * (likewise V).  k_seq_stride = 0 means one segment shared by every sequence
 * (its keys are read once for all of them).  n_keys = 0 is a legal, empty
 * segment.  Pointers, strides and row sizes must be multiples of the row's
 * load width (16 bytes for f32/f16 rows, 8 for block rows whose size is a
 * multiple of 8, else 4).  The result does not depend on the order of
 * positions inside a view (softmax attention is invariant to a joint
 * permutation of the (k, v) pairs). */
typedef struct rkv_kv_view {
    const void *k;
    const void *v;
    int32_t k_type;
    int32_t v_type;
    int64_t n_keys;
    int64_t k_pos_stride, v_pos_stride;
    int64_t k_head_stride, v_head_stride;
    int64_t k_seq_stride, v_seq_stride;
    /* Absolute position of the view's first key: key j of the view sits at
     * position pos0 + j.  Read only by a call whose descriptor carries query
     * positions (q_pos); a window view of positions [0, wc) has pos0 = 0,
     * its tail pos0 = wc. */
    int64_t pos0;
} rkv_kv_view;

/* ---- the attention problem ------------------------------------------------
 * Decode: one query token per sequence.  Query head h of a sequence attends
 * KV head q_to_kv[h] (NULL: contiguous groups h / (n_q_heads / n_kv_heads),
 * which needs n_q_heads % n_kv_heads == 0).  Scores are
 *     s_j = scale * (q . k_j),  then  s_j = softcap * tanh(s_j / softcap)  if softcap > 0,
 * and the softmax and LSE are taken over the final s_j.  Limits:
 * head_dim in {64, 128, 256, 512}; n_q_heads <= 256; n_kv_heads <= 64;
 * n_seq * n_q_heads <= 65535.
 *
 * Several query rows of one sequence -- a prefill chunk or the draft tokens
 * of a verify step ("F5 M7 -- Rolling KV", section "2026-07-12 -- #582-P2
 * SHIPPED", bug-2161: the n_q > 1 path over window and tail; section
 * "2026-07-14 -- bug-2172 SHIPPED": the mask is indexed by absolute key
 * position, -inf for hidden keys) -- are passed as n_seq "sequences" over views with
 * sequence stride 0, each with its position in q_pos: the row at position p
 * sees the keys at absolute positions <= p (a key's absolute position is the
 * view's pos0 plus its index).  A row that sees no key of a call gets o = 0
 * and lse = -inf, the empty-segment result, so that the segment merge gives it
 * weight 0.  With q_pos, n_seq <= 64. */
typedef struct rkv_attn_desc {
    int32_t n_seq;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    float scale;
    float softcap;          /* 0 = off */
    const int32_t *q_to_kv; /* host array of n_q_heads, or NULL */
    const int64_t *q_pos;   /* host array of n_seq (absolute query positions), or NULL: no mask */
} rkv_attn_desc;

/* Workspace bytes rkv_attend_segment needs for this problem and segment
 * (written to *bytes; 0 when no workspace is needed).  The workspace holds
 * per-split partial results; its contents need no initialisation.  Calls
 * that overlap in time must not share a workspace. */
int rkv_attend_workspace_bytes(const rkv_attn_desc *desc, const rkv_kv_view *seg, size_t *bytes);

/*
 * rkv_attend_segment -- normalised attention output and LSE of one segment.
 *
 *   q    [n_seq][n_q_heads][head_dim] binary32, device.
 *   seg  the segment (device memory).
 *   o    [n_seq][n_q_heads][head_dim] binary32, device (written).
 *   lse  [n_seq][n_q_heads] binary32 natural-log LSE, device (written).
 *   ws   device workspace of at least rkv_attend_workspace_bytes bytes.
 *
 * An empty segment gives o = 0 and lse = -inf (combine weight 0).  The result
 * is deterministic: the same inputs give the same bits on every run.
 * Errors: RKV_E_INVAL (null / host pointers, misaligned strides, small
 * workspace, bad head map), RKV_E_UNSUPPORTED (type / head_dim / head
 * counts outside the limits).
 */
int rkv_attend_segment(const rkv_attn_desc *desc, const float *q, const rkv_kv_view *seg,
                       float *o, float *lse, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * rkv_attend_split -- attention over the union of n_segments segments in one
 * launch: each segment is attended by its own key splits and all partials
 * are merged by the LSE combine of the segment results ("F5 M7 -- Rolling
 * KV", header note: window [0, wc) and tail [wc, n_kv) attended separately
 * and merged; the result equals softmax attention over all their keys).
 * This is the window + tail (+ tail tiles) step of one layer as a single
 * call; rkv_attend_segment is the case n_segments == 1.
 *
 *   segs  1..4 views.  Segments of one K type, one V type and one sequence
 *         sharing (all shared by every sequence, or all per sequence) go to
 *         one launch of the attention kernel; segments that differ in these
 *         -- a window and a tail stored at different types ("F5 M7 -- Rolling
 *         KV", "2026-07-12 -- #582-P2 SHIPPED": each segment read at its own
 *         type), a shared prefix and private suffixes -- get one launch per
 *         group, all writing one set of partials, merged once.  Empty segments
 *         are allowed; if every segment is empty o = 0 and lse = -inf.
 *   q, o, lse, ws, stream: as for rkv_attend_segment.
 *
 * The merge order is fixed, so results are deterministic; they agree with
 * rkv_attend_segment per segment + rkv_lse_combine to rounding, not bit for
 * bit.
 */
int rkv_attend_split_workspace_bytes(const rkv_attn_desc *desc, int n_segments, const rkv_kv_view *segs,
                                     size_t *bytes);
int rkv_attend_split(const rkv_attn_desc *desc, const float *q, int n_segments, const rkv_kv_view *segs, float *o,
                     float *lse, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * rkv_attend_split_noalloc -- rkv_attend_split for callers that cannot
 * allocate device memory: code under stream or graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The same launches and arithmetic
 * (the same bits as rkv_attend_split), with the per-split partials in a fixed
 * array of the library's own instead of a caller's workspace: each GPU the
 * library runs on holds one array of RKV_NOALLOC_MAX_BYTES, from module load
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * library allocation) and creates nothing; the caller passes q, o, lse and
 * the segments as for rkv_attend_split.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it has to start at zero: every partial is written
 * before it is read): calls that overlap in time on one GPU (on different
 * streams, or from different threads without ordering) race and give wrong
 * results.  A call whose partials need more than RKV_NOALLOC_MAX_BYTES (see
 * rkv_attend_split_workspace_bytes) returns RKV_E_UNSUPPORTED and enqueues
 * nothing.  Other errors as for rkv_attend_split.
 */
#define RKV_NOALLOC_MAX_BYTES ((size_t)32 << 20)
int rkv_attend_split_noalloc(const rkv_attn_desc *desc, const float *q, int n_segments, const rkv_kv_view *segs,
                             float *o, float *lse, hipStream_t stream);

/*
 * The two phases of rkv_attend_split as separate calls, for callers that
 * time them or put other work between them:
 *   rkv_attend_split_partials  the attention kernel: every key split writes
 *       its partial (running max, denominator, weighted sum) into ws, in a
 *       layout of the library's own; when the launch has a single split, or
 *       no keys at all, the final o / lse are written here instead.
 *   rkv_attend_split_merge  the fixed-order merge of those partials into o /
 *       lse (nothing to do in the single-split and no-key cases).
 * Called in this order on one stream with the same desc, segments (the same
 * sizes and types) and workspace, they enqueue exactly what rkv_attend_split
 * enqueues and give the same bits.  ws must not be reused in between.
 * Arguments and errors as for rkv_attend_split (the merge takes no query).
 */
int rkv_attend_split_partials(const rkv_attn_desc *desc, const float *q, int n_segments, const rkv_kv_view *segs,
                              float *o, float *lse, void *ws, size_t ws_bytes, hipStream_t stream);
int rkv_attend_split_merge(const rkv_attn_desc *desc, int n_segments, const rkv_kv_view *segs, float *o, float *lse,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * rkv_lse_combine -- merge per-segment results ("F5 M7 -- Rolling KV",
 * "Implementation decomposition, refined", S2):
 *     M = max_t lse_t;  w_t = e^{lse_t - M};
 *     o = sum_t w_t o_t / sum_t w_t;  lse = M + ln sum_t w_t.
 *
 *   o_parts[t]   [n_rows][head_dim] binary32, device;  lse_parts[t] [n_rows], device.
 *   o_parts and lse_parts are HOST arrays of n_parts device pointers.
 *
 * A part with lse = -inf has weight 0.  When every part of a row is empty the
 * row gets o = 0, lse = -inf (and the call succeeds).  A row with a single
 * non-empty part gets that part's values bit for bit.  o_out may alias
 * o_parts[0] and lse_out may alias lse_parts[0].  1 <= n_parts <= 64.
 */
int rkv_lse_combine(int n_parts, const float *const *o_parts, const float *const *lse_parts,
                    int64_t n_rows, int32_t head_dim, float *o_out, float *lse_out, hipStream_t stream);

/*
 * rkv_dequant_q8_0 / rkv_dequant_q4_0 -- blocks (device) to n_values binary32
 * values (device), bit-exact: the products d*q and d*(n-8) are exact in
 * binary32.  n_values % 32 != 0 -> RKV_E_INVAL.  Not used by the attention
 * path (which reads blocks in registers); provided for checking and tools.
 */
int rkv_dequant_q8_0(const void *blocks, int64_t n_values, float *out, hipStream_t stream);
int rkv_dequant_q4_0(const void *blocks, int64_t n_values, float *out, hipStream_t stream);
/*
 * rkv_dequant_tbq3 -- TBQ3 blocks (device) to n_values binary32 values of the
 * original space x = R^T y (device); n_values % 128 != 0 -> RKV_E_INVAL.
 * Computed in binary32 (the levels, the norm product and the transform
 * round), so the values agree with their binary64 definition to a few units
 * in the last place of the block's largest value, not bit for bit.
 */
int rkv_dequant_tbq3(const void *blocks, int64_t n_values, float *out, hipStream_t stream);

/* ---- streamed tail --------------------------------------------------------
 * A ring of n_slots device staging slots, each holding one tile of K and one
 * of V, filled from pinned host memory by asynchronous copies on a copy
 * stream.  The copy into a slot waits until the attention of the slot's
 * previous tile has read it; the attention of a tile waits for its slot's
 * copy_done event ("F5 M7 -- Rolling KV", "CUDA stream graph").  The first of
 * these waits is taken on the host: the kernel after a tile's attention
 * kernel on the stream (the layer's next tile, or its merge) writes the
 * tile's sequence number to a per-slot word in pinned host memory when it
 * starts, and a copier thread owned by the ring watches that word and then
 * enqueues the slot's
 * copies (DMA-engine hipMemcpyAsync) and copy_done record.  So the copy
 * stream carries no wait on a compute-queue event (such a wait costs a
 * DMA-engine copy tens of microseconds even when the event has long
 * completed) and the compute stream records no event per tile.  The order of copies is one flat sequence over
 * (layer, tile) for a whole decode step, kept n_slots ahead of compute
 * across layer boundaries ("Rolling-KV: step/graph-level tail prefetch
 * (design)", "The fix: a persistent, step-spanning tail-prefetch ring"), so a
 * layer's tail can load while earlier layers compute.
 */
typedef struct rkv_ring rkv_ring;

/* Create a ring.  n_slots >= 2 (<= 16).  slot_k_bytes / slot_v_bytes: bytes
 * of one tile of K / V (tile_keys * pos_stride of the tail views).
 * copy_stream: NULL makes the ring create and own a non-blocking stream.
 * The ring owns its slots, its copy_done events (created here, timing
 * disabled), its progress words (128 bytes of pinned host memory), a stream
 * it created and its copier thread (started here, on the current device).
 * Errors: RKV_E_INVAL, RKV_E_NOMEM, RKV_E_HIP. */
int rkv_ring_create(int n_slots, size_t slot_k_bytes, size_t slot_v_bytes, hipStream_t copy_stream,
                    rkv_ring **out);
/* Stop the copier (copies it has not enqueued yet are dropped), wait for the
 * ring's enqueued copies and for the attention of every tile already handed
 * to rkv_stream_tail to finish reading its slot, then free it.  A GPU that
 * does not finish within 60 s gives RKV_E_HIP (the ring is freed anyway).
 * NULL is a no-op. */
int rkv_ring_destroy(rkv_ring *ring);

/* Plan one step: the tails of n_layers layers (host_tails[l], one sequence
 * or shared by all sequences), cut into tiles of tile_keys keys (the last tile
 * of a layer may be partial; an empty tail has no tiles; at most 63 tiles per
 * layer).  A tail in pinned host memory is streamed through the slots; a tail
 * in device memory is attended where it is, tile by tile, with the same
 * launches and the same merge and no copies (the step's results are then the
 * same bits as with that tail streamed).  Hands the first n_slots copies to
 * the copier (each waits for the previous step's last use of its slot).  The
 * tail buffers must stay alive and unchanged until the step's attention has
 * completed.  Errors: RKV_E_INVAL (pageable host memory, a streamed tile
 * larger than a slot, misaligned), RKV_E_UNSUPPORTED (more than 63 tiles in a
 * layer), RKV_E_STATE (previous step not ended). */
int rkv_ring_begin_step(rkv_ring *ring, int n_layers, const rkv_kv_view *host_tails, int64_t tile_keys);

/* Workspace bytes rkv_stream_tail needs for a layer of the current plan. */
int rkv_stream_tail_workspace_bytes(const rkv_ring *ring, int layer, const rkv_attn_desc *desc, size_t *bytes);

/*
 * rkv_stream_tail -- attention over layer `layer`'s tail, tile by tile from
 * the ring, merged with the window's result.
 *
 * For each tile: the call waits on the host until the copier has enqueued
 * the tile's copy (at most until the GPU has finished the compute n_slots
 * items earlier); the compute stream waits copy_done of its slot and attends
 * the slot, and the kernel after the split kernel signals the slot free;
 * then the refill of that slot with the item n_slots further on in the flat
 * order is handed to the copier.  Tiles may run on different compute
 * streams.  A slot whose previous reader has not finished within 60 s of the
 * copier starting to wait fails the ring's copier (RKV_E_HIP at the next
 * call).
 * Each tile's key splits write their partials into one set for the layer,
 * and one fixed-order merge (the S2 combine applied to the window's result
 * and every split's partial, in the order window, tile 0's splits, tile 1's
 * splits, ...) gives o and lse; lse_window may be NULL (no window; o_window is
 * then ignored).  A slot is released when the kernel after the tile's
 * attention kernel (the next tile's, or the merge) starts.  The result does not depend on n_slots, and equals, bit
 * for bit, the same call with the layer's tail in device memory (attended in
 * place); it agrees with rkv_attend_segment per tile + rkv_lse_combine to
 * rounding.  Layers must be consumed in plan order.
 * Errors: RKV_E_STATE (layer out of order / no step), RKV_E_INVAL, RKV_E_HIP
 * (also a failure of the copier).  A failure once the tiles have started
 * aborts the step: later calls return RKV_E_STATE until the next begin_step.
 */
int rkv_stream_tail(rkv_ring *ring, int layer, const rkv_attn_desc *desc, const float *q,
                    const float *o_window, const float *lse_window, float *o, float *lse,
                    void *ws, size_t ws_bytes, hipStream_t compute_stream);

/* End the step: every planned layer must have been consumed (else
 * RKV_E_STATE).  Does not wait for the GPU. */
int rkv_ring_end_step(rkv_ring *ring);

/* Pure host logic of the schedule, for checking: with n_slots slots and
 * tiles_per_layer[l] tiles per layer, item j of the flat order goes to slot
 * j % n_slots and its copy waits for the compute of item j - n_slots.
 * Writes, for each item j < n_items: layer_of[j], tile_of[j], slot_of[j],
 * waits_on[j] (item index or -1).  Returns the number of items, or a
 * negative status.  Any output pointer may be NULL. */
int64_t rkv_ring_schedule(int n_layers, const int64_t *tiles_per_layer, int n_slots, int64_t max_items,
                          int32_t *layer_of, int64_t *tile_of, int32_t *slot_of, int64_t *waits_on);

/* ---- write path ------------------------------------------------------------
 * rkv_append_kv -- store the K and V rows of n_tokens new tokens of one layer
 * and one sequence at the consecutive positions pos0, pos0 + 1, ..., each in
 * the storage type of the region it lands in.
 *
 * Routing ("Rolling-KV: step/graph-level tail prefetch (design)", section
 * "Staged plan", S0 / bug-1341: a layer's writes follow that layer's own
 * window size, so a layer without a tail writes everything to its window;
 * "F5 M7 -- Rolling KV", section "2026-07-14 -- bug-2172 SHIPPED": each new
 * row goes to the window or the tail by its position): position p goes to
 * window row p when p < window->n_keys, else to tail row p - window->n_keys.
 * Here n_keys of window and tail is read as the region's capacity in
 * positions; NULL is a region of capacity 0.  pos0 + n_tokens must not exceed
 * the two capacities together (RKV_E_INVAL, nothing written).
 *
 * Storage (block formats of "F5 M6 -- PolyKV", section "S0 -- Bootstrap"; the
 * pages print no rule for making codes, the one used is the common rule for
 * these formats, in binary32 arithmetic without fused multiply-add):
 *   RKV_F32  the value; RKV_F16 the nearest binary16 (ties to even);
 *   RKV_Q8_0 d = amax / 127, q = round-half-away-from-zero(x * (1/d));
 *   RKV_Q4_0 m = the first value of largest magnitude in the block (+0 if
 *            all are zero), d = m / -8, n = min(15, trunc(x * (1/d) + 8.5));
 *   1/d is 0 when d = 0; the block scale is stored as the binary16 nearest
 *   the binary32 d (ties to even) and the codes are made from the binary32 d.
 * Values must be finite.
 *
 * k_new, v_new: device binary32 [n_tokens][n_kv_heads][head_dim], contiguous,
 *   4-byte aligned.  head_dim 64, 128, 256 or 512.
 * window: device memory.  tail: device memory or pinned host memory (then
 *   the kernel makes its stores visible system-wide before it ends).  Both are
 *   position-major with the byte strides of the view; seq selects the
 *   sequence (seq * seq_stride); pointers and strides must be even, the rows
 *   of one position must fit in its position stride.  Window and tail may
 *   have different types.
 * fresh (optional, device memory): receives the tail-routed rows as well, row
 *   j = the j-th of them (n_keys >= their count), in fresh's own types, so the
 *   step that writes them can attend them from device memory (the ring's
 *   copies of a step may have started before the step's own appends).
 * ring (optional) with layer in [0, 1024): when tail rows are written, a
 *   one-thread kernel after the append marks the layer written (a host-visible
 *   word of the ring); copies of that layer's tail in steps begun with
 *   rkv_ring_begin_step after this call wait on the host until the append has
 *   finished.  Appends to one layer that name a ring must be ordered (one
 *   stream, or the caller's own ordering), and must be issued from the thread
 *   that calls rkv_ring_begin_step, or ordered with it.
 * Enqueued on stream; allocates nothing.  Errors: RKV_E_INVAL,
 * RKV_E_UNSUPPORTED, RKV_E_HIP.
 */
int rkv_append_kv(int n_kv_heads, int head_dim, int n_tokens, int64_t pos0, int seq, const float *k_new,
                  const float *v_new, const rkv_kv_view *window, const rkv_kv_view *tail, const rkv_kv_view *fresh,
                  rkv_ring *ring, int layer, hipStream_t stream);

/* ---- residency planner (host only) ----------------------------------------
 * rkv_plan_residency -- choose, for a decode step over n_layers layers of
 * n_kv positions, the window (positions per layer kept in device memory),
 * the tail tile and the ring's slot count, and estimate what streaming the
 * tail costs.  Pure host arithmetic in binary64 on measured inputs; no GPU
 * call.  The steps:
 *  - bw_eff = min(link_bw, host_ram_bw), host_ram_bw <= 0 meaning unknown
 *    ("T*-aware auto rolling-KV spill", T* section: the host-to-device rate
 *    is bound by the slower of the link and the host memory read).
 *  - The whole cache within kv_budget_bytes: RKV_RESIDENT, window = n_kv
 *    ("F5 M7 -- Rolling KV", runtime tactic table: a layer that fits stays
 *    hot).
 *  - Otherwise tile_keys = floor(compute_s_per_layer * bw_eff * safety /
 *    bytes_per_key) (>= 1, "F5 M7 -- Rolling KV", section "Slot pool"); the
 *    window is what the budget holds after two slots; a tail of more than 63
 *    tiles per layer grows the tile (one combine merges the window and at most
 *    63 tiles) and the window is sized again; n_slots = clamp(budget left /
 *    slot bytes, 2, 4).
 *  - t_resident = (weights_bytes + whole KV) / vram_bw; drop = (c_engage_s +
 *    tail bytes / bw_eff) / t_resident; T* = (target_drop * t_resident -
 *    c_engage_s) * bw_eff ("T*-aware auto rolling-KV spill", T* section).  A
 *    tail of at most T* bytes (all layers): RKV_STREAM; more: RKV_QUANTIZE (the
 *    spill costs more than the target drop; a smaller cache type should be
 *    chosen).
 *  - predicted_step_s = max(step compute, tail DMA) + c_engage_s, free zone =
 *    step compute * bw_eff, predicted_hidden = min(compute, DMA) / DMA
 *    ("Rolling-KV: step/graph-level tail prefetch (design)", section "Bounded
 *    win (be honest)").
 * Units: bytes, bytes per second, seconds.  Errors: RKV_E_INVAL (NULL,
 * non-positive or non-finite rates, a budget below two slots of one
 * position); the message is rkv_plan_last_error().
 */
enum { RKV_RESIDENT = 0, RKV_STREAM = 1, RKV_QUANTIZE = 2 };
enum { RKV_LINK_BOUND = 0, RKV_HOST_RAM_BOUND = 1 };

typedef struct rkv_residency_in {
    int32_t n_layers;
    int64_t n_kv;               /* positions per layer */
    int64_t bytes_per_key;      /* K + V bytes of one position of one layer, all KV heads, stored types */
    int64_t kv_budget_bytes;    /* device memory for the windows and the ring slots */
    int64_t weights_bytes;      /* other bytes a step reads from device memory (active weights) */
    double vram_bw;             /* device memory read rate, bytes/s */
    double link_bw;             /* pinned host-to-device copy rate, bytes/s (measured) */
    double host_ram_bw;         /* host memory read rate, bytes/s; <= 0 unknown */
    double c_engage_s;          /* fixed cost per step of engaging the split path, s (measured) */
    double compute_s_per_layer; /* one layer's step time with its window resident, s (measured) */
    double target_drop;         /* tolerated throughput drop of a spill, e.g. 0.20 */
    double safety;              /* tile sizing safety factor in (0, 1], e.g. 0.8 */
} rkv_residency_in;

typedef struct rkv_residency_plan {
    int32_t tactic;       /* RKV_RESIDENT, RKV_STREAM or RKV_QUANTIZE */
    int32_t binding;      /* RKV_LINK_BOUND or RKV_HOST_RAM_BOUND */
    int64_t window_keys;  /* positions per layer in device memory */
    int64_t tail_keys;    /* positions per layer in the tail */
    int64_t tile_keys;    /* positions per ring tile (0 without a tail) */
    int32_t n_slots;      /* ring slots (0 without a tail) */
    double bw_eff;        /* binding host-to-device rate, bytes/s */
    double t_resident_s;  /* step time with the whole cache resident (model) */
    double t_star_bytes;  /* tolerable tail bytes at target_drop (<= 0: never spill) */
    double drop;          /* modelled throughput drop of this plan's tail */
    double free_zone_bytes;
    double predicted_step_s;
    double predicted_hidden; /* fraction of the tail DMA hidden under compute */
} rkv_residency_plan;

int rkv_plan_residency(const rkv_residency_in *in, rkv_residency_plan *out);
/* Message of the last failing rkv_plan_residency call on this thread. */
const char *rkv_plan_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RKV_H */
