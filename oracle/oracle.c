/*
 * oracle.c -- plain, slow, obviously correct CPU reference for position-split
 * decode attention.  TEST INFRASTRUCTURE ONLY: nothing on the product path
 * links, loads or calls this file.  Only the test-suite, the smoke check and
 * the benchmark's CPU-baseline leg may use it.
 *
 * Everything is computed in IEEE binary64 from the stored bytes.  The file
 * shares no code, header, table or helper with the HIP library: the binary16
 * decoder, the block readers and the softmax are written out here from their
 * definitions.
 *
 * What it follows (pages are cited by title and section):
 *  - "F5 M7 -- Rolling KV: position-windowed KV residency", header note and
 *    section "Implementation decomposition, refined" (S2): attention over a
 *    key-position window [0,wc) and a tail [wc,n_kv), each segment giving a
 *    normalised output O_t and lse_t = m_t + log d_t, merged in F32 by
 *    O = sum_t O_t exp(lse_t - M) / sum_t exp(lse_t - M), M = max_t lse_t.
 *    The merge is stated to be exact online-softmax, so the plain definition
 *    of what the split path computes is softmax attention over the unsplit
 *    key set; orc_attend computes exactly that.  orc_lse_combine is the merge
 *    itself, written in binary64, and is used only by the invariant tests.
 *  - "F5 M6 -- PolyKV", section "S0 -- Bootstrap" and the tier-family table
 *    (q8_0 1.062 / q4_0 0.562 bytes per value): 32-value blocks with one
 *    binary16 scale; q8_0 holds 32 signed bytes (x = d*q), q4_0 holds 16
 *    bytes of 4-bit codes (x = d*(n-8)).  Nibble order (element i < 16 is the
 *    low nibble of byte i, element i >= 16 the high nibble of byte i-16) is a
 *    reading: the pages name the stock type but do not print its layout.
 *  - Logit softcap c*tanh(s/c) applied after the scale (reading: the pages
 *    list softcap among the score modifiers of the streaming path but do not
 *    order it; the softmax and the LSE are taken over the capped scores).
 *  - The write path (orc_route, orc_encode_row).  Routing: "Rolling-KV:
 *    step/graph-level tail prefetch (design)", section "Staged plan" (S0,
 *    bug-1341: a layer's writes follow that layer's own window size; a layer
 *    without a tail writes everything to its window) and "F5 M7 -- Rolling
 *    KV", section "2026-07-14 -- bug-2172 SHIPPED" (each new row goes to the
 *    window or to the tail by its destination position).  A row at position
 *    p goes to window row p when p < wc, else to tail row p - wc.
 *    Storing a binary32 row in the cache's type (quantise on append) is not
 *    spelled out by the pages, which only name the block types; the reading
 *    taken is the common rule for these formats, in binary32 arithmetic:
 *    q8_0 d = amax / 127, q = round-half-away-from-zero(x * (1 / d)); q4_0
 *    m = the first value of largest magnitude (+0 for a block of zeros),
 *    d = m / -8, n = min(15, trunc(x * (1 / d) + 8.5)); 1/d is taken as 0
 *    when d = 0; the scale is stored as the binary16 nearest to the binary32
 *    d (ties to even), the codes come from the binary32 d.  The codes are
 *    integers decided by binary32 arithmetic, so they are computed here in
 *    binary32, as the kernel computes them, and compared bit for bit.
 *  - TBQ3, the 3-bit value tier ("F5 M6 -- PolyKV", section "S2 --
 *    TurboQuant tier family (TBQ8_0 / TBQ4_0 / TBQ3_0)": a fast
 *    Walsh-Hadamard rotation spreads a block's energy over its values, then
 *    each value takes the nearest level of a Lloyd-Max (MSE-optimal)
 *    codebook; the same page lists the 3-bit type's fields as a binary16
 *    norm, 2-bit indices and one sign bit per value over a 128-value block,
 *    and names seed 42 for the rotation; section "S2 perf-path Level B": the
 *    rotation is a Q forward / O inverse pair, exact by Parseval).  The pages
 *    print neither the codebook, nor the signs, nor a byte order; the
 *    readings taken: the codebook is the 8-level Lloyd-Max quantiser of
 *    N(0,1) (symmetric: a 2-bit index m picks the magnitude c_m, the sign
 *    bit the sign), solved here from its two optimality conditions; the
 *    rotation of a 128-value block is R = S2 H S1 / sqrt(128), H the
 *    Sylvester Hadamard matrix (H[i][j] = (-1)^popcount(i & j)), S1 / S2
 *    diagonal signs from bits 0..127 of the first two / next two outputs of
 *    splitmix64 seeded with 42 (bit set = -1); a block stores
 *    n = ||x||_2 of its original values (binary16, nearest even), two zero
 *    bytes (alignment), the 2-bit magnitude index of value i at bits
 *    2(i%4) of byte 4 + i/4 and its sign bit at bit i%8 of byte 36 + i/8
 *    (52 bytes).  A stored block means y_i = +-c_m n / sqrt(128) in the
 *    rotated space, and x = R^T y = S1 H S2 y / sqrt(128) in the original one.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_Q8_0 = 2, ORC_Q4_0 = 3, ORC_TBQ3 = 4 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0 -> subnormal m * 2^-24; exponent 31 -> inf / nan. */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

static uint16_t rd_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Bytes of one row of D values of a given storage type (0 on a bad type). */
int64_t orc_row_bytes(int type, int64_t d)
{
    switch (type) {
    case ORC_F32: return 4 * d;
    case ORC_F16: return 2 * d;
    case ORC_Q8_0: return (d % 32) ? 0 : (d / 32) * 34;
    case ORC_Q4_0: return (d % 32) ? 0 : (d / 32) * 18;
    case ORC_TBQ3: return (d % 128) ? 0 : (d / 128) * 52;
    default: return 0;
    }
}

/* One q8_0 value: binary16 scale times a signed byte.  The product of an
 * 11-bit significand and an 8-bit integer is exact in binary32, so the
 * binary64 product rounded to float is the exact dequantised value. */
static double q8_0_value(const uint8_t *blk, int i)
{
    double d = orc_f16_to_f64(rd_u16(blk));
    int8_t q = (int8_t)blk[2 + i];
    return d * (double)q;
}

static double q4_0_value(const uint8_t *blk, int i)
{
    double d = orc_f16_to_f64(rd_u16(blk));
    uint8_t byte = blk[2 + (i & 15)];
    int n = (i < 16) ? (byte & 0x0f) : (byte >> 4);
    return d * (double)(n - 8);
}

/* ---- TBQ3 (readings in the header) ---- */

/* splitmix64: the state advances by 0x9e3779b97f4a7c15 and each output is
 * the state passed through two xor-shift-multiply steps and a final
 * xor-shift (Vigna's published generator). */
void orc_splitmix64(uint64_t seed, int n, uint64_t *out)
{
    uint64_t s = seed;
    int i;
    for (i = 0; i < n; ++i) {
        uint64_t z;
        s += 0x9e3779b97f4a7c15ull;
        z = s;
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        out[i] = z ^ (z >> 31);
    }
}

static double std_normal_pdf(double x) { return isinf(x) ? 0.0 : exp(-0.5 * x * x) / sqrt(2.0 * acos(-1.0)); }
static double std_normal_above(double x) { return isinf(x) ? 0.0 : 0.5 * erfc(x / sqrt(2.0)); } /* P(X > x) */

/* The positive half c[0] < c[1] < c[2] < c[3] of the 8-level Lloyd-Max
 * quantiser of N(0,1): Lloyd's iteration of its two conditions, thresholds
 * t_j = (c_{j-1} + c_j) / 2 (t_0 = 0, t_4 = inf) and levels
 * c_j = E[X | t_j < X < t_{j+1}] = (pdf(t_j) - pdf(t_{j+1})) / P(t_j < X < t_{j+1}),
 * from a uniform start until no level moves. */
static void tbq3_solve_levels(double c[4])
{
    int it, j;
    c[0] = 0.5; c[1] = 1.0; c[2] = 1.5; c[3] = 2.0;
    for (it = 0; it < 100000; ++it) {
        double t[5], nc[4], moved = 0.0;
        t[0] = 0.0;
        for (j = 1; j < 4; ++j) t[j] = 0.5 * (c[j - 1] + c[j]);
        t[4] = INFINITY;
        for (j = 0; j < 4; ++j) {
            const double mass = std_normal_above(t[j]) - std_normal_above(t[j + 1]);
            nc[j] = (std_normal_pdf(t[j]) - std_normal_pdf(t[j + 1])) / mass;
            if (fabs(nc[j] - c[j]) > moved) moved = fabs(nc[j] - c[j]);
        }
        for (j = 0; j < 4; ++j) c[j] = nc[j];
        if (moved == 0.0) break;
    }
}

static double tbq3_lv[4];
static int tbq3_s1[128], tbq3_s2[128];
static int tbq3_ready;

/* Fill the codebook and the rotation signs (called outside parallel regions). */
static void tbq3_init(void)
{
    uint64_t w[4];
    int i;
    if (tbq3_ready) return;
    tbq3_solve_levels(tbq3_lv);
    orc_splitmix64(42, 4, w);
    for (i = 0; i < 128; ++i) {
        tbq3_s1[i] = ((w[i >> 6] >> (i & 63)) & 1) ? -1 : 1;
        tbq3_s2[i] = ((w[2 + (i >> 6)] >> (i & 63)) & 1) ? -1 : 1;
    }
    tbq3_ready = 1;
}

void orc_tbq3_levels(double out[4])
{
    tbq3_init();
    memcpy(out, tbq3_lv, sizeof tbq3_lv);
}

void orc_tbq3_signs(int32_t out[256])
{
    int i;
    tbq3_init();
    for (i = 0; i < 128; ++i) {
        out[i] = tbq3_s1[i];
        out[128 + i] = tbq3_s2[i];
    }
}

/* Entry (i, j) of the 128 x 128 Sylvester Hadamard matrix. */
static int hadamard(int i, int j) { return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1; }

/* One TBQ3 block: its 128 values in the original space, x = S1 H S2 y / sqrt(128). */
static void tbq3_block_values(const uint8_t *blk, double *out)
{
    const double n = orc_f16_to_f64(rd_u16(blk));
    double y[128];
    int i, j;
    for (i = 0; i < 128; ++i) {
        const int m = (blk[4 + i / 4] >> (2 * (i % 4))) & 3;
        const int neg = (blk[36 + i / 8] >> (i % 8)) & 1;
        y[i] = (neg ? -1.0 : 1.0) * tbq3_lv[m] * n / sqrt(128.0);
    }
    for (i = 0; i < 128; ++i) {
        double acc = 0.0;
        for (j = 0; j < 128; ++j) acc += hadamard(i, j) * tbq3_s2[j] * y[j];
        out[i] = tbq3_s1[i] * acc / sqrt(128.0);
    }
}

/* Standalone TBQ3 dequantisation: n_values (a multiple of 128) original-space
 * values, each the binary64 value rounded to binary32. */
int orc_dequant_tbq3(const void *blocks, int64_t n_values, float *out)
{
    int64_t b;
    double v[128];
    int i;
    if (n_values % 128) return -1;
    tbq3_init();
    for (b = 0; b < n_values / 128; ++b) {
        tbq3_block_values((const uint8_t *)blocks + 52 * b, v);
        for (i = 0; i < 128; ++i) out[128 * b + i] = (float)v[i];
    }
    return 0;
}

/* Dequantise one row of D values to binary64. */
static void dequant_row(int type, const uint8_t *row, int d, double *out)
{
    int i;
    switch (type) {
    case ORC_F32:
        for (i = 0; i < d; ++i) {
            float f;
            memcpy(&f, row + 4 * i, 4);
            out[i] = (double)f;
        }
        break;
    case ORC_F16:
        for (i = 0; i < d; ++i) out[i] = orc_f16_to_f64(rd_u16(row + 2 * i));
        break;
    case ORC_Q8_0:
        for (i = 0; i < d; ++i) out[i] = q8_0_value(row + 34 * (i / 32), i % 32);
        break;
    case ORC_Q4_0:
        for (i = 0; i < d; ++i) out[i] = q4_0_value(row + 18 * (i / 32), i % 32);
        break;
    case ORC_TBQ3:
        for (i = 0; i < d; i += 128) tbq3_block_values(row + 52 * (i / 128), out + i);
        break;
    }
}

/* Standalone block dequantisation to binary32 (the exact values). */
int orc_dequant_q8_0(const void *blocks, int64_t n_values, float *out)
{
    int64_t i;
    if (n_values % 32) return -1;
    for (i = 0; i < n_values; ++i)
        out[i] = (float)q8_0_value((const uint8_t *)blocks + 34 * (i / 32), (int)(i % 32));
    return 0;
}

int orc_dequant_q4_0(const void *blocks, int64_t n_values, float *out)
{
    int64_t i;
    if (n_values % 32) return -1;
    for (i = 0; i < n_values; ++i)
        out[i] = (float)q4_0_value((const uint8_t *)blocks + 18 * (i / 32), (int)(i % 32));
    return 0;
}

/* binary32 -> IEEE 754 binary16, round to nearest, ties to even.  Written
 * from the format's definition in binary64 (every binary32 value and every
 * scaling by a power of two below is exact there): subnormal results are
 * multiples of 2^-24; a normal result 2^e (1 + m / 1024) has 1024 + m the
 * nearest integer to |x| 2^(10 - e); |x| >= 65520 (the midpoint between the
 * largest finite value 65504 and 2^16) rounds to infinity. */
static uint16_t f64_to_f16(double f)
{
    const double v = fabs(f);
    const uint16_t sign = signbit(f) ? 0x8000 : 0;
    double m;
    int ex, e;
    if (isnan(f)) return sign | 0x7e00;
    if (v >= 65520.0) return sign | 0x7c00;
    if (v < ldexp(1.0, -14)) /* rint gives 1024 for values that round up to 2^-14: the encoding 0x0400 */
        return sign | (uint16_t)rint(ldexp(v, 24));
    (void)frexp(v, &ex);
    e = ex - 1; /* 2^e <= v < 2^(e+1) */
    m = rint(ldexp(v, 10 - e));
    if (m == 2048.0) {
        m = 1024.0;
        ++e;
    }
    return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

uint16_t orc_f32_to_f16(float f) { return f64_to_f16((double)f); }

static void wr_u16(uint8_t *p, uint16_t h)
{
    p[0] = (uint8_t)(h & 0xff);
    p[1] = (uint8_t)(h >> 8);
}

/* One q8_0 block from 32 binary32 values (rule in the header). */
static void quant_q8_0_block(const float *x, uint8_t *blk)
{
    float amax = 0.0f, d, id;
    int i;
    for (i = 0; i < 32; ++i)
        if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
    d = amax / 127.0f;
    id = d != 0.0f ? 1.0f / d : 0.0f;
    wr_u16(blk, orc_f32_to_f16(d));
    for (i = 0; i < 32; ++i) {
        const float v = x[i] * id;
        blk[2 + i] = (uint8_t)(int8_t)roundf(v);
    }
}

/* One q4_0 block from 32 binary32 values (rule in the header). */
static void quant_q4_0_block(const float *x, uint8_t *blk)
{
    float amax = 0.0f, m = 0.0f, d, id;
    int i, n[32];
    for (i = 0; i < 32; ++i)
        if (fabsf(x[i]) > amax) {
            amax = fabsf(x[i]);
            m = x[i];
        }
    d = m / -8.0f;
    id = d != 0.0f ? 1.0f / d : 0.0f;
    wr_u16(blk, orc_f32_to_f16(d));
    for (i = 0; i < 32; ++i) {
        const float v = x[i] * id;
        const float w = v + 8.5f;
        int c = (int)w;
        if (c > 15) c = 15;
        n[i] = c;
    }
    for (i = 0; i < 16; ++i) blk[2 + i] = (uint8_t)(n[i] | (n[i + 16] << 4));
}

/* One TBQ3 block from 128 binary32 values (readings in the header):
 * n = ||x||_2, y = S2 H S1 x / sqrt(128), z = y sqrt(128) / n; value i takes
 * the level nearest to z_i (magnitude index m = the number of thresholds
 * (c_{j-1} + c_j) / 2 strictly below |z_i|; sign bit set when z_i < 0); a
 * block of zeros stores n = 0 and index 0.  Used by the oracle's own tests
 * (round trip, nearest level); the attention reads whatever bytes it gets. */
static void quant_tbq3_block(const float *x, uint8_t *blk)
{
    double n = 0.0, y[128];
    int i, j;
    for (i = 0; i < 128; ++i) n += (double)x[i] * (double)x[i];
    n = sqrt(n);
    for (i = 0; i < 128; ++i) {
        double acc = 0.0;
        for (j = 0; j < 128; ++j) acc += hadamard(i, j) * tbq3_s1[j] * (double)x[j];
        y[i] = tbq3_s2[i] * acc / sqrt(128.0);
    }
    memset(blk, 0, 52);
    wr_u16(blk, f64_to_f16(n));
    if (n == 0.0) return;
    for (i = 0; i < 128; ++i) {
        const double z = y[i] * sqrt(128.0) / n, a = fabs(z);
        int m = 0;
        for (j = 1; j < 4; ++j)
            if (a > 0.5 * (tbq3_lv[j - 1] + tbq3_lv[j])) m = j;
        blk[4 + i / 4] |= (uint8_t)(m << (2 * (i % 4)));
        if (z < 0.0) blk[36 + i / 8] |= (uint8_t)(1 << (i % 8));
    }
}

/* Store one row of D binary32 values in a cache type: binary32 bytes as
 * they are, binary16 rounded to nearest even, or D/32 blocks.  Returns 0, or
 * -1 for a bad type or a block type with D % 32 != 0. */
int orc_encode_row(int type, const float *x, int64_t d, uint8_t *out)
{
    int64_t i;
    if (!orc_row_bytes(type, d)) return -1;
    switch (type) {
    case ORC_F32:
        memcpy(out, x, 4 * d);
        break;
    case ORC_F16:
        for (i = 0; i < d; ++i) wr_u16(out + 2 * i, orc_f32_to_f16(x[i]));
        break;
    case ORC_Q8_0:
        for (i = 0; i < d / 32; ++i) quant_q8_0_block(x + 32 * i, out + 34 * i);
        break;
    case ORC_Q4_0:
        for (i = 0; i < d / 32; ++i) quant_q4_0_block(x + 32 * i, out + 18 * i);
        break;
    case ORC_TBQ3:
        tbq3_init();
        for (i = 0; i < d / 128; ++i) quant_tbq3_block(x + 128 * i, out + 52 * i);
        break;
    }
    return 0;
}

/* Where a new row at absolute position pos goes, for a layer whose window
 * holds positions [0, window_cap) and whose tail holds [window_cap,
 * window_cap + tail_cap): returns 0 (window) or 1 (tail) and the row index
 * inside that region in *row, or -1 when the position fits neither. */
int orc_route(int64_t pos, int64_t window_cap, int64_t tail_cap, int64_t *row)
{
    if (pos < 0) return -1;
    if (pos < window_cap) {
        *row = pos;
        return 0;
    }
    if (pos - window_cap < tail_cap) {
        *row = pos - window_cap;
        return 1;
    }
    return -1;
}

/* A segment of the KV cache: positions [0, n_keys) of a view.  Byte strides:
 * between positions, between KV heads inside a position, between sequences
 * (0 = one segment shared by every sequence). */
typedef struct {
    const void *k, *v;
    int32_t k_type, v_type;
    int64_t n_keys;
    int64_t k_pos_stride, v_pos_stride;
    int64_t k_head_stride, v_head_stride;
    int64_t k_seq_stride, v_seq_stride;
} orc_view;

/* The causal mask: sequence b's query sees key position t iff t <= q_pos[b]
 * (every key when there is no mask). */
static int key_seen(const int64_t *q_pos, int b, int64_t t)
{
    return !q_pos || t <= q_pos[b];
}

/*
 * Unsplit softmax attention of one query token per sequence over the keys of
 * all n_views views taken together (view 0's keys, then view 1's, ...).
 *
 * q:     [n_seq][n_q_heads][head_dim] binary32.
 * rows:  optional list of flattened (seq * n_q_heads + head) indices to
 *        compute; NULL computes every row.  o[r*head_dim + d] and lse[r] are
 *        written for the r-th listed row (or row r when rows is NULL).
 * q_to_kv: optional map query head -> KV head; NULL means contiguous groups
 *        h / (n_q_heads / n_kv_heads).
 * q_pos: optional causal mask by absolute key position for several query
 *        rows ("F5 M7 -- Rolling KV", section "2026-07-14 -- bug-2172
 *        SHIPPED": the streaming attention's mask is per cell and indexed by
 *        absolute key position, -inf for hidden keys; section "2026-07-12 --
 *        #582-P2 SHIPPED", bug-2161: the n_q > 1 prefill path over window and
 *        tail).  Key t of the concatenation
 *        (t = 0, 1, ... over view 0's keys, then view 1's, ...) sits at
 *        absolute position t; sequence b's query sits at q_pos[b] and sees
 *        the keys with t <= q_pos[b].  NULL: every key is seen.
 * A row that sees no key (an empty key set, or q_pos[b] < 0) gives o = 0 and
 * lse = -inf.
 */
int orc_attend(int n_seq, int n_q_heads, int n_kv_heads, int head_dim,
               double scale, double softcap, const int32_t *q_to_kv, const int64_t *q_pos,
               const float *q, int n_views, const orc_view *views,
               const int64_t *rows, int64_t n_rows, double *o, double *lse)
{
    int64_t n_total = 0, r;
    int vi, err = 0;
    if (n_seq <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0) return -1;
    if (!q_to_kv && (n_q_heads % n_kv_heads)) return -1;
    for (vi = 0; vi < n_views; ++vi) {
        if (!orc_row_bytes(views[vi].k_type, head_dim) || !orc_row_bytes(views[vi].v_type, head_dim))
            return -1;
        n_total += views[vi].n_keys;
    }
    if (!rows) n_rows = (int64_t)n_seq * n_q_heads;
    tbq3_init();

#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < n_rows; ++r) {
        int64_t row = rows ? rows[r] : r;
        int b = (int)(row / n_q_heads), h = (int)(row % n_q_heads);
        int g = q_to_kv ? q_to_kv[h] : h / (n_q_heads / n_kv_heads);
        double *s = (double *)malloc(sizeof(double) * (n_total > 0 ? n_total : 1));
        double *kv = (double *)malloc(sizeof(double) * head_dim);
        double *qd = (double *)malloc(sizeof(double) * head_dim);
        double *acc = o + r * head_dim;
        double mx = -INFINITY, z = 0.0;
        int64_t j, t;
        int d, w_i;
        if (!s || !kv || !qd) {
#pragma omp atomic write
            err = -4;
            free(s); free(kv); free(qd);
            continue;
        }
        for (d = 0; d < head_dim; ++d) qd[d] = (double)q[row * head_dim + d];

        /* scores s_j = scale * q . k_j, then the optional cap */
        t = 0;
        for (w_i = 0; w_i < n_views; ++w_i) {
            const orc_view *w = &views[w_i];
            const uint8_t *kb = (const uint8_t *)w->k + (int64_t)b * w->k_seq_stride + (int64_t)g * w->k_head_stride;
            for (j = 0; j < w->n_keys; ++j, ++t) {
                double dot = 0.0;
                if (!key_seen(q_pos, b, t)) continue; /* hidden key: no score */
                dequant_row(w->k_type, kb + j * w->k_pos_stride, head_dim, kv);
                for (d = 0; d < head_dim; ++d) dot += qd[d] * kv[d];
                s[t] = scale * dot;
                if (softcap > 0.0) s[t] = softcap * tanh(s[t] / softcap);
                if (s[t] > mx) mx = s[t];
            }
        }

        /* softmax-weighted sum of the value rows */
        for (d = 0; d < head_dim; ++d) acc[d] = 0.0;
        if (mx == -INFINITY) { /* no key seen */
            lse[r] = -INFINITY;
            free(s); free(kv); free(qd);
            continue;
        }
        t = 0;
        for (w_i = 0; w_i < n_views; ++w_i) {
            const orc_view *w = &views[w_i];
            const uint8_t *vb = (const uint8_t *)w->v + (int64_t)b * w->v_seq_stride + (int64_t)g * w->v_head_stride;
            for (j = 0; j < w->n_keys; ++j, ++t) {
                double p;
                if (!key_seen(q_pos, b, t)) continue;
                p = exp(s[t] - mx);
                z += p;
                dequant_row(w->v_type, vb + j * w->v_pos_stride, head_dim, kv);
                for (d = 0; d < head_dim; ++d) acc[d] += p * kv[d];
            }
        }
        for (d = 0; d < head_dim; ++d) acc[d] /= z;
        lse[r] = mx + log(z);
        free(s); free(kv); free(qd);
    }
    return err;
}

/*
 * The segment merge, in binary64: M = max_t lse_t,
 * O = sum_t O_t e^{lse_t - M} / sum_t e^{lse_t - M}, LSE = M + ln sum_t e^{lse_t - M}.
 * A part with lse = -inf has weight 0; when every part is empty the result is
 * O = 0, LSE = -inf.
 */
int orc_lse_combine(int n_parts, const double *const *o_parts, const double *const *lse_parts,
                    int64_t n_rows, int head_dim, double *o_out, double *lse_out)
{
    int64_t r;
    if (n_parts <= 0 || head_dim <= 0) return -1;
    for (r = 0; r < n_rows; ++r) {
        double mx = -INFINITY, z = 0.0;
        int t, d;
        for (t = 0; t < n_parts; ++t)
            if (lse_parts[t][r] > mx) mx = lse_parts[t][r];
        if (mx == -INFINITY) {
            for (d = 0; d < head_dim; ++d) o_out[r * head_dim + d] = 0.0;
            lse_out[r] = -INFINITY;
            continue;
        }
        for (d = 0; d < head_dim; ++d) o_out[r * head_dim + d] = 0.0;
        for (t = 0; t < n_parts; ++t) {
            double w = exp(lse_parts[t][r] - mx);
            z += w;
            for (d = 0; d < head_dim; ++d) o_out[r * head_dim + d] += w * o_parts[t][r * head_dim + d];
        }
        for (d = 0; d < head_dim; ++d) o_out[r * head_dim + d] /= z;
        lse_out[r] = mx + log(z);
    }
    return 0;
}

/* Threads the OpenMP runtime will use (1 without OpenMP). */
int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
