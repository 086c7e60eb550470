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
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_Q8_0 = 2, ORC_Q4_0 = 3 };

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
 * An empty key set gives o = 0 and lse = -inf.
 */
int orc_attend(int n_seq, int n_q_heads, int n_kv_heads, int head_dim,
               double scale, double softcap, const int32_t *q_to_kv,
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
                dequant_row(w->k_type, kb + j * w->k_pos_stride, head_dim, kv);
                for (d = 0; d < head_dim; ++d) dot += qd[d] * kv[d];
                s[t] = scale * dot;
                if (softcap > 0.0) s[t] = softcap * tanh(s[t] / softcap);
                if (s[t] > mx) mx = s[t];
            }
        }

        /* softmax-weighted sum of the value rows */
        for (d = 0; d < head_dim; ++d) acc[d] = 0.0;
        t = 0;
        for (w_i = 0; w_i < n_views; ++w_i) {
            const orc_view *w = &views[w_i];
            const uint8_t *vb = (const uint8_t *)w->v + (int64_t)b * w->v_seq_stride + (int64_t)g * w->v_head_stride;
            for (j = 0; j < w->n_keys; ++j, ++t) {
                double p = exp(s[t] - mx);
                z += p;
                dequant_row(w->v_type, vb + j * w->v_pos_stride, head_dim, kv);
                for (d = 0; d < head_dim; ++d) acc[d] += p * kv[d];
            }
        }
        if (n_total == 0) {
            lse[r] = -INFINITY;
        } else {
            for (d = 0; d < head_dim; ++d) acc[d] /= z;
            lse[r] = mx + log(z);
        }
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
