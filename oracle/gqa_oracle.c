/*
 * gqa_oracle.c -- fp64 CPU oracle for grouped-query attention (GQA).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls this
 * file; only the tests, the package's smoke check and the benchmark's CPU-baseline
 * leg do. It shares no source, header, table or helper with the HIP kernels.
 *
 * What it computes (plain definition, no blocking, fusion or reordering):
 *
 *   GQA splits H query heads into G groups of R = H / G consecutive heads; every
 *   head of group g reads the same key/value head g, so G = H is multi-head
 *   attention and G = 1 is multi-query attention
 *     [GQA paper digest page (51969.com), section "Grouped-query attention (GQA)"
 *      and its Figure 2; "LLM principles -- code implementation of multi-head
 *      attention (MQA and GQA)", section 5, where the group of a head is its index
 *      divided by the heads per group].
 *   Query head h therefore reads KV head g = h / R (integer division).
 *
 *   For one query row q (length D) against n key/value rows:
 *     s_j   = scale * sum_d q[d] * k[j][d]                    (scaled dot product)
 *     p_j   = exp(s_j - max_j s_j) / sum_j exp(s_j - max_j s_j)  (softmax over keys)
 *     out_d = sum_j p_j * v[j][d]
 *   ["LLM principles -- code ...", sections 3 and 5: Q times K transposed, divided
 *    by the square root of the head size, softmax over the last axis, times V].
 *   Subtracting the maximum changes nothing in exact arithmetic; it only keeps
 *   exp() finite.
 *
 *   Prefill (causal): row i attends to keys j <= i; the upper triangle above the
 *   diagonal is masked to -inf before the softmax, which is the same as leaving
 *   those keys out ["LLM principles -- code ...", section 3, the triu mask with
 *   diagonal 1]. Non-causal prefill attends to all T keys.
 *
 *   Decode: the current token has already been appended to the cache (the cache is
 *   concatenated before the scores are formed, same page, sections 3 and 5), so the
 *   query attends to all rows 0 .. L_b-1 of its sequence, itself included.
 *   Readings where the pages say nothing: L_b <= 0 gives a zero row, L_b > T_cap is
 *   clamped to T_cap.
 *
 *   fp8 KV storage ("GQA revolution: how xformers speeds up LLM inference",
 *   section on mixed-precision KV storage): a stored value is code * scale with one
 *   fp32 scale per (sequence, KV head). The code is OCP 8-bit E4M3FN: 1 sign bit,
 *   4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal
 *   (value 2^-6 * m/8); S.1111.111 is NaN and there are no infinities, so the
 *   largest finite magnitude is 2^8 * 1.75 = 448.
 *
 *   INT4 KV storage (same page and section, which names 4-bit storage for K/V and gives
 *   no format; this oracle's reading): each 4-bit field u in 0..15 stands for
 *   (u - 8) * scale, one fp32 scale per (sequence, KV head); two fields per byte, the
 *   low four bits holding the even head dim. A value x is stored as the integer nearest
 *   to x / scale (the quotient in fp32, ties to even), clamped to -8 .. 7, plus 8.
 *
 * Layouts (all contiguous, head dimension innermost):
 *   decode  q, out [B][H][D]; k_cache, v_cache [B][G][T_cap][D]; seq_lens [B]
 *   prefill q, out [B][H][T][D]; k, v [B][G][T][D]
 *
 * All arithmetic is IEEE double. Build: gcc -O2 -fopenmp (no -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One output row: attention of q over rows 0..n-1 of K and V (row stride D).
 * s is caller scratch of at least n doubles. n <= 0 writes zeros. */
static void attend_row(const double *q, const double *K, const double *V, long n, int D,
                       double scale, double *out, double *s)
{
    long j;
    int d;
    if (n <= 0) {
        for (d = 0; d < D; ++d) out[d] = 0.0;
        return;
    }
    double m = -INFINITY;
    for (j = 0; j < n; ++j) {
        double dot = 0.0;
        for (d = 0; d < D; ++d) dot += q[d] * K[j * (long)D + d];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    double denom = 0.0;
    for (j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        denom += s[j];
    }
    for (d = 0; d < D; ++d) {
        double acc = 0.0;
        for (j = 0; j < n; ++j) acc += s[j] * V[j * (long)D + d];
        out[d] = acc / denom;
    }
}

/* Decode's own coding of the same definition (every prefill row goes through attend_row
 * above): the softmax is normalised through the log of its denominator,
 * p_t = exp(s_t - lse) with lse = m + log(sum_t exp(s_t - m)), and the output is built one
 * value row at a time, out += p_t * v_t. In exact arithmetic it equals attend_row; it is
 * written apart so that the pin "incremental decode equals causal prefill" compares two
 * codings of the definition, not one with itself. w is caller scratch of at least n doubles;
 * n <= 0 writes zeros. */
static void decode_row(const double *q, const double *K, const double *V, long n, int D,
                       double scale, double *out, double *w)
{
    long t;
    int e;
    for (e = 0; e < D; ++e) out[e] = 0.0;
    if (n <= 0) return;
    double top = -INFINITY;
    for (t = 0; t < n; ++t) {
        const double *kt = K + t * (long)D;
        double qk = 0.0;
        for (e = 0; e < D; ++e) qk += kt[e] * q[e];
        w[t] = qk * scale;
        if (w[t] > top) top = w[t];
    }
    double z = 0.0;
    for (t = 0; t < n; ++t) z += exp(w[t] - top);
    const double lse = top + log(z);
    for (t = 0; t < n; ++t) {
        const double p = exp(w[t] - lse);
        const double *vt = V + t * (long)D;
        for (e = 0; e < D; ++e) out[e] += p * vt[e];
    }
}

static int kv_head_of(int h, int H, int G) { return h / (H / G); }

int gqa_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void gqa_oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Decode: out[b][h] = attention of q[b][h] over cache rows 0..L_b-1 of KV head h/R. */
int gqa_oracle_decode(const double *q, const double *k_cache, const double *v_cache,
                      const int32_t *seq_lens, double *out, int B, int H, int G, int D,
                      int T_cap, double scale)
{
    if (B < 1 || H < 1 || G < 1 || D < 1 || T_cap < 1 || H % G != 0) return 1;
    long bh, nbh = (long)B * H;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)T_cap);
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (bh = 0; bh < nbh; ++bh) {
                int b = (int)(bh / H), h = (int)(bh % H);
                int g = kv_head_of(h, H, G);
                long L = seq_lens[b];
                if (L > T_cap) L = T_cap;
                const double *K = k_cache + ((long)b * G + g) * T_cap * D;
                const double *V = v_cache + ((long)b * G + g) * T_cap * D;
                decode_row(q + bh * D, K, V, L, D, scale, out + bh * D, s);
            }
            free(s);
        }
    }
    return fail ? 2 : 0;
}

/* Decode, selected rows only: rows[r] = b*H + h; out_rows[r][D]. */
int gqa_oracle_decode_rows(const double *q, const double *k_cache, const double *v_cache,
                           const int32_t *seq_lens, int B, int H, int G, int D, int T_cap,
                           double scale, const int64_t *rows, long nrows, double *out_rows)
{
    if (B < 1 || H < 1 || G < 1 || D < 1 || T_cap < 1 || H % G != 0) return 1;
    long r;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)T_cap);
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (r = 0; r < nrows; ++r) {
                long bh = rows[r];
                int b = (int)(bh / H), h = (int)(bh % H);
                int g = kv_head_of(h, H, G);
                long L = seq_lens[b];
                if (L > T_cap) L = T_cap;
                const double *K = k_cache + ((long)b * G + g) * T_cap * D;
                const double *V = v_cache + ((long)b * G + g) * T_cap * D;
                decode_row(q + bh * D, K, V, L, D, scale, out_rows + r * D, s);
            }
            free(s);
        }
    }
    return fail ? 2 : 0;
}

/* Prefill: out[b][h][i] = attention of q[b][h][i] over keys 0..i (causal) or 0..T-1. */
int gqa_oracle_prefill(const double *q, const double *k, const double *v, double *out, int B,
                       int T, int H, int G, int D, double scale, int causal)
{
    if (B < 1 || T < 1 || H < 1 || G < 1 || D < 1 || H % G != 0) return 1;
    long row, nrow = (long)B * H * T;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)T);
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (row = 0; row < nrow; ++row) {
                int i = (int)(row % T);
                long bh = row / T;
                int b = (int)(bh / H), h = (int)(bh % H);
                int g = kv_head_of(h, H, G);
                long n = causal ? (long)i + 1 : (long)T;
                const double *K = k + ((long)b * G + g) * T * D;
                const double *V = v + ((long)b * G + g) * T * D;
                attend_row(q + row * D, K, V, n, D, scale, out + row * D, s);
            }
            free(s);
        }
    }
    return fail ? 2 : 0;
}

/*
 * Prefill of a chunk of Tq query positions against a cache that already holds earlier
 * tokens ("LLM principles -- code implementation of multi-head attention (MQA and GQA)",
 * sections 3 and 5: new keys and values are concatenated to the cache before the scores, and
 * the causal mask hides later keys). q, out [B,H,Tq,D]; k, v [B,G,T_cap,D]; seq_lens[b] = L_b
 * counts every valid cache row, the chunk included, so query i of sequence b sits at
 * position p = L_b - Tq + i. It sees keys 0 .. p (causal) or 0 .. L_b - 1 (not causal), never
 * beyond L_b - 1; L_b is clamped to 0 .. T_cap as in decode. A row that sees no key (p < 0)
 * is zero. With Tq = 1 this is decode; with L_b = Tq = T_cap it is the plain prefill.
 */
int gqa_oracle_prefill_cached(const double *q, const double *k, const double *v, const int32_t *seq_lens,
                              double *out, int B, int Tq, int H, int G, int D, long T_cap, double scale,
                              int causal)
{
    if (B < 1 || Tq < 1 || H < 1 || G < 1 || D < 1 || T_cap < 1 || H % G != 0) return 1;
    long row, nrow = (long)B * H * Tq;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)T_cap);
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (row = 0; row < nrow; ++row) {
                int i = (int)(row % Tq);
                long bh = row / Tq;
                int b = (int)(bh / H), h = (int)(bh % H);
                int g = kv_head_of(h, H, G);
                long L = seq_lens[b] < 0 ? 0 : (seq_lens[b] > T_cap ? T_cap : seq_lens[b]);
                long p = L - Tq + i;
                long n = causal ? (p + 1 < L ? p + 1 : L) : L;
                const double *K = k + ((long)b * G + g) * T_cap * D;
                const double *V = v + ((long)b * G + g) * T_cap * D;
                attend_row(q + row * D, K, V, n, D, scale, out + row * D, s);
            }
            free(s);
        }
    }
    return fail ? 2 : 0;
}

/* Prefill, selected rows only: rows[r] = (b*H + h)*T + i; out_rows[r][D]. */
int gqa_oracle_prefill_rows(const double *q, const double *k, const double *v, int B, int T,
                            int H, int G, int D, double scale, int causal, const int64_t *rows,
                            long nrows, double *out_rows)
{
    if (B < 1 || T < 1 || H < 1 || G < 1 || D < 1 || H % G != 0) return 1;
    long r;
    int fail = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)T);
        if (!s) {
#pragma omp atomic write
            fail = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (r = 0; r < nrows; ++r) {
                long row = rows[r];
                int i = (int)(row % T);
                long bh = row / T;
                int b = (int)(bh / H), h = (int)(bh % H);
                int g = kv_head_of(h, H, G);
                long n = causal ? (long)i + 1 : (long)T;
                const double *K = k + ((long)b * G + g) * T * D;
                const double *V = v + ((long)b * G + g) * T * D;
                attend_row(q + row * D, K, V, n, D, scale, out_rows + r * D, s);
            }
            free(s);
        }
    }
    return fail ? 2 : 0;
}

/* OCP E4M3FN code -> its exact value (NaN for S.1111.111). */
double gqa_oracle_e4m3fn_value(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Quantise one value to OCP E4M3FN: the finite code whose value is nearest to q, ties to
 * the code with an even mantissa (its last bit clear), the sign kept (a negative q that
 * rounds to zero gives the code of -0). Magnitudes beyond the largest code, 448, give 448:
 * a cache with fixed per-(sequence, KV head) scales saturates tokens that outgrow them
 * (reading; "GQA revolution ...", section on mixed-precision KV storage, stores code *
 * scale but does not say what happens out of range). NaN gives the NaN code 0x7F.
 * Written as an exhaustive search over the 127 non-negative finite codes. */
uint8_t gqa_oracle_e4m3fn_encode(float q)
{
    if (isnan(q)) return 0x7F;
    const int neg = signbit(q) ? 1 : 0;
    const double a = fabs((double)q);
    int best = 0;
    double best_err = INFINITY;
    int c;
    for (c = 0; c <= 0x7E; ++c) {
        /* differences of a float and a 4-significant-bit value are exact in double */
        const double err = fabs(a - gqa_oracle_e4m3fn_value((uint8_t)c));
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(best | (neg << 7));
}

/* Quantise n values: codes[i] = encode(x[i] / scale), the quotient taken in fp32. */
void gqa_oracle_quant_e4m3fn(const float *x, float scale, long n, uint8_t *codes)
{
    long i;
    for (i = 0; i < n; ++i) codes[i] = gqa_oracle_e4m3fn_encode(x[i] / scale);
}

/* Dequantise fp8 slabs: out[s][i] = value(codes[s][i]) * scales[s], s < nslab, i < slab_len. */
void gqa_oracle_dequant_e4m3fn(const uint8_t *codes, const float *scales, long nslab,
                               long slab_len, double *out)
{
    long s;
#pragma omp parallel for schedule(static)
    for (s = 0; s < nslab; ++s) {
        double sc = (double)scales[s];
        long i;
        for (i = 0; i < slab_len; ++i)
            out[s * slab_len + i] = gqa_oracle_e4m3fn_value(codes[s * slab_len + i]) * sc;
    }
}

/* INT4 field u (0..15) -> its value in units of the scale: u - 8. */
int gqa_oracle_int4_value(int u) { return (u & 15) - 8; }

/* Field for the fp32 quotient q: the nearest integer, ties to even, clamped to -8 .. 7,
 * then + 8. NaN stores the field of 0 (8). */
int gqa_oracle_int4_encode(float q)
{
    double x = (double)q, r, f;
    if (isnan(x)) return 8;
    r = floor(x);
    f = x - r;
    if (f > 0.5 || (f == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    if (r < -8.0) r = -8.0;
    if (r > 7.0) r = 7.0;
    return (int)r + 8;
}

/* Quantise n values (n even) to packed fields: byte i holds x[2i] (low) and x[2i+1] (high),
 * each the field of x / scale, the quotient taken in fp32. */
void gqa_oracle_quant_int4(const float *x, float scale, long n, uint8_t *packed)
{
    long i;
    for (i = 0; i + 1 < n; i += 2) {
        int lo = gqa_oracle_int4_encode(x[i] / scale), hi = gqa_oracle_int4_encode(x[i + 1] / scale);
        packed[i / 2] = (uint8_t)(lo | (hi << 4));
    }
}

/* Packed INT4 slabs -> float64 values: out[s][i] = (field i of slab s - 8) * scales[s];
 * slab_len counts values (even). */
void gqa_oracle_dequant_int4(const uint8_t *packed, const float *scales, long nslab, long slab_len, double *out)
{
    long s;
#pragma omp parallel for schedule(static)
    for (s = 0; s < nslab; ++s) {
        double sc = (double)scales[s];
        long i;
        for (i = 0; i < slab_len; ++i) {
            uint8_t byte = packed[(s * slab_len + i) / 2];
            int u = (i & 1) ? (byte >> 4) : (byte & 15);
            out[s * slab_len + i] = (double)gqa_oracle_int4_value(u) * sc;
        }
    }
}
