/*
 * FP64 CPU oracle for dense noncausal attention and its prefix-cached variant.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it. It shares no code with the HIP library.
 *
 * What it computes (page "Audit SGLang interfaces and refresh validated kernel
 * solutions"):
 *   - definitions/dense_attention/noncausal_dense_attention_h32_d128.json and
 *     ..._h32_d64.json, field "reference": scores = einsum(bqhd,bkhd->bhqk) of Q and
 *     K in float, times head_dim ** -0.5; probabilities = softmax over k;
 *     output = einsum(bhqk,bkhd->bqhd) of the probabilities and V.
 *   - definitions/block_causal_attention/prefix_cached_block_causal_h32_d128.json,
 *     field "reference" (post-change text): keys and values are the concatenation
 *     along the sequence axis of (K_prefix, K_current) and (V_prefix, V_current);
 *     every query sees every key; scale 128 ** -0.5.
 *   - definitions/block_causal_attention/prefix_cached_block_causal_h32_d128_prefix0.json,
 *     field "reference" (post-change text): with positions 0..N-1 and image_ids [N]
 *     (text = -1), query i may see key j when j <= i, or when image_ids[i] >= 0 and
 *     image_ids[i] == image_ids[j]; the other scores are filled with -inf before the
 *     softmax; scale 128 ** -0.5 (head_dim ** -0.5 here).
 * The pages evaluate in FP32; this oracle evaluates the same formula in FP64 and
 * returns the unrounded FP64 result (the pages' final BF16 cast is left to the
 * comparison).
 *
 * Tensors are [B, N, H, D], contiguous, holding BF16 bit patterns (uint16).
 * Widening BF16 to FP64 is exact: the 16 bits are the top half of an FP32.
 *
 * The key sequence is the concatenation of segment 0 (n0 rows, e.g. the prefix)
 * and segment 1 (n1 rows, e.g. the current keys). Dense attention is n1 == 0.
 *
 * Softmax is evaluated row by row as exp(s_j - max_j s_j) / sum_j exp(s_j - max_j s_j),
 * which is the softmax of the row (the subtracted maximum cancels exactly).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_f64(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Pointer to element [b, j, h, 0] of the concatenated key (or value) sequence. */
static const uint16_t* seq_row(const uint16_t* s0, long n0, const uint16_t* s1, long n1,
                               long b, long j, long H, long D, long h) {
    if (j < n0) return s0 + ((b * n0 + j) * H + h) * D;
    return s1 + ((b * n1 + (j - n0)) * H + h) * D;
}

/*
 * Computes output rows of attention in FP64.
 *
 * rows: flat indices r = (b * Nq + i) * H + h into the [B, Nq, H] row space, or
 *       NULL for every row in order. nrows: how many.
 * out:  [nrows, D] FP64 outputs (unrounded).
 * lse:  optional [nrows] natural-log log-sum-exp of the scaled scores.
 * psum: optional [nrows] sum of the normalised probabilities (should be 1).
 * scale_override: <= 0 means head_dim ** -0.5, the pages' fixed scale.
 * Returns 0, -1 on bad arguments, -2 on a row index out of range, -3 on allocation
 * failure.
 */
int oracle_attn_rows(const uint16_t* q, const uint16_t* k0, const uint16_t* v0, long n0,
                     const uint16_t* k1, const uint16_t* v1, long n1, long B, long Nq,
                     long H, long D, const long* rows, long nrows, double* out, double* lse,
                     double* psum, double scale_override) {
    if (!q || !out || B < 1 || Nq < 1 || H < 1 || D < 1 || n0 < 0 || n1 < 0) return -1;
    if (n0 + n1 < 1) return -1;
    if (n0 > 0 && (!k0 || !v0)) return -1;
    if (n1 > 0 && (!k1 || !v1)) return -1;
    const long nk = n0 + n1;
    const long total = B * Nq * H;
    if (!rows) nrows = total;
    const double scale = scale_override > 0 ? scale_override : pow((double)D, -0.5);
    int fail = 0;

#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)nk);
        double* qd = (double*)malloc(sizeof(double) * (size_t)D);
        if (!s || !qd) {
#pragma omp atomic write
            fail = 3;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (long t = 0; t < nrows; ++t) {
                const long r = rows ? rows[t] : t;
                if (r < 0 || r >= total) {
#pragma omp atomic write
                    fail = 2;
                    continue;
                }
                const long h = r % H;
                const long bi = r / H;
                const long i = bi % Nq;
                const long b = bi / Nq;
                const uint16_t* qr = q + ((b * Nq + i) * H + h) * D;
                for (long d = 0; d < D; ++d) qd[d] = bf16_to_f64(qr[d]);

                /* scores s_j = scale * <q_i, k_j> over the concatenated keys */
                double mx = -INFINITY;
                for (long j = 0; j < nk; ++j) {
                    const uint16_t* kr = seq_row(k0, n0, k1, n1, b, j, H, D, h);
                    double dot = 0.0;
                    for (long d = 0; d < D; ++d) dot += qd[d] * bf16_to_f64(kr[d]);
                    s[j] = dot * scale;
                    if (s[j] > mx) mx = s[j];
                }
                /* softmax: e_j = exp(s_j - max), l = sum e_j, p_j = e_j / l */
                double l = 0.0;
                for (long j = 0; j < nk; ++j) {
                    s[j] = exp(s[j] - mx);
                    l += s[j];
                }
                double* o = out + t * D;
                for (long d = 0; d < D; ++d) o[d] = 0.0;
                double ps = 0.0;
                for (long j = 0; j < nk; ++j) {
                    const double p = s[j] / l;
                    ps += p;
                    const uint16_t* vr = seq_row(v0, n0, v1, n1, b, j, H, D, h);
                    for (long d = 0; d < D; ++d) o[d] += p * bf16_to_f64(vr[d]);
                }
                if (lse) lse[t] = mx + log(l);
                if (psum) psum[t] = ps;
            }
        }
        free(s);
        free(qd);
    }
    return fail ? -fail : 0;
}

/*
 * Block-causal attention without a prefix (the "_prefix0" definition): Q, K, V are
 * [B, N, H, D] and ids is image_ids [N], shared by every batch entry. Only the
 * allowed keys of a row enter its softmax (a -inf score contributes exp(-inf) = 0).
 * Arguments and return codes as oracle_attn_rows (keys = queries, N of them);
 * returns -4 if a row has no allowed key (cannot happen: j = i is always allowed).
 */
int oracle_block_causal_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const int32_t* ids, long B, long N, long H, long D,
                             const long* rows, long nrows, double* out, double* lse,
                             double* psum) {
    if (!q || !k || !v || !ids || !out || B < 1 || N < 1 || H < 1 || D < 1) return -1;
    const long total = B * N * H;
    if (!rows) nrows = total;
    const double scale = pow((double)D, -0.5);
    int fail = 0;

#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
        unsigned char* allowed = (unsigned char*)malloc((size_t)N);
        double* qd = (double*)malloc(sizeof(double) * (size_t)D);
        if (!s || !allowed || !qd) {
#pragma omp atomic write
            fail = 3;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (long t = 0; t < nrows; ++t) {
                const long r = rows ? rows[t] : t;
                if (r < 0 || r >= total) {
#pragma omp atomic write
                    fail = 2;
                    continue;
                }
                const long h = r % H;
                const long bi = r / H;
                const long i = bi % N;
                const long b = bi / N;
                const uint16_t* qr = q + ((b * N + i) * H + h) * D;
                for (long d = 0; d < D; ++d) qd[d] = bf16_to_f64(qr[d]);

                /* visibility of key j for query i, then the allowed scores */
                double mx = -INFINITY;
                long seen = 0;
                for (long j = 0; j < N; ++j) {
                    const int same_image = ids[i] >= 0 && ids[i] == ids[j];
                    allowed[j] = (unsigned char)(j <= i || same_image);
                    if (!allowed[j]) continue;
                    ++seen;
                    const uint16_t* kr = k + ((b * N + j) * H + h) * D;
                    double dot = 0.0;
                    for (long d = 0; d < D; ++d) dot += qd[d] * bf16_to_f64(kr[d]);
                    s[j] = dot * scale;
                    if (s[j] > mx) mx = s[j];
                }
                if (seen == 0) {
#pragma omp atomic write
                    fail = 4;
                    continue;
                }
                double l = 0.0;
                for (long j = 0; j < N; ++j) {
                    if (!allowed[j]) continue;
                    s[j] = exp(s[j] - mx);
                    l += s[j];
                }
                double* o = out + t * D;
                for (long d = 0; d < D; ++d) o[d] = 0.0;
                double ps = 0.0;
                for (long j = 0; j < N; ++j) {
                    if (!allowed[j]) continue;
                    const double p = s[j] / l;
                    ps += p;
                    const uint16_t* vr = v + ((b * N + j) * H + h) * D;
                    for (long d = 0; d < D; ++d) o[d] += p * bf16_to_f64(vr[d]);
                }
                if (lse) lse[t] = mx + log(l);
                if (psum) psum[t] = ps;
            }
        }
        free(s);
        free(allowed);
        free(qd);
    }
    return fail ? -fail : 0;
}

/* Window of odd size k around position i on an axis of length L (k <= L): the k
 * consecutive positions centred on i, moved inside [0, L) at the ends, so every query
 * has exactly k neighbours on the axis. This is the neighborhood the pages' 3-D
 * neighborhood attention delegates to (natten.functional.na3d with its defaults); the
 * pages do not spell it out, and this is NATTEN's published definition. */
static void na_window(long i, long k, long L, long* lo, long* hi) {
    long s = i - k / 2;
    if (s > L - k) s = L - k;
    if (s < 0) s = 0;
    *lo = s;
    *hi = s + k;
}

/*
 * 3-D neighborhood attention (page "Audit SGLang interfaces and refresh validated
 * kernel solutions", definitions/neighborhood_attention/
 * neighborhood_attention_3d_h{4,8,16,32}_d64_kt*_ky*_kx*, called as
 * natten.functional.na3d(query, key, value, kernel_size, scale=1.0); the model's scale
 * is already in Q). q, k, v and out rows use the layout [B, T, Y, X, H, D]. Query
 * (b, t, y, x, h) attends to the kt*ky*kx keys (b, t', y', x', h) with t' in the
 * window of t on the T axis, y' in that of y, x' in that of x (na_window); its score
 * with a key is the plain dot product (scale 1).
 *
 * rows: flat query indices ((((b*T + t)*Y + y)*X + x)*H + h), or NULL for all.
 * Returns 0; -1 bad arguments (null, size < 1, even window or window longer than its
 * axis); -2 row index out of range; -3 allocation failure.
 */
int oracle_na3d_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, long B, long T,
                     long Y, long X, long H, long D, long kt, long ky, long kx,
                     const long* rows, long nrows, double* out) {
    if (!q || !k || !v || !out || B < 1 || T < 1 || Y < 1 || X < 1 || H < 1 || D < 1) return -1;
    if (kt < 1 || ky < 1 || kx < 1 || kt % 2 == 0 || ky % 2 == 0 || kx % 2 == 0) return -1;
    if (kt > T || ky > Y || kx > X) return -1;
    const long total = B * T * Y * X * H;
    if (!rows) nrows = total;
    const long nkeys = kt * ky * kx;
    int fail = 0;

#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)nkeys);
        long* kidx = (long*)malloc(sizeof(long) * (size_t)nkeys);
        double* qd = (double*)malloc(sizeof(double) * (size_t)D);
        if (!s || !kidx || !qd) {
#pragma omp atomic write
            fail = 3;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (long r_i = 0; r_i < nrows; ++r_i) {
                const long r = rows ? rows[r_i] : r_i;
                if (r < 0 || r >= total) {
#pragma omp atomic write
                    fail = 2;
                    continue;
                }
                const long h = r % H;
                const long pos = r / H;
                const long x = pos % X;
                const long y = (pos / X) % Y;
                const long t = (pos / (X * Y)) % T;
                const long b = pos / (X * Y * T);
                const uint16_t* qr = q + (pos * H + h) * D;
                for (long d = 0; d < D; ++d) qd[d] = bf16_to_f64(qr[d]);

                long t0, t1, y0, y1, x0, x1;
                na_window(t, kt, T, &t0, &t1);
                na_window(y, ky, Y, &y0, &y1);
                na_window(x, kx, X, &x0, &x1);
                long n = 0;
                double mx = -INFINITY;
                for (long tt = t0; tt < t1; ++tt)
                    for (long yy = y0; yy < y1; ++yy)
                        for (long xx = x0; xx < x1; ++xx) {
                            const long kp = ((b * T + tt) * Y + yy) * X + xx;
                            const uint16_t* kr = k + (kp * H + h) * D;
                            double dot = 0.0;
                            for (long d = 0; d < D; ++d) dot += qd[d] * bf16_to_f64(kr[d]);
                            kidx[n] = kp;
                            s[n] = dot;
                            if (dot > mx) mx = dot;
                            ++n;
                        }
                double l = 0.0;
                for (long j = 0; j < n; ++j) {
                    s[j] = exp(s[j] - mx);
                    l += s[j];
                }
                double* o = out + r_i * D;
                for (long d = 0; d < D; ++d) o[d] = 0.0;
                for (long j = 0; j < n; ++j) {
                    const double pj = s[j] / l;
                    const uint16_t* vr = v + (kidx[j] * H + h) * D;
                    for (long d = 0; d < D; ++d) o[d] += pj * bf16_to_f64(vr[d]);
                }
            }
        }
        free(s);
        free(kidx);
        free(qd);
    }
    return fail ? -fail : 0;
}

/* Number of OpenMP threads the oracle will use (1 when built without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
