/*
 * TriAttention KV-cache pruning: reference oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, fp64 CPU implementation of
 * what the pruning path computes.  It exists to check the HIP library against;
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  It shares no code, header, table or constant with the HIP library.
 *
 * Sources (web pages describing TriAttention; their formulas were lost in
 * extraction, so every step below restates the prose in my own notation):
 *   [YY] "实现单卡4090跑通OpenClaw!英伟达&浙大等提出长上下文推理KV压缩新方法
 *        TriAttention" (yeyulingfeng.com), section 主要方法.
 *   [ZN] "TriAttention：用三角级数压缩KV缓存，让长推理模型跑在消费级显卡上"
 *        (zingnex.cn), sections 预RoPE空间的发现 and
 *        TriAttention的核心机制：三角级数距离建模.
 *
 * Notation.  d = head_dim, F = d/2 rotary bands.  Band f of a stored (post-RoPE)
 * row x is the complex number x[f] + i x[f+F] (half-split pairing) with angular
 * frequency w_f = theta^(-2f/d).  A key stored at position p is the pre-RoPE key
 * k_f rotated by e^{i w_f p}.  A query head h has an offline centre per band
 * with magnitude M[h][f], phase phi[h][f] and concentration R[h][f] (mean
 * resultant length).  t is the position of the next query; O is the offset set.
 *
 * Parity status: every function here is pinned by a CPU test (closed forms,
 * invariants, brute force on tiny inputs, hand-worked fixtures) except that no
 * check can reach the paper's own (lost) score formula: the score is this
 * reconstruction, see orc_score_segment.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* Exact value of stored element i (fp32, or bf16 widened by a 16-bit shift). */
static double stored_value(const void* base, int dtype, int64_t i) {
    if (dtype == ORC_F32) return (double)((const float*)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * Key importance scores of one segment (one KV head of one layer of one
 * sequence) for its G query heads.
 *
 * Steps, in the order [YY] 主要方法 gives them:
 *  1. Un-rotate.  The key's band representation in the pre-RoPE space:
 *     magnitude |k_f| = |x_f| (a rotation keeps length) and phase
 *     psi_f = arg(x_f) - w_f p.
 *  2. Trigonometric-series term.  Under RoPE the query/key logit is a sum over
 *     bands of a cosine of (w_f * relative distance + phase difference); with
 *     the query replaced by its offline centre it depends on the distance only
 *     ([YY] 主要方法, paragraph on rewriting the RoPE logit; [ZN] 核心机制).
 *     The key is scored at each future query position t+o, o in O, and the
 *     scores are averaged ([YY] 主要方法, paragraph on geometric future offsets):
 *        trig_h = (1/|O|) sum_o sum_f M[h][f] |k_f| cos(w_f (t+o-p) + phi[h][f] - psi_f)
 *  3. Norm term, which compensates for the centre approximation and is
 *     suppressed where the band is concentrated and boosted where it is not
 *     ([YY] 主要方法, paragraph on the norm score; [ZN] 核心机制, Q/K norms as an
 *     auxiliary signal).  Reading: linear weight (1 - R):
 *        norm_h = sum_f (1 - R[h][f]) M[h][f] |k_f|
 *  4. Fusion into one importance score ([YY] 主要方法): S_h = trig_h + norm_h.
 *     Reading: plain sum, no 1/sqrt(d) (z-scoring makes a common scale moot).
 *
 * K: [N][d] stored rows; pos: [N]; M, phi, R: [G][F]; offsets: [n_off].
 * S: [G][N] output.  trig_out / norm_out: optional [G][N] outputs of the two
 * parts.  Returns 0, or -1 on bad arguments.
 */
/* Score variants (the ablated components the pages name, [YY] 主实验结果: the
 * trigonometric score, the adaptive weighting and the geometric offsets; plus
 * the alternative reading of the centre magnitude).  Linear offsets need no
 * flag: they are a different offset set. */
#define ORC_VAR_TRIG_ONLY 1        /* drop the norm term                        */
#define ORC_VAR_NORM_ONLY 2        /* drop the trigonometric term               */
#define ORC_VAR_FIXED_WEIGHT 4     /* norm weight M instead of (1 - R) M        */
#define ORC_VAR_R_WEIGHTED_TRIG 8  /* trigonometric term with R M instead of M  */

int orc_score_segment_variant(const void* K, int dtype, const int32_t* pos, int64_t N, int d,
                              double theta, int64_t t, const float* M, const float* phi,
                              const float* R, int G, const int64_t* offsets, int n_off, int variant,
                              double* S, double* trig_out, double* norm_out);

int orc_score_segment(const void* K, int dtype, const int32_t* pos, int64_t N, int d,
                      double theta, int64_t t, const float* M, const float* phi,
                      const float* R, int G, const int64_t* offsets, int n_off,
                      double* S, double* trig_out, double* norm_out) {
    return orc_score_segment_variant(K, dtype, pos, N, d, theta, t, M, phi, R, G, offsets, n_off, 0, S, trig_out,
                                     norm_out);
}

int orc_score_segment_variant(const void* K, int dtype, const int32_t* pos, int64_t N, int d,
                              double theta, int64_t t, const float* M, const float* phi,
                              const float* R, int G, const int64_t* offsets, int n_off, int variant,
                              double* S, double* trig_out, double* norm_out) {
    if (d <= 0 || (d & 1) || G <= 0 || n_off <= 0 || N < 0) return -1;
    if ((variant & ~15) || ((variant & ORC_VAR_TRIG_ONLY) && (variant & ORC_VAR_NORM_ONLY))) return -1;
    const int F = d / 2;
    double* w = (double*)malloc(sizeof(double) * F);
    double* mag = (double*)malloc(sizeof(double) * F);
    double* psi = (double*)malloc(sizeof(double) * F);
    if (!w || !mag || !psi) {
        free(w); free(mag); free(psi);
        return -1;
    }
    for (int f = 0; f < F; ++f) w[f] = pow(theta, -2.0 * (double)f / (double)d);

    for (int64_t i = 0; i < N; ++i) {
        const double p = (double)pos[i];
        /* step 1 */
        for (int f = 0; f < F; ++f) {
            const double re = stored_value(K, dtype, i * d + f);
            const double im = stored_value(K, dtype, i * d + f + F);
            mag[f] = hypot(re, im);
            psi[f] = atan2(im, re) - w[f] * p;
        }
        for (int h = 0; h < G; ++h) {
            const float* Mh = M + (int64_t)h * F;
            const float* ph = phi + (int64_t)h * F;
            const float* Rh = R + (int64_t)h * F;
            /* step 2: brute force over every offset and band */
            double trig = 0.0;
            for (int o = 0; o < n_off; ++o) {
                const double delta = (double)(t + offsets[o]) - p;
                for (int f = 0; f < F; ++f) {
                    const double c = (variant & ORC_VAR_R_WEIGHTED_TRIG) ? (double)Rh[f] * (double)Mh[f] : (double)Mh[f];
                    trig += c * mag[f] * cos(w[f] * delta + (double)ph[f] - psi[f]);
                }
            }
            trig /= (double)n_off;
            /* step 3 */
            double norm = 0.0;
            for (int f = 0; f < F; ++f) {
                const double wt = (variant & ORC_VAR_FIXED_WEIGHT) ? 1.0 : 1.0 - (double)Rh[f];
                norm += wt * (double)Mh[f] * mag[f];
            }
            if (variant & ORC_VAR_TRIG_ONLY) norm = 0.0;
            if (variant & ORC_VAR_NORM_ONLY) trig = 0.0;
            /* step 4 */
            S[(int64_t)h * N + i] = trig + norm;
            if (trig_out) trig_out[(int64_t)h * N + i] = trig;
            if (norm_out) norm_out[(int64_t)h * N + i] = norm;
        }
    }
    free(w); free(mag); free(psi);
    return 0;
}

/*
 * GQA aggregation ([YY] 主要方法, paragraph on GQA): z-score the scores inside
 * each query head, then take the maximum over the query heads that share the
 * KV head, so that heads are comparable.
 * Readings: population mean/standard deviation over all N keys of the segment
 * (two passes); a head whose scores are all equal (sigma = 0) contributes z = 0.
 * S: [G][N]; mu, sigma: [G] outputs; A: [N] output.
 */
int orc_zscore_max(const double* S, int G, int64_t N, double* mu, double* sigma, double* A) {
    if (G <= 0 || N < 0) return -1;
    for (int h = 0; h < G; ++h) {
        const double* Sh = S + (int64_t)h * N;
        /* mean = x0 + mean(x - x0): the same number, but a head whose scores are
         * all equal gets that value back exactly, so its spread is exactly 0 */
        const double x0 = N > 0 ? Sh[0] : 0.0;
        double sum = 0.0;
        for (int64_t i = 0; i < N; ++i) sum += Sh[i] - x0;
        const double m = N > 0 ? x0 + sum / (double)N : 0.0;
        double ss = 0.0;
        for (int64_t i = 0; i < N; ++i) ss += (Sh[i] - m) * (Sh[i] - m);
        mu[h] = m;
        sigma[h] = N > 0 ? sqrt(ss / (double)N) : 0.0;
    }
    for (int64_t i = 0; i < N; ++i) {
        double best = -INFINITY;
        for (int h = 0; h < G; ++h) {
            const double z = sigma[h] > 0.0 ? (S[(int64_t)h * N + i] - mu[h]) / sigma[h] : 0.0;
            if (z > best) best = z;
        }
        A[i] = best;
    }
    return 0;
}

typedef struct {
    double a;
    int32_t pos;
    int32_t slot;
} ranked_key;

/* Higher aggregated score first; among equal scores the earlier position
 * first, and among equal positions the lower slot. */
static int by_score_then_position(const void* x, const void* y) {
    const ranked_key* p = (const ranked_key*)x;
    const ranked_key* q = (const ranked_key*)y;
    if (p->a > q->a) return -1;
    if (p->a < q->a) return 1;
    if (p->pos != q->pos) return p->pos < q->pos ? -1 : 1;
    return (p->slot > q->slot) - (p->slot < q->slot);
}

static int ascending_i32(const void* x, const void* y) {
    const int32_t a = *(const int32_t*)x, b = *(const int32_t*)y;
    return (a > b) - (a < b);
}

/*
 * Budgeted selection ([YY] 主要方法, paragraph on windowed batch pruning): when
 * the segment holds more than B keys keep only the B best by aggregated score;
 * otherwise keep everything.  Reading: among keys whose scores tie at the cut,
 * the earlier position (the key generated first) is kept; keys that share a
 * position as well go by lower slot.  pos: [N] positions of the slots, or
 * NULL when slot order is position order.  The kept slots are returned in
 * ascending order.
 * A: [N]; idx: [min(N,B)] output; *n_kept = min(N, B).
 */
int orc_select_topb(const double* A, const int32_t* pos, int64_t N, int64_t B, int32_t* idx, int64_t* n_kept) {
    if (B <= 0 || N < 0) return -1;
    if (N <= B) {
        for (int64_t i = 0; i < N; ++i) idx[i] = (int32_t)i;
        *n_kept = N;
        return 0;
    }
    ranked_key* r = (ranked_key*)malloc(sizeof(ranked_key) * (size_t)N);
    if (!r) return -1;
    for (int64_t i = 0; i < N; ++i) {
        r[i].a = A[i];
        r[i].pos = pos ? pos[i] : (int32_t)i;
        r[i].slot = (int32_t)i;
    }
    qsort(r, (size_t)N, sizeof(ranked_key), by_score_then_position);
    for (int64_t j = 0; j < B; ++j) idx[j] = r[j].slot;
    qsort(idx, (size_t)B, sizeof(int32_t), ascending_i32);
    free(r);
    *n_kept = B;
    return 0;
}

/* Same selection on single-precision scores (widened exactly to double, so
 * -0 and +0 compare equal, as IEEE comparison has them). */
int orc_select_topb_f32(const float* A, const int32_t* pos, int64_t N, int64_t B, int32_t* idx, int64_t* n_kept) {
    if (N < 0) return -1;
    double* a = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    if (!a) return -1;
    for (int64_t i = 0; i < N; ++i) a[i] = (double)A[i];
    const int rc = orc_select_topb(a, pos, N, B, idx, n_kept);
    free(a);
    return rc;
}

/* Compaction: dst row j = src row idx[j], byte for byte, j < n. */
int orc_gather_rows(const void* src, int64_t row_bytes, const int32_t* idx, int64_t n, void* dst) {
    if (row_bytes <= 0 || n < 0) return -1;
    for (int64_t j = 0; j < n; ++j)
        memcpy((char*)dst + j * row_bytes, (const char*)src + (int64_t)idx[j] * row_bytes,
               (size_t)row_bytes);
    return 0;
}

/*
 * Arrangement of a segment pruned in place in the "fill freed slots" mode, a
 * mode a caller asks for explicitly.  The pages fix which keys survive a prune
 * ([YY] 主要方法: keep the top-B keys), not where they sit afterwards; attention
 * and later prunes read each key with its stored position, so any arrangement
 * of the kept rows in slots [0, n_kept) is a valid cache.  The default
 * arrangement, in place or not, is slot order (the gather above).  In this
 * mode a kept key already below n_kept stays in its slot, and the kept keys at
 * or above n_kept fill the freed slots below n_kept, the lowest such key
 * going to the lowest freed slot, and so on.
 * kept: the kept slots in ascending order, n of them, all < N.
 * src_of: [n] output; slot j of the pruned segment holds the key that was in
 * slot src_of[j] before the prune.
 */
int orc_fill_freed_layout(const int32_t* kept, int64_t n, int64_t N, int32_t* src_of) {
    if (n < 0 || n > N) return -1;
    for (int64_t i = 0; i < n; ++i)
        if (kept[i] < 0 || kept[i] >= N || (i > 0 && kept[i] <= kept[i - 1])) return -1;
    char* is_kept = (char*)calloc((size_t)(N > 0 ? N : 1), 1);
    if (!is_kept) return -1;
    for (int64_t i = 0; i < n; ++i) is_kept[kept[i]] = 1;
    int64_t next_mover = 0;                       /* first kept entry at or above n */
    while (next_mover < n && kept[next_mover] < n) ++next_mover;
    for (int64_t j = 0; j < n; ++j) {
        if (is_kept[j]) src_of[j] = (int32_t)j;   /* stays where it is */
        else src_of[j] = kept[next_mover++];      /* freed slot: next key from above */
    }
    free(is_kept);
    return next_mover == n ? 0 : -1;
}

/* A paged segment read out in slot order: slot i lives in row (i % page_size)
 * of page page_table[i / page_size] of the pool. */
int orc_paged_rows(const void* pool, int64_t row_bytes, const int32_t* page_table,
                   int page_size, int64_t n, void* dst) {
    if (row_bytes <= 0 || page_size <= 0 || n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t page = page_table[i / page_size];
        const int64_t row = page * page_size + i % page_size;
        memcpy((char*)dst + i * row_bytes, (const char*)pool + row * row_bytes, (size_t)row_bytes);
    }
    return 0;
}

/*
 * Single-query decode attention over a (pruned) cache for the G query heads
 * that share one KV head: out_h = sum_i softmax_i(scale * q_h . k_i) v_i.
 * The pages describe decode as re-attending to the whole cache for every new
 * token ([ZN] 长推理的内存困境); this is that textbook softmax attention.
 * q: [G][d] stored; K, V: [N][d] stored; out: [G][d] (fp64).
 */
int orc_decode_attn(const void* q, int q_dtype, const void* K, const void* V, int kv_dtype,
                    int64_t N, int d, int G, double scale, double* out) {
    if (d <= 0 || G <= 0 || N <= 0) return -1;
    double* logit = (double*)malloc(sizeof(double) * (size_t)N);
    if (!logit) return -1;
    for (int h = 0; h < G; ++h) {
        double mx = -INFINITY;
        for (int64_t i = 0; i < N; ++i) {
            double dot = 0.0;
            for (int e = 0; e < d; ++e)
                dot += stored_value(q, q_dtype, (int64_t)h * d + e) * stored_value(K, kv_dtype, i * d + e);
            logit[i] = scale * dot;
            if (logit[i] > mx) mx = logit[i];
        }
        double den = 0.0;
        for (int64_t i = 0; i < N; ++i) {
            logit[i] = exp(logit[i] - mx);
            den += logit[i];
        }
        for (int e = 0; e < d; ++e) {
            double acc = 0.0;
            for (int64_t i = 0; i < N; ++i) acc += logit[i] * stored_value(V, kv_dtype, i * d + e);
            out[(int64_t)h * d + e] = acc / den;
        }
    }
    free(logit);
    return 0;
}

/*
 * Offline calibration of one query head from sampled pre-RoPE queries
 * ([YY] 主要方法: pre-RoPE queries gather around fixed non-zero centres, and
 * the concentration of a band is the mean resultant length R, closer to 1
 * meaning more concentrated directions).  Band f of a sample is the complex
 * number q[f] + i q[f+F]; over the n samples:
 *   M[f]   = mean of |q_f|                       (centre magnitude)
 *   phi[f] = arg of the sum of q_f               (centre phase; 0 when the sum is 0)
 *   R[f]   = | mean of q_f / |q_f| |             (mean resultant length; a sample
 *                                                 with q_f = 0 adds a zero vector)
 * q: [n][d] stored rows; M, phi, R: [F] outputs.  Returns 0, or -1 on bad arguments.
 */
int orc_calibrate(const void* q, int dtype, int64_t n, int d, double* M, double* phi, double* R) {
    if (!q || n <= 0 || d <= 0 || (d & 1) || !M || !phi || !R) return -1;
    const int F = d / 2;
    for (int f = 0; f < F; ++f) {
        double mag = 0.0, sre = 0.0, sim = 0.0, ure = 0.0, uim = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            const double re = stored_value(q, dtype, i * d + f);
            const double im = stored_value(q, dtype, i * d + f + F);
            const double r = hypot(re, im);
            mag += r;
            sre += re;
            sim += im;
            if (r > 0.0) {
                ure += re / r;
                uim += im / r;
            }
        }
        M[f] = mag / (double)n;
        phi[f] = (sre == 0.0 && sim == 0.0) ? 0.0 : atan2(sim, sre);
        R[f] = hypot(ure, uim) / (double)n;
    }
    return 0;
}
