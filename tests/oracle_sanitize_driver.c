/*
 * Drives every oracle function on small inputs (edge cases included) so that a
 * build with AddressSanitizer + UndefinedBehaviorSanitizer, or with
 * ThreadSanitizer (-DTHREADS: the same calls from several threads at once, as
 * the Python thread pool makes them), can report memory errors, undefined
 * behaviour or data races.  Test infrastructure: built and run by
 * tests/test_sanitizers.py.  Exit status 0 and "ok" on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#ifdef THREADS
#include <pthread.h>
#endif

int orc_score_segment(const void* K, int dtype, const int32_t* pos, int64_t N, int d, double theta, int64_t t,
                      const float* M, const float* phi, const float* R, int G, const int64_t* offsets, int n_off,
                      double* S, double* trig_out, double* norm_out);
int orc_score_segment_variant(const void* K, int dtype, const int32_t* pos, int64_t N, int d, double theta,
                              int64_t t, const float* M, const float* phi, const float* R, int G,
                              const int64_t* offsets, int n_off, int variant, double* S, double* trig_out,
                              double* norm_out);
int orc_zscore_max(const double* S, int G, int64_t N, double* mu, double* sigma, double* A);
int orc_select_topb(const double* A, const int32_t* pos, int64_t N, int64_t B, int32_t* idx, int64_t* n_kept);
int orc_select_topb_f32(const float* A, const int32_t* pos, int64_t N, int64_t B, int32_t* idx, int64_t* n_kept);
int orc_gather_rows(const void* src, int64_t row_bytes, const int32_t* idx, int64_t n, void* dst);
int orc_fill_freed_layout(const int32_t* kept, int64_t n, int64_t N, int32_t* src_of);
int orc_paged_rows(const void* pool, int64_t row_bytes, const int32_t* page_table, int page_size, int64_t n,
                   void* dst);
int orc_decode_attn(const void* q, int q_dtype, const void* K, const void* V, int kv_dtype, int64_t N, int d, int G,
                    double scale, double* out);
int orc_calibrate(const void* q, int dtype, int64_t n, int d, double* M, double* phi, double* R);

static double urand(uint64_t* st) {              /* xorshift64, [0, 1) */
    *st ^= *st << 13;
    *st ^= *st >> 7;
    *st ^= *st << 17;
    return (double)(*st >> 11) / 9007199254740992.0;
}

#define CHECK(x)                                                     \
    do {                                                             \
        if (!(x)) {                                                  \
            fprintf(stderr, "check failed: %s (line %d)\n", #x, __LINE__); \
            exit(1);                                                 \
        }                                                            \
    } while (0)

/* One segment through every step; returns the number kept. */
static int64_t one_segment(int64_t N, int d, int G, int64_t B, int dtype, unsigned seed) {
    uint64_t rs = 0x9E3779B97F4A7C15ull * (seed + 1);
    uint64_t* st = &rs;
    const int F = d / 2;
    const int64_t offs[3] = {1, 2, 4};
    float* M = malloc(sizeof(float) * G * F);
    float* phi = malloc(sizeof(float) * G * F);
    float* R = malloc(sizeof(float) * G * F);
    for (int i = 0; i < G * F; ++i) {
        M[i] = (float)(0.5 + 1.5 * urand(st));
        phi[i] = (float)(6.28 * urand(st));
        R[i] = (float)(0.3 + 0.69 * urand(st));
    }
    const size_t es = dtype ? 2 : 4;
    void* K = malloc(es * (size_t)(N > 0 ? N : 1) * d);
    void* V = malloc(es * (size_t)(N > 0 ? N : 1) * d);
    int32_t* pos = malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
    for (int64_t i = 0; i < N * d; ++i) {
        const float x = (float)(2.0 * urand(st) - 1.0);
        if (dtype) {
            uint32_t b;
            memcpy(&b, &x, 4);
            ((uint16_t*)K)[i] = (uint16_t)(b >> 16);
            ((uint16_t*)V)[i] = (uint16_t)(b >> 16);
        } else {
            ((float*)K)[i] = x;
            ((float*)V)[i] = -x;
        }
    }
    for (int64_t i = 0; i < N; ++i) pos[i] = (int32_t)((i * 7) % (N > 0 ? N : 1));   /* not in slot order */
    double* S = malloc(sizeof(double) * G * (size_t)(N > 0 ? N : 1));
    double* tr = malloc(sizeof(double) * G * (size_t)(N > 0 ? N : 1));
    double* nr = malloc(sizeof(double) * G * (size_t)(N > 0 ? N : 1));
    double* A = malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double mu[8], sg[8];
    CHECK(orc_score_segment(K, dtype, pos, N, d, 1e4, N, M, phi, R, G, offs, 3, S, tr, nr) == 0);
    for (int v = 1; v <= 8; v <<= 1)
        CHECK(orc_score_segment_variant(K, dtype, pos, N, d, 1e4, N, M, phi, R, G, offs, 3, v, S, NULL, NULL) == 0);
    CHECK(orc_score_segment(K, dtype, pos, N, d, 1e4, N, M, phi, R, G, offs, 3, S, NULL, NULL) == 0);
    CHECK(orc_zscore_max(S, G, N, mu, sg, A) == 0);
    int32_t* idx = malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
    int64_t nk = -1;
    CHECK(orc_select_topb(A, pos, N, B, idx, &nk) == 0);
    CHECK(nk == (N < B ? N : B));
    CHECK(orc_select_topb(A, NULL, N, B, idx, &nk) == 0);
    float* Af = malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
    for (int64_t i = 0; i < N; ++i) Af[i] = (float)floor(A[i]);          /* many ties */
    CHECK(orc_select_topb_f32(Af, pos, N, B, idx, &nk) == 0);
    void* Kd = malloc(es * (size_t)(nk > 0 ? nk : 1) * d);
    CHECK(orc_gather_rows(K, (int64_t)es * d, idx, nk, Kd) == 0);
    int32_t* src_of = malloc(sizeof(int32_t) * (size_t)(nk > 0 ? nk : 1));
    CHECK(orc_fill_freed_layout(idx, nk, N, src_of) == 0);
    if (N > 0) {
        double* out = malloc(sizeof(double) * G * d);
        float* q = malloc(sizeof(float) * G * d);
        for (int i = 0; i < G * d; ++i) q[i] = (float)(urand(st) - 0.5);
        CHECK(orc_decode_attn(q, 0, K, V, dtype, N, d, G, 0.125, out) == 0);
        free(out);
        free(q);
    }
    free(M); free(phi); free(R); free(K); free(V); free(pos); free(S); free(tr); free(nr); free(A);
    free(idx); free(Af); free(Kd); free(src_of);
    return nk;
}

static void edge_cases(void) {
    /* bad arguments are refused without touching memory */
    int32_t kept_bad[2] = {3, 1}, out2[2];
    CHECK(orc_fill_freed_layout(kept_bad, 2, 5, out2) != 0);
    double A1[1] = {1.0};
    int32_t idx1[1];
    int64_t nk;
    CHECK(orc_select_topb(A1, NULL, 1, 0, idx1, &nk) != 0);
    CHECK(orc_score_segment(A1, 0, idx1, 1, 3, 1e4, 0, NULL, NULL, NULL, 1, NULL, 1, NULL, NULL, NULL) != 0);
    /* paged read-out with a page size that does not divide n */
    uint16_t pool[5 * 3 * 4];
    for (int i = 0; i < 60; ++i) pool[i] = (uint16_t)i;
    int32_t pt[3] = {4, 0, 2};
    uint16_t dst[7 * 4];
    CHECK(orc_paged_rows(pool, 8, pt, 3, 7, dst) == 0);
    CHECK(dst[0] == 48 && dst[4 * 6] == 24);
    /* calibration: zero samples, zero rows, bf16 */
    float q[4 * 4] = {0};
    double Mc[2], Pc[2], Rc[2];
    CHECK(orc_calibrate(q, 0, 0, 4, Mc, Pc, Rc) != 0);
    CHECK(orc_calibrate(q, 0, 4, 4, Mc, Pc, Rc) == 0);
    CHECK(Mc[0] == 0.0 && Rc[0] == 0.0 && Pc[0] == 0.0);
    uint16_t qb[3 * 8];
    for (int i = 0; i < 24; ++i) qb[i] = (uint16_t)(0x3f80 + i);
    double Mb[4], Pb[4], Rb[4];
    CHECK(orc_calibrate(qb, 1, 3, 8, Mb, Pb, Rb) == 0);
}

#ifdef THREADS
static void* worker(void* arg) {
    const unsigned id = (unsigned)(uintptr_t)arg;
    for (int r = 0; r < 3; ++r) one_segment(200 + 37 * id, 64, 4, 50, (int)(id & 1), id * 10 + r);
    return NULL;
}
#endif

int main(void) {
    edge_cases();
    const int64_t Ns[] = {0, 1, 2, 5, 64, 300};
    for (int i = 0; i < 6; ++i) {
        one_segment(Ns[i], 64, 4, 3, 0, (unsigned)i);
        one_segment(Ns[i], 128, 8, 64, 1, (unsigned)(i + 10));
        one_segment(Ns[i], 16, 1, 400, 1, (unsigned)(i + 20));
    }
#ifdef THREADS
    pthread_t th[8];
    for (uintptr_t i = 0; i < 8; ++i) CHECK(pthread_create(&th[i], NULL, worker, (void*)i) == 0);
    for (int i = 0; i < 8; ++i) pthread_join(th[i], NULL);
#endif
    printf("ok\n");
    return 0;
}
