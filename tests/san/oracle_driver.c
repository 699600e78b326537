/*
 * Host sanitizer driver for the fp64 oracle (oracle/gdn_oracle.c): built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py
 * and run on small inputs that reach every branch the oracle has -- empty and
 * one-token sequences, ragged chunk tails, GQA groups, d_k != d_v, conv with
 * and without bias and history, decode with skipped slots.  Exits non-zero
 * when a result is not finite or the chunked form disagrees with the
 * step-by-step one; the sanitizers abort on any invalid access or undefined
 * operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct {
    int64_t num_seqs, total_tokens, h_k, h_v, d_k, d_v, conv_width, qk_l2norm;
    double l2_eps, scale;
} gdn_oracle_dims;

int gdn_oracle_prologue(const gdn_oracle_dims* d, const int64_t* cu, const double* q_raw, const double* k_raw,
                        const double* v_raw, const double* conv_w, const double* conv_b,
                        const double* conv_state_in, double* conv_state_out, double* q_out, double* k_out,
                        double* v_out, int nthreads);
int gdn_oracle_recurrent(const gdn_oracle_dims* d, const int64_t* cu, const double* q, const double* k,
                         const double* v, const double* g, const double* beta, const double* initial_state,
                         double* o, double* final_state, int nthreads);
int gdn_oracle_chunked(const gdn_oracle_dims* d, const int64_t* cu, int64_t chunk, const double* q, const double* k,
                       const double* v, const double* g, const double* beta, const double* initial_state,
                       double* o, double* final_state, int nthreads);
int gdn_oracle_decode(const gdn_oracle_dims* d, const double* q_raw, const double* k_raw, const double* v_raw,
                      const double* g, const double* beta, const double* conv_w, const double* conv_b,
                      double* conv_state_pool, double* state_pool, const int64_t* state_indices, double* o,
                      int nthreads);

static uint64_t rng = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in (-1, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return ((double)(rng >> 11) / 9007199254740992.0) * 2.0 - 1.0;
}
static double* arr(size_t n, double scale) {
    double* a = malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; i++) a[i] = scale * urand();
    return a;
}
static int all_finite(const double* a, size_t n) {
    for (size_t i = 0; i < n; i++)
        if (!isfinite(a[i])) return 0;
    return 1;
}

static int run_prefill(int64_t hk, int64_t hv, int64_t dk, int64_t dvv, const int64_t* lens, int64_t N,
                       int conv, int bias, int hist, int init) {
    int64_t cu[16];
    cu[0] = 0;
    for (int64_t n = 0; n < N; n++) cu[n + 1] = cu[n] + lens[n];
    const int64_t T = cu[N], C = 2 * hk * dk + hv * dvv;
    gdn_oracle_dims d = {N, T, hk, hv, dk, dvv, conv ? 4 : 0, 1, 1e-6, 1.0 / sqrt((double)dk)};
    double *qr = arr(T * hk * dk, 1), *kr = arr(T * hk * dk, 1), *vr = arr(T * hv * dvv, 1);
    double *g = arr(T * hv, 1), *b = arr(T * hv, 0.5);
    for (int64_t i = 0; i < T * hv; i++) { g[i] = -fabs(g[i]); b[i] = 0.5 + b[i]; }
    double *w = arr(C * 4, 0.5), *cb = arr(C, 0.1), *csi = arr(N * C * 3, 1), *cso = arr(N * C * 3, 0);
    double *q = arr(T * hk * dk, 0), *k = arr(T * hk * dk, 0), *v = arr(T * hv * dvv, 0);
    double *h0 = arr(N * hv * dk * dvv, 0.02);
    double *o1 = arr(T * hv * dvv, 0), *f1 = arr(N * hv * dk * dvv, 0);
    double *o2 = arr(T * hv * dvv, 0), *f2 = arr(N * hv * dk * dvv, 0);
    int bad = 0;
    bad |= gdn_oracle_prologue(&d, cu, qr, kr, vr, conv ? w : NULL, (conv && bias) ? cb : NULL,
                               (conv && hist) ? csi : NULL, conv ? cso : NULL, q, k, v, 2) != 0;
    bad |= gdn_oracle_recurrent(&d, cu, q, k, v, g, b, init ? h0 : NULL, o1, f1, 2) != 0;
    for (int64_t chunk = 1; chunk <= 70; chunk += 23) {
        bad |= gdn_oracle_chunked(&d, cu, chunk, q, k, v, g, b, init ? h0 : NULL, o2, f2, 2) != 0;
        double err = 0.0, ref = 1e-300;
        for (int64_t i = 0; i < T * hv * dvv; i++) { err = fmax(err, fabs(o1[i] - o2[i])); ref = fmax(ref, fabs(o1[i])); }
        for (int64_t i = 0; i < N * hv * dk * dvv; i++) { err = fmax(err, fabs(f1[i] - f2[i])); ref = fmax(ref, fabs(f1[i])); }
        if (err > 1e-9 * ref) { fprintf(stderr, "chunked %lld differs: %g\n", (long long)chunk, err / ref); bad = 1; }
    }
    bad |= !all_finite(o1, T * hv * dvv) || !all_finite(f1, N * hv * dk * dvv) || (conv && !all_finite(cso, N * C * 3));
    free(qr); free(kr); free(vr); free(g); free(b); free(w); free(cb); free(csi); free(cso);
    free(q); free(k); free(v); free(h0); free(o1); free(f1); free(o2); free(f2);
    return bad;
}

static int run_decode(int64_t hk, int64_t hv, int64_t dk, int64_t dvv, int conv) {
    const int64_t N = 4, P = 6, C = 2 * hk * dk + hv * dvv;
    const int64_t idx[4] = {5, -1, 0, 3};
    gdn_oracle_dims d = {N, N, hk, hv, dk, dvv, conv ? 4 : 0, 1, 1e-6, 1.0 / sqrt((double)dk)};
    double *q = arr(N * hk * dk, 1), *k = arr(N * hk * dk, 1), *v = arr(N * hv * dvv, 1);
    double *g = arr(N * hv, 1), *b = arr(N * hv, 0.5);
    for (int64_t i = 0; i < N * hv; i++) { g[i] = -fabs(g[i]); b[i] = 0.5 + b[i]; }
    double *w = arr(C * 4, 0.5), *cpool = arr(P * C * 3, 1), *pool = arr(P * hv * dk * dvv, 0.02);
    double* o = arr(N * hv * dvv, 0);
    int bad = gdn_oracle_decode(&d, q, k, v, g, b, conv ? w : NULL, NULL, conv ? cpool : NULL, pool, idx, o, 2) != 0;
    bad |= !all_finite(o, N * hv * dvv) || !all_finite(pool, P * hv * dk * dvv);
    free(q); free(k); free(v); free(g); free(b); free(w); free(cpool); free(pool); free(o);
    return bad;
}

int main(void) {
    const int64_t lens_a[5] = {0, 1, 63, 130, 3};
    const int64_t lens_b[3] = {64, 0, 65};
    int bad = 0;
    bad |= run_prefill(2, 4, 16, 16, lens_a, 5, 1, 1, 1, 1);
    bad |= run_prefill(1, 3, 8, 24, lens_b, 3, 1, 0, 0, 0);
    bad |= run_prefill(2, 2, 24, 8, lens_a, 5, 0, 0, 0, 1);
    bad |= run_decode(2, 4, 16, 16, 1);
    bad |= run_decode(1, 2, 8, 24, 0);
    printf(bad ? "oracle driver: FAILED\n" : "oracle driver: ok\n");
    return bad;
}
