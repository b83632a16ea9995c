/*
 * The C oracle (oracle/gdn_oracle.c) under AddressSanitizer and UndefinedBehaviorSanitizer, on
 * small packed problems that reach every branch: empty and one-token sequences, NULL h0 and hT,
 * a subset of heads. Checks that chained decode steps reproduce the forward pass, and the
 * closed form with beta = 0 (the state only decays: S_T = prod(alpha) h0, o_t = S_t q_t).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdn_oracle_forward(const double *q, const double *k, const double *v, const double *g,
                       const double *beta, const double *h0, double *o, double *hT,
                       const int64_t *seg, int N, int H, int dk, int dv, const int32_t *heads, int nh);
int gdn_oracle_decode(double *state, const double *q, const double *k, const double *v,
                      const double *g, const double *beta, double *o, long NH, int dk, int dv);

static uint64_t rs = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in [0, 1) */
    rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17;
    return (double)(rs >> 11) / 9007199254740992.0;
}
static double nrand(void) { return sqrt(-2.0 * log(urand() + 1e-300)) * cos(6.283185307179586 * urand()); }

static int fail = 0;
static void check(const char *what, double got, double want, double tol) {
    if (!(fabs(got - want) <= tol * (1.0 + fabs(want)))) {
        fprintf(stderr, "%s: got %.17g want %.17g\n", what, got, want);
        fail = 1;
    }
}

int main(void) {
    enum { N = 5, H = 3, DK = 8, DV = 5 };
    const int64_t lens[N] = {7, 0, 1, 70, 3};
    int64_t seg[N + 1] = {0};
    for (int n = 0; n < N; ++n) seg[n + 1] = seg[n] + lens[n];
    const long T = seg[N];
    double *q = malloc(sizeof(double) * T * H * DK), *k = malloc(sizeof(double) * T * H * DK);
    double *v = malloc(sizeof(double) * T * H * DV), *g = malloc(sizeof(double) * T * H);
    double *b = malloc(sizeof(double) * T * H), *b0 = calloc((size_t)T * H, sizeof(double));
    double *h0 = malloc(sizeof(double) * N * H * DV * DK);
    double *o = malloc(sizeof(double) * T * H * DV), *hT = malloc(sizeof(double) * N * H * DV * DK);
    for (long i = 0; i < T * H * DK; ++i) { q[i] = nrand() / sqrt(DK); k[i] = nrand() / sqrt(DK); }
    for (long i = 0; i < T * H * DV; ++i) v[i] = nrand();
    for (long i = 0; i < T * H; ++i) { g[i] = -log1p(exp(nrand())) * 0.1; b[i] = 2.0 / (1.0 + exp(-nrand())); }
    for (long i = 0; i < N * H * DV * DK; ++i) h0[i] = nrand();

    /* forward with h0, all heads */
    gdn_oracle_forward(q, k, v, g, b, h0, o, hT, seg, N, H, DK, DV, NULL, 0);
    /* chained decode steps, one sequence-head pair at a time */
    for (int n = 0; n < N; ++n)
        for (int h = 0; h < H; ++h) {
            double S[DV * DK], od[DV];
            memcpy(S, h0 + ((size_t)n * H + h) * DV * DK, sizeof S);
            for (int64_t t = seg[n]; t < seg[n + 1]; ++t) {
                const size_t th = (size_t)t * H + h;
                gdn_oracle_decode(S, q + th * DK, k + th * DK, v + th * DV, g + th, b + th, od, 1, DK, DV);
                for (int c = 0; c < DV; ++c) check("decode o", od[c], o[th * DV + c], 1e-12);
            }
            for (int e = 0; e < DV * DK; ++e) check("decode state", S[e], hT[((size_t)n * H + h) * DV * DK + e], 1e-12);
        }

    /* beta = 0: S_t = alpha_t S_{t-1}; heads 2 and 0 only, NULL hT elsewhere left untouched */
    const int32_t heads[2] = {2, 0};
    for (long i = 0; i < T * H * DV; ++i) o[i] = NAN;
    gdn_oracle_forward(q, k, v, g, b0, h0, o, hT, seg, N, H, DK, DV, heads, 2);
    for (int n = 0; n < N; ++n)
        for (int hi = 0; hi < 2; ++hi) {
            const int h = heads[hi];
            double decay = 1.0;
            for (int64_t t = seg[n]; t < seg[n + 1]; ++t) {
                const size_t th = (size_t)t * H + h;
                decay *= exp(g[th]);
                for (int c = 0; c < DV; ++c) {
                    double want = 0.0;
                    for (int j = 0; j < DK; ++j) want += decay * h0[(((size_t)n * H + h) * DV + c) * DK + j] * q[th * DK + j];
                    check("beta=0 o", o[th * DV + c], want, 1e-12);
                }
            }
            for (int e = 0; e < DV * DK; ++e)
                check("beta=0 hT", hT[((size_t)n * H + h) * DV * DK + e], decay * h0[((size_t)n * H + h) * DV * DK + e], 1e-12);
        }
    /* NULL h0 and hT */
    gdn_oracle_forward(q, k, v, g, b, NULL, o, NULL, seg, N, H, DK, DV, NULL, 0);
    for (long i = 0; i < T * H * DV; ++i)
        if (!isfinite(o[i])) { fprintf(stderr, "non-finite o\n"); fail = 1; break; }

    free(q); free(k); free(v); free(g); free(b); free(b0); free(h0); free(o); free(hT);
    if (!fail) printf("oracle driver: all checks passed\n");
    return fail;
}
