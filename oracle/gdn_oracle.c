/*
 * CPU fp64 oracle of the gated delta rule, token by token (C twin of recurrence.py).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the CPU
 * baseline leg of the benchmark may load or run it. It shares no code with the HIP
 * library: no headers, no helpers, no tables.
 *
 * Recurrence, per sequence and head, with state S [d_v][d_k] row-major:
 *     S_t = S_{t-1} . alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
 * (paper note "Gated Delta Networks: Improving Mamba2 with Delta Rule", mechanism
 * paragraph; record "LIT-137", section "Standing in the anthology"). The old memory
 * is decayed first, the delta write follows, and the query reads the updated memory
 * (module page "Gated DeltaNet", sections "How It Works" and "Math Or Compute
 * Schema"). The step is evaluated as alpha S + beta (v - alpha S k) k^T, the product
 * form distributed out.
 *
 * Independent (sequence, head) pairs run in parallel with OpenMP; the token loop of
 * each pair is sequential. No blocking, no reordering of the recurrence.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token on one head. S is updated in place; o receives S_t q_t. */
static void oracle_step(double *S, const double *q, const double *k, const double *v,
                        double g, double beta, double *o, int dk, int dv) {
    const double a = exp(g);
    for (int i = 0; i < dv; ++i) {
        double *row = S + (size_t)i * dk;
        double u = 0.0;
        for (int j = 0; j < dk; ++j) {
            row[j] *= a;                 /* decay the old memory */
            u += row[j] * k[j];          /* what the decayed memory stores under k */
        }
        const double w = beta * (v[i] - u);
        double r = 0.0;
        for (int j = 0; j < dk; ++j) {
            row[j] += w * k[j];          /* delta-rule write along k */
            r += row[j] * q[j];          /* read of the updated memory */
        }
        o[i] = r;
    }
}

/*
 * Forward pass over packed sequences.
 * q, k [Ttot][H][dk]; v [Ttot][H][dv]; g, beta [Ttot][H]; seg [N+1] token offsets;
 * h0 [N][H][dv][dk] or NULL (zeros); o [Ttot][H][dv]; hT [N][H][dv][dk] or NULL.
 * heads: list of nh head indices to process (NULL: all H). Returns the number of
 * OpenMP threads used.
 */
int gdn_oracle_forward(const double *q, const double *k, const double *v, const double *g,
                       const double *beta, const double *h0, double *o, double *hT,
                       const int64_t *seg, int N, int H, int dk, int dv,
                       const int32_t *heads, int nh) {
    if (heads == NULL) nh = H;
    int used = 1;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
#pragma omp for schedule(dynamic, 1)
        for (long p = 0; p < (long)N * nh; ++p) {
            const int n = (int)(p / nh);
            const int h = heads ? heads[p % nh] : (int)(p % nh);
            const size_t sbase = ((size_t)n * H + h) * (size_t)dk * dv;
            if (h0) memcpy(S, h0 + sbase, sizeof(double) * (size_t)dk * dv);
            else memset(S, 0, sizeof(double) * (size_t)dk * dv);
            for (int64_t t = seg[n]; t < seg[n + 1]; ++t) {
                const size_t th = (size_t)t * H + h;
                oracle_step(S, q + th * dk, k + th * dk, v + th * dv, g[th], beta[th],
                            o + th * dv, dk, dv);
            }
            if (hT) memcpy(hT + sbase, S, sizeof(double) * (size_t)dk * dv);
        }
        free(S);
    }
    return used;
}

/*
 * One decode step for every (sequence, head), in place on state [NH][dv][dk];
 * q, k [NH][dk]; v, o [NH][dv]; g, beta [NH]. Returns the threads used.
 */
int gdn_oracle_decode(double *state, const double *q, const double *k, const double *v,
                      const double *g, const double *beta, double *o, long NH, int dk, int dv) {
    int used = 1;
#pragma omp parallel
    {
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
#pragma omp for schedule(static)
        for (long p = 0; p < NH; ++p)
            oracle_step(state + (size_t)p * dk * dv, q + (size_t)p * dk, k + (size_t)p * dk,
                        v + (size_t)p * dv, g[p], beta[p], o + (size_t)p * dv, dk, dv);
    }
    return used;
}
