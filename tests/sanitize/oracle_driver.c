/* Runs every function of the fp64 oracle once on small ragged shapes, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer: any out-of-bounds access, use of
 * freed memory or undefined operation aborts with a report.  Values are only checked
 * for finiteness; the oracle's numerics are pinned by the Python tests. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "hf_oracle.h"

static uint64_t rng_state = 88172645463325252ull;
static double rnd(void) {   /* xorshift64, uniform in [-1, 1) */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double *fill(int64_t n) {
    double *p = (double *)malloc((size_t)n * sizeof(double));
    for (int64_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
}
static double *zeros(int64_t n) { return (double *)calloc((size_t)n, sizeof(double)); }
static int finite_all(const double *p, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}
#define CHECK(cond, what)                                  \
    do {                                                   \
        if (!(cond)) {                                     \
            fprintf(stderr, "oracle driver: %s\n", what);  \
            return 1;                                      \
        }                                                  \
    } while (0)

int main(void) {
    /* 2 planes, 40 queries (blocks of 16: ragged), 72 keys (blocks of 16: ragged), D 8,
     * frames of 24 tokens (so blocks straddle frames) */
    const int64_t BH = 2, Nq = 40, Nk = 72, D = 8, bq = 16, bk = 16, T = 24;
    const int64_t nqb = (Nq + bq - 1) / bq, nkb = (Nk + bk - 1) / bk, k = 3;
    hfo_set_num_threads(2);
    CHECK(hfo_num_threads() >= 1, "threads");
    CHECK(fabs(hfo_phi(0.5) - 1.5) < 1e-15 && hfo_phi(-1.0) > 0.0, "phi");

    double *Q = fill(BH * Nq * D), *K = fill(BH * Nk * D), *V = fill(BH * Nk * D);
    double *qbar = zeros(BH * nqb * D), *kbar = zeros(BH * nkb * D), *s = zeros(BH * nqb * nkb);
    int32_t *idx = (int32_t *)calloc((size_t)(BH * nqb * k), sizeof(int32_t));
    hfo_pool(BH, Nq, D, bq, Q, qbar);
    hfo_pool(BH, Nk, D, bk, K, kbar);
    hfo_block_scores(BH, nqb, nkb, D, qbar, kbar, s);
    hfo_select(BH, nqb, nkb, k, s, idx);
    for (int64_t i = 0; i < BH * nqb * k; ++i) CHECK(idx[i] >= 0 && idx[i] < nkb, "idx range");

    double *out = zeros(BH * Nq * D), *out2 = zeros(BH * Nq * D);
    hfo_sparse_attn(BH, Nq, Nk, D, bq, bk, k, Q, K, V, idx, NULL, 0, out);
    const int64_t blocks[4] = {0, nqb - 1, 1, 0};
    hfo_sparse_attn(BH, Nq, Nk, D, bq, bk, k, Q, K, V, idx, blocks, 2, out2);
    hfo_sparse_attn_rope(BH, Nq, Nk, D, bq, bk, k, T, 4, 1, 10000.0, Q, K, V, idx, NULL, 0, out2);
    CHECK(finite_all(out, BH * Nq * D) && finite_all(out2, BH * Nq * D), "attention finite");

    double *S = zeros(BH * D * D), *z = zeros(BH * D);
    hfo_absorb(BH, Nk, D, K, V, S, z);
    double *r = zeros(BH * Nq * D);
    hfo_linear_readout(BH, Nq, D, bq, Q, S, z, 1e-6, NULL, 0, r);
    hfo_linear_readout(BH, Nq, D, bq, Q, S, z, 1e-6, blocks, 2, r);
    CHECK(finite_all(S, BH * D * D) && finite_all(r, BH * Nq * D), "readout finite");

    int32_t *idx2 = (int32_t *)calloc((size_t)(BH * nqb * k), sizeof(int32_t));
    double *step = zeros(BH * Nq * D), *sc = zeros(BH * nqb * nkb);
    hfo_hybrid_step(BH, Nq, Nk, D, bq, bk, k, 1e-6, Q, K, V, S, z, NULL, 0, idx2, sc, step);
    hfo_hybrid_step(BH, Nq, Nk, D, bq, bk, k, 1e-6, Q, K, V, S, z, blocks, 2, idx2, NULL, step);
    CHECK(finite_all(step, BH * Nq * D), "step finite");

    double *dO = fill(BH * Nq * D), *dQ = zeros(BH * Nq * D), *dK = zeros(BH * Nk * D), *dV = zeros(BH * Nk * D);
    double *dS = zeros(BH * D * D), *dz = zeros(BH * D);
    hfo_sparse_attn_bwd(BH, Nq, Nk, D, bq, bk, k, Q, K, V, idx, dO, dQ, dK, dV);
    hfo_linear_readout_bwd(BH, Nq, D, Q, S, z, 1e-6, dO, dQ, dS, dz);
    hfo_absorb_bwd(BH, Nk, D, K, V, dS, dz, dK, dV);
    CHECK(finite_all(dQ, BH * Nq * D) && finite_all(dK, BH * Nk * D) && finite_all(dV, BH * Nk * D), "grads finite");

    free(Q); free(K); free(V); free(qbar); free(kbar); free(s); free(idx); free(out); free(out2);
    free(S); free(z); free(r); free(idx2); free(step); free(sc); free(dO); free(dQ); free(dK); free(dV);
    free(dS); free(dz);
    puts("oracle driver: ok");
    return 0;
}
