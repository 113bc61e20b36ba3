/*
 * hf_oracle.c -- plain fp64 CPU oracle of the Hybrid Forcing hybrid attention step.
 *
 * TEST INFRASTRUCTURE ONLY (see hf_oracle.h).  Straight loops in double precision,
 * one plane or one query block at a time; OpenMP only distributes independent
 * planes / blocks over threads and never changes any summation order.
 */
#include "hf_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

double hfo_phi(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

int hfo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void hfo_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------- pooling */

void hfo_pool(int64_t BH, int64_t N, int64_t D, int64_t blk, const double *X, double *out) {
    const int64_t nb = ceil_div(N, blk);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t p = 0; p < BH; ++p) {
        for (int64_t b = 0; b < nb; ++b) {
            const int64_t t0 = b * blk, t1 = min64(t0 + blk, N);
            double *o = out + (p * nb + b) * D;
            for (int64_t d = 0; d < D; ++d) {
                double sum = 0.0;
                for (int64_t t = t0; t < t1; ++t) sum += X[(p * N + t) * D + d];
                o[d] = sum / (double)(t1 - t0);
            }
        }
    }
}

/* ---------------------------------------------------------------- scores */

void hfo_block_scores(int64_t BH, int64_t nqb, int64_t nkb, int64_t D,
                      const double *qbar, const double *kbar, double *s) {
    const double scale = 1.0 / sqrt((double)D);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t p = 0; p < BH; ++p) {
        for (int64_t i = 0; i < nqb; ++i) {
            const double *q = qbar + (p * nqb + i) * D;
            for (int64_t j = 0; j < nkb; ++j) {
                const double *kk = kbar + (p * nkb + j) * D;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += q[d] * kk[d];
                s[(p * nqb + i) * nkb + j] = dot * scale;
            }
        }
    }
}

/* ---------------------------------------------------------------- selection */

typedef struct {
    double s;
    int32_t j;
} scored_block;

/* Strict total order: higher score first, then lower block index. */
static int by_score_then_index(const void *pa, const void *pb) {
    const scored_block *a = (const scored_block *)pa, *b = (const scored_block *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

static int by_int(const void *pa, const void *pb) {
    const int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

void hfo_select(int64_t BH, int64_t nqb, int64_t nkb, int64_t k, const double *s, int32_t *idx) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t p = 0; p < BH; ++p) {
        for (int64_t i = 0; i < nqb; ++i) {
            scored_block *row = (scored_block *)malloc((size_t)nkb * sizeof(scored_block));
            for (int64_t j = 0; j < nkb; ++j) {
                row[j].s = s[(p * nqb + i) * nkb + j];
                row[j].j = (int32_t)j;
            }
            qsort(row, (size_t)nkb, sizeof(scored_block), by_score_then_index);
            int32_t *o = idx + (p * nqb + i) * k;
            for (int64_t r = 0; r < k; ++r) o[r] = row[r].j;
            qsort(o, (size_t)k, sizeof(int32_t), by_int);
            free(row);
        }
    }
}

/* ---------------------------------------------------------------- sparse attention */

/* One query block: softmax over the union of its kept key blocks. */
/* Relative temporal rotary embedding of the softmax branch ([HF-de] §2.C "Relative
 * RoPE", [HF-pt] §2.B.2): the temporal position index is capped and taken as an offset
 * between frames.  Reading: a query of window frame fq scored against a key of window
 * frame fk sees the query rotated by the offset delta = clamp(fq - fk, -cap, cap), so
 * the score is the standard rotary one whenever |fq - fk| <= cap.  Feature pair
 * (2i, 2i+1), i < DT/2, turns by the angle delta * base^(-2i/DT); features DT.. D-1
 * (the spatial part) are left as they are. */
typedef struct {
    int64_t T;       /* tokens per frame: window frame of key u is u / T */
    int64_t DT;      /* rotated (temporal) features; 0 = no rotation */
    int64_t cap;
    double base;
} rope_cfg;

static void rope_rotate_query(const double *q, int64_t D, const rope_cfg *rp, int64_t delta, double *qr) {
    for (int64_t d = 0; d < D; ++d) qr[d] = q[d];
    for (int64_t i = 0; i < rp->DT / 2; ++i) {
        const double angle = (double)delta * pow(rp->base, -2.0 * (double)i / (double)rp->DT);
        const double c = cos(angle), s = sin(angle);
        qr[2 * i] = q[2 * i] * c - q[2 * i + 1] * s;
        qr[2 * i + 1] = q[2 * i] * s + q[2 * i + 1] * c;
    }
}

/* One query block.  `rp` NULL: plain scores q . k; else q rotated per key frame as above
 * (query t of the chunk lies in window frame (Nk - Nq + t) / T).  `qr` holds D doubles. */
static void sparse_block(int64_t Nq, int64_t Nk, int64_t D, int64_t bq, int64_t bk, int64_t k,
                         const double *Q, const double *K, const double *V, const int32_t *sel,
                         int64_t i, const rope_cfg *rp, double *out, double *logit, double *qr) {
    const double scale = 1.0 / sqrt((double)D);
    const int64_t t0 = i * bq, t1 = min64(t0 + bq, Nq);
    for (int64_t t = t0; t < t1; ++t) {
        const double *q = Q + t * D;
        int64_t qr_frame = -1;   /* key frame the rotated query in qr was made for */
        /* logits over the kept keys, in kept-block order */
        int64_t n = 0;
        double m = -INFINITY;
        for (int64_t r = 0; r < k; ++r) {
            const int64_t u0 = (int64_t)sel[r] * bk, u1 = min64(u0 + bk, Nk);
            for (int64_t u = u0; u < u1; ++u) {
                const double *qu = q;
                if (rp) {
                    const int64_t fk = u / rp->T;
                    if (fk != qr_frame) {
                        int64_t delta = (Nk - Nq + t) / rp->T - fk;
                        if (delta > rp->cap) delta = rp->cap;
                        if (delta < -rp->cap) delta = -rp->cap;
                        rope_rotate_query(q, D, rp, delta, qr);
                        qr_frame = fk;
                    }
                    qu = qr;
                }
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += qu[d] * K[u * D + d];
                logit[n] = dot * scale;
                if (logit[n] > m) m = logit[n];
                ++n;
            }
        }
        double denom = 0.0;
        for (int64_t e = 0; e < n; ++e) {
            logit[e] = exp(logit[e] - m);
            denom += logit[e];
        }
        double *o = out + t * D;
        for (int64_t c = 0; c < D; ++c) o[c] = 0.0;
        n = 0;
        for (int64_t r = 0; r < k; ++r) {
            const int64_t u0 = (int64_t)sel[r] * bk, u1 = min64(u0 + bk, Nk);
            for (int64_t u = u0; u < u1; ++u) {
                const double w = logit[n++];
                for (int64_t c = 0; c < D; ++c) o[c] += w * V[u * D + c];
            }
        }
        for (int64_t c = 0; c < D; ++c) o[c] /= denom;
    }
}

static void sparse_attn(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, int64_t bq, int64_t bk,
                        int64_t k, const rope_cfg *rp, const double *Q, const double *K, const double *V,
                        const int32_t *idx, const int64_t *blocks, int64_t n_blocks, double *out) {
    const int64_t nqb = ceil_div(Nq, bq);
    const int64_t total = blocks ? n_blocks : BH * nqb;
#pragma omp parallel
    {
        double *logit = (double *)malloc((size_t)(k * bk) * sizeof(double));
        double *qr = (double *)malloc((size_t)D * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t w = 0; w < total; ++w) {
            const int64_t p = blocks ? blocks[2 * w] : w / nqb;
            const int64_t i = blocks ? blocks[2 * w + 1] : w % nqb;
            sparse_block(Nq, Nk, D, bq, bk, k, Q + p * Nq * D, K + p * Nk * D, V + p * Nk * D,
                         idx + (p * nqb + i) * k, i, rp, out + p * Nq * D, logit, qr);
        }
        free(qr);
        free(logit);
    }
}

void hfo_sparse_attn(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, int64_t bq, int64_t bk,
                     int64_t k, const double *Q, const double *K, const double *V,
                     const int32_t *idx, const int64_t *blocks, int64_t n_blocks, double *out) {
    sparse_attn(BH, Nq, Nk, D, bq, bk, k, NULL, Q, K, V, idx, blocks, n_blocks, out);
}

void hfo_sparse_attn_rope(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, int64_t bq, int64_t bk,
                          int64_t k, int64_t T, int64_t DT, int64_t cap, double base, const double *Q,
                          const double *K, const double *V, const int32_t *idx, const int64_t *blocks,
                          int64_t n_blocks, double *out) {
    const rope_cfg rp = {T, DT, cap, base};
    sparse_attn(BH, Nq, Nk, D, bq, bk, k, &rp, Q, K, V, idx, blocks, n_blocks, out);
}

/* ---------------------------------------------------------------- linear branch */

void hfo_linear_readout(int64_t BH, int64_t Nq, int64_t D, int64_t bq, const double *Q,
                        const double *S, const double *z, double eps,
                        const int64_t *blocks, int64_t n_blocks, double *out) {
    const int64_t nqb = ceil_div(Nq, bq);
    const int64_t total = blocks ? n_blocks : BH * nqb;
#pragma omp parallel
    {
        double *a = (double *)malloc((size_t)D * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t w = 0; w < total; ++w) {
            const int64_t p = blocks ? blocks[2 * w] : w / nqb;
            const int64_t i = blocks ? blocks[2 * w + 1] : w % nqb;
            const double *Sp = S + p * D * D, *zp = z + p * D;
            for (int64_t t = i * bq; t < min64((i + 1) * bq, Nq); ++t) {
                const double *q = Q + (p * Nq + t) * D;
                for (int64_t d = 0; d < D; ++d) a[d] = hfo_phi(q[d]);
                double den = 0.0;
                for (int64_t d = 0; d < D; ++d) den += a[d] * zp[d];
                double *o = out + (p * Nq + t) * D;
                for (int64_t c = 0; c < D; ++c) {
                    double num = 0.0;
                    for (int64_t d = 0; d < D; ++d) num += a[d] * Sp[d * D + c];
                    o[c] = num / (den + eps);
                }
            }
        }
        free(a);
    }
}

void hfo_absorb(int64_t BH, int64_t n, int64_t D, const double *K, const double *V,
                double *S, double *z) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t p = 0; p < BH; ++p) {
        for (int64_t a = 0; a < D; ++a) {
            const double *Kp = K + p * n * D, *Vp = V + p * n * D;
            double *Srow = S + (p * D + a) * D;
            double zsum = 0.0;
            for (int64_t u = 0; u < n; ++u) {
                const double f = hfo_phi(Kp[u * D + a]);
                zsum += f;
                for (int64_t c = 0; c < D; ++c) Srow[c] += f * Vp[u * D + c];
            }
            z[p * D + a] += zsum;
        }
    }
}

/* ---------------------------------------------------------------- the step */

void hfo_hybrid_step(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, int64_t bq, int64_t bk,
                     int64_t k, double eps, const double *Q, const double *K, const double *V,
                     const double *S, const double *z, const int64_t *blocks, int64_t n_blocks,
                     int32_t *idx_out, double *scores_out, double *out) {
    const int64_t nqb = ceil_div(Nq, bq), nkb = ceil_div(Nk, bk);
    double *qbar = (double *)malloc((size_t)(BH * nqb * D) * sizeof(double));
    double *kbar = (double *)malloc((size_t)(BH * nkb * D) * sizeof(double));
    double *s = scores_out ? scores_out : (double *)malloc((size_t)(BH * nqb * nkb) * sizeof(double));
    double *lin = (double *)calloc((size_t)(BH * Nq * D), sizeof(double));

    hfo_pool(BH, Nq, D, bq, Q, qbar);
    hfo_pool(BH, Nk, D, bk, K, kbar);
    hfo_block_scores(BH, nqb, nkb, D, qbar, kbar, s);
    hfo_select(BH, nqb, nkb, k, s, idx_out);
    hfo_sparse_attn(BH, Nq, Nk, D, bq, bk, k, Q, K, V, idx_out, blocks, n_blocks, out);
    hfo_linear_readout(BH, Nq, D, bq, Q, S, z, eps, blocks, n_blocks, lin);

    /* sum of the two branches, on the computed query blocks only */
    const int64_t total = blocks ? n_blocks : BH * nqb;
    for (int64_t w = 0; w < total; ++w) {
        const int64_t p = blocks ? blocks[2 * w] : w / nqb;
        const int64_t i = blocks ? blocks[2 * w + 1] : w % nqb;
        for (int64_t t = i * bq; t < min64((i + 1) * bq, Nq); ++t)
            for (int64_t c = 0; c < D; ++c) out[(p * Nq + t) * D + c] += lin[(p * Nq + t) * D + c];
    }

    free(lin);
    if (!scores_out) free(s);
    free(kbar);
    free(qbar);
}

/* ---------------------------------------------------------------- backward */

static double phi_prime(double x) { return x > 0.0 ? 1.0 : exp(x); }

/* One plane, every query in order (dK, dV accumulate over queries, so the plane is the
 * unit of parallel work and the summation order is fixed). */
static void sparse_plane_bwd(int64_t Nq, int64_t Nk, int64_t D, int64_t bq, int64_t bk, int64_t k,
                             const double *Q, const double *K, const double *V, const int32_t *sel_all,
                             const double *dO, double *dQ, double *dK, double *dV, double *P,
                             double *dP, int64_t *key) {
    const double scale = 1.0 / sqrt((double)D);
    const int64_t nqb = ceil_div(Nq, bq);
    for (int64_t t = 0; t < Nq; ++t) {
        const int32_t *sel = sel_all + (t / bq) * k;
        const double *q = Q + t * D, *g = dO + t * D;
        /* the kept keys of t's block, their logits and softmax weights */
        int64_t n = 0;
        double m = -INFINITY;
        for (int64_t r = 0; r < k; ++r) {
            const int64_t u0 = (int64_t)sel[r] * bk, u1 = min64(u0 + bk, Nk);
            for (int64_t u = u0; u < u1; ++u) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += q[d] * K[u * D + d];
                key[n] = u;
                P[n] = dot * scale;
                if (P[n] > m) m = P[n];
                ++n;
            }
        }
        double denom = 0.0;
        for (int64_t e = 0; e < n; ++e) {
            P[e] = exp(P[e] - m);
            denom += P[e];
        }
        for (int64_t e = 0; e < n; ++e) P[e] /= denom;
        /* dP and Delta */
        double delta = 0.0;
        for (int64_t e = 0; e < n; ++e) {
            const double *v = V + key[e] * D;
            double s = 0.0;
            for (int64_t c = 0; c < D; ++c) s += g[c] * v[c];
            dP[e] = s;
            delta += P[e] * s;
        }
        for (int64_t e = 0; e < n; ++e) {
            const int64_t u = key[e];
            const double G = P[e] * (dP[e] - delta);
            for (int64_t d = 0; d < D; ++d) {
                dQ[t * D + d] += G * K[u * D + d] * scale;
                dK[u * D + d] += G * q[d] * scale;
                dV[u * D + d] += P[e] * g[d];
            }
        }
    }
    (void)nqb;
}

void hfo_sparse_attn_bwd(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, int64_t bq, int64_t bk,
                         int64_t k, const double *Q, const double *K, const double *V,
                         const int32_t *idx, const double *dO, double *dQ, double *dK, double *dV) {
    const int64_t nqb = ceil_div(Nq, bq);
#pragma omp parallel
    {
        double *P = (double *)malloc((size_t)(k * bk) * sizeof(double));
        double *dP = (double *)malloc((size_t)(k * bk) * sizeof(double));
        int64_t *key = (int64_t *)malloc((size_t)(k * bk) * sizeof(int64_t));
#pragma omp for schedule(dynamic, 1)
        for (int64_t p = 0; p < BH; ++p)
            sparse_plane_bwd(Nq, Nk, D, bq, bk, k, Q + p * Nq * D, K + p * Nk * D, V + p * Nk * D,
                             idx + p * nqb * k, dO + p * Nq * D, dQ + p * Nq * D, dK + p * Nk * D,
                             dV + p * Nk * D, P, dP, key);
        free(key);
        free(dP);
        free(P);
    }
}

void hfo_linear_readout_bwd(int64_t BH, int64_t Nq, int64_t D, const double *Q, const double *S,
                            const double *z, double eps, const double *dO, double *dQ, double *dS,
                            double *dz) {
#pragma omp parallel
    {
        double *a = (double *)malloc((size_t)D * sizeof(double));
        double *num = (double *)malloc((size_t)D * sizeof(double));
        double *dn = (double *)malloc((size_t)D * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t p = 0; p < BH; ++p) {
            const double *Sp = S + p * D * D, *zp = z + p * D;
            double *dSp = dS + p * D * D, *dzp = dz + p * D;
            for (int64_t t = 0; t < Nq; ++t) {
                const double *q = Q + (p * Nq + t) * D, *g = dO + (p * Nq + t) * D;
                for (int64_t d = 0; d < D; ++d) a[d] = hfo_phi(q[d]);
                double den = eps;
                for (int64_t d = 0; d < D; ++d) den += a[d] * zp[d];
                double gn = 0.0;
                for (int64_t c = 0; c < D; ++c) {
                    double s = 0.0;
                    for (int64_t d = 0; d < D; ++d) s += a[d] * Sp[d * D + c];
                    num[c] = s;
                    gn += g[c] * s;
                }
                const double dden = -gn / (den * den);
                for (int64_t c = 0; c < D; ++c) dn[c] = g[c] / den;
                for (int64_t d = 0; d < D; ++d) {
                    double da = zp[d] * dden;
                    for (int64_t c = 0; c < D; ++c) {
                        da += Sp[d * D + c] * dn[c];
                        dSp[d * D + c] += a[d] * dn[c];
                    }
                    dzp[d] += a[d] * dden;
                    dQ[(p * Nq + t) * D + d] += da * phi_prime(q[d]);
                }
            }
        }
        free(dn);
        free(num);
        free(a);
    }
}

void hfo_absorb_bwd(int64_t BH, int64_t n, int64_t D, const double *K, const double *V,
                    const double *dS, const double *dz, double *dK, double *dV) {
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < BH; ++p) {
        const double *dSp = dS + p * D * D, *dzp = dz + p * D;
        for (int64_t u = 0; u < n; ++u) {
            const double *ku = K + (p * n + u) * D, *vu = V + (p * n + u) * D;
            for (int64_t c = 0; c < D; ++c) {
                double s = 0.0;
                for (int64_t a = 0; a < D; ++a) s += hfo_phi(ku[a]) * dSp[a * D + c];
                dV[(p * n + u) * D + c] += s;
            }
            for (int64_t a = 0; a < D; ++a) {
                double s = dzp[a];
                for (int64_t c = 0; c < D; ++c) s += dSp[a * D + c] * vu[c];
                dK[(p * n + u) * D + a] += s * phi_prime(ku[a]);
            }
        }
    }
}
