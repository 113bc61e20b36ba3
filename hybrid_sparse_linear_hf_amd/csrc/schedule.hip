// Chunk-aware growth (CAG) sparsity schedule: host arithmetic only.
//
// [LF-de] §2.1 "Chunk-bewusstes Wachstum": the first chunk of a stream gets dense
// attention and later chunks get progressively sparser; chunk i's sparsity is
// s_i = s_base - alpha_i * beta, alpha_i scales as one over a square root (read here as
// 1 / sqrt(i + 1) of the chunk's position), and beta is set so that the total attention
// work meets a target sparsity.  Work of chunk i = its kept key blocks per query block,
// k_i = ceil((1 - s_i) n_kb[i]) clamped to [1, n_kb[i]]; beta is the smallest value whose
// schedule keeps at least (1 - s_target) of the dense total, found by bisection.
#include <cmath>

#include "hf_internal.h"

#pragma clang fp contract(off)

namespace {

double cag_alpha(int i) { return 1.0 / std::sqrt((double)(i + 1)); }

double cag_sparsity(int i, double s_base, double s_max, double beta) {
    if (i == 0) return 0.0;                    // the first chunk is dense
    const double s = s_base - cag_alpha(i) * beta;
    return std::fmin(std::fmax(s, 0.0), s_max);
}

int cag_keep(double s, int nkb) {
    double k = std::ceil((1.0 - s) * (double)nkb);
    if (k < 1.0) k = 1.0;
    if (k > (double)nkb) k = (double)nkb;
    return (int)k;
}

long long cag_work(int n, const int32_t *nkb, double s_base, double s_max, double beta) {
    long long w = 0;
    for (int i = 0; i < n; ++i) w += cag_keep(cag_sparsity(i, s_base, s_max, beta), nkb[i]);
    return w;
}

}  // namespace

hf_status hf_cag_schedule_impl(int32_t n, const int32_t *nkb, double s_base, double s_target, double s_max,
                               int32_t *top_k, double *sparsity, double *beta_out) {
    double dense = 0.0;
    for (int i = 0; i < n; ++i) dense += (double)nkb[i];
    const double target = (1.0 - s_target) * dense;
    double beta = 0.0;
    if ((double)cag_work(n, nkb, s_base, s_max, 0.0) < target) {
        // at hi every s_i is clamped to 0 (dense), which meets any target
        double lo = 0.0, hi = s_base * std::sqrt((double)n) + 1.0;
        for (int it = 0; it < 200; ++it) {
            const double mid = 0.5 * (lo + hi);
            if (mid <= lo || mid >= hi) break;
            if ((double)cag_work(n, nkb, s_base, s_max, mid) >= target)
                hi = mid;
            else
                lo = mid;
        }
        beta = hi;
    }
    for (int i = 0; i < n; ++i) {
        const double s = cag_sparsity(i, s_base, s_max, beta);
        top_k[i] = cag_keep(s, nkb[i]);
        if (sparsity) sparsity[i] = s;
    }
    if (beta_out) *beta_out = beta;
    return HF_OK;
}
