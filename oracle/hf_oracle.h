/*
 * hf_oracle.h -- plain fp64 CPU oracle of the Hybrid Forcing hybrid attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, obviously-correct reference the
 * HIP library is checked against.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the product path never does.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Sources (web pages on the method; no code exists on them):
 *   [HF-de]  gist.science (German), "Long-Horizon Streaming Video Generation via
 *            Hybrid Attention with Decoupled Distillation", technical summary.
 *   [HF-pt]  gist.science (Portuguese), same paper, technical summary.
 *   [HF-abs] arxivdaily.com page of the same paper, English abstract.
 *   [LF-de]  gist.science (German), "Light Forcing: Accelerating Autoregressive
 *            Video Diffusion via Sparse Attention", technical summary.
 *
 * Layouts: every array is dense row-major fp64.  A "plane" is one (batch, head)
 * pair; BH planes are stored one after another.
 *   Q      [BH][Nq][D]     queries of the current chunk
 *   K, V   [BH][Nk][D]     window keys/values in logical order (oldest frame first;
 *                          the last Nq rows are the current chunk)
 *   S      [BH][D][D]      linear state, S[a][c]
 *   z      [BH][D]         linear normaliser state
 *   idx    [BH][nqb][k]    kept key-block indices per query block, ascending
 *
 * Geometry: query block i holds tokens [i*bq, min((i+1)*bq, Nq)); key block j holds
 * [j*bk, min((j+1)*bk, Nk)).  Blocks run over the concatenated window and may cross
 * frame boundaries; a short last block is pooled over its real tokens only.
 *
 * Parity pins: every function here is pinned by the CPU test-suite (brute force,
 * closed forms, invariants).  What is NOT pinned is agreement with the authors'
 * own implementation: the pages fix neither the feature map, nor epsilon, nor the
 * block-scoring rule, nor the keep rounding; those are readings (see the design
 * notes) -- "parity unpinned" with respect to the authors' code.
 */
#ifndef HF_ORACLE_H
#define HF_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Feature map of the linear branch: phi(x) = elu(x) + 1, i.e. x + 1 for x > 0 and
 * exp(x) otherwise (positive, so the normaliser never vanishes).  The pages name a
 * "linear attention" ([HF-de] §2.A, [HF-pt] §2.A.1) without a feature map; elu+1 is
 * the reading taken. */
double hfo_phi(double x);

/* Mean of each block of `blk` consecutive rows (a short last block averages its real
 * rows only).  X [BH][N][D] -> out [BH][ceil(N/blk)][D].  Token compression by
 * mean pooling as in [LF-de] §2.2 "Token-Kompression". */
void hfo_pool(int64_t BH, int64_t N, int64_t D, int64_t blk, const double *X, double *out);

/* Block importance: s[bh][i][j] = qbar_i . kbar_j / sqrt(D).  [HF-de] §2.A keeps the
 * most important (Top-K) blocks; the importance score is the reading of pooled
 * query-key affinity ([LF-de] §2.2). */
void hfo_block_scores(int64_t BH, int64_t nqb, int64_t nkb, int64_t D,
                      const double *qbar, const double *kbar, double *s);

/* Top-k per query block: order key blocks by score descending, equal scores by
 * lower index first; keep the first k; write them in ascending index order.
 * s [BH][nqb][nkb] -> idx [BH][nqb][k].  Requires 1 <= k <= nkb. */
void hfo_select(int64_t BH, int64_t nqb, int64_t nkb, int64_t k, const double *s, int32_t *idx);

/* Block-sparse softmax attention ([HF-de] §2.A "Block-Sparse Sliding Window
 * Attention", [HF-pt] §2.A.2): each query of block i attends, with softmax weights
 * exp(q.k/sqrt(D)), to exactly the keys of its kept blocks idx[bh][i][0..k).
 * Writes out[bh][t][:] for the query blocks listed in `blocks` (pairs bh, i;
 * n_blocks pairs), or for every query block when blocks == NULL.  Rows of
 * unlisted blocks are left untouched. */
void hfo_sparse_attn(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, int64_t bq, int64_t bk,
                     int64_t k, const double *Q, const double *K, const double *V,
                     const int32_t *idx, const int64_t *blocks, int64_t n_blocks, double *out);

/* hfo_sparse_attn with the relative temporal rotary embedding ([HF-de] §2.C "Relative
 * RoPE", [HF-pt] §2.B.2: the temporal RoPE index is capped and expressed as a relative
 * offset).  Reading: with T tokens per frame, key u lies in window frame fk = u / T and
 * query t of the chunk in frame fq = (Nk - Nq + t) / T (the chunk is the window's last Nq
 * rows); the score of (t, u) is (R(delta) q_t) . k_u / sqrt(D) with
 * delta = clamp(fq - fk, -cap, cap), where R(delta) turns feature pair (2i, 2i+1),
 * i < DT/2, by the angle delta * base^(-2i/DT) and leaves features DT..D-1 unchanged.
 * For |fq - fk| <= cap this equals the usual rotary score (R(a_t) q_t) . (R(a_u) k_u)
 * with absolute positions a.  The rest is as hfo_sparse_attn. */
void hfo_sparse_attn_rope(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, int64_t bq, int64_t bk,
                          int64_t k, int64_t T, int64_t DT, int64_t cap, double base, const double *Q,
                          const double *K, const double *V, const int32_t *idx, const int64_t *blocks,
                          int64_t n_blocks, double *out);

/* Linear temporal readout ([HF-de] §2.A "Lineare Zeit-Aufmerksamkeit", [HF-abs]):
 * out[t][c] = sum_a phi(Q[t][a]) S[a][c] / (sum_a phi(Q[t][a]) z[a] + eps).
 * Same `blocks` convention as hfo_sparse_attn (query blocks of size bq). */
void hfo_linear_readout(int64_t BH, int64_t Nq, int64_t D, int64_t bq, const double *Q,
                        const double *S, const double *z, double eps,
                        const int64_t *blocks, int64_t n_blocks, double *out);

/* Absorb evicted tokens into the compact state ([HF-abs]: the state incrementally
 * absorbs evicted tokens; [HF-de] §2.A: evicted frames are aggregated into it):
 * S[a][c] += sum_u phi(K[u][a]) V[u][c],  z[a] += sum_u phi(K[u][a]).
 * K, V [BH][n][D]; S, z updated in place. */
void hfo_absorb(int64_t BH, int64_t n, int64_t D, const double *K, const double *V,
                double *S, double *z);

/* The whole step: pool, score, select, sparse attention, readout, and the sum of
 * the two branches ([HF-de] §2.A "Kombination", [HF-pt] §2.A "Resultado").
 * idx_out [BH][nqb][k] receives the selection; scores_out ([BH][nqb][nkb]) may be
 * NULL.  `blocks` as above restricts which query blocks are computed (selection is
 * always computed for all). */
void hfo_hybrid_step(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, int64_t bq, int64_t bk,
                     int64_t k, double eps, const double *Q, const double *K, const double *V,
                     const double *S, const double *z, const int64_t *blocks, int64_t n_blocks,
                     int32_t *idx_out, double *scores_out, double *out);

/* ---- backward of the step (the selection idx is held fixed: it is piecewise constant)
 * Each function below is the chain rule of the forward function above it, written out
 * term by term; gradients are ADDED into the output arrays (the caller zeroes them). */

/* Sparse attention: with P the softmax weights of query t over its kept keys u,
 * o_t = sum_u P_tu v_u, dP_tu = dO_t . v_u, Delta_t = sum_u P_tu dP_tu,
 * G_tu = P_tu (dP_tu - Delta_t):  dQ_t += G_tu k_u / sqrt(D),  dK_u += G_tu q_t / sqrt(D),
 * dV_u += P_tu dO_t.  Every query block is computed. */
void hfo_sparse_attn_bwd(int64_t BH, int64_t Nq, int64_t Nk, int64_t D, int64_t bq, int64_t bk,
                         int64_t k, const double *Q, const double *K, const double *V,
                         const int32_t *idx, const double *dO, double *dQ, double *dK, double *dV);

/* Linear readout r_t = n_t / den_t, n_t[c] = sum_a a_t[a] S[a][c], den_t = a_t . z + eps,
 * a_t = phi(q_t):  dn = dO_t / den_t, dden = -(dO_t . n_t) / den_t^2,
 * dS[a][c] += a_t[a] dn[c], dz[a] += a_t[a] dden, da[a] = sum_c S[a][c] dn[c] + z[a] dden,
 * dQ_t[a] += da[a] phi'(q_t[a]) with phi'(x) = 1 for x > 0, e^x otherwise. */
void hfo_linear_readout_bwd(int64_t BH, int64_t Nq, int64_t D, const double *Q, const double *S,
                            const double *z, double eps, const double *dO, double *dQ, double *dS,
                            double *dz);

/* Absorb S += sum_u phi(k_u)^T v_u, z += sum_u phi(k_u), given the gradients dS, dz of
 * the state after it:  dV_u[c] += sum_a phi(k_u[a]) dS[a][c],
 * dK_u[a] += (sum_c dS[a][c] v_u[c] + dz[a]) phi'(k_u[a]).  K, V [BH][n][D]. */
void hfo_absorb_bwd(int64_t BH, int64_t n, int64_t D, const double *K, const double *V,
                    const double *dS, const double *dz, double *dK, double *dV);

/* Number of OpenMP threads the oracle runs on (1 when built without OpenMP). */
int hfo_num_threads(void);
void hfo_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
