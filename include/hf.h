/*
 * hf.h -- C ABI of the MI355X (gfx950) hybrid attention step of Hybrid Forcing.
 *
 * The method (pages, cited by title and section):
 *   [HF-de]  gist.science (German) summary of "Long-Horizon Streaming Video Generation
 *            via Hybrid Attention with Decoupled Distillation", §2.A "Hybride
 *            Aufmerksamkeitsmechanismen".
 *   [HF-pt]  gist.science (Portuguese) summary of the same paper, §2.A "Mecanismo de
 *            Atenção Híbrida" (2.A.1 linear temporal attention, 2.A.2 sparse window
 *            attention, "Resultado").
 *   [HF-abs] the paper's English abstract (arxivdaily.com page of the same paper).
 *   [LF-de]  gist.science (German) summary of "Light Forcing: Accelerating Autoregressive
 *            Video Diffusion via Sparse Attention", §2.2 "Hierarchische Spärliche
 *            Attention" (mean-pooled block tokens).
 *
 * Each chunk of latent frames attends to a sliding window of recent frames kept in a
 * KV cache.  Its output is the sum of (a) block-sparse softmax attention over the
 * window, computed only on the top-k key blocks of each query block, and (b) a linear
 * attention readout from a compact state (S, z) that absorbs the tokens evicted from
 * the window ([HF-de] §2.A, [HF-pt] §2.A, [HF-abs]).
 *
 * Readings where the pages are silent (the same ones the fp64 oracle takes):
 *   feature map phi(x) = elu(x) + 1; readout phi(q)^T S / (phi(q) . z + eps), eps as
 *   passed (1e-6 by default); softmax and block scores scaled by 1/sqrt(D); block score
 *   = mean-pooled query block . mean-pooled key block; top-k ties go to the lower key
 *   block index; no causal mask inside the window; the two branches are summed with no
 *   weight; a step reads (S, z) as they were before its own evictions.
 *
 * ---------------------------------------------------------------------------------
 * Conventions shared by every entry point
 *
 *  * Memory: every pointer argument named *_dev is DEVICE memory owned by the caller;
 *    hf_dims / hf_kv_ring structs and `bytes` out-parameters are HOST memory.  The
 *    library never allocates, frees, or keeps a pointer after returning (the one entry
 *    point for callers that cannot allocate, hf_hybrid_step_noalloc, uses a fixed device
 *    array the library holds per GPU).
 *  * Asynchrony: work is enqueued on `stream` (0 = the null stream) and the call
 *    returns without waiting.  A device fault surfaces at the caller's next
 *    synchronisation.
 *  * Validation happens before anything is enqueued.  A call that returns an error has
 *    enqueued nothing and changed nothing (buffers and ring descriptor untouched); the
 *    reason is kept in a thread-local string read by hf_last_error().
 *  * Dtypes: Q/K/V are bfloat16 (raw 16-bit storage); S, z and the output are fp32;
 *    block indices int32.
 *  * Supported shapes: D in {64, 128}; bq in {16, 32, 64}; bk in {16, 32, 64, 128};
 *    T a positive multiple of 8; 1 <= C <= W; B, H >= 1; total sizes below 2^31
 *    elements per tensor.  Anything else -> HF_ERR_UNSUPPORTED or HF_ERR_SHAPE.
 *  * Determinism: no floating-point atomics; the same inputs give bit-identical
 *    outputs, independent of the ring's physical head position.
 *  * Overlap: calls on different streams must not share an output or workspace buffer.
 * ---------------------------------------------------------------------------------
 */
#ifndef HF_H
#define HF_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HF_ABI_VERSION 1

typedef enum {
    HF_OK = 0,
    HF_ERR_NULL = 1,         /* a required pointer is NULL */
    HF_ERR_SHAPE = 2,        /* inconsistent sizes (e.g. top_k > number of key blocks) */
    HF_ERR_UNSUPPORTED = 3,  /* valid but not supported (D, block sizes, T % 8 != 0) */
    HF_ERR_RING_STATE = 4,   /* ring descriptor out of range (head, n_committed) */
    HF_ERR_WORKSPACE = 5,    /* workspace missing or smaller than hf_workspace_size() */
    HF_ERR_HIP = 6           /* a HIP launch failed (message holds hipGetErrorString) */
} hf_status;

/* Problem geometry (host struct).
 *   B  independent streams (batch)         H  heads            D  head dim (64 | 128)
 *   T  tokens per latent frame             C  frames per chunk (the current chunk)
 *   W  window frames incl. the current chunk (the sliding window of [HF-de] §1)
 *   bq, bk  query / key block sizes of the block-sparse attention ([HF-de] §2.A). */
typedef struct {
    int32_t B, H, D;
    int32_t T, C, W;
    int32_t bq, bk;
} hf_dims;

/* KV cache as a ring of W frame slots (the windowed KV cache with eviction of
 * [HF-de] §1 / [HF-pt] §1).
 *   k_dev   bf16 [B][H][W][T][D]       key frames, row-major (D contiguous)
 *   vg_dev  bf16 [B][H][W][T/8][D][8]  value frames in 8-token GROUPS: for each group of 8
 *                                      consecutive tokens of a frame, D rows of the 8
 *                                      tokens' values (value feature f of token 8g + j at
 *                                      [g][f][j]); a 16-byte row is the 8-key slice of one
 *                                      feature that the matrix cores take as an operand, and
 *                                      the keys of a group are one contiguous 16*D bytes
 *   head         slot holding the oldest frame of the window, 0 <= head < W
 *   n_committed  frames already committed to the window, 0 <= n_committed <= W - C
 * Logical window frame f (0 = oldest) lives in slot (head + f) % W.  A step's window
 * is the n_committed committed frames followed by the C frames of the current chunk
 * (logical frames n_committed .. n_committed+C-1), so it holds
 * Nk = (n_committed + C) * T keys; key j is token j % T of logical frame j / T.
 * Query blocks cut the current chunk's Nq = C*T queries; key blocks cut the window,
 * across frame boundaries; a short last block is allowed. */
typedef struct {
    void *k_dev;
    void *vg_dev;
    int32_t head;
    int32_t n_committed;
} hf_kv_ring;

/* hf_hybrid_step flag: after attending, commit the current chunk to the window and
 * evict (absorb into S, z) the oldest frames beyond W - C committed frames. */
#define HF_STEP_COMMIT 1u

/* Optional timing hooks for hf_hybrid_step: any non-NULL event is recorded on the
 * step's stream at that point: ev[0] and ev[1] at the beginning (the ring append runs as
 * extra workgroups of the selection's second launch, so it has no interval of its own),
 * ev[2] and ev[3] after block selection (whose first launch also prepares the readout
 * operands, so the two mark the same point), ev[4] after the attention launch (whose extra
 * workgroups also form the absorb partials of the evicted frames), ev[5] after the state
 * pass that adds them to the state (the end of the step).
 * Events must have been created by the caller with hipEventCreate. */
typedef struct {
    hipEvent_t ev[6];
} hf_step_events;

int hf_abi_version(void);
const char *hf_status_str(hf_status s);
/* Detail of the last failed call on this thread ("" if none). */
const char *hf_last_error(void);

/* Bytes of device workspace the entry points need for these dims and top_k, for a
 * window of up to W frames (host call, no GPU work).  The same workspace serves every
 * entry point; it holds transient per-call data only and needs no initialisation. */
hf_status hf_workspace_size(const hf_dims *d, int32_t top_k, size_t *bytes);

/* Describe an empty ring over caller-owned storage (host only, no GPU work): checks the
 * dims, then sets *out = {k_store_dev, vg_store_dev, head 0, n_committed 0}.  The storage
 * must hold B*H*W*T*D bf16 values each (layouts above); its contents are not read until
 * frames are committed.  Errors: those of the dims, HF_ERR_NULL for a NULL pointer. */
hf_status hf_ring_init(const hf_dims *d, void *k_store_dev, void *vg_store_dev, hf_kv_ring *out);

/* Copy the current chunk into the ring: k_cur_dev, v_cur_dev are bf16 [B][H][C*T][D]
 * (row-major).  Frame c of the chunk goes to logical frame n_committed + c; values are
 * written in 8-token groups (see hf_kv_ring).  The descriptor is not changed. */
hf_status hf_ring_append(const hf_dims *d, const hf_kv_ring *ring, const void *k_cur_dev,
                         const void *v_cur_dev, hipStream_t stream);

/* Block selection ([HF-de] §2.A, item "Block-Sparse Sliding Window Attention"; [HF-pt]
 * §2.A.2; pooling as in [LF-de] §2.2, item "Token-Kompression").
 * For each (b, h, query block i): qbar_i = mean of Q over block i, kbar_j = mean of the
 * window keys over key block j, score s_ij = qbar_i . kbar_j / sqrt(D) (pooled and
 * scored in fp64); keep the top_k largest, ties to the lower j, written in ASCENDING
 * order.  The pooled sums are exact in fp64, so independent of summation order, when the
 * nonzero magnitudes summed into one pooled feature span at most 2^(45 - ceil(log2 n))
 * (n rows summed: 2^39 for 64-row blocks, 2^34 for 1560-token frames); beyond that
 * span a score may differ from an exact evaluation in its last bits.
 *   q_dev          bf16 [B][H][C*T][D] current chunk queries
 *   idx_dev        int32 [B][H][n_qb][top_k] out, n_qb = ceil(C*T/bq)
 *   scores_dev     fp64 [B][H][n_qb][n_kb] out (may be NULL), n_kb = ceil(Nk/bk)
 * Requires 1 <= top_k <= n_kb (HF_ERR_SHAPE otherwise); n_kb of a full window must not exceed
 * 1536 (HF_ERR_UNSUPPORTED). */
hf_status hf_block_select(const hf_dims *d, const void *q_dev, const hf_kv_ring *ring, int32_t top_k,
                          int32_t *idx_dev, double *scores_dev, void *workspace_dev,
                          size_t workspace_bytes, hipStream_t stream);

/* Hierarchical (coarse-to-fine) block selection ([LF-de] §2.2 "Hierarchische Spärliche
 * Attention": queries and keys compressed by mean pooling at block and frame level; per
 * query block, frame selection with the frame-level keys, then block selection inside the
 * selected frames).  For each (b, h, query block i):
 *   frame score  sf_if = qbar_i . fbar_f / sqrt(D), fbar_f the mean of window frame f's
 *                T keys; keep the top_frames best frames, ties to the lower frame;
 *   block score  s_ij as hf_block_select; keep the top_k best key blocks among those that
 *                touch (share a key with) a kept frame, ties to the lower block;
 * pooled and scored in fp64, indices written in ASCENDING order.
 *   idx_dev           int32 [B][H][n_qb][top_k] out (feeds hf_sparse_window_attn)
 *   frames_dev        NULL or int32 [B][H][n_qb][top_frames] out: kept frames, ascending
 *                     (logical window frames, 0 = oldest)
 *   scores_dev        NULL or fp64 [B][H][n_qb][n_kb] out: every block score
 *   frame_scores_dev  NULL or fp64 [B][H][n_qb][F] out, F = n_committed + C frames
 * Requires bk <= T, F <= 64, 1 <= top_frames <= F and 1 <= top_k <= min(n_kb,
 * top_frames * ceil(T / bk) - (top_frames - 1)) (the key blocks any top_frames frames are
 * sure to touch).  Errors: HF_ERR_UNSUPPORTED (bk > T, F > 64), HF_ERR_SHAPE (bounds), plus
 * those of hf_block_select. */
hf_status hf_block_select_hier(const hf_dims *d, const void *q_dev, const hf_kv_ring *ring, int32_t top_frames,
                               int32_t top_k, int32_t *idx_dev, int32_t *frames_dev, double *scores_dev,
                               double *frame_scores_dev, void *workspace_dev, size_t workspace_bytes,
                               hipStream_t stream);

/* Block-sparse window attention plus linear readout ([HF-de] §2.A, [HF-pt] §2.A.1,
 * 2.A.2 and "Resultado"; [HF-abs]).
 * out[b,h,t,:] = sum_{u in kept blocks of t's block} softmax_u(q_t.k_u / sqrt(D)) v_u
 *              + phi(q_t)^T S[b,h] / (phi(q_t) . z[b,h] + eps)
 *   q_dev    bf16 [B][H][C*T][D]
 *   idx_dev  int32 [B][H][n_qb][top_k]: kept key blocks, each in [0, n_kb), STRICTLY
 *            ASCENDING per query block (hf_block_select's output qualifies).  Other lists
 *            give unspecified values, but every access stays inside the window.
 *   S_dev    fp32 [B][H][D][D] (S[a][c]) and z_dev fp32 [B][H][D]: the linear state;
 *            both NULL -> the linear branch is skipped (sparse part only)
 *   out_dev  fp32 [B][H][C*T][D] out
 * Numerics: bf16 matrix-core products with fp32 accumulation and fp32 online softmax;
 * the readout multiplies bf16-rounded phi(q) and S with fp32 accumulation. */
hf_status hf_sparse_window_attn(const hf_dims *d, const void *q_dev, const hf_kv_ring *ring,
                                const int32_t *idx_dev, int32_t top_k, const float *S_dev,
                                const float *z_dev, float eps, float *out_dev, void *workspace_dev,
                                size_t workspace_bytes, hipStream_t stream);

/* Absorb evicted tokens into the state ([HF-abs]: a compact key-value state that
 * incrementally absorbs evicted tokens; [HF-de] §2.A; [HF-pt] §2.A.1):
 *   S[a][c] += sum_u phi(K_u[a]) V_u[c],   z[a] += sum_u phi(K_u[a])
 *   k_ev_dev, v_ev_dev  bf16 [B][H][n_tok][D] row-major evicted tokens
 *   S_dev, z_dev        fp32 state, updated in place
 * n_tok >= 0 (0 is a no-op).  Products use bf16 hi+lo halves of phi(K) so S keeps
 * fp32-grade accuracy.  The token range is cut into a fixed number of splits (set by
 * B, H, D and n_tok only); each split's partial sum goes to the workspace and a second
 * kernel adds them to (S, z) in split order, so the result is deterministic. */
hf_status hf_linear_absorb(const hf_dims *d, const void *k_ev_dev, const void *v_ev_dev, int64_t n_tok,
                           float *S_dev, float *z_dev, void *workspace_dev, size_t workspace_bytes,
                           hipStream_t stream);

/* Chunk-aware growth sparsity schedule ([LF-de] §2.1 "Chunk-bewusstes Wachstum"): the
 * keep counts of a stream of n_chunks chunks, the first dense and later ones sparser.
 * Host call, no GPU work; every pointer is HOST memory.
 *   n_kb[i]      key blocks in chunk i's window (>= 1)
 *   s_base       base sparsity, s_target the sparsity the whole stream must meet, s_max
 *                the cap of any chunk's sparsity; each in [0, 1)
 *   top_k[i]     out: kept key blocks per query block for chunk i (pass to hf_block_select
 *                or hf_hybrid_step)
 *   sparsity[i]  out (may be NULL): s_i;  beta out (may be NULL): the fitted beta
 * Schedule: s_0 = 0; s_i = min(max(s_base - beta / sqrt(i + 1), 0), s_max) for i >= 1;
 * top_k[i] = ceil((1 - s_i) n_kb[i]) clamped to [1, n_kb[i]]; beta >= 0 is the smallest
 * value (to double precision, by bisection) with sum_i top_k[i] >= (1 - s_target) sum_i
 * n_kb[i].  Readings: the page's alpha_i "proportional to 1/sqrt(T)" is taken as
 * 1/sqrt(i + 1) of the chunk's position, and "total FLOPs" as the kept key blocks summed
 * over the chunks (every chunk has the same query blocks).  Errors: HF_ERR_NULL,
 * HF_ERR_SHAPE (n_chunks < 1, n_kb[i] < 1, a ratio outside [0, 1) or NaN). */
hf_status hf_cag_schedule(int32_t n_chunks, const int32_t *n_kb, double s_base, double s_target, double s_max,
                          int32_t *top_k, double *sparsity, double *beta);

/* One hybrid attention step on the ring:
 *   1. if k_cur_dev and v_cur_dev are given: hf_ring_append (else the caller has
 *      already written the current chunk into its slots);
 *   2. block selection as hf_block_select -> idx_dev ([B][H][n_qb][top_k], an output);
 *   3. the readout operands are taken from (S, z) as they are (in the same launch as the
 *      selection's pooling);
 *   4. block-sparse attention with the fused readout, as hf_sparse_window_attn -> out_dev;
 *   5. with HF_STEP_COMMIT, when committing the chunk leaves more than W - C committed
 *      frames, the e oldest window frames are the evicted ones: they are absorbed into
 *      (S, z) -- S += sum phi(K_ev)^T V_ev, z += sum phi(K_ev), fp32 with bf16 hi/lo
 *      products as hf_linear_absorb: extra workgroups of the attention launch form split
 *      partial sums straight from the frames' ring slots (those frames stay in the ring
 *      until the next append), and a state pass adds them in split order;
 *   6. with HF_STEP_COMMIT: n_committed += C - e and head = (head + e) % W.
 * The output therefore reads the state before this step's evictions, and on return the
 * state includes them.  `ring` is updated on success only.  S_dev/z_dev may be NULL only
 * without HF_STEP_COMMIT (sparse part only).  `events` may be NULL. */
hf_status hf_hybrid_step(const hf_dims *d, const void *q_dev, const void *k_cur_dev, const void *v_cur_dev,
                         hf_kv_ring *ring, int32_t top_k, uint32_t flags, float *S_dev, float *z_dev,
                         float eps, int32_t *idx_dev, float *out_dev, void *workspace_dev,
                         size_t workspace_bytes, const hf_step_events *events, hipStream_t stream);

/* hf_hybrid_step for callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): the same step, the same kernels
 * and arguments, but no workspace -- its transient data live in a fixed device array of
 * 32 MiB that the library holds on each GPU it runs on until the process ends.  The call
 * allocates and frees nothing.  Calls that overlap in time on one GPU (different streams
 * or threads) race on that array; calls in one stream order are safe.  The stream's device
 * (the current device for the null stream) runs the work.  Errors: those of hf_hybrid_step,
 * HF_ERR_UNSUPPORTED when the step's transient data would exceed 32 MiB (the 832x480 layer
 * with 12 heads needs about 19 MiB, four such streams batched about 27 MiB), HF_ERR_HIP when
 * the array's device address cannot be obtained. */
hf_status hf_hybrid_step_noalloc(const hf_dims *d, const void *q_dev, const void *k_cur_dev, const void *v_cur_dev,
                                 hf_kv_ring *ring, int32_t top_k, uint32_t flags, float *S_dev, float *z_dev,
                                 float eps, int32_t *idx_dev, float *out_dev, const hf_step_events *events,
                                 hipStream_t stream);

/* ---- Relative temporal rotary embedding of the softmax branch ([HF-de] §2.C "Relative
 * RoPE", [HF-pt] §2.B.2: the temporal RoPE index is capped and expressed as an offset
 * between positions).  With it, the score of query t (window frame fq) and key u (window
 * frame fk) is (R(delta) q_t) . k_u / sqrt(D) with delta = clamp(fq - fk, -cap, cap), where
 * R(delta) turns feature pair (2i, 2i+1), i < temporal_dims / 2, by the angle
 * delta * base^(-2i / temporal_dims) and leaves the other features as they are.  Within the
 * cap this is the usual rotary score with absolute frame positions.  Block selection and
 * the linear branch use the raw q and k.  The turned query enters the matrix cores in
 * bf16.  Forward only: the backward entry points below do not take it. */
typedef struct {
    int32_t temporal_dims;   /* 16 or 32: the rotated leading features */
    int32_t cap;             /* largest |frame offset| the rotation sees, 0 .. 1024 */
    float base;              /* frequency base, finite and > 1 */
} hf_rope;

/* hf_sparse_window_attn with the rotary embedding; rope must not be NULL (HF_ERR_NULL);
 * fields outside the ranges above give HF_ERR_SHAPE. */
hf_status hf_sparse_window_attn_rope(const hf_dims *d, const void *q_dev, const hf_kv_ring *ring,
                                     const int32_t *idx_dev, int32_t top_k, const float *S_dev,
                                     const float *z_dev, float eps, const hf_rope *rope, float *out_dev,
                                     void *workspace_dev, size_t workspace_bytes, hipStream_t stream);

/* hf_hybrid_step with the rotary embedding in its attention (step 4); rope as above. */
hf_status hf_hybrid_step_rope(const hf_dims *d, const void *q_dev, const void *k_cur_dev, const void *v_cur_dev,
                              hf_kv_ring *ring, int32_t top_k, uint32_t flags, float *S_dev, float *z_dev,
                              float eps, const hf_rope *rope, int32_t *idx_dev, float *out_dev,
                              void *workspace_dev, size_t workspace_bytes, const hf_step_events *events,
                              hipStream_t stream);

/* ---- Backward of the step (training).  The block selection is held fixed: it is
 * piecewise constant in the inputs, so no gradient flows through it.  Gradients of a loss
 * L given dL/dout; for query t with kept keys u and softmax weights P_tu ([HF-de] §2.A,
 * [HF-pt] §2.A.1, 2.A.2, "Resultado"; [HF-abs]):
 *   dq_t = sum_u G_tu k_u / sqrt(D) + (S dn_t + z dden_t) * phi'(q_t),
 *   dk_u = sum_t G_tu q_t / sqrt(D),  dv_u = sum_t P_tu dout_t,
 *   dS = sum_t phi(q_t) dn_t^T,  dz = sum_t phi(q_t) dden_t,
 * with G_tu = P_tu (dout_t . v_u - dout_t . (out_t - r_t)), r_t the readout,
 * dn_t = dout_t / den_t, dden_t = -dout_t . (S^T phi(q_t)) / den_t^2,
 * den_t = phi(q_t) . z + eps, phi'(x) = 1 for x > 0 and e^x otherwise.
 * Products run on bf16 matrix cores with fp32 accumulation (P and G rounded to bf16 as
 * operands); every sum has a fixed order, so results are deterministic. */

/* Forward for training: hf_sparse_window_attn, plus lse_dev fp32 [B][H][C*T] out: for each
 * query, log2 of its softmax denominator over the kept keys, in base-2 logits
 * (lse_t = log2 sum_u 2^(q_t.k_u log2(e) / sqrt(D))), which hf_hybrid_attn_backward uses. */
hf_status hf_sparse_window_attn_lse(const hf_dims *d, const void *q_dev, const hf_kv_ring *ring,
                                    const int32_t *idx_dev, int32_t top_k, const float *S_dev,
                                    const float *z_dev, float eps, float *out_dev, float *lse_dev,
                                    void *workspace_dev, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace hf_hybrid_attn_backward needs for these dims and top_k (any
 * window of up to W frames); host call.  Contents need no initialisation. */
hf_status hf_backward_workspace_size(const hf_dims *d, int32_t top_k, size_t *bytes);

/* Backward of out = sparse window attention + linear readout (the forward of
 * hf_sparse_window_attn_lse with the same q, ring, idx, S, z, eps):
 *   inputs   q_dev bf16 [B][H][C*T][D]; ring, idx_dev, top_k, S_dev, z_dev, eps as in the
 *            forward (S and z required); out_dev and lse_dev fp32 from that forward;
 *            dout_dev fp32 [B][H][C*T][D] = dL/dout
 *   outputs  (written, not accumulated) dq_dev fp32 [B][H][C*T][D]; dk_dev, dv_dev fp32
 *            [B][H][Nk][D] for the window's keys in LOGICAL order (key j = f T + t of
 *            logical frame f; keys no query block kept get 0); dS_dev fp32 [B][H][D][D];
 *            dz_dev fp32 [B][H][D]
 *   workspace_dev of at least hf_backward_workspace_size bytes (HF_ERR_WORKSPACE otherwise).
 * Errors as hf_sparse_window_attn; the kept lists must be those of the forward. */
hf_status hf_hybrid_attn_backward(const hf_dims *d, const void *q_dev, const hf_kv_ring *ring,
                                  const int32_t *idx_dev, int32_t top_k, const float *S_dev,
                                  const float *z_dev, float eps, const float *out_dev,
                                  const float *lse_dev, const float *dout_dev, float *dq_dev,
                                  float *dk_dev, float *dv_dev, float *dS_dev, float *dz_dev,
                                  void *workspace_dev, size_t workspace_bytes, hipStream_t stream);

/* Backward of hf_linear_absorb ([HF-abs]: S += sum_u phi(k_u)^T v_u, z += sum_u phi(k_u)):
 * given dS_dev fp32 [B][H][D][D] and dz_dev fp32 [B][H][D], the gradients of the state
 * after the absorb, writes dk_dev, dv_dev fp32 [B][H][n_tok][D]:
 *   dv_u = phi(k_u) dS,   dk_u = (dS v_u + dz) * phi'(k_u)
 * (bf16 matrix-core products, fp32 accumulation).  The gradient with respect to the state
 * before the absorb is dS, dz themselves.  workspace_dev as for hf_linear_absorb. */
hf_status hf_linear_absorb_backward(const hf_dims *d, const void *k_ev_dev, const void *v_ev_dev,
                                    int64_t n_tok, const float *dS_dev, const float *dz_dev,
                                    float *dk_dev, float *dv_dev, void *workspace_dev,
                                    size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* HF_H */
