// Block selection for the block-sparse window attention.
//
// [HF-de] §2.A / [HF-pt] §2.A.2 keep only the most important (top-K) key blocks of the
// window for each query block; the importance score is the dot product of the
// mean-pooled query block and the mean-pooled key block ([LF-de] §2.2 token
// compression by mean pooling), scaled by 1/sqrt(D).  Ties go to the lower key block.
//
// Hierarchical variant ([LF-de] §2.2 "Hierarchische Spärliche Attention", coarse to fine):
// keys are also pooled per window frame; each query block first keeps its top_frames
// frames by pooled query block . frame-pooled keys / sqrt(D), then its top-k key blocks
// among the blocks that touch a kept frame.  The frame pooling reads no key twice: the
// pool kernel keeps each key block's rows of its two frames apart, frame_pool_kernel adds
// those parts per frame.
//
// Two launches (three for the hierarchical variant):
//   pool_kernel        HBM-bound: one workgroup per query or key block sums its rows in
//                      fp64 and stores the block mean.  The sums are exact while the
//                      magnitudes in one feature span at most 2^39 over 64 rows (8 bits of
//                      a bf16 significand + 6 bits of carries + the span fit in 53).
//                      In a hybrid step the same launch carries extra workgroups that
//                      prepare the readout operands, and the chunk's key blocks are
//                      pooled from the chunk input.
//   score_topk_kernel  one wave per query block: its fp64 scores against every pooled
//                      key block, each evaluated as sum_d (qbar_d * kbar_d) in index
//                      order with separately rounded products and sums (pooled keys staged
//                      through LDS in chunks of 64), kept in LDS; then a radix select of the
//                      k-th largest (score, -index) key and an ascending emit of the kept
//                      indices.  In a hybrid step the same launch carries the ring append of
//                      the chunk as extra workgroups, whose copying overlaps the scoring.
// The hierarchical variant pools per frame as well (frame_pool_kernel, between the two),
// and its score_topk_kernel instance scores the frames first, through the same LDS path
// and summation order, and selects them before the blocks.
#include "append_tile.h"
#include "state_tile.h"

namespace hf {
namespace {

__device__ __forceinline__ double bf16_to_f64(uint32_t bits) { return (double)__uint_as_float(bits << 16); }

// Row pointer of window key j (logical order): in the ring, or, for the current chunk's
// frames when the step appends them in the same launch, in the chunk input.
__device__ __forceinline__ const uint16_t *key_row(const hf_select_args &a, int bh, int j) {
    const int f = j / a.T, t = j - f * a.T;
    if (a.k_cur && f >= a.ncom) return a.k_cur + ((size_t)bh * a.Nq + (size_t)(f - a.ncom) * a.T + t) * a.D;
    int slot = a.head + f;
    if (slot >= a.W) slot -= a.W;
    return a.ring_k + (((size_t)bh * a.W + slot) * a.T + t) * a.D;
}

// Position of feature d of row ro in the pool's fp64 reduction array: bits 5-6 of d and
// bit 0 of ro XORed into bits 0-2, so that a write (lanes v = 0 .. 15 of two rows, features
// 8 v + e) and a read (consecutive features of one row) touch distinct banks.  Values and
// summation order are unchanged.
__device__ __forceinline__ int rpos(int ro, int d) { return d ^ (((d >> 5) & 3) | ((ro & 1) << 2)); }

template <int D, bool SPLIT>
__global__ __launch_bounds__(256) void pool_kernel(hf_select_args a) {
    constexpr int kVec = D / 8;              // 16-byte vectors per row
    constexpr int kRowsPerPass = 256 / kVec;
    __shared__ double red[kRowsPerPass][D];

    const int per_plane = a.nqb + a.nkb;
    if ((int)blockIdx.x >= a.BH * per_plane) {
        const int x = (int)blockIdx.x - a.BH * per_plane;
        if (x < a.prep_tiles)   // readout operands of a hybrid step (independent of the selection)
            state_tile<D>(a.prep, x, reinterpret_cast<float(*)[33]>(&red[0][0]));
        return;
    }
    const int bh = blockIdx.x / per_plane;
    const int blk = blockIdx.x % per_plane;
    const bool is_q = blk < a.nqb;
    const int b = is_q ? blk : blk - a.nqb;
    const int bs = is_q ? a.bq : a.bk;
    const int N = is_q ? a.Nq : a.Nk;
    // hierarchical: rows from `fend` on lie in the key block's second frame; their sum is
    // kept apart (both parts are exact sums, so the block sum is unchanged)
    const bool split = SPLIT && !is_q;
    const int fend = split ? min((b * bs / a.T + 1) * a.T, N) : N;
    const int r0 = b * bs, r1 = min(r0 + bs, N);

    const int v = threadIdx.x % kVec, ro = threadIdx.x / kVec;
    double acc[8], acc2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc2[e] = 0.0;
    // this thread's rows r0 + ro, r0 + ro + kRowsPerPass, ... below `end`, from `r` on
    auto add_rows = [&](int r, int end, double (&s)[8]) __attribute__((always_inline)) {
#pragma unroll 4
        for (; r < end; r += kRowsPerPass) {
            const uint16_t *row = is_q ? a.q + ((size_t)bh * a.Nq + r) * D : key_row(a, bh, r);
            const u32x4 w = *reinterpret_cast<const u32x4 *>(row + v * 8);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s[2 * e] += bf16_to_f64(ws[e] & 0xFFFFu);
                s[2 * e + 1] += bf16_to_f64(ws[e] >> 16);
            }
        }
        return r;
    };
    // the first frame's rows into acc, the second's (hierarchical key blocks) into acc2
    const int r = add_rows(r0 + ro, min(fend, r1), acc);
    if constexpr (SPLIT) add_rows(r, r1, acc2);
    if constexpr (SPLIT) {
        if (split) {
            // the two frame parts of this key block, for the frame pooling, reduced one after
            // the other through the same LDS (one array keeps the launch at eight workgroups
            // per CU); the block's sum is their sum (both exact, so it is the exact block sum)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[ro][rpos(ro, v * 8 + e)] = acc[e];
            __syncthreads();
            double s0 = 0.0, s1 = 0.0;
            if (threadIdx.x < D)
                for (int k = 0; k < kRowsPerPass; ++k) s0 += red[k][rpos(k, threadIdx.x)];
            if (fend < r1) {                  // the block reaches into the next frame (uniform)
                __syncthreads();
#pragma unroll
                for (int e = 0; e < 8; ++e) red[ro][rpos(ro, v * 8 + e)] = acc2[e];
                __syncthreads();
                if (threadIdx.x < D)
                    for (int k = 0; k < kRowsPerPass; ++k) s1 += red[k][rpos(k, threadIdx.x)];
            }
            if (threadIdx.x < D) {
                double *pp = a.part + (((size_t)bh * a.nkb + b) * 2) * D;
                pp[threadIdx.x] = s0;
                pp[D + threadIdx.x] = s1;
                a.kbar[((size_t)bh * a.nkb + b) * D + threadIdx.x] = (s0 + s1) / (double)(r1 - r0);
            }
            return;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[ro][rpos(ro, v * 8 + e)] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
        double s = 0.0;
        for (int k = 0; k < kRowsPerPass; ++k) s += red[k][rpos(k, threadIdx.x)];
        double *dst = is_q ? a.qbar + ((size_t)bh * a.nqb + b) * D : a.kbar + ((size_t)bh * a.nkb + b) * D;
        dst[threadIdx.x] = s / (double)(r1 - r0);
    }
}

// Frame-pooled keys (hierarchical selection): frame f's key sum is assembled, in key block
// order, from the parts of the key blocks that touch it -- a block's first-frame part when
// the block starts in f, its second-frame part when it starts in f - 1 (bk <= T, so a
// block touches at most two frames).  The parts are exact sums, so the frame sum is the
// exact sum of its T rows; then the mean.
template <int D>
__global__ __launch_bounds__(D) void frame_pool_kernel(hf_select_args a) {
    const int bh = blockIdx.x / a.nfr, f = blockIdx.x % a.nfr;
    const int j0 = f * a.T / a.bk, j1 = ((f + 1) * a.T - 1) / a.bk;
    constexpr int kBatch = 16;                                 // loads in flight before the adds
    double s = 0.0;
    for (int jb = j0; jb <= j1; jb += kBatch) {
        double v[kBatch];
#pragma unroll
        for (int e = 0; e < kBatch; ++e) {
            const int j = jb + e;
            const int second = (j * a.bk / a.T) != f;          // block j starts in frame f - 1
            v[e] = j <= j1 ? a.part[(((size_t)bh * a.nkb + j) * 2 + second) * D + threadIdx.x] : 0.0;
        }
#pragma unroll
        for (int e = 0; e < kBatch; ++e)
            if (jb + e <= j1) s += v[e];
    }
    a.fbar[((size_t)bh * a.nfr + f) * D + threadIdx.x] = s / (double)a.T;
}

__device__ __forceinline__ uint64_t order_key(double s) {
    const uint64_t u = (uint64_t)__double_as_longlong(s + 0.0);  // -0 -> +0
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Radix select over one wave: the k-th largest of the keys held in registers (KPL per
// lane; key 0 marks an absent candidate and is below every real key).  Returns that key
// and how many of the keys equal to it are kept (the lowest-indexed ones).
template <int KPL>
__device__ __forceinline__ uint64_t kth_key(const uint64_t (&key)[KPL], int k, int &need_eq) {
    // largest v with #{key >= v} >= k (v = 0 is only reached if fewer than k real keys
    // exist, which the callers' bounds on k rule out), found bit by bit from the top.  The
    // search stops early once exactly k keys lie at or above the prefix: those k are the
    // kept set, whatever their remaining bits.
    uint64_t prefix = 0;
    for (int bit = 63; bit >= 0; --bit) {
        const uint64_t cand = prefix | (1ull << bit);
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < KPL; ++e) cnt += __popcll(__ballot(key[e] >= cand));
        if (cnt >= k) prefix = cand;
        if (cnt == k) break;
    }
    int gt = 0;
#pragma unroll
    for (int e = 0; e < KPL; ++e) gt += __popcll(__ballot(key[e] > prefix));
    need_eq = k - gt;  // keys equal to the returned value that are kept (0 after an early stop
                       // where none equals it)
    return prefix;
}

// Ascending emit of the kept candidates (index lane + 64 e) to out[0 .. k); returns the
// kept set as a bit mask when KPL == 1.
template <int KPL>
__device__ __forceinline__ uint64_t emit_kept(const uint64_t (&key)[KPL], int n, uint64_t prefix, int need_eq,
                                              int32_t *out, int lane) {
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int written = 0, eq_seen = 0;
    uint64_t kept = 0;
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
        const int j = lane + 64 * e;
        const bool valid = j < n;
        const bool is_gt = valid && key[e] > prefix;
        const bool is_eq = valid && key[e] == prefix;
        const uint64_t eq_b = __ballot(is_eq);
        const int eq_rank = eq_seen + __popcll(eq_b & lt_mask);
        const bool sel = is_gt || (is_eq && eq_rank < need_eq);
        const uint64_t sel_b = __ballot(sel);
        if (sel && out) out[written + __popcll(sel_b & lt_mask)] = j;
        written += __popcll(sel_b);
        eq_seen += __popcll(eq_b);
        if (e == 0) kept = sel_b;
    }
    return kept;
}

// Flat selection, scores and top-k in one launch: a workgroup takes kRows query blocks of
// one plane (one wave each).  The plane's pooled key blocks pass through LDS in chunks of
// 64 (the next chunk is loaded into registers while the current one is scored); lane l of
// wave w scores query block w against key block (chunk start + l) as a sequential sum in
// index order with separately rounded products and sums, as the oracle does.  The row of
// scores stays in LDS for the wave's radix select.  HIER (hierarchical selection): before
// the key blocks the plane's frame-pooled keys pass through the same LDS (at most 64
// frames), lane f scoring frame f the same way; each wave keeps its top_frames best frames
// (radix select, ties to the lower frame), and only the key blocks touching a kept frame
// enter the block select.
constexpr int kRows = 4;
template <int D, int KPL, bool HIER = false>
__global__ __launch_bounds__(64 * kRows) void score_topk_kernel(hf_select_args a, double scale) {
    constexpr int P = D + 2;                  // row pitch in doubles (16-byte aligned rows)
    constexpr int CH = 64;                    // key blocks per chunk
    constexpr int kPer = CH * D / 2 / (64 * kRows);   // 16-byte loads per thread per chunk
    typedef __attribute__((ext_vector_type(2))) double f64x2;
    __shared__ __align__(16) double qs[kRows][P];
    __shared__ __align__(16) double ks[CH][P];
    __shared__ double srow[kRows][KPL * 64];
    const int groups = (a.nqb + kRows - 1) / kRows;
    if ((int)blockIdx.x >= a.BH * groups) {
        // a hybrid step's ring append: pure copying, which fills the slots this latency-bound
        // scoring leaves idle (nothing here reads the ring: the current chunk's keys were
        // pooled from the chunk input)
        append_tile<D>(a.app, (int)blockIdx.x - a.BH * groups, reinterpret_cast<u32x4 *>(&ks[0][0]));
        return;
    }
    const int bh = blockIdx.x / groups, i0 = (blockIdx.x % groups) * kRows;
    const int tid = threadIdx.x, w = tid / 64, lane = tid % 64;
    const int i = i0 + w;                     // this wave's query block (past the end: idle)
    for (int t = tid; t < kRows * D / 2; t += 64 * kRows) {
        const int r = t / (D / 2), d = 2 * (t % (D / 2));
        *reinterpret_cast<f64x2 *>(&qs[r][d]) =
            *reinterpret_cast<const f64x2 *>(a.qbar + ((size_t)bh * a.nqb + min(i0 + r, a.nqb - 1)) * D + d);
    }
    const double *kb = a.kbar + (size_t)bh * a.nkb * D;
    f64x2 nxt[kPer];
    auto load_rows = [&](const double *base, int nrows, int c0) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int t = tid + 64 * kRows * e, r = t / (D / 2), d = 2 * (t % (D / 2));
            nxt[e] = *reinterpret_cast<const f64x2 *>(base + (size_t)min(c0 + r, nrows - 1) * D + d);
        }
    };
    auto load_chunk = [&](int c0) { load_rows(kb, a.nkb, c0); };
    auto stage = [&]() {
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int t = tid + 64 * kRows * e, r = t / (D / 2), d = 2 * (t % (D / 2));
            *reinterpret_cast<f64x2 *>(&ks[r][d]) = nxt[e];
        }
    };
    // score of query block w against staged row `lane`
    auto row_score = [&]() -> double {
        double acc = 0.0;
        {
#pragma clang fp contract(off)
#pragma unroll 8
            for (int d = 0; d < D; d += 2) {
                const f64x2 q = *reinterpret_cast<const f64x2 *>(&qs[w][d]);
                const f64x2 k = *reinterpret_cast<const f64x2 *>(&ks[lane][d]);
                acc = acc + q.x * k.x;
                acc = acc + q.y * k.y;
            }
            acc = acc * scale;
        }
        return acc;
    };
    uint64_t frames = ~0ull;                  // kept frames of this wave's query block (bit f)
    if constexpr (HIER) {
        load_rows(a.fbar + (size_t)bh * a.nfr * D, a.nfr, 0);
        stage();
        __syncthreads();                      // qs and the frame rows are in place
        load_chunk(0);
        const double sf = row_score();
        const size_t row = (size_t)bh * a.nqb + i;
        if (a.fscores && i < a.nqb && lane < a.nfr) a.fscores[row * a.nfr + lane] = sf;
        const uint64_t fkey[1] = {lane < a.nfr ? order_key(sf) : 0};
        int need_eq;
        const uint64_t prefix = kth_key<1>(fkey, a.top_frames, need_eq);
        frames = emit_kept<1>(fkey, a.nfr, prefix, need_eq,
                              a.fidx && i < a.nqb ? a.fidx + row * a.top_frames : nullptr, lane);
    } else {
        load_chunk(0);
    }
    for (int c0 = 0; c0 < a.nkb; c0 += CH) {
        __syncthreads();                      // everyone is done with the previous chunk
        stage();
        __syncthreads();
        if (c0 + CH < a.nkb) load_chunk(c0 + CH);
        const int j = c0 + lane;
        const double acc = row_score();
        if (j < a.nkb) {
            srow[w][j] = acc;
            if (a.scores && i < a.nqb) a.scores[((size_t)bh * a.nqb + i) * a.nkb + j] = acc;
        }
    }
    if (i >= a.nqb) return;                   // uniform per wave; no barrier follows
    uint64_t key[KPL];
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
        const int j = lane + 64 * e;
        bool ok = j < a.nkb;
        if constexpr (HIER) {
            if (ok) {
                // frames touched by key block j: f0 .. f1 (bk <= T: at most two)
                const int f0 = j * a.bk / a.T, f1 = (min((j + 1) * a.bk, a.Nk) - 1) / a.T;
                ok = ((frames >> f0) & ((2ull << (f1 - f0)) - 1)) != 0;
            }
        }
        key[e] = ok ? order_key(srow[w][j]) : 0;
    }
    int need_eq;
    const uint64_t prefix = kth_key<KPL>(key, a.top_k, need_eq);
    emit_kept<KPL>(key, a.nkb, prefix, need_eq, a.idx + ((size_t)bh * a.nqb + i) * a.top_k, lane);
}

}  // namespace
}  // namespace hf

template <int D, bool HIER = false>
static void launch_score_topk(int kpl, const hf_select_args &a, double scale, hipStream_t s) {
    const dim3 grid((unsigned)(a.BH * ((a.nqb + hf::kRows - 1) / hf::kRows) + a.app_tiles));
    const dim3 block(64 * hf::kRows);
    if (kpl <= 1) hipLaunchKernelGGL((hf::score_topk_kernel<D, 1, HIER>), grid, block, 0, s, a, scale);
    else if (kpl <= 2) hipLaunchKernelGGL((hf::score_topk_kernel<D, 2, HIER>), grid, block, 0, s, a, scale);
    else if (kpl <= 3) hipLaunchKernelGGL((hf::score_topk_kernel<D, 3, HIER>), grid, block, 0, s, a, scale);
    else if (kpl <= 4) hipLaunchKernelGGL((hf::score_topk_kernel<D, 4, HIER>), grid, block, 0, s, a, scale);
    else if (kpl <= 8) hipLaunchKernelGGL((hf::score_topk_kernel<D, 8, HIER>), grid, block, 0, s, a, scale);
    else if (kpl <= 16) hipLaunchKernelGGL((hf::score_topk_kernel<D, 16, HIER>), grid, block, 0, s, a, scale);
    else hipLaunchKernelGGL((hf::score_topk_kernel<D, 24, HIER>), grid, block, 0, s, a, scale);
}

hipError_t hf_launch_block_select(const hf_select_args &a, hipStream_t s) {
    // a step's ring append runs as extra workgroups of the score + top-k launch (flat
    // selection; the hierarchical path is never given one)
    const dim3 grid_pool((unsigned)(a.BH * (a.nqb + a.nkb) + a.prep_tiles));
    const double scale = 1.0 / sqrt((double)a.D);
    const int kpl = (a.nkb + 63) / 64;
    if (a.top_frames == 0) {
        // flat: pool, then scores and top-k in one launch
        if (a.D == 64) {
            hipLaunchKernelGGL((hf::pool_kernel<64, false>), grid_pool, dim3(256), 0, s, a);
            launch_score_topk<64>(kpl, a, scale, s);
        } else {
            hipLaunchKernelGGL((hf::pool_kernel<128, false>), grid_pool, dim3(256), 0, s, a);
            launch_score_topk<128>(kpl, a, scale, s);
        }
        return hipGetLastError();
    }
    // hierarchical: pool (keeping each key block's frame parts), frame means, then frame
    // scores, frame top-k, block scores and the block top-k among the kept frames' blocks in
    // one launch
    if (a.D == 64) {
        hipLaunchKernelGGL((hf::pool_kernel<64, true>), grid_pool, dim3(256), 0, s, a);
        hipLaunchKernelGGL(hf::frame_pool_kernel<64>, dim3((unsigned)(a.BH * a.nfr)), dim3(64), 0, s, a);
        launch_score_topk<64, true>(kpl, a, scale, s);
    } else {
        hipLaunchKernelGGL((hf::pool_kernel<128, true>), grid_pool, dim3(256), 0, s, a);
        hipLaunchKernelGGL(hf::frame_pool_kernel<128>, dim3((unsigned)(a.BH * a.nfr)), dim3(128), 0, s, a);
        launch_score_topk<128, true>(kpl, a, scale, s);
    }
    return hipGetLastError();
}
