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
// Flat selection, two launches:
//   pool_kernel        HBM-bound: one workgroup per query or key block sums its rows in
//                      fp64 (sums of bf16 values are exact in fp64) and stores the block
//                      mean.  In a hybrid step the same launch carries extra workgroups
//                      that prepare the readout operands and append the chunk to the ring
//                      (the chunk's key blocks are then pooled from the chunk input).
//   score_topk_kernel  one wave per query block: its fp64 scores against every pooled
//                      key block, each evaluated as sum_d (qbar_d * kbar_d) in index
//                      order with separately rounded products and sums (pooled keys staged
//                      through LDS in chunks of 64), kept in LDS; then a radix select of the
//                      k-th largest (score, -index) key and an ascending emit of the kept
//                      indices.
// The hierarchical variant pools per frame as well (frame_pool_kernel), scores with the
// tiled score_kernel (16 x 16 tiles, one wave each, same summation order) over block pairs
// and over (query block, frame) pairs, and lets topk_kernel select the frames before the
// blocks.
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
        else                    // the step's ring append
            append_tile<D>(a.app, x - a.prep_tiles);
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
#pragma unroll 4
    for (int r = r0 + ro; r < r1; r += kRowsPerPass) {
        const uint16_t *row = is_q ? a.q + ((size_t)bh * a.Nq + r) * D : key_row(a, bh, r);
        const u32x4 w = *reinterpret_cast<const u32x4 *>(row + v * 8);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double lo = bf16_to_f64(ws[e] & 0xFFFFu), hi = bf16_to_f64(ws[e] >> 16);
            if constexpr (SPLIT) {
                const bool first = r < fend;           // adding 0.0 leaves a sum unchanged
                acc[2 * e] += first ? lo : 0.0;
                acc[2 * e + 1] += first ? hi : 0.0;
                acc2[2 * e] += first ? 0.0 : lo;
                acc2[2 * e + 1] += first ? 0.0 : hi;
            } else {
                acc[2 * e] += lo;
                acc[2 * e + 1] += hi;
            }
        }
    }
    if (SPLIT && split) {
        // the two frame parts of this key block, for the frame pooling (one LDS buffer,
        // reduced twice)
        double *pp = a.part + (((size_t)bh * a.nkb + b) * 2) * D;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int e = 0; e < 8; ++e) red[ro][v * 8 + e] = h == 0 ? acc[e] : acc2[e];
            __syncthreads();
            if (threadIdx.x < D) {
                double s = 0.0;
                for (int k = 0; k < kRowsPerPass; ++k) s += red[k][threadIdx.x];
                pp[h * D + threadIdx.x] = s;
            }
            __syncthreads();
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += acc2[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[ro][v * 8 + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
        double s = 0.0;
        for (int k = 0; k < kRowsPerPass; ++k) s += red[k][threadIdx.x];
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

constexpr int kTile = 16;   // score tile: 16 query blocks x 16 key blocks per workgroup

// Scores of a 16 x 16 tile of (query block, key block) pairs, one wave per tile: both
// pooled tiles are staged in LDS (every staging load issued before the first LDS write),
// then each lane forms a 2 x 2 block of dot products, each a sequential sum in index
// order, reading two features per 16-byte LDS load.
template <int D>
__global__ __launch_bounds__(64) void score_kernel(hf_select_args a, double scale) {
    constexpr int P = D + 2;                 // row pitch in doubles (16-byte aligned rows)
    __shared__ __align__(16) double qs[kTile][P];
    __shared__ __align__(16) double ks[kTile][P];
    typedef __attribute__((ext_vector_type(2))) double f64x2;
    const int ti_n = (a.nqb + kTile - 1) / kTile, tj_n = (a.nkb + kTile - 1) / kTile;
    const int bh = blockIdx.x / (ti_n * tj_n);
    const int i0 = ((blockIdx.x / tj_n) % ti_n) * kTile, j0 = (blockIdx.x % tj_n) * kTile;
    const int tid = threadIdx.x;
    {
        // rows past the end re-read the last row and are zeroed
        constexpr int kPer = kTile * D / 2 / 64;        // 16-byte loads per lane per matrix
        constexpr int kBatch = 8;
#pragma unroll
        for (int e0 = 0; e0 < kPer; e0 += kBatch) {
            f64x2 qv[kBatch], kv[kBatch];
#pragma unroll
            for (int e = 0; e < kBatch; ++e) {
                const int idx = tid + 64 * (e0 + e), r = idx / (D / 2), d = 2 * (idx % (D / 2));
                qv[e] = *reinterpret_cast<const f64x2 *>(a.qbar + ((size_t)bh * a.nqb + min(i0 + r, a.nqb - 1)) * D + d);
                kv[e] = *reinterpret_cast<const f64x2 *>(a.kbar + ((size_t)bh * a.nkb + min(j0 + r, a.nkb - 1)) * D + d);
            }
#pragma unroll
            for (int e = 0; e < kBatch; ++e) {
                const int idx = tid + 64 * (e0 + e), r = idx / (D / 2), d = 2 * (idx % (D / 2));
                const f64x2 z = {0.0, 0.0};
                *reinterpret_cast<f64x2 *>(&qs[r][d]) = i0 + r < a.nqb ? qv[e] : z;
                *reinterpret_cast<f64x2 *>(&ks[r][d]) = j0 + r < a.nkb ? kv[e] : z;
            }
        }
    }
    __syncthreads();
    const int ti = 2 * (tid / 8), tj = 2 * (tid % 8);
    double acc[2][2] = {{0.0, 0.0}, {0.0, 0.0}};
    {
        // products and sums rounded separately (no fused multiply-add), in index order
#pragma clang fp contract(off)
#pragma unroll 4
        for (int d = 0; d < D; d += 2) {
            const f64x2 q0 = *reinterpret_cast<const f64x2 *>(&qs[ti][d]);
            const f64x2 q1 = *reinterpret_cast<const f64x2 *>(&qs[ti + 1][d]);
            const f64x2 k0 = *reinterpret_cast<const f64x2 *>(&ks[tj][d]);
            const f64x2 k1 = *reinterpret_cast<const f64x2 *>(&ks[tj + 1][d]);
            acc[0][0] = acc[0][0] + q0.x * k0.x;
            acc[0][1] = acc[0][1] + q0.x * k1.x;
            acc[1][0] = acc[1][0] + q1.x * k0.x;
            acc[1][1] = acc[1][1] + q1.x * k1.x;
            acc[0][0] = acc[0][0] + q0.y * k0.y;
            acc[0][1] = acc[0][1] + q0.y * k1.y;
            acc[1][0] = acc[1][0] + q1.y * k0.y;
            acc[1][1] = acc[1][1] + q1.y * k1.y;
        }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) acc[x][y] = acc[x][y] * scale;
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
        const int i = i0 + ti + x;
        if (i >= a.nqb) continue;
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            const int j = j0 + tj + y;
            if (j >= a.nkb) continue;
            a.sc[((size_t)bh * a.nqb + i) * a.nkb + j] = acc[x][y];
            if (a.scores) a.scores[((size_t)bh * a.nqb + i) * a.nkb + j] = acc[x][y];
        }
    }
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

// One wave per (plane, query block): radix select of the k-th largest (score, -index)
// key, then an ascending emit of the kept block indices.  Lane l holds keys of blocks
// l, l + 64, ... in registers (KPL of them).  HIER: the candidates are first restricted
// to the key blocks touching the query block's top_frames best window frames (lane f
// holds frame f's score).
template <int KPL, bool HIER>
__global__ __launch_bounds__(256) void topk_kernel(hf_select_args a) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int row = blockIdx.x * 4 + wave;                    // (bh, i) flattened
    if (row >= a.BH * a.nqb) return;
    uint64_t frames = ~0ull;                                  // kept frames (bit f)
    if constexpr (HIER) {
        const uint64_t fkey[1] = {lane < a.nfr ? order_key(a.fsc[(size_t)row * a.nfr + lane]) : 0};
        int need_eq;
        const uint64_t prefix = kth_key<1>(fkey, a.top_frames, need_eq);
        frames = emit_kept<1>(fkey, a.nfr, prefix, need_eq,
                              a.fidx ? a.fidx + (size_t)row * a.top_frames : nullptr, lane);
    }
    const double *src = a.sc + (size_t)row * a.nkb;
    uint64_t key[KPL];
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
        const int j = lane + 64 * e;
        bool ok = j < a.nkb;
        if constexpr (HIER) {
            if (ok) {
                // frames touched by key block j: f0 .. f1 (at most 17 of them: bk <= 128, T >= 8)
                const int f0 = j * a.bk / a.T, f1 = (min((j + 1) * a.bk, a.Nk) - 1) / a.T;
                ok = ((frames >> f0) & ((2ull << (f1 - f0)) - 1)) != 0;
            }
        }
        key[e] = ok ? order_key(src[j]) : 0;
    }
    int need_eq;
    const uint64_t prefix = kth_key<KPL>(key, a.top_k, need_eq);
    emit_kept<KPL>(key, a.nkb, prefix, need_eq, a.idx + (size_t)row * a.top_k, lane);
}

// Flat selection, scores and top-k in one launch: a workgroup takes kRows query blocks of
// one plane (one wave each).  The plane's pooled key blocks pass through LDS in chunks of
// 64 (the next chunk is loaded into registers while the current one is scored); lane l of
// wave w scores query block w against key block (chunk start + l) as a sequential sum in
// index order with separately rounded products and sums, exactly as the tiled kernel
// does.  The row of scores stays in LDS for the wave's radix select.
constexpr int kRows = 4;
template <int D, int KPL>
__global__ __launch_bounds__(64 * kRows) void score_topk_kernel(hf_select_args a, double scale) {
    constexpr int P = D + 2;                  // row pitch in doubles (16-byte aligned rows)
    constexpr int CH = 64;                    // key blocks per chunk
    constexpr int kPer = CH * D / 2 / (64 * kRows);   // 16-byte loads per thread per chunk
    typedef __attribute__((ext_vector_type(2))) double f64x2;
    __shared__ __align__(16) double qs[kRows][P];
    __shared__ __align__(16) double ks[CH][P];
    __shared__ double srow[kRows][KPL * 64];
    const int groups = (a.nqb + kRows - 1) / kRows;
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
    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int t = tid + 64 * kRows * e, r = t / (D / 2), d = 2 * (t % (D / 2));
            nxt[e] = *reinterpret_cast<const f64x2 *>(kb + (size_t)min(c0 + r, a.nkb - 1) * D + d);
        }
    };
    load_chunk(0);
    for (int c0 = 0; c0 < a.nkb; c0 += CH) {
        __syncthreads();                      // everyone is done with the previous chunk
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int t = tid + 64 * kRows * e, r = t / (D / 2), d = 2 * (t % (D / 2));
            *reinterpret_cast<f64x2 *>(&ks[r][d]) = nxt[e];
        }
        __syncthreads();
        if (c0 + CH < a.nkb) load_chunk(c0 + CH);
        const int j = c0 + lane;
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
        key[e] = j < a.nkb ? order_key(srow[w][j]) : 0;
    }
    int need_eq;
    const uint64_t prefix = kth_key<KPL>(key, a.top_k, need_eq);
    emit_kept<KPL>(key, a.nkb, prefix, need_eq, a.idx + ((size_t)bh * a.nqb + i) * a.top_k, lane);
}

}  // namespace
}  // namespace hf

static void launch_topk(int kpl, dim3 grid, const hf_select_args &a, hipStream_t s) {
    if (kpl <= 1) hipLaunchKernelGGL((hf::topk_kernel<1, true>), grid, dim3(256), 0, s, a);
    else if (kpl <= 2) hipLaunchKernelGGL((hf::topk_kernel<2, true>), grid, dim3(256), 0, s, a);
    else if (kpl <= 3) hipLaunchKernelGGL((hf::topk_kernel<3, true>), grid, dim3(256), 0, s, a);
    else if (kpl <= 4) hipLaunchKernelGGL((hf::topk_kernel<4, true>), grid, dim3(256), 0, s, a);
    else if (kpl <= 8) hipLaunchKernelGGL((hf::topk_kernel<8, true>), grid, dim3(256), 0, s, a);
    else if (kpl <= 16) hipLaunchKernelGGL((hf::topk_kernel<16, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((hf::topk_kernel<24, true>), grid, dim3(256), 0, s, a);
}

template <int D>
static void launch_score_topk(int kpl, const hf_select_args &a, double scale, hipStream_t s) {
    const dim3 grid((unsigned)(a.BH * ((a.nqb + hf::kRows - 1) / hf::kRows)));
    const dim3 block(64 * hf::kRows);
    if (kpl <= 1) hipLaunchKernelGGL((hf::score_topk_kernel<D, 1>), grid, block, 0, s, a, scale);
    else if (kpl <= 2) hipLaunchKernelGGL((hf::score_topk_kernel<D, 2>), grid, block, 0, s, a, scale);
    else if (kpl <= 3) hipLaunchKernelGGL((hf::score_topk_kernel<D, 3>), grid, block, 0, s, a, scale);
    else if (kpl <= 4) hipLaunchKernelGGL((hf::score_topk_kernel<D, 4>), grid, block, 0, s, a, scale);
    else if (kpl <= 8) hipLaunchKernelGGL((hf::score_topk_kernel<D, 8>), grid, block, 0, s, a, scale);
    else if (kpl <= 16) hipLaunchKernelGGL((hf::score_topk_kernel<D, 16>), grid, block, 0, s, a, scale);
    else hipLaunchKernelGGL((hf::score_topk_kernel<D, 24>), grid, block, 0, s, a, scale);
}

hipError_t hf_launch_block_select(const hf_select_args &a, hipStream_t s) {
    const dim3 grid_pool((unsigned)(a.BH * (a.nqb + a.nkb) + a.prep_tiles + a.app_tiles));
    const int ti_n = (a.nqb + hf::kTile - 1) / hf::kTile, tj_n = (a.nkb + hf::kTile - 1) / hf::kTile;
    const dim3 grid_score((unsigned)(a.BH * ti_n * tj_n));
    const dim3 grid_topk((unsigned)((a.BH * a.nqb + 3) / 4));
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
    // hierarchical: pool (keeping each key block's frame parts), frame means, block and
    // frame scores, then the two-level top-k
    if (a.D == 64) {
        hipLaunchKernelGGL((hf::pool_kernel<64, true>), grid_pool, dim3(256), 0, s, a);
        hipLaunchKernelGGL(hf::score_kernel<64>, grid_score, dim3(64), 0, s, a, scale);
    } else {
        hipLaunchKernelGGL((hf::pool_kernel<128, true>), grid_pool, dim3(256), 0, s, a);
        hipLaunchKernelGGL(hf::score_kernel<128>, grid_score, dim3(64), 0, s, a, scale);
    }
    const dim3 grid_fp((unsigned)(a.BH * a.nfr));
    if (a.D == 64)
        hipLaunchKernelGGL(hf::frame_pool_kernel<64>, grid_fp, dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL(hf::frame_pool_kernel<128>, grid_fp, dim3(128), 0, s, a);
    // frame scores: the score kernel over (query block, frame) pairs
    hf_select_args f = a;
    f.kbar = a.fbar;
    f.nkb = a.nfr;
    f.sc = a.fsc;
    f.scores = a.fscores;
    const dim3 grid_fs((unsigned)(a.BH * ti_n * ((a.nfr + hf::kTile - 1) / hf::kTile)));
    if (a.D == 64)
        hipLaunchKernelGGL(hf::score_kernel<64>, grid_fs, dim3(64), 0, s, f, scale);
    else
        hipLaunchKernelGGL(hf::score_kernel<128>, grid_fs, dim3(64), 0, s, f, scale);
    launch_topk(kpl, grid_topk, a, s);
    return hipGetLastError();
}
