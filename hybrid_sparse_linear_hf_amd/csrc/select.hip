// Block selection for the block-sparse window attention.
//
// [HF-de] §2.A / [HF-pt] §2.A.2 keep only the most important (top-K) key blocks of the
// window for each query block; the importance score is the dot product of the
// mean-pooled query block and the mean-pooled key block ([LF-de] §2.2 token
// compression by mean pooling), scaled by 1/sqrt(D).  Ties go to the lower key block.
//
// Three launches:
//   pool_kernel   HBM-bound: one workgroup per query or key block sums its rows in fp64
//                 (sums of bf16 values are exact in fp64) and stores the block mean.
//   score_kernel  16 x 16 tiles of fp64 scores, each evaluated as sum_d (qbar_d * kbar_d) in
//                 index order with separately rounded products and sums (the pooled
//                 tiles are staged in LDS, every load issued up front).
//   topk_kernel   one wave per query block: radix select of the k-th largest
//                 (score, -index) key and an ascending emit of the kept indices.
#include "hf_internal.h"

namespace hf {
namespace {

__device__ __forceinline__ double bf16_to_f64(uint32_t bits) { return (double)__uint_as_float(bits << 16); }

// Row pointer of window key j (logical order) in the ring.
__device__ __forceinline__ const uint16_t *key_row(const hf_select_args &a, int bh, int j) {
    const int f = j / a.T, t = j - f * a.T;
    int slot = a.head + f;
    if (slot >= a.W) slot -= a.W;
    return a.ring_k + (((size_t)bh * a.W + slot) * a.T + t) * a.D;
}

template <int D>
__global__ __launch_bounds__(256) void pool_kernel(hf_select_args a) {
    constexpr int kVec = D / 8;              // 16-byte vectors per row
    constexpr int kRowsPerPass = 256 / kVec;
    __shared__ double red[kRowsPerPass][D];

    const int per_plane = a.nqb + a.nkb;
    const int bh = blockIdx.x / per_plane;
    const int blk = blockIdx.x % per_plane;
    const bool is_q = blk < a.nqb;
    const int b = is_q ? blk : blk - a.nqb;
    const int bs = is_q ? a.bq : a.bk;
    const int N = is_q ? a.Nq : a.Nk;
    const int r0 = b * bs, r1 = min(r0 + bs, N);

    const int v = threadIdx.x % kVec, ro = threadIdx.x / kVec;
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll 4
    for (int r = r0 + ro; r < r1; r += kRowsPerPass) {
        const uint16_t *row = is_q ? a.q + ((size_t)bh * a.Nq + r) * D : key_row(a, bh, r);
        const u32x4 w = *reinterpret_cast<const u32x4 *>(row + v * 8);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += bf16_to_f64(ws[e] & 0xFFFFu);
            acc[2 * e + 1] += bf16_to_f64(ws[e] >> 16);
        }
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

__device__ __forceinline__ uint64_t order_key(double s) {
    const uint64_t u = (uint64_t)__double_as_longlong(s + 0.0);  // -0 -> +0
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

constexpr int kTile = 16;   // score tile: 16 query blocks x 16 key blocks per workgroup

// Scores of a 16 x 16 tile of (query block, key block) pairs: both pooled tiles are staged
// in LDS (every staging load issued before the first LDS write), then each thread forms one
// dot product as a sequential sum in index order.
template <int D>
__global__ __launch_bounds__(256) void score_kernel(hf_select_args a, double scale) {
    __shared__ double qs[kTile][D + 1];
    __shared__ double ks[kTile][D + 1];
    const int ti_n = (a.nqb + kTile - 1) / kTile, tj_n = (a.nkb + kTile - 1) / kTile;
    const int bh = blockIdx.x / (ti_n * tj_n);
    const int i0 = ((blockIdx.x / tj_n) % ti_n) * kTile, j0 = (blockIdx.x % tj_n) * kTile;
    const int tid = threadIdx.x;
    {
        // rows past the end re-read the last row and are zeroed
        typedef __attribute__((ext_vector_type(2))) double f64x2;
        constexpr int kPer = kTile * D / 2 / 256;       // 16-byte loads per thread per matrix
        f64x2 qv[kPer], kv[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int idx = tid + 256 * e, r = idx / (D / 2), d = 2 * (idx % (D / 2));
            qv[e] = *reinterpret_cast<const f64x2 *>(a.qbar + ((size_t)bh * a.nqb + min(i0 + r, a.nqb - 1)) * D + d);
            kv[e] = *reinterpret_cast<const f64x2 *>(a.kbar + ((size_t)bh * a.nkb + min(j0 + r, a.nkb - 1)) * D + d);
        }
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int idx = tid + 256 * e, r = idx / (D / 2), d = 2 * (idx % (D / 2));
            const bool qok = i0 + r < a.nqb, kok = j0 + r < a.nkb;
            qs[r][d] = qok ? qv[e].x : 0.0;
            qs[r][d + 1] = qok ? qv[e].y : 0.0;
            ks[r][d] = kok ? kv[e].x : 0.0;
            ks[r][d + 1] = kok ? kv[e].y : 0.0;
        }
    }
    __syncthreads();
    const int ti = tid / kTile, tj = tid % kTile;
    const int i = i0 + ti, j = j0 + tj;
    if (i >= a.nqb || j >= a.nkb) return;
    double acc = 0.0;
    {
        // products and sums rounded separately (no fused multiply-add), in index order
#pragma clang fp contract(off)
#pragma unroll 8
        for (int d = 0; d < D; ++d) acc = acc + qs[ti][d] * ks[tj][d];
        acc = acc * scale;
    }
    a.sc[((size_t)bh * a.nqb + i) * a.nkb + j] = acc;
    if (a.scores) a.scores[((size_t)bh * a.nqb + i) * a.nkb + j] = acc;
}

// One wave per (plane, query block): radix select of the k-th largest (score, -index)
// key, then an ascending emit of the kept block indices.  Lane l holds keys of blocks
// l, l + 64, ... in registers (KPL of them).
template <int KPL>
__global__ __launch_bounds__(256) void topk_kernel(hf_select_args a) {
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int row = blockIdx.x * 4 + wave;                    // (bh, i) flattened
    if (row >= a.BH * a.nqb) return;
    const double *src = a.sc + (size_t)row * a.nkb;
    uint64_t key[KPL];
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
        const int j = lane + 64 * e;
        key[e] = j < a.nkb ? order_key(src[j]) : 0;          // 0 is below every real key
    }
    const int k = a.top_k;

    // largest v with #{key >= v} >= k, i.e. the k-th largest key (padding keys are 0 and
    // never counted once v > 0; v = 0 is only reached if fewer than k real keys exist,
    // which the caller's 1 <= k <= n_kb rules out)
    uint64_t prefix = 0;
    for (int bit = 63; bit >= 0; --bit) {
        const uint64_t cand = prefix | (1ull << bit);
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < KPL; ++e) cnt += __popcll(__ballot(key[e] >= cand));
        if (cnt >= k) prefix = cand;
    }
    int gt = 0;
#pragma unroll
    for (int e = 0; e < KPL; ++e) gt += __popcll(__ballot(key[e] > prefix));
    const int need_eq = k - gt;  // >= 1 by construction
    int32_t *out = a.idx + (size_t)row * k;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int written = 0, eq_seen = 0;
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
        const int j = lane + 64 * e;
        const bool valid = j < a.nkb;
        const bool is_gt = valid && key[e] > prefix;
        const bool is_eq = valid && key[e] == prefix;
        const uint64_t eq_b = __ballot(is_eq);
        const int eq_rank = eq_seen + __popcll(eq_b & lt_mask);
        const bool sel = is_gt || (is_eq && eq_rank < need_eq);
        const uint64_t sel_b = __ballot(sel);
        if (sel) out[written + __popcll(sel_b & lt_mask)] = j;
        written += __popcll(sel_b);
        eq_seen += __popcll(eq_b);
    }
}

}  // namespace
}  // namespace hf

hipError_t hf_launch_block_select(const hf_select_args &a, hipStream_t s) {
    const dim3 grid_pool((unsigned)(a.BH * (a.nqb + a.nkb)));
    const int ti_n = (a.nqb + hf::kTile - 1) / hf::kTile, tj_n = (a.nkb + hf::kTile - 1) / hf::kTile;
    const dim3 grid_score((unsigned)(a.BH * ti_n * tj_n));
    const dim3 grid_topk((unsigned)((a.BH * a.nqb + 3) / 4));
    const double scale = 1.0 / sqrt((double)a.D);
    if (a.D == 64) {
        hipLaunchKernelGGL(hf::pool_kernel<64>, grid_pool, dim3(256), 0, s, a);
        hipLaunchKernelGGL(hf::score_kernel<64>, grid_score, dim3(256), 0, s, a, scale);
    } else {
        hipLaunchKernelGGL(hf::pool_kernel<128>, grid_pool, dim3(256), 0, s, a);
        hipLaunchKernelGGL(hf::score_kernel<128>, grid_score, dim3(256), 0, s, a, scale);
    }
    const int kpl = (a.nkb + 63) / 64;
    if (kpl <= 1) hipLaunchKernelGGL(hf::topk_kernel<1>, grid_topk, dim3(256), 0, s, a);
    else if (kpl <= 2) hipLaunchKernelGGL(hf::topk_kernel<2>, grid_topk, dim3(256), 0, s, a);
    else if (kpl <= 3) hipLaunchKernelGGL(hf::topk_kernel<3>, grid_topk, dim3(256), 0, s, a);
    else if (kpl <= 4) hipLaunchKernelGGL(hf::topk_kernel<4>, grid_topk, dim3(256), 0, s, a);
    else if (kpl <= 8) hipLaunchKernelGGL(hf::topk_kernel<8>, grid_topk, dim3(256), 0, s, a);
    else if (kpl <= 16) hipLaunchKernelGGL(hf::topk_kernel<16>, grid_topk, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(hf::topk_kernel<24>, grid_topk, dim3(256), 0, s, a);
    return hipGetLastError();
}
