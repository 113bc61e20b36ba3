// Block selection for the block-sparse window attention.
//
// [HF-de] §2.A / [HF-pt] §2.A.2 keep only the most important (top-K) key blocks of the
// window for each query block; the importance score is the dot product of the
// mean-pooled query block and the mean-pooled key block ([LF-de] §2.2 token
// compression by mean pooling), scaled by 1/sqrt(D).  Ties go to the lower key block.
//
// Two launches:
//   pool_kernel   HBM-bound: one workgroup per query or key block sums its rows in fp64
//                 (sums of bf16 values are exact in fp64) and stores the block mean.
//   score_topk    one workgroup per (plane, 4 query blocks): fp64 scores against every
//                 key block, evaluated as sum_d (qbar_d * kbar_d) in index order with
//                 separately rounded products and sums, then a wavefront radix select
//                 of the k-th largest (score, -index) key and an ascending emit.
#include "hf_internal.h"

namespace hf {
namespace {

constexpr int kQPerWG = 4;  // query blocks per score_topk workgroup (one wave each)

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

template <int D>
__global__ __launch_bounds__(256) void score_topk_kernel(hf_select_args a, double scale) {
    extern __shared__ __align__(16) unsigned char smem[];
    double *qb = reinterpret_cast<double *>(smem);                 // [kQPerWG][D]
    uint64_t *keys = reinterpret_cast<uint64_t *>(qb + kQPerWG * D);  // [kQPerWG][nkb]

    const int groups = (a.nqb + kQPerWG - 1) / kQPerWG;
    const int bh = blockIdx.x / groups;
    const int i0 = (blockIdx.x % groups) * kQPerWG;
    const int nq = min(kQPerWG, a.nqb - i0);

    for (int e = threadIdx.x; e < kQPerWG * D; e += 256) {
        const int g = e / D;
        qb[e] = g < nq ? a.qbar[((size_t)bh * a.nqb + i0 + g) * D + e % D] : 0.0;
    }
    __syncthreads();

    // scores: thread per key block, all query blocks of the group at once
    for (int j = threadIdx.x; j < a.nkb; j += 256) {
        // products and sums rounded separately (no fused multiply-add), as in the definition
#pragma clang fp contract(off)
        const double *kb = a.kbar + ((size_t)bh * a.nkb + j) * D;
        double acc[kQPerWG];
#pragma unroll
        for (int g = 0; g < kQPerWG; ++g) acc[g] = 0.0;
#pragma unroll 1
        for (int d0 = 0; d0 < D; d0 += 8) {
            double kv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) kv[e] = kb[d0 + e];
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int g = 0; g < kQPerWG; ++g) acc[g] = acc[g] + qb[g * D + d0 + e] * kv[e];
        }
#pragma unroll
        for (int g = 0; g < kQPerWG; ++g) {
            if (g < nq) {
                const double s = acc[g] * scale;
                if (a.scores) a.scores[((size_t)bh * a.nqb + i0 + g) * a.nkb + j] = s;
                keys[g * a.nkb + j] = order_key(s);
            }
        }
    }
    __syncthreads();

    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    if (wave >= nq) return;
    const uint64_t *K = keys + wave * a.nkb;
    const int k = a.top_k;

    // radix select: largest v with #{key >= v} >= k, i.e. the k-th largest key
    uint64_t prefix = 0;
    for (int bit = 63; bit >= 0; --bit) {
        const uint64_t cand = prefix | (1ull << bit);
        int cnt = 0;
        for (int j0 = 0; j0 < a.nkb; j0 += 64) {
            const int j = j0 + lane;
            cnt += __popcll(__ballot(j < a.nkb && K[j] >= cand));
        }
        if (cnt >= k) prefix = cand;
    }
    int gt = 0;
    for (int j0 = 0; j0 < a.nkb; j0 += 64) {
        const int j = j0 + lane;
        gt += __popcll(__ballot(j < a.nkb && K[j] > prefix));
    }
    const int need_eq = k - gt;  // >= 1 by construction
    int32_t *out = a.idx + ((size_t)bh * a.nqb + i0 + wave) * k;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int written = 0, eq_seen = 0;
    for (int j0 = 0; j0 < a.nkb; j0 += 64) {
        const int j = j0 + lane;
        const bool valid = j < a.nkb;
        const uint64_t key = valid ? K[j] : 0;
        const bool is_gt = valid && key > prefix;
        const bool is_eq = valid && key == prefix;
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
    const int groups = (a.nqb + hf::kQPerWG - 1) / hf::kQPerWG;
    const dim3 grid_sel((unsigned)(a.BH * groups));
    const size_t smem = (size_t)hf::kQPerWG * a.D * sizeof(double) + (size_t)hf::kQPerWG * a.nkb * sizeof(uint64_t);
    const double scale = 1.0 / sqrt((double)a.D);
    if (a.D == 64) {
        hipLaunchKernelGGL(hf::pool_kernel<64>, grid_pool, dim3(256), 0, s, a);
        hipLaunchKernelGGL(hf::score_topk_kernel<64>, grid_sel, dim3(256), smem, s, a, scale);
    } else {
        hipLaunchKernelGGL(hf::pool_kernel<128>, grid_pool, dim3(256), 0, s, a);
        hipLaunchKernelGGL(hf::score_topk_kernel<128>, grid_sel, dim3(256), smem, s, a, scale);
    }
    return hipGetLastError();
}
