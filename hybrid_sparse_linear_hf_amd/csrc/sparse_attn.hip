// Block-sparse window attention with the linear readout fused into its epilogue.
//
// Sparse branch ([HF-de] §2.A "Block-Sparse Sliding Window Attention", [HF-pt] §2.A.2):
// every query of query block i attends with softmax weights to the keys of its kept key
// blocks only.  Linear branch ([HF-de] §2.A "Lineare Zeit-Aufmerksamkeit", [HF-pt]
// §2.A.1, [HF-abs]): phi(q)^T S / (phi(q) . z + eps) from the compact state.  The output
// is their sum ([HF-de] §2.A "Kombination", [HF-pt] §2.A "Resultado").
//
// gfx950 design
//   * One wavefront per (plane, query block) owns up to 64 queries as two 32-column
//     tiles.  It computes S^T = K Q^T and O^T += V^T P^T on 32x32x16 bf16 matrix cores,
//     so the softmax probabilities leave the first product already in the register
//     layout the second product consumes (no LDS round trip, no lane shuffles).
//   * Key rows feed the first product's A operand in the order perm32(m), which makes
//     each lane hold 16 consecutive keys of its query; the second product's contraction
//     index is matched to those keys, and value frames are stored transposed ([D][T]) in
//     the ring, so every operand is a single 16-byte load straight from global memory.
//   * fp32 online softmax in base 2 with the 1/sqrt(D) scale folded into one FMA; the
//     running maximum is only raised when a tile exceeds it by more than 2^8, so the
//     accumulator rescale is rare.
//   * The next kept 32-key subtile is loaded while the current one is computed.
//   * Workgroup ids are remapped so that the query blocks of one plane run on one XCD
//     and share its L2 for the window's K/V.
#include "hf_internal.h"

namespace hf {
namespace {

constexpr float kLazyRescaleLog2 = 8.0f;

template <int D>
struct KVFrag {
    u32x4 k[D / 16];          // K rows: A operand of S^T, contraction over d
    u32x4 v[D / 32][2];       // V^T rows: A operand of O^T, contraction over keys
};

__device__ __forceinline__ int div_T(int n, uint32_t magic, int T) {
    int q = (int)__umulhi((uint32_t)n, magic);
    q -= (q * T > n);
    return q;
}

template <int D>
__device__ __forceinline__ void load_kv(const hf_attn_args &a, uint32_t magicT, int bh, int key0, int kend,
                                        int n, int g, KVFrag<D> &f) {
    // K: lane supplies key key0 + perm32(n), d range [16s + 8g, +8)
    int key = key0 + perm32(n);
    if (key >= kend) key = key0;
    int fr = div_T(key, magicT, a.T);
    int t = key - fr * a.T;
    int slot = a.head + fr;
    if (slot >= a.W) slot -= a.W;
    const uint16_t *kp = a.ring_k + (((size_t)bh * a.W + slot) * a.T + t) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) f.k[s] = *reinterpret_cast<const u32x4 *>(kp + 16 * s);
    // V^T: lane supplies d = 32*dt + perm32(n), keys [key0 + 16g + 8ks, +8)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        int k8 = key0 + 16 * g + 8 * ks;
        if (k8 >= kend) k8 = key0;
        int fv = div_T(k8, magicT, a.T);
        int tv = k8 - fv * a.T;
        int sv = a.head + fv;
        if (sv >= a.W) sv -= a.W;
        const uint16_t *vp = a.ring_vt + ((size_t)bh * a.W + sv) * (size_t)D * a.T + tv;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
            f.v[dt][ks] = *reinterpret_cast<const u32x4 *>(vp + (size_t)(32 * dt + perm32(n)) * a.T);
    }
}

template <int D, int QT>
__global__ __launch_bounds__(64) void sparse_attn_kernel(hf_attn_args a, uint32_t magicT, float c_log2,
                                                         int per_xcd) {
    const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (item >= a.BH * a.nqb) return;
    const int bh = item / a.nqb, qb = item - bh * a.nqb;
    const int lane = threadIdx.x, n = lane & 31, g = lane >> 5;
    const int q0 = qb * a.bq, qend = min(q0 + a.bq, a.Nq);

    // Q^T fragments (B operand): query column n of tile qt, d range [16s + 8g, +8).  They
    // are parked in a per-lane LDS slot (conflict-free 16-byte reads) to leave the
    // registers to the double-buffered K/V fragments and the accumulators.
    __shared__ u32x4 qs[QT][D / 16][64];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        int row = q0 + 32 * qt + n;
        if (row >= qend) row = q0;
        const uint16_t *qp = a.q + ((size_t)bh * a.Nq + row) * D + 8 * g;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qs[qt][s][lane] = *reinterpret_cast<const u32x4 *>(qp + 16 * s);
    }

    f32x16 acc[QT][D / 32];
    float m[QT], l[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        m[qt] = -INFINITY;
        l[qt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[qt][dt] = f32x16{};
    }

    const int32_t *sel = a.idx + ((size_t)bh * a.nqb + qb) * a.top_k;
    const int nsub = (a.bk + 31) / 32;
    const int total = a.top_k * nsub;

    // subtile it -> [key0, kend)
    auto subtile = [&](int it, int &key0, int &kend) {
        const int r = it / nsub, st = it - r * nsub;
        // out-of-range indices (a caller error) are clamped so that no load leaves the window
        const int j = min(max(__builtin_amdgcn_readfirstlane(sel[r]), 0), a.nkb - 1);
        key0 = j * a.bk + 32 * st;
        kend = min(min(j * a.bk + a.bk, a.Nk), key0 + 32);
    };

    KVFrag<D> cur, nxt;
    int key0, kend, nkey0 = 0, nkend = 0;
    subtile(0, key0, kend);
    if (kend > key0) load_kv<D>(a, magicT, bh, key0, kend, n, g, cur);

    for (int it = 0; it < total; ++it) {
        if (it + 1 < total) {
            subtile(it + 1, nkey0, nkend);
            if (nkend > nkey0) load_kv<D>(a, magicT, bh, nkey0, nkend, n, g, nxt);
        }
        if (kend > key0) {
            const int nvalid = kend - key0;
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                f32x16 sc = {};
#pragma unroll
                for (int s = 0; s < D / 16; ++s) sc = mfma32(as_bf16x8(cur.k[s]), as_bf16x8(qs[qt][s][lane]), sc);
                if (nvalid < 32) {
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (16 * g + i >= nvalid) sc[i] = -INFINITY;
                }
                float mx = sc[0];
#pragma unroll
                for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const bool raise = (mx - m[qt]) * c_log2 > kLazyRescaleLog2;
                if (__any(raise)) {
                    const float mn = fmaxf(m[qt], mx);
                    const float alpha = __builtin_amdgcn_exp2f((m[qt] - mn) * c_log2);
                    m[qt] = mn;
                    l[qt] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                        for (int i = 0; i < 16; ++i) acc[qt][dt][i] *= alpha;
                }
                const float mc = m[qt] * c_log2;
                float p[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], c_log2, -mc));
                    l[qt] += p[i];
                }
                u32x4 pf[2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    pf[ks].x = pack_bf16x2(p[8 * ks + 0], p[8 * ks + 1]);
                    pf[ks].y = pack_bf16x2(p[8 * ks + 2], p[8 * ks + 3]);
                    pf[ks].z = pack_bf16x2(p[8 * ks + 4], p[8 * ks + 5]);
                    pf[ks].w = pack_bf16x2(p[8 * ks + 6], p[8 * ks + 7]);
                }
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        acc[qt][dt] = mfma32(as_bf16x8(cur.v[dt][ks]), as_bf16x8(pf[ks]), acc[qt][dt]);
            }
        }
        cur = nxt;
        key0 = nkey0;
        kend = nkend;
    }

    // ---- epilogue: normalise, add the linear readout, store fp32
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const float lt = l[qt] + __shfl_xor(l[qt], 32);
        const float inv_l = 1.f / lt;
        const int row = q0 + 32 * qt + n;
        const bool row_ok = row < qend;
        float *op = a.out + ((size_t)bh * a.Nq + (row_ok ? row : q0)) * D + 16 * g;

        if (a.S) {
            // phi(q) as the B operand (same fragment layout as Q^T) and the normaliser
            u32x4 pq[D / 16];
            float den = 0.f;
            const float *zp = a.z + (size_t)bh * D + 8 * g;
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const u32x4 qv = qs[qt][s][lane];
                const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
                const f32x4 z0 = *reinterpret_cast<const f32x4 *>(zp + 16 * s);
                const f32x4 z1 = *reinterpret_cast<const f32x4 *>(zp + 16 * s + 4);
                const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
                float ph[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ph[2 * e] = phi_f32(bf16_lo_to_f32(w[e]));
                    ph[2 * e + 1] = phi_f32(bf16_hi_to_f32(w[e]));
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) den += ph[e] * zz[e];
                pq[s].x = pack_bf16x2(ph[0], ph[1]);
                pq[s].y = pack_bf16x2(ph[2], ph[3]);
                pq[s].z = pack_bf16x2(ph[4], ph[5]);
                pq[s].w = pack_bf16x2(ph[6], ph[7]);
            }
            den += __shfl_xor(den, 32);
            const float inv_den = 1.f / (den + a.eps);
            const uint16_t *stp = a.st + (size_t)bh * D * D + 8 * g;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                f32x16 lin = {};
                const uint16_t *srow = stp + (size_t)(32 * dt + perm32(n)) * D;
#pragma unroll
                for (int s = 0; s < D / 16; ++s)
                    lin = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(srow + 16 * s)), as_bf16x8(pq[s]), lin);
                if (row_ok) {
                    f32x4 *o4 = reinterpret_cast<f32x4 *>(op + 32 * dt);
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        o4[v] = f32x4{acc[qt][dt][4 * v] * inv_l + lin[4 * v] * inv_den,
                                      acc[qt][dt][4 * v + 1] * inv_l + lin[4 * v + 1] * inv_den,
                                      acc[qt][dt][4 * v + 2] * inv_l + lin[4 * v + 2] * inv_den,
                                      acc[qt][dt][4 * v + 3] * inv_l + lin[4 * v + 3] * inv_den};
                }
            }
        } else if (row_ok) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                f32x4 *o4 = reinterpret_cast<f32x4 *>(op + 32 * dt);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    o4[v] = f32x4{acc[qt][dt][4 * v] * inv_l, acc[qt][dt][4 * v + 1] * inv_l,
                                  acc[qt][dt][4 * v + 2] * inv_l, acc[qt][dt][4 * v + 3] * inv_l};
            }
        }
    }
}

// S fp32 [BH][a][c] -> S^T bf16 [BH][c][a] (the A operand layout of the readout product)
template <int D>
__global__ __launch_bounds__(256) void state_transpose_kernel(const float *S, uint16_t *st) {
    __shared__ float tile[32][33];
    const int tiles = D / 32;
    const int bh = blockIdx.x / (tiles * tiles);
    const int ta = (blockIdx.x / tiles) % tiles, tc = blockIdx.x % tiles;
    const float *src = S + (size_t)bh * D * D;
    uint16_t *dst = st + (size_t)bh * D * D;
    const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;
    for (int r = ty; r < 32; r += 8) tile[r][tx] = src[(size_t)(32 * ta + r) * D + 32 * tc + tx];
    __syncthreads();
    for (int r = ty; r < 32; r += 8)
        dst[(size_t)(32 * tc + r) * D + 32 * ta + tx] = (uint16_t)f32_to_bf16_bits(tile[tx][r]);
}

}  // namespace
}  // namespace hf

hipError_t hf_launch_sparse_attn(const hf_attn_args &a, hipStream_t s) {
    if (a.S) {
        const int tiles = a.D / 32;
        const dim3 g((unsigned)(a.BH * tiles * tiles));
        if (a.D == 64)
            hipLaunchKernelGGL(hf::state_transpose_kernel<64>, g, dim3(256), 0, s, a.S, a.st);
        else
            hipLaunchKernelGGL(hf::state_transpose_kernel<128>, g, dim3(256), 0, s, a.S, a.st);
    }
    const int items = a.BH * a.nqb;
    const int per_xcd = (items + 7) / 8;
    const dim3 grid((unsigned)(per_xcd * 8));
    const uint32_t magicT = (uint32_t)((0x100000000ull + (uint64_t)a.T - 1) / (uint64_t)a.T);
    const float c_log2 = (float)(1.4426950408889634 / sqrt((double)a.D));
    const bool two = a.bq > 32;
    if (a.D == 64) {
        if (two)
            hipLaunchKernelGGL((hf::sparse_attn_kernel<64, 2>), grid, dim3(64), 0, s, a, magicT, c_log2, per_xcd);
        else
            hipLaunchKernelGGL((hf::sparse_attn_kernel<64, 1>), grid, dim3(64), 0, s, a, magicT, c_log2, per_xcd);
    } else {
        if (two)
            hipLaunchKernelGGL((hf::sparse_attn_kernel<128, 2>), grid, dim3(64), 0, s, a, magicT, c_log2, per_xcd);
        else
            hipLaunchKernelGGL((hf::sparse_attn_kernel<128, 1>), grid, dim3(64), 0, s, a, magicT, c_log2, per_xcd);
    }
    return hipGetLastError();
}
