// Absorb evicted tokens into the linear attention state.
//
// [HF-abs]: a compact key-value state incrementally absorbs the tokens evicted from the
// sliding window; [HF-de] §2.A / [HF-pt] §2.A.1: information of frames leaving the window
// is aggregated into that state through a linear attention.  With feature map
// phi = elu + 1:   S[a][c] += sum_u phi(K_u[a]) V_u[c],   z[a] += sum_u phi(K_u[a]).
//
// gfx950 design (HBM-bound: ~60 flop per byte against a ~315 flop/byte ridge)
//   * The state is cut into 64x64 tiles; each workgroup owns one tile and a contiguous
//     range of 64-token chunks, so a plane's K and V are streamed once per tile row /
//     column pair and the re-reads stay in the XCD's L2.
//   * Per chunk, phi(K) is evaluated in fp32, split into bf16 hi + lo halves and written
//     transposed to LDS; V arrives transposed ([D][T] frames of the ring, or transposed
//     here for row-major input) so both contraction operands are 16-byte LDS reads.  Each
//     of the 4 waves accumulates a 32x32 sub-tile with 2 matrix-core products per 16
//     tokens (hi and lo), keeping fp32-grade accuracy in S.
//   * Token-split partial tiles are reduced by the last workgroup of each tile to finish
//     (integer ticket, no floating-point atomics), always in split order, then added to
//     the old state: the result is deterministic.
#include "hf_internal.h"

namespace hf {
namespace {

constexpr int kChunk = 64;
constexpr int kPitch = kChunk + 8;   // LDS row pitch (bf16) of the transposed tiles
constexpr int kTileElems = 64 * 64;

struct AbsorbGeom {
    int nta;      // 64-wide tiles along a (and along c)
    int P;        // token splits per tile
    int nch;      // 64-token chunks
};

// Splits per tile aim at ~256 workgroups (one per CU) whatever the number of planes.
__host__ __device__ inline int absorb_max_splits(int BH, int D) {
    const int tiles = BH * (D / 64) * (D / 64);
    const int P = (256 + tiles / 2) / tiles;
    return P < 1 ? 1 : P;
}

__host__ __device__ inline AbsorbGeom absorb_geom(int BH, int D, int64_t n_tok) {
    AbsorbGeom g;
    g.nta = D / 64;
    const int64_t nch = (n_tok + kChunk - 1) / kChunk;   // callers keep n_tok * D below 2^31
    g.nch = (int)nch;
    const int P = absorb_max_splits(BH, D);
    g.P = nch < 1 ? 1 : (nch < P ? (int)nch : P);
    return g;
}

// Raw registers of one chunk for one thread: 2 tokens x 8 features of K and of V.
struct ChunkRaw {
    u32x4 k[2];
    u32x4 v[2];
};

template <bool kRing>
struct Src {
    const hf_absorb_args &a;
    int bh;
    // pointer to 8 consecutive K features (a0 .. a0+7) of token u (u < n_tok)
    __device__ const uint16_t *k_row(int64_t u, int a0) const {
        if constexpr (kRing) {
            const int f = (int)(u / a.T), t = (int)(u - (int64_t)f * a.T);
            int slot = a.head + f;
            slot %= a.W;
            return a.ring_k + (((size_t)bh * a.W + slot) * a.T + t) * a.D + a0;
        } else {
            return a.k + ((size_t)bh * a.n_tok + u) * a.D + a0;
        }
    }
};

template <int D, bool kRing>
__device__ __forceinline__ void load_chunk(const hf_absorb_args &a, int bh, int64_t u0, int a0, int c0, int tid,
                                           ChunkRaw &r) {
    const int pr = tid >> 3, sub = tid & 7;
    const Src<kRing> src{a, bh};
    // K: tokens u0 + 2*pr + {0,1}, features a0 + 8*sub ..
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int64_t u = u0 + 2 * pr + e;
        r.k[e] = u < a.n_tok ? *reinterpret_cast<const u32x4 *>(src.k_row(u, a0 + 8 * sub)) : u32x4{0, 0, 0, 0};
    }
    if constexpr (kRing) {
        // V^T rows c0 + pr + 32e, tokens u0 + 8*sub .. +8 (one frame: T % 8 == 0)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int64_t u = u0 + 8 * sub;
            if (u < a.n_tok) {
                const int f = (int)(u / a.T), t = (int)(u - (int64_t)f * a.T);
                const int slot = (a.head + f) % a.W;
                const uint16_t *p = a.ring_vt + ((size_t)bh * a.W + slot) * (size_t)D * a.T +
                                    (size_t)(c0 + pr + 32 * e) * a.T + t;
                r.v[e] = *reinterpret_cast<const u32x4 *>(p);
            } else {
                r.v[e] = u32x4{0, 0, 0, 0};
            }
        }
    } else {
        // V rows: tokens u0 + 2*pr + {0,1}, features c0 + 8*sub ..
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int64_t u = u0 + 2 * pr + e;
            r.v[e] = u < a.n_tok ? *reinterpret_cast<const u32x4 *>(a.v + ((size_t)bh * a.n_tok + u) * D + c0 + 8 * sub)
                                 : u32x4{0, 0, 0, 0};
        }
    }
}

template <int D, bool kRing>
__global__ __launch_bounds__(256) void absorb_kernel(hf_absorb_args a, int per_xcd) {
    __shared__ __align__(16) uint16_t kh[64][kPitch];
    __shared__ __align__(16) uint16_t kl[64][kPitch];
    __shared__ __align__(16) uint16_t vt[64][kPitch];
    __shared__ float zred[32][65];
    __shared__ int s_last;

    const AbsorbGeom geo = absorb_geom(a.BH, D, a.n_tok);
    const int items = a.BH * geo.nta * geo.nta * geo.P;
    const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (item >= items) return;
    const int p = item % geo.P;
    const int tile = item / geo.P;                 // (bh, qa, qc)
    const int qc = tile % geo.nta, qa = (tile / geo.nta) % geo.nta, bh = tile / (geo.nta * geo.nta);
    const int a0 = 64 * qa, c0 = 64 * qc;
    const int ch0 = (int)((int64_t)p * geo.nch / geo.P), ch1 = (int)((int64_t)(p + 1) * geo.nch / geo.P);
    const bool do_z = (qc == 0);

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 31, g = lane >> 5;
    const int ta = w >> 1, tc = w & 1;
    const int pr = tid >> 3, sub = tid & 7;

    f32x16 acc = {};
    float zacc[8] = {0, 0, 0, 0, 0, 0, 0, 0};

    ChunkRaw cur, nxt;
    if (ch0 < ch1) load_chunk<D, kRing>(a, bh, (int64_t)ch0 * kChunk, a0, c0, tid, cur);
    for (int ch = ch0; ch < ch1; ++ch) {
        if (ch + 1 < ch1) load_chunk<D, kRing>(a, bh, (int64_t)(ch + 1) * kChunk, a0, c0, tid, nxt);
        const int64_t u0 = (int64_t)ch * kChunk;
        // phi(K) -> hi/lo bf16, transposed into LDS: kh[a][u]
        {
            const bool ok0 = u0 + 2 * pr < a.n_tok, ok1 = u0 + 2 * pr + 1 < a.n_tok;
            const uint32_t w0[4] = {cur.k[0].x, cur.k[0].y, cur.k[0].z, cur.k[0].w};
            const uint32_t w1[4] = {cur.k[1].x, cur.k[1].y, cur.k[1].z, cur.k[1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t b0 = (e & 1) ? (w0[e >> 1] >> 16) : (w0[e >> 1] & 0xFFFFu);
                const uint32_t b1 = (e & 1) ? (w1[e >> 1] >> 16) : (w1[e >> 1] & 0xFFFFu);
                const float f0 = ok0 ? phi_f32(__uint_as_float(b0 << 16)) : 0.f;
                const float f1 = ok1 ? phi_f32(__uint_as_float(b1 << 16)) : 0.f;
                zacc[e] += f0;
                zacc[e] += f1;
                const uint32_t h0 = f32_to_bf16_bits(f0), h1 = f32_to_bf16_bits(f1);
                const uint32_t l0 = f32_to_bf16_bits(f0 - __uint_as_float(h0 << 16));
                const uint32_t l1 = f32_to_bf16_bits(f1 - __uint_as_float(h1 << 16));
                *reinterpret_cast<uint32_t *>(&kh[8 * sub + e][2 * pr]) = h0 | (h1 << 16);
                *reinterpret_cast<uint32_t *>(&kl[8 * sub + e][2 * pr]) = l0 | (l1 << 16);
            }
        }
        if constexpr (kRing) {
#pragma unroll
            for (int e = 0; e < 2; ++e) *reinterpret_cast<u32x4 *>(&vt[pr + 32 * e][8 * sub]) = cur.v[e];
        } else {
            const uint32_t w0[4] = {cur.v[0].x, cur.v[0].y, cur.v[0].z, cur.v[0].w};
            const uint32_t w1[4] = {cur.v[1].x, cur.v[1].y, cur.v[1].z, cur.v[1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t b0 = (e & 1) ? (w0[e >> 1] >> 16) : (w0[e >> 1] & 0xFFFFu);
                const uint32_t b1 = (e & 1) ? (w1[e >> 1] >> 16) : (w1[e >> 1] & 0xFFFFu);
                *reinterpret_cast<uint32_t *>(&vt[8 * sub + e][2 * pr]) = b0 | (b1 << 16);
            }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < kChunk / 16; ++s) {
            const bf16x8 ah = as_bf16x8(*reinterpret_cast<const u32x4 *>(&kh[32 * ta + n][16 * s + 8 * g]));
            const bf16x8 al = as_bf16x8(*reinterpret_cast<const u32x4 *>(&kl[32 * ta + n][16 * s + 8 * g]));
            const bf16x8 bv = as_bf16x8(*reinterpret_cast<const u32x4 *>(&vt[32 * tc + n][16 * s + 8 * g]));
            acc = mfma32(ah, bv, acc);
            acc = mfma32(al, bv, acc);
        }
        __syncthreads();
        cur = nxt;
    }

    // z partial of this split: features a0 + 8*sub + e summed over the 32 token pairs
    if (do_z) {
#pragma unroll
        for (int e = 0; e < 8; ++e) zred[pr][8 * sub + e] = zacc[e];
    }
    __syncthreads();
    float zsum = 0.f;
    if (do_z && tid < 64)
        for (int k = 0; k < 32; ++k) zsum += zred[k][tid];

    // accumulator slot i holds row a0 + 32*ta + 8*(i/4) + 4*g + i%4, column c0 + 32*tc + n
    float *Sp = a.S + (size_t)bh * D * D;
    if (geo.P == 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = a0 + 32 * ta + 8 * (i >> 2) + 4 * g + (i & 3);
            float *dst = Sp + (size_t)r * D + c0 + 32 * tc + n;
            *dst = *dst + acc[i];
        }
        if (do_z && tid < 64) a.z[(size_t)bh * D + a0 + tid] += zsum;
        return;
    }

    float *part = a.part + (size_t)item * kTileElems + w * 1024 + lane;
#pragma unroll
    for (int i = 0; i < 16; ++i) part[i * 64] = acc[i];
    float *zpart = a.part + (size_t)items * kTileElems + ((size_t)(bh * geo.nta + qa) * geo.P + p) * 64;
    if (do_z && tid < 64) zpart[tid] = zsum;

    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&a.counters[tile], 1u) == (unsigned)(geo.P - 1));
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    float sum[16];
    const float *pt = a.part + (size_t)tile * geo.P * kTileElems + w * 1024 + lane;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum[i] = pt[i * 64];
    for (int q = 1; q < geo.P; ++q) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sum[i] += pt[(size_t)q * kTileElems + i * 64];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = a0 + 32 * ta + 8 * (i >> 2) + 4 * g + (i & 3);
        float *dst = Sp + (size_t)r * D + c0 + 32 * tc + n;
        *dst = *dst + sum[i];
    }
    if (do_z && tid < 64) {
        const float *zp = a.part + (size_t)items * kTileElems + (size_t)(bh * geo.nta + qa) * geo.P * 64 + tid;
        float zs = zp[0];
        for (int q = 1; q < geo.P; ++q) zs += zp[(size_t)q * 64];
        a.z[(size_t)bh * D + a0 + tid] += zs;
    }
    if (tid == 0) atomicExch(&a.counters[tile], 0u);
}

}  // namespace
}  // namespace hf

// Workspace bytes of one absorb call over n_tok tokens: tile counters (padded to 256
// bytes), then P partial 64x64 tiles per state tile, then P partial z slices per 64 rows.
size_t hf_absorb_required_bytes(int BH, int D, int64_t n_tok) {
    const hf::AbsorbGeom g = hf::absorb_geom(BH, D, n_tok);
    const size_t tiles = (size_t)BH * g.nta * g.nta;
    const size_t counters = (tiles * sizeof(uint32_t) + 255) & ~(size_t)255;
    const size_t part = tiles * g.P * hf::kTileElems * sizeof(float) + (size_t)BH * g.nta * g.P * 64 * sizeof(float);
    return counters + part;
}

// Upper bound of hf_absorb_required_bytes over every token count.
size_t hf_absorb_workspace_bytes(int BH, int D) {
    const size_t tiles = (size_t)BH * (D / 64) * (D / 64);
    const size_t P = (size_t)hf::absorb_max_splits(BH, D);
    const size_t counters = (tiles * sizeof(uint32_t) + 255) & ~(size_t)255;
    return counters + tiles * P * hf::kTileElems * sizeof(float) + (size_t)BH * (D / 64) * P * 64 * sizeof(float);
}

hipError_t hf_launch_absorb(const hf_absorb_args &a, hipStream_t s) {
    if (a.n_tok <= 0) return hipSuccess;
    const hf::AbsorbGeom g = hf::absorb_geom(a.BH, a.D, a.n_tok);
    const int items = a.BH * g.nta * g.nta * g.P;
    const int per_xcd = (items + 7) / 8;
    const dim3 grid((unsigned)(per_xcd * 8));
    const bool ring = a.ring_k != nullptr;
    if (a.D == 64) {
        if (ring)
            hipLaunchKernelGGL((hf::absorb_kernel<64, true>), grid, dim3(256), 0, s, a, per_xcd);
        else
            hipLaunchKernelGGL((hf::absorb_kernel<64, false>), grid, dim3(256), 0, s, a, per_xcd);
    } else {
        if (ring)
            hipLaunchKernelGGL((hf::absorb_kernel<128, true>), grid, dim3(256), 0, s, a, per_xcd);
        else
            hipLaunchKernelGGL((hf::absorb_kernel<128, false>), grid, dim3(256), 0, s, a, per_xcd);
    }
    return hipGetLastError();
}
