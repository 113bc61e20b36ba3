// Absorb evicted tokens into the linear attention state.
//
// [HF-abs]: a compact key-value state incrementally absorbs the tokens evicted from the
// sliding window; [HF-de] §2.A / [HF-pt] §2.A.1: information of frames leaving the window
// is aggregated into that state through a linear attention.  With feature map
// phi = elu + 1:   S[a][c] += sum_u phi(K_u[a]) V_u[c],   z[a] += sum_u phi(K_u[a]).
//
// gfx950 design (HBM-bound: ~60 flop per byte against a ~315 flop/byte ridge)
//   * absorb_partial: each workgroup owns 64 rows of S (all D columns) and a contiguous
//     range of 64-token chunks, so phi(K) is evaluated exactly once per element; it
//     writes its 64 x D partial sum and its 64 partial z values to the workspace.  No
//     workgroup waits for another: no fences, counters or atomics.
//   * Chunks are pipelined: registers hold the loads of the next two chunks while the
//     matrix cores consume a double-buffered LDS stage.
//   * phi(K) is evaluated in fp32, split into bf16 hi + lo halves and written transposed to
//     LDS; V arrives transposed ([D][T] frames of the ring, or transposed here for row-major
//     input), so both contraction operands are 16-byte LDS reads.  The 16-byte groups of
//     each LDS row are XOR-swizzled by the row so the transposing writes spread over all
//     banks.  Two matrix-core products per 16 tokens (hi and lo) keep fp32-grade accuracy.
//   * The partials are summed in split order and added to the old state by the state
//     pass (state.hip), standalone or fused with the preparation that precedes the
//     attention kernel of a hybrid step.  The result is deterministic and independent of
//     the token source (ring or row-major buffers).
#include "hf_internal.h"

namespace hf {
namespace {

constexpr int kChunk = 64;
constexpr int kPitch = kChunk + 8;   // LDS row pitch (bf16) of the transposed tiles

// Raw registers of one chunk for one thread: 2 tokens x 8 features of K, and D/32
// 16-byte vectors of V.
template <int D>
struct ChunkRaw {
    u32x4 k[2];
    u32x4 v[D / 32];
};

// Loads of one chunk.  Token indices past n_tok are clamped to the last token (valid,
// finite data; their phi(K) is zeroed when staged), so the loads are branch-free.
template <int D, bool kRing>
__device__ __forceinline__ void load_chunk(const hf_absorb_args &a, int bh, int u0, int a0, int tid,
                                           ChunkRaw<D> &r) {
    const int pr = tid >> 3, sub = tid & 7;
    const int nt = (int)a.n_tok;
    // K: tokens u0 + 2*pr + {0,1}, features a0 + 8*sub ..
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int u = min(u0 + 2 * pr + e, nt - 1);
        size_t row;
        if constexpr (kRing) {
            const int f = fast_div(u, a.magicT, a.T);
            int slot = a.head + f;
            if (slot >= a.W) slot -= a.W;
            row = ((size_t)bh * a.W + slot) * a.T + (u - f * a.T);
        } else {
            row = (size_t)bh * nt + u;
        }
        r.k[e] = *reinterpret_cast<const u32x4 *>((kRing ? a.ring_k : a.k) + row * D + a0 + 8 * sub);
    }
    if constexpr (kRing) {
        // V^T rows pr + 32e, tokens u0 + 8*sub .. +8 (within one frame: T % 8 == 0 and the
        // evicted range is a whole number of frames)
        const int u = min(u0 + 8 * sub, nt - 8);
        const int f = fast_div(u, a.magicT, a.T);
        int slot = a.head + f;
        if (slot >= a.W) slot -= a.W;
        const uint16_t *p = a.ring_vt + ((size_t)bh * a.W + slot) * (size_t)D * a.T + (u - f * a.T);
#pragma unroll
        for (int e = 0; e < D / 32; ++e) r.v[e] = *reinterpret_cast<const u32x4 *>(p + (size_t)(pr + 32 * e) * a.T);
    } else {
        // V rows: tokens u0 + 2*pr + (e & 1), features 64*(e >> 1) + 8*sub ..
#pragma unroll
        for (int e = 0; e < D / 32; ++e) {
            const int u = min(u0 + 2 * pr + (e & 1), nt - 1);
            r.v[e] = *reinterpret_cast<const u32x4 *>(a.v + ((size_t)bh * nt + u) * D + 64 * (e >> 1) + 8 * sub);
        }
    }
}

__device__ __forceinline__ uint32_t word(const u32x4 &v, int e) {
    return e < 2 ? (e == 0 ? v.x : v.y) : (e == 2 ? v.z : v.w);
}

// Element column of token u in LDS row `row`: 16-byte groups XOR-swizzled by row / 8.
__device__ __forceinline__ int swz(int row, int u) { return ((((u >> 3) ^ (row >> 3)) & 7) << 3) | (u & 7); }

template <int D>
struct Stage {
    uint16_t kh[64][kPitch];   // phi(K)^T, bf16 high half: [feature a][token]
    uint16_t kl[64][kPitch];   // phi(K)^T, bf16 low half
    uint16_t vt[D][kPitch];    // V^T: [feature c][token]
};

// Registers -> LDS stage for the chunk starting at token u0 (tokens >= nt contribute 0).
template <int D, bool kRing>
__device__ __forceinline__ void store_chunk(const ChunkRaw<D> &cur, Stage<D> &st, int u0, int nt, int tid,
                                            float *zacc) {
    const int pr = tid >> 3, sub = tid & 7;
    const bool ok0 = u0 + 2 * pr < nt, ok1 = u0 + 2 * pr + 1 < nt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t w0 = word(cur.k[0], e), w1 = word(cur.k[1], e);
        float f0[2], f1[2];
        f0[0] = ok0 ? phi_f32(bf16_lo_to_f32(w0)) : 0.f;
        f0[1] = ok0 ? phi_f32(bf16_hi_to_f32(w0)) : 0.f;
        f1[0] = ok1 ? phi_f32(bf16_lo_to_f32(w1)) : 0.f;
        f1[1] = ok1 ? phi_f32(bf16_hi_to_f32(w1)) : 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            zacc[2 * e + h] += f0[h];
            zacc[2 * e + h] += f1[h];
            const int row = 8 * sub + 2 * e + h;
            const uint32_t hi = pack_bf16x2(f0[h], f1[h]);            // (token 2pr, token 2pr+1)
            const uint32_t lo = pack_bf16x2(f0[h] - bf16_lo_to_f32(hi), f1[h] - bf16_hi_to_f32(hi));
            *reinterpret_cast<uint32_t *>(&st.kh[row][swz(row, 2 * pr)]) = hi;
            *reinterpret_cast<uint32_t *>(&st.kl[row][swz(row, 2 * pr)]) = lo;
        }
    }
    if constexpr (kRing) {
#pragma unroll
        for (int e = 0; e < D / 32; ++e) {
            const int row = pr + 32 * e;
            *reinterpret_cast<u32x4 *>(&st.vt[row][swz(row, 8 * sub)]) = cur.v[e];
        }
    } else {
#pragma unroll
        for (int e2 = 0; e2 < D / 64; ++e2) {
            const u32x4 &t0 = cur.v[2 * e2], &t1 = cur.v[2 * e2 + 1];   // tokens 2pr, 2pr+1
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w0 = word(t0, e), w1 = word(t1, e);
                const int r0 = 64 * e2 + 8 * sub + 2 * e, r1 = r0 + 1;
                *reinterpret_cast<uint32_t *>(&st.vt[r0][swz(r0, 2 * pr)]) = (w0 & 0xFFFFu) | (w1 << 16);
                *reinterpret_cast<uint32_t *>(&st.vt[r1][swz(r1, 2 * pr)]) = (w0 >> 16) | (w1 & 0xFFFF0000u);
            }
        }
    }
}

// Wave w: rows 32*(w & 1) .. +32 of the 64-row block, columns (w >> 1)*(D/2) .. + D/2 in
// NT = D/64 tiles of 32; 2 products (hi, lo) per tile per 16 tokens.
template <int D>
__device__ __forceinline__ void mma_chunk(const Stage<D> &st, int w, int n, int g, f32x16 (&acc)[D / 64]) {
    const int ra = 32 * (w & 1) + n;
#pragma unroll
    for (int s = 0; s < kChunk / 16; ++s) {
        const int col = swz(ra, 16 * s + 8 * g);
        const bf16x8 ah = as_bf16x8(*reinterpret_cast<const u32x4 *>(&st.kh[ra][col]));
        const bf16x8 al = as_bf16x8(*reinterpret_cast<const u32x4 *>(&st.kl[ra][col]));
#pragma unroll
        for (int t = 0; t < D / 64; ++t) {
            const int rc = (w >> 1) * (D / 2) + 32 * t + n;
            const bf16x8 bv = as_bf16x8(*reinterpret_cast<const u32x4 *>(&st.vt[rc][swz(rc, 16 * s + 8 * g)]));
            acc[t] = mfma32(ah, bv, acc[t]);
            acc[t] = mfma32(al, bv, acc[t]);
        }
    }
}

template <int D, bool kRing>
__global__ __launch_bounds__(256, 2) void absorb_partial_kernel(hf_absorb_args a, int P, int nch, int per_xcd) {
    __shared__ Stage<D> stage[2];
    constexpr int nta = D / 64;

    const int items = a.BH * nta * P;
    const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (item >= items) return;
    const int p = item % P, rowblk = item / P;              // rowblk = bh * nta + qa
    const int qa = rowblk % nta, bh = rowblk / nta;
    const int a0 = 64 * qa;
    const int ch0 = (int)((int64_t)p * nch / P), ch1 = (int)((int64_t)(p + 1) * nch / P);
    const int nt = (int)a.n_tok;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 31, g = lane >> 5;
    const int pr = tid >> 3, sub = tid & 7;

    f32x16 acc[D / 64];
#pragma unroll
    for (int t = 0; t < D / 64; ++t) acc[t] = f32x16{};
    float zacc[8] = {0, 0, 0, 0, 0, 0, 0, 0};

    // Pipeline: stage (i & 1) holds chunk ch0 + i; registers run two chunks ahead.  Loads
    // past the range repeat the last chunk (unconditional, so no wait lands on the younger
    // prefetch) and are staged as empty chunks (token index >= nt).
    const int last = ch1 - 1;                      // ch1 > ch0: every split owns >= 1 chunk
    auto chunk_u0 = [&](int ch) { return ch <= last ? ch * kChunk : nt; };
    ChunkRaw<D> r0, r1;
    load_chunk<D, kRing>(a, bh, ch0 * kChunk, a0, tid, r0);
    load_chunk<D, kRing>(a, bh, min(ch0 + 1, last) * kChunk, a0, tid, r1);
    store_chunk<D, kRing>(r0, stage[0], chunk_u0(ch0), nt, tid, zacc);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int ch = ch0; ch <= last; ch += 2) {
        load_chunk<D, kRing>(a, bh, min(ch + 2, last) * kChunk, a0, tid, r0);
        __builtin_amdgcn_sched_barrier(0);
        mma_chunk<D>(stage[0], w, n, g, acc);
        __builtin_amdgcn_sched_barrier(0);
        store_chunk<D, kRing>(r1, stage[1], chunk_u0(ch + 1), nt, tid, zacc);
        __syncthreads();
        if (ch + 1 > last) break;
        load_chunk<D, kRing>(a, bh, min(ch + 3, last) * kChunk, a0, tid, r1);
        __builtin_amdgcn_sched_barrier(0);
        mma_chunk<D>(stage[1], w, n, g, acc);
        __builtin_amdgcn_sched_barrier(0);
        store_chunk<D, kRing>(r0, stage[0], chunk_u0(ch + 2), nt, tid, zacc);
        __syncthreads();
    }

    // partial S rows a0 .. a0+63 of this split: part[item][row][c]
    float *part = a.part + (size_t)item * 64 * D;
#pragma unroll
    for (int t = 0; t < D / 64; ++t) {
        const int c = (w >> 1) * (D / 2) + 32 * t + n;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 32 * (w & 1) + 8 * (i >> 2) + 4 * g + (i & 3);
            part[(size_t)r * D + c] = acc[t][i];
        }
    }
    // partial z: features a0 + 8*sub + e summed over the 32 token pairs (the LDS stages are
    // free once the last barrier of the loop has passed)
    float(*zred)[65] = reinterpret_cast<float(*)[65]>(&stage[0]);
#pragma unroll
    for (int e = 0; e < 8; ++e) zred[pr][8 * sub + e] = zacc[e];
    __syncthreads();
    if (tid < 64) {
        float zs = 0.f;
        for (int k = 0; k < 32; ++k) zs += zred[k][tid];
        a.part[(size_t)items * 64 * D + (size_t)item * 64 + tid] = zs;
    }
}

}  // namespace
}  // namespace hf

// ------------------------------------------------------------------ host side

// Splits per 64-row block aim at no more than ~256 workgroups (about one per CU) whatever
// the number of planes, and never exceed the number of 64-token chunks.
int hf_absorb_splits(int BH, int D, int64_t n_tok) {
    const int blocks = BH * (D / 64);
    int P = 256 / blocks;
    P = P < 1 ? 1 : P;
    const int64_t nch = (n_tok + hf::kChunk - 1) / hf::kChunk;
    return nch < P ? (int)(nch > 0 ? nch : 1) : P;
}

// Workspace floats of the partials for P splits: BH*D/64*P blocks of 64 x D, then as many
// blocks of 64 z values.
size_t hf_absorb_partial_floats(int BH, int D, int P) {
    const size_t items = (size_t)BH * (D / 64) * P;
    return items * 64 * D + items * 64;
}

size_t hf_absorb_workspace_bytes(int BH, int D) {
    return hf_absorb_partial_floats(BH, D, hf_absorb_splits(BH, D, (int64_t)1 << 30)) * sizeof(float);
}

hipError_t hf_launch_absorb_partial(const hf_absorb_args &a, hipStream_t s) {
    if (a.n_tok <= 0) return hipSuccess;
    const int P = hf_absorb_splits(a.BH, a.D, a.n_tok);
    const int nch = (int)((a.n_tok + hf::kChunk - 1) / hf::kChunk);
    const int items = a.BH * (a.D / 64) * P;
    const int per_xcd = (items + 7) / 8;
    const dim3 grid((unsigned)(per_xcd * 8));
    hf_absorb_args b = a;
    b.magicT = hf::div_magic((uint32_t)(a.T > 0 ? a.T : 1));
    const bool ring = a.ring_k != nullptr;
    if (a.D == 64) {
        if (ring)
            hipLaunchKernelGGL((hf::absorb_partial_kernel<64, true>), grid, dim3(256), 0, s, b, P, nch, per_xcd);
        else
            hipLaunchKernelGGL((hf::absorb_partial_kernel<64, false>), grid, dim3(256), 0, s, b, P, nch, per_xcd);
    } else {
        if (ring)
            hipLaunchKernelGGL((hf::absorb_partial_kernel<128, true>), grid, dim3(256), 0, s, b, P, nch, per_xcd);
        else
            hipLaunchKernelGGL((hf::absorb_partial_kernel<128, false>), grid, dim3(256), 0, s, b, P, nch, per_xcd);
    }
    return hipGetLastError();
}
