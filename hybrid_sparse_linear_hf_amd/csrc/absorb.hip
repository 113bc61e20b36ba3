// Absorb evicted tokens into the linear attention state.
//
// [HF-abs]: a compact key-value state incrementally absorbs the tokens evicted from the
// sliding window; [HF-de] §2.A / [HF-pt] §2.A.1: information of frames leaving the window
// is aggregated into that state through a linear attention.  With feature map
// phi = elu + 1:   S[a][c] += sum_u phi(K_u[a]) V_u[c],   z[a] += sum_u phi(K_u[a]).
//
// gfx950 design (HBM-bound: ~60 flop per byte against a ~315 flop/byte ridge)
//   * Each workgroup owns 64 rows of S (all D columns) and a contiguous range of 64-token
//     chunks, so phi(K) is evaluated exactly once per element; it writes its 64 x D
//     partial sum and its 64 partial z values to the workspace.  No workgroup waits for
//     another: no fences, counters or atomics.
//   * Source: the caller's row-major evicted tokens (the absorb of a hybrid step runs
//     inside its attention launch instead).  Registers hold the loads of the next two
//     chunks, and V is transposed on its way into LDS; phi(K) is evaluated in fp32, split
//     into bf16 hi + lo halves and written transposed to an LDS tile.
//   * Two matrix-core products per 16 tokens (hi and lo) keep fp32-grade accuracy: V is
//     exact in bf16, phi(K) = hi + lo to ~2^-17 relative.
//   * The partials are summed in split order and added to the old state by the state
//     pass (state.hip).  The result is deterministic.
#include <type_traits>

#include "hf_internal.h"

namespace hf {
namespace {

constexpr int kChunk = 64;
constexpr int kPitch = kChunk + 8;   // LDS row pitch (bf16) of the transposed phi(K) tiles

// Element column of token u in LDS row `row` of a phi(K) tile: 16-byte groups
// XOR-swizzled by row / 8.
__device__ __forceinline__ int swz(int row, int u) { return ((((u >> 3) ^ (row >> 3)) & 7) << 3) | (u & 7); }

__device__ __forceinline__ uint32_t word(const u32x4 &v, int e) {
    return e < 2 ? (e == 0 ? v.x : v.y) : (e == 2 ? v.z : v.w);
}

// phi(K)^T of one chunk, bf16 high and low halves: [feature a][token].  col(row, u) is
// the element column of token u in row `row`.
struct PhiTile {
    uint16_t kh[64][kPitch];
    uint16_t kl[64][kPitch];
    static __device__ __forceinline__ int col(int row, int u) { return swz(row, u); }
};
// A thread holds tokens 2pr, 2pr+1 (k0, k1: 2 NWORD bf16 features each, a0 + fbase ..):
// phi in fp32, z accumulation, hi/lo split, transposed pair writes into the tile.  m0, m1
// are all-ones for tokens to absorb and 0 for padding: a bit mask, so no branch is taken
// and padding reads zero whatever bits its LDS held (inf or NaN included).
__device__ __forceinline__ float keep_if(float f, uint32_t m) { return __uint_as_float(__float_as_uint(f) & m); }

template <int NWORD, bool kMask = true, typename Tile = PhiTile>
__device__ __forceinline__ void stage_phi(const uint32_t (&k0)[NWORD], const uint32_t (&k1)[NWORD], uint32_t m0,
                                          uint32_t m1, int pr, int fbase, Tile &t, float *zacc) {
#pragma unroll
    for (int e = 0; e < NWORD; ++e) {
        const uint32_t w0 = k0[e], w1 = k1[e];
        float f0[2], f1[2];
        f0[0] = phi_f32(bf16_lo_to_f32(w0));
        f0[1] = phi_f32(bf16_hi_to_f32(w0));
        f1[0] = phi_f32(bf16_lo_to_f32(w1));
        f1[1] = phi_f32(bf16_hi_to_f32(w1));
        if constexpr (kMask) {
            f0[0] = keep_if(f0[0], m0);
            f0[1] = keep_if(f0[1], m0);
            f1[0] = keep_if(f1[0], m1);
            f1[1] = keep_if(f1[1], m1);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            zacc[2 * e + h] += f0[h];
            zacc[2 * e + h] += f1[h];
            const int row = fbase + 2 * e + h;
            const uint32_t hi = pack_bf16x2(f0[h], f1[h]);            // (token 2pr, token 2pr+1)
            const uint32_t lo = pack_bf16x2(f0[h] - bf16_lo_to_f32(hi), f1[h] - bf16_hi_to_f32(hi));
            *reinterpret_cast<uint32_t *>(&t.kh[row][Tile::col(row, 2 * pr)]) = hi;
            *reinterpret_cast<uint32_t *>(&t.kl[row][Tile::col(row, 2 * pr)]) = lo;
        }
    }
}

// Wave w: rows 32*(w & 1) .. +32 of the 64-row block, columns (w >> 1)*(D/2) .. + D/2 in
// D/64 tiles of 32; 2 products (hi, lo) per tile per 16 tokens.  vrow(rc, tseg) gives the
// 16 bytes of V^T row rc, tokens 8 tseg .. 8 tseg + 7.
template <int D, typename VRow>
__device__ __forceinline__ void mma_chunk(const PhiTile &t, int w, int n, int g, f32x16 (&acc)[D / 64], VRow vrow) {
    const int ra = 32 * (w & 1) + n;
#pragma unroll
    for (int s = 0; s < kChunk / 16; ++s) {
        const int col = swz(ra, 16 * s + 8 * g);
        const bf16x8 ah = as_bf16x8(*reinterpret_cast<const u32x4 *>(&t.kh[ra][col]));
        const bf16x8 al = as_bf16x8(*reinterpret_cast<const u32x4 *>(&t.kl[ra][col]));
#pragma unroll
        for (int j = 0; j < D / 64; ++j) {
            const int rc = (w >> 1) * (D / 2) + 32 * j + n;
            const bf16x8 bv = as_bf16x8(vrow(rc, 2 * s + g));
            acc[j] = mfma32(ah, bv, acc[j]);
            acc[j] = mfma32(al, bv, acc[j]);
        }
    }
}

// Partial S rows a0 .. a0+63 of split `item` (part[item][row][c]) and, through LDS scratch
// `zred` (>= 32 x 65 floats, free to overwrite), its 64 partial z values.
template <int D>
__device__ __forceinline__ void write_partials(const hf_absorb_args &a, int items, int item, int tid,
                                               const f32x16 (&acc)[D / 64], const float *zacc, float *zred_mem) {
    const int w = tid >> 6, lane = tid & 63, n = lane & 31, g = lane >> 5;
    const int pr = tid >> 3, sub = tid & 7;
    float *part = a.part + (size_t)item * 64 * D;
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
        const int c = (w >> 1) * (D / 2) + 32 * j + n;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 32 * (w & 1) + 8 * (i >> 2) + 4 * g + (i & 3);
            part[(size_t)r * D + c] = acc[j][i];
        }
    }
    float(*zred)[65] = reinterpret_cast<float(*)[65]>(zred_mem);
#pragma unroll
    for (int e = 0; e < 8; ++e) zred[pr][8 * sub + e] = zacc[e];
    __syncthreads();
    if (tid < 64) {
        float zs = 0.f;
        for (int k = 0; k < 32; ++k) zs += zred[k][tid];
        a.part[(size_t)items * 64 * D + (size_t)item * 64 + tid] = zs;
    }
}

// Work item of a workgroup: 64-row block `qa` of plane `bh`, split `p` of the chunks.
// Items are numbered (bh, p, qa) with qa fastest, so the D/64 row blocks of one split --
// which read the same V^T -- are adjacent: they land on one XCD (whose L2 then serves the
// second read) and run at the same time.  The partial-sum slot of an item is
// (bh * (D/64) + qa) * P + p, the layout the state pass reads.
struct Item {
    int item, slot, p, qa, bh, ch0, ch1;
};
__device__ __forceinline__ bool get_item(const hf_absorb_args &a, int P, int nch, int per_xcd, Item &it) {
    const int nta = a.D / 64;
    const int items = a.BH * nta * P;
    it.item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (it.item >= items) return false;
    it.qa = it.item % nta;
    it.p = (it.item / nta) % P;
    it.bh = it.item / (nta * P);
    it.slot = (it.bh * nta + it.qa) * P + it.p;
    it.ch0 = (int)((int64_t)it.p * nch / P);
    it.ch1 = (int)((int64_t)(it.p + 1) * nch / P);
    return true;
}

// ------------------------------------------------------------------ row-major source

template <int D>
struct RowsRaw {
    u32x4 k[2];         // tokens 2 pr, 2 pr + 1: 8 features of K each
    u32x4 v[D / 32];    // tokens 2 pr + (e & 1), features 64 (e >> 1) + 8 sub ..
};

// Token indices past n_tok are clamped to the last token (finite data; staged with
// phi = 0), so the loads are branch-free.
template <int D>
__device__ __forceinline__ void load_rows(const hf_absorb_args &a, int bh, int u0, int a0, int tid, RowsRaw<D> &r) {
    const int pr = tid >> 3, sub = tid & 7;
    const int nt = (int)a.n_tok;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int u = min(u0 + 2 * pr + e, nt - 1);
        r.k[e] = *reinterpret_cast<const u32x4 *>(a.k + ((size_t)bh * nt + u) * D + a0 + 8 * sub);
    }
#pragma unroll
    for (int e = 0; e < D / 32; ++e) {
        const int u = min(u0 + 2 * pr + (e & 1), nt - 1);
        r.v[e] = *reinterpret_cast<const u32x4 *>(a.v + ((size_t)bh * nt + u) * D + 64 * (e >> 1) + 8 * sub);
    }
}

template <int D>
struct RowsStage {
    PhiTile phi;
    uint16_t vt[D][kPitch];    // V^T: [feature c][token], swizzled like the phi tile
};

template <int D>
__device__ __forceinline__ void store_rows(const RowsRaw<D> &cur, RowsStage<D> &st, int u0, int nt, int tid,
                                           float *zacc) {
    const int pr = tid >> 3, sub = tid & 7;
    const uint32_t k0[4] = {cur.k[0].x, cur.k[0].y, cur.k[0].z, cur.k[0].w};
    const uint32_t k1[4] = {cur.k[1].x, cur.k[1].y, cur.k[1].z, cur.k[1].w};
    stage_phi<4>(k0, k1, u0 + 2 * pr < nt ? ~0u : 0u, u0 + 2 * pr + 1 < nt ? ~0u : 0u, pr, 8 * sub, st.phi, zacc);
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

template <int D>
__global__ __launch_bounds__(256, 2) void absorb_rows_kernel(hf_absorb_args a, int P, int nch, int per_xcd) {
    __shared__ RowsStage<D> stage[2];
    Item it;
    if (!get_item(a, P, nch, per_xcd, it)) return;
    const int items = a.BH * (D / 64) * P;
    const int a0 = 64 * it.qa, nt = (int)a.n_tok, bh = it.bh;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 31, g = lane >> 5;

    f32x16 acc[D / 64];
#pragma unroll
    for (int j = 0; j < D / 64; ++j) acc[j] = f32x16{};
    float zacc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    auto vrow = [](const RowsStage<D> &st) {
        const RowsStage<D> *sp = &st;
        return [sp](int rc, int tseg) {
            return *reinterpret_cast<const u32x4 *>(&sp->vt[rc][swz(rc, 8 * tseg)]);
        };
    };

    // Pipeline: stage (i & 1) holds chunk ch0 + i; registers run two chunks ahead.  Loads
    // past the range repeat the last chunk (unconditional, so no wait lands on the younger
    // prefetch) and are staged as empty chunks (token index >= nt).
    const int ch0 = it.ch0, last = it.ch1 - 1;    // every split owns >= 1 chunk
    auto chunk_u0 = [&](int ch) { return ch <= last ? ch * kChunk : nt; };
    RowsRaw<D> r0, r1;
    load_rows<D>(a, bh, ch0 * kChunk, a0, tid, r0);
    load_rows<D>(a, bh, min(ch0 + 1, last) * kChunk, a0, tid, r1);
    store_rows<D>(r0, stage[0], chunk_u0(ch0), nt, tid, zacc);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int ch = ch0; ch <= last; ch += 2) {
        load_rows<D>(a, bh, min(ch + 2, last) * kChunk, a0, tid, r0);
        __builtin_amdgcn_sched_barrier(0);
        mma_chunk<D>(stage[0].phi, w, n, g, acc, vrow(stage[0]));
        __builtin_amdgcn_sched_barrier(0);
        store_rows<D>(r1, stage[1], chunk_u0(ch + 1), nt, tid, zacc);
        __syncthreads();
        if (ch + 1 > last) break;
        load_rows<D>(a, bh, min(ch + 3, last) * kChunk, a0, tid, r1);
        __builtin_amdgcn_sched_barrier(0);
        mma_chunk<D>(stage[1].phi, w, n, g, acc, vrow(stage[1]));
        __builtin_amdgcn_sched_barrier(0);
        store_rows<D>(r0, stage[0], chunk_u0(ch + 2), nt, tid, zacc);
        __syncthreads();
    }
    // (the last barrier of the loop has passed: the stages are free for the z reduction)
    write_partials<D>(a, items, it.slot, tid, acc, zacc, reinterpret_cast<float *>(&stage[0]));
}

}  // namespace
}  // namespace hf

// ------------------------------------------------------------------ host side

// Splits per 64-row block aim at about 512 workgroups (two per CU, the most the kernel's
// two LDS stages allow, so that one workgroup's products overlap the other's staging)
// whatever the number of planes, and never exceed the number of 64-token chunks.
int hf_absorb_splits(int BH, int D, int64_t n_tok) {
    const int blocks = BH * (D / 64);
    int P = 512 / blocks;
    P = P < 1 ? 1 : P;
    const int64_t nch = (n_tok + hf::kChunk - 1) / hf::kChunk;
    return nch < P ? (int)(nch > 0 ? nch : 1) : P;
}

// Splits of a hybrid step's absorb, which runs beside the attention: about 72 workgroups in
// all -- enough to stream the evicted frames while the attention runs, few enough to leave
// it its slots -- and at least one 16-token step each.  Never more than hf_absorb_splits
// allows for these planes, so the partials fit the same workspace.
int hf_step_absorb_splits(int BH, int D, int64_t n_tok) {
    const int64_t steps = (n_tok + 15) / 16;
    int64_t P = 72 / BH;
    const int64_t cap = hf_absorb_splits(BH, D, (int64_t)1 << 30);
    P = P < cap ? P : cap;
    P = P < steps ? P : steps;
    return (int)(P < 1 ? 1 : P);
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
    if (a.D == 64)
        hipLaunchKernelGGL(hf::absorb_rows_kernel<64>, grid, dim3(256), 0, s, a, P, nch, per_xcd);
    else
        hipLaunchKernelGGL(hf::absorb_rows_kernel<128>, grid, dim3(256), 0, s, a, P, nch, per_xcd);
    return hipGetLastError();
}
