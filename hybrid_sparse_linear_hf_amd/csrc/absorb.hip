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
//   * Ring source (the evictions of a step): the raw K rows and V^T rows of each chunk are
//     fetched with direct-to-LDS buffer loads into a ring of four LDS stages, three chunks
//     ahead of the compute, so ~70 KB per workgroup are in flight and no register holds
//     staging data.  16-byte slots are XOR-swizzled by row so that the matrix-core operand
//     reads hit distinct banks.  Each chunk's phi(K) is then evaluated in fp32 from LDS,
//     split into bf16 hi + lo halves and written transposed to a second LDS tile.
//   * Row-major source (standalone absorb of caller buffers): registers hold the loads of
//     the next two chunks, and V is transposed on its way into LDS.
//   * Two matrix-core products per 16 tokens (hi and lo) keep fp32-grade accuracy: V is
//     exact in bf16, phi(K) = hi + lo to ~2^-17 relative.
//   * The partials are summed in split order and added to the old state by the state
//     pass (state.hip), standalone or fused with the preparation that precedes the
//     attention kernel of a hybrid step.  The result is deterministic and independent of
//     the token source (ring or row-major buffers).
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
// Unpadded variant: 128-byte rows whose 16-byte groups are XOR-swizzled by
// (row >> 1) ^ (row >> 4), so 16 consecutive rows read at one group hit 16 distinct bank
// groups (64 banks of 4 bytes: a 128-byte row covers half of them), and the transform's
// pair writes touch every bank group at most twice.
struct PhiTile128 {
    uint16_t kh[64][64];
    uint16_t kl[64][64];
    static __device__ __forceinline__ int col(int row, int u) {
        return ((((u >> 3) ^ (row >> 1) ^ (row >> 4)) & 7) << 3) | (u & 7);
    }
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

// ------------------------------------------------------------------ ring source

constexpr int kStages = 5;
constexpr int kBufDword3 = 0x00020000;        // raw buffer resource word 3 (gfx9 family)
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef __attribute__((address_space(3))) void *LdsPtr;

__device__ __forceinline__ Rsrc make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufDword3);
}

// One fetched chunk: K rows [token][64 features] and V^T rows [feature][64 tokens], 128
// bytes each.  Slot j of K row r holds the row's 16-byte group j ^ (r & 7) (the transform
// reads whole rows); slot j of V^T row r holds group j ^ ((r >> 1) & 7), so 16 consecutive
// rows read at one group hit 16 distinct bank groups.
template <int D>
struct RawChunk {
    unsigned char k[64 * 128];
    unsigned char v[D * 128];
};
__device__ __forceinline__ int vt_slot(int row, int grp) { return grp ^ ((row >> 1) & 7); }

template <int D>
struct RingLds {
    RawChunk<D> st[kStages];
    PhiTile128 phi[2];
};
// the final reductions reuse the stages: 32 KB of accumulator halves, then 32 x 65 floats
static_assert(sizeof(RawChunk<64>) * kStages >= 32768 + 32 * 65 * 4, "reduction scratch");

// Ring-source geometry: NW = D / 16 waves.  Wave w multiplies rows 32 (w & 1) .. +32 by
// columns 64 ((w >> 1) % (D / 64)) .. +64 (two 32 x 32 tiles) over one half of each
// chunk's tokens (the contraction half w / (NW / 2)); the two halves are added at the
// end.  The phi transform gives each thread 2 tokens x FPT features.
template <int D>
struct RingShape {
    static constexpr int NW = D / 16;
    static constexpr int kThreads = 64 * NW;
    static constexpr int FPT = 2048 / kThreads;          // features per thread in the transform
    static constexpr int TPR = 64 / FPT;                 // threads per token pair
    static constexpr int KPW = 8 / NW;                   // K fetch instructions per wave and chunk
    static constexpr int VPW = D / 8 / NW;               // V^T fetch instructions per wave and chunk
    static constexpr int kPerChunk = KPW + VPW;
};

// Direct-to-LDS fetch of chunk u0 .. u0+63 of plane bh: 8 K and D/8 V^T instructions of
// 64 x 16 bytes, spread over the waves.  Lane l of instruction j fills slot l & 7 of row
// 8 j + l / 8, so it fetches that row's group (l & 7) ^ (l >> 3) for K and
// vt_slot(row, l & 7) for V^T.
//   T >= 64: the chunk spans at most two frames; their slots and the split point are
//   uniform (scalar) values, and each lane only selects between two bases.  Tokens past
//   n_tok are fetched from the frame that follows (a valid slot: finite data) and are
//   staged with phi = 0.
//   T < 64: each lane maps its own token to its frame and slot, clamped to n_tok - 1.
template <int D>
__device__ __forceinline__ void fetch_chunk(const hf_absorb_args &a, Rsrc rk, Rsrc rv, RawChunk<D> &dst, int u0,
                                            int a0, int w, int lane) {
    using RS = RingShape<D>;
    const int grp = (lane & 7) ^ (lane >> 3);
    if (a.T >= kChunk) {
        const int f0 = fast_div(u0, a.magicT, a.T);
        int s0 = a.head + f0;
        s0 = s0 >= a.W ? s0 - a.W : s0;
        const int s1 = s0 + 1 >= a.W ? s0 + 1 - a.W : s0 + 1;
        const int split = (f0 + 1) * a.T - u0;           // tokens of the chunk in frame f0
        // byte offsets of chunk token 0 as if every token lay in frame f0 (k0, v0) or f0+1 (k1, v1)
        const int k0 = (s0 * a.T + u0 - f0 * a.T) * D * 2, k1 = (s1 * a.T - split) * D * 2;
        const int v0 = (s0 * D * a.T + u0 - f0 * a.T) * 2, v1 = (s1 * D * a.T - split) * 2;
#pragma unroll
        for (int jj = 0; jj < RS::KPW; ++jj) {
            const int j = RS::KPW * w + jj;
            const int t = 8 * j + (lane >> 3);
            const uint32_t off = (uint32_t)((t < split ? k0 : k1) + (t * D + a0 + 8 * grp) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LdsPtr)(dst.k + j * 1024), 16, (int)off, 0, 0, 0);
        }
#pragma unroll
        for (int jj = 0; jj < RS::VPW; ++jj) {
            const int j = RS::VPW * w + jj;
            const int c = 8 * j + (lane >> 3);
            const int vg = vt_slot(c, lane & 7);
            const uint32_t off = (uint32_t)((8 * vg < split ? v0 : v1) + (c * a.T + 8 * vg) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LdsPtr)(dst.v + j * 1024), 16, (int)off, 0, 0, 0);
        }
        return;
    }
    const int nt = (int)a.n_tok;
#pragma unroll
    for (int jj = 0; jj < RS::KPW; ++jj) {
        const int j = RS::KPW * w + jj;
        const int u = min(u0 + 8 * j + (lane >> 3), nt - 1);
        const int f = fast_div(u, a.magicT, a.T);
        int slot = a.head + f;
        if (slot >= a.W) slot -= a.W;
        const uint32_t off = (uint32_t)((((slot * a.T) + (u - f * a.T)) * D + a0 + 8 * grp) * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LdsPtr)(dst.k + j * 1024), 16, (int)off, 0, 0, 0);
    }
#pragma unroll
    for (int jj = 0; jj < RS::VPW; ++jj) {
        const int j = RS::VPW * w + jj;
        const int c = 8 * j + (lane >> 3);
        const int u = min(u0 + 8 * vt_slot(c, lane & 7), nt - 8);   // 8 tokens of one frame (T % 8 == 0)
        const int f = fast_div(u, a.magicT, a.T);
        int slot = a.head + f;
        if (slot >= a.W) slot -= a.W;
        const uint32_t off = (uint32_t)((((slot * D) + c) * a.T + (u - f * a.T)) * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LdsPtr)(dst.v + j * 1024), 16, (int)off, 0, 0, 0);
    }
}

template <int D>
__global__ __launch_bounds__(RingShape<D>::kThreads, 1) void absorb_ring_kernel(hf_absorb_args a, int P, int nch,
                                                                               int per_xcd) {
    using RS = RingShape<D>;
    constexpr int FPT = RS::FPT;
    __shared__ RingLds<D> lds;
    Item it;
    if (!get_item(a, P, nch, per_xcd, it)) return;
    const int items = a.BH * (D / 64) * P;
    const int a0 = 64 * it.qa, nt = (int)a.n_tok;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 31, g = lane >> 5;
    const int pr = tid / RS::TPR, q = tid % RS::TPR;
    const size_t plane = (size_t)a.W * a.T * D;
    const Rsrc rk = make_rsrc(a.ring_k + (size_t)it.bh * plane, (uint32_t)(plane * 2));
    const Rsrc rv = make_rsrc(a.ring_vt + (size_t)it.bh * plane, (uint32_t)(plane * 2));

    float zacc[FPT];
#pragma unroll
    for (int e = 0; e < FPT; ++e) zacc[e] = 0.f;

    // phi(K) of local chunk i (raw K in stage i % kStages) into phi tile `buf`; chunks past
    // the split, and tokens past n_tok, are staged with phi = 0 (kMask: per-token masks).
    const int cnt = it.ch1 - it.ch0;               // >= 1
    auto transform = [&](int i, int buf, auto masked) {
        const RawChunk<D> &c = lds.st[i % kStages];
        const int t0 = 2 * pr, t1 = 2 * pr + 1;
        const int u0 = (it.ch0 + i) * kChunk;
        const int byte = 2 * FPT * q;              // of the 128-byte K row
        const unsigned char *p0 = c.k + t0 * 128 + 16 * ((byte >> 4) ^ (t0 & 7)) + (byte & 15);
        const unsigned char *p1 = c.k + t1 * 128 + 16 * ((byte >> 4) ^ (t1 & 7)) + (byte & 15);
        uint32_t k0[FPT / 2], k1[FPT / 2];
        if constexpr (FPT == 8) {
            const u32x4 v0 = *reinterpret_cast<const u32x4 *>(p0), v1 = *reinterpret_cast<const u32x4 *>(p1);
            k0[0] = v0.x, k0[1] = v0.y, k0[2] = v0.z, k0[3] = v0.w;
            k1[0] = v1.x, k1[1] = v1.y, k1[2] = v1.z, k1[3] = v1.w;
        } else {
            const u32x2 v0 = *reinterpret_cast<const u32x2 *>(p0), v1 = *reinterpret_cast<const u32x2 *>(p1);
            k0[0] = v0.x, k0[1] = v0.y;
            k1[0] = v1.x, k1[1] = v1.y;
        }
        const bool live = i < cnt;
        stage_phi<FPT / 2, decltype(masked)::value>(k0, k1, live && u0 + t0 < nt ? ~0u : 0u,
                                                    live && u0 + t1 < nt ? ~0u : 0u, pr, FPT * q, lds.phi[buf], zacc);
    };
    // chunk i needs no masks when it is one of this split's and lies below n_tok
    auto unmasked = [&](int i) { return i < cnt && (it.ch0 + i + 1) * kChunk <= nt; };

    // Pipeline: the fetches run kStages - 1 chunks ahead; step i multiplies chunk i (its phi
    // tile and V^T) while it evaluates phi of chunk i + 1, one barrier per chunk.  Two waves
    // share each SIMD, so one's matrix-core work overlaps the other's phi evaluation.
#pragma unroll
    for (int c = 0; c < kStages - 1; ++c)
        if (c < cnt) fetch_chunk<D>(a, rk, rv, lds.st[c], (it.ch0 + c) * kChunk, a0, w, lane);
    if (kStages - 2 < cnt)
        wait_vm<RS::kPerChunk * (kStages - 2)>();
    else
        wait_vm<0>();
    lds_barrier();
    if (unmasked(0))
        transform(0, 0, std::false_type{});
    else
        transform(0, 0, std::true_type{});

    constexpr int kHalves = RS::NW / 2;                  // waves per contraction half
    const int ra = 32 * (w & 1) + n, cb = 64 * ((w >> 1) % (D / 64)), sh = w / kHalves;
    f32x16 acc[2] = {f32x16{}, f32x16{}};
    for (int i = 0; i < cnt; ++i) {
        // chunk i + 1 has landed once at most the fetches of the chunks after it are pending
        if (i + kStages - 2 < cnt)
            wait_vm<RS::kPerChunk * (kStages - 3)>();
        else
            wait_vm<0>();
        lds_barrier();     // phi of chunk i is complete, chunk i+1 is in LDS, chunk i-1 is consumed
        if (i + kStages - 1 < cnt)
            fetch_chunk<D>(a, rk, rv, lds.st[(i + kStages - 1) % kStages], (it.ch0 + i + kStages - 1) * kChunk, a0,
                           w, lane);
        const RawChunk<D> &cur = lds.st[i % kStages];
        const PhiTile128 &ph = lds.phi[i & 1];
        auto mma = [&]() {
#pragma unroll
            for (int ss = 0; ss < 2; ++ss) {
                const int s = 2 * sh + ss, tg = 2 * s + g;     // 16-token step, 8-token group
                const int col = PhiTile128::col(ra, 8 * tg);
                const bf16x8 ah = as_bf16x8(*reinterpret_cast<const u32x4 *>(&ph.kh[ra][col]));
                const bf16x8 al = as_bf16x8(*reinterpret_cast<const u32x4 *>(&ph.kl[ra][col]));
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int rc = cb + 32 * j + n;
                    const bf16x8 bv = as_bf16x8(*reinterpret_cast<const u32x4 *>(cur.v + rc * 128 + 16 * vt_slot(rc, tg)));
                    acc[j] = mfma32(ah, bv, acc[j]);
                    acc[j] = mfma32(al, bv, acc[j]);
                }
            }
        };
        // the matrix-core products of chunk i interleave with phi of chunk i + 1
        if (unmasked(i + 1)) {
            mma();
            transform(i + 1, (i + 1) & 1, std::false_type{});
        } else {
            mma();
            transform(i + 1, (i + 1) & 1, std::true_type{});
        }
    }
    lds_barrier();     // the LDS stages are free for the reductions

    // partial S: the two contraction halves added, rows a0 .. a0+63 (part[item][row][c])
    unsigned char *red = reinterpret_cast<unsigned char *>(&lds.st[0]);
    f32x16 *hand = reinterpret_cast<f32x16 *>(red);               // [kHalves][2][64 lanes], <= 32 KB
    if (sh == 1) {
#pragma unroll
        for (int j = 0; j < 2; ++j) hand[((w - kHalves) * 2 + j) * 64 + lane] = acc[j];
    }
    __syncthreads();
    if (sh == 0) {
        float *part = a.part + (size_t)it.slot * 64 * D;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const f32x16 t = acc[j] + hand[(w * 2 + j) * 64 + lane];
            const int c = cb + 32 * j + n;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 32 * (w & 1) + 8 * (i >> 2) + 4 * g + (i & 3);
                part[(size_t)r * D + c] = t[i];
            }
        }
    }
    // partial z: features FPT q + e summed over the 32 token pairs
    float(*zred)[65] = reinterpret_cast<float(*)[65]>(red + 32768);
#pragma unroll
    for (int e = 0; e < FPT; ++e) zred[pr][FPT * q + e] = zacc[e];
    __syncthreads();
    if (tid < 64) {
        float zs = 0.f;
        for (int k = 0; k < 32; ++k) zs += zred[k][tid];
        a.part[(size_t)items * 64 * D + (size_t)it.slot * 64 + tid] = zs;
    }
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
    if (a.ring_k != nullptr) {
        // per-plane buffer resources take 32-bit byte offsets
        if ((uint64_t)a.W * a.T * a.D * 2 >= (1ull << 31) || a.T % 8 != 0) return hipErrorInvalidValue;
        b.magicT = hf::div_magic((uint32_t)a.T);
        if (a.D == 64)
            hipLaunchKernelGGL(hf::absorb_ring_kernel<64>, grid, dim3(hf::RingShape<64>::kThreads), 0, s, b, P, nch,
                               per_xcd);
        else
            hipLaunchKernelGGL(hf::absorb_ring_kernel<128>, grid, dim3(hf::RingShape<128>::kThreads), 0, s, b, P, nch,
                               per_xcd);
    } else {
        if (a.D == 64)
            hipLaunchKernelGGL(hf::absorb_rows_kernel<64>, grid, dim3(256), 0, s, b, P, nch, per_xcd);
        else
            hipLaunchKernelGGL(hf::absorb_rows_kernel<128>, grid, dim3(256), 0, s, b, P, nch, per_xcd);
    }
    return hipGetLastError();
}
