// Backward of the hybrid step output with the block selection held fixed (the selection is
// piecewise constant in the inputs).  For query t with kept keys u, P_tu = softmax of
// q_t.k_u / sqrt(D), r_t = phi(q_t)^T S / (phi(q_t).z + eps), out_t = sum_u P_tu v_u + r_t
// ([HF-de] §2.A, [HF-pt] §2.A.1, 2.A.2 and "Resultado"; [HF-abs]).  Given dO = dL/dout:
//   sparse part  dP_tu = dO_t.v_u, Delta_t = dO_t.(out_t - r_t), G_tu = P_tu (dP_tu - Delta_t),
//                dq_t += sum_u G_tu k_u / sqrt(D), dk_u = sum_t G_tu q_t / sqrt(D),
//                dv_u = sum_t P_tu dO_t;
//   readout      n_t = S^T phi(q_t), den_t = phi(q_t).z + eps, dn = dO_t / den_t,
//                dden = -(dO_t.n_t) / den_t^2, dS += phi(q_t) dn^T, dz += phi(q_t) dden,
//                dq_t += (S dn + z dden) * phi'(q_t);
//   absorb       (S += phi(K)^T V, z += sum phi(K)):  dV = phi(K) dS, dK = (V dS^T + dz) * phi'(K).
//
// gfx950 design.  A prep launch copies the window into logical order in bf16 -- K rows and
// V rows -- so that the passes below never touch the ring's frame arithmetic, and S into
// bf16 rows and transposed rows.
//   * readout pass: one workgroup per (plane, split of the queries), S staged in LDS once;
//     n = S^T phi(q) on the matrix cores, per-query terms in fp32 (Delta, 1 / den, dden);
//     dS and dz as split partials (phi(q) and dn staged transposed in LDS), added in split
//     order by a second launch.  It reads every dO row and writes it back in bf16 for the
//     passes below.
//   * dq pass: one workgroup per query block, one wave per 32-query tile, walking the kept
//     key blocks in 32-key subtiles staged in LDS (two stages filled by direct-to-LDS
//     loads, one subtile ahead): S^T = K Q^T, dP^T = V dO^T,
//     G^T = P^T (dP^T - Delta) and dq^T += K^T G^T (K^T read from the staged K rows by
//     transposing LDS reads); then the readout's term S dn + z dden, times phi'(q), with S
//     staged in the same LDS, and one store of dq.
//   * dk/dv pass: one workgroup per key block, one wave per (32-key tile, 32-query tile),
//     walking the query blocks that kept it (a per-plane transpose of the selection, in
//     ascending order), their Q and dO rows fetched into LDS ahead of their use:
//     S = Q K^T, dP = dO V^T, G = P (dP - Delta), dv^T += dO^T P, dk^T += Q^T G, the
//     transposed operands read from the same rows by transposing LDS reads.
//   Products in bf16 with fp32 accumulation; P and G rounded to bf16 as matrix-core
//   operands.  Every sum has a fixed order: results are deterministic.
#include "hf_internal.h"

namespace hf {
namespace {

constexpr int kQB = 64;   // query-block stages hold 64 rows (a short block repeats its last query)

// int32 data a kernel only reads and an earlier launch wrote, addressed through the
// constant address space so that uniform reads become scalar loads
typedef const __attribute__((address_space(4))) int32_t *cint32_p;

__device__ __forceinline__ float pair_sum_b(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float phi_prime(float x) {
    const float e = __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
    return x > 0.f ? 1.f : e;
}

// ---------------------------------------------------------------- prep

// A fp32 [BH][D][D] matrix into bf16 rows and bf16 transposed rows, one workgroup per
// 32 x 32 tile.
template <int D>
__device__ void mat_copies(const float *M, uint16_t *mb, uint16_t *mtb, int tile, float (*t)[33]) {
    constexpr int nt = D / 32;
    const int bh = tile / (nt * nt), ti = (tile / nt) % nt, tj = tile % nt;
    const float *src = M + (size_t)bh * D * D;
    for (int e = threadIdx.x; e < 32 * 32; e += 256) {
        const int r = e / 32, c = e % 32;
        const float v = src[(size_t)(32 * ti + r) * D + 32 * tj + c];
        t[r][c] = v;
        mb[(size_t)bh * D * D + (size_t)(32 * ti + r) * D + 32 * tj + c] = (uint16_t)f32_to_bf16_bits(v);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 32 * 32; e += 256) {
        const int r = e / 32, c = e % 32;   // transposed element (c, r) of the tile
        mtb[(size_t)bh * D * D + (size_t)(32 * tj + r) * D + 32 * ti + c] = (uint16_t)f32_to_bf16_bits(t[c][r]);
    }
}

// One workgroup per (plane, 64-key tile of the logical window): K rows and V rows, rows
// past the window zeroed.  Threads 0..127 turn V back from the ring's 8-token groups
// ([D][8] per group) into rows: each owns 8 keys x 8 features, loads the 8 features' 16-byte
// key runs (128 contiguous bytes), transposes the 8x8 block of 16-bit values in registers
// (byte permutes) and stores 8 16-byte row pieces; threads 128..255 copy the K rows.  Keys
// j0 .. j0 + 63 in aligned groups of 8 stay in one frame (T % 8 == 0).  Every load of a
// thread is issued before its first store.  Extra workgroups copy S into bf16 rows and
// transposed rows (mat_copies).
template <int D>
__global__ __launch_bounds__(256) void prep_keys_kernel(hf_bwd_args a) {
    const int tiles = a.NkP / 64;
    if ((int)blockIdx.x >= a.BH * tiles) {
        __shared__ float t[32][33];
        mat_copies<D>(a.S, a.sb, a.stb, (int)blockIdx.x - a.BH * tiles, t);
        return;
    }
    const int bh = blockIdx.x / tiles, j0 = (blockIdx.x % tiles) * 64;
    auto ring_off = [&](int j) {     // element offset of window key j's row (K) or group (V)
        const int f = j / a.T, t = j - f * a.T;
        int s = a.head + f;
        s = s >= a.W ? s - a.W : s;
        return (((size_t)bh * a.W + s) * a.T + t) * D;
    };
    const int tid = threadIdx.x;
    if (tid < 128) {
        const int fg = tid % 16, tg = tid / 16;             // feature octet, key group
        if (fg >= D / 8) return;
        const int j = j0 + 8 * tg;
        u32x4 in[8];
        if (j < a.Nk) {
            const uint16_t *src = a.ring_vg + ring_off(j) + 64 * fg;   // features 8 fg .. + 7, 8 keys each
#pragma unroll
            for (int i = 0; i < 8; ++i) in[i] = *reinterpret_cast<const u32x4 *>(src + 8 * i);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) in[i] = u32x4{0u, 0u, 0u, 0u};
        }
        // out[k] = key k's features 8 fg .. + 7: word w takes feature 2w and 2w+1 of key k
        uint16_t *dst = a.vr + ((size_t)bh * a.NkP + j) * D + 8 * fg;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
            uint32_t o[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) o[w] = __builtin_amdgcn_perm(in[2 * w + 1][k >> 1], in[2 * w][k >> 1], sel);
            *reinterpret_cast<u32x4 *>(dst + (size_t)k * D) = u32x4{o[0], o[1], o[2], o[3]};
        }
    } else {
        constexpr int kVecPerRow = D / 8, kIters = 64 * kVecPerRow / 128;
        u32x4 kv[kIters];
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int e = tid - 128 + 128 * it, r = e / kVecPerRow, c8 = (e % kVecPerRow) * 8, j = j0 + r;
            kv[it] = j < a.Nk ? *reinterpret_cast<const u32x4 *>(a.ring_k + ring_off(j) + c8) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int e = tid - 128 + 128 * it, r = e / kVecPerRow, c8 = (e % kVecPerRow) * 8;
            *reinterpret_cast<u32x4 *>(a.kr + ((size_t)bh * a.NkP + j0 + r) * D + c8) = kv[it];
        }
    }
}

// The dk/dv pass's work order.  Key blocks (bh * nkb + j) are cut into 8 contiguous shares,
// one per XCD (dispatch places workgroup x on XCD x % 8, and the pass maps it to slot
// (x % 8) * share + x / 8), so that one XCD's L2 holds the Q and dO rows of about one and a
// half planes; within each share the key blocks are sorted by descending number of query
// blocks that kept them (counting sort, one workgroup per share), so that the longest work
// starts first.  Ties are ordered by the atomics, which changes timing only: every workgroup
// writes its own key block.
constexpr int kOrderBuckets = 2048;
__global__ __launch_bounds__(1024) void order_kernel(hf_bwd_args a) {
    __shared__ int start[kOrderBuckets];
    __shared__ int part[1024];
    const int items = a.BH * a.nkb, share = (items + 7) / 8, t = threadIdx.x;
    const int lo = (int)blockIdx.x * share, hi = min(lo + share, items);
    auto bucket = [&](int it) {
        const int32_t *off = a.qoff + (size_t)(it / a.nkb) * (a.nkb + 1);
        const int j = it % a.nkb;
        return kOrderBuckets - 1 - min(off[j + 1] - off[j], kOrderBuckets - 1);
    };
    start[2 * t] = start[2 * t + 1] = 0;
    __syncthreads();
    for (int it = lo + t; it < hi; it += 1024) atomicAdd(&start[bucket(it)], 1);
    __syncthreads();
    // exclusive scan over the buckets: thread t holds buckets 2t, 2t+1; Hillis-Steele over
    // the 1024 pair sums
    const int c0 = start[2 * t], c1 = start[2 * t + 1];
    part[t] = c0 + c1;
    __syncthreads();
    for (int d = 1; d < 1024; d *= 2) {
        const int v = t >= d ? part[t - d] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    const int base = part[t] - (c0 + c1);
    start[2 * t] = base;
    start[2 * t + 1] = base + c0;
    __syncthreads();
    for (int it = lo + t; it < hi; it += 1024) a.korder[lo + atomicAdd(&start[bucket(it)], 1)] = it;
}

// Per plane, the query blocks that kept each key block, ascending: count (LDS atomics over
// the kept entries, which are also staged in LDS when they fit), exclusive scan (one wave),
// then the fill.  When the plane's (key block, query block) bitmap fits in LDS, every entry
// finds its own slot: query block i goes to the key block's list at the number of query
// blocks below i that kept it (a population count of the bitmap row), all entries at once.
// Otherwise a fill walks the query blocks in order.  A kept list holds distinct blocks, so
// entries never collide; entries outside [0, n_kb), a caller error, are skipped.
constexpr int kCsrStaged = 8192;   // kept entries of a plane staged in LDS for the fill
constexpr int kCsrBitWords = 4096; // 64-bit words of the bitmap (n_kb * ceil(n_qb / 64))
__global__ __launch_bounds__(256) void csr_kernel(hf_bwd_args a) {
    __shared__ int cnt[kMaxKeyBlocks];
    __shared__ int pos[kMaxKeyBlocks];
    __shared__ int32_t sel_s[kCsrStaged];
    __shared__ unsigned long long bits[kCsrBitWords];
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int total = a.nqb * a.top_k;
    const bool staged = total <= kCsrStaged;          // uniform
    const int words = (a.nqb + 63) / 64;              // bitmap words per key block
    const bool by_rank = a.nkb * words <= kCsrBitWords;   // uniform
    const int32_t *sel = a.idx + (size_t)bh * total;
    for (int j = tid; j < a.nkb; j += 256) cnt[j] = 0;
    if (by_rank)
        for (int e = tid; e < a.nkb * words; e += 256) bits[e] = 0ull;
    __syncthreads();
    // the kept entries, twelve loads per thread issued before the first is used
    constexpr int U = 12;
    for (int e0 = tid; e0 < total; e0 += 256 * U) {
        int jv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) jv[u] = e0 + 256 * u < total ? sel[e0 + 256 * u] : -1;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = e0 + 256 * u, j = jv[u];
            if (e >= total) break;
            if (staged) sel_s[e] = j;
            if (j >= 0 && j < a.nkb) {
                atomicAdd(&cnt[j], 1);
                if (by_rank) {
                    const int i = e / a.top_k;
                    atomicOr(&bits[j * words + (i >> 6)], 1ull << (i & 63));
                }
            }
        }
    }
    __syncthreads();
    const int32_t *fsel = staged ? sel_s : sel;        // the fill reads LDS when it can
    int32_t *off = a.qoff + (size_t)bh * (a.nkb + 1);
    if (tid < 64) {
        int base = 0;
        for (int j0 = 0; j0 < a.nkb; j0 += 64) {
            const int j = j0 + tid;
            const int c = j < a.nkb ? cnt[j] : 0;
            int x = c;
            for (int d = 1; d < 64; d <<= 1) {
                const int y = __shfl_up(x, d);
                if (tid >= d) x += y;
            }
            if (j < a.nkb) {
                off[j] = base + x - c;
                pos[j] = base + x - c;
            }
            base += __shfl(x, 63);
        }
        if (tid == 0) off[a.nkb] = base;
    }
    __syncthreads();
    int32_t *list = a.qlist + (size_t)bh * a.nqb * a.top_k;
    if (by_rank) {
        for (int e = tid; e < total; e += 256) {
            const int j = fsel[e];
            if (j < 0 || j >= a.nkb) continue;
            const int i = e / a.top_k, wi = i >> 6;
            const unsigned long long *row = &bits[j * words];
            int rank = __popcll(row[wi] & ((1ull << (i & 63)) - 1ull));
            for (int q = 0; q < wi; ++q) rank += __popcll(row[q]);
            list[pos[j] + rank] = i;
        }
        return;
    }
    for (int i = 0; i < a.nqb; ++i) {
        for (int r = tid; r < a.top_k; r += 256) {
            const int j = fsel[(size_t)i * a.top_k + r];
            if (j >= 0 && j < a.nkb) list[pos[j]++] = i;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- staged-row helpers

// 16-byte chunk swizzle of staged rows of D (S in the readout pass, Q and dO rows in the dk/dv
// pass, K rows in the dq pass): chunk c of row r sits at slot c ^ swz_row(r).  For D = 128 the row's two low
// bits go to slot bits 2-3, bit 2 to bit 0 and bit 4 to bit 1, so that (a) the fragment
// reads of rows 32 x + perm32(n), one chunk per 16 lanes, hit 16 distinct bank groups, and
// (b) the transposing reads -- four consecutive rows, chunk offsets 0 and 2 within them --
// land on 16 distinct (chunk, half) slots.
template <int D>
__device__ __forceinline__ int swz_row(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 1) | (((r >> 4) & 1) << 1);
    else return ((r >> 1) & 3) | ((r >> 2) & 4);
}

// Transposing LDS read (gfx950): within each 16-lane group, lane i receives element i % 4 of
// the 4-element vectors that lanes i / 4, i / 4 + 4, i / 4 + 8, i / 4 + 12 of the group point
// at (one per returned element).
typedef short v4s16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t *p) {
    const v4s16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s16 *)(const_cast<uint16_t *>(p)));
    return u32x2{(uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16),
                 (uint32_t)(uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16)};
}

// Matrix-core A fragment of X^T from staged, chunk-swizzled rows of D (swz_row): lane
// (n, g) receives features 32 ft + perm32(n) of rows q0 .. q0 + 7 (q0 for its lane half),
// as two transposing reads of four rows.  In a 16-lane group (n = 16 G + i) lane s points
// at row q0 + 4 h + s / 4, features 32 ft + 8 G + 16 ((s % 4) & 1) + 4 ((s % 4) >> 1) .. + 3,
// so that lane i receives feature 32 ft + perm32(16 G + i).
template <int D>
__device__ __forceinline__ u32x4 xt_frag(const uint16_t *X, int q0, int ft, int lane) {
    const int s = lane & 15, t = s & 3, G = (lane >> 4) & 1;
    const int d = 32 * ft + 8 * G + 16 * (t & 1) + 4 * (t >> 1);
    u32x2 h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int r = q0 + 4 * hh + (s >> 2);
        const int e = r * D + (((d >> 3) ^ swz_row<D>(r)) << 3) + (d & 7);
        h[hh] = ds_read_tr16(X + e);
    }
    return u32x4{h[0].x, h[0].y, h[1].x, h[1].y};
}

constexpr int kBufDword3 = 0x00020000;        // raw buffer resource word 3 (gfx9 family)
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef __attribute__((address_space(3))) void *LdsPtr;

__device__ __forceinline__ Rsrc make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufDword3);
}

// 16 bytes per lane from the buffer into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(Rsrc r, unsigned char *lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)lds, 16, (int)voff, 0, 0, 0);
}

// ---------------------------------------------------------------- readout pass

// One workgroup (two waves) per (plane, split); split s takes 64-query chunks
// s, s + splits, ...  Each wave owns 32 queries of the chunk.
template <int D>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 1))) void readout_bwd_kernel(hf_bwd_args a) {
    __shared__ __align__(16) uint16_t phT[D][kQB + 8];
    __shared__ __align__(16) uint16_t dnT[D][kQB + 8];
    __shared__ __align__(16) float dden_s[kQB];
    // S in bf16, staged once for all the workgroup's chunks as chunk-swizzled rows of D
    // (swz_row): its row fragments are read directly, those of S^T by transposing reads
    __shared__ __align__(16) uint16_t s_sw[D * D];
    const int bh = blockIdx.x / a.splits, sp = blockIdx.x % a.splits;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31, g = lane >> 5;
    const int nchunks = (a.Nq + kQB - 1) / kQB;
    // z at the features 16 ks + 8 g .. + 8 this lane's phi(q) holds, in registers for every chunk
    f32x4 zr[D / 16][2];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) zr[ks][h] = *reinterpret_cast<const f32x4 *>(a.z + (size_t)bh * D + 16 * ks + 8 * g + 4 * h);
    {
        // direct-to-LDS loads, 1 KB (RPI whole rows) per instruction, all issued before the
        // first wait: lane l of instruction j fills slot l % LPR of row RPI j + l / LPR,
        // which holds the row's chunk (l % LPR) ^ swz_row
        constexpr int LPR = D / 8, RPI = 64 / LPR, NI = D * D * 2 / 1024;
        const Rsrc rs = make_rsrc(a.sb + (size_t)__builtin_amdgcn_readfirstlane(bh) * D * D, (uint32_t)(D * D * 2));
#pragma unroll
        for (int jj = 0; jj < NI / 2; ++jj) {
            const int j = 2 * jj + __builtin_amdgcn_readfirstlane(w), r = RPI * j + lane / LPR;
            dma16(rs, reinterpret_cast<unsigned char *>(s_sw) + j * 1024,
                  (uint32_t)(r * D * 2 + (((lane % LPR) ^ swz_row<D>(r)) << 4)));
        }
        wait_vm<0>();
        __syncthreads();
    }
    // partial dS: wave w owns output tiles (a-tile XT w + x, c-tile y), x < XT = D/64,
    // y < D/32
    constexpr int NT = D / 32, XT = NT / 2;
    f32x16 accS[XT][NT];
#pragma unroll
    for (int x = 0; x < XT; ++x)
#pragma unroll
        for (int y = 0; y < NT; ++y) accS[x][y] = f32x16{};
    float dz_acc = 0.f;
    for (int ch = sp; ch < nchunks; ch += a.splits) {
        const int t = ch * kQB + 32 * w + n;
        const bool valid = t < a.Nq;
        const size_t row = (size_t)bh * a.Nq + (valid ? t : 0);
        // phi(q) in the B layout (features 16 ks + 8 g .. + 8) and the denominator
        // every load of the chunk first (the LDS use holds this pass to one wave per SIMD, so
        // the registers are there): q, and the dO and output features this lane meets below
        u32x4 pq[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) pq[ks] = *reinterpret_cast<const u32x4 *>(a.q + row * D + 16 * ks + 8 * g);
        f32x4 gva[NT][4], ova[NT][4];
#pragma unroll
        for (int ft = 0; ft < NT; ++ft)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                gva[ft][v] = *reinterpret_cast<const f32x4 *>(a.dout + row * D + 32 * ft + 16 * g + 4 * v);
                ova[ft][v] = *reinterpret_cast<const f32x4 *>(a.out + row * D + 32 * ft + 16 * g + 4 * v);
            }
        // the dO row in bf16 (round to nearest even) for the dq and dk / dv passes
        if (valid) {
#pragma unroll
            for (int ft = 0; ft < NT; ++ft)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const f32x4 x = gva[ft][2 * h], y = gva[ft][2 * h + 1];
                    *reinterpret_cast<u32x4 *>(a.gr + row * D + 32 * ft + 16 * g + 8 * h) =
                        u32x4{pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w), pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w)};
                }
        }
        float den = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const u32x4 qv = pq[ks];
            const uint32_t wv[4] = {qv.x, qv.y, qv.z, qv.w};
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f0 = phi_f32(bf16_lo_to_f32(wv[e])), f1 = phi_f32(bf16_hi_to_f32(wv[e]));
                den = __builtin_fmaf(f0, zr[ks][e >> 1][2 * (e & 1)], den);
                den = __builtin_fmaf(f1, zr[ks][e >> 1][2 * (e & 1) + 1], den);
                o[e] = pack_bf16x2(f0, f1);
            }
            pq[ks] = u32x4{o[0], o[1], o[2], o[3]};
        }
        den = pair_sum_b(den) + a.eps;
        const float inv_den = 1.f / den;
        // n^T = S^T phi(q): lane holds n[c], c = 32 ft + 16 g + i, and reads dO[c], staging
        // dn = dO / den (bf16) transposed, zero for rows past the queries, for the partials
        // (the previous chunk's partials are done with dnT: the loop's closing barrier)
        const int col = 32 * w + n;
        float gn = 0.f, go = 0.f;
#pragma unroll
        for (int ft = 0; ft < NT; ++ft) {
            // S^T rows 32 ft + perm32(n), features 16 ks + 8 g .. + 8: every fragment read
            // before the first product
            u32x4 sf[D / 16];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) sf[ks] = xt_frag<D>(s_sw, 16 * ks + 8 * g, ft, lane);
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) acc = mfma32(as_bf16x8(sf[ks]), as_bf16x8(pq[ks]), acc);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const f32x4 gv = gva[ft][v], ov = ova[ft][v];
                gn += gv.x * acc[4 * v] + gv.y * acc[4 * v + 1] + gv.z * acc[4 * v + 2] + gv.w * acc[4 * v + 3];
                go += gv.x * ov.x + gv.y * ov.y + gv.z * ov.z + gv.w * ov.w;
                const float gg[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dnT[32 * ft + 16 * g + 4 * v + e][col] = valid ? (uint16_t)f32_to_bf16_bits(gg[e] * inv_den) : 0;
            }
        }
        gn = pair_sum_b(gn);
        go = pair_sum_b(go);
        const float dden = -gn * inv_den * inv_den;
        if (valid && g == 0) a.delta[(size_t)bh * a.NqP + t] = go - gn * inv_den;
        // the readout's term of dq, (S dn + z dden) * phi'(q), is formed by the dq pass from
        // these two per-query values
        if (valid && g == 0) {
            float *rp = a.rod + ((size_t)bh * a.NqP + t) * 2;
            rp[0] = inv_den;
            rp[1] = dden;
        }
        // stage phi(q) transposed, zero for rows past the queries, for the partials
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const uint32_t pw[4] = {pq[ks].x, pq[ks].y, pq[ks].z, pq[ks].w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                phT[16 * ks + 8 * g + e][col] = valid ? (uint16_t)((e & 1) ? (pw[e >> 1] >> 16) : (pw[e >> 1] & 0xFFFF)) : 0;
        }
        if (g == 0) dden_s[col] = valid ? dden : 0.f;
        __syncthreads();
        // dS partial += phi^T dn over the chunk's 64 queries (4 contraction steps of 16)
#pragma unroll
        for (int x = 0; x < XT; ++x) {
            const int ar = 32 * (XT * w + x) + n;
#pragma unroll
            for (int kq = 0; kq < kQB / 16; ++kq) {
                const bf16x8 av = as_bf16x8(*reinterpret_cast<const u32x4 *>(&phT[ar][16 * kq + 8 * g]));
#pragma unroll
                for (int y = 0; y < NT; ++y) {
                    const bf16x8 bv = as_bf16x8(*reinterpret_cast<const u32x4 *>(&dnT[32 * y + n][16 * kq + 8 * g]));
                    accS[x][y] = mfma32(av, bv, accS[x][y]);
                }
            }
        }
        if (threadIdx.x < D) {
            // dz partial of feature threadIdx.x over the chunk's queries, in query order;
            // eight queries per 16-byte read
            float s = 0.f;
#pragma unroll
            for (int q8 = 0; q8 < kQB; q8 += 8) {
                const u32x4 pv = *reinterpret_cast<const u32x4 *>(&phT[threadIdx.x][q8]);
                const f32x4 d0 = *reinterpret_cast<const f32x4 *>(&dden_s[q8]);
                const f32x4 d1 = *reinterpret_cast<const f32x4 *>(&dden_s[q8 + 4]);
                s = __builtin_fmaf(bf16_lo_to_f32(pv.x), d0.x, s);
                s = __builtin_fmaf(bf16_hi_to_f32(pv.x), d0.y, s);
                s = __builtin_fmaf(bf16_lo_to_f32(pv.y), d0.z, s);
                s = __builtin_fmaf(bf16_hi_to_f32(pv.y), d0.w, s);
                s = __builtin_fmaf(bf16_lo_to_f32(pv.z), d1.x, s);
                s = __builtin_fmaf(bf16_hi_to_f32(pv.z), d1.y, s);
                s = __builtin_fmaf(bf16_lo_to_f32(pv.w), d1.z, s);
                s = __builtin_fmaf(bf16_hi_to_f32(pv.w), d1.w, s);
            }
            dz_acc += s;
        }
        __syncthreads();
    }
    // partials: tile (x, y) element i of lane l is (a, c) = (32(XT w+x) + 8(i/4) + 4g + i%4, 32y + n)
    float *dsp = a.dsp + ((size_t)bh * a.splits + sp) * D * D;
#pragma unroll
    for (int x = 0; x < XT; ++x)
#pragma unroll
        for (int y = 0; y < NT; ++y)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int ar = 32 * (XT * w + x) + 8 * (i / 4) + 4 * g + (i % 4);
                dsp[(size_t)ar * D + 32 * y + n] = accS[x][y][i];
            }
    if (threadIdx.x < D) a.dzp[((size_t)bh * a.splits + sp) * D + threadIdx.x] = dz_acc;
}

// Sum of `splits` partials p at src[p * stride] in split order; the loads of sixteen splits
// are issued before their adds, which keep the order (so the result is the serial sum).
__device__ __forceinline__ float ordered_split_sum(const float *src, size_t stride, int splits) {
    float s = 0.f;
    for (int p0 = 0; p0 < splits; p0 += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = p0 + u < splits ? src[(size_t)(p0 + u) * stride] : 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u)
            if (p0 + u < splits) s += v[u];
    }
    return s;
}

// dS, dz = sum of the split partials in split order: one element of dS per thread
// (D * D / 256 workgroups per plane); the plane's first workgroup also adds dz.
template <int D>
__global__ __launch_bounds__(256) void reduce_readout_kernel(hf_bwd_args a) {
    constexpr int per = D * D / 256;
    const int bh = blockIdx.x / per, tile = blockIdx.x % per;
    {
        const int e = 256 * tile + threadIdx.x;
        a.dS[(size_t)bh * D * D + e] = ordered_split_sum(a.dsp + (size_t)bh * a.splits * D * D + e, (size_t)D * D, a.splits);
    }
    if (tile == 0 && threadIdx.x < D)
        a.dz[(size_t)bh * D + threadIdx.x] =
            ordered_split_sum(a.dzp + (size_t)bh * a.splits * D + threadIdx.x, (size_t)D, a.splits);
}

// ---------------------------------------------------------------- dq pass

// One workgroup per query block, one wave per 32-query tile, walking the kept key blocks in
// 32-key subtiles.  Each subtile's K and V rows (both chunk-swizzled, swz_row) reach LDS by
// direct-to-LDS loads into one of two stages, the next subtile's while the current one is
// computed.  The loads go through buffer resources bounded by the plane's rows, so rows past
// the padded window read as zero.
template <int D>
struct DqStage {
    uint16_t k[32 * D];
    uint16_t v[32 * D];
};

// Fragments of four contraction steps (k-steps k0 .. k0 + 3) of the rows that lane reads in
// the S and dP products -- K at the four addresses, V at the same offsets in the V rows --
// in one asm block that waits for all eight reads at its end (every output is complete when
// it ends); left to itself the compiler, short of registers, issues each step's reads just
// before its products and waits for each pair.
template <int D>
__device__ __forceinline__ void dq_kv_reads(const uint32_t (&ad)[2], u32x4 (&fk)[2], u32x4 (&fv)[2]) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %2, %4 offset:%6\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %3, %5 offset:%6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(fk[0]), "=&v"(fk[1]), "=&v"(fv[0]), "=&v"(fv[1])
        : "v"(ad[0]), "v"(ad[1]), "i"(32 * D * 2)
        : "memory");
}

// Every transposed fragment of 16 staged rows for one set of products -- xt_frag(X, r0 +
// 8 ks, ft) for every ft and ks = 0, 1 (r0 a multiple of 16) -- read in one asm block that
// waits once at its end (left to itself the compiler waits for each fragment's pair of
// reads before its product).  Per lane the reads of ks = 1 lie 8 rows (16 D bytes) past
// those of ks = 0: the row swizzle ignores bit 3 of the row.
template <int D>
__device__ __forceinline__ void xt_frags(const uint16_t *X, int r0, int lane, u32x4 (&f)[D / 32][2]) {
    static_assert(D == 64 || D == 128, "head dimension");
    const int s = lane & 15, t = s & 3, G = (lane >> 4) & 1;
    uint32_t ad[D / 32][2];
#pragma unroll
    for (int ft = 0; ft < D / 32; ++ft)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int r = r0 + 4 * hh + (s >> 2);
            const int d = 32 * ft + 8 * G + 16 * (t & 1) + 4 * (t >> 1);
            const int e = r * D + (((d >> 3) ^ swz_row<D>(r)) << 3) + (d & 7);
            ad[ft][hh] = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint16_t *)(X + e);
        }
    u32x2 h[D / 32][2][2];   // [ft][ks][hh]
    if constexpr (D == 128) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %16\n\t"
            "ds_read_b64_tr_b16 %1, %17\n\t"
            "ds_read_b64_tr_b16 %2, %16 offset:%24\n\t"
            "ds_read_b64_tr_b16 %3, %17 offset:%24\n\t"
            "ds_read_b64_tr_b16 %4, %18\n\t"
            "ds_read_b64_tr_b16 %5, %19\n\t"
            "ds_read_b64_tr_b16 %6, %18 offset:%24\n\t"
            "ds_read_b64_tr_b16 %7, %19 offset:%24\n\t"
            "ds_read_b64_tr_b16 %8, %20\n\t"
            "ds_read_b64_tr_b16 %9, %21\n\t"
            "ds_read_b64_tr_b16 %10, %20 offset:%24\n\t"
            "ds_read_b64_tr_b16 %11, %21 offset:%24\n\t"
            "ds_read_b64_tr_b16 %12, %22\n\t"
            "ds_read_b64_tr_b16 %13, %23\n\t"
            "ds_read_b64_tr_b16 %14, %22 offset:%24\n\t"
            "ds_read_b64_tr_b16 %15, %23 offset:%24\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(h[0][0][0]), "=&v"(h[0][0][1]), "=&v"(h[0][1][0]), "=&v"(h[0][1][1]),
              "=&v"(h[1][0][0]), "=&v"(h[1][0][1]), "=&v"(h[1][1][0]), "=&v"(h[1][1][1]),
              "=&v"(h[2][0][0]), "=&v"(h[2][0][1]), "=&v"(h[2][1][0]), "=&v"(h[2][1][1]),
              "=&v"(h[3][0][0]), "=&v"(h[3][0][1]), "=&v"(h[3][1][0]), "=&v"(h[3][1][1])
            : "v"(ad[0][0]), "v"(ad[0][1]), "v"(ad[1][0]), "v"(ad[1][1]), "v"(ad[2][0]), "v"(ad[2][1]),
              "v"(ad[3][0]), "v"(ad[3][1]), "i"(16 * D)
            : "memory");
    } else {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8\n\t"
            "ds_read_b64_tr_b16 %1, %9\n\t"
            "ds_read_b64_tr_b16 %2, %8 offset:%12\n\t"
            "ds_read_b64_tr_b16 %3, %9 offset:%12\n\t"
            "ds_read_b64_tr_b16 %4, %10\n\t"
            "ds_read_b64_tr_b16 %5, %11\n\t"
            "ds_read_b64_tr_b16 %6, %10 offset:%12\n\t"
            "ds_read_b64_tr_b16 %7, %11 offset:%12\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(h[0][0][0]), "=&v"(h[0][0][1]), "=&v"(h[0][1][0]), "=&v"(h[0][1][1]),
              "=&v"(h[1][0][0]), "=&v"(h[1][0][1]), "=&v"(h[1][1][0]), "=&v"(h[1][1][1])
            : "v"(ad[0][0]), "v"(ad[0][1]), "v"(ad[1][0]), "v"(ad[1][1]), "i"(16 * D)
            : "memory");
    }
#pragma unroll
    for (int ft = 0; ft < D / 32; ++ft)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            f[ft][ks] = u32x4{h[ft][ks][0].x, h[ft][ks][0].y, h[ft][ks][1].x, h[ft][ks][1].y};
}

template <int D, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(NW, 2))) void dq_kernel(hf_bwd_args a, float c_log2, float inv_sqrt_d, int lsh) {
    constexpr int LPR = D / 8, RPI = 64 / LPR;      // chunks per row, rows per load instruction
    constexpr int NI = 32 * D * 2 / 1024;           // load instructions per operand and subtile
    constexpr int PW = NI / NW;                     // ... per wave
    static_assert(NI % NW == 0, "load split");
    // one __shared__ object per stage, addressed only with compile-time stage numbers, so
    // that the compiler tells one stage's direct-to-LDS writes from the other's reads
    __shared__ __align__(16) DqStage<D> S0, S1;
    const int bh = blockIdx.x / a.nqb, qb = blockIdx.x % a.nqb;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31, g = lane >> 5;
    const int q0 = qb * a.bq, qend = min(q0 + a.bq, a.Nq);
    const int t = q0 + 32 * w + n;
    const bool valid = t < qend;
    const size_t row = (size_t)bh * a.Nq + (valid ? t : q0);
    u32x4 qf[D / 16], gf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        qf[ks] = *reinterpret_cast<const u32x4 *>(a.q + row * D + 16 * ks + 8 * g);
        gf[ks] = *reinterpret_cast<const u32x4 *>(a.gr + row * D + 16 * ks + 8 * g);
    }
    const float Lq = a.lse[row], Dl = a.delta[(size_t)bh * a.NqP + (valid ? t : q0)];
    const uint32_t plane_bytes = (uint32_t)((size_t)a.NkP * D * 2);
    const Rsrc rk = make_rsrc(a.kr + (size_t)bh * a.NkP * D, plane_bytes);
    const Rsrc rv = make_rsrc(a.vr + (size_t)bh * a.NkP * D, plane_bytes);
    f32x16 acc[D / 32];
#pragma unroll
    for (int ft = 0; ft < D / 32; ++ft) acc[ft] = f32x16{};
    // the kept list through scalar loads (constant address space: written by an earlier
    // launch), so that no vector load sits among the counted direct-to-LDS fetches
    const cint32_p sel = (cint32_p)(a.idx + ((size_t)bh * a.nqb + qb) * a.top_k);
    auto kept = [&](int e) { return min(max(sel[e], 0), a.nkb - 1); };
    // subtiles: 2^lsh per kept block, minus the empty tail of a short last block (the list
    // is ascending, so that block can only be the final entry)
    const int nsub_blk = 1 << lsh;
    int nsubt = a.top_k << lsh;
    {
        const int lastb = kept(a.top_k - 1);
        if (lastb == a.nkb - 1 && a.bk >= 32) nsubt -= nsub_blk - (a.Nk - lastb * a.bk + 31) / 32;
    }
    auto key0_of = [&](int u) { return kept(u >> lsh) * a.bk + ((u & (nsub_blk - 1)) << 5); };
    // this wave's load instructions jj: rows RPI j + lane / LPR of the subtile (j = w PW + jj),
    // LDS slot lane % LPR holding chunk slot ^ swz_row(row)
    uint32_t lo[PW];
#pragma unroll
    for (int jj = 0; jj < PW; ++jj) {
        const int r = RPI * (w * PW + jj) + lane / LPR;
        lo[jj] = (uint32_t)((r * D + 8 * ((lane % LPR) ^ swz_row<D>(r))) * 2);
    }
    // (the whole offset goes in the per-lane operand, which the buffer's range check covers)
    auto fetch = [&](int u, DqStage<D> &st) {
        const uint32_t base = (uint32_t)(key0_of(u) * D * 2);
#pragma unroll
        for (int jj = 0; jj < PW; ++jj) {
            const int j = w * PW + jj;
            dma16(rk, reinterpret_cast<unsigned char *>(st.k) + j * 1024, base + lo[jj]);
            dma16(rv, reinterpret_cast<unsigned char *>(st.v) + j * 1024, base + lo[jj]);
        }
    };
    const int kr = perm32(n), ksw = swz_row<D>(kr);
    auto step = [&](int u, DqStage<D> &cur, DqStage<D> &nxt) __attribute__((always_inline)) {
        // this wave's loads of subtile u have landed, then everyone's, and everyone is done
        // with the other stage, which takes subtile u + 1
        wait_vm<0>();
        lds_barrier();
        if (u + 1 < nsubt) fetch(u + 1, nxt);
        const int k0 = key0_of(u);
        const int b = k0 / a.bk;
        const int nv = min(32, min(b * a.bk + a.bk, a.Nk) - k0);
        // S^T = K Q^T and dP^T = V dO^T: lane holds keys 16 g + i of the subtile for query n
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int k0s = 0; k0s < D / 16; k0s += 2) {
            uint32_t ad[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                ad[kk] = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint16_t *)(
                    cur.k + kr * D + (((2 * (k0s + kk) + g) ^ ksw) << 3));
            u32x4 fk[2], fv[2];
            dq_kv_reads<D>(ad, fk, fv);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                s = mfma32(as_bf16x8(fk[kk]), as_bf16x8(qf[k0s + kk]), s);
                dp = mfma32(as_bf16x8(fv[kk]), as_bf16x8(gf[k0s + kk]), dp);
            }
        }
        // (keys past the subtile's valid ones are masked; a full subtile has none)
        float gt[16];
        auto terms = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c_log2, -Lq));
                if constexpr (decltype(masked)::value) p = 16 * g + i < nv ? p : 0.f;
                gt[i] = p * (dp[i] - Dl);
            }
        };
        if (nv >= 32) terms(std::false_type{});   // uniform per wave
        else terms(std::true_type{});
        u32x4 gfr[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            gfr[ks] = u32x4{pack_bf16x2(gt[8 * ks], gt[8 * ks + 1]), pack_bf16x2(gt[8 * ks + 2], gt[8 * ks + 3]),
                            pack_bf16x2(gt[8 * ks + 4], gt[8 * ks + 5]), pack_bf16x2(gt[8 * ks + 6], gt[8 * ks + 7])};
        // dq^T += K^T G^T: K^T rows 32 ft + perm32(n), keys 16 g + 8 ks .. + 8
        u32x4 kt[D / 32][2];
        xt_frags<D>(cur.k, 16 * g, lane, kt);
#pragma unroll
        for (int ft = 0; ft < D / 32; ++ft)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) acc[ft] = mfma32(as_bf16x8(kt[ft][ks]), as_bf16x8(gfr[ks]), acc[ft]);
    };
    fetch(0, S0);
    int u = 0;
    for (; u + 1 < nsubt; u += 2) {
        step(u, S0, S1);
        step(u + 1, S1, S0);
    }
    if (u < nsubt) step(u, S0, S1);
    // the readout's term, (S dn + z dden) * phi'(q) with dn = dO / den (the bf16 dO rows
    // scaled, rounded to bf16 as the matrix-core operand) and 1 / den, dden from the readout
    // pass; S (bf16 rows, chunk-swizzled like the K rows) is staged in the stages' LDS,
    // 64 rows per stage object
    lds_barrier();             // everyone is done with the last subtile (no load is in flight)
    {
        const Rsrc rs = make_rsrc(a.sb + (size_t)bh * D * D, (uint32_t)(D * D * 2));
        constexpr int NIH = 64 * D * 2 / 1024;      // load instructions per 64 rows
        static_assert(NIH % NW == 0 && sizeof(DqStage<D>) == 64 * D * 2, "S staging");
#pragma unroll
        for (int h = 0; h < D / 64; ++h) {
            unsigned char *dst = reinterpret_cast<unsigned char *>(h == 0 ? &S0 : &S1);
#pragma unroll
            for (int jj = 0; jj < NIH / NW; ++jj) {
                const int j = w * (NIH / NW) + jj, r = RPI * j + lane / LPR;
                dma16(rs, dst + j * 1024, (uint32_t)(((64 * h + r) * D + 8 * ((lane % LPR) ^ swz_row<D>(r))) * 2));
            }
        }
    }
    const float2 rd = *reinterpret_cast<const float2 *>(a.rod + ((size_t)bh * a.NqP + (valid ? t : q0)) * 2);
    u32x4 dnf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const uint32_t wv[4] = {gf[ks].x, gf[ks].y, gf[ks].z, gf[ks].w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(bf16_lo_to_f32(wv[e]) * rd.x, bf16_hi_to_f32(wv[e]) * rd.x);
        dnf[ks] = u32x4{o[0], o[1], o[2], o[3]};
    }
    wait_vm<0>();
    lds_barrier();
#pragma unroll
    for (int ft = 0; ft < D / 32; ++ft) {
        // S rows 32 ft + perm32(n), features 16 ks + 8 g .. + 8: lane holds features 32 ft + 16 g + i
        const int sr = 32 * ft + perm32(n), lr = sr % 64;
        const unsigned char *sb = reinterpret_cast<const unsigned char *>(sr < 64 ? &S0 : &S1) + lr * D * 2;
        f32x16 ro = {};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            ro = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(sb + (((2 * ks + g) ^ swz_row<D>(lr)) << 4))),
                        as_bf16x8(dnf[ks]), ro);
        if (valid) {
            const int a0 = 32 * ft + 16 * g;
            const u32x4 q0v = *reinterpret_cast<const u32x4 *>(a.q + row * D + a0);
            const u32x4 q1v = *reinterpret_cast<const u32x4 *>(a.q + row * D + a0 + 8);
            const uint32_t qw[8] = {q0v.x, q0v.y, q0v.z, q0v.w, q1v.x, q1v.y, q1v.z, q1v.w};
            const float *zr = a.z + (size_t)bh * D + a0;
            float *dqp = a.dq + row * D + a0;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const f32x4 z4 = *reinterpret_cast<const f32x4 *>(zr + 4 * v);
                const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
                float r[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * v + e;
                    const float qx = (i & 1) ? bf16_hi_to_f32(qw[i >> 1]) : bf16_lo_to_f32(qw[i >> 1]);
                    r[e] = acc[ft][i] * inv_sqrt_d + (ro[i] + zz[e] * rd.y) * phi_prime(qx);
                }
                *reinterpret_cast<f32x4 *>(dqp + 4 * v) = f32x4{r[0], r[1], r[2], r[3]};
            }
        }
    }
}

// ---------------------------------------------------------------- dk / dv pass



// One query block's operands, staged unpadded with swizzled chunks by direct-to-LDS loads:
// Q and dO rows (rows of D, chunk c of row r at slot c ^ swz_row(r)), and the block's lse
// and Delta values.
template <int D>
struct QStage {
    uint16_t q[kQB * D], g[kQB * D];
    float aux[2][kQB];            // lse, Delta
};
constexpr int kStagesKV = 4;   // query-block stages: up to three blocks ahead are in flight

// One workgroup per key block: wave (kt, qt) owns the block's 32-key tile kt and the
// 32-query tile qt of every query block that kept it (NKT key tiles x NQT query tiles).
// Each query block's Q and dO rows reach LDS once for all the waves by direct-to-LDS loads,
// kStagesKV - 1 blocks ahead of their use; the products that contract over queries read
// their Q^T / dO^T operands from the same rows with transposing LDS reads.  The two
// query-tile halves of each key tile are added at the end.
// MODE 0 forms dv and dk together (one wave per SIMD: both accumulator sets and the key
// tile's K and V fragments).  MODE 1 forms dv only and MODE 2 dk only, each with two
// query-block stages (one block ahead), so that two workgroups -- two waves per SIMD --
// share a CU; the pair recomputes S and fetches the Q and dO rows twice, and is still the
// faster at 64 x 64 blocks.
template <int D, int NKT, int NQT, int MODE = 0>
__global__ __launch_bounds__(64 * NKT * NQT) __attribute__((amdgpu_waves_per_eu(MODE ? 2 : 1))) void dkdv_kernel(hf_bwd_args a, float c_log2, float inv_sqrt_d) {
    constexpr int NW = NKT * NQT;
    constexpr int NTF = D / 32;                    // 32-feature tiles of dk, dv
    constexpr int LPR = D / 8, RPI = 64 / LPR;    // chunks per row, rows per load instruction
    constexpr int NI = kQB * D * 2 / 1024;         // load instructions per operand (16 for D = 128)
    static_assert(NI % NW == 0, "load split");
    // loads each wave issues per query block: its share of the Q and dO rows, and the lse
    // (even waves) or Delta (odd waves) row -- both when the workgroup has one wave
    constexpr int PER = 2 * (NI / NW) + (NW == 1 ? 2 : 1);
    // stages: one fewer when the loads of two blocks ahead would not fit the wait counter
    constexpr int NS = MODE != 0 ? 2 : (2 * PER < 64 ? kStagesKV : kStagesKV - 1);
    static_assert(PER * (NS - 2) < 64, "vmcnt range");
    // one __shared__ object per stage, addressed only with compile-time stage numbers: the
    // compiler then tells each stage's direct-to-LDS writes from the reads of the others and
    // does not wait for the fetches in flight before reading the current stage
    __shared__ __align__(16) QStage<D> S0, S1, S2, S3;
    static_assert(sizeof(S0) >= (size_t)2 * D * 32 * 4, "reduction space");
    auto stage = [&](auto ic) -> QStage<D> & {
        constexpr int k = decltype(ic)::value % NS;
        if constexpr (k == 0) return S0;
        else if constexpr (k == 1) return S1;
        else if constexpr (k == 2) return S2;
        else return S3;
    };
    // this XCD's share of the key blocks, longest work first
    const int items = a.BH * a.nkb, share = (items + 7) / 8;
    const int slot = (blockIdx.x & 7) * share + (blockIdx.x >> 3);
    if (slot >= items) return;   // uniform per workgroup, before any barrier
    const int item = ((cint32_p)a.korder)[slot];
    const int bh = item / a.nkb, j = item % a.nkb;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, n = lane & 31, g = lane >> 5;
    const int kt = w % NKT, qt = w / NKT;
    const int kj0 = j * a.bk + 32 * kt;
    const int nvk = min(32, min(j * a.bk + a.bk, a.Nk) - kj0);   // keys of this wave (<= 0: none)
    const int key = kj0 + n;                                     // < NkP whenever nvk > 0
    const bool kvalid = n < nvk;
    f32x16 accV[NTF], accK[NTF];
#pragma unroll
    for (int fi = 0; fi < NTF; ++fi) accV[fi] = accK[fi] = f32x16{};
    u32x4 kf[D / 16], vf[D / 16];
    {
        const size_t krow = ((size_t)bh * a.NkP + (nvk > 0 ? key : j * a.bk)) * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            kf[ks] = *reinterpret_cast<const u32x4 *>(a.kr + krow + 16 * ks);
            if constexpr (MODE != 1) vf[ks] = *reinterpret_cast<const u32x4 *>(a.vr + krow + 16 * ks);
        }
    }
    const Rsrc rq = make_rsrc(a.q + (size_t)bh * a.Nq * D, (uint32_t)((size_t)a.Nq * D * 2));
    const Rsrc rg = make_rsrc(a.gr + (size_t)bh * a.Nq * D, (uint32_t)((size_t)a.Nq * D * 2));
    const Rsrc rl = make_rsrc(a.lse + (size_t)bh * a.Nq, (uint32_t)((size_t)a.Nq * 4));
    const Rsrc rd = make_rsrc(a.delta + (size_t)bh * a.NqP, (uint32_t)((size_t)a.NqP * 4));
    // the work lists are read through scalar loads (constant address space: written by
    // earlier launches, read-only here), so that no vector load -- and no wait for one -- sits
    // among the direct-to-LDS fetches, whose counted waits assume they are the only vector
    // memory operations in flight
    const cint32_p off = (cint32_p)(a.qoff + (size_t)bh * (a.nkb + 1));
    const cint32_p list = (cint32_p)(a.qlist + (size_t)bh * a.nqb * a.top_k);
    const int p0 = off[j], p1 = off[j + 1];
    // fetch query block p into stage T: every wave issues its PER instructions
    auto fetch = [&](int p, QStage<D> &T) {
        const int i = min(max(list[p], 0), a.nqb - 1);
        const int q0 = i * a.bq, nqv = min(a.bq, a.Nq - q0);
#pragma unroll
        for (int jj = w * (NI / NW); jj < (w + 1) * (NI / NW); ++jj) {
            // rows of D: lane -> row RPI jj + lane / LPR, slot lane % LPR
            const int r = RPI * jj + lane / LPR, c = (lane % LPR) ^ swz_row<D>(r);
            const uint32_t ro = (uint32_t)(((q0 + min(r, nqv - 1)) * D + 8 * c) * 2);
            dma16(rq, reinterpret_cast<unsigned char *>(T.q) + jj * 1024, ro);
            dma16(rg, reinterpret_cast<unsigned char *>(T.g) + jj * 1024, ro);
        }
        const uint32_t eo = (uint32_t)((q0 + min(lane, nqv - 1)) * 4);
        if (NW == 1 || (w & 1) == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (LdsPtr)&T.aux[0][0], 4, (int)eo, 0, 0, 0);
        if (NW == 1 || (w & 1) == 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (LdsPtr)&T.aux[1][0], 4, (int)eo, 0, 0, 0);
    };
    // (a key block no query block kept skips the loop and writes zero gradients)
    // Every step fetches, past the end repeating the last block into a stage that is not
    // read again, so that exactly NS - 2 blocks' loads follow block p's at its wait: one
    // constant count, which the compiler's own wait tracking follows exactly (a fetch under
    // a branch makes it fall back to waiting for every load in flight).
    if (p0 < p1) {
        fetch(p0, stage(std::integral_constant<int, 0>{}));
        if constexpr (NS > 2) fetch(min(p0 + 1, p1 - 1), stage(std::integral_constant<int, 1>{}));
        if constexpr (NS > 3) fetch(min(p0 + 2, p1 - 1), stage(std::integral_constant<int, 2>{}));
    }
    // block p (the ST-th of its group of NS) is in stage ST
    auto step = [&](int p, auto ic) __attribute__((always_inline)) {
        constexpr int ST = decltype(ic)::value;
        QStage<D> &cur = stage(ic);
        const int i = min(max(list[p], 0), a.nqb - 1);
        const int nqv = min(a.bq, a.Nq - i * a.bq);
        // this wave's loads of block p have landed (the next NS - 2 blocks' may still fly);
        // then everyone's, and everyone is done with block p - 1, whose stage is refilled next
        wait_vm<(NS - 2) * PER>();
        lds_barrier();   // not __syncthreads(): its fence would wait for the fetches in flight
        fetch(min(p + NS - 1, p1 - 1), stage(std::integral_constant<int, ST + NS - 1>{}));
        if (nvk <= 0 || 32 * qt >= nqv) return;   // uniform per wave; the barrier is above
        const uint16_t *Lq = cur.q, *Lg = cur.g;
        const float *s_lse = cur.aux[0], *s_delta = cur.aux[1];
        // S and dP for queries 32 qt + (rows in perm32 order), this wave's keys
        const int qr = 32 * qt + perm32(n);
        const int qsw = swz_row<D>(qr);
        f32x16 s = {}, dp = {};
        // the Q and dO fragments of four contraction steps are read in one asm block that
        // waits for all eight reads at its end (every output is complete when it ends): left
        // to itself the compiler, short of registers at one wave per SIMD, issues each
        // step's two reads just before its two products and waits for each pair.  A
        // stage's dO rows sit kQB * D * 2 bytes after its Q rows.
#pragma unroll
        for (int k0 = 0; k0 < D / 16; k0 += 4) {
            uint32_t ad[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                ad[kk] = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint16_t *)(Lq + qr * D + ((2 * (k0 + kk) + g) ^ qsw) * 8);
            u32x4 fq[4], fg[4];
            asm volatile(
                "ds_read_b128 %0, %8\n\t"
                "ds_read_b128 %4, %8 offset:%12\n\t"
                "ds_read_b128 %1, %9\n\t"
                "ds_read_b128 %5, %9 offset:%12\n\t"
                "ds_read_b128 %2, %10\n\t"
                "ds_read_b128 %6, %10 offset:%12\n\t"
                "ds_read_b128 %3, %11\n\t"
                "ds_read_b128 %7, %11 offset:%12\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(fq[0]), "=&v"(fq[1]), "=&v"(fq[2]), "=&v"(fq[3]), "=&v"(fg[0]), "=&v"(fg[1]), "=&v"(fg[2]), "=&v"(fg[3])
                : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "i"(kQB * D * 2)
                : "memory");
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                s = mfma32(as_bf16x8(fq[kk]), as_bf16x8(kf[k0 + kk]), s);
                if constexpr (MODE != 1) dp = mfma32(as_bf16x8(fg[kk]), as_bf16x8(vf[k0 + kk]), dp);
            }
        }
        // lane (key n) holds queries 32 qt + 16 g + i.  Only query rows past the block's end
        // are masked (they repeat its last query): a key past the end feeds only its own
        // columns of dv, dk, which are never stored.
        const int qb0 = 32 * qt + 16 * g;
        float lv[16], dl[16];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const f32x4 l4 = *reinterpret_cast<const f32x4 *>(s_lse + qb0 + 4 * v);
            const f32x4 d4 = *reinterpret_cast<const f32x4 *>(s_delta + qb0 + 4 * v);
            lv[4 * v] = l4.x, lv[4 * v + 1] = l4.y, lv[4 * v + 2] = l4.z, lv[4 * v + 3] = l4.w;
            dl[4 * v] = d4.x, dl[4 * v + 1] = d4.y, dl[4 * v + 2] = d4.z, dl[4 * v + 3] = d4.w;
        }
        float pv[16], gv[16];
        auto terms = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
            for (int i2 = 0; i2 < 16; ++i2) {
                float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i2], c_log2, -lv[i2]));
                if constexpr (decltype(masked)::value) pr = qb0 + i2 < nqv ? pr : 0.f;
                pv[i2] = pr;
                if constexpr (MODE != 1) gv[i2] = pr * (dp[i2] - dl[i2]);
            }
        };
        if (32 * qt + 32 <= nqv) terms(std::false_type{});   // uniform per wave
        else terms(std::true_type{});
        u32x4 pf[2], gfr[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            pf[ks] = u32x4{pack_bf16x2(pv[8 * ks], pv[8 * ks + 1]), pack_bf16x2(pv[8 * ks + 2], pv[8 * ks + 3]),
                           pack_bf16x2(pv[8 * ks + 4], pv[8 * ks + 5]), pack_bf16x2(pv[8 * ks + 6], pv[8 * ks + 7])};
            if constexpr (MODE != 1)
            gfr[ks] = u32x4{pack_bf16x2(gv[8 * ks], gv[8 * ks + 1]), pack_bf16x2(gv[8 * ks + 2], gv[8 * ks + 3]),
                            pack_bf16x2(gv[8 * ks + 4], gv[8 * ks + 5]), pack_bf16x2(gv[8 * ks + 6], gv[8 * ks + 7])};
        }
        // dv^T += dO^T P, dk^T += Q^T G (rows d in perm32 order; this lane half's queries
        // 32 qt + 16 g + 8 ks .. + 8, the order in which P and G are packed).  Rows past the
        // block's end repeat its last query and meet P = G = 0.
        // all transposed fragments of one operand are read before its products
        u32x4 xg[NTF][2];
        if constexpr (MODE != 2) {
        xt_frags<D>(Lg, 32 * qt + 16 * g, lane, xg);
#pragma unroll
        for (int fi = 0; fi < NTF; ++fi)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) accV[fi] = mfma32(as_bf16x8(xg[fi][ks]), as_bf16x8(pf[ks]), accV[fi]);
        }
        if constexpr (MODE != 1) {
        xt_frags<D>(Lq, 32 * qt + 16 * g, lane, xg);
#pragma unroll
        for (int fi = 0; fi < NTF; ++fi)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) accK[fi] = mfma32(as_bf16x8(xg[fi][ks]), as_bf16x8(gfr[ks]), accK[fi]);
        }
    };
    int p = p0;
    for (; p + NS <= p1; p += NS) {
        step(p, std::integral_constant<int, 0>{});
        step(p + 1, std::integral_constant<int, 1>{});
        if constexpr (NS > 2) step(p + 2, std::integral_constant<int, 2>{});
        if constexpr (NS > 3) step(p + 3, std::integral_constant<int, 3>{});
    }
    if (p < p1) step(p, std::integral_constant<int, 0>{});
    if (p + 1 < p1) step(p + 1, std::integral_constant<int, 1>{});
    if (NS > 3 && p + 2 < p1) step(p + 2, std::integral_constant<int, 2>{});
    __builtin_amdgcn_s_waitcnt(0x0F70);   // no load in flight before the stages are reused
    if constexpr (NQT > 1) {
        // query-tile halves, one key tile at a time: the waves with qt = 1 hand their sums
        // to the waves with qt = 0
        float *red = reinterpret_cast<float *>(&S0);
        for (int kk = 0; kk < NKT; ++kk) {
            __syncthreads();
            if (qt == 1 && kt == kk) {
#pragma unroll
                for (int fi = 0; fi < NTF; ++fi)
#pragma unroll
                    for (int i2 = 0; i2 < 16; ++i2) {
                        if constexpr (MODE != 2) red[(0 * (D / 32) + fi) * 16 * 64 + i2 * 64 + lane] = accV[fi][i2];
                        if constexpr (MODE != 1) red[(1 * (D / 32) + fi) * 16 * 64 + i2 * 64 + lane] = accK[fi][i2];
                    }
            }
            __syncthreads();
            if (qt == 0 && kt == kk) {
#pragma unroll
                for (int fi = 0; fi < NTF; ++fi)
#pragma unroll
                    for (int i2 = 0; i2 < 16; ++i2) {
                        if constexpr (MODE != 2) accV[fi][i2] += red[(0 * (D / 32) + fi) * 16 * 64 + i2 * 64 + lane];
                        if constexpr (MODE != 1) accK[fi][i2] += red[(1 * (D / 32) + fi) * 16 * 64 + i2 * 64 + lane];
                    }
            }
        }
        if (qt != 0) return;
    }
    if (kvalid) {
        // lane (key n) holds features 32 fi + 16 g + i of its feature tiles fi
        float *dvp = a.dv + ((size_t)bh * a.Nk + key) * D + 16 * g;
        float *dkp = a.dk + ((size_t)bh * a.Nk + key) * D + 16 * g;
#pragma unroll
        for (int fi = 0; fi < NTF; ++fi) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                if constexpr (MODE != 2)
                *reinterpret_cast<f32x4 *>(dvp + 32 * fi + 4 * v) =
                    f32x4{accV[fi][4 * v], accV[fi][4 * v + 1], accV[fi][4 * v + 2], accV[fi][4 * v + 3]};
                if constexpr (MODE != 1)
                *reinterpret_cast<f32x4 *>(dkp + 32 * fi + 4 * v) =
                    f32x4{accK[fi][4 * v] * inv_sqrt_d, accK[fi][4 * v + 1] * inv_sqrt_d,
                          accK[fi][4 * v + 2] * inv_sqrt_d, accK[fi][4 * v + 3] * inv_sqrt_d};
            }
        }
    }
}

// ---------------------------------------------------------------- absorb backward

template <int D>
__global__ __launch_bounds__(256) void absorb_bwd_prep_kernel(hf_absorb_bwd_args a) {
    __shared__ float t[32][33];
    mat_copies<D>(a.dS, a.sb, a.stb, blockIdx.x, t);
}

// One wave per (plane, 32 tokens): dv^T = dS^T phi(K)^T and dphi^T = dS V^T on the matrix
// cores (rows in perm32 order, so each lane holds 16 consecutive features of its token).
template <int D>
__global__ __launch_bounds__(64) void absorb_bwd_kernel(hf_absorb_bwd_args a) {
    const int64_t tiles = (a.n_tok + 31) / 32;
    const int bh = (int)(blockIdx.x / tiles);
    const int64_t u0 = (blockIdx.x % tiles) * 32;
    const int lane = threadIdx.x, n = lane & 31, g = lane >> 5;
    const int64_t u = u0 + n;
    const bool valid = u < a.n_tok;
    const size_t row = ((size_t)bh * a.n_tok + (valid ? u : u0)) * D;
    u32x4 phf[D / 16], vf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 kv = *reinterpret_cast<const u32x4 *>(a.k + row + 16 * ks + 8 * g);
        const uint32_t wv[4] = {kv.x, kv.y, kv.z, kv.w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(phi_f32(bf16_lo_to_f32(wv[e])), phi_f32(bf16_hi_to_f32(wv[e])));
        phf[ks] = u32x4{o[0], o[1], o[2], o[3]};
        vf[ks] = *reinterpret_cast<const u32x4 *>(a.v + row + 16 * ks + 8 * g);
    }
    const uint16_t *sbp = a.sb + (size_t)bh * D * D, *stp = a.stb + (size_t)bh * D * D;
    const float *dzp = a.dz + (size_t)bh * D;
#pragma unroll
    for (int ft = 0; ft < D / 32; ++ft) {
        f32x16 dvt = {}, dpt = {};
        const uint16_t *r1 = stp + (size_t)(32 * ft + perm32(n)) * D + 8 * g;
        const uint16_t *r2 = sbp + (size_t)(32 * ft + perm32(n)) * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            dvt = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(r1 + 16 * ks)), as_bf16x8(phf[ks]), dvt);
            dpt = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(r2 + 16 * ks)), as_bf16x8(vf[ks]), dpt);
        }
        if (valid) {
            const int a0 = 32 * ft + 16 * g;
            const u32x4 k0 = *reinterpret_cast<const u32x4 *>(a.k + row + a0);
            const u32x4 k1 = *reinterpret_cast<const u32x4 *>(a.k + row + a0 + 8);
            const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float r[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * v + e;
                    const float kx = (i & 1) ? bf16_hi_to_f32(kw[i >> 1]) : bf16_lo_to_f32(kw[i >> 1]);
                    r[e] = (dpt[i] + dzp[a0 + i]) * phi_prime(kx);
                }
                *reinterpret_cast<f32x4 *>(a.dk + row + a0 + 4 * v) = f32x4{r[0], r[1], r[2], r[3]};
                *reinterpret_cast<f32x4 *>(a.dv + row + a0 + 4 * v) = f32x4{dvt[4 * v], dvt[4 * v + 1], dvt[4 * v + 2], dvt[4 * v + 3]};
            }
        }
    }
}

template <int D>
hipError_t launch_attn_backward(const hf_bwd_args &a, hipStream_t s) {
    const int nt = D / 32;
    const float c_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    const float inv_sqrt_d = (float)(1.0 / sqrt((double)D));
    const int lsh = a.bk >= 128 ? 2 : (a.bk >= 64 ? 1 : 0);
    hipLaunchKernelGGL(prep_keys_kernel<D>, dim3((unsigned)(a.BH * (a.NkP / 64) + a.BH * nt * nt)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(csr_kernel, dim3((unsigned)a.BH), dim3(256), 0, s, a);
    hipLaunchKernelGGL(order_kernel, dim3(8), dim3(1024), 0, s, a);
    hipLaunchKernelGGL(readout_bwd_kernel<D>, dim3((unsigned)(a.BH * a.splits)), dim3(128), 0, s, a);
    hipLaunchKernelGGL(reduce_readout_kernel<D>, dim3((unsigned)(a.BH * (D * D / 256))), dim3(256), 0, s, a);
    if (a.bq > 32)
        hipLaunchKernelGGL((dq_kernel<D, 2>), dim3((unsigned)(a.BH * a.nqb)), dim3(128), 0, s, a, c_log2, inv_sqrt_d, lsh);
    else
        hipLaunchKernelGGL((dq_kernel<D, 1>), dim3((unsigned)(a.BH * a.nqb)), dim3(64), 0, s, a, c_log2, inv_sqrt_d, lsh);
    const dim3 gk((unsigned)((a.BH * a.nkb + 7) / 8 * 8));
    // key tiles (bk / 32, at least 1) x query tiles (bq / 32, at least 1) waves; 64 x 64
    // blocks take the dv and dk launches apart
    if (a.bq > 32) {
        if (a.bk > 64) hipLaunchKernelGGL((dkdv_kernel<D, 4, 2>), gk, dim3(512), 0, s, a, c_log2, inv_sqrt_d);
        else if (a.bk > 32) {
            hipLaunchKernelGGL((dkdv_kernel<D, 2, 2, 1>), gk, dim3(256), 0, s, a, c_log2, inv_sqrt_d);
            hipLaunchKernelGGL((dkdv_kernel<D, 2, 2, 2>), gk, dim3(256), 0, s, a, c_log2, inv_sqrt_d);
        } else hipLaunchKernelGGL((dkdv_kernel<D, 1, 2>), gk, dim3(128), 0, s, a, c_log2, inv_sqrt_d);
    } else {
        if (a.bk > 64) hipLaunchKernelGGL((dkdv_kernel<D, 4, 1>), gk, dim3(256), 0, s, a, c_log2, inv_sqrt_d);
        else if (a.bk > 32) hipLaunchKernelGGL((dkdv_kernel<D, 2, 1>), gk, dim3(128), 0, s, a, c_log2, inv_sqrt_d);
        else hipLaunchKernelGGL((dkdv_kernel<D, 1, 1>), gk, dim3(64), 0, s, a, c_log2, inv_sqrt_d);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_absorb_backward(const hf_absorb_bwd_args &a, hipStream_t s) {
    const int nt = D / 32;
    hipLaunchKernelGGL(absorb_bwd_prep_kernel<D>, dim3((unsigned)(a.BH * nt * nt)), dim3(256), 0, s, a);
    const int64_t tiles = (a.n_tok + 31) / 32;
    hipLaunchKernelGGL(absorb_bwd_kernel<D>, dim3((unsigned)(a.BH * tiles)), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace
}  // namespace hf

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int bwd_splits(int BH, int Nq) {
    const int chunks = (Nq + hf::kQB - 1) / hf::kQB;
    int s = 512 / BH;   // the readout pass fits two workgroups per CU
    s = s < 1 ? 1 : s;
    return s < chunks ? s : chunks;
}

// Workspace: K rows, V rows, dO rows, S / S^T bf16, Delta,
// the selection transpose, readout partials (each region 256-byte aligned).
static size_t bwd_layout(hf_bwd_args *a, int BH, int D, int Nq, int Nk, int bq, int bk, int top_k, char *base) {
    const int nqb = (Nq + bq - 1) / bq, nkb = (Nk + bk - 1) / bk;
    const int NkP = (Nk + 63) / 64 * 64, NqP = nqb * bq;
    const int splits = bwd_splits(BH, Nq);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += align256(bytes);
        return base ? base + at : nullptr;
    };
    char *kr = take((size_t)BH * NkP * D * 2), *vr = take((size_t)BH * NkP * D * 2);
    char *gr = take((size_t)BH * Nq * D * 2);
    char *sb = take((size_t)BH * D * D * 2), *stb = take((size_t)BH * D * D * 2);
    char *delta = take((size_t)BH * NqP * 4), *rod = take((size_t)BH * NqP * 2 * 4);
    char *qoff = take((size_t)BH * (nkb + 1) * 4), *qlist = take((size_t)BH * nqb * top_k * 4);
    char *korder = take((size_t)BH * nkb * 4);
    char *dsp = take((size_t)BH * splits * D * D * 4), *dzp = take((size_t)BH * splits * D * 4);
    if (a) {
        a->NkP = NkP;
        a->NqP = NqP;
        a->splits = splits;
        a->kr = reinterpret_cast<uint16_t *>(kr);
        a->vr = reinterpret_cast<uint16_t *>(vr);
        a->gr = reinterpret_cast<uint16_t *>(gr);
        a->sb = reinterpret_cast<uint16_t *>(sb);
        a->stb = reinterpret_cast<uint16_t *>(stb);
        a->delta = reinterpret_cast<float *>(delta);
        a->rod = reinterpret_cast<float *>(rod);
        a->qoff = reinterpret_cast<int32_t *>(qoff);
        a->qlist = reinterpret_cast<int32_t *>(qlist);
        a->korder = reinterpret_cast<int32_t *>(korder);
        a->dsp = reinterpret_cast<float *>(dsp);
        a->dzp = reinterpret_cast<float *>(dzp);
    }
    return o;
}

size_t hf_bwd_workspace_bytes(int BH, int D, int Nq, int Nk, int bq, int bk, int top_k) {
    return bwd_layout(nullptr, BH, D, Nq, Nk, bq, bk, top_k, nullptr);
}

void hf_bwd_layout(hf_bwd_args &a, void *ws) {
    bwd_layout(&a, a.BH, a.D, a.Nq, a.Nk, a.bq, a.bk, a.top_k, static_cast<char *>(ws));
}

hipError_t hf_launch_attn_backward(const hf_bwd_args &a, hipStream_t s) {
    if (a.nkb > kMaxKeyBlocks) return hipErrorInvalidValue;
    return a.D == 64 ? hf::launch_attn_backward<64>(a, s) : hf::launch_attn_backward<128>(a, s);
}

hipError_t hf_launch_absorb_backward(const hf_absorb_bwd_args &a, hipStream_t s) {
    if (a.n_tok <= 0) return hipSuccess;
    return a.D == 64 ? hf::launch_absorb_backward<64>(a, s) : hf::launch_absorb_backward<128>(a, s);
}
