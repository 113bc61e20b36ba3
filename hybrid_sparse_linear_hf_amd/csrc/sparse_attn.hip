// Block-sparse window attention with the linear readout fused into its epilogue.
//
// Sparse branch ([HF-de] §2.A "Block-Sparse Sliding Window Attention", [HF-pt] §2.A.2):
// every query of query block i attends with softmax weights to the keys of its kept key
// blocks only.  Linear branch ([HF-de] §2.A "Lineare Zeit-Aufmerksamkeit", [HF-pt]
// §2.A.1, [HF-abs]): phi(q)^T S / (phi(q) . z + eps) from the compact state.  The output
// is their sum ([HF-de] §2.A "Kombination", [HF-pt] §2.A "Resultado").
//
// gfx950 design
//   * A workgroup owns one query block; each of its wavefronts owns one 32-query tile
//     (two waves for 64-query blocks).  At most 256 registers per wave, so two waves share
//     a SIMD and the hardware overlaps one wave's softmax with the other's matrix-core
//     work.  Workgroup ids are remapped so that the query blocks of one plane run on one
//     XCD and share its L2 for the window's K/V.
//   * The kept key blocks are walked in 32-key subtiles.  Each subtile's K rows and V^T
//     columns are fetched with direct-to-LDS buffer loads (16 bytes per lane, whole 256-byte
//     K rows and 64-byte V^T row segments per instruction, so every load is coalesced) into
//     a double-buffered LDS stage, one subtile ahead of the compute; the two waves share
//     the fetch.  Chunk positions are XOR-swizzled per row, so that the 16-byte reads in
//     matrix-core operand order hit distinct LDS banks.
//   * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16: the probabilities leave
//     the first product in the register layout the second consumes.  Key rows are read in
//     the order perm32(m), so each lane holds 16 consecutive keys of its query column, and
//     value rows (features) likewise, so each lane holds 16 consecutive output features.
//   * Relative temporal rotary embedding (instances KT > 0; [HF-de] §2.C "Relative RoPE",
//     [HF-pt] §2.B.2): a query scored against a key of window frame f uses its first DT
//     features turned pairwise by the clamped frame offset clamp(fq - f, -cap, cap).
//     The kept list is ascending, so the key frame changes at most once per frame of the
//     window: the turned fragments (bf16, like every matrix-core operand) are rebuilt in
//     registers only then.  A subtile that spans several frames runs the temporal
//     products once per frame on top of a shared spatial product and picks each key's
//     row.  The readout uses the raw query.
//   * Softmax in base 2 with the 1/sqrt(D) scale folded into one FMA.  Full subtiles use a
//     FIXED reference per query row -- the exact row maximum of the first subtile -- so
//     nothing is ever rescaled; should a later score exceed it by so much that the row sum
//     reaches 2^32, the block is recomputed with an online (rescaling) softmax.  Short
//     subtiles (the tail of a short last key block; every subtile when bk < 32) use the
//     online softmax with masking.
#include <type_traits>

#include "hf_internal.h"

namespace hf {
namespace {

constexpr int kSub = 32;                      // keys per subtile
constexpr int kBufDword3 = 0x00020000;        // raw buffer resource word 3 (gfx9 family)
constexpr float kLazyRescaleLog2 = 8.0f;
constexpr float kFixedRefLimit = 4294967296.0f;   // 2^32

typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef __attribute__((address_space(3))) void *LdsPtr;

__device__ __forceinline__ Rsrc make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufDword3);
}

// 16 bytes per lane from the buffer into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(Rsrc r, unsigned char *lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)lds, 16, (int)voff, 0, 0, 0);
}

// Reductions over the lane pair (l, l ^ 32) that holds the two key halves of one query.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS chunk swizzles (16-byte chunks).  K rows hold D/8 chunks; V^T rows (one feature,
// the subtile's 32 keys) hold 4.  Chosen so that the operand reads below touch 16 distinct
// bank groups per 16 lanes.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
    if constexpr (D == 128) return ((r & 3) << 1) | ((r >> 2) & 1) | ((r >> 1) & 8);
    else return ((r >> 1) & 3) | ((r >> 2) & 4);
}
__device__ __forceinline__ int swz_v(int f) { return ((f >> 4) & 1) | (((f >> 2) & 1) << 1); }

struct SmState {
    float m;     // reference maximum of s * c_log2 (base-2 logits)
    float l;     // this lane's partial row sum
};

__device__ __forceinline__ float tile_max_log2(const f32x16 &s, float c_log2) {
    float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
    mx = fmaxf(mx, s[15]);
    return pair_max(mx) * c_log2;
}

__device__ __forceinline__ void pack_p(const float (&p)[16], u32x4 (&pf)[2]) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        pf[ks].x = pack_bf16x2(p[8 * ks + 0], p[8 * ks + 1]);
        pf[ks].y = pack_bf16x2(p[8 * ks + 2], p[8 * ks + 3]);
        pf[ks].z = pack_bf16x2(p[8 * ks + 4], p[8 * ks + 5]);
        pf[ks].w = pack_bf16x2(p[8 * ks + 6], p[8 * ks + 7]);
    }
}

__device__ __forceinline__ float sum16(const float (&p)[16]) {
    return (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]))) +
           (((p[8] + p[9]) + (p[10] + p[11])) + ((p[12] + p[13]) + (p[14] + p[15])));
}

// Full tile against the fixed reference: p = 2^(s c - m).
__device__ __forceinline__ void softmax_fixed(const f32x16 &s, float c_log2, float moff, float &l, u32x4 (&pf)[2]) {
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c_log2, moff));
    l += sum16(p);
    pack_p(p, pf);
}

// Masked online softmax (keys 16g + i >= nval excluded); returns the factor the output
// accumulator must be scaled by (1 when unchanged).
__device__ __forceinline__ float softmax_online(f32x16 s, int nval, int g, float c_log2, SmState &st, u32x4 (&pf)[2]) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (16 * g + i >= nval) s[i] = -INFINITY;
    const float mx = tile_max_log2(s, c_log2);
    const float mnew = (mx > st.m + kLazyRescaleLog2) ? mx : st.m;
    const float alpha = (mnew == st.m) ? 1.f : __builtin_amdgcn_exp2f(st.m - mnew);
    st.m = mnew;
    const float moff = -fmaxf(mnew, -3.0e38f);   // finite even while every key so far was masked
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c_log2, moff));
    st.l = __builtin_fmaf(st.l, alpha, sum16(p));
    pack_p(p, pf);
    return alpha;
}

constexpr int kWaitVm0 = 0x0F70;   // s_waitcnt vmcnt(0), other counters untouched

// D = head dim; NW = waves per workgroup = 32-query tiles per query block (2 when bq == 64);
// KT = temporal fragments of the relative rotation (DT / 16; 0: no rotation).
template <int D, int NW, int KT>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2))) void
sparse_attn_kernel(hf_attn_args a, uint32_t magicT, float c_log2, int per_xcd, int lsh) {
    constexpr int LPR = D / 8;            // 16-byte chunks per K row
    constexpr int RPI = 64 / LPR;         // K rows per load instruction
    constexpr int NK = kSub / RPI;        // K load instructions per subtile
    constexpr int NV = D / 16;            // V^T load instructions per subtile (16 feature rows each)
    constexpr int KW = NK / NW, VW = NV / NW;
    constexpr int KBYTES = kSub * D * 2, VBYTES = D * 64;

    // dynamic LDS: [K stage 0][K stage 1][V stage 0][V stage 1][kept list][NW flags]
    extern __shared__ __align__(16) unsigned char dyn[];
    const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (item >= a.BH * a.nqb) return;   // uniform per workgroup
    const int bh = item / a.nqb, qb = item - bh * a.nqb;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, n = lane & 31, g = lane >> 5;
    const int q0 = qb * a.bq, qend = min(q0 + a.bq, a.Nq);
    unsigned char *const kst = dyn, *const vst = dyn + 2 * KBYTES;
    int32_t *s_blist = reinterpret_cast<int32_t *>(dyn + 2 * (KBYTES + VBYTES));
    int *s_flag = reinterpret_cast<int *>(s_blist + a.top_k);

    // kept blocks -> LDS (out-of-range entries, a caller error, are clamped so that no load
    // leaves the window)
    const int32_t *sel = a.idx + ((size_t)bh * a.nqb + qb) * a.top_k;
    for (int t = threadIdx.x; t < a.top_k; t += 64 * NW) s_blist[t] = min(max(sel[t], 0), a.nkb - 1);

    // this wave's Q^T B fragments: query q0 + 32w + n (clamped into the block), features
    // 16ks + 8g .. + 8
    u32x4 qf[D / 16];
    {
        int row = q0 + 32 * w + n;
        row = row < qend ? row : q0;
        const uint16_t *qp = a.q + ((size_t)bh * a.Nq + row) * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const u32x4 *>(qp + 16 * ks);
    }
    __syncthreads();

    // rotation: this lane's query frame (window order) and the KT temporal fragments of Q^T
    // turned for key frame qt_f
    constexpr bool ROPE = KT > 0;
    int fq = 0, qt_f = -1;
    u32x4 qt[ROPE ? KT : 1];
    if constexpr (ROPE) {
        const int row = q0 + 32 * w + n;
        fq = a.ncom + fast_div(row < qend ? row : q0, magicT, a.T);
    }
    // feature pair 8ks + 4g + j of the fragments turns by clamp(fq - f, -cap, cap) *
    // theta_i, theta_i = base^(-2i/DT) = 2^(i * rope_c1)
    auto set_qt = [&](int f) __attribute__((always_inline)) {
        if (f == qt_f) return;
        qt_f = f;
        const float off = (float)min(max(fq - f, -a.rope_cap), a.rope_cap);
        // |angle| = 2^(i * rope_c1 + log2|off|): formed from the offset (0 for off = 0), so
        // that no per-pair frequency stays live in registers between frame changes
        const float lg = __log2f(fabsf(off));
#pragma unroll
        for (int ks = 0; ks < KT; ++ks) {
            const uint32_t wv[4] = {qf[ks].x, qf[ks].y, qf[ks].z, qf[ks].w};
            uint32_t o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float ang = copysignf(__builtin_amdgcn_exp2f(__builtin_fmaf((float)(8 * ks + 4 * g + j), a.rope_c1, lg)), off);
                const float sn = __sinf(ang), cs = __cosf(ang);
                const float x0 = bf16_lo_to_f32(wv[j]), x1 = bf16_hi_to_f32(wv[j]);
                o[j] = pack_bf16x2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
            }
            qt[ks] = u32x4{o[0], o[1], o[2], o[3]};
        }
    };

    const size_t plane = (size_t)bh * a.W * a.T * D;
    const uint32_t plane_bytes = (uint32_t)((size_t)a.W * a.T * D * 2);
    const Rsrc rk = make_rsrc(a.ring_k + plane, plane_bytes);
    const Rsrc rv = make_rsrc(a.ring_vt + plane, plane_bytes);
    const int T = a.T, W = a.W, head = a.head;

    // ---- subtile list: 2^lsh subtiles per kept block, minus the empty tail of a short last
    // block (the list is ascending, so that block can only be the final entry)
    const int nsub_blk = 1 << lsh;
    int nsubt = a.top_k << lsh;
    int nfull = (a.bk >= kSub && T >= kSub) ? nsubt : 0;
    {
        const int lastb = s_blist[a.top_k - 1];
        if (lastb == a.nkb - 1 && a.bk >= kSub) {
            const int len = a.Nk - lastb * a.bk;
            nsubt -= nsub_blk - (len + kSub - 1) / kSub;
            if (nfull) nfull = nsubt - ((len & (kSub - 1)) ? 1 : 0);
        }
    }
    auto key0_of = [&](int u) -> int {
        const int b = __builtin_amdgcn_readfirstlane(s_blist[u >> lsh]);
        return b * a.bk + ((u & (nsub_blk - 1)) << 5);
    };
    auto nval_of = [&](int k0) -> int {
        const int b = k0 / a.bk;
        return min(min(kSub, b * a.bk + a.bk - k0), a.Nk - k0);
    };
    auto slot_of = [&](int f) -> int {
        const int s = head + f;
        return s >= W ? s - W : s;
    };

    // ---- per-lane load plan; this wave issues K instructions w*KW .. and V instructions w*VW ..
    // Both stages are row-major with chunk positions swizzled per row: K row r (key r of the
    // subtile) holds D/8 chunks, V^T row f (feature f) the subtile's 4 eight-key chunks.
    // One instruction fetches RPI whole K rows, or 16 whole V^T row segments.
    // Subtiles start at multiples of 32 keys and T is a multiple of 8, so a frame boundary
    // inside a subtile falls on a multiple of 8 keys and never inside a K instruction's rows:
    // the K frame choice is a scalar offset.  A V^T instruction spans all 32 keys, so a
    // subtile that crosses a frame boundary takes a per-lane path.
    uint32_t kvo[KW], vvo[VW];
    int krow[KW], vkr[VW];
#pragma unroll
    for (int jj = 0; jj < KW; ++jj) {
        const int j = w * KW + jj;
        const int r = RPI * j + lane / LPR;
        const int c = (lane % LPR) ^ swz_k<D>(r);
        krow[jj] = r;
        kvo[jj] = (uint32_t)((lane / LPR) * D * 2 + c * 16);      // within the instruction's rows
    }
#pragma unroll
    for (int jj = 0; jj < VW; ++jj) {
        const int f = 16 * (w * VW + jj) + (lane >> 2);
        const int c = (lane & 3) ^ swz_v(f);
        vkr[jj] = 8 * c;
        vvo[jj] = (uint32_t)(f * T * 2 + c * 16);
    }
    // Frame geometry of a full subtile (T >= 32): its keys lie in frame f0 from token t0 on
    // and, from key `split` (a multiple of 8) on, in frame f0 + 1.  Wave-uniform scalars.
    struct Geo {
        uint32_t kb0, kb1, vb0, vb1;
        int split;
    };
    auto geo_of = [&](int k0) -> Geo {
        const int f0 = fast_div(k0, magicT, T);
        const int t0 = k0 - f0 * T;
        const int split = T - t0;
        const int s0 = slot_of(f0), s1 = slot_of(f0 + 1);
        return Geo{(uint32_t)((s0 * T + t0) * D * 2), (uint32_t)((s1 * T - split) * D * 2),
                   (uint32_t)(s0 * D * T * 2 + t0 * 2), (uint32_t)(s1 * D * T * 2 - split * 2), split};
    };
    auto dma_full_k = [&](const Geo &ge, int st) {
#pragma unroll
        for (int jj = 0; jj < KW; ++jj) {
            const int j = w * KW + jj;
            const uint32_t so = (RPI * j < ge.split ? ge.kb0 : ge.kb1) + (uint32_t)(RPI * j * D * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (LdsPtr)(kst + st * KBYTES + j * 1024), 16, (int)kvo[jj], (int)so, 0, 0);
        }
    };
    auto dma_full_v = [&](const Geo &ge, int st) {
        if (ge.split >= kSub) {
#pragma unroll
            for (int jj = 0; jj < VW; ++jj)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LdsPtr)(vst + st * VBYTES + (w * VW + jj) * 1024), 16, (int)vvo[jj],
                                                         (int)ge.vb0, 0, 0);
        } else {
#pragma unroll
            for (int jj = 0; jj < VW; ++jj)
                dma16(rv, vst + st * VBYTES + (w * VW + jj) * 1024, (vkr[jj] < ge.split ? ge.vb0 : ge.vb1) + vvo[jj]);
        }
    };
    // General plan (short subtiles, any T): rows past the valid keys re-read the last one.
    auto dma_any = [&](int k0, int st) {
        const int nv = nval_of(k0);
#pragma unroll
        for (int jj = 0; jj < KW; ++jj) {
            const int j = k0 + min(krow[jj], nv - 1);
            const int f = fast_div(j, magicT, T);
            const uint32_t off = (uint32_t)((slot_of(f) * T + (j - f * T)) * D * 2) + (kvo[jj] - (uint32_t)((lane / LPR) * D * 2));
            dma16(rk, kst + st * KBYTES + (w * KW + jj) * 1024, off);
        }
#pragma unroll
        for (int jj = 0; jj < VW; ++jj) {
            const int j = k0 + min(vkr[jj], (nv - 1) & ~7);
            const int f = fast_div(j, magicT, T);
            const uint32_t off = (uint32_t)(slot_of(f) * D * T * 2 + (j - f * T) * 2) + (vvo[jj] - (uint32_t)(vkr[jj] * 2));
            dma16(rv, vst + st * VBYTES + (w * VW + jj) * 1024, off);
        }
    };

    // ---- per-lane operand reads (swizzled chunk positions)
    const int rk_row = perm32(n);
    const int rk_swz = swz_k<D>(rk_row);
    // per-lane byte offsets of the operand fragments within a stage (stage offsets are
    // added as instruction immediates where the stage is known at compile time)
    uint32_t koff[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) koff[ks] = (uint32_t)(rk_row * D * 2 + (((2 * ks + g) ^ rk_swz) << 4));
    uint32_t voff[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) voff[ks] = (uint32_t)(rk_row * 64 + (((2 * g + ks) ^ swz_v(rk_row)) << 4));
    auto qk_from = [&](const unsigned char *kb) -> f32x16 {
        u32x4 kfr[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) kfr[ks] = *reinterpret_cast<const u32x4 *>(kb + koff[ks]);
        f32x16 s = {};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) s = mfma32(as_bf16x8(kfr[ks]), as_bf16x8(qf[ks]), s);
        return s;
    };
    f32x16 acc[D / 32];
#pragma unroll
    for (int ft = 0; ft < D / 32; ++ft) acc[ft] = f32x16{};
    auto pv_from = [&](const unsigned char *vb, const u32x4 (&pf)[2]) {
        u32x4 vfr[D / 32][2];
#pragma unroll
        for (int ft = 0; ft < D / 32; ++ft)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                vfr[ft][ks] = *reinterpret_cast<const u32x4 *>(vb + ft * 2048 + voff[ks]);
#pragma unroll
        for (int ft = 0; ft < D / 32; ++ft)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) acc[ft] = mfma32(as_bf16x8(vfr[ft][ks]), as_bf16x8(pf[ks]), acc[ft]);
    };
    // Rotated scores of the nk keys from window key k0 on (keys past nk are masked later).
    // The spatial fragments do not depend on the frame.  The temporal products run once
    // per frame of the subtile (more than one only where a frame boundary falls inside it)
    // into the same accumulator, each with the K fragments of the other frames' keys
    // zeroed: this lane supplies the A row of key k0 + perm32(n).
    auto qk_rope = [&](const unsigned char *kb, int k0, int nk) __attribute__((always_inline)) -> f32x16 {
        const int fa = fast_div(k0, magicT, T), fb = fast_div(k0 + nk - 1, magicT, T);
        const int myf = fast_div(k0 + rk_row, magicT, T);
        const u32x4 zero = {0u, 0u, 0u, 0u};
        set_qt(fa);
        u32x4 kfr[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) kfr[ks] = *reinterpret_cast<const u32x4 *>(kb + koff[ks]);
        f32x16 s = {};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            if (ks < KT) s = mfma32(as_bf16x8(myf == fa ? kfr[ks] : zero), as_bf16x8(qt[ks < KT ? ks : 0]), s);
            else s = mfma32(as_bf16x8(kfr[ks]), as_bf16x8(qf[ks]), s);
        }
        for (int f = fa + 1; f <= fb; ++f) {     // K fragments read again: nothing stays live
            set_qt(f);
#pragma unroll
            for (int ks = 0; ks < KT; ++ks) {
                const u32x4 kk = *reinterpret_cast<const u32x4 *>(kb + koff[ks]);
                s = mfma32(as_bf16x8(myf == f ? kk : zero), as_bf16x8(qt[ks]), s);
            }
        }
        return s;
    };
    auto qk_tile = [&](int st) -> f32x16 { return qk_from(kst + st * KBYTES); };
    auto pv_tile = [&](int st, const u32x4 (&pf)[2]) { pv_from(vst + st * VBYTES, pf); };
    auto rescale = [&](float alpha) {
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
            for (int ft = 0; ft < D / 32; ++ft)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[ft][i] *= alpha;
        }
    };
    // wait for this wave's loads, then for the other wave's (and for both to be done with
    // the stage about to be refilled)
    auto stage_ready = [&]() {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();
    };

    SmState sm{-INFINITY, 0.f};
    int ustart = 0;            // first subtile of the online loop
    if (nfull > 0) {
        // ---- fast path over the full subtiles, software-pipelined: step u computes
        // S_{u+1} = K_{u+1} Q^T while the softmax of S_u runs, then O += V_u P_u.  K runs one
        // subtile ahead of V, so K_{u+2} and V_{u+1} are fetched during step u into the K / V
        // stages that step u-1 finished with (the barrier closing each step orders this).
        // Past the last subtile the fetches repeat it and the extra product is discarded.
        const int last = nfull - 1;
        const Geo g0 = geo_of(key0_of(0));
        Geo g1 = geo_of(key0_of(min(1, last)));
        dma_full_k(g0, 0);
        dma_full_v(g0, 0);
        dma_full_k(g1, 1);
        stage_ready();
        f32x16 s_a, s_b;
        if constexpr (ROPE) s_a = qk_rope(kst, key0_of(0), kSub);
        else s_a = qk_tile(0);
        sm.m = tile_max_log2(s_a, c_log2);
        const float moff = -sm.m;
        __syncthreads();            // K stage 0 is refilled in step 0
        // one step with stage parity P (compile-time): S_u in s_cur, S_{u+1} -> s_nxt
        auto step = [&](int u, auto par, const f32x16 &s_cur, f32x16 &s_nxt) {
            constexpr int P = decltype(par)::value;
            const Geo g2 = geo_of(key0_of(min(u + 2, last)));
            dma_full_k(g2, P);
            dma_full_v(g1, 1 - P);
            g1 = g2;
            if constexpr (ROPE) s_nxt = qk_rope(kst + (1 - P) * KBYTES, key0_of(min(u + 1, last)), kSub);
            else s_nxt = qk_from(kst + (1 - P) * KBYTES);
            u32x4 pf[2];
            softmax_fixed(s_cur, c_log2, moff, sm.l, pf);
            pv_from(vst + P * VBYTES, pf);
            stage_ready();
        };
        int u = 0;
        for (; u + 1 < nfull; u += 2) {
            step(u, std::integral_constant<int, 0>{}, s_a, s_b);
            step(u + 1, std::integral_constant<int, 1>{}, s_b, s_a);
        }
        if (u < nfull) step(u, std::integral_constant<int, 0>{}, s_a, s_b);
        // a score far above its reference (row sum >= 2^32): recompute the block online
        const int bad = __builtin_amdgcn_ballot_w64(!(sm.l < kFixedRefLimit)) != 0;
        if (lane == 0) s_flag[w] = bad;
        __syncthreads();
        int any_bad = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) any_bad |= s_flag[i];
        if (any_bad) {
            sm = SmState{-INFINITY, 0.f};
#pragma unroll
            for (int ft = 0; ft < D / 32; ++ft) acc[ft] = f32x16{};
            ustart = 0;
        } else {
            ustart = nfull;
        }
    }

    // ---- online path: short subtiles, or every subtile after a fallback
    if (ustart < nsubt) {
        dma_any(key0_of(ustart), ustart & 1);
        for (int u = ustart; u < nsubt; ++u) {
            stage_ready();
            if (u + 1 < nsubt) dma_any(key0_of(u + 1), (u + 1) & 1);
            const int k0 = key0_of(u);
            const int nv = nval_of(k0);
            f32x16 s;
            if constexpr (ROPE) s = qk_rope(kst + (u & 1) * KBYTES, k0, nv);
            else s = qk_tile(u & 1);
            u32x4 pf[2];
            const float al = softmax_online(s, nv, g, c_log2, sm, pf);
            rescale(al);
            pv_tile(u & 1, pf);
        }
    }

    // ---- epilogue: normalise, add the linear readout, store fp32
    const float lsum = pair_sum(sm.l);
    const float inv_l = 1.f / lsum;
#pragma unroll
    for (int ft = 0; ft < D / 32; ++ft)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[ft][i] *= inv_l;
    if (a.st) {
        // B operand phi(q) / (phi(q) . z + eps) in the Q^T fragment layout, so that the
        // readout accumulates straight onto the normalised sparse output
        const float *zp = a.zc + (size_t)bh * D + 8 * g;
        float den = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const uint32_t wv[4] = {qf[ks].x, qf[ks].y, qf[ks].z, qf[ks].w};
            const f32x4 z0 = *reinterpret_cast<const f32x4 *>(zp + 16 * ks);
            const f32x4 z1 = *reinterpret_cast<const f32x4 *>(zp + 16 * ks + 4);
            const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                den = __builtin_fmaf(phi_f32(bf16_lo_to_f32(wv[e])), zz[2 * e], den);
                den = __builtin_fmaf(phi_f32(bf16_hi_to_f32(wv[e])), zz[2 * e + 1], den);
            }
        }
        const float inv_den = 1.f / (pair_sum(den) + a.eps);
        u32x4 pq[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const uint32_t wv[4] = {qf[ks].x, qf[ks].y, qf[ks].z, qf[ks].w};
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                o[e] = pack_bf16x2(phi_f32(bf16_lo_to_f32(wv[e])) * inv_den, phi_f32(bf16_hi_to_f32(wv[e])) * inv_den);
            pq[ks] = u32x4{o[0], o[1], o[2], o[3]};
        }
        const uint16_t *stp = a.st + (size_t)bh * D * D + 8 * g;
#pragma unroll
        for (int ft = 0; ft < D / 32; ++ft) {
            const uint16_t *srow = stp + (size_t)(32 * ft + perm32(n)) * D;
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks)
                acc[ft] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(srow + 16 * ks)), as_bf16x8(pq[ks]), acc[ft]);
        }
    }
    const int row = q0 + 32 * w + n;
    if (a.lse && g == 0 && row < qend) a.lse[(size_t)bh * a.Nq + row] = sm.m + __log2f(lsum);
    if (row < qend) {
        float *op = a.out + ((size_t)bh * a.Nq + row) * D + 16 * g;
#pragma unroll
        for (int ft = 0; ft < D / 32; ++ft) {
            f32x4 *o4 = reinterpret_cast<f32x4 *>(op + 32 * ft);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                o4[v] = f32x4{acc[ft][4 * v], acc[ft][4 * v + 1], acc[ft][4 * v + 2], acc[ft][4 * v + 3]};
        }
    }
}

}  // namespace
}  // namespace hf

hipError_t hf_launch_sparse_attn(const hf_attn_args &a, hipStream_t s) {
    const int items = a.BH * a.nqb;
    const int per_xcd = (items + 7) / 8;
    const dim3 grid((unsigned)(per_xcd * 8));
    const uint32_t magicT = hf::div_magic((uint32_t)a.T);
    const float c_log2 = (float)(1.4426950408889634 / sqrt((double)a.D));
    const int lsh = a.bk >= 128 ? 2 : (a.bk >= 64 ? 1 : 0);     // 32-key subtiles per key block = 2^lsh
    const int nw = a.bq > 32 ? 2 : 1;
    const size_t dyn = 2 * (size_t)128 * a.D + (size_t)a.top_k * sizeof(int32_t) + nw * sizeof(int);   // 2 K + 2 V stages
    auto go = [&](auto kern, int threads) {
        hipLaunchKernelGGL(kern, grid, dim3(threads), dyn, s, a, magicT, c_log2, per_xcd, lsh);
    };
    // one instance per (D, waves, temporal fragments of the rotation)
    auto pick = [&](auto dc, auto nwc) {
        constexpr int Dc = decltype(dc)::value, NWc = decltype(nwc)::value;
        switch (a.rope_dt / 16) {
        case 1: go(hf::sparse_attn_kernel<Dc, NWc, 1>, 64 * NWc); break;
        case 2: go(hf::sparse_attn_kernel<Dc, NWc, 2>, 64 * NWc); break;
        default: go(hf::sparse_attn_kernel<Dc, NWc, 0>, 64 * NWc); break;
        }
    };
    using I64 = std::integral_constant<int, 64>;
    using I128 = std::integral_constant<int, 128>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if (a.D == 64) nw == 2 ? pick(I64{}, I2{}) : pick(I64{}, I1{});
    else nw == 2 ? pick(I128{}, I2{}) : pick(I128{}, I1{});
    return hipGetLastError();
}
