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
//   * The kept key blocks are walked in 32-key subtiles.  Each subtile's K rows and its four
//     8-key V groups (the ring keeps values as [8-token group][D][8]) are fetched with
//     direct-to-LDS buffer loads (16 bytes per lane, 1 KB of contiguous whole cache lines per
//     instruction) into a double-buffered LDS stage, one subtile ahead of the compute; the
//     two waves share the fetch.  16-byte chunk positions are XOR-swizzled, so that the
//     reads in matrix-core operand order hit distinct LDS banks.
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
#include <algorithm>
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

// LDS swizzles (16-byte chunks) of the operand reads below.  K rows hold D/8 chunks,
// permuted per row, so that the 16 lanes of a read touch 16 distinct bank groups.  A V
// group holds D 16-byte feature rows; feature f sits at position vslot(f), which flips bits
// 2 and 3 where bit 4 is set (an involution that leaves bits 4 and up alone).  The lanes of
// a read take features perm32(0 .. 31) = {0-3, 16-19, 4-7, 20-23, 8-11, 24-27, 12-15, 28-31}
// (+ 32 ft) of group ks and, lanes 32-63, of group 2 + ks.  Counted with SQ_LDS_BANK_CONFLICT
// on gfx950 for these exact 64-lane patterns: no conflict cycles, where flipping bit 3 alone
// cost one extra pass per read (2-way).
template <int D>
__device__ __forceinline__ int swz_k(int r) {
    if constexpr (D == 128) return ((r & 3) << 1) | ((r >> 2) & 1) | ((r >> 1) & 8);
    else return ((r >> 1) & 3) | ((r >> 2) & 4);
}
__device__ __forceinline__ int vslot(int f) { return f ^ (((f >> 4) & 1) * 12); }

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

// ------------------------------------------------------------------ absorb role
// In a committed step, extra workgroups at the front of the attention launch absorb the
// evicted tokens -- the ab_E oldest keys of the window, still in their ring slots -- into
// split partial sums of the linear state, which grows by every token that leaves the
// window ([HF-abs]; [HF-de] §2.A "Lineare Zeit-Aufmerksamkeit"; [HF-pt] §2.A.1):
//     S[a][c] += sum_u phi(K_u[a]) V_u[c],      z[a] += sum_u phi(K_u[a]).
// The attention's readout reads a copy of the state made before the launch, so the two
// roles never touch the same data, and the absorb runs beside the attention instead of
// after it; the state pass that follows the launch adds the partials in split order.
//   * Work item = (plane, split of the token range[, 64-row half of S when one wave cannot
//     hold all rows]).  Each wave owns 64 rows of S (32 for D = 64 with two waves) and all
//     D columns, and the workgroup walks its split in 16-token steps.
//   * The steps stream through a ring of kAbStages LDS stages with direct-to-LDS loads,
//     kAbStages - 1 steps ahead (counted waits, one LDS-only barrier per step): K rows (the
//     item's features of each token) and the two 8-token V groups.  gfx950's
//     transposing LDS read (within each 16-lane group, lane i receives element i % 4 of the
//     4-element vectors lanes i / 4 + 4 e point at) turns the K rows into the phi(K)^T
//     operand (8 tokens of one feature per lane); phi is evaluated in fp32 and split into
//     bf16 hi + lo halves, so with V exact in bf16 the two products per fragment keep
//     fp32-grade accuracy.
//   * Each wave writes its rows' partial (and z) straight from its accumulators into the
//     split's slot of the workspace: no atomics, the result is deterministic.

constexpr int kAbStages = 4;                 // LDS stages (steps in flight + 1)

template <int D, int NW>
struct AbShape {
    static constexpr int R = (D / NW < 64) ? D / NW : 64;   // rows of S per wave
    static constexpr int RTW = R / 32;                       // 32-row tiles per wave
    static constexpr int CT = D / 32;                        // 32-column tiles
    static constexpr int ROWS = R * NW;                      // rows (features) per item
    static constexpr int GROUPS = D / ROWS;                  // items per (plane, split)
    static constexpr int RW = ROWS * 2;                      // bytes per staged K row
    static constexpr int RC = RW / 16;                       // 16-byte chunks per K row
    static constexpr int KB = 16 * RW;                       // K stage bytes (16 tokens)
    static constexpr int SB = KB + D * 32;                   // stage bytes (+ V: two 8-token groups)
    static constexpr int KI = KB / 1024, VI = D * 32 / 1024; // load instructions per step
    static constexpr int PW = (KI + VI) / NW;                // ... per wave
};

// K stage swizzle: 16-byte chunk c of token row r sits at slot c ^ ((RC / 4) (r % 4)), so the
// four rows a transposing read touches hit distinct bank groups.
template <int RC>
__device__ __forceinline__ int ab_kswz(int r) { return (RC / 4) * (r & 3); }

// LDS reads of one absorb step, in one asm block that also waits for them: per 32-row tile
// two transposing reads of K (token rows 0-3 and 4-7 from the lane's base, 4 RW bytes
// apart) and CT 16-byte V fragments (512 bytes apart).  Written out so that the compiler, which
// cannot tell which direct-to-LDS load an LDS read depends on, adds no wait for every load
// in flight: the caller's counted wait covers the step's loads.  Every output is complete
// when the block ends.
template <int RTW, int CT, int RW>
__device__ __forceinline__ void ab_lds_reads(const uint32_t (&ka)[RTW], uint32_t va, u32x2 (&r)[RTW][2],
                                             u32x4 (&vf)[CT]) {
    if constexpr (RTW == 2 && CT == 4) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8\n\t"
            "ds_read_b64_tr_b16 %1, %8 offset:%11\n\t"
            "ds_read_b64_tr_b16 %2, %9\n\t"
            "ds_read_b64_tr_b16 %3, %9 offset:%11\n\t"
            "ds_read_b128 %4, %10\n\t"
            "ds_read_b128 %5, %10 offset:512\n\t"
            "ds_read_b128 %6, %10 offset:1024\n\t"
            "ds_read_b128 %7, %10 offset:1536\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(vf[0]), "=&v"(vf[1]),
              "=&v"(vf[2]), "=&v"(vf[3])
            : "v"(ka[0]), "v"(ka[1]), "v"(va), "i"(4 * RW)
            : "memory");
    } else if constexpr (RTW == 2 && CT == 2) {
        asm volatile(
            "ds_read_b64_tr_b16 %0, %6\n\t"
            "ds_read_b64_tr_b16 %1, %6 offset:%9\n\t"
            "ds_read_b64_tr_b16 %2, %7\n\t"
            "ds_read_b64_tr_b16 %3, %7 offset:%9\n\t"
            "ds_read_b128 %4, %8\n\t"
            "ds_read_b128 %5, %8 offset:512\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(vf[0]), "=&v"(vf[1])
            : "v"(ka[0]), "v"(ka[1]), "v"(va), "i"(4 * RW)
            : "memory");
    } else {
        static_assert(RTW == 1 && CT == 2, "absorb tile shape");
        asm volatile(
            "ds_read_b64_tr_b16 %0, %4\n\t"
            "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
            "ds_read_b128 %2, %5\n\t"
            "ds_read_b128 %3, %5 offset:512\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(vf[0]), "=&v"(vf[1])
            : "v"(ka[0]), "v"(va), "i"(4 * RW)
            : "memory");
    }
}

__device__ __forceinline__ uint32_t lds_addr(const unsigned char *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char *)p;
}

template <int D, int NW>
__device__ __forceinline__ void absorb_role(const hf_attn_args &a, int ab, unsigned char *lds, uint32_t magicT) {
    using A = AbShape<D, NW>;
    constexpr int RTW = A::RTW, CT = A::CT, RW = A::RW, RC = A::RC, SB = A::SB;
    const int P = a.ab_P;
    const int grp = ab % A::GROUPS, p = (ab / A::GROUPS) % P, bh = ab / (A::GROUPS * P);
    const int E = a.ab_E, nsteps = (E + 15) >> 4;
    const int s0 = (int)((int64_t)p * nsteps / P), s1 = (int)((int64_t)(p + 1) * nsteps / P);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, n = lane & 31, g = lane >> 5;
    const int T = a.T, W = a.W, head = a.head;
    const int F0 = grp * A::ROWS;            // the item's first feature (row of S)
    const size_t plane = (size_t)bh * W * T * D;
    const uint32_t plane_bytes = (uint32_t)((size_t)W * T * D * 2);
    const Rsrc rk = make_rsrc(a.ring_k + plane, plane_bytes);
    const Rsrc rv = make_rsrc(a.ring_vg + plane, plane_bytes);
    auto slot_of = [&](int f) -> int {
        const int s = head + f;
        return s >= W ? s - W : s;
    };
    // Step h (tokens 16 h ..) into stage st; h is clamped to the split's last step (loads of
    // padding steps are never consumed).  Instruction j of the step is issued by wave j % NW.
    //   K, j < KI: lane -> token row (64 j + lane) / RC, slot (64 j + lane) % RC holding chunk
    //     slot ^ ab_kswz(row) of the item's features.
    //   V, j >= KI: 1 KB of the step's two 8-token groups as they lie in the ring ([group]
    //     [D][8]; a group is 8 tokens of one frame: T and E are multiples of 8).
    // Tokens at or past E re-read the last ones (finite data; their phi is masked to 0).
    auto fetch = [&](int h, int st) {
        h = min(h, s1 - 1);
        unsigned char *kd = lds + st * SB, *vd = kd + A::KB;
        const int kb = 16 * h;
#pragma unroll
        for (int jj = 0; jj < A::PW; ++jj) {
            const int j = w + NW * jj;
            if (j < A::KI) {
                const int e = 64 * j + lane, r = e / RC, c = (e % RC) ^ ab_kswz<RC>(r);
                const int t = min(kb + r, E - 1);
                const int ft = fast_div(t, magicT, T);
                dma16(rk, kd + j * 1024, (uint32_t)(((slot_of(ft) * T + (t - ft * T)) * D + F0 + 8 * c) * 2));
            } else {
                constexpr int VIG = D / 64;       // instructions per group
                const int jv = j - A::KI;
                const int t8 = min(kb + 8 * (jv / VIG), E - 8);
                const int f8 = fast_div(t8, magicT, T);
                dma16(rv, vd + jv * 1024, (uint32_t)((slot_of(f8) * T + (t8 - f8 * T)) * D * 2 + (jv % VIG) * 1024 + lane * 16));
            }
        }
    };

    // Per 32-row tile of the wave: transposing-read address in a K stage -- token row s16 / 4
    // (+ the 8-token base of the lane half), features 16 Gh + 4 (s16 % 4) .. + 3 of the tile,
    // so lane i of 16-lane group Gh receives feature 16 Gh + i of four consecutive tokens.
    // V fragment of column tile ct: group g, feature row 32 ct + n.
    const int s16 = lane & 15, Gh = (lane >> 4) & 1;
    int kro[RTW];
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
        const int r = 8 * g + (s16 >> 2);
        const int fo = w * A::R + 32 * t + 16 * Gh + 4 * (s16 & 3);   // feature within the item
        kro[t] = r * RW + (((fo >> 3) ^ ab_kswz<RC>(r)) << 4) + (fo & 7) * 2;
    }
    const int vro = A::KB + g * D * 16 + n * 16;
    f32x16 acc[RTW][CT];
#pragma unroll
    for (int t = 0; t < RTW; ++t)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[t][ct] = f32x16{};
    float zs[RTW];
#pragma unroll
    for (int t = 0; t < RTW; ++t) zs[t] = 0.f;

#pragma unroll
    for (int i = 0; i < kAbStages - 1; ++i) fetch(s0 + i, i);
    for (int h = s0; h < s1; ++h) {
        const int st = (h - s0) % kAbStages;
        wait_vm<A::PW * (kAbStages - 2)>();       // this wave's loads of step h have landed
        lds_barrier();                            // every wave's; step h - 1's stage is free
        fetch(h + kAbStages - 1, (h - s0 + kAbStages - 1) % kAbStages);
        const unsigned char *sb = lds + st * SB;
        uint32_t ka[RTW];
#pragma unroll
        for (int t = 0; t < RTW; ++t) ka[t] = lds_addr(sb + kro[t]);
        u32x2 r[RTW][2];
        u32x4 vf[CT];
        ab_lds_reads<RTW, CT, RW>(ka, lds_addr(sb + vro), r, vf);
        const int nv = E - 16 * h - 8 * g;        // tokens of the lane's 8 that are absorbed
#pragma unroll
        for (int t = 0; t < RTW; ++t) {
            const uint32_t raw[4] = {r[t][0].x, r[t][0].y, r[t][1].x, r[t][1].y};
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float f0 = phi_f32(bf16_lo_to_f32(raw[e])), f1 = phi_f32(bf16_hi_to_f32(raw[e]));
                f0 = 2 * e < nv ? f0 : 0.f;
                f1 = 2 * e + 1 < nv ? f1 : 0.f;
                zs[t] += f0;
                zs[t] += f1;
                hi[e] = pack_bf16x2(f0, f1);
                lo[e] = pack_bf16x2(f0 - bf16_lo_to_f32(hi[e]), f1 - bf16_hi_to_f32(hi[e]));
            }
            const bf16x8 ah = as_bf16x8(u32x4{hi[0], hi[1], hi[2], hi[3]});
            const bf16x8 al = as_bf16x8(u32x4{lo[0], lo[1], lo[2], lo[3]});
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                acc[t][ct] = mfma32(ah, as_bf16x8(vf[ct]), acc[t][ct]);
                acc[t][ct] = mfma32(al, as_bf16x8(vf[ct]), acc[t][ct]);
            }
        }
    }
    wait_vm<0>();     // the padding steps' loads land before the workgroup releases its LDS

    // partials in the state pass's layout: 64-row block rb of plane bh, split p at slot
    // (bh (D / 64) + rb) P + p, 64 x D floats; z partials after all of them
    const size_t items = (size_t)a.BH * (D / 64) * P;
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
        const int rbase = F0 + w * A::R + 32 * t;      // the tile's first row (feature)
        const size_t slot = ((size_t)bh * (D / 64) + rbase / 64) * P + p;
        float *part = a.ab_part + slot * 64 * D + (size_t)(rbase % 64) * D;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 16; ++i) part[(size_t)(8 * (i >> 2) + 4 * g + (i & 3)) * D + 32 * ct + n] = acc[t][ct][i];
        const float zt = pair_sum(zs[t]);
        if (g == 0) a.ab_part[items * 64 * D + slot * 64 + rbase % 64 + n] = zt;
    }
}

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

    // dynamic LDS: [K stage 0][K stage 1][V stage 0][V stage 1][V stage 2] (40 KB at D = 128,
    // so that four workgroups share a CU's 160 KB)
    extern __shared__ __align__(16) unsigned char dyn[];
    // the absorb role's workgroups come first (a multiple of 8 of them, so that the
    // attention's workgroup-to-XCD remap below is unchanged)
    if ((int)blockIdx.x < a.ab_nab) {
        if ((int)blockIdx.x < a.ab_items) absorb_role<D, NW>(a, blockIdx.x, dyn, magicT);
        return;
    }
    const int bid = (int)blockIdx.x - a.ab_nab;
    const int item = (bid & 7) * per_xcd + (bid >> 3);
    if (item >= a.BH * a.nqb) return;   // uniform per workgroup
    const int bh = item / a.nqb, qb = item - bh * a.nqb;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, n = lane & 31, g = lane >> 5;
    const int q0 = qb * a.bq, qend = min(q0 + a.bq, a.Nq);
    unsigned char *const kst = dyn, *const vst = dyn + 2 * KBYTES;   // 2 K stages, 3 V stages

    // kept blocks -> LDS (out-of-range entries, a caller error, are clamped so that no load
    // leaves the window)
    typedef const __attribute__((address_space(4))) int32_t *KeptPtr;
    const KeptPtr sel = (KeptPtr)(a.idx + ((size_t)bh * a.nqb + qb) * a.top_k);
    auto kept = [&](int t) -> int { return min(max(sel[t], 0), a.nkb - 1); };

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
    const Rsrc rv = make_rsrc(a.ring_vg + plane, plane_bytes);
    const int T = a.T, W = a.W, head = a.head;

    // ---- subtile list: 2^lsh subtiles per kept block, minus the empty tail of a short last
    // block (the list is ascending, so that block can only be the final entry)
    const int nsub_blk = 1 << lsh;
    int nsubt = a.top_k << lsh;
    int nfull = (a.bk >= kSub && T >= kSub) ? nsubt : 0;
    {
        const int lastb = kept(a.top_k - 1);
        if (lastb == a.nkb - 1 && a.bk >= kSub) {
            const int len = a.Nk - lastb * a.bk;
            nsubt -= nsub_blk - (len + kSub - 1) / kSub;
            if (nfull) nfull = nsubt - ((len & (kSub - 1)) ? 1 : 0);
        }
    }
    auto key0_of = [&](int u) -> int {
        const int b = kept(u >> lsh);
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
    // The K stage is row-major with chunk positions swizzled per row (K row r = key r of the
    // subtile, D/8 chunks); one instruction fetches RPI whole K rows.  The V stage holds the
    // subtile's four 8-key groups as they lie in the ring ([group][D][8], 16 D bytes each,
    // the 16-byte row of feature f at position vslot(f)); one instruction fetches 1 KB of a
    // group, whole cache lines.  In the ring the rows of key j and the group of keys j .. j+7
    // (j a multiple of 8) both start at byte (slot T + t) D 2, t = j's token in its frame.
    // Subtiles start at multiples of 32 keys and T is a multiple of 8, so a frame boundary
    // inside a subtile falls on a multiple of 8 keys, never inside an instruction's rows or
    // group: every frame choice is a scalar offset.
    constexpr int VIG = D / 64;           // V instructions per 8-key group
    uint32_t kvo[KW];
    int krow[KW];
#pragma unroll
    for (int jj = 0; jj < KW; ++jj) {
        const int j = w * KW + jj;
        const int r = RPI * j + lane / LPR;
        const int c = (lane % LPR) ^ swz_k<D>(r);
        krow[jj] = r;
        kvo[jj] = (uint32_t)((lane / LPR) * D * 2 + c * 16);      // within the instruction's rows
    }
    // LDS position 64 h + lane of a group holds feature vslot(64 h + lane) (an involution
    // that leaves bits 5 and up alone)
    const uint32_t vlo = (uint32_t)(vslot(lane) * 16);
    // Frame geometry of a full subtile (T >= 32): its keys lie in frame f0 from token t0 on
    // and, from key `split` (a multiple of 8) on, in frame f0 + 1.  Wave-uniform scalars:
    // kb0 + 2 D i is the byte offset of the subtile's key i (and of its group) if i < split,
    // kb1 + 2 D i otherwise.
    struct Geo {
        uint32_t kb0, kb1;
        int split;
    };
    auto geo_of = [&](int k0) -> Geo {
        const int f0 = fast_div(k0, magicT, T);
        const int t0 = k0 - f0 * T;
        const int split = T - t0;
        const int s0 = slot_of(f0), s1 = slot_of(f0 + 1);
        return Geo{(uint32_t)((s0 * T + t0) * D * 2), (uint32_t)((s1 * T - split) * D * 2), split};
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
#pragma unroll
        for (int jj = 0; jj < VW; ++jj) {
            const int j = w * VW + jj;
            const uint32_t so = (8 * (j / VIG) < ge.split ? ge.kb0 : ge.kb1) + (uint32_t)(j * 1024);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (LdsPtr)(vst + st * VBYTES + j * 1024), 16, (int)vlo, (int)so, 0, 0);
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
            const int jv = w * VW + jj;
            const int j = k0 + min(8 * (jv / VIG), (nv - 1) & ~7);
            const int f = fast_div(j, magicT, T);
            const uint32_t off = (uint32_t)((slot_of(f) * T + (j - f * T)) * D * 2 + (jv % VIG) * 1024) + vlo;
            dma16(rv, vst + st * VBYTES + jv * 1024, off);
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
    // V fragment of product ks: the lane's 8 keys are group 2 g + ks (the key order the
    // probabilities leave the QK product in), feature row 32 ft + rk_row
    uint32_t voff[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) voff[ks] = (uint32_t)((2 * g + ks) * D * 16 + vslot(rk_row) * 16);
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
                vfr[ft][ks] = *reinterpret_cast<const u32x4 *>(vb + ft * 512 + voff[ks]);
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
        // S_{u+1} = K_{u+1} Q^T while the softmax of S_u runs, then O += V_u P_u.  K streams
        // through two stages and V through three, so K_{u+2} and V_{u+2} are fetched during
        // step u into the stages that step u-1 finished with (the barrier closing each step
        // orders this): every K fetch has a step to land, every V fetch two.
        // Past the last subtile the fetches repeat it and the extra product is discarded.
        const int last = nfull - 1;
        const Geo g0 = geo_of(key0_of(0));
        const Geo g1 = geo_of(key0_of(min(1, last)));
        dma_full_k(g0, 0);
        dma_full_v(g0, 0);
        dma_full_k(g1, 1);
        dma_full_v(g1, 1);
        wait_vm<0>();
        lds_barrier();
        f32x16 s_a, s_b;
        if constexpr (ROPE) s_a = qk_rope(kst, key0_of(0), kSub);
        else s_a = qk_tile(0);
        sm.m = tile_max_log2(s_a, c_log2);
        const float moff = -sm.m;
        lds_barrier();              // K stage 0 is refilled in step 0
        // step u: fetch K_{u+2} into K stage u % 2, then V_{u+2} into V stage (u+2) % 3 (V_{u-1}'s);
        // QK of u+1 from K stage (u+1) % 2, softmax of u, PV of u from V stage u % 3; close by
        // waiting for all but the V_{u+2} loads
        // step u with K parity KP = u % 2 (compile-time) and V stages vp = u % 3, vf =
        // (u + 2) % 3: compile-time too (loop unrolled by six) where the registers allow
        // it, else wave-uniform runtime values (unrolled by two)
        auto step = [&](int u, auto kp, auto vpc, auto vfc, const f32x16 &s_cur, f32x16 &s_nxt) {
            constexpr int KP = decltype(kp)::value;
            const int vp = vpc, vf = vfc;
            const Geo g2 = geo_of(key0_of(min(u + 2, last)));
            dma_full_k(g2, KP);
            dma_full_v(g2, vf);
            if constexpr (ROPE) s_nxt = qk_rope(kst + (1 - KP) * KBYTES, key0_of(min(u + 1, last)), kSub);
            else s_nxt = qk_from(kst + (1 - KP) * KBYTES);
            u32x4 pf[2];
            softmax_fixed(s_cur, c_log2, moff, sm.l, pf);
            pv_from(vst + vp * VBYTES, pf);
            wait_vm<VW>();
            lds_barrier();
        };
        using C0 = std::integral_constant<int, 0>;
        using C1 = std::integral_constant<int, 1>;
        using C2 = std::integral_constant<int, 2>;
        int u = 0;
        if constexpr (!ROPE && NW == 2) {
            for (; u + 5 < nfull; u += 6) {
                step(u, C0{}, C0{}, C2{}, s_a, s_b);
                step(u + 1, C1{}, C1{}, C0{}, s_b, s_a);
                step(u + 2, C0{}, C2{}, C1{}, s_a, s_b);
                step(u + 3, C1{}, C0{}, C2{}, s_b, s_a);
                step(u + 4, C0{}, C1{}, C0{}, s_a, s_b);
                step(u + 5, C1{}, C2{}, C1{}, s_b, s_a);
            }
            const int rem = nfull - u;
            if (rem > 0) step(u, C0{}, C0{}, C2{}, s_a, s_b);
            if (rem > 1) step(u + 1, C1{}, C1{}, C0{}, s_b, s_a);
            if (rem > 2) step(u + 2, C0{}, C2{}, C1{}, s_a, s_b);
            if (rem > 3) step(u + 3, C1{}, C0{}, C2{}, s_b, s_a);
            if (rem > 4) step(u + 4, C0{}, C1{}, C0{}, s_a, s_b);
        } else {
            auto next3 = [](int x) { return x == 2 ? 0 : x + 1; };
            int vp = 0, vf = 2;
            for (; u + 1 < nfull; u += 2) {
                step(u, C0{}, vp, vf, s_a, s_b);
                vp = next3(vp);
                vf = next3(vf);
                step(u + 1, C1{}, vp, vf, s_b, s_a);
                vp = next3(vp);
                vf = next3(vf);
            }
            if (u < nfull) step(u, C0{}, vp, vf, s_a, s_b);
        }
        wait_vm<0>();
        lds_barrier();
        // a score far above its reference (row sum >= 2^32): recompute the block online
        int *const s_flag = reinterpret_cast<int *>(vst + 2 * VBYTES);
        const int bad = __builtin_amdgcn_ballot_w64(!(sm.l < kFixedRefLimit)) != 0;
        if (lane == 0) s_flag[w] = bad;
        lds_barrier();
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
        // S^T (bf16, row r = output feature r) is staged once per workgroup in the LDS the
        // K/V stages used, its rows laid out and swizzled like K rows, while the readout's
        // B operand phi(q) / (phi(q) . z + eps) is formed in the Q^T fragment layout (the
        // readout then accumulates straight onto the normalised sparse output)
        lds_barrier();              // every wave is done with the stages
        {
            const Rsrc rs = make_rsrc(a.st + (size_t)bh * D * D, (uint32_t)(D * D * 2));
#pragma unroll
            for (int ft = 0; ft < D / 32; ++ft)
#pragma unroll
                for (int jj = 0; jj < KW; ++jj) {
                    const int j = w * KW + jj;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LdsPtr)(dyn + ft * KBYTES + j * 1024), 16, (int)kvo[jj],
                                                             (32 * ft + RPI * j) * D * 2, 0, 0);
                }
        }
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
        wait_vm<0>();
        lds_barrier();
#pragma unroll
        for (int ft = 0; ft < D / 32; ++ft) {
            // row 32 ft + perm32(n), features 16 ks + 8 g .. + 7 (the K-row read pattern)
            u32x4 sf[D / 16];
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) sf[ks] = *reinterpret_cast<const u32x4 *>(dyn + ft * KBYTES + koff[ks]);
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) acc[ft] = mfma32(as_bf16x8(sf[ks]), as_bf16x8(pq[ks]), acc[ft]);
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

hipError_t hf_launch_sparse_attn(const hf_attn_args &a_in, hipStream_t s) {
    hf_attn_args a = a_in;
    const int nw = a.bq > 32 ? 2 : 1;
    // absorb items: (plane, split[, 64-row half of S for one-wave workgroups at D = 128])
    a.ab_P = a.ab_E > 0 ? hf_step_absorb_splits(a.BH, a.D, a.ab_E) : 1;
    a.ab_items = a.ab_E > 0 ? a.BH * a.ab_P * ((a.D == 128 && nw == 1) ? 2 : 1) : 0;
    a.ab_nab = (a.ab_items + 7) & ~7;
    const int items = a.BH * a.nqb;
    const int per_xcd = (items + 7) / 8;
    const dim3 grid((unsigned)(a.ab_nab + per_xcd * 8));
    const uint32_t magicT = hf::div_magic((uint32_t)a.T);
    const float c_log2 = (float)(1.4426950408889634 / sqrt((double)a.D));
    const int lsh = a.bk >= 128 ? 2 : (a.bk >= 64 ? 1 : 0);     // 32-key subtiles per key block = 2^lsh
    const size_t dyn = 5 * (size_t)64 * a.D;     // 2 K stages + 3 V stages
    // a step's absorb role streams through kAbStages stages within the attention's LDS
    static_assert(hf::kAbStages * hf::AbShape<128, 2>::SB <= 2 * 128 * 128, "absorb LDS, D=128");
    static_assert(hf::kAbStages * hf::AbShape<128, 1>::SB <= 2 * 128 * 128, "absorb LDS, D=128, one wave");
    static_assert(hf::kAbStages * hf::AbShape<64, 2>::SB <= 2 * 128 * 64, "absorb LDS, D=64");
    static_assert(hf::kAbStages * hf::AbShape<64, 1>::SB <= 2 * 128 * 64, "absorb LDS, D=64, one wave");
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
