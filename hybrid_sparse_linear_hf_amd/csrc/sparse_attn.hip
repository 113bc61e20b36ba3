// Block-sparse window attention with the linear readout fused into its epilogue.
//
// Sparse branch ([HF-de] §2.A "Block-Sparse Sliding Window Attention", [HF-pt] §2.A.2):
// every query of query block i attends with softmax weights to the keys of its kept key
// blocks only.  Linear branch ([HF-de] §2.A "Lineare Zeit-Aufmerksamkeit", [HF-pt]
// §2.A.1, [HF-abs]): phi(q)^T S / (phi(q) . z + eps) from the compact state.  The output
// is their sum ([HF-de] §2.A "Kombination", [HF-pt] §2.A "Resultado").
//
// gfx950 design
//   * A workgroup of 4 waves owns two adjacent query blocks of one plane (two 32-query
//     tiles each).  Adjacent query blocks keep largely the same key blocks, so the
//     workgroup walks the UNION of their two kept lists and loads every 32-key K/V subtile
//     once for both: fewer bytes per matrix-core flop than one block per workgroup.
//   * Subtiles are staged cooperatively (coalesced 16-byte loads) through registers four
//     subtiles ahead, into a double-buffered LDS stage, with rows stored in the lane order
//     the matrix-core operands read them (conflict-free 16-byte LDS reads).
//   * Each wave computes S^T = K Q^T and O^T += V^T P^T on 32x32x16 bf16 matrix cores, so
//     the probabilities leave the first product already in the register layout the second
//     consumes.  Feeding key rows in the order perm32(m) makes each lane hold 16
//     consecutive keys of its query; value frames are stored transposed ([D][T]) in the
//     ring, so the V operand needs no transpose either.
//   * fp32 online softmax in base 2 with the 1/sqrt(D) scale folded into one FMA; the
//     running maximum is only raised when a tile exceeds it by more than 2^8, so the
//     accumulator rescale is rare.
//   * At most 256 registers per wave, so two workgroups share a CU and one wave's memory
//     waits overlap the other's matrix-core work.
//   * Workgroup ids are remapped so that the query blocks of one plane run on one XCD
//     and share its L2 for the window's K/V.
#include "hf_internal.h"

namespace hf {
namespace {

constexpr float kLazyRescaleLog2 = 8.0f;
constexpr int kSub = 32;          // keys per subtile

// Inverse of perm32: LDS row that holds logical row k.
__device__ __forceinline__ int inv_perm32(int k) { return (((k >> 2) & 3) << 3) | ((k >> 4) << 2) | (k & 3); }

template <int D>
struct Stage {
    uint16_t k[kSub][D + 8];      // row m holds key perm32(m) of the subtile
    uint16_t vt[D][kSub + 8];     // row 32*dt + m holds feature 32*dt + perm32(m), keys in order
};

// Per-thread share of one subtile: D/64 K vectors and D/64 V^T vectors of 16 bytes.
template <int D>
struct Regs {
    u32x4 k[D / 64];
    u32x4 v[D / 64];
};

struct SubInfo {
    int key0, nval, flags;
};

__device__ __forceinline__ SubInfo sub_info(const int2 *ulist, int us) {
    const int2 e = ulist[us];
    return SubInfo{e.x, e.y & 0xFF, e.y >> 8};
}

// Frame geometry of a subtile, uniform across the workgroup: the subtile's 32 keys lie in
// frame f0 (from token t0 on) and, past the frame end, in frame f0 + 1.
struct SubGeom {
    uint32_t krow0, krow1;     // ring row (in units of D) of token 0 of frames f0, f0 + 1
    uint32_t vcol0, vcol1;     // element offset of V^T frame f0, f0 + 1
    int t0, nval;
};

__device__ __forceinline__ SubGeom sub_geom(const hf_attn_args &a, uint32_t magicT, int bh, SubInfo si) {
    const int key0 = __builtin_amdgcn_readfirstlane(si.key0);
    const int f0 = fast_div(key0, magicT, a.T);
    int s0 = a.head + f0;
    s0 -= (s0 >= a.W) ? a.W : 0;
    int s1 = s0 + 1;
    s1 -= (s1 >= a.W) ? a.W : 0;
    SubGeom g;
    g.t0 = key0 - f0 * a.T;
    g.krow0 = (uint32_t)((bh * a.W + s0) * a.T);
    g.krow1 = (uint32_t)((bh * a.W + s1) * a.T) - (uint32_t)a.T;   // + t with t >= T
    g.vcol0 = g.krow0 * (uint32_t)a.D;
    g.vcol1 = (uint32_t)((bh * a.W + s1) * a.T) * (uint32_t)a.D - (uint32_t)a.T;
    g.nval = __builtin_amdgcn_readfirstlane(si.nval);
    return g;
}

// Per-thread constants of the cooperative subtile load (see load_sub).
template <int D>
struct LoadPlan {
    int kr[D / 64];            // subtile key row of the thread's K vector
    uint32_t kcol[D / 64];     // byte offset of its 8 features in the row
    int kg8[D / 64];           // first key (0, 8, 16, 24) of the thread's V^T vector
    uint32_t dT[D / 64];       // feature row d of the V^T vector, times T
};

template <int D>
__device__ __forceinline__ LoadPlan<D> load_plan(int tid, int T) {
    LoadPlan<D> p;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
        const int v = tid + 256 * e;
        p.kr[e] = v / (D / 8);
        p.kcol[e] = (uint32_t)(v % (D / 8)) * 16u;
        p.kg8[e] = 8 * (v % 4);
        p.dT[e] = (uint32_t)(v / 4) * (uint32_t)T;
    }
    return p;
}

// Global -> registers for one subtile.  Rows past the subtile's valid keys re-read its
// first key (finite data; their scores are masked).  Byte offsets stay below 2^32 (the
// ring holds fewer than 2^31 elements), so each load is a 32-bit offset from the ring base.
template <int D>
__device__ __forceinline__ void load_sub(const hf_attn_args &a, const SubGeom &g, const LoadPlan<D> &p,
                                         Regs<D> &r) {
    const char *kbase = reinterpret_cast<const char *>(a.ring_k);
    const char *vbase = reinterpret_cast<const char *>(a.ring_vt);
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
        const int t = g.t0 + (p.kr[e] < g.nval ? p.kr[e] : 0);
        const uint32_t row = (t >= a.T ? g.krow1 : g.krow0) + (uint32_t)t;
        r.k[e] = *reinterpret_cast<const u32x4 *>(kbase + (row * (uint32_t)(D * 2) + p.kcol[e]));
        const int tv = g.t0 + (p.kg8[e] < g.nval ? p.kg8[e] : 0);
        const uint32_t col = (tv >= a.T ? g.vcol1 : g.vcol0) + p.dT[e] + (uint32_t)tv;
        r.v[e] = *reinterpret_cast<const u32x4 *>(vbase + col * 2u);
    }
}

template <int D>
__device__ __forceinline__ void store_sub(const Regs<D> &r, Stage<D> &st, int tid) {
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
        const int v = tid + 256 * e;
        const int kr = v / (D / 8), col8 = v % (D / 8);
        *reinterpret_cast<u32x4 *>(&st.k[inv_perm32(kr)][8 * col8]) = r.k[e];
        const int d = v / 4, kg = v % 4;
        *reinterpret_cast<u32x4 *>(&st.vt[32 * (d / 32) + inv_perm32(d % 32)][8 * kg]) = r.v[e];
    }
}

template <int D>
__global__ __launch_bounds__(256, 2) void sparse_attn_kernel(hf_attn_args a, uint32_t magicT, float c_log2,
                                                             int per_xcd, int npairs) {
    __shared__ Stage<D> stage[2];
    extern __shared__ __align__(16) unsigned char dyn[];
    const int nsub = (a.bk + kSub - 1) / kSub;
    int2 *ulist = reinterpret_cast<int2 *>(dyn);                                   // [nkb * nsub]
    unsigned char *fa = dyn + (size_t)a.nkb * nsub * sizeof(int2);                 // [nkb]
    unsigned char *fb = fa + a.nkb;                                                // [nkb]
    __shared__ int s_usub;

    const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (item >= a.BH * npairs) return;
    const int bh = item / npairs, pair = item - bh * npairs;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 31, g = lane >> 5;
    const int qbA = 2 * pair, qbB = 2 * pair + 1;
    const bool hasB = qbB < a.nqb;

    // ---- union of the two kept lists, as a list of non-empty 32-key subtiles in key order
    for (int j = tid; j < a.nkb; j += 256) fa[j] = fb[j] = 0;
    __syncthreads();
    {
        const int32_t *selA = a.idx + ((size_t)bh * a.nqb + qbA) * a.top_k;
        const int32_t *selB = a.idx + ((size_t)bh * a.nqb + (hasB ? qbB : qbA)) * a.top_k;
        for (int t = tid; t < a.top_k; t += 256) {
            // out-of-range indices (a caller error) are clamped so that no load leaves the window
            fa[min(max(selA[t], 0), a.nkb - 1)] = 1;
            if (hasB) fb[min(max(selB[t], 0), a.nkb - 1)] = 1;
        }
    }
    __syncthreads();
    if (w == 0) {
        const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        int base = 0;
        for (int j0 = 0; j0 < a.nkb; j0 += 64) {
            const int j = j0 + lane;
            const int flags = j < a.nkb ? (fa[j] | (fb[j] << 1)) : 0;
            const int kb0 = j * a.bk, kb1 = min(kb0 + a.bk, a.Nk);
            const int cnt = flags ? min(nsub, (kb1 - kb0 + kSub - 1) / kSub) : 0;
            int before = 0, total = 0;
            for (int s = 0; s < nsub; ++s) {
                const uint64_t b = __ballot(cnt > s);
                before += __popcll(b & lt_mask);
                total += __popcll(b);
            }
            for (int s = 0; s < cnt; ++s) {
                const int key0 = kb0 + kSub * s;
                ulist[base + before + s] = int2{key0, min(kSub, kb1 - key0) | (flags << 8)};
            }
            base += total;
        }
        if (lane == 0) s_usub = base;
    }
    __syncthreads();
    const int usub = s_usub;

    // ---- this wave's 32 queries: query block (w >> 1), tile (w & 1)
    const int myblk = w >> 1;
    const int qb = myblk ? qbB : qbA;
    const int q0 = qb * a.bq, qend = min(q0 + a.bq, a.Nq);
    const int qrow0 = q0 + 32 * (w & 1);
    const bool active = (myblk == 0 || hasB) && qrow0 < qend;
    const int myflag = 1 << myblk;

    u32x4 qf[D / 16];
    {
        int row = qrow0 + n;
        if (!active || row >= qend) row = min(q0, a.Nq - 1);
        const uint16_t *qp = a.q + ((size_t)bh * a.Nq + row) * D + 8 * g;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qf[s] = *reinterpret_cast<const u32x4 *>(qp + 16 * s);
    }
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
    float m = -INFINITY, l = 0.f;

    auto compute = [&](int us, const Stage<D> &st) {
        const SubInfo si = sub_info(ulist, us);
        if (!active || !(si.flags & myflag)) return;
        f32x16 sc = {};
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            sc = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(&st.k[n][16 * s + 8 * g])), as_bf16x8(qf[s]), sc);
        if (si.nval < kSub) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (16 * g + i >= si.nval) sc[i] = -INFINITY;
        }
        float mx = sc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (__any((mx - m) * c_log2 > kLazyRescaleLog2)) {
            const float mn = fmaxf(m, mx);
            const float alpha = __builtin_amdgcn_exp2f((m - mn) * c_log2);
            m = mn;
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
        }
        const float mc = m * c_log2;
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], c_log2, -mc));
            l += p[i];
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
                acc[dt] = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(&st.vt[32 * dt + n][16 * g + 8 * ks])),
                                 as_bf16x8(pf[ks]), acc[dt]);
    };

    // ---- main loop.  LDS stage (us & 1) holds subtile us; four register buffers carry the
    // loads of subtiles us+1 .. us+4, so a load has three steps to land before it is staged.
    // Loads are issued unconditionally (past the end they repeat the last subtile) so that
    // the wait for a staged subtile never covers the younger prefetches behind it.
    const int last = usub - 1;   // >= 0: every kept block holds at least one key
    const LoadPlan<D> plan = load_plan<D>(tid, a.T);
    auto fetch = [&](int us, Regs<D> &r) {
        load_sub<D>(a, sub_geom(a, magicT, bh, sub_info(ulist, min(us, last))), plan, r);
    };
    Regs<D> r0, r1, r2, r3;
    fetch(0, r0);
    fetch(1, r1);
    fetch(2, r2);
    fetch(3, r3);
    store_sub<D>(r0, stage[0], tid);
    // Drain every load issued so far (the Q fragments included) once, so that inside the
    // loop only the prefetch of later subtiles is outstanding.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // one step: prefetch subtile us+4 into `ld` (free: its subtile us is already staged),
    // compute subtile us, stage subtile us+1 from `nx`
    // (the scheduling barriers keep the prefetch ahead of the compute: the memory counter is
    // in order, so a prefetch sunk below the staging store would be waited for there)
    auto step = [&](int us, Regs<D> &ld, const Stage<D> &cs, const Regs<D> &nx, Stage<D> &ns) {
        fetch(us + 4, ld);
        __builtin_amdgcn_sched_barrier(0);
        compute(us, cs);
        __builtin_amdgcn_sched_barrier(0);
        store_sub<D>(nx, ns, tid);
        __syncthreads();
    };
    for (int us = 0; us < usub; us += 4) {
        step(us, r0, stage[0], r1, stage[1]);
        if (us + 1 >= usub) break;
        step(us + 1, r1, stage[1], r2, stage[0]);
        if (us + 2 >= usub) break;
        step(us + 2, r2, stage[0], r3, stage[1]);
        if (us + 3 >= usub) break;
        step(us + 3, r3, stage[1], r0, stage[0]);
    }
    if (!active) return;

    // ---- epilogue: normalise, add the linear readout, store fp32
    const float inv_l = 1.f / (l + __shfl_xor(l, 32));
    const int row = qrow0 + n;
    const bool row_ok = row < qend;
    float *op = a.out + ((size_t)bh * a.Nq + (row_ok ? row : q0)) * D + 16 * g;
    if (a.st) {
        // phi(q) as the B operand (same fragment layout as Q^T) and the normaliser
        u32x4 pq[D / 16];
        float den = 0.f;
        const float *zp = a.zc + (size_t)bh * D + 8 * g;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const uint32_t wv[4] = {qf[s].x, qf[s].y, qf[s].z, qf[s].w};
            const f32x4 z0 = *reinterpret_cast<const f32x4 *>(zp + 16 * s);
            const f32x4 z1 = *reinterpret_cast<const f32x4 *>(zp + 16 * s + 4);
            const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
            float ph[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ph[2 * e] = phi_f32(bf16_lo_to_f32(wv[e]));
                ph[2 * e + 1] = phi_f32(bf16_hi_to_f32(wv[e]));
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
                    o4[v] = f32x4{acc[dt][4 * v] * inv_l + lin[4 * v] * inv_den,
                                  acc[dt][4 * v + 1] * inv_l + lin[4 * v + 1] * inv_den,
                                  acc[dt][4 * v + 2] * inv_l + lin[4 * v + 2] * inv_den,
                                  acc[dt][4 * v + 3] * inv_l + lin[4 * v + 3] * inv_den};
            }
        }
    } else if (row_ok) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            f32x4 *o4 = reinterpret_cast<f32x4 *>(op + 32 * dt);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                o4[v] = f32x4{acc[dt][4 * v] * inv_l, acc[dt][4 * v + 1] * inv_l, acc[dt][4 * v + 2] * inv_l,
                              acc[dt][4 * v + 3] * inv_l};
        }
    }
}

}  // namespace
}  // namespace hf

hipError_t hf_launch_sparse_attn(const hf_attn_args &a, hipStream_t s) {
    const int npairs = (a.nqb + 1) / 2;
    const int items = a.BH * npairs;
    const int per_xcd = (items + 7) / 8;
    const dim3 grid((unsigned)(per_xcd * 8));
    const uint32_t magicT = hf::div_magic((uint32_t)a.T);
    const float c_log2 = (float)(1.4426950408889634 / sqrt((double)a.D));
    const int nsub = (a.bk + hf::kSub - 1) / hf::kSub;
    const size_t dyn = (size_t)a.nkb * nsub * sizeof(int2) + 2 * (size_t)a.nkb;
    if (a.D == 64)
        hipLaunchKernelGGL((hf::sparse_attn_kernel<64>), grid, dim3(256), dyn, s, a, magicT, c_log2, per_xcd, npairs);
    else
        hipLaunchKernelGGL((hf::sparse_attn_kernel<128>), grid, dim3(256), dyn, s, a, magicT, c_log2, per_xcd, npairs);
    return hipGetLastError();
}
