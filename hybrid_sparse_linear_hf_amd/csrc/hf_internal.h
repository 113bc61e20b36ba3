// Internal declarations shared by the HIP sources of libhf (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hf.h"

namespace hf {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// ------------------------------------------------------------------ bf16 helpers

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two fp32 -> packed bf16 pair (round to nearest even; one v_cvt_pk_bf16_f32), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// fp32 -> bf16 bits (round to nearest even).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// elu(x) + 1, branch-free: exp(x) as exp2(x log2 e) on the transcendental unit, selected
// for x <= 0.
__device__ __forceinline__ float phi_f32(float x) {
    const float e = __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
    return x > 0.f ? x + 1.f : e;
}

// n / d for 0 <= n < 2^31 with magic = ceil(2^32 / d) (one correction step suffices).
__host__ __device__ inline uint32_t div_magic(uint32_t d) {
    return (uint32_t)((0x100000000ull + (uint64_t)d - 1) / (uint64_t)d);
}
__device__ __forceinline__ int fast_div(int n, uint32_t magic, int d) {
    int q = (int)__umulhi((uint32_t)n, magic);
    q -= (q * d > n);
    return q;
}

// ------------------------------------------------------------------ LDS pipelines
// Workgroup barrier that orders LDS accesses only.  __syncthreads() also orders global
// memory, which makes the compiler wait for every load in flight -- including the
// direct-to-LDS fetches of later stages that this barrier must not wait for.  The empty
// asm statements keep the compiler from moving memory accesses across; the wait drains
// this wave's LDS reads and writes before the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited on
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt with vmcnt(n), expcnt and lgkmcnt at their maxima (no wait on those).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// ------------------------------------------------------------------ matrix cores
// D = A * B + C on a 32x32x16 bf16 tile.  Lane l supplies A row (l % 32) and B column
// (l % 32), 8 contraction elements each (the same 8 for A and B); the accumulator of
// lane l holds rows 8*(i/4) + 4*(l/32) + (i%4), i = 0..15, of column l % 32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Accumulator rows held by a lane are {8*(i/4) + 4*g + i%4}.  Feeding operand row
// perm32(m) from lane m makes lane group g hold the 16 CONSECUTIVE logical rows
// 16*g + i, i = 0..15, in accumulator slot i.
__device__ __forceinline__ int perm32(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }


}  // namespace hf

// ------------------------------------------------------------------ host-side launch API
// (implemented in the .hip files, called from hf_api.cpp)

struct hf_state_args {
    int BH, D;
    float *S, *z;              // state, read (and updated when part != null)
    const float *part;         // absorb partials to add (null: none), P splits
    int P;
    uint16_t *st;              // out: S^T bf16 of the state as read (null: skip)
    float *zc;                 // out: copy of z as read (null: skip)
};
hipError_t hf_launch_state(const hf_state_args &a, hipStream_t s);

struct hf_append_args {
    int BH, D, T, W, head, first_frame, C;
    const uint16_t *k_cur, *v_cur;
    uint16_t *ring_k, *ring_vg;
};

struct hf_select_args {
    int BH, D, T, W, head, Nq, Nk, bq, bk, nqb, nkb, top_k;
    const uint16_t *q, *ring_k;
    double *qbar, *kbar;       // workspace: pooled blocks
    int32_t *idx;
    double *scores;            // may be null
    // hierarchical selection (top_frames > 0): frames of the window, pooled per frame
    int nfr, top_frames;
    double *fbar;              // workspace: frame-pooled keys [BH][nfr][D]
    double *part;              // workspace: per key block, sums of its rows in its first frame
                               // and in the next one [BH][nkb][2][D] (needs bk <= T)
    // readout preparation run as extra workgroups of the pool launch (prep_tiles > 0)
    hf_state_args prep;
    int prep_tiles;
    // a hybrid step's ring append, run as extra workgroups of the score + top-k launch
    // (app_tiles > 0); the pool then reads the keys of the current chunk (logical frames
    // >= ncom) from k_cur, not the ring
    hf_append_args app;
    int app_tiles;
    const uint16_t *k_cur;     // null: every key from the ring
    int ncom;
    int32_t *fidx;             // may be null: kept frames [BH][nqb][top_frames], ascending
    double *fscores;           // may be null: frame scores [BH][nqb][nfr]
};
constexpr int kMaxHierFrames = 64;   // window frames the hierarchical selection handles
constexpr int kMaxKeyBlocks = 1536;  // key blocks of a window (sizes the attention's LDS lists)
hipError_t hf_launch_block_select(const hf_select_args &a, hipStream_t s);

struct hf_attn_args {
    int BH, D, T, W, head, Nq, Nk, bq, bk, nqb, nkb, top_k;
    const uint16_t *q, *ring_k, *ring_vg;
    const int32_t *idx;
    const uint16_t *st;        // S^T in bf16 [BH][D][D] (null: sparse part only)
    const float *zc;           // z [BH][D] as read by this step
    float eps;
    float *out;
    float *lse;                // null, or [BH][Nq]: log2 of each query's softmax sum (base-2 logits)
    // relative temporal rotation: rope_dt rotated features (0 = off, 16 or 32),
    // offsets clamped to +-rope_cap, theta_i = 2^(i * rope_c1); ncom = window frames before the chunk
    int rope_dt, rope_cap, ncom;
    float rope_c1;
    // absorb of the ab_E oldest window tokens (the frames a committed step evicts), run by
    // extra workgroups of the same launch (ab_E = 0: none): split partial sums into ab_part
    // (workspace, hf_absorb_partial_floats floats, the layout the state pass adds up)
    int ab_E;
    float *ab_part;
    int ab_P, ab_items, ab_nab;   // set by the launcher: splits, work items, workgroups (items rounded up to 8)
};
hipError_t hf_launch_sparse_attn(const hf_attn_args &a, hipStream_t s);

// Backward of the step output (backward.hip); arguments validated by the caller.
struct hf_bwd_args {
    int BH, D, T, W, head, Nq, Nk, bq, bk, nqb, nkb, top_k, NkP, NqP, splits;
    const uint16_t *q, *ring_k, *ring_vg;
    const int32_t *idx;
    const float *S, *z, *out, *lse, *dout;
    float eps;
    float *dq, *dk, *dv, *dS, *dz;
    // workspace
    uint16_t *kr, *vr;         // window K rows, V rows [BH][NkP][D] (logical order, zero pad)
    uint16_t *gr;              // dO rows in bf16 [BH][NqP][D]
    uint16_t *sb, *stb;        // S and S^T in bf16 [BH][D][D]
    float *delta;              // [BH][NqP]: dO . (sparse part of out)
    float *rod;                // [BH][NqP][2]: 1 / den and dden of each query (readout pass -> dq pass)
    int32_t *qoff, *qlist;     // per key block, the query blocks that kept it: [BH][nkb+1], [BH][nqb*top_k]
    int32_t *korder;           // [BH*nkb] key blocks (bh * nkb + j) by descending kept-by count
    float *dsp, *dzp;          // readout partials [BH][splits][D][D], [BH][splits][D]
};
size_t hf_bwd_workspace_bytes(int BH, int D, int Nq, int Nk, int bq, int bk, int top_k);
void hf_bwd_layout(hf_bwd_args &a, void *ws);
hipError_t hf_launch_attn_backward(const hf_bwd_args &a, hipStream_t s);

struct hf_absorb_bwd_args {
    int BH, D;
    int64_t n_tok;
    const uint16_t *k, *v;     // evicted tokens [BH][n_tok][D]
    const float *dS, *dz;
    uint16_t *sb, *stb;        // workspace: dS and dS^T in bf16 [BH][D][D]
    float *dk, *dv;            // [BH][n_tok][D]
};
hipError_t hf_launch_absorb_backward(const hf_absorb_bwd_args &a, hipStream_t s);

struct hf_absorb_args {
    int BH, D;
    int64_t n_tok;
    const uint16_t *k, *v;     // row-major evicted tokens [BH][n_tok][D]
    float *part;               // workspace: partial sums (hf_absorb_partial_floats floats)
};
int hf_absorb_splits(int BH, int D, int64_t n_tok);
int hf_step_absorb_splits(int BH, int D, int64_t n_tok);   // the absorb inside a step's attention launch
size_t hf_absorb_partial_floats(int BH, int D, int P);
size_t hf_absorb_workspace_bytes(int BH, int D);
hipError_t hf_launch_absorb_partial(const hf_absorb_args &a, hipStream_t s);


// Chunk-aware growth schedule (schedule.hip); arguments validated by the caller.
hf_status hf_cag_schedule_impl(int32_t n, const int32_t *nkb, double s_base, double s_target, double s_max,
                               int32_t *top_k, double *sparsity, double *beta_out);

hipError_t hf_launch_ring_append(const hf_append_args &a, hipStream_t s);
int hf_append_tiles(const hf_append_args &a);   // workgroups of an append

// A hybrid step split into validation and enqueue (hf_api.hip), so that entry points with
// another source of workspace memory share both.
hf_status hf_step_validate(const hf_dims *d, const void *q, const void *k_cur, const void *v_cur,
                           const hf_kv_ring *ring, int32_t top_k, uint32_t flags, const float *S, const float *z,
                           float eps, const int32_t *idx, const float *out);
size_t hf_step_workspace_bytes(const hf_dims *d);   // dims validated
hf_status hf_step_enqueue(const hf_dims *d, const void *q, const void *k_cur, const void *v_cur, hf_kv_ring *ring,
                          int32_t top_k, uint32_t flags, float *S, float *z, float eps, const hf_rope *rope,
                          int32_t *idx, float *out, void *ws, const hf_step_events *events, hipStream_t stream);
hf_status hf_fail_unsupported(const char *msg, size_t need, size_t have);
hf_status hf_fail_hip(hipError_t e, const char *what);
