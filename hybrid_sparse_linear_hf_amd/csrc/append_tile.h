// Ring append tile, shared by the append launch and the hybrid step's fused selection
// launch: write one 64-token tile of the current chunk's key/value frames into their window
// slots.  Keys are copied as they are ([T][D] per frame); values are regrouped per 8 tokens
// to [T/8][D][8], the layout in which the attention and absorb kernels fetch them (whole
// cache lines) and feed them to the matrix cores.  Pure data movement, bound by HBM
// bandwidth.
#pragma once

#include "hf_internal.h"

namespace hf {

constexpr int kTileTok = 64;

// One tile per (plane, chunk frame, 64 tokens), for a workgroup of 256 threads.  Threads
// 0..127 regroup V: each owns an 8-token x 8-feature block, loads its 8 rows (16 bytes
// each), transposes the 8x8 block of 16-bit values in registers (byte permutes) and puts
// the 8 features' 16-byte token rows into `vbuf` (LDS, 64 / 8 * D pieces of 16 bytes) at
// their positions in the tile's groups.  Lane t of the regrouping threads takes feature
// group t % 16 and token group t / 16, so the 16 lanes of a token group read whole V
// rows.  Threads 128..255 copy the tile's K rows, 8 16-byte vectors each, every load
// issued before the first store.  Then all 256 threads store the tile's groups, one
// contiguous run of the slot, from `vbuf`: every store instruction writes whole lines.
// LDS position of value piece f (feature f of a token group) within its group's D pieces:
// bits 4-6 of f XORed into bits 0-2, so that the 16 lanes of a piece write (features
// 8 fg + i, fg = 0 .. 15) and of a piece read (16 consecutive features) each touch 16
// distinct 16-byte bank groups
__device__ __forceinline__ int vpos(int f) { return f ^ ((f >> 4) & 7); }

template <int D>
__device__ void append_tile(const hf_append_args &a, int tile, u32x4 *vbuf) {
    const int tiles_per_frame = (a.T + kTileTok - 1) / kTileTok;
    const int tile_id = tile % tiles_per_frame;
    const int fc = (tile / tiles_per_frame) % a.C;   // frame within the chunk
    const int bh = tile / (tiles_per_frame * a.C);
    const int t0 = tile_id * kTileTok;
    const int ntok = min(kTileTok, a.T - t0);               // a multiple of 8 (T % 8 == 0)
    int slot = a.head + a.first_frame + fc;
    slot %= a.W;

    const size_t src_row0 = ((size_t)bh * a.C + fc) * a.T + t0;           // in rows of D
    const int tid = threadIdx.x;
    if (tid < 128) {
        const int fg = tid % 16, tg = tid / 16;             // feature group, token group
        if (fg < D / 8 && 8 * tg < ntok) {
            const uint16_t *src = a.v_cur + (src_row0 + 8 * tg) * D + 8 * fg;
            u32x4 in[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) in[r] = *reinterpret_cast<const u32x4 *>(src + (size_t)r * D);
            // piece i = feature 8fg + i over tokens 8tg .. 8tg + 7, at LDS position tg D + 8fg + i
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
                uint32_t o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t wa = in[2 * j][i >> 1], wb = in[2 * j + 1][i >> 1];
                    o[j] = __builtin_amdgcn_perm(wb, wa, sel);
                }
                vbuf[tg * D + vpos(8 * fg + i)] = u32x4{o[0], o[1], o[2], o[3]};
            }
        }
    } else {
        constexpr int kVecPerRow = D / 8;
        constexpr int kIters = kTileTok * kVecPerRow / 128;
        const uint16_t *ksrc = a.k_cur + src_row0 * D;
        uint16_t *kdst = a.ring_k + (((size_t)bh * a.W + slot) * a.T + t0) * D;
        u32x4 kv[kIters];
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int e = tid - 128 + 128 * it;
            const int r = min(e / kVecPerRow, ntok - 1), c8 = (e % kVecPerRow) * 8;
            kv[it] = *reinterpret_cast<const u32x4 *>(ksrc + (size_t)r * D + c8);
        }
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int e = tid - 128 + 128 * it;
            const int r = e / kVecPerRow, c8 = (e % kVecPerRow) * 8;
            if (r < ntok) *reinterpret_cast<u32x4 *>(kdst + (size_t)r * D + c8) = kv[it];
        }
    }
    __syncthreads();
    // the tile's groups are one contiguous run of the slot: piece e of the run is LDS piece e
    uint16_t *vdst = a.ring_vg + (((size_t)bh * a.W + slot) * a.T + t0) * D;
    const int npieces = (ntok / 8) * D;
    for (int e = tid; e < npieces; e += 256) *reinterpret_cast<u32x4 *>(vdst + 8 * e) = vbuf[(e & ~(D - 1)) | vpos(e & (D - 1))];
}


inline int append_tiles(const hf_append_args &a) { return a.BH * a.C * ((a.T + kTileTok - 1) / kTileTok); }

}  // namespace hf
