// Ring append tile, shared by the append launch and the hybrid step's fused selection
// launch: write one 64-token tile of the current chunk's key/value frames into their window
// slots.  Keys are copied as they are ([T][D] per frame); values are transposed per frame
// to [D][T], the layout in which the attention and absorb kernels feed them to the matrix
// cores.  Pure data movement, bound by HBM bandwidth.
#pragma once

#include "hf_internal.h"

namespace hf {

constexpr int kTileTok = 64;

// One tile per (plane, chunk frame, 64 tokens), for a workgroup of 256 threads.  Threads 0..127 transpose V: each
// owns an 8-token x 8-feature block, loads its 8 rows (16 bytes each), transposes the 8x8
// block of 16-bit values in registers (byte permutes) and stores 8 rows of V^T.  Lane t of
// the transposing threads takes token group t % 8 and feature group t / 8, so each store
// instruction writes eight whole 128-byte V^T row segments (64 tokens) and each load reads
// 128-byte halves of V rows.  Threads 128..255 copy the tile's K rows, 8 16-byte vectors
// each.  Every load of a thread is issued before its first store.
template <int D>
__device__ void append_tile(const hf_append_args &a, int tile) {
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
        const int tg = tid % 8, fg = tid / 8;               // token group, feature group
        if (fg < D / 8 && 8 * tg < ntok) {
            const uint16_t *src = a.v_cur + (src_row0 + 8 * tg) * D + 8 * fg;
            u32x4 in[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) in[r] = *reinterpret_cast<const u32x4 *>(src + (size_t)r * D);
            // out[i] = feature 8fg + i over tokens 8tg .. 8tg + 7
            uint16_t *dst = a.ring_vt + (((size_t)bh * a.W + slot) * D + 8 * fg) * a.T + t0 + 8 * tg;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
                uint32_t o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t wa = in[2 * j][i >> 1], wb = in[2 * j + 1][i >> 1];
                    o[j] = __builtin_amdgcn_perm(wb, wa, sel);
                }
                *reinterpret_cast<u32x4 *>(dst + (size_t)i * a.T) = u32x4{o[0], o[1], o[2], o[3]};
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
}


inline int append_tiles(const hf_append_args &a) { return a.BH * a.C * ((a.T + kTileTok - 1) / kTileTok); }

}  // namespace hf
