// One 32 x 32 tile of the state pass (see state.hip), shared by the state kernel and by
// the block-select launch of a hybrid step, which runs the readout preparation as extra
// workgroups.
#pragma once

#include "hf_internal.h"

namespace hf {

constexpr int kStateGroup = 16;   // partial loads in flight per thread

// Tile t (of BH * (D/32)^2) of the state pass, run by a 256-thread workgroup; `tile` is
// 32 x 33 floats of LDS.
template <int D>
__device__ __forceinline__ void state_tile(const hf_state_args &a, int t, float (*tile)[33]) {
    constexpr int tiles = D / 32;
    const int bh = t / (tiles * tiles);
    const int ta = (t / tiles) % tiles, tc = t % tiles;
    // one float4 of the tile per thread: row r, columns c4 .. c4 + 3
    const int r = threadIdx.x >> 3, c4 = (threadIdx.x & 7) * 4;
    const int row = 32 * ta + r, col = 32 * tc + c4;
    float *Sp = a.S + ((size_t)bh * D + row) * D + col;
    const f32x4 old = *reinterpret_cast<const f32x4 *>(Sp);
    if (a.part) {
        // the partials are loaded 16 splits at a time, all before the first add; the sum
        // runs in split order
        const float *pp = a.part + ((size_t)(bh * (D / 64) + row / 64) * a.P) * 64 * D + (size_t)(row % 64) * D + col;
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
        for (int q0 = 0; q0 < a.P; q0 += kStateGroup) {
            f32x4 v[kStateGroup];
#pragma unroll
            for (int i = 0; i < kStateGroup; ++i)
                v[i] = q0 + i < a.P ? *reinterpret_cast<const f32x4 *>(pp + (size_t)(q0 + i) * 64 * D) : f32x4{};
#pragma unroll
            for (int i = 0; i < kStateGroup; ++i)
                if (q0 + i < a.P) sum += v[i];
        }
        *reinterpret_cast<f32x4 *>(Sp) = old + sum;
    }
    tile[r][c4] = old.x;
    tile[r][c4 + 1] = old.y;
    tile[r][c4 + 2] = old.z;
    tile[r][c4 + 3] = old.w;
    if (tc == 0 && threadIdx.x < 32) {
        const int zr = 32 * ta + threadIdx.x;
        const float zold = a.z[(size_t)bh * D + zr];
        if (a.zc) a.zc[(size_t)bh * D + zr] = zold;
        if (a.part) {
            const size_t items = (size_t)a.BH * (D / 64) * a.P;        // partial blocks
            const float *zp = a.part + items * 64 * D + ((size_t)(bh * (D / 64) + zr / 64) * a.P) * 64 + zr % 64;
            float sum = 0.f;
            for (int q0 = 0; q0 < a.P; q0 += kStateGroup) {
                float v[kStateGroup];
#pragma unroll
                for (int i = 0; i < kStateGroup; ++i) v[i] = q0 + i < a.P ? zp[(size_t)(q0 + i) * 64] : 0.f;
#pragma unroll
                for (int i = 0; i < kStateGroup; ++i)
                    if (q0 + i < a.P) sum += v[i];
            }
            a.z[(size_t)bh * D + zr] = zold + sum;
        }
    }
    if (!a.st) return;
    __syncthreads();
    // S^T in bf16: output row 32 tc + cc (a column of the tile), 4 consecutive tile rows
    const int cc = threadIdx.x >> 3, rr = (threadIdx.x & 7) * 4;
    uint16_t *dst = a.st + ((size_t)bh * D + 32 * tc + cc) * D + 32 * ta + rr;
    const uint32_t w0 = pack_bf16x2(tile[rr][cc], tile[rr + 1][cc]);
    const uint32_t w1 = pack_bf16x2(tile[rr + 2][cc], tile[rr + 3][cc]);
    *reinterpret_cast<u32x2 *>(dst) = u32x2{w0, w1};
}

}  // namespace hf
