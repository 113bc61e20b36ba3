// State pass over the linear attention state (S, z).
//
// One launch does any of:
//   * prepare the readout operands of this step from the state as it is (a step reads the
//     state before its own evictions are absorbed): S^T rounded to bf16 ([c][a], the
//     matrix-core operand layout of phi(q)^T S) and a copy of z;
//   * finish an absorb ([HF-abs]; [HF-de] §2.A): add the partial sums written by
//     absorb_partial, taken in split order, to S and z.
// Each workgroup owns one 32x32 tile of S (and the matching 32 entries of z), so reading
// the old value and writing the new one never race.  Pure data movement, HBM/L2-bound.
#include "hf_internal.h"

namespace hf {
namespace {

constexpr int kGroup = 16;   // partial loads in flight per thread

template <int D>
__global__ __launch_bounds__(256) void state_kernel(hf_state_args a) {
    __shared__ float tile[32][33];
    constexpr int tiles = D / 32;
    const int bh = blockIdx.x / (tiles * tiles);
    const int ta = (blockIdx.x / tiles) % tiles, tc = blockIdx.x % tiles;
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
        for (int q0 = 0; q0 < a.P; q0 += kGroup) {
            f32x4 v[kGroup];
#pragma unroll
            for (int i = 0; i < kGroup; ++i)
                v[i] = q0 + i < a.P ? *reinterpret_cast<const f32x4 *>(pp + (size_t)(q0 + i) * 64 * D) : f32x4{};
#pragma unroll
            for (int i = 0; i < kGroup; ++i)
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
            for (int q0 = 0; q0 < a.P; q0 += kGroup) {
                float v[kGroup];
#pragma unroll
                for (int i = 0; i < kGroup; ++i) v[i] = q0 + i < a.P ? zp[(size_t)(q0 + i) * 64] : 0.f;
#pragma unroll
                for (int i = 0; i < kGroup; ++i)
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

}  // namespace
}  // namespace hf

hipError_t hf_launch_state(const hf_state_args &a, hipStream_t s) {
    const int tiles = a.D / 32;
    const dim3 grid((unsigned)(a.BH * tiles * tiles));
    if (a.D == 64)
        hipLaunchKernelGGL(hf::state_kernel<64>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(hf::state_kernel<128>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}
