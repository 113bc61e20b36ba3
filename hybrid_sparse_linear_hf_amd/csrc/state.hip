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

template <int D>
__global__ __launch_bounds__(256) void state_kernel(hf_state_args a) {
    __shared__ float tile[32][33];
    constexpr int tiles = D / 32;
    const int bh = blockIdx.x / (tiles * tiles);
    const int ta = (blockIdx.x / tiles) % tiles, tc = blockIdx.x % tiles;
    float *S = a.S + (size_t)bh * D * D;
    const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;
    const size_t items = (size_t)a.BH * (D / 64) * a.P;        // partial blocks
    for (int r = ty; r < 32; r += 8) {
        const int row = 32 * ta + r, col = 32 * tc + tx;
        const float old = S[(size_t)row * D + col];
        tile[r][tx] = old;
        if (a.part) {
            const float *pp = a.part + ((size_t)(bh * (D / 64) + row / 64) * a.P) * 64 * D + (size_t)(row % 64) * D + col;
            float sum = pp[0];
            for (int q = 1; q < a.P; ++q) sum += pp[(size_t)q * 64 * D];
            S[(size_t)row * D + col] = old + sum;
        }
    }
    if (tc == 0 && threadIdx.x < 32) {
        const int row = 32 * ta + threadIdx.x;
        const float old = a.z[(size_t)bh * D + row];
        if (a.zc) a.zc[(size_t)bh * D + row] = old;
        if (a.part) {
            const float *zp = a.part + items * 64 * D + ((size_t)(bh * (D / 64) + row / 64) * a.P) * 64 + row % 64;
            float sum = zp[0];
            for (int q = 1; q < a.P; ++q) sum += zp[(size_t)q * 64];
            a.z[(size_t)bh * D + row] = old + sum;
        }
    }
    if (!a.st) return;
    __syncthreads();
    uint16_t *dst = a.st + (size_t)bh * D * D;
    for (int r = ty; r < 32; r += 8)
        dst[(size_t)(32 * tc + r) * D + 32 * ta + tx] = (uint16_t)f32_to_bf16_bits(tile[tx][r]);
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
