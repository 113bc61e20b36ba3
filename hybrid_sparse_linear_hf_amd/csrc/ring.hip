// Ring append: write the current chunk's key/value frames into their window slots.
// Keys are copied as they are ([T][D] per frame); values are transposed per frame to
// [D][T], the layout in which the attention and absorb kernels feed them to the matrix
// cores.  Pure data movement, bound by HBM bandwidth.
#include "hf_internal.h"

namespace hf {
namespace {

constexpr int kTileTok = 64;

// One workgroup per (plane, chunk frame, 64-token tile): K rows copied, V tile transposed
// through LDS.
template <int D>
__global__ __launch_bounds__(256) void ring_append_kernel(hf_append_args a) {
    __shared__ uint16_t tile[kTileTok][D + 8];
    const int tiles_per_frame = (a.T + kTileTok - 1) / kTileTok;
    const int tile_id = blockIdx.x % tiles_per_frame;
    const int fc = (blockIdx.x / tiles_per_frame) % a.C;   // frame within the chunk
    const int bh = blockIdx.x / (tiles_per_frame * a.C);
    const int t0 = tile_id * kTileTok;
    const int ntok = min(kTileTok, a.T - t0);
    int slot = a.head + a.first_frame + fc;
    slot %= a.W;

    const size_t src_row0 = ((size_t)bh * a.C + fc) * a.T + t0;           // in rows of D
    const size_t dst_k_row0 = ((size_t)bh * a.W + slot) * a.T + t0;
    const uint16_t *ksrc = a.k_cur + src_row0 * D;
    const uint16_t *vsrc = a.v_cur + src_row0 * D;
    uint16_t *kdst = a.ring_k + dst_k_row0 * D;

    constexpr int kVecPerRow = D / 8;                                     // 16-byte vectors per row
    for (int e = threadIdx.x; e < ntok * kVecPerRow; e += 256) {
        const int r = e / kVecPerRow, c8 = (e % kVecPerRow) * 8;
        const u32x4 kv = *reinterpret_cast<const u32x4 *>(ksrc + (size_t)r * D + c8);
        *reinterpret_cast<u32x4 *>(kdst + (size_t)r * D + c8) = kv;
        const u32x4 vv = *reinterpret_cast<const u32x4 *>(vsrc + (size_t)r * D + c8);
        *reinterpret_cast<u32x4 *>(&tile[r][c8]) = vv;
    }
    __syncthreads();

    // V^T[d][t0 .. t0+ntok): each thread writes 8 consecutive tokens of one d row.
    uint16_t *vdst = a.ring_vt + ((size_t)bh * a.W + slot) * (size_t)D * a.T + t0;
    const int groups = ntok / 8;                                          // T % 8 == 0
    for (int e = threadIdx.x; e < D * groups; e += 256) {
        const int d = e / groups, g8 = (e % groups) * 8;
        u32x4 w;
        w.x = (uint32_t)tile[g8 + 0][d] | ((uint32_t)tile[g8 + 1][d] << 16);
        w.y = (uint32_t)tile[g8 + 2][d] | ((uint32_t)tile[g8 + 3][d] << 16);
        w.z = (uint32_t)tile[g8 + 4][d] | ((uint32_t)tile[g8 + 5][d] << 16);
        w.w = (uint32_t)tile[g8 + 6][d] | ((uint32_t)tile[g8 + 7][d] << 16);
        *reinterpret_cast<u32x4 *>(vdst + (size_t)d * a.T + g8) = w;
    }
}

}  // namespace
}  // namespace hf

hipError_t hf_launch_ring_append(const hf_append_args &a, hipStream_t s) {
    const int tiles = (a.T + hf::kTileTok - 1) / hf::kTileTok;
    const dim3 grid((unsigned)(a.BH * a.C * tiles));
    if (a.D == 64)
        hipLaunchKernelGGL(hf::ring_append_kernel<64>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(hf::ring_append_kernel<128>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}
