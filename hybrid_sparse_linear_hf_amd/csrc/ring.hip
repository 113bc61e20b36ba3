// Ring append: write the current chunk's key/value frames into their window slots (one
// workgroup per 64-token tile; the tile code is shared with the hybrid step's fused
// selection launch).
#include "append_tile.h"

namespace hf {
namespace {

template <int D>
__global__ __launch_bounds__(256) void ring_append_kernel(hf_append_args a) {
    __shared__ u32x4 vbuf[kTileTok / 8 * D];
    append_tile<D>(a, blockIdx.x, vbuf);
}

}  // namespace
}  // namespace hf

hipError_t hf_launch_ring_append(const hf_append_args &a, hipStream_t s) {
    const dim3 grid((unsigned)hf::append_tiles(a));
    if (a.D == 64)
        hipLaunchKernelGGL(hf::ring_append_kernel<64>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(hf::ring_append_kernel<128>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

int hf_append_tiles(const hf_append_args &a) { return hf::append_tiles(a); }
