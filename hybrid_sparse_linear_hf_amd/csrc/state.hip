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
#include "state_tile.h"

namespace hf {
namespace {

template <int D>
__global__ __launch_bounds__(256) void state_kernel(hf_state_args a) {
    __shared__ float tile[32][33];
    state_tile<D>(a, blockIdx.x, tile);
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
