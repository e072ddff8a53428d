// Stable counting sort of the (token, slot) pairs by expert: one workgroup of 16 wavefronts
// running permute_block.
#include "permute_device.h"

namespace moeq {

constexpr int kPermWaves = 16;

__global__ void __launch_bounds__(64 * kPermWaves) permute_kernel(const int32_t* __restrict__ ids,
                                                                   int P, int E,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ sorted_pair,
                                                                   int32_t* __restrict__ pair_pos) {
    permute_block<kPermWaves>(ids, P, E, offsets, sorted_pair, pair_pos);
}

void launch_permute(const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pair,
                    int32_t* pair_pos, hipStream_t stream) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(64 * kPermWaves), 0, stream, ids, P, E,
                       offsets, sorted_pair, pair_pos);
}

}  // namespace moeq
