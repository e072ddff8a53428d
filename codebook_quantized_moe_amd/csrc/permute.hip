// Stable counting sort of the (token, slot) pairs by expert: one workgroup of 16 wavefronts
// running permute_block.
#include "permute_device.h"
#include "route_device.h"

namespace moeq {

constexpr int kPermWaves = 16;

__global__ void __launch_bounds__(64 * kPermWaves) permute_kernel(const int32_t* __restrict__ ids,
                                                                   int P, int E,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ sorted_pair,
                                                                   int32_t* __restrict__ pair_pos) {
    permute_block<kPermWaves>(ids, P, E, offsets, sorted_pair, pair_pos);
}

// Routing and permutation in one workgroup of 16 wavefronts (few tokens: one launch instead
// of two): wavefront w routes tokens w, w + 16, ...; then the permutation of their pairs.
__global__ void __launch_bounds__(64 * kPermWaves) route_permute_kernel(
    const float* __restrict__ logits, int T, int E, int k, int sigmoid, int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos) {
    for (int t = threadIdx.x >> 6; t < T; t += kPermWaves)
        route_token(logits, t, E, k, sigmoid != 0, ids, w);
    __syncthreads();
    permute_block<kPermWaves>(ids, T * k, E, offsets, sorted_pair, pair_pos);
}

void launch_route_permute(const float* logits, int T, int E, int k, bool sigmoid, int32_t* ids,
                          float* w, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                          hipStream_t stream) {
    hipLaunchKernelGGL(route_permute_kernel, dim3(1), dim3(64 * kPermWaves), 0, stream, logits, T,
                       E, k, sigmoid ? 1 : 0, ids, w, offsets, sorted_pair, pair_pos);
}

void launch_permute(const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pair,
                    int32_t* pair_pos, hipStream_t stream) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(64 * kPermWaves), 0, stream, ids, P, E,
                       offsets, sorted_pair, pair_pos);
}

}  // namespace moeq
