// Top-k routing kernel: one wavefront per token, four tokens per workgroup (the per-token
// selection and gate values are route_token).
#include "route_device.h"

namespace moeq {

__global__ void __launch_bounds__(256) route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int sigmoid,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    route_token(logits, t, E, k, sigmoid != 0, ids, w);
}

void launch_route_topk(const float* logits, int T, int E, int k, bool sigmoid, int32_t* ids,
                       float* w, hipStream_t stream) {
    const int blocks = (T + 3) / 4;
    hipLaunchKernelGGL(route_topk_kernel, dim3(blocks), dim3(256), 0, stream, logits, T, E, k,
                       sigmoid ? 1 : 0, ids, w);
}

}  // namespace moeq
