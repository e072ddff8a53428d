// Unpermute and combine: each token's k expert rows (gate weights already applied by the down
// projection) are summed in fixed slot order in fp32, then the optional shared-expert row and
// the optional residual are added, and the row is rounded to bf16 (README of
// GLM-5.2-EXL3-TR3v4-3.5bpw-MTP78, "Shared residual rotations": expert outputs are
// routing-weighted and summed back into the residual space; "Checkpoint layout update": one
// shared expert per layer beside the routed ones).
// One workgroup per (token, 1024-column chunk), flattened into one grid dimension; 16-byte loads
// of yp, 8-byte stores of y.
#include "combine_device.h"

namespace moeq {

__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ yp,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const int32_t* __restrict__ offsets, int k,
                                                      int E, int H,
                                                      const float* __restrict__ shared_z,
                                                      const uint16_t* residual, uint16_t* y) {
    const int nchunk = (H / 4 + 255) / 256;
    const int t = blockIdx.x / nchunk;
    const int h = ((blockIdx.x % nchunk) * 256 + threadIdx.x) * 4;
    if (h >= H) return;
    combine_cols(yp, pair_pos, offsets[E], t, h, k, H, shared_z, residual, y);
}

void launch_combine(const float* yp, const int32_t* pair_pos, const int32_t* offsets, int T, int k,
                    int E, int H, const float* shared_z, const uint16_t* residual, uint16_t* y,
                    hipStream_t stream) {
    const int nchunk = (H / 4 + 255) / 256;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T * nchunk), dim3(256), 0, stream, yp,
                       pair_pos, offsets, k, E, H, shared_z, residual, y);
}

// The shared expert's routing: every token to expert 0 (one slot), in token order, weight 1.
__global__ void __launch_bounds__(256) identity_routing_kernel(int T, int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_pair,
                                                               float* __restrict__ w) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < T) {
        sorted_pair[i] = i;
        w[i] = 1.0f;
    }
    if (i == 0) {
        offsets[0] = 0;
        offsets[1] = T;
    }
}

void launch_identity_routing(int T, int32_t* offsets, int32_t* sorted_pair, float* w,
                             hipStream_t stream) {
    hipLaunchKernelGGL(identity_routing_kernel, dim3((T + 255) / 256), dim3(256), 0, stream, T,
                       offsets, sorted_pair, w);
}

}  // namespace moeq
