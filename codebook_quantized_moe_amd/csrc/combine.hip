// Unpermute and combine: each token's k expert rows (gate weights already applied by the down
// projection) are summed in fixed slot order in fp32, then the optional shared-expert row and
// the optional residual are added, and the row is rounded to bf16 (README of
// GLM-5.2-EXL3-TR3v4-3.5bpw-MTP78, "Shared residual rotations": expert outputs are
// routing-weighted and summed back into the residual space; "Checkpoint layout update": one
// shared expert per layer beside the routed ones).
// One workgroup per (token, 1024-column chunk), flattened into one grid dimension; 16-byte loads
// of yp, 8-byte stores of y.
#include "moeq_device.h"

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
    const int valid = offsets[E];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    bool bad = false;
    // the k rows' loads go out back to back (no branch around a load: an invalid position
    // reads row 0 and only marks the result); yp is read once, hence non-temporal
    for (int j0 = 0; j0 < k; j0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int pos = j0 + j < k ? pair_pos[(size_t)t * k + j0 + j] : 0;
            bad |= j0 + j < k && pos >= valid;
            pos = pos < valid ? pos : 0;
            v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yp + (size_t)pos * H + h));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j0 + j < k) { acc.x += v[j][0]; acc.y += v[j][1]; acc.z += v[j][2]; acc.w += v[j][3]; }
    }
    if (shared_z) {
        const f32x4 v = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(shared_z + (size_t)t * H + h));
        acc.x += v[0]; acc.y += v[1]; acc.z += v[2]; acc.w += v[3];
    }
    if (residual) {
        const uint2 r = *reinterpret_cast<const uint2*>(residual + (size_t)t * H + h);
        acc.x += bf16_to_f32(r.x & 0xFFFFu); acc.y += bf16_to_f32(r.x >> 16);
        acc.z += bf16_to_f32(r.y & 0xFFFFu); acc.w += bf16_to_f32(r.y >> 16);
    }
    if (bad) acc = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                               __builtin_nanf(""));
    uint2 o;
    o.x = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
    o.y = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
    *reinterpret_cast<uint2*>(y + (size_t)t * H + h) = o;
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
