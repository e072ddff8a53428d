// Unpermute and combine of one token's 4 columns h .. h + 3: its k expert rows (gate weights
// already applied by the down projection) summed in fixed slot order in fp32, then the
// optional shared-expert row and the optional residual, rounded to bf16 (README of
// GLM-5.2-EXL3-TR3v4-3.5bpw-MTP78, "Shared residual rotations": expert outputs are
// routing-weighted and summed back into the residual space).
#pragma once

#include "moeq_device.h"

namespace moeq {

// valid: expert_offsets[E] (positions at or past it hold pairs with an invalid expert id,
// whose token becomes NaN)
__device__ inline void combine_cols(const float* __restrict__ yp,
                                    const int32_t* __restrict__ pair_pos, int valid, int t, int h,
                                    int k, int H, const float* __restrict__ shared_z,
                                    const uint16_t* residual, uint16_t* y) {
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

}  // namespace moeq
