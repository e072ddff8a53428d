// Top-k routing of one token by one wavefront ("Round 7" brief, Model geometry: top-8 of 256).
//
// Each lane holds up to 4 of the token's E <= 256 logits as 64-bit keys
// (totalOrder(logit) << 32 | ~expert): the maximum key is the largest logit, and among equal
// logits the lowest expert id. k rounds of a wave-wide max select the experts in order. The
// gate values are a softmax over the k selected logits, or (sigmoid gating) the selected
// logits' sigmoids renormalised to sum one; both in fp32 with a fixed reduction order.
#pragma once

#include "moeq_device.h"

namespace moeq {

__device__ __forceinline__ uint32_t total_order_key(float f) {
    const uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// One DPP step of a max reduction: each lane takes the larger of its key and the key that the
// DPP pattern CTRL brings from another lane of its row of 16.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > v ? o : v;
}

__device__ __forceinline__ uint64_t read_lane_u64(uint64_t v, int lane) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, lane);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// Wave-wide maximum of a 64-bit key, the same value in every lane: the maximum of each row of
// 16 lanes with DPP moves (swap neighbours, swap pairs, rotate the row by 4, then by 8), then
// the four row maxima through scalar registers. DPP steps are plain VALU operations, where a
// lane shuffle would go through the LDS crossbar with its longer latency.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = dpp_max_step<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v = dpp_max_step<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v = dpp_max_step<0x124>(v);   // row_ror 4
    v = dpp_max_step<0x128>(v);   // row_ror 8
    const uint64_t r0 = read_lane_u64(v, 0), r1 = read_lane_u64(v, 16);
    const uint64_t r2 = read_lane_u64(v, 32), r3 = read_lane_u64(v, 48);
    const uint64_t a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
    return a > b ? a : b;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Route token t (the whole wavefront calls it): ids[t*k + j], w[t*k + j] for j < k; the ids
// also into lds_ids[t*k + j] when it is given.
__device__ inline void route_token(const float* __restrict__ logits, int t, int E, int k,
                                   bool sigmoid, int32_t* __restrict__ ids,
                                   float* __restrict__ w, int32_t* lds_ids = nullptr) {
    const int lane = threadIdx.x & 63;
    const float* row = logits + (size_t)t * E;
    uint64_t key[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        // padding entries: key 0 with an id above every real expert, never chosen first
        key[j] = e < E ? ((uint64_t)total_order_key(row[e]) << 32) | (uint32_t)(~e)
                       : (uint64_t)(uint32_t)(~(256 + e));
    }
    // slot r (0 <= r < k <= 256) is kept by lane r % 64 in its register r / 64
    int my_id[4] = {0, 0, 0, 0};
    float my_val[4] = {0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < k; ++r) {
        uint64_t best = key[0];
#pragma unroll
        for (int j = 1; j < 4; ++j) best = key[j] > best ? key[j] : best;
        best = wave_max_u64(best);
        const int win = (int)(~(uint32_t)best);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (key[j] == best) key[j] = 0;   // taken (keys are unique: ids differ)
        if (lane == (r & 63)) {
            const uint32_t kb = (uint32_t)(best >> 32);
            const float v = __uint_as_float((kb & 0x80000000u) ? (kb & 0x7FFFFFFFu) : ~kb);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if ((r >> 6) == j) { my_id[j] = win; my_val[j] = v; }
        }
    }
    const float l0 = __shfl(my_val[0], 0, 64);   // slot 0 holds the largest logit
    float ex[4], part = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float l = my_val[j];
        float s;
        if (!sigmoid) {
            s = expf(l - l0);
        } else if (l0 < 0.0f) {
            // every selected logit is negative: sigmoid(l) = e^l / (1 + e^l); the common
            // factor e^l0 is taken out so no term underflows and slot 0 contributes >= 1/2
            s = expf(l - l0) / (1.0f + expf(l));
        } else if (l >= 0.0f) {
            s = 1.0f / (1.0f + expf(-l));
        } else {
            const float e = expf(l);
            s = e / (1.0f + e);
        }
        ex[j] = (64 * j + lane < k) ? s : 0.0f;
        part += ex[j];
    }
    const float sum = wave_sum_f32(part);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int slot = 64 * j + lane;
        if (slot < k) {
            ids[(size_t)t * k + slot] = my_id[j];
            w[(size_t)t * k + slot] = ex[j] / sum;
            if (lds_ids) lds_ids[t * k + slot] = my_id[j];
        }
    }
}

}  // namespace moeq
