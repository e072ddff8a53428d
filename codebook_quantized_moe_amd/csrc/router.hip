// Router logits: logits[T, E] = x[T, H] . Wr[E, H]^T over bf16 values with fp32 accumulation
// (GLM-5.2-EXL3-DENSE6-MTP78 model card, "Quant recipe": the router is kept in BF16; Round 7
// brief, "Target pipeline": a layer's routing is the router applied to its activations).
//
// Many tokens: an LDS-tiled bf16 GEMM. A workgroup of 4 wavefronts computes 64 tokens x 128
// experts, K in steps of 64: each thread keeps the 16-byte chunks of the next six steps in flight
// in registers while the current step is multiplied out of LDS (rows padded to 72 bf16, so the
// 16-byte reads of 8 consecutive rows hit disjoint banks), and a wavefront owns 32 tokens x
// 64 experts (two v_mfma_f32_32x32x16_bf16 tiles sharing the token operand). Steps past H / 64
// read zeros, so the loop runs whole groups of six.
// Few tokens (decode): see the second kernel below.
// In both, rows past T or E read zeros (out-of-range buffer loads), and workgroups are numbered
// so that the expert tiles of one token tile run on one XCD (workgroup b runs on XCD b % 8):
// that XCD's L2 serves the token rows to all of them, and every XCD keeps its own copy of the
// router weight (E * H * 2 bytes, 3 MiB for 256 x 6144).
#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

typedef float f32x16r __attribute__((ext_vector_type(16)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t r_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

constexpr int kTM = 64, kTN = 128, kTK = 64, kLdsRow = kTK + 8;
constexpr int kSets = 6;   // register sets of the load pipeline (even: steps alternate LDS buffers)

__device__ __forceinline__ int xcd_tile(int b, int n) {
    // tile q = (b % 8) * (n / 8) + b / 8 when the n workgroups split evenly over the 8 XCDs
    return (n % 8 == 0) ? (b % 8) * (n / 8) + b / 8 : b;
}

__global__ void __launch_bounds__(256) router_logits_tiled_kernel(const uint16_t* __restrict__ x,
                                                                  int T, int H,
                                                                  const uint16_t* __restrict__ wr,
                                                                  int E,
                                                                  float* __restrict__ logits) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kTM * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kTN * kLdsRow];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cl = lane & 31, h = lane >> 5;
    const int q = xcd_tile(blockIdx.x, gridDim.x);
    const int ne = (E + kTN - 1) / kTN;
    const int t0 = (q / ne) * kTM, e0 = (q % ne) * kTN;
    const __amdgpu_buffer_rsrc_t rx = r_rsrc(x, (uint32_t)T * H * 2);
    const __amdgpu_buffer_rsrc_t rw = r_rsrc(wr, (uint32_t)E * H * 2);
    const uint32_t kOut = 0x80000000u;
    const int ns = H / kTK;
    // chunk c = tid + 256 j of a step: row c / 8, 16 bytes at column 8 (c % 8)
    uint32_t ga[2], gb[4];
    int la[2], lb[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int c = tid + 256 * j, r = c >> 3, k8 = (c & 7) * 8;
        ga[j] = t0 + r < T ? ((uint32_t)(t0 + r) * H + k8) * 2u : kOut;
        la[j] = r * kLdsRow + k8;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = tid + 256 * j, r = c >> 3, k8 = (c & 7) * 8;
        gb[j] = e0 + r < E ? ((uint32_t)(e0 + r) * H + k8) * 2u : kOut;
        lb[j] = r * kLdsRow + k8;
    }
    auto gload = [&](int st, u32x4* a, u32x4* bb) {
        const bool in = st < ns;
        const uint32_t d = 2u * kTK * st;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            a[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rx, in ? ga[j] + d : kOut, 0, 0));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bb[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rw, in ? gb[j] + d : kOut, 0, 0));
    };
    auto lstore = [&](int buf, const u32x4* a, const u32x4* bb) {
#pragma unroll
        for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4*>(&As[buf][la[j]]) = a[j];
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(&Bs[buf][lb[j]]) = bb[j];
    };
    // wavefront tile: tokens 32 (wave & 1) .. + 32, experts 64 (wave >> 1) .. + 64
    const int ar = (32 * (wave & 1) + cl) * kLdsRow + 8 * h;
    const int br = (64 * (wave >> 1) + cl) * kLdsRow + 8 * h;
    f32x16r acc0, acc1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { acc0[r] = 0.f; acc1[r] = 0.f; }
    auto compute = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < kTK / 16; ++ks) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(&As[buf][ar + 16 * ks]);
            const u32x4 b0 = *reinterpret_cast<const u32x4*>(&Bs[buf][br + 16 * ks]);
            const u32x4 b1 = *reinterpret_cast<const u32x4*>(&Bs[buf][br + 32 * kLdsRow + 16 * ks]);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                           __builtin_bit_cast(bf16x8, b0), acc0,
                                                           0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                           __builtin_bit_cast(bf16x8, b1), acc1,
                                                           0, 0, 0);
        }
    };
    // step j travels in register set j % kSets: loaded kSets steps before it is multiplied,
    // stored to LDS buffer j % 2 at the end of step j - 1. The loads are pinned ahead of each
    // step's MFMAs (the scheduler would sink them below).
    u32x4 ra[kSets][2], rb[kSets][4];
#pragma unroll
    for (int i = 0; i < kSets; ++i) gload(i, ra[i], rb[i]);
    lstore(0, ra[0], rb[0]);
    __syncthreads();
    for (int st = 0; st < ns; st += kSets) {
#pragma unroll
        for (int i = 0; i < kSets; ++i) {
            gload(st + i + kSets, ra[i], rb[i]);
            __builtin_amdgcn_sched_barrier(0);
            compute(i & 1);
            lstore((i + 1) & 1, ra[(i + 1) % kSets], rb[(i + 1) % kSets]);
            __syncthreads();
        }
    }
    // lane holds experts e0 + 64 (wave >> 1) + cl (acc0) and + 32 (acc1), tokens
    // t0 + 32 (wave & 1) + 8 (r / 4) + 4 h + r % 4
    const int e = e0 + 64 * (wave >> 1) + cl;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int t = t0 + 32 * (wave & 1) + 8 * (r >> 2) + 4 * h + (r & 3);
        if (t < T) {
            if (e < E) logits[(size_t)t * E + e] = acc0[r];
            if (e + 32 < E) logits[(size_t)t * E + e + 32] = acc1[r];
        }
    }
}

// Few tokens (decode): the time is the latency of reading the router weight, so the tiles are
// 16 tokens x 16 experts (v_mfma_f32_16x16x32_bf16: lane l holds token row / router row l % 16,
// K 8 (l / 16) .. + 7 of each 32-wide step; result register r of lane l is token 4 (l / 16) + r,
// expert l % 16), E / 16 workgroups of NW wavefronts split K NW ways, and each wavefront issues
// the loads of 12 steps (384 K) before the first MFMA, so one memory round trip covers them.
typedef float f32x4r __attribute__((ext_vector_type(4)));
constexpr int kSkinnySteps = 12;

template <int NW>
__global__ void __launch_bounds__(64 * NW) router_logits_skinny_kernel(
    const uint16_t* __restrict__ x, int T, int H, const uint16_t* __restrict__ wr, int E,
    float* __restrict__ logits) {
    __shared__ f32x4r part[NW - 1][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cl = lane & 15, g = lane >> 4;
    const int q = xcd_tile(blockIdx.x, gridDim.x);
    const int ne = (E + 15) / 16;
    const int t0 = (q / ne) * 16, e0 = (q % ne) * 16;
    const __amdgpu_buffer_rsrc_t rx = r_rsrc(x, (uint32_t)T * H * 2);
    const __amdgpu_buffer_rsrc_t rw = r_rsrc(wr, (uint32_t)E * H * 2);
    const uint32_t kOut = 0x80000000u;
    const int kw = H / NW;                                  // K of a wavefront (multiple of 32)
    const int kbeg = wave * kw;
    const uint32_t ax = t0 + cl < T ? ((uint32_t)(t0 + cl) * H + kbeg + 8 * g) * 2u : kOut;
    const uint32_t bw = e0 + cl < E ? ((uint32_t)(e0 + cl) * H + kbeg + 8 * g) * 2u : kOut;
    f32x4r acc = {0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb < kw; kb += 32 * kSkinnySteps) {
        u32x4 a[kSkinnySteps], bb[kSkinnySteps];
#pragma unroll
        for (int s = 0; s < kSkinnySteps; ++s) {
            const int kk = kb + 32 * s;
            const bool in = kk < kw;
            a[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rx, in ? ax + 2u * kk : kOut, 0, 0));
            bb[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rw, in ? bw + 2u * kk : kOut, 0, 0));
        }
        __builtin_amdgcn_sched_barrier(0);     // every load of the block is issued first
#pragma unroll
        for (int s = 0; s < kSkinnySteps; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                          __builtin_bit_cast(bf16x8, bb[s]),
                                                          acc, 0, 0, 0);
    }
    if (wave > 0) part[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
#pragma unroll 1
    for (int w = 0; w < NW - 1; ++w) {
        const f32x4r p = part[w][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] += p[r];
    }
    const int e = e0 + cl;
    if (e >= E) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = t0 + 4 * g + r;
        if (t < T) logits[(size_t)t * E + e] = acc[r];
    }
}

// Token counts up to this take the few-tokens kernel.
constexpr int kSkinnyMaxT = 64;

void launch_router_logits(const uint16_t* x, int T, int H, const uint16_t* wr, int E,
                          float* logits, hipStream_t stream) {
    if (T <= kSkinnyMaxT) {
        const dim3 grid(((T + 15) / 16) * ((E + 15) / 16));
        if (H % 512 == 0)
            hipLaunchKernelGGL(router_logits_skinny_kernel<16>, grid, dim3(1024), 0, stream, x, T,
                               H, wr, E, logits);
        else if (H % 128 == 0)
            hipLaunchKernelGGL(router_logits_skinny_kernel<4>, grid, dim3(256), 0, stream, x, T, H,
                               wr, E, logits);
        else
            hipLaunchKernelGGL(router_logits_skinny_kernel<2>, grid, dim3(128), 0, stream, x, T, H,
                               wr, E, logits);
        return;
    }
    const dim3 grid(((T + kTM - 1) / kTM) * ((E + kTN - 1) / kTN));
    hipLaunchKernelGGL(router_logits_tiled_kernel, grid, dim3(256), 0, stream, x, T, H, wr, E,
                       logits);
}

}  // namespace moeq
