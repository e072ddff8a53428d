// Stable counting sort of the (token, slot) pairs by expert (the walks are permute_range):
// up to 64 pairs one wavefront (permute_wave); below 4096 pairs one workgroup of 16
// wavefronts; from 4096 pairs three launches over blocks of pairs (below); and, for few tokens,
// routing followed by the permutation in one workgroup.
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

// P <= 64 pairs: one wavefront
__global__ void __launch_bounds__(64) permute_wave_kernel(const int32_t* __restrict__ ids, int P,
                                                          int E, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pair,
                                                          int32_t* __restrict__ pair_pos) {
    const int lane = threadIdx.x;
    permute_wave(lane < P ? ids[lane] : 0, P, E, offsets, sorted_pair, pair_pos);
}

// Routing and permutation in one workgroup of 16 wavefronts (few tokens: one launch instead
// of two): wavefront w routes tokens w, w + 16, ...; then the permutation of their pairs.
__global__ void __launch_bounds__(64 * kPermWaves) route_permute_kernel(
    const float* __restrict__ logits, int T, int E, int k, int sigmoid, int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos) {
    const int P = T * k;
    if (P <= 64) {
        // the ids stay in LDS for the one-wavefront permutation
        __shared__ int32_t sid[64];
        for (int t = threadIdx.x >> 6; t < T; t += kPermWaves)
            route_token(logits, t, E, k, sigmoid != 0, ids, w, sid);
        __syncthreads();
        if (threadIdx.x < 64)
            permute_wave(threadIdx.x < P ? sid[threadIdx.x] : 0, P, E, offsets, sorted_pair,
                         pair_pos);
        return;
    }
    for (int t = threadIdx.x >> 6; t < T; t += kPermWaves)
        route_token(logits, t, E, k, sigmoid != 0, ids, w);
    __syncthreads();
    permute_block<kPermWaves>(ids, P, E, offsets, sorted_pair, pair_pos);
}

void launch_route_permute(const float* logits, int T, int E, int k, bool sigmoid, int32_t* ids,
                          float* w, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                          hipStream_t stream) {
    hipLaunchKernelGGL(route_permute_kernel, dim3(1), dim3(64 * kPermWaves), 0, stream, logits, T,
                       E, k, sigmoid ? 1 : 0, ids, w, offsets, sorted_pair, pair_pos);
}

// Many pairs: three launches over blocks of kPermChunk pairs (the last block takes the rest,
// so every block holds at least kPermChunk >= 257 pairs). The outputs double as scratch:
//   1. count: block b's per-bucket counts into sorted_pair[257 b ..];
//   2. scan (one workgroup): per bucket, exclusive sums over the blocks into
//      pair_pos[kPermChunk b ..] (inside block b's own pairs), then over the buckets
//      (expert_offsets);
//   3. place: block b reads its first positions (expert_offsets + its block sums), then places
//      its pairs (pair_pos of its own pairs, sorted_pair anywhere: the counts are no longer
//      needed).
// Within every bucket the blocks are in order and each block keeps pair order: the result is
// the single-workgroup permutation's.
constexpr int kPermChunk = 1024;

__device__ __forceinline__ void chunk_range(int b, int nb, int P, int* pb, int* pe) {
    *pb = b * kPermChunk;
    *pe = b + 1 == nb ? P : (b + 1) * kPermChunk;
}

__global__ void __launch_bounds__(64 * kPermWaves) permute_count_kernel(
    const int32_t* __restrict__ ids, int P, int E, int32_t* __restrict__ counts) {
    int pb, pe;
    chunk_range(blockIdx.x, gridDim.x, P, &pb, &pe);
    permute_range<kPermWaves, kPermCount>(ids, pb, pe, E, nullptr, nullptr, nullptr,
                                          counts + (size_t)blockIdx.x * kBuckets, nullptr);
}

__global__ void __launch_bounds__(1024) permute_scan_kernel(const int32_t* __restrict__ counts,
                                                            int nb, int E,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ bases) {
    __shared__ int tot[kBuckets];
    const int t = threadIdx.x, lane = t & 63;
    constexpr int kU = 16;                               // loads in flight per thread
    if (t <= E) {
        int run = 0;
        for (int b0 = 0; b0 < nb; b0 += kU) {
            int c[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u)
                c[u] = b0 + u < nb ? counts[(size_t)(b0 + u) * kBuckets + t] : 0;
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (b0 + u < nb) {
                    bases[(size_t)(b0 + u) * kPermChunk + t] = run;
                    run += c[u];
                }
        }
        tot[t] = run;
    }
    __syncthreads();
    if (t < 64) {
        int local[5];
        int s = 0;
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int b = lane * 5 + j;
            local[j] = b <= E ? tot[b] : 0;
            s += local[j];
        }
        const int incl = wave_inclusive_scan(s);
        int run = incl - s;
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int b = lane * 5 + j;
            if (b <= E) offsets[b] = run;
            run += local[j];
        }
    }
}

__global__ void __launch_bounds__(64 * kPermWaves) permute_place_kernel(
    const int32_t* __restrict__ ids, int P, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
    int pb, pe;
    chunk_range(blockIdx.x, gridDim.x, P, &pb, &pe);
    permute_range<kPermWaves, kPermPlace>(ids, pb, pe, E, offsets, sorted_pair, pair_pos, nullptr,
                                          pair_pos + (size_t)blockIdx.x * kPermChunk);
}

void launch_permute(const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pair,
                    int32_t* pair_pos, hipStream_t stream) {
    if (P <= 64) {
        hipLaunchKernelGGL(permute_wave_kernel, dim3(1), dim3(64), 0, stream, ids, P, E, offsets,
                           sorted_pair, pair_pos);
        return;
    }
    if (P < 4 * kPermChunk) {
        hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(64 * kPermWaves), 0, stream, ids, P, E,
                           offsets, sorted_pair, pair_pos);
        return;
    }
    const int nb = P / kPermChunk;
    hipLaunchKernelGGL(permute_count_kernel, dim3(nb), dim3(64 * kPermWaves), 0, stream, ids, P,
                       E, sorted_pair);
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, stream, sorted_pair, nb, E,
                       offsets, pair_pos);
    hipLaunchKernelGGL(permute_place_kernel, dim3(nb), dim3(64 * kPermWaves), 0, stream, ids, P,
                       E, offsets, sorted_pair, pair_pos);
}

}  // namespace moeq
