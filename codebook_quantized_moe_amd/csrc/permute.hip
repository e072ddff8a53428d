// Stable counting sort of the T*k (token, slot) pairs by expert, in one workgroup of 1024
// threads (16 wavefronts), with no atomics on the order:
//   1. expert histogram (LDS integer atomics: the counts do not depend on their order);
//   2. wavefront prefix scan of the counts -> expert_offsets (bucket E collects invalid ids);
//   3. pairs in chunks of 1024: the rank of a pair among the earlier same-expert pairs of its
//      wavefront comes from ballots over the 9 bits of its bucket; a scan over the 16
//      wavefronts per bucket gives each wavefront's starting position; positions then follow
//      pair order within every bucket.
#include "moeq_device.h"

namespace moeq {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kBuckets = 257;   // experts 0..255 and one bucket for invalid ids

// inclusive scan of one value per lane across a wavefront
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    return v;
}

__global__ void __launch_bounds__(kPermThreads) permute_kernel(const int32_t* __restrict__ ids,
                                                               int P, int E,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_pair,
                                                               int32_t* __restrict__ pair_pos) {
    __shared__ int cnt[kBuckets];
    __shared__ int base[kBuckets];
    __shared__ int whist[kPermWaves][kBuckets];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int b = tid; b < kBuckets; b += kPermThreads) cnt[b] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += kPermThreads) {
        const int e = ids[p];
        atomicAdd(&cnt[(e >= 0 && e < E) ? e : E], 1);
    }
    __syncthreads();

    // exclusive scan over buckets 0..E (E + 1 <= 257 entries): wave 0, 5 entries per lane
    if (wave == 0) {
        int local[5];
        int s = 0;
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int b = lane * 5 + j;
            local[j] = b <= E ? cnt[b] : 0;
            s += local[j];
        }
        const int incl = wave_inclusive_scan(s);
        int run = incl - s;
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int b = lane * 5 + j;
            if (b <= E) {
                base[b] = run;
                offsets[b] = run;           // offsets[E] = number of valid pairs
            }
            run += local[j];
        }
    }
    __syncthreads();

    const uint64_t lanes_below = (1ull << lane) - 1ull;
    for (int p0 = 0; p0 < P; p0 += kPermThreads) {
        for (int i = tid; i < kPermWaves * kBuckets; i += kPermThreads)
            (&whist[0][0])[i] = 0;
        const int p = p0 + tid;
        const bool live = p < P;
        int bucket = 0;
        if (live) {
            const int e = ids[p];
            bucket = (e >= 0 && e < E) ? e : E;
        }
        uint64_t same = __ballot(live);
#pragma unroll
        for (int bit = 0; bit < 9; ++bit) {
            const uint64_t m = __ballot((bucket >> bit) & 1);
            same &= ((bucket >> bit) & 1) ? m : ~m;
        }
        const int rank = __popcll(same & lanes_below);
        __syncthreads();   // whist cleared
        if (live && rank == 0) whist[wave][bucket] = __popcll(same);
        __syncthreads();
        for (int b = tid; b <= E; b += kPermThreads) {
            int run = base[b];
#pragma unroll
            for (int w = 0; w < kPermWaves; ++w) {
                const int c = whist[w][b];
                whist[w][b] = run;
                run += c;
            }
            base[b] = run;
        }
        __syncthreads();
        if (live) {
            const int pos = whist[wave][bucket] + rank;
            sorted_pair[pos] = p;
            pair_pos[p] = pos;
        }
        __syncthreads();   // before the next chunk clears whist
    }
}

void launch_permute(const int32_t* ids, int P, int E, int32_t* offsets, int32_t* sorted_pair,
                    int32_t* pair_pos, hipStream_t stream) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, stream, ids, P, E, offsets,
                       sorted_pair, pair_pos);
}

}  // namespace moeq
