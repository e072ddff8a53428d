// Stable counting sort of the T*k (token, slot) pairs by expert, in one workgroup of NW
// wavefronts, with no atomics on the order. Wavefront w owns one contiguous span
// of pairs and walks it 64 pairs at a time; within such a group, a pair's rank among the
// earlier pairs of its bucket comes from ballots over the 9 bits of the bucket (experts
// 0..E-1; bucket E collects ids outside [0, E)), and the group's first pair of each bucket
// (its leader) adds the bucket's count to the wavefront's running counter.
//   1. counting walk: per-wavefront bucket counts;
//   2. per bucket, exclusive scans over the wavefronts and then over the buckets give every
//      wavefront its first position in every bucket (and expert_offsets);
//   3. placing walk: the same groups again; position = running counter + rank.
// Positions therefore follow pair order within every bucket.
#pragma once

#include "moeq_device.h"

namespace moeq {

constexpr int kBuckets = 257;   // experts 0..255 and one bucket for invalid ids
constexpr int kBatch = 8;       // groups of 64 pairs per load batch

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

struct PairClass {
    int bucket;
    uint64_t same;    // lanes of this group in the same bucket (live lanes only)
    bool live;
};

__device__ __forceinline__ PairClass classify(int e, bool live, int E) {
    PairClass c;
    c.live = live;
    c.bucket = live ? ((e >= 0 && e < E) ? e : E) : 0;
    uint64_t same = __ballot(live);
#pragma unroll
    for (int bit = 0; bit < 9; ++bit) {
        const uint64_t m = __ballot((c.bucket >> bit) & 1);
        same &= ((c.bucket >> bit) & 1) ? m : ~m;
    }
    c.same = same;
    return c;
}

// What permute_range does with the pairs [pb0, pe0) (every thread of the workgroup calls it):
//   kPermFull:  the whole permutation (the range is all pairs); writes expert_offsets;
//   kPermCount: only the range's per-bucket counts, into counts_out[0..E];
//   kPermPlace: the range's pairs placed from the first positions offsets[e] + base_in[e] it
//               has in every bucket (base_in may lie in pair_pos inside the range: it is read
//               first).
constexpr int kPermFull = 0, kPermCount = 1, kPermPlace = 2;

template <int NW, int MODE>
__device__ inline void permute_range(const int32_t* __restrict__ ids, int pb0, int pe0, int E,
                                     int32_t* __restrict__ offsets,
                                     int32_t* __restrict__ sorted_pair,
                                     int32_t* __restrict__ pair_pos,
                                     int32_t* __restrict__ counts_out, const int32_t* base_in) {
    __shared__ int wcnt[NW][kBuckets];   // counts, then running positions
    __shared__ int base[kBuckets];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t lanes_below = (1ull << lane) - 1ull;

    for (int i = tid; i < NW * kBuckets; i += (64 * NW)) (&wcnt[0][0])[i] = 0;
    __syncthreads();

    // this wavefront's span of the range (a multiple of 64 long, except at the range's end)
    const int n = pe0 - pb0;
    const int span = ((n + 64 * NW - 1) / (64 * NW)) * 64;
    const int pb = pb0 + wave * span;
    const int pe = min(pe0, pb + span);

    // the ids of kBatch groups are loaded before the first of them is classified (one memory
    // round trip per batch instead of one per group)
    int idv[kBatch];
    auto load_batch = [&](int p0) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int p = p0 + 64 * j + lane;
            idv[j] = p < pe ? ids[p] : 0;
        }
    };

    for (int p0 = pb; p0 < pe; p0 += 64 * kBatch) {
        load_batch(p0);
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int p = p0 + 64 * j + lane;
            const PairClass c = classify(idv[j], p < pe, E);
            if (c.live && __popcll(c.same & lanes_below) == 0)
                wcnt[wave][c.bucket] += __popcll(c.same);
        }
    }
    __syncthreads();

    // per bucket: exclusive scan over the wavefronts (in place), total into base
    for (int b = tid; b <= E; b += (64 * NW)) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int c = wcnt[w][b];
            wcnt[w][b] = run;
            run += c;
        }
        if (MODE == kPermCount) counts_out[b] = run;
        else if (MODE == kPermPlace) base[b] = offsets[b] + base_in[b];
        else base[b] = run;
    }
    if (MODE == kPermCount) return;
    __syncthreads();

    // exclusive scan over buckets 0..E (E + 1 <= 257 entries): wave 0, 5 entries per lane
    if (MODE == kPermFull && wave == 0) {
        int local[5];
        int s = 0;
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int b = lane * 5 + j;
            local[j] = b <= E ? base[b] : 0;
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

    for (int p0 = pb; p0 < pe; p0 += 64 * kBatch) {
        load_batch(p0);
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int p = p0 + 64 * j + lane;
            const PairClass c = classify(idv[j], p < pe, E);
            const int rank = __popcll(c.same & lanes_below);
            if (c.live) {
                const int pos = base[c.bucket] + wcnt[wave][c.bucket] + rank;
                sorted_pair[pos] = p;
                pair_pos[p] = pos;
            }
            // every lane has read its running position before the leaders advance them
            if (c.live && rank == 0) wcnt[wave][c.bucket] += __popcll(c.same);
        }
    }
}

// The whole permutation of P <= 64 pairs by one wavefront (all its lanes call it; lane p
// holds the expert id e of pair p, any value for p >= P). A pair's position is the number of
// pairs in lower buckets plus the number of earlier pairs in its own bucket; both sets come
// from the 9 ballots of the bucket bits, taken from the most significant bit down (a lane that
// differs from this one first at bit j is in a lower bucket when its bit j is 0). The buckets
// in sorted order go to LDS, and expert_offsets[x] (x = 0..E) is the count of them below x, a
// lower-bound search. No barrier: the wavefront's LDS operations complete in order.
__device__ inline void permute_wave(int e, int P, int E, int32_t* __restrict__ offsets,
                                    int32_t* __restrict__ sorted_pair,
                                    int32_t* __restrict__ pair_pos) {
    __shared__ int sb[64];
    const int lane = threadIdx.x & 63;
    const bool live = lane < P;
    const int bucket = (e >= 0 && e < E) ? e : E;
    uint64_t eq = __ballot(live), lt = 0;
#pragma unroll
    for (int bit = 8; bit >= 0; --bit) {
        const bool one = (bucket >> bit) & 1;
        const uint64_t m = __ballot(live && one);
        if (one) {
            lt |= eq & ~m;
            eq &= m;
        } else {
            eq &= ~m;
        }
    }
    const int pos = __popcll(lt) + __popcll(eq & ((1ull << lane) - 1ull));
    if (live) {
        sorted_pair[pos] = lane;
        pair_pos[lane] = pos;
        sb[pos] = bucket;
    }
    // lanes read buckets other lanes wrote: one wavefront, whose LDS accesses complete in
    // order; the barrier keeps the compiler from moving the reads above the writes
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        const int x = lane + 64 * j;
        if (x <= E) {
            int lo = 0;
#pragma unroll
            for (int step = 64; step >= 1; step >>= 1)
                if (lo + step <= P && sb[lo + step - 1] < x) lo += step;
            offsets[x] = lo;
        }
    }
}

// The whole permutation, by one workgroup of NW wavefronts (every thread calls it).
template <int NW>
__device__ inline void permute_block(const int32_t* __restrict__ ids, int P, int E,
                                     int32_t* __restrict__ offsets,
                                     int32_t* __restrict__ sorted_pair,
                                     int32_t* __restrict__ pair_pos) {
    permute_range<NW, kPermFull>(ids, 0, P, E, offsets, sorted_pair, pair_pos, nullptr, nullptr);
}

}  // namespace moeq
