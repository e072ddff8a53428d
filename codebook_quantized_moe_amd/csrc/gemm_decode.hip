// Grouped projections for few rows per expert (decode): the expert weights are the traffic.
//
// MFMA shape. v_mfma_f32_4x4x4_16b_bf16 runs 16 independent 4x4x4 products; lane 4b + q holds
// row q of block b's A (4 K values), column q of block b's B, and column q (rows 0..3) of
// block b's result. The 16 blocks are used as 16 slices of K of one 4-row x 4-column product
// and summed across lanes (permlane swaps, DPP rotations) when an item is complete. A tile
// therefore has M = 4 token rows (the size of an expert's share of a decode batch) instead of
// a 16-row operand that would be mostly padding.
//
// Memory path. On MI355X the vector-memory address path, not HBM, bounds a weight stream that
// is fetched with narrow or out-of-range loads: a wavefront instruction costs about the same
// whether it moves 64 bytes or 1 KiB. So the hot loop issues only full 16-byte, in-range
// loads of codes -- lane (b, q) reads 32 codes of weight row 4g + q at K 32b .. 32b + 31 of a
// 512-wide K-step, one instruction per column group g covering 4 rows x 256 contiguous bytes,
// with the non-temporal hint (each byte is read once) -- and everything else comes from LDS:
//   * the tile's activation rows and the scale bytes of the workgroup's 128 weight rows are
//     staged per 2048-wide K-chunk by the whole workgroup with 16-byte loads, double-buffered
//     (one barrier per chunk), and shared by its 8 wavefronts;
//   * the exact bf16 decode tables (one 16-byte entry per table and scale byte).
// The codes of the next K-step stay in flight per wavefront, across chunk and item boundaries.
//
// Work item = (tile of <= 4 sorted rows of one expert, block of 64 channels for gate|up or
// 128 output rows for down); a workgroup (8 wavefronts) takes one item at a time, wavefront w
// takes 16 weight rows of it over the whole K.
// gate|up ("Round 7" brief, decision 4): wavefront w decodes the gate rows and the up rows of
// the same 8 channels, so bf16(silu(g) * u) is formed in registers.
// down ("Round 7" brief, decision 6; README "What had to be fixed": router weighting in the
// down epilogue): writes topk_w[p] * (I . Wd) in fp32.
// The grid is persistent; expert row counts are read from expert_offsets on the device.
#include "combine_device.h"
#include "moeq_device.h"
#include "moeq_kernels.h"
#include "permute_device.h"
#include "route_device.h"

#include <algorithm>

namespace moeq {

constexpr int kTileRows = 4;
constexpr int kStepK = 512;                       // K per step: lane b covers 32 codes

// Shape of a decode launch: WAVES wavefronts per workgroup (16 weight rows each), K staged
// in chunks of CHUNK.
#define GATEUP_COLS(w) (8 * (w))
template <int WAVES, int CHUNK>
struct DecShape {
    static constexpr int kWaves = WAVES;
    static constexpr int kThreads = 64 * WAVES;
    static constexpr int kChunkK = CHUNK;
    static constexpr int kRowsPerWG = 16 * WAVES;                 // weight rows per item
    static constexpr int kChannelsPerWG = GATEUP_COLS(WAVES);   // gate|up channels per item
    static constexpr int kARowUnits = CHUNK / 8 + 1;              // 16-byte units per row (+1)
    static constexpr int kABufBytes = kTileRows * kARowUnits * 16;
    // a weight row's CHUNK / 32 scale bytes, staged from the 16-byte boundary below them
    static constexpr int kSRowBytes = CHUNK / 32 + 16;
    static constexpr int kSBufBytes = kRowsPerWG * kSRowBytes;
};

constexpr uint32_t kOutOfRange = 0x80000000u;

// s_waitcnt until at most n vector-memory loads are outstanding (loads return in order)
#define MOEQ_DEC_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))
// non-temporal: the weight streams are read once (a plain read kernel reaches ~4.9 TB/s
// with the default policy and ~6.8 TB/s with this hint on MI355X)
constexpr int kStreamPolicy = 2;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

template <int POLICY>
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
}

__device__ __forceinline__ f32x4 mfma4x4x4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                           f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, u32x2{a0, a1}),
                                                  __builtin_bit_cast(s16x4, u32x2{b0, b1}), c, 0,
                                                  0, 0);
}

// Per active expert (ascending ids), in LDS: its id, first sorted row, row count, decode
// table id and the prefix count of its kTileRows-row tiles. Everything the K loop needs about
// an item then comes from LDS: a vector-memory load inside the loop would have to wait for
// every code load issued before it (loads return in order) and drain the prefetch.
// The tiles of the few-rows kernels: at most 4096 rows (every expert adds at most one partial
// tile of 4): 1024 + 256.
constexpr int kMaxTiles = 1280;

struct ExpertMeta {
    int active[256];
    int tpre[257];
    int beg[256];
    int cnt[256];
    int tsel[256];
    uint16_t t2a[kMaxTiles];        // tile -> index of its active expert (when MAP)
    int n;
};

// What the first wavefront reads for the expert map: lane l takes experts 4 l .. 4 l + 3.
// The indexes are clamped into the arrays (offsets has E + 1 entries, E >= 1), so the loads
// need no branches and go out together; an expert e >= E gets zero rows.
struct MetaLoads {
    int beg[4], end[4], tsel[4];
};

__device__ __forceinline__ MetaLoads load_meta(const int32_t* offsets, const uint8_t* table_id,
                                               int E) {
    const int lane = threadIdx.x & 63;
    MetaLoads l;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = lane * 4 + j;
        l.beg[j] = offsets[min(e, E)];
        l.end[j] = offsets[min(e + 1, E)];
        l.tsel[j] = table_id[min(e, E - 1)];
    }
    return l;
}

// Fills m from the first wavefront's loads ml (all threads call it; ends with a barrier), and
// with MAP the tile -> expert map. Returns the count of active experts.
template <bool MAP>
__device__ inline int active_tiles(const MetaLoads& ml, ExpertMeta& m) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < 64) {
        int rows[4], beg[4], c = 0, nt = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            beg[j] = ml.beg[j];
            rows[j] = ml.end[j] - ml.beg[j];
            c += rows[j] > 0;
            nt += (rows[j] + kTileRows - 1) / kTileRows;
        }
        int ic = c, it = nt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int oc = __shfl_up(ic, off, 64), ot = __shfl_up(it, off, 64);
            if (lane >= off) { ic += oc; it += ot; }
        }
        int pos = ic - c, pre = it - nt;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (rows[j] > 0) {
                const int e = lane * 4 + j;
                m.active[pos] = e;
                m.tpre[pos] = pre;
                m.beg[pos] = beg[j];
                m.cnt[pos] = rows[j];
                m.tsel[pos] = ml.tsel[j];
                ++pos;
                pre += (rows[j] + kTileRows - 1) / kTileRows;
            }
        if (lane == 63) {
            m.n = ic;
            m.tpre[ic] = it;
        }
    }
    __syncthreads();
    if constexpr (MAP) {
        const int nact = m.n;
        for (int a = threadIdx.x; a < nact; a += blockDim.x) {
            const int t1 = min(m.tpre[a + 1], kMaxTiles);
            for (int t = m.tpre[a]; t < t1; ++t) m.t2a[t] = (uint16_t)a;
        }
        __syncthreads();
    }
    return m.n;
}

// Sums over the 16 K-slices of an MFMA result (lane bits 2..5 of lane 4 b + q).
// split_bit5(x, y): lanes with bit 5 clear get x summed over bit 5, the others y (the sum of
// the two outputs of v_permlane32_swap); split_bit4 likewise over bit 4 with v_permlane16_swap.
__device__ __forceinline__ float split_bit5(float x, float y) {
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
__device__ __forceinline__ float split_bit4(float x, float y) {
    const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
// every lane gets the sum over lane bits 2 and 3 (DPP row rotations by 4 and 8, fused into
// the adds)
__device__ __forceinline__ float sum_bits23(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
    return v;
}
__device__ __forceinline__ float sum_bits234(float v) { return sum_bits23(split_bit4(v, v)); }

struct Item {
    int e, cb, r0, rows, tsel;
};

template <bool MAP>
__device__ __forceinline__ Item locate(long item, int ncb, int nact, const ExpertMeta& m) {
    Item it;
    int lo = 0, tile;
    if constexpr (MAP) {
        // one LDS read: the map of active_tiles<true> (items < 2^31)
        const int idx = (int)item;
        tile = idx / ncb;
        it.cb = idx - tile * ncb;
        lo = __builtin_amdgcn_readfirstlane((int)m.t2a[tile]);
    } else {
        tile = (int)(item / ncb);
        it.cb = (int)(item % ncb);
        // last a < nact with tpre[a] <= tile: a fixed, unrolled search (no loop in the K loop)
#pragma unroll
        for (int step = 128; step >= 1; step >>= 1) {
            const int c = lo + step;
            if (c < nact && m.tpre[c] <= tile) lo = c;
        }
        lo = __builtin_amdgcn_readfirstlane(lo);
    }
    it.e = __builtin_amdgcn_readfirstlane(m.active[lo]);
    const int m0 = (tile - __builtin_amdgcn_readfirstlane(m.tpre[lo])) * kTileRows;
    it.r0 = __builtin_amdgcn_readfirstlane(m.beg[lo]) + m0;
    it.rows = min(kTileRows, __builtin_amdgcn_readfirstlane(m.cnt[lo]) - m0);
    it.tsel = __builtin_amdgcn_readfirstlane(m.tsel[lo]);
    return it;
}

// Weight row (within its matrix) of column group g, lane q, wavefront w; mat = 1 for up rows.
template <bool GATEUP, class S>
__device__ __forceinline__ int weight_row(int cb, int w, int g, int q, int* mat) {
    if (GATEUP) {
        *mat = g >> 1;
        return cb * S::kChannelsPerWG + w * 8 + (g & 1) * 4 + q;
    }
    *mat = 0;
    return cb * S::kRowsPerWG + w * 16 + g * 4 + q;
}

// An output element: a plain store, or (COH) a device-coherent one, which goes through the
// XCD's L2 to memory, so that workgroups on the other XCDs can read it in the same launch.
template <bool COH, class T>
__device__ __forceinline__ void put(T* p, T v) {
    if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *p = v;
}

// One projection over the whole persistent grid (every workgroup calls it; it returns when
// the workgroup's items are done). smem: the launch's dynamic LDS; meta: LDS for the item map.
// SALIGN (only when K is a multiple of the chunk, so every K-step lies inside K and every
// weight row's scale bytes start on a 16-byte boundary) stages 16 fewer scale bytes per row
// and checks no K bounds; the other form works for any K.
// COH: outputs by device-coherent stores (single launch). build: fill the decode tables
// (false when the launch has already filled them for these tables).
template <bool GATEUP, class S, bool SALIGN, bool COH = false>
__device__ __forceinline__ void decode_body(const SkinnyArgs& a, uint8_t* smem, ExpertMeta& meta,
                                            bool build = true) {
    constexpr int kChunkK = S::kChunkK, kRowsPerWG = S::kRowsPerWG;
    constexpr int kARowUnits = S::kARowUnits, kABufBytes = S::kABufBytes;
    constexpr int kSBufBytes = S::kSBufBytes, kSRowBytes = S::kSRowBytes;
    u32x4* tab = reinterpret_cast<u32x4*>(smem);
    uint8_t* abuf = smem + (size_t)a.tables.n * 256 * 16;
    uint8_t* sbuf = abuf + 2 * kABufBytes;
    // per sorted row: gate|up the token (x row), down the gate weight topk_w[pair]
    uint8_t* rowinfo = sbuf + 2 * kSBufBytes;
    uint16_t* row_tok = reinterpret_cast<uint16_t*>(rowinfo);
    float* row_w = reinterpret_cast<float*>(rowinfo);
    // the prologue's first loads go out before the table build, which hides their latency
    const int P = a.T * a.k;
    const bool has_row = (int)threadIdx.x < P;
    const int p0 = has_row ? a.sorted_pair[threadIdx.x] : 0;
    MetaLoads ml;
    if (threadIdx.x < 64) ml = load_meta(a.offsets, a.table_id, a.E);
    if (build) build_decode_tables(a.tables, tab);
    for (int r = threadIdx.x; r < P; r += blockDim.x) {
        const int p = r == (int)threadIdx.x ? p0 : a.sorted_pair[r];
        if (GATEUP) row_tok[r] = (uint16_t)(p / a.k);
        else row_w[r] = a.topk_w[p];
    }
    const int nact = active_tiles<SALIGN && !GATEUP>(ml, meta);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = lane >> 2, q = lane & 3;
    const int K = a.K, N = a.N;
    const int ncb = GATEUP ? (N + S::kChannelsPerWG - 1) / S::kChannelsPerWG
                           : (N + kRowsPerWG - 1) / kRowsPerWG;
    const long items = (long)__builtin_amdgcn_readfirstlane(meta.tpre[nact]) * ncb;
    // whole chunks of K-steps (steps past K load nothing in range and add zeros), so that
    // every chunk issues the same number of code loads after its staging DMA
    const int nsteps = (K + kChunkK - 1) / kChunkK * (kChunkK / kStepK);
    const long first = blockIdx.x, stride = gridDim.x;
    const long nmine = items > first ? (items - first + stride - 1) / stride : 0;
    const long total = nmine * nsteps;
    if (total == 0) return;                       // uniform per workgroup
    const uint32_t kb = (uint32_t)K / 2, ks = (uint32_t)K / 32;
    const uint32_t mc = (uint32_t)N * kb, ms = (uint32_t)N * ks;
    const __amdgpu_buffer_rsrc_t ract = make_rsrc(a.act, a.act_bytes);

    // ---------------- one item's sources ----------------
    // Items past the end (the "next" of the last item) are empty: every load falls out of
    // range and returns zeros, so the loop below needs no branches around its loads.
    struct Src {
        __amdgpu_buffer_rsrc_t c0, c1;            // gate (or down) and up codes of the expert
        uint32_t off[4];                          // this lane's code row per group (or none)
        int e, cb, r0, rows, tsel;
    };
    auto make_src = [&](long item) {
        Src sr;
        const bool valid = item < items;
        const Item it = locate<SALIGN && !GATEUP>(valid ? item : first, ncb, nact, meta);
        sr.e = it.e;
        sr.cb = it.cb;
        sr.r0 = it.r0;
        sr.rows = valid ? it.rows : 0;
        sr.tsel = it.tsel;
        sr.c0 = make_rsrc(a.codes0 + (size_t)it.e * mc, mc);
        sr.c1 = GATEUP ? make_rsrc(a.codes1 + (size_t)it.e * mc, mc) : sr.c0;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            int mat;
            const int row = weight_row<GATEUP, S>(it.cb, wave, g, q, &mat);
            sr.off[g] = (valid && row < N) ? (uint32_t)row * kb + (uint32_t)b * 16 : kOutOfRange;
        }
        return sr;
    };
    // codes of K-step st: lane (b, q) of group g reads 32 codes of row 4 g + q at K 32 b
    auto load_group = [&](const Src& sr, int st, int g) {
        const int kk = st * kStepK;
        // SALIGN (whole chunks): every step is inside K, and a row past N (kOutOfRange) stays
        // past the end of the buffer after adding kk / 2 < 2^30
        if constexpr (SALIGN) return bload16<kStreamPolicy>((GATEUP && g >= 2) ? sr.c1 : sr.c0, sr.off[g] + kk / 2);
        const bool ok = kk + b * 32 < K;
        const uint32_t off = (ok && sr.off[g] != kOutOfRange) ? sr.off[g] + kk / 2 : kOutOfRange;
        return bload16<kStreamPolicy>((GATEUP && g >= 2) ? sr.c1 : sr.c0, off);
    };
    auto load_step = [&](const Src& sr, int st, u32x4 (&c)[4]) {
#pragma unroll
        for (int g = 0; g < 4; ++g) c[g] = load_group(sr, st, g);
    };

    // ---------------- staging of activations and scales (per workgroup, per chunk) -------
    // Both go global -> LDS by LDS-DMA (16 bytes per lane, lane-contiguous), issued at the
    // start of the chunk before and waited for at its end:
    //   * activations: kTileRows rows x kARowUnits 16-byte units (the last unit of a row is
    //     padding, so that the 4 rows of an MFMA operand read sit in different banks);
    //     the intermediate is stored in pair-split K order; x (natural order) is put into it
    //     by the wavefront that staged it (split_own below), or comes split (single launch);
    //   * scales: row R of the item (gate|up: R = 64 mat + channel, so gate rows and up rows
    //     fill separate DMA loads) gets kSRow bytes from the 16-byte boundary at or below its
    //     first scale byte of the chunk; readers add the row's offset (row * K/32 mod 16, zero
    //     when SALIGN, which needs no extra 16 bytes per row). Bytes past a row's K are masked
    //     at read time.
    constexpr int kAUnits = kTileRows * kARowUnits;
    constexpr int kALoads = (kAUnits + 63) / 64;
    constexpr int kSRow = SALIGN ? kChunkK / 32 : kSRowBytes;
    constexpr int kSLoads = kRowsPerWG * kSRow / 1024;
    constexpr int kSUnitsPerRow = kSRow / 16;
    static_assert(kRowsPerWG * kSRow <= kSBufBytes && (kRowsPerWG / 2) * kSRow % 1024 == 0,
                  "scale staging: whole DMA loads, gate and up rows in separate loads");
    auto stage_dma = [&](const Src& sr, int chunk, int sbufi) {
        const int kc = chunk * kChunkK;
        uint8_t* ab = abuf + sbufi * kABufBytes;
        uint8_t* sbb = sbuf + sbufi * kSBufBytes;
        // Activation loads whose units all lie past the item's last real unit (the rows past
        // its row count, and that row's padding unit) are not issued: those rows only reach
        // outputs that are never written. An item past the end issues nothing.
        const int na =
            min(kALoads, ((sr.rows - 1) * kARowUnits + kChunkK / 8 + 63) / 64);
        const int nall = sr.rows > 0 ? na + kSLoads : 0;
        for (int i = wave; i < nall; i += S::kWaves) {
            if (i < na) {
                const int u = i * 64 + lane;
                const int row = u / kARowUnits, p = u % kARowUnits;
                uint32_t off = kOutOfRange;
                if (row < sr.rows && p < kChunkK / 8 && kc + 8 * p < K) {
                    const uint32_t src = GATEUP ? (uint32_t)row_tok[sr.r0 + row]
                                                : (uint32_t)(sr.r0 + row);
                    off = (src * (uint32_t)K + (uint32_t)(kc + 8 * p)) * 2u;
                }
                if (u < kAUnits)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ract, ab + i * 1024, 16, off, 0, 0, 0);
            } else {
                const int j = i - na;
                const int u = j * 64 + lane;
                const int R = u / kSUnitsPerRow, piece = u % kSUnitsPerRow;
                int wrow, mat;
                if (GATEUP) {
                    mat = R / (kRowsPerWG / 2);
                    wrow = sr.cb * S::kChannelsPerWG + R % (kRowsPerWG / 2);
                } else {
                    mat = 0;
                    wrow = sr.cb * kRowsPerWG + R;
                }
                const uint8_t* sbase = (mat ? a.scales1 : a.scales0) + (size_t)sr.e * ms;
                const __amdgpu_buffer_rsrc_t rs = make_rsrc(sbase, ms);
                const uint32_t first_b = (uint32_t)wrow * ks + (uint32_t)(kc / 32);
                const uint32_t off = (sr.rows > 0 && wrow < N)
                                         ? (first_b & ~15u) + 16u * (uint32_t)piece : kOutOfRange;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, sbb + j * 1024, 16, off, 0, 0,
                                                         kStreamPolicy);
            }
        }
    };

    // x in natural K order (gate|up from moeq_gateup_swiglu): each wavefront puts the
    // activation units its own staging loads wrote into pair-split order once they have landed
    // (its vmcnt wait), before the barrier that publishes the buffer to the other wavefronts.
    // The same units (and no others) as stage_dma's activation loads of this wavefront.
    const bool natural = GATEUP && a.act_natural != 0;
    auto split_own = [&](const Src& sr, int sbufi) {
        if constexpr (!GATEUP) return;
        if (!natural || sr.rows <= 0) return;
        const int na =
            min(kALoads, ((sr.rows - 1) * kARowUnits + kChunkK / 8 + 63) / 64);
        uint8_t* ab = abuf + sbufi * kABufBytes;
        for (int i = wave; i < na; i += S::kWaves) {
            const int u = i * 64 + lane;
            if (u < kAUnits) {
                u32x4* pu = reinterpret_cast<u32x4*>(ab + (size_t)u * 16);
                *pu = pair_split(*pu);
            }
        }
    };

    // ---------------- main loop ----------------
    // Per chunk of kSteps K-steps: the next chunk (of this item or the next one) is staged by
    // DMA into the other buffers; the codes of K-step s sit in one of two register slots (cA
    // for even steps, cB for odd ones), and as soon as group g of step s is decoded its
    // registers take the load of group g of step s + 2 (of this item or the next): about one
    // and a half K-steps of codes stay in flight per wavefront, with no register beyond the two
    // slots. After the chunk the DMA is waited for (the 4 kSteps code loads issued after it may
    // stay in flight) and one barrier switches the buffers.
    constexpr int kSteps = kChunkK / kStepK;
    static_assert(kSteps % 2 == 0 && kSteps >= 2, "even K-steps per chunk");
    const int nchunks = nsteps / kSteps;
    Src cur = make_src(first);
    Src nxt = make_src(first + stride);
    stage_dma(cur, 0, 0);
    u32x4 cA[4], cB[4];
    load_step(cur, 0, cA);
    load_step(cur, 1, cB);         // an item has at least kSteps >= 2 K-steps
    MOEQ_DEC_WAIT_VMCNT(8);        // the staging has landed; the 8 code loads may be in flight
    asm volatile("" ::: "memory");
    split_own(cur, 0);
    __syncthreads();
    int buf = 0;

    for (long n = 0; n < nmine; ++n) {
        const bool badtab = cur.tsel >= a.tables.n;
        const u32x4* mytab = tab + (badtab ? 0 : cur.tsel) * 256;
        int soff[4];
        f32x4 acc[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            int mat;
            const int wrow = weight_row<GATEUP, S>(cur.cb, wave, g, q, &mat);
            const int R = GATEUP ? mat * (kRowsPerWG / 2) + (wrow - cur.cb * S::kChannelsPerWG)
                                 : wrow - cur.cb * kRowsPerWG;
            soff[g] = SALIGN ? R * kSRow : R * kSRow + (int)(((uint32_t)wrow * ks) & 15u);
            acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // step kk / kStepK from slot c; group g's registers then load step rst of rs
        auto compute = [&](u32x4 (&c)[4], int kk, const Src& rs, int rst) {
            // activation operands: tile row q, K 32 b .. 32 b + 31 of the step (pair-split)
            const uint8_t* ap = abuf + buf * kABufBytes + q * kARowUnits * 16 +
                                ((kk % kChunkK) / 8 + b * 4) * 16;
            u32x4 A[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) A[j] = *reinterpret_cast<const u32x4*>(ap + 16 * j);
            const uint8_t* sp = sbuf + buf * kSBufBytes + (kk % kChunkK) / 32 + b;
            const bool kin = SALIGN || kk + 32 * b < K;
            // the four scale bytes, then their four table entries: two LDS round trips per
            // K-step instead of two per group
            uint32_t sc[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) sc[g] = kin ? (uint32_t)sp[soff[g]] : 0u;
            u32x4 t[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) t[g] = mytab[sc[g]];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32x4 w = decode8(c[g][j], t[g]);
                    acc[g] = mfma4x4x4(A[j][0], A[j][1], w[0], w[1], acc[g]);
                    acc[g] = mfma4x4x4(A[j][2], A[j][3], w[2], w[3], acc[g]);
                }
                c[g] = load_group(rs, rst, g);
            }
        };
        for (int ch = 0; ch < nchunks; ++ch) {
            const bool lastc = ch + 1 == nchunks;
            const Src& ns = lastc ? nxt : cur;     // source of the next chunk
            stage_dma(ns, lastc ? 0 : ch + 1, buf ^ 1);
#pragma unroll
            for (int j = 0; j < kSteps; ++j) {
                const int st = ch * kSteps + j;
                // step st + 2: in this item, or (last chunk, last two steps) step j + 2 - kSteps
                // of the next one
                const bool nx = lastc && j + 2 >= kSteps;
                compute((j & 1) ? cB : cA, st * kStepK, nx ? nxt : cur,
                        nx ? j + 2 - kSteps : st + 2);
            }
            MOEQ_DEC_WAIT_VMCNT(4 * kSteps);
            asm volatile("" ::: "memory");
            split_own(ns, buf ^ 1);
            __syncthreads();
            buf ^= 1;
        }

        // ---- item complete: sum the 16 K-slices (lane bits 2..5) of the item's rows (the
        // others are never written). The permlane swaps split the sums of two values between
        // the two halves of the lane bit they exchange, so each lane ends with the totals it
        // stores: gate|up, bit 5 picks h and the lane keeps gate and up of channel 4 h + q;
        // down, bits 5 and 4 pick the column group g. The other bits are summed by DPP. ----
        if (GATEUP) {
            uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
            const int h = lane >> 5;
            const int ch = cur.cb * S::kChannelsPerWG + wave * 8 + h * 4 + q;
            const int slot = (ch & ~7) | (((ch & 1) << 2) | ((ch & 7) >> 1));
            const bool st = (lane & 0x1C) == 0 && ch < N;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (r >= cur.rows) continue;          // uniform per wavefront
                const float gv = sum_bits234(split_bit5(acc[0][r], acc[1][r]));
                const float uv = sum_bits234(split_bit5(acc[2][r], acc[3][r]));
                if (st) {
                    const float v = badtab ? __builtin_nanf("") : silu_mul(gv, uv);
                    put<COH>(out + (size_t)(cur.r0 + r) * a.out_ld + slot,
                             (uint16_t)f32_to_bf16_rne(v));
                }
            }
        } else {
            float* out = reinterpret_cast<float*>(a.out);
            const int g = ((lane >> 5) << 1) | ((lane >> 4) & 1);
            const int col = cur.cb * kRowsPerWG + wave * 16 + g * 4 + q;
            const bool st = (lane & 0x0C) == 0 && col < N;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (r >= cur.rows) continue;          // uniform per wavefront
                const float v = sum_bits23(split_bit4(split_bit5(acc[0][r], acc[2][r]),
                                                      split_bit5(acc[1][r], acc[3][r])));
                if (st) {
                    const size_t row = (size_t)(cur.r0 + r);
                    put<COH>(out + row * a.out_ld + col,
                             badtab ? __builtin_nanf("") : row_w[row] * v);
                }
            }
        }
        cur = nxt;
        nxt = make_src(first + (n + 2) * stride);
    }
}

template <bool GATEUP, class S, bool SALIGN>
__global__ void __launch_bounds__(S::kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
decode_kernel(const SkinnyArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ ExpertMeta meta;
    decode_body<GATEUP, S, SALIGN>(a, smem, meta);
}

// scale rows of K/32 bytes all start on a 16-byte boundary
// whole chunks of K (which also puts every scale row on a 16-byte boundary)
template <class S>
static bool whole_chunks(const SkinnyArgs& a) { return a.K % S::kChunkK == 0; }

template <class S>
static void launch_shape(const SkinnyArgs& a, bool gateup, long items, int cus, hipStream_t stream) {
    const size_t lds = (size_t)a.tables.n * 256 * 16 + 2 * S::kABufBytes + 2 * S::kSBufBytes +
                       (size_t)a.T * a.k * (gateup ? 2 : 4);
    const int per_cu = 16 / S::kWaves;                    // 4 wavefronts per SIMD
    const long blocks = std::max(1L, std::min(items, (long)cus * per_cu));
    const bool al = whole_chunks<S>(a);
    if (gateup && al)
        hipLaunchKernelGGL((decode_kernel<true, S, true>), dim3(blocks), dim3(S::kThreads), lds,
                           stream, a);
    else if (gateup)
        hipLaunchKernelGGL((decode_kernel<true, S, false>), dim3(blocks), dim3(S::kThreads), lds,
                           stream, a);
    else if (al)
        hipLaunchKernelGGL((decode_kernel<false, S, true>), dim3(blocks), dim3(S::kThreads), lds,
                           stream, a);
    else
        hipLaunchKernelGGL((decode_kernel<false, S, false>), dim3(blocks), dim3(S::kThreads),
                           lds, stream, a);
}

int decode_tile_rows() { return kTileRows; }

// shape 0: 8 wavefronts, 2048-wide chunks; 2: 8 wavefronts, 1024; 4: 16 wavefronts, 2048
// (tuning alternatives; any other value selects shape 0)
void launch_decode(const SkinnyArgs& a, bool gateup, long tiles, int cus, int shape,
                   hipStream_t stream) {
    auto items = [&](int cols) { return tiles * ((a.N + cols - 1) / cols); };
    switch (shape) {
    case 2: launch_shape<DecShape<8, 1024>>(a, gateup, items(gateup ? 64 : 128), cus, stream); break;
    case 4: launch_shape<DecShape<16, 2048>>(a, gateup, items(gateup ? 128 : 256), cus, stream); break;
    default: launch_shape<DecShape<8, 2048>>(a, gateup, items(gateup ? 64 : 128), cus, stream); break;
    }
}

// ---------------------------------------------------------------------------------------------
// The whole decode layer in one cooperative launch: routing and permutation (workgroup 0, while
// the others fill their decode tables), gate|up, down and the combine over the whole grid. The
// grid is co-resident (a cooperative launch fails rather than run it otherwise).
//
// Coherence across the 8 XCDs (each has its own L2) without cache maintenance in the grid
// barriers: every value that one phase writes and a later phase reads on another XCD is written
// with device-coherent stores (the projections' outputs) and, at the time it is read, was never
// read in this launch before, so no L2 or L1 holds a stale copy of its line (the launch starts
// with clean caches, and every 128-byte line of the intermediate and of the expert outputs has
// one writing workgroup). A barrier then only needs each thread's stores to have completed
// before its workgroup arrives. The routing arrays are written with plain stores by workgroup 0
// alone, which writes its XCD's L2 back once before it raises the ready flag.
// Waits give up after about a second and record that in the barrier header, so a broken
// barrier ends the kernel instead of hanging it.
//
// Barrier header (ints): 0 arrivals, 1 failure flag, 2..11 the clock stamps, 12 routing ready.
// ---------------------------------------------------------------------------------------------
constexpr int kBarrierSpinLimit = 1 << 22;
constexpr int kBarReady = 12;

// thread 0 waits until *p >= target (bounded); the whole workgroup then continues
__device__ inline void wait_at_least(int* bar, int* p, int target) {
    if (threadIdx.x == 0) {
        int spins = 0;
        while (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins > kBarrierSpinLimit) {
                __hip_atomic_fetch_or(&bar[1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

// all workgroups: this workgroup's (device-coherent) stores are complete, then it arrives
__device__ inline void grid_barrier(int* bar, int target) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(&bar[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_at_least(bar, &bar[0], target);
}

template <class S, bool SALIGN>
__global__ void __launch_bounds__(S::kThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
decode_layer_kernel(const DecodeLayerArgs L) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ ExpertMeta meta;
    const int nwg = gridDim.x, tid = threadIdx.x;
    const int P = L.T * L.k;
    // workgroup 0 records when it starts and leaves each phase (64-bit constant-rate clock,
    // 100 MHz) in the barrier header: bar[2 + 2 i], i = 0..4
    auto stamp = [&](int i) {
        if (blockIdx.x == 0 && tid == 0)
            reinterpret_cast<unsigned long long*>(L.barrier)[1 + i] = __builtin_amdgcn_s_memrealtime();
    };
    stamp(0);
    // phase 1
    if (blockIdx.x == 0) {
        for (int t = tid >> 6; t < L.T; t += S::kWaves)
            route_token(L.logits, t, L.E, L.k, L.sigmoid != 0, L.ids, L.w);
        __syncthreads();
        permute_block<S::kWaves>(L.ids, P, L.E, L.offsets, L.sorted_pair, L.pair_pos);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");    // L2 write-back of this XCD
            __builtin_amdgcn_s_waitcnt(0);                        // ... completed
            __hip_atomic_store(&L.barrier[kBarReady], 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // the decode tables (the same for both projections) while workgroup 0 routes
    build_decode_tables(L.gu.tables, reinterpret_cast<u32x4*>(smem));
    wait_at_least(L.barrier, &L.barrier[kBarReady], 1);
    stamp(1);
    decode_body<true, S, SALIGN, true>(L.gu, smem, meta, false);
    grid_barrier(L.barrier, nwg);
    stamp(2);
    decode_body<false, S, SALIGN, true>(L.dn, smem, meta, false);
    grid_barrier(L.barrier, 2 * nwg);
    stamp(3);
    // phase 4: combine, 4 columns per thread
    const int quads = L.H / 4;
    const int valid = L.offsets[L.E];
    for (long u = (long)blockIdx.x * S::kThreads + tid; u < (long)L.T * quads;
         u += (long)nwg * S::kThreads) {
        const int t = (int)(u / quads), h = (int)(u % quads) * 4;
        combine_cols(L.yp, L.pair_pos, valid, t, h, L.k, L.H, nullptr, L.residual, L.y);
    }
    stamp(4);
}

__global__ void zero_barrier_kernel(int* bar) {
    if (threadIdx.x < 16) bar[threadIdx.x] = 0;
}

// Launch geometry of the fused kernel: dynamic LDS and the largest co-resident grid.
static size_t decode_layer_lds(const DecodeLayerArgs& L) {
    using S = DecShape<8, 2048>;
    return (size_t)L.gu.tables.n * 256 * 16 + 2 * S::kABufBytes + 2 * S::kSBufBytes +
           (size_t)L.T * L.k * 4;
}

template <bool SALIGN>
static int launch_layer(const DecodeLayerArgs& L, int cus, hipStream_t stream) {
    using S = DecShape<8, 2048>;
    const size_t lds = decode_layer_lds(L);
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_layer_kernel<S, SALIGN>,
                                                     S::kThreads, lds) != hipSuccess || per_cu < 1)
        return -1;
    const int blocks = cus * per_cu;
    hipLaunchKernelGGL(zero_barrier_kernel, dim3(1), dim3(64), 0, stream, L.barrier);
    DecodeLayerArgs arg = L;
    void* params[] = {&arg};
    if (hipLaunchCooperativeKernel(reinterpret_cast<const void*>(decode_layer_kernel<S, SALIGN>),
                                   dim3(blocks), dim3(S::kThreads), params, (unsigned)lds,
                                   stream) != hipSuccess)
        return -2;
    return blocks;
}

int launch_decode_layer(const DecodeLayerArgs& L, int cus, hipStream_t stream) {
    using S = DecShape<8, 2048>;
    return whole_chunks<S>(L.gu) && whole_chunks<S>(L.dn) ? launch_layer<true>(L, cus, stream)
                                                                : launch_layer<false>(L, cus, stream);
}

}  // namespace moeq
