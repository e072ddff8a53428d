// Grouped projections for many rows per expert (prefill): the MFMA work dominates.
//
// Tiles. A workgroup of 4 wavefronts computes a 128 (sorted rows of one expert) x 128 (weight
// rows) tile over the whole K, in stages of 64 along K, with v_mfma_f32_32x32x16_bf16 (fp32
// accumulation); the wavefronts form a 2 x 2 grid of 64 x 64 sub-tiles (2 x 2 MFMA tiles each).
// Every stage, the workgroup
//   * gathers the tile's 128 activation rows (x rows through sorted_pair for gate|up, the
//     intermediate's rows for down) with 16-byte loads and stores them to LDS -- x is put into
//     the decode's pair-split K order on the way;
//   * loads the 128 x 64 codes (16 bytes per thread, non-temporal) and their scale bytes and
//     decodes them (decode8: exact LDS tables + byte permutes) into a bf16 LDS tile;
// both tiles are double-buffered: the global loads of stage s + 1 are in flight while stage s
// runs its 16 MFMAs per wavefront, then stage s + 1 is decoded into the other buffer and one
// barrier closes the stage. LDS rows are 128 bytes with the 16-byte units XOR-swizzled by
// (row / 2) % 8, so the 32 rows read by an MFMA operand load hit distinct banks.
//
// gate|up ("Round 7" brief, decision 4): the 128 weight rows of a tile are 64 channels in
// blocks of 32 -- gate c0..c0+31, up c0..c0+31, gate c0+32.., up c0+32.. -- so a wavefront's two
// N sub-tiles are the gate and up rows of the same 32 channels and bf16(silu(g) * u) is formed
// in registers. down ("Round 7" brief, decision 6; README "What had to be fixed"): the epilogue
// writes topk_w[p] * (I . Wd) in fp32.
// Items (expert, 128-row block, 128-weight-row block) are enumerated on the device from
// expert_offsets; the persistent grid walks them so that the workgroups of one XCD take
// consecutive items, which share their activation rows and their expert's weights in the
// XCD's L2.
#include "moeq_device.h"
#include "moeq_kernels.h"

#include <algorithm>

namespace moeq {

constexpr int kPBM = 128, kPBN = 128, kPBK = 64;
constexpr int kPThreads = 256;
constexpr int kPTileBytes = 128 * kPBK * 2;       // one 128 x 64 bf16 tile: 16 KiB
constexpr uint32_t kPOutOfRange = 0x80000000u;
constexpr int kPStreamPolicy = 2;                 // codes are read once per tile: non-temporal

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t p_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// byte offset of 16-byte unit u (0..7) of row r in a 128-byte-row tile
__device__ __forceinline__ int swz(int r, int u) { return r * 128 + ((u ^ ((r >> 1) & 7)) << 4); }

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4 a, const u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Active experts and the prefix count of their 128-row blocks (as in the decode kernel).
__device__ inline int p_active_tiles(const int32_t* offsets, int E, int* active, int* tpre,
                                     int* n_s) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < 64) {
        int rows[4], c = 0, nt = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane * 4 + j;
            rows[j] = e < E ? offsets[e + 1] - offsets[e] : 0;
            c += rows[j] > 0;
            nt += (rows[j] + kPBM - 1) / kPBM;
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
                active[pos] = lane * 4 + j;
                tpre[pos] = pre;
                ++pos;
                pre += (rows[j] + kPBM - 1) / kPBM;
            }
        if (lane == 63) {
            *n_s = ic;
            tpre[ic] = it;
        }
    }
    __syncthreads();
    return *n_s;
}

template <bool GATEUP>
__global__ void __launch_bounds__(kPThreads) prefill_kernel(const SkinnyArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int active[256];
    __shared__ int tpre[257];
    __shared__ int n_active_s;
    u32x4* tab = reinterpret_cast<u32x4*>(smem);
    uint8_t* atile = smem + (size_t)a.tables.n * 256 * 16;       // [2][128 x 128 B]
    uint8_t* btile = atile + 2 * kPTileBytes;                      // [2][128 x 128 B]
    build_decode_tables(a.tables, tab);
    const int nact = p_active_tiles(a.offsets, a.E, active, tpre, &n_active_s);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int K = a.K, N = a.N;
    const int ncb = GATEUP ? (N + 63) / 64 : (N + kPBN - 1) / kPBN;
    const long items = (long)__builtin_amdgcn_readfirstlane(tpre[nact]) * ncb;
    const int nstages = K / kPBK;
    const uint32_t kb = (uint32_t)K / 2, ks = (uint32_t)K / 32;
    const uint32_t mc = (uint32_t)N * kb, ms = (uint32_t)N * ks;
    const __amdgpu_buffer_rsrc_t ract = p_rsrc(a.act, a.act_bytes);

    // XCD-contiguous walk: workgroup g runs on XCD g % 8; the workgroups of one XCD take a
    // contiguous run of items each round
    const long G = gridDim.x;
    const long per_xcd = G / 8;
    const long slot = (G % 8 == 0) ? (long)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8
                                   : (long)blockIdx.x;

    // this thread's share of the global loads of a stage
    const int ld_row = tid >> 1, ld_half = tid & 1;

    for (long item = slot; item < items; item += G) {
        const int tile = (int)(item / ncb), cb = (int)(item % ncb);
        int lo = 0, hi = nact - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tpre[mid] <= tile) lo = mid; else hi = mid - 1;
        }
        const int e = __builtin_amdgcn_readfirstlane(active[lo]);
        const int m0 = (tile - __builtin_amdgcn_readfirstlane(tpre[lo])) * kPBM;
        const int beg = __builtin_amdgcn_readfirstlane(a.offsets[e]);
        const int end = __builtin_amdgcn_readfirstlane(a.offsets[e + 1]);
        const int r0 = beg + m0, rows = min(kPBM, end - r0);
        const int tsel = a.table_id[e];
        const bool badtab = tsel >= a.tables.n;
        const u32x4* mytab = tab + (badtab ? 0 : tsel) * 256;

        // activation row of this thread's loads (out of range past the expert's rows)
        uint32_t abase = kPOutOfRange;
        if (ld_row < rows) {
            const uint32_t src = GATEUP ? (uint32_t)(a.sorted_pair[r0 + ld_row] / a.k)
                                        : (uint32_t)(r0 + ld_row);
            abase = (src * (uint32_t)K + (uint32_t)ld_half * 32u) * 2u;
        }
        // weight row of this thread's code loads
        int wrow, mat = 0;
        if (GATEUP) {
            const int blk = ld_row >> 5;                  // gate, up, gate, up (32 rows each)
            mat = blk & 1;
            wrow = cb * 64 + (blk >> 1) * 32 + (ld_row & 31);
        } else {
            wrow = cb * kPBN + ld_row;
        }
        const __amdgpu_buffer_rsrc_t rc =
            p_rsrc((mat ? a.codes1 : a.codes0) + (size_t)e * mc, mc);
        const __amdgpu_buffer_rsrc_t rs =
            p_rsrc((mat ? a.scales1 : a.scales0) + (size_t)e * ms, ms);
        const uint32_t cbase = wrow < N ? (uint32_t)wrow * kb + (uint32_t)ld_half * 16u : kPOutOfRange;
        const uint32_t sbase = wrow < N ? (uint32_t)wrow * ks + (uint32_t)ld_half : kPOutOfRange;

        struct Stage {
            u32x4 x[4];
            u32x4 c;
            uint32_t s;
        };
        auto gload = [&](int st) {
            Stage g;
            const uint32_t koff = (uint32_t)st * kPBK;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                g.x[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    ract, abase == kPOutOfRange ? kPOutOfRange : abase + koff * 2u + 16u * j, 0, 0));
            g.c = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                rc, cbase == kPOutOfRange ? kPOutOfRange : cbase + koff / 2u, 0, kPStreamPolicy));
            g.s = __builtin_amdgcn_raw_buffer_load_b8(
                rs, sbase == kPOutOfRange ? kPOutOfRange : sbase + koff / 32u, 0, kPStreamPolicy);
            return g;
        };
        auto sstore = [&](const Stage& g, int buf) {
            uint8_t* at = atile + buf * kPTileBytes;
            uint8_t* bt = btile + buf * kPTileBytes;
            const u32x4 t = mytab[g.s & 0xFFu];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 x = GATEUP ? pair_split(g.x[j]) : g.x[j];   // x arrives natural
                *reinterpret_cast<u32x4*>(at + swz(ld_row, ld_half * 4 + j)) = x;
                *reinterpret_cast<u32x4*>(bt + swz(ld_row, ld_half * 4 + j)) = decode8(g.c[j], t);
            }
        };

        f32x16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

        {
            const Stage g0 = gload(0);
            sstore(g0, 0);
        }
        __syncthreads();
        for (int st = 0; st < nstages; ++st) {
            const int buf = st & 1;
            Stage nxt;
            const bool more = st + 1 < nstages;
            if (more) nxt = gload(st + 1);
            const uint8_t* at = atile + buf * kPTileBytes;
            const uint8_t* bt = btile + buf * kPTileBytes;
#pragma unroll
            for (int kq = 0; kq < kPBK / 16; ++kq) {
                const int u = kq * 2 + (lane >> 5);      // 16-byte unit: K 16 kq + 8 (lane / 32)
                u32x4 af[2], bf[2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    af[i] = *reinterpret_cast<const u32x4*>(at + swz(wm * 64 + i * 32 + (lane & 31), u));
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    bf[j] = *reinterpret_cast<const u32x4*>(bt + swz(wn * 64 + j * 32 + (lane & 31), u));
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(af[i], bf[j], acc[i][j]);
            }
            if (more) sstore(nxt, buf ^ 1);
            __syncthreads();
        }

        // ---- epilogue: lane holds rows 8 (r / 4) + 4 (lane / 32) + r % 4 of column lane % 32 ----
        const int cl = lane & 31;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row >= rows) continue;
                const size_t grow = (size_t)(r0 + row);
                if (GATEUP) {
                    const int ch = cb * 64 + wn * 32 + cl;
                    if (ch >= N) continue;
                    const float h = badtab ? __builtin_nanf("") : silu_mul(acc[i][0][r], acc[i][1][r]);
                    const int slotc = (ch & ~7) | (((ch & 1) << 2) | ((ch & 7) >> 1));
                    reinterpret_cast<uint16_t*>(a.out)[grow * a.out_ld + slotc] =
                        (uint16_t)f32_to_bf16_rne(h);
                } else {
                    const float wgt = a.topk_w[a.sorted_pair[grow]];
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int col = cb * kPBN + wn * 64 + j * 32 + cl;
                        if (col >= N) continue;
                        reinterpret_cast<float*>(a.out)[grow * a.out_ld + col] =
                            badtab ? __builtin_nanf("") : wgt * acc[i][j][r];
                    }
                }
            }
    }
}

int prefill_tile_rows() { return kPBM; }

void launch_prefill(const SkinnyArgs& a, bool gateup, long tiles, int cus, hipStream_t stream) {
    const size_t lds = (size_t)a.tables.n * 256 * 16 + 4 * kPTileBytes;
    const long ncb = gateup ? (a.N + 63) / 64 : (a.N + kPBN - 1) / kPBN;
    const long items = tiles * ncb;
    long blocks = std::min(items, (long)cus * 2);                 // 2 workgroups per CU
    if (blocks >= 8) blocks -= blocks % 8;                       // whole rounds over the XCDs
    blocks = std::max(1L, blocks);
    if (gateup)
        hipLaunchKernelGGL(prefill_kernel<true>, dim3(blocks), dim3(kPThreads), lds, stream, a);
    else
        hipLaunchKernelGGL(prefill_kernel<false>, dim3(blocks), dim3(kPThreads), lds, stream, a);
}

}  // namespace moeq
