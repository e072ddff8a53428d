// Grouped projections for many rows per expert (prefill): the MFMA work dominates.
//
// Tile. A workgroup of 8 wavefronts (one workgroup per CU, two wavefronts per SIMD) computes
// 128 sorted rows of one expert against 512 weight rows over the whole K, in stages of 64
// along K, with v_mfma_f32_32x32x16_bf16 (fp32 accumulation). Every wavefront owns 64 weight
// rows (two 32-column MFMA tiles) across all 128 rows (four 32-row MFMA tiles).
//   * Both operands are staged in LDS by LDS-DMA (buffer loads that write LDS directly), so
//     that every global request is a whole 64-byte sector: the 128 x 64 bf16 activation tile
//     of a stage (x rows through sorted_pair for gate|up, the intermediate's rows for down;
//     both already in the pair-split K order of the decoder) three stages ahead, and the code
//     bytes of the 512 weight rows for a super-stage of S stages (S = 2: 64 bytes a row) about
//     two stages ahead. The workgroup thus fetches each activation and code byte once per
//     item, and a CU keeps more data per request in flight than with per-lane register loads.
//   * A lane holds one weight row and one 32-wide half of the stage's K: 16 code bytes (read
//     from LDS one stage ahead) and exactly one E8M0 scale byte per stage (one decode-table
//     lookup for 32 weights). The scales are loaded to registers, 16 bytes a row (four
//     super-stages) at a time. The weights are decoded in registers into the MFMA B operand.
//   * Activation rows in LDS are 128 bytes with their 16-byte units XOR-swizzled by
//     (r1, r0 ^ r2, r0 ^ r3); weight rows hold their 2S units XOR-ed with a function of the
//     row, so the per-lane operand reads (16 consecutive rows, one unit) cover all 64 banks.
// The MFMA K index is mapped so that lane half h of kq-step q holds K 32 S h + 32 s + 8 q +
// (the pair-split order of 0..7) of super-stage stage s: the B lane's 32 weights are one
// contiguous, single-scale block of its row, and the A operand reads unit 4 h + q of its row.
// An expert's last tile is partial: the 32-row MFMA tiles past its rows are skipped
// (wavefront-uniform branches); their activation loads fall out of range and return zeros.
//
// gate|up ("Round 7" brief, decision 4): a wavefront's two column tiles are the gate and up
// rows of the same 32 channels, so bf16(silu(g) * u) is formed in registers; the workgroup
// covers 256 channels. down ("Round 7" brief, decision 6; README "What had to be fixed"): the
// epilogue writes topk_w[p] * (I . Wd) in fp32.
// Items (expert, 128-row block, weight-row block) are enumerated on the device from
// expert_offsets; the persistent grid walks them so that the workgroups of one XCD take
// consecutive items (the column blocks of the same rows first), which share their activation
// rows and their expert's weights in the XCD's L2.
#include "moeq_device.h"
#include "moeq_kernels.h"

#include <algorithm>
#include <type_traits>

namespace moeq {

constexpr int kPBM = 128, kPBK = 64;
constexpr int kPThreads = 512;                    // 8 wavefronts
constexpr int kPRowsW = 512;                      // weight rows of an item
constexpr int kPATile = kPBM * kPBK * 2;          // one 128 x 64 bf16 activation tile: 16 KiB
constexpr int kPABufs = 4;                        // activation tiles in LDS: DMA 3 stages ahead
constexpr int kPWBytes = 64 * 1024;               // weight tiles in LDS (2 x 32 KiB or 4 x 16 KiB)
constexpr uint32_t kPOutOfRange = 0x80000000u;
constexpr int kPQueues = 8;                       // work queues, one per XCD

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t p_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// byte offset of 16-byte unit u (0..7) of row r in a 128-byte-row tile; the unit index is
// XOR-ed with (r1, r0 ^ r2, r0 ^ r3) (bits of r)
__device__ __forceinline__ int swz(int r, int u) {
    const int g = ((r >> 1) & 1) | (((r ^ (r >> 2)) & 1) << 1) | (((r ^ (r >> 3)) & 1) << 2);
    return r * 128 + ((u ^ g) << 4);
}

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4 a, const u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Active experts (ascending) and the prefix count of their 128-row tiles.
__device__ inline int p_active_tiles(const int32_t* offsets, int E, int* active, int* tpre,
                                     int* n_s) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < 64) {
        int rows[4], c = 0, nt = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // clamped indexes (offsets has E + 1 entries): no branches between the loads, and
            // an expert e >= E gets no rows
            const int e = lane * 4 + j;
            rows[j] = (offsets[min(e + 1, E)] - offsets[min(e, E)] + kPBM - 1) / kPBM;
            c += rows[j] > 0;
            nt += rows[j];
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
                pre += rows[j];
            }
        if (lane == 63) {
            *n_s = ic;
            tpre[ic] = it;
        }
    }
    __syncthreads();
    return *n_s;
}

// x [T, H] -> the same rows with every 8-element group in pair-split order (the K order in
// which decode8 produces weights), so the gate|up tiles can be staged without permutes.
__global__ void __launch_bounds__(256) pair_split_rows_kernel(const u32x4* __restrict__ x,
                                                               u32x4* __restrict__ xs, long units) {
    const long stride = (long)gridDim.x * blockDim.x;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < units; i += stride)
        xs[i] = pair_split(__builtin_nontemporal_load(x + i));
}

// s_waitcnt that waits until at most n vector-memory loads are outstanding (other counters
// untouched); loads return in order.
#define MOEQ_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// Workgroup barrier that waits for the wavefront's own LDS reads but not for its vector-memory
// loads. __syncthreads() also makes the compiler wait for every LDS-DMA load in flight,
// including the ones issued for stages ahead; the stage loop instead waits for the one it
// needs with MOEQ_WAIT_VMCNT. The LDS reads issued in kq-step 2 of a stage (the activation
// fragments of kq-step 3 from the stage's own tile, the next stage's code bytes from a weight
// tile that the loads after the barrier may refill) are only consumed in kq-step 3, after the
// barrier; s_barrier does not wait for them, so lgkmcnt(0) comes first: once a wavefront is
// past the barrier, every LDS read of every wavefront issued before it has returned its data,
// and the LDS-DMA refills issued after it cannot overwrite a tile under a pending read. The
// empty asm statements keep the compiler from moving memory accesses across the barrier.
#define MOEQ_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14))
#define MOEQ_STAGE_BARRIER()                 \
    do {                                     \
        asm volatile("" ::: "memory");       \
        MOEQ_WAIT_LGKM0();                   \
        __builtin_amdgcn_s_barrier();        \
        asm volatile("" ::: "memory");       \
    } while (0)

// Stage-loop waits, by S and stage position r in a group of 8: the number of vector-memory
// loads issued after the one waited for (loads return in order; the issue schedule is the
// one of prefill_kernel's issue()). kPWaitA: before the barrier of stage st, for the
// activations of stage st + 1 (issued in stage st - 3); kPWaitW: before the code bytes of
// stage st + 1 are read, for their weights (issued in stage st - 3; S = 2: odd r only, when
// stage st + 1 starts a super-stage; 0 = no wait).
constexpr int kPWaitA[2][8] = {{16, 16, 16, 16, 16, 16, 16, 16}, {8, 12, 10, 14, 10, 12, 8, 12}};
constexpr int kPWaitW[2][8] = {{14, 14, 14, 14, 14, 14, 14, 14}, {0, 8, 0, 10, 0, 8, 0, 8}};

// S: stages per weight super-stage: 2 when K % 128 == 0 (a weight row's 64 code bytes of a
// super-stage are one sector; its scale bytes are read 16 at a time, four super-stages), else
// 1 (32 code bytes a row per stage, one scale byte per stage and lane).
template <bool GATEUP, int S>
__global__ void __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
    prefill_kernel(const SkinnyArgs a) {
    constexpr int MT = 4, NT = 2;                 // 32 x 32 MFMA tiles per wavefront
    constexpr int U = 2 * S;                      // 16-byte units of a weight row per super-stage
    constexpr int WROW = 32 * S;                  // bytes of a weight row per super-stage
    constexpr int NWB = 4 / S;                    // weight tiles in LDS
    constexpr int WTILE = kPRowsW * WROW;         // bytes of one weight tile
    static_assert(NWB * WTILE == kPWBytes, "weight tiles");

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int active[256];
    __shared__ int tpre[257];
    __shared__ int n_active_s;
    u32x4* tab = reinterpret_cast<u32x4*>(smem);
    uint8_t* atile = smem + (size_t)a.tables.n * 256 * 16;       // [kPABufs][128 x 128 B]
    uint8_t* wtile = atile + kPABufs * kPATile;                   // [NWB][512 x WROW B]
    build_decode_tables(a.tables, tab);
    const int nact = p_active_tiles(a.offsets, a.E, active, tpre, &n_active_s);

    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, cl = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = a.K, N = a.N;
    const int cols = GATEUP ? 256 : 512;          // output columns (gate|up: channels) per item
    const int ncb = (N + cols - 1) / cols;
    const long items = (long)__builtin_amdgcn_readfirstlane(tpre[nact]) * ncb;
    const int nstages = K / kPBK;
    const int nsuper = nstages / S;
    const int ngroups = (nstages + 7) / 8;        // scale loads (S = 2): 8 stages each
    const uint32_t kb = (uint32_t)K / 2, ks = (uint32_t)K / 32;
    const uint32_t mcode = (uint32_t)N * kb, mscale = (uint32_t)N * ks;
    const __amdgpu_buffer_rsrc_t ract = p_rsrc(a.act, a.act_bytes);

    // Work queues: a.queue holds one counter per XCD (zero at launch; workgroup g runs on XCD
    // g % 8). Queue x hands out, in order, the items of item groups x, x + 8, x + 16, ..., a
    // group being the column blocks of 4 row tiles, which share activations and weights in the
    // XCD's L2. A workgroup drains its own XCD's queue first, then the other queues, so the
    // work balances across workgroups whatever the items cost.
    const int myx = (int)(blockIdx.x % 8);
    const long grp = 4L * ncb;
    __shared__ int s_claim;
    __shared__ float s_roww[kPBM];                // down: topk_w of the item's rows

    // MFMA A operand of kq-step q, row tile i: swz(32 i + cl, 4 h + q) = a_rd0 ^ 16 q + 4096 i
    // (the swizzle depends on the row's low 4 bits only; (4 h + q) ^ g = (4 h ^ g) ^ q)
    const int a_rd0 = swz(cl, 4 * h);
    // Activation staging: load j (0, 1) of wavefront w fills tile rows 16 w + 8 j .. + 7, lane
    // L the 16 bytes at physical unit L % 8 of row 16 w + 8 j + L / 8, i.e. logical unit
    // d_u[j] (the row's low 4 bits are 8 j + L / 8).
    const int d_row = lane >> 3;
    int d_u[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int r = 8 * p + d_row;
        const int g = ((r >> 1) & 1) | (((r ^ (r >> 2)) & 1) << 1) | (((r ^ (r >> 3)) & 1) << 2);
        d_u[p] = (lane & 7) ^ g;
    }
    // Weight tile rows: 0 .. 255 gate, 256 .. 511 up (same channels), or 512 down rows. Unit
    // k of row R sits at position k ^ wsw(R), wsw(R) = (R / (16 / U)) % U: the 16 lanes of an
    // operand read (rows R0 .. R0 + 15, one unit k) then hit 16 distinct bank groups.
    auto wsw = [](int R) { return (R / (16 / U)) % U; };
    // weight staging: load i (0 .. 2S - 1) of a wavefront fills the 32 / S tile rows from
    // wd_row0[i], lane L row wd_row0[i] + L / U, position L % U (fixed-size arrays throughout:
    // hipcc's host pass drops this kernel's stubs when its lambdas capture template-sized
    // arrays or call one another)
    int wd_row0[4];
#pragma unroll
    for (int i = 0; i < 2 * S; ++i)
        wd_row0[i] = GATEUP ? (i < S ? 32 * wave + (32 / S) * i : 256 + 32 * wave + (32 / S) * (i - S))
                            : 64 * wave + (32 / S) * i;
    const int wd_t = lane % U;
    // the tile rows of this lane's two column tiles, and the LDS offsets of its unit for
    // stage s of a super-stage (unit S h + s)
    uint32_t wr_off[NT][2];                       // [NT][S]
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int R = GATEUP ? j * 256 + 32 * wave + cl : 64 * wave + 32 * j + cl;
#pragma unroll
        for (int sp = 0; sp < S; ++sp)
            wr_off[j][sp] = (uint32_t)(R * WROW + 16 * ((S * h + sp) ^ wsw(R)));
    }
    const uint32_t hsh = 16u * (uint32_t)h;       // S = 2: bit offset of the lane's scale bytes

    // s_claim is written by thread 0 only after a barrier that every wavefront reaches after
    // reading its previous value: the staging barrier of an item, or the barrier below when a
    // queue is drained (the previous item's epilogue ends without one).
    int qx = 0;                                   // queues drained: myx .. myx + qx - 1
    if (tid == 0) s_claim = atomicAdd(&a.queue[myx], 1);
    __syncthreads();
    int claim = __builtin_amdgcn_readfirstlane(s_claim);
    for (;;) {
        const int qcur = (myx + qx) & 7;
        const long item = ((long)(claim / grp) * 8 + qcur) * grp + claim % grp;
        if (item >= items) {                      // queue qcur is drained: take the next one
            if (++qx == 8) break;
            __syncthreads();                      // every wavefront has read the last claim
            if (tid == 0) s_claim = atomicAdd(&a.queue[(myx + qx) & 7], 1);
            __syncthreads();
            claim = __builtin_amdgcn_readfirstlane(s_claim);
            continue;
        }
        const int tile = (int)(item / ncb), cb = (int)(item % ncb);
        int nclaim = 0;                           // the next claim of queue qcur (thread 0)
        int row_pair = 0;                         // down, thread t < 128: pair of row t
        float row_w = 0.f;                        // and its router weight
        int lo = 0, hi = nact - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tpre[mid] <= tile) lo = mid; else hi = mid - 1;
        }
        const int e = __builtin_amdgcn_readfirstlane(active[lo]);
        const int beg = __builtin_amdgcn_readfirstlane(a.offsets[e]);
        const int end = __builtin_amdgcn_readfirstlane(a.offsets[e + 1]);
        const int r0 = beg + (tile - __builtin_amdgcn_readfirstlane(tpre[lo])) * kPBM;
        const int rows = min(kPBM, end - r0);
        const int mt_act = (rows + 31) >> 5;      // 32-row MFMA tiles holding rows
        const int tsel = a.table_id[e];
        const bool badtab = tsel >= a.tables.n;
        const u32x4* mytab = tab + (badtab ? 0 : tsel) * 256;

        // Stage st = S m + s: unit u of an activation row holds K = 64 S m + (u / 4) 32 S +
        // 32 s + 8 (u % 4) .. + 7, i.e. row byte offset rb + 64 S (u / 4) + 128 S m + 64 s.
        // (rb is 16-byte aligned; its bit 0 carries u / 4, the K half of the lane's unit)
        uint32_t rb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int rr = wave * 16 + j * 8 + d_row;
            const int u = d_u[j];
            rb[j] = kPOutOfRange;
            if (rr < rows) {
                const uint32_t src = GATEUP ? (uint32_t)(a.sorted_pair[r0 + rr] / a.k)
                                            : (uint32_t)(r0 + rr);
                rb[j] = src * (uint32_t)K * 2u + 16u * (uint32_t)(u & 3);
            }
            rb[j] |= (uint32_t)(u >> 2);
        }
        // weight staging sources: a wavefront stages exactly the 64 tile rows it reads (gate|up:
        // loads 0 .. S - 1 its gate rows, S .. 2S - 1 its up rows), so the weights need no
        // barrier, only the wavefront's own memory-counter waits
        const __amdgpu_buffer_rsrc_t rcw0 = p_rsrc(a.codes0 + (size_t)e * mcode, mcode);
        const __amdgpu_buffer_rsrc_t rcw1 =
            GATEUP ? p_rsrc(a.codes1 + (size_t)e * mcode, mcode) : rcw0;
        uint32_t wdoff[4];                        // [2 S]
#pragma unroll
        for (int i = 0; i < 2 * S; ++i) {
            const int R = wd_row0[i] + lane / U;
            const int grow = GATEUP ? cb * 256 + (R & 255) : cb * 512 + R;
            wdoff[i] = grow < N ? (uint32_t)grow * kb + 16u * (uint32_t)(wd_t ^ wsw(R))
                                : kPOutOfRange;
        }
        // scale rows of the lane's column tiles
        __amdgpu_buffer_rsrc_t rs[NT];
        uint32_t sw[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const uint8_t* sm = (GATEUP && j == 1) ? a.scales1 : a.scales0;
            rs[j] = p_rsrc(sm + (size_t)e * mscale, mscale);
            const int srow = GATEUP ? cb * 256 + 32 * wave + cl : cb * 512 + 64 * wave + 32 * j + cl;
            sw[j] = srow < N ? (uint32_t)srow * ks : kPOutOfRange;
        }

        // ---- staging (steps past the end re-load the last stage: no branches around loads,
        // so the memory-counter waits below stay exact) ----
        auto dma_a = [&](int st, int pos) {          // activations of stage st -> tile pos % 4
            const int sc = min(st, nstages - 1);
            const int m = sc / S, sp = sc % S;
            const uint32_t koff = 128u * S * (uint32_t)m + 64u * (uint32_t)sp;
            uint8_t* dst = atile + (pos % kPABufs) * kPATile + wave * 2048;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ract, dst + j * 1024, 16, (rb[j] & ~1u) + (rb[j] & 1u) * 64u * S + koff, 0, 0, 0);
        };
        auto dma_w = [&](int msup, int mpos) {       // weights of super-stage msup -> tile mpos
            const int mc = min(msup, nsuper - 1);
            uint8_t* dst = wtile + (mpos % NWB) * WTILE;
#pragma unroll
            for (int i = 0; i < 2 * S; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(i < S ? rcw0 : rcw1,
                                                         dst + wd_row0[i] * WROW, 16,
                                                         wdoff[i] + (uint32_t)WROW * mc, 0, 0, 0);
        };
        // scales: S = 2, 16 bytes a row (stages 8 g .. 8 g + 7; byte 4 (p / 2) + 2 h + p % 2 for
        // stage 8 g + p); S = 1, one byte per stage in a ring of four
        u32x4 wsc[NT], wscn[NT];
        uint32_t wsb[NT][4];
        auto sload2 = [&](int g, u32x4* dst) {
            const int gc = min(g, ngroups - 1);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                dst[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       rs[j], sw[j] + 16u * (uint32_t)gc, 0, 0));
        };
        auto sload1 = [&](int st, int pos) {
            const int sc = min(st, nstages - 1);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                wsb[j][pos % 4] = __builtin_amdgcn_raw_buffer_load_b8(
                    rs[j], sw[j] + 2u * (uint32_t)sc + (uint32_t)h, 0, 0);
        };

        f32x16 acc[MT][NT];
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

        // Operands in flight: the A fragments of the next kq-step (each 32-row fragment is
        // re-read as soon as its MFMAs are issued), the decoded weights of this kq-step and the
        // next, the lane's 16 code bytes and decode-table entries of one stage. A stage at
        // unrolled position pos (0 .. 7; 8 = the next group's first) uses activation tile
        // pos % 4 and weight tile (pos / S) % NWB.
        u32x4 av[MT], b[2][NT], tt[NT], wcur[NT];
        auto read_a = [&](int pos, int q, int i) {
            const uint8_t* at = atile + (pos % kPABufs) * kPATile;
            av[i] = *reinterpret_cast<const u32x4*>(at + (a_rd0 ^ (16 * q)) + i * 32 * 128);
        };
        auto read_w = [&](int pos) {
            const uint8_t* wt = wtile + ((pos / S) % NWB) * WTILE;
#pragma unroll
            for (int j = 0; j < NT; ++j)
                wcur[j] = *reinterpret_cast<const u32x4*>(wt + wr_off[j][pos % S]);
        };
        auto tables_of = [&](int pos) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                uint32_t sbyte;
                if constexpr (S == 2) {
                    const u32x4 src = pos >= 8 ? wscn[j] : wsc[j];
                    const int p = pos % 8;
                    sbyte = __builtin_amdgcn_ubfe(src[p / 2], hsh + 8u * (uint32_t)(p & 1), 8);
                } else {
                    sbyte = wsb[j][pos % 4];
                }
                tt[j] = mytab[sbyte];
            }
        };
        // Loads issued in stage st (position r of a group of 8 stages), after its barrier: the
        // activations of stage st + 4 (into the tile of stage st); S = 2: for even r the weights
        // of super-stage st / 2 + 2 (into the tile of super-stage st / 2), for r = 1 the next
        // group's scales; S = 1: the weights of stage st + 4 and the scale bytes of stage st + 3.
        auto issue = [&](int st, int r) {
            dma_a(st + 4, r + 4);
            if (S == 2) {
                if ((r & 1) == 0) dma_w(st / 2 + 2, r / 2 + 2);
                if (r == 1) sload2(st / 8 + 1, wscn);
            } else {
                dma_w(st + 4, r + 4);
                sload1(st + 3, r + 3);
            }
        };
        // waits: kPWaitA / kPWaitW (namespace scope)
        auto wait_n = [](int n) {
            switch (n) {
                case 16: MOEQ_WAIT_VMCNT(16); break;
                case 14: MOEQ_WAIT_VMCNT(14); break;
                case 12: MOEQ_WAIT_VMCNT(12); break;
                case 10: MOEQ_WAIT_VMCNT(10); break;
                case 8: MOEQ_WAIT_VMCNT(8); break;
                default: MOEQ_WAIT_VMCNT(0); break;
            }
        };
        // FULL: all four 32-row MFMA tiles hold rows (no branches inside the stage). Stage st
        // (position r) starts with its kq-step 0 operands in av, b[0]. In kq-step 2 it reads the
        // code bytes and table entries of stage st + 1 (its own staged weights); after kq-step 2
        // (the last reads of its activation tile) the workgroup barrier makes the activations
        // of stage st + 1 visible and frees the tile of stage st, which the loads of the stage
        // then refill; kq-step 3 fetches the A fragments and first decoded weights of stage
        // st + 1, so the next stage starts with MFMAs at once.
        auto compute = [&](auto full, int st, int r) {
            constexpr bool FULL = decltype(full)::value;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int cur = q & 1, nxt = cur ^ 1;
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    if (FULL || i < mt_act)
#pragma unroll
                        for (int j = 0; j < NT; ++j)
                            acc[i][j] = mfma32x32x16(av[i], b[cur][j], acc[i][j]);
                    if (FULL || i < mt_act) {
                        if (q < 3) read_a(r, q + 1, i);
                        else read_a(r + 1, 0, i);
                    }
                    if (q < 3 && i < NT) b[nxt][i] = decode8(wcur[i][q + 1], tt[i]);
                    if (q == 2 && i == 2) {
                        __builtin_amdgcn_sched_barrier(0);
                        if (kPWaitW[S - 1][r]) wait_n(kPWaitW[S - 1][r]);
                        asm volatile("" ::: "memory");
                        tables_of(r + 1);
                        read_w(r + 1);
                    }
                    if (q == 3 && i >= 2) b[nxt][i - 2] = decode8(wcur[i - 2][0], tt[i - 2]);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (q == 2) {
                    wait_n(kPWaitA[S - 1][r]);
                    MOEQ_STAGE_BARRIER();
                    issue(st, r);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        auto run = [&](auto full) {
#pragma unroll
            for (int st = 0; st < 4; ++st) dma_a(st, st);
            if (S == 2) {
                dma_w(0, 0);
                dma_w(1, 1);
                sload2(0, wsc);
            } else {
#pragma unroll
                for (int st = 0; st < 4; ++st) dma_w(st, st);
#pragma unroll
                for (int st = 0; st < 3; ++st) sload1(st, st);
            }
            MOEQ_WAIT_VMCNT(0);
            __syncthreads();
            if (tid == 0) s_claim = nclaim;           // read by all after the item's last barrier
            if (!GATEUP && tid < kPBM && tid < rows) row_w = a.topk_w[row_pair];
            tables_of(0);
            read_w(0);
#pragma unroll
            for (int i = 0; i < MT; ++i) read_a(0, 0, i);
#pragma unroll
            for (int j = 0; j < NT; ++j) b[0][j] = decode8(wcur[j][0], tt[j]);
            // whole groups of 8 stages as straight-line code (branches between the loads would
            // make the compiler's own waits for the scale registers drain every load in flight),
            // then the last group's stages one by one
            int st0 = 0;
            for (; st0 + 8 <= nstages; st0 += 8) {
#pragma unroll
                for (int r = 0; r < 8; ++r) compute(full, st0 + r, r);
                if (S == 2) {
#pragma unroll
                    for (int j = 0; j < NT; ++j) wsc[j] = wscn[j];
                }
            }
            if (st0 < nstages) {
#pragma unroll
                for (int r = 0; r < 8; ++r)
                    if (st0 + r < nstages) compute(full, st0 + r, r);
            }
            if (!GATEUP && tid < kPBM) s_roww[tid] = row_w;
            // the last stage's kq-step 3 read the (unused) tile past the end: all wavefronts
            // are done with LDS before the next item stages into it
            MOEQ_WAIT_VMCNT(0);
            __syncthreads();
        };
        // the next item of this queue is claimed now: the staging's wait covers the atomic,
        // and its result is published after the staging's barrier
        if (tid == 0) nclaim = atomicAdd(&a.queue[qcur], 1);
        // down: thread t < 128 fetches the router weight of row t (its pair index now, under
        // the staging's wait; the weight after the staging barrier) and parks it in LDS at the
        // end of the stage loop, where the load has long arrived: the epilogue then reads LDS
        // instead of two dependent global loads per output row
        if (!GATEUP && tid < kPBM && tid < rows) row_pair = a.sorted_pair[r0 + tid];
        if (mt_act == MT) run(std::true_type{});
        else run(std::false_type{});

        // ---- epilogue: lane holds rows 8 (r / 4) + 4 h + r % 4 of column cl; row offsets are
        // split into the lane's 4 h and a wavefront-uniform rest ----
        int el = lane;
        asm volatile("" : "+v"(el));              // computed here, not kept live across the loop
        const int hr = 4 * (el >> 5), ecl = el & 31;
        if (GATEUP) {
            // Each 32-row block of the wavefront's 32 channels goes through LDS (64 bytes a row
            // in pair-split slot order, in the wavefront's own 2 KB of activation tile 0; see the
            // down epilogue below), so that a lane stores 16 contiguous bytes (8 slots) instead
            // of 2.
            uint16_t* own = reinterpret_cast<uint16_t*>(atile + wave * 2048);
            const int ch = cb * 256 + wave * 32 + ecl;
            const int sl = (ecl & ~7) | (((ecl & 1) << 2) | ((ecl & 7) >> 1));  // slot in the 32
            int rd = lane;
            asm volatile("" : "+v"(rd));                 // computed here, not kept live across the loop
            const int gslot = cb * 256 + wave * 32 + 8 * (rd & 3);
            uint16_t* ob = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                if (i >= mt_act) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int c = hr + 8 * (r >> 2) + (r & 3);
                    const float v =
                        badtab ? __builtin_nanf("") : silu_mul(acc[i][0][r], acc[i][1][r]);
                    own[c * 32 + sl] = (uint16_t)f32_to_bf16_rne(v);
                }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const int rb = (rd >> 2) + 16 * k;        // row of the block
                    const int row = 32 * i + rb;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(own + rb * 32 + 8 * (rd & 3));
                    if (row < rows && gslot < N)
                        *reinterpret_cast<u32x4*>(ob + (size_t)(r0 + row) * a.out_ld + gslot) = v;
                }
                __builtin_amdgcn_wave_barrier();
            }
            (void)ch;
            MOEQ_WAIT_LGKM0();
        } else {
            // Each 32-row block of the wavefront's 64 columns goes through LDS, so that a lane
            // stores 16 contiguous bytes (16 lanes one 256-byte output row, 4 rows a store)
            // instead of 4: the block (32 rows x 256 bytes) sits in the wavefront's own part of
            // the four activation tiles (bytes 2048 w .. + 2047 of each, which only this
            // wavefront's staging loads fill), 8 rows a tile. After run()'s barrier no other
            // wavefront reads them, and the LDS reads are waited for before this wavefront's
            // next staging loads.
            uint8_t* own = atile + wave * 2048;
            auto blk = [&](int row, int col) { return own + (row >> 3) * kPATile + (row & 7) * 256 + col * 4; };
            int rd = lane;
            asm volatile("" : "+v"(rd));                 // computed here, not kept live across the loop
            const int rl = rd >> 4, c4 = (rd & 15) * 4;   // read side: rows rl + 4 k, 4 columns
            const int gcol = cb * 512 + wave * 64 + c4;
            float* ob = reinterpret_cast<float*>(a.out);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                if (i >= mt_act) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int c = hr + 8 * (r >> 2) + (r & 3);
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        *reinterpret_cast<float*>(blk(c, ecl + 32 * j)) = acc[i][j][r];
                }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int row = 32 * i + rl + 4 * k;      // row of the item
                    const f32x4 v = *reinterpret_cast<const f32x4*>(blk(rl + 4 * k, c4));
                    if (row < rows && gcol < N) {
                        const float wgt = badtab ? __builtin_nanf("") : s_roww[row];
                        *reinterpret_cast<f32x4*>(ob + (size_t)(r0 + row) * a.out_ld + gcol) = wgt * v;
                    }
                }
                __builtin_amdgcn_wave_barrier();
            }
            MOEQ_WAIT_LGKM0();
        }
        claim = __builtin_amdgcn_readfirstlane(s_claim);
    }
}

__global__ void __launch_bounds__(64) zero_queue_kernel(int32_t* q) {
    if (threadIdx.x < kPQueues) q[threadIdx.x] = 0;
}

int prefill_tile_rows() { return kPBM; }

size_t prefill_split_bytes(int T, int H) { return ((size_t)T * H * 2 + 255) & ~(size_t)255; }

size_t prefill_queue_bytes() { return 256; }

void launch_pair_split_rows(const uint16_t* x, int T, int H, uint16_t* xs, int cus,
                            hipStream_t stream) {
    const long units = (long)T * H / 8;
    const long blocks = std::max(1L, std::min((units + 255) / 256, (long)cus * 8));
    hipLaunchKernelGGL(pair_split_rows_kernel, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x4*>(xs), units);
}

// tiles: host upper bound of the 128-row tiles the device will find
void launch_prefill(const SkinnyArgs& a, bool gateup, long tiles, int cus, int max_groups,
                    hipStream_t stream) {
    hipLaunchKernelGGL(zero_queue_kernel, dim3(1), dim3(64), 0, stream, a.queue);
    const size_t lds = (size_t)a.tables.n * 256 * 16 + kPABufs * kPATile + kPWBytes;
    const long ncb = gateup ? (a.N + 255) / 256 : (a.N + 511) / 512;
    long blocks = std::min(tiles * ncb, (long)cus);
    if (blocks >= 8) blocks -= blocks % 8;                       // whole rounds over the XCDs
    if (max_groups > 0) blocks = std::min(blocks, (long)max_groups);
    blocks = std::max(1L, blocks);
    const bool wide = a.K % 128 == 0;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(kPThreads), lds, stream, a);
    };
    if (gateup) {
        if (wide) go(prefill_kernel<true, 2>); else go(prefill_kernel<true, 1>);
    } else {
        if (wide) go(prefill_kernel<false, 2>); else go(prefill_kernel<false, 1>);
    }
}

}  // namespace moeq
