// Grouped projections for many rows per expert (prefill): the MFMA work dominates.
//
// Tile. A workgroup of 4 wavefronts computes 128 sorted rows of one expert against 256 weight
// rows over the whole K, in stages of 64 along K, with v_mfma_f32_32x32x16_bf16 (fp32
// accumulation). Every wavefront owns 64 weight rows (two 32-column MFMA tiles) across all
// 128 rows (four 32-row MFMA tiles), so the weights a wavefront needs are its own:
//   * weights go global -> registers -> decoded in registers -> MFMA B operand. A lane holds
//     one weight row and one 32-wide half of the stage's K, i.e. 16 code bytes and exactly one
//     E8M0 scale byte per stage (one decode-table lookup for 32 weights). The code and scale
//     loads run two stages ahead in a ring of three register sets.
//   * activations are shared by the four wavefronts and go through LDS: each stage the
//     workgroup loads the 128 x 64 bf16 tile (x rows through sorted_pair for gate|up, the
//     intermediate's rows for down; both already in the pair-split K order of the decoder)
//     one stage ahead into registers and stores it into the other half of a double-buffered
//     LDS tile; one barrier closes the stage. LDS rows are 128 bytes with their 16-byte units
//     XOR-swizzled by (r1, r0 ^ r2, r0 ^ r3), so that the MFMA operand reads (16 consecutive
//     rows, one unit) and the staging writes cover all 64 banks.
// The MFMA K index is mapped so that lane half h of kq-step q holds stage K 32 h + 8 q + (the
// pair-split order of 0..7): the B lane's 32 weights are one contiguous, single-scale block,
// and the A operand reads unit 4 h + q of its row.
// An expert's last tile is partial: the 32-row MFMA tiles past its rows are skipped
// (wavefront-uniform branches); their activation loads fall out of range and return zeros.
//
// gate|up ("Round 7" brief, decision 4): a wavefront's two column tiles are the gate and up
// rows of the same 32 channels, so bf16(silu(g) * u) is formed in registers; the workgroup
// covers 128 channels. down ("Round 7" brief, decision 6; README "What had to be fixed"): the
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
constexpr int kPThreads = 256;
constexpr int kPATile = kPBM * kPBK * 2;          // one 128 x 64 bf16 activation tile: 16 KiB
constexpr uint32_t kPOutOfRange = 0x80000000u;
// Weight loads use the default (cached) policy: a lane reads 32 of the 128 bytes of a cache
// line per stage and the next three stages read the rest, and the items of the other row
// tiles of the same expert read the same lines -- non-temporal loads made every stage fetch
// its line from HBM again.
constexpr int kPWeightPolicy = 0;

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
            const int e = lane * 4 + j;
            rows[j] = e < E ? (offsets[e + 1] - offsets[e] + kPBM - 1) / kPBM : 0;
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

// S: stages per weight super-stage. S = 4 when K % 128 == 0: a lane then reads the 64 code
// bytes of its row for four stages at once (whole cache lines) and one aligned scale dword;
// otherwise S = 1 (16 code bytes and the scale byte's dword per stage).
template <bool GATEUP, int S>
__global__ void __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
    prefill_kernel(const SkinnyArgs a) {
    constexpr int MT = 4, NT = 2;                 // 32 x 32 MFMA tiles per wavefront

    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int active[256];
    __shared__ int tpre[257];
    __shared__ int n_active_s;
    u32x4* tab = reinterpret_cast<u32x4*>(smem);
    uint8_t* atile = smem + (size_t)a.tables.n * 256 * 16;       // [2][128 x 128 B]
    build_decode_tables(a.tables, tab);
    const int nact = p_active_tiles(a.offsets, a.E, active, tpre, &n_active_s);

    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, cl = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = a.K, N = a.N;
    const int cols = GATEUP ? 128 : 256;          // weight rows (gate|up: channels) per item
    const int ncb = (N + cols - 1) / cols;
    const long items = (long)__builtin_amdgcn_readfirstlane(tpre[nact]) * ncb;
    const int nstages = K / kPBK;
    const int nsuper = (nstages + S - 1) / S;
    const uint32_t kb = (uint32_t)K / 2, ks = (uint32_t)K / 32;
    const uint32_t mcode = (uint32_t)N * kb, mscale = (uint32_t)N * ks;
    const __amdgpu_buffer_rsrc_t ract = p_rsrc(a.act, a.act_bytes);

    // XCD-contiguous walk: workgroup g runs on XCD g % 8; the workgroups of one XCD take a
    // contiguous run of items each round
    const long G = gridDim.x;
    const long per_xcd = G / 8;
    const long slot = (G % 8 == 0) ? (long)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8
                                   : (long)blockIdx.x;

    // MFMA A operand of kq-step q, row tile i: swz(32 i + cl, 4 h + q) = a_rd[q] + 4096 i (the
    // swizzle depends on the row's low 4 bits only)
    // ((4 h + q) ^ g = (4 h ^ g) ^ q for q < 4, so a_rd[q] = a_rd0 ^ 16 q)
    const int a_rd0 = swz(cl, 4 * h);
    // Activation staging by LDS-DMA: load j (0..3) of wavefront w fills tile rows 32 w + 8 j ..
    // + 7, lane L the 16 bytes at physical unit L % 8 of row 32 w + 8 j + L / 8, i.e. logical
    // unit d_u[j % 2] (the row's low 4 bits are 8 (j % 2) + L / 8).
    const int d_row = lane >> 3;
    int d_u[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int r = 8 * p + d_row;
        const int g = ((r >> 1) & 1) | (((r ^ (r >> 2)) & 1) << 1) | (((r ^ (r >> 3)) & 1) << 2);
        d_u[p] = (lane & 7) ^ g;
    }

    for (long item = slot; item < items; item += G) {
        const int tile = (int)(item / ncb), cb = (int)(item % ncb);
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

        // Stage st of super-stage m (st = S m + s, ms stages in m): unit u of an LDS row holds
        // K = 64 S m + (u / 4) 32 ms + 32 s + 8 (u % 4) .. + 7, so that the lane half h of the
        // B operand covers a contiguous 32 ms-wide K range of its weight row per super-stage.
        // Row byte offset of a DMA lane: rb + 64 ms (u / 4) + 128 S m + 64 s.
        // (rb is 16-byte aligned; its bit 0 carries u / 4, the K half of the lane's unit)
        uint32_t rb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = wave * 32 + j * 8 + d_row;
            const int u = d_u[j & 1];
            rb[j] = kPOutOfRange;
            if (rr < rows) {
                const uint32_t src = GATEUP ? (uint32_t)(a.sorted_pair[r0 + rr] / a.k)
                                            : (uint32_t)(r0 + rr);
                rb[j] = src * (uint32_t)K * 2u + 16u * (uint32_t)(u & 3);
            }
            rb[j] |= (uint32_t)(u >> 2);
        }
        // the weight rows of this lane: column tile j of the wavefront
        // (gate|up: both tiles use the same rows of the two matrices; down: the second tile
        // starts 32 rows further)
        __amdgpu_buffer_rsrc_t rc[NT], rs[NT];
        const int wrow0 = GATEUP ? cb * 128 + wave * 32 + cl : cb * 256 + wave * 64 + cl;
        const uint32_t cw0 = (uint32_t)wrow0 * kb, sw0 = (uint32_t)wrow0 * ks;
        uint32_t cw[NT], sw[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int jr = GATEUP ? 0 : 32 * j;
            const uint8_t* cm = (GATEUP && j == 1) ? a.codes1 : a.codes0;
            const uint8_t* sm = (GATEUP && j == 1) ? a.scales1 : a.scales0;
            rc[j] = p_rsrc(cm + (size_t)e * mcode, mcode);
            rs[j] = p_rsrc(sm + (size_t)e * mscale, mscale);
            cw[j] = wrow0 + jr < N ? cw0 + (uint32_t)jr * kb : kPOutOfRange;
            sw[j] = wrow0 + jr < N ? sw0 + (uint32_t)jr * ks : kPOutOfRange;
        }

        // Weights: chunk c (16 code bytes per column tile) of super-stage m is used at stage
        // S m + c. For S = 4 the chunk registers are shared by consecutive super-stages: chunks
        // 0, 1 of super-stage m + 1 (with its scale dwords, which alternate between two sets)
        // are loaded at stage S m + 2, after chunks 0, 1 of m were used; chunks 2, 3 of
        // m + 1 at its own stage 0. A row's 128-byte line is thus read in two bursts.
        // (S = 1: two chunk slots alternate, slot = stage parity)
        u32x4 wc[NT][S == 1 ? 2 : S];
        uint32_t wsc[2][NT], wsh[2];
        // Loads past the end re-read the last super-stage (cache hits, never used), so the
        // stage loop has no branches around loads and the memory-counter waits stay exact.
        auto wload = [&](int m, int c0, int nc, bool scales, int set) {
            const int mc = min(m, nsuper - 1);
            const uint32_t ms = (uint32_t)min(S, nstages - S * mc);
            const uint32_t coff = 32u * S * (uint32_t)mc + 16u * ms * (uint32_t)h;
            const uint32_t soff = 2u * S * (uint32_t)mc + ms * (uint32_t)h;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
#pragma unroll
                for (int c = c0; c < c0 + nc; ++c)       // S = 1: chunk 0 into slot c0
                    wc[j][c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        rc[j], cw[j] + coff + 16u * (S == 1 ? 0 : c), 0, kPWeightPolicy));
                if (scales)
                    wsc[set][j] = __builtin_amdgcn_raw_buffer_load_b32(
                        rs[j], (sw[j] + soff) & ~3u, 0, kPWeightPolicy);
            }
            if (scales) wsh[set] = ((sw[0] + soff) & 3u) * 8u;
        };
        auto dma = [&](int st) {
            const int sc = min(st, nstages - 1);
            const int m = sc / S, sp = sc % S;
            const uint32_t ms = (uint32_t)min(S, nstages - S * m);
            const uint32_t koff = 128u * S * (uint32_t)m + 64u * (uint32_t)sp;
            uint8_t* dst = atile + (st & 1) * kPATile + wave * 4096;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ract, dst + j * 1024, 16, (rb[j] & ~1u) + (rb[j] & 1u) * 64u * ms + koff, 0, 0, 0);
        };

        f32x16 acc[MT][NT];
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

        // FULL: all four 32-row MFMA tiles hold rows (no branches inside the stage)
        // sp: sub-stage within the super-stage (scale byte), slot: chunk registers
        auto compute = [&](auto full, int st, int set, int slot, int sp) {
            constexpr bool FULL = decltype(full)::value;
            const uint8_t* at = atile + (st & 1) * kPATile;
            u32x4 t[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j)
                t[j] = mytab[__builtin_amdgcn_ubfe(wsc[set][j], wsh[set] + 8u * sp, 8)];
            // software pipeline over the four kq-steps: the A fragments and decoded weights of
            // step q + 1 are produced while the MFMAs of step q run
            u32x4 av[2][MT], b[2][NT];
            auto read_a = [&](int q, u32x4* dst) {
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    if (FULL || i < mt_act)
                        dst[i] = *reinterpret_cast<const u32x4*>(at + (a_rd0 ^ (16 * q)) + i * 32 * 128);
            };
            read_a(0, av[0]);
#pragma unroll
            for (int j = 0; j < NT; ++j) b[0][j] = decode8(wc[j][slot][0], t[j]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int cur = q & 1, nxt = cur ^ 1;
                if (q < 3) read_a(q + 1, av[nxt]);
                __builtin_amdgcn_sched_barrier(0);
                if (q < 3) {
#pragma unroll
                    for (int j = 0; j < NT; ++j) b[nxt][j] = decode8(wc[j][slot][q + 1], t[j]);
                }
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    if (FULL || i < mt_act)
#pragma unroll
                        for (int j = 0; j < NT; ++j)
                            acc[i][j] = mfma32x32x16(av[cur][i], b[cur][j], acc[i][j]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // Stage st: the activations of stage st + 1 go out by DMA into the other LDS buffer,
        // then the weight loads of this stage (if any); stage st computes; the activations of
        // stage st + 1 are waited for (loads return in order, so the weights issued after them
        // stay in flight) and one barrier closes the stage. The scale sets alternate by
        // unrolling two super-stages; the steps past the last stage only load.
        auto run = [&](auto full) {
            wload(0, 0, S == 4 ? 2 : 1, true, 0);
            dma(0);
            MOEQ_WAIT_VMCNT(0);
            __syncthreads();
            for (int st0 = 0; st0 < nstages; st0 += 2 * S) {
#pragma unroll
                for (int r = 0; r < 2 * S; ++r) {
                    const int st = st0 + r;
                    const int m = st0 / S + r / S, sp = r % S, set = (r / S) & 1;
                    dma(st + 1);
                    int nw = 0;
                    if (S == 1) {
                        wload(m + 1, set ^ 1, 1, true, set ^ 1);
                        nw = 2 * NT;
                    } else if (sp == 0) {
                        wload(m, 2, 2, false, set);
                        nw = 2 * NT;
                    } else if (sp == 2) {
                        wload(m + 1, 0, 2, true, set ^ 1);
                        nw = 3 * NT;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if (st < nstages) compute(full, st, set, S == 1 ? set : sp, sp);
                    __builtin_amdgcn_sched_barrier(0);
                    if (nw == 3 * NT) MOEQ_WAIT_VMCNT(3 * NT);
                    else if (nw == 2 * NT) MOEQ_WAIT_VMCNT(2 * NT);
                    else MOEQ_WAIT_VMCNT(0);
                    __syncthreads();
                }
            }
        };
        if (mt_act == MT) run(std::true_type{});
        else run(std::false_type{});

        // ---- epilogue: lane holds rows 8 (r / 4) + 4 h + r % 4 of column cl; row offsets are
        // split into the lane's 4 h and a wavefront-uniform rest ----
        int el = lane;
        asm volatile("" : "+v"(el));              // computed here, not kept live across the loop
        const int hr = 4 * (el >> 5), ecl = el & 31;
        if (GATEUP) {
            const int ch = cb * 128 + wave * 32 + ecl;
            const int slotc = (ch & ~7) | (((ch & 1) << 2) | ((ch & 7) >> 1));
            uint16_t* ob = reinterpret_cast<uint16_t*>(a.out) + (size_t)(r0 + hr) * a.out_ld + slotc;
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                if (i >= mt_act) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int c = i * 32 + 8 * (r >> 2) + (r & 3);
                    if (hr >= rows - c || ch >= N) continue;
                    const float v =
                        badtab ? __builtin_nanf("") : silu_mul(acc[i][0][r], acc[i][1][r]);
                    ob[(size_t)c * a.out_ld] = (uint16_t)f32_to_bf16_rne(v);
                }
            }
        } else {
            const int col = cb * 256 + wave * 64 + ecl;
            float* ob = reinterpret_cast<float*>(a.out) + (size_t)(r0 + hr) * a.out_ld + col;
            const int32_t* sp = a.sorted_pair + r0 + hr;
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                if (i >= mt_act) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int c = i * 32 + 8 * (r >> 2) + (r & 3);
                    if (hr >= rows - c) continue;
                    const float wgt = badtab ? __builtin_nanf("") : a.topk_w[sp[c]];
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        if (col + 32 * j < N) ob[(size_t)c * a.out_ld + 32 * j] = wgt * acc[i][j][r];
                }
            }
        }
    }
}

int prefill_tile_rows() { return kPBM; }

size_t prefill_split_bytes(int T, int H) { return ((size_t)T * H * 2 + 255) & ~(size_t)255; }

void launch_pair_split_rows(const uint16_t* x, int T, int H, uint16_t* xs, int cus,
                            hipStream_t stream) {
    const long units = (long)T * H / 8;
    const long blocks = std::max(1L, std::min((units + 255) / 256, (long)cus * 8));
    hipLaunchKernelGGL(pair_split_rows_kernel, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x4*>(xs), units);
}

// tiles: host upper bound of the 128-row tiles the device will find
void launch_prefill(const SkinnyArgs& a, bool gateup, long tiles, int cus, hipStream_t stream) {
    const size_t lds = (size_t)a.tables.n * 256 * 16 + 2 * kPATile;
    const long ncb = gateup ? (a.N + 127) / 128 : (a.N + 255) / 256;
    long blocks = std::min(tiles * ncb, (long)cus * 2);
    if (blocks >= 8) blocks -= blocks % 8;                       // whole rounds over the XCDs
    blocks = std::max(1L, blocks);
    const bool wide = a.K % 128 == 0;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(kPThreads), lds, stream, a);
    };
    if (gateup) {
        if (wide) go(prefill_kernel<true, 4>); else go(prefill_kernel<true, 1>);
    } else {
        if (wide) go(prefill_kernel<false, 4>); else go(prefill_kernel<false, 1>);
    }
}

}  // namespace moeq
