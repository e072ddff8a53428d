// Grouped projections for few rows per expert (decode): the weights are the traffic.
//
// Work item = (active expert e, block of 16 weight rows). One wavefront owns an item and
// streams its weight rows once along K, decoding the codes in registers straight into MFMA
// B-operands (no LDS round trip for weights), for all of the expert's sorted rows in blocks
// of 16 (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// Per K-step of 256, lane (n = lane & 15, g = lane >> 4) loads 32 contiguous code bytes of
// weight row n (64 codes = two E8M0 blocks; 16 rows x 128 contiguous bytes per wavefront) and
// the two scale bytes, fetches the two decode tables of those scale bytes from LDS, and
// feeds 8 MFMAs; MFMA d contracts the K indices 64g + 8d + {0,2,4,6,1,3,5,7} of the step
// (the decode's pair-split order), which the activation operand mirrors.
//
// gate|up ("Round 7" brief, decision 4): the gate row and the up row of the same channel are
// decoded side by side into two accumulators; the epilogue writes bf16(silu(g) * u).
// down ("Round 7" brief, decision 6; README "What had to be fixed": router weighting in the
// down epilogue): the epilogue writes topk_w[p] * (I . Wd) in fp32.
// The grid is persistent: each workgroup builds the decode tables and the active-expert list
// once, then its wavefronts stride over the items. No host synchronisation is needed: the
// expert row counts are read from expert_offsets on the device.
#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

constexpr int kSkinnyWaves = 4;

__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Compact list of experts with at least one row, ascending; returns the count. All threads.
__device__ inline int active_experts(const int32_t* offsets, int E, int* active, int* n_s) {
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < 64) {
        int has[4], c = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane * 4 + j;
            has[j] = (e < E) && (offsets[e + 1] > offsets[e]);
            c += has[j];
        }
        int incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        int pos = incl - c;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (has[j]) active[pos++] = lane * 4 + j;
        if (lane == 63) *n_s = incl;
    }
    __syncthreads();
    return *n_s;
}

template <bool GATEUP>
__global__ void __launch_bounds__(64 * kSkinnyWaves) skinny_kernel(const SkinnyArgs a) {
    extern __shared__ u32x4 tab[];
    __shared__ int active[256];
    __shared__ int n_active_s;
    build_decode_tables(a.tables, tab);
    const int nact = active_experts(a.offsets, a.E, active, &n_active_s);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nl = lane & 15, g = lane >> 4;
    const int nblk = a.N / 16;
    const long items = (long)nact * nblk;
    const int kb = a.K / 2, ks = a.K / 32;

    for (long item = (long)blockIdx.x * kSkinnyWaves + wave; item < items;
         item += (long)gridDim.x * kSkinnyWaves) {
        const int e = active[item / nblk];
        const int nb = (int)(item % nblk);
        const int r0 = a.offsets[e];
        const int Me = a.offsets[e + 1] - r0;
        const int tsel = a.table_id[e];
        const bool badtab = tsel >= a.tables.n;
        const u32x4* mytab = tab + (badtab ? 0 : tsel) * 256;
        const size_t wrow = (size_t)e * a.N + (size_t)nb * 16 + nl;
        const uint8_t* c0 = a.codes0 + wrow * kb + g * 32;
        const uint8_t* s0 = a.scales0 + wrow * ks + g * 2;
        const uint8_t* c1 = GATEUP ? a.codes1 + wrow * kb + g * 32 : nullptr;
        const uint8_t* s1 = GATEUP ? a.scales1 + wrow * ks + g * 2 : nullptr;

        for (int m0 = 0; m0 < Me; m0 += 16) {
            const int am = m0 + nl;                       // this lane's activation row
            const bool arow = am < Me;
            const uint16_t* ap = nullptr;
            if (arow) {
                const size_t src = GATEUP ? (size_t)(a.sorted_pair[r0 + am] / a.k)
                                          : (size_t)(r0 + am);
                ap = a.act + src * a.K + g * 64;
            }
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
            for (int kk = 0; kk < a.K; kk += 256) {
                const bool kval = kk + g * 64 < a.K;
                u32x4 cg0 = {0, 0, 0, 0}, cg1 = {0, 0, 0, 0}, cu0 = {0, 0, 0, 0},
                      cu1 = {0, 0, 0, 0};
                uint32_t sg = 127u | (127u << 8), su = sg;
                if (kval) {
                    cg0 = ld16(c0 + kk / 2);
                    cg1 = ld16(c0 + kk / 2 + 16);
                    sg = *reinterpret_cast<const uint16_t*>(s0 + kk / 32);
                    if (GATEUP) {
                        cu0 = ld16(c1 + kk / 2);
                        cu1 = ld16(c1 + kk / 2 + 16);
                        su = *reinterpret_cast<const uint16_t*>(s1 + kk / 32);
                    }
                }
                const u32x4 tg0 = mytab[sg & 0xFFu], tg1 = mytab[(sg >> 8) & 0xFFu];
                u32x4 tu0 = tg0, tu1 = tg1;
                if (GATEUP) { tu0 = mytab[su & 0xFFu]; tu1 = mytab[(su >> 8) & 0xFFu]; }
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    u32x4 A = {0, 0, 0, 0};
                    if (arow && kval) {
                        A = ld16(ap + kk + 8 * d);
                        if (GATEUP) A = pair_split(A);    // x is stored in natural order
                    }
                    const uint32_t cw = d < 4 ? cg0[d & 3] : cg1[d & 3];
                    acc0 = mfma16x16x32(A, decode8(cw, d < 4 ? tg0 : tg1), acc0);
                    if (GATEUP) {
                        const uint32_t cv = d < 4 ? cu0[d & 3] : cu1[d & 3];
                        acc1 = mfma16x16x32(A, decode8(cv, d < 4 ? tu0 : tu1), acc1);
                    }
                }
            }
            // C layout: lane holds rows 4g + i (i = 0..3) of column nl
            const int col = nb * 16 + nl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mm = m0 + 4 * g + i;
                if (mm >= Me) continue;
                const size_t r = (size_t)(r0 + mm);
                if (GATEUP) {
                    const float h = badtab ? __builtin_nanf("") : silu_mul(acc0[i], acc1[i]);
                    uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
                    const int slot = (col & ~7) | (((col & 1) << 2) | ((col & 7) >> 1));
                    out[r * a.out_ld + slot] = (uint16_t)f32_to_bf16_rne(h);
                } else {
                    const float wgt = a.topk_w[a.sorted_pair[r]];
                    float* out = reinterpret_cast<float*>(a.out);
                    out[r * a.out_ld + col] = badtab ? __builtin_nanf("") : wgt * acc0[i];
                }
            }
        }
    }
}

void launch_skinny(const SkinnyArgs& a, bool gateup, int blocks, hipStream_t stream) {
    const size_t lds = (size_t)a.tables.n * 256 * sizeof(u32x4);
    if (gateup)
        hipLaunchKernelGGL(skinny_kernel<true>, dim3(blocks), dim3(64 * kSkinnyWaves), lds, stream,
                           a);
    else
        hipLaunchKernelGGL(skinny_kernel<false>, dim3(blocks), dim3(64 * kSkinnyWaves), lds,
                           stream, a);
}

// ---------------------------------------------------------------------------------------------
// debug decode: whole matrices through decode8 + the LDS tables, written in natural K order
// ---------------------------------------------------------------------------------------------

__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, int E,
                                                      int N, int K, const uint8_t* table_id,
                                                      TableArgs ta, uint16_t* __restrict__ out) {
    extern __shared__ u32x4 tab[];
    build_decode_tables(ta, tab);
    const size_t dw_per_row = (size_t)K / 8;
    const size_t total = (size_t)E * N * dw_per_row;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        const size_t row = i / dw_per_row;
        const int dd = (int)(i % dw_per_row);
        const int e = (int)(row / N);
        const int tsel = table_id[e];
        const uint32_t c = *reinterpret_cast<const uint32_t*>(codes + row * (K / 2) + dd * 4);
        const int s = scales[row * (K / 32) + dd / 4];
        u32x4 v;
        if (tsel >= ta.n) {
            v = u32x4{0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
        } else {
            v = pair_join(decode8(c, tab[tsel * 256 + s]));
        }
        *reinterpret_cast<u32x4*>(out + row * K + (size_t)dd * 8) = v;
    }
}

void launch_dequant(const uint8_t* codes, const uint8_t* scales, int E, int N, int K,
                    const uint8_t* table_id, const TableArgs& ta, uint16_t* out, int blocks,
                    hipStream_t stream) {
    const size_t lds = (size_t)ta.n * 256 * sizeof(u32x4);
    hipLaunchKernelGGL(dequant_kernel, dim3(blocks), dim3(256), lds, stream, codes, scales, E, N,
                       K, table_id, ta, out);
}

}  // namespace moeq
