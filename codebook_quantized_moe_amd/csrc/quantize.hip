// Encoding bf16 expert weights into the 4-bit format, the weighted Lloyd-Max statistics of a
// grid fit, and the per-expert choice between two tables (GLM-5.2-NF4-Lloyd-Experts-GPTQ
// model card). "Codes are indices into the per-layer grid": a block of 32 along K takes the
// least exponent e for which the grid's top magnitude times 2^e reaches the block's largest
// magnitude, stored as the byte e + 127, and each weight the grid magnitude nearest to
// |w| / 2^e. "What this is": the layer's magnitudes come from a Lloyd-Max fit to those
// ratios over all experts' matrices together, a ratio weighted by (2^e)^2. "Provenance":
// each expert keeps whichever of the fitted grid and an E2M1 control table encodes it better.
//
// One wavefront per weight row, 16 blocks of 32 at a time: lane l holds 8 weights (one
// 16-byte load; the wavefront reads 1 KiB of the row contiguously) of block l / 4, the four
// lanes of a block agree on its maximum through two DPP swaps, and each stores its 4 code
// bytes (64 lanes: 256 contiguous bytes). The ratio |w| / 2^e of a bf16 weight is exact in
// fp64, and so are the midpoints of two fp32 magnitudes, so the nearest-magnitude decision
// (ties to the lower) is exact. It is taken in fp32 where that is exact too: the ratio is an
// fp32 value unless it falls below the normal range (then fp64 decides), and for an fp32 r,
// r > m exactly when r is above the largest fp32 value not above m. The kernel is specialised
// on its outputs (codes and scales, row errors, or both), so the packing pass does no error
// work. Sums are fp64, each lane's in block order, then across lanes in a fixed butterfly, then
// across rows in row order: the same inputs give the same bits.
#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

constexpr int kQThreads = 256;
constexpr int kQWaves = kQThreads / 64;

struct BlockCode {
    int s;          // scale byte (255: a weight of the block is not finite)
    int e;          // exponent the ratios use
};

// Scale byte of a block whose largest magnitude has bf16 bits amax (sign cleared): the
// smallest e with gmax * 2^e >= amax, clamped to [-127, 127]; 0 for an all-zero block.
__device__ inline BlockCode block_code(uint32_t amax, float gmax) {
    BlockCode bc;
    if (amax >= 0x7F80u || !(gmax > 0.0f)) { bc.s = 255; bc.e = 0; return bc; }
    if (amax == 0) { bc.s = 0; bc.e = -127; return bc; }
    const double a = (double)__uint_as_float(amax << 16);
    const double g = (double)gmax;
    int ea, eg;
    (void)frexp(a, &ea);
    (void)frexp(g, &eg);
    int e = ea - eg;
    while (ldexp(g, e) < a) ++e;
    while (ldexp(g, e - 1) >= a) --e;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    bc.s = e + 127;
    bc.e = e;
    return bc;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Lane l of a wavefront at group i of a row: block 16 i + l / 4, weights 8 (l % 4) .. + 7 of it
// as 4 dwords (two weights each, even K low); zeros past the row's last block.
__device__ __forceinline__ u32x4 load_quarter(const uint16_t* row, int nb, int i, int lane) {
    const int b = 16 * i + (lane >> 2);
    if (b >= nb) return u32x4{0u, 0u, 0u, 0u};
    return __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(row + (size_t)b * 32 + (lane & 3) * 8));
}

// largest bf16 magnitude of the block of 32 that a quad of lanes holds (in all four lanes)
__device__ __forceinline__ uint32_t quad_amax(const u32x4 h) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, max(h[i] & 0x7FFFu, (h[i] >> 16) & 0x7FFFu));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
    return m;
}

// index of the magnitude nearest to ratio r (mid: the 7 exact midpoints, ascending)
__device__ __forceinline__ int nearest(double r, const double (&mid)[7]) {
    int m = 0;
#pragma unroll
    for (int i = 0; i < 7; ++i) m += r > mid[i];
    return m;
}

// index of the magnitude nearest to an fp32 ratio r, exact when r is: for an fp32 value r and a
// real midpoint m, r > m exactly when r > the largest fp32 value not above m (mid32)
__device__ __forceinline__ int nearest32(float r, const float (&mid32)[7]) {
    int m = 0;
#pragma unroll
    for (int i = 0; i < 7; ++i) m += r > mid32[i];
    return m;
}

// CODES: write codes and/or scales (whichever is given); ERR: the row's squared reconstruction
// error (either or both)
template <bool CODES, bool ERR>
__global__ void __launch_bounds__(kQThreads) quantize_kernel(const uint16_t* __restrict__ w,
                                                             long long rows, int K, int N,
                                                             TableArgs ta,
                                                             const uint8_t* __restrict__ table_id,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales,
                                                             double* __restrict__ row_err) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * kQWaves + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int t = table_id[row / N];
    const bool badtab = t >= ta.n;
    float g[8];
    double mid[7];
    float mid32[7];
#pragma unroll
    for (int m = 0; m < 8; ++m) g[m] = badtab ? 0.f : ta.v[t][m];
#pragma unroll
    for (int i = 0; i < 7; ++i) {
        mid[i] = 0.5 * ((double)g[i] + (double)g[i + 1]);          // exact in fp64
        float f = (float)mid[i];
        if ((double)f > mid[i]) f = __uint_as_float(__float_as_uint(f) - 1u);   // f > 0 here
        mid32[i] = f;
    }
    const uint16_t* wr = w + (size_t)row * K;
    const int nb = K / 32;
    const int q = lane & 3;
    double err = 0.0;
    for (int i = 0; 16 * i < nb; ++i) {
        const int b = 16 * i + (lane >> 2);
        const u32x4 h = load_quarter(wr, nb, i, lane);
        // an unknown table id encodes NaN blocks (gmax is then 0: block_code gives 255)
        const BlockCode bc = block_code(quad_amax(h), g[7]);
        const double inv = ldexp(1.0, -bc.e);
        const float invf = (float)inv;                              // a power of two: exact
        // the block's 8 reconstructions bf16(g[m] * 2^e): lane q of the quad forms those of
        // magnitudes 2q and 2q + 1, and four DPP broadcasts give every lane all four pairs
        uint32_t pr[4] = {0u, 0u, 0u, 0u};
        if (ERR) {
            const float ga = q == 0 ? g[0] : q == 1 ? g[2] : q == 2 ? g[4] : g[6];
            const float gb = q == 0 ? g[1] : q == 1 ? g[3] : q == 2 ? g[5] : g[7];
            const int own = (int)(scaled_bf16_bits(ga, bc.s) | (scaled_bf16_bits(gb, bc.s) << 16));
            pr[0] = (uint32_t)__builtin_amdgcn_update_dpp(0, own, 0x00, 0xF, 0xF, false);
            pr[1] = (uint32_t)__builtin_amdgcn_update_dpp(0, own, 0x55, 0xF, 0xF, false);
            pr[2] = (uint32_t)__builtin_amdgcn_update_dpp(0, own, 0xAA, 0xF, 0xF, false);
            pr[3] = (uint32_t)__builtin_amdgcn_update_dpp(0, own, 0xFF, 0xF, 0xF, false);
        }
        if (b >= nb) continue;
        uint32_t packed = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t hb = (h[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
            const uint32_t mag_bits = hb & 0x7FFFu;
            const bool neg = (hb & 0x8000u) && mag_bits != 0;
            // |w| / 2^e is a bf16 value times a power of two: exact in fp32 unless it falls
            // below the normal range, where the decision is taken in fp64
            const float magf = bf16_to_f32(mag_bits);
            const float rf = magf * invf;
            int m = nearest32(rf, mid32);
            if (rf < 0x1p-126f && mag_bits != 0) m = nearest((double)magf * inv, mid);
            if (ERR) {
                const double x = (double)bf16_to_f32(hb);
                const uint32_t pm = m < 2 ? pr[0] : m < 4 ? pr[1] : m < 6 ? pr[2] : pr[3];
                const float rm = bf16_to_f32((m & 1) ? pm >> 16 : pm & 0xFFFFu);
                const double d = x - (neg ? -(double)rm : (double)rm);
                err += d * d;
            }
            const uint32_t code = bc.s == 255 ? 0u : (uint32_t)m | (neg ? 8u : 0u);
            packed |= code << (4 * j);
        }
        if (ERR && bc.s == 255) err += __builtin_nan("");
        if (CODES) {
            if (codes)
                *reinterpret_cast<uint32_t*>(codes + (size_t)row * (K / 2) + (size_t)b * 16 + q * 4) =
                    packed;
            if (scales && q == 0) scales[(size_t)row * nb + b] = (uint8_t)bc.s;
        }
    }
    if (ERR) {
        err = wave_sum_f64(err);
        if (lane == 0) row_err[row] = err;
    }
}

// Per workgroup (its 4 waves' rows), 24 fp64 sums: for magnitude m, sum (2^e)^2 r, sum (2^e)^2 and
// sum (2^e)^2 (r - g[m])^2 over the ratios nearest to it; e for the top magnitude gmax.
// Each lane adds (2^e)^2 r, (2^e)^2 and (2^e)^2 r^2 into its own LDS slots of the weight's
// magnitude (slot [wave][sum][m][lane]: no two lanes share a slot, so the adds of a slot
// happen in the lane's program order); the squared distance is formed from the three sums
// at the end, in fp64.
constexpr int kLloydStats = 24;

__global__ void __launch_bounds__(kQThreads) lloyd_stats_kernel(const uint16_t* __restrict__ w,
                                                                long long rows, int K, Table8 tab,
                                                                float gmax,
                                                                double* __restrict__ part) {
    __shared__ double slot[kQWaves][3][8][64];
    __shared__ double wsum[kQWaves][kLloydStats];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double mid[7];
#pragma unroll
    for (int i = 0; i < 7; ++i) mid[i] = 0.5 * ((double)tab.v[i] + (double)tab.v[i + 1]);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        slot[wave][0][m][lane] = 0.0;
        slot[wave][1][m][lane] = 0.0;
        slot[wave][2][m][lane] = 0.0;
    }
    // rows blockIdx.x * 4 + wave, then every gridDim.x * 4 rows after it
    for (long long row = (long long)blockIdx.x * kQWaves + wave; row < rows;
         row += (long long)gridDim.x * kQWaves) {
        const uint16_t* wr = w + (size_t)row * K;
        const int nb = K / 32;
        for (int i = 0; 16 * i < nb; ++i) {
            const u32x4 h = load_quarter(wr, nb, i, lane);
            const BlockCode bc = block_code(quad_amax(h), gmax);
            if (16 * i + (lane >> 2) >= nb || bc.s == 255) continue;   // past the row; non-finite
            const double inv = ldexp(1.0, -bc.e);
            const double wt = ldexp(1.0, 2 * bc.e);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t hb = (h[j >> 1] >> (16 * (j & 1))) & 0x7FFFu;
                const double r = (double)bf16_to_f32(hb) * inv;
                const int m = nearest(r, mid);
                const double wr1 = wt * r;
                __hip_atomic_fetch_add(&slot[wave][0][m][lane], wr1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_add(&slot[wave][1][m][lane], wt, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_add(&slot[wave][2][m][lane], wr1 * r, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const double a = wave_sum_f64(slot[wave][0][m][lane]);
        const double c = wave_sum_f64(slot[wave][1][m][lane]);
        const double q = wave_sum_f64(slot[wave][2][m][lane]);
        if (lane == 0) {
            const double g = (double)tab.v[m];
            wsum[wave][m] = a;
            wsum[wave][8 + m] = c;
            wsum[wave][16 + m] = q - 2.0 * g * a + g * g * c;
        }
    }
    __syncthreads();
    if (threadIdx.x < kLloydStats) {
        double v = 0.0;
#pragma unroll
        for (int q = 0; q < kQWaves; ++q) v += wsum[q][threadIdx.x];
        part[(size_t)blockIdx.x * kLloydStats + threadIdx.x] = v;
    }
}

// stats[i] (+)= the sum of the nparts partial sums of statistic i (workgroup i): thread t adds
// parts t, t + 256, ... in order, then a fixed tree over the 256 threads.
__global__ void __launch_bounds__(256) lloyd_reduce_kernel(const double* __restrict__ part,
                                                           int nparts, int accumulate,
                                                           double* __restrict__ stats) {
    __shared__ double t[256];
    const int i = blockIdx.x;
    double v = 0.0;
    for (int p = threadIdx.x; p < nparts; p += 256) v += part[(size_t)p * kLloydStats + i];
    t[threadIdx.x] = v;
    __syncthreads();
    for (int n = 128; n > 0; n >>= 1) {
        if (threadIdx.x < n) t[threadIdx.x] += t[threadIdx.x + n];
        __syncthreads();
    }
    if (threadIdx.x == 0) stats[i] = accumulate ? stats[i] + t[0] : t[0];
}

// Per expert: the row errors of two encodings summed in row order (added to expert_err when
// accumulating over several matrices of the experts); table id 1 when the second total is
// strictly smaller.
__global__ void __launch_bounds__(64) select_arms_kernel(const double* __restrict__ err_a,
                                                         const double* __restrict__ err_b,
                                                         int N, int accumulate,
                                                         uint8_t* __restrict__ table_id,
                                                         double* __restrict__ expert_err) {
    const int e = blockIdx.x, lane = threadIdx.x;
    double a = 0.0, b = 0.0;
    for (int r = lane; r < N; r += 64) {
        a += err_a[(size_t)e * N + r];
        b += err_b[(size_t)e * N + r];
    }
    a = wave_sum_f64(a);
    b = wave_sum_f64(b);
    if (lane == 0) {
        if (accumulate) { a += expert_err[2 * e]; b += expert_err[2 * e + 1]; }
        table_id[e] = b < a ? 1 : 0;
        if (expert_err) { expert_err[2 * e] = a; expert_err[2 * e + 1] = b; }
    }
}

void launch_quantize(const uint16_t* w, long long rows, int K, int N, const TableArgs& ta,
                     const uint8_t* table_id, uint8_t* codes, uint8_t* scales, double* row_err,
                     hipStream_t stream) {
    const long long blocks = (rows + kQWaves - 1) / kQWaves;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kQThreads), 0, stream, w, rows, K,
                           N, ta, table_id, codes, scales, row_err);
    };
    // CODES: codes or scales (or both) are written; ERR: row errors
    const bool want_codes = codes != nullptr || scales != nullptr;
    if (want_codes && row_err) go(quantize_kernel<true, true>);
    else if (want_codes) go(quantize_kernel<true, false>);
    else if (row_err) go(quantize_kernel<false, true>);
}

// workgroups of the statistics pass: enough to fill the chip (3 per CU by LDS), few enough that
// the partial sums stay small
constexpr long long kLloydMaxGroups = 2048;

static int lloyd_groups(long long rows) {
    const long long g = (rows + kQWaves - 1) / kQWaves;
    return (int)(g < kLloydMaxGroups ? g : kLloydMaxGroups);
}

size_t lloyd_workspace_bytes(long long rows) {
    return (size_t)lloyd_groups(rows) * kLloydStats * sizeof(double);
}

void launch_lloyd_stats(const uint16_t* w, long long rows, int K, const Table8& tab, float gmax,
                        double* part, int accumulate, double* stats, hipStream_t stream) {
    const int groups = lloyd_groups(rows);
    hipLaunchKernelGGL(lloyd_stats_kernel, dim3(groups), dim3(kQThreads), 0, stream, w, rows, K,
                       tab, gmax, part);
    hipLaunchKernelGGL(lloyd_reduce_kernel, dim3(kLloydStats), dim3(256), 0, stream, part, groups,
                       accumulate, stats);
}

void launch_select_arms(const double* err_a, const double* err_b, int E, int N, int accumulate,
                        uint8_t* table_id, double* expert_err, hipStream_t stream) {
    hipLaunchKernelGGL(select_arms_kernel, dim3(E), dim3(64), 0, stream, err_a, err_b, N,
                       accumulate, table_id, expert_err);
}

}  // namespace moeq
