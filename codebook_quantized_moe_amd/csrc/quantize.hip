// Encoding bf16 expert weights into the 4-bit format, the weighted Lloyd-Max statistics of a
// grid fit, and the per-expert choice between two tables (GLM-5.2-NF4-Lloyd-Experts-GPTQ
// model card). "Codes are indices into the per-layer grid": a block of 32 along K takes the
// least exponent e for which the grid's top magnitude times 2^e reaches the block's largest
// magnitude, stored as the byte e + 127, and each weight the grid magnitude nearest to
// |w| / 2^e. "What this is": the layer's magnitudes come from a Lloyd-Max fit to those
// ratios over all experts' matrices together, a ratio weighted by (2^e)^2. "Provenance":
// each expert keeps whichever of the fitted grid and an E2M1 control table encodes it better.
//
// A wavefront takes 8 consecutive weight rows, one after the other, 16 blocks of 32 at a time
// (the next 16 loaded while these are encoded): lane l holds 8 weights (one 16-byte load; the
// wavefront reads 1 KiB of the row contiguously) of block l / 4, the four
// lanes of a block agree on its maximum through two DPP swaps, and each stores its 4 code
// bytes (64 lanes: 256 contiguous bytes). The ratio |w| / 2^e of a bf16 weight is exact in
// fp64, and so are the midpoints of two fp32 magnitudes, so the nearest-magnitude decision
// (ties to the lower) is exact. Almost every block takes it, its scale byte and its
// reconstructions in integer arithmetic on bf16 bits, two weights per instruction (the block
// maximum's and the top magnitude's exponent fields give the scale byte; thresholds and
// reconstructions scale by adding e << 7 while they stay normal). The other blocks (a
// subnormal maximum, thresholds below the normal range) decide on the ratio: in fp32 where
// that is exact (for an fp32 r, r > m exactly when r is above the largest fp32 value not above
// m), in fp64 below fp32's normal range. The kernel is specialised on its outputs (codes and
// scales, row errors, or both), so the packing pass does no error work. Sums are fp64, each lane's in block order, then across lanes in a fixed butterfly, then
// across rows in row order: the same inputs give the same bits.
#include "moeq_device.h"
#include "moeq_kernels.h"

namespace moeq {

constexpr int kQThreads = 256;
constexpr int kQWaves = kQThreads / 64;
constexpr int kQRowsPerWave = 8;     // consecutive rows per wavefront (one table while N % 8 == 0)

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

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// The nearest-magnitude decision in bf16 bits, two weights at a time. For a bf16 magnitude |w|
// and a real threshold M >= 0, |w| > M exactly when bits(|w|) > bits(floor_bf16(M)) (the bits
// of non-negative bf16 values are ordered as the values). With M = mid_i * 2^e:
// floor_bf16(mid_i * 2^e) = floor_bf16(mid_i) * 2^e while both stay normal, whose bits are
// bits(floor_bf16(mid_i)) + (e << 7); above the largest finite value the threshold saturates
// to 0x7FFF, which no finite magnitude exceeds. floor_bf16(mid_i) is the top half of the bits
// of floor_fp32(mid_i). So a row keeps q_i = bits(floor_bf16(mid_i)) - (127 << 7) and a block
// adds s << 7 (s = e + 127) with signed saturation. The thresholds ascend with i (the tables
// do), so the index is a binary search of three tests, [|w| > t] = bit 15 of (t - |w|) mod
// 2^16 (t and |w| both below 2^15), the result of one test selecting the next threshold.
struct FastRow {
    i16x2 q[7];
    int pexp;          // smallest exponent field of the floor_bf16(mid_i)
    int gexp;          // exponent field and mantissa bits of the top magnitude (fp32)
    uint32_t gmant;
    bool ok;           // every floor_bf16(mid_i) is normal and the top magnitude is a normal fp32
};

// Round-to-nearest-even of a finite fp32 to bf16 bits.
__device__ __forceinline__ uint32_t rne16(uint32_t b) { return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16; }

// The thresholds of a row: q_i, the smallest exponent field, and whether the fast decision
// applies to the row at all; the block exponent's inputs from the top magnitude gmax.
__device__ __forceinline__ void fast_row(FastRow& fr, const float (&mid32)[7], float gmax) {
    fr.pexp = 255;
    fr.ok = true;
#pragma unroll
    for (int i = 0; i < 7; ++i) {
        const uint32_t p = __float_as_uint(mid32[i]) >> 16;         // floor_bf16(mid_i)
        fr.ok = fr.ok && p >= 0x80u;
        fr.pexp = min(fr.pexp, (int)(p >> 7));
        const int16_t q = (int16_t)((int)p - (127 << 7));
        fr.q[i] = i16x2{q, q};
    }
    const uint32_t gb = __float_as_uint(gmax);
    fr.gexp = (int)(gb >> 23);
    fr.gmant = gb & 0x7FFFFFu;
    fr.ok = fr.ok && fr.gexp >= 1 && fr.gexp <= 254;
}

// Scale byte of a block from exponent fields, when the block maximum amax (bf16 bits, sign
// clear) is zero or normal and the row is fast: the least e with gmax * 2^e >= amax is the
// exponent difference, plus one when gmax's significand is below amax's (the rule block_code
// applies in fp64). Returns false when the block needs block_code or the exact decision: a
// non-finite or subnormal maximum, or thresholds that would leave the normal range.
__device__ __forceinline__ bool fast_scale(const FastRow& fr, uint32_t amax, int& s) {
    s = 0;
    if (!fr.ok || amax >= 0x7F80u) return false;
    if (amax == 0) return true;
    if (amax < 0x80u) return false;
    int e = (int)(amax >> 7) - fr.gexp + (fr.gmant < ((amax & 0x7Fu) << 16) ? 1 : 0);
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    s = e + 127;
    return s + fr.pexp >= 128;
}

// The 7 thresholds of a fast block, two copies per dword (an all-zero block takes thresholds
// above every magnitude: index 0 throughout)
__device__ __forceinline__ void block_thresholds(const FastRow& fr, uint32_t amax, int s,
                                                 uint32_t (&tt)[7]) {
    const int16_t sh = (int16_t)((amax == 0 ? 254 : s) << 7);
#pragma unroll
    for (int k = 0; k < 7; ++k)
        tt[k] = __builtin_bit_cast(uint32_t, __builtin_elementwise_add_sat(fr.q[k], i16x2{sh, sh}));
}

__device__ __forceinline__ uint32_t bitsel(uint32_t mask, uint32_t a, uint32_t b) {
    return (mask & a) | (~mask & b);                            // v_bfi_b32
}

// 0xFFFF in a half where |w| > t, else 0 (bit 15 of t - |w| spread by an arithmetic shift).
// The shift is written as the one instruction so that the compiler keeps the result a plain
// 32-bit mask (as a vector compare it would split every select below into halves).
__device__ __forceinline__ uint32_t above(uint32_t t2, uint32_t mag2) {
    const uint32_t d = as_u32(as_u16x2(t2) - as_u16x2(mag2));
    uint32_t m;
    asm("v_pk_ashrrev_i16 %0, 15, %1 op_sel_hi:[0,1]" : "=v"(m) : "v"(d));
    return m;
}

// magnitude indexes of the two weights of mag2 (one per half) against ascending thresholds t
__device__ __forceinline__ uint32_t nearest_pair(uint32_t mag2, const uint32_t (&t)[7]) {
    const uint32_t a2 = above(t[3], mag2);
    const uint32_t a1 = above(bitsel(a2, t[5], t[1]), mag2);
    const uint32_t t0 = bitsel(a1, bitsel(a2, t[6], t[2]), bitsel(a2, t[4], t[0]));
    const uint32_t a0 = above(t0, mag2);
    return (a2 & 0x00040004u) | (a1 & 0x00020002u) | (a0 & 0x00010001u);
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
    const long long row0 = ((long long)blockIdx.x * kQWaves + (threadIdx.x >> 6)) * kQRowsPerWave;
    if (row0 >= rows) return;
    const int nrow = rows - row0 < kQRowsPerWave ? (int)(rows - row0) : kQRowsPerWave;
    float g[8];
    double mid[7];
    float mid32[7];
    FastRow fr;
    // reconstructions by integer scaling: bf16(g * 2^e) = bf16(g) * 2^e while it is normal (the
    // rounding commutes with a power of two), i.e. bits(bf16(g)) + (e << 7), Inf above the
    // largest finite value. This lane's two magnitudes 2q, 2q + 1: r - (127 << 7) per half,
    // and a mask that keeps zero magnitudes zero.
    int rexp = 255;
    bool rok = true;
    uint32_t rq = 0u, rnz = 0u;
    // the constants of a row's table (recomputed when the table changes between rows)
    auto setup = [&](int t) __attribute__((always_inline)) {
        const bool badtab = t >= ta.n;
#pragma unroll
        for (int m = 0; m < 8; ++m) g[m] = badtab ? 0.f : ta.v[t][m];
#pragma unroll
        for (int i = 0; i < 7; ++i) {
            mid[i] = 0.5 * ((double)g[i] + (double)g[i + 1]);      // exact in fp64
            float f = (float)mid[i];
            if ((double)f > mid[i]) f = __uint_as_float(__float_as_uint(f) - 1u);   // f > 0 here
            mid32[i] = f;
        }
        fast_row(fr, mid32, g[7]);
        if (ERR) {
            rexp = 255;
            rok = true;
            rq = rnz = 0u;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const uint32_t r = rne16(__float_as_uint(g[m]));
                if (r != 0u) {
                    rexp = min(rexp, (int)(r >> 7));
                    rok = rok && (r >> 7) >= 1u && (r >> 7) <= 254u;
                }
                if ((m >> 1) == (lane & 3)) {
                    const int sh = 16 * (m & 1);
                    rq |= (((r - (127u << 7)) & 0xFFFFu) << sh);
                    rnz |= (r != 0u ? 0xFFFFu : 0u) << sh;
                }
            }
        }
    };
    const int nb = K / 32;
    const int iters = (nb + 15) / 16;
    const int q = lane & 3;
    int tcur = -1;
    double err = 0.0;
    // the wavefront's rows one after the other, each block's weights loaded one step ahead
    u32x4 hn = load_quarter(w + (size_t)row0 * K, nb, 0, lane);
    for (int r = 0, i = 0; r < nrow;) {
        const long long row = row0 + r;
        if (i == 0) {
            const int t = __builtin_amdgcn_readfirstlane((int)table_id[row / N]);
            if (t != tcur) { setup(t); tcur = t; }
            err = 0.0;
        }
        const u32x4 h = hn;
        const int ni = i + 1 == iters ? 0 : i + 1;
        const int nr = i + 1 == iters ? r + 1 : r;
        if (nr < nrow) hn = load_quarter(w + (size_t)(row0 + nr) * K, nb, ni, lane);
        const int b = 16 * i + (lane >> 2);
        const uint32_t amax = quad_amax(h);
        int sf;
        const bool fast = fast_scale(fr, amax, sf);
        // an unknown table id encodes NaN blocks (gmax is then 0: block_code gives 255)
        BlockCode bc;
        if (fast) { bc.s = sf; bc.e = sf - 127; }
        else bc = block_code(amax, g[7]);
        // the block's 8 reconstructions bf16(g[m] * 2^e): lane q of the quad forms those of
        // magnitudes 2q and 2q + 1, and four DPP broadcasts give every lane all four pairs
        uint32_t pr[4] = {0u, 0u, 0u, 0u};
        if (ERR) {
            uint32_t own;
            if (fast && rok && bc.s + rexp >= 128) {
                const int16_t sh = (int16_t)(bc.s << 7);
                const u16x2 v = __builtin_bit_cast(
                    u16x2, __builtin_elementwise_add_sat(__builtin_bit_cast(i16x2, rq), i16x2{sh, sh}));
                own = as_u32(__builtin_elementwise_min(v, u16x2{0x7F80, 0x7F80})) & rnz;
            } else {
                const float ga = q == 0 ? g[0] : q == 1 ? g[2] : q == 2 ? g[4] : g[6];
                const float gb = q == 0 ? g[1] : q == 1 ? g[3] : q == 2 ? g[5] : g[7];
                own = scaled_bf16_bits(ga, bc.s) | (scaled_bf16_bits(gb, bc.s) << 16);
            }
            pr[0] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)own, 0x00, 0xF, 0xF, false);
            pr[1] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)own, 0x55, 0xF, 0xF, false);
            pr[2] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)own, 0xAA, 0xF, 0xF, false);
            pr[3] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)own, 0xFF, 0xF, 0xF, false);
        }
        uint32_t packed = 0u;
        if (b >= nb) {
            // past the row's last block
        } else if (bc.s == 255) {
            // a non-finite weight: codes 0, the row's error NaN
            if (ERR) err += __builtin_nan("");
        } else if (fast) {
            uint32_t tt[7];
            block_thresholds(fr, amax, bc.s, tt);
            // reconstruction bytes by magnitude: low bytes of magnitudes 0..3 and 4..7, high
            // bytes likewise (v_perm selects byte m of the pair {x1, x0} for m = 0..7)
            const uint32_t lo0 = __builtin_amdgcn_perm(pr[1], pr[0], 0x06040200u);
            const uint32_t lo1 = __builtin_amdgcn_perm(pr[3], pr[2], 0x06040200u);
            const uint32_t hi0 = __builtin_amdgcn_perm(pr[1], pr[0], 0x07050301u);
            const uint32_t hi1 = __builtin_amdgcn_perm(pr[3], pr[2], 0x07050301u);
            uint32_t byte[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t hv = h[k];
                const uint32_t mag2 = hv & 0x7FFF7FFFu;
                const uint32_t m2 = nearest_pair(mag2, tt);
                if (CODES) {
                    // sign bit of a code: a negative weight other than -0
                    const uint32_t nz = as_u32(u16x2{0, 0} - as_u16x2(mag2));   // bit 15: |w| != 0
                    const uint32_t c2 = m2 | (((hv & nz) >> 12) & 0x00080008u);
                    byte[k] = c2 | (c2 >> 12);                  // low byte: even code | odd << 4
                }
                if (ERR) {
                    // reconstructions of the two weights with the weights' signs (a -0 weight
                    // takes -w_hat: the square is the same)
                    const uint32_t qv = __builtin_amdgcn_perm(lo1, lo0, m2 | 0x0C000C00u) |
                                        __builtin_amdgcn_perm(hi1, hi0, (m2 << 8) | 0x000C000Cu) |
                                        (hv & 0x80008000u);
                    const double d0 = (double)__uint_as_float(hv << 16) -
                                      (double)__uint_as_float(qv << 16);
                    err += d0 * d0;
                    const double d1 = (double)__uint_as_float(hv & 0xFFFF0000u) -
                                      (double)__uint_as_float(qv & 0xFFFF0000u);
                    err += d1 * d1;
                }
            }
            if (CODES)
                packed = __builtin_amdgcn_perm(byte[1], byte[0], 0x0C0C0400u) |
                         __builtin_amdgcn_perm(byte[3], byte[2], 0x04000C0Cu);
        } else {
            const double inv = ldexp(1.0, -bc.e);
            const float invf = (float)inv;                          // a power of two: exact
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t hb = (h[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
                const uint32_t mag_bits = hb & 0x7FFFu;
                const bool neg = (hb & 0x8000u) && mag_bits != 0;
                // |w| / 2^e is a bf16 value times a power of two: exact in fp32 unless it
                // falls below the normal range, where the decision is taken in fp64
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
                packed |= (uint32_t)(m | (neg ? 8 : 0)) << (4 * j);
            }
        }
        if (CODES && b < nb) {
            if (codes)
                *reinterpret_cast<uint32_t*>(codes + (size_t)row * (K / 2) + (size_t)b * 16 + q * 4) =
                    packed;
            if (scales && q == 0) scales[(size_t)row * nb + b] = (uint8_t)bc.s;
        }
        if (ERR && ni == 0) {
            const double tot = wave_sum_f64(err);
            if (lane == 0) row_err[row] = tot;
        }
        i = ni;
        r = nr;
    }
}

// Per workgroup (its 4 waves' rows), 24 fp64 sums: for magnitude m, sum (2^e)^2 r, sum (2^e)^2 and
// sum (2^e)^2 (r - g[m])^2 over the ratios nearest to it; e for the top magnitude gmax.
// Each lane adds (2^e)^2 r and (2^e)^2 r^2 into its own LDS slots of the weight's magnitude
// (slot [wave][sum][m][lane]: no two lanes share a slot, so the adds of a slot happen in the
// lane's program order) and keeps sum (2^e)^2 per magnitude in registers, as (2^e)^2 times
// the block's count; the squared distance is formed from the three sums at the end, in fp64.
constexpr int kLloydStats = 24;

__global__ void __launch_bounds__(kQThreads) lloyd_stats_kernel(const uint16_t* __restrict__ w,
                                                                long long rows, int K, Table8 tab,
                                                                float gmax,
                                                                double* __restrict__ part) {
    __shared__ double slot[kQWaves][2][8][64];
    __shared__ double wsum[kQWaves][kLloydStats];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double mid[7];
    float mid32[7];
#pragma unroll
    for (int i = 0; i < 7; ++i) {
        mid[i] = 0.5 * ((double)tab.v[i] + (double)tab.v[i + 1]);
        float f = (float)mid[i];
        if ((double)f > mid[i]) f = __uint_as_float(__float_as_uint(f) - 1u);
        mid32[i] = f;
    }
    FastRow fr;
    fast_row(fr, mid32, gmax);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        slot[wave][0][m][lane] = 0.0;
        slot[wave][1][m][lane] = 0.0;
    }
    // sum (2^e)^2 per magnitude: (2^e)^2 times the block's count, kept in registers
    double wsq[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) wsq[m] = 0.0;
    // (2^e)^2 r = 2^e |w| and (2^e)^2 r^2 = |w|^2 into the slots of the weight's magnitude m
    // (both products exact in fp64); cnt counts the lane's weights per magnitude, 4 bits each
    auto add2 = [&](int m, double a, double q2, uint32_t& cnt) __attribute__((always_inline)) {
        __hip_atomic_fetch_add(&slot[wave][0][m][lane], a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_add(&slot[wave][1][m][lane], q2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        cnt += 1u << (4 * m);
    };
    // rows blockIdx.x * 4 + wave, then every gridDim.x * 4 rows after it; each block's weights
    // are loaded one step ahead
    const long long rstep = (long long)gridDim.x * kQWaves;
    const int nb = K / 32;
    const int iters = (nb + 15) / 16;
    long long row = (long long)blockIdx.x * kQWaves + wave;
    u32x4 hn = row < rows ? load_quarter(w + (size_t)row * K, nb, 0, lane) : u32x4{0u, 0u, 0u, 0u};
    for (int i = 0; row < rows;) {
        const u32x4 h = hn;
        const int ni = i + 1 == iters ? 0 : i + 1;
        const long long nrow = i + 1 == iters ? row + rstep : row;
        if (nrow < rows) hn = load_quarter(w + (size_t)nrow * K, nb, ni, lane);
        const int bi = i;
        i = ni;
        row = nrow;
        {
            const uint32_t amax = quad_amax(h);
            int sf;
            const bool fast = fast_scale(fr, amax, sf);
            const BlockCode bc = fast ? BlockCode{sf, sf - 127} : block_code(amax, gmax);
            if (16 * bi + (lane >> 2) >= nb || bc.s == 255) continue;  // past the row; non-finite
            const double p2e = ldexp(1.0, bc.e);
            const double wt = ldexp(1.0, 2 * bc.e);
            uint32_t cnt = 0u;
            if (fast) {
                uint32_t tt[7];
                block_thresholds(fr, amax, bc.s, tt);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t mag2 = h[k] & 0x7FFF7FFFu;
                    const uint32_t m2 = nearest_pair(mag2, tt);
                    const double a0 = (double)__uint_as_float(mag2 << 16);
                    add2((int)(m2 & 7u), a0 * p2e, a0 * a0, cnt);
                    const double a1 = (double)__uint_as_float(mag2 & 0xFFFF0000u);
                    add2((int)(m2 >> 16), a1 * p2e, a1 * a1, cnt);
                }
            } else {
                const double inv = ldexp(1.0, -bc.e);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t hb = (h[j >> 1] >> (16 * (j & 1))) & 0x7FFFu;
                    const double r = (double)bf16_to_f32(hb) * inv;
                    const int m = nearest(r, mid);
                    const double wr1 = wt * r;
                    add2(m, wr1, wr1 * r, cnt);
                }
            }
#pragma unroll
            for (int m = 0; m < 8; ++m) wsq[m] += wt * (double)((cnt >> (4 * m)) & 15u);
        }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const double a = wave_sum_f64(slot[wave][0][m][lane]);
        const double c = wave_sum_f64(wsq[m]);
        const double q = wave_sum_f64(slot[wave][1][m][lane]);
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
    const long long per = (long long)kQWaves * kQRowsPerWave;
    const long long blocks = (rows + per - 1) / per;
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
