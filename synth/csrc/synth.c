/*
 * Seeded synthetic inputs for the routed-expert MoE layer over 4-bit codebook experts.
 *
 * This file only PRODUCES inputs: Gaussian expert weights, drawn from a counter-based
 * generator, and their round-to-nearest (RTN) encoding into 4-bit sign+magnitude codes with
 * E8M0 block-32 scales. It holds no part of the forward pass (no decoding, no contraction,
 * no routing). Both the GPU library and the CPU oracle consume its bytes; neither is linked
 * against it.
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014). The state of draw i under key K is K + (i+1)*gamma, and the
 * output is SplitMix64's finaliser of that state, so any element can be drawn on its own.
 * Normals: Box-Muller on the two 32-bit halves of one 64-bit draw; draw i yields elements
 * 2i (cosine branch) and 2i+1 (sine branch) of the logical matrix.
 *
 * Encoding rule (GLM-5.2-NF4-Lloyd-Experts-GPTQ model card, "Codes are indices into the
 * per-layer grid"): the grid holds absolute magnitudes; a block of 32 weights along K gets
 * the smallest power of two 2^e with gmax * 2^e >= amax, is stored as byte e + 127, and each
 * weight stores the index of its nearest grid magnitude in bits 0..2 and its sign in bit 3.
 * Ties between two magnitudes go to the lower index; a block whose amax is 0 gets byte 0
 * and all-zero codes. Two codes per byte: the even K index in the low nibble ("Contents").
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Derive a stream key from up to 6 integer components. */
uint64_t synth_key(int64_t a, int64_t b, int64_t c, int64_t d, int64_t e, int64_t f) {
    const int64_t comp[6] = {a, b, c, d, e, f};
    uint64_t h = 0x6A09E667F3BCC908ULL;
    for (int i = 0; i < 6; ++i) h = sm64_mix(h + (uint64_t)comp[i] * GAMMA + GAMMA);
    return h;
}

/* Normal draws (synth_normal.c). Row buffer out[0..K) for stored row rn of a Kl-column
 * logical matrix, columns col_src (NULL = identity). */
void synth_normal_row(uint64_t key, int64_t rn, int64_t K, int64_t Kl, int64_t k0, float sigma,
                      const int32_t* col_src, float* out);

/*
 * Dense fp32 N(0, sigma) matrix, stored [N, K]. Stored element (n, k) is logical element
 * (row_src[n], col_src[k]) of a Kl-column matrix (identity when the maps are NULL).
 */
void synth_normal_f32(uint64_t key, int64_t N, int64_t K, int64_t Kl, double sigma,
                      const int32_t* row_src, const int32_t* col_src, float* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        synth_normal_row(key, row_src ? row_src[n] : n, K, Kl, 0, (float)sigma, col_src,
                         out + n * K);
}

/* Smallest e with gmax * 2^e >= amax (amax > 0, gmax > 0). */
static int block_exponent(double amax, double gmax) {
    int ex;
    (void)frexp(amax / gmax, &ex);
    int e = ex;
    while (ldexp(gmax, e) < amax) ++e;
    while (ldexp(gmax, e - 1) >= amax) --e;
    return e;
}

/* Largest float <= m: for a float r, (r > m) == (r > float_floor(m)) exactly. */
static float float_floor(double m) {
    float f = (float)m;
    if ((double)f > m) f = nextafterf(f, -INFINITY);
    return f;
}

/* Encode nb consecutive 32-blocks of one row; returns the number of clamped exponents. */
static int64_t encode_blocks(const float* row, int64_t nb, const double* mid, double gmax,
                             uint8_t* codes, uint8_t* scales) {
    float midf[7];
    for (int i = 0; i < 7; ++i) midf[i] = float_floor(mid[i]);
    int64_t clamped = 0;
    for (int64_t b = 0; b < nb; ++b) {
        const float* blk = row + b * 32;
        float amax = 0.0f;
        for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(blk[j]));
        uint8_t* cb = codes + b * 16;
        if (amax == 0.0f) {
            scales[b] = 0;
            memset(cb, 0, 16);
            continue;
        }
        int e = block_exponent((double)amax, gmax);
        if (e < -127) { e = -127; ++clamped; }
        if (e > 127) { e = 127; ++clamped; }
        scales[b] = (uint8_t)(e + 127);
        /* |w| * 2^-e, computed in double (exact) then compared against the float floors of
         * the midpoints, which is the exact comparison against the double midpoints. */
        const double inv = ldexp(1.0, -e);
        uint8_t code[32];
        for (int j = 0; j < 32; ++j) {
            const double rd = (double)fabsf(blk[j]) * inv;
            /* rd is a float times a power of two; when it is a normal float, (float)rd is
             * exact. Outside that range fall back to the double comparison. */
            int idx = 0;
            if (rd >= 1.1754943508222875e-38 && rd <= 3.4028234663852886e38) {
                const float r = (float)rd;
                for (int i = 0; i < 7; ++i) idx += (r > midf[i]);
            } else {
                for (int i = 0; i < 7; ++i) idx += (rd > mid[i]);
            }
            code[j] = (uint8_t)(idx | (blk[j] < 0.0f ? 8 : 0));
        }
        for (int j = 0; j < 16; ++j) cb[j] = (uint8_t)(code[2 * j] | (code[2 * j + 1] << 4));
    }
    return clamped;
}

static void grid_midpoints(const float* grid, double* mid) {
    for (int i = 0; i < 7; ++i) mid[i] = 0.5 * ((double)grid[i] + (double)grid[i + 1]);
}

/*
 * RTN-encode one fp32 matrix [N, K] (K % 32 == 0) against 8 ascending grid magnitudes.
 * codes: [N, K/2], scales: [N, K/32]. Returns the number of blocks whose exponent fell
 * outside the E8M0 range [-127, 127] (those are clamped); 0 on normal data.
 */
int64_t synth_rtn_encode(const float* w, int64_t N, int64_t K, const float* grid,
                         uint8_t* codes, uint8_t* scales) {
    double mid[7];
    grid_midpoints(grid, mid);
    int64_t clamped = 0;
    #pragma omp parallel for schedule(static) reduction(+ : clamped)
    for (int64_t n = 0; n < N; ++n)
        clamped += encode_blocks(w + n * K, K / 32, mid, grid[7], codes + n * (K / 2),
                                 scales + n * (K / 32));
    return clamped;
}

/*
 * Draw and encode in one pass, row-parallel, without materialising the fp32 matrix:
 * stored row n is logical row row_src[n], stored column k is logical column col_src[k]
 * of a Kl-column logical matrix with N(0, sigma) entries.
 */
int64_t synth_rtn_normal(uint64_t key, int64_t N, int64_t K, int64_t Kl, double sigma,
                         const int32_t* row_src, const int32_t* col_src, const float* grid,
                         uint8_t* codes, uint8_t* scales) {
    double mid[7];
    grid_midpoints(grid, mid);
    int64_t clamped = 0;
    #pragma omp parallel for schedule(static) reduction(+ : clamped)
    for (int64_t n = 0; n < N; ++n) {
        float row[4096];
        const int64_t rn = row_src ? row_src[n] : n;
        for (int64_t k0 = 0; k0 < K; k0 += 4096) {
            const int64_t kn = (K - k0) < 4096 ? (K - k0) : 4096;
            synth_normal_row(key, rn, kn, Kl, k0, (float)sigma, col_src, row);
            clamped += encode_blocks(row, kn / 32, mid, grid[7], codes + n * (K / 2) + k0 / 2,
                                     scales + n * (K / 32) + k0 / 32);
        }
    }
    return clamped;
}
