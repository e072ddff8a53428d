/*
 * Counter-based N(0, sigma) draws for the synthetic expert weights (built with fast math:
 * only the statistical distribution matters here, not bit-reproducibility across builds).
 *
 * SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): draw i under key K is the SplitMix64
 * finaliser of K + (i+1)*gamma. Box-Muller turns the two 23-bit halves of draw i into
 * logical elements 2i (cosine branch) and 2i+1 (sine branch).
 */
#include <math.h>
#include <stdint.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline void uniform_pair(uint64_t key, uint64_t pair, float* u1, float* u2) {
    const uint64_t r = sm64_mix(key + (pair + 1) * GAMMA);
    *u1 = ((float)(uint32_t)(r >> 41) + 0.5f) * (1.0f / 8388608.0f);
    *u2 = ((float)(uint32_t)(r & 0x7FFFFF) + 0.5f) * (1.0f / 8388608.0f);
}

#define CHUNK 256

/* out[k] = sigma * normal(logical element (rn, col(k0 + k))) for k in [0, K). */
void synth_normal_row(uint64_t key, int64_t rn, int64_t K, int64_t Kl, int64_t k0, float sigma,
                      const int32_t* col_src, float* out) {
    const uint64_t base = (uint64_t)(rn * Kl);
    float u1[CHUNK], u2[CHUNK], z0[CHUNK], z1[CHUNK];
    if (!col_src && ((base + (uint64_t)k0) % 2 == 0) && (K % 2 == 0)) {
        const uint64_t p0 = (base + (uint64_t)k0) >> 1;
        for (int64_t j0 = 0; j0 < K / 2; j0 += CHUNK) {
            const int n = (K / 2 - j0) < CHUNK ? (int)(K / 2 - j0) : CHUNK;
            for (int j = 0; j < n; ++j) uniform_pair(key, p0 + (uint64_t)(j0 + j), &u1[j], &u2[j]);
            for (int j = 0; j < n; ++j) {
                const float rad = sigma * sqrtf(-2.0f * logf(u1[j]));
                const float ang = 6.28318530717958647692f * u2[j];
                z0[j] = rad * cosf(ang);
                z1[j] = rad * sinf(ang);
            }
            for (int j = 0; j < n; ++j) {
                out[2 * (j0 + j)] = z0[j];
                out[2 * (j0 + j) + 1] = z1[j];
            }
        }
        return;
    }
    for (int64_t k = 0; k < K; ++k) {
        const uint64_t idx = base + (uint64_t)(col_src ? col_src[k0 + k] : (k0 + k));
        float a, b;
        uniform_pair(key, idx >> 1, &a, &b);
        const float rad = sigma * sqrtf(-2.0f * logf(a));
        const float ang = 6.28318530717958647692f * b;
        out[k] = (idx & 1) ? rad * sinf(ang) : rad * cosf(ang);
    }
}
