// Device-side building blocks shared by the libmoeq kernels (gfx950, wave64).
//
// Decoding 4-bit codes (GLM-5.2-NF4-Lloyd-Experts-GPTQ model card, "Contents" and "Codes are
// indices into the per-layer grid"): a byte holds two codes, even K in the low nibble; code c
// of a row block with scale byte s decodes to (-1)^(c>>3) * table[c & 7] * 2^(s - 127).
//
// How it is done here. For every (table, scale byte) pair the 8 exact magnitudes
// bf16(table[m] * 2^(s - 127)) are precomputed once per workgroup into LDS, split into a
// high-byte table and a low-byte table (8 bytes each, two dwords each). A dword of 8 codes is
// then decoded with byte permutes (v_perm_b32): the 3-bit magnitude indices select bytes from
// the two tables, bit 3 of each code is OR-ed in as the bf16 sign bit, and two more permutes
// interleave low and high bytes into bf16 pairs. The result is bit-exact (every value comes
// from the exact table and a sign flip, which commutes with round-to-nearest-even) and costs
// 14 VALU ops per 8 weights, with no per-weight conversion or multiply.
//
// The 8 decoded values come out in the order k = 0, 2, 4, 6, 1, 3, 5, 7 of their 8-group
// ("pair-split" order). MFMA contracts over K, so the order only has to agree between the
// two operands: activation operands are permuted the same way (X on the fly, the
// intermediate by storing it in that order).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq {

constexpr int kMaxTables = 4;

struct TableArgs {
    float v[kMaxTables][8];
    int n;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
    // selector byte values 0..3 pick bytes of `lo`, 4..7 pick bytes of `hi`
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// bf16 bits of round-to-nearest-even(t * 2^(s - 127)), t a finite non-negative fp32 value.
// s == 255 gives NaN (0x7FC0). Integer arithmetic only: the exact product is M * 2^E with a
// 24-bit integer M; it is shifted down to the bf16 quantum (2^(q-7) for a normal result in
// [2^q, 2^(q+1)), 2^-133 in the subnormal range) with round-half-even on the dropped bits.
__device__ inline uint32_t scaled_bf16_bits(float t, int s) {
    if (s == 255) return 0x7FC0u;
    const uint32_t b = __float_as_uint(t);
    const uint32_t ex = b >> 23, man = b & 0x7FFFFFu;
    if (ex == 0 && man == 0) return 0u;
    uint32_t M;
    int E;
    if (ex == 0) { M = man; E = -149; } else { M = man | 0x800000u; E = (int)ex - 150; }
    E += s - 127;
    const int L = 31 - __clz((int)M);
    int q = L + E;
    if (q > 127) return 0x7F80u;
    const bool normal = q >= -126;
    const int qe = normal ? (q - 7) : -133;
    const int sh = qe - E;
    uint32_t r;
    if (sh <= 0) {
        r = M << (-sh);
    } else if (sh > 31) {
        r = 0;
    } else {
        const uint32_t rem = M & ((1u << sh) - 1u);
        const uint32_t half = 1u << (sh - 1);
        r = M >> sh;
        if (rem > half || (rem == half && (r & 1u))) ++r;
    }
    if (!normal) return r;            // r == 128 is the smallest normal, bits 0x0080
    if (r == 256u) { r = 128u; ++q; if (q > 127) return 0x7F80u; }
    return ((uint32_t)(q + 127) << 7) | (r & 0x7Fu);
}

// Fill the LDS decode tables: tab[t * 256 + s] = {hi bytes m0..3, hi bytes m4..7,
// lo bytes m0..3, lo bytes m4..7} of bf16(table_t[m] * 2^(s - 127)). Called by all threads
// of a workgroup; ends with a barrier.
__device__ inline void build_decode_tables(const TableArgs& ta, u32x4* tab) {
    for (int i = threadIdx.x; i < ta.n * 256; i += blockDim.x) {
        // t is the same in every lane of a wavefront (blockDim is a multiple of 64): as a
        // scalar, its 8 magnitudes come by one scalar load instead of 8 dependent vector loads
        const int t = __builtin_amdgcn_readfirstlane(i >> 8), s = i & 255;
        uint32_t h0 = 0, h1 = 0, l0 = 0, l1 = 0;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint32_t v = scaled_bf16_bits(ta.v[t][m], s);
            const uint32_t hb = v >> 8, lb = v & 0xFFu;
            if (m < 4) { h0 |= hb << (8 * m); l0 |= lb << (8 * m); }
            else { h1 |= hb << (8 * (m - 4)); l1 |= lb << (8 * (m - 4)); }
        }
        tab[i] = u32x4{h0, h1, l0, l1};
    }
    __syncthreads();
}

// Decode one dword of 8 codes (bytes b0..b3; byte j = codes of k = 2j (low) and 2j+1 (high))
// with the decode table `tb` of its scale block. Output: 4 dwords of bf16 pairs
// (k0,k2), (k4,k6), (k1,k3), (k5,k7).
__device__ __forceinline__ u32x4 decode8(uint32_t c, const u32x4 tb) {
    const uint32_t se = c & 0x07070707u;
    const uint32_t so = (c >> 4) & 0x07070707u;
    uint32_t he = perm_b32(tb[1], tb[0], se);
    const uint32_t le = perm_b32(tb[3], tb[2], se);
    uint32_t ho = perm_b32(tb[1], tb[0], so);
    const uint32_t lo = perm_b32(tb[3], tb[2], so);
    he |= (c << 4) & 0x80808080u;   // bit 3 of each low nibble -> bf16 sign
    ho |= c & 0x80808080u;          // bit 3 of each high nibble -> bf16 sign
    return u32x4{perm_b32(he, le, 0x05010400u), perm_b32(he, le, 0x07030602u),
                 perm_b32(ho, lo, 0x05010400u), perm_b32(ho, lo, 0x07030602u)};
}

// Natural-order 8 bf16 (dwords (x0,x1), (x2,x3), (x4,x5), (x6,x7)) -> pair-split order.
__device__ __forceinline__ u32x4 pair_split(const u32x4 n) {
    return u32x4{perm_b32(n[1], n[0], 0x05040100u), perm_b32(n[3], n[2], 0x05040100u),
                 perm_b32(n[1], n[0], 0x07060302u), perm_b32(n[3], n[2], 0x07060302u)};
}

// Inverse of pair_split.
__device__ __forceinline__ u32x4 pair_join(const u32x4 p) {
    return u32x4{perm_b32(p[2], p[0], 0x05040100u), perm_b32(p[2], p[0], 0x07060302u),
                 perm_b32(p[3], p[1], 0x05040100u), perm_b32(p[3], p[1], 0x07060302u)};
}

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4 a, const u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN with the input's sign.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t b = __float_as_uint(f);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return ((b >> 16) & 0x8000u) | 0x7FC0u;
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace moeq
