// fa_philox.h -- dropout keep bits on the GPU.
//
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds, each two 32 x 32 -> 64-bit products
// of counter words 0 and 2 with 0xD2511F53 and 0xCD9E8D57, the high halves
// mixed with words 1 and 3 and the key, the key bumped by 0x9E3779B9 and
// 0xBB67AE85 between rounds.  One call gives the random words of four
// consecutive keys of one query row: element (i, j) of query head h of
// sequence b uses word j % 4 of the call at counter (j / 4, i, b * H + h,
// offset lo) with key (seed lo, seed hi ^ offset hi), and is kept iff that
// word is >= floor(p * 2^32) (the keep test of the Triton FA2 teaching page's
// dropout_mask, read so that kept values scaled by 1 / (1 - p) keep the
// expectation).
#pragma once

#include "fa_internal.h"

namespace fa {

// a ^ b ^ k in one instruction: gfx950's three-input bit operation with
// truth table 0x96 (inputs 0xF0, 0xCC, 0xAA); the compiler leaves the two
// xors of each Philox round separate otherwise.
__device__ inline uint32_t xor3_sk(uint32_t a, uint32_t b, uint32_t k)
{
    return __builtin_amdgcn_bitop3_b32(a, b, k, 0x96);
}

// Keep bits of keys 4*c0 .. 4*c0+3 of query row c1 (bit x: key 4*c0 + x).
// c2 = b * H + h.  The key and the last counter word are wave-uniform.
// X3: each round's two xors as one three-input operation (about a tenth of
// the vector instructions of a dropout kernel fewer; the dQ kernel, which
// has no register left, spills with it and keeps the two-xor form).
template <bool X3 = true>
__device__ inline uint32_t keep_nibble(uint32_t c0, uint32_t c1, uint32_t c2, const Params &p)
{
    uint32_t w0 = c0, w1 = c1, w2 = c2, w3 = p.drop_c3;
    uint32_t k0 = p.drop_k0, k1 = p.drop_k1;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * w0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * w2;
        uint32_t n0, n2;
        if constexpr (X3) {
            n0 = xor3_sk((uint32_t)(p1 >> 32), w1, k0);
            n2 = xor3_sk((uint32_t)(p0 >> 32), w3, k1);
        } else {
            n0 = (uint32_t)(p1 >> 32) ^ w1 ^ k0;
            n2 = (uint32_t)(p0 >> 32) ^ w3 ^ k1;
        }
        w1 = (uint32_t)p1;
        w3 = (uint32_t)p0;
        w0 = n0;
        w2 = n2;
    }
    const uint32_t t = p.drop_thr;
    return (w0 >= t ? 1u : 0u) | (w1 >= t ? 2u : 0u) | (w2 >= t ? 4u : 0u) | (w3 >= t ? 8u : 0u);
}

// Nibble r (bits 4r .. 4r+3) of a 16-bit value moved to bits 8r .. 8r+3.
__device__ inline uint32_t spread_nibbles(uint32_t x)
{
    x = (x | (x << 8)) & 0x00FF00FFu;
    return (x | (x << 4)) & 0x0F0F0F0Fu;
}

// The inverse: nibbles 0, 2, 4, 6 of x into nibbles 0 .. 3.
__device__ inline uint32_t gather_nibbles(uint32_t x)
{
    x &= 0x0F0F0F0Fu;
    x = (x | (x >> 4)) & 0x00FF00FFu;
    return (x | (x >> 8)) & 0x0000FFFFu;
}

// Dropout multiplier of a keep bit: 1 / (1 - p) if set, else 0 (the bit
// sign-extended to a full mask and ANDed with inv's bits: two operations,
// no compare).
__device__ inline float keep_mult(uint32_t bits, int pos, float inv)
{
    const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)bits, pos, 1);
    return __builtin_bit_cast(float, m & __builtin_bit_cast(uint32_t, inv));
}

}  // namespace fa
