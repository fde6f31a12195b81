// kq_decode.h -- in-register k-quant decoders for gfx950, shared by the
// matvec kernels and the unpack/dequant debug kernels.
//
// Layouts: muser-book Ch 6 "The kquant family on the reference lane",
// Figures 6.2 (Q4_K), 6.3 (the 6-bit scale strip), 6.4 (Q5_K), 6.5 (Q6_K).
//
// Codes are produced two per 32-bit word, one in each 16-bit half, as the
// bit pattern of a binary16 SUBNORMAL: a half holding the integer v
// (0 <= v < 1024) is the binary16 value v * 2^-24, exactly.  v_fma_mix_f32
// widens such a half to float32 inside the multiply-add, so one instruction
// both converts a code and accumulates code * x.  Codes taken from a high
// nibble are left in place (v = 16 * code, value code * 2^-20); the kernels
// fold the 2^-24 / 2^-20 factors into the per-block scale.  Every value
// here stays below 1024, the limit of the subnormal range.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

// The 12-byte strip of Q4_K/Q5_K (Ch 6 section 6.2, the get_scale_min rule)
// as four words holding one 6-bit field per byte: sc_0..3, sc_4..7, m_0..3,
// m_4..7.  s0, s1, s2 are strip bytes 0-3, 4-7, 8-11 (little-endian).
struct K4Scales {
    uint32_t sc_lo, sc_hi, m_lo, m_hi;
};

__device__ __forceinline__ K4Scales k4_scales(uint32_t s0, uint32_t s1, uint32_t s2) {
    K4Scales r;
    r.sc_lo = s0 & 0x3F3F3F3Fu;                                  // j < 4: low six bits of s[j]
    r.m_lo = s1 & 0x3F3F3F3Fu;                                   //        and of s[j+4]
    r.sc_hi = (s2 & 0x0F0F0F0Fu) | ((s0 >> 2) & 0x30303030u);    // j >= 4: low nibble of s[j+4], top 2 of s[j-4]
    r.m_hi = ((s2 >> 4) & 0x0F0F0F0Fu) | ((s1 >> 2) & 0x30303030u); //     high nibble of s[j+4], top 2 of s[j]
    return r;
}

// Field j (0..7) of a K4Scales as an integer.
__device__ __forceinline__ uint32_t k4_sc(const K4Scales& s, int j) {
    return ((j < 4 ? s.sc_lo : s.sc_hi) >> (8 * (j & 3))) & 0xFFu;
}
__device__ __forceinline__ uint32_t k4_m(const K4Scales& s, int j) {
    return ((j < 4 ? s.m_lo : s.m_hi) >> (8 * (j & 3))) & 0xFFu;
}

// Four packed code words for one 32-bit word `q` of Q4_K/Q5_K qs bytes
// l..l+3 of group g (Ch 6 section 6.2: the low nibble of qs[32g+l] is
// element 64g+l, the high nibble element 64g+32+l).
//   lo02: elements l+0 | l+2 of sub-block 2g      (halves: v = code)
//   lo13: elements l+1 | l+3 of sub-block 2g
//   hi02: elements l+0 | l+2 of sub-block 2g+1    (halves: v = 16*code)
//   hi13: elements l+1 | l+3 of sub-block 2g+1
struct Packed4 {
    uint32_t lo02, lo13, hi02, hi13;
};

__device__ __forceinline__ Packed4 k4_codes(uint32_t q) {
    Packed4 p;
    uint32_t q8 = q >> 8;
    p.lo02 = q & 0x000F000Fu;
    p.lo13 = q8 & 0x000F000Fu;
    p.hi02 = q & 0x00F000F0u;
    p.hi13 = q8 & 0x00F000F0u;
    return p;
}

// Q5_K: the same four words with the fifth bit merged in.  h holds qh
// bytes l..l+3; bit j of qh[l] is the fifth code bit of element l of
// sub-block j (the reading of Ch 6 Figure 6.4 stated in the design notes).
// G is the group (0..3), so the sub-blocks are 2G and 2G+1.
template <int G>
__device__ __forceinline__ Packed4 k5_codes(uint32_t q, uint32_t h) {
    constexpr int J0 = 2 * G, J1 = 2 * G + 1;
    Packed4 p = k4_codes(q);
    uint32_t b02;                                                   // bit J0 of bytes 0,2 -> bits 4, 20
    if constexpr (J0 <= 4) b02 = h << (4 - J0);
    else b02 = h >> (J0 - 4);
    p.lo02 |= b02 & 0x00100010u;
    p.lo13 |= (h >> (4 + J0)) & 0x00100010u;                        // bytes 1,3 -> bits 4, 20
    p.hi02 |= (h << (8 - J1)) & 0x01000100u;                        // bit J1 of bytes 0,2 -> bits 8, 24
    p.hi13 |= (h >> J1) & 0x01000100u;                              // bytes 1,3 -> bits 8, 24
    return p;
}

// Q6_K: eight packed words for dword k (0..7) of half n, from
//   a = ql bytes 64n+4k..+3, b = ql bytes 64n+32+4k..+3, h = qh bytes 32n+4k..+3.
// Quarter c of the half (elements 128n + 32c + l) takes the low (c < 2) or
// high (c >= 2) nibble of a (c even) or b (c odd) and bits 2c, 2c+1 of qh
// (the reading of Ch 6 section 6.4 stated in the design notes).  Codes are
// the unsigned 6-bit values 0..63 (the -32 offset is applied by the caller);
// quarters 2 and 3 are left scaled by 16.
struct Packed6 {
    uint32_t c02[4], c13[4];   // [quarter]: elements l+0|l+2 and l+1|l+3
};

__device__ __forceinline__ Packed6 k6_codes(uint32_t a, uint32_t b, uint32_t h) {
    Packed6 p;
    uint32_t a8 = a >> 8, b8 = b >> 8;
    uint32_t h4l = h << 4, h2l = h << 2, h4r = h >> 4, h6r = h >> 6;
    p.c02[0] = (a & 0x000F000Fu) | (h4l & 0x00300030u);
    p.c13[0] = (a8 & 0x000F000Fu) | (h4r & 0x00300030u);
    p.c02[1] = (b & 0x000F000Fu) | (h2l & 0x00300030u);
    p.c13[1] = (b8 & 0x000F000Fu) | (h6r & 0x00300030u);
    p.c02[2] = (a & 0x00F000F0u) | (h4l & 0x03000300u);
    p.c13[2] = (a8 & 0x00F000F0u) | (h4r & 0x03000300u);
    p.c02[3] = (b & 0x00F000F0u) | (h2l & 0x03000300u);
    p.c13[3] = (b8 & 0x00F000F0u) | (h6r & 0x03000300u);
    return p;
}

// binary16 bits -> float32 (exact, subnormals kept).
__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Low / high half of a packed code word as the binary16 subnormal it
// encodes, widened to float32: v * 2^-24.
__device__ __forceinline__ _Float16 half_lo(uint32_t w) { return __builtin_bit_cast(_Float16, (uint16_t)w); }
__device__ __forceinline__ _Float16 half_hi(uint32_t w) { return __builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// Shift a run of 32-bit words right by two bytes: out[i] = bytes 2..5 of
// the pair (in[i], in[i+1]).  Used for Q6_K blocks that start two bytes
// into a word.
__device__ __forceinline__ uint32_t align2(uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_alignbit(hi, lo, 16);
}

}  // namespace kq
