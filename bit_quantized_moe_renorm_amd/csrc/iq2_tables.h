// iq2_tables.h - decoding IQ2-style codebook groups on gfx950.
//
// The codebook format ("Redis 作者出手！ds4...", section 2.3: block_iq2_xxs, 66
// bytes per 256 weights) stores per group of 8 weights one codebook index and
// 7 sign bits (the 8th sign makes the count of negatives even), and per 32
// weights a 4-bit scale.  The library keeps each sub-block's canonical 8 bytes
// (4 index bytes, then the sign/scale word) in its qs plane.
//
// The 256-entry codebook is expanded once per workgroup into an LDS table of
// unsigned levels (2c+1) for all 8 coordinates (16 bytes per entry, packed
// pairs).  The table is replicated 16 times with the replicas interleaved at
// 16-byte granularity (entry e, replica r at byte 256 e + 16 r), and lane l
// reads replica l & 15: replica r always sits in bank quad r (of 64 banks), so
// the 16 lanes served together by a ds_read_b128 never conflict, whatever
// indices they look up.  Signs are applied with XOR masks
// built from the sign bits by rotates (v_alignbit) and one v_bitop3 each.
#pragma once
#include "common.h"

namespace ds4 {

constexpr int IQ2_REPL = 16;
constexpr int IQ2_LUT_BYTES = 256 * IQ2_REPL * 16;  // 64 KB

// Unsigned level (2c+1) bit patterns, c in 0..3.
__device__ __forceinline__ uint32_t iq2_level_bf16(uint32_t c) {
    return (c == 0) ? 0x3F80u : (c == 1) ? 0x4040u : (c == 2) ? 0x40A0u : 0x40E0u;
}
__device__ __forceinline__ uint32_t iq2_level_f16(uint32_t c) {
    return (c == 0) ? 0x3C00u : (c == 1) ? 0x4200u : (c == 2) ? 0x4500u : 0x4700u;
}

// One entry of the replicated table (entry e, replica r at uint4 index e*R +
// r) from its codebook word c.
template <bool FP16, int R = IQ2_REPL>
__device__ __forceinline__ void iq2_lut_entry(uint4 *T, int e, uint32_t c) {
    uint32_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = FP16 ? iq2_level_f16((c >> (2 * k)) & 3u) : iq2_level_bf16((c >> (2 * k)) & 3u);
    const uint4 q = make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
#pragma unroll
    for (int r = 0; r < R; ++r) T[e * R + r] = q;
}
// Build the replicated table: each thread loads whole codebook entries once
// and writes their R replicas.
template <bool FP16, int R = IQ2_REPL>
__device__ __forceinline__ void iq2_build_lut(uint4 *T, const uint16_t *__restrict__ codebook, int tid, int nthreads) {
    for (int e = tid; e < 256; e += nthreads) iq2_lut_entry<FP16, R>(T, e, codebook[e]);
}

// Rotate right (v_alignbit_b32 with both sources equal).  Written as one
// instruction so the compiler cannot fold the rotate and the following mask
// into a quarter-rate 32-bit multiply.
template <int R>
__device__ __forceinline__ uint32_t rotr(uint32_t v) {
    uint32_t r;
    asm("v_alignbit_b32 %0, %1, %1, %2" : "=v"(r) : "v"(v), "i"(R));
    return r;
}

// Apply the signs of one group to its unsigned levels L (4 dwords of packed
// pairs w0|w1 .. w6|w7): s7 = stored sign bits of weights 0..6.
__device__ __forceinline__ uint4 iq2_apply_signs(uint4 L, uint32_t s7) {
    // 8th sign: the group holds an even number of negatives (bit 7 = parity;
    // bits 8-9 receive the rest of the count and are never selected below)
    const uint32_t s8 = s7 | (__builtin_popcount(s7) << 7);
    // copy A of the signs at bits 0-9, copy B at bits 15-24
    const uint32_t S = s8 | (s8 << 15);
    // dword j holds weights (2j, 2j+1): their sign bits go to bit 15 (from copy A,
    // bit 2j) and bit 31 (from copy B, bit 2j+1).  Rotating S left by 15-2j (a
    // right rotate by 17+2j with v_alignbit) puts both there at once.
    const uint32_t M = 0x80008000u;
    L.x ^= rotr<17>(S) & M;
    L.y ^= rotr<19>(S) & M;
    L.z ^= rotr<21>(S) & M;
    L.w ^= rotr<23>(S) & M;
    return L;
}

// Signed levels of one group: idx = codebook index, s7 = stored sign bits of
// weights 0..6.  Returns 4 dwords of packed pairs (w0|w1, w2|w3, w4|w5, w6|w7).
template <int R = IQ2_REPL>
__device__ __forceinline__ uint4 iq2_group_levels(const uint4 *T, uint32_t idx, uint32_t s7, int rep) {
    return iq2_apply_signs(T[idx * R + rep], s7);
}

// ---------------------------------------------------------------- byte tables
// For fp16 dot products a group fits in 8 bytes.  The levels 1, 3, 5, 7 are
// fp16 numbers whose low byte is zero (0x3C00, 0x4200, 0x4500, 0x4700), and
// the fp16 sign is bit 7 of the high byte.  So one table holds each codebook
// entry's 8 level bytes and another each sign pattern's 8 sign bytes (the 8th
// sign from the parity of the 7 stored ones).  A group's signed levels are
// the XOR of the two 8-byte words, spread into 4 fp16 pairs by v_perm.
constexpr int IQ2B_REPL = 16;  // replicas of both byte tables (8 bytes each)

__device__ __forceinline__ uint32_t iq2_level_f16hi(uint32_t c) {
    return (c == 0) ? 0x3Cu : (c == 1) ? 0x42u : (c == 2) ? 0x45u : 0x47u;
}
// Level bytes of codebook entry cb (coordinate i in bits 2i..2i+1): byte i.
__device__ __forceinline__ uint2 iq2_level_bytes(uint32_t cb) {
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = iq2_level_f16hi((cb >> (2 * i)) & 3u);
    return make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
}
// Sign bytes of the 7 stored sign bits s7: bit 7 of byte i is weight i's sign.
__device__ __forceinline__ uint2 iq2_sign_bytes(uint32_t s7) {
    const uint32_t s8 = s7 | ((__builtin_popcount(s7) & 1u) << 7);
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = ((s8 >> i) & 1u) << 7;
    return make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
}
// 8 signed level bytes -> 4 fp16 pairs (weights 2j | 2j+1 << 16 in dword j).
__device__ __forceinline__ uint4 iq2_expand_f16(uint2 v) {
    return make_uint4(__builtin_amdgcn_perm(0u, v.x, 0x010C000Cu), __builtin_amdgcn_perm(0u, v.x, 0x030C020Cu),
                      __builtin_amdgcn_perm(0u, v.y, 0x010C000Cu), __builtin_amdgcn_perm(0u, v.y, 0x030C020Cu));
}

}  // namespace ds4
