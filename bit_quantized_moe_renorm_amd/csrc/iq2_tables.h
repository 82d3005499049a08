// iq2_tables.h - LDS lookup tables for the IQ2-style codebook blocks.
//
// The codebook format (2-bit codebook weights, "Redis 作者出手！ds4...", section 2.3:
// block_iq2_xxs, 66 bytes per 256 weights) stores per group of 8 weights one
// codebook index and 7 sign bits; the 8th sign follows from parity.  In the
// library's repacked layout each group is one 16-bit field (see common.h).
//
// Two 4096-entry tables, built per workgroup in LDS from the 256-entry codebook,
// turn a field into 8 signed levels +-(2c+1) without any per-weight bit work:
//   T[0    + (field & 0xFFF)]        -> levels of weights 0..3 (4 x 16 bit)
//   T[4096 + ((field >> 3) & 0xFFF)] -> levels of weights 4..7
// Each entry is a uint2 holding two packed pairs (w0|w1<<16, w2|w3<<16).  The
// levels are bf16 (decode dot products) or fp16 (MFMA operands scaled by
// packed fp16 multiplies); both are exact for the small odd integers 1..7.
#pragma once
#include "common.h"

namespace ds4 {

constexpr int IQ2_TABLE_ENTRIES = 8192;  // 64 KB of uint2

template <bool FP16>
__device__ __forceinline__ uint32_t iq2_level_bits(uint32_t c, uint32_t neg) {
    // +-(2c+1) for c in 0..3
    uint32_t v;
    if (FP16)
        v = (c == 0) ? 0x3C00u : (c == 1) ? 0x4200u : (c == 2) ? 0x4500u : 0x4700u;
    else
        v = (c == 0) ? 0x3F80u : (c == 1) ? 0x4040u : (c == 2) ? 0x40A0u : 0x40E0u;
    return v | (neg << 15);
}

// Fill T[0..8191] from the codebook cb[256] (already in LDS); caller syncs after.
template <bool FP16>
__device__ __forceinline__ void iq2_build_tables(uint2 *T, const uint16_t *cb, int tid, int nthreads) {
    for (int i = tid; i < IQ2_TABLE_ENTRIES; i += nthreads) {
        uint32_t s[4], codes, idx;
        if (i < 4096) {
            uint32_t P = (i >> 3) & 1;
            idx = (i >> 4) & 0xFF;
            s[0] = i & 1;
            s[1] = (i >> 1) & 1;
            s[2] = (i >> 2) & 1;
            s[3] = P ^ s[0] ^ s[1] ^ s[2];
            codes = cb[idx] & 0xFF;
        } else {
            int j = i - 4096;
            uint32_t P = j & 1;
            idx = (j >> 1) & 0xFF;
            s[0] = (j >> 9) & 1;
            s[1] = (j >> 10) & 1;
            s[2] = (j >> 11) & 1;
            s[3] = P ^ s[0] ^ s[1] ^ s[2];
            codes = cb[idx] >> 8;
        }
        uint32_t v0 = iq2_level_bits<FP16>(codes & 3, s[0]);
        uint32_t v1 = iq2_level_bits<FP16>((codes >> 2) & 3, s[1]);
        uint32_t v2 = iq2_level_bits<FP16>((codes >> 4) & 3, s[2]);
        uint32_t v3 = iq2_level_bits<FP16>((codes >> 6) & 3, s[3]);
        T[i] = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
    }
}

// Levels of the two groups packed in one dword D (group fields D & 0xFFFF, D >> 16).
// Byte offsets are formed directly from the field bits (entry size 8 bytes).
struct Iq2Pair {
    uint2 a0, a1;  // low group: weights 0..3, 4..7
    uint2 b0, b1;  // high group
};

__device__ __forceinline__ Iq2Pair iq2_lookup(const uint2 *T, uint32_t D) {
    const char *Tb = reinterpret_cast<const char *>(T);
    Iq2Pair p;
    p.a0 = *reinterpret_cast<const uint2 *>(Tb + ((D << 3) & 0x7FF8u));
    p.a1 = *reinterpret_cast<const uint2 *>(Tb + 32768 + (D & 0x7FF8u));
    p.b0 = *reinterpret_cast<const uint2 *>(Tb + ((D >> 13) & 0x7FF8u));
    p.b1 = *reinterpret_cast<const uint2 *>(Tb + 32768 + ((D >> 16) & 0x7FF8u));
    return p;
}

// Sub-block scale ls from the sub-block's two dwords (bit 15 of each group field).
__device__ __forceinline__ uint32_t iq2_ls(uint32_t D0, uint32_t D1) {
    return ((D0 >> 15) & 1u) | ((D0 >> 30) & 2u) | ((D1 >> 13) & 4u) | ((D1 >> 28) & 8u);
}

// Repack one canonical sub-block (4 index bytes + sign/scale word) into the
// four 16-bit group fields, returned as two dwords (groups 0|1, 2|3).
__host__ __device__ inline void iq2_encode_subblock(const uint8_t idx[4], uint32_t word, uint32_t &D0,
                                                    uint32_t &D1) {
    uint32_t ls = word >> 28;
    uint32_t f[4];
    for (int g = 0; g < 4; ++g) {
        uint32_t s7 = (word >> (7 * g)) & 0x7Fu;
        uint32_t P = (s7 ^ (s7 >> 1) ^ (s7 >> 2) ^ (s7 >> 3)) & 1u;
        f[g] = (s7 & 7u) | (P << 3) | ((uint32_t)idx[g] << 4) | (((s7 >> 4) & 7u) << 12) |
               (((ls >> g) & 1u) << 15);
    }
    D0 = f[0] | (f[1] << 16);
    D1 = f[2] | (f[3] << 16);
}

}  // namespace ds4
