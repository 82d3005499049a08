// mfma_ops.h - MFMA operand helpers shared by the grouped GEMMs (gemm.hip)
// and the small-batch kernels (small.hip).
//
// Operand roles of v_mfma_f32_16x16x32_f16: A = 16 tokens x 32 K, B = 32 K x 16
// weight rows, C = 16 tokens x 16 rows.  Lane l holds B column l % 16 (one
// weight row) and K 8(l/16)..+8, and C rows 4(l/16)..+3 of that column.  Within
// a 256-K block, step cc (0..7) has lane group g = l / 16 supply K 64 g + 8 cc
// ..+8, so each lane needs only its own quarter of every weight row block.
#pragma once
#include "common.h"
#include "iq2_tables.h"

namespace ds4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma_f16(half8 a, half8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_bf16(uint4 a, uint4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ half8 as_half8(uint4 v) { return __builtin_bit_cast(half8, v); }

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ uint16_t f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// B operand of the routed gate/up GEMM: for the lane's 16-byte quarter w of
// an IQ2 row block (sub-blocks 2 g and 2 g + 1: words x, y and z, w) and
// step cc (0..7), the 8 weights K 64 g + 8 cc .. + 7 in fp16: the signed
// table level times fp16(d (2 ls + 1) / 64), rounded once more in the
// product.  scl caches the scale over a sub-block's 4 steps (set at cc % 4
// == 0), so steps go in order.  The debug entry decodes through this same
// function.
// In two parts, so a caller can issue the table lookup a step ahead of the
// arithmetic: iq2_b_lookup reads the unsigned levels of the step's group from
// the table, iq2_b_finish applies the signs and the scale.
__device__ __forceinline__ uint4 iq2_b_lookup(const uint4 *T, const uint4 &w, int cc, int rl) {
    const uint32_t ib = (cc < 4) ? w.x : w.z;
    return T[((ib >> (8 * (cc & 3))) & 0xFFu) * IQ2_REPL + rl];
}
__device__ __forceinline__ half8 iq2_b_finish(const uint4 &lv, const uint4 &w, uint16_t d, int cc, half2v &scl) {
    const uint32_t sw = (cc < 4) ? w.y : w.w;
    if ((cc & 3) == 0) {
        const _Float16 s = (_Float16)(half_to_f32(d) * (0.015625f * (float)(2u * (sw >> 28) + 1u)));
        scl = half2v{s, s};
    }
    const uint4 sg = iq2_apply_signs(lv, (sw >> (7 * (cc & 3))) & 0x7Fu);
    return as_half8(sg) * __builtin_shufflevector(scl, scl, 0, 1, 0, 1, 0, 1, 0, 1);
}
__device__ __forceinline__ half8 iq2_b_operand(const uint4 *T, const uint4 &w, uint16_t d, int cc, int rl,
                                               half2v &scl) {
    return iq2_b_finish(iq2_b_lookup(T, w, cc, rl), w, d, cc, scl);
}

// Sign masks from a table instead of bit arithmetic: entry s7 (the 7 stored
// sign bits of a group) holds the group's four XOR masks (bit 15 and bit 31
// of dword j for weights 2j and 2j+1, the 8th sign from the parity), that is
// iq2_apply_signs of zero levels, so the signed levels are identical.  128
// entries, IQ2S_REPL replicas interleaved at 16-byte granularity (entry s,
// replica r at uint4 index s IQ2S_REPL + r); lane l reads replica l & 7, so at
// most two of the 16 lanes served together share a bank quad.  Five VALU
// operations per group fewer than the bit arithmetic, one more LDS read: it
// pays where the IQ2 decode is shared by few token tiles (the A operand's LDS
// reads are then few).
constexpr int IQ2S_REPL = 8;
__device__ __forceinline__ void iq2_build_sign_table(uint4 *ST, int tid, int nthreads) {
    for (int i = tid; i < 128 * IQ2S_REPL; i += nthreads)
        ST[i] = iq2_apply_signs(make_uint4(0u, 0u, 0u, 0u), (uint32_t)i / IQ2S_REPL);
}
__device__ __forceinline__ uint4 iq2_s_lookup(const uint4 *ST, const uint4 &w, int cc, int rl) {
    const uint32_t sw = (cc < 4) ? w.y : w.w;
    return ST[((sw >> (7 * (cc & 3))) & 0x7Fu) * IQ2S_REPL + (rl & 7)];
}
// iq2_b_finish with the signs as looked-up masks sm.
__device__ __forceinline__ half8 iq2_b_finish_masked(uint4 lv, const uint4 &sm, const uint4 &w, uint16_t d, int cc,
                                                     half2v &scl) {
    const uint32_t sw = (cc < 4) ? w.y : w.w;
    if ((cc & 3) == 0) {
        const _Float16 s = (_Float16)(half_to_f32(d) * (0.015625f * (float)(2u * (sw >> 28) + 1u)));
        scl = half2v{s, s};
    }
    lv.x ^= sm.x, lv.y ^= sm.y, lv.z ^= sm.z, lv.w ^= sm.w;
    return as_half8(lv) * __builtin_shufflevector(scl, scl, 0, 1, 0, 1, 0, 1, 0, 1);
}

// Q2_K B decode: a table of the four 2-bit values of each qs byte as fp16
// (8 bytes per entry), 16 replicas interleaved per entry; lane l reads replica l % 16.
constexpr int QT_REPL = 16;
__device__ __forceinline__ void q2k_build_table(uint2 *QT, int tid, int nthreads) {
    for (int i = tid; i < 256 * QT_REPL; i += nthreads) {
        const uint32_t byte = (uint32_t)i / QT_REPL;
        uint32_t h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t q = (byte >> (2 * j)) & 3u;
            h[j] = (q == 0) ? 0u : (q == 1) ? 0x3C00u : (q == 2) ? 0x4000u : 0x4200u;
        }
        QT[i] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    }
}

// B operand of the routed down GEMM: for the lane's 16 quant bytes q of a
// Q2_K row block (weights 64 g .. 64 g + 63), its 4 scale bytes sc
// (sub-blocks 4 g .. 4 g + 3) and dd = d | dmin << 16, step cc (0..7) gives
// the 8 weights K 64 g + 8 cc .. + 7 in fp16 as fma(q, fp16(d sc),
// fp16(-dmin m)).  dsc and msc cache the scale and min over a sub-block's 2
// steps (set at even cc), so steps go in order.  The debug entry decodes
// through this same function.
// In two parts like the IQ2 operand: q2k_b_lookup reads the step's 8 codes
// as fp16 from the table, q2k_b_finish applies the sub-block's scale and min.
__device__ __forceinline__ uint4 q2k_b_lookup(const uint2 *QT, const uint4 &q, int cc, int rl) {
    const uint32_t dw = (cc < 2) ? q.x : (cc < 4) ? q.y : (cc < 6) ? q.z : q.w;
    const int sh = 16 * (cc & 1);
    const uint2 lo = QT[((dw >> sh) & 0xFFu) * QT_REPL + rl];
    const uint2 hi = QT[((dw >> (sh + 8)) & 0xFFu) * QT_REPL + rl];
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}
__device__ __forceinline__ half8 q2k_b_finish(const uint4 &qv8, uint32_t sc, uint32_t dd, int cc, half8 &dsc,
                                              half8 &msc) {
    if ((cc & 1) == 0) {
        // sub-block 4 g + cc / 2: scale and min nibbles of its scale byte
        const uint32_t sb8 = (sc >> (8 * (cc >> 1))) & 0xFFu;
        const float d = half_to_f32((uint16_t)(dd & 0xFFFFu));
        const float dmin = half_to_f32((uint16_t)(dd >> 16));
        const _Float16 ds = (_Float16)(d * (float)(sb8 & 0xFu));
        const _Float16 ms = (_Float16)(-dmin * (float)(sb8 >> 4));
        dsc = half8{ds, ds, ds, ds, ds, ds, ds, ds};
        msc = half8{ms, ms, ms, ms, ms, ms, ms, ms};
    }
    return __builtin_elementwise_fma(as_half8(qv8), dsc, msc);
}
__device__ __forceinline__ half8 q2k_b_operand(const uint2 *QT, const uint4 &q, uint32_t sc, uint32_t dd, int cc,
                                               int rl, half8 &dsc, half8 &msc) {
    return q2k_b_finish(q2k_b_lookup(QT, q, cc, rl), sc, dd, cc, dsc, msc);
}

}  // namespace ds4
