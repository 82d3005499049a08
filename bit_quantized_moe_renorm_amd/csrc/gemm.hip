// gemm.hip - batched path (prefill and batches beyond the GEMV limit): the
// routed and shared expert projections as grouped MFMA GEMMs with the weight
// decode fused into the B-operand load.
//
// Operand roles (v_mfma_f32_16x16x32_{f16,bf16}): A = 16 tokens x 32 K from an
// LDS stage, B = 32 K x 16 weight rows decoded in registers, C = 16 tokens x 16
// rows.  Lane l holds B column l % 16 (one weight row) and K 8(l/16)..+8, which
// is exactly one 8-weight codebook group of an IQ2 sub-block, and C rows
// 4(l/16)..+3 of that same column, so every per-row factor (block scale d,
// sub-block scale, Q2_K d / dmin) is lane-local.
//
// Numerics: the routed experts' B operand is the dequantized weight rounded
// to fp16 (IQ2: signed level (2c+1) times fp16(d (2ls+1) / 64); Q2_K:
// fma(q, fp16(d sc), fp16(-dmin m)); "Redis 作者出手！ds4...", section 2.3), and
// their activations (x, and h = silu(gate) * up) are rounded to fp16; fp16
// overflow turns into inf in the output rather than a silent error.  The
// shared expert keeps its bf16 weights and takes bf16 activations split into a
// high and a low part (two MFMAs), so its only rounding is fp32 accumulation.
#include "common.h"
#include "iq2_tables.h"
#include "mfma_ops.h"

#include <algorithm>

namespace ds4 {

constexpr int CH_TOK = 64;                     // tokens (routed: slots) per chunk
constexpr int STG_PITCH = 80;                  // LDS stage row: 32 16-bit values + 16 B pad
constexpr int STG_BYTES = CH_TOK * STG_PITCH;  // one K-chunk of A for a chunk of tokens
constexpr int GU_ROWS = 128;                   // n_ff rows per gate/up workgroup (32 per wave)
constexpr int DN_ROWS = 256;                   // n_embd rows per down workgroup (64 per wave)

bool gemm_enabled() { return true; }

int gemm_max_chunks(int n_tok, int NE, int k) {
    const int nq = n_tok * k;
    return min(NE, nq) + (nq + CH_TOK - 1) / CH_TOK;
}

// ---------------------------------------------------------------- routing -> chunks
// Splits every expert's token list into chunks of at most CH_TOK slots:
// chunk = (expert, first list position, count), experts ascending.  By one
// workgroup of 256 threads (thread e: expert e).
__device__ void build_chunks(int NE, const Work &W) {
    __shared__ int wsum[4];
    const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
    int beg = 0, m = 0;
    if (e < NE) {
        beg = W.offsets[e];
        m = W.offsets[e + 1] - beg;
    }
    const int nc = (m + CH_TOK - 1) / CH_TOK;
    int v = nc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int t = __shfl_up(v, off, 64);
        if (lane >= off) v += t;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int pre = 0;
    for (int w = 0; w < wave; ++w) pre += wsum[w];
    const int start = pre + v - nc;
    for (int i = 0; i < nc; ++i)
        W.chunks[start + i] = make_int4(e, beg + i * CH_TOK, min(CH_TOK, m - i * CH_TOK), 0);
    if (e == 255) *W.nchunks = pre + v;
}

// ---------------------------------------------------------------- activation copies
// x (bf16 or fp32) -> fp16 for the routed GEMMs; for fp32 x also the bf16 high
// and low parts used by the shared expert.
// Workgroup 0 also builds the chunk table (one launch instead of two).
template <bool XBF16>
__global__ __launch_bounds__(256) void k_prep_x(const void *__restrict__ x, int64_t n, uint16_t *__restrict__ x16,
                                                uint16_t *__restrict__ xhi, uint16_t *__restrict__ xlo, int NE,
                                                Work W) {
    if (blockIdx.x == 0) build_chunks(NE, W);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        float v;
        if (XBF16) {
            v = bf16_to_f32(static_cast<const uint16_t *>(x)[i]);
        } else {
            v = static_cast<const float *>(x)[i];
            const uint16_t hi = f32_to_bf16_rne(v);
            xhi[i] = hi;
            xlo[i] = f32_to_bf16_rne(v - bf16_to_f32(hi));
        }
        x16[i] = f16_bits(v);
    }
}

// ---------------------------------------------------------------- LDS stage helpers
// The stage holds one K-chunk (32 values, 64 bytes) of A for CH_TOK token rows;
// thread t moves 16 bytes: row t / 4, quarter t % 4.
__device__ __forceinline__ void stage_put(uint8_t *stg, int tid, uint4 v) {
    *reinterpret_cast<uint4 *>(stg + (tid >> 2) * STG_PITCH + (tid & 3) * 16) = v;
}
// A fragment of token tile i: lane (rl, grp) reads row 16 i + rl, K 8 grp..+8.
__device__ __forceinline__ uint4 stage_get(const uint8_t *stg, int i, int rl, int grp) {
    return *reinterpret_cast<const uint4 *>(stg + (16 * i + rl) * STG_PITCH + grp * 16);
}

// ---------------------------------------------------------------- routed experts: block-staged GEMMs
// Both routed kernels work one 256-K block at a time.  The block of A (64
// token rows x 256 K, fp16) sits in an LDS stage (double-buffered, one barrier
// per block), and the MFMA K order is permuted inside the block: in step c
// (0..7) lane group g = l / 16 supplies K 64 g + 8 c..+8.  Each lane therefore
// needs only its own quarter of every weight row block: IQ2 sub-blocks 2g and
// 2g + 1 (16 bytes), Q2_K qs bytes 16 g..16 g+15 (16 bytes) and scale bytes
// 4 g..4 g+3, loaded once per block as one vector per fragment.
//
// The B operand is the dequantized weight rounded to fp16 (relative error at
// most 2^-11 per weight): IQ2 = signed level (2c+1) times fp16(d (2ls+1) / 64),
// Q2_K = fma(q, fp16(d sc), fp16(-dmin m)) in packed fp16, so the MFMAs
// accumulate the whole K range into one fp32 accumulator per tile.
constexpr int RB_WAVES = 16;                      // waves per routed workgroup (1 workgroup per CU)
constexpr int RB_THREADS = 64 * RB_WAVES;
constexpr int GU_FR = 1;                          // gate/up: 16-row fragments per matrix per wave
constexpr int GU_NF = 2 * GU_FR;                  // fragments per wave (gate ones, then up ones)
constexpr int DN_NF = 2;                          // down: 16-row fragments per wave
constexpr int RB_PITCH = 2 * QK + 16;             // stage row: 256 fp16 + 16 B pad (conflict-free A reads)
constexpr int RB_STAGE = CH_TOK * RB_PITCH;       // 33792 bytes
constexpr int RGU_ROWS = RB_WAVES * 16 * GU_FR;   // n_ff rows per gate/up workgroup
constexpr int RDN_ROWS = RB_WAVES * 16 * DN_NF;   // n_embd rows per down workgroup
constexpr int LD_V = CH_TOK * QK * 2 / 16 / RB_THREADS;  // 16-byte vectors per thread per stage
constexpr int LD_PER_ROW = 32 / LD_V;             // threads per token row

// Block stage loader: thread t moves LD_V x 16 bytes: token row t / LD_PER_ROW,
// K 8 LD_V (t % LD_PER_ROW)..+8 LD_V.  Every load is unconditional (a load
// under a condition leaves a path without it, and the first use after the
// join would then wait for every load in flight): rows past the chunk read
// the chunk's last row, whose products land in accumulator rows never stored.
struct BlockLoader {
    const uint16_t *src;   // row start + K offset
    int lds_off;
    __device__ void init(const uint16_t *row, int tid) {
        const int p = tid % LD_PER_ROW;
        src = row + 8 * LD_V * p;
        lds_off = (tid / LD_PER_ROW) * RB_PITCH + 16 * LD_V * p;
    }
    __device__ void load(int bi, uint4 (&r)[LD_V]) const {
#pragma unroll
        for (int j = 0; j < LD_V; ++j) r[j] = *reinterpret_cast<const uint4 *>(src + QK * bi + 8 * j);
    }
    __device__ void store(uint8_t *stg, const uint4 (&r)[LD_V]) const {
#pragma unroll
        for (int j = 0; j < LD_V; ++j) *reinterpret_cast<uint4 *>(stg + lds_off + 16 * j) = r[j];
    }
};
// A fragment for step c of token tile i: row 16 i + rl, K 64 grp + 8 c.
__device__ __forceinline__ half8 block_a(const uint8_t *stg, int i, int c, int rl, int grp) {
    return as_half8(*reinterpret_cast<const uint4 *>(stg + (16 * i + rl) * RB_PITCH + 128 * grp + 16 * c));
}

// Main loop and epilogue of the routed gate/up GEMM for a chunk of NT token
// tiles (NT is a template parameter so the step bodies have no branches).
template <int NT>
__device__ __forceinline__ void gateup_routed_tiles(const Layer &L, const Work &W, const uint4 *T, const uint4 *ST,
                                                    uint8_t *stg0,
                                                    uint8_t *stg1, const BlockLoader &ld, uint4 (&xr)[LD_V],
                                                    const uint8_t *qg, const uint16_t *dg, int fq, int fd, int f0,
                                                    int beg, int cnt, int rl, int grp, int nbe, float *part,
                                                    int nq) {
    const int F = L.n_ff;
    // gate and up planes sit at a fixed distance from each other
    const int64_t qdu = L.iq2_qs[1] - L.iq2_qs[0], ddu = L.iq2_d[1] - L.iq2_d[0];
    auto wload = [&](int fi, int bi) {
        return *reinterpret_cast<const uint4 *>(qg + ((fi >= GU_FR) ? qdu : 0) + (fi % GU_FR) * fq + 64 * bi);
    };
    auto dload = [&](int fi, int bi) { return dg[((fi >= GU_FR) ? ddu : 0) + (fi % GU_FR) * fd + bi]; };
    // weights LA blocks ahead in LA + 1 named buffers used in rotation (the
    // loop is unrolled by LA + 1): a buffer is first read LA blocks after its
    // loads are issued, and nothing copies a value that may still be in flight
    // (a copy would wait for it).  Two blocks ahead for one or two token tiles,
    // whose blocks compute in less than a load's latency, when there are at
    // least 4 blocks; one otherwise (more tiles: their registers would not
    // fit two)
    constexpr int LAM = NT <= 2 ? 2 : 1;
    const int LA = (LAM == 2 && nbe >= 4) ? 2 : 1;
    uint4 w0[GU_NF], w1[GU_NF], w2[GU_NF];
    uint16_t d0[GU_NF], d1[GU_NF], d2[GU_NF];
#pragma unroll
    for (int fi = 0; fi < GU_NF; ++fi) {
        w0[fi] = wload(fi, 0), d0[fi] = dload(fi, 0);
        // unconditionally (with one block ahead, block 0 loads it again)
        w1[fi] = wload(fi, min(1, nbe - 1)), d1[fi] = dload(fi, min(1, nbe - 1));
    }

    floatx4 acc[NT][GU_NF];
    const floatx4 zf = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int fi = 0; fi < GU_NF; ++fi) acc[i][fi] = zf;

    // block bi from (wcur, dcur); block bi + LA's weights into (wl, dl)
    auto block = [&](int bi, const uint4 (&wcur)[GU_NF], const uint16_t (&dcur)[GU_NF], uint4 (&wl)[GU_NF],
                     uint16_t (&dl)[GU_NF]) __attribute__((always_inline)) {
        const bool more = bi + 1 < nbe;
        {
            // the next block's x, then the weights LA blocks ahead (the last
            // block again past the end: unused), unconditionally
            ld.load(min(bi + 1, nbe - 1), xr);
            const int b2 = min(bi + LA, nbe - 1);
#pragma unroll
            for (int fi = 0; fi < GU_NF; ++fi) wl[fi] = wload(fi, b2), dl[fi] = dload(fi, b2);
        }
        const uint8_t *cur = (bi & 1) ? stg1 : stg0;
        half2v scl[GU_NF];
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
            // signs from the mask table for one or two token tiles; with more
            // tiles the A reads keep the LDS busy and the bit arithmetic is
            // cheaper (2048-token prefill: 698 -> 782 us with the table)
            half8 b[GU_NF];
#pragma unroll
            for (int fi = 0; fi < GU_NF; ++fi)
                b[fi] = NT <= 2 ? iq2_b_finish_masked(iq2_b_lookup(T, wcur[fi], cc, rl), iq2_s_lookup(ST, wcur[fi], cc, rl),
                                                      wcur[fi], dcur[fi], cc, scl[fi])
                                : iq2_b_operand(T, wcur[fi], dcur[fi], cc, rl, scl[fi]);
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const half8 a = block_a(cur, i, cc, rl, grp);
#pragma unroll
                for (int fi = 0; fi < GU_NF; ++fi) acc[i][fi] = mfma_f16(a, b[fi], acc[i][fi]);
            }
        }
        if (more) ld.store((bi & 1) ? stg0 : stg1, xr);
        __syncthreads();
    };
    if (LAM == 2 && LA == 2) {
        for (int bi = 0; bi < nbe; bi += 3) {
            block(bi, w0, d0, w2, d2);
            if (bi + 1 >= nbe) break;
            block(bi + 1, w1, d1, w0, d0);
            if (bi + 2 >= nbe) break;
            block(bi + 2, w2, d2, w1, d1);
        }
    } else {
        for (int bi = 0; bi < nbe; bi += 2) {
            block(bi, w0, d0, w1, d1);
            if (bi + 1 >= nbe) break;
            block(bi + 1, w1, d1, w0, d0);
        }
    }

    if (part) {
        // this K range's gate and up sums, slot-major
#pragma unroll
        for (int i = 0; i < NT; ++i) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tt = 16 * i + 4 * grp + v;
                if (tt >= cnt) continue;
                float *prow = part + ((int64_t)blockIdx.z * nq + W.list[beg + tt]) * (2 * F) + f0 + rl;
#pragma unroll
                for (int fp = 0; fp < GU_FR; ++fp) {
                    prow[16 * fp] = acc[i][fp][v];
                    prow[F + 16 * fp] = acc[i][fp + GU_FR][v];
                }
            }
        }
        return;
    }
    // epilogue: h = silu(gate) * up -> fp16 slot rows
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int tt = 16 * i + 4 * grp + v;
            if (tt >= cnt) continue;
            const int q = W.list[beg + tt];
#pragma unroll
            for (int fp = 0; fp < GU_FR; ++fp) {
                const float h = silu(acc[i][fp][v]) * acc[i][fp + GU_FR][v];
                W.hbuf16[(int64_t)q * F + f0 + 16 * fp + rl] = f16_bits(h);
            }
        }
    }
}

// XCD-aware tile order for the routed GEMMs.  Workgroups go to the 8 XCDs
// round-robin by linear id, so the gx row groups of one chunk (consecutive
// ids), which all read that chunk's activation rows, would sit on 8 XCDs with
// 8 separate L2s and each fetch the rows from memory.  Here, within each run
// of 8 gx ids, id 8 m + j takes row group m of chunk 8 g + j: a chunk's row
// groups share one XCD's L2.  Ids past the last whole run keep the plain
// order.  The map is a bijection of the (gx, gy) grid, per K split.
__device__ __forceinline__ void xcd_tile(int gx, int gy, int &tx, int &ty) {
    const int lin = blockIdx.x + gx * blockIdx.y;
    const int run = 8 * gx;
    if (lin < (gy / 8) * run) {
        const int g = lin / run, r = lin - g * run;
        ty = 8 * g + (r & 7);
        tx = r >> 3;
    } else {
        ty = lin / gx;
        tx = lin - ty * gx;
    }
}

// grid: (n_ff / RGU_ROWS, max chunks), RB_THREADS threads.  Wave w covers
// n_ff rows f0..f0+16 GU_FR-1 of gate and up for all tokens of the chunk
// (1..4 token tiles), over the whole n_embd.
// blockIdx.z = K split: 256-K blocks bps z .. bps z + bps - 1.  With part (more
// than one split) the raw sums go to part[z][slot][2 n_ff] for
// k_routed_gu_reduce; nq = slots of the call.
__global__ __launch_bounds__(RB_THREADS, 1) void k_gemm_gateup_routed(Layer L, Work W, int bps, float *part, int nq) {
    int tx, c;
    xcd_tile(gridDim.x, gridDim.y, tx, c);
    if (c >= *W.nchunks) return;
    const int4 ch = W.chunks[c];
    const int e = ch.x, beg = ch.y, cnt = ch.z;
    __shared__ uint4 T[256 * IQ2_REPL];
    __shared__ uint4 ST[128 * IQ2S_REPL];
    __shared__ __align__(16) uint8_t stg[2][RB_STAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = lane & 15, grp = lane >> 4;
    const int E = L.n_embd, F = L.n_ff, k = L.top_k, nbe = L.nbe, b0 = blockIdx.z * bps;

    BlockLoader ld;
    {
        const int sr = tid / LD_PER_ROW;
        ld.init(W.x16 + (int64_t)(W.list[beg + min(sr, cnt - 1)] / k) * E + QK * b0, tid);
    }
    const int f0 = tx * RGU_ROWS + wave * 16 * GU_FR;
    // fragment fi: matrix fi / GU_FR (gate, up), rows f0 + 16 (fi % GU_FR) + rl
    const int64_t rb = ((int64_t)expert_slot(L, e) * F + f0 + rl) * nbe;
    const uint8_t *qg = L.iq2_qs[0] + (rb + b0) * 64 + 16 * grp;  // + 64 bi (up: + iq2_qs[1] - iq2_qs[0])
    const uint16_t *dg = L.iq2_d[0] + rb + b0;                    // + bi
    const int fq = 16 * nbe * 64, fd = 16 * nbe;
    uint4 xr[LD_V];
    ld.load(0, xr);
    iq2_build_lut<true>(T, L.codebook, tid, RB_THREADS);
    if (cnt <= 32) iq2_build_sign_table(ST, tid, RB_THREADS);
    ld.store(stg[0], xr);
    __syncthreads();
    switch ((cnt + 15) >> 4) {
        case 1: gateup_routed_tiles<1>(L, W, T, ST, stg[0], stg[1], ld, xr, qg, dg, fq, fd, f0, beg, cnt, rl, grp, bps, part, nq); break;
        case 2: gateup_routed_tiles<2>(L, W, T, ST, stg[0], stg[1], ld, xr, qg, dg, fq, fd, f0, beg, cnt, rl, grp, bps, part, nq); break;
        case 3: gateup_routed_tiles<3>(L, W, T, ST, stg[0], stg[1], ld, xr, qg, dg, fq, fd, f0, beg, cnt, rl, grp, bps, part, nq); break;
        default: gateup_routed_tiles<4>(L, W, T, ST, stg[0], stg[1], ld, xr, qg, dg, fq, fd, f0, beg, cnt, rl, grp, bps, part, nq); break;
    }
}

template <int NT>
__device__ __forceinline__ void down_routed_tiles(const Layer &L, const Work &W, float *__restrict__ out,
                                                  const uint2 *QT, uint8_t *stg0, uint8_t *stg1, const BlockLoader &ld,
                                                  uint4 (&xr)[LD_V], const uint8_t *qb, const uint8_t *sb,
                                                  const uint32_t *db, int fq, int fs, int fd, bool active, int r0,
                                                  int beg, int cnt, int rl, int grp, int nbf) {
    const int E = L.n_embd;
    // loads are unconditional (inactive waves read row 0: in bounds, unused)
    uint4 qcur[DN_NF], qnext[DN_NF];
    uint32_t scur[DN_NF], snext[DN_NF], dcur[DN_NF], dnext[DN_NF];
#pragma unroll
        for (int fi = 0; fi < DN_NF; ++fi) {
            qcur[fi] = *reinterpret_cast<const uint4 *>(qb + fi * fq);
            scur[fi] = *reinterpret_cast<const uint32_t *>(sb + fi * fs);
            dcur[fi] = db[fi * fd];
        }

    floatx4 acc[NT][DN_NF];
    const floatx4 zf = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int fi = 0; fi < DN_NF; ++fi) acc[i][fi] = zf;

    for (int bi = 0; bi < nbf; ++bi) {
        const bool more = bi + 1 < nbf;
        {
            // the next block (the last one again past the end: unused), unconditionally
            const int bn = min(bi + 1, nbf - 1);
            ld.load(bn, xr);
#pragma unroll
            for (int fi = 0; fi < DN_NF; ++fi) {
                qnext[fi] = *reinterpret_cast<const uint4 *>(qb + fi * fq + 64 * bn);
                snext[fi] = *reinterpret_cast<const uint32_t *>(sb + fi * fs + 16 * bn);
                dnext[fi] = db[fi * fd + bn];
            }
        }
        if (active) {
            const uint8_t *cur = (bi & 1) ? stg1 : stg0;
            half8 dsc[DN_NF], msc[DN_NF];
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                half8 b[DN_NF];
#pragma unroll
                for (int fi = 0; fi < DN_NF; ++fi)
                    b[fi] = q2k_b_operand(QT, qcur[fi], scur[fi], dcur[fi], cc, rl, dsc[fi], msc[fi]);
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    const half8 a = block_a(cur, i, cc, rl, grp);
#pragma unroll
                    for (int fi = 0; fi < DN_NF; ++fi) acc[i][fi] = mfma_f16(a, b[fi], acc[i][fi]);
                }
            }
        }
        if (more) {
            ld.store((bi & 1) ? stg0 : stg1, xr);
#pragma unroll
            for (int fi = 0; fi < DN_NF; ++fi) qcur[fi] = qnext[fi], scur[fi] = snext[fi], dcur[fi] = dnext[fi];
        }
        __syncthreads();
    }
    if (!active) return;

    // epilogue: out[token][row] += w * y
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int tt = 16 * i + 4 * grp + v;
            if (tt >= cnt) continue;
            const int q = W.list[beg + tt];
            const float wgt = W.w[q];
            float *orow = out + (int64_t)(q / L.top_k) * E + r0 + rl;
#pragma unroll
            for (int fi = 0; fi < DN_NF; ++fi) atomicAdd(orow + 16 * fi, wgt * acc[i][fi][v]);
        }
    }
}

// grid: (ceil(n_embd / RDN_ROWS), max chunks), RB_THREADS threads.  Wave w
// covers n_embd rows r0..r0+16 DN_NF-1 for all tokens of the chunk over the
// whole n_ff; waves whose rows lie past n_embd only help with the staging.
// blockIdx.z = K split (256-K blocks bps z ..): every split adds its share of
// w y into out with the same atomics.
__global__ __launch_bounds__(RB_THREADS, 1) void k_gemm_down_routed(Layer L, Work W, float *__restrict__ out, int bps) {
    int tx, c;
    xcd_tile(gridDim.x, gridDim.y, tx, c);
    if (c >= *W.nchunks) return;
    const int4 ch = W.chunks[c];
    const int e = ch.x, beg = ch.y, cnt = ch.z;
    __shared__ uint2 QT[256 * QT_REPL];
    __shared__ __align__(16) uint8_t stg[2][RB_STAGE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = lane & 15, grp = lane >> 4;
    const int E = L.n_embd, F = L.n_ff, nbf = L.nbf, b0 = blockIdx.z * bps;

    BlockLoader ld;
    {
        const int sr = tid / LD_PER_ROW;
        ld.init(W.hbuf16 + (int64_t)W.list[beg + min(sr, cnt - 1)] * F + QK * b0, tid);
    }
    const int r0 = tx * RDN_ROWS + wave * 16 * DN_NF;
    const bool active = r0 < E;
    // fragment fi = rows r0 + 16 fi + rl; one base per plane, fragments 16 rows apart
    const int64_t rb = ((int64_t)expert_slot(L, e) * E + (active ? r0 + rl : 0)) * nbf;
    const uint8_t *qb = L.q2k_qs + (rb + b0) * 64 + 16 * grp;   // + fi * fq + 64 bi
    const uint8_t *sb = L.q2k_sc + (rb + b0) * 16 + 4 * grp;    // + fi * fs + 16 bi
    const uint32_t *db = L.q2k_dd + rb + b0;                    // + fi * fd + bi
    const int fq = 16 * nbf * 64, fs = 16 * nbf * 16, fd = 16 * nbf;
    uint4 xr[LD_V];
    ld.load(0, xr);
    q2k_build_table(QT, tid, RB_THREADS);
    ld.store(stg[0], xr);
    __syncthreads();
    switch ((cnt + 15) >> 4) {
        case 1: down_routed_tiles<1>(L, W, out, QT, stg[0], stg[1], ld, xr, qb, sb, db, fq, fs, fd, active, r0, beg, cnt, rl, grp, bps); break;
        case 2: down_routed_tiles<2>(L, W, out, QT, stg[0], stg[1], ld, xr, qb, sb, db, fq, fs, fd, active, r0, beg, cnt, rl, grp, bps); break;
        case 3: down_routed_tiles<3>(L, W, out, QT, stg[0], stg[1], ld, xr, qb, sb, db, fq, fs, fd, active, r0, beg, cnt, rl, grp, bps); break;
        default: down_routed_tiles<4>(L, W, out, QT, stg[0], stg[1], ld, xr, qb, sb, db, fq, fs, fd, active, r0, beg, cnt, rl, grp, bps); break;
    }
}

// ---------------------------------------------------------------- shared expert gate/up
// grid: (n_ff / GU_ROWS, ceil(n_tok / CH_TOK)).  bf16 weights straight from
// memory; A = x as bf16 (SPLIT: high and low bf16 parts of fp32 x).
// blockIdx.z = K split: this workgroup covers K chunks kcs z .. kcs z + kcs - 1
// (32 values each).  With part, its raw gate and up sums go to
// part[z][token][2 n_ff] for k_shared_gu_reduce; without (one split), h is
// stored directly.
template <bool SPLIT>
__global__ __launch_bounds__(256, 2) void k_gemm_gateup_shared(Layer L, Work W, const uint16_t *__restrict__ xhi,
                                                               const uint16_t *__restrict__ xlo, int n_tok, int kcs,
                                                               float *__restrict__ part) {
    const int t0 = blockIdx.y * CH_TOK;
    const int cnt = min(CH_TOK, n_tok - t0);
    __shared__ __align__(16) uint8_t stg[2][2][STG_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = lane & 15, grp = lane >> 4;
    const int E = L.n_embd, F = L.n_ff;
    const int nt = (cnt + 15) >> 4;
    const int nkc = kcs, kc0 = blockIdx.z * kcs;
    // unconditional loads from clamped addresses (see the shared down kernel)
    const int sr = tid >> 2;
    const int64_t xo = (int64_t)(t0 + min(sr, cnt - 1)) * E + 8 * (tid & 3) + 32 * kc0;

    const int f0 = blockIdx.x * GU_ROWS + wave * 32;
    const uint4 *wp[4];
#pragma unroll
    for (int fi = 0; fi < 4; ++fi) {
        const uint16_t *base = (fi >> 1) ? L.sh_up : L.sh_gate;
        wp[fi] = reinterpret_cast<const uint4 *>(base + (int64_t)(f0 + 16 * (fi & 1) + rl) * E + 8 * grp) +
                 4 * kc0;  // kc: wp[fi][4 kc]
    }
    floatx4 acc[4][4];
    const floatx4 zf = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) acc[i][fi] = zf;
    if constexpr (!SPLIT) {
        // one part of x: the stage's second plane holds the next K chunk, so
        // each barrier covers two chunks (kcs is even)
        uint4 xh[2], wr[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            xh[s] = *reinterpret_cast<const uint4 *>(xhi + xo + 32 * s);
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) wr[s][fi] = wp[fi][4 * s];
        }
        stage_put(stg[0][0], tid, xh[0]);
        stage_put(stg[0][1], tid, xh[1]);
#pragma unroll
        for (int s = 0; s < 2; ++s) xh[s] = *reinterpret_cast<const uint4 *>(xhi + xo + 32 * min(2 + s, nkc - 1));
        __syncthreads();
        for (int k0 = 0; k0 < nkc; k0 += 2) {
            const int buf = (k0 >> 1) & 1;
            uint4 b[2][4];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int fi = 0; fi < 4; ++fi) {
                    b[s][fi] = wr[s][fi];
                    wr[s][fi] = wp[fi][4 * min(k0 + 2 + s, nkc - 1)];
                }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (i < nt) {
                        const uint4 a = stage_get(stg[buf][s], i, rl, grp);
#pragma unroll
                        for (int fi = 0; fi < 4; ++fi) acc[i][fi] = mfma_bf16(a, b[s][fi], acc[i][fi]);
                    }
                }
            if (k0 + 2 < nkc) {
                stage_put(stg[buf ^ 1][0], tid, xh[0]);
                stage_put(stg[buf ^ 1][1], tid, xh[1]);
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    xh[s] = *reinterpret_cast<const uint4 *>(xhi + xo + 32 * min(k0 + 4 + s, nkc - 1));
            }
            __syncthreads();
        }
    } else {
        constexpr int SPF = 2;
        uint4 xh[SPF], xl[SPF], wr[SPF][4];
    #pragma unroll
        for (int s = 0; s < SPF; ++s) {
            const int kq = min(s, nkc - 1);
            xh[s] = *reinterpret_cast<const uint4 *>(xhi + xo + 32 * kq);
            if (SPLIT) xl[s] = *reinterpret_cast<const uint4 *>(xlo + xo + 32 * kq);
    #pragma unroll
            for (int fi = 0; fi < 4; ++fi) wr[s][fi] = wp[fi][4 * kq];
        }
        stage_put(stg[0][0], tid, xh[0]);
        if (SPLIT) stage_put(stg[0][1], tid, xl[0]);
        {
            const int kq = min(SPF, nkc - 1);
            xh[0] = *reinterpret_cast<const uint4 *>(xhi + xo + 32 * kq);
            if (SPLIT) xl[0] = *reinterpret_cast<const uint4 *>(xlo + xo + 32 * kq);
        }
        __syncthreads();


        for (int k0 = 0; k0 < nkc; k0 += SPF) {
    #pragma unroll
            for (int s = 0; s < SPF; ++s) {
                const int kc = k0 + s;
                if (kc >= nkc) break;
                uint4 b[4];
    #pragma unroll
                for (int fi = 0; fi < 4; ++fi) {
                    b[fi] = wr[s][fi];
                    wr[s][fi] = wp[fi][4 * min(kc + SPF, nkc - 1)];
                }
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (i < nt) {
                        const uint4 a = stage_get(stg[kc & 1][0], i, rl, grp);
    #pragma unroll
                        for (int fi = 0; fi < 4; ++fi) acc[i][fi] = mfma_bf16(a, b[fi], acc[i][fi]);
                        if (SPLIT) {
                            const uint4 al = stage_get(stg[kc & 1][1], i, rl, grp);
    #pragma unroll
                            for (int fi = 0; fi < 4; ++fi) acc[i][fi] = mfma_bf16(al, b[fi], acc[i][fi]);
                        }
                    }
                }
                const int sn = (s + 1) & (SPF - 1);
                if (kc + 1 < nkc) {
                    stage_put(stg[(kc + 1) & 1][0], tid, xh[sn]);
                    if (SPLIT) stage_put(stg[(kc + 1) & 1][1], tid, xl[sn]);
                    const int kq = min(kc + 1 + SPF, nkc - 1);
                    xh[sn] = *reinterpret_cast<const uint4 *>(xhi + xo + 32 * kq);
                    if (SPLIT) xl[sn] = *reinterpret_cast<const uint4 *>(xlo + xo + 32 * kq);
                }
                __syncthreads();
            }
        }
    }
    if (part) {
        // this K range's gate and up sums
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i >= nt) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tt = 16 * i + 4 * grp + v;
                if (tt >= cnt) continue;
                float *prow = part + ((int64_t)blockIdx.z * n_tok + t0 + tt) * (2 * F) + f0 + rl;
#pragma unroll
                for (int fp = 0; fp < 2; ++fp) {
                    prow[16 * fp] = acc[i][fp][v];
                    prow[F + 16 * fp] = acc[i][fp + 2][v];
                }
            }
        }
        return;
    }
    // h = silu(gate) * up, stored as bf16 high and low parts
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i >= nt) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int tt = 16 * i + 4 * grp + v;
            if (tt >= cnt) continue;
#pragma unroll
            for (int fp = 0; fp < 2; ++fp) {
                const float h = silu(acc[i][fp][v]) * acc[i][fp + 2][v];
                const uint16_t hi = f32_to_bf16_rne(h);
                const int64_t o = (int64_t)(t0 + tt) * F + f0 + 16 * fp + rl;
                W.hsh_hi[o] = hi;
                W.hsh_lo[o] = f32_to_bf16_rne(h - bf16_to_f32(hi));
            }
        }
    }
}

// ---------------------------------------------------------------- shared expert down
// grid: (n_embd / DN_ROWS, ceil(n_tok / CH_TOK)).  A = h (high and low bf16
// parts), B = bf16 rows of the shared down matrix; out[token][row] += y.
// blockIdx.z = K split as in the shared gate/up GEMM; with part, this K
// range's sums go to part[z][token][n_embd] for k_shared_dn_reduce.
__global__ __launch_bounds__(256, 2) void k_gemm_down_shared(Layer L, Work W, int n_tok, float *__restrict__ out,
                                                             int kcs, float *__restrict__ part) {
    const int t0 = blockIdx.y * CH_TOK;
    const int cnt = min(CH_TOK, n_tok - t0);
    __shared__ __align__(16) uint8_t stg[2][2][STG_BYTES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = lane & 15, grp = lane >> 4;
    const int E = L.n_embd, F = L.n_ff;
    const int nt = (cnt + 15) >> 4;
    const int nkc = kcs, kc0 = blockIdx.z * kcs;
    // loads never depend on a condition (a select between a load and a zero
    // vector becomes a flat load from a stack slot, waited on at once): rows
    // past the chunk read the chunk's last row (their results are dropped),
    // and prefetches past the last K chunk re-read it (unused)
    const int sr = tid >> 2;
    const int64_t ho = (int64_t)(t0 + min(sr, cnt - 1)) * F + 8 * (tid & 3) + 32 * kc0;

    const int r0 = blockIdx.x * DN_ROWS + wave * 64;
    const uint4 *wp[4];
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
        wp[fi] = reinterpret_cast<const uint4 *>(L.sh_down + (int64_t)(r0 + 16 * fi + rl) * F + 8 * grp) + 4 * kc0;
    constexpr int SPF = 2;
    uint4 xh[SPF], xl[SPF], wr[SPF][4];
#pragma unroll
    for (int s = 0; s < SPF; ++s) {
        const int kq = min(s, nkc - 1);
        xh[s] = *reinterpret_cast<const uint4 *>(W.hsh_hi + ho + 32 * kq);
        xl[s] = *reinterpret_cast<const uint4 *>(W.hsh_lo + ho + 32 * kq);
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) wr[s][fi] = wp[fi][4 * kq];
    }
    stage_put(stg[0][0], tid, xh[0]);
    stage_put(stg[0][1], tid, xl[0]);
    {
        const int kq = min(SPF, nkc - 1);
        xh[0] = *reinterpret_cast<const uint4 *>(W.hsh_hi + ho + 32 * kq);
        xl[0] = *reinterpret_cast<const uint4 *>(W.hsh_lo + ho + 32 * kq);
    }
    __syncthreads();

    floatx4 acc[4][4];
    const floatx4 zf = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) acc[i][fi] = zf;

    for (int k0 = 0; k0 < nkc; k0 += SPF) {
#pragma unroll
        for (int s = 0; s < SPF; ++s) {
            const int kc = k0 + s;
            if (kc >= nkc) break;
            uint4 b[4];
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) {
                b[fi] = wr[s][fi];
                wr[s][fi] = wp[fi][4 * min(kc + SPF, nkc - 1)];
            }
            // the high parts for every tile, then the low parts: no MFMA
            // waits on the one just issued
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < nt) {
                    const uint4 a = stage_get(stg[kc & 1][0], i, rl, grp);
#pragma unroll
                    for (int fi = 0; fi < 4; ++fi) acc[i][fi] = mfma_bf16(a, b[fi], acc[i][fi]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i < nt) {
                    const uint4 al = stage_get(stg[kc & 1][1], i, rl, grp);
#pragma unroll
                    for (int fi = 0; fi < 4; ++fi) acc[i][fi] = mfma_bf16(al, b[fi], acc[i][fi]);
                }
            }
            const int sn = (s + 1) & (SPF - 1);
            if (kc + 1 < nkc) {
                stage_put(stg[(kc + 1) & 1][0], tid, xh[sn]);
                stage_put(stg[(kc + 1) & 1][1], tid, xl[sn]);
                const int kq = min(kc + 1 + SPF, nkc - 1);
                xh[sn] = *reinterpret_cast<const uint4 *>(W.hsh_hi + ho + 32 * kq);
                xl[sn] = *reinterpret_cast<const uint4 *>(W.hsh_lo + ho + 32 * kq);
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i >= nt) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int tt = 16 * i + 4 * grp + v;
            if (tt >= cnt) continue;
            if (part) {
                float *prow = part + ((int64_t)blockIdx.z * n_tok + t0 + tt) * E + r0 + rl;
#pragma unroll
                for (int fi = 0; fi < 4; ++fi) prow[16 * fi] = acc[i][fi][v];
                continue;
            }
            // each output element gets exactly one shared contribution, and
            // nothing else writes out meanwhile: a plain read-modify-write
            float *orow = out + (int64_t)(t0 + tt) * E + r0 + rl;
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) orow[16 * fi] += acc[i][fi][v];
        }
    }
}

// ---------------------------------------------------------------- K-split reductions
// h[t][f] = silu(sum_z gate) * sum_z up over the ks splits in order, as bf16 high
// and low parts.
__global__ __launch_bounds__(256) void k_shared_gu_reduce(Work W, const float *__restrict__ part, int n_tok, int F,
                                                          int ks) {
    const int64_t n = (int64_t)n_tok * F;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t t = i / F, f = i - t * F;
        float g = 0.0f, u = 0.0f;
        for (int z = 0; z < ks; ++z) {
            const float *p = part + ((int64_t)z * n_tok + t) * (2 * F);
            g += p[f];
            u += p[F + f];
        }
        const float h = silu(g) * u;
        const uint16_t hi = f32_to_bf16_rne(h);
        W.hsh_hi[i] = hi;
        W.hsh_lo[i] = f32_to_bf16_rne(h - bf16_to_f32(hi));
    }
}
// out[t][r] += sum_z part[z][t][r] over the ks splits in order.
__global__ __launch_bounds__(256) void k_shared_dn_reduce(const float *__restrict__ part, int n_tok, int E, int ks,
                                                          float *__restrict__ out) {
    const int64_t n = (int64_t)n_tok * E;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        float s = 0.0f;
        for (int z = 0; z < ks; ++z) s += part[(int64_t)z * n + i];
        out[i] += s;
    }
}

// h[q][f] = silu(sum_z gate) * sum_z up over the ks splits in order, as fp16,
// for the nq routed slots.
__global__ __launch_bounds__(256) void k_routed_gu_reduce(Work W, const float *__restrict__ part, int nq, int F, int ks) {
    const int64_t n = (int64_t)nq * F;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t q = i / F, f = i - q * F;
        float g = 0.0f, u = 0.0f;
        for (int z = 0; z < ks; ++z) {
            const float *p = part + ((int64_t)z * nq + q) * (2 * F);
            g += p[f];
            u += p[F + f];
        }
        W.hbuf16[i] = f16_bits(silu(g) * u);
    }
}

// K splits for a routed GEMM of wgs workgroups (the grid's chunk rows are an
// upper bound of the work) over nb 256-K blocks: none from 256 workgroups up
// (at 8 tokens splits measured no faster), else about 512 workgroups in all,
// at least 2 blocks per split, at most 8 splits; rows (the slots when the
// splits write partial sums, else 0) times splits within the partial-sum buffer.
static int routed_ksplit(int wgs, int nb, int rows) {
    int ks = 1;
    if (wgs >= 256) return ks;
    while (wgs * ks < 512 && ks < 8 && nb / (2 * ks) >= 2 && 2 * ks * rows <= PART_ROWS) ks *= 2;
    return ks;
}

// K splits for a shared-expert GEMM of wgs workgroups over nkc K chunks: about
// 512 workgroups in all, at least 2 chunks per split, at most 16 splits, and
// splits times tokens within the partial-sum buffer.
static int shared_ksplit(int wgs, int nkc, int n_tok) {
    int ks = 1;
    while (wgs * ks < 512 && ks < 16 && nkc / (2 * ks) >= 2 && 2 * ks * n_tok <= PART_ROWS) ks *= 2;
    return ks;
}

// ---------------------------------------------------------------- launchers
hipError_t launch_gemm_prep(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s) {
    const int64_t nx = (int64_t)n_tok * L.n_embd;
    const int pg = (int)std::min<int64_t>((nx + 255) / 256, 4096);
    if (L.act_dtype == 1)
        hipLaunchKernelGGL(k_prep_x<true>, dim3(pg), dim3(256), 0, s, x, nx, W.x16, nullptr, nullptr, L.n_expert, W);
    else
        hipLaunchKernelGGL(k_prep_x<false>, dim3(pg), dim3(256), 0, s, x, nx, W.x16, W.xhi, W.xlo, L.n_expert, W);
    return hipGetLastError();
}

hipError_t launch_gemm_gateup_routed(const Layer &L, const Work &W, int n_tok, hipStream_t s) {
    const int mc = gemm_max_chunks(n_tok, L.n_expert, L.top_k), gx = L.n_ff / RGU_ROWS, nq = n_tok * L.top_k;
    const int ks = routed_ksplit(gx * mc, L.nbe, nq);
    float *part = ks > 1 ? W.part : nullptr;
    hipLaunchKernelGGL(k_gemm_gateup_routed, dim3(gx, mc, ks), dim3(RB_THREADS), 0, s, L, W, L.nbe / ks, part, nq);
    if (ks > 1) {
        const int nb = (int)std::min<int64_t>(((int64_t)nq * L.n_ff + 255) / 256, 2048);
        hipLaunchKernelGGL(k_routed_gu_reduce, dim3(nb), dim3(256), 0, s, W, W.part, nq, L.n_ff, ks);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_gateup_shared(const Layer &L, const Work &W, const void *x, int n_tok, hipStream_t s) {
    const int gx = L.n_ff / GU_ROWS, gy = (n_tok + CH_TOK - 1) / CH_TOK, nkc = L.n_embd / 32;
    const int ks = shared_ksplit(gx * gy, nkc, n_tok);
    const dim3 g(gx, gy, ks);
    float *part = ks > 1 ? W.part : nullptr;
    if (L.act_dtype == 1)
        hipLaunchKernelGGL(k_gemm_gateup_shared<false>, g, dim3(256), 0, s, L, W, static_cast<const uint16_t *>(x),
                           nullptr, n_tok, nkc / ks, part);
    else
        hipLaunchKernelGGL(k_gemm_gateup_shared<true>, g, dim3(256), 0, s, L, W, W.xhi, W.xlo, n_tok, nkc / ks,
                           part);
    if (ks > 1) {
        const int nb = (int)std::min<int64_t>(((int64_t)n_tok * L.n_ff + 255) / 256, 2048);
        hipLaunchKernelGGL(k_shared_gu_reduce, dim3(nb), dim3(256), 0, s, W, W.part, n_tok, L.n_ff, ks);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_down_routed(const Layer &L, const Work &W, int n_tok, float *out, hipStream_t s) {
    const int mc = gemm_max_chunks(n_tok, L.n_expert, L.top_k), gx = (L.n_embd + RDN_ROWS - 1) / RDN_ROWS;
    const int ks = routed_ksplit(gx * mc, L.nbf, 0);
    hipLaunchKernelGGL(k_gemm_down_routed, dim3(gx, mc, ks), dim3(RB_THREADS), 0, s, L, W, out, L.nbf / ks);
    return hipGetLastError();
}

hipError_t launch_gemm_down_shared(const Layer &L, const Work &W, int n_tok, float *out, hipStream_t s) {
    const int gx = L.n_embd / DN_ROWS, gy = (n_tok + CH_TOK - 1) / CH_TOK, nkc = L.n_ff / 32;
    const int ks = shared_ksplit(gx * gy, nkc, n_tok);
    float *part = ks > 1 ? W.part : nullptr;
    hipLaunchKernelGGL(k_gemm_down_shared, dim3(gx, gy, ks), dim3(256), 0, s, L, W, n_tok, out, nkc / ks, part);
    if (ks > 1) {
        const int nb = (int)std::min<int64_t>(((int64_t)n_tok * L.n_embd + 255) / 256, 2048);
        hipLaunchKernelGGL(k_shared_dn_reduce, dim3(nb), dim3(256), 0, s, W.part, n_tok, L.n_embd, ks, out);
    }
    return hipGetLastError();
}

// Debug: one routed expert matrix exactly as the grouped GEMMs feed it to
// the MFMAs, through iq2_b_operand and q2k_b_operand (which 0 gate, 1 up:
// [n_ff][n_embd]; 2 down: [n_embd][n_ff]), each fp16 value widened to fp32.
// IQ2 values are also decoded with the sign-mask table (iq2_b_finish_masked);
// a value on which the two decodes differ in any bit is written as NaN.
// One thread per (row, 256-K block, lane quarter g), its 8 steps in order.
__global__ __launch_bounds__(256) void k_debug_gemm_b(Layer L, int which, int expert, float *__restrict__ dst) {
    __shared__ uint4 T[256 * IQ2_REPL];
    __shared__ uint4 ST[128 * IQ2S_REPL];
    __shared__ uint2 QT[256 * QT_REPL];
    const int tid = threadIdx.x;
    if (which < 2) {
        iq2_build_lut<true>(T, L.codebook, tid, 256);
        iq2_build_sign_table(ST, tid, 256);
    } else
        q2k_build_table(QT, tid, 256);
    __syncthreads();
    const int rows = which < 2 ? L.n_ff : L.n_embd, nb = which < 2 ? L.nbe : L.nbf;
    const int64_t i = (int64_t)blockIdx.x * 256 + tid;
    if (i >= (int64_t)rows * nb * 4) return;
    const int g = (int)(i & 3);
    const int64_t rbk = i >> 2;
    const int row = (int)(rbk / nb), bi = (int)(rbk % nb);
    const int rl = tid & 15;
    const int64_t rb = ((int64_t)expert * rows + row) * nb + bi;
    float *o = dst + (int64_t)row * nb * QK + (int64_t)bi * QK + 64 * g;
    if (which < 2) {
        const uint4 w = *reinterpret_cast<const uint4 *>(L.iq2_qs[which] + rb * 64 + 16 * g);
        const uint16_t d = L.iq2_d[which][rb];
        half2v scl, scl2;
        for (int cc = 0; cc < 8; ++cc) {
            const half8 b = iq2_b_operand(T, w, d, cc, rl, scl);
            const half8 b2 = iq2_b_finish_masked(iq2_b_lookup(T, w, cc, rl), iq2_s_lookup(ST, w, cc, rl), w, d, cc, scl2);
            const uint4 u = __builtin_bit_cast(uint4, b), u2 = __builtin_bit_cast(uint4, b2);
            const uint32_t dx[4] = {u.x ^ u2.x, u.y ^ u2.y, u.z ^ u2.z, u.w ^ u2.w};
            for (int j = 0; j < 8; ++j)
                o[8 * cc + j] = ((dx[j >> 1] >> (16 * (j & 1))) & 0xFFFFu) ? __builtin_nanf("") : (float)b[j];
        }
    } else {
        const uint4 q = *reinterpret_cast<const uint4 *>(L.q2k_qs + rb * 64 + 16 * g);
        const uint32_t sc = *reinterpret_cast<const uint32_t *>(L.q2k_sc + rb * 16 + 4 * g);
        const uint32_t dd = L.q2k_dd[rb];
        half8 dsc, msc;
        for (int cc = 0; cc < 8; ++cc) {
            const half8 b = q2k_b_operand(QT, q, sc, dd, cc, rl, dsc, msc);
            for (int j = 0; j < 8; ++j) o[8 * cc + j] = (float)b[j];
        }
    }
}

hipError_t launch_debug_gemm_b(const Layer &L, int which, int expert, float *dst, hipStream_t s) {
    const int rows = which < 2 ? L.n_ff : L.n_embd, nb = which < 2 ? L.nbe : L.nbf;
    const int64_t n = (int64_t)rows * nb * 4;
    hipLaunchKernelGGL(k_debug_gemm_b, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, L, which, expert, dst);
    return hipGetLastError();
}

}  // namespace ds4
