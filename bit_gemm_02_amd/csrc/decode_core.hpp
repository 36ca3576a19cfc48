// decode_core.hpp — the decode product's block body (16 * RG weight rows of one problem of
// a grouped launch, four waves splitting K), its batch layout and host-side builders.
// Included by decode.hip (the decode launches) and mixed.hip (prefill tiles and decode
// blocks in one grid).  The design is described at the top of decode.hip.
#pragma once

#include <algorithm>

#include "common.hpp"

namespace bl {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kSuperWords = 16;    // words per row per super-step
constexpr int kDecXldsMaxM = BL_LINEAR_FUSED_MAX_M;       // activations staged in LDS for at
constexpr int kDecXldsBytes = BL_LINEAR_FUSED_MAX_BYTES;  // most this many tokens and bytes
constexpr int kDecCQ = 12;    // fused form, one token: quads per lane kept in registers

struct FwdDev {
    const int8_t *Xq;
    const float *sx;
    const uint32_t *W;
    const float *gamma;
    float *Y;
    int32_t *acc;
    int M, N, K;
    int block_begin;
    const float *R;     // residual added to the output, or NULL
    // Fused decode form only: raw activations, norm, and optional copies of codes / scales.
    const void *X;
    const float *g;
    int8_t *Xq_out;
    float *sx_out;
    float eps;
    int bf16;
    // Layer-call epilogue (fused form): the up projection of a gated pair and the activation.
    const uint32_t *W2;
    const float *gamma2;
    int act;
};


struct FwdBatch {
    FwdDev p[BL_MAX_GROUP];
    int count;
};

// Four activations (fp32 or bf16) of row resource `xr`, elements 4j .. 4j+3, as fp32.
__device__ __forceinline__ float4 load_quad(rsrc_t xr, int j, bool bf16)
{
    if (bf16) {
        const uint32_t lo = buf_load4(xr, (uint32_t)j * 8u), hi = buf_load4(xr, (uint32_t)j * 8u + 4u);
        return make_float4(__uint_as_float(lo << 16), __uint_as_float(lo & 0xFFFF0000u),
                           __uint_as_float(hi << 16), __uint_as_float(hi & 0xFFFF0000u));
    }
    const v4u v = buf_load16(xr, (uint32_t)j * 16u);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                       __uint_as_float(v.w));
}

// Base-3 weights (five codes per byte in blocks of 80 weights per 16 bytes; byte b of a block
// holds weights 4b .. 4b+3 and 64 + b as sum_i (c + 1) * 3^i): the four dwords of a block give
// five 16-byte MFMA operands, weights 0..15, 16..31, 32..47, 48..63 and 64..79 of the block,
// each byte 64 * c as in the two-bit planes.  Each block keeps a 256-entry table in LDS:
// entry v holds the codes of byte value v, the first four (consecutive weights) in one dword
// and the fifth in the low byte of a second.  Dword d of the block (bytes 4d .. 4d+3) then
// gives operand d as the four first dwords of its bytes' entries, unchanged, and dword d of
// operand 4 from the four second dwords with two v_perm_b32 selects.  (Digits extracted
// arithmetically, q = (v * 171) >> 9 = floor(v / 3) in 16-bit lanes, and a layout that
// needed a 4 x 4 byte transpose after the lookup both measured slower.)
__device__ __forceinline__ void b3_table_entry(uint32_t v, uint32_t &lo, uint32_t &hi)
{
    uint32_t c[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const uint32_t d = v % 3u;                     // digit = code + 1
        c[i] = d == 0 ? 0xC0u : (d == 1 ? 0x00u : 0x40u);
        v /= 3u;
    }
    lo = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    hi = c[4];
}

// Dword d of a block -> operand d (four dwords) and dword d of operand 4.
__device__ __forceinline__ void unpack_b3_dword(uint32_t w, const uint32_t *lut, v4i &op, uint32_t &op4)
{
    uint32_t a[4], b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t idx = (w >> (8 * e)) & 0xFFu;
        const v2u ent = *reinterpret_cast<const v2u *>(lut + 2 * idx);
        a[e] = ent.x;
        b[e] = ent.y;
    }
    op = v4i{(int)a[0], (int)a[1], (int)a[2], (int)a[3]};
    op4 = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u) | __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);
}

// FULL_K: every problem of the launch has K % 256 == 0, so super-steps never run past a
// row and rows are 64-byte aligned (one 16-byte load per lane, no tail masking).
// QUANT (with XLDS): the fused decode form.  The activations arrive unquantized;
// each wave reduces absmax (and the sum of squares for the norm) over its K piece of every
// token row, the four waves combine them through LDS in a fixed order, and each wave then
// quantizes its piece straight into the LDS operand buffer (the same quant4 / act_scale
// arithmetic as the activation-quantization kernels).  The first block of a problem also
// writes the codes and scales out when asked to.
// PAIR (fused form only): a gated pair of projections with one set of activations; the
// block's first RG/2 row groups are rows of W, the other RG/2 the same rows of W2, and the
// epilogue combines the two outputs of each row through the activation.
// B3 (fused form only): base-3 weights; a super-step is 320 weights (four 16-byte blocks a
// row, one per lane group), five MFMAs per row group.
template <int RG, bool XLDS, bool QUANT, bool FULL_K, bool PAIR = false, bool BF16 = false,
          bool B3 = false>
__device__ __forceinline__ void decode_block(const FwdBatch &b, int bid)
{
    static_assert(!QUANT || XLDS, "the fused form stages codes in LDS");
    static_assert(!PAIR || (QUANT && RG % 2 == 0), "pairs: fused form, even row groups");
    static_assert(!B3 || QUANT, "base-3 weights: fused form");
    constexpr int EPS = B3 ? 320 : 256;    // weights per super-step
    // Base-3 decode table (ready after the quantization phase's barrier).
    __shared__ __align__(8) uint32_t b3lut[B3 ? 512 : 2];
    if (B3) {
        uint32_t lo, hi;
        b3_table_entry(threadIdx.x, lo, hi);     // 256 threads, one entry each
        *reinterpret_cast<v2u *>(b3lut + 2 * threadIdx.x) = v2u{lo, hi};
    }
    constexpr int GN = PAIR ? RG / 2 : RG;    // row groups of output rows per block
    constexpr int ROWS = 16 * GN;
    // Super-steps per chunk (two chunks of loads in flight).  Four per chunk measured slower:
    // the dead loads past a short wave's range cost more than the deeper queue gains.
    constexpr int kDecPF = 2;
    __shared__ v4i red[kDecWaves][RG][kWave];
    // XLDS: the activations X[0..M)[0..K) staged in LDS (row stride K), each wave copying
    // only its own K piece, followed by one zeroed 16-byte chunk per wave.
    extern __shared__ __align__(16) unsigned char xs[];

    int prob = 0;
#pragma unroll 1
    while (prob + 1 < b.count && bid >= b.p[prob + 1].block_begin)
        ++prob;
    const FwdDev &p = b.p[prob];
    const int n0 = (bid - p.block_begin) * ROWS;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int r = lane & 15;
    const int g = lane >> 4;
    const int row_bytes = B3 ? 16 * ((p.K + 79) / 80) : p.K / 4;
    const int words = row_bytes / 4;
    // Weight rows n0 .. n0+ROWS-1 (rows past N read as zero); tokens 0 .. M-1 (rows past M
    // read as zero: their offsets r * K + ... lie at or past M * K).
    const rsrc_t wres = make_rsrc(p.W + (int64_t)n0 * words, rows_bytes(n0, ROWS, p.N, row_bytes));
    const rsrc_t wres2 = PAIR ? make_rsrc(p.W2 + (int64_t)n0 * words, rows_bytes(n0, ROWS, p.N, row_bytes))
                              : wres;
    const rsrc_t xres = make_rsrc(p.Xq, (uint32_t)p.M * (uint32_t)p.K);
    const uint32_t wbase = (uint32_t)r * row_bytes;
    const uint32_t xbase = (uint32_t)r * p.K;
    const uint32_t gstride = 16u * (uint32_t)row_bytes;   // bytes between row groups
    const uint32_t zero_off = (uint32_t)p.M * (uint32_t)p.K + 16u * (uint32_t)wave;

    const int supers = (words + kSuperWords - 1) / kSuperWords;
    const int t_begin = (supers * wave) / kDecWaves;
    const int t_end = (supers * (wave + 1)) / kDecWaves;

    struct Chunk {
        v4u x[kDecPF][4];
        v4u w[kDecPF][RG];
    };
    // Super-steps t0 .. t0+PF-1; those at or past t_end load zeros (offset "infinity"), so
    // every chunk issues the same loads and the wait before a chunk's use is a fixed count.
    auto load = [&](Chunk &c, int t0) {
#pragma unroll
        for (int u = 0; u < kDecPF; ++u) {
            const int w = (t0 + u) * kSuperWords + 4 * g;
            const bool live = (t0 + u) < t_end;
#pragma unroll
            for (int q = 0; q < RG; ++q) {
                const bool second = PAIR && q >= GN;
                const rsrc_t res = second ? wres2 : wres;
                const uint32_t rowoff = wbase + (uint32_t)(second ? q - GN : q) * gstride;
                if (B3) {
                    // Rows are whole 16-byte blocks: a block is all in or all past the row.
                    const int blk = (t0 + u) * 4 + g;
                    c.w[u][q] = buf_load16(res, live && blk < row_bytes / 16 ? rowoff + 16u * blk : kOOB);
                } else if (FULL_K) {
                    c.w[u][q] = buf_load16(res, live ? rowoff + 4u * w : kOOB);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bool ok = live && (w + j) < words;
                        c.w[u][q][j] = buf_load4(res, ok ? rowoff + 4u * (w + j) : kOOB);
                    }
                }
            }
            if (!XLDS) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool ok = live && (FULL_K || (w + j) < words);
                    c.x[u][j] = buf_load16(xres, ok ? xbase + 16u * (w + j) : kOOB);
                }
            }
        }
    };
    // Activation operand of super-step t, word j: from registers, or read from LDS (token
    // rows past M, dead super-steps and words past K read the zero chunk).
    auto xop = [&](const Chunk &c, int t0, int u, int j) -> v4i {
        if (!XLDS)
            return v4i{(int)c.x[u][j].x, (int)c.x[u][j].y, (int)c.x[u][j].z, (int)c.x[u][j].w};
        const int w = (t0 + u) * kSuperWords + 4 * g + j;
        const bool ok = r < p.M && (t0 + u) < t_end && (FULL_K || w < words);
        return *reinterpret_cast<const v4i *>(xs + (ok ? xbase + 16u * w : zero_off));
    };
    v4i acc[RG];
#pragma unroll
    for (int q = 0; q < RG; ++q)
        acc[q] = v4i{0, 0, 0, 0};
    auto compute = [&](const Chunk &c, int t0) {
        if constexpr (B3) {
#pragma unroll
            for (int u = 0; u < kDecPF; ++u) {
                // Operand i of lane group g's block: 16-weight chunk 20 (t0 + u) + 5g + i.
                v4i a[5];
#pragma unroll
                for (int i = 0; i < 5; ++i) {
                    const int ch = (t0 + u) * 20 + 5 * g + i;
                    const bool ok = r < p.M && (t0 + u) < t_end && ch < p.K / 16;
                    a[i] = *reinterpret_cast<const v4i *>(xs + (ok ? xbase + 16u * ch : zero_off));
                }
#pragma unroll
                for (int q = 0; q < RG; ++q) {
                    v4i op[4];
                    uint32_t op4[4];
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        unpack_b3_dword(c.w[u][q][v], b3lut, op[v], op4[v]);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], op[i], acc[q], 0, 0, 0);
                    acc[q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        a[4], v4i{(int)op4[0], (int)op4[1], (int)op4[2], (int)op4[3]}, acc[q], 0, 0, 0);
                }
            }
            return;
        }
#pragma unroll
        for (int u = 0; u < kDecPF; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4i a = xop(c, t0, u, j);
#pragma unroll
                for (int q = 0; q < RG; ++q)
                    acc[q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, unpack_word64(c.w[u][q][j]),
                                                                  acc[q], 0, 0, 0);
            }
    };

    // Epilogue inputs first (gamma, the row scales of this lane's tokens m = 4g + v): the
    // epilogue then does not wait on a memory round trip of its own.
    const rsrc_t sres = make_rsrc(p.sx, QUANT ? 0u : (uint32_t)p.M * 4u);   // past M: 0
    float sxv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        sxv[v] = QUANT ? 0.0f : __uint_as_float(buf_load4(sres, (uint32_t)(4 * g + v) * 4u));
    const float gammaf = __uint_as_float(buf_load4(make_rsrc(p.gamma, 4u), 0u));
    const float gamma2f = PAIR ? __uint_as_float(buf_load4(make_rsrc(p.gamma2, 4u), 0u)) : 0.0f;
    __builtin_amdgcn_sched_barrier(0);

    // Two chunks of weight loads in flight from the start; then the activation piece is
    // staged (its loads queue behind them); then each step multiplies the older chunk and
    // refills it with the chunk two ahead (past the wave's range, loads and multiplies see
    // zeros).  (The scheduling barrier keeps the refill where it
    // is: left alone, the compiler sinks it below the next multiplies, halving the loads in
    // flight.)
    // Fused form: this wave's piece of the activations, elements [e0, e1) of each token row.
    const int e0 = t_begin * EPS;
    const int e1 = min(t_end * EPS, p.K);
    const int quads = (e1 - e0) / 4;
    const bool norm = QUANT && p.g != nullptr;
    constexpr bool bf16 = BF16;      // the activation dtype is a launch-wide constant
    constexpr int esize = bf16 ? 2 : 4;
    const rsrc_t gr = make_rsrc(p.g, norm ? (uint32_t)p.K * 4u : 0u);
    auto row = [&](int m) {
        return make_rsrc(static_cast<const unsigned char *>(p.X) + (int64_t)m * p.K * esize,
                         (uint32_t)p.K * esize);
    };
    auto quad_g = [&](int j) {
        const v4u v = buf_load16(gr, (uint32_t)j * 16u);
        return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                           __uint_as_float(v.w));
    };
    // One token whose row takes up to kDecCQ quads per thread: the row is quantized block-wide
    // in 16-byte chunks (4 fp32 or 8 bf16 values; thread t takes chunks t, t + 256, ...), in
    // the same order as the one-token call (gemv.hip) — per thread over its chunks, then
    // across lanes and across waves in a fixed order — so the two give the same scale bit for
    // bit.  Every activation (and norm weight) load is issued before the weight loads, so the
    // quantization does not wait behind the weight stream (loads complete in issue order), and
    // the loads land in raw registers that are converted only after the weight loads are out
    // (a use next to a load makes the wave wait for it, which would serialize the loads).
    // Otherwise each wave quantizes its own piece of every token row, four quads per lane at a
    // time after the weight loads, re-read for the quantization pass.
    constexpr int QPC = BF16 ? 2 : 1;                 // quads per chunk
    constexpr int CH = kDecCQ / QPC;                  // chunks per thread kept in registers
    const int nchunk = p.K * (BF16 ? 2 : 4) / 16;
    const bool cached = QUANT && p.M == 1 && nchunk <= CH * kDecThreads;
    v4u rx[CH], rgw[kDecCQ];
    if (cached) {
        const rsrc_t xr = row(0);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int i = (int)threadIdx.x + c * kDecThreads;
            rx[c] = v4u{0, 0, 0, 0};
#pragma unroll
            for (int h = 0; h < QPC; ++h)
                rgw[QPC * c + h] = v4u{0, 0, 0, 0};
            if (c * kDecThreads < nchunk) {      // block-uniform: no loads past the row
                rx[c] = buf_load16(xr, i < nchunk ? 16u * (uint32_t)i : kOOB);
                if (norm) {
#pragma unroll
                    for (int h = 0; h < QPC; ++h)
                        rgw[QPC * c + h] = buf_load16(gr, i < nchunk ? 16u * (uint32_t)(QPC * i + h) : kOOB);
                }
            }
        }
    }
    // Chunk c of the cached row as QPC quads of fp32 values.
    auto chunk_quads = [&](int c, float4 *x) {
        const v4u v = rx[c];
        if (BF16) {
            x[0] = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                               __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
            x[QPC - 1] = make_float4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xFFFF0000u),
                                     __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xFFFF0000u));
        } else {
            x[0] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                               __uint_as_float(v.w));
        }
    };
    auto g_quad = [&](int c, int h) {
        const v4u v = rgw[QPC * c + h];
        return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                           __uint_as_float(v.w));
    };
    __builtin_amdgcn_sched_barrier(0);

    Chunk c0, c1;
    load(c0, t_begin);
    __builtin_amdgcn_sched_barrier(0);
    load(c1, t_begin + kDecPF);
    __builtin_amdgcn_sched_barrier(0);
    __shared__ float q_amax[kDecWaves][kDecXldsMaxM];
    __shared__ double q_ss[kDecWaves][kDecXldsMaxM];
    if (QUANT) {
        // Partial absmax of u (u = x, or fl32(x * g)) and sum of x^2 over this wave's piece.
        const bool first = bid == p.block_begin;
        if (cached) {
            float amax = 0.0f;
            double ss = 0.0;
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                if (c * kDecThreads < nchunk) {
                    float4 x[QPC];
                    chunk_quads(c, x);
#pragma unroll
                    for (int h = 0; h < QPC; ++h) {
                        const float4 u = norm ? mul4(x[h], g_quad(c, h)) : x[h];
                        amax = fmaxf(amax, absmax4(u));
                        if (norm)
                            ss = sumsq4(ss, x[h]);
                    }
                }
            }
            amax = wave_max(amax);
            if (norm)
                ss = wave_sum_fixed(ss);
            if (lane == 0) {
                q_amax[wave][0] = amax;
                q_ss[wave][0] = ss;
            }
        } else {
#pragma unroll
            for (int m = 0; m < kDecXldsMaxM; ++m) {
                if (m < p.M) {
                    const rsrc_t xr = row(m);
                    float amax = 0.0f;
                    double ss = 0.0;
                    for (int q0 = lane; q0 < quads; q0 += 4 * kWave) {
                        float4 f[4], gq[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) {     // four loads in flight (zeros past)
                            const int q = q0 + u * kWave;
                            const int j = q < quads ? e0 / 4 + q : (int)(kOOB / 16u);
                            f[u] = load_quad(xr, j, bf16);
                            if (norm)
                                gq[u] = quad_g(j);
                        }
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const float4 uu = norm ? mul4(f[u], gq[u]) : f[u];
                            amax = fmaxf(amax, absmax4(uu));
                            if (norm)
                                ss = sumsq4(ss, f[u]);
                        }
                    }
                    amax = wave_max(amax);
                    if (norm)
                        ss = wave_sum_fixed(ss);
                    if (lane == 0) {
                        q_amax[wave][m] = amax;
                        q_ss[wave][m] = ss;
                    }
                }
            }
        }
        __syncthreads();
        if (cached) {
            float a = q_amax[0][0];
#pragma unroll
            for (int w = 1; w < kDecWaves; ++w)
                a = fmaxf(a, q_amax[w][0]);
            const float inv = a == 0.0f ? 0.0f : 127.0f / a;  // correctly rounded division
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int i = (int)threadIdx.x + c * kDecThreads;
                if (c * kDecThreads < nchunk && i < nchunk) {
                    float4 x[QPC];
                    chunk_quads(c, x);
#pragma unroll
                    for (int h = 0; h < QPC; ++h) {
                        const int q = QPC * i + h;
                        const char4 cq = quant4(norm ? mul4(x[h], g_quad(c, h)) : x[h], inv);
                        *reinterpret_cast<char4 *>(xs + 4u * q) = cq;
                        if (first && p.Xq_out)
                            *reinterpret_cast<char4 *>(p.Xq_out + 4 * q) = cq;
                    }
                }
            }
        } else {
#pragma unroll
            for (int m = 0; m < kDecXldsMaxM; ++m) {
                if (m < p.M) {
                    float a = q_amax[0][m];
#pragma unroll
                    for (int w = 1; w < kDecWaves; ++w)
                        a = fmaxf(a, q_amax[w][m]);
                    const float inv = a == 0.0f ? 0.0f : 127.0f / a;  // correctly rounded division
                    const rsrc_t xr = row(m);
                    for (int q0 = lane; q0 < quads; q0 += 4 * kWave) {
                        float4 f[4], gq[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int q = q0 + u * kWave;
                            const int j = q < quads ? e0 / 4 + q : (int)(kOOB / 16u);
                            f[u] = load_quad(xr, j, bf16);
                            if (norm)
                                gq[u] = quad_g(j);
                        }
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int q = q0 + u * kWave;
                            if (q < quads) {
                                const int j = e0 / 4 + q;
                                const char4 c = quant4(norm ? mul4(f[u], gq[u]) : f[u], inv);
                                *reinterpret_cast<char4 *>(xs + (uint32_t)m * p.K + 4u * j) = c;
                                if (first && p.Xq_out)
                                    *reinterpret_cast<char4 *>(p.Xq_out + (int64_t)m * p.K + 4 * j) = c;
                            }
                        }
                    }
                }
            }
        }
        // Scales of this lane's epilogue tokens m = 4g + v (and the optional copy).
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = 4 * g + v;
            if (m < p.M) {
                float a = q_amax[0][m];
                double ss = q_ss[0][m];
#pragma unroll
                for (int w = 1; w < kDecWaves; ++w) {
                    a = fmaxf(a, q_amax[w][m]);
                    ss += q_ss[w][m];
                }
                sxv[v] = act_scale(a, ss, p.K, p.eps, norm);
                if (first && p.sx_out && wave == 0 && r == 0)
                    p.sx_out[m] = sxv[v];
            }
        }
        if (lane == 0)
            *reinterpret_cast<v4u *>(xs + zero_off) = v4u{0, 0, 0, 0};
        if (cached) {
            // The block-wide form: every wave reads codes other waves wrote.
            __syncthreads();
        } else {
            // Each wave reads only the codes it wrote: LDS operations of one wave complete in
            // order, so a wave-scope fence (no instruction, no wait) suffices.
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    } else if (XLDS) {
        // Copy this wave's piece, rows 0 .. M-1, k in [16 * kw0, 16 * kw1), 16 bytes per lane.
        const int kw0 = t_begin * kSuperWords;
        const int kw1 = min(t_end * kSuperWords, words);
        const int span = kw1 - kw0;
        const int chunks = p.M * span;
        for (int c = lane; c < chunks; c += kWave) {
            const int m = c / span, kw = kw0 + c % span;
            const uint32_t off = (uint32_t)m * p.K + 16u * (uint32_t)kw;
            *reinterpret_cast<v4u *>(xs + off) = buf_load16(xres, off);
        }
        if (lane == 0)
            *reinterpret_cast<v4u *>(xs + zero_off) = v4u{0, 0, 0, 0};
        // Lanes read what other lanes of the same wave wrote: LDS operations of one wave
        // complete in order, so a wave-scope fence (no instruction, no wait) suffices.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    for (int t = t_begin; t < t_end; t += 2 * kDecPF) {
        compute(c0, t);
        load(c0, t + 2 * kDecPF);
        __builtin_amdgcn_sched_barrier(0);
        compute(c1, t + kDecPF);       // all zeros when past t_end
        load(c1, t + 3 * kDecPF);
        __builtin_amdgcn_sched_barrier(0);
    }

#pragma unroll
    for (int q = 0; q < RG; ++q)
        red[wave][q][lane] = acc[q];
    __syncthreads();
    if (wave >= GN)
        return;
    v4i s = red[0][wave][lane];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w)
        s += red[w][wave][lane];
    v4i s2 = v4i{0, 0, 0, 0};
    if (PAIR) {
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w)
            s2 += red[w][wave + GN][lane];
    }

    // s holds 64 * D[m][n] for m = 4 * g + v (v = register index), n = n0 + 16 * wave + r.
    const int n = n0 + 16 * wave + r;
    if (n >= p.N)
        return;
    const double gamma = (double)gammaf;
    const int accv[4] = {s.x, s.y, s.z, s.w};
    const int accv2[4] = {s2.x, s2.y, s2.z, s2.w};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m < p.M) {
            const int a = accv[v] >> 6;  // exact: the sum is a multiple of 64
            const double scale = gamma * (double)sxv[v];
            float y = (float)((double)a * scale);
            if (PAIR) {
                const float y2 = (float)((double)(accv2[v] >> 6) * ((double)gamma2f * (double)sxv[v]));
                y = ffn_act(p.act, y, y2);
            } else if (QUANT && p.act != BL_ACT_NONE) {
                y = ffn_act(p.act, y, 0.0f);
            }
            if (p.R)
                y = y + p.R[(int64_t)m * p.N + n];
            p.Y[(int64_t)m * p.N + n] = y;
            if (!QUANT && p.acc)
                p.acc[(int64_t)m * p.N + n] = a;
        }
    }
}

// Fused decode problems (longest K first) -> batch; returns the block count (ROWS weight rows
// per block) and whether every K is a multiple of 256.
template <int RG, bool PAIR>
static int build_linear_batch(const bl_linear_ex_problem *const *q, int count, FwdBatch &b,
                              bool &full_k)
{
    constexpr int ROWS = 16 * (PAIR ? RG / 2 : RG);
    int order[BL_MAX_GROUP];
    for (int i = 0; i < count; ++i)
        order[i] = i;
    std::stable_sort(order, order + count, [&](int a, int c) { return q[a]->K > q[c]->K; });
    int blocks = 0;
    full_k = true;
    for (int o = 0; o < count; ++o) {
        const bl_linear_ex_problem &s = *q[order[o]];
        full_k = full_k && (s.K % 256 == 0);
        FwdDev &d = b.p[o];
        d.W = s.W_packed;
        d.gamma = s.gamma;
        d.Y = s.Y;
        d.R = s.residual;
        d.M = (int)s.M;
        d.N = (int)s.N;
        d.K = (int)s.K;
        d.block_begin = blocks;
        d.X = s.X;
        d.g = s.norm_weight;
        d.Xq_out = s.X_q;
        d.sx_out = s.x_scale;
        d.eps = s.eps;
        d.bf16 = s.x_dtype == BL_BF16;
        d.W2 = s.W2_packed;
        d.gamma2 = s.gamma2;
        d.act = s.act;
        blocks += (d.N + ROWS - 1) / ROWS;
    }
    b.count = count;
    return blocks;
}

// Dynamic LDS of the staged-activation form: every problem's M x K codes plus one zeroed
// 16-byte chunk per wave.
inline size_t decode_xlds_bytes(const FwdBatch &b)
{
    size_t lds = 0;
    for (int i = 0; i < b.count; ++i)
        lds = std::max(lds, (size_t)b.p[i].M * (size_t)b.p[i].K + 16 * kDecWaves);
    return lds;
}

}  // namespace bl
