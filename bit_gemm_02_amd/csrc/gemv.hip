// gemv.hip — the one-token decode call: activation quantization and the streaming ternary
// product of a single token row in one launch.
//
// At one token the product reads every packed weight once and does almost no arithmetic per
// byte, so it is bound by HBM (SLM750-Edge card, "Performance": single-token decode is
// bandwidth-bound).  A launch over a whole layer set moves only a few tens of MB — a few
// microseconds at full bandwidth — which is about as long as a handful of memory round trips
// under load.  A wave that streams its weights in several dependent rounds (issue, wait,
// multiply, issue the next) therefore finishes well after the rest of the chip, with its
// later rounds queued behind everybody's first.  This kernel cuts the work so that each wave
// has one round: a wave owns one group of 16 weight rows (two for a gated pair: the same rows
// of both projections) over one slice of K, and has every load of that slice in flight before
// it multiplies.  Long rows are split into 2 or 4 slices (one per wave of the block, summed
// through LDS at the end, exactly, in a fixed order) so that every wave moves about the same
// number of bytes whatever the projection's shape; short rows give each wave of a block its
// own row group.
//
// The token's int8 codes need the absmax of the whole row (BitDistill article: INT8
// activations; absmax scale per token), so every block quantizes the row itself, with the same
// arithmetic as the activation-quantization kernels (quant4, act_scale): its four waves copy
// the row into LDS with direct-to-LDS loads issued before any weight load, the partial maxima
// (and sums of squares) meet in LDS in a fixed order, and the codes go to LDS, where the waves
// read them as the MFMA's activation operand.  The row copies get no priority in the memory
// system: with every wave's full round of weight loads ahead of them they arrived microseconds
// late (per-wave timestamps), so each wave sends only its first four super-steps of weights
// before it waits for the row, and the rest right after the quantization.
//
// Product: v_mfma_i32_16x16x64_i8 with 16 weight rows as the B operand (a lane (r, g) holds
// words 16t + 4g .. 16t + 4g + 3 of row r, one 16-byte load per super-step t of 256 weights,
// expanded to 64 * c with one shift and one mask per four weights; see plane64) and the
// token's codes as the A operand.  On decode tiles the same codes are stored plane-major with
// three of the four planes offset by one, which leaves one mask per four weights and no shift
// (the instruction count of the expansion set the kernel's tail); the offsets are removed
// exactly with the sum of the affected activation codes.  Only row 0 of the output is used: every lane reads the
// token's codes for its k range (lanes of one lane group read the same 16 bytes, a broadcast),
// so the other 15 rows of the result repeat row 0 and are ignored.
#include <algorithm>

#include "decode_core.hpp"

namespace bl {

constexpr int kGvThreads = 256;
constexpr int kGvWaves = kGvThreads / kWave;
constexpr int kGvLoadsPerWave = 12;  // target 16-byte weight loads per lane per wave (one round)
constexpr int kGvQuads = 12;         // activation quads per thread: rows up to 12288 values
constexpr size_t kGvMaxLds = 64 * 1024;

// Dynamic LDS of a launch: the raw row of the longest problem in whole 1 KB copies, then the
// codes of its super-steps.
static void gemv_lds(const bl_linear_ex_problem *const *q, int count, bool bf16, bool b3,
                     int &c_off, size_t &bytes)
{
    int k_max = 16;
    for (int i = 0; i < count; ++i)
        k_max = std::max(k_max, (int)q[i]->K);
    const int supers = b3 ? ((k_max + 79) / 80 + 3) / 4 : (k_max / 16 + 15) / 16;
    c_off = (k_max * (bf16 ? 2 : 4) + 1023) / 1024 * 1024;
    bytes = (size_t)c_off + (size_t)(b3 ? 320 : 256) * supers;
}

bool gemv_fits(const bl_linear_ex_problem *const *q, int count, bool bf16, bool b3)
{
    for (int i = 0; i < count; ++i)
        if (q[i]->K > kGvThreads * 4 * kGvQuads || (!b3 && q[i]->K % 64 != 0))
            return false;
    int c_off;
    size_t bytes;
    gemv_lds(q, count, bf16, b3, c_off, bytes);
    return bytes <= kGvMaxLds;
}

struct GvDev {
    const void *X;          // [K] fp32 or bf16
    const float *g;         // [K] RMSNorm weight or NULL
    const uint32_t *W;      // [N][K/16] packed codes (the gate projection of a pair)
    const uint32_t *W2;     // pair: the up projection
    const float *gamma;
    const float *gamma2;
    const float *R;         // [N] residual or NULL
    float *Y;               // [N]
    int8_t *Xq_out;         // optional copies of the codes and the scale
    float *sx_out;
    float eps;
    int N, K;
    int ks_log2;            // slices per row group: 1, 2 or 4 (log2)
    int act;
    int block_begin;
};

struct GvBatch {
    GvDev p[BL_MAX_GROUP];
    int count;
    int c_off;              // LDS offset of the codes (the raw row comes first)
};

// S: super-steps (16-byte loads per lane and row group) in one round; BF16: activation dtype;
// PAIR: gated pair (two row groups per wave, the epilogue applies the activation); NORM: every
// problem of the launch has an RMSNorm weight (held in registers: rows of at most 12288); B3:
// base-3 rows (16-byte blocks of 80 weights, see b3_table_entry; a super-step is then 320
// weights and five MFMAs per row group, the expansion a table lookup in LDS).  Two-bit rows
// have K % 64 == 0, so a lane's 16 bytes never straddle the end of a row.
template <int S, bool BF16, bool PAIR, bool NORM, bool B3, bool TL>
__global__ __launch_bounds__(kGvThreads) void gemv_kernel(GvBatch b)
{
    static_assert(!(TL && (PAIR || B3)), "decode tiles: single two-bit projections");
    constexpr int G = PAIR ? 2 : 1;
    static_assert(!B3 || !PAIR, "base-3 rows: single projections");
    __shared__ __align__(8) uint32_t b3lut[B3 ? 512 : 2];
    if (B3) {
        uint32_t lo, hi;
        b3_table_entry(threadIdx.x, lo, hi);     // 256 threads, one entry each
        *reinterpret_cast<v2u *>(b3lut + 2 * threadIdx.x) = v2u{lo, hi};
    }
    __shared__ float s_amax[kGvWaves];
    __shared__ double s_ss[kGvWaves];
    __shared__ int s_red[kGvWaves][G][16];
    __shared__ int s_csum[kGvWaves];        // decode tiles: per wave, sum of offset-plane codes
    extern __shared__ __align__(16) unsigned char lds[];

    int prob = 0;
#pragma unroll 1
    while (prob + 1 < b.count && (int)blockIdx.x >= b.p[prob + 1].block_begin)
        ++prob;
    const GvDev &p = b.p[prob];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int r = lane & 15;
    const int g = lane >> 4;
    const int ksl = p.ks_log2;
    const int rg = (((int)blockIdx.x - p.block_begin) << (2 - ksl)) + (wave >> ksl);
    const int slice = wave & ((1 << ksl) - 1);
    const int n0 = rg * 16;
    const int n = n0 + r;                 // output row of lanes 0..15
    const int K = p.K;
    const int words = K >> 4;
    const int nblk = (K + 79) / 80;       // base-3 blocks per row
    const int row_bytes = B3 ? 16 * nblk : K >> 2;
    const int supers = B3 ? (nblk + 3) >> 2 : (words + 15) >> 4;
    const int t_begin = (supers * slice) >> ksl;
    const int t_end = (supers * (slice + 1)) >> ksl;
    const bool first = (int)blockIdx.x == p.block_begin;
    unsigned char *const xraw = lds;
    unsigned char *const codes = lds + b.c_off;

    // ---- epilogue inputs first, so the epilogue does not wait on a round trip of its own
    const float gammaf = __uint_as_float(buf_load4(make_rsrc(p.gamma, 4u), 0u));
    const float gamma2f = PAIR ? __uint_as_float(buf_load4(make_rsrc(p.gamma2, 4u), 0u)) : 0.0f;
    const bool out_lane = lane < 16 && n < p.N;
    const float resid = __uint_as_float(
        buf_load4(make_rsrc(p.R, p.R ? (uint32_t)p.N * 4u : 0u), out_lane ? (uint32_t)n * 4u : kOOB));

    // ---- the activation row straight into LDS, before any weight load: loads return in
    // issue order, and these hit L2 after the first block.  Wave w copies 1 KB chunks w,
    // w + 4, ... (the tail of the last chunk reads as zeros).
    constexpr int esize = BF16 ? 2 : 4;
    const int xbytes = K * esize;
    const v4i xdesc = make_desc(p.X, (uint32_t)xbytes);
    for (int c = wave; c * 1024 < xbytes; c += kGvWaves)
        dma16(xdesc, lds_addr(xraw + 1024 * c), (uint32_t)(1024 * c + 16 * lane));
    // The row in 16-byte chunks (4 fp32 or 8 bf16 values): thread t takes chunks t, t + 256,
    // ...; its norm weights (one 16-byte quad per 4 values) go to registers, also ahead of the
    // weights.
    constexpr int QPC = BF16 ? 2 : 1;                 // quads per chunk
    constexpr int CH = kGvQuads / QPC;                // chunks per thread
    const int nchunk = xbytes / 16;
    v4u rgw[NORM ? kGvQuads : 1];
    if (NORM) {
        const rsrc_t gr = make_rsrc(p.g, (uint32_t)K * 4u);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int i = tid + c * kGvThreads;
#pragma unroll
            for (int h = 0; h < QPC; ++h)
                rgw[QPC * c + h] = buf_load16(gr, i < nchunk ? 16u * (uint32_t)(QPC * i + h) : kOOB);
        }
    }

    // ---- weight loads: rows n0 .. n0+15 (rows past N read as zero), the first round of
    // this wave's super-steps [t_begin, t_end)
    // Decode tiles (TL): the row group's super-step T is one contiguous KB at T * 1024, lane l
    // at byte 16 l: the codes this lane loads from the two-bit rows, arranged plane-major so
    // that each MFMA operand is one mask per word.  Field j of byte b of dword i holds the
    // code of k = 256 T + 64 g + 16 j + 4 i + b: for j = 3 (the byte's top bits) in two's
    // complement, so the masked byte is 64 c; for j < 3 as c + 1, so the masked byte is
    // 4^j (c + 1) and the sum over plane j exceeds 4^j times its share of the dot product by
    // 4^j times the sum of its activation codes, removed once in the epilogue (s_csum).
    const int64_t tile_bytes = (int64_t)supers * 1024;
    const unsigned char *const wrow = reinterpret_cast<const unsigned char *>(p.W) +
                                      (TL ? (int64_t)rg * tile_bytes : (int64_t)n0 * row_bytes);
    // (A wave whose row group lies past N gets an empty resource: every load reads zero.)
    const rsrc_t wres = make_rsrc(wrow, TL ? (n0 < p.N ? (uint32_t)tile_bytes : 0u)
                                           : rows_bytes(n0, 16, p.N, row_bytes));
    const rsrc_t wres2 = PAIR ? make_rsrc(p.W2 + (int64_t)n0 * words, rows_bytes(n0, 16, p.N, row_bytes))
                              : wres;
    const uint32_t wbase = TL ? 16u * (uint32_t)lane : (uint32_t)r * row_bytes;
    v4u w[G][S];
    // Super-steps lo .. hi-1 of the round starting at super-step `base` (non-temporal: the
    // weights are read once).
    auto load_round = [&](int base, int lo, int hi) {
#pragma unroll
        for (int t = 0; t < S; ++t) {
            if (t < lo || t >= hi)
                continue;
            const int T = base + t;
            const bool live = T < t_end;
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                const rsrc_t res = gi ? wres2 : wres;
                if (B3) {
                    const int blk = 4 * T + g;
                    w[gi][t] = buf_load16_nt(res, live && blk < nblk ? wbase + 16u * blk : kOOB);
                } else if (TL) {
                    w[gi][t] = buf_load16_nt(res, live ? (uint32_t)T * 1024u + wbase : kOOB);
                } else {
                    const int wd = 16 * T + 4 * g;
                    w[gi][t] = buf_load16_nt(res, live && wd < words ? wbase + 4u * wd : kOOB);
                }
            }
        }
    };
    // Only the first few super-steps go out before the row is waited for: the row copies get
    // no priority in the memory system, and a full round from every wave ahead of them delays
    // them (and so every block's quantization) by microseconds; the rest follows the
    // quantization.  The copies (and norm weights) were issued before these G * EARLY loads.
    constexpr int EARLY = S < 4 ? S : 4;
    load_round(t_begin, 0, EARLY);
    __builtin_amdgcn_sched_barrier(0);
    wait_stage<G * EARLY>();
    block_sync();

    // The quantization's two barriers hand over LDS data only (the partial maxima, then the
    // codes).  On decode tiles they do not wait for the first super-steps' weight loads, so a
    // block issues the rest of its round as soon as its codes are written; on the two-bit rows
    // the full __syncthreads (which does wait for them) measured faster.
    auto quant_barrier = [] {
        if constexpr (TL)
            lds_barrier();
        else
            __syncthreads();
    };

    // ---- activation quantization, block-wide: absmax of u = x or fl32(x * g) and the sum of
    // x^2 (per thread in chunk order, then across lanes and waves in a fixed order), four
    // chunks' LDS reads in flight at a time
    auto chunk_quads = [&](const v4u &v, float4 *x) {
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
    auto gq = [&](int c, int h) {
        const v4u v = rgw[NORM ? QPC * c + h : 0];
        return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                           __uint_as_float(v.w));
    };
    auto read4 = [&](int c0, v4u *v) {     // chunks c0 .. c0+3 of this thread (zeros past the row)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = tid + (c0 + u) * kGvThreads;
            const v4u t = *reinterpret_cast<const v4u *>(xraw + 16 * (i < nchunk ? i : 0));
            v[u] = i < nchunk ? t : v4u{0, 0, 0, 0};
        }
    };
    float amax = 0.0f;
    double ss = 0.0;
    int csum = 0;
#pragma unroll
    for (int c0 = 0; c0 < CH; c0 += 4) {
        if (c0 * kGvThreads < nchunk) {      // block-uniform
            v4u v[4];
            read4(c0, v);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float4 x[QPC];
                chunk_quads(v[u], x);
#pragma unroll
                for (int h = 0; h < QPC; ++h) {
                    const float4 uu = NORM ? mul4(x[h], gq(c0 + u, h)) : x[h];
                    amax = fmaxf(amax, absmax4(uu));
                    if (NORM)
                        ss = sumsq4(ss, x[h]);
                }
            }
        }
    }
    amax = wave_max(amax);
    if (NORM)
        ss = wave_sum_fixed(ss);
    if (lane == 0) {
        s_amax[wave] = amax;
        s_ss[wave] = ss;
    }
    quant_barrier();
    float a = s_amax[0];
    double sst = s_ss[0];
#pragma unroll
    for (int v = 1; v < kGvWaves; ++v) {
        a = fmaxf(a, s_amax[v]);
        sst += s_ss[v];
    }
    const float inv = a == 0.0f ? 0.0f : 127.0f / a;   // correctly rounded division
    const float sx = act_scale(a, sst, K, p.eps, NORM);
#pragma unroll
    for (int c0 = 0; c0 < CH; c0 += 4) {
        if (c0 * kGvThreads < nchunk) {
            v4u v[4];
            read4(c0, v);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = tid + (c0 + u) * kGvThreads;
                if (i < nchunk) {
                    float4 x[QPC];
                    chunk_quads(v[u], x);
#pragma unroll
                    for (int h = 0; h < QPC; ++h) {
                        const int q = QPC * i + h;
                        const char4 cq = quant4(NORM ? mul4(x[h], gq(c0 + u, h)) : x[h], inv);
                        *reinterpret_cast<char4 *>(codes + 4 * q) = cq;
                        if (TL && ((q >> 2) & 3) != 3) {
                            int cw;
                            __builtin_memcpy(&cw, &cq, 4);
                            csum = __builtin_amdgcn_sdot4(cw, 0x01010101, csum, false);
                        }
                        if (first && p.Xq_out)
                            *reinterpret_cast<char4 *>(p.Xq_out + 4 * q) = cq;
                    }
                }
            }
        }
    }
    if (first && p.sx_out && tid == 0)
        p.sx_out[0] = sx;
    // Codes past the row, up to the end of the last super-step, meet zero weights; clear them
    // so that every value fed to the matrix unit is defined.
    constexpr int EPS = B3 ? 320 : 256;      // weights per super-step
    for (int q = K / 4 + tid; q < EPS / 4 * supers; q += kGvThreads)
        *reinterpret_cast<uint32_t *>(codes + 4 * q) = 0u;
    if (TL) {
        // Integer sums, exact in any order: each row of 16 lanes by shifts (lane 15 of the
        // row ends with the row's sum), then the four rows' last lanes.
        csum += __builtin_amdgcn_update_dpp(0, csum, 0x111, 0xF, 0xF, false);   // row_shr:1
        csum += __builtin_amdgcn_update_dpp(0, csum, 0x112, 0xF, 0xF, false);   // row_shr:2
        csum += __builtin_amdgcn_update_dpp(0, csum, 0x114, 0xF, 0xF, false);   // row_shr:4
        csum += __builtin_amdgcn_update_dpp(0, csum, 0x118, 0xF, 0xF, false);   // row_shr:8
        const int wsum = __builtin_amdgcn_readlane(csum, 15) + __builtin_amdgcn_readlane(csum, 31) +
                         __builtin_amdgcn_readlane(csum, 47) + __builtin_amdgcn_readlane(csum, 63);
        if (lane == 0)
            s_csum[wave] = wsum;
    }
    quant_barrier();
    load_round(t_begin, EARLY, S);
    __builtin_amdgcn_sched_barrier(0);

    // ---- product over this wave's super-steps, S per round
    v4i acc[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
        acc[gi] = v4i{0, 0, 0, 0};
    v4i accp[TL ? 4 : 1];                    // decode tiles: one accumulator per plane
#pragma unroll
    for (int j = 0; j < (TL ? 4 : 1); ++j)
        accp[j] = v4i{0, 0, 0, 0};
    for (int base = t_begin; base < t_end; base += S) {
        if (base != t_begin) {
            load_round(base, 0, S);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int t = 0; t < S; ++t) {
            const int T = base + t;
            if (T < t_end && B3) {
                // Operand i of lane group g's block: 16-weight chunk 20 T + 5 g + i.
                v4i av[5];
#pragma unroll
                for (int i = 0; i < 5; ++i)
                    av[i] = *reinterpret_cast<const v4i *>(codes + 16 * (20 * T + 5 * g + i));
                v4i op[4];
                uint32_t op4[4];
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    unpack_b3_dword(w[0][t][v], b3lut, op[v], op4[v]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[i], op[i], acc[0], 0, 0, 0);
                acc[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                    av[4], v4i{(int)op4[0], (int)op4[1], (int)op4[2], (int)op4[3]}, acc[0], 0, 0, 0);
            } else if (TL && T < t_end) {    // wave-uniform
                // Plane j of the lane's four words holds the codes of k = 256 T + 64 g + 16 j
                // + 0..15 in byte order (see tile_plane): one mask per word, no shift.
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v4i av = *reinterpret_cast<const v4i *>(codes + 256 * T + 64 * g + 16 * j);
                    const v4u ww = w[0][t];
                    const uint32_t m = 0x03030303u << (2 * j);
                    accp[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                        av, v4i{(int)(ww.x & m), (int)(ww.y & m), (int)(ww.z & m), (int)(ww.w & m)}, accp[j],
                        0, 0, 0);
                }
            } else if (T < t_end) {          // wave-uniform
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v4i av = *reinterpret_cast<const v4i *>(codes + 256 * T + 64 * g + 16 * j);
#pragma unroll
                    for (int gi = 0; gi < G; ++gi)
                        acc[gi] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, unpack_word64(w[gi][t][j]),
                                                                       acc[gi], 0, 0, 0);
                }
            }
        }
    }

    // ---- slices of one row group meet in LDS (integer sums: exact, fixed order)
    int s1 = acc[0].x, s2 = acc[G - 1].x;    // lanes 0..15: 64 * D[0][n0 + r]
    if (TL)    // 64x the slice's sum with the offset planes' codes counted once too many
        s1 = accp[3].x + 4 * accp[2].x + 16 * accp[1].x + 64 * accp[0].x;
    if (ksl > 0) {
        if (lane < 16) {
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
                s_red[wave][gi][lane] = gi ? s2 : s1;
        }
        __syncthreads();
        if (slice != 0)
            return;
        if (lane < 16) {
            s1 = 0;
            s2 = 0;
            for (int v = 0; v < (1 << ksl); ++v) {
                s1 += s_red[wave + v][0][lane];
                s2 += s_red[wave + v][G - 1][lane];
            }
        }
    }
    if (!out_lane)
        return;
    if (TL)
        for (int v = 0; v < kGvWaves; ++v)
            s1 -= 64 * s_csum[v];
    // y = fl32(acc * gamma * s_x): gamma * s_x is exact in fp64 (two 24-bit significands),
    // so this is the correctly rounded value of the exact product.
    float y = (float)((double)(s1 >> 6) * ((double)gammaf * (double)sx));
    if (PAIR)
        y = ffn_act(p.act, y, (float)((double)(s2 >> 6) * ((double)gamma2f * (double)sx)));
    else if (p.act != BL_ACT_NONE)
        y = ffn_act(p.act, y, 0.0f);
    if (p.R)
        y = y + resid;
    p.Y[n] = y;
}

template <int S, bool BF16, bool PAIR, bool B3, bool TL>
static void launch_s(const GvBatch &b, int blocks, size_t lds, bool norm, hipStream_t stream)
{
    if (norm)
        hipLaunchKernelGGL((gemv_kernel<S, BF16, PAIR, true, B3, TL>), dim3(blocks), dim3(kGvThreads), lds,
                           stream, b);
    else
        hipLaunchKernelGGL((gemv_kernel<S, BF16, PAIR, false, B3, TL>), dim3(blocks), dim3(kGvThreads), lds,
                           stream, b);
}

// One launch for problems of one kind (pair or single, one activation dtype, all with or all
// without a norm) that gemv_fits; every problem has M == 1.  Slices per row group: the fewest
// (1, 2 or 4) that keep a wave's loads per lane within kGvLoadsPerWave; the round length S is
// the longest slice, rounded up to 4, 8, 12 or 16 (longer slices take several rounds).
// Longest rows first.
template <bool BF16, bool PAIR, bool B3, bool TL>
static hipError_t launch_kind(const bl_linear_ex_problem *const *q, int count, hipStream_t stream)
{
    if (count == 0)
        return hipSuccess;
    constexpr int G = PAIR ? 2 : 1;
    int order[BL_MAX_GROUP];
    for (int i = 0; i < count; ++i)
        order[i] = i;
    std::stable_sort(order, order + count, [&](int a, int c) { return q[a]->K > q[c]->K; });
    GvBatch b{};
    int blocks = 0, longest = 1;
    for (int o = 0; o < count; ++o) {
        const bl_linear_ex_problem &s = *q[order[o]];
        GvDev &d = b.p[o];
        const int K = (int)s.K;
        const int supers = B3 ? ((K + 79) / 80 + 3) / 4 : (K / 16 + 15) / 16;
        int ksl = 0;
        while (ksl < 2 && G * ((supers + (1 << ksl) - 1) >> ksl) > kGvLoadsPerWave)
            ++ksl;
        longest = std::max(longest, (supers + (1 << ksl) - 1) >> ksl);
        d.X = s.X;
        d.g = s.norm_weight;
        d.W = s.W_packed;
        d.W2 = s.W2_packed;
        d.gamma = s.gamma;
        d.gamma2 = s.gamma2;
        d.R = s.residual;
        d.Y = s.Y;
        d.Xq_out = s.X_q;
        d.sx_out = s.x_scale;
        d.eps = s.eps;
        d.N = (int)s.N;
        d.K = K;
        d.ks_log2 = ksl;
        d.act = s.act;
        d.block_begin = blocks;
        const int groups = (d.N + 15) / 16, per_block = 4 >> ksl;
        blocks += (groups + per_block - 1) / per_block;
    }
    b.count = count;
    const bool norm = q[0]->norm_weight != nullptr;
    size_t lds;
    gemv_lds(q, count, BF16, B3, b.c_off, lds);
    // A pair's wave holds two row groups' loads: rounds of at most 8 super-steps (more would
    // not fit the register budget of three waves per SIMD).
    if (longest <= 4)
        launch_s<4, BF16, PAIR, B3, TL>(b, blocks, lds, norm, stream);
    else if (longest <= 8 || PAIR)
        launch_s<8, BF16, PAIR, B3, TL>(b, blocks, lds, norm, stream);
    else if (longest <= 12)
        launch_s<12, BF16, false, B3, TL>(b, blocks, lds, norm, stream);
    else
        launch_s<16, BF16, false, B3, TL>(b, blocks, lds, norm, stream);
    return hipGetLastError();
}

// Problems of one kind, split into those with and without a norm (one launch each).
template <bool BF16, bool PAIR, bool B3, bool TL>
static hipError_t launch_split(const bl_linear_ex_problem *const *q, int count, hipStream_t stream)
{
    const bl_linear_ex_problem *part[2][BL_MAX_GROUP];
    int n[2] = {0, 0};
    for (int i = 0; i < count; ++i) {
        const int k = q[i]->norm_weight ? 1 : 0;
        part[k][n[k]++] = q[i];
    }
    hipError_t e = launch_kind<BF16, PAIR, B3, TL>(part[0], n[0], stream);
    if (e == hipSuccess)
        e = launch_kind<BF16, PAIR, B3, TL>(part[1], n[1], stream);
    return e;
}

hipError_t launch_gemv(const bl_linear_ex_problem *const *q, int count, bool pair, bool bf16,
                       hipStream_t stream)
{
    if (pair)
        return bf16 ? launch_split<true, true, false, false>(q, count, stream)
                    : launch_split<false, true, false, false>(q, count, stream);
    return bf16 ? launch_split<true, false, false, false>(q, count, stream)
                : launch_split<false, false, false, false>(q, count, stream);
}

hipError_t launch_gemv_b3(const bl_linear_ex_problem *const *q, int count, bool bf16,
                          hipStream_t stream)
{
    return bf16 ? launch_split<true, false, true, false>(q, count, stream)
                : launch_split<false, false, true, false>(q, count, stream);
}

hipError_t launch_gemv_tiles(const bl_linear_ex_problem *const *q, int count, bool bf16,
                             hipStream_t stream)
{
    return bf16 ? launch_split<true, false, false, true>(q, count, stream)
                : launch_split<false, false, false, true>(q, count, stream);
}

// Decode tiles from two-bit rows: output chunk c (16 bytes) of tile (row group rg, super-step
// T) holds, for lane l = c % 64 (r = l % 16, g = l / 16), words 16 T + 4 g .. + 3 of row
// 16 rg + r; words past the row and rows past N are zero.
__global__ __launch_bounds__(256) void pack_tiles_kernel(const uint32_t *__restrict__ P, int N,
                                                         int words, int supers, int64_t chunks,
                                                         uint4 *__restrict__ out)
{
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= chunks)
        return;
    const int l = (int)(c & 63);
    const int64_t tile = c >> 6;
    const int T = (int)(tile % supers);
    const int64_t rg = tile / supers;
    const int64_t row = rg * 16 + (l & 15);
    const int w0 = 16 * T + 4 * (l >> 4);
    // Row words w0 + j hold k = 256 T + 64 g + 16 j + 4 i + b at bits 8 b + 2 i (two-bit rows);
    // the chunk's dword i holds the same code at bits 8 b + 2 j, offset by one for j < 3.
    uint32_t v[4] = {0u, 0u, 0u, 0u};
    if (row < N) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (w0 + j < words)
                v[j] = P[row * words + w0 + j];
    }
    uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t f = (v[j] >> (8 * b + 2 * i)) & 3u;
                o[i] |= (j < 3 ? (f + 1u) & 3u : f) << (8 * b + 2 * j);
            }
    out[c] = make_uint4(o[0], o[1], o[2], o[3]);
}

int64_t tiles_bytes(int64_t N, int64_t K)
{
    return ((N + 15) / 16) * ((K / 16 + 15) / 16) * 1024;
}

hipError_t launch_pack_tiles(const uint32_t *P, int64_t N, int64_t K, uint32_t *out,
                             hipStream_t stream)
{
    const int words = (int)(K / 16), supers = (words + 15) / 16;
    const int64_t chunks = tiles_bytes(N, K) / 16;
    if (chunks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(pack_tiles_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream,
                       P, (int)N, words, supers, chunks, reinterpret_cast<uint4 *>(out));
    return hipGetLastError();
}

}  // namespace bl
