// prefill_core.hpp — the prefill product's block body (one 2-D tile of one problem of a
// grouped launch), its tile configurations and its host-side batch builder.  Included by
// prefill.hip (the prefill launches) and mixed.hip (prefill tiles and decode blocks in one
// grid).  The design of the pipeline is described at the top of prefill.hip.
#pragma once

#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "common.hpp"

namespace bl {

struct PreDev {
    const int8_t *Xq;
    const float *sx;
    const uint32_t *W;
    const float *gamma;
    float *Y;
    int32_t *acc;
    const float *R;     // residual added to the output, or NULL
    int M, N, K;
    int tiles_n;
    int block_begin;
};

struct PreBatch {
    PreDev p[BL_MAX_GROUP];
    int count;
    int blocks;
};

// Tile configuration: BM x BN block tile split over WM x WN waves (wave tile BM/WM x BN/WN,
// MFMA tiles 16 x 16), KS weights of K per pipeline stage, NST stages in LDS, EA bytes per
// activation (1: int8 codes on the int8 matrix unit; 2: bf16 activations on the bf16 one).
template <int BM_, int BN_, int WM_, int WN_, int KS_, int NST_, int EA_ = 1, int WPE_ = 1>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, KS = KS_, NST = NST_, EA = EA_;
    static constexpr int WPE = WPE_;                     // waves per SIMD the registers must allow
    static constexpr int WAVES = WM * WN;
    static constexpr int THREADS = WAVES * 64;
    static constexpr int TM = BM / WM, TN = BN / WN;     // wave tile
    static constexpr int MI = TM / 16, NI = TN / 16;     // MFMA tiles per wave, each direction
    static constexpr int XROW = KS * EA;                 // activation bytes per row per stage
    static constexpr int CPR = XROW / 16;                // 16-byte activation chunks per row
    static constexpr int WPS = KS / 16;                  // packed words per weight row
    static constexpr int LPW = WPS / 4;                  // words per lane (one MFMA k-step each)
    static constexpr int WROW = KS / 4;                  // bytes per weight row per stage
    static constexpr int XBYTES = BM * XROW;
    static constexpr int WBYTES = BN * WROW;
    static constexpr int STAGE = XBYTES + WBYTES;
    static constexpr int XINST = XBYTES / 1024 / WAVES;  // 1 KB direct loads per wave per stage
    static constexpr int WINST = WBYTES / 1024 / WAVES;
    static constexpr int LOADS = XINST + WINST;          // vector-memory ops per wave per stage
    static_assert(LPW >= 1 && LPW <= 4, "1..4 words per lane");
    static_assert(XINST >= 1 && WINST >= 1, "every wave loads part of each operand");
    static_assert(XINST * WAVES * 1024 == XBYTES && WINST * WAVES * 1024 == WBYTES, "even split");
    static_assert(NST * STAGE <= 160 * 1024, "LDS budget");
    static_assert((NST - 2) * LOADS < 64, "vmcnt range");
};

// Activation chunk swizzle: chunk c of tile row m sits at position c ^ f(m).  For 128-byte
// rows (CPR = 8, int8 stages) f(m) = (m & 7) ^ ((m >> 3) & 1): an LDS probe of the fragment
// read (lane (r, g) reads chunk (2g + j) ^ f(r) of row r) measured 186 bytes per clock per CU
// with it, the rate of a linear read, against 128 with f(m) = (m / 2) & 7, which puts the 16
// rows in 16 different 16-byte slots of 256 bytes but still conflicts in the hardware's lane
// grouping.  Other row lengths: f(m) = (m / (16 / CPR)) % CPR.
template <int CPR>
__device__ __forceinline__ int xswz(int row)
{
    if constexpr (CPR == 8)
        return (row & 7) ^ ((row >> 3) & 1);
    else
        return (row / (16 / CPR)) & (CPR - 1);
}

// Weight chunk swizzle (16-byte chunks, WCH per row): rows m and m + 8 of a 16-row B-operand
// read would share banks at a 32-byte row pitch; flipping the chunk order on every other
// group of 8 rows separates them.
template <int WCH>
__device__ __forceinline__ int wswz(int row)
{
    return WCH > 1 ? ((row >> 3) & 1) : 0;
}

// One LDS buffer per pipeline stage, as distinct variables: the compiler can then tell that
// a direct-to-LDS load into one stage does not alias reads from another, and does not force
// a wait for every outstanding load before each LDS read.
template <int S, int BYTES>
__device__ __forceinline__ unsigned char *stage_buf()
{
    __shared__ __align__(1024) unsigned char buf[BYTES];
    return buf;
}

template <int N>
struct IC {
    static constexpr int value = N;
};

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(IC<B>{});
        static_for<B + 1, E>(f);
    }
}

// The prefill kernel.  Per stage, activations (BM rows x KS bytes, swizzled) and packed
// weights (BN rows x KS/4 bytes) travel global -> LDS by direct buffer loads; NST - 1 stages
// are in flight while one is computed, and one barrier per stage orders reuse of the buffers.
// FULL_K: every problem has K % KS == 0 (no stage runs past a row).  QR: the packed weights
// are in the quad-row layout (quad_row_word), so each 1 KB weight load reads eight whole
// 128-byte lines (four rows' 32-byte stage pieces each) instead of 32 rows x 32 bytes.
template <class T, bool FULL_K, bool QR = false>
__device__ __forceinline__ void prefill_block(const PreBatch &b, int bid)
{
    constexpr int BM = T::BM, BN = T::BN, KS = T::KS, NST = T::NST, WAVES = T::WAVES;
    constexpr int MI = T::MI, NI = T::NI, CPR = T::CPR, LPW = T::LPW, WROW = T::WROW;
    constexpr int EA = T::EA, XROW = T::XROW;
    constexpr bool BF = EA == 2;      // bf16 activations: the weight-only product
    constexpr int AH = EA;            // activation fragments per packed word (16 / 8 weights)
    using AccT = typename std::conditional<BF, f32x4, v4i>::type;

    int prob = 0;
#pragma unroll 1
    while (prob + 1 < b.count && bid >= b.p[prob + 1].block_begin)
        ++prob;
    const PreDev &p = b.p[prob];
    // XCD-aware order inside each problem, so every XCD gets its share of every problem.
    const int ntiles = (prob + 1 < b.count ? b.p[prob + 1].block_begin : b.blocks) - p.block_begin;
    const int tile = xcd_order(bid - p.block_begin, ntiles);
    // On large grids, consecutive tiles of one XCD walk two activation panels side by side,
    // so each weight panel fetched into that XCD's L2 serves two tiles; small grids keep
    // the plain row-major order (one panel of each is all an XCD holds anyway).
    const int gm_max = ntiles >= 1024 ? 2 : 1;
    const int tiles_m = ntiles / p.tiles_n;
    const int grp = tile / (gm_max * p.tiles_n), within = tile % (gm_max * p.tiles_n);
    const int gm = min(gm_max, tiles_m - grp * gm_max);
    const int m0 = (grp * gm_max + within % gm) * BM;
    const int n0 = (within / gm) * BN;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
    const int wm = wave / T::WN, wn = wave % T::WN;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int K = p.K;
    const int row_bytes = K / 4;
    const int stages = (K + KS - 1) / KS;

    // Activation rows m0 .. m0+BM-1 and weight rows n0 .. n0+BN-1; rows past M / N read zero.
    const v4i xres = make_desc(reinterpret_cast<const unsigned char *>(p.Xq) + (int64_t)m0 * K * EA,
                               rows_bytes(m0, BM, p.M, K * EA));
    const v4i wres = make_desc(p.W + (int64_t)n0 * (K / 16), rows_bytes(n0, BN, p.N, row_bytes));

    // Load plan.  Activations: wave w fills rows w*BM/WAVES .. +BM/WAVES, 64/CPR rows per 1 KB
    // load; lane l -> row (l / CPR), position l % CPR, global chunk position ^ swizzle.
    // Weights: wave w fills rows w*BN/WAVES .. +BN/WAVES, 1024/WROW rows per load; lane l ->
    // row l / (WROW/16), position l % (WROW/16), global chunk position ^ swizzle.
    // Past-the-row chunks (only when !FULL_K) read as zero for activations; weight words past
    // K meet those zero activations.
    constexpr int XR = 64 / CPR;            // activation rows per load
    constexpr int WCH = WROW / 16;          // 16-byte weight chunks per row
    constexpr int WR = 64 / WCH;            // weight rows per load
    const int xrow_l = lane / CPR, xpos = lane % CPR;
    const int wrow_l = lane / WCH, wcol = lane % WCH;
    // A stage at or past `stages` is still issued, from out-of-range offsets: it writes zeros
    // into a buffer nobody reads again, and keeps the number of loads in flight per stage
    // constant, so a single compile-time vmcnt wait fits every iteration.
    // (The dead-stage flag is folded into bit 31 of the offset arithmetically: a select on a
    // uniform flag would be turned into branches around the loads, and the compiler then
    // waits conservatively for all of them before reading LDS.)
    auto issue = [&](auto S, int t) {
        unsigned char *st = stage_buf<decltype(S)::value, T::STAGE>();
        const uint32_t dead = (uint32_t)(t >= stages) << 31;   // == kOOB for a dead stage
#pragma unroll
        for (int i = 0; i < T::XINST; ++i) {
            const int row0 = wave * (BM / WAVES) + i * XR;
            const int row = row0 + xrow_l;
            const int c = xpos ^ xswz<CPR>(row);
            const int k = t * KS + c * (16 / EA);                     // first element of the chunk
            uint32_t off = ((uint32_t)row * K + (uint32_t)k) * EA | dead;
            if (!FULL_K)
                off = k < K ? off : kOOB;
            dma16(xres, lds_addr(st + row0 * XROW), off);
        }
#pragma unroll
        for (int i = 0; i < T::WINST; ++i) {
            const int row0 = wave * (BN / WAVES) + i * WR;
            const int row = row0 + wrow_l;
            uint32_t off;
            if constexpr (QR) {
                // Row `row`'s piece of stage t in the line of rows 4 (row / 4) .. + 3 (K % 128
                // == 0 on this path: no stage runs past a row).
                static_assert(WROW == 32, "quad-row lines hold four 32-byte stage pieces");
                off = ((uint32_t)((row >> 2) * stages + t) * 128u +
                       (uint32_t)(32 * (row & 3) + 16 * (wcol ^ wswz<WCH>(row)))) | dead;
            } else {
                const int kb = t * WROW + 16 * (wcol ^ wswz<WCH>(row));   // byte offset in the row
                off = ((uint32_t)row * row_bytes + (uint32_t)kb) | dead;
                if (!FULL_K)
                    off = kb < row_bytes ? off : kOOB;
            }
            dma16(wres, lds_addr(st + T::XBYTES + row0 * WROW), off);
        }
    };

    AccT acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = AccT{0, 0, 0, 0};

    // Per-lane LDS offsets inside a stage.  Lane (r, g) reads words g*LPW .. +LPW-1 of its
    // weight row: 16-byte chunk (g*LPW*4) / 16 (swizzled) at byte (g*LPW*4) % 16.
    const int arow = (wm * T::TM + r) * XROW;                // + mi * 16 * XROW
    const int aswz = xswz<CPR>(wm * T::TM + r);              // same for every mi (16 | mi*16)
    const int bch = (g * LPW * 4) / 16, bin = (g * LPW * 4) % 16;
    const int brow = T::XBYTES + (wn * T::TN + r) * WROW +
                     16 * (bch ^ wswz<WCH>(wn * T::TN + r)) + bin;           // + ni * 16 * WROW

    // The last k-step of each stage is deferred to the next stage: its operands (activation
    // fragments and raw packed words) stay in registers, and its MFMAs are issued right after
    // the next stage's barrier and LDS reads, so the matrix pipe has work while those reads
    // are in flight instead of idling after every barrier.  (Zero operands before the first
    // stage add nothing.)
    v4i da[AH][MI];
    uint32_t dw[NI];
#pragma unroll
    for (int h = 0; h < AH; ++h)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
            da[h][mi] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
        dw[ni] = 0;
    // One packed word per lane and weight row: int8, its four planes as one 16 x 16 x 64
    // operand; bf16, its two halves of eight codes as two 16 x 16 x 32 operands.
    auto mfma_step = [&](const uint32_t (&w)[NI], const v4i (&a)[AH][MI]) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            if constexpr (BF) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const v4u b = ternary_bf16(w[ni], h);
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
                        acc[mi][ni] = mfma_bf16(b, __builtin_bit_cast(v4u, a[h][mi]), acc[mi][ni]);
                }
            } else {
                const v4i b = unpack_word64(w[ni]);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    acc[mi][ni] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, a[0][mi], acc[mi][ni], 0, 0, 0);
            }
        }
    };
    // Activations of word j of the lane's share: 16 int8 (one chunk), or 16 bf16 (two
    // chunks, one per half).
    auto read_a = [&](const unsigned char *st, int j, v4i (&a)[AH][MI]) {
#pragma unroll
        for (int h = 0; h < AH; ++h) {
            const int pos = 16 * ((AH * (g * LPW + j) + h) ^ aswz);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
                a[h][mi] = *reinterpret_cast<const v4i *>(st + arow + mi * 16 * XROW + pos);
        }
    };

    auto compute = [&](auto S) {
        const unsigned char *st = stage_buf<decltype(S)::value, T::STAGE>();
        uint32_t wq[NI][LPW];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            const unsigned char *src = st + brow + ni * 16 * WROW;
            if constexpr (LPW == 4) {
                const v4u v = *reinterpret_cast<const v4u *>(src);
                wq[ni][0] = v.x; wq[ni][1] = v.y; wq[ni][2] = v.z; wq[ni][3] = v.w;
            } else if constexpr (LPW == 2) {
                const uint2 v = *reinterpret_cast<const uint2 *>(src);
                wq[ni][0] = v.x; wq[ni][1] = v.y;
            } else {
                wq[ni][0] = *reinterpret_cast<const uint32_t *>(src);
            }
        }
        v4i a0[AH][MI];
        read_a(st, 0, a0);
        mfma_step(dw, da);          // previous stage's last k-step
        static_assert(LPW >= 2, "one k-step per stage is deferred");
#pragma unroll
        for (int j = 0; j < LPW - 1; ++j) {
            uint32_t w[NI];
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                w[ni] = wq[ni][j];
            if (j == 0) {
                mfma_step(w, a0);
            } else {
                v4i a[AH][MI];
                read_a(st, j, a);
                mfma_step(w, a);
            }
        }
        read_a(st, LPW - 1, da);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
            dw[ni] = wq[ni][LPW - 1];
    };

    // The int8 product as a rolling pipeline of units.  A unit (stage t, k-step j, row block
    // mi) is the NI MFMAs of one activation fragment with the NI expanded weight words of step
    // j; right after them the fragment's registers are refilled with the fragment the next
    // unit of that row block needs (step j + 1, or step 0 of stage t + 1), so every LDS read
    // is issued MI units (MI * NI MFMAs) before its use, with no registers beyond one fragment
    // per row block.  Stage t + 1 is entered in the middle of stage t's last step, after unit
    // X: by then every read of stage t has been issued for X units (and has returned at the
    // lgkmcnt(0) wait), the wait for stage t + 1's loads and the barrier follow, then the
    // refill of stage t's buffer and the first reads of stage t + 1, which the remaining
    // MI - X units of stage t (operands already in registers) cover.  (The compiler, left to
    // schedule the deferred-step form below, sank the reads behind the MFMAs and waited for
    // each read right after issuing it.)  Used for the 128 x 256 tile (MI = 8: four units of
    // cover on each side of the barrier; the Qwen3-1.7B set at 4096 tokens: 176-184 -> 171 us,
    // the Qwen3-4B set at 8192 tokens unchanged); the 128 x 128 tile (MI = 4, two units)
    // measured about 1 us slower with it on the Distillix-125M set at 2048 tokens and keeps
    // the deferred-step form.
    auto rolling_pipeline = [&](auto &acc_) {
        constexpr int X = MI / 2;
        v4i a[MI];
        v4i bw[NI];
        uint32_t wq[NI][LPW];
        auto read_w = [&](const unsigned char *st) {
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const unsigned char *src = st + brow + ni * 16 * WROW;
                if constexpr (LPW == 4) {
                    const v4u v = *reinterpret_cast<const v4u *>(src);
                    wq[ni][0] = v.x; wq[ni][1] = v.y; wq[ni][2] = v.z; wq[ni][3] = v.w;
                } else if constexpr (LPW == 2) {
                    const uint2 v = *reinterpret_cast<const uint2 *>(src);
                    wq[ni][0] = v.x; wq[ni][1] = v.y;
                } else {
                    wq[ni][0] = *reinterpret_cast<const uint32_t *>(src);
                }
            }
        };
        auto read_a1 = [&](const unsigned char *st, int j, int mi) {
            const int pos = 16 * ((g * LPW + j) ^ aswz);
            a[mi] = *reinterpret_cast<const v4i *>(st + arow + mi * 16 * XROW + pos);
        };
        auto unpack_b = [&](int j) {
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
                bw[ni] = unpack_word64(wq[ni][j]);
        };
        // Enter stage tn (buffer S): its loads have landed in every wave, every LDS read of
        // the buffer refilled next has returned; refill it, read the stage's weight words and
        // the fragments of row blocks 0 .. X-1 (whose registers are free by now).
        auto enter = [&](auto S, int tn) {
            wait_stage<(NST - 2) * T::LOADS>();
            block_sync();
            issue(IC<(decltype(S)::value + NST - 1) % NST>{}, tn + NST - 1);
            const unsigned char *st = stage_buf<decltype(S)::value, T::STAGE>();
            read_w(st);
#pragma unroll
            for (int mi = 0; mi < X; ++mi)
                read_a1(st, 0, mi);
        };

        static_for<0, NST - 1>([&](auto S) { issue(S, S.value); });
        enter(IC<0>{}, 0);
        {
            const unsigned char *st0 = stage_buf<0, T::STAGE>();
#pragma unroll
            for (int mi = X; mi < MI; ++mi)
                read_a1(st0, 0, mi);
        }
        unpack_b(0);
        // Unrolled by NST so that every buffer is a compile-time choice.  Past the last stage
        // the same steps run on a dead stage (zeros loaded, reads unused), without branches.
        for (int t0 = 0; t0 < stages; t0 += NST) {
            static_for<0, NST>([&](auto S) {
                constexpr int SN = (decltype(S)::value + 1) % NST;
                const int t = t0 + S.value;
                if (t < stages) {
                    const unsigned char *st = stage_buf<decltype(S)::value, T::STAGE>();
                    const unsigned char *sn = stage_buf<SN, T::STAGE>();
#pragma unroll
                    for (int j = 0; j < LPW; ++j) {
#pragma unroll
                        for (int mi = 0; mi < MI; ++mi) {
                            if (j == LPW - 1 && mi == X)
                                enter(IC<SN>{}, t + 1);
                            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                            for (int ni = 0; ni < NI; ++ni)
                                acc_[mi][ni] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bw[ni], a[mi], acc_[mi][ni],
                                                                                    0, 0, 0);
                            if (j < LPW - 1)
                                read_a1(st, j + 1, mi);
                            else if (mi >= X)
                                read_a1(sn, 0, mi);
                            if (mi == MI - 1)
                                unpack_b(j < LPW - 1 ? j + 1 : 0);
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                }
            });
        }
        // Dead stages issued past the end land before the block ends.
        __builtin_amdgcn_s_waitcnt((0 & 15) | (0 << 14) | (7 << 4) | (15 << 8));
    };

    // Row scales and gamma, loaded before the pipeline starts: older than every stage load,
    // they have landed by the first stage wait, and the epilogue does not wait on memory.
    float sxv[MI];
    {
        const rsrc_t sres = make_rsrc(p.sx, BF ? 0u : (uint32_t)p.M * 4u);   // bf16: unused
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int m = m0 + wm * T::TM + mi * 16 + r;   // rows past M read 0
            sxv[mi] = __uint_as_float(buf_load4(sres, (uint32_t)m * 4u));
        }
    }
    const float gammaf = __uint_as_float(buf_load4(make_rsrc(p.gamma, 4u), 0u));

    if constexpr (!BF && MI >= 8) {
        rolling_pipeline(acc);
    } else {
    // Prologue: stages 0 .. NST-2 in flight.
    static_for<0, NST - 1>([&](auto S) { issue(S, S.value); });
    // Main loop, unrolled by NST so every stage buffer is a compile-time choice.  Stage t has
    // landed once only the NST - 2 stages issued after it are still in flight; the buffer
    // refilled after the barrier (stage t - 1's) is free once every wave's reads of it have
    // returned.
    for (int t0 = 0; t0 < stages; t0 += NST) {
        static_for<0, NST>([&](auto S) {
            const int t = t0 + S.value;
            if (t < stages) {
                wait_stage<(NST - 2) * T::LOADS>();
                block_sync();
                issue(IC<(decltype(S)::value + NST - 1) % NST>{}, t + NST - 1);
                compute(S);
            }
        });
    }
    mfma_step(dw, da);              // the last stage's deferred k-step
    }

    // Epilogue.  The MFMA takes the weights as its row operand, so acc[mi][ni] register v
    // holds 64 * D[m][n] for m = m0 + wm * TM + mi * 16 + r and n = n0 + wn * TN + ni * 16 +
    // 4 * g + v: each lane owns four consecutive outputs of one row and writes them with one
    // 16-byte store (scalar stores when the row pitch or the base is not 16-byte aligned, and
    // in a ragged last column group).
    if constexpr (BF) {
        // Weight-only product: y = fl32(gamma * acc), acc the fp32 matrix-unit sum.
        const bool vecb = (p.N & 3) == 0 && ((uintptr_t)p.Y & 15) == 0;
        // A full tile: whole-line non-temporal stores (store_pair_lines_nt), as below.
        if (vecb && m0 + BM <= p.M && n0 + BN <= p.N && (int64_t)BM * p.N * 4 <= (int64_t)0xFFFFFFFFu) {
            static_assert(NI % 2 == 0, "column groups in pairs");
            const rsrc_t yres = make_rsrc(p.Y + (int64_t)m0 * p.N, (uint32_t)BM * (uint32_t)p.N * 4u);
            const bool lo = r < 8;
            const uint32_t pitch8 = 8u * (uint32_t)p.N * 4u;
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const uint32_t base = (uint32_t)(wm * T::TM + mi * 16 + (r & 7)) * (uint32_t)p.N * 4u +
                                      (uint32_t)(n0 + wn * T::TN + 4 * g + (lo ? 0 : 16)) * 4u;
#pragma unroll
                for (int pp = 0; pp < NI / 2; ++pp) {
                    const f32x4 ye = acc[mi][2 * pp] * gammaf;
                    const f32x4 yo = acc[mi][2 * pp + 1] * gammaf;
                    store_pair_lines_nt(yres, base + (uint32_t)(pp * 32 * 4), pitch8, lo,
                                        __builtin_bit_cast(v4u, ye), __builtin_bit_cast(v4u, yo));
                }
            }
            return;
        }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int m = m0 + wm * T::TM + mi * 16 + r;
            if (m >= p.M)
                continue;
            float *yrow = p.Y + (int64_t)m * p.N;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const int n = n0 + wn * T::TN + ni * 16 + 4 * g;
                const f32x4 y = acc[mi][ni] * gammaf;
                if (vecb && n + 3 < p.N) {
                    *reinterpret_cast<float4 *>(yrow + n) = make_float4(y[0], y[1], y[2], y[3]);
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (n + v < p.N)
                            yrow[n + v] = y[v];
                }
            }
        }
        return;
    } else {
    const double gamma = (double)gammaf;
    // A full tile with neither residual nor int32 copy (every tile of a product whose M and
    // N are multiples of the tile): straight-line code with whole-line,
    // non-temporal stores (store_pair_lines_nt: column groups 2p and 2p + 1 exchanged
    // between lanes r and r ^ 8, each store a whole 128-byte row segment).  The stores bypass
    // the caches, which then keep the operand panels the other tiles read.
    // Measured on the Qwen3-4B set at 8192 tokens: product 707-718 -> 672-677 us, step
    // 1.132-1.139 -> 1.099-1.105 ms (non-temporal 64-byte pieces were slower than plain
    // stores in the step, whole lines without the hint no faster); Distillix-125M set at
    // 2048 tokens (128 x 128 tiles): product 25.9-26.7 -> 23.3-24.8 us.  The general form
    // below, with its per-group branches and 64-bit addresses, measured 6-7 us per 128 x 256
    // tile whether or not it stored anything (the unrolled code is large and runs once per
    // tile); this one 2.3 us plus the stores' drain.
    if (!p.R && !p.acc && m0 + BM <= p.M && n0 + BN <= p.N && (p.N & 3) == 0 &&
        ((uintptr_t)p.Y & 15) == 0 && (int64_t)BM * p.N * 4 <= (int64_t)0xFFFFFFFFu) {
        static_assert(NI % 2 == 0, "column groups in pairs");
        const rsrc_t yres = make_rsrc(p.Y + (int64_t)m0 * p.N, (uint32_t)BM * (uint32_t)p.N * 4u);
        const bool lo = r < 8;
        const uint32_t pitch8 = 8u * (uint32_t)p.N * 4u;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const double scale = gamma * (double)sxv[mi];
            // Lanes r < 8 store the pair's first 16 columns, lanes r >= 8 its last 16, of row
            // (r & 7), then of row (r & 7) + 8.
            const uint32_t base = (uint32_t)(wm * T::TM + mi * 16 + (r & 7)) * (uint32_t)p.N * 4u +
                                  (uint32_t)(n0 + wn * T::TN + 4 * g + (lo ? 0 : 16)) * 4u;
#pragma unroll
            for (int pp = 0; pp < NI / 2; ++pp) {
                v4u ye, yo;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    ye[v] = __float_as_uint((float)((double)(acc[mi][2 * pp][v] >> 6) * scale));
                    yo[v] = __float_as_uint((float)((double)(acc[mi][2 * pp + 1][v] >> 6) * scale));
                }
                store_pair_lines_nt(yres, base + (uint32_t)(pp * 32 * 4), pitch8, lo, ye, yo);
            }
        }
    } else {
    const bool vec = (p.N & 3) == 0 && ((uintptr_t)p.Y & 15) == 0 &&
                     (!p.acc || ((uintptr_t)p.acc & 15) == 0) &&
                     (!p.R || ((uintptr_t)p.R & 15) == 0);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        const int m = m0 + wm * T::TM + mi * 16 + r;
        if (m >= p.M)
            continue;
        const double scale = gamma * (double)sxv[mi];
        float *yrow = p.Y + (int64_t)m * p.N;
        const float *rrow = p.R ? p.R + (int64_t)m * p.N : nullptr;
        int32_t *arow_out = p.acc ? p.acc + (int64_t)m * p.N : nullptr;
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
            const int n = n0 + wn * T::TN + ni * 16 + 4 * g;
            int a[4];
            float y[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                a[v] = acc[mi][ni][v] >> 6;
                y[v] = (float)((double)a[v] * scale);
            }
            if (vec && n + 3 < p.N) {
                if (rrow) {
                    const float4 rv = *reinterpret_cast<const float4 *>(rrow + n);
                    y[0] = y[0] + rv.x;
                    y[1] = y[1] + rv.y;
                    y[2] = y[2] + rv.z;
                    y[3] = y[3] + rv.w;
                }
                *reinterpret_cast<float4 *>(yrow + n) = make_float4(y[0], y[1], y[2], y[3]);
                if (arow_out)
                    *reinterpret_cast<int4 *>(arow_out + n) = make_int4(a[0], a[1], a[2], a[3]);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    if (n + v < p.N) {
                        yrow[n + v] = rrow ? y[v] + rrow[n + v] : y[v];
                        if (arow_out)
                            arow_out[n + v] = a[v];
                    }
                }
            }
        }
    }
    }
    }
}

template <class T>
static int build_batch(const bl_forward_ex_problem *q, int count, PreBatch &b, bool &full_k)
{
    // Longest-K problems first: their tiles take longest, so they should not start last.
    int order[BL_MAX_GROUP];
    int n = 0;
    for (int i = 0; i < count; ++i)
        if (q[i].M > 0 && q[i].N > 0)
            order[n++] = i;
    for (int i = 1; i < n; ++i)
        for (int j = i; j > 0 && q[order[j]].K > q[order[j - 1]].K; --j) {
            const int t = order[j];
            order[j] = order[j - 1];
            order[j - 1] = t;
        }
    int blocks = 0;
    full_k = true;
    for (int i = 0; i < n; ++i) {
        const bl_forward_ex_problem &s = q[order[i]];
        PreDev &d = b.p[i];
        d.Xq = s.X_q;
        d.sx = s.x_scale;
        d.W = s.W_packed;
        d.gamma = s.gamma;
        d.Y = s.Y;
        d.acc = s.acc;
        d.R = s.residual;
        d.M = (int)s.M;
        d.N = (int)s.N;
        d.K = (int)s.K;
        d.tiles_n = (d.N + T::BN - 1) / T::BN;
        d.block_begin = blocks;
        blocks += ((d.M + T::BM - 1) / T::BM) * d.tiles_n;
        full_k = full_k && (d.K % T::KS == 0);
    }
    b.count = n;
    b.blocks = blocks;
    return blocks;
}

// Large grids: 128 tokens x 256 weight rows, four waves side by side in N (each wave 128
// tokens x 64 rows: 8 x 4 MFMA tiles, so each expanded weight word feeds eight MFMAs), a 3-stage
// 72 KB ring and registers for two waves per SIMD: two blocks per CU, so one block's epilogue
// (fp32 stores) and pipeline fill overlap the other's products.  Measured on the Qwen3-4B set
// against 256 x 256 tiles with one 160 KB block per CU (4 x 2 waves: 770 us; 2 x 4 waves:
// 735 us) and 128 x 256 with 2 x 2 waves (746 us): 710-723 us.
using TileBig = Tile<128, 256, 1, 4, 128, 3, 1, 2>;
// Small tiles: a 3-stage ring (60 KB LDS, two blocks per CU) measured faster than 4 stages
// (80 KB, Distillix-125M set at 2048 tokens: 27.3 -> 25.9 us) and than 2 stages (40 KB, four blocks per CU).
using TileSmall = Tile<128, 128, 2, 2, 128, 3>;

// The weight-only product with bf16 activations (the W1.58.A16 forward and the input gradient
// with bf16 dY): the same pipeline with 2-byte activations and the bf16 matrix unit.
using TileWBig = Tile<256, 256, 4, 2, 128, 2, 2>;     // 144 KB LDS, one block per CU
using TileWSmall = Tile<128, 128, 2, 2, 128, 2, 2>;   // 72 KB, two blocks per CU

// Measurement-only knob to A/B the two tile layouts (BITLINEAR_PREFILL_TILE=big|small):
// 0 = automatic, 1 = large, 2 = small.
inline int tile_override()
{
    static int v = [] {
        const char *e = getenv("BITLINEAR_PREFILL_TILE");
        if (!e)
            return 0;
        if (!strcmp(e, "big")) return 1;
        if (!strcmp(e, "small")) return 2;
        return 0;
    }();
    return v;
}

// Large (128 x 256) tiles when the set is big: at least 256 units of 256 x 256 outputs (512
// such tiles, one per slot of two blocks per CU); otherwise 128 x 128.  (At 512 units the
// Qwen3-4B layer chain ran its o and down projections, 320 units each, on 128 x 128 tiles:
// 1018-1023 us per layer at 8192 tokens, against 1008-1009 us on 128 x 256.)
inline bool prefill_big_tiles(const bl_forward_ex_problem *q, int count)
{
    switch (tile_override()) {
    case 1: return true;
    case 2: return false;
    default: break;
    }
    int64_t big = 0;
    for (int i = 0; i < count; ++i)
        big += ((q[i].M + 255) / 256) * ((q[i].N + 255) / 256);
    return big >= 256;
}

}  // namespace bl
