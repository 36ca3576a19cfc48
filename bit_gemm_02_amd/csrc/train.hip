// train.hip — the training-side products on the bf16 matrix cores.
//
// (1) The weight-only ternary forward (bitone README, "Features": the QAT forward computes
//     Y = X @ W_q^T x gamma with full-precision activations): Y = gamma * X C^T.
// (2) The input gradient through the straight-through estimator (Distillix README, "Key
//     Innovations 1": gradients pass through quantization unchanged): dX = gamma * dY C.
//     It is (1) with the transposed code matrix, so (3) re-packs C^T once per weight update
//     and the same kernel runs it.
// (4) The weight gradient: dW = grad_scale(W / gamma) . (dY^T X_hat), X_hat = q * s_x the
//     dequantized activations the forward multiplied; grad_scale is 1 (pass-through), the
//     hard mask |W / gamma| <= 1, or sech^2(beta W / gamma) (bitone README, "Soft-STE").
//
// The codes are exact in bf16 (0, +-1.0) and so are int8 activation codes, so products on
// the bf16 matrix unit (v_mfma_f32_16x16x32_bf16, fp32 accumulation) lose nothing on that
// side.  fp32 operands are split x = hi + lo with hi = bf16(x) and lo = bf16(x - hi)
// (x - hi is exact in fp32): two MFMAs per fragment carry 16 significant bits of x, a
// relative representation error of at most 2^-16 (2^-8 of 2^-8), below the fp32 accumulation error of any
// contraction longer than a few hundred terms.  bf16 operands take one MFMA.
//
// Both GEMMs stage operands through LDS in bf16 with the contraction index contiguous (the
// MFMA operand layout): (1)/(2) read activation rows and packed code rows that are already
// contraction-major and expand the 2-bit codes to bf16 in registers; (4) contracts over
// tokens, which are the slow index of both dY and q, so its staging loads four token rows
// at once and writes them transposed (four tokens per 8-byte LDS store).  (1)/(2) with bf16
// activations need no conversion while staging and run on the prefill product's pipeline
// instead (prefill.hip: direct-to-LDS loads, the bf16 form of its kernel).
#include <algorithm>

#include "common.hpp"

namespace bl {


typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 values as a bf16 pair (x0 in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float x0, float x1)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
}

// hi / lo parts of a pair: hi = bf16(x), lo = bf16(x - hi) (the difference is exact).
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t &hi, uint32_t &lo)
{
    hi = pack_bf16(x0, x1);
    lo = pack_bf16(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xFFFF0000u));
}

// ------------------------------------------------------- (1)/(2): Y = gamma * A T^T

struct WgDev {
    const void *A;        // [M][Kc] fp32 or bf16, row-major
    const uint32_t *T;    // [O][Kc/16] packed codes
    const float *gamma;
    float *Y;             // [M][O]
    int M, O, Kc;
    int tiles_o;
    int block_begin;
};

struct WgBatch {
    WgDev p[BL_MAX_GROUP];
    int count;
    int blocks;
};

constexpr int kWgThreads = 512;              // 2 x 4 waves, 64 x 64 outputs each
constexpr int kWgBM = 128, kWgBO = 256;      // block tile: A rows x code rows
constexpr int kWgKC = 64;                    // contraction per stage (4 packed words a row)
constexpr int kWgPitch = 2 * kWgKC + 16;     // LDS bytes per bf16 A row (padded: no bank
                                             // conflicts between the 16 rows of a read)
constexpr int kWgABytes = kWgBM * kWgPitch;
constexpr int kWgTBytes = kWgBO * 16;

// F32: A is fp32, split into hi / lo parts while staging.  Block tile 128 x 256 (twice as
// many code rows as A rows: each split A value then feeds twice the MFMAs), stages of
// 64 contraction indices double-buffered in LDS: the next stage's global loads are in
// flight while the current one is multiplied, one barrier per stage.  Lane (r, g) reads the
// A fragment of row r, contraction 16g + 8j .. +7 (16 bytes of LDS) and word g of its code
// row, expanded to the same eight contraction indices (half j).
template <bool F32>
__global__ __launch_bounds__(kWgThreads) void wgemm_kernel(WgBatch b)
{
    constexpr int PARTS = F32 ? 2 : 1;
    constexpr int STAGE = PARTS * kWgABytes + kWgTBytes;
    constexpr int ESZ = F32 ? 4 : 2;
    constexpr int CHUNKS = kWgBM * kWgKC * ESZ / 16 / kWgThreads;   // 16-byte A loads a thread
    constexpr int CPR = kWgKC * ESZ / 16;                            // 16-byte chunks per row
    __shared__ __align__(16) unsigned char lds[2][STAGE];

    int prob = 0;
#pragma unroll 1
    while (prob + 1 < b.count && (int)blockIdx.x >= b.p[prob + 1].block_begin)
        ++prob;
    const WgDev &p = b.p[prob];
    // XCD-aware order inside the problem: neighbouring tiles share an activation row panel.
    const int ntiles = (prob + 1 < b.count ? b.p[prob + 1].block_begin : b.blocks) - p.block_begin;
    const int tile = xcd_order(blockIdx.x - p.block_begin, ntiles);
    const int m0 = (tile / p.tiles_o) * kWgBM;
    const int o0 = (tile % p.tiles_o) * kWgBO;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave >> 2, wn = wave & 3;
    const int r = lane & 15, g = lane >> 4;
    const int Kc = p.Kc;
    const int words = Kc / 16;
    const int stages = (Kc + kWgKC - 1) / kWgKC;

    // Rows past M / O read as zero.  Activation chunks past Kc read as zero (offset kOOB);
    // code words past Kc may belong to the next row: they meet those zero activations.
    const rsrc_t ares = make_rsrc(static_cast<const unsigned char *>(p.A) + (int64_t)m0 * Kc * ESZ,
                                  rows_bytes(m0, kWgBM, p.M, Kc * ESZ));
    const rsrc_t tres = make_rsrc(p.T + (int64_t)o0 * words, rows_bytes(o0, kWgBO, p.O, words * 4));

    // One stage's global loads, held in registers until they are written to LDS (issued
    // before the previous stage is multiplied).  (Two alternating register sets, two stages
    // in flight, measured slower: past 256 registers a SIMD holds one wave instead of two.)
    struct Regs {
        v4u a[CHUNKS];
        v4u t;
    };
    auto load = [&](Regs &R, int s) {
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int q = tid + kWgThreads * i;
            const int row = q / CPR, c = (q % CPR) * (16 / ESZ);   // c: element in the stage
            const int k = s * kWgKC + c;
            R.a[i] = buf_load16(ares, k < Kc ? (uint32_t)(row * Kc + k) * ESZ : kOOB);
        }
        R.t = v4u{0, 0, 0, 0};
        if (tid < kWgBO) {
            const uint32_t off = (uint32_t)(tid * words + s * 4) * 4u;
            if ((words & 3) == 0) {
                R.t = buf_load16(tres, off);
            } else {
                // A 16-byte load running past the resource may come back all zero: with a
                // ragged word count take the row's words one by one (past the row: zero).
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    R.t[j] = buf_load4(tres, s * 4 + j < words ? off + 4u * j : kOOB);
            }
        }
    };
    auto store = [&](const Regs &R, int buf) {
        unsigned char *st = lds[buf];
#pragma unroll
        for (int i = 0; i < CHUNKS; ++i) {
            const int q = tid + kWgThreads * i;
            const int row = q / CPR, c = (q % CPR) * (16 / ESZ);
            unsigned char *dst = st + row * kWgPitch + 2 * c;
            if (F32) {
                uint32_t h0, l0, h1, l1;
                split_pair(__uint_as_float(R.a[i].x), __uint_as_float(R.a[i].y), h0, l0);
                split_pair(__uint_as_float(R.a[i].z), __uint_as_float(R.a[i].w), h1, l1);
                *reinterpret_cast<v2u *>(dst) = v2u{h0, h1};
                *reinterpret_cast<v2u *>(dst + kWgABytes) = v2u{l0, l1};
            } else {
                *reinterpret_cast<v4u *>(dst) = R.a[i];
            }
        }
        if (tid < kWgBO)
            *reinterpret_cast<v4u *>(st + PARTS * kWgABytes + tid * 16) = R.t;
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
            acc[mi][ni] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int buf) {
        const unsigned char *st = lds[buf];
        uint32_t wd[4];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
            wd[ni] = *reinterpret_cast<const uint32_t *>(st + PARTS * kWgABytes +
                                                         (wn * 64 + ni * 16 + r) * 16 + 4 * g);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            v4u bw[4];
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                bw[ni] = ternary_bf16(wd[ni], j);
#pragma unroll
            for (int part = 0; part < PARTS; ++part)
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    const v4u a = *reinterpret_cast<const v4u *>(
                        st + part * kWgABytes + (wm * 64 + mi * 16 + r) * kWgPitch + 32 * g + 16 * j);
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni)
                        acc[mi][ni] = mfma_bf16(bw[ni], a, acc[mi][ni]);
                }
        }
    };

    const float gammaf = __uint_as_float(buf_load4(make_rsrc(p.gamma, 4u), 0u));
    Regs R;
    load(R, 0);
    store(R, 0);
    __syncthreads();
    for (int s = 0; s < stages; ++s) {
        const bool more = s + 1 < stages;
        if (more)
            load(R, s + 1);
        compute(s & 1);
        if (more)
            store(R, (s + 1) & 1);
        __syncthreads();
    }

    // acc[mi][ni] register v: D[o][m] for o = o0 + wn * 64 + ni * 16 + 4g + v and
    // m = m0 + wm * 64 + mi * 16 + r (the codes are the MFMA's row operand): four
    // consecutive outputs of one row per lane.
    const bool vec = (p.O & 3) == 0 && ((uintptr_t)p.Y & 15) == 0;
    // A full tile: whole-line non-temporal stores (store_pair_lines_nt), as in the prefill
    // product's epilogue.
    if (vec && m0 + kWgBM <= p.M && o0 + kWgBO <= p.O && (int64_t)kWgBM * p.O * 4 <= (int64_t)0xFFFFFFFFu) {
        const rsrc_t yres = make_rsrc(p.Y + (int64_t)m0 * p.O, (uint32_t)kWgBM * (uint32_t)p.O * 4u);
        const bool lo = r < 8;
        const uint32_t pitch8 = 8u * (uint32_t)p.O * 4u;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const uint32_t base = (uint32_t)(wm * 64 + mi * 16 + (r & 7)) * (uint32_t)p.O * 4u +
                                  (uint32_t)(o0 + wn * 64 + 4 * g + (lo ? 0 : 16)) * 4u;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const f32x4 ye = acc[mi][2 * pp] * gammaf;
                const f32x4 yo = acc[mi][2 * pp + 1] * gammaf;
                store_pair_lines_nt(yres, base + (uint32_t)(pp * 32 * 4), pitch8, lo,
                                    __builtin_bit_cast(v4u, ye), __builtin_bit_cast(v4u, yo));
            }
        }
        return;
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int m = m0 + wm * 64 + mi * 16 + r;
        if (m >= p.M)
            continue;
        float *yrow = p.Y + (int64_t)m * p.O;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int o = o0 + wn * 64 + ni * 16 + 4 * g;
            const f32x4 y = acc[mi][ni] * gammaf;
            if (vec && o + 3 < p.O) {
                *reinterpret_cast<float4 *>(yrow + o) = make_float4(y[0], y[1], y[2], y[3]);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (o + v < p.O)
                        yrow[o + v] = y[v];
            }
        }
    }
}

hipError_t launch_wgemm(const WgProblem *q, int count, hipStream_t stream)
{
    // bf16 activations: the prefill pipeline (direct-to-LDS loads, no conversion to stage).
    hipError_t e0 = launch_wonly_prefill(q, count, stream);
    if (e0 != hipSuccess)
        return e0;
    for (int f32 = 1; f32 < 2; ++f32) {
        WgBatch b{};
        int blocks = 0;
        for (int i = 0; i < count; ++i) {
            const WgProblem &s = q[i];
            if (s.f32 != (f32 != 0) || s.M == 0 || s.O == 0)
                continue;
            WgDev &d = b.p[b.count++];
            d.A = s.A;
            d.T = s.T;
            d.gamma = s.gamma;
            d.Y = s.Y;
            d.M = (int)s.M;
            d.O = (int)s.O;
            d.Kc = (int)s.Kc;
            d.tiles_o = (d.O + kWgBO - 1) / kWgBO;
            d.block_begin = blocks;
            blocks += ((d.M + kWgBM - 1) / kWgBM) * d.tiles_o;
        }
        if (!blocks)
            continue;
        b.blocks = blocks;
        if (f32)
            hipLaunchKernelGGL((wgemm_kernel<true>), dim3(blocks), dim3(kWgThreads), 0, stream, b);
        else
            hipLaunchKernelGGL((wgemm_kernel<false>), dim3(blocks), dim3(kWgThreads), 0, stream, b);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// ------------------------------------------------------- (3): packed C -> packed C^T

// Block: 64 code rows (n) x 64 columns (k).  Each thread loads one input word into LDS, then
// assembles one output word: column k's codes of 16 consecutive rows, in the canonical field
// layout (row 16w' + 4i + b of the output word at bits 8b + 2i).
__global__ __launch_bounds__(256) void transpose_packed_kernel(const uint32_t *P, int N, int K,
                                                                uint32_t *Pt, int tiles_k)
{
    __shared__ uint32_t in[64][5];
    const int n0 = (blockIdx.x / tiles_k) * 64, k0 = (blockIdx.x % tiles_k) * 64;
    const int words = K / 16, owords = N / 16;
    const int t = threadIdx.x;
    {
        const int n = n0 + (t >> 2), w = k0 / 16 + (t & 3);
        in[t >> 2][t & 3] = (n < N && w < words) ? P[(int64_t)n * words + w] : 0u;
    }
    __syncthreads();
    const int kk = t >> 2, ow = t & 3;
    const int k = k0 + kk, wo = n0 / 16 + ow;
    if (k >= K || wo >= owords)
        return;
    const int kin = kk & 15;
    const int sh_in = 8 * (kin & 3) + 2 * (kin >> 2);
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint32_t f = (in[16 * ow + j][kk >> 4] >> sh_in) & 3u;
        out |= f << (8 * (j & 3) + 2 * (j >> 2));
    }
    Pt[(int64_t)k * owords + wo] = out;
}

hipError_t launch_transpose_packed(const uint32_t *P, int64_t N, int64_t K, uint32_t *Pt,
                                   hipStream_t stream)
{
    if (N == 0)
        return hipSuccess;
    const int tiles_n = (int)((N + 63) / 64), tiles_k = (int)((K + 63) / 64);
    hipLaunchKernelGGL(transpose_packed_kernel, dim3(tiles_n * tiles_k), dim3(256), 0, stream,
                       P, (int)N, (int)K, Pt, tiles_k);
    return hipGetLastError();
}

// ------------------------------------------------------- (4): weight gradient

struct GwDev {
    const float *dY;      // [M][N]
    const int8_t *Xq;     // [M][K]
    const float *sx;      // [M]
    const float *W;       // [N][K] (hard / soft scale) or NULL
    const float *gamma;
    float *dW;            // [N][K]
    int M, N, K;
    int ste;
    float beta;
    int tiles_k;
    int block_begin;
};

struct GwBatch {
    GwDev p[BL_MAX_GROUP];
    int count;
    int blocks;
};

constexpr int kGwThreads = 512;              // 2 x 4 waves, 64 x 64 outputs each
constexpr int kGwBN = 128, kGwBK = 256;      // block tile: dW rows (n) x columns (k)
constexpr int kGwKC = 32;                    // tokens per stage (one MFMA k-step)
constexpr int kGwPitch = 2 * kGwKC + 16;     // LDS bytes per bf16 row (padded)
constexpr int kGwPartY = kGwBN * kGwPitch;   // one bf16 part of the dY tile
constexpr int kGwPartQ = kGwBK * kGwPitch;   // the q tile
constexpr int kGwStage = 2 * kGwPartY + kGwPartQ;   // dY hi, dY lo, q

// Stage s covers tokens 32s .. 32s+31.  Staging: dY is scaled by s_x (one fp32 product, as
// the dequantized activation q * s_x is folded into dY's side) and split, q converted
// (exact), and both land transposed: row = column of dW, contiguous in tokens.  The tile is
// twice as wide in k as in n because the dY conversion (product, split) costs several
// instructions per value and q's one: every staged dY value then feeds twice the MFMAs.
__global__ __launch_bounds__(kGwThreads) void gradw_kernel(GwBatch b)
{
    __shared__ __align__(16) unsigned char lds[2][kGwStage];

    int prob = 0;
#pragma unroll 1
    while (prob + 1 < b.count && (int)blockIdx.x >= b.p[prob + 1].block_begin)
        ++prob;
    const GwDev &p = b.p[prob];
    // XCD-aware order inside the problem: neighbouring tiles share a dY column panel, and
    // run through the tokens together, so the panel's current stage is read once per XCD.
    const int ntiles = (prob + 1 < b.count ? b.p[prob + 1].block_begin : b.blocks) - p.block_begin;
    const int tile = xcd_order(blockIdx.x - p.block_begin, ntiles);
    const int n0 = (tile / p.tiles_k) * kGwBN;
    const int k0 = (tile % p.tiles_k) * kGwBK;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave >> 2, wn = wave & 3;
    const int r = lane & 15, g = lane >> 4;
    const int M = p.M, N = p.N, K = p.K;
    const int stages = (M + kGwKC - 1) / kGwKC;
    const rsrc_t sres = make_rsrc(p.sx, (uint32_t)M * 4u);

    // Per stage: the tokens' rows from column n0 (k0) on; tokens past M read zero.  Columns
    // past N (K) belong to the next row: they only reach dW rows (columns) that are not
    // stored.  dY: thread t takes tokens 4 (t % 8) + 2 (t / 256) + {0, 1} of the four columns
    // 4 ((t / 8) % 32) .. +3 (two 16-byte loads) and writes each (column, token pair) with
    // one 4-byte store per part; q: tokens 4 (t % 8) .. +3 of the columns 4 (t / 8) .. +3 (four
    // dword loads), one 8-byte store per column.  In both, lane l of a half-wave takes token
    // quad l % 8 and column quad l / 8, so a store instruction's lanes fall in 32 distinct
    // banks (columns four apart are 320 bytes apart, 64 modulo the 256-byte bank cycle, and
    // the token quads fill the 64), where token-quad-major lanes collided 8 ways.
    const int tq = tid & 7;
    const int yc = ((tid >> 3) & 31) * 4, yh = tid >> 8;   // dY: column quad, token pair
    const int qc = (tid >> 3) * 4;                          // q: column quad
    struct Regs {
        v4u y[2];      // [token of the pair]: four dY columns
        float s[2];
        uint32_t q[4]; // [token]: four q columns
    };
    auto load = [&](Regs &R, int st) {
        const int t0 = st * kGwKC;
        const int live = min(kGwKC, M - t0);
        const int64_t ybytes = (int64_t)live * N * 4 - (int64_t)n0 * 4;
        const int64_t qbytes = (int64_t)live * K - (int64_t)k0;
        const rsrc_t yres = make_rsrc(p.dY + (int64_t)t0 * N + n0, ybytes > 0 ? (uint32_t)ybytes : 0u);
        const rsrc_t qres = make_rsrc(p.Xq + (int64_t)t0 * K + k0, qbytes > 0 ? (uint32_t)qbytes : 0u);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int t = 4 * tq + 2 * yh + h;
            const uint32_t off = (uint32_t)(t * N + yc) * 4u;
            if ((N & 3) == 0) {
                R.y[h] = buf_load16(yres, off);
            } else {
                // Rows not 16-byte multiples: one dword at a time (see wgemm_kernel).
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    R.y[h][e] = buf_load4(yres, off + 4u * e);
            }
            R.s[h] = __uint_as_float(buf_load4(sres, (uint32_t)(t0 + t) * 4u));
        }
#pragma unroll
        for (int h = 0; h < 4; ++h)
            R.q[h] = buf_load4(qres, (uint32_t)((4 * tq + h) * K + qc));
    };
    auto store = [&](const Regs &R, int buf) {
        unsigned char *st = lds[buf];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t hi, lo;
            split_pair(__uint_as_float(R.y[0][e]) * R.s[0], __uint_as_float(R.y[1][e]) * R.s[1], hi, lo);
            unsigned char *dy = st + (yc + e) * kGwPitch + 8 * tq + 4 * yh;
            *reinterpret_cast<uint32_t *>(dy) = hi;
            *reinterpret_cast<uint32_t *>(dy + kGwPartY) = lo;
            float f[4];
#pragma unroll
            for (int h = 0; h < 4; ++h)
                f[h] = (float)((int)(R.q[h] << (24 - 8 * e)) >> 24);   // exact in bf16
            *reinterpret_cast<v2u *>(st + 2 * kGwPartY + (qc + e) * kGwPitch + 8 * tq) =
                v2u{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3])};
        }
    };

    f32x4 acc[4][4];   // [ni][mi]
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
            acc[ni][mi] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int buf) {
        const unsigned char *st = lds[buf];
        v4u bq[4];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
            bq[ni] = *reinterpret_cast<const v4u *>(st + 2 * kGwPartY + (wn * 64 + ni * 16 + r) * kGwPitch + 16 * g);
#pragma unroll
        for (int part = 0; part < 2; ++part)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const v4u a = *reinterpret_cast<const v4u *>(st + part * kGwPartY +
                                                             (wm * 64 + mi * 16 + r) * kGwPitch + 16 * g);
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[ni][mi] = mfma_bf16(bq[ni], a, acc[ni][mi]);
            }
    };

    const float gammaf = __uint_as_float(buf_load4(make_rsrc(p.gamma, 4u), 0u));
    Regs R;
    if (stages > 0) {
        load(R, 0);
        store(R, 0);
    }
    __syncthreads();
    for (int s = 0; s < stages; ++s) {
        const bool more = s + 1 < stages;
        if (more)
            load(R, s + 1);
        compute(s & 1);
        if (more)
            store(R, (s + 1) & 1);
        __syncthreads();
    }

    // acc[ni][mi] register v: dW[n][k] for k = k0 + wn * 64 + ni * 16 + 4g + v and
    // n = n0 + wm * 64 + mi * 16 + r.  Gradient scale from t = fl32(W / gamma) (the
    // quantizer's division; gamma == 0 gives t = 0).
    const bool vec = ((uintptr_t)p.dW & 15) == 0 && (!p.W || ((uintptr_t)p.W & 15) == 0);
    const double beta = (double)p.beta;
    // The four outputs of group (mi, ni): row n, columns k .. k + 3.
    auto outputs = [&](int mi, int ni, int n, int k, float (&y)[4]) {
        float w[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (p.ste != 0) {
            const float *wrow = p.W + (int64_t)n * K + k;
            if (vec) {
                const float4 wv = *reinterpret_cast<const float4 *>(wrow);
                w[0] = wv.x; w[1] = wv.y; w[2] = wv.z; w[3] = wv.w;
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    w[v] = wrow[v];
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float a = acc[ni][mi][v];
            if (p.ste == 0) {
                y[v] = a;
            } else {
                const float t = gammaf == 0.0f ? 0.0f : w[v] / gammaf;   // correctly rounded
                if (p.ste == 1) {
                    y[v] = fabsf(t) <= 1.0f ? a : 0.0f;
                } else {
                    // sech^2(x) = 4 e / (1 + e)^2 with e = exp(-2 |x|): one exponential.
                    const double e = exp(-2.0 * fabs(beta * (double)t));
                    const double d = 1.0 + e;
                    y[v] = (float)((4.0 * e / (d * d)) * (double)a);
                }
            }
        }
    };
    // A full tile: whole-line non-temporal stores (store_pair_lines_nt), as in the prefill
    // product's epilogue.
    if (vec && n0 + kGwBN <= N && k0 + kGwBK <= K && (int64_t)kGwBN * K * 4 <= (int64_t)0xFFFFFFFFu) {
        const rsrc_t dres = make_rsrc(p.dW + (int64_t)n0 * K, (uint32_t)kGwBN * (uint32_t)K * 4u);
        const bool lo = r < 8;
        const uint32_t pitch8 = 8u * (uint32_t)K * 4u;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            const int n = n0 + wm * 64 + mi * 16 + r;
            const uint32_t base = (uint32_t)(wm * 64 + mi * 16 + (r & 7)) * (uint32_t)K * 4u +
                                  (uint32_t)(k0 + wn * 64 + 4 * g + (lo ? 0 : 16)) * 4u;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                float ye[4], yo[4];
                outputs(mi, 2 * pp, n, k0 + wn * 64 + 2 * pp * 16 + 4 * g, ye);
                outputs(mi, 2 * pp + 1, n, k0 + wn * 64 + (2 * pp + 1) * 16 + 4 * g, yo);
                const v4u e = {__float_as_uint(ye[0]), __float_as_uint(ye[1]), __float_as_uint(ye[2]), __float_as_uint(ye[3])};
                const v4u o = {__float_as_uint(yo[0]), __float_as_uint(yo[1]), __float_as_uint(yo[2]), __float_as_uint(yo[3])};
                store_pair_lines_nt(dres, base + (uint32_t)(pp * 32 * 4), pitch8, lo, e, o);
            }
        }
        return;
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
        const int n = n0 + wm * 64 + mi * 16 + r;
        if (n >= N)
            continue;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
            const int k = k0 + wn * 64 + ni * 16 + 4 * g;
            if (k >= K)
                continue;     // K % 16 == 0: the four columns are all in or all out
            float y[4];
            outputs(mi, ni, n, k, y);
            float *dst = p.dW + (int64_t)n * K + k;
            if (vec) {
                *reinterpret_cast<float4 *>(dst) = make_float4(y[0], y[1], y[2], y[3]);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    dst[v] = y[v];
            }
        }
    }
}

hipError_t launch_grad_weight(const bl_grad_weight_problem *q, int count, hipStream_t stream)
{
    GwBatch b{};
    int blocks = 0;
    for (int i = 0; i < count; ++i) {
        const bl_grad_weight_problem &s = q[i];
        if (s.N == 0)
            continue;
        GwDev &d = b.p[b.count++];
        d.dY = s.dY;
        d.Xq = s.X_q;
        d.sx = s.x_scale;
        d.W = s.W;
        d.gamma = s.gamma;
        d.dW = s.dW;
        d.M = (int)s.M;
        d.N = (int)s.N;
        d.K = (int)s.K;
        d.ste = s.ste;
        d.beta = s.beta;
        d.tiles_k = (d.K + kGwBK - 1) / kGwBK;
        d.block_begin = blocks;
        blocks += ((d.N + kGwBN - 1) / kGwBN) * d.tiles_k;
    }
    if (!blocks)
        return hipSuccess;
    b.blocks = blocks;
    hipLaunchKernelGGL(gradw_kernel, dim3(blocks), dim3(kGwThreads), 0, stream, b);
    return hipGetLastError();
}

}  // namespace bl
