// quant.hip — weight scale, ternary quantize-and-pack, code packing and int8 activation
// quantization kernels for gfx950.
//
// Weight path (Distillix README, "1. BitNet b1.58 Core": W_q = round(clip(W / mean|W|, -1, 1));
// bitone README, "Features": gamma from a separate one-dimensional reduction over W, and the
// quantized weights never materialized in HBM):
//   gamma_partial_kernel  reads W once, writes up to kGammaParts fp64 partial sums per tensor;
//   quant_pack_kernel     reduces the partials (same fixed order in every wave, so every wave
//                         sees the same gamma), reads W again and writes packed words.
//
// Activation path (BitDistill article: INT8 activations, SubLN before the attention and FFN
// output projections; SLM750-Edge card: RMSNorm epsilon 1e-6):
//   act_quant_wave_kernel   one wave per token row (K <= 4096);
//   act_quant_block_kernel  one block per token row for longer rows;
//   both: absmax (+ fixed-order sum of squares for the norm), then q = rint(u * (127 / a))
//   and the row scale.
//
// Rounding-sensitive arithmetic is written so that it matches IEEE-754 fp32 semantics:
// the library is built with -ffp-contract=off, fp32 division is correctly rounded (the HIP
// default), and rintf lowers to round-to-nearest-even.
#include <stdlib.h>

#include <algorithm>

#include "common.hpp"

namespace bl {

constexpr int kGammaParts = 256;    // partial sums per tensor; fixed, so the order is fixed
constexpr int kGammaThreads = 256;
constexpr int kPackThreads = 256;
constexpr int kPackUnroll = 8;      // float4 chunks per thread in quant_pack_kernel
constexpr int kActThreads = 256;

// ----------------------------------------------------------------------------- gamma

struct WeightDev {
    const float4 *W;
    uint32_t *packed;
    float *gamma;
    double *partials;   // [parts]
    int64_t chunks;     // N * K / 4 float4 chunks
    int parts;          // partial sums (blocks of gamma_partial_kernel) for this tensor
    int part_begin;     // first block of this tensor in gamma_partial_kernel's grid
    int pack_begin;     // first block of this tensor in quant_pack_kernel's grid
    uint32_t quad_wpr;  // 0: rows [N][K/16]; else K/16, and the words go to the quad-row layout
    // One-read form only (the workspace regions of this tensor; see one_read_pass_kernel):
    double *sample;     // [kSampleBlocks][2]: sum |w| and sum w^2 of the sampled pieces
    float *band;        // [2]: the band (lo, hi) the pass used; lo > hi: the pass listed nothing
    uint32_t *counts;   // [parts * 4]: chunks each wave listed
    uint32_t *keys;     // [parts * 4][cap]: chunk index << 4 | mask of its band weights
    v4u *vals;          // [parts * 4][cap]: the chunk's four fp32 values
    uint32_t cap;       // list entries per wave
    int sparts;         // sample blocks of this tensor
    int sample_begin;   // first block of this tensor in the sample grid
};

struct WeightBatch {
    WeightDev p[BL_MAX_GROUP];
    int count;
};

// Number of partial sums for a tensor: about 4 float4 chunks per thread, at most kGammaParts.
// A function of the shape only, so the summation order is fixed for a given shape.
static int gamma_parts(int64_t chunks)
{
    const int64_t per = 4 * kGammaThreads;
    const int64_t parts = (chunks + per - 1) / per;
    return (int)(parts < 1 ? 1 : parts > kGammaParts ? kGammaParts : parts);
}

__device__ __forceinline__ void gamma_partial_block(const WeightBatch &b, int bid)
{
    __shared__ double lds[kGammaThreads / kWave];
    int prob = 0;
#pragma unroll 1
    while (prob + 1 < b.count && bid >= b.p[prob + 1].part_begin)
        ++prob;
    const WeightDev &p = b.p[prob];
    const int part = bid - p.part_begin;
    const int64_t stride = (int64_t)p.parts * kGammaThreads;
    double s = 0.0;
    int64_t i = (int64_t)part * kGammaThreads + threadIdx.x;
    auto add4 = [&s](float x, float y, float z, float w) {
        s += fabs((double)x); s += fabs((double)y);
        s += fabs((double)z); s += fabs((double)w);
    };
    if (p.chunks * 16 < ((int64_t)1 << 31)) {
        // Eight loads in flight per thread through a buffer resource (chunks past the tensor
        // read as zeros and add nothing); the additions stay in index order.  Non-temporal:
        // the masters are streamed, and left uncached they do not evict the packed words and
        // activation codes the product reads next (weight quantization of the Qwen3-4B set
        // 141 -> 131-133 us; the same hint on the activation rows was slower).
        const rsrc_t wr = make_rsrc(p.W, (uint32_t)(p.chunks * 16));
        for (; i < p.chunks; i += 8 * stride) {
            v4u v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t j = i + u * stride;
                v[u] = buf_load16_nt(wr, j < p.chunks ? (uint32_t)(j * 16) : kOOB);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                add4(__uint_as_float(v[u].x), __uint_as_float(v[u].y), __uint_as_float(v[u].z),
                     __uint_as_float(v[u].w));
        }
    } else {
        // Tensors of 2 GiB and more: four loads in flight, plain pointers.
        for (; i + 3 * stride < p.chunks; i += 4 * stride) {
            const float4 v0 = p.W[i], v1 = p.W[i + stride], v2 = p.W[i + 2 * stride],
                         v3 = p.W[i + 3 * stride];
            add4(v0.x, v0.y, v0.z, v0.w);
            add4(v1.x, v1.y, v1.z, v1.w);
            add4(v2.x, v2.y, v2.z, v2.w);
            add4(v3.x, v3.y, v3.z, v3.w);
        }
        for (; i < p.chunks; i += stride) {
            const float4 v = p.W[i];
            add4(v.x, v.y, v.z, v.w);
        }
    }
    // Fixed-order block sum: wave butterfly, then the waves in index order.
    s = wave_sum_fixed(s);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0)
        lds[wave] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = lds[0];
#pragma unroll
        for (int w = 1; w < kGammaThreads / kWave; ++w)
            t = t + lds[w];
        p.partials[part] = t;
    }
}

// ------------------------------------------------------------------- quantize + pack
//
// Code rule without a per-element division.  For gamma > 0 and the fp32 quotient
// t = fl(W / gamma) (correctly rounded, hence monotone in W):
//   t > 0.5  <=>  W / gamma > 0.5 + 2^-25  (0.5 + 2^-25 is the midpoint between 0.5 and the
//            next fp32; a tie there rounds to the even 0.5)
//           <=>  W > T,  T = gamma * (0.5 + 2^-25)  (exact in fp64: 24 x 25 significant bits)
//           <=>  W > tau, tau = the largest fp32 <= T   (W is an fp32)
// and symmetrically t < -0.5 <=> -W > tau.  So c = sign(W) when |W| > tau, else 0, which is
// bit-identical to round_clip(fl(W / gamma)) for every fp32 W, including infinities and
// subnormals; NaN compares false and gives 0.  gamma == 0 (and NaN) must give all zeros:
// tau = +inf (NaN) achieves that.
__device__ __forceinline__ float code_threshold(float gamma)
{
    if (!(gamma > 0.0f))
        return gamma == 0.0f ? __builtin_inff() : gamma;  // 0 -> +inf; NaN stays NaN
    const double T = (double)gamma * (0.5 + 0x1p-25);
    float tau = (float)T;                                  // round to nearest
    if ((double)tau > T)
        tau = __int_as_float(__float_as_int(tau) - 1);     // step down to the largest <= T
    return tau;
}

__device__ __forceinline__ uint32_t quad_or(uint32_t v)
{
    // OR over the four lanes of a quad (DPP quad_perm [1,0,3,2] then [2,3,0,1]).
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
    v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
    return v;
}

__global__ __launch_bounds__(kGammaThreads) void gamma_partial_kernel(WeightBatch b)
{
    gamma_partial_block(b, blockIdx.x);
}

__global__ __launch_bounds__(kPackThreads) void quant_pack_kernel(WeightBatch b)
{
    int prob = 0;
#pragma unroll 1
    while (prob + 1 < b.count && (int)blockIdx.x >= b.p[prob + 1].pack_begin)
        ++prob;
    const WeightDev &p = b.p[prob];
    const int blk = blockIdx.x - p.pack_begin;

    // Issue this block's weight loads first (they do not depend on gamma), then reduce gamma
    // while they are in flight.  Out-of-range chunks of the last block read as zero.  The
    // masters are streamed with the non-temporal hint, as in the gamma pass.
    const int64_t base = (int64_t)blk * kPackThreads * kPackUnroll;
    const int64_t live = p.chunks - base < kPackThreads * kPackUnroll ? p.chunks - base
                                                                       : kPackThreads * kPackUnroll;
    const rsrc_t wres = make_rsrc(p.W + base, live > 0 ? (uint32_t)live * 16u : 0u);
    v4u raw[kPackUnroll];
#pragma unroll
    for (int u = 0; u < kPackUnroll; ++u)
        raw[u] = buf_load16_nt(wres, (uint32_t)(u * kPackThreads + threadIdx.x) * 16u);

    // gamma = fl32(sum / count).  Every wave reduces the partial sums itself in the same
    // fixed order (lane-sequential, then the wave butterfly), so every wave of every block
    // holds the same gamma without a barrier.
    const int lane = threadIdx.x & (kWave - 1);
    double part = 0.0;
    {
        // All of a lane's partials (parts <= 256: four) loaded at once; slots past the
        // partials read as zeros and add nothing.
        const rsrc_t pr = make_rsrc(p.partials, (uint32_t)p.parts * 8u);
        v2u v[kGammaParts / kWave];
#pragma unroll
        for (int k = 0; k < kGammaParts / kWave; ++k)
            v[k] = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(
                                               pr, (lane + k * kWave) * 8, 0, 0));
#pragma unroll
        for (int k = 0; k < kGammaParts / kWave; ++k)
            part += __longlong_as_double((long long)(((uint64_t)v[k].y << 32) | v[k].x));
    }
    const double sum = wave_sum_fixed(part);
    const double count = (double)(p.chunks * 4);
    const float gamma = p.chunks > 0 ? (float)(sum / count) : 0.0f;
    if (blk == 0 && threadIdx.x == 0)
        *p.gamma = gamma;
    const float tau = code_threshold(gamma);

    // Each lane turns 4 consecutive weights (one float4) into its plane of a packed word:
    // chunk j covers k = 4j .. 4j + 3, i.e. word j / 4, plane i = j % 4, bytes b = 0..3.
    // The four lanes of a quad hold the four planes of one word and OR them together.
#pragma unroll
    for (int u = 0; u < kPackUnroll; ++u) {
        const int64_t j = base + (int64_t)u * kPackThreads + threadIdx.x;
        const float vx = __uint_as_float(raw[u].x), vy = __uint_as_float(raw[u].y);
        const float vz = __uint_as_float(raw[u].z), vw = __uint_as_float(raw[u].w);
        const int sh = 2 * (int)(j & 3);
        uint32_t bits = code_field(fabsf(vx) > tau, vx < 0.0f) << (0 + sh);
        bits |= code_field(fabsf(vy) > tau, vy < 0.0f) << (8 + sh);
        bits |= code_field(fabsf(vz) > tau, vz < 0.0f) << (16 + sh);
        bits |= code_field(fabsf(vw) > tau, vw < 0.0f) << (24 + sh);
        bits = quad_or(bits);
        if (j < p.chunks && (j & 3) == 0)
            p.packed[p.quad_wpr ? quad_row_word((uint32_t)(j >> 2), p.quad_wpr) : j >> 2] = bits;
    }
}

// --------------------------------------------------------- one-read quantize + pack
//
// The two passes above read W twice: the codes need gamma, and gamma needs all of W.  The
// one-read form reads W once and still gives the codes of the exact rule above, bit for bit:
//
//   sample     (sample_block)  reads one 4 KB piece out of every 64 KB of W and sums |w| and
//              w^2 in fp64: an estimate g of gamma and its standard error;
//   pass       (one_read_pass_kernel) is the gamma pass (the same blocks, loads and summation
//              order, so the partial sums and gamma are the same bits), and meanwhile writes
//              each weight's code against a band lo < hi around the estimated threshold g/2:
//              |w| > hi gives sign(w), |w| <= lo gives 0, and a weight inside the band gets 0
//              for now; a chunk (four weights) holding such a weight is listed (its index, a
//              mask of those weights, its four values) in its wave's region;
//   fix-up     (one_read_fix_kernel) reduces gamma and tau exactly as quant_pack_kernel does,
//              checks lo <= tau <= hi, and then ORs the code of every listed weight with
//              |w| > tau into its word.
//
// With lo <= tau <= hi, an unlisted |w| > hi exceeds tau and an unlisted |w| <= lo does not,
// so every unlisted code equals the exact rule's; the listed ones are decided against tau
// itself.  The estimate therefore sets only how many weights are listed, never a code.  When
// the check fails (an unrepresentative sample, gamma == 0, a NaN or an infinity in W, a band
// too wide to be useful) or a wave's list overflowed, the fix-up block reads its own chunks
// of W again and writes their codes from tau, as the pack pass would.  A block's chunks are
// the gamma pass's (chunk i = part * 256 + t + r * parts * 256), so the words of different
// blocks are disjoint and a block may rewrite its words while other blocks OR fields into
// theirs.

constexpr int kSampleBlocks = 256;        // sample partial sums per tensor (at most)
constexpr int64_t kSampleGroup = 4096;    // chunks per 64 KB group; its first 256 are sampled
constexpr int kSampleChunks = 256;
constexpr double kBandSigmas = 8.0;       // band half-width in standard errors of the estimate
constexpr double kBandFloor = 0x1p-12;    // ... plus this relative floor
constexpr double kBandMax = 0.03;         // wider bands (small samples): no listing, one re-read
constexpr int kListShare = 16;            // list capacity: one chunk in 16 per wave, plus 64

__host__ __device__ inline int64_t sample_groups(int64_t chunks)
{
    return (chunks + kSampleGroup - 1) / kSampleGroup;
}

// Weights the sample covers: every group's first 256 chunks (fewer in a short last group).
__host__ __device__ inline double sample_weights(int64_t chunks)
{
    const int64_t g = sample_groups(chunks);
    if (g == 0)
        return 0.0;
    const int64_t last = chunks - (g - 1) * kSampleGroup;
    return 4.0 * (double)((g - 1) * kSampleChunks + (last < kSampleChunks ? last : kSampleChunks));
}

__device__ __forceinline__ void sample_block(const WeightBatch &b, int bid)
{
    __shared__ double lds[2][kGammaThreads / kWave];
    int prob = 0;
#pragma unroll 1
    while (prob + 1 < b.count && bid >= b.p[prob + 1].sample_begin)
        ++prob;
    const WeightDev &p = b.p[prob];
    const int s = bid - p.sample_begin;
    const int64_t groups = sample_groups(p.chunks);
    const rsrc_t wr = make_rsrc(p.W, (uint32_t)(p.chunks * 16));
    double a = 0.0, q = 0.0;
    for (int64_t g = s; g < groups; g += 4 * (int64_t)p.sparts) {
        v4u v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t j = (g + u * (int64_t)p.sparts) * kSampleGroup + threadIdx.x;
            const bool in = g + u * (int64_t)p.sparts < groups && j < p.chunks;
            v[u] = buf_load16_nt(wr, in ? (uint32_t)(j * 16) : kOOB);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float x[4] = {__uint_as_float(v[u].x), __uint_as_float(v[u].y),
                                __uint_as_float(v[u].z), __uint_as_float(v[u].w)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a += fabs((double)x[e]);
                q += (double)x[e] * (double)x[e];
            }
        }
    }
    a = wave_sum_fixed(a);
    q = wave_sum_fixed(q);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
        lds[0][wave] = a;
        lds[1][wave] = q;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double ta = lds[0][0], tq = lds[1][0];
#pragma unroll
        for (int w = 1; w < kGammaThreads / kWave; ++w) {
            ta = ta + lds[0][w];
            tq = tq + lds[1][w];
        }
        p.sample[2 * s] = ta;
        p.sample[2 * s + 1] = tq;
    }
}

__global__ __launch_bounds__(kGammaThreads) void sample_kernel(WeightBatch b)
{
    sample_block(b, blockIdx.x);
}

// The band from the sample: the estimated threshold g/2 widened by kBandSigmas standard errors
// of g (plus kBandFloor), relative.  lo > hi (no band) when the sample says nothing useful.
// Every wave of the pass computes it from the same sums in the same order, so all agree.
__device__ __forceinline__ void one_read_band(const WeightDev &p, int lane, float &lo, float &hi)
{
    double a = 0.0, q = 0.0;
#pragma unroll
    for (int k = 0; k < kSampleBlocks / kWave; ++k) {
        const int s = lane + k * kWave;
        a += s < p.sparts ? p.sample[2 * s] : 0.0;
        q += s < p.sparts ? p.sample[2 * s + 1] : 0.0;
    }
    a = wave_sum_fixed(a);
    q = wave_sum_fixed(q);
    const double n = sample_weights(p.chunks);
    const double g = a / n;
    const double var = q / n - g * g;                  // of |w|
    const double d = kBandSigmas * sqrt(fmax(var, 0.0) / n) / g + kBandFloor;
    lo = 1.0f;
    hi = 0.0f;
    if (g > 0.0 && g < 1e30 && d < kBandMax) {
        const double t = 0.5 * g;
        lo = (float)(t * (1.0 - d));
        hi = (float)(t * (1.0 + d));
    }
}

// Byte e of the result is the top byte of v[e].
__device__ __forceinline__ uint32_t top_bytes(const uint32_t (&v)[4])
{
    return __builtin_amdgcn_perm(v[1], v[0], 0x0c0c0703u) | __builtin_amdgcn_perm(v[3], v[2], 0x07030c0cu);
}

// The one-read kernels index in 32 bits: their tensors are below 2 GiB (2^27 chunks).
__device__ __forceinline__ uint32_t word_index(uint32_t quad_wpr, uint32_t j)
{
    return quad_wpr ? quad_row_word(j >> 2, quad_wpr) : j >> 2;
}

// Each wave lists, in a region of its own, the chunks (four weights) that hold a weight inside
// the band: entry e of wave w (of the tensor's parts * 4 waves) sits at slot w * cap + e, its
// key (chunk index << 4 | mask of the band's weights) in keys[slot] and the four fp32 values in
// vals[slot].  The lanes that list a chunk at the same step take consecutive slots (a ballot
// and a count of the lower lanes), so the stores are contiguous and no lane waits for another.
__global__ __launch_bounds__(kGammaThreads) void one_read_pass_kernel(WeightBatch b)
{
    __shared__ double lds[kGammaThreads / kWave];
    const int bid = blockIdx.x;
    int prob = 0;
#pragma unroll 1
    while (prob + 1 < b.count && bid >= b.p[prob + 1].part_begin)
        ++prob;
    const WeightDev &p = b.p[prob];
    const int part = bid - p.part_begin;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
    float lo, hi;
    one_read_band(p, lane, lo, hi);
    const bool spec = lo <= hi;
    if (part == 0 && threadIdx.x == 0) {
        p.band[0] = lo;
        p.band[1] = hi;
    }
    // The band compared on the bits of |w| (non-negative floats order as their bits).  A NaN
    // or an infinity in W compares above hi and gets a provisional code, but it also makes
    // gamma NaN or infinite, so the fix-up's check fails and codes this tensor again.
    const uint32_t lo_bits = __float_as_uint(lo), hi_bits = __float_as_uint(hi);
    const int wave_global = part * (kGammaThreads / kWave) + wave;
    // Every store goes through a buffer resource: buffer stores complete in order with the
    // weight loads, so the loop waits for each load alone (with flat stores in the loop the
    // compiler had to wait for all of a step's loads before coding its first chunk), and the
    // list's stores past this wave's capacity are dropped by the resource's range check.
    const uint32_t cap = (uint32_t)__builtin_amdgcn_readfirstlane((int)p.cap);
    const rsrc_t keys = make_rsrc(p.keys + (size_t)wave_global * cap, cap * 4u);
    const rsrc_t vals = make_rsrc(p.vals + (size_t)wave_global * cap, cap * 16u);
    const uint32_t wpr = (uint32_t)__builtin_amdgcn_readfirstlane((int)p.quad_wpr);
    uint32_t listed = 0;
    const uint32_t stride = (uint32_t)p.parts * kGammaThreads;
    const uint32_t chunks = (uint32_t)p.chunks;
    const rsrc_t wr = make_rsrc(p.W, chunks * 16u);
    const rsrc_t pk = make_rsrc(p.packed, chunks);    // chunks / 4 words of 4 bytes
    const uint32_t q = (uint32_t)lane & 3u;      // this lane's place in its quad
    double s = 0.0;
    auto add4 = [&s](float x, float y, float z, float w) {
        s += fabs((double)x); s += fabs((double)y);
        s += fabs((double)z); s += fabs((double)w);
    };
    // The loop runs while the wave's first lane has chunks, so every lane takes part in the
    // quad OR; a lane past the tensor loads zeros, which add nothing to its sum (the gamma
    // pass's thread would have stopped with the same sum).
    for (uint32_t iw = (uint32_t)(part * kGammaThreads + wave * kWave); iw < chunks; iw += 8 * stride) {
        const uint32_t i = iw + lane;
        v4u v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t j = i + u * stride;
            v[u] = buf_load16_nt(wr, j < chunks ? j * 16u : kOOB);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            add4(__uint_as_float(v[u].x), __uint_as_float(v[u].y), __uint_as_float(v[u].z),
                 __uint_as_float(v[u].w));
        if (!spec)
            continue;
        // Chunk i + u * stride covers word (i + u * stride) / 4, plane q: the lane's byte
        // plane of the word; the quad OR assembles the word in all four lanes, and the quad's
        // lane q keeps the words of u = q (wa) and u = q + 4 (wb) to store.
        uint32_t wa = 0, wb = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t j = i + u * stride;
            const uint32_t x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            // Comparisons as sign bits, no compare instructions: with a = |w| and hi below 2^31,
            // hi - a is negative exactly when a > hi, lo - a when a > lo, and (lo - a) & ~(hi - a)
            // when lo < a <= hi.  Three byte permutes gather the four weights' top bytes.
            uint32_t d[4], nb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t a = x[e] & 0x7FFFFFFFu;
                d[e] = hi_bits - a;
                nb[e] = (lo_bits - a) & ~d[e];
            }
            const uint32_t dtop = top_bytes(d);                // bit 7 of byte e: |w_e| > hi
            const uint32_t xtop = top_bytes(x);                // bit 7 of byte e: w_e < 0
            const uint32_t ntop = top_bytes(nb) & 0x80808080u; // bit 7 of byte e: in the band
            // Byte e: 01 for +1, 11 for -1, 00 for 0 (code_field's fields).
            const uint32_t bits = ((dtop >> 7) & 0x01010101u) | (((dtop & xtop) >> 6) & 0x02020202u);
            const uint32_t word = quad_or(bits << (2 * q));
            if (u < 4)
                wa = q == (uint32_t)u ? word : wa;
            else
                wb = q == (uint32_t)(u - 4) ? word : wb;
            const bool list = ntop != 0 && j < chunks;
            const uint64_t mask = __ballot(list);
            if (mask) {
                const uint32_t at = listed + __builtin_amdgcn_mbcnt_hi(
                                                 (uint32_t)(mask >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                if (list) {
                    // The band's weights as a 4-bit mask (bit e of m: weight e).
                    const uint32_t m = (((ntop >> 7) * 0x01020408u) >> 24) & 15u;
                    __builtin_amdgcn_raw_buffer_store_b32((j << 4) | m, keys, (int)(at * 4u), 0, 0);
                    buf_store16(vals, at * 16u, v[u]);
                }
                listed += (uint32_t)__popcll(mask);
            }
        }
        const uint32_t ja = i - q + q * stride;               // the quad's chunks for u = q
        const uint32_t jb = ja + 4 * stride;
        __builtin_amdgcn_raw_buffer_store_b32(wa, pk, (int)(ja < chunks ? 4u * word_index(wpr, ja) : kOOB), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(wb, pk, (int)(jb < chunks ? 4u * word_index(wpr, jb) : kOOB), 0, 0);
    }
    if (spec && lane == 0)
        p.counts[wave_global] = listed;
    // The gamma pass's block sum, in its order.
    s = wave_sum_fixed(s);
    if (lane == 0)
        lds[wave] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = lds[0];
#pragma unroll
        for (int w = 1; w < kGammaThreads / kWave; ++w)
            t = t + lds[w];
        p.partials[part] = t;
    }
}

__device__ __forceinline__ void one_read_fix_block(const WeightBatch &b, int bid)
{
    int prob = 0;
#pragma unroll 1
    while (prob + 1 < b.count && bid >= b.p[prob + 1].part_begin)
        ++prob;
    const WeightDev &p = b.p[prob];
    const int part = bid - p.part_begin;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int wave_global = part * (kGammaThreads / kWave) + wave;

    // gamma and tau exactly as in quant_pack_kernel (the same partial sums, the same order).
    double part_sum = 0.0;
    {
        const rsrc_t pr = make_rsrc(p.partials, (uint32_t)p.parts * 8u);
        v2u v[kGammaParts / kWave];
#pragma unroll
        for (int k = 0; k < kGammaParts / kWave; ++k)
            v[k] = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(
                                               pr, (lane + k * kWave) * 8, 0, 0));
#pragma unroll
        for (int k = 0; k < kGammaParts / kWave; ++k)
            part_sum += __longlong_as_double((long long)(((uint64_t)v[k].y << 32) | v[k].x));
    }
    const double sum = wave_sum_fixed(part_sum);
    const double count = (double)(p.chunks * 4);
    const float gamma = p.chunks > 0 ? (float)(sum / count) : 0.0f;
    if (part == 0 && threadIdx.x == 0)
        *p.gamma = gamma;
    const float tau = code_threshold(gamma);

    const float lo = p.band[0], hi = p.band[1];
    const bool in_band = lo <= hi && lo <= tau && tau <= hi;     // block-uniform
    const uint32_t n = in_band ? p.counts[wave_global] : 0u;
    // Every wave of the block must have kept all its entries.
    const bool listed_ok = in_band && !__syncthreads_or(n > p.cap);
    if (listed_ok) {
        for (uint32_t e = lane; e < n; e += kWave) {
            const size_t slot = (size_t)wave_global * p.cap + e;
            const uint32_t key = p.keys[slot];
            const v4u v = p.vals[slot];
            const uint32_t j = key >> 4, m = key & 15u;
            const uint32_t x[4] = {v.x, v.y, v.z, v.w};
            uint32_t bits = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float f = __uint_as_float(x[k]);
                if ((m >> k) & 1u)
                    bits |= code_field(fabsf(f) > tau, f < 0.0f) << (8 * k);
            }
            if (bits)
                atomicOr(&p.packed[word_index(p.quad_wpr, j)], bits << (2 * (j & 3u)));
        }
        return;
    }
    // This block's chunks again, coded from tau.
    const uint32_t stride = (uint32_t)p.parts * kGammaThreads;
    const uint32_t chunks = (uint32_t)p.chunks;
    const rsrc_t wr = make_rsrc(p.W, chunks * 16u);
    for (uint32_t iw = (uint32_t)(part * kGammaThreads + wave * kWave); iw < chunks; iw += 8 * stride) {
        const uint32_t i = iw + lane;
        v4u v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t j = i + u * stride;
            v[u] = buf_load16_nt(wr, j < chunks ? j * 16u : kOOB);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t j = i + u * stride;
            const int sh = 2 * (int)(j & 3);
            const float vx = __uint_as_float(v[u].x), vy = __uint_as_float(v[u].y);
            const float vz = __uint_as_float(v[u].z), vw = __uint_as_float(v[u].w);
            uint32_t bits = code_field(fabsf(vx) > tau, vx < 0.0f) << (0 + sh);
            bits |= code_field(fabsf(vy) > tau, vy < 0.0f) << (8 + sh);
            bits |= code_field(fabsf(vz) > tau, vz < 0.0f) << (16 + sh);
            bits |= code_field(fabsf(vw) > tau, vw < 0.0f) << (24 + sh);
            bits = quad_or(bits);
            if (j < chunks && (j & 3) == 0)
                p.packed[word_index(p.quad_wpr, j)] = bits;
        }
    }
}

__global__ __launch_bounds__(kGammaThreads) void one_read_fix_kernel(WeightBatch b)
{
    one_read_fix_block(b, blockIdx.x);
}

size_t quantize_weights_workspace(int count)
{
    return (size_t)count * kGammaParts * sizeof(double);
}

// Tensors are processed in groups of at most group_bytes() of fp32 weights, each group as
// one gamma launch followed by one pack launch, so that the pack launch can re-read W from
// the 256 MB last-level cache (MALL) instead of HBM.  Default: one group (2 launches);
// BITLINEAR_WQ_GROUP_MB is a measurement-only knob to A/B smaller groups.
static int64_t group_bytes()
{
    static int64_t v = [] {
        const char *e = getenv("BITLINEAR_WQ_GROUP_MB");
        return e ? (int64_t)atoll(e) << 20 : (int64_t)1 << 62;
    }();
    return v;
}

// Tensors i0 .. (returned end) - 1 of one launch pair: the γ-pass blocks (parts) and the pack
// pass blocks (blocks).
static int build_weight_batch(const bl_weight_problem *q, int i0, int count, void *workspace,
                              WeightBatch &b, int &parts, int &blocks, bool quad)
{
    parts = 0;
    blocks = 0;
    int64_t bytes = 0;
    int i = i0;
    for (; i < count; ++i) {
        const int64_t tb = q[i].N * q[i].K * 4;
        if (i > i0 && bytes + tb > group_bytes())
            break;
        bytes += tb;
        WeightDev &d = b.p[b.count++];
        d.W = reinterpret_cast<const float4 *>(q[i].W);
        d.packed = q[i].W_packed;
        d.gamma = q[i].gamma;
        d.partials = static_cast<double *>(workspace) + (size_t)i * kGammaParts;
        d.chunks = q[i].N * q[i].K / 4;
        d.quad_wpr = quad ? (uint32_t)(q[i].K / 16) : 0u;
        d.parts = gamma_parts(d.chunks);
        d.part_begin = parts;
        parts += d.parts;
        const int64_t per_block = (int64_t)kPackThreads * kPackUnroll;
        int pb = (int)((d.chunks + per_block - 1) / per_block);
        if (pb == 0)
            pb = 1;  // still writes gamma (= 0 for an empty tensor)
        d.pack_begin = blocks;
        blocks += pb;
    }
    return i;
}

// ---- one-read form: workspace layout, eligibility, launches
//
// Workspace: the count * kGammaParts partial sums of the two-pass form, then per tensor (each
// piece 256-byte aligned) its sample sums, band, per-wave list counts and list.
constexpr int64_t kOneReadMinBytes = (int64_t)64 << 20;   // smaller sets keep the two passes

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct OneReadRegion {
    size_t sample, band, counts, keys, vals, end;
    uint32_t cap;
};

static OneReadRegion one_read_region(int64_t chunks, size_t at)
{
    OneReadRegion r;
    const int64_t parts = gamma_parts(chunks);
    const int64_t per_lane = (chunks + parts * kGammaThreads - 1) / (parts * kGammaThreads);
    r.cap = (uint32_t)(per_lane * kWave / kListShare + kWave);
    r.sample = at;
    at = align256(at + kSampleBlocks * 2 * sizeof(double));
    r.band = at;
    at = align256(at + 2 * sizeof(float));
    const size_t waves = (size_t)parts * (kGammaThreads / kWave);
    r.counts = at;
    at = align256(at + waves * sizeof(uint32_t));
    r.keys = at;
    at = align256(at + waves * r.cap * sizeof(uint32_t));
    r.vals = at;
    at = align256(at + waves * r.cap * sizeof(v4u));
    r.end = at;
    return r;
}

size_t quantize_weights_one_read_workspace(const bl_weight_problem *q, int count)
{
    size_t at = align256((size_t)count * kGammaParts * sizeof(double));
    for (int i = 0; i < count; ++i)
        at = one_read_region(q[i].N * q[i].K / 4, at).end;
    return at;
}

// The one-read form runs when the set is large enough for one read to pay, every tensor is
// below 2 GiB (32-bit buffer offsets, list keys) and the workspace holds its regions.
static bool one_read_eligible(const bl_weight_problem *q, int count, size_t workspace_bytes)
{
    if (count <= 0 || workspace_bytes == 0)
        return false;
    int64_t bytes = 0;
    for (int i = 0; i < count; ++i) {
        const int64_t b = q[i].N * q[i].K * 4;
        if (b >= ((int64_t)1 << 31))
            return false;
        bytes += b;
    }
    return bytes >= kOneReadMinBytes && workspace_bytes >= quantize_weights_one_read_workspace(q, count);
}

static void build_one_read_batch(const bl_weight_problem *q, int count, void *workspace,
                                 WeightBatch &b, int &sblocks, int &parts, bool quad)
{
    char *ws = static_cast<char *>(workspace);
    size_t region[BL_MAX_GROUP];
    size_t at = align256((size_t)count * kGammaParts * sizeof(double));
    for (int i = 0; i < count; ++i) {
        region[i] = at;
        at = one_read_region(q[i].N * q[i].K / 4, at).end;
    }
    // Largest tensors first in the grids (their blocks run longest); the block-to-chunk map
    // of each tensor, and so every result, does not depend on the order.
    int order[BL_MAX_GROUP];
    for (int i = 0; i < count; ++i) {
        int j = i;
        for (; j > 0 && q[order[j - 1]].N * q[order[j - 1]].K < q[i].N * q[i].K; --j)
            order[j] = order[j - 1];
        order[j] = i;
    }
    sblocks = 0;
    parts = 0;
    b.count = 0;
    for (int k = 0; k < count; ++k) {
        const int i = order[k];
        WeightDev &d = b.p[b.count++];
        d.W = reinterpret_cast<const float4 *>(q[i].W);
        d.packed = q[i].W_packed;
        d.gamma = q[i].gamma;
        d.partials = reinterpret_cast<double *>(ws) + (size_t)i * kGammaParts;
        d.chunks = q[i].N * q[i].K / 4;
        d.quad_wpr = quad ? (uint32_t)(q[i].K / 16) : 0u;
        d.parts = gamma_parts(d.chunks);
        d.part_begin = parts;
        parts += d.parts;
        d.pack_begin = 0;
        const OneReadRegion r = one_read_region(d.chunks, region[i]);
        d.sample = reinterpret_cast<double *>(ws + r.sample);
        d.band = reinterpret_cast<float *>(ws + r.band);
        d.counts = reinterpret_cast<uint32_t *>(ws + r.counts);
        d.keys = reinterpret_cast<uint32_t *>(ws + r.keys);
        d.vals = reinterpret_cast<v4u *>(ws + r.vals);
        d.cap = r.cap;
        const int64_t g = sample_groups(d.chunks);
        d.sparts = (int)(g < kSampleBlocks ? g : kSampleBlocks);
        d.sample_begin = sblocks;
        sblocks += d.sparts;
    }
}

// The pass and the fix-up (the sample has run before them on the same stream).
static hipError_t launch_one_read_fix(const WeightBatch &b, int parts, hipStream_t stream);

static hipError_t launch_one_read_passes(const WeightBatch &b, int parts, hipStream_t stream)
{
    hipLaunchKernelGGL(one_read_pass_kernel, dim3(parts), dim3(kGammaThreads), 0, stream, b);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? launch_one_read_fix(b, parts, stream) : e;
}

hipError_t launch_quantize_weights(const bl_weight_problem *q, int count, void *workspace,
                                   hipStream_t stream, bool quad, size_t workspace_bytes)
{
    if (one_read_eligible(q, count, workspace_bytes)) {
        WeightBatch b{};
        int sblocks, parts;
        build_one_read_batch(q, count, workspace, b, sblocks, parts, quad);
        if (sblocks) {
            hipLaunchKernelGGL(sample_kernel, dim3(sblocks), dim3(kGammaThreads), 0, stream, b);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
        return launch_one_read_passes(b, parts, stream);
    }
    int i0 = 0;
    while (i0 < count) {
        WeightBatch b{};
        int parts, blocks;
        i0 = build_weight_batch(q, i0, count, workspace, b, parts, blocks, quad);
        hipLaunchKernelGGL(gamma_partial_kernel, dim3(parts), dim3(kGammaThreads), 0, stream, b);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(quant_pack_kernel, dim3(blocks), dim3(kPackThreads), 0, stream, b);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// ------------------------------------------------------------------------ pack codes

__global__ __launch_bounds__(256) void pack_codes_kernel(const uint4 *codes, uint32_t *packed,
                                                          int64_t words)
{
    const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (w >= words)
        return;
    const uint4 c = codes[w];  // 16 int8 codes: k = 16w + 4q + b is byte b of component q
    const uint32_t comp[4] = {c.x, c.y, c.z, c.w};
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)  // q = plane index i (k = 16w + 4i + b)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
            word |= ((comp[q] >> (8 * bb)) & 3u) << (8 * bb + 2 * q);
    packed[w] = word;
}

hipError_t launch_pack_codes(const int8_t *codes, int64_t N, int64_t K, uint32_t *W_packed,
                             hipStream_t stream)
{
    const int64_t words = N * K / 16;
    if (words == 0)
        return hipSuccess;
    const int64_t blocks = (words + 255) / 256;
    hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint4 *>(codes), W_packed, words);
    return hipGetLastError();
}

// ------------------------------------------------------------------- quad rows

// Two-bit rows [N][K/16] -> the quad-row layout (a permutation of the same words; see
// quad_row_word): one thread per four words, which stay consecutive in both layouts.
__global__ __launch_bounds__(256) void pack_quad_rows_kernel(const uint4 *__restrict__ P,
                                                              uint4 *__restrict__ out,
                                                              uint32_t wpr, uint32_t quads)
{
    const uint32_t c = blockIdx.x * 256u + threadIdx.x;      // 16-byte chunk of the output
    if (c >= quads)
        return;
    // Output words 4c .. 4c + 3: line L = 4c / 32 (rows 4q .. 4q + 3 of stage t), row
    // 4q + i, words 8t + j .. 8t + j + 3 with i = (4c % 32) / 8, j = 4c % 8.
    const uint32_t o = 4u * c, S = wpr / 8u;
    const uint32_t L = o / 32u, i = (o % 32u) / 8u, j = o % 8u;
    const uint32_t q = L / S, t = L % S;
    out[c] = P[((4u * q + i) * wpr + 8u * t + j) / 4u];
}

hipError_t launch_pack_quad_rows(const uint32_t *P, int64_t N, int64_t K, uint32_t *out,
                                 hipStream_t stream)
{
    const int64_t quads = N * K / 64;                        // 16-byte chunks
    if (quads == 0)
        return hipSuccess;
    hipLaunchKernelGGL(pack_quad_rows_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0,
                       stream, reinterpret_cast<const uint4 *>(P), reinterpret_cast<uint4 *>(out),
                       (uint32_t)(K / 16), (uint32_t)quads);
    return hipGetLastError();
}

// ---------------------------------------------------------------- activation quant

struct ActDev {
    const void *X;
    const float *g;
    int8_t *Xq;
    float *sx;
    int M, K;
    int bf16;
    float eps;
    int row_begin;  // first row of this problem in the launch's row space
    const float *x2;  // FFN activation's second input (GLU kinds), or NULL
    int act;          // bl_act_kind
};

struct ActBatch {
    ActDev p[BL_MAX_GROUP];
    int count;
};

// Raw storage of one 16-byte group of activations (four fp32 or eight bf16 values, kept packed
// in registers and widened exactly when used).  Group j covers activations EPG*j .. +EPG-1.
template <bool BF16>
struct Group {
    static constexpr int EPG = BF16 ? 8 : 4;
    v4u v;
    __device__ __forceinline__ void load(rsrc_t r, int j) { v = buf_load16(r, (uint32_t)j * 16u); }
    // Non-temporal, for the step call's inputs (see kStepNT).
    __device__ __forceinline__ void load_nt(rsrc_t r, int j) { v = buf_load16_nt(r, (uint32_t)j * 16u); }
    // The group's values as one (fp32) or two (bf16: lo then hi) float4.
    __device__ __forceinline__ float4 f(int half) const
    {
        if (BF16) {
            const uint32_t a = half ? v.z : v.x, b = half ? v.w : v.y;
            return make_float4(__uint_as_float(a << 16), __uint_as_float(a & 0xFFFF0000u),
                               __uint_as_float(b << 16), __uint_as_float(b & 0xFFFF0000u));
        }
        return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                           __uint_as_float(v.w));
    }
};

__device__ __forceinline__ rsrc_t row_rsrc(const ActDev &p, int m)
{
    const int esize = p.bf16 ? 2 : 4;
    return make_rsrc(static_cast<const unsigned char *>(p.X) + (int64_t)m * p.K * esize,
                     (uint32_t)p.K * esize);
}

__device__ __forceinline__ float4 load_g(rsrc_t g, int j)
{
    const v4u v = buf_load16(g, (uint32_t)j * 16u);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                       __uint_as_float(v.w));
}

__device__ __forceinline__ void write_scale(const ActDev &p, int m, float a, double ss, bool norm)
{
    p.sx[m] = act_scale(a, ss, p.K, p.eps, norm);
}

template <typename T>
__device__ __forceinline__ int find_problem(const T &b, int key)
{
    int prob = 0;
#pragma unroll 1
    while (prob + 1 < b.count && key >= b.p[prob + 1].row_begin)
        ++prob;
    return prob;
}

// One wave per token row, K <= 256 * CACHE: the grid has a wave for every row and the
// hardware keeps each CU full as waves retire (a persistent grid that prefetched its next row
// measured slower: at a few rows per wave the prefetch never paid for its second register
// set).  The row's activations stay in registers (raw), the row is read from HBM once, and
// all reductions are wave-local (no LDS, no barriers).  Groups past the row load from
// outside the buffer resource (zeros).
// Lane l holds the 16-byte groups c * 64 + l (CACHE fp32 groups, or CACHE / 2 bf16 groups).
// The step call (bitlinear_quantize_step*) reads its activation rows with the non-temporal
// hint: a step's inputs are read once, and left uncached they do not evict the codes (and
// packed weights) written just before the product that reads them.  On the Qwen3-4B step,
// with the activation rows quantized last: 0.947-0.958 -> 0.909-0.927 ms.  The standalone
// activation calls keep cached loads: in the layer chain a row was written by the previous
// product and may still be in the caches (there the hint cost 969-974 -> 983-990 us per layer).
constexpr bool kStepNT = true;

template <int CACHE, bool BF16>
struct RowBuf {
    static constexpr int NG = BF16 ? CACHE / 2 : CACHE;
    Group<BF16> x[NG];
};

__device__ __forceinline__ rsrc_t act_row_rsrc(const ActBatch &b, int row, int rows, int &prob)
{
    if (row >= rows) {
        prob = 0;
        return make_rsrc(b.p[0].X, 0u);
    }
    prob = find_problem(b, row);
    return row_rsrc(b.p[prob], row - b.p[prob].row_begin);
}

template <int CACHE, bool BF16, bool NT>
__device__ __forceinline__ void act_load(RowBuf<CACHE, BF16> &r, rsrc_t xr, int lane)
{
#pragma unroll
    for (int c = 0; c < RowBuf<CACHE, BF16>::NG; ++c) {  // groups past the row read as zero
        if constexpr (NT)
            r.x[c].load_nt(xr, c * kWave + lane);
        else
            r.x[c].load(xr, c * kWave + lane);
    }
}

// RMSNorm weights of a row's problem (zeros, unused, without a norm): the fp32 quads that
// match the lane's groups.
template <int CACHE>
struct NormBuf {
    float4 g[CACHE];
};

template <int CACHE, bool BF16>
__device__ __forceinline__ void norm_load(NormBuf<CACHE> &n, const ActDev &p, int lane)
{
    const rsrc_t gr = make_rsrc(p.g, p.g ? (uint32_t)p.K * 4u : 0u);
    constexpr int H = BF16 ? 2 : 1;
#pragma unroll
    for (int c = 0; c < CACHE / H; ++c)
#pragma unroll
        for (int h = 0; h < H; ++h)
            n.g[c * H + h] = load_g(gr, (c * kWave + lane) * H + h);
}

template <int CACHE, bool BF16>
__device__ __forceinline__ void act_quant_row(const RowBuf<CACHE, BF16> &r, const NormBuf<CACHE> &n,
                                              const ActDev &p, int m, int lane)
{
    constexpr int NG = RowBuf<CACHE, BF16>::NG, H = BF16 ? 2 : 1;
    const int groups = p.K / Group<BF16>::EPG;
    const bool norm = p.g != nullptr;
    float amax = 0.0f;
    double ss = 0.0;
    float4 u[CACHE];
#pragma unroll
    for (int c = 0; c < NG; ++c)
#pragma unroll
        for (int h = 0; h < H; ++h) {
            const float4 f = r.x[c].f(h);
            u[c * H + h] = norm ? mul4(f, n.g[c * H + h]) : f;
            amax = fmaxf(amax, absmax4(u[c * H + h]));
            if (norm)
                ss = sumsq4(ss, f);  // groups past the row are zero and add nothing
        }
    const float a = wave_max(amax);
    if (norm)
        ss = wave_sum_fixed(ss);
    char4 *q4 = reinterpret_cast<char4 *>(p.Xq + (int64_t)m * p.K);
    const float inv = a == 0.0f ? 0.0f : 127.0f / a;  // correctly rounded fp32 division
#pragma unroll
    for (int c = 0; c < NG; ++c) {
        const int j = c * kWave + lane;
        if (j < groups) {
            if (BF16) {
                const char4 lo = quant4(u[2 * c], inv), hi = quant4(u[2 * c + 1], inv);
                uint2 w;
                __builtin_memcpy(&w.x, &lo, 4);
                __builtin_memcpy(&w.y, &hi, 4);
                reinterpret_cast<uint2 *>(q4)[j] = w;
            } else {
                q4[j] = quant4(u[c], inv);
            }
        }
    }
    if (lane == 0)
        write_scale(p, m, a, ss, norm);
}

template <int CACHE, bool BF16, bool NT = false>
__device__ __forceinline__ void act_wave_block(const ActBatch &b, int rows, int bid)
{
    const int lane = threadIdx.x & (kWave - 1);
    // Wave-uniform row index (readfirstlane keeps the problem lookup and the buffer
    // descriptors in scalar registers; otherwise every load is wrapped in a per-lane loop).
    const int r = bid * (kActThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (r >= rows)
        return;
    RowBuf<CACHE, BF16> A;
    NormBuf<CACHE> G;
    int pa;
    act_load<CACHE, BF16, NT>(A, act_row_rsrc(b, r, rows, pa), lane);
    norm_load<CACHE, BF16>(G, b.p[pa], lane);
    act_quant_row(A, G, b.p[pa], r - b.p[pa].row_begin, lane);
}

template <int CACHE, bool BF16, bool NT>
__global__ __launch_bounds__(kActThreads) void act_quant_wave_kernel(ActBatch b, int rows)
{
    act_wave_block<CACHE, BF16, NT>(b, rows, blockIdx.x);
}

// The γ partial sums of a weight set and the activation quantization of an input set in one
// grid: the two are independent (γ needs only W, the codes only X), so their blocks share a
// launch, γ blocks first; the pack pass follows as its own launch.  Each block runs exactly the
// code of its own kernel.
static_assert(kGammaThreads == kActThreads, "one block size for both kinds of block");
template <int CACHE, bool BF16>
__global__ __launch_bounds__(kActThreads) void gamma_act_kernel(WeightBatch wb, int gblocks, ActBatch ab,
                                                               int rows)
{
    const int bid = blockIdx.x;
    if (bid < gblocks)
        gamma_partial_block(wb, bid);
    else
        act_wave_block<CACHE, BF16, kStepNT>(ab, rows, bid - gblocks);
}

// One block per token row for rows longer than the largest wave class.  Thread t handles the
// 16-byte groups j = t + 256 c of the row (four fp32 or eight bf16 activations each); the first
// C groups per thread stay in registers between the reduction and the quantization, any
// remainder is read again (from L2).  Groups past the row load zeros.  The norm weights are
// read per group in both passes (L2 hits: every row of the problem shares them).
template <int C, bool BF16, bool NT>
__device__ __forceinline__ void act_block_body(const ActBatch &b, int bid)
{
    constexpr int EPG = BF16 ? 8 : 4;   // activations per 16-byte group
    __shared__ float lds_max[kActThreads / kWave];
    __shared__ double lds_sum[kActThreads / kWave];
    const ActDev &p = b.p[find_problem(b, bid)];
    const int m = bid - p.row_begin;
    const int groups = p.K / EPG;
    const bool norm = p.g != nullptr;
    const rsrc_t xr = row_rsrc(p, m);
    const rsrc_t gr = make_rsrc(p.g, norm ? (uint32_t)p.K * 4u : 0u);
    const int tid = threadIdx.x;

    auto widen = [&](const v4u &r, float4 &lo, float4 &hi) {
        if (BF16) {
            lo = make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u),
                             __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xFFFF0000u));
            hi = make_float4(__uint_as_float(r.z << 16), __uint_as_float(r.z & 0xFFFF0000u),
                             __uint_as_float(r.w << 16), __uint_as_float(r.w & 0xFFFF0000u));
        } else {
            lo = make_float4(__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z),
                             __uint_as_float(r.w));
            hi = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    };
    // u = x (or fl32(x * g)) for the group's activations; ss gets x^2 in element order.
    auto absmax_group = [&](const v4u &r, int j, float &amax, double &ss) {
        float4 lo, hi;
        widen(r, lo, hi);
        const uint32_t goff = j < groups ? (uint32_t)j * EPG * 4u : kOOB;
        const float4 ulo = norm ? mul4(lo, load_g(gr, (int)(goff / 16u))) : lo;
        amax = fmaxf(amax, absmax4(ulo));
        if (norm)
            ss = sumsq4(ss, lo);
        if (BF16) {
            const float4 uhi = norm ? mul4(hi, load_g(gr, (int)(goff / 16u) + 1)) : hi;
            amax = fmaxf(amax, absmax4(uhi));
            if (norm)
                ss = sumsq4(ss, hi);
        }
    };
    auto quant_group = [&](const v4u &r, int j, float inv) {
        float4 lo, hi;
        widen(r, lo, hi);
        const int gj = j * EPG / 4;
        const char4 q0 = quant4(norm ? mul4(lo, load_g(gr, gj)) : lo, inv);
        if (BF16) {
            const char4 q1 = quant4(norm ? mul4(hi, load_g(gr, gj + 1)) : hi, inv);
            char4 *dst = reinterpret_cast<char4 *>(p.Xq + (int64_t)m * p.K + (int64_t)j * EPG);
            dst[0] = q0;
            dst[1] = q1;
        } else {
            reinterpret_cast<char4 *>(p.Xq + (int64_t)m * p.K)[j] = q0;
        }
    };

    v4u raw[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int j = c * kActThreads + tid;
        raw[c] = NT ? buf_load16_nt(xr, j < groups ? (uint32_t)j * 16u : kOOB)
                    : buf_load16(xr, j < groups ? (uint32_t)j * 16u : kOOB);
    }
    float amax = 0.0f;
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < C; ++c)
        absmax_group(raw[c], c * kActThreads + tid, amax, ss);
    for (int j = C * kActThreads + tid; j < groups; j += kActThreads)
        absmax_group(buf_load16(xr, (uint32_t)j * 16u), j, amax, ss);

    // Block max (exact, order-free) and fixed-order block sum of squares.
    amax = wave_max(amax);
    if (norm)
        ss = wave_sum_fixed(ss);
    const int wave = tid / kWave;
    if ((tid & (kWave - 1)) == 0) {
        lds_max[wave] = amax;
        lds_sum[wave] = ss;
    }
    __syncthreads();
    float a = lds_max[0];
    double sum = lds_sum[0];
#pragma unroll
    for (int w = 1; w < kActThreads / kWave; ++w) {
        a = fmaxf(a, lds_max[w]);
        sum = sum + lds_sum[w];
    }

    const float inv = a == 0.0f ? 0.0f : 127.0f / a;  // correctly rounded fp32 division
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int j = c * kActThreads + tid;
        if (j < groups)
            quant_group(raw[c], j, inv);
    }
    for (int j = C * kActThreads + tid; j < groups; j += kActThreads)
        quant_group(buf_load16(xr, (uint32_t)j * 16u), j, inv);
    if (tid == 0)
        write_scale(p, m, a, sum, norm);
}

template <int C, bool BF16, bool NT>
__global__ __launch_bounds__(kActThreads) void act_quant_block_kernel(ActBatch b)
{
    act_block_body<C, BF16, NT>(b, blockIdx.x);
}

// The one-read form's fix-up beside the block kernel's activation rows (the longest rows of a
// step): blocks [0, fblocks) are fix-up blocks, the rest activation rows; each block runs
// exactly the code of its own kernel.  The fix-up's short, latency-bound blocks then run
// under the rows' stream instead of as a launch of their own.
static_assert(kGammaThreads == kActThreads, "one block size for both kinds of block");
template <int C, bool BF16>
__global__ __launch_bounds__(kActThreads) void fix_act_kernel(WeightBatch wb, int fblocks, ActBatch ab)
{
    const int bid = blockIdx.x;
    if (bid < fblocks)
        one_read_fix_block(wb, bid);
    else
        act_block_body<C, BF16, kStepNT>(ab, bid - fblocks);
}

// One block per token row of an FFN hidden state: h = act(gate, up) from two fp32 rows, then
// the same absmax (+ SubLN over h) quantization as the block kernel.  The first C groups of
// four per thread of h stay in registers between the two passes (the activation is evaluated
// once per element there); groups past them are re-read and re-evaluated (the same value).
template <int C>
__global__ __launch_bounds__(kActThreads) void act_quant_ffn_kernel(ActBatch b)
{
    __shared__ float lds_max[kActThreads / kWave];
    __shared__ double lds_sum[kActThreads / kWave];
    __shared__ double exp_tab[64];         // 2^(j/64) for ffn_act_tab
    const ActDev &p = b.p[find_problem(b, (int)blockIdx.x)];
    const int m = blockIdx.x - p.row_begin;
    const int groups = p.K / 4;
    const bool norm = p.g != nullptr;
    const int kind = p.act;
    const rsrc_t xr = row_rsrc(p, m);
    const rsrc_t x2r = make_rsrc(p.x2 ? p.x2 + (int64_t)m * p.K : p.x2, p.x2 ? (uint32_t)p.K * 4u : 0u);
    const rsrc_t gr = make_rsrc(p.g, norm ? (uint32_t)p.K * 4u : 0u);
    const int tid = threadIdx.x;

    auto f4 = [](const v4u &r) {
        return make_float4(__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z),
                           __uint_as_float(r.w));
    };
    auto h_at = [&](int j) {
        return ffn_act4_tab(kind, f4(buf_load16(xr, (uint32_t)j * 16u)),
                            f4(buf_load16(x2r, (uint32_t)j * 16u)), exp_tab);
    };
    auto absmax_group = [&](const float4 &h, int j, float &amax, double &ss) {
        const float4 u = norm ? mul4(h, load_g(gr, j < groups ? j : (int)(kOOB / 16u))) : h;
        amax = fmaxf(amax, absmax4(u));
        if (norm)
            ss = sumsq4(ss, h);
    };
    auto quant_group = [&](const float4 &h, int j, float inv) {
        reinterpret_cast<char4 *>(p.Xq + (int64_t)m * p.K)[j] =
            quant4(norm ? mul4(h, load_g(gr, j)) : h, inv);
    };

    float4 h[C];
    {
        v4u raw[C], raw2[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int j = c * kActThreads + tid;
            const uint32_t off = j < groups ? (uint32_t)j * 16u : kOOB;
            raw[c] = buf_load16(xr, off);
            raw2[c] = buf_load16(x2r, off);
        }
        // The exp table, built while the row is in flight.
        if (tid < 64)
            exp_tab[tid] = exp2((double)tid * (1.0 / 64.0));
        __syncthreads();
#pragma unroll
        for (int c = 0; c < C; ++c)
            h[c] = ffn_act4_tab(kind, f4(raw[c]), f4(raw2[c]), exp_tab);   // zeros past the row: h = 0
    }
    float amax = 0.0f;
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < C; ++c)
        absmax_group(h[c], c * kActThreads + tid, amax, ss);
    for (int j = C * kActThreads + tid; j < groups; j += kActThreads)
        absmax_group(h_at(j), j, amax, ss);

    amax = wave_max(amax);
    if (norm)
        ss = wave_sum_fixed(ss);
    const int wave = tid / kWave;
    if ((tid & (kWave - 1)) == 0) {
        lds_max[wave] = amax;
        lds_sum[wave] = ss;
    }
    __syncthreads();
    float a = lds_max[0];
    double sum = lds_sum[0];
#pragma unroll
    for (int w = 1; w < kActThreads / kWave; ++w) {
        a = fmaxf(a, lds_max[w]);
        sum = sum + lds_sum[w];
    }

    const float inv = a == 0.0f ? 0.0f : 127.0f / a;  // correctly rounded fp32 division
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int j = c * kActThreads + tid;
        if (j < groups)
            quant_group(h[c], j, inv);
    }
    for (int j = C * kActThreads + tid; j < groups; j += kActThreads)
        quant_group(h_at(j), j, inv);
    if (tid == 0)
        write_scale(p, m, a, sum, norm);
}

// Groups per thread kept in registers by the block kernel: the smallest class that holds
// the longest row of the launch (longer rows re-read the rest).
constexpr int kActBlockClasses[] = {4, 8, 16};

// Row-length classes of the wave kernel (chunks of 4 per lane): K <= 256 * class.  Longer
// rows go to the block kernel.
constexpr int kActClasses[] = {4, 8, 16};
constexpr int kActNumClasses = 3;

template <int CACHE, bool BF16, bool NT>
static void launch_wave(const ActBatch &b, int rows, hipStream_t stream)
{
    const int per_block = kActThreads / kWave;
    hipLaunchKernelGGL((act_quant_wave_kernel<CACHE, BF16, NT>), dim3((rows + per_block - 1) / per_block),
                       dim3(kActThreads), 0, stream, b, rows);
}

// Weight quantization and activation quantization of one step: the γ pass and the activation
// codes in one launch (gamma_act_kernel), then the pack pass.  Taken when every non-empty
// activation problem fits the wave kernel (K <= 4096, no FFN activation) with one dtype and
// the weights form one launch pair; otherwise the two calls' own launches.
// The wave-kernel batch of activation problems idx[0 .. n) (one dtype, bf), longest rows first
// (the row-to-block map changes nothing in the results: every row is quantized on its own).
static void build_wave_acts(const bl_act_ex_problem *aq, int *idx, int n, int bf, ActBatch &ab,
                            int &rows, int &cls)
{
    for (int i = 1; i < n; ++i)
        for (int j = i; j > 0 && aq[idx[j]].K > aq[idx[j - 1]].K; --j) {
            const int t = idx[j];
            idx[j] = idx[j - 1];
            idx[j - 1] = t;
        }
    ab.count = 0;
    rows = 0;
    cls = 0;
    for (int i = 0; i < n; ++i) {
        const bl_act_ex_problem &s = aq[idx[i]];
        const int cpl = (int)((s.K / 4 + kWave - 1) / kWave);
        int c = 0;
        while (cpl > kActClasses[c])
            ++c;
        cls = std::max(cls, c);
        ActDev &d = ab.p[ab.count++];
        d.X = s.X;
        d.g = s.norm_weight;
        d.Xq = s.X_q;
        d.sx = s.x_scale;
        d.M = (int)s.M;
        d.K = (int)s.K;
        d.bf16 = bf;
        d.eps = s.eps;
        d.row_begin = rows;
        d.x2 = nullptr;
        d.act = BL_ACT_NONE;
        rows += d.M;
    }
}

// One launch: `wblocks` γ-pass blocks and then the wave-kernel activation blocks.
static hipError_t launch_weight_act(const WeightBatch &wb, int wblocks, const ActBatch &ab, int rows,
                                    int cls, int bf, hipStream_t stream)
{
    const dim3 grid((unsigned)(wblocks + (rows + kActThreads / kWave - 1) / (kActThreads / kWave)));
    if (bf) {
        if (cls == 0) hipLaunchKernelGGL((gamma_act_kernel<4, true>), grid, dim3(kActThreads), 0, stream, wb, wblocks, ab, rows);
        else if (cls == 1) hipLaunchKernelGGL((gamma_act_kernel<8, true>), grid, dim3(kActThreads), 0, stream, wb, wblocks, ab, rows);
        else hipLaunchKernelGGL((gamma_act_kernel<16, true>), grid, dim3(kActThreads), 0, stream, wb, wblocks, ab, rows);
    } else {
        if (cls == 0) hipLaunchKernelGGL((gamma_act_kernel<4, false>), grid, dim3(kActThreads), 0, stream, wb, wblocks, ab, rows);
        else if (cls == 1) hipLaunchKernelGGL((gamma_act_kernel<8, false>), grid, dim3(kActThreads), 0, stream, wb, wblocks, ab, rows);
        else hipLaunchKernelGGL((gamma_act_kernel<16, false>), grid, dim3(kActThreads), 0, stream, wb, wblocks, ab, rows);
    }
    return hipGetLastError();
}

static hipError_t launch_one_read_fix(const WeightBatch &b, int parts, hipStream_t stream)
{
    hipLaunchKernelGGL(one_read_fix_kernel, dim3(parts), dim3(kGammaThreads), 0, stream, b);
    return hipGetLastError();
}

// The fix-up's `parts` blocks and the block kernel's rows of q[0 .. n) (every row longer than
// 4096 values, one dtype bf) in one launch, longest rows first.
static hipError_t launch_fix_acts(const WeightBatch &wb, int parts, const bl_act_ex_problem *q, int n,
                                  int bf, hipStream_t stream)
{
    int order[BL_MAX_GROUP];
    for (int i = 0; i < n; ++i) {
        int j = i;
        for (; j > 0 && q[order[j - 1]].K < q[i].K; --j)
            order[j] = order[j - 1];
        order[j] = i;
    }
    ActBatch ab{};
    int rows = 0, gpt = 0;   // gpt: 16-byte groups per thread of the longest row
    for (int i = 0; i < n; ++i) {
        const bl_act_ex_problem &s = q[order[i]];
        ActDev &d = ab.p[ab.count++];
        d.X = s.X;
        d.g = s.norm_weight;
        d.Xq = s.X_q;
        d.sx = s.x_scale;
        d.M = (int)s.M;
        d.K = (int)s.K;
        d.bf16 = bf;
        d.eps = s.eps;
        d.row_begin = rows;
        d.x2 = nullptr;
        d.act = BL_ACT_NONE;
        rows += d.M;
        gpt = std::max(gpt, (int)((s.K / (bf ? 8 : 4) + kActThreads - 1) / kActThreads));
    }
    const dim3 grid((unsigned)(parts + rows));
    if (bf) {
        if (gpt <= kActBlockClasses[0])
            hipLaunchKernelGGL((fix_act_kernel<kActBlockClasses[0], true>), grid, dim3(kActThreads), 0, stream, wb, parts, ab);
        else if (gpt <= kActBlockClasses[1])
            hipLaunchKernelGGL((fix_act_kernel<kActBlockClasses[1], true>), grid, dim3(kActThreads), 0, stream, wb, parts, ab);
        else
            hipLaunchKernelGGL((fix_act_kernel<kActBlockClasses[2], true>), grid, dim3(kActThreads), 0, stream, wb, parts, ab);
    } else {
        if (gpt <= kActBlockClasses[0])
            hipLaunchKernelGGL((fix_act_kernel<kActBlockClasses[0], false>), grid, dim3(kActThreads), 0, stream, wb, parts, ab);
        else if (gpt <= kActBlockClasses[1])
            hipLaunchKernelGGL((fix_act_kernel<kActBlockClasses[1], false>), grid, dim3(kActThreads), 0, stream, wb, parts, ab);
        else
            hipLaunchKernelGGL((fix_act_kernel<kActBlockClasses[2], false>), grid, dim3(kActThreads), 0, stream, wb, parts, ab);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_step(const bl_weight_problem *wq, int nw, void *workspace,
                                size_t workspace_bytes, const bl_act_ex_problem *aq, int na,
                                hipStream_t stream, bool quad)
{
    int order[BL_MAX_GROUP];
    int n = 0, bf = -1;
    if (one_read_eligible(wq, nw, workspace_bytes)) {
        // One read of W: the sample, the pass, then the fix-up sharing a launch with the
        // activation rows the block kernel takes (longer than 4096 values, one dtype), and the
        // other activation rows last.  The codes are then written right before the product
        // that reads them, while the last-level cache still holds them: on the Qwen3-4B set
        // the product ran 7 us faster than with the activation rows ahead of the weight pass.
        WeightBatch wb{};
        int sblocks, parts;
        build_one_read_batch(wq, nw, workspace, wb, sblocks, parts, quad);
        bl_act_ex_problem wide[BL_MAX_GROUP], other[BL_MAX_GROUP];
        int nwide = 0, nother = 0, wbf = -1;
        for (int i = 0; i < na; ++i) {
            if (aq[i].M == 0)
                continue;
            const int cpl = (int)((aq[i].K / 4 + kWave - 1) / kWave);
            const int dt = aq[i].x_dtype == BL_BF16 ? 1 : 0;
            if (aq[i].act == BL_ACT_NONE && cpl > kActClasses[kActNumClasses - 1] && (wbf < 0 || wbf == dt)) {
                wbf = dt;
                wide[nwide++] = aq[i];
            } else {
                other[nother++] = aq[i];
            }
        }
        hipError_t e = hipSuccess;
        if (sblocks) {
            hipLaunchKernelGGL(sample_kernel, dim3(sblocks), dim3(kGammaThreads), 0, stream, wb);
            e = hipGetLastError();
        }
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(one_read_pass_kernel, dim3(parts), dim3(kGammaThreads), 0, stream, wb);
        e = hipGetLastError();
        if (e == hipSuccess)
            e = nwide ? launch_fix_acts(wb, parts, wide, nwide, wbf, stream)
                      : launch_one_read_fix(wb, parts, stream);
        if (e == hipSuccess && nother)
            e = launch_quantize_acts(other, nother, stream, kStepNT);
        return e;
    }
    bool ok = nw > 0;
    for (int i = 0; i < na && ok; ++i) {
        if (aq[i].M == 0)
            continue;
        const int cpl = (int)((aq[i].K / 4 + kWave - 1) / kWave);
        const int dt = aq[i].x_dtype == BL_BF16 ? 1 : 0;
        ok = aq[i].act == BL_ACT_NONE && cpl <= kActClasses[kActNumClasses - 1] && (bf < 0 || bf == dt);
        bf = dt;
        order[n++] = i;
    }
    WeightBatch wb{};
    int parts = 0, blocks = 0;
    ok = ok && n > 0 && build_weight_batch(wq, 0, nw, workspace, wb, parts, blocks, quad) == nw;
    if (!ok) {
        const hipError_t e = launch_quantize_weights(wq, nw, workspace, stream, quad, 0);
        return e == hipSuccess ? launch_quantize_acts(aq, na, stream, kStepNT) : e;
    }
    ActBatch ab{};
    int rows, cls;
    build_wave_acts(aq, order, n, bf, ab, rows, cls);
    hipError_t e = launch_weight_act(wb, parts, ab, rows, cls, bf, stream);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(quant_pack_kernel, dim3(blocks), dim3(kPackThreads), 0, stream, wb);
    return hipGetLastError();
}

template <bool NT>
static hipError_t launch_acts(const bl_act_ex_problem *q, int count, hipStream_t stream)
{
    // Problems with rows up to 4096 share one wave-kernel launch per dtype, sized by their
    // longest row (shorter rows load zeros past their end); longer rows use the block kernel.
    // Longest rows first inside a launch.
    int order[BL_MAX_GROUP];
    int n = 0;
    for (int i = 0; i < count; ++i)
        if (q[i].M > 0 && q[i].act == BL_ACT_NONE)
            order[n++] = i;
    for (int i = 1; i < n; ++i)
        for (int j = i; j > 0 && q[order[j]].K > q[order[j - 1]].K; --j) {
            const int t = order[j];
            order[j] = order[j - 1];
            order[j - 1] = t;
        }
    for (int wide = 0; wide < 2; ++wide) {
        for (int bf = 0; bf < 2; ++bf) {
            ActBatch b{};
            int rows = 0, cls = 0;
            for (int i = 0; i < n; ++i) {
                const bl_act_ex_problem &s = q[order[i]];
                const int cpl = (int)((s.K / 4 + kWave - 1) / kWave);  // chunks per lane
                int c = 0;
                while (c < kActNumClasses && cpl > kActClasses[c])
                    ++c;
                if ((c == kActNumClasses) != (wide == 1) || (s.x_dtype == BL_BF16) != (bf == 1))
                    continue;
                if (c > cls)
                    cls = c;
                ActDev &d = b.p[b.count++];
                d.X = s.X;
                d.g = s.norm_weight;
                d.Xq = s.X_q;
                d.sx = s.x_scale;
                d.M = (int)s.M;
                d.K = (int)s.K;
                d.bf16 = bf;
                d.eps = s.eps;
                d.row_begin = rows;
                d.x2 = nullptr;
                d.act = BL_ACT_NONE;
                rows += d.M;
            }
            if (!rows)
                continue;
            if (wide) {
                int gpt = 0;   // 16-byte groups per thread of the longest row
                for (int i = 0; i < b.count; ++i) {
                    const int groups = b.p[i].K / (bf ? 8 : 4);
                    gpt = std::max(gpt, (groups + kActThreads - 1) / kActThreads);
                }
                if (bf) {
                    if (gpt <= kActBlockClasses[0])
                        hipLaunchKernelGGL((act_quant_block_kernel<kActBlockClasses[0], true, NT>), dim3(rows), dim3(kActThreads), 0, stream, b);
                    else if (gpt <= kActBlockClasses[1])
                        hipLaunchKernelGGL((act_quant_block_kernel<kActBlockClasses[1], true, NT>), dim3(rows), dim3(kActThreads), 0, stream, b);
                    else
                        hipLaunchKernelGGL((act_quant_block_kernel<kActBlockClasses[2], true, NT>), dim3(rows), dim3(kActThreads), 0, stream, b);
                } else {
                    if (gpt <= kActBlockClasses[0])
                        hipLaunchKernelGGL((act_quant_block_kernel<kActBlockClasses[0], false, NT>), dim3(rows), dim3(kActThreads), 0, stream, b);
                    else if (gpt <= kActBlockClasses[1])
                        hipLaunchKernelGGL((act_quant_block_kernel<kActBlockClasses[1], false, NT>), dim3(rows), dim3(kActThreads), 0, stream, b);
                    else
                        hipLaunchKernelGGL((act_quant_block_kernel<kActBlockClasses[2], false, NT>), dim3(rows), dim3(kActThreads), 0, stream, b);
                }
            } else if (bf) {
                if (cls == 0) launch_wave<4, true, NT>(b, rows, stream);
                else if (cls == 1) launch_wave<8, true, NT>(b, rows, stream);
                else launch_wave<16, true, NT>(b, rows, stream);
            } else {
                if (cls == 0) launch_wave<4, false, NT>(b, rows, stream);
                else if (cls == 1) launch_wave<8, false, NT>(b, rows, stream);
                else launch_wave<16, false, NT>(b, rows, stream);
            }
            hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
    }
    // Problems with an FFN activation: one block-kernel launch (fp32 inputs).
    {
        ActBatch b{};
        int rows = 0, gpt = 0;
        for (int i = 0; i < count; ++i) {
            const bl_act_ex_problem &s = q[i];
            if (s.M == 0 || s.act == BL_ACT_NONE)
                continue;
            ActDev &d = b.p[b.count++];
            d.X = s.X;
            d.g = s.norm_weight;
            d.Xq = s.X_q;
            d.sx = s.x_scale;
            d.M = (int)s.M;
            d.K = (int)s.K;
            d.bf16 = 0;
            d.eps = s.eps;
            d.row_begin = rows;
            d.x2 = s.X2;
            d.act = s.act;
            rows += d.M;
            gpt = std::max(gpt, (int)((s.K / 4 + kActThreads - 1) / kActThreads));
        }
        if (rows) {
            if (gpt <= 4)
                hipLaunchKernelGGL((act_quant_ffn_kernel<4>), dim3(rows), dim3(kActThreads), 0, stream, b);
            else
                hipLaunchKernelGGL((act_quant_ffn_kernel<12>), dim3(rows), dim3(kActThreads), 0, stream, b);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
    }
    return hipSuccess;
}

hipError_t launch_quantize_acts(const bl_act_ex_problem *q, int count, hipStream_t stream, bool nt)
{
    return nt ? launch_acts<true>(q, count, stream) : launch_acts<false>(q, count, stream);
}

// Two-bit packed rows -> base-3 rows (five codes per byte, 80 weights per 16-byte block; byte
// b of block j holds weights 80j + 4b + i, i = 0..3, and 80j + 64 + b as sum_i (c + 1) * 3^i).
// One thread per output block, which reads input words 5j .. 5j+4 (word 5j + w holds weights
// 80j + 16w .. +15); words past the row are padding (code 0).
__global__ __launch_bounds__(256) void pack_b3_kernel(const uint32_t *P, int K, uint8_t *out,
                                                      int64_t total)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= total)
        return;
    const int bpr = (K + 79) / 80, words = K / 16;
    const int64_t n = t / bpr;
    const int j = (int)(t % bpr);
    uint32_t w[5];
#pragma unroll
    for (int i = 0; i < 5; ++i)
        w[i] = 5 * j + i < words ? P[n * words + 5 * j + i] : 0u;
    v4u o = v4u{0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 16; ++b) {
        uint32_t v = 0, pw = 1;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int k = i < 4 ? 4 * b + i : 64 + b;          // weight within the block
            const int kk = k & 15;                              // = 4 * plane + byte in its word
            const uint32_t f = (w[k >> 4] >> (8 * (kk & 3) + 2 * (kk >> 2))) & 3u;   // 00, 01, 11
            v += ((f + 1u) & 3u) * pw;                          // digit c + 1
            pw *= 3u;
        }
        o[b >> 2] |= v << (8 * (b & 3));
    }
    *reinterpret_cast<v4u *>(out + n * 16 * bpr + 16 * j) = o;
}

hipError_t launch_pack_b3(const uint32_t *P, int64_t N, int64_t K, uint8_t *out, hipStream_t stream)
{
    const int64_t total = N * ((K + 79) / 80);
    if (total == 0)
        return hipSuccess;
    hipLaunchKernelGGL(pack_b3_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       P, (int)K, out, total);
    return hipGetLastError();
}

}  // namespace bl
