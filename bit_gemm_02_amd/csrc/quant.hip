// quant.hip — weight scale, ternary quantize-and-pack, code packing and int8 activation
// quantization kernels for gfx950.
//
// Weight path (Distillix README, "1. BitNet b1.58 Core": W_q = round(clip(W / mean|W|, -1, 1));
// bitone README, "Features": gamma from a separate one-dimensional reduction over W, and the
// quantized weights never materialized in HBM):
//   gamma_partial_kernel  reads W once, writes kGammaParts fp64 partial sums per tensor;
//   quant_pack_kernel     reduces the partials (same fixed order in every block, so every
//                         block sees the same gamma), reads W again and writes packed words.
//
// Activation path (BitDistill article: INT8 activations, SubLN before the attention and FFN
// output projections; SLM750-Edge card: RMSNorm epsilon 1e-6):
//   act_quant_wave_kernel   one wave per token row (K <= 4096), row held in registers;
//   act_quant_block_kernel  one block per token row for longer rows;
//   both: absmax (+ fixed-order sum of squares for the norm), then q = rint(u * (127 / a))
//   and the row scale.
//
// Rounding-sensitive arithmetic is written so that it matches IEEE-754 fp32 semantics:
// the library is built with -ffp-contract=off, fp32 division is correctly rounded (the HIP
// default), and rintf lowers to round-to-nearest-even.
#include "common.hpp"

namespace bl {

constexpr int kGammaParts = 256;    // partial sums per tensor; fixed, so the order is fixed
constexpr int kGammaThreads = 512;
constexpr int kPackThreads = 256;
constexpr int kPackUnroll = 8;      // float4 chunks per thread in quant_pack_kernel
constexpr int kActThreads = 256;
constexpr int kActCache = 16;       // 4-element chunks per thread kept in registers (block kernel)

// ----------------------------------------------------------------------------- gamma

struct WeightDev {
    const float4 *W;
    uint32_t *packed;
    float *gamma;
    double *partials;   // [kGammaParts]
    int64_t chunks;     // N * K / 4 float4 chunks
    int pack_blocks;    // blocks of quant_pack_kernel for this tensor
    int pack_begin;     // first block of this tensor in quant_pack_kernel's grid
};

struct WeightBatch {
    WeightDev p[BL_MAX_GROUP];
    int count;
};

// Block sum of one fp64 value per thread in a fixed order (wave butterfly, then waves in
// index order).  Result valid in every thread.
template <int THREADS>
__device__ __forceinline__ double block_sum_fixed(double v, double *lds)
{
    constexpr int W = THREADS / kWave;
    v = wave_sum_fixed(v);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0)
        lds[wave] = v;
    __syncthreads();
    double s = lds[0];
#pragma unroll
    for (int i = 1; i < W; ++i)
        s = s + lds[i];
    __syncthreads();
    return s;
}

__global__ __launch_bounds__(kGammaThreads) void gamma_partial_kernel(WeightBatch b)
{
    __shared__ double lds[kGammaThreads / kWave];
    const int prob = blockIdx.x / kGammaParts;
    const int part = blockIdx.x % kGammaParts;
    const WeightDev &p = b.p[prob];
    const int64_t stride = (int64_t)kGammaParts * kGammaThreads;
    double s = 0.0;
    int64_t i = (int64_t)part * kGammaThreads + threadIdx.x;
    // Four loads in flight per thread; the additions stay in index order.
    for (; i + 3 * stride < p.chunks; i += 4 * stride) {
        float4 v0 = p.W[i], v1 = p.W[i + stride], v2 = p.W[i + 2 * stride],
               v3 = p.W[i + 3 * stride];
        s += fabs((double)v0.x); s += fabs((double)v0.y);
        s += fabs((double)v0.z); s += fabs((double)v0.w);
        s += fabs((double)v1.x); s += fabs((double)v1.y);
        s += fabs((double)v1.z); s += fabs((double)v1.w);
        s += fabs((double)v2.x); s += fabs((double)v2.y);
        s += fabs((double)v2.z); s += fabs((double)v2.w);
        s += fabs((double)v3.x); s += fabs((double)v3.y);
        s += fabs((double)v3.z); s += fabs((double)v3.w);
    }
    for (; i < p.chunks; i += stride) {
        float4 v = p.W[i];
        s += fabs((double)v.x); s += fabs((double)v.y);
        s += fabs((double)v.z); s += fabs((double)v.w);
    }
    s = block_sum_fixed<kGammaThreads>(s, lds);
    if (threadIdx.x == 0)
        p.partials[part] = s;
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

__global__ __launch_bounds__(kPackThreads) void quant_pack_kernel(WeightBatch b)
{
    __shared__ double lds[kPackThreads / kWave];
    int prob = 0;
#pragma unroll 1
    while (prob + 1 < b.count && (int)blockIdx.x >= b.p[prob + 1].pack_begin)
        ++prob;
    const WeightDev &p = b.p[prob];
    const int blk = blockIdx.x - p.pack_begin;

    // gamma = fl32(sum / count), the partial sums reduced in the same order in every block.
    double part = 0.0;
    for (int i = threadIdx.x; i < kGammaParts; i += kPackThreads)
        part += p.partials[i];
    const double sum = block_sum_fixed<kPackThreads>(part, lds);
    const double count = (double)(p.chunks * 4);
    const float gamma = p.chunks > 0 ? (float)(sum / count) : 0.0f;
    if (blk == 0 && threadIdx.x == 0)
        *p.gamma = gamma;
    const float tau = code_threshold(gamma);

    // Each lane turns 4 consecutive weights (one float4) into its plane of a packed word:
    // chunk j covers k = 4j .. 4j + 3, i.e. word j / 4, plane i = j % 4, bytes b = 0..3.
    // The four lanes of a quad hold the four planes of one word and OR them together.
    // All loads first (out-of-range chunks of the last block read as zero), then the codes.
    const int64_t base = (int64_t)blk * kPackThreads * kPackUnroll;
    const int64_t live = p.chunks - base < kPackThreads * kPackUnroll ? p.chunks - base
                                                                       : kPackThreads * kPackUnroll;
    const rsrc_t wres = make_rsrc(p.W + base, live > 0 ? (uint32_t)live * 16u : 0u);
    v4u raw[kPackUnroll];
#pragma unroll
    for (int u = 0; u < kPackUnroll; ++u)
        raw[u] = buf_load16(wres, (uint32_t)(u * kPackThreads + threadIdx.x) * 16u);
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
            p.packed[j >> 2] = bits;
    }
}

size_t quantize_weights_workspace(int count)
{
    return (size_t)count * kGammaParts * sizeof(double);
}

hipError_t launch_quantize_weights(const bl_weight_problem *q, int count, void *workspace,
                                   hipStream_t stream)
{
    WeightBatch b{};
    b.count = count;
    int blocks = 0;
    for (int i = 0; i < count; ++i) {
        WeightDev &d = b.p[i];
        d.W = reinterpret_cast<const float4 *>(q[i].W);
        d.packed = q[i].W_packed;
        d.gamma = q[i].gamma;
        d.partials = static_cast<double *>(workspace) + (size_t)i * kGammaParts;
        d.chunks = q[i].N * q[i].K / 4;
        const int64_t per_block = (int64_t)kPackThreads * kPackUnroll;
        d.pack_blocks = (int)((d.chunks + per_block - 1) / per_block);
        if (d.pack_blocks == 0)
            d.pack_blocks = 1;  // still writes gamma (= 0 for an empty tensor)
        d.pack_begin = blocks;
        blocks += d.pack_blocks;
    }
    hipLaunchKernelGGL(gamma_partial_kernel, dim3(count * kGammaParts), dim3(kGammaThreads), 0,
                       stream, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(quant_pack_kernel, dim3(blocks), dim3(kPackThreads), 0, stream, b);
    return hipGetLastError();
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

// ---------------------------------------------------------------- activation quant

struct ActDev {
    const void *X;
    const float *g;
    int8_t *Xq;
    float *sx;
    int M, K;
    int bf16;
    float eps;
    int row_begin;  // first block (row) of this problem in the grid
};

struct ActBatch {
    ActDev p[BL_MAX_GROUP];
    int count;
};

// Chunk j (4 activations) of a row through the row's buffer resource: fp32 rows use 16-byte
// loads, bf16 rows 8-byte loads widened exactly to fp32.  Chunks past the row read as zero.
__device__ __forceinline__ float4 load_chunk(rsrc_t row, int bf16, int j)
{
    if (bf16) {
        const uint32_t lo = buf_load4(row, (uint32_t)j * 8u);
        const uint32_t hi = buf_load4(row, (uint32_t)j * 8u + 4u);
        return make_float4(__uint_as_float(lo << 16), __uint_as_float(lo & 0xFFFF0000u),
                           __uint_as_float(hi << 16), __uint_as_float(hi & 0xFFFF0000u));
    }
    const v4u v = buf_load16(row, (uint32_t)j * 16u);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                       __uint_as_float(v.w));
}

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

__device__ __forceinline__ int8_t quant_one(float u, float inv)
{
    const float v = __builtin_rintf(u * inv);  // fp32 product, round half to even
    if (v > 127.0f)
        return 127;
    if (v < -127.0f)
        return -127;
    if (v != v)
        return 0;
    return (int8_t)(int)v;
}

// Quantize one row given its absmax a: q = clamp(rint(u * fl32(127 / a))).
__device__ __forceinline__ char4 quant4(float4 u, float inv)
{
    return make_char4(quant_one(u.x, inv), quant_one(u.y, inv), quant_one(u.z, inv),
                      quant_one(u.w, inv));
}

__device__ __forceinline__ float4 mul4(float4 a, float4 b)
{
    return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}

__device__ __forceinline__ float absmax4(float4 u)
{
    return fmaxf(fmaxf(fabsf(u.x), fabsf(u.y)), fmaxf(fabsf(u.z), fabsf(u.w)));
}

__device__ __forceinline__ double sumsq4(double s, float4 x)
{
    s += (double)x.x * (double)x.x;
    s += (double)x.y * (double)x.y;
    s += (double)x.z * (double)x.z;
    s += (double)x.w * (double)x.w;
    return s;
}

__device__ __forceinline__ void write_scale(const ActDev &p, int m, float a, double ss, bool norm)
{
    if (a == 0.0f) {
        p.sx[m] = 0.0f;
    } else if (!norm) {
        p.sx[m] = a / 127.0f;  // correctly rounded fp32 division
    } else {
        const double r = 1.0 / sqrt(ss / (double)p.K + (double)p.eps);
        p.sx[m] = (float)((double)a * r / 127.0);
    }
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

// One wave per token row, for K <= 256 * CACHE: each lane keeps its CACHE chunks of 4
// activations in registers, so the row is read from HBM once; reductions are wave-local
// (no LDS, no barriers).  Four rows per block.
template <int CACHE>
__global__ __launch_bounds__(kActThreads) void act_quant_wave_kernel(ActBatch b, int rows)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int grow = blockIdx.x * (kActThreads / kWave) + threadIdx.x / kWave;
    if (grow >= rows)
        return;
    const ActDev &p = b.p[find_problem(b, grow)];
    const int m = grow - p.row_begin;
    const int chunks = p.K / 4;
    const bool norm = p.g != nullptr;
    const rsrc_t xr = row_rsrc(p, m);
    const rsrc_t gr = make_rsrc(p.g, norm ? (uint32_t)p.K * 4u : 0u);

    float4 x[CACHE], u[CACHE];
#pragma unroll
    for (int c = 0; c < CACHE; ++c)
        x[c] = load_chunk(xr, p.bf16, c * kWave + lane);
    float amax = 0.0f;
    double ss = 0.0;
    if (norm) {
#pragma unroll
        for (int c = 0; c < CACHE; ++c) {
            u[c] = mul4(x[c], load_g(gr, c * kWave + lane));
            amax = fmaxf(amax, absmax4(u[c]));
            ss = sumsq4(ss, x[c]);   // chunks past the row are zero and add nothing
        }
    } else {
#pragma unroll
        for (int c = 0; c < CACHE; ++c) {
            u[c] = x[c];
            amax = fmaxf(amax, absmax4(u[c]));
        }
    }
    const float a = wave_max(amax);
    if (norm)
        ss = wave_sum_fixed(ss);
    char4 *q4 = reinterpret_cast<char4 *>(p.Xq) + (int64_t)m * chunks;
    const float inv = a == 0.0f ? 0.0f : 127.0f / a;  // correctly rounded fp32 division
#pragma unroll
    for (int c = 0; c < CACHE; ++c) {
        const int j = c * kWave + lane;
        if (j < chunks)
            q4[j] = quant4(u[c], inv);
    }
    if (lane == 0)
        write_scale(p, m, a, ss, norm);
}

// One block per token row for long rows (K > 4096): the first kActCache chunks per thread
// stay in registers, any remainder is read again (from L2) in the second pass.
__global__ __launch_bounds__(kActThreads) void act_quant_block_kernel(ActBatch b)
{
    __shared__ float lds_max[kActThreads / kWave];
    __shared__ double lds_sum[kActThreads / kWave];
    const ActDev &p = b.p[find_problem(b, (int)blockIdx.x)];
    const int m = blockIdx.x - p.row_begin;
    const int chunks = p.K / 4;
    const bool norm = p.g != nullptr;
    const rsrc_t xr = row_rsrc(p, m);
    const rsrc_t gr = make_rsrc(p.g, norm ? (uint32_t)p.K * 4u : 0u);

    float4 cache[kActCache];
#pragma unroll
    for (int c = 0; c < kActCache; ++c)
        cache[c] = load_chunk(xr, p.bf16, c * kActThreads + threadIdx.x);
    float amax = 0.0f;
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < kActCache; ++c) {
        const int j = c * kActThreads + threadIdx.x;
        amax = fmaxf(amax, absmax4(norm ? mul4(cache[c], load_g(gr, j)) : cache[c]));
        if (norm)
            ss = sumsq4(ss, cache[c]);
    }
    for (int j = kActCache * kActThreads + threadIdx.x; j < chunks; j += kActThreads) {
        const float4 x = load_chunk(xr, p.bf16, j);
        amax = fmaxf(amax, absmax4(norm ? mul4(x, load_g(gr, j)) : x));
        if (norm)
            ss = sumsq4(ss, x);
    }

    // Block max (exact, order-free) and fixed-order block sum of squares.
    amax = wave_max(amax);
    if (norm)
        ss = wave_sum_fixed(ss);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
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

    char4 *q4 = reinterpret_cast<char4 *>(p.Xq) + (int64_t)m * chunks;
    const float inv = a == 0.0f ? 0.0f : 127.0f / a;  // correctly rounded fp32 division
#pragma unroll
    for (int c = 0; c < kActCache; ++c) {
        const int j = c * kActThreads + threadIdx.x;
        if (j < chunks)
            q4[j] = quant4(norm ? mul4(cache[c], load_g(gr, j)) : cache[c], inv);
    }
    for (int j = kActCache * kActThreads + threadIdx.x; j < chunks; j += kActThreads) {
        const float4 x = load_chunk(xr, p.bf16, j);
        q4[j] = quant4(norm ? mul4(x, load_g(gr, j)) : x, inv);
    }
    if (threadIdx.x == 0)
        write_scale(p, m, a, sum, norm);
}

hipError_t launch_quantize_acts(const bl_act_problem *q, int count, hipStream_t stream)
{
    // Rows up to 4096 wide go to the wave-per-row kernel, longer rows to the block kernel.
    ActBatch wave_b{}, block_b{};
    int wave_rows = 0, block_rows = 0, max_wave_k = 0;
    for (int i = 0; i < count; ++i) {
        if (q[i].M == 0)
            continue;
        const bool wide = q[i].K > 4096;
        ActBatch &b = wide ? block_b : wave_b;
        int &rows = wide ? block_rows : wave_rows;
        ActDev &d = b.p[b.count++];
        d.X = q[i].X;
        d.g = q[i].norm_weight;
        d.Xq = q[i].X_q;
        d.sx = q[i].x_scale;
        d.M = (int)q[i].M;
        d.K = (int)q[i].K;
        d.bf16 = q[i].x_dtype == BL_BF16;
        d.eps = q[i].eps;
        d.row_begin = rows;
        rows += d.M;
        if (!wide && d.K > max_wave_k)
            max_wave_k = d.K;
    }
    if (wave_rows) {
        const int per_block = kActThreads / kWave;
        const dim3 grid((wave_rows + per_block - 1) / per_block);
        if (max_wave_k <= 1024)
            hipLaunchKernelGGL(act_quant_wave_kernel<4>, grid, dim3(kActThreads), 0, stream, wave_b, wave_rows);
        else if (max_wave_k <= 2048)
            hipLaunchKernelGGL(act_quant_wave_kernel<8>, grid, dim3(kActThreads), 0, stream, wave_b, wave_rows);
        else
            hipLaunchKernelGGL(act_quant_wave_kernel<16>, grid, dim3(kActThreads), 0, stream, wave_b, wave_rows);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (block_rows) {
        hipLaunchKernelGGL(act_quant_block_kernel, dim3(block_rows), dim3(kActThreads), 0, stream, block_b);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace bl
