// prefill.hip — ternary x int8 product for many tokens (M > 16): the prefill path.
//
// With hundreds of tokens the product is a dense contraction (2 M N K integer operations;
// zeros are multiplied, the method computes the dense ternary product), so it belongs on the
// int8 matrix cores: v_mfma_i32_16x16x64_i8.  bitone README, "Features": the quantized
// weights stay in on-chip memory inside the GEMM and are never materialized in HBM; here the
// packed 2-bit words go straight from global memory into registers and are expanded there
// (plane64: one shift and one mask per four weights, giving 64 * c as int8), while the int8
// activations are staged through LDS because every wave of the block reads them.
//
// Block tile 128 (tokens) x 128 (weight rows); 4 waves in a 2 x 2 arrangement, each owning a
// 64 x 64 sub-tile = 4 x 4 MFMA tiles.  The K loop advances in super-steps of 256 weights
// (16 packed words per row): lane (r = l % 16, g = l / 16) loads words 4g .. 4g+3 of its
// weight row with one 16-byte load and uses word 4g + j in MFMA j; the matching activation
// bytes 16 (4g + j) .. +15 of its token row come from LDS with one 16-byte read.  The next
// super-step's activations and weights are loaded into registers while the current one is
// computed, and LDS is double-buffered, so one barrier per super-step suffices.
// Epilogue: y = fl32(fp64(acc * gamma * s_x[m])), acc = (MFMA sum) / 64 (exact shift).
#include "common.hpp"

namespace bl {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kPreThreads = 256;
constexpr int kSuper = 256;                 // weights (k) per super-step
constexpr int kXRow = kSuper + 16;          // LDS bytes per token row (16 B pad: no conflicts)
constexpr int kXStage = kBM * kXRow;        // bytes per LDS buffer
constexpr int kXLoads = kBM * kSuper / 16 / kPreThreads;  // 16-byte loads per thread per stage

struct PreDev {
    const int8_t *Xq;
    const float *sx;
    const uint32_t *W;
    const float *gamma;
    float *Y;
    int32_t *acc;
    int M, N, K;
    int tiles_n;
    int block_begin;
};

struct PreBatch {
    PreDev p[BL_MAX_GROUP];
    int count;
};

__device__ __forceinline__ uint4 load_w4(const uint32_t *row, int w, int words, bool aligned)
{
    if (aligned && w + 3 < words)
        return *reinterpret_cast<const uint4 *>(row + w);
    uint4 r;
    r.x = w + 0 < words ? row[w + 0] : 0u;
    r.y = w + 1 < words ? row[w + 1] : 0u;
    r.z = w + 2 < words ? row[w + 2] : 0u;
    r.w = w + 3 < words ? row[w + 3] : 0u;
    return r;
}

__global__ __launch_bounds__(kPreThreads) void prefill_kernel(PreBatch b)
{
    __shared__ __align__(16) unsigned char smem[2 * kXStage];

    int prob = 0;
#pragma unroll 1
    while (prob + 1 < b.count && (int)blockIdx.x >= b.p[prob + 1].block_begin)
        ++prob;
    const PreDev &p = b.p[prob];
    const int tile = blockIdx.x - p.block_begin;
    const int m0 = (tile / p.tiles_n) * kBM;
    const int n0 = (tile % p.tiles_n) * kBN;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int K = p.K;
    const int words = K / 16;
    const bool aligned = (words & 3) == 0;
    const int supers = (K + kSuper - 1) / kSuper;

    // Weight rows of this lane, one per n sub-tile.
    const uint32_t *wrow[4];
    bool wok[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        const int n = n0 + wn * 64 + ni * 16 + r;
        wok[ni] = n < p.N;
        wrow[ni] = p.W + (int64_t)(wok[ni] ? n : 0) * words;
    }

    // Activation staging: chunk c = i * 256 + tid -> token row c / 16, 16-byte column c % 16.
    auto load_x = [&](int t, int4 (&xr)[kXLoads]) {
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) {
            const int c = i * kPreThreads + tid;
            const int row = c >> 4, col = c & 15;
            const int m = m0 + row;
            const int k = t * kSuper + col * 16;
            xr[i] = (m < p.M && k < K)
                        ? *reinterpret_cast<const int4 *>(p.Xq + (int64_t)m * K + k)
                        : make_int4(0, 0, 0, 0);
        }
    };
    auto store_x = [&](int buf, const int4 (&xr)[kXLoads]) {
        unsigned char *base = smem + buf * kXStage;
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) {
            const int c = i * kPreThreads + tid;
            const int row = c >> 4, col = c & 15;
            *reinterpret_cast<int4 *>(base + row * kXRow + col * 16) = xr[i];
        }
    };
    auto load_w = [&](int t, uint4 (&wr)[4]) {
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
            wr[ni] = wok[ni] ? load_w4(wrow[ni], t * 16 + 4 * g, words, aligned)
                             : make_uint4(0, 0, 0, 0);
    };

    v4i acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
            acc[mi][ni] = v4i{0, 0, 0, 0};

    int4 xr[kXLoads];
    uint4 wcur[4], wnext[4];
    load_x(0, xr);
    load_w(0, wcur);
    store_x(0, xr);
    __syncthreads();

    for (int t = 0; t < supers; ++t) {
        const bool more = t + 1 < supers;
        if (more) {
            load_x(t + 1, xr);
            load_w(t + 1, wnext);
        }
        const unsigned char *xs = smem + (t & 1) * kXStage + (wm * 64 + r) * kXRow + 64 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v4i bop[4];
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const uint32_t wj = j == 0 ? wcur[ni].x : j == 1 ? wcur[ni].y
                                  : j == 2 ? wcur[ni].z : wcur[ni].w;
                bop[ni] = unpack_word64(wj);
            }
            v4i aop[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                aop[mi] = *reinterpret_cast<const v4i *>(xs + mi * 16 * kXRow + 16 * j);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[mi], bop[ni],
                                                                       acc[mi][ni], 0, 0, 0);
        }
        if (more) {
            store_x((t + 1) & 1, xr);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                wcur[ni] = wnext[ni];
        }
        __syncthreads();
    }

    // Epilogue: acc[mi][ni] register v holds 64 * D[m][n] for
    // m = m0 + wm * 64 + mi * 16 + 4 * g + v and n = n0 + wn * 64 + ni * 16 + r.
    const double gamma = (double)*p.gamma;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = m0 + wm * 64 + mi * 16 + 4 * g + v;
            if (m >= p.M)
                continue;
            const double scale = gamma * (double)p.sx[m];
            float *yrow = p.Y + (int64_t)m * p.N;
            int32_t *arow = p.acc ? p.acc + (int64_t)m * p.N : nullptr;
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const int n = n0 + wn * 64 + ni * 16 + r;
                if (n >= p.N)
                    continue;
                const int s = v == 0 ? acc[mi][ni].x : v == 1 ? acc[mi][ni].y
                            : v == 2 ? acc[mi][ni].z : acc[mi][ni].w;
                const int a = s >> 6;
                yrow[n] = (float)((double)a * scale);
                if (arow)
                    arow[n] = a;
            }
        }
    }
}

hipError_t launch_forward_prefill(const bl_forward_problem *q, int count, hipStream_t stream)
{
    PreBatch b{};
    int blocks = 0, n = 0;
    for (int i = 0; i < count; ++i) {
        if (q[i].M == 0 || q[i].N == 0)
            continue;
        PreDev &d = b.p[n++];
        d.Xq = q[i].X_q;
        d.sx = q[i].x_scale;
        d.W = q[i].W_packed;
        d.gamma = q[i].gamma;
        d.Y = q[i].Y;
        d.acc = q[i].acc;
        d.M = (int)q[i].M;
        d.N = (int)q[i].N;
        d.K = (int)q[i].K;
        d.tiles_n = (d.N + kBN - 1) / kBN;
        d.block_begin = blocks;
        blocks += ((d.M + kBM - 1) / kBM) * d.tiles_n;
    }
    b.count = n;
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(prefill_kernel, dim3(blocks), dim3(kPreThreads), 0, stream, b);
    return hipGetLastError();
}

}  // namespace bl
