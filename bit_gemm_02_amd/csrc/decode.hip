// decode.hip — ternary x int8 product for few tokens (M <= 16): the decode path.
//
// At decode the product reads every packed weight once and does little work per byte, so
// it is bound by HBM bandwidth (SLM750-Edge card: decode is "bandwidth-bound"; bitone README:
// ternary weights make the product additions and subtractions only).  The kernel streams
// 2-bit words straight from HBM into registers, expands them in registers (one shift and
// one mask per four weights, see plane64) and lets the int8 matrix unit do the sums:
// v_mfma_i32_16x16x64_i8 with the tokens as the 16-row A operand (rows >= M are zero) and
// 16 weight rows as the B operand.  Wasting MFMA rows costs nothing here: the MFMA pipe and
// the VALU both have several times the throughput the memory stream needs.
//
// Work split: one block = 4 waves = 16 weight rows.  The K range of those rows is cut into
// four contiguous pieces, one per wave; each wave walks its piece in "super-steps" of 16
// words (256 weights) per row: lane (r = l % 16, g = l / 16) loads words 4g .. 4g+3 of row
// n0 + r with one 16-byte load and feeds them to four MFMAs.  In MFMA j, lane group g
// contributes word 16t + 4g + j; the A operand of the same lane takes the matching 16 int8
// activations, so both operands see the same k in the same byte positions whatever order
// the hardware uses inside a lane group.  The four waves' integer partial sums are added
// through LDS (exact, order-free) and wave 0 applies the epilogue
// y = fl32(fp64(acc * gamma * s_x[m])).
#include "common.hpp"

namespace bl {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kDecRows = 16;       // weight rows per block
constexpr int kSuperWords = 16;    // words per row per super-step
constexpr int kDecUnroll = 2;      // super-steps with loads in flight per wave

struct FwdDev {
    const int8_t *Xq;
    const float *sx;
    const uint32_t *W;
    const float *gamma;
    float *Y;
    int32_t *acc;
    int M, N, K;
    int block_begin;
};

struct FwdBatch {
    FwdDev p[BL_MAX_GROUP];
    int count;
};

// FULL_K: every problem of the launch has K % 256 == 0, so super-steps never run past a
// row and rows are 64-byte aligned (one 16-byte load per lane, no tail masking).
template <bool FULL_K>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(FwdBatch b)
{
    __shared__ v4i red[kDecWaves - 1][kWave];

    int prob = 0;
#pragma unroll 1
    while (prob + 1 < b.count && (int)blockIdx.x >= b.p[prob + 1].block_begin)
        ++prob;
    const FwdDev &p = b.p[prob];
    const int n0 = (blockIdx.x - p.block_begin) * kDecRows;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
    const int r = lane & 15;
    const int g = lane >> 4;
    const int words = p.K / 16;
    const int row_bytes = p.K / 4;
    // Weight rows n0 .. n0+15 (rows past N read as zero); tokens 0 .. M-1 (rows past M zero).
    const rsrc_t wres = make_rsrc(p.W + (int64_t)n0 * words, rows_bytes(n0, kDecRows, p.N, row_bytes));
    const rsrc_t xres = make_rsrc(p.Xq, (uint32_t)p.M * (uint32_t)p.K);
    const uint32_t wbase = (uint32_t)r * row_bytes;
    const uint32_t xbase = (uint32_t)r * p.K;

    const int supers = (words + kSuperWords - 1) / kSuperWords;
    const int t_begin = (supers * wave) / kDecWaves;
    const int t_end = (supers * (wave + 1)) / kDecWaves;

    v4i acc = {0, 0, 0, 0};
    for (int t = t_begin; t < t_end; t += kDecUnroll) {
        v4u wv[kDecUnroll];
        v4u xv[kDecUnroll][4];
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
            const int w = (t + u) * kSuperWords + 4 * g;
            // A super-step past this wave's range is loaded from offset "infinity" (zeros).
            const bool live = (t + u) < t_end;
            if (FULL_K) {
                wv[u] = buf_load16(wres, live ? wbase + 4u * w : kOOB);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool ok = live && (w + j) < words;
                    wv[u][j] = buf_load4(wres, ok ? wbase + 4u * (w + j) : kOOB);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool ok = live && (FULL_K || (w + j) < words);
                xv[u][j] = buf_load16(xres, ok ? xbase + 16u * (w + j) : kOOB);
            }
        }
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4i a = {(int)xv[u][j].x, (int)xv[u][j].y, (int)xv[u][j].z, (int)xv[u][j].w};
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, unpack_word64(wv[u][j]), acc, 0, 0, 0);
            }
        }
    }

    if (wave > 0)
        red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0)
        return;
#pragma unroll
    for (int w = 0; w < kDecWaves - 1; ++w)
        acc += red[w][lane];

    // acc holds 64 * D[m][n] for m = 4 * g + v (v = register index), n = n0 + r.
    const int n = n0 + r;
    if (n >= p.N)
        return;
    const double gamma = (double)*p.gamma;
    const int accv[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m < p.M) {
            const int a = accv[v] >> 6;  // exact: the sum is a multiple of 64
            const double scale = gamma * (double)p.sx[m];
            p.Y[(int64_t)m * p.N + n] = (float)((double)a * scale);
            if (p.acc)
                p.acc[(int64_t)m * p.N + n] = a;
        }
    }
}

hipError_t launch_forward_decode(const bl_forward_problem *q, int count, hipStream_t stream)
{
    FwdBatch b{};
    int blocks = 0, n = 0;
    bool full_k = true;
    for (int i = 0; i < count; ++i) {
        if (q[i].M == 0 || q[i].N == 0)
            continue;
        full_k = full_k && (q[i].K % 256 == 0);
        FwdDev &d = b.p[n++];
        d.Xq = q[i].X_q;
        d.sx = q[i].x_scale;
        d.W = q[i].W_packed;
        d.gamma = q[i].gamma;
        d.Y = q[i].Y;
        d.acc = q[i].acc;
        d.M = (int)q[i].M;
        d.N = (int)q[i].N;
        d.K = (int)q[i].K;
        d.block_begin = blocks;
        blocks += (d.N + kDecRows - 1) / kDecRows;
    }
    b.count = n;
    if (blocks == 0)
        return hipSuccess;
    if (full_k)
        hipLaunchKernelGGL(decode_kernel<true>, dim3(blocks), dim3(kDecThreads), 0, stream, b);
    else
        hipLaunchKernelGGL(decode_kernel<false>, dim3(blocks), dim3(kDecThreads), 0, stream, b);
    return hipGetLastError();
}

}  // namespace bl
