// prefill.hip — ternary x int8 product for many tokens (M > 16): the prefill path.
//
// With hundreds of tokens the product is a dense contraction (2 M N K integer operations;
// zeros are multiplied, the method computes the dense ternary product), so it belongs on the
// int8 matrix cores: v_mfma_i32_16x16x64_i8.  bitone README, "Features": the quantized
// weights stay in on-chip memory inside the GEMM and are never materialized in HBM; here the
// packed 2-bit words (0.25 B per weight) travel to LDS and are expanded to int8 in registers
// right before the multiply (plane64: one shift and one mask per four weights, giving 64 * c).
//
// Block tile BM (tokens) x BN (weight rows), 128 x 256 with 4 waves side by side in N (large
// grids; two blocks per CU) or 128 x 128 with 4 waves (2 x 2); each wave owns a (BM/WM) x
// (BN/WN) sub-tile of 16 x 16 MFMA tiles.  The K loop runs in stages of KS = 128 weights
// through a ring of NST = 3 LDS buffers:
// activation rows (BM x 128 bytes) and packed weight rows (BN x 32 bytes) go global -> LDS
// by gfx950 direct-to-LDS buffer loads, NST - 1 stages in flight while one is multiplied,
// one barrier per stage.  Per stage and lane (r = l % 16, g = l / 16): the packed words of its
// weight rows from LDS, expanded into B operands; the A operands (16 activation bytes of
// token row r, k group g) from LDS with one 16-byte read each.  The 128 x 256 tile runs these
// reads as a rolling pipeline (each fragment re-read right after its last use, the stage
// barrier in the middle of the last k-step); the 128 x 128 tile defers each stage's last
// k-step past the next barrier.
// Epilogue: y = fl32(fp64(acc * gamma * s_x[m])), acc = (MFMA sum) / 64 (exact shift); full
// tiles store whole 128-byte row segments with the non-temporal hint.
#include "prefill_core.hpp"

namespace bl {

template <class T, bool FULL_K, bool QR>
__global__ __launch_bounds__(T::THREADS, T::WPE) void prefill_kernel(PreBatch b)
{
    prefill_block<T, FULL_K, QR>(b, blockIdx.x);
}

template <class T, bool QR = false>
static hipError_t launch_tiles(const bl_forward_ex_problem *q, int count, hipStream_t stream)
{
    PreBatch b{};
    bool full_k;
    const int blocks = build_batch<T>(q, count, b, full_k);
    if (blocks == 0)
        return hipSuccess;
    if (QR)     // K % 128 == 0 for every problem (checked at the boundary): one form
        hipLaunchKernelGGL((prefill_kernel<T, true, true>), dim3(blocks), dim3(T::THREADS), 0, stream, b);
    else if (full_k)
        hipLaunchKernelGGL((prefill_kernel<T, true, false>), dim3(blocks), dim3(T::THREADS), 0, stream, b);
    else
        hipLaunchKernelGGL((prefill_kernel<T, false, false>), dim3(blocks), dim3(T::THREADS), 0, stream, b);
    return hipGetLastError();
}

hipError_t launch_wonly_prefill(const WgProblem *q, int count, hipStream_t stream)
{
    bl_forward_ex_problem ex[BL_MAX_GROUP];
    int n = 0;
    int64_t big = 0;
    for (int i = 0; i < count; ++i) {
        if (q[i].f32 || q[i].M == 0 || q[i].O == 0)
            continue;
        ex[n++] = bl_forward_ex_problem{static_cast<const int8_t *>(q[i].A), nullptr, q[i].T,
                                        q[i].gamma, q[i].Y, nullptr, nullptr, q[i].M, q[i].O,
                                        q[i].Kc};
        big += ((q[i].M + 255) / 256) * ((q[i].O + 255) / 256);
    }
    if (n == 0)
        return hipSuccess;
    if (big >= 512)
        return launch_tiles<TileWBig>(ex, n, stream);
    return launch_tiles<TileWSmall>(ex, n, stream);
}

hipError_t launch_forward_prefill(const bl_forward_ex_problem *q, int count, hipStream_t stream,
                                  bool quad)
{
    if (prefill_big_tiles(q, count))
        return quad ? launch_tiles<TileBig, true>(q, count, stream) : launch_tiles<TileBig>(q, count, stream);
    return quad ? launch_tiles<TileSmall, true>(q, count, stream) : launch_tiles<TileSmall>(q, count, stream);
}

}  // namespace bl
