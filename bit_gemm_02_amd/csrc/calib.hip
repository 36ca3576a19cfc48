// calib.hip — measurement helpers: what this GPU attains on a plain HBM read stream and on
// the matrix units alone, the "measured peaks" that the kernels' rooflines are also quoted
// against (beside the published peaks).  Not part of the method.
//
//   calib_stream_kernel  reads a buffer once with 16-byte loads (eight in flight per thread)
//                        and XORs every dword into one word, so no load can be dropped;
//   calib_mfma_kernel    runs a loop of independent matrix-unit operations per wave (int8
//                        16x16x64 or bf16 16x16x32) on operands of ones; the sums it stores
//                        have a closed form the tests check.
#include "common.hpp"

namespace bl {

constexpr int kCalibThreads = 256;
constexpr int kCalibChains = 8;     // independent accumulators per wave
// Steps per chain between loop back-edges: the compiler copies the loop-carried accumulators
// between matrix registers at every back-edge (about 56 moves), so a long unrolled body keeps
// those copies to a few percent of the loop.
constexpr int kCalibBlock = 64;

__global__ __launch_bounds__(kCalibThreads) void calib_stream_kernel(const v4u *buf, int64_t chunks,
                                                                     uint32_t *out)
{
    const int64_t stride = (int64_t)gridDim.x * kCalibThreads;
    uint32_t x = 0;
    int64_t i = (int64_t)blockIdx.x * kCalibThreads + threadIdx.x;
    for (; i + 7 * stride < chunks; i += 8 * stride) {
        v4u v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = buf[i + u * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < chunks; i += stride) {
        const v4u v = buf[i];
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // Wave XOR, then one device atomic per wave.
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        x ^= (uint32_t)__shfl_xor((int)x, off, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0)
        atomicXor(out, x);
}

// Every wave: kCalibChains accumulators, `iters` operations on each, operands `a` and `b`
// (kernel arguments, so nothing is folded): int8 bytes of value 1 give 64 per step per
// element, bf16 1.0 (0x3F80) gives 32.  Lane l stores a quarter of the sum over its chains of
// all four accumulator elements to out[block * 256 + thread].
template <bool BF>
__global__ __launch_bounds__(kCalibThreads) void calib_mfma_kernel(int iters, uint32_t a, uint32_t b, int32_t *out)
{
    const v4u op = v4u{a, a, a, a};
    const v4u opb = v4u{b, b, b, b};
    if constexpr (BF) {
        f32x4 acc[kCalibChains];
#pragma unroll
        for (int c = 0; c < kCalibChains; ++c)
            acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        int it = 0;
#pragma unroll 1
        for (; it + kCalibBlock <= iters; it += kCalibBlock)
#pragma unroll
            for (int u = 0; u < kCalibBlock; ++u)
#pragma unroll
                for (int c = 0; c < kCalibChains; ++c)
                    acc[c] = mfma_bf16(op, opb, acc[c]);
#pragma unroll 1
        for (; it < iters; ++it)
#pragma unroll
            for (int c = 0; c < kCalibChains; ++c)
                acc[c] = mfma_bf16(op, opb, acc[c]);
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < kCalibChains; ++c)
            s += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
        out[blockIdx.x * kCalibThreads + threadIdx.x] = (int32_t)(s * 0.25f);
    } else {
        const v4i opi = __builtin_bit_cast(v4i, op), opj = __builtin_bit_cast(v4i, opb);
        v4i acc[kCalibChains];
#pragma unroll
        for (int c = 0; c < kCalibChains; ++c)
            acc[c] = v4i{0, 0, 0, 0};
        int it = 0;
#pragma unroll 1
        for (; it + kCalibBlock <= iters; it += kCalibBlock)
#pragma unroll
            for (int u = 0; u < kCalibBlock; ++u)
#pragma unroll
                for (int c = 0; c < kCalibChains; ++c)
                    acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(opi, opj, acc[c], 0, 0, 0);
#pragma unroll 1
        for (; it < iters; ++it)
#pragma unroll
            for (int c = 0; c < kCalibChains; ++c)
                acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(opi, opj, acc[c], 0, 0, 0);
        int32_t s = 0;
#pragma unroll
        for (int c = 0; c < kCalibChains; ++c)
            s += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
        out[blockIdx.x * kCalibThreads + threadIdx.x] = s / 4;
    }
}

hipError_t launch_calib_stream(const void *buf, int64_t bytes, uint32_t *out, hipStream_t stream)
{
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return e;
    const int64_t chunks = bytes / 16;
    int64_t blocks = (chunks + kCalibThreads - 1) / kCalibThreads;
    if (blocks > (int64_t)cus * 8)
        blocks = (int64_t)cus * 8;
    if (blocks < 1)
        blocks = 1;
    hipLaunchKernelGGL(calib_stream_kernel, dim3((unsigned)blocks), dim3(kCalibThreads), 0, stream,
                       static_cast<const v4u *>(buf), chunks, out);
    return hipGetLastError();
}

hipError_t launch_calib_mfma(int kind, int iters, int blocks, int32_t *out, hipStream_t stream)
{
    if (kind == 1)
        hipLaunchKernelGGL(calib_mfma_kernel<true>, dim3(blocks), dim3(kCalibThreads), 0, stream,
                           iters, 0x3F803F80u, 0x3F803F80u, out);
    else
        hipLaunchKernelGGL(calib_mfma_kernel<false>, dim3(blocks), dim3(kCalibThreads), 0, stream,
                           iters, 0x01010101u, 0x01010101u, out);
    return hipGetLastError();
}

}  // namespace bl
