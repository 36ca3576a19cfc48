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
// Work split: one block = 4 waves = RG groups of 16 weight rows.  The K range of those rows
// is cut into four contiguous pieces, one per wave; each wave walks its piece in
// "super-steps" of 256 weights (16 packed words) per row: lane (r = l % 16, g = l / 16)
// loads words 4g .. 4g+3 of row r of every row group with one 16-byte load per group and
// feeds them to four MFMAs per group.  In MFMA j, lane group g contributes word 16t + 4g + j;
// the A operand of the same lane takes the matching 16 int8 activations, loaded once and
// used by all RG groups (so the activation loads, L2 hits, are 4/RG of the weight loads).
// Super-steps go in chunks of PF with the next chunk's loads in flight while one chunk is
// multiplied.  The four waves' integer partial sums are added through LDS (exact, order-
// free); wave q applies the epilogue y = fl32(fp64(acc * gamma * s_x[m])) to row group q.
#include "decode_core.hpp"

namespace bl {

template <int RG, bool XLDS, bool QUANT, bool FULL_K, bool PAIR = false, bool BF16 = false,
          bool B3 = false>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(FwdBatch b)
{
    decode_block<RG, XLDS, QUANT, FULL_K, PAIR, BF16, B3>(b, blockIdx.x);
}

template <int RG, bool XLDS, bool QUANT = false, bool PAIR = false, bool BF16 = false, bool B3 = false>
static hipError_t launch_batch(FwdBatch &b, int blocks, bool full_k, hipStream_t stream)
{
    if (blocks == 0)
        return hipSuccess;
    const size_t lds = XLDS ? decode_xlds_bytes(b) : 0;
    if (B3)      // rows are whole blocks: no ragged-word form
        hipLaunchKernelGGL((decode_kernel<RG, XLDS, QUANT, true, PAIR, BF16, B3>), dim3(blocks),
                           dim3(kDecThreads), lds, stream, b);
    else if (full_k)
        hipLaunchKernelGGL((decode_kernel<RG, XLDS, QUANT, true, PAIR, BF16>), dim3(blocks),
                           dim3(kDecThreads), lds, stream, b);
    else
        hipLaunchKernelGGL((decode_kernel<RG, XLDS, QUANT, false, PAIR, BF16>), dim3(blocks),
                           dim3(kDecThreads), lds, stream, b);
    return hipGetLastError();
}

template <int RG, bool XLDS>
static hipError_t launch_rg(const bl_forward_ex_problem *q, int count, hipStream_t stream)
{
    // Longest-K problems first: their blocks take longest, so they should not start last.
    int order[BL_MAX_GROUP];
    int m = 0;
    for (int i = 0; i < count; ++i)
        if (q[i].M > 0 && q[i].N > 0)
            order[m++] = i;
    std::stable_sort(order, order + m, [&](int a, int c) { return q[a].K > q[c].K; });
    FwdBatch b{};
    int blocks = 0, n = 0;
    bool full_k = true;
    for (int o = 0; o < m; ++o) {
        const bl_forward_ex_problem &s = q[order[o]];
        full_k = full_k && (s.K % 256 == 0);
        FwdDev &d = b.p[n++];
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
        d.block_begin = blocks;
        blocks += (d.N + 16 * RG - 1) / (16 * RG);
    }
    b.count = n;
    return launch_batch<RG, XLDS>(b, blocks, full_k, stream);
}

// Row groups per block: as many as still leave at least one block per compute unit
// (fewer activation loads per weight byte), else one (more blocks for small layers).
hipError_t launch_forward_decode(const bl_forward_ex_problem *q, int count, hipStream_t stream)
{
    int64_t rows = 0;
    bool xlds = true;
    for (int i = 0; i < count; ++i)
        if (q[i].M > 0 && q[i].N > 0) {
            rows += q[i].N;
            xlds = xlds && q[i].M <= kDecXldsMaxM && q[i].M * q[i].K <= kDecXldsBytes;
        }
    if (xlds)
        return launch_rg<1, true>(q, count, stream);
    if (rows >= 256 * 64)
        return launch_rg<4, false>(q, count, stream);
    if (rows >= 256 * 32)
        return launch_rg<2, false>(q, count, stream);
    return launch_rg<1, false>(q, count, stream);
}

// The fused decode form: every problem has M <= 4 and M * K <= the LDS budget (checked by
// the caller).  Longest K first, one launch per kind (single projections, gated pairs).
// Every block quantizes the token rows it needs from the raw activations, so larger blocks
// (more row groups) read them fewer times: row groups as in the unfused decode launch, by
// weight rows (a pair's block holds both projections' rows).
template <int RG, bool PAIR, bool BF16, bool B3 = false>
static hipError_t launch_linear_rg(const bl_linear_ex_problem *const *q, int count,
                                   hipStream_t stream)
{
    FwdBatch b{};
    bool full_k;
    const int blocks = build_linear_batch<RG, PAIR>(q, count, b, full_k);
    return launch_batch<RG, true, true, PAIR, BF16, B3>(b, blocks, full_k, stream);
}

// Row groups per block by weight rows (a pair's block holds both projections' rows; pairs
// need an even count).
template <bool PAIR, bool BF16>
static hipError_t launch_linear_kind(const bl_linear_ex_problem *const *q, int n, int64_t wrows,
                                     hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    bool one_token = true;
    for (int i = 0; i < n; ++i)
        one_token = one_token && q[i]->M == 1;
    if (one_token && gemv_fits(q, n, BF16, false))
        return launch_gemv(q, n, PAIR, BF16, stream);
    if (wrows >= 256 * 64)
        return launch_linear_rg<4, PAIR, BF16>(q, n, stream);
    if constexpr (PAIR) {
        return launch_linear_rg<2, PAIR, BF16>(q, n, stream);
    } else {
        if (wrows >= 256 * 32)
            return launch_linear_rg<2, PAIR, BF16>(q, n, stream);
        return launch_linear_rg<1, PAIR, BF16>(q, n, stream);
    }
}

// One launch per kind present: single projections or gated pairs, fp32 or bf16 activations.
hipError_t launch_linear_decode(const bl_linear_ex_problem *q, int count, hipStream_t stream)
{
    const bl_linear_ex_problem *part[4][BL_MAX_GROUP];
    int n[4] = {0, 0, 0, 0};
    int64_t rows[4] = {0, 0, 0, 0};
    for (int i = 0; i < count; ++i) {
        if (q[i].M == 0 || q[i].N == 0)
            continue;
        const int k = (q[i].W2_packed ? 2 : 0) + (q[i].x_dtype == BL_BF16 ? 1 : 0);
        part[k][n[k]++] = &q[i];
        rows[k] += (q[i].W2_packed ? 2 : 1) * q[i].N;
    }
    hipError_t e = launch_linear_kind<false, false>(part[0], n[0], rows[0], stream);
    if (e == hipSuccess)
        e = launch_linear_kind<false, true>(part[1], n[1], rows[1], stream);
    if (e == hipSuccess)
        e = launch_linear_kind<true, false>(part[2], n[2], rows[2], stream);
    if (e == hipSuccess)
        e = launch_linear_kind<true, true>(part[3], n[3], rows[3], stream);
    return e;
}

// The fused decode call on base-3 weights (single projections, no epilogue stages): row
// groups as for the two-bit form, by weight rows.
template <bool BF16>
static hipError_t launch_b3_kind(const bl_linear_ex_problem *const *q, int n, int64_t rows,
                                 hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    bool one_token = true;
    for (int i = 0; i < n; ++i)
        one_token = one_token && q[i]->M == 1;
    if (one_token && gemv_fits(q, n, BF16, true))
        return launch_gemv_b3(q, n, BF16, stream);
    if (rows >= 256 * 64)
        return launch_linear_rg<4, false, BF16, true>(q, n, stream);
    if (rows >= 256 * 32)
        return launch_linear_rg<2, false, BF16, true>(q, n, stream);
    return launch_linear_rg<1, false, BF16, true>(q, n, stream);
}

hipError_t launch_linear_decode_b3(const bl_linear_ex_problem *q, int count, hipStream_t stream)
{
    const bl_linear_ex_problem *part[2][BL_MAX_GROUP];
    int n[2] = {0, 0};
    int64_t rows[2] = {0, 0};
    for (int i = 0; i < count; ++i) {
        if (q[i].M == 0 || q[i].N == 0)
            continue;
        const int k = q[i].x_dtype == BL_BF16 ? 1 : 0;
        part[k][n[k]++] = &q[i];
        rows[k] += q[i].N;
    }
    hipError_t e = launch_b3_kind<false>(part[0], n[0], rows[0], stream);
    if (e == hipSuccess)
        e = launch_b3_kind<true>(part[1], n[1], rows[1], stream);
    return e;
}

}  // namespace bl
