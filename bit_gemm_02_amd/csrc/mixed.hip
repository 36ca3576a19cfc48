// mixed.hip — one launch for a mixed batch: the prefill products of one chunk of tokens and
// the fused decode calls of a few other tokens, the two phases a serving step batches
// together (SLM750-Edge card, "Performance": prompt processing and single-token decode, the
// latter bandwidth-bound; both run the same BitLinear forward).
//
// The two sets of problems are independent, so their blocks can share one grid: prefill
// tiles take block indices [0, P) (their XCD-aware tile order is unchanged) and decode
// blocks [P, P + D).  Blocks are dispatched in index order, so the decode blocks start as
// prefill tiles retire and run on the compute units the product leaves idle in its tail
// (its long-K tiles finish last), instead of waiting for the whole product to drain and
// paying a launch boundary of their own.  Every block runs exactly the code of its own
// launch (prefill_block, decode_block), so the results are bit-identical to the two
// launches.  The grid uses the 128 x 128 prefill tile (four waves, the decode block's size);
// its LDS is the sum of both bodies' static buffers (60 KB + 4 KB) plus the decode block's
// staged activations (M * K bytes): two blocks per compute unit while those stay under about
// 16 KB, one block per compute unit for larger decode rows (up to the fused form's 48 KB).
#include "decode_core.hpp"
#include "prefill_core.hpp"

namespace bl {

static_assert(TileSmall::THREADS == kDecThreads, "one block size for both kinds of block");
static_assert(sizeof(PreBatch) + sizeof(FwdBatch) <= 4096, "kernel arguments");

template <bool PFULL, bool DFULL, bool BF16>
__global__ __launch_bounds__(kDecThreads) void mixed_kernel(PreBatch pb, FwdBatch db)
{
    const int bid = blockIdx.x;
    if (bid < pb.blocks)
        prefill_block<TileSmall, PFULL>(pb, bid);
    else
        decode_block<1, true, true, DFULL, false, BF16, false>(db, bid - pb.blocks);
}

bool mixed_eligible(const bl_forward_ex_problem *pre, int npre, const bl_linear_ex_problem *dec,
                    int ndec)
{
    if (npre <= 0 || ndec <= 0)
        return false;
    for (int i = 0; i < npre; ++i)
        if (pre[i].M <= kDecodeMaxM)
            return false;
    if (prefill_big_tiles(pre, npre))
        return false;
    for (int i = 0; i < ndec; ++i)
        if (dec[i].W2_packed || dec[i].act != BL_ACT_NONE || dec[i].residual ||
            dec[i].x_dtype != dec[0].x_dtype || dec[i].M > BL_LINEAR_FUSED_MAX_M ||
            dec[i].M * dec[i].K > BL_LINEAR_FUSED_MAX_BYTES)
            return false;
    return true;
}

template <bool PFULL, bool DFULL>
static void launch_mixed_dt(bool bf16, int blocks, size_t lds, hipStream_t stream,
                            const PreBatch &pb, const FwdBatch &db)
{
    if (bf16)
        hipLaunchKernelGGL((mixed_kernel<PFULL, DFULL, true>), dim3(blocks), dim3(kDecThreads), lds,
                           stream, pb, db);
    else
        hipLaunchKernelGGL((mixed_kernel<PFULL, DFULL, false>), dim3(blocks), dim3(kDecThreads), lds,
                           stream, pb, db);
}

hipError_t launch_mixed(const bl_forward_ex_problem *pre, int npre, const bl_linear_ex_problem *dec,
                        int ndec, hipStream_t stream)
{
    PreBatch pb{};
    bool pfull;
    const int pblocks = build_batch<TileSmall>(pre, npre, pb, pfull);
    const bl_linear_ex_problem *dq[BL_MAX_GROUP];
    for (int i = 0; i < ndec; ++i)
        dq[i] = &dec[i];
    FwdBatch db{};
    bool dfull;
    const int dblocks = build_linear_batch<1, false>(dq, ndec, db, dfull);
    const int blocks = pblocks + dblocks;
    if (blocks == 0)
        return hipSuccess;
    const size_t lds = decode_xlds_bytes(db);
    const bool bf16 = dec[0].x_dtype == BL_BF16;
    if (pfull && dfull)
        launch_mixed_dt<true, true>(bf16, blocks, lds, stream, pb, db);
    else if (pfull)
        launch_mixed_dt<true, false>(bf16, blocks, lds, stream, pb, db);
    else if (dfull)
        launch_mixed_dt<false, true>(bf16, blocks, lds, stream, pb, db);
    else
        launch_mixed_dt<false, false>(bf16, blocks, lds, stream, pb, db);
    return hipGetLastError();
}

}  // namespace bl
