// api.hip — the C ABI entry points (include/bitlinear.h): argument validation, problem
// tables and kernel dispatch.  Validation follows the input checks the bitone README lists
// for its native bridge (null pointers, shapes/bounds, alignment, dtype) and runs entirely on
// the host before anything is launched, so a rejected call touches no device memory.
#include <limits.h>

#include <mutex>

#include "common.hpp"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bl_status check_k(int64_t K)
{
    if (K <= 0 || K % 16 != 0 || K > BL_MAX_K)
        return BL_ERR_SHAPE;
    return BL_OK;
}

bl_status check_rows(int64_t R)
{
    if (R < 0 || R > BL_MAX_ROWS)
        return BL_ERR_SHAPE;
    return BL_OK;
}

bl_status check_weight(const bl_weight_problem &p)
{
    // An empty tensor (N == 0) may come with NULL data pointers; gamma is still written.
    if (!p.gamma || (p.N != 0 && (!p.W || !p.W_packed)))
        return BL_ERR_NULL;
    bl_status s = check_rows(p.N);
    if (s == BL_OK)
        s = check_k(p.K);
    if (s != BL_OK)
        return s;
    if (p.N * p.K / 4 > (int64_t)INT_MAX * 4096)
        return BL_ERR_SHAPE;  // keeps the pack grid within 2^31 blocks
    if (!aligned16(p.W) || !aligned16(p.W_packed) || (reinterpret_cast<uintptr_t>(p.gamma) & 3u))
        return BL_ERR_ALIGN;
    return BL_OK;
}

// The quad-row layout's shape limits: whole groups of four rows and whole 128-weight stages
// (so the layout is a permutation of the rows with no padding), and word indices below 2^32.
bl_status check_quad(int64_t N, int64_t K)
{
    if (N % 4 != 0 || K % 128 != 0 || N * (K / 16) > (int64_t)UINT_MAX)
        return BL_ERR_SHAPE;
    return BL_OK;
}

bl_status check_act(const bl_act_problem &p)
{
    if (p.M != 0 && (!p.X || !p.X_q || !p.x_scale))
        return BL_ERR_NULL;
    if (p.x_dtype != BL_F32 && p.x_dtype != BL_BF16)
        return BL_ERR_DTYPE;
    bl_status s = check_rows(p.M);
    if (s == BL_OK)
        s = check_k(p.K);
    if (s != BL_OK)
        return s;
    if (!aligned16(p.X) || !aligned16(p.X_q) || (reinterpret_cast<uintptr_t>(p.x_scale) & 3u) ||
        (p.norm_weight && !aligned16(p.norm_weight)))
        return BL_ERR_ALIGN;
    return BL_OK;
}

bl_status check_forward(const bl_forward_problem &p)
{
    // Empty products (M == 0 or N == 0) launch nothing and may pass NULL for empty tensors.
    const bool empty = p.M == 0 || p.N == 0;
    if (!p.gamma || (!empty && (!p.X_q || !p.x_scale || !p.W_packed || !p.Y)))
        return BL_ERR_NULL;
    bl_status s = check_rows(p.M);
    if (s == BL_OK)
        s = check_rows(p.N);
    if (s == BL_OK)
        s = check_k(p.K);
    if (s != BL_OK)
        return s;
    if (!aligned16(p.X_q) || !aligned16(p.W_packed) || (reinterpret_cast<uintptr_t>(p.x_scale) & 3u) ||
        (reinterpret_cast<uintptr_t>(p.gamma) & 3u) || (reinterpret_cast<uintptr_t>(p.Y) & 3u) ||
        (reinterpret_cast<uintptr_t>(p.acc) & 3u))
        return BL_ERR_ALIGN;
    return BL_OK;
}

bl_status check_act_ex(const bl_act_ex_problem &p)
{
    bl_act_problem base{p.X, p.norm_weight, p.X_q, p.x_scale, p.M, p.K, p.x_dtype, p.eps};
    bl_status s = check_act(base);
    if (s != BL_OK)
        return s;
    if (p.act < BL_ACT_NONE || p.act > BL_ACT_RELU2)
        return BL_ERR_DTYPE;
    if (p.act != BL_ACT_NONE && p.x_dtype != BL_F32)
        return BL_ERR_DTYPE;
    const bool glu = p.act == BL_ACT_SWIGLU || p.act == BL_ACT_RELU2_GLU;
    if (glu && p.M != 0 && !p.X2)
        return BL_ERR_NULL;
    if (glu && !aligned16(p.X2))
        return BL_ERR_ALIGN;
    return BL_OK;
}

bl_status check_forward_ex(const bl_forward_ex_problem &p)
{
    bl_forward_problem base{p.X_q, p.x_scale, p.W_packed, p.gamma, p.Y, p.acc, p.M, p.N, p.K};
    bl_status s = check_forward(base);
    if (s != BL_OK)
        return s;
    if (reinterpret_cast<uintptr_t>(p.residual) & 3u)
        return BL_ERR_ALIGN;
    return BL_OK;
}

bl_act_ex_problem to_ex(const bl_act_problem &p)
{
    return bl_act_ex_problem{p.X, nullptr, p.norm_weight, p.X_q, p.x_scale, p.M, p.K,
                             p.x_dtype, BL_ACT_NONE, p.eps};
}

bl_forward_ex_problem to_ex(const bl_forward_problem &p)
{
    return bl_forward_ex_problem{p.X_q, p.x_scale, p.W_packed, p.gamma, p.Y, p.acc, nullptr,
                                 p.M, p.N, p.K};
}

bl_status from_hip(hipError_t e) { return e == hipSuccess ? BL_OK : BL_ERR_HIP; }

// ---- fixed scratch of the allocation-free weight quantization
//
// The γ pass's fp64 partial sums (2 KiB per tensor) for a grouped call of up to BL_MAX_GROUP
// tensors, in a device array of the library instead of a caller-provided workspace.  Each GPU
// holds its own copy at its own address, for as long as the process lives.  In host code the
// array's name is only a stand-in for the symbol: its device address is looked up once per
// device (with that device current) and only that address is handed to kernels.
constexpr size_t kScratchBytes = (size_t)BL_MAX_GROUP * 256 * sizeof(double);
constexpr int kScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on device `dev`, or NULL if it cannot be had.
void *scratch_address(int dev)
{
    static std::mutex mu;
    static void *addr[kScratchDevices] = {};
    if (dev < 0 || dev >= kScratchDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess)
            return nullptr;
        if (cur != dev && hipSetDevice(dev) != hipSuccess)
            return nullptr;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev)
            (void)hipSetDevice(cur);
        if (e != hipSuccess || !p)
            return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

// Validated problems -> launches: act quant of any form in one call.
bl_status run_acts(const bl_act_ex_problem *q, int count, void *stream)
{
    int64_t rows = 0;
    for (int i = 0; i < count; ++i)
        rows += q[i].M;
    if (rows > INT_MAX)
        return BL_ERR_SHAPE;
    return from_hip(bl::launch_quantize_acts(q, count, static_cast<hipStream_t>(stream)));
}

// Validated products -> one decode launch (M <= 16) and one prefill launch (the rest).
bl_status run_forward(const bl_forward_ex_problem *q, int count, void *stream)
{
    bl_forward_ex_problem dec[BL_MAX_GROUP], pre[BL_MAX_GROUP];
    int nd = 0, np = 0;
    int64_t dec_blocks = 0, pre_blocks = 0;
    for (int i = 0; i < count; ++i) {
        const bl_forward_ex_problem &p = q[i];
        if (p.M <= bl::kDecodeMaxM) {
            dec[nd++] = p;
            dec_blocks += (p.N + 15) / 16;
        } else {
            pre[np++] = p;
            pre_blocks += ((p.M + 127) / 128) * ((p.N + 127) / 128);
        }
    }
    if (dec_blocks > INT_MAX || pre_blocks > INT_MAX)
        return BL_ERR_SHAPE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (nd) {
        bl_status s = from_hip(bl::launch_forward_decode(dec, nd, st));
        if (s != BL_OK)
            return s;
    }
    if (np)
        return from_hip(bl::launch_forward_prefill(pre, np, st));
    return BL_OK;
}

bool linear_fused(const bl_linear_problem &p)
{
    return p.M <= BL_LINEAR_FUSED_MAX_M && p.M * p.K <= BL_LINEAR_FUSED_MAX_BYTES;
}

bl_status check_linear(const bl_linear_problem &p)
{
    const bool empty = p.M == 0 || p.N == 0;
    if (!p.gamma || (!empty && (!p.X || !p.W_packed || !p.Y)))
        return BL_ERR_NULL;
    if (p.x_dtype != BL_F32 && p.x_dtype != BL_BF16)
        return BL_ERR_DTYPE;
    bl_status s = check_rows(p.M);
    if (s == BL_OK)
        s = check_rows(p.N);
    if (s == BL_OK)
        s = check_k(p.K);
    if (s != BL_OK)
        return s;
    // The two-step form needs the intermediate codes and scales.
    if (!empty && !linear_fused(p) && (!p.X_q || !p.x_scale))
        return BL_ERR_NULL;
    if (!aligned16(p.X) || !aligned16(p.W_packed) || !aligned16(p.X_q) ||
        (p.norm_weight && !aligned16(p.norm_weight)) ||
        (reinterpret_cast<uintptr_t>(p.x_scale) & 3u) || (reinterpret_cast<uintptr_t>(p.gamma) & 3u) ||
        (reinterpret_cast<uintptr_t>(p.Y) & 3u))
        return BL_ERR_ALIGN;
    return BL_OK;
}

bl_status check_linear_ex(const bl_linear_ex_problem &p)
{
    bl_linear_problem base{p.X, p.norm_weight, p.W_packed, p.gamma, p.Y, p.X_q, p.x_scale,
                           p.M, p.N, p.K, p.x_dtype, p.eps};
    const bool empty = p.M == 0 || p.N == 0;
    if (!empty && !linear_fused(base))
        return BL_ERR_SHAPE;       // only the fused form exists
    bl_status s = check_linear(base);
    if (s != BL_OK)
        return s;
    if (p.act < BL_ACT_NONE || p.act > BL_ACT_RELU2)
        return BL_ERR_DTYPE;
    const bool glu = p.act == BL_ACT_SWIGLU || p.act == BL_ACT_RELU2_GLU;
    if (glu && (!p.gamma2 || (!empty && !p.W2_packed)))
        return BL_ERR_NULL;
    if (!glu && p.W2_packed)
        return BL_ERR_DTYPE;
    if (!aligned16(p.W2_packed) || (reinterpret_cast<uintptr_t>(p.gamma2) & 3u) ||
        (reinterpret_cast<uintptr_t>(p.residual) & 3u))
        return BL_ERR_ALIGN;
    return BL_OK;
}

bool a4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bl_status check_wonly(const bl_wonly_problem &p)
{
    const bool empty = p.M == 0 || p.N == 0;
    if (!p.gamma || (!empty && (!p.X || !p.W_packed || !p.Y)))
        return BL_ERR_NULL;
    if (p.x_dtype != BL_F32 && p.x_dtype != BL_BF16)
        return BL_ERR_DTYPE;
    bl_status s = check_rows(p.M);
    if (s == BL_OK)
        s = check_rows(p.N);
    if (s == BL_OK)
        s = check_k(p.K);
    if (s != BL_OK)
        return s;
    if (!aligned16(p.X) || !aligned16(p.W_packed) || !a4(p.gamma) || !a4(p.Y))
        return BL_ERR_ALIGN;
    return BL_OK;
}

bl_status check_grad_input(const bl_grad_input_problem &p)
{
    const bool empty = p.M == 0;
    if (!p.gamma || (!empty && (!p.dY || !p.Wt_packed || !p.dX)))
        return BL_ERR_NULL;
    if (p.dy_dtype != BL_F32 && p.dy_dtype != BL_BF16)
        return BL_ERR_DTYPE;
    bl_status s = check_rows(p.M);
    if (s == BL_OK)
        s = check_k(p.N);            // the contraction: N % 16 == 0, 0 < N <= BL_MAX_K
    if (s == BL_OK)
        s = check_k(p.K);
    if (s != BL_OK)
        return s;
    if (!aligned16(p.dY) || !aligned16(p.Wt_packed) || !a4(p.gamma) || !a4(p.dX))
        return BL_ERR_ALIGN;
    return BL_OK;
}

bl_status check_grad_weight(const bl_grad_weight_problem &p)
{
    const bool empty = p.N == 0;
    if (p.ste < BL_STE_PASS || p.ste > BL_STE_SOFT)
        return BL_ERR_DTYPE;
    if (!p.gamma || (!empty && (!p.dW || (p.M != 0 && (!p.dY || !p.X_q || !p.x_scale)) ||
                                (p.ste != BL_STE_PASS && !p.W))))
        return BL_ERR_NULL;
    bl_status s = check_rows(p.M);
    if (s == BL_OK && (p.N < 0 || p.N > BL_MAX_K))
        s = BL_ERR_SHAPE;
    if (s == BL_OK)
        s = check_k(p.K);
    if (s != BL_OK)
        return s;
    if (!aligned16(p.dY) || !aligned16(p.X_q) || !aligned16(p.W) || !aligned16(p.dW) ||
        !a4(p.gamma) || !a4(p.x_scale))
        return BL_ERR_ALIGN;
    return BL_OK;
}

bl_linear_ex_problem to_ex(const bl_linear_problem &p)
{
    return bl_linear_ex_problem{p.X, p.norm_weight, p.W_packed, p.gamma, nullptr, nullptr,
                                p.Y, nullptr, p.X_q, p.x_scale, p.M, p.N, p.K, p.x_dtype,
                                BL_ACT_NONE, p.eps};
}

}  // namespace

extern "C" {

const char *bitlinear_status_string(int status)
{
    switch (status) {
    case BL_OK: return "ok";
    case BL_ERR_NULL: return "null pointer argument";
    case BL_ERR_SHAPE: return "invalid shape (negative size, K not a positive multiple of 16, or above limits)";
    case BL_ERR_ALIGN: return "misaligned pointer (tensors need 16-byte alignment)";
    case BL_ERR_DTYPE: return "unknown activation dtype";
    case BL_ERR_WORKSPACE: return "workspace too small";
    case BL_ERR_HIP: return "HIP launch failed";
    case BL_ERR_COUNT: return "invalid problem count";
    default: return "unknown status";
    }
}

int bitlinear_abi_version(void) { return 104; }

size_t bitlinear_quantize_weights_workspace(int64_t N, int64_t K)
{
    (void)N;
    (void)K;
    return bl::quantize_weights_workspace(1);
}

size_t bitlinear_workspace_bytes(int64_t N, int64_t K)
{
    return bitlinear_quantize_weights_workspace(N, K);
}

size_t bitlinear_quantize_weights_grouped_workspace(int count)
{
    if (count <= 0 || count > BL_MAX_GROUP)
        return 0;
    return bl::quantize_weights_workspace(count);
}

size_t bitlinear_quantize_weights_one_read_workspace(const bl_weight_problem *problems, int count)
{
    if (!problems || count <= 0 || count > BL_MAX_GROUP)
        return 0;
    for (int i = 0; i < count; ++i)
        if (check_rows(problems[i].N) != BL_OK || check_k(problems[i].K) != BL_OK ||
            problems[i].N * problems[i].K / 4 > (int64_t)INT_MAX * 4096)
            return 0;
    return bl::quantize_weights_one_read_workspace(problems, count);
}

bl_status bitlinear_quantize_weights_grouped(const bl_weight_problem *problems, int count,
                                             void *workspace, size_t workspace_bytes,
                                             void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    for (int i = 0; i < count; ++i) {
        bl_status s = check_weight(problems[i]);
        if (s != BL_OK)
            return s;
    }
    if (!workspace)
        return BL_ERR_NULL;
    if (!aligned16(workspace))
        return BL_ERR_ALIGN;
    if (workspace_bytes < bl::quantize_weights_workspace(count))
        return BL_ERR_WORKSPACE;
    return from_hip(bl::launch_quantize_weights(problems, count, workspace,
                                                static_cast<hipStream_t>(stream), false,
                                                workspace_bytes));
}

bl_status bitlinear_quantize_weights_grouped_noalloc(const bl_weight_problem *problems, int count,
                                                     void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    for (int i = 0; i < count; ++i) {
        bl_status s = check_weight(problems[i]);
        if (s != BL_OK)
            return s;
    }
    if (bl::quantize_weights_workspace(count) > kScratchBytes)
        return BL_ERR_WORKSPACE;      // more partial sums than the fixed scratch holds
    // The scratch of the device the stream belongs to (NULL: the current device).
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = -1;
    if ((st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev)) != hipSuccess)
        return BL_ERR_HIP;
    void *ws = scratch_address(dev);
    if (!ws)
        return BL_ERR_HIP;
    return from_hip(bl::launch_quantize_weights(problems, count, ws, st));
}

bl_status bitlinear_quantize_weights(const float *W, int64_t N, int64_t K, uint32_t *W_packed,
                                     float *gamma, void *workspace, size_t workspace_bytes,
                                     void *stream)
{
    bl_weight_problem p{W, W_packed, gamma, N, K};
    return bitlinear_quantize_weights_grouped(&p, 1, workspace, workspace_bytes, stream);
}

bl_status bitlinear_pack_codes(const int8_t *codes, int64_t N, int64_t K, uint32_t *W_packed,
                               void *stream)
{
    bl_status s = check_rows(N);
    if (s == BL_OK && N != 0 && (!codes || !W_packed))
        return BL_ERR_NULL;
    if (s == BL_OK)
        s = check_k(K);
    if (s != BL_OK)
        return s;
    if (N * K / 16 > (int64_t)INT_MAX * 256)
        return BL_ERR_SHAPE;
    if (!aligned16(codes) || !aligned16(W_packed))
        return BL_ERR_ALIGN;
    return from_hip(bl::launch_pack_codes(codes, N, K, W_packed, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_quantize_acts_grouped(const bl_act_problem *problems, int count, void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    bl_act_ex_problem ex[BL_MAX_GROUP];
    for (int i = 0; i < count; ++i) {
        bl_status s = check_act(problems[i]);
        if (s != BL_OK)
            return s;
        ex[i] = to_ex(problems[i]);
    }
    return run_acts(ex, count, stream);
}

static bl_status quantize_step(const bl_weight_problem *weights, int nw, void *workspace,
                               size_t workspace_bytes, const bl_act_problem *acts, int na,
                               void *stream, bool quad)
{
    if (nw < 0 || na < 0 || nw > BL_MAX_GROUP || na > BL_MAX_GROUP || nw + na == 0)
        return BL_ERR_COUNT;
    if ((nw && !weights) || (na && !acts))
        return BL_ERR_NULL;
    // Every problem is validated before anything is launched.
    for (int i = 0; i < nw; ++i) {
        bl_status s = check_weight(weights[i]);
        if (s == BL_OK && quad)
            s = check_quad(weights[i].N, weights[i].K);
        if (s != BL_OK)
            return s;
    }
    bl_act_ex_problem ex[BL_MAX_GROUP];
    int64_t rows = 0;
    for (int i = 0; i < na; ++i) {
        bl_status s = check_act(acts[i]);
        if (s != BL_OK)
            return s;
        ex[i] = to_ex(acts[i]);
        rows += acts[i].M;
    }
    if (rows > INT_MAX)
        return BL_ERR_SHAPE;
    if (nw) {
        if (!workspace)
            return BL_ERR_NULL;
        if (!aligned16(workspace))
            return BL_ERR_ALIGN;
        if (workspace_bytes < bl::quantize_weights_workspace(nw))
            return BL_ERR_WORKSPACE;
    }
    return from_hip(bl::launch_quantize_step(weights, nw, workspace, workspace_bytes, ex, na,
                                             static_cast<hipStream_t>(stream), quad));
}

bl_status bitlinear_quantize_step(const bl_weight_problem *weights, int nw, void *workspace,
                                  size_t workspace_bytes, const bl_act_problem *acts, int na,
                                  void *stream)
{
    return quantize_step(weights, nw, workspace, workspace_bytes, acts, na, stream, false);
}

bl_status bitlinear_quantize_step_quad_rows(const bl_weight_problem *weights, int nw,
                                            void *workspace, size_t workspace_bytes,
                                            const bl_act_problem *acts, int na, void *stream)
{
    return quantize_step(weights, nw, workspace, workspace_bytes, acts, na, stream, true);
}

bl_status bitlinear_quantize_acts_ex_grouped(const bl_act_ex_problem *problems, int count,
                                             void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    for (int i = 0; i < count; ++i) {
        bl_status s = check_act_ex(problems[i]);
        if (s != BL_OK)
            return s;
    }
    return run_acts(problems, count, stream);
}

bl_status bitlinear_quantize_acts(const void *X, int x_dtype, int64_t M, int64_t K,
                                  const float *norm_weight, float eps, int8_t *X_q,
                                  float *x_scale, void *stream)
{
    bl_act_problem p{X, norm_weight, X_q, x_scale, M, K, x_dtype, eps};
    return bitlinear_quantize_acts_grouped(&p, 1, stream);
}

bl_status bitlinear_forward_grouped(const bl_forward_problem *problems, int count, void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    bl_forward_ex_problem ex[BL_MAX_GROUP];
    for (int i = 0; i < count; ++i) {
        bl_status s = check_forward(problems[i]);
        if (s != BL_OK)
            return s;
        ex[i] = to_ex(problems[i]);
    }
    return run_forward(ex, count, stream);
}

bl_status bitlinear_forward_ex_grouped(const bl_forward_ex_problem *problems, int count,
                                       void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    for (int i = 0; i < count; ++i) {
        bl_status s = check_forward_ex(problems[i]);
        if (s != BL_OK)
            return s;
    }
    return run_forward(problems, count, stream);
}

bl_status bitlinear_forward(const int8_t *X_q, const float *x_scale, const uint32_t *W_packed,
                            const float *gamma, int64_t M, int64_t N, int64_t K, float *Y,
                            int32_t *acc, void *stream)
{
    bl_forward_problem p{X_q, x_scale, W_packed, gamma, Y, acc, M, N, K};
    return bitlinear_forward_grouped(&p, 1, stream);
}

bl_status bitlinear_pack_quad_rows(const uint32_t *W_packed, int64_t N, int64_t K, uint32_t *W_quad,
                                   void *stream)
{
    bl_status s = check_rows(N);
    if (s == BL_OK && N != 0 && (!W_packed || !W_quad))
        return BL_ERR_NULL;
    if (s == BL_OK)
        s = check_k(K);
    if (s == BL_OK)
        s = check_quad(N, K);
    if (s != BL_OK)
        return s;
    if (!aligned16(W_packed) || !aligned16(W_quad))
        return BL_ERR_ALIGN;
    return from_hip(bl::launch_pack_quad_rows(W_packed, N, K, W_quad, static_cast<hipStream_t>(stream)));
}

// The prefill products of a set on quad rows: every non-empty problem needs M > 16, N % 4 == 0
// and K % 128 == 0; problems are validated before anything is launched.
static bl_status forward_quad(const bl_forward_ex_problem *q, int count, void *stream)
{
    bl_forward_ex_problem ex[BL_MAX_GROUP];
    int n = 0;
    int64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        const bl_forward_ex_problem &p = q[i];
        if (p.M == 0 || p.N == 0)
            continue;
        if (p.M <= bl::kDecodeMaxM)
            return BL_ERR_SHAPE;         // the quad-row layout feeds the prefill product only
        const bl_status s = check_quad(p.N, p.K);
        if (s != BL_OK)
            return s;
        ex[n++] = p;
        blocks += ((p.M + 127) / 128) * ((p.N + 127) / 128);
    }
    if (blocks > INT_MAX)
        return BL_ERR_SHAPE;
    if (n == 0)
        return BL_OK;
    return from_hip(bl::launch_forward_prefill(ex, n, static_cast<hipStream_t>(stream), true));
}

bl_status bitlinear_forward_quad_rows_grouped(const bl_forward_problem *problems, int count,
                                              void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    bl_forward_ex_problem ex[BL_MAX_GROUP];
    for (int i = 0; i < count; ++i) {
        const bl_status s = check_forward(problems[i]);
        if (s != BL_OK)
            return s;
        ex[i] = to_ex(problems[i]);
    }
    return forward_quad(ex, count, stream);
}

bl_status bitlinear_forward_ex_quad_rows_grouped(const bl_forward_ex_problem *problems, int count,
                                                 void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    for (int i = 0; i < count; ++i) {
        const bl_status s = check_forward_ex(problems[i]);
        if (s != BL_OK)
            return s;
    }
    return forward_quad(problems, count, stream);
}

bl_status bitlinear_linear_grouped(const bl_linear_problem *problems, int count, void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    bl_linear_ex_problem fused[BL_MAX_GROUP];
    bl_act_ex_problem act[BL_MAX_GROUP];
    bl_forward_ex_problem fwd[BL_MAX_GROUP];
    int nf = 0, nt = 0;
    int64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        const bl_linear_problem &p = problems[i];
        bl_status s = check_linear(p);
        if (s != BL_OK)
            return s;
        if (p.M == 0 || p.N == 0)
            continue;
        if (linear_fused(p)) {
            fused[nf++] = to_ex(p);
            blocks += (p.N + 15) / 16;
        } else {
            act[nt] = bl_act_ex_problem{p.X, nullptr, p.norm_weight, p.X_q, p.x_scale, p.M, p.K,
                                        p.x_dtype, BL_ACT_NONE, p.eps};
            fwd[nt] = bl_forward_ex_problem{p.X_q, p.x_scale, p.W_packed, p.gamma, p.Y, nullptr,
                                            nullptr, p.M, p.N, p.K};
            ++nt;
        }
    }
    if (blocks > INT_MAX)
        return BL_ERR_SHAPE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (nf) {
        bl_status s = from_hip(bl::launch_linear_decode(fused, nf, st));
        if (s != BL_OK)
            return s;
    }
    if (nt) {
        bl_status s = run_acts(act, nt, stream);
        if (s != BL_OK)
            return s;
        return run_forward(fwd, nt, stream);
    }
    return BL_OK;
}

bl_status bitlinear_forward_mixed(const bl_forward_ex_problem *prefill, int npre,
                                  const bl_linear_problem *decode, int ndec, void *stream)
{
    if (npre < 0 || ndec < 0 || npre > BL_MAX_GROUP || ndec > BL_MAX_GROUP || npre + ndec == 0)
        return BL_ERR_COUNT;
    if ((npre && !prefill) || (ndec && !decode))
        return BL_ERR_NULL;
    // Every problem is validated before anything is launched.
    bl_forward_ex_problem pre[BL_MAX_GROUP];
    bl_linear_ex_problem dec[BL_MAX_GROUP];
    int np = 0, nd = 0;
    int64_t pre_blocks = 0, dec_blocks = 0;
    for (int i = 0; i < npre; ++i) {
        bl_status s = check_forward_ex(prefill[i]);
        if (s != BL_OK)
            return s;
        if (prefill[i].M > 0 && prefill[i].N > 0) {
            pre[np++] = prefill[i];
            pre_blocks += ((prefill[i].M + 127) / 128) * ((prefill[i].N + 127) / 128);
        }
    }
    bool fused = true;
    for (int i = 0; i < ndec; ++i) {
        bl_status s = check_linear(decode[i]);
        if (s != BL_OK)
            return s;
        if (decode[i].M > 0 && decode[i].N > 0) {
            fused = fused && linear_fused(decode[i]);
            dec[nd++] = to_ex(decode[i]);
            dec_blocks += (decode[i].N + 15) / 16;
        }
    }
    if (pre_blocks + dec_blocks > INT_MAX)
        return BL_ERR_SHAPE;
    if (fused && bl::mixed_eligible(pre, np, dec, nd))
        return from_hip(bl::launch_mixed(pre, np, dec, nd, static_cast<hipStream_t>(stream)));
    // Otherwise the two calls, prefill first.
    if (npre) {
        bl_status s = bitlinear_forward_ex_grouped(prefill, npre, stream);
        if (s != BL_OK)
            return s;
    }
    return ndec ? bitlinear_linear_grouped(decode, ndec, stream) : BL_OK;
}

bl_status bitlinear_linear_ex_grouped(const bl_linear_ex_problem *problems, int count,
                                      void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    int64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        bl_status s = check_linear_ex(problems[i]);
        if (s != BL_OK)
            return s;
        blocks += (problems[i].N + 15) / 16;
    }
    if (blocks > INT_MAX)
        return BL_ERR_SHAPE;
    return from_hip(bl::launch_linear_decode(problems, count, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_forward_wonly_grouped(const bl_wonly_problem *problems, int count, void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    bl::WgProblem q[BL_MAX_GROUP];
    int64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        const bl_wonly_problem &p = problems[i];
        bl_status s = check_wonly(p);
        if (s != BL_OK)
            return s;
        q[i] = bl::WgProblem{p.X, p.x_dtype == BL_F32, p.W_packed, p.gamma, p.Y, p.M, p.N, p.K};
        blocks += ((p.M + 127) / 128) * ((p.N + 127) / 128);
    }
    if (blocks > INT_MAX)
        return BL_ERR_SHAPE;
    return from_hip(bl::launch_wgemm(q, count, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_transpose_packed(const uint32_t *W_packed, int64_t N, int64_t K,
                                     uint32_t *Wt_packed, void *stream)
{
    if (N < 0 || N > BL_MAX_K || N % 16 != 0)
        return BL_ERR_SHAPE;
    bl_status s = check_k(K);
    if (s != BL_OK)
        return s;
    if (N != 0 && (!W_packed || !Wt_packed))
        return BL_ERR_NULL;
    if (!aligned16(W_packed) || !aligned16(Wt_packed))
        return BL_ERR_ALIGN;
    return from_hip(bl::launch_transpose_packed(W_packed, N, K, Wt_packed,
                                                static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_grad_input_grouped(const bl_grad_input_problem *problems, int count,
                                       void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    bl::WgProblem q[BL_MAX_GROUP];
    int64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        const bl_grad_input_problem &p = problems[i];
        bl_status s = check_grad_input(p);
        if (s != BL_OK)
            return s;
        // dX = gamma * dY C = gamma * dY (C^T)^T: the weight-only product with A = dY and the
        // transposed codes (K rows of N/16 words).
        q[i] = bl::WgProblem{p.dY, p.dy_dtype == BL_F32, p.Wt_packed, p.gamma, p.dX, p.M, p.K, p.N};
        blocks += ((p.M + 127) / 128) * ((p.K + 127) / 128);
    }
    if (blocks > INT_MAX)
        return BL_ERR_SHAPE;
    return from_hip(bl::launch_wgemm(q, count, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_grad_weight_grouped(const bl_grad_weight_problem *problems, int count,
                                        void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    int64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        bl_status s = check_grad_weight(problems[i]);
        if (s != BL_OK)
            return s;
        blocks += ((problems[i].N + 127) / 128) * ((problems[i].K + 127) / 128);
    }
    if (blocks > INT_MAX)
        return BL_ERR_SHAPE;
    return from_hip(bl::launch_grad_weight(problems, count, static_cast<hipStream_t>(stream)));
}

int64_t bitlinear_b3_row_bytes(int64_t K)
{
    return K <= 0 ? 0 : 16 * ((K + 79) / 80);
}

bl_status bitlinear_pack_b3(const uint32_t *W_packed, int64_t N, int64_t K, uint8_t *W_b3,
                            void *stream)
{
    bl_status s = check_rows(N);
    if (s == BL_OK && N != 0 && (!W_packed || !W_b3))
        return BL_ERR_NULL;
    if (s == BL_OK)
        s = check_k(K);
    if (s != BL_OK)
        return s;
    if (N * ((K + 79) / 80) > (int64_t)INT_MAX * 256)
        return BL_ERR_SHAPE;
    if (!aligned16(W_packed) || !aligned16(W_b3))
        return BL_ERR_ALIGN;
    return from_hip(bl::launch_pack_b3(W_packed, N, K, W_b3, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_linear_b3_grouped(const bl_linear_problem *problems, int count, void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    bl_linear_ex_problem ex[BL_MAX_GROUP];
    int64_t blocks = 0;
    for (int i = 0; i < count; ++i) {
        const bl_linear_problem &p = problems[i];
        const bool empty = p.M == 0 || p.N == 0;
        if (!empty && !linear_fused(p))
            return BL_ERR_SHAPE;         // only the fused form exists
        bl_status s = check_linear(p);
        if (s != BL_OK)
            return s;
        ex[i] = to_ex(p);
        blocks += (p.N + 15) / 16;
    }
    if (blocks > INT_MAX)
        return BL_ERR_SHAPE;
    return from_hip(bl::launch_linear_decode_b3(ex, count, static_cast<hipStream_t>(stream)));
}

int64_t bitlinear_tiles_bytes(int64_t N, int64_t K)
{
    return (N < 0 || K <= 0 || K % 16 != 0) ? 0 : bl::tiles_bytes(N, K);
}

bl_status bitlinear_pack_tiles(const uint32_t *W_packed, int64_t N, int64_t K, uint32_t *W_tiles,
                               void *stream)
{
    bl_status s = check_rows(N);
    if (s == BL_OK && N != 0 && (!W_packed || !W_tiles))
        return BL_ERR_NULL;
    if (s == BL_OK)
        s = check_k(K);
    if (s != BL_OK)
        return s;
    if (bl::tiles_bytes(N, K) / 16 > (int64_t)INT_MAX * 256)
        return BL_ERR_SHAPE;
    if (!aligned16(W_packed) || !aligned16(W_tiles))
        return BL_ERR_ALIGN;
    return from_hip(bl::launch_pack_tiles(W_packed, N, K, W_tiles, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_linear_tiles_grouped(const bl_linear_problem *problems, int count, void *stream)
{
    if (!problems)
        return BL_ERR_NULL;
    if (count <= 0 || count > BL_MAX_GROUP)
        return BL_ERR_COUNT;
    bl_linear_ex_problem ex[BL_MAX_GROUP];
    const bl_linear_ex_problem *part[2][BL_MAX_GROUP];
    int n[2] = {0, 0};
    for (int i = 0; i < count; ++i) {
        const bl_linear_problem &p = problems[i];
        bl_status s = check_linear(p);
        if (s != BL_OK)
            return s;
        if (p.M == 0 || p.N == 0)
            continue;
        if (p.M != 1)
            return BL_ERR_SHAPE;         // the tile layout feeds the one-token product only
        ex[i] = to_ex(p);
        const int k = p.x_dtype == BL_BF16 ? 1 : 0;
        part[k][n[k]++] = &ex[i];
    }
    for (int k = 0; k < 2; ++k)
        if (n[k] && !bl::gemv_fits(part[k], n[k], k == 1, false))
            return BL_ERR_SHAPE;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    for (int k = 0; k < 2 && e == hipSuccess; ++k)
        if (n[k])
            e = bl::launch_gemv_tiles(part[k], n[k], k == 1, st);
    return from_hip(e);
}

bl_status bitlinear_calib_stream(const void *buf, int64_t bytes, uint32_t *xor_out, void *stream)
{
    if (bytes < 0 || bytes % 16 != 0)
        return BL_ERR_SHAPE;
    if (!xor_out || (bytes > 0 && !buf))
        return BL_ERR_NULL;
    if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(xor_out) & 3u))
        return BL_ERR_ALIGN;
    if (bytes == 0)
        return BL_OK;
    return from_hip(bl::launch_calib_stream(buf, bytes, xor_out, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_calib_mfma(int kind, int iters, int blocks, int32_t *out, void *stream)
{
    if (kind != 0 && kind != 1)
        return BL_ERR_DTYPE;
    if (iters <= 0 || blocks <= 0 || iters > (kind == 1 ? (1 << 16) : (1 << 21)))
        return BL_ERR_SHAPE;
    if (!out)
        return BL_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(out) & 3u)
        return BL_ERR_ALIGN;
    return from_hip(bl::launch_calib_mfma(kind, iters, blocks, out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
