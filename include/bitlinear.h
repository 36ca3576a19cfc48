/*
 * bitlinear.h — C ABI of the BitNet b1.58 BitLinear forward for AMD Instinct MI355X (gfx950).
 *
 * The forward has five steps (Distillix README, "Key Innovations 1. BitNet b1.58 Core";
 * bitone README, "Features": Triton-fused BitLinear forward; SLM750-Edge 1.58-bit model card,
 * §3.1 "Ternary Weight Quantization"; BitDistill article, "Stage 1 — Architectural refinement
 * with SubLN" and its INT8-activation deployment):
 *
 *   1. gamma = mean(|W|) over one weight tensor W [N][K]          bitlinear_quantize_weights
 *   2. ternary codes c = round(clip(W / gamma, -1, 1)), packed    bitlinear_quantize_weights
 *      2 bits per weight, 16 per uint32                           (or bitlinear_pack_codes)
 *   3. per-token absmax int8 activations (optionally with the     bitlinear_quantize_acts
 *      SubLN RMSNorm folded in)
 *   4. acc = X_q · c^T, exact int32                               bitlinear_forward
 *   5. Y = acc · gamma · s_x, fp32                                bitlinear_forward
 *
 * General rules for every entry point:
 *   * Deliberate differences from a textbook C signature: the stream is passed as void* (a
 *     hipStream_t, NULL = the legacy default stream), so that a plain C caller or a ctypes
 *     binding needs no HIP header; the activation dtype is passed as int (a bl_dtype value),
 *     for the same reason; and K is limited to BL_MAX_K (below), far under the 127 * K < 2^31
 *     bound of the exact int32 product, because the kernels accumulate 64 * acc.
 *   * Every pointer argument is a DEVICE pointer (HIP device memory visible to the GPU that
 *     owns `stream`), owned by the caller, 16-byte aligned, and the tensor behind it is dense
 *     row-major.  Pointers to empty tensors (a zero dimension) may be NULL.  The library never
 *     allocates, frees, copies to the host or synchronizes.
 *   * `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).  All work
 *     is enqueued on it and the call returns at once; results are ready when the stream is.
 *   * A non-zero status means the arguments were rejected: nothing was launched and no output
 *     was written.  BL_ERR_HIP means a launch failed after validation (outputs undefined).
 *     Faults inside kernels surface asynchronously, at the caller's next synchronization.
 *   * Data values are not checked (NaN/Inf are outside the method's domain; see below for
 *     the degenerate cases that are defined).
 *   * Calls are stateless and thread-safe; two calls on different streams may run
 *     concurrently when their output buffers do not overlap.
 *
 * Packed weight layout (the pages fix only the density — Distillix README, "Memory
 * Footprint": ~25 MB for ~100M weights, 2 bits each): row n of W_packed holds K/16 uint32
 * words; word w holds k in [16w, 16w+16); the code of weight k = 16w + 4i + b sits at bits
 * [8b + 2i, 8b + 2i + 1] as a 2-bit two's complement value (+1 -> 01, 0 -> 00, -1 -> 11;
 * 10 is never written and undefined on input).  Shifting a word left by 6 - 2i and masking
 * with 0xC0C0C0C0 yields four int8 lanes equal to 64 * c for k = 16w + 4i + 0..3, which is
 * how the kernels feed the integer dot-product and matrix units.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BL_OK = 0,
    BL_ERR_NULL = -1,      /* a required pointer is NULL */
    BL_ERR_SHAPE = -2,     /* a size is negative, K % 16 != 0, or K / M / N above the limits */
    BL_ERR_ALIGN = -3,     /* a pointer is not 16-byte aligned */
    BL_ERR_DTYPE = -4,     /* unknown activation dtype */
    BL_ERR_WORKSPACE = -5, /* workspace smaller than bitlinear_quantize_weights_workspace() */
    BL_ERR_HIP = -6,       /* a HIP launch failed */
    BL_ERR_COUNT = -7      /* grouped call: count <= 0 or above BL_MAX_GROUP */
} bl_status;

typedef enum { BL_F32 = 0, BL_BF16 = 1 } bl_dtype;

/* K limit: 64 * 127 * K must fit in int32.  The kernels feed the int8 matrix unit the codes as
 * 64 * c (one shift and one mask per four weights, see the layout above) and divide the int32
 * sum by 64 at the end, so the bound is 64 * 127 * K < 2^31, not 127 * K < 2^31. */
#define BL_MAX_K 262144
/* M and N limit (row counts are held in 32-bit integers inside the kernels). */
#define BL_MAX_ROWS 2147483647LL
/* Largest number of problems one grouped call accepts. */
#define BL_MAX_GROUP 16

/* Human-readable name of a status code (static string, never NULL). */
const char *bitlinear_status_string(int status);

/* ABI version of this library (major * 100 + minor). */
int bitlinear_abi_version(void);

/* ---------------------------------------------------------------------------------------
 * Steps 1 + 2: weight quantization.
 *
 * Distillix README, "1. BitNet b1.58 Core": W_q = round(clip(W / mean(|W|), -1, 1)).
 * bitone README, "Features": gamma = mean(|W|) comes from a separate one-dimensional
 * reduction over W, and the quantized weights are never materialized as int8/fp tensors.
 * SLM750-Edge card §3.1: round_clip(x) = +1 for x > 0.5, 0 for |x| <= 0.5, -1 below -0.5.
 *
 *   W          [N][K] fp32, row-major (N = output features, K = input features).
 *   W_packed   [N][K/16] uint32 out, layout above.
 *   gamma      [1] fp32 out: fl32(sum_{n,k} |W[n][k]| / (N K)), the sum taken in fp64 in a
 *              fixed order (so repeated calls on the same data give the same bits).
 *   workspace  device scratch of at least bitlinear_quantize_weights_workspace(N, K) bytes;
 *              it may be reused between calls on the same stream.
 * Codes are round_clip(fl32(W / gamma)) for every element, with the division rounded to
 * nearest even; gamma == 0 gives all-zero codes.  N == 0 writes gamma = 0 and nothing else.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE (N < 0, K <= 0, K % 16 != 0, K > BL_MAX_K),
 * BL_ERR_ALIGN, BL_ERR_WORKSPACE.
 * ------------------------------------------------------------------------------------- */
size_t bitlinear_quantize_weights_workspace(int64_t N, int64_t K);

/* The same size under the name this library's first specification gave the query (the
 * workspace holds per-tensor partial sums, so the size does not depend on N or K). */
size_t bitlinear_workspace_bytes(int64_t N, int64_t K);

bl_status bitlinear_quantize_weights(const float *W, int64_t N, int64_t K, uint32_t *W_packed,
                                     float *gamma, void *workspace, size_t workspace_bytes,
                                     void *stream);

/* One weight tensor of a grouped weight quantization. */
typedef struct {
    const float *W;
    uint32_t *W_packed;
    float *gamma;
    int64_t N, K;
} bl_weight_problem;

/* Grouped form: up to BL_MAX_GROUP independent tensors in two kernel launches.  Each problem
 * has the same semantics as bitlinear_quantize_weights; the workspace must hold at least
 * bitlinear_quantize_weights_grouped_workspace(count) bytes. */
size_t bitlinear_quantize_weights_grouped_workspace(int count);

bl_status bitlinear_quantize_weights_grouped(const bl_weight_problem *problems, int count,
                                             void *workspace, size_t workspace_bytes,
                                             void *stream);

/* Workspace with which bitlinear_quantize_weights_grouped, bitlinear_quantize_step and
 * bitlinear_quantize_step_quad_rows read every fp32 master once instead of twice (steps 1 and
 * 2 as above, the same codes and gamma bit for bit).  The one-read form samples one 4 KB piece
 * of every 64 KB of W for an estimate of gamma, and during the gamma pass writes each code
 * against a band around the estimated threshold, listing the weights inside the band; a short
 * fix-up pass then reduces gamma exactly, checks that the exact threshold lies inside the
 * band and decides the listed weights against it (or, where the check fails or a list
 * overflowed, codes that part of W again from gamma).  It is taken for sets of at least 64 MB
 * of fp32 weights with every tensor below 2 GiB, when workspace_bytes is at least this size
 * (about 0.31 N K bytes plus 1.3 MiB per tensor); otherwise the calls read W twice, as with the
 * smaller workspace.  Returns 0 for an invalid array, count or shape (the errors the calls
 * report as BL_ERR_NULL, BL_ERR_COUNT and BL_ERR_SHAPE).  The workspace may be reused between
 * calls on the same stream; calls that overlap on different streams need their own. */
size_t bitlinear_quantize_weights_one_read_workspace(const bl_weight_problem *problems, int count);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): bitlinear_quantize_weights_grouped
 * without a workspace argument.  The partial sums go to a fixed scratch array inside the
 * library (2 KiB per tensor, room for BL_MAX_GROUP tensors: 32 KiB per GPU, held until the
 * process ends); the call allocates nothing.  Every call on one GPU shares that GPU's array,
 * so two such calls that overlap on one GPU (different streams, or host threads) race and
 * must be serialized by the caller; a call writes every partial sum it reads, so nothing has
 * to be cleared between calls.  Results are bit for bit those of
 * bitlinear_quantize_weights_grouped.  Errors: as for bitlinear_quantize_weights_grouped
 * (BL_ERR_WORKSPACE if the call needed more partial sums than the scratch holds), and
 * BL_ERR_HIP if the stream's device or the scratch's address cannot be had. */
bl_status bitlinear_quantize_weights_grouped_noalloc(const bl_weight_problem *problems, int count,
                                                     void *stream);

/* ---------------------------------------------------------------------------------------
 * Step 2 for weights that are already ternary (pre-ternarized checkpoints): pack int8 codes.
 *
 *   codes      [N][K] int8 in {-1, 0, +1}; any other value gives an undefined field.
 *   W_packed   [N][K/16] uint32 out.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN.
 * ------------------------------------------------------------------------------------- */
bl_status bitlinear_pack_codes(const int8_t *codes, int64_t N, int64_t K, uint32_t *W_packed,
                               void *stream);

/* ---------------------------------------------------------------------------------------
 * Step 3: per-token absmax int8 activation quantization, optionally with SubLN RMSNorm.
 *
 * BitDistill article: ternary weights with INT8 activations; SubLN is inserted before the
 * attention output projection and before the FFN output projection.  SLM750-Edge card,
 * "Key Architectural Features": RMSNorm with epsilon 1e-6.
 *
 *   X          [M][K] fp32 (x_dtype = BL_F32) or bf16 (BL_BF16), row-major.
 *   norm_weight NULL: u = x.  Otherwise [K] fp32 RMSNorm weight g, u = fl32(x * g).
 *   eps        RMSNorm epsilon (ignored without norm_weight).
 *   X_q        [M][K] int8 out: q = clamp(rint(fl32(u * fl32(127 / a))), -127, 127) with
 *              a = max_k |u_k| and rint rounding half to even.
 *   x_scale    [M] fp32 out: a / 127 without norm; fl32(a * r / 127) with norm, where
 *              r = 1 / sqrt(mean_k(x_k^2) + eps) in fp64.  The RMS factor r > 0 cancels in
 *              the codes, so it enters only the scale.
 * A row with a == 0 gives q = 0 and x_scale = 0.  M == 0 is a no-op.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE (M < 0, K <= 0, K % 16 != 0, K > BL_MAX_K),
 * BL_ERR_ALIGN, BL_ERR_DTYPE.
 * ------------------------------------------------------------------------------------- */
bl_status bitlinear_quantize_acts(const void *X, int x_dtype, int64_t M, int64_t K,
                                  const float *norm_weight, float eps, int8_t *X_q,
                                  float *x_scale, void *stream);

/* One activation matrix of a grouped activation quantization. */
typedef struct {
    const void *X;
    const float *norm_weight;
    int8_t *X_q;
    float *x_scale;
    int64_t M, K;
    int x_dtype;
    float eps;
} bl_act_problem;

/* Grouped form: up to BL_MAX_GROUP independent matrices in one kernel launch. */
bl_status bitlinear_quantize_acts_grouped(const bl_act_problem *problems, int count,
                                          void *stream);

/* ---------------------------------------------------------------------------------------
 * Steps 1 + 2 and step 3 of one forward step in one call: a weight set's quantization and an
 * input set's activation quantization.
 *
 * Distillix README, "1. BitNet b1.58 Core", and bitone README, "Features": a training-style
 * step re-quantizes the weights (gamma, then the codes) and quantizes the step's activations;
 * the two depend on different inputs (W, X), so the gamma reduction and the activation codes
 * can run side by side.
 *
 *   weights, nw, workspace, workspace_bytes   as for bitlinear_quantize_weights_grouped
 *                   (0 <= nw <= BL_MAX_GROUP; weights may be NULL and the workspace is not
 *                   needed when nw == 0).
 *   acts, na        as for bitlinear_quantize_acts_grouped (0 <= na <= BL_MAX_GROUP; may be
 *                   NULL when na == 0).
 * Results: bit for bit those of the two grouped calls.  With the one-read workspace
 * (bitlinear_quantize_weights_one_read_workspace) and a large enough weight set: the sample,
 * the one-read pass, the fix-up beside the activation rows longer than 4096 values, then the
 * other activation rows.  Otherwise, when every non-empty activation problem has K <= 4096 and
 * one dtype, the gamma pass and the activation quantization share one launch and the pack pass
 * follows (two launches instead of three), else the two calls run in order.  The activation
 * rows are read with the non-temporal hint (a step's inputs are read once; left uncached they
 * do not evict the codes that the step's product reads next); bitlinear_quantize_acts_grouped
 * reads them through the caches.  The two sets run concurrently: no buffer one set writes may
 * be read or written by the other.
 * Errors: BL_ERR_COUNT (nw or na outside 0 .. BL_MAX_GROUP, or both 0), BL_ERR_NULL (a NULL
 * array with a nonzero count, or no workspace with nw > 0), then each problem's errors as for
 * the two calls, BL_ERR_ALIGN / BL_ERR_WORKSPACE for the workspace, and BL_ERR_SHAPE when the
 * activation rows exceed 2^31 - 1.  Every problem is validated before anything is launched.
 * ------------------------------------------------------------------------------------- */
bl_status bitlinear_quantize_step(const bl_weight_problem *weights, int nw, void *workspace,
                                  size_t workspace_bytes, const bl_act_problem *acts, int na,
                                  void *stream);

/* ---------------------------------------------------------------------------------------
 * Steps 4 + 5: ternary x int8 product with int32 accumulation and the rescale epilogue.
 *
 * bitone README, "Features": Y = X @ W_q^T x gamma, weights [out, in] (nn.Linear layout);
 * bitone README, "What is bitone?": ternary weights turn the product into additions and
 * subtractions; the int8-activation scale s_x joins gamma in the epilogue.
 *
 *   X_q        [M][K] int8 (from bitlinear_quantize_acts).
 *   x_scale    [M] fp32.
 *   W_packed   [N][K/16] uint32.
 *   gamma      [1] fp32 (device pointer, so a re-quantized gamma never visits the host).
 *   Y          [M][N] fp32 out: fl32(fp64(acc * gamma * x_scale[m])).
 *   acc        [M][N] int32 out, or NULL: acc[m][n] = sum_k X_q[m][k] * c[n][k], exact.
 * M <= 16 runs a bandwidth-bound streaming kernel (decode); larger M runs the int8
 * matrix-core kernel (prefill).  M == 0 or N == 0 is a no-op.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE (M < 0, N < 0, K <= 0, K % 16 != 0, K > BL_MAX_K),
 * BL_ERR_ALIGN.
 * ------------------------------------------------------------------------------------- */
bl_status bitlinear_forward(const int8_t *X_q, const float *x_scale, const uint32_t *W_packed,
                            const float *gamma, int64_t M, int64_t N, int64_t K, float *Y,
                            int32_t *acc, void *stream);

/* One product of a grouped forward. */
typedef struct {
    const int8_t *X_q;
    const float *x_scale;
    const uint32_t *W_packed;
    const float *gamma;
    float *Y;
    int32_t *acc;
    int64_t M, N, K;
} bl_forward_problem;

/* Grouped form: up to BL_MAX_GROUP independent products.  Problems with M <= 16 share one
 * decode launch and problems with M > 16 share one prefill launch. */
bl_status bitlinear_forward_grouped(const bl_forward_problem *problems, int count,
                                    void *stream);

/* ---------------------------------------------------------------------------------------
 * Steps 3 + 4 + 5 for a few tokens in one launch: the decode form of the layer call.
 *
 * Same arithmetic as bitlinear_quantize_acts followed by bitlinear_forward (BitDistill
 * article: INT8 activations into ternary-weight projections, SubLN before the output
 * projections), for the decode case where the activations are a handful of tokens and two
 * launches would cost more than the work: each block of the product quantizes the token rows
 * itself (absmax and, with a norm, the sum of squares over the whole row) and feeds the codes
 * to the product without a trip through global memory.
 *
 *   X, x_dtype, norm_weight, eps   as for bitlinear_quantize_acts ([M][K] activations).
 *   W_packed, gamma, Y             as for bitlinear_forward.
 *   X_q, x_scale                   optional outputs ([M][K] int8, [M] fp32), or NULL: the
 *                                  codes and scales the product used, identical to what
 *                                  bitlinear_quantize_acts returns for the same input.
 * The codes equal bitlinear_quantize_acts' bit for bit; x_scale and Y equal the two-call
 * result except that, with a norm, the sum of squares is added in another fixed order (the
 * scale may differ in its last bit).
 * Fused when M <= 4 and M * K <= 49152; other problems take the two-step path and then need
 * X_q and x_scale as the intermediate buffers (BL_ERR_NULL otherwise).  M == 0 or N == 0 is
 * a no-op.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_DTYPE.
 * ------------------------------------------------------------------------------------- */
typedef struct {
    const void *X;
    const float *norm_weight;
    const uint32_t *W_packed;
    const float *gamma;
    float *Y;
    int8_t *X_q;
    float *x_scale;
    int64_t M, N, K;
    int x_dtype;
    float eps;
} bl_linear_problem;

/* Largest token count and activation bytes (M * K) of the fused decode form. */
#define BL_LINEAR_FUSED_MAX_M 4
#define BL_LINEAR_FUSED_MAX_BYTES 49152

/* Up to BL_MAX_GROUP independent layer calls; all fused ones share one launch. */
bl_status bitlinear_linear_grouped(const bl_linear_problem *problems, int count, void *stream);

/* ---------------------------------------------------------------------------------------
 * Layer chain: the two extensions the BitLinear sub-graph of a transformer layer needs.
 *
 * BitDistill article, "Stage 1 — Architectural refinement with SubLN": SubLN before the
 * attention output projection and before the FFN output projection.  SLM750-Edge card, "Key
 * Architectural Features": FFN activation ReLU2 = relu(x)^2, RMSNorm epsilon 1e-6; §2.3: a
 * gate, an up and a down matrix per layer.  The Distillix and Qwen3-shaped layer sets name
 * SwiGLU gate/up projections.
 *
 * (1) Activation quantization with the FFN activation in front (the down projection's input):
 *     h = act(X, X2) per element, evaluated in fp64 from the fp32 inputs and rounded to fp32
 *     once, then quantized exactly as bitlinear_quantize_acts quantizes x (with the optional
 *     SubLN RMSNorm over h: codes from fl32(h * g), scale from the RMS of h):
 *       BL_ACT_SWIGLU     h = silu(X) * X2, silu(g) = g / (1 + exp(-g))
 *       BL_ACT_RELU2_GLU  h = relu(X)^2 * X2
 *       BL_ACT_RELU2      h = relu(X)^2            (X2 unused, may be NULL)
 *     With an activation, X and X2 are fp32 (the gate and up products' outputs) [M][K].
 *     Otherwise (BL_ACT_NONE) the problem is exactly a bitlinear_quantize_acts problem.
 *     The fp64 exp is the device library's; it may differ from another libm in its last
 *     bit, which changes the fp32 h only when that value lies within 2^-52 (relative) of an
 *     fp32 rounding midpoint.
 * (2) Products with a residual: Y = fl32(fl32(fp64(acc * gamma * x_scale[m])) + R[m][n]) —
 *     the projection's output added to the residual stream in the epilogue, R fp32 [M][N]
 *     (may alias Y; each element is read before it is written by the same thread).
 * ------------------------------------------------------------------------------------- */
typedef enum { BL_ACT_NONE = 0, BL_ACT_SWIGLU = 1, BL_ACT_RELU2_GLU = 2, BL_ACT_RELU2 = 3 } bl_act_kind;

typedef struct {
    const void *X;            /* [M][K]; the gate output for the GLU kinds */
    const float *X2;          /* [M][K] fp32 up output for the GLU kinds, else NULL */
    const float *norm_weight; /* [K] SubLN / RMSNorm weight, or NULL */
    int8_t *X_q;
    float *x_scale;
    int64_t M, K;
    int x_dtype;              /* BL_F32 or BL_BF16 (BL_F32 whenever act != BL_ACT_NONE) */
    int act;                  /* bl_act_kind */
    float eps;
} bl_act_ex_problem;

/* Up to BL_MAX_GROUP activation problems of either form in one call.  Errors as for
 * bitlinear_quantize_acts_grouped, plus BL_ERR_DTYPE for an unknown act kind or a bf16
 * input with an activation, and BL_ERR_NULL for a GLU kind without X2. */
bl_status bitlinear_quantize_acts_ex_grouped(const bl_act_ex_problem *problems, int count,
                                             void *stream);

typedef struct {
    const int8_t *X_q;
    const float *x_scale;
    const uint32_t *W_packed;
    const float *gamma;
    float *Y;
    int32_t *acc;
    const float *residual;    /* [M][N] fp32 added to the output, or NULL */
    int64_t M, N, K;
} bl_forward_ex_problem;

/* Up to BL_MAX_GROUP products, each with an optional residual.  Errors as for
 * bitlinear_forward_grouped (BL_ERR_ALIGN also for a residual not 4-byte aligned). */
bl_status bitlinear_forward_ex_grouped(const bl_forward_ex_problem *problems, int count,
                                       void *stream);

/* ---------------------------------------------------------------------------------------
 * Mixed batch: one chunk of prompt tokens (prefill) and a few decode tokens in one call.
 *
 * SLM750-Edge card, "Performance": inference has a prompt-processing phase and a single-token
 * decode phase (the latter bandwidth-bound); both run the same BitLinear forward (steps 3 to
 * 5), and a serving step that batches a prompt chunk with other requests' decode tokens runs
 * both sets of products.
 *
 *   prefill, npre   products with quantized activations, as for bitlinear_forward_ex_grouped
 *                   (0 <= npre <= BL_MAX_GROUP; may be NULL when npre == 0).
 *   decode, ndec    layer calls, as for bitlinear_linear_grouped (0 <= ndec <= BL_MAX_GROUP;
 *                   may be NULL when ndec == 0).
 * Results: bit for bit those of bitlinear_forward_ex_grouped(prefill, npre) followed by
 * bitlinear_linear_grouped(decode, ndec).  When every non-empty prefill product has M > 16
 * and the products take 128 x 128 tiles (they do while the set has fewer than 256 units of
 * 256 x 256 outputs; larger sets take 128 x 256 tiles), and every
 * non-empty decode call takes the fused form with one activation dtype, both sets share one
 * launch: the decode blocks run on the compute units the product's last tiles leave idle.
 * Otherwise the two calls run in that order on the stream.
 * The two sets run concurrently: no buffer one set writes may be read or written by the
 * other.
 * Errors: BL_ERR_COUNT (npre or ndec outside 0 .. BL_MAX_GROUP, or both 0), BL_ERR_NULL (a
 * NULL array with a nonzero count), then each problem's errors as for the two calls, and
 * BL_ERR_SHAPE when the launch would exceed 2^31 - 1 blocks.  Every problem is validated
 * before anything is launched.
 * ------------------------------------------------------------------------------------- */
bl_status bitlinear_forward_mixed(const bl_forward_ex_problem *prefill, int npre,
                                  const bl_linear_problem *decode, int ndec, void *stream);

/* ---------------------------------------------------------------------------------------
 * (3) The decode form of a layer's product calls: bitlinear_linear_grouped's fused call
 *     (activation quantization inside the product) with the layer's output stages in the
 *     epilogue, so that a layer's BitLinear sub-graph at a few tokens takes three launches
 *     (attention projections, FFN gate/up, FFN down) instead of six.
 *
 *   X, x_dtype, norm_weight, eps, X_q, x_scale   as for bl_linear_problem.
 *   W_packed, gamma    the projection (or the gate projection of a gated pair), [N][K/16].
 *   W2_packed, gamma2  the up projection of a gated pair ([N][K/16], the same codes layout),
 *                      or NULL for a single projection.
 *   act                BL_ACT_NONE or BL_ACT_RELU2 for a single projection; BL_ACT_SWIGLU or
 *                      BL_ACT_RELU2_GLU for a gated pair.
 *   residual           [M][N] fp32 added last, or NULL (may alias Y).
 *   Y                  [M][N] fp32:
 *     y1 = fl32(fp64(acc1 * gamma * x_scale[m]))   (the bitlinear_forward output)
 *     y2 = fl32(fp64(acc2 * gamma2 * x_scale[m]))  (gated pairs: the up output)
 *     h  = act(y1, y2) as in (1): fp64 evaluation from the fp32 inputs, one fp32 rounding
 *          (BL_ACT_NONE: h = y1)
 *     Y  = residual ? fl32(h + residual) : h
 *   So Y equals bitlinear_forward of both projections followed by the activation (and the
 *   residual add) element for element; only the fused form exists: every problem with
 *   M > 0 and N > 0 needs M <= BL_LINEAR_FUSED_MAX_M and M * K <= BL_LINEAR_FUSED_MAX_BYTES.
 *   M == 0 or N == 0 is a no-op.
 * Errors: BL_ERR_NULL (X, W_packed, gamma or Y missing; W2_packed or gamma2 missing for a
 * gated kind), BL_ERR_DTYPE (unknown x_dtype or act, a gated kind without a pair or a pair
 * with a single kind), BL_ERR_SHAPE (as for bl_linear_problem, and sizes past the fused
 * form), BL_ERR_ALIGN (16 bytes for X, W_packed, W2_packed, X_q, norm_weight; 4 bytes for
 * the fp32 arrays).  Pair problems and single problems of one call take one launch each.
 * ------------------------------------------------------------------------------------- */
typedef struct {
    const void *X;
    const float *norm_weight;
    const uint32_t *W_packed;
    const float *gamma;
    const uint32_t *W2_packed;
    const float *gamma2;
    float *Y;
    const float *residual;
    int8_t *X_q;
    float *x_scale;
    int64_t M, N, K;
    int x_dtype;
    int act;
    float eps;
} bl_linear_ex_problem;

bl_status bitlinear_linear_ex_grouped(const bl_linear_ex_problem *problems, int count,
                                      void *stream);

/* ---------------------------------------------------------------------------------------
 * Training side: the weight-only forward and the straight-through backward.
 *
 * bitone README, "Features": the QAT forward Y = X @ W_q^T x gamma with full-precision
 * activations, and "Soft-STE": the weight gradient's hard mask and its smooth replacement
 * grad_scale = 1 - tanh^2(beta * W / gamma) = sech^2(beta * W / gamma), beta 2 by default.
 * Distillix README, "Key Innovations 1" and the BitDistill article: gradients pass through
 * the quantizers unchanged (STE).
 *
 * Arithmetic: the products run on the bf16 matrix cores with fp32 accumulation.  Codes
 * (0, +-1) and int8 activation codes are exact in bf16; fp32 operands are carried as two
 * bf16 parts (16 significant bits, relative error <= 2^-16 per term); bf16 operands are
 * exact.  Results are the exact sums up to fp32 accumulation: for a contraction of length L
 * over terms a_i, |error| <= (L * 2^-24 + 2^-16 [fp32 operands] ) * sum |a_i| + one fp32
 * rounding of the scaled result.  Sums are not bit-reproducible against a serial order.
 * ------------------------------------------------------------------------------------- */

/* (1) Weight-only ternary forward: Y[m][n] = fp32(gamma * sum_k X[m][k] * c[n][k]).
 *   X          [M][K] fp32 or bf16 (x_dtype), 16-byte aligned.
 *   W_packed   [N][K/16] packed codes (the bitlinear_quantize_weights layout).
 *   gamma      [1] fp32.   Y  [M][N] fp32.
 * M == 0 or N == 0 is a no-op.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE (as bitlinear_forward), BL_ERR_ALIGN, BL_ERR_DTYPE. */
typedef struct {
    const void *X;
    const uint32_t *W_packed;
    const float *gamma;
    float *Y;
    int64_t M, N, K;
    int x_dtype;
} bl_wonly_problem;

bl_status bitlinear_forward_wonly_grouped(const bl_wonly_problem *problems, int count,
                                          void *stream);

/* (2) The transposed code matrix: Wt_packed [K][N/16] holds c[n][k] at row k, field n, in the
 * same packed layout (needs N % 16 == 0 and N <= BL_MAX_K).  Run once per weight update; the
 * input gradient reads it.  N == 0 is a no-op.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN. */
bl_status bitlinear_transpose_packed(const uint32_t *W_packed, int64_t N, int64_t K,
                                     uint32_t *Wt_packed, void *stream);

/* (3) Input gradient: dX[m][k] = fp32(gamma * sum_n dY[m][n] * c[n][k]) (through the
 * activation quantizer unchanged; the caller applies the norm's backward if the forward
 * fused one).
 *   dY         [M][N] fp32 or bf16 (dy_dtype).
 *   Wt_packed  [K][N/16]: bitlinear_transpose_packed of the forward's W_packed.
 *   gamma      the forward's gamma.   dX  [M][K] fp32.
 * Needs N % 16 == 0, N <= BL_MAX_K, K > 0, K % 16 == 0.  M == 0 is a no-op. */
typedef struct {
    const void *dY;
    const uint32_t *Wt_packed;
    const float *gamma;
    float *dX;
    int64_t M, N, K;
    int dy_dtype;
} bl_grad_input_problem;

bl_status bitlinear_grad_input_grouped(const bl_grad_input_problem *problems, int count,
                                       void *stream);

/* (4) Weight gradient: dW[n][k] = fp32(scale(W[n][k]) * sum_m dY[m][n] * X_q[m][k] * x_scale[m])
 * (dY times the dequantized activations the forward multiplied, through the weight
 * quantizer by the STE), scale from t = fl32(W / gamma) (the quantizer's division; gamma ==
 * 0 gives t = 0):
 *   BL_STE_PASS  1                      (W may be NULL)
 *   BL_STE_HARD  1 if |t| <= 1, else 0
 *   BL_STE_SOFT  sech^2(beta * t), evaluated in fp64
 *   dY [M][N] fp32; X_q [M][K] int8 and x_scale [M] from the forward's activation
 *   quantization; W [N][K] fp32 masters; dW [N][K] fp32 (M == 0 writes zeros).
 * Needs K > 0, K % 16 == 0, K <= BL_MAX_K, N <= BL_MAX_K.  N == 0 is a no-op.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN (16 bytes for every array but gamma and
 * x_scale), BL_ERR_DTYPE (unknown ste kind). */
typedef enum { BL_STE_PASS = 0, BL_STE_HARD = 1, BL_STE_SOFT = 2 } bl_ste_kind;

typedef struct {
    const float *dY;
    const int8_t *X_q;
    const float *x_scale;
    const float *W;
    const float *gamma;
    float *dW;
    int64_t M, N, K;
    int ste;
    float beta;
} bl_grad_weight_problem;

bl_status bitlinear_grad_weight_grouped(const bl_grad_weight_problem *problems, int count,
                                        void *stream);

/* ---------------------------------------------------------------------------------------
 * Base-3 weights: five codes per byte, 1.6 bits per weight.
 *
 * bitone README, "What is bitone?" and its size table: a 3B-parameter model in 600 MB (700M in
 * 0.14 GB, 8B in 1.6 GB), i.e. 1.6 bits per weight (3^5 = 243 <= 256).  Layout (a reading; the
 * pages give only the density): each row of K weights is cut into blocks of 80 weights stored
 * in 16 bytes (the last block padded with code 0); byte b of block j holds the five weights
 * k = 80j + 4b + 0..3 and 80j + 64 + b, as the base-3 number sum_i (c_{k_i} + 1) * 3^i (0..242:
 * digit i of the first four is weight 4b + i).  A row takes
 * bitlinear_b3_row_bytes(K) = 16 * ceil(K / 80) bytes; rows are contiguous.  The decode product
 * reads 20 % fewer weight bytes than the two-bit layout (K a multiple of 80) and expands the
 * codes with integer arithmetic in registers.
 * ------------------------------------------------------------------------------------- */
int64_t bitlinear_b3_row_bytes(int64_t K);

/* Two-bit packed codes W_packed [N][K/16] -> base-3 bytes W_b3 [N][bitlinear_b3_row_bytes(K)].
 * N == 0 is a no-op.  Errors: BL_ERR_NULL, BL_ERR_SHAPE (as bitlinear_pack_codes),
 * BL_ERR_ALIGN (both 16-byte aligned). */
bl_status bitlinear_pack_b3(const uint32_t *W_packed, int64_t N, int64_t K, uint8_t *W_b3,
                            void *stream);

/* The fused decode layer call (bitlinear_linear_grouped's fused form: activation quantization,
 * product and epilogue in one launch) on base-3 weights: each problem's W_packed points to the
 * problem's base-3 bytes [N][bitlinear_b3_row_bytes(K)] (16-byte aligned).  Results are
 * bit-identical to bitlinear_linear_grouped on the same codes in the two-bit layout.  Every
 * problem with M > 0 and N > 0 needs M <= BL_LINEAR_FUSED_MAX_M and M * K <=
 * BL_LINEAR_FUSED_MAX_BYTES (BL_ERR_SHAPE otherwise); X_q and x_scale are optional outputs.
 * Errors as for bitlinear_linear_grouped. */
bl_status bitlinear_linear_b3_grouped(const bl_linear_problem *problems, int count, void *stream);

/* ---------------------------------------------------------------------------------------
 * Decode tiles: the same two-bit codes arranged for the one-token product.
 *
 * SLM750-Edge card, "Performance": single-token decode is bandwidth-bound, so its weight
 * stream should run at the memory's rate.  The one-token product feeds the int8 matrix unit
 * 16 weight rows at a time, one 16-byte piece of each of 16 rows per lane group, and from
 * [N][K/16] rows each of its load instructions gathers 16 rows x 64 bytes (measured: 3.55
 * TB/s, against 5.0 TB/s for 1 KB contiguous per instruction).  The tile layout (this
 * library's own, not the pages') stores every group of 16 rows (16 rg .. 16 rg + 15) and every
 * 256 weights of K (super-step T) as one contiguous KB: 16-byte chunk l = 16 g + r (r, g in
 * 0..15, 0..3) holds the codes of row 16 rg + r for k = 256 T + 64 g .. 256 T + 64 g + 63 (the
 * weights that the chunk's lane multiplies) as four 32-bit little-endian dwords i = 0..3, and
 * bits 8 b + 2 j .. 8 b + 2 j + 1 of dword i hold the code c of k = 256 T + 64 g + 16 j + 4 i + b:
 * as c mod 4 (two's complement) for j = 3, as c + 1 for j = 0, 1, 2.  With one mask per dword
 * the product then reads every plane j as int8 values 4^j (c + 1) or 64 c, without shifts.
 * Rows past N and k past K hold c = 0.  Tile (rg, T) starts at byte (rg * ceil(K / 256) + T) *
 * 1024.  Same codes, same bytes per weight (plus the padding).
 * ------------------------------------------------------------------------------------- */

/* Bytes of the tile layout of an N x K weight matrix: ceil(N / 16) * ceil(K / 256) * 1024
 * (0 for N < 0 or K not a positive multiple of 16). */
int64_t bitlinear_tiles_bytes(int64_t N, int64_t K);

/* Two-bit packed codes W_packed [N][K/16] -> W_tiles [bitlinear_tiles_bytes(N, K) bytes].
 * N == 0 is a no-op.  Errors: BL_ERR_NULL, BL_ERR_SHAPE (K not a positive multiple of 16, or
 * past the limits of bitlinear_pack_codes), BL_ERR_ALIGN (both 16-byte aligned). */
bl_status bitlinear_pack_tiles(const uint32_t *W_packed, int64_t N, int64_t K, uint32_t *W_tiles,
                               void *stream);

/* The fused one-token layer call (bitlinear_linear_grouped's fused form at M == 1:
 * activation quantization, product and epilogue in one launch) on tiled weights: each
 * problem's W_packed points to the problem's tiles (16-byte aligned).  Results are
 * bit-identical to bitlinear_linear_grouped on the same codes in the two-bit layout.  Every
 * problem with N > 0 needs M == 1 (or M == 0: skipped), K % 64 == 0 and K <= 12288 (the
 * one-token kernel's limits), BL_ERR_SHAPE otherwise; X_q and x_scale are optional outputs.
 * Other errors as for bitlinear_linear_grouped; nothing is launched on an error. */
bl_status bitlinear_linear_tiles_grouped(const bl_linear_problem *problems, int count, void *stream);

/* ---------------------------------------------------------------------------------------
 * Quad rows: the same two-bit words arranged for the prefill product's weight loads.
 *
 * bitone README, "Features": the fused BitLinear GEMM (Y = X @ W_q^T x gamma).  The prefill
 * product stages 128 weights of K at a time, i.e. 32 bytes of each of its weight rows, and
 * from [N][K/16] rows every 128-byte line it touches serves one row's stage piece (a quarter
 * of the line per request; measured: the 8192-token product of the Qwen3-4B set 5 % faster
 * with whole-line requests).  The quad-row layout (this library's own, not the pages')
 * needs N % 4 == 0 and K % 128 == 0 and permutes the words of every four rows: for rows
 * 4 q .. 4 q + 3 and stage t (words 8 t .. 8 t + 7 of each row), one 128-byte line holds the
 * four rows' 32-byte pieces in row order.  Word w of row n sits at word
 * ((n / 4) * (K / 128) + w / 8) * 32 + 8 * (n % 4) + w % 8; same size as the rows (N * K / 4
 * bytes), no padding.
 * ------------------------------------------------------------------------------------- */

/* Two-bit rows W_packed [N][K/16] -> W_quad (N * K / 4 bytes, not overlapping W_packed).
 * N == 0 is a no-op.  Errors: BL_ERR_NULL, BL_ERR_SHAPE (N % 4 != 0, K % 128 != 0, the
 * limits of bitlinear_pack_codes, or N * K / 16 >= 2^32), BL_ERR_ALIGN (both 16-byte
 * aligned). */
bl_status bitlinear_pack_quad_rows(const uint32_t *W_packed, int64_t N, int64_t K, uint32_t *W_quad,
                                   void *stream);

/* bitlinear_quantize_step with every weight problem's W_packed receiving the quad-row layout
 * (the same words as bitlinear_quantize_step writes, permuted; gamma and the activation
 * results unchanged).  Every weight problem needs N % 4 == 0, K % 128 == 0 and
 * N * K / 16 < 2^32 (BL_ERR_SHAPE); other errors as for bitlinear_quantize_step. */
bl_status bitlinear_quantize_step_quad_rows(const bl_weight_problem *weights, int nw,
                                            void *workspace, size_t workspace_bytes,
                                            const bl_act_problem *acts, int na, void *stream);

/* bitlinear_forward_grouped on weights in the quad-row layout: one prefill launch, results
 * (Y and the optional int32 acc) bit-identical to bitlinear_forward_grouped on the same codes
 * in rows.  Every problem with M > 0 and N > 0 needs M > 16 (the prefill product; decode-sized
 * products read rows), N % 4 == 0, K % 128 == 0 and N * K / 16 < 2^32, BL_ERR_SHAPE
 * otherwise; empty problems are skipped.  Other errors as for bitlinear_forward_grouped;
 * nothing is launched on an error. */
bl_status bitlinear_forward_quad_rows_grouped(const bl_forward_problem *problems, int count,
                                              void *stream);

/* bitlinear_forward_ex_grouped (the layer chain's products, with the optional residual added
 * in the epilogue) on weights in the quad-row layout: the same limits and errors as
 * bitlinear_forward_quad_rows_grouped, otherwise as bitlinear_forward_ex_grouped; results
 * bit-identical to bitlinear_forward_ex_grouped on the same codes in rows. */
bl_status bitlinear_forward_ex_quad_rows_grouped(const bl_forward_ex_problem *problems, int count,
                                                 void *stream);

/* ---------------------------------------------------------------------------------------
 * Measurement helpers (not part of the method): what this GPU attains, so that a kernel's
 * roofline can be quoted against a measured peak beside the published one.
 * ------------------------------------------------------------------------------------- */

/* Reads buf [bytes] once with 16-byte loads (a grid of up to 8 blocks per compute unit,
 * eight loads in flight per thread) and XORs all its 32-bit words into *xor_out, which the
 * caller zeroes first (so the result is the XOR of the buffer's words and no load can be
 * skipped).  bytes % 16 == 0; buf 16-byte aligned, xor_out 4-byte aligned; bytes == 0 is a
 * no-op.  Errors: BL_ERR_SHAPE, BL_ERR_NULL, BL_ERR_ALIGN. */
bl_status bitlinear_calib_stream(const void *buf, int64_t bytes, uint32_t *xor_out, void *stream);

/* `blocks` blocks of 256 threads; every wave runs 8 independent accumulators through `iters`
 * matrix-unit operations on constant operands: kind 0 = int8 16x16x64 (A = B = 1; 32768
 * operations each), kind 1 = bf16 16x16x32 (A = B = 1.0; 16384 floating-point operations
 * each).  Total operations = blocks * 4 * 8 * iters * (32768 or 16384).  Thread t of block b
 * writes out[256 b + t] = 8 * iters * 64 (int8) or 8 * iters * 32 (bf16).  1 <= iters <= 2^21
 * (int8) or 2^16 (bf16, so the sums stay exact in fp32); out holds 256 * blocks int32.
 * Errors: BL_ERR_DTYPE (kind), BL_ERR_SHAPE, BL_ERR_NULL, BL_ERR_ALIGN. */
bl_status bitlinear_calib_mfma(int kind, int iters, int blocks, int32_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
