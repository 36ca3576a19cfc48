/*
 * oracle.c — plain, slow CPU oracle for the BitNet b1.58 BitLinear forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this file:
 * it is used by the test suite, by the package's smoke check and by the benchmark's CPU
 * baseline, and nowhere else.  It shares no code, header or table with the GPU library.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC (x86-64, SSE2,
 * round-to-nearest-even environment).  Every function is single-threaded and written as the
 * plain definition of its step, one element at a time.
 *
 * The five steps, with the passages they follow:
 *   O1  gamma    — absmean weight scale gamma = mean(|W|) over one weight tensor.
 *                  Distillix README, "Key Innovations 1. BitNet b1.58 Core" (W_q formula);
 *                  bitone README, "Features": Triton BitLinear forward (separate 1-D
 *                  reduction for gamma = mean(|W|)); SLM750-Edge card §3.1 "every linear
 *                  weight tensor" (its alpha formula is garbled into a mean of a max; the
 *                  mean-|W| reading of the other two pages is taken).
 *   O2  codes    — W_q = round(clip(W / gamma, -1, 1)), spelled out as the SLM750-Edge card
 *                  §3.1 round_clip rule: +1 if x > 0.5, 0 if |x| <= 0.5, -1 if x < -0.5
 *                  (the card's third case is cut off; -1 below -0.5 follows by symmetry).
 *   O3  packing  — 2 bits per weight, 16 weights per uint32 word, rows of K/16 words.
 *                  The pages fix only the density (Distillix README "Memory Footprint":
 *                  ~25 MB for ~100M weights = 2 bits each).  Field layout (a reading):
 *                  word w of row n holds k in [16w, 16w+16); weight k = 16w + 4i + b sits
 *                  at bits [8b + 2i, 8b + 2i + 1]; the field holds the code in 2-bit two's
 *                  complement (+1 -> 01, 0 -> 00, -1 -> 11; 10 is never written).
 *   O4  act quant— per-token absmax int8 quantization with scale absmax/127 (BitDistill
 *                  article: "activations are quantized to INT8"), optionally preceded by the
 *                  SubLN RMSNorm (BitDistill article, "Stage 1 — Architectural refinement
 *                  with SubLN"; SLM750-Edge card, "Key Architectural Features": RMSNorm,
 *                  epsilon 1e-6).  Fused-norm reading: the RMS factor r > 0 cancels in
 *                  q = round(y * 127 / max|y|) for y = r * (x . g), so codes come from
 *                  u = x . g and r enters only the scale.
 *   O5  matmul   — acc[m][n] = sum_k q[m][k] * c[n][k], exact integer (Y = X W_q^T, bitone
 *                  README "Features": Triton forward computes Y = X @ W_q^T x gamma).
 *   O6  epilogue — y[m][n] = fp32(acc * gamma * s_x[m]) evaluated in fp64.
 *
 * Layer chain (the BitLinear sub-graph of one transformer layer, for the chain tests):
 *   O7  FFN act  — the activation between the gate/up products and the down product's
 *                  quantization.  SLM750-Edge card, "Key Architectural Features": FFN
 *                  activation ReLU2 = relu(x)^2, and §2.3: a gate, an up and a down matrix per
 *                  layer, read as h = relu(gate)^2 * up (gated) or h = relu(x)^2 (one input);
 *                  the Distillix and Qwen3-shaped layer sets name SwiGLU gate/up projections:
 *                  h = silu(gate) * up with silu(g) = g / (1 + exp(-g)).  Each is evaluated in
 *                  fp64 from the fp32 inputs and rounded to fp32 once (a reading).
 *   O8  residual — y_out = fp32(y + r): the BitLinear output added to the residual stream,
 *                  y from O6, one fp32 addition.
 *
 * Weight-only forward and the straight-through backward (training-side rows):
 *   O9  fwd W1.58A16 — y[m][n] = fp32(gamma * sum_k x[m][k] * c[n][k]), x fp32 (bf16 widened
 *                  exactly), the sum in fp64 in k order (bitone README, "Features": the QAT
 *                  forward Y = X @ W_q^T x gamma with full-precision activations).
 *   O10 grad X   — dx[m][k] = fp32(gamma * sum_n dy[m][n] * c[n][k]), the sum in fp64 in n
 *                  order: the product's input gradient through the dequantized weights
 *                  gamma * c, the activation quantizer passing it unchanged (Distillix README,
 *                  "Key Innovations 1": STE, gradients pass through quantization unchanged;
 *                  BitDistill article: gradients through the quantizer use the STE).
 *   O11 STE scale— grad_scale(t) for t = fp32(W / gamma) (the O2 division): pass-through 1;
 *                  hard: 1 if |t| <= 1 else 0; soft: sech^2(beta t) = 1 - tanh^2(beta t), beta
 *                  2 by default (bitone README, "Soft-STE": the hard mask and its smooth
 *                  replacement).  fp64, sech^2 as 1 / cosh^2 (the same function without the
 *                  cancellation of 1 - tanh^2 for large |beta t|).
 *   O12 grad W   — dw[n][k] = fp32(grad_scale(t[n][k]) * sum_m dy[m][n] * xh[m][k]), the sum in
 *                  fp64 in m order, xh[m][k] = q[m][k] * s_x[m] the dequantized activation the
 *                  forward multiplied (fp64 product), or a full-precision x for the weight-only
 *                  forward.  gamma's own dependence on W is not differentiated (a reading: the
 *                  STE treats W_q * gamma as W).
 *
 * Base-3 packing (the denser weight format, for the decode product):
 *   O13 packing  — five ternary codes per byte (3^5 = 243 <= 256), 1.6 bits per weight: the
 *                  bitone README's "3B parameter model fits in 600 MB" and its size table
 *                  (700M -> 0.14 GB, 3B -> 0.6 GB, 8B -> 1.6 GB) are 1.6 bits per weight.  Layout (a
 *                  reading; the pages give only the density): a row of K weights is cut into
 *                  blocks of 80 (16 bytes, the last block padded with code 0); byte b of block j
 *                  holds the five weights k_0..k_4 = 80j + 4b + 0..3 and 80j + 64 + b as the
 *                  base-3 number sum_i (c_{k_i} + 1) * 3^i (values 0..242).  Row n takes
 *                  16 * ceil(K / 80) bytes.
 *
 * Degenerate data (defined here, the pages are silent): gamma == 0 gives all codes 0; a row
 * with absmax 0 gives q = 0 and s_x = 0.  NaN inputs are outside the method's domain; where
 * a comparison meets a NaN the result is code 0.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

/* ---------------------------------------------------------------- O1: gamma = mean |W| */

/* Sum |W| over all `count` elements in row-major order in fp64, divide by the element
 * count in fp64, round to fp32 (round to nearest even).  The fp64 mean is returned through
 * `gamma64` when it is non-NULL (used to locate rounding-boundary weights). */
float oracle_gamma(const float *W, int64_t count, double *gamma64)
{
    double sum = 0.0;
    for (int64_t i = 0; i < count; ++i)
        sum += fabs((double)W[i]);
    double mean = count > 0 ? sum / (double)count : 0.0;
    if (gamma64)
        *gamma64 = mean;
    return (float)mean;
}

/* ------------------------------------------------- O2: ternary codes, round_clip(W/gamma) */

static int8_t round_clip(float x)
{
    if (x > 0.5f)
        return 1;
    if (x < -0.5f)
        return -1;
    return 0; /* |x| <= 0.5, ties included; NaN also lands here */
}

void oracle_ternary_codes(const float *W, int64_t count, float gamma, int8_t *codes)
{
    for (int64_t i = 0; i < count; ++i) {
        if (gamma == 0.0f) {
            codes[i] = 0;
            continue;
        }
        float t = W[i] / gamma; /* one IEEE-754 fp32 division, round to nearest even */
        codes[i] = round_clip(t);
    }
}

/* ---------------------------------------------------------------- O3: 2-bit packing */

static unsigned field_shift(int64_t j) /* j = position inside the 16-weight group */
{
    int64_t i = j / 4, b = j % 4;
    return (unsigned)(8 * b + 2 * i);
}

/* codes [N][K] int8 in {-1,0,+1} -> packed [N][K/16] uint32.  Returns 0, or -1 when K is
 * not a multiple of 16, or -2 when a code is outside {-1, 0, +1}. */
int oracle_pack(const int8_t *codes, int64_t N, int64_t K, uint32_t *packed)
{
    if (K % 16 != 0)
        return -1;
    int64_t words = K / 16;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t w = 0; w < words; ++w) {
            uint32_t word = 0;
            for (int64_t j = 0; j < 16; ++j) {
                int c = codes[n * K + 16 * w + j];
                uint32_t field;
                if (c == 1)
                    field = 1u;
                else if (c == 0)
                    field = 0u;
                else if (c == -1)
                    field = 3u;
                else
                    return -2;
                word |= field << field_shift(j);
            }
            packed[n * words + w] = word;
        }
    }
    return 0;
}

/* packed [N][K/16] -> codes [N][K].  Returns 0, -1 for K % 16 != 0, -3 for a 10 field. */
int oracle_unpack(const uint32_t *packed, int64_t N, int64_t K, int8_t *codes)
{
    if (K % 16 != 0)
        return -1;
    int64_t words = K / 16;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t w = 0; w < words; ++w) {
            uint32_t word = packed[n * words + w];
            for (int64_t j = 0; j < 16; ++j) {
                uint32_t field = (word >> field_shift(j)) & 3u;
                int8_t c;
                if (field == 1u)
                    c = 1;
                else if (field == 0u)
                    c = 0;
                else if (field == 3u)
                    c = -1;
                else
                    return -3;
                codes[n * K + 16 * w + j] = c;
            }
        }
    }
    return 0;
}

/* O1 + O2 + O3 on one weight tensor W [N][K]. */
int oracle_quantize_weights(const float *W, int64_t N, int64_t K, int8_t *codes_scratch,
                            uint32_t *packed, float *gamma_out)
{
    float gamma = oracle_gamma(W, N * K, NULL);
    oracle_ternary_codes(W, N * K, gamma, codes_scratch);
    *gamma_out = gamma;
    return oracle_pack(codes_scratch, N, K, packed);
}

/* ------------------------------------------------ O4: per-token absmax int8 act quant */

static int8_t to_int8_clamped(float v)
{
    if (v > 127.0f)
        return 127;
    if (v < -127.0f)
        return -127;
    if (v != v)
        return 0;
    return (int8_t)v; /* v is already an integer value in [-127, 127] */
}

/* One token row x[0..K) (already widened to fp32).  g == NULL: plain absmax quantization.
 * g != NULL: SubLN RMSNorm with weight g and epsilon eps, fused as described in the header. */
static void quantize_row(const float *x, int64_t K, const float *g, float eps, int8_t *q,
                         float *s_x)
{
    float a = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float u = g ? x[k] * g[k] : x[k];
        float mag = fabsf(u);
        if (mag > a)
            a = mag;
    }
    if (a == 0.0f) {
        for (int64_t k = 0; k < K; ++k)
            q[k] = 0;
        *s_x = 0.0f;
        return;
    }
    float inv = 127.0f / a;
    for (int64_t k = 0; k < K; ++k) {
        float u = g ? x[k] * g[k] : x[k];
        float v = rintf(u * inv); /* round half to even */
        q[k] = to_int8_clamped(v);
    }
    if (!g) {
        *s_x = a / 127.0f;
    } else {
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k)
            ss += (double)x[k] * (double)x[k];
        double r = 1.0 / sqrt(ss / (double)K + (double)eps);
        *s_x = (float)((double)a * r / 127.0);
    }
}

void oracle_quantize_acts_f32(const float *X, int64_t M, int64_t K, const float *g, float eps,
                              int8_t *Xq, float *s_x)
{
    for (int64_t m = 0; m < M; ++m)
        quantize_row(X + m * K, K, g, eps, Xq + m * K, s_x + m);
}

/* bf16 rows are widened exactly to fp32 (the bf16 bits are the top half of the fp32 bits),
 * then quantized as above.  `row` is caller-provided scratch of K floats. */
void oracle_quantize_acts_bf16(const uint16_t *X, int64_t M, int64_t K, const float *g,
                               float eps, float *row, int8_t *Xq, float *s_x)
{
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) {
            union { uint32_t u; float f; } cv;
            cv.u = (uint32_t)X[m * K + k] << 16;
            row[k] = cv.f;
        }
        quantize_row(row, K, g, eps, Xq + m * K, s_x + m);
    }
}

/* ---------------------------------------------------- O5 + O6: integer product, rescale */

/* acc[m][n] = sum_k Xq[m][k] * C[n][k], summed in int64.  Returns 0, or -4 if a sum does not
 * fit in int32 (cannot happen for |q| <= 127 and K < 2^24). */
int oracle_matmul(const int8_t *Xq, const int8_t *C, int64_t M, int64_t N, int64_t K,
                  int32_t *acc)
{
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)Xq[m * K + k] * (int64_t)C[n * K + k];
            if (s > INT32_MAX || s < INT32_MIN)
                return -4;
            acc[m * N + n] = (int32_t)s;
        }
    }
    return 0;
}

/* y[m][n] = fp32( (double)acc * (double)gamma * (double)s_x[m] ), left to right in fp64. */
void oracle_epilogue(const int32_t *acc, const float *s_x, float gamma, int64_t M, int64_t N,
                     float *Y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            Y[m * N + n] = (float)((double)acc[m * N + n] * (double)gamma * (double)s_x[m]);
}

/* O5 + O6 for selected output entries (m_idx[i], n_idx[i]) of a product whose weights are
 * given packed [N][K/16]: each entry unpacks its weight row and sums K products.  Used to
 * check large shapes at sampled positions. */
int oracle_forward_entries(const int8_t *Xq, const float *s_x, const uint32_t *packed,
                           float gamma, int64_t K, const int64_t *m_idx, const int64_t *n_idx,
                           int64_t count, int8_t *row_scratch, int32_t *acc, float *Y)
{
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = m_idx[i], n = n_idx[i];
        int rc = oracle_unpack(packed + n * (K / 16), 1, K, row_scratch);
        if (rc)
            return rc;
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k)
            s += (int64_t)Xq[m * K + k] * (int64_t)row_scratch[k];
        if (s > INT32_MAX || s < INT32_MIN)
            return -4;
        acc[i] = (int32_t)s;
        Y[i] = (float)((double)acc[i] * (double)gamma * (double)s_x[m]);
    }
    return 0;
}

/* ---------------------------------------------------------- O7: FFN activation (chain) */

/* Activation kinds: 1 = SwiGLU h = silu(x) * x2, 2 = gated ReLU^2 h = relu(x)^2 * x2,
 * 3 = ReLU^2 h = relu(x)^2 (x2 unused).  fp64 evaluation; this is the fp64 value before the
 * one rounding to fp32 (tests use it to tell where that rounding is close to a tie). */
double oracle_ffn_act1_f64(int kind, float x, float x2)
{
    double v;
    if (kind == 1) {
        v = ((double)x / (1.0 + exp(-(double)x))) * (double)x2;
    } else if (kind == 2) {
        double r = x > 0.0f ? (double)x : 0.0;
        v = r * r * (double)x2;
    } else {
        double r = x > 0.0f ? (double)x : 0.0;
        v = r * r;
    }
    return v;
}

/* The activation rounded once to fp32. */
float oracle_ffn_act1(int kind, float x, float x2)
{
    return (float)oracle_ffn_act1_f64(kind, x, x2);
}

/* H = act(X, X2) elementwise over `count` values (X2 may be NULL for kind 3). */
void oracle_ffn_act(int kind, const float *X, const float *X2, int64_t count, float *H)
{
    for (int64_t i = 0; i < count; ++i)
        H[i] = oracle_ffn_act1(kind, X[i], X2 ? X2[i] : 0.0f);
}

/* The same, unrounded: H64 = the fp64 value of each activation. */
void oracle_ffn_act_f64(int kind, const float *X, const float *X2, int64_t count, double *H64)
{
    for (int64_t i = 0; i < count; ++i)
        H64[i] = oracle_ffn_act1_f64(kind, X[i], X2 ? X2[i] : 0.0f);
}

/* ------------------------------------------------------- O8: residual epilogue (chain) */

/* y[m][n] = fp32( fp32((double)acc * (double)gamma * (double)s_x[m]) + r[m][n] ). */
void oracle_epilogue_residual(const int32_t *acc, const float *s_x, float gamma,
                              const float *R, int64_t M, int64_t N, float *Y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float y = (float)((double)acc[m * N + n] * (double)gamma * (double)s_x[m]);
            Y[m * N + n] = y + R[m * N + n];
        }
}

/* ------------------------------------------- O9: weight-only ternary forward (W1.58A16) */

/* Y[m][n] = fp32(gamma * sum_k X[m][k] * c[n][k]); codes [N][K] int8. */
void oracle_forward_wonly(const float *X, const int8_t *C, float gamma, int64_t M, int64_t N,
                          int64_t K, float *Y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += (double)X[m * K + k] * (double)C[n * K + k];
            Y[m * N + n] = (float)((double)gamma * s);
        }
}

/* ---------------------------------------------------- O10: input gradient through the STE */

/* dX[m][k] = fp32(gamma * sum_n dY[m][n] * c[n][k]); dY [M][N], codes [N][K]. */
void oracle_grad_input(const float *dY, const int8_t *C, float gamma, int64_t M, int64_t N,
                       int64_t K, float *dX)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            double s = 0.0;
            for (int64_t n = 0; n < N; ++n)
                s += (double)dY[m * N + n] * (double)C[n * K + k];
            dX[m * K + k] = (float)((double)gamma * s);
        }
}

/* ---------------------------------------------------------- O11: STE gradient scale */

/* kind 0: pass-through, 1: hard mask, 2: soft sech^2(beta t).  t = fp32(w / gamma) as in O2
 * (gamma == 0: t is taken as 0, the scale of a zero tensor's weights). */
double oracle_ste_scale(int kind, float w, float gamma, double beta)
{
    const float t = gamma == 0.0f ? 0.0f : w / gamma;
    if (kind == 0)
        return 1.0;
    if (kind == 1)
        return fabsf(t) <= 1.0f ? 1.0 : 0.0;
    const double c = cosh(beta * (double)t);
    return 1.0 / (c * c);
}

/* --------------------------------------------------------- O12: weight gradient (STE) */

/* dW[n][k] = fp32(scale(W[n][k]) * sum_m dY[m][n] * xh[m][k]) with xh = Xq * s_x (Xq != NULL)
 * or xh = Xf.  W may be NULL for the pass-through kind.  dY [M][N], activations [M][K]. */
void oracle_grad_weight(const float *dY, const int8_t *Xq, const float *s_x, const float *Xf,
                        const float *W, float gamma, int kind, double beta, int64_t M,
                        int64_t N, int64_t K, float *dW)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            double s = 0.0;
            for (int64_t m = 0; m < M; ++m) {
                const double xh = Xq ? (double)Xq[m * K + k] * (double)s_x[m] : (double)Xf[m * K + k];
                s += (double)dY[m * N + n] * xh;
            }
            const double sc = kind == 0 ? 1.0 : oracle_ste_scale(kind, W[n * K + k], gamma, beta);
            dW[n * K + k] = (float)(sc * s);
        }
}

/* ------------------------------------------------------------- O13: base-3 packing */

/* Weight index of digit i of byte b in block j. */
static int64_t b3_weight(int64_t j, int b, int i)
{
    return 80 * j + (i < 4 ? 4 * b + i : 64 + b);
}

/* Bytes per row of the base-3 layout. */
int64_t oracle_b3_row_bytes(int64_t K)
{
    return 16 * ((K + 79) / 80);
}

/* codes [N][K] in {-1, 0, +1} -> bytes [N][16 * ceil(K/80)].  Returns 0, or -2 for a code
 * outside {-1, 0, +1}. */
int oracle_pack_b3(const int8_t *codes, int64_t N, int64_t K, uint8_t *out)
{
    const int64_t rb = oracle_b3_row_bytes(K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < rb / 16; ++j)
            for (int b = 0; b < 16; ++b) {
                unsigned v = 0, p = 1;
                for (int i = 0; i < 5; ++i) {
                    const int64_t k = b3_weight(j, b, i);
                    int c = 0;
                    if (k < K) {
                        c = codes[n * K + k];
                        if (c < -1 || c > 1)
                            return -2;
                    }
                    v += (unsigned)(c + 1) * p;
                    p *= 3;
                }
                out[n * rb + 16 * j + b] = (uint8_t)v;
            }
    return 0;
}

/* bytes [N][16 * ceil(K/80)] -> codes [N][K].  Returns 0, or -3 for a byte above 242. */
int oracle_unpack_b3(const uint8_t *in, int64_t N, int64_t K, int8_t *codes)
{
    const int64_t rb = oracle_b3_row_bytes(K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < rb / 16; ++j)
            for (int b = 0; b < 16; ++b) {
                unsigned v = in[n * rb + 16 * j + b];
                if (v > 242)
                    return -3;
                for (int i = 0; i < 5; ++i) {
                    const int64_t k = b3_weight(j, b, i);
                    if (k < K)
                        codes[n * K + k] = (int8_t)((int)(v % 3) - 1);
                    v /= 3;
                }
            }
    return 0;
}
