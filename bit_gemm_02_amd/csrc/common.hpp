// common.hpp — device helpers and launcher declarations shared by the BitLinear kernels.
//
// Internal to libbitlinear: nothing here is part of the C ABI (include/bitlinear.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bitlinear.h"

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ----------------------------------------------------------------- buffer loads
//
// Raw buffer loads through a buffer resource: an offset at or past `bytes` returns zeros
// instead of touching memory, so ragged tiles need no per-lane branch (a branch around a
// load forces the compiler to wait for it inside the branch).  Offsets are 32-bit, so each
// resource covers at most one tile's rows (always far below 4 GiB).
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// An offset that is out of range for every resource (each covers < 2^31 bytes) and does not
// wrap when the access size is added: loads from it return zeros.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    // Third descriptor word for gfx9-family raw (untyped) buffer access.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ v4u buf_load16(rsrc_t r, uint32_t offset)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)offset, 0, 0);
}

// The same with the non-temporal policy, for data read once per launch (a weight stream):
// it is not kept in the caches for reuse.
__device__ __forceinline__ v4u buf_load16_nt(rsrc_t r, uint32_t offset)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)offset, 0, 2);
}

__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t offset)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)offset, 0, 0);
}

__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t offset, v4u value)
{
    __builtin_amdgcn_raw_buffer_store_b128(value, r, (int)offset, 0, 0);
}

// The same with the non-temporal policy, for output written once and not read back by the
// launch: it is not kept in the caches (evicting operands other blocks still read).
__device__ __forceinline__ void buf_store16_nt(rsrc_t r, uint32_t offset, v4u value)
{
    __builtin_amdgcn_raw_buffer_store_b128(value, r, (int)offset, 0, 2);
}

// Whole-line output stores from a 16 x 16 MFMA result layout.  Lane (r, g), r = lane % 16,
// g = lane / 16, holds four consecutive fp32 outputs of tile row r at columns 4g .. 4g + 3 of
// two adjacent 16-column groups: e (columns 0-15) and o (columns 16-31).  Lanes r and r ^ 8
// exchange one piece (a DPP rotation by 8 within each row of 16 lanes), after which one
// 16-byte store per lane writes tile rows 0-7 and a second one rows 8-15, each row as one
// 128-byte segment of 32 outputs (instead of 16 rows of 64 bytes per store), with the
// non-temporal policy.  `off` is the byte offset of row (r & 7), column 4g + (r < 8 ? 0 : 16)
// in `res`; `pitch8` is eight rows' bytes.
__device__ __forceinline__ void store_pair_lines_nt(rsrc_t res, uint32_t off, uint32_t pitch8,
                                                    bool lo, v4u e, v4u o)
{
    v4u v1, v2;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        // r < 8 sends its piece of o to r + 8 and receives that lane's piece of e; r >= 8 the
        // other way round.
        const uint32_t snd = lo ? o[v] : e[v];
        const uint32_t rcv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)snd, 0x128, 0xF, 0xF, false);
        v1[v] = lo ? e[v] : rcv;      // row (r & 7)
        v2[v] = lo ? rcv : o[v];      // row (r & 7) + 8
    }
    buf_store16_nt(res, off, v1);
    buf_store16_nt(res, off + pitch8, v2);
}

// Bytes of rows [r0, min(r0 + rows, R)) of a row-major matrix with `row_bytes` per row.
__device__ __forceinline__ uint32_t rows_bytes(int r0, int rows, int R, int row_bytes)
{
    const int live = R - r0 < rows ? R - r0 : rows;
    return live > 0 ? (uint32_t)live * (uint32_t)row_bytes : 0u;
}

// Dispatch order -> work order.  Workgroups are handed to the 8 XCDs round-robin
// (block b runs on XCD b % 8); remapping gives each XCD a contiguous range of a problem's
// nb tiles, so tiles that share an operand panel run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_order(int b, int nb)
{
    const int xcd = b & 7, i = b >> 3;
    const int q = nb >> 3, r = nb & 7;
    return xcd < r ? xcd * (q + 1) + i : r * (q + 1) + (xcd - r) * q + i;
}

// ----------------------------------------------------------------- direct-to-LDS loads

// Raw buffer descriptor as four scalar dwords: base address, stride 0, size in bytes, and
// the gfx9-family raw-access word.  Offsets at or past `bytes` read zero.
__device__ __forceinline__ v4i make_desc(const void *base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)base;
    v4i d;
    d.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    d.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFFu));
    d.z = __builtin_amdgcn_readfirstlane((int)bytes);
    d.w = 0x00020000;
    return d;
}

// LDS byte address of a shared-memory pointer, wave-uniform.
__device__ __forceinline__ uint32_t lds_addr(const unsigned char *p)
{
    typedef __attribute__((address_space(3))) const unsigned char lds_uchar;
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_uchar *)p);
}

// Direct-to-LDS 16-byte buffer load (gfx950): lane l's 16 bytes land at LDS address
// lds + 16 * l; an out-of-range offset writes zeros.  Issued from inline assembly so that the
// compiler does not model it: modelled, it cannot tell buffers in flight apart and drains
// every load before the first LDS read that follows.  The instruction has no register
// result; its completion is ordered by the caller's explicit vmcnt waits and barriers, and
// the "memory" clobber keeps LDS accesses from moving across it.  (The compiler's own waits
// stay correct: they count only the loads it knows of, and waiting for a later load also
// waits for every earlier one, these included.)
__device__ __forceinline__ void dma16(v4i desc, uint32_t lds, uint32_t offset)
{
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(offset), "s"(desc)
                 : "memory", "m0");
}

// Workgroup barrier that is also a compiler barrier for memory operations (the barrier
// instruction alone does not stop the compiler from moving LDS accesses across it), without
// the waits a memory fence would add.
__device__ __forceinline__ void block_sync()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Barrier for LDS traffic only: every LDS access of this wave has completed (lgkmcnt(0)),
// then s_barrier.  __syncthreads() also waits for every outstanding vector-memory load of the
// wave (vmcnt(0)); where loads still in flight do not feed the LDS data being handed over,
// this barrier lets the waves go on without them.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xF | (3 << 14) | (7 << 4) | (0 << 8));   // vmcnt max, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) lgkmcnt(0): wait until at most N vector-memory loads of this wave
// (direct-to-LDS ones included) are still in flight and every LDS read of this wave has
// returned.  The second part matters before a barrier that hands an LDS buffer back to
// the loads: a read of the buffer about to be refilled may have been issued before the
// barrier and not yet returned, and it could still be queued behind other LDS traffic when
// another wave's refill lands (a bare s_barrier does not wait for LDS reads).
template <int N>
__device__ __forceinline__ void wait_stage()
{
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// ----------------------------------------------------------------- packed-code planes
//
// A packed word holds 16 codes; the code of weight k = 16w + 4i + b lives at bits
// [8b + 2i, 8b + 2i + 1] in 2-bit two's complement.  Shifting left by 6 - 2i moves plane i
// to the top two bits of every byte; masking with 0xC0C0C0C0 leaves four int8 lanes holding
// 64 * c for k = 16w + 4i + 0..3 (01 -> 0x40 = 64, 11 -> 0xC0 = -64, 00 -> 0).  Integer
// dot products of these bytes are therefore exactly 64x the ternary dot product; the kernels
// divide by 64 (an exact arithmetic shift) before the epilogue.
__device__ __forceinline__ uint32_t plane64(uint32_t word, int i)
{
    return (word << (6 - 2 * i)) & 0xC0C0C0C0u;
}

// The four planes of a word, as the 16-byte operand of one 16x16x64 int8 MFMA lane:
// byte 4i + b of the result is 64 * c for k = 16w + 4i + b (natural k order).
__device__ __forceinline__ v4i unpack_word64(uint32_t word)
{
    v4i r;
    r.x = (int)plane64(word, 0);
    r.y = (int)plane64(word, 1);
    r.z = (int)plane64(word, 2);
    r.w = (int)plane64(word, 3);
    return r;
}

// Quad-row layout of packed words (N % 4 == 0, K % 128 == 0; the same words as the rows
// [N][K/16], permuted within every group of four rows): for rows 4q .. 4q + 3 and every 128
// weights of K (stage t, words 8t .. 8t + 7 of a row), one 128-byte line holds the four
// rows' 32-byte pieces in row order.  Word w of row n, with wpr = K / 16 words per row, sits
// at word ((n / 4) * (wpr / 8) + w / 8) * 32 + 8 * (n % 4) + w % 8.  `wi` is the word's
// index in the rows layout, n * wpr + w (below 2^32).
__device__ __forceinline__ uint32_t quad_row_word(uint32_t wi, uint32_t wpr)
{
    const uint32_t n = wi / wpr, w = wi - n * wpr;
    return ((n >> 2) * (wpr >> 3) + (w >> 3)) * 32u + 8u * (n & 3u) + (w & 7u);
}

// 2-bit field of one code (+1 -> 01, 0 -> 00, -1 -> 11), from "is nonzero" and "is negative".
__device__ __forceinline__ uint32_t code_field(bool nonzero, bool negative)
{
    return nonzero ? (negative ? 3u : 1u) : 0u;
}

// ----------------------------------------------------------------- wave reductions

// Wave maximum with DPP lane moves (no LDS round trips): quad permutes and row mirrors give
// every lane its 16-lane row maximum, two row broadcasts carry rows 0-2 into row 3, and lane
// 63 is read back.  max is exact, so the order does not matter.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max(float v)
{
    const int o = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK,
                                              0xF, false);
    return fmaxf(v, __int_as_float(o));
}

__device__ __forceinline__ float wave_max(float v)
{
    v = dpp_max<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_max<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_max<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_max<0x140, 0xF>(v);  // row_mirror
    v = dpp_max<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_max<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Fixed butterfly order: every lane ends with the same value, and the order of additions
// depends only on the lane layout, so the result is reproducible bit for bit.
__device__ __forceinline__ double wave_sum_fixed(double v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = v + __shfl_xor(v, off, kWave);
    return v;
}

// ----------------------------------------------------------------- activation quantization
//
// Shared by the activation-quantization kernels and the fused decode path, so both produce
// the same codes and scales from the same absmax (and sum of squares).

// q = clamp(rint(u * inv), -127, 127) as an integer.  rint of the fp32 product (round half
// to even), then an exact integer clamp; the conversion maps NaN to 0 and saturates
// infinities, so the degenerate rows (127/a overflowing to inf, 0 * inf = NaN) give the
// same codes as clamping in floating point and sending NaN to 0.
__device__ __forceinline__ int quant_one(float u, float inv)
{
    const int i = (int)__builtin_rintf(u * inv);
    return min(max(i, -127), 127);
}

__device__ __forceinline__ char4 quant4(float4 u, float inv)
{
    const uint32_t b0 = (uint32_t)quant_one(u.x, inv) & 0xFFu;
    const uint32_t b1 = (uint32_t)quant_one(u.y, inv) & 0xFFu;
    const uint32_t b2 = (uint32_t)quant_one(u.z, inv) & 0xFFu;
    const uint32_t b3 = (uint32_t)quant_one(u.w, inv) & 0xFFu;
    const uint32_t w = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    char4 c;
    __builtin_memcpy(&c, &w, 4);
    return c;
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

// s_x of a row: a / 127, or a * r / 127 with r = 1 / sqrt(sum(x^2) / K + eps) in fp64 when the
// RMSNorm is fused; 0 for an all-zero row.
__device__ __forceinline__ float act_scale(float a, double ss, int K, float eps, bool norm)
{
    if (a == 0.0f)
        return 0.0f;
    if (!norm)
        return a / 127.0f;  // correctly rounded fp32 division
    const double r = 1.0 / sqrt(ss / (double)K + (double)eps);
    return (float)((double)a * r / 127.0);
}

// FFN activation (the down projection's input): h = act(x, x2) evaluated in fp64 from the
// fp32 inputs, rounded to fp32 once (SwiGLU: silu(x) * x2 with
// silu(g) = g / (1 + exp(-g)); gated ReLU^2: relu(x)^2 * x2; ReLU^2: relu(x)^2).
__device__ __forceinline__ float ffn_act(int kind, float x, float x2)
{
    double v;
    if (kind == BL_ACT_SWIGLU) {
        v = ((double)x / (1.0 + exp(-(double)x))) * (double)x2;
    } else if (kind == BL_ACT_RELU2_GLU) {
        const double r = x > 0.0f ? (double)x : 0.0;
        v = r * r * (double)x2;
    } else {
        const double r = x > 0.0f ? (double)x : 0.0;
        v = r * r;
    }
    return (float)v;
}

__device__ __forceinline__ float4 ffn_act4(int kind, float4 x, float4 x2)
{
    return make_float4(ffn_act(kind, x.x, x2.x), ffn_act(kind, x.y, x2.y),
                       ffn_act(kind, x.z, x2.z), ffn_act(kind, x.w, x2.w));
}

// The same activation for the bulk kernels, with a table-driven fp64 exp: e^t = 2^(k/64) e^r,
// k = rint(64 t / ln 2), r = t - k ln2/64 (two-part constant, |r| <= ln2/128), e^r by its
// degree-6 Taylor polynomial (truncation < 2^-64), 2^(j/64) = tab[j] from a 64-entry table in
// LDS (tab[j] = exp2(j / 64), built by the caller), then ldexp; silu(g) = g * (1 / (1 + e))
// with the reciprocal refined by one Newton step.  A few fp64 ulps from the exact value (the
// general-purpose exp and division are one to two ulps), so h, rounded to fp32, differs from
// that of any accurate fp64 evaluation only within a few 2^-52 of an fp32 midpoint.  Large
// |g| saturates as the library's exp does (e^800 = inf, e^-800 = 0); NaN propagates.
// About 12 fp64 operations per element instead of about 40.
// (Host-callable as well, so that it can be checked against the host library on the CPU.)
__host__ __device__ inline double exp_f64_tab(double t, const double *tab)
{
    t = t < -800.0 ? -800.0 : (t > 800.0 ? 800.0 : t);          // NaN compares false: kept
    constexpr double kInvStep = 92.332482616893656877;           // 64 / ln 2
    constexpr double kStepHi = 0x1.62e42fefa39efp-7;             // ln 2 / 64, leading part
    constexpr double kStepLo = 0x1.abc9e3b39803fp-62;            // ln 2 / 64 - kStepHi
    const double k = __builtin_rint(t * kInvStep);
    const int ki = (int)k;                                       // NaN -> 0: index stays valid
    double r = __builtin_fma(-k, kStepHi, t);
    r = __builtin_fma(-k, kStepLo, r);
    double q = __builtin_fma(r, 1.0 / 720.0, 1.0 / 120.0);
    q = __builtin_fma(q, r, 1.0 / 24.0);
    q = __builtin_fma(q, r, 1.0 / 6.0);
    q = __builtin_fma(q, r, 0.5);
    q = __builtin_fma(q, r, 1.0);
    q = __builtin_fma(q, r, 1.0);
    return __builtin_ldexp(tab[ki & 63] * q, ki >> 6);
}

__device__ __forceinline__ float ffn_act_tab(int kind, float x, float x2, const double *tab)
{
    if (kind != BL_ACT_SWIGLU)
        return ffn_act(kind, x, x2);
    const double g = (double)x;
    const double d = 1.0 + exp_f64_tab(-g, tab);                 // >= 1, or inf, or NaN
    double y = __builtin_amdgcn_rcp(d);
    y = __builtin_fma(y, __builtin_fma(-d, y, 1.0), y);         // one Newton step
    y = d == __builtin_inf() ? 0.0 : y;                          // 1 / inf = 0 (the step gives NaN)
    return (float)((g * y) * (double)x2);
}

__device__ __forceinline__ float4 ffn_act4_tab(int kind, float4 x, float4 x2, const double *tab)
{
    return make_float4(ffn_act_tab(kind, x.x, x2.x, tab), ffn_act_tab(kind, x.y, x2.y, tab),
                       ffn_act_tab(kind, x.z, x2.z, tab), ffn_act_tab(kind, x.w, x2.w, tab));
}

// ----------------------------------------------------------------- bf16 matrix operands
//
// Ternary codes as bf16 MFMA operands (the weight-only product and the input gradient).

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma_bf16(v4u a, v4u b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Eight codes of a packed word as eight bf16 values (0, +1.0, -1.0): half j holds weights
// 8j .. 8j+7 of the word's 16, i.e. planes 2j and 2j+1 (weight 4i + b at bits 8b + 2i).
// Each byte of t = (w >> 2i) & 0x03030303 is one 2-bit field f (00 -> 0, 01 -> +1, 11 -> -1);
// v_perm_b32 looks the bf16 bytes up: selector byte f picks the low byte from kLutLo
// (0x00 or 0x80) and f + 4 the high byte from kLutHi (0x00, 0x3F or 0xBF).  The unused field
// value 10 maps to 0.
constexpr uint32_t kLutLo = 0x80008000u;   // bytes for f = 0..3: 00 80 00 80
constexpr uint32_t kLutHi = 0xBF003F00u;   // bytes for f = 0..3: 00 3F 00 BF

__device__ __forceinline__ uint32_t bf16_pair(uint32_t t, uint32_t t4, uint32_t sel)
{
    // sel picks [t.byte a, t4.byte a, t.byte a+1, t4.byte a+1] = [f, f + 4, f', f' + 4].
    return __builtin_amdgcn_perm(kLutHi, kLutLo, __builtin_amdgcn_perm(t4, t, sel));
}

__device__ __forceinline__ v4u ternary_bf16(uint32_t w, int j)
{
    const uint32_t t0 = (w >> (4 * j)) & 0x03030303u;
    const uint32_t t1 = (w >> (4 * j + 2)) & 0x03030303u;
    const uint32_t u0 = t0 + 0x04040404u, u1 = t1 + 0x04040404u;
    return v4u{bf16_pair(t0, u0, 0x05010400u), bf16_pair(t0, u0, 0x07030602u),
               bf16_pair(t1, u1, 0x05010400u), bf16_pair(t1, u1, 0x07030602u)};
}

// ----------------------------------------------------------------- launchers

// quad: write the packed words in the quad-row layout (quad_row_word) instead of rows.
// workspace_bytes: with at least quantize_weights_one_read_workspace(p, count) bytes, a large
// enough set reads W once (the one-read form, same codes and gamma); else W is read twice.
hipError_t launch_quantize_weights(const bl_weight_problem *p, int count, void *workspace,
                                   hipStream_t stream, bool quad = false, size_t workspace_bytes = 0);
size_t quantize_weights_workspace(int count);
size_t quantize_weights_one_read_workspace(const bl_weight_problem *p, int count);
hipError_t launch_pack_codes(const int8_t *codes, int64_t N, int64_t K, uint32_t *W_packed,
                             hipStream_t stream);
// nt: read the rows with the non-temporal hint (a step's fresh inputs, read once).
hipError_t launch_quantize_acts(const bl_act_ex_problem *p, int count, hipStream_t stream,
                                bool nt = false);
hipError_t launch_forward_decode(const bl_forward_ex_problem *p, int count, hipStream_t stream);
// Fused decode form: every problem has M <= BL_LINEAR_FUSED_MAX_M and M * K within
// BL_LINEAR_FUSED_MAX_BYTES.
hipError_t launch_linear_decode(const bl_linear_ex_problem *p, int count, hipStream_t stream);
// One-token form of the fused decode call (gemv.hip): every problem has M == 1; one kind per
// launch (single projections or gated pairs, one activation dtype); gemv_fits says whether the
// problems' rows fit its LDS budget.
bool gemv_fits(const bl_linear_ex_problem *const *p, int count, bool bf16, bool b3);
hipError_t launch_gemv(const bl_linear_ex_problem *const *p, int count, bool pair, bool bf16,
                       hipStream_t stream);
// The same on base-3 rows (single projections; W_packed holds bitlinear_pack_b3's rows).
hipError_t launch_gemv_b3(const bl_linear_ex_problem *const *p, int count, bool bf16,
                          hipStream_t stream);
hipError_t launch_gemv_tiles(const bl_linear_ex_problem *const *q, int count, bool bf16,
                             hipStream_t stream);
int64_t tiles_bytes(int64_t N, int64_t K);
hipError_t launch_pack_tiles(const uint32_t *P, int64_t N, int64_t K, uint32_t *out,
                             hipStream_t stream);
// quad: W_packed of every problem is in the quad-row layout (N % 4 == 0, K % 128 == 0).
hipError_t launch_forward_prefill(const bl_forward_ex_problem *p, int count, hipStream_t stream,
                                  bool quad = false);
hipError_t launch_pack_quad_rows(const uint32_t *P, int64_t N, int64_t K, uint32_t *out,
                                 hipStream_t stream);
// Weight quantization + activation quantization of one step.  One-read form (workspace large
// enough, set of 64 MB or more): sample, pass, fix-up beside the block kernel's activation rows,
// then the other activation rows; else the γ pass and the activation codes in one launch when
// every activation problem takes the wave kernel with one dtype, then the pack pass.  The
// activation rows are read non-temporally (a step's inputs, read once).
hipError_t launch_quantize_step(const bl_weight_problem *wq, int nw, void *workspace,
                                size_t workspace_bytes, const bl_act_ex_problem *aq, int na,
                                hipStream_t stream, bool quad = false);
// Mixed batch (prefill products + fused decode calls) in one launch: eligible when every
// prefill product has M > 16 and takes the 128 x 128 tile, and every decode call is a fused
// single projection (no pair, activation or residual) with one activation dtype.
bool mixed_eligible(const bl_forward_ex_problem *pre, int npre, const bl_linear_ex_problem *dec,
                    int ndec);
hipError_t launch_mixed(const bl_forward_ex_problem *pre, int npre, const bl_linear_ex_problem *dec,
                        int ndec, hipStream_t stream);

// Training-side products (train.hip).  Y[M][O] = gamma * A[M][Kc] T^T with T packed codes
// [O][Kc/16] and A fp32 or bf16: the weight-only forward, and the input gradient with the
// transposed codes.
struct WgProblem {
    const void *A;
    bool f32;
    const uint32_t *T;
    const float *gamma;
    float *Y;
    int64_t M, O, Kc;
};
hipError_t launch_wgemm(const WgProblem *p, int count, hipStream_t stream);
// The bf16-activation problems of a set, on the prefill pipeline (prefill.hip).
hipError_t launch_wonly_prefill(const WgProblem *p, int count, hipStream_t stream);
hipError_t launch_transpose_packed(const uint32_t *P, int64_t N, int64_t K, uint32_t *Pt,
                                   hipStream_t stream);
hipError_t launch_grad_weight(const bl_grad_weight_problem *p, int count, hipStream_t stream);

// Base-3 weights (five codes per byte): the packer and the fused decode call on them.
hipError_t launch_pack_b3(const uint32_t *P, int64_t N, int64_t K, uint8_t *out, hipStream_t stream);
hipError_t launch_linear_decode_b3(const bl_linear_ex_problem *p, int count, hipStream_t stream);
hipError_t launch_calib_stream(const void *buf, int64_t bytes, uint32_t *out, hipStream_t stream);
hipError_t launch_calib_mfma(int kind, int iters, int blocks, int32_t *out, hipStream_t stream);

// Token count up to which bitlinear_forward uses the decode (streaming) kernel.
constexpr int64_t kDecodeMaxM = 16;

}  // namespace bl
