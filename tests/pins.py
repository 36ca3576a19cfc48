"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

Every pin takes an oracle handle (``oracle.Oracle``) and raises ``AssertionError`` when the
oracle disagrees with the fact it checks.  The same pins run against the real oracle
(``test_oracle_pins.py``) and against copies of the oracle with a planted mistake
(``test_oracle_mutants.py``), where at least one pin must fail for every mistake.

None of these pins re-types the oracle's own code: they use hand-derived fixtures
(``tests/golden``), exact rational arithmetic, closed forms of the Gaussian, invariants of
the quantizers, numpy's library routines (``rint``, ``clip``, ``matmul``) on special cases,
and brute force on tiny inputs.
"""

from __future__ import annotations

import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32_of_fraction(fr: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) fp32 value of an exact rational."""
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    fr = abs(fr)
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1
    e = max(e, -126)  # below the normal range the spacing stays 2^-149
    scaled = fr * Fraction(2) ** (23 - e)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    value = Fraction(n) * Fraction(2) ** (e - 23)
    return np.float32(sign * float(value))


def _rng(*key):
    return np.random.Generator(np.random.PCG64([7, *key]))


# ------------------------------------------------------------------ O1: gamma = mean |W|

def pin_gamma_exact_rational(orc):
    """gamma equals the correctly rounded exact mean of |W| on small tensors."""
    for t in range(40):
        g = _rng(1, t)
        n = int(g.integers(1, 64))
        W = (g.standard_normal(n) * 0.02).astype(np.float32)
        exact = sum(Fraction(float(abs(w))) for w in W) / n
        got, _ = orc.gamma(W)
        assert got == f32_of_fraction(exact), (t, got, f32_of_fraction(exact))


def pin_gamma_hand_example(orc):
    fx = golden("round_clip_ties.json")
    W = np.array(fx["W"], dtype=np.float32)
    got, g64 = orc.gamma(W)
    assert got == np.float32(fx["gamma"]) and g64 == fx["gamma"]


def pin_gamma_closed_forms(orc):
    """Constant magnitude gives that magnitude; all-zero gives 0; scaling by 2^j is exact."""
    W = np.full((4, 32), -0.375, dtype=np.float32)
    W[::2] *= -1
    assert orc.gamma(W)[0] == np.float32(0.375)
    assert orc.gamma(np.zeros((3, 16), np.float32))[0] == 0.0
    X = workloads.gaussian((8, 64), (11,), 0.02)
    g0 = orc.gamma(X)[0]
    for j in (-3, 5):
        assert orc.gamma(X * np.float32(2.0 ** j))[0] == g0 * np.float32(2.0 ** j)


def pin_gamma_gaussian(orc):
    """W ~ N(0, s^2): E|W| = s * sqrt(2/pi); std of the mean of |z| is sqrt(1 - 2/pi)/sqrt(n)."""
    s = 0.02
    W = workloads.gaussian((1024, 1024), (12,), s)
    g, _ = orc.gamma(W)
    n = W.size
    tol = 5 * math.sqrt(1 - 2 / math.pi) / math.sqrt(n)
    assert abs(float(g) / s - math.sqrt(2 / math.pi)) < tol, float(g) / s


# ------------------------------------------------------------- O2: ternary codes

def pin_codes_tie_example(orc):
    fx = golden("round_clip_ties.json")
    W = np.array(fx["W"], dtype=np.float32)
    g, _ = orc.gamma(W)
    assert orc.ternary_codes(W, g).tolist() == fx["codes"]


def pin_codes_boundaries(orc):
    fx = golden("round_clip_ties.json")["boundary_cases_gamma_2"]
    ulp_up = 2.0 ** -24
    ulp_dn = 2.0 ** -25
    xs = [0.5, -0.5, 0.5 + ulp_up, -(0.5 + ulp_up), 0.5 - ulp_dn, -(0.5 - ulp_dn), 1, -1, 7, -7, 0]
    W = np.array([2.0 * x for x in xs], dtype=np.float32)
    assert orc.ternary_codes(W, np.float32(2.0)).tolist() == fx["codes"]


def pin_codes_match_rint_clip(orc):
    """round_clip(W/gamma) equals numpy rint(clip(W/gamma, -1, 1)) (round half to even) for
    finite inputs, on a dense sweep of ratios around the boundaries and at random."""
    gamma = np.float32(0.0173)
    t = np.concatenate([np.linspace(-2, 2, 4001, dtype=np.float32),
                        workloads.gaussian((4096,), (13,), 1.0)])
    W = (t * gamma).astype(np.float32)
    ref = np.rint(np.clip(W / gamma, np.float32(-1), np.float32(1))).astype(np.int8)
    assert np.array_equal(orc.ternary_codes(W, gamma), ref)


def pin_codes_ternary_and_gaussian_mix(orc):
    """Codes lie in {-1, 0, +1}; for Gaussian W the zero share is P(|z| <= sqrt(2/pi)/2)."""
    W = workloads.gaussian((1024, 1024), (14,), 0.02)
    g, _ = orc.gamma(W)
    c = orc.ternary_codes(W, g)
    assert set(np.unique(c).tolist()) <= {-1, 0, 1}
    n = c.size
    p0 = math.erf(math.sqrt(2 / math.pi) / 2 / math.sqrt(2))
    pm = (1 - p0) / 2
    tol = 5 * math.sqrt(0.25 / n)
    assert abs(np.mean(c == 0) - p0) < tol, (np.mean(c == 0), p0)
    assert abs(np.mean(c == 1) - pm) < tol and abs(np.mean(c == -1) - pm) < tol


def pin_codes_scaled_ternary_roundtrip(orc):
    """quantize(alpha * C) == C for ternary C with a nonzero entry and alpha > 0."""
    for t, alpha in enumerate((0.021, 1.0, 3.5e-3, 17.0)):
        C = workloads.ternary((64, 96), (15, t))
        W = (np.float32(alpha) * C.astype(np.float32)).astype(np.float32)
        g, _ = orc.gamma(W)
        assert np.array_equal(orc.ternary_codes(W, g), C)


def pin_codes_zero_gamma(orc):
    W = np.zeros((2, 16), np.float32)
    assert not orc.ternary_codes(W, np.float32(0.0)).any()


# ------------------------------------------------------------------ O3: packing

def pin_pack_golden_word(orc):
    fx = golden("pack_word.json")
    codes = np.array([fx["codes"]], dtype=np.int8)
    assert int(orc.pack(codes)[0, 0]) == int(fx["word_hex"], 16)


def pin_pack_roundtrip_and_density(orc):
    C = workloads.ternary((48, 160), (16,))
    P = orc.pack(C)
    assert P.shape == (48, 10) and P.nbytes == C.size // 4
    assert np.array_equal(orc.unpack(P, 160), C)
    fx = golden("footprint.json")
    assert fx["weights"] / 4 / 1e6 == fx["packed_megabytes_2bit"]


def pin_pack_fields_in_range(orc):
    """Every 2-bit field is 00, 01 or 11; field 10 never appears."""
    C = workloads.ternary((16, 256), (17,))
    P = orc.pack(C).astype(np.uint64)
    for s in range(0, 32, 2):
        assert not np.any(((P >> np.uint64(s)) & np.uint64(3)) == 2)


def pin_pack_locality(orc):
    """Changing the code at (n, k) changes only word (n, k // 16)."""
    C = workloads.ternary((4, 64), (18,))
    base = orc.pack(C)
    for n, k in ((0, 0), (1, 17), (3, 63), (2, 40)):
        D = C.copy()
        D[n, k] = 1 if C[n, k] != 1 else -1
        diff = np.argwhere(orc.pack(D) != base)
        assert diff.tolist() == [[n, k // 16]], (n, k, diff)


# ------------------------------------------------------------ O4: activation quant

def pin_acts_golden_ties(orc):
    fx = golden("act_quant_ties.json")
    q, s = orc.quantize_acts(np.array(fx["x"], dtype=np.float32))
    assert q.tolist() == fx["q"] and s.tolist() == fx["s_x"]


def pin_acts_properties(orc):
    X = workloads.gaussian((33, 200), (19,), 1.0)
    q, s = orc.quantize_acts(X)
    assert q.min() >= -127 and q.max() <= 127
    a = np.max(np.abs(X), axis=1)
    assert np.array_equal(s, (a / np.float32(127)).astype(np.float32))
    idx = np.argmax(np.abs(X), axis=1)
    peak = q[np.arange(33), idx]
    assert np.array_equal(peak, np.where(X[np.arange(33), idx] > 0, 127, -127))
    # One-hot rows.
    H = np.zeros((3, 64), np.float32)
    H[0, 5], H[1, 0], H[2, 63] = 0.37, -2.0, 1e-3
    qh, sh = orc.quantize_acts(H)
    assert qh[0, 5] == 127 and qh[1, 0] == -127 and qh[2, 63] == 127
    assert np.count_nonzero(qh) == 3
    # Power-of-two scaling leaves codes unchanged and scales s_x exactly.
    for j in (-4, 3):
        q2, s2 = orc.quantize_acts(X * np.float32(2.0 ** j))
        assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(2.0 ** j))
    # All-zero row.
    qz, sz = orc.quantize_acts(np.zeros((1, 32), np.float32))
    assert not qz.any() and sz[0] == 0.0


def pin_acts_match_fp64_rounding(orc):
    """Codes equal round-half-even(u * 127 / a) evaluated in fp64, except possibly where the
    fp32 and fp64 products straddle a .5 boundary (at most a one-step difference there)."""
    X = workloads.gaussian((64, 512), (20,), 1.0)
    q, _ = orc.quantize_acts(X)
    a = np.max(np.abs(X.astype(np.float64)), axis=1, keepdims=True)
    ref = np.rint(X.astype(np.float64) * 127.0 / a)
    diff = np.abs(q.astype(np.float64) - ref)
    assert diff.max() <= 1 and np.count_nonzero(diff) <= 3, np.count_nonzero(diff)


def pin_acts_bf16_widening(orc):
    X = workloads.gaussian((9, 128), (21,), 1.0)
    bits = workloads.f32_to_bf16_bits(X)
    wide = workloads.bf16_bits_to_f32(bits)
    g = workloads.gaussian((128,), (22,), 0.1) + np.float32(1)
    for gg in (None, g):
        qa, sa = orc.quantize_acts(bits, gg, bf16=True)
        qb, sb = orc.quantize_acts(wide, gg)
        assert np.array_equal(qa, qb) and np.array_equal(sa, sb)


def pin_norm_constant_row(orc):
    """x = c * 1, g = 1: every code is sign(c) * 127 and s_x = |c| / (127 sqrt(c^2 + eps))."""
    getcontext().prec = 50
    eps = np.float32(1e-6)
    for c in (0.75, -3.0, 2.0 ** -9):
        x = np.full((1, 96), c, np.float32)
        q, s = orc.quantize_acts(x, np.ones(96, np.float32), float(eps))
        assert np.all(q == (127 if c > 0 else -127))
        ref = Decimal(abs(c)) / (Decimal(127) * (Decimal(c) ** 2 + Decimal(float(eps))).sqrt())
        assert abs(float(s[0]) - float(ref)) <= 1e-7 * float(ref), (c, s[0], ref)


def pin_norm_equals_normalize_then_quantize(orc):
    """Fused SubLN + quant equals RMSNorm (fp64) followed by absmax quantization (fp64):
    same codes except at rounding ties, same scale to fp32 precision."""
    X = workloads.gaussian((32, 384), (23,), 1.0)
    g = (np.float32(1) + workloads.gaussian((384,), (24,), 0.1)).astype(np.float32)
    eps = 1e-6
    q, s = orc.quantize_acts(X, g, eps)
    x64 = X.astype(np.float64)
    r = 1.0 / np.sqrt(np.mean(x64 * x64, axis=1, keepdims=True) + np.float64(np.float32(eps)))
    y = x64 * r * g.astype(np.float64)
    a = np.max(np.abs(y), axis=1, keepdims=True)
    ref_q = np.rint(y * 127.0 / a)
    ref_s = a[:, 0] / 127.0
    diff = np.abs(q - ref_q)
    assert diff.max() <= 1 and np.count_nonzero(diff) <= 3
    assert np.max(np.abs(s / ref_s - 1)) < 1e-6


# ------------------------------------------------------------ O5 + O6: product

def pin_matmul_library(orc):
    """acc equals numpy's int64 matmul Xq @ C^T on non-square shapes."""
    Xq = _rng(25).integers(-127, 128, size=(5, 48), dtype=np.int8)
    C = workloads.ternary((7, 48), (26,))
    acc = orc.matmul(Xq, C)
    assert acc.shape == (5, 7)
    assert np.array_equal(acc, Xq.astype(np.int64) @ C.astype(np.int64).T)


def pin_matmul_freivalds(orc):
    """acc v == Xq (C^T v) exactly for random integer vectors v."""
    Xq = _rng(27).integers(-127, 128, size=(40, 320), dtype=np.int8)
    C = workloads.ternary((72, 320), (28,))
    acc = orc.matmul(Xq, C).astype(np.int64)
    for t in range(3):
        v = _rng(29, t).integers(-1000, 1000, size=72)
        lhs = acc @ v
        rhs = Xq.astype(np.int64) @ (C.astype(np.int64).T @ v)
        assert np.array_equal(lhs, rhs)


def pin_forward_dequantized_product(orc):
    """Tiny brute force: Y equals the fp64 product of the dequantized operands
    (q * s_x) (c * gamma)^T to within fp32 output rounding."""
    W = workloads.gaussian((24, 64), (30,), 0.02)
    X = workloads.gaussian((6, 64), (31,), 1.0)
    P, g, C = orc.quantize_weights(W)
    q, s = orc.quantize_acts(X)
    acc, Y = orc.forward(q, s, P, g)
    deq = (q.astype(np.float64) * s.astype(np.float64)[:, None]) @ \
        (C.astype(np.float64) * np.float64(g)).T
    assert np.all(np.abs(Y.astype(np.float64) - deq) <= 2.0 ** -23 * np.abs(deq) + 1e-30)
    assert np.array_equal(acc, q.astype(np.int64) @ C.astype(np.int64).T)


def pin_forward_one_hot(orc):
    """A one-hot token with value a at k gives y[n] = gamma * a * c[n, k] (within rounding)."""
    W = workloads.gaussian((32, 48), (32,), 0.02)
    P, g, C = orc.quantize_weights(W)
    a, k = np.float32(1.75), 13
    x = np.zeros((1, 48), np.float32)
    x[0, k] = a
    q, s = orc.quantize_acts(x)
    _, Y = orc.forward(q, s, P, g)
    ref = float(g) * float(a) * C[:, k].astype(np.float64)
    assert np.allclose(Y[0], ref, rtol=3e-7, atol=0)


def pin_forward_entries_match_full(orc):
    W = workloads.gaussian((40, 96), (33,), 0.02)
    X = workloads.gaussian((9, 96), (34,), 1.0)
    P, g, _ = orc.quantize_weights(W)
    q, s = orc.quantize_acts(X)
    acc, Y = orc.forward(q, s, P, g)
    m = np.array([0, 8, 3, 5]), np.array([39, 0, 17, 22])
    ea, ey = orc.forward_entries(q, s, P, g, *m)
    assert np.array_equal(ea, acc[m]) and np.array_equal(ey, Y[m])


def pin_quantize_weights_chain(orc):
    """The packed output of the whole weight chain unpacks to round_clip(W/gamma)."""
    W = workloads.gaussian((20, 80), (35,), 0.02)
    P, g, C = orc.quantize_weights(W)
    g_ref = f32_of_fraction(sum(Fraction(float(abs(w))) for w in W.ravel()) / W.size)
    assert g == g_ref
    t = W.astype(np.float32) / g
    ref = np.where(t > 0.5, 1, np.where(t < -0.5, -1, 0)).astype(np.int8)
    assert np.array_equal(orc.unpack(P, 80), ref) and np.array_equal(C, ref)


# ------------------------------------------------- O7 / O8: layer-chain FFN act, residual

def _f32(x):
    return np.float32(x)


def _ulp32(v):
    v = abs(float(v))
    return float(np.spacing(np.float32(v))) if v > 0 else float(np.float32(1.4e-45))


def pin_relu2_exact(orc):
    """ReLU^2 (SLM750-Edge card, "Key Architectural Features": relu(x)^2) is the correctly
    rounded square of the positive part: exact rational arithmetic, including 0, -0,
    subnormal inputs, squares that overflow fp32 and negative inputs (all zero)."""
    xs = list(_rng(70).standard_normal(400).astype(np.float32) * np.float32(3))
    xs += [0.0, -0.0, 1e-40, -1e-40, 1.5, -1.5, 3e19, 2.0 ** -75, 65504.0, 1.0 + 2.0 ** -23]
    for x in xs:
        x = _f32(x)
        want = f32_of_fraction(Fraction(float(x)) ** 2) if x > 0 else np.float32(0.0)
        got = orc.ffn_act1(orc.RELU2, x)
        assert got == want or (np.isinf(want) and np.isinf(got)), (x, got, want)


def pin_relu2_glu_near_exact(orc):
    """Gated ReLU^2 h = relu(g)^2 * u against exact rationals: within one fp32 ulp always and
    equal to the correctly rounded value in all but a sliver of cases (the fp64 evaluation
    rounds twice); exact zeros for g <= 0 or u = 0, and relu(g)^2 for u = 1."""
    r = _rng(71)
    G = r.standard_normal(2000).astype(np.float32) * np.float32(2)
    U = r.standard_normal(2000).astype(np.float32)
    H = orc.ffn_act(orc.RELU2_GLU, G, U)
    equal = 0
    for g, u, h in zip(G, U, H):
        want = f32_of_fraction(Fraction(float(g)) ** 2 * Fraction(float(u))) if g > 0 else np.float32(0.0)
        assert abs(float(h) - float(want)) <= _ulp32(want), (g, u, h, want)
        equal += h == want
    assert equal >= 1995, equal
    for g in (-2.0, -0.0, 0.0):
        assert orc.ffn_act1(orc.RELU2_GLU, g, 5.0) == 0.0
    assert orc.ffn_act1(orc.RELU2_GLU, 3.0, 0.0) == 0.0
    assert orc.ffn_act1(orc.RELU2_GLU, 1.25, 1.0) == np.float32(1.5625)


def _silu_times(g, u):
    """silu(g) * u correctly rounded to fp32, from a 60-digit decimal evaluation."""
    getcontext().prec = 60
    dg = Decimal(float(g))
    val = dg / (Decimal(1) + (-dg).exp()) * Decimal(float(u))
    return f32_of_fraction(Fraction(val))


def pin_swiglu_high_precision(orc):
    """SwiGLU h = silu(g) * u, silu(g) = g / (1 + e^-g), against a 60-digit decimal evaluation:
    within one fp32 ulp always, equal in all but a sliver of cases; silu(0) = 0; for large g
    silu(g) * u rounds to g * u; for very negative g the product underflows to zero."""
    r = _rng(72)
    G = r.standard_normal(600).astype(np.float32) * np.float32(4)
    U = r.standard_normal(600).astype(np.float32)
    H = orc.ffn_act(orc.SWIGLU, G, U)
    equal = 0
    for g, u, h in zip(G, U, H):
        want = _silu_times(g, u)
        assert abs(float(h) - float(want)) <= _ulp32(want), (g, u, h, want)
        equal += h == want
    assert equal >= 597, equal
    assert orc.ffn_act1(orc.SWIGLU, 0.0, 3.0) == 0.0
    assert orc.ffn_act1(orc.SWIGLU, 200.0, 1.5) == np.float32(300.0)
    assert orc.ffn_act1(orc.SWIGLU, -300.0, 1.0) == 0.0
    # silu(x) - silu(-x) = x (odd part), checked through one rounding each.
    for x in (0.5, 1.0, 2.5, 7.0):
        a, b = float(orc.ffn_act1(orc.SWIGLU, x, 1.0)), float(orc.ffn_act1(orc.SWIGLU, -x, 1.0))
        assert abs((a - b) - x) <= 2 * _ulp32(x), (x, a, b)


def _silu_times_exact(g, u):
    """silu(g) * u as a 60-digit decimal."""
    getcontext().prec = 60
    dg = Decimal(float(g))
    return dg / (Decimal(1) + (-dg).exp()) * Decimal(float(u))


def pin_ffn_act_fp64_values(orc):
    """The activations' fp64 values before the fp32 rounding (what the parity tests use to
    decide whether an fp32 difference sits at a rounding tie): SwiGLU within 4 fp64 ulps of a
    60-digit decimal evaluation (one correctly rounded exp, an addition, a division and a
    product; each at most an ulp or so), exact zeros where g or u is 0; ReLU^2 of an fp32 is
    exact in fp64 (a 24-bit significand squared) and gated ReLU^2 one fp64 rounding of the
    exact product; each fp64 value rounds to the fp32 activation."""
    r = _rng(73)
    G = r.standard_normal(800).astype(np.float32) * np.float32(5)
    U = r.standard_normal(800).astype(np.float32)
    G[:6] = np.array([0.0, -0.0, 1e-40, -30.0, 80.0, -700.0], np.float32)
    H64 = orc.ffn_act_f64(orc.SWIGLU, G, U)
    assert np.array_equal(H64.astype(np.float32), orc.ffn_act(orc.SWIGLU, G, U))
    for g, u, h in zip(G, U, H64):
        exact = _silu_times_exact(g, u)
        if exact == 0:
            assert h == 0.0, (g, u, h)
            continue
        err = abs(Fraction(float(h)) - Fraction(exact)) / abs(Fraction(exact))
        assert err <= Fraction(4, 2 ** 52), (g, u, float(h), float(err))
    X = r.standard_normal(300).astype(np.float32) * np.float32(3)
    H2 = orc.ffn_act_f64(orc.RELU2, X)
    for x, h in zip(X, H2):
        assert Fraction(float(h)) == (Fraction(float(x)) ** 2 if x > 0 else 0), (x, h)
    H3 = orc.ffn_act_f64(orc.RELU2_GLU, X, U[:300])
    for x, u, h in zip(X, U[:300], H3):
        exact = Fraction(float(x)) ** 2 * Fraction(float(u)) if x > 0 else Fraction(0)
        assert Fraction(float(h)) == exact or abs(Fraction(float(h)) - exact) <= abs(exact) / 2 ** 53, (x, u, h)


def pin_residual_epilogue_exact(orc):
    """Residual epilogue: fp32(fp32(acc * gamma * s_x) + r), the second step one exactly
    rounded fp32 addition; r = 0 gives the plain epilogue, r = -y gives +0."""
    r = _rng(73)
    M, N = 5, 37
    acc = r.integers(-200000, 200000, (M, N)).astype(np.int32)
    sx = (r.random(M) * 0.05).astype(np.float32)
    gamma = np.float32(0.021)
    R = (r.standard_normal((M, N)) * 3).astype(np.float32)
    Y0 = orc.epilogue(acc, sx, gamma)
    Y = orc.epilogue_residual(acc, sx, gamma, R)
    for m in range(M):
        for n in range(N):
            want = f32_of_fraction(Fraction(float(Y0[m, n])) + Fraction(float(R[m, n])))
            assert Y[m, n] == want, (m, n, Y[m, n], want)
    assert np.array_equal(orc.epilogue_residual(acc, sx, gamma, np.zeros_like(R)), Y0)
    Z = orc.epilogue_residual(acc, sx, gamma, -Y0)
    assert np.all(Z == 0.0) and not np.any(np.signbit(Z[Y0 != 0]))


# ------------------------------------------- O9: weight-only ternary forward (W1.58A16)

def _dyadic(shape, key, bits=3, span=8):
    """Values k / 2^bits with |k| < span * 2^bits: sums of a few of them are exact in fp64."""
    return (_rng(*key).integers(-span * 2 ** bits, span * 2 ** bits, size=shape)
            / 2.0 ** bits).astype(np.float32)


def pin_wonly_brute_force(orc):
    """Tiny brute force in exact rationals: y = fp32(gamma * sum_k x c)."""
    X = _dyadic((3, 16), (60,))
    C = workloads.ternary((5, 16), (61,))
    g = np.float32(0.0213)
    Y = orc.forward_wonly(X, C, g)
    for m in range(3):
        for n in range(5):
            exact = sum(Fraction(float(X[m, k])) * int(C[n, k]) for k in range(16))
            assert Y[m, n] == f32_of_fraction(Fraction(float(g)) * exact), (m, n)


def pin_wonly_integer_inputs_match_int_path(orc):
    """Integer-valued activations: the weight-only forward equals the int8 path's epilogue
    with unit row scales, bit for bit (both are fp32(gamma * exact integer sum))."""
    q = _rng(62).integers(-127, 128, size=(4, 96), dtype=np.int8)
    C = workloads.ternary((33, 96), (63,))
    g = np.float32(0.0187)
    Y = orc.forward_wonly(q.astype(np.float32), C, g)
    ref = orc.epilogue(q.astype(np.int64) @ C.astype(np.int64).T, np.ones(4, np.float32), g)
    assert np.array_equal(Y, ref)


def pin_wonly_one_hot(orc):
    """A one-hot token with value a at k gives y[n] = fp32(gamma * a * c[n, k])."""
    C = workloads.ternary((20, 48), (64,))
    g, a, k = np.float32(0.031), np.float32(-2.625), 29
    X = np.zeros((2, 48), np.float32)
    X[1, k] = a
    Y = orc.forward_wonly(X, C, g)
    assert np.count_nonzero(Y[0]) == 0
    for n in range(20):
        assert Y[1, n] == f32_of_fraction(Fraction(float(g)) * Fraction(float(a)) * int(C[n, k]))


# ------------------------------------------------------------ O10: input gradient (STE)

def pin_grad_input_adjoint(orc):
    """<dY, X W^T> == <dX, X> with dX = dY W (the adjoint of the weight-only product),
    non-square and square shapes, to the accuracy of the fp32 outputs."""
    for (M, N, K), key in (((5, 24, 40), 65), ((3, 32, 32), 66)):
        C = workloads.ternary((N, K), (key, 1))
        X = workloads.gaussian((M, K), (key, 2), 1.0)
        dY = workloads.gaussian((M, N), (key, 3), 1.0)
        g = np.float32(0.027)
        Y = orc.forward_wonly(X, C, g).astype(np.float64)
        dX = orc.grad_input(dY, C, g).astype(np.float64)
        lhs = np.sum(dY.astype(np.float64) * Y)
        rhs = np.sum(dX * X.astype(np.float64))
        scale = np.sum(np.abs(dY.astype(np.float64)) @ np.abs(C.astype(np.float64))
                       * np.abs(X.astype(np.float64))) * float(g)
        assert abs(lhs - rhs) <= 1e-6 * scale, (M, N, K, lhs, rhs)


def pin_grad_input_one_hot(orc):
    """dY one-hot at (m, n) with value a: dx[m] = fp32(gamma * a * c[n, :]), other rows 0."""
    C = workloads.ternary((12, 40), (67,))
    g, a = np.float32(0.019), np.float32(1.375)
    dY = np.zeros((3, 12), np.float32)
    dY[2, 7] = a
    dX = orc.grad_input(dY, C, g)
    assert np.count_nonzero(dX[:2]) == 0
    for k in range(40):
        assert dX[2, k] == f32_of_fraction(Fraction(float(g)) * Fraction(float(a)) * int(C[7, k]))


def pin_grad_input_brute_force(orc):
    dY = _dyadic((2, 9), (68,))
    C = workloads.ternary((9, 16), (69,))
    g = np.float32(0.0411)
    dX = orc.grad_input(dY, C, g)
    for m in range(2):
        for k in range(16):
            exact = sum(Fraction(float(dY[m, n])) * int(C[n, k]) for n in range(9))
            assert dX[m, k] == f32_of_fraction(Fraction(float(g)) * exact), (m, k)


# --------------------------------------------------------------- O11: STE gradient scale

def pin_ste_scale_page_values(orc):
    """bitone README, Soft-STE: scale 1 at w/gamma = 0, about 0.07 at 1, effectively zero but
    positive at 3 (beta = 2); the hard mask keeps |w/gamma| <= 1 (boundary included)."""
    S, H, P = orc.STE_SOFT, orc.STE_HARD, orc.STE_PASS
    assert orc.ste_scale(S, 0.0, 0.5) == 1.0
    assert abs(orc.ste_scale(S, 0.5, 0.5) - 0.07) < 1e-3          # t = 1 exactly
    assert abs(orc.ste_scale(S, 0.5, 0.5) - (1.0 - math.tanh(2.0) ** 2)) < 1e-15
    v3 = orc.ste_scale(S, 1.5, 0.5)                                   # t = 3
    assert 0.0 < v3 < 1e-4
    assert orc.ste_scale(H, 0.5, 0.5) == 1.0
    assert orc.ste_scale(H, -0.5, 0.5) == 1.0
    assert orc.ste_scale(H, float(np.nextafter(np.float32(0.5), np.float32(1))), 0.5) == 0.0
    assert orc.ste_scale(H, 0.0, 0.5) == 1.0
    assert orc.ste_scale(P, 123.0, 0.5) == 1.0
    # Symmetric in w.
    assert orc.ste_scale(S, -0.3, 0.5) == orc.ste_scale(S, 0.3, 0.5)


def pin_ste_soft_is_tanh_derivative(orc):
    """The soft scale is d/dt [tanh(beta t) / beta] (central differences, beta 2 and 1), and
    is computed from t = fp32(w / gamma)."""
    for beta in (2.0, 1.0):
        for t in (-2.2, -0.7, 0.0, 0.35, 1.0, 1.9, 4.5):
            w = np.float32(t) * np.float32(0.25)
            tt = float(np.float32(w) / np.float32(0.25))
            h = 1e-5
            fd = (math.tanh(beta * (tt + h)) - math.tanh(beta * (tt - h))) / (2 * h * beta)
            s = orc.ste_scale(orc.STE_SOFT, w, 0.25, beta)
            assert abs(s - fd) <= 1e-8 + 1e-8 * abs(fd), (beta, t, s, fd)


# --------------------------------------------------------------- O12: weight gradient (STE)

def pin_grad_weight_adjoint(orc):
    """Pass-through: <dW, gamma c> == <dY, Y> for Y the int8-path forward of the same
    codes and activations (dW = dY^T (q s_x) is the adjoint of W -> X_hat W^T)."""
    M, N, K = 6, 20, 48
    C = workloads.ternary((N, K), (70,))
    X = workloads.gaussian((M, K), (71,), 1.0)
    dY = workloads.gaussian((M, N), (72,), 1.0)
    g = np.float32(0.023)
    q, s = orc.quantize_acts(X)
    Y = orc.epilogue(orc.matmul(q, C), s, g).astype(np.float64)
    dW = orc.grad_weight(dY, orc.STE_PASS, Xq=q, sx=s).astype(np.float64)
    lhs = np.sum(dW * C.astype(np.float64)) * float(g)
    rhs = np.sum(dY.astype(np.float64) * Y)
    scale = float(g) * np.sum(np.abs(dY.astype(np.float64)).T @ np.abs(q * s[:, None].astype(np.float64)))
    assert abs(lhs - rhs) <= 1e-6 * scale


def pin_grad_weight_masks_elementwise(orc):
    """Hard and soft gradients are the pass-through gradient times the scale of the same
    weight (non-square: a transposed mask index fails), with t spanning both sides of 1."""
    M, N, K = 5, 12, 32
    Xf = workloads.gaussian((M, K), (73,), 1.0)
    dY = workloads.gaussian((M, N), (74,), 1.0)
    W = workloads.gaussian((N, K), (75,), 0.03)
    g = np.float32(0.02)
    base = orc.grad_weight(dY, orc.STE_PASS, Xf=Xf).astype(np.float64)
    hard = orc.grad_weight(dY, orc.STE_HARD, W=W, gamma=g, Xf=Xf)
    soft = orc.grad_weight(dY, orc.STE_SOFT, W=W, gamma=g, beta=2.0, Xf=Xf)
    t = (W / g).astype(np.float32)
    assert 0 < np.count_nonzero(np.abs(t) > 1) < t.size
    ref_h = np.where(np.abs(t) <= 1, base, 0.0).astype(np.float32)
    assert np.array_equal(hard, ref_h)
    ref_s = base / np.cosh(2.0 * t.astype(np.float64)) ** 2
    assert np.all(np.abs(soft - ref_s) <= 2.0 ** -23 * np.abs(ref_s) + 1e-37)


def pin_grad_weight_brute_force(orc):
    """Tiny brute force in exact rationals, dequantized activations q * s_x."""
    dY = _dyadic((3, 4), (76,))
    q = _rng(77).integers(-127, 128, size=(3, 16), dtype=np.int8)
    s = np.array([0.5, 0.0078125, 3.25], np.float32)
    dW = orc.grad_weight(dY, orc.STE_PASS, Xq=q, sx=s)
    for n in range(4):
        for k in range(16):
            exact = sum(Fraction(float(dY[m, n])) * int(q[m, k]) * Fraction(float(s[m]))
                        for m in range(3))
            assert dW[n, k] == f32_of_fraction(exact), (n, k)


# ------------------------------------------------------------------ O13: base-3 packing

def pin_b3_golden_block(orc):
    """The hand-derived block of tests/golden/b3_block.json, and the extreme bytes."""
    gold = golden("b3_block.json")
    C = np.zeros((1, 80), np.int8)
    for k, c in gold["block_codes_nonzero"].items():
        C[0, int(k)] = c
    assert list(orc.pack_b3(C)[0]) == gold["bytes"]
    ex = gold["extremes"]
    assert set(orc.pack_b3(np.ones((1, 80), np.int8))[0]) == {ex["all_plus_one"]}
    assert set(orc.pack_b3(-np.ones((1, 80), np.int8))[0]) == {ex["all_minus_one"]}
    assert set(orc.pack_b3(np.zeros((1, 80), np.int8))[0]) == {ex["all_zero"]}


def pin_b3_density_matches_the_pages(orc):
    """1.6 bits per weight: the bitone README's model sizes follow from the row bytes."""
    for n, gb in golden("b3_block.json")["model_sizes_gb"].items():
        K = 80 * 1000
        per_weight = orc.b3_row_bytes(K) / K
        assert abs(int(n) * per_weight / 1e9 - gb) < 1e-9, (n, gb)
    assert orc.b3_row_bytes(2560) == 512 and orc.b3_row_bytes(768) == 160
    assert orc.b3_row_bytes(16) == 16 and orc.b3_row_bytes(80) == 16 and orc.b3_row_bytes(96) == 32


def pin_b3_roundtrip_and_range(orc):
    """unpack(pack(C)) == C for ragged K; every byte <= 242; padding weights are code 0."""
    for K in (16, 80, 96, 768, 2000):
        C = workloads.ternary((7, K), (80, K))
        B = orc.pack_b3(C)
        assert B.max() <= 242
        assert np.array_equal(orc.unpack_b3(B, K), C)
    C = workloads.ternary((3, 16), (81,))
    B = orc.pack_b3(C).astype(int)
    # K = 16: bytes 0..3 hold weights 4b .. 4b+3 and the padding weight 64 + b (digit 1);
    # bytes 4..15 hold padding only.
    for b in range(4):
        v = sum((C[:, 4 * b + i].astype(int) + 1) * 3 ** i for i in range(4)) + 81
        assert np.array_equal(B[:, b], v)
    assert np.all(B[:, 4:] == 121)


def pin_b3_digit_weights_and_locality(orc):
    """Changing the code of weight k by +1 changes exactly one byte, by 3^i: within block
    j = k // 80, r = k % 80 < 64 is digit r % 4 of byte r // 4, r >= 64 digit 4 of byte r - 64."""
    C = np.zeros((2, 400), np.int8)
    base = orc.pack_b3(C).astype(int)
    for k in (0, 3, 15, 16, 63, 64, 79, 80, 163, 399):
        D = C.copy()
        D[1, k] = 1
        diff = orc.pack_b3(D).astype(int) - base
        j, r = k // 80, k % 80
        b, i = (r // 4, r % 4) if r < 64 else (r - 64, 4)
        assert np.count_nonzero(diff) == 1 and diff[1, 16 * j + b] == 3 ** i, k


def pin_b3_agrees_with_two_bit_packing(orc):
    """The same codes through both layouts: unpack_b3(pack_b3(C)) == unpack(pack(C))."""
    C = workloads.ternary((9, 320), (82,))
    assert np.array_equal(orc.unpack_b3(orc.pack_b3(C), 320), orc.unpack(orc.pack(C), 320))


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
