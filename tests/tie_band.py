"""Parity where an fp64 value is rounded to fp32 near a tie (the SwiGLU activation).

The kernels evaluate SwiGLU's h = silu(g) * u in fp64 and round it to fp32 once, as the oracle
does, but with another exp: a table-driven one in the bulk FFN quantizer (exp_f64_tab) and
the device library's in the decode epilogue, where the oracle has the host library's.  Each
fp64 value is within a few fp64 ulps of the exact one (the oracle's: pinned within 4 ulps by
pin_ffn_act_fp64_values; the table exp: a 2^(j/64) table entry, a degree-6 polynomial and a
Newton-refined reciprocal, each within an ulp or so), so two evaluations can round to
different fp32 values only where the exact value, and with it the oracle's fp64 value, lies
within a few fp64 ulps of an fp32 rounding midpoint.

These helpers accept an fp32 difference only there: the oracle's fp64 value must lie within
BAND (16 fp64 ulps, relative 2^-48) of the midpoint between the oracle's fp32 value and the
GPU's, and the GPU's value must be the other rounding across that midpoint.  Anything
downstream of such an h (its int8 code, the row's scale, a residual sum) must then be exactly
what the oracle gives for the h with that other rounding.
"""

import numpy as np

BAND = 16 * 2.0 ** -52


def alternate(h64):
    """For fp64 values h64: (h32, alt, in_band): h32 = fl32(h64); alt = the fp32 value on the
    other side of the rounding midpoint nearest to h64; in_band = whether h64 lies within BAND
    (relative) of that midpoint."""
    h64 = np.asarray(h64, np.float64)
    h32 = h64.astype(np.float32)
    above = h64 >= h32.astype(np.float64)
    alt = np.where(above, np.nextafter(h32, np.float32(np.inf)), np.nextafter(h32, np.float32(-np.inf)))
    mid = (h32.astype(np.float64) + alt.astype(np.float64)) / 2.0     # exact in fp64
    in_band = np.abs(h64 - mid) <= BAND * np.abs(h64)
    return h32, alt.astype(np.float32), in_band


def check_values(got, h64, label, add=None):
    """got: the GPU's fp32 values of fl32(h64) (plus `add`, an fp32 array added in fp32, when
    given).  Every difference from the oracle must come from an h at a tie taking its other
    rounding.  Returns the number of such differences."""
    h32, alt, inb = alternate(h64)
    want = h32 if add is None else (h32 + add).astype(np.float32)
    bad = got != want
    if not np.any(bad):
        return 0
    assert np.all(inb[bad]), (label, "differences away from a tie", np.nonzero(bad & ~inb)[0][:8])
    other = alt if add is None else (alt + add).astype(np.float32)
    assert np.array_equal(got[bad], other[bad]), (label, "not the other rounding")
    return int(np.count_nonzero(bad))


def _scale_ok(s, s_ref, norm):
    if s_ref == 0 or s == 0:
        return s == s_ref
    return s == s_ref if not norm else abs(float(s) / float(s_ref) - 1.0) <= 1e-6


def check_act_codes(q, s, H64, g, orc, label):
    """q [M, K], s [M]: the GPU's int8 codes and scales of the quantization (with RMSNorm
    weight g, or None) of h = fl32(H64).  A row whose codes or scale differ from the oracle's
    must equal, codes bit for bit and scale as the oracle's (bit for bit without a norm, within
    1e-6 with one), the oracle's quantization of a row in which only elements at a tie take
    their other rounding: those whose codes differ, and the row's largest |u| if the scale
    still differs.  Returns the number of such elements."""
    H, alt, inb = alternate(H64)
    q_ref, s_ref = orc.quantize_acts(H, g, 1e-6)
    norm = g is not None
    flips = 0
    for m in range(q.shape[0]):
        if np.array_equal(q[m], q_ref[m]) and _scale_ok(s[m], s_ref[m], norm):
            continue
        idx = list(np.nonzero(q[m] != q_ref[m])[0])
        assert all(inb[m, idx]), (label, m, "code differences away from a tie")
        row = H[m].copy()
        row[idx] = alt[m, idx]
        qa, sa = orc.quantize_acts(row[None], g, 1e-6)
        if not _scale_ok(s[m], sa[0], norm):
            u = np.abs(row * g.astype(np.float32)) if norm else np.abs(row)
            k = int(np.argmax(u))
            assert inb[m, k] and k not in idx, (label, m, "scale differs away from a tie")
            row[k] = alt[m, k]
            idx.append(k)
            qa, sa = orc.quantize_acts(row[None], g, 1e-6)
        assert np.array_equal(qa[0], q[m]), (label, m, "codes not explained by ties")
        assert _scale_ok(s[m], sa[0], norm), (label, m, "scale not explained by ties")
        flips += len(idx)
    return flips
