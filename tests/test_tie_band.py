"""The tie-band parity helpers on the CPU: a difference is accepted only where the oracle's fp64
value sits at an fp32 rounding tie and the GPU took the other rounding; planted differences
anywhere else are refused."""

import numpy as np
import pytest

import tie_band


def _tie(lo):
    """An fp64 value just above the midpoint between fp32 lo and the next fp32 value."""
    lo = np.float32(lo)
    hi = np.nextafter(lo, np.float32(np.inf))
    mid = (float(lo) + float(hi)) / 2.0
    return mid + abs(mid) * 2.0 ** -50


def test_alternate():
    h64 = np.array([_tie(2.5), 2.5, 1.0 / 3.0, 0.0, -_tie(7.0)])
    h32, alt, inb = tie_band.alternate(h64)
    assert list(inb) == [True, False, False, False, True]
    assert h32[0] == np.nextafter(np.float32(2.5), np.float32(3)) and alt[0] == np.float32(2.5)
    assert alt[4] == np.float32(-7.0)
    assert np.all(np.abs(alt.astype(np.float64) - h32) > 0)


def test_check_values():
    h64 = np.array([_tie(2.5), 1.0 / 3.0, -0.75, _tie(-1e-3)])
    h32, alt, _ = tie_band.alternate(h64)
    assert tie_band.check_values(h32.copy(), h64, "same") == 0
    got = h32.copy()
    got[0] = alt[0]
    got[3] = alt[3]
    assert tie_band.check_values(got, h64, "ties") == 2
    # With a residual added in fp32 a one-ulp difference of h can vanish (element 3 here).
    R = np.array([1.0, 2.0, 3.0, 4.0], np.float32)
    assert tie_band.check_values((got + R).astype(np.float32), h64, "ties+R", add=R) == 1
    bad = h32.copy()
    bad[1] = np.nextafter(bad[1], np.float32(1))      # one ulp off, but not at a tie
    with pytest.raises(AssertionError):
        tie_band.check_values(bad, h64, "planted")
    bad = h32.copy()
    bad[0] = np.nextafter(alt[0], np.float32(-1))     # at a tie, but not the other rounding
    with pytest.raises(AssertionError):
        tie_band.check_values(bad, h64, "planted")


def test_check_act_codes(orc):
    # Row 0: absmax 127 (inv = 1), so the code of an element is rint(h); element 1 sits at the
    # tie between 2.5 and the next fp32 value: one rounding gives code 2, the other 3.
    # Row 1: its absmax element sits at a tie, so the other rounding changes the scale.
    H64 = np.array([[127.0, _tie(2.5), -5.25, 0.5],
                    [_tie(100.0), 3.0, -40.0, 1.0]])
    H, alt, inb = tie_band.alternate(H64)
    q_ref, s_ref = orc.quantize_acts(H)
    assert tie_band.check_act_codes(q_ref, s_ref, H64, None, orc, "same") == 0
    # A GPU that rounded element (0, 1) the other way.
    H_alt = H.copy()
    H_alt[0, 1] = alt[0, 1]
    q_alt, s_alt = orc.quantize_acts(H_alt)
    assert q_alt[0, 1] != q_ref[0, 1]
    assert tie_band.check_act_codes(q_alt, s_alt, H64, None, orc, "tie code") == 1
    # A GPU that rounded row 1's absmax the other way: new scale, possibly other codes.
    H_alt = H.copy()
    H_alt[1, 0] = alt[1, 0]
    q_alt, s_alt = orc.quantize_acts(H_alt)
    assert s_alt[1] != s_ref[1]
    assert tie_band.check_act_codes(q_alt, s_alt, H64, None, orc, "tie scale") >= 1
    # Planted: a code one off where h is not at a tie.
    q_bad = q_ref.copy()
    q_bad[0, 2] += 1
    with pytest.raises(AssertionError):
        tie_band.check_act_codes(q_bad, s_ref, H64, None, orc, "planted code")
    # Planted: a scale off by one ulp with no tie at the row's absmax.
    s_bad = s_ref.copy()
    s_bad[0] = np.nextafter(s_bad[0], np.float32(2))
    with pytest.raises(AssertionError):
        tie_band.check_act_codes(q_ref, s_bad, H64, None, orc, "planted scale")
