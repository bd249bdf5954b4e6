"""Number formats of the FP4 global KV cache (oracle; test infrastructure only).

Element format: FP4 E2M1; one E4M3 scale per 16 channels of the 512-channel
latent [P3 section 二 "how it was compressed", second route; P2 "same notes,
many layers": the main KV goes from FP8 to FP4].  A 4-bit code has 2^4 = 16
levels [P1 section 五].  The page's range argument puts the largest
representable magnitude at 448 x 6 = 2688 [P3 section 三]: 448 is the largest
E4M3 value of the OCP "FN" variant and 6 the largest E2M1 magnitude, which
fixes both variants (the FNUZ E4M3 variant tops out at 240).

Readings taken here (the pages give no bit layouts):
  * E2M1 is the OCP microscaling element type: sign bit, 2 exponent bits
    (bias 1), 1 mantissa bit, no Inf/NaN; magnitudes {0,.5,1,1.5,2,3,4,6}.
  * E4M3 is OCP E4M3FN: bias 7, subnormals, no Inf, only S.1111.111 is NaN.
  * Rounding is to nearest, ties to the even code (LSB 0), saturating at the
    largest finite magnitude.

All encoders here decide exactly: a value is compared against the exact
midpoints of the grid; every product formed for that comparison has at most
8 significant bits, so it is exact in float64.
"""
from fractions import Fraction

import numpy as np

# ---- E2M1 ---------------------------------------------------------------

E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
E2M1_MAX = 6.0

# value of each of the 16 nibbles: bit 3 is the sign
E2M1_TABLE = np.array([(-1.0 if n & 8 else 1.0) * E2M1_MAGNITUDES[n & 7]
                       for n in range(16)], dtype=np.float64)

# midpoints between consecutive magnitudes (index k sits between code k and k+1)
E2M1_MIDPOINTS = np.array([(E2M1_MAGNITUDES[k] + E2M1_MAGNITUDES[k + 1]) / 2
                           for k in range(7)], dtype=np.float64)


def e2m1_value(nibble: int) -> float:
    """Real value of one E2M1 code (0..15)."""
    return float(E2M1_TABLE[nibble & 15])


# ---- E4M3FN -------------------------------------------------------------

E4M3_MAX = 448.0
E4M3_NAN_BYTES = (0x7F, 0xFF)


def e4m3_value(byte: int) -> float:
    """Real value of one E4M3FN byte (NaN for 0x7F / 0xFF)."""
    byte &= 0xFF
    sign = -1.0 if byte & 0x80 else 1.0
    e = (byte >> 3) & 0xF
    m = byte & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
    return sign * (8 + m) * 2.0 ** (e - 10)  # (1 + m/8) * 2^(e-7)


E4M3_TABLE = np.array([e4m3_value(b) for b in range(256)], dtype=np.float64)

# The non-negative finite codes 0x00..0x7E are increasing in value.
_E4M3_POS = E4M3_TABLE[:0x7F]
assert np.all(np.diff(_E4M3_POS) > 0)
# midpoint k lies between codes k and k+1 (k = 0..125)
E4M3_MIDPOINTS = (_E4M3_POS[:-1] + _E4M3_POS[1:]) / 2


def _rne_index(y_cmp, mids_cmp):
    """Index of the nearest grid point, ties to the even index.

    ``mids_cmp[k]`` is the (exact) midpoint between grid points k and k+1, in
    the same units as ``y_cmp``; values beyond the last midpoint saturate to
    the last grid point.  Both arrays must hold exact values.
    """
    y_cmp = np.asarray(y_cmp, dtype=np.float64)
    k = np.searchsorted(mids_cmp, y_cmp, side="left")  # midpoints strictly below y
    # y sits exactly on midpoint k: the tie is between k and k+1; take the even one
    kk = np.minimum(k, len(mids_cmp) - 1)
    tie = (k < len(mids_cmp)) & (mids_cmp[kk] == y_cmp)
    return np.where(tie & (k % 2 == 1), k + 1, k)


def e4m3_scale_byte(amax):
    """E4M3FN byte of RNE(amax / 6), saturating at 448, for amax >= 0.

    The comparison amax/6 <> mid is done as amax <> 6*mid: 6*mid has at most
    8 significant bits, so it is exact in float64 and the decision is exact.
    Results below half the smallest subnormal (2^-10) round to 0; 2^-10 itself
    ties to the even code 0.
    """
    amax = np.asarray(amax, dtype=np.float64)
    if np.any(~np.isfinite(amax)) or np.any(amax < 0):
        raise ValueError("amax must be finite and non-negative")
    return _rne_index(amax, 6.0 * E4M3_MIDPOINTS).astype(np.uint8)


def e2m1_magnitude_code(absx, s):
    """3-bit magnitude code of RNE(|x| / s), saturating at 6; 0 where s == 0.

    Compared as |x| <> s*mid: s has at most 4 significant bits and each
    midpoint at most 3, so s*mid is exact.  The code is the number of
    midpoints strictly below |x|, plus one when |x| sits exactly on a
    midpoint whose upper neighbour has the even code (0.75, 1.75, 3.5).
    """
    absx = np.asarray(absx, dtype=np.float64)
    s_b = np.broadcast_to(np.asarray(s, dtype=np.float64), absx.shape)
    code = np.zeros(absx.shape, dtype=np.uint8)
    for k, mid in enumerate(E2M1_MIDPOINTS):
        thr = s_b * mid                                   # exact
        code += (absx > thr)
        if k % 2 == 1:                                    # tie between codes k and k+1, k+1 even
            code += (absx == thr)
    return np.where(s_b == 0, 0, code).astype(np.uint8)


# ---- exact helpers used by the pins ------------------------------------

def as_fraction(v) -> Fraction:
    """Exact rational value of a finite float."""
    return Fraction(float(v))
