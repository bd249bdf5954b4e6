"""Row quantiser of the FP4 global KV cache (oracle; test infrastructure only).

One cached position holds the 512-channel global-KV latent [P3 section 三].
It is stored as 512 E2M1 codes plus 32 E4M3 scales, one per 16 consecutive
channels [P3 section 二, second route].  Per position that is
256 + 32 = 288 bytes; 4-bit storage alone is a quarter of 16-bit storage
[P3 section 二].  Positions sit at a fixed stride so that a kernel can find a
position from its index and dequantise it in parallel [P1 section 五].

Readings (the pages do not give the quantiser):
  * scale s = RNE_E4M3(amax / 6) of the group's largest magnitude, exact,
    saturating at 448; no second, per-tensor scale (the page's 448 x 6 =
    2688 range is scale x code with nothing on top).
  * element code = RNE_E2M1(|x| / s), exact, saturating at 6; sign kept as
    the code's top bit, so -0.0 and negatives rounding to 0 give code 0x8;
    s == 0 gives magnitude 0.
  * channel 2j goes to the low nibble and 2j+1 to the high nibble of byte j;
    group g covers channels 16g..16g+15 and its scale is byte g.
"""
import numpy as np

from .formats import (E2M1_TABLE, E4M3_TABLE, e2m1_magnitude_code,
                      e4m3_scale_byte)

D = 512            # latent channels
GROUP = 16         # channels per scale
NGROUPS = D // GROUP
CODE_BYTES = D // 2
SCALE_BYTES = NGROUPS
BYTES_PER_TOKEN = CODE_BYTES + SCALE_BYTES   # 288


def quantize_rows(x):
    """float32 [R, 512] -> (codes uint8 [R, 256], scales uint8 [R, 32]).

    Raises ValueError on non-finite input.
    """
    x = np.asarray(x)
    if x.dtype != np.float32 or x.ndim != 2 or x.shape[1] != D:
        raise ValueError("expected float32 [R, 512]")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input row")
    R = x.shape[0]
    g = x.reshape(R, NGROUPS, GROUP)
    amax = np.abs(g).max(axis=2)                          # exact
    sbyte = e4m3_scale_byte(amax)                         # [R, 32]
    s = E4M3_TABLE[sbyte]                                 # exact float64
    mag = e2m1_magnitude_code(np.abs(g), s[..., None])    # [R, 32, 16]
    sign = np.signbit(g).astype(np.uint8)
    code = (sign << 3) | mag                              # nibble per channel
    code = code.reshape(R, D)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, sbyte


def unpack_codes(codes):
    """uint8 [R, 256] -> nibble per channel uint8 [R, 512]."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (D,), dtype=np.uint8)
    out[..., 0::2] = codes & 0xF
    out[..., 1::2] = codes >> 4
    return out


def dequantize_rows(codes, scales):
    """(codes [R, 256], scales [R, 32]) -> float32 [R, 512], exact.

    Each value is code x scale: at most 2 + 4 significant bits and within
    [2^-10, 2688], so the float32 result is the exact product.
    """
    nib = unpack_codes(codes)
    v = E2M1_TABLE[nib]                                   # float64
    s = E4M3_TABLE[np.asarray(scales, dtype=np.uint8)]
    if np.any(np.isnan(s)):
        raise ValueError("NaN scale byte in cache")
    out = v.reshape(v.shape[:-1] + (NGROUPS, GROUP)) * s[..., None]
    return out.reshape(v.shape).astype(np.float32)
