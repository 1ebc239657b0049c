"""Number formats of the KV cache, written out value by value.

* BF16: the upper 16 bits of an IEEE float32.
* E4M3 (FP8): the cache format of ``paged_decode_attn_splitk_fp8`` and of the
  per-16 scales of the NVFP4 cache [metrale: reshape_and_cache_nvfp4,
  paged_decode_attn_splitk_fp8]. The pages only name the format; the reading
  taken is OCP E4M3FN (R1): 1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits, exponent 0 encodes subnormals m/8 * 2^-6, S.1111.111 is NaN,
  no infinities, largest finite magnitude 448 (the FP8 calibration divides the
  absmax by 448).
* E2M1 (FP4): the NVFP4 element format [metrale: reshape_and_cache_nvfp4]:
  1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit; magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6.

Encoders round to the nearest representable value with ties going to the even
code, the sign of the input kept (R2-R5, R9); the quotient x/scale is taken as
an IEEE float32 division before rounding (R2).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def bf16_to_f64(bits) -> np.ndarray:
    """BF16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_values() -> np.ndarray:
    """float64 value of each of the 256 E4M3FN codes (NaN for 0x7F, 0xFF)."""
    codes = np.arange(256)
    sign = np.where(codes & 0x80, -1.0, 1.0)
    e = (codes >> 3) & 0xF
    m = (codes & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64))
    subnormal = (m / 8.0) * 2.0 ** -6
    vals = sign * np.where(e == 0, subnormal, normal)
    vals[(e == 15) & ((codes & 0x7) == 7)] = np.nan
    return vals


_E4M3 = e4m3_values()
_E4M3_MAGS = _E4M3[:127]            # codes 0x00..0x7E, strictly increasing


def e4m3_decode(codes) -> np.ndarray:
    """E4M3FN codes (uint8) -> float64 values."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def _nearest_code(mag: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the entry of the increasing, non-negative ``table`` nearest to
    each magnitude in ``mag`` (float64, within the table's range); an exact tie
    between two neighbours picks the even index."""
    hi = np.searchsorted(table, mag, side="left")
    hi = np.clip(hi, 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    d_lo = mag - table[lo]
    d_hi = table[hi] - mag
    tie_pick = np.where(lo % 2 == 0, lo, hi)
    return np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, tie_pick))


def e4m3_encode(x, scale) -> np.ndarray:
    """Quantize ``x`` (taken as float32) with per-tensor ``scale`` to E4M3FN.

    y = float32(x) / float32(scale) (IEEE float32 division, R2); NaN -> 0x7F
    (R3); |y| >= 448 saturates to +-448 (R4); otherwise the nearest code with
    ties to the even code; the sign bit is the sign bit of y, so a negative
    value that rounds to zero is 0x80 (R5); scale == 0 gives code 0 (R6).
    """
    x32 = np.asarray(x, dtype=np.float32)
    s32 = np.float32(scale)
    if s32 == 0:
        return np.zeros(x32.shape, dtype=np.uint8)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        y = x32 / s32
    mag = np.abs(y).astype(np.float64)
    finite_mag = np.where(np.isnan(mag), 0.0, np.minimum(mag, E4M3_MAX))
    idx = _nearest_code(finite_mag, _E4M3_MAGS)
    idx = np.where(mag >= E4M3_MAX, 126, idx)
    code = idx.astype(np.uint8) | (np.signbit(y).astype(np.uint8) << np.uint8(7))
    code = np.where(np.isnan(y), np.uint8(0x7F), code)
    return code.astype(np.uint8)


def e2m1_values() -> np.ndarray:
    """float64 value of each of the 16 E2M1 codes."""
    codes = np.arange(16)
    sign = np.where(codes & 0x8, -1.0, 1.0)
    e = (codes >> 1) & 0x3
    m = (codes & 0x1).astype(np.float64)
    normal = (1.0 + m / 2.0) * np.exp2((e - 1).astype(np.float64))
    subnormal = m / 2.0
    return sign * np.where(e == 0, subnormal, normal)


_E2M1 = e2m1_values()
_E2M1_MAGS = _E2M1[:8]               # 0, .5, 1, 1.5, 2, 3, 4, 6


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 codes (low 4 bits of each uint8) -> float64 values."""
    return _E2M1[np.asarray(codes, dtype=np.uint8) & 0xF]


def e2m1_encode(y) -> np.ndarray:
    """Round float32 ``y`` to E2M1: nearest magnitude, ties to the even code,
    |y| >= 6 saturates to 6, sign bit from the sign of y (-0 -> 0x8) (R9).
    NaN inputs are outside the contract (they give 0x7 with y's sign)."""
    y32 = np.asarray(y, dtype=np.float32)
    mag = np.abs(y32).astype(np.float64)
    finite_mag = np.where(np.isnan(mag), E2M1_MAX, np.minimum(mag, E2M1_MAX))
    idx = _nearest_code(finite_mag, _E2M1_MAGS)
    idx = np.where(mag >= E2M1_MAX, 7, idx)
    idx = np.where(np.isnan(mag), 7, idx)
    return (idx.astype(np.uint8) | (np.signbit(y32).astype(np.uint8) << np.uint8(3))).astype(np.uint8)


def nvfp4_encode_groups(x):
    """NVFP4 quantization of groups of 16 consecutive values (last axis = 16)
    [metrale: reshape_and_cache_nvfp4: E2M1 values, one E4M3 scale per 16].

    For each group: amax = max |x| (float32); the scale code is the E4M3FN
    rounding of float32(amax) / 6 (IEEE float32 division, saturating; no
    per-tensor second-level scale, R7); S is its value. If S == 0 every
    element code is 0x0 (R8); otherwise code_i = E2M1(float32(x_i) / S) with
    the division in float32 (R9).

    Returns (codes uint8 [..., 16] in the low nibble, scale_codes uint8 [...]).
    """
    x32 = np.asarray(x, dtype=np.float32)
    assert x32.shape[-1] == 16, "groups of 16 along the last axis"
    amax = np.max(np.abs(x32), axis=-1)
    with np.errstate(over="ignore", invalid="ignore"):
        s_code = e4m3_encode(amax / np.float32(6.0), 1.0)
    S = e4m3_decode(s_code).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        y = x32 / np.where(S == 0, np.float32(1.0), S)[..., None]
    codes = e2m1_encode(y)
    codes = np.where((S == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes, s_code


def nvfp4_decode_groups(codes, scale_codes) -> np.ndarray:
    """E2M1 codes [..., 16] and their E4M3 scale codes [...] -> float64 values
    (exact: at most 6 significant bits)."""
    return e2m1_decode(codes) * e4m3_decode(scale_codes)[..., None]
