"""Pins of the oracle's number formats (CPU only).

E4M3FN is pinned to torch's float8_e4m3fn decode and cast (a library routine,
valid where torch does not overflow to NaN, |y| < 464), to a brute-force
nearest-code search over all 127 non-negative finite codes, and to values of
the OCP format worked out by hand. E2M1 is pinned to its 8 magnitudes worked
out by hand and to a brute-force search. NVFP4 groups are pinned by hand-made
examples and a round trip on representable groups.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F


def _sweep_f32():
    """Every finite BF16 pattern as float32, plus midpoints between adjacent
    E4M3 magnitudes and their float32 neighbours."""
    bits = np.arange(65536, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    mags = F.e4m3_values()[:127]
    mid = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    mid_up = np.nextafter(mid, np.float32(np.inf))
    mid_dn = np.nextafter(mid, np.float32(0))
    extra = np.concatenate([mid, mid_up, mid_dn, mags.astype(np.float32)])
    extra = np.concatenate([extra, -extra])
    return np.concatenate([x, extra]).astype(np.float32)


def _brute_e4m3(y):
    """Nearest code by scanning every magnitude; ties to the even code."""
    mags = F.e4m3_values()[:127]
    a = np.abs(y.astype(np.float64))
    out = np.empty(y.shape, np.uint8)
    for start in range(0, y.size, 4096):
        aa = np.minimum(a[start:start + 4096], 448.0)
        d = np.abs(aa[:, None] - mags[None, :])
        best = d.min(axis=1, keepdims=True)
        cand = d == best
        # among the (at most two) nearest codes prefer the even one
        even = cand & (np.arange(127)[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        out[start:start + 4096] = pick
    return out | (np.signbit(y).astype(np.uint8) << 7)


def test_e4m3_values_at_hand_computed_points():
    v = F.e4m3_values()
    assert v[0x00] == 0.0 and not np.signbit(v[0x00])
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9            # smallest subnormal 1/8 * 2^-6
    assert v[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert v[0x08] == 2.0 ** -6            # smallest normal
    assert v[0x38] == 1.0                  # exponent 7 = bias
    assert v[0x3C] == 1.5
    assert v[0x7E] == 448.0                # 1.75 * 2^8
    assert v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isnan(v).sum() == 2
    assert np.all(np.diff(v[:127]) > 0)


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], ours[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(ours[ok]))


@pytest.mark.parametrize("scale", [1.0, 3.0, 0.37, 1.0 / 448.0, 2.0 ** -5, 1000.0, 7.123e-3])
def test_e4m3_encode_matches_torch_cast_in_range(scale):
    x = _sweep_f32()
    y = x / np.float32(scale)
    ours = F.e4m3_encode(x, scale)
    inrange = np.abs(y) < 464.0          # torch turns |y| >= 464 into NaN
    ref = torch.from_numpy(y[inrange]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours[inrange], ref)


@pytest.mark.parametrize("scale", [1.0, 0.37, 1.0 / 448.0])
def test_e4m3_encode_matches_bruteforce(scale):
    x = _sweep_f32()
    y = x / np.float32(scale)
    assert np.array_equal(F.e4m3_encode(x, scale), _brute_e4m3(y))


def test_e4m3_encode_specials():
    enc = lambda v, s=1.0: int(F.e4m3_encode(np.array([v], np.float32), s)[0])
    assert enc(449.0) == 0x7E and enc(1e30) == 0x7E and enc(np.inf) == 0x7E
    assert enc(-500.0) == 0xFE and enc(-np.inf) == 0xFE
    assert enc(np.nan) == 0x7F
    assert enc(-1e-30) == 0x80 and enc(-0.0) == 0x80 and enc(0.0) == 0x00
    assert enc(2.0 ** -10) == 0x00            # tie between 0 and 2^-9 -> even code 0
    assert enc(3 * 2.0 ** -10) == 0x02        # tie between codes 1 and 2 -> 2
    assert enc(1.0625) == 0x38                # tie between 1.0 (0x38) and 1.125 (0x39)
    assert enc(1.1875) == 0x3A                # tie between 0x39 and 0x3A -> 0x3A
    assert enc(5.0, 0.0) == 0x00              # zero scale gives code 0
    assert enc(10.0, 2.0) == enc(5.0)         # the quotient is what is rounded


def test_e4m3_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    for s in (2.0 ** -8, 1.0, 32.0):
        vals = (F.e4m3_decode(codes) * s).astype(np.float32)
        assert np.array_equal(F.e4m3_encode(vals, s), codes)


def test_e2m1_values_hand_computed():
    v = F.e2m1_values()
    assert list(v[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(v[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert np.signbit(v[8])


def test_e2m1_encode_hand_computed():
    enc = lambda y: int(F.e2m1_encode(np.array([y], np.float32))[0])
    assert enc(0.25) == 0x0       # tie 0 / 0.5 -> even code 0
    assert enc(0.2500001) == 0x1
    assert enc(0.75) == 0x2       # tie 0.5 (code 1) / 1.0 (code 2)
    assert enc(1.25) == 0x2       # tie 1.0 (code 2) / 1.5 (code 3)
    assert enc(1.75) == 0x4       # tie 1.5 / 2.0
    assert enc(2.5) == 0x4        # tie 2 (code 4) / 3 (code 5)
    assert enc(3.5) == 0x6        # tie 3 / 4
    assert enc(5.0) == 0x6        # tie 4 (code 6) / 6 (code 7)
    assert enc(5.0001) == 0x7
    assert enc(6.0) == 0x7 and enc(100.0) == 0x7 and enc(np.inf) == 0x7
    assert enc(-6.5) == 0xF
    assert enc(-0.0) == 0x8 and enc(-0.1) == 0x8 and enc(0.0) == 0x0
    assert enc(-2.9) == 0xD


def test_e2m1_encode_matches_bruteforce():
    rng = np.random.default_rng(0)
    y = np.concatenate([
        rng.uniform(-8, 8, 200000).astype(np.float32),
        np.array([0, .25, .75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0], np.float32),
    ])
    y = np.concatenate([y, np.nextafter(y, np.float32(np.inf)), np.nextafter(y, np.float32(-np.inf)), -y])
    mags = F.e2m1_values()[:8]
    a = np.minimum(np.abs(y.astype(np.float64)), 6.0)
    d = np.abs(a[:, None] - mags[None, :])
    cand = d == d.min(axis=1, keepdims=True)
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    ref = pick.astype(np.uint8) | (np.signbit(y).astype(np.uint8) << 3)
    assert np.array_equal(F.e2m1_encode(y), ref)


def test_nvfp4_group_hand_example():
    # amax = 3 -> 3/6 = 0.5 is exactly E4M3 (code 0x30); element codes of x/0.5
    x = np.zeros(16, np.float32)
    x[:6] = [3.0, -1.2, 0.1, 0.125, -0.5, 1.4]
    codes, s = F.nvfp4_encode_groups(x)
    assert int(s) == 0x30 and F.e4m3_decode(s) == 0.5
    # y = 6, -2.4, 0.2, 0.25, -1.0, 2.8 -> 6 (7), -2 (0xC), 0 (0), tie .25 -> 0, -1 (0xA), 3 (5)
    assert list(codes[:6]) == [0x7, 0xC, 0x0, 0x0, 0xA, 0x5]
    assert list(codes[6:]) == [0] * 10


def test_nvfp4_group_scale_rounding_and_saturation():
    # amax = 1.0: 1/6 = 0.1666.. -> nearest E4M3 is 0.171875 (1.375 * 2^-3)
    x = np.array([1.0] + [0.0] * 15, np.float32)
    codes, s = F.nvfp4_encode_groups(x)
    assert F.e4m3_decode(s) == 0.171875 and int(codes[0]) == 0x7   # 1/0.171875 = 5.8 -> 6
    # amax = 0.9: 0.15 -> E4M3 neighbours 0.140625 / 0.15625 -> 0.15625 is nearer
    x = np.array([0.9, -0.9] + [0.0] * 14, np.float32)
    codes, s = F.nvfp4_encode_groups(x)
    assert F.e4m3_decode(s) == 0.15625 and list(codes[:2]) == [0x7, 0xF]   # 5.76 -> 6
    # a group whose scale rounds down saturates its largest element to 6
    x = np.array([6.2 * 0.140625] + [0.0] * 15, np.float32)   # amax/6 -> 0.1453 -> 0.140625
    codes, s = F.nvfp4_encode_groups(x)
    assert F.e4m3_decode(s) == 0.140625 and int(codes[0]) == 0x7
    # all-zero / tiny groups: scale 0 -> every code 0, even for negative inputs
    x = np.array([-1e-5] * 16, np.float32)
    codes, s = F.nvfp4_encode_groups(x)
    assert int(s) == 0 and np.all(codes == 0)


def test_nvfp4_round_trip_on_representable_groups():
    rng = np.random.default_rng(1)
    n = 4000
    s_codes = rng.integers(0x08, 0x70, n).astype(np.uint8)     # normal scales, 6*S stays < 448*..
    codes = rng.integers(0, 16, (n, 16)).astype(np.uint8)
    codes[:, 0] = 0x7 | (codes[:, 0] & 0x8)                   # one element at +-6 -> amax = 6 S
    x = F.nvfp4_decode_groups(codes, s_codes).astype(np.float32)
    c2, s2 = F.nvfp4_encode_groups(x)
    assert np.array_equal(s2, s_codes)
    assert np.array_equal(c2, codes)


def test_nvfp4_decode_bound():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((5000, 16)) * rng.uniform(0.01, 50, (5000, 1))).astype(np.float32)
    codes, s = F.nvfp4_encode_groups(x)
    dec = F.nvfp4_decode_groups(codes, s)
    S = F.e4m3_decode(s)
    assert np.all(np.abs(dec) <= 6 * S[:, None])
    # every element is within half a step of the grid unless it saturated
    amax = np.abs(x).max(axis=1)
    unsat = 6 * S >= amax
    err = np.abs(dec - x)[unsat]
    assert np.all(err <= S[unsat][:, None])        # widest E2M1 step is 2 (4 -> 6)


def test_bf16_decode():
    assert F.bf16_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert F.bf16_to_f64(np.array([0xC000], np.uint16))[0] == -2.0
    assert F.bf16_to_f64(np.array([0x0001], np.uint16))[0] == 2.0 ** -133
    assert np.isnan(F.bf16_to_f64(np.array([0x7FC0], np.uint16))[0])
    t = torch.randn(1000).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_to_f64(bits), t.to(torch.float64).numpy())
