"""Pins of the oracle's building blocks against hand-derived values, exact
arithmetic and library routines (CPU only).

The pages fix 4-bit integer transport with a high-precision sum
("Tensor-parallel traffic drops to 4 bits", Interpretation; "Echo:
Error-Compensated 4-Bit Tensor-Parallel Communication", Abstract); the group
size, code range, scale rule,
rounding and nibble order are the stated readings, checked here by values
worked out by hand (tests/golden/quantizer_hand_cases.json) and by exact
rational re-derivation.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantizer_hand_cases.json")


@pytest.fixture(scope="module")
def hand():
    with open(GOLDEN) as f:
        return json.load(f)


def test_hand_quantizer_cases(hand):
    for case in hand["quantizer"]:
        v = np.array([float.fromhex(t) for t in case["v"]], dtype=np.float32)
        q, s = orc.quantize_group(v)
        assert s == float.fromhex(case["scale"]), case["name"]
        assert q.tolist() == case["codes"], case["name"]


def test_hand_quantizer_cases_8bit(hand):
    for case in hand["quantizer8"]:
        v = np.array([float.fromhex(t) for t in case["v"]], dtype=np.float32)
        q, s = orc.quantize_group_q(v, 127)
        assert s == float.fromhex(case["scale"]), case["name"]
        assert q.tolist() == case["codes"], case["name"]


def test_hand_byte_codes_8bit(hand):
    for case in hand["pack8"]:
        assert orc.pack_codes(np.array(case["q"], np.int8), bits=8).tolist() == case["bytes"]
        assert orc.unpack_codes(np.array(case["bytes"], np.uint8), 4, bits=8).tolist() == case["q"]


def test_hand_pack_cases(hand):
    for case in hand["pack"]:
        assert orc.pack(np.array(case["q"], np.int8)).tolist() == [case["byte"]], case["why"]
        assert orc.unpack(np.array([case["byte"]], np.uint8), 2).tolist() == case["q"]


def test_pack_roundtrip_exhaustive():
    vals = np.arange(-8, 8, dtype=np.int8)
    a, b = np.meshgrid(vals, vals, indexing="ij")
    q = np.stack([a.ravel(), b.ravel()], axis=1).ravel()
    codes = orc.pack(q)
    assert np.array_equal(orc.unpack(codes, q.size), q)
    # 256 distinct pairs give 256 distinct bytes: a bijection
    assert len(set(codes.tolist())) == 256


def test_hand_bf16_cases(hand):
    for case in hand["bf16"]:
        f = np.array([case["f32"]], dtype=np.uint32).view(np.float32)
        assert int(orc.f32_to_bf16(f)[0]) == case["bf16"], case["why"]


def test_bf16_matches_torch_cast():
    """Round-to-nearest-even narrowing agrees with torch's float32->bfloat16
    cast on every finite upper half (sign, exponent and the 7 kept mantissa
    bits), each with exact, tie, near-tie and other lower halves."""
    hi = np.arange(1 << 16, dtype=np.uint32)
    hi = hi[(hi & 0x7F80) != 0x7F80]  # finite only
    lows = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xC000], np.uint32)
    bits = ((hi[:, None] << 16) | lows[None, :]).ravel()
    f = bits.view(np.float32)
    ours = orc.f32_to_bf16(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _is_nearest_f32(s: float, exact: Fraction) -> bool:
    """s is a binary32 value closest to `exact` (ties allowed either way here)."""
    s32 = np.float32(s)
    lo = np.nextafter(s32, np.float32(-np.inf))
    hi = np.nextafter(s32, np.float32(np.inf))
    d = abs(Fraction(float(s32)) - exact)
    return d <= abs(Fraction(float(lo)) - exact) and d <= abs(Fraction(float(hi)) - exact)


def _groups(rng):
    yield rng.standard_normal(128).astype(np.float32)
    yield (rng.standard_normal(128) * 1e-3).astype(np.float32)
    t = rng.standard_normal(128)
    t[rng.integers(0, 128)] *= 30
    yield t.astype(np.float32)
    yield (rng.standard_t(3, 128) * 1e5).astype(np.float32)
    yield rng.uniform(-1, 1, 128).astype(np.float32)
    yield np.round(rng.uniform(-7, 7, 128) * 2) / 2  # many exact half-integers
    yield (rng.integers(-3, 4, 128) * 2.0 ** -140).astype(np.float32)  # denormal scale


@pytest.mark.parametrize("qmax", [7, 127])
def test_quantizer_is_nearest_code_exact_arithmetic(qmax):
    """Every code is the exact nearest of the 2*qmax+1 codes to v (ties to the
    even code), with s the correctly rounded binary32 value of amax/qmax;
    values whose v/s lies within 2^-20 of a half-integer are decided by the
    binary32 quotient and checked against numpy's IEEE division instead."""
    rng = np.random.default_rng(1 + qmax)
    n_checked = n_boundary = 0
    for _ in range(20 if qmax == 7 else 6):
        for v in _groups(rng):
            v = np.ascontiguousarray(v, np.float32)
            if qmax == 127:
                v = v * np.float32(127.0 / 7.0)  # keep the half-integer family on the grid
                v = np.ascontiguousarray(v, np.float32)
            q, s = orc.quantize_group_q(v, qmax)
            amax = Fraction(float(np.max(np.abs(v))))
            if s == 0.0:
                # all-zero group, or amax/qmax below half the smallest denormal
                assert amax / qmax <= Fraction(2.0 ** -150)
                assert not q.any()
                continue
            assert _is_nearest_f32(s, amax / qmax)
            S = Fraction(s)
            for vi, qi in zip(v.tolist(), q.tolist()):
                t = Fraction(vi) / S
                frac = t - (t.numerator // t.denominator)
                if abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 20):
                    n_boundary += 1
                    ref = np.clip(np.rint(np.float32(vi) / np.float32(s)), -qmax, qmax)
                    assert qi == int(ref)
                    continue
                if qmax == 7:  # brute force over the whole code set
                    pool = range(-qmax, qmax + 1)
                else:  # the nearest code is one of the two integers around v/s, clamped
                    lo = max(-qmax, min(qmax, t.numerator // t.denominator))
                    pool = {lo, max(-qmax, min(qmax, lo + 1))}
                cands = sorted(pool, key=lambda c: (abs(Fraction(vi) - c * S), c % 2))
                assert qi == cands[0], (vi, s, qi, cands[:2])
                n_checked += 1
    assert n_checked > 3000 and n_boundary > 20


def test_quantizer_error_bound():
    """|d - v| <= s/2 for every value (exact arithmetic), the textbook bound
    of round-to-nearest with step s when no value is clamped."""
    rng = np.random.default_rng(2)
    for _ in range(50):
        for v in _groups(rng):
            v = np.ascontiguousarray(v, np.float32)
            q, s = orc.quantize_group(v)
            if s == 0.0:
                continue
            S = Fraction(s)
            for vi, qi in zip(v.tolist(), q.tolist()):
                err = abs(Fraction(qi) * S - Fraction(vi))
                # slack covers amax/s slightly above 7 after rounding s
                assert err <= S / 2 + Fraction(abs(vi)) * Fraction(1, 1 << 21)


def test_quantizer_codes_in_range_and_amax_hits_qmax():
    rng = np.random.default_rng(3)
    for _ in range(200):
        v = (rng.standard_normal(128) * rng.uniform(1e-3, 1e3)).astype(np.float32)
        q, s = orc.quantize_group(v)
        assert q.min() >= -7 and q.max() <= 7
        assert abs(int(q[np.argmax(np.abs(v))])) == 7


def test_ema_closed_form():
    """k refreshes with a constant r from zero give m = r (1 - beta^k)."""
    r = np.array([1.0, -3.5, 1e-3, 250.0], np.float32)
    mf = np.zeros_like(r)
    ms = np.zeros_like(r)
    for k in range(1, 41):
        orc.ema_refresh(mf, ms, r)
        want_f = r.astype(np.float64) * (1 - orc.BETA_FAST ** k)
        want_s = r.astype(np.float64) * (1 - orc.BETA_SLOW ** k)
        np.testing.assert_allclose(mf, want_f, rtol=2e-6 * k, atol=0)
        np.testing.assert_allclose(ms, want_s, rtol=2e-6 * k, atol=0)
    # r = 0 keeps a zero state at zero, and decays a nonzero one geometrically
    mf = np.full(4, 8.0, np.float32)
    ms = np.full(4, 8.0, np.float32)
    orc.ema_refresh(mf, ms, np.zeros(4, np.float32))
    assert mf.tolist() == [4.0] * 4 and ms.tolist() == [7.0] * 4


def test_update_from_zero_state_is_alpha_times_residual():
    """From a zero state the correction is 0, so x' = x, r = d1 - x and the
    averages become A_F r and A_S r (products by powers of two are exact)."""
    rng = np.random.default_rng(4)
    n, P = 1024, 4
    x = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16).copy()
    mf = np.zeros(n, np.float32)
    ms = np.zeros(n, np.float32)
    codes, scales = orc.encode(xb, mf, ms)
    q = orc.unpack(codes, n).astype(np.float64)
    # q * s is exact in float64 (3-bit by 24-bit), so one cast to float32 is
    # the correctly rounded binary32 product
    d1 = (q * np.repeat(scales.astype(np.float64), 128)).astype(np.float32).astype(np.float64)
    xf = x.float().numpy().astype(np.float64)
    e2 = rng.standard_normal(n // P).astype(np.float32) * 1e-2
    orc.update(xb, mf, ms, codes, scales, e2, nranks=P, rank=1)
    r = (d1 - xf).astype(np.float32)  # the float64 difference is exact here
    r[n // P:2 * n // P] = r[n // P:2 * n // P] + e2
    assert np.array_equal(mf, (0.5 * r.astype(np.float64)).astype(np.float32))
    assert np.array_equal(ms, (0.125 * r.astype(np.float64)).astype(np.float32))


def _round_f32(q: Fraction) -> float:
    """The binary32 value nearest to the exact rational q (ties to the even
    significand), found by exact comparison among q's neighbourhood; q is
    nonzero and inside the normal range here."""
    f = np.float32(float(q))
    cands = [f]
    for _ in range(2):
        cands = [np.nextafter(cands[0], np.float32(-np.inf))] + cands + \
                [np.nextafter(cands[-1], np.float32(np.inf))]
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - q)
        even = (int(np.float32(c).view(np.uint32)) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, c)
    return float(best[1])


def test_update_rounds_each_operation_in_the_written_order():
    """The refresh is m <- (B * m) + (A * r) with each product and the sum
    rounded once, in that order (reading 19), checked against exact rational
    arithmetic with IEEE rounding applied step by step.  B_S = 7/8 makes
    B_S * m inexact, so a reassociated form such as m + A (r - m) rounds
    differently on many elements."""
    rng = np.random.default_rng(19)
    n, P, rank = 128 * 16, 4, 2
    x = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16).copy()
    mf = (rng.standard_normal(n) * 0.3).astype(np.float32)
    ms = (rng.standard_normal(n) * 0.3).astype(np.float32)
    codes, scales = orc.encode(xb, mf, ms)
    e2 = (rng.standard_normal(n // P) * 1e-2).astype(np.float32)
    mf0, ms0 = mf.copy(), ms.copy()
    r = orc.update(xb, mf, ms, codes, scales, e2, nranks=P, rank=rank, want_r=True)
    BF, AF = Fraction(float(orc.BETA_FAST)), Fraction(float(orc.ALPHA_FAST))
    BS, AS = Fraction(float(orc.BETA_SLOW)), Fraction(float(orc.ALPHA_SLOW))

    def refresh(B, A, m, ri):
        bm = _round_f32(B * Fraction(float(m))) if m != 0 else 0.0
        ar = _round_f32(A * Fraction(float(ri))) if ri != 0 else 0.0
        s = Fraction(bm) + Fraction(ar)
        return _round_f32(s) if s != 0 else 0.0

    for i in range(n):
        assert float(mf[i]) == refresh(BF, AF, mf0[i], r[i]), i
        assert float(ms[i]) == refresh(BS, AS, ms0[i], r[i]), i
