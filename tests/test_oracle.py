"""Pins of the CPU oracle against things other than itself: closed forms,
independent library routines (scipy, mpmath, PyTorch's bf16 cast), brute
force on small inputs, invariants, and the figures the pages print
(tests/golden/pages_figures.json).  CPU only."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def f32_ulp(x) -> float:
    x = np.float32(abs(x))
    return float(np.nextafter(x, np.float32(np.inf), dtype=np.float32) - x)


# --------------------------------------------------------------------------
# bf16 rounding
# --------------------------------------------------------------------------
def test_bf16_rounding_matches_torch():
    import torch

    rng = np.random.default_rng(7)
    f = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-40], np.float32),
    ])
    # exact ties: low 16 bits 0x8000, both parities of the kept part
    ties = (rng.integers(0, 2**15, 4000).astype(np.uint32) << 16) | np.uint32(0x8000)
    f = np.concatenate([f, ties.view(np.float32)[np.isfinite(ties.view(np.float32))]])
    ours = oracle.f32_to_bf16_bits(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_widen_exact():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_bits_to_f32(bits)
    back = oracle.f32_to_bf16_bits(f)
    finite = np.isfinite(f)
    assert np.array_equal(back[finite], bits[finite])


# --------------------------------------------------------------------------
# Standard normal quantile
# --------------------------------------------------------------------------
def test_normal_quantile_vs_scipy_and_cdf():
    from scipy import special

    for p in np.linspace(0.5, 0.99, 491):
        x = oracle.normal_quantile(float(p))
        assert x == pytest.approx(float(special.ndtri(p)), rel=1e-14, abs=1e-15)
        # closed-form round trip through the CDF Phi(x) = erfc(-x/sqrt2)/2
        assert 0.5 * math.erfc(-x / math.sqrt(2.0)) == pytest.approx(float(p), rel=1e-14)
    assert oracle.normal_quantile(0.5) == 0.0
    assert oracle.normal_quantile(0.975) == pytest.approx(-oracle.normal_quantile(0.025), rel=1e-15)


# --------------------------------------------------------------------------
# Codebook
# --------------------------------------------------------------------------
def test_codebook_invariants():
    L = oracle.codebook()
    assert L.dtype == np.float32 and L.shape == (16,)
    assert np.all(np.diff(L) > 0)
    assert L[0] == np.float32(-1.0) and L[7] == np.float32(0.0) and L[15] == np.float32(1.0)
    assert np.sum(L < 0) == 7 and np.sum(L > 0) == 8
    assert np.all(np.abs(L) <= 1)
    # dense near 0, sparse at the ends (mlqm.cn article, section 3.2):
    # gaps grow monotonically moving away from zero on each side.
    gaps = np.diff(L.astype(np.float64))
    assert np.all(np.diff(gaps[7:]) > 0)      # positive side, 0 -> +1
    assert np.all(np.diff(gaps[:7]) < 0)      # negative side, -1 -> 0


def test_codebook_is_correctly_rounded_exact_quantiles():
    """Recompute each level in 50-digit arithmetic (mpmath erfinv) from the
    stated construction; the oracle's binary32 level must be the correctly
    rounded value."""
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    d = mpmath.mpf(1) - mpmath.mpf(1) / 2 * (mpmath.mpf(1) / 30 + mpmath.mpf(1) / 32)

    def q(p):
        return mpmath.sqrt(2) * mpmath.erfinv(2 * p - 1)

    top = q(d)
    half = mpmath.mpf(1) / 2
    pos = [q(d + i * (half - d) / 8) / top for i in range(8)]
    neg = [-q(d + i * (half - d) / 7) / top for i in range(7)]
    exact = sorted(neg + [mpmath.mpf(0)] + pos)
    L = oracle.codebook()
    for li, ei in zip(L, exact):
        err = abs(mpmath.mpf(float(li)) - ei)
        assert err <= mpmath.mpf(f32_ulp(li)) / 2 * (1 + mpmath.mpf(2) ** -20) + mpmath.mpf(10) ** -45


def test_codebook_levels_are_the_stated_quantiles():
    """Phi(L_i * Phi^-1(offset)) must give back the evenly spaced
    probabilities (positive side: 8 steps from the offset toward 1/2; negative
    side mirrored, 7 steps)."""
    from scipy.stats import norm

    L = oracle.codebook().astype(np.float64)
    top = oracle.normal_quantile(nf4.NF4_OFFSET)
    d = nf4.NF4_OFFSET
    pos = L[8:][::-1]      # +1 .. smallest positive
    neg = -L[:7]           # 1 .. smallest |negative|
    for i, v in enumerate(pos):
        assert norm.cdf(v * top) == pytest.approx(d + i * (0.5 - d) / 8, abs=3e-8)
    for i, v in enumerate(neg):
        assert norm.cdf(v * top) == pytest.approx(d + i * (0.5 - d) / 7, abs=3e-8)


# --------------------------------------------------------------------------
# Thresholds and encode
# --------------------------------------------------------------------------
def test_thresholds_bracket_midpoints():
    L = oracle.codebook().astype(np.float64)
    T = oracle.thresholds(oracle.codebook())
    for i in range(15):
        m = Fraction(float(L[i])) / 2 + Fraction(float(L[i + 1])) / 2
        assert Fraction(float(T[i])) > m
        below = np.nextafter(T[i], np.float32(-np.inf), dtype=np.float32)
        assert Fraction(float(below)) <= m


def brute_codes(x: np.ndarray) -> np.ndarray:
    """argmin_i |x - L_i| in binary64 (exact for binary32 x), lowest index
    on ties -- independent of the threshold table."""
    L = oracle.codebook().astype(np.float64)
    d = np.abs(x.astype(np.float64)[:, None] - L[None, :])
    return np.argmin(d, axis=1).astype(np.uint8)  # argmin returns the first minimum


def _encode_unit(x):
    # a block absmax of exactly 1 makes the normalisation the identity
    x = np.asarray(x, dtype=np.float32)
    n = x.size
    pad = (-n) % 64
    xx = np.concatenate([x, np.zeros(pad, np.float32)])
    a = np.ones(xx.size // 64, dtype=np.float32)
    return oracle.encode(xx, a, oracle.thresholds(oracle.codebook()))[:n]


def test_encode_matches_bruteforce_near_every_threshold():
    T = oracle.thresholds(oracle.codebook())
    xs = []
    for t in T:
        v = np.float32(t)
        lo = hi = v
        xs.append(v)
        for _ in range(64):
            lo = np.nextafter(lo, np.float32(-np.inf), dtype=np.float32)
            hi = np.nextafter(hi, np.float32(np.inf), dtype=np.float32)
            xs += [lo, hi]
    rng = np.random.default_rng(11)
    xs = np.concatenate([np.array(xs, np.float32),
                         rng.uniform(-1, 1, 200000).astype(np.float32),
                         np.array([-1.0, 1.0, 0.0, -0.0], np.float32)])
    assert np.array_equal(_encode_unit(xs), brute_codes(xs))


def test_exact_midpoint_ties_go_to_lower_index():
    L = oracle.codebook().astype(np.float64)
    found = 0
    for i in range(15):
        m = (L[i] + L[i + 1]) / 2
        if float(np.float32(m)) == m:         # midpoint representable in binary32
            found += 1
            c = _encode_unit(np.array([m], np.float32))[0]
            assert c == i
            assert brute_codes(np.array([m], np.float32))[0] == i
    assert found >= 1


def test_encode_exhaustive_bf16_against_bruteforce():
    """Every finite bf16 weight, in blocks whose absmax sweeps many binades;
    codes from the full quantize path vs brute-force nearest level of
    x = fl32(w * fl32(1/a))."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_bits_to_f32(allbits)
    rng = np.random.default_rng(5)
    anchors = oracle.f32_to_bf16_bits(
        np.float32(2.0) ** rng.uniform(-30, 30, 24).astype(np.float32) *
        rng.uniform(1, 2, 24).astype(np.float32))
    anchors = np.concatenate([anchors, oracle.f32_to_bf16_bits(np.array([1.0, 0.02, 3.0], np.float32))])
    for ab in anchors:
        a = oracle.bf16_bits_to_f32(np.array([ab]))[0]
        ok = np.isfinite(f) & (np.abs(f) <= a)
        w = allbits[ok]
        # lay out blocks of 63 weights + the anchor so each block's absmax is a
        nblk = -(-w.size // 63)
        body = np.zeros(nblk * 63, np.uint16)
        body[:w.size] = w
        blocks = np.concatenate([body.reshape(nblk, 63),
                                 np.full((nblk, 1), ab, np.uint16)], axis=1).ravel()
        q = oracle.quantize(blocks, False)
        assert np.all(q["absmax"] == a)
        r = np.float32(1.0) / np.float32(a)
        x = (oracle.bf16_bits_to_f32(blocks) * r).astype(np.float32)
        assert np.array_equal(q["codes"], brute_codes(x))


def test_reconstruction_error_bound():
    """|w - L[c] * a_b| <= a_b * (largest half gap) (+ binary32 slack), and
    per element within half the gap around its level."""
    L = oracle.codebook().astype(np.float64)
    hmax = np.max(np.diff(L)) / 2
    rng = np.random.default_rng(3)
    for sigma in (0.02, 1.0, 300.0):
        w = oracle.f32_to_bf16_bits(rng.standard_normal(64 * 500).astype(np.float32) * np.float32(sigma))
        q = oracle.quantize(w, False)
        wf = oracle.bf16_bits_to_f32(w).astype(np.float64)
        a = np.repeat(q["absmax"].astype(np.float64), 64)
        rec = L[q["codes"]] * a
        assert np.all(np.abs(wf - rec) <= a * hmax * (1 + 2.0 ** -20))
        # bf16 dequant adds at most half a bf16 ulp
        deq = oracle.bf16_bits_to_f32(oracle.dequantize(q["packed"], q)).astype(np.float64)
        assert np.all(np.abs(wf - deq) <= a * hmax * (1 + 2.0 ** -20) + np.abs(rec) * 2.0 ** -8)


def test_reconstruction_error_bound_tiny_blocks():
    """Blocks whose absmax lies anywhere from the smallest bf16 subnormal
    (2^-133) up past 2^-100, with zeros and both signs inside: every code is
    still the nearest level and the bound holds.  Without the 2^64
    pre-scaling the reciprocal of an absmax at or below 2^-128 overflows and
    a block's zeros would take code 0 (dequantized to -absmax)."""
    L = oracle.codebook().astype(np.float64)
    hmax = np.max(np.diff(L)) / 2
    rng = np.random.default_rng(17)
    blocks = []
    for e in list(range(-133, -96)) + [-126, -127, -128]:
        a = np.float32(2.0 ** e)
        for mant in (1.0, 1.5, 1.9921875):
            am = np.float32(a * np.float32(mant))
            blk = np.zeros(64, np.float32)
            blk[0] = am
            blk[1] = -am
            blk[2:40] = (rng.uniform(-1, 1, 38) * am).astype(np.float32)
            blocks.append(blk)
    w = oracle.f32_to_bf16_bits(np.concatenate(blocks))
    for qt in ("nf4", "fp4"):
        q = oracle.quantize(w, False, quant_type=qt)
        Lq = oracle.levels_by_code(qt).astype(np.float64)
        hq = np.max(np.diff(np.sort(np.unique(Lq)))) / 2
        wf = oracle.bf16_bits_to_f32(w).astype(np.float64)
        a = np.repeat(q["absmax"].astype(np.float64), 64)
        assert np.all(a > 0)
        rec = Lq[q["codes"]] * a
        assert np.all(np.abs(wf - rec) <= a * hq * (1 + 2.0 ** -20))
        zero_code = 7 if qt == "nf4" else 0
        assert np.all(q["codes"][wf == 0] == zero_code)
        if qt == "nf4":
            assert hq == hmax


def test_tiny_block_prescale_only_changes_overflowing_blocks():
    """x = fl32(fl32(w * 2^64) * fl32(1 / (a * 2^64))) equals the plain
    fl32(w * fl32(1 / a)) bit for bit for every bf16 absmax a in
    (2^-128, 2^-100) (all of them) against weights spread over [-a, a]: the
    pre-scaling only alters blocks whose plain reciprocal overflowed."""
    bits = np.arange(0x0000, 0x8000, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_bits_to_f32(bits)
    a = vals[(vals > np.float32(2.0 ** -128)) & (vals < np.float32(2.0 ** -100))]
    assert a.size > 3000
    frac = np.linspace(-1.0, 1.0, 257, dtype=np.float64)
    w = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(
        (a[:, None].astype(np.float64) * frac[None, :]).astype(np.float32)))
    with np.errstate(over="ignore"):
        plain = (w * (np.float32(1.0) / a)[:, None]).astype(np.float32)
        pre = np.float32(2.0 ** 64)
        scaled = ((w * pre).astype(np.float32) *
                  (np.float32(1.0) / (a * pre).astype(np.float32))[:, None]).astype(np.float32)
    assert np.all(np.isfinite(plain))
    assert np.array_equal(plain.view(np.uint32), scaled.view(np.uint32))
    # and at 2^-128 itself the plain reciprocal overflows
    with np.errstate(over="ignore", divide="ignore"):
        assert np.isinf(np.float32(1.0) / np.float32(2.0 ** -128))


def test_zero_block_and_partial_block():
    w = np.zeros(64 + 10, dtype=np.uint16)            # one zero block + a 10-wide tail
    w[64:] = oracle.f32_to_bf16_bits(np.linspace(-0.5, 0.5, 10).astype(np.float32))
    q = oracle.quantize(w, False)
    assert q["absmax"].size == 2 and q["absmax"][0] == 0 and q["absmax"][1] == np.float32(0.5)
    assert np.all(q["codes"][:64] == 7)
    assert q["codes"][64] == 0 and q["codes"][73] == 15
    deq = oracle.dequantize(q["packed"], q, w.size)
    assert np.all(deq[:64] == 0)      # +0.0, not -0.0


def test_pack_nibbles_hand_built():
    codes = np.array([1, 2, 3, 4, 15, 0, 7, 8], np.uint8)
    packed = oracle.pack_nibbles(codes)
    assert packed.tolist() == [0x12, 0x34, 0xF0, 0x78]
    assert np.array_equal(oracle.unpack_nibbles(packed), codes)
    with pytest.raises(ValueError):
        oracle.pack_nibbles(np.zeros(3, np.uint8))


# --------------------------------------------------------------------------
# Double quantization
# --------------------------------------------------------------------------
def test_double_quant_hand_example():
    a = np.array([1.0, 2.0, 3.0], np.float32)
    q, s, mean = oracle.double_quant(a)
    assert mean == np.float32(2.0)
    assert s.tolist() == [1.0]
    assert q.tolist() == [-127, 0, 127]


def test_double_quant_mean_is_exact_then_rounded():
    rng = np.random.default_rng(9)
    a = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(
        np.abs(rng.standard_normal(3000)).astype(np.float32) * np.float32(0.05)))
    a[::97] *= np.float32(2.0 ** 12)         # spread over many binades
    q, s, mean = oracle.double_quant(a)
    exact = sum(Fraction(float(v)) for v in a) / a.size
    assert abs(Fraction(float(mean)) - exact) <= Fraction(f32_ulp(mean)) / 2 * (1 + Fraction(1, 2 ** 20))


def test_double_quant_bounds_and_saturation():
    rng = np.random.default_rng(4)
    for nb in (1, 255, 256, 257, 1000, 4096 + 3):
        a = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(
            np.abs(rng.standard_normal(nb)).astype(np.float32) * np.float32(0.06)))
        q, s, mean = oracle.double_quant(a)
        ng = -(-nb // 256)
        assert q.shape == (nb,) and s.shape == (ng,)
        assert np.all(q >= -127) and np.all(q <= 127)
        g = np.arange(nb) // 256
        for gi in range(ng):
            sel = g == gi
            if s[gi] > 0:
                assert np.max(np.abs(q[sel].astype(int))) == 127
            else:
                assert np.all(q[sel] == 0)
        state = {"double_quant": True, "absmax": q, "absmax2": s, "absmax_mean": mean}
        ahat = oracle.block_scales(state).astype(np.float64)
        slack = 4 * np.array([f32_ulp(max(abs(float(mean)), float(s[gi]), float(ai)))
                              for gi, ai in zip(g, a)])
        assert np.all(np.abs(ahat - a) <= s[g].astype(np.float64) / 254 + slack)


def test_double_quant_exact_ties_round_half_even():
    """Constructed scales where fl32(fl32(c_b / s_g) * 127) lands exactly on
    k + 1/2 with k even: q takes k (ties to even), where rounding half away
    from zero would take k + 1.  Scales [0, 2m, m + c, m - c] have mean m, so
    c_b = -m, m, c, -c and s_g = m.  First a binary32 case (m = 1, tie at
    32.5), then one in bf16 values (m = 15.875, c = 1/16: u = 1/2 exactly)
    that the GPU quantize test reaches from real weights."""
    for m, c, k in ((1.0, None, 32), (15.875, 0.0625, 0)):
        m = np.float32(m)
        if c is None:
            # the binary32 c nearest (k + 1/2) / 127 whose product rounds to the tie
            c0 = np.float32((k + 0.5) / 127.0)
            cands = [np.array([int(c0.view(np.uint32)) + d], np.uint32).view(np.float32)[0]
                     for d in range(-8, 9)]
            c = next(cc for cc in cands
                     if float(np.float32(np.float32(cc / m) * np.float32(127.0))) == k + 0.5)
        c = np.float32(c)
        a = np.array([0.0, 2 * m, m + c, m - c], np.float32)
        assert float(a[2]) == float(m) + float(c) and float(a[3]) == float(m) - float(c)
        q, s, mean = oracle.double_quant(a)
        assert mean == m and s.tolist() == [float(m)]
        u = np.float32(np.float32(c / m) * np.float32(127.0))
        assert float(u) == k + 0.5
        assert q.tolist() == [-127, 127, k, -k]
        away = int(np.floor(float(u) + 0.5))
        assert away == k + 1 and away != q[2]


def test_double_quant_constant_scales():
    a = np.full(300, 0.25, np.float32)
    q, s, mean = oracle.double_quant(a)
    assert mean == np.float32(0.25) and np.all(s == 0) and np.all(q == 0)
    state = {"double_quant": True, "absmax": q, "absmax2": s, "absmax_mean": mean}
    assert np.all(oracle.block_scales(state) == np.float32(0.25))


# --------------------------------------------------------------------------
# The "dynamic" 8-bit second-level map
# --------------------------------------------------------------------------
def decode_dynamic_bits(code: int) -> float:
    """Value of an 8-bit dynamic-tree code read from its bit fields: bit 7
    the sign, then E zero bits (decimal exponent 10^-E), a one bit, and
    6 - E fraction bits f naming the midpoint of the f-th of 2^(6-E) equal
    bins of [0.1, 1].  Seven zero bits leave no indicator: the value 0."""
    sign = -1.0 if code & 0x80 else 1.0
    rest = code & 0x7F
    if rest == 0:
        return 0.0
    e = 7 - rest.bit_length()
    nbits = 6 - e
    f = rest & ((1 << nbits) - 1)
    return sign * (10.0 ** -e) * (0.1 + 0.9 * (f + 0.5) / (1 << nbits))


def test_dynamic_map_is_the_bit_layout():
    """The sorted map equals the values the 256 bit patterns decode to (both
    zero codes give 0), with 1.0 in the place of the second zero."""
    m = oracle.dynamic_map().astype(np.float64)
    decoded = sorted(set(float(np.float32(decode_dynamic_bits(c))) for c in range(256)) | {1.0})
    assert len(decoded) == 256
    assert np.array_equal(m, np.array(decoded))


def test_dynamic_map_structure():
    m = oracle.dynamic_map()
    assert m.dtype == np.float32 and m.size == 256
    assert np.all(np.diff(m.astype(np.float64)) > 0)
    assert m[-1] == np.float32(1.0) and m[0] == np.float32(-0.99296875)
    assert np.count_nonzero(m == 0) == 1
    assert np.count_nonzero(m < 0) == 127 and np.count_nonzero(m > 0) == 128
    mag = np.abs(m[m > 0].astype(np.float64))[:-1]    # without 1.0
    for e in range(7):
        lo, hi = 0.1 * 10.0 ** -e, 10.0 ** -e
        d = np.sort(mag[(mag > lo) & (mag < hi)])
        assert d.size == 2 ** (6 - e)                  # 2^(6-E) bins per decade
        step = 0.9 * hi / 2 ** (6 - e)
        if d.size > 1:                                 # equal bins, to binary32 rounding
            assert np.allclose(np.diff(d), step, rtol=0, atol=4 * hi * 2.0 ** -24)
        assert abs(d[0] - (lo + step / 2)) <= hi * 2.0 ** -24
    assert np.array_equal(-m[:127][::-1], m[128:255])  # symmetric but for 1.0


def test_dynamic_double_quant_hand_example():
    q, s, mean = oracle.double_quant_dynamic(np.array([1.0, 2.0, 3.0], np.float32))
    assert mean == np.float32(2.0) and s.tolist() == [1.0]
    assert q.tolist() == [0, 127, 255]
    state = {"double_quant": True, "dq_map": "dynamic", "absmax": q, "absmax2": s,
             "absmax_mean": mean}
    ahat = oracle.block_scales(state)
    assert ahat.tolist() == [float(np.float32(np.float32(-0.99296875) + np.float32(2.0))), 2.0, 3.0]
    # a group scale other than 1: each binary32 operation's exact result is a
    # binary64 value here, so one rounding of it to binary32 is the format
    a = np.array([0.0, 1.5, 0.8125, 0.6875, 0.703125], np.float32)
    q, s, mean = oracle.double_quant_dynamic(a)
    m = oracle.dynamic_map()
    state = {"double_quant": True, "dq_map": "dynamic", "absmax": q, "absmax2": s,
             "absmax_mean": mean}
    ahat = oracle.block_scales(state)
    for i in range(a.size):
        prod = np.float32(float(m[q[i]]) * float(s[0]))
        assert ahat[i] == np.float32(float(prod) + float(mean))


def test_dynamic_codes_are_the_nearest_map_value():
    """Scales [0, 2, 1 + c, 1 - c] have mean 1 and group scale 1, so the
    normalised value of the last two is exactly +-c: their codes must be the
    brute-force nearest map index (lowest index on a tie), for c spread over
    every decade, on the map values and on both sides of every midpoint."""
    m = oracle.dynamic_map().astype(np.float64)
    mids = (m[:-1] + m[1:]) / 2
    cs = set()
    rng = np.random.default_rng(12)
    for v in np.concatenate([np.abs(m), np.abs(mids), 10.0 ** rng.uniform(-7, 0, 400)]):
        for c in (v, v * (1 + 2.0 ** -20), v * (1 - 2.0 ** -20)):
            c = float(np.float32(c))
            # 1 + c and 1 - c must be binary32 values for the construction
            if 0 < c < 1 and float(np.float32(1 + c)) == 1 + c and float(np.float32(1 - c)) == 1 - c:
                cs.add(c)
    cs = sorted(cs)
    assert len(cs) > 100
    for c in cs:
        a = np.array([0.0, 2.0, 1.0 + c, 1.0 - c], np.float32)
        q, s, mean = oracle.double_quant_dynamic(a)
        assert mean == 1.0 and s[0] == 1.0
        for t, code in ((c, q[2]), (-c, q[3])):
            dist = np.abs(m - t)
            best = int(np.flatnonzero(dist == dist.min())[0])
            assert code == best, (t, code, best)


def test_dynamic_double_quant_bounds():
    """|a_hat - a| <= s_g * (largest half gap of the map) + rounding slack;
    a group with s_g = 0 dequantizes to the mean exactly."""
    m = oracle.dynamic_map().astype(np.float64)
    hmax = np.max(np.diff(m)) / 2
    rng = np.random.default_rng(14)
    for nb in (1, 255, 256, 257, 1000, 4096 + 3):
        a = oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(
            np.abs(rng.standard_normal(nb)).astype(np.float32) * np.float32(0.06)))
        q, s, mean = oracle.double_quant_dynamic(a)
        g = np.arange(nb) // 256
        state = {"double_quant": True, "dq_map": "dynamic", "absmax": q, "absmax2": s,
                 "absmax_mean": mean}
        ahat = oracle.block_scales(state).astype(np.float64)
        slack = 4 * np.array([f32_ulp(max(abs(float(mean)), float(s[gi]), float(ai)))
                              for gi, ai in zip(g, a)])
        assert np.all(np.abs(ahat - a) <= s[g].astype(np.float64) * hmax + slack)
    a = np.full(300, 0.25, np.float32)
    q, s, mean = oracle.double_quant_dynamic(a)
    assert np.all(s == 0) and np.all(oracle.dynamic_map()[q] == 0)
    state = {"double_quant": True, "dq_map": "dynamic", "absmax": q, "absmax2": s,
             "absmax_mean": mean}
    assert np.all(oracle.block_scales(state) == np.float32(0.25))


def test_dynamic_map_quantize_state():
    w = oracle.f32_to_bf16_bits(np.random.default_rng(15).standard_normal(64 * 600)
                                .astype(np.float32) * np.float32(0.02))
    lin = oracle.quantize(w, True)
    dyn = oracle.quantize(w, True, dq_map="dynamic")
    assert np.array_equal(lin["packed"], dyn["packed"])       # codes use the true a_b
    assert dyn["absmax"].dtype == np.uint8 and dyn["dq_map"] == "dynamic"
    assert dyn["absmax_mean"] == lin["absmax_mean"]
    assert np.array_equal(dyn["absmax2"], lin["absmax2"])
    with pytest.raises(ValueError):
        oracle.quantize(w, True, dq_map="quantile")


# --------------------------------------------------------------------------
# Dequant and matmul
# --------------------------------------------------------------------------
def test_dequant_with_unit_absmax_returns_levels():
    L = oracle.codebook()
    lv = oracle.f32_to_bf16_bits(L)
    # 4 copies of the 16 levels -> one block of 64 whose absmax is exactly 1
    w = np.tile(lv, 4)
    q = oracle.quantize(w, False)
    assert q["absmax"][0] == 1.0
    assert np.array_equal(q["codes"], np.tile(np.arange(16, dtype=np.uint8), 4))
    assert np.array_equal(oracle.dequantize(q["packed"], q), w)


def test_matmul_unit_vector_is_exact_column():
    from synth import normal_bf16

    N, K = 48, 128
    w = normal_bf16((N, K), 0.02, 99)
    for dq in (False, True):
        q = oracle.quantize(w, dq)
        what = oracle.dequantize(q["packed"], q).reshape(N, K)
        for k in (0, 5, 127):
            x = np.zeros((1, K), np.uint16)
            x[0, k] = 0x3F80                   # bf16 1.0
            y = oracle.dequant_matmul_ref(x, q["packed"], q, N, K)
            assert np.array_equal(y[0], oracle.bf16_bits_to_f32(what[:, k]).astype(np.float64))


def test_matmul_bruteforce_loops():
    from synth import normal_bf16

    M, N, K = 2, 3, 64
    x = normal_bf16((M, K), 1.0, 5)
    w = normal_bf16((N, K), 0.5, 6)
    y = oracle.matmul_ref(x, w)
    xf = oracle.bf16_bits_to_f32(x).reshape(M, K)
    wf = oracle.bf16_bits_to_f32(w).reshape(N, K)
    for m in range(M):
        for n in range(N):
            acc = math.fsum(float(xf[m, k]) * float(wf[n, k]) for k in range(K))
            assert y[m, n] == pytest.approx(acc, rel=1e-13, abs=1e-13)


def test_rel_frobenius():
    assert oracle.rel_frobenius([3.0, 4.0], [3.0, 4.0]) == 0.0
    assert oracle.rel_frobenius([3.0, 5.0], [3.0, 4.0]) == pytest.approx(0.2)


# --------------------------------------------------------------------------
# Memory arithmetic and the pages' figures
# --------------------------------------------------------------------------
def test_storage_bits_per_weight():
    n = 4096 * 4096
    assert oracle.storage_bytes(n, False) * 8 / n == pytest.approx(4.5)
    bits_dq = oracle.storage_bytes(n, True) * 8 / n
    assert bits_dq == pytest.approx(4 + 8 / 64 + 32 / (64 * 256), abs=1e-5)
    # sizes the quantizer actually returns agree with the formula
    from synth import normal_bf16
    w = normal_bf16((64, 1024), 0.02, 8)
    for dq in (False, True):
        q = oracle.quantize(w, dq)
        got = q["packed"].nbytes + q["absmax"].nbytes
        if dq:
            got += q["absmax2"].nbytes + 4
        assert got == oracle.storage_bytes(w.size, dq)


def test_pages_memory_figures():
    g = json.load(open(GOLDEN))
    n7 = 7e9
    # fp16 = 2 bytes per parameter reproduces both fp16 figures the pages print
    assert n7 * 2 / 1e9 == pytest.approx(g["fp16_7b_model_gb"]["value"])
    assert g["gpt3_params"]["value"] * 2 / 1e9 == pytest.approx(g["gpt3_fp16_gb_about"]["value"])
    # NF4 + double quant: 7B weights take ~3.6 GB, i.e. "about 4 GB" (the rest
    # of a real model, embeddings and norms, stays 16-bit)
    n = 4096 * 4096
    per_weight = oracle.storage_bytes(n, True) / n
    gb = n7 * per_weight / 1e9
    assert 3.0 < gb <= g["nf4_dq_7b_model_gb_about"]["value"]
    # 4-bit saves about three quarters of 16-bit storage
    saving = 1 - oracle.storage_bytes(n, False) / (2 * n)
    assert saving == pytest.approx(g["four_bit_saving_fraction"]["value"], abs=0.05)
    # double quant saves "a few tenths of a bit" per parameter
    lo, hi = g["double_quant_saving_bits_per_param"]["range"]
    d = (oracle.storage_bytes(n, False) - oracle.storage_bytes(n, True)) * 8 / n
    assert lo <= d <= hi and d == pytest.approx(0.373, abs=1e-3)
    # the measured table's ordering is the ordering of bits per weight
    t = g["qwen2_5_1_5b_allocated_mb"]
    assert t["nf4_double_quant"] < t["fp4"] < t["int8"] < t["fp16"]


def test_nf4_error_below_uniform_int4():
    """Direction of the pages' figure (NF4 error about 0.6x INT4, section
    3.2): on normal weights in blocks of 64, NF4 mean squared error is below
    that of blockwise absmax INT4 with 15 symmetric levels."""
    rng = np.random.default_rng(12)
    wf = rng.standard_normal(64 * 4000).astype(np.float32)
    w = oracle.f32_to_bf16_bits(wf)
    wf = oracle.bf16_bits_to_f32(w).astype(np.float64)
    q = oracle.quantize(w, False)
    L = oracle.codebook().astype(np.float64)
    a = np.repeat(q["absmax"].astype(np.float64), 64)
    mse_nf4 = np.mean((wf - L[q["codes"]] * a) ** 2)
    int4 = np.round(wf / a * 7) / 7 * a
    mse_int4 = np.mean((wf - int4) ** 2)
    g = json.load(open(GOLDEN))
    assert mse_nf4 < mse_int4
    assert mse_nf4 / mse_int4 < 1.0 and g["nf4_vs_int4_error_ratio_about"]["value"] < 1.0


# --------------------------------------------------------------------------
# FP4, the other 4-bit quant type (mlqm.cn article, section 4)
# --------------------------------------------------------------------------
# The E2M1 element values as the OCP Microscaling Formats specification
# (v1.0, FP4 E2M1 table) lists them for codes 0b0000 .. 0b0111; codes with
# bit 3 set are their negatives.  Typed in from the standard, independent of
# the oracle's bit-field decoding.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_fp4_levels_are_the_e2m1_table():
    L = oracle.fp4_codebook()
    want = np.array(E2M1_TABLE + [-v for v in E2M1_TABLE], dtype=np.float64) / 6.0
    assert np.array_equal(L, want.astype(np.float32))
    assert L[7] == 1.0 and L[15] == -1.0 and L[0] == 0.0 and L[8] == 0.0
    assert np.all(L[8:] == -L[:8])
    assert np.max(np.abs(L)) == 1.0


def test_fp4_sorted_codes():
    L = oracle.fp4_codebook()
    order = oracle.sorted_codes("fp4")
    assert order.size == 15 and 8 not in order.tolist()
    assert np.all(np.diff(L[order].astype(np.float64)) > 0)
    assert list(order[:8]) == [15, 14, 13, 12, 11, 10, 9, 0]
    assert np.array_equal(oracle.sorted_codes("nf4"), np.arange(16))


def brute_fp4_codes(x: np.ndarray) -> np.ndarray:
    """Nearest of the 15 distinct FP4 levels in binary64, the lower value on
    ties, as its code: a direct search over the codes, independent of the
    threshold table and of the code order used by the encoder."""
    L = oracle.fp4_codebook().astype(np.float64)
    codes = [c for c in range(16) if c != 8]
    best = np.full(x.size, -1, dtype=np.int64)
    bestd = np.full(x.size, np.inf)
    xd = x.astype(np.float64)
    for c in codes:
        d = np.abs(xd - L[c])
        better = (d < bestd) | ((d == bestd) & (L[c] < L[np.maximum(best, 0)]))
        best = np.where(better, c, best)
        bestd = np.where(better, d, bestd)
    return best.astype(np.uint8)


def _quantize_unit_fp4(x):
    # blocks of 63 values plus a +1 anchor: the absmax is exactly 1, so the
    # normalisation is the identity
    x = np.asarray(x, dtype=np.float32)
    nblk = -(-x.size // 63)
    body = np.zeros(nblk * 63, np.float32)
    body[:x.size] = x
    w = np.concatenate([body.reshape(nblk, 63), np.ones((nblk, 1), np.float32)], axis=1).ravel()
    bits = oracle.f32_to_bf16_bits(w)
    assert np.array_equal(oracle.bf16_bits_to_f32(bits), w)   # inputs are bf16 values
    q = oracle.quantize(bits, False, quant_type="fp4")
    assert np.all(q["absmax"] == 1.0)
    return q["codes"].reshape(nblk, 64)[:, :63].ravel()[:x.size]


def test_fp4_encode_matches_bruteforce():
    L = oracle.fp4_codebook().astype(np.float64)
    order = oracle.sorted_codes("fp4")
    xs = []
    for a, b in zip(L[order][:-1], L[order][1:]):     # bf16 values around each midpoint
        m = np.float32((a + b) / 2)
        bits = oracle.f32_to_bf16_bits(np.array([m], np.float32))[0].astype(np.int32)
        xs += [oracle.bf16_bits_to_f32(np.array([(bits + k) & 0xFFFF], np.uint16))[0]
               for k in range(-40, 41)]
    rng = np.random.default_rng(21)
    xs = np.concatenate([np.array(xs, np.float32),
                         oracle.bf16_bits_to_f32(oracle.f32_to_bf16_bits(
                             rng.uniform(-1, 1, 60000).astype(np.float32))),
                         np.array([-1.0, 1.0, 0.0, -0.0, -2.0 ** -100, 2.0 ** -100], np.float32)])
    xs = xs[np.abs(xs) <= 1]
    assert np.array_equal(_quantize_unit_fp4(xs), brute_fp4_codes(xs))


def test_fp4_exact_midpoint_ties_go_to_lower_value():
    L = oracle.fp4_codebook().astype(np.float64)
    order = oracle.sorted_codes("fp4")
    found = 0
    for i in range(14):
        m = (L[order[i]] + L[order[i + 1]]) / 2
        if float(np.float32(m)) == m:
            found += 1
            x = np.array([m], np.float32)
            assert oracle.encode(x, np.ones(1, np.float32),
                                 oracle.thresholds(L[order].astype(np.float32)),
                                 order=order, zero_code=0)[0] == order[i]
            assert brute_fp4_codes(x)[0] == order[i]
    assert found >= 2     # the two midpoints next to 0 (+-fl32(1/12)/2) are exact


def test_fp4_zero_block_negative_zero_never_emitted():
    w = np.zeros(64 + 64, dtype=np.uint16)
    rng = np.random.default_rng(8)
    tail = rng.standard_normal(64).astype(np.float32) * np.float32(1e-6)
    tail[0] = 5.0
    w[64:] = oracle.f32_to_bf16_bits(tail)
    q = oracle.quantize(w, False, quant_type="fp4")
    assert np.all(q["codes"][:64] == 0)
    assert not np.any(q["codes"] == 8)
    assert np.all(q["codes"][65:] == 0)          # tiny values of either sign -> +0
    deq = oracle.dequantize(q["packed"], q, w.size)
    assert np.all(deq[:64] == 0) and np.all(deq[65:] == 0)


def test_fp4_reconstruction_error_bound():
    L = oracle.fp4_codebook().astype(np.float64)
    srt = np.sort(np.unique(L))
    hmax = np.max(np.diff(srt)) / 2
    assert abs(hmax - 1.0 / 6.0) < 1e-7        # the 2/3 .. 1 gap
    rng = np.random.default_rng(4)
    for dq in (False, True):
        w = oracle.f32_to_bf16_bits(rng.standard_normal(64 * 600).astype(np.float32) * np.float32(0.02))
        q = oracle.quantize(w, dq, quant_type="fp4")
        wf = oracle.bf16_bits_to_f32(w).astype(np.float64)
        a = np.repeat(q["absmax_fp32"].astype(np.float64), 64)
        rec = L[q["codes"]] * a
        assert np.all(np.abs(wf - rec) <= a * hmax * (1 + 2.0 ** -20))


def test_fp4_dequant_with_unit_absmax_returns_levels():
    L = oracle.fp4_codebook()
    order = oracle.sorted_codes("fp4")
    vals = np.concatenate([L[order], L[order], L[order], L[order][:19]])   # 64 values, max 1
    w = oracle.f32_to_bf16_bits(vals)
    q = oracle.quantize(w, False, quant_type="fp4")
    assert q["absmax"][0] == 1.0
    assert np.array_equal(q["codes"], np.concatenate([order, order, order, order[:19]]))
    assert np.array_equal(oracle.dequantize(q["packed"], q), oracle.f32_to_bf16_bits(vals))


# --------------------------------------------------------------------------
# FP16 compute dtype (mlqm.cn article, section 4)
# --------------------------------------------------------------------------
def test_f16_rounding_hand_cases():
    f = np.array([65504.0, 65519.996, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25,
                  1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, -2.0, 0.0, -0.0, 2.0 ** -14], np.float32)
    want = [0x7BFF, 0x7BFF, 0x7C00, 0x0001, 0x0000, 0x0002,
            0x3C00, 0x3C02, 0xC000, 0x0000, 0x8000, 0x0400]
    assert oracle.f32_to_f16_bits(f).tolist() == want
    assert oracle.f16_bits_to_f32(np.array(want[:2], np.uint16)).tolist() == [65504.0, 65504.0]


def test_f16_rounding_matches_torch():
    import torch

    rng = np.random.default_rng(9)
    f = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-6).astype(np.float32),      # subnormal range
        (rng.standard_normal(2000) * 7e4).astype(np.float32),       # around overflow
    ])
    # binary32 values exactly halfway between two binary16 neighbours
    h = rng.integers(0, 0x7BFF, 4000).astype(np.uint16)
    lo = oracle.f16_bits_to_f32(h).astype(np.float64)
    hi = oracle.f16_bits_to_f32(h + np.uint16(1)).astype(np.float64)
    f = np.concatenate([f, ((lo + hi) / 2).astype(np.float32)])
    ours = oracle.f32_to_f16_bits(f)
    ref = torch.from_numpy(f).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_dequant_hand_example():
    L = oracle.codebook()
    lv = oracle.f32_to_bf16_bits(L * np.float32(3.0))
    w = np.tile(lv, 4)                               # absmax 3, every level once per 16
    q = oracle.quantize(w, False)
    assert q["absmax"][0] == 3.0
    deq = oracle.dequantize(q["packed"], q, dtype="f16")
    assert deq[15] == 0x4200 and deq[0] == 0xC200 and deq[7] == 0x0000   # 3, -3, +0
    want = oracle.f32_to_f16_bits((L * np.float32(3.0)).astype(np.float32))
    assert np.array_equal(deq, np.tile(want, 4))


def test_dx_reference_is_the_transposed_product():
    """dX = dY . W_hat: for dY = e_n (one-hot rows) it is row n of W_hat, and
    <dX, X> = <dY, X . W_hat^T> for any X (the adjoint identity between the
    forward product and its input gradient), by brute-force loops."""
    rng = np.random.default_rng(41)
    N, K, M = 64, 128, 3
    w = oracle.f32_to_bf16_bits(rng.standard_normal(N * K).astype(np.float32) * np.float32(0.05))
    for qt in ("nf4", "fp4"):
        q = oracle.quantize(w, True, quant_type=qt)
        what = oracle.bf16_bits_to_f32(oracle.dequantize(q["packed"], q)).astype(np.float64)
        what = what.reshape(N, K)
        eye = np.zeros((N, N), np.uint16)
        eye[np.arange(N), np.arange(N)] = 0x3F80
        assert np.array_equal(oracle.dequant_matmul_dx_ref(eye, q["packed"], q, N, K), what)
        dy = oracle.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
        x = oracle.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
        dx = oracle.dequant_matmul_dx_ref(dy, q["packed"], q, N, K)
        y = oracle.dequant_matmul_ref(x, q["packed"], q, N, K)
        dyf = oracle.bf16_bits_to_f32(dy).astype(np.float64)
        xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
        lhs = sum(dx[m, k] * xf[m, k] for m in range(M) for k in range(K))
        rhs = sum(dyf[m, n] * y[m, n] for m in range(M) for n in range(N))
        assert abs(lhs - rhs) <= 1e-9 * (abs(lhs) + 1)


def test_lora_reference_adds_the_low_rank_term():
    """Y = X . W_hat^T + XA . B^T: with B = 0 it is the plain product, and
    with XA one-hot (row m picks rank k) the added term is column k of B,
    checked by brute-force loops."""
    rng = np.random.default_rng(43)
    N, K, M, r = 32, 128, 4, 16
    w = oracle.f32_to_bf16_bits(rng.standard_normal(N * K).astype(np.float32) * np.float32(0.05))
    q = oracle.quantize(w, True)
    x = oracle.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    base = oracle.dequant_matmul_ref(x, q["packed"], q, N, K)
    zero_b = np.zeros((N, r), np.uint16)
    xa = oracle.f32_to_bf16_bits(rng.standard_normal((M, r)).astype(np.float32))
    assert np.array_equal(oracle.lora_matmul_ref(x, q["packed"], q, N, K, xa, zero_b), base)
    onehot = np.zeros((M, r), np.uint16)
    for m in range(M):
        onehot[m, (3 * m) % r] = 0x3F80
    b = oracle.f32_to_bf16_bits(rng.standard_normal((N, r)).astype(np.float32))
    bf = oracle.bf16_bits_to_f32(b).astype(np.float64)
    got = oracle.lora_matmul_ref(x, q["packed"], q, N, K, onehot, b) - base
    for m in range(M):
        for n in range(N):
            assert abs(got[m, n] - bf[n, (3 * m) % r]) <= 1e-12


def test_lora_down_reference_pins():
    """XA = s . X . A^T: one-hot rows of X pick scaled columns of A exactly,
    a brute-force triple loop agrees on a small case, and s = 0 gives 0."""
    rng = np.random.default_rng(77)
    M, K, r = 5, 64, 16
    a_f = rng.standard_normal((r, K)).astype(np.float32)
    a = oracle.f32_to_bf16_bits(a_f)
    a64 = oracle.bf16_bits_to_f32(a).astype(np.float64).reshape(r, K)
    ks = [0, 7, 31, 32, 63]
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), ks] = 0x3F80                          # 1.0
    got = oracle.lora_down_ref(x, a, 0.5, M, K)
    assert np.array_equal(got, 0.5 * a64[:, ks].T)
    xf = rng.standard_normal((M, K)).astype(np.float32)
    xb = oracle.f32_to_bf16_bits(xf)
    x64 = oracle.bf16_bits_to_f32(xb).astype(np.float64).reshape(M, K)
    want = np.zeros((M, r))
    for m in range(M):
        for j in range(r):
            acc = 0.0
            for k in range(K):
                acc += x64[m, k] * a64[j, k]
            want[m, j] = 2.0 * acc
    assert np.allclose(oracle.lora_down_ref(xb, a, 2.0, M, K), want, rtol=1e-12, atol=1e-12)
    assert not np.any(oracle.lora_down_ref(xb, a, 0.0, M, K))

