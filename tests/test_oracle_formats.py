"""Pins for the oracle's number formats (CPU only).

Each test checks the oracle against something other than itself: the OCP MX
format tables (tests/golden/ocp_mx_element_values.txt), brute-force nearest
searches, closed forms, exhaustive enumeration, or exact rational arithmetic.
"""

import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_values():
    rows = []
    with open(os.path.join(GOLDEN, "ocp_mx_element_values.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fmt, code, val = line.split()
            rows.append((fmt, int(code, 16), float(val)))
    return rows


def test_golden_element_tables():
    for fmt, code, val in _golden_values():
        if fmt == "e2m1":
            got = float(F.e2m1_value(code))
        elif fmt == "e4m3":
            got = float(F.e4m3_value(code))
        else:
            got = 2.0 ** (code - 127)
        assert got == val and np.signbit(got) == np.signbit(val), (fmt, hex(code), got, val)


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = F.bf16_bits_to_f32(b)
    return x[np.isfinite(x)]


def _brute_nearest(mag, grid, even_of):
    """Nearest grid value by exhaustive search; ties go to the candidate whose
    code is even (even_of(index) tells the code's parity)."""
    d = np.abs(mag[:, None] - grid[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    out = np.empty(len(mag), dtype=np.int64)
    for n in range(len(mag)):
        idx = np.nonzero(cand[n])[0]
        if len(idx) == 1:
            out[n] = idx[0]
        else:
            ev = [i for i in idx if even_of(i)]
            assert len(ev) == 1
            out[n] = ev[0]
    return out


def test_e2m1_rounding_brute_force():
    # every bf16 value scaled into the E2M1 range, plus all midpoints
    x = _all_finite_bf16().astype(np.float64)
    x = x[np.abs(x) < 16]
    x = np.concatenate([x, F._E2M1_MIDS, -F._E2M1_MIDS, [7.99, 100.0]])
    codes = F.e2m1_round_code(x)
    mag = np.minimum(np.abs(x), 6.0)
    want = _brute_nearest(mag, F.E2M1_VALUES, lambda i: i % 2 == 0)
    assert np.array_equal(codes & 7, want)
    assert np.array_equal((codes >> 3) & 1, np.signbit(x).astype(np.uint8))


def test_e2m1_grid_round_trips_through_mxfp4():
    # every grid value times 2**e, in a block whose max fixes the scale to e
    for e in (-127, -20, -1, 0, 3, 40, 125):
        vals = np.concatenate([F.E2M1_VALUES, -F.E2M1_VALUES[1:]])
        blk = np.zeros(32)
        blk[: len(vals)] = vals
        blk[31] = 4.0  # amax in [4, 8) -> shared exponent 0 before scaling
        x = np.ldexp(blk, e).astype(np.float32)
        if not np.all(np.ldexp(x.astype(np.float64), -e) == blk):
            continue  # not representable in float32 at this e
        codes, scales = F.quantize_mxfp4(x[None, :])
        assert int(scales[0, 0]) == e + 127
        back = F.dequantize_mxfp4(codes, scales)[0]
        assert np.array_equal(back, x.astype(np.float64))


def test_e8m0_closed_form():
    rng = np.random.default_rng(0)
    for k in range(-126, 127):
        mant = rng.uniform(1.0, 2.0, size=8)
        amax = np.ldexp(mant, k)
        e4 = F.e8m0_exponent(amax, 2)
        e8 = F.e8m0_exponent(amax, 8)
        assert np.all(e4 + 127 == np.clip(125 + k, 0, 254))
        assert np.all(e8 + 127 == np.clip(119 + k, 0, 254))
    assert F.e8m0_exponent(np.array([0.0]), 2)[0] == -127
    assert F.e8m0_exponent(np.array([2.0 ** -140]), 8)[0] == -127


def test_e4m3_codes_round_trip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = F.e4m3_value(codes)
    assert np.array_equal(F.e4m3_round_code(vals), codes)
    assert float(F.e4m3_value(0x7E)) == 448.0
    assert F.e4m3_round_code(np.array([1e9]))[0] == 0x7E
    assert F.e4m3_round_code(np.array([-1e9]))[0] == 0xFE


def test_e4m3_rounding_brute_force():
    x = _all_finite_bf16().astype(np.float64)
    x = x[np.abs(x) < 600]
    x = np.concatenate([x, F._E4M3_MIDS])
    codes = F.e4m3_round_code(x)
    grid = F._E4M3_MAGS
    want = _brute_nearest(np.minimum(np.abs(x), 448.0), grid, lambda i: i % 2 == 0)
    assert np.array_equal(codes & 0x7F, want)


def test_mxfp8_keys_layout_and_scale():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((2, 64, 8)).astype(np.float32)
    v[0, 5, 3] = 300.0
    codes, scales = F.quantize_mxfp8_keys(v)
    assert codes.shape == (2, 8, 64) and scales.shape == (2, 8, 2)
    # block (b=0, d=3, keys 0..31) has amax 300 in [256, 512) -> e = 8 - 8 = 0
    assert scales[0, 3, 0] == 127
    back = F.dequantize_mxfp8_keys(codes, scales)
    assert back.shape == v.shape
    assert back[0, 5, 3] == 288.0  # E4M3 steps by 32 in [256, 512): 300 -> 288
    # element-wise error: half a step of a 3-bit mantissa (<= |x| * 2**-4) unless
    # |x| / 2**e lies in (448, 512), where the OCP rule clips it to 448
    err = np.abs(back - v)
    e = (scales.astype(np.int64) - 127).repeat(32, axis=2).swapaxes(1, 2)
    scaled = np.abs(v) / 2.0 ** e
    clipped = scaled > 464
    assert np.all(err[~clipped] <= np.abs(v[~clipped]) * 2.0 ** -4 + 2.0 ** -20)
    assert np.all(back[clipped] == np.sign(v[clipped]) * 448 * 2.0 ** e[clipped])


def test_f16_rounding_brute_force():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-6, 4, 4000),
                        rng.uniform(-70000, 70000, 100)])
    allh = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    fin = np.isfinite(allh)
    hv = allh[fin].astype(np.float64)
    hb = np.arange(1 << 16)[fin]
    got = F.round_f16(x).astype(np.float64)
    for n in range(len(x)):
        if abs(x[n]) >= 65520:
            assert np.isinf(got[n])
            continue
        d = np.abs(hv - x[n])
        best = d.min()
        cand = np.nonzero(d == best)[0]
        if len(cand) > 1:
            cand = [c for c in cand if hb[c] % 2 == 0]
        assert got[n] == hv[cand[0]] or (got[n] == 0 and hv[cand[0]] == 0)


def _round_fraction_f32(q: Fraction) -> np.float32:
    f = np.float32(float(q))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - q)
        key = (d, int(np.array(cand, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def test_fma_f32_exact_rounding():
    rng = np.random.default_rng(7)
    a = (rng.standard_normal(3000) * 10.0 ** rng.integers(-3, 4, 3000)).astype(np.float32)
    b = (rng.standard_normal(3000) * 10.0 ** rng.integers(-3, 4, 3000)).astype(np.float32)
    c = (rng.standard_normal(3000) * 10.0 ** rng.integers(-3, 4, 3000)).astype(np.float32)
    # constructed cases: c = -round(a*b) leaves the tiny exact residual;
    # c = 6144.0 lands a*b + c near float32 ties on the 2**-11 grid
    a2 = rng.uniform(-50, 50, 2000).astype(np.float32)
    b2 = np.full(2000, np.float32(0.12752323))
    c2 = np.full(2000, np.float32(6144.0 + 8 - 17))
    aa = np.concatenate([a, a, a2])
    bb = np.concatenate([b, b, b2])
    cc = np.concatenate([c, -(a.astype(np.float64) * b).astype(np.float32), c2])
    got = F.fma_f32(aa, bb, cc)
    for n in range(len(aa)):
        exact = Fraction(float(aa[n])) * Fraction(float(bb[n])) + Fraction(float(cc[n]))
        assert got[n] == _round_fraction_f32(exact), (aa[n], bb[n], cc[n])
    # an exact tie resolved by the sign of the residual
    x = np.float32(1.0) + np.float32(2.0 ** -23)
    y = np.float32(1.0 + 2.0 ** -23)
    tie = F.fma_f32(np.array([x]), np.array([y]), np.array([np.float32(-1.0)]))
    assert tie[0] == _round_fraction_f32(Fraction(float(x)) * Fraction(float(y)) - 1)


def test_p_exponent_grid_is_nearest_grid_point():
    rng = np.random.default_rng(11)
    s = (rng.standard_normal(5000) * 40).astype(np.float32)
    c = np.float32(0.12752323)
    m = np.ceil((s.astype(np.float64) * float(c)).max()).astype(np.float32) + rng.integers(0, 12, 5000).astype(np.float32)
    xq = F.p_exponent_grid(s, c, m)
    for n in range(len(s)):
        exact = Fraction(float(s[n])) * Fraction(float(c)) - Fraction(float(m[n])) + 8
        k = exact * 2048
        lo = k.numerator // k.denominator
        frac = k - lo
        if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1):
            lo += 1
        assert Fraction(float(xq[n])) == Fraction(lo, 2048), (s[n], m[n])
    assert np.isneginf(F.p_exponent_grid(np.array([-np.inf], np.float32), c, np.float32(3))[0])


def test_p_e4m3_code_every_grid_point_vs_decimal():
    """Exhaustive: every x on the 2**-11 grid in [-11, 8] against 40-digit
    decimal exp2 and an exact nearest-even E4M3 decision."""
    getcontext().prec = 40
    ln2 = Decimal(2).ln()
    ks = np.arange(-11 * 2048, 8 * 2048 + 1)
    xq = ks / 2048.0
    got = F.p_e4m3_code(xq)
    mags = [Decimal(float(v)) for v in F._E4M3_MAGS]
    for n, k in enumerate(ks):
        y = (Decimal(int(k)) / 2048 * ln2).exp()
        # nearest E4M3 value with ties to the even code, by search
        lo = max(i for i in range(len(mags)) if mags[i] <= y) if y >= 0 else 0
        if lo == len(mags) - 1:
            want = lo
        else:
            dl, dh = y - mags[lo], mags[lo + 1] - y
            want = lo if dl < dh else lo + 1 if dh < dl else (lo if lo % 2 == 0 else lo + 1)
        assert int(got[n]) == want, (k, float(y), int(got[n]), want)
    assert F.p_e4m3_code(np.array([-np.inf]))[0] == 0
    assert F.p_e4m3_code(np.array([-10.0]))[0] == 0      # exact tie 2**-10 -> even code 0
    assert F.p_e4m3_code(np.array([8.0]))[0] == 0x78     # 256


def test_int4_g32_definition_and_bounds():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((50, 64)) * 3).astype(np.float32)
    x[3, :32] = 1.25                       # constant group -> s = 0, codes 0
    codes, s, z = F.quantize_int4_g32(x)
    assert codes.max() <= 15
    assert s[3, 0] == 0 and np.all(codes[3, :32] == 0)
    xh = F.dequantize_int4_g32(codes, s, z)
    assert np.all(xh[3, :32] == np.float32(np.float16(1.25)))
    # brute force: the code is the nearest integer (ties even) to fl32(fl32(x-z)/s), clamped
    sf = s.astype(np.float32).repeat(32, axis=1)
    zf = z.astype(np.float32).repeat(32, axis=1)
    for r in range(50):
        for d in range(64):
            if sf[r, d] == 0:
                assert codes[r, d] == 0
                continue
            t = np.float32(np.float32(x[r, d] - zf[r, d]) / sf[r, d])
            dist = [abs(float(t) - c) for c in range(16)]
            best = min(dist)
            cand = [c for c in range(16) if dist[c] == best]
            want = cand[0] if len(cand) == 1 else [c for c in cand if c % 2 == 0][0]
            assert codes[r, d] == want
    # reconstruction error: at most half a step plus the fp16 rounding of s and z
    step = sf
    err = np.abs(xh - x)
    ok = sf > 0
    assert np.all(err[ok] <= 0.5 * step[ok] * (1 + 2 ** -9) + np.abs(zf[ok]) * 2 ** -10 + 15 * step[ok] * 2 ** -10)
    # exact lattice: values z + k*s with representable s, z round-trip exactly
    lat = (np.float32(-1.5) + np.arange(32) % 16 * np.float32(0.25)).astype(np.float32)
    c2, s2, z2 = F.quantize_int4_g32(lat[None, :])
    assert s2[0, 0] == np.float16(0.25) and z2[0, 0] == np.float16(-1.5)
    assert np.array_equal(c2[0], np.arange(32) % 16)
    assert np.array_equal(F.dequantize_int4_g32(c2, s2, z2)[0], lat)


def test_pack_unpack_nibbles():
    c = np.arange(64, dtype=np.uint8) % 16
    p = F.pack_nibbles(c)
    assert p[0] == 0x10 and p[1] == 0x32
    assert np.array_equal(F.unpack_nibbles(p), c)


def test_bf16_round_trip():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = F.bf16_bits_to_f32(b)
    fin = np.isfinite(x)
    assert np.array_equal(F.f32_to_bf16_bits(x[fin]), b[fin])
