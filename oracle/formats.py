"""Number formats used on the attention path: plain definitions, slow and exact.

Test infrastructure only (see ``oracle/__init__``).

Sources: the ThriftAttention abstract (block-scaled quantisation moves
attention to 4-bit; selected blocks stay FP16), the "Attention Quantization"
topic page overview (block-scaled FP8/FP4 and integer formats), and the
public OCP Microscaling v1.0 rules for E2M1, E4M3 and the E8M0 shared scale.
Readings R2-R5, R7, R15, R17 and R19 are implemented here; each function
states the rule it follows.
"""

from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# bf16 <-> fp32
# --------------------------------------------------------------------------


def bf16_bits_to_f32(u16: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32.  Exact (reading R1)."""
    u16 = np.asarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 (ties to even) and return the bits."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = (b + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


# --------------------------------------------------------------------------
# E2M1 (FP4) elements
# --------------------------------------------------------------------------

#: magnitudes of the eight E2M1 codes 0..7 (sign is bit 3)
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1_MIDS = (E2M1_VALUES[:-1] + E2M1_VALUES[1:]) / 2.0


def _nearest_code_ties_even(mag: np.ndarray, mids: np.ndarray) -> np.ndarray:
    """Index of the grid value nearest to ``mag``; a tie picks the even index.

    ``mids`` are the midpoints between consecutive grid values (exact).
    Above the last midpoint the last index is returned (saturation).
    """
    lo = np.searchsorted(mids, mag, side="left")   # midpoints strictly below
    hi = np.searchsorted(mids, mag, side="right")  # midpoints at or below
    tie = lo != hi
    return np.where(tie, np.where(lo % 2 == 0, lo, lo + 1), lo).astype(np.int64)


def e2m1_round_code(v: np.ndarray) -> np.ndarray:
    """Round to E2M1 (reading R3): nearest of {0,.5,1,1.5,2,3,4,6}, ties to the
    even code, saturating at 6.  The sign bit always copies the sign of ``v``
    (so -0.0 and tiny negatives give code 8)."""
    v = np.asarray(v, dtype=np.float64)
    code = _nearest_code_ties_even(np.abs(v), _E2M1_MIDS)
    return (code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def e2m1_value(code: np.ndarray) -> np.ndarray:
    code = np.asarray(code, dtype=np.int64)
    mag = E2M1_VALUES[code & 7]
    return np.where(code & 8, -mag, mag)


# --------------------------------------------------------------------------
# E4M3 (OCP FP8) elements
# --------------------------------------------------------------------------


def e4m3_value(code: np.ndarray) -> np.ndarray:
    """Decode OCP E4M3 (bias 7, no infinities; 0x7F/0xFF are NaN)."""
    code = np.asarray(code, dtype=np.int64)
    e = (code >> 3) & 15
    m = code & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((code & 0x7F) == 0x7F, np.nan, mag)
    return np.where(code & 0x80, -mag, mag)


_E4M3_MAGS = e4m3_value(np.arange(127))          # codes 0..126: 0 .. 448
_E4M3_MIDS = (_E4M3_MAGS[:-1] + _E4M3_MAGS[1:]) / 2.0


def e4m3_round_code(v: np.ndarray) -> np.ndarray:
    """Round to OCP E4M3 (reading R5): nearest value, ties to the even code,
    magnitudes above 448 saturate to 448, subnormals kept, sign follows ``v``,
    NaN never produced.  Exact for float64 input."""
    v = np.asarray(v, dtype=np.float64)
    code = _nearest_code_ties_even(np.abs(v), _E4M3_MIDS)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


# --------------------------------------------------------------------------
# E8M0 shared scale (OCP MX rule, reading R2)
# --------------------------------------------------------------------------


def e8m0_exponent(amax: np.ndarray, emax_elem: int) -> np.ndarray:
    """Shared exponent e = floor(log2(amax)) - emax_elem, clamped to
    [-127, 127]; amax == 0 gives -127.  floor(log2) is taken exactly from the
    binary exponent (frexp), never from a rounded logarithm."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)          # amax = f * 2**ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1 - emax_elem
    e = np.clip(e, -127, 127)
    return np.where(amax == 0.0, -127, e)


# --------------------------------------------------------------------------
# MXFP4: blocks of 32 along the last axis (head_dim), readings R2-R4, R6
# --------------------------------------------------------------------------


def quantize_mxfp4(x: np.ndarray):
    """Quantise float32 ``x[..., D]`` to MXFP4 with one E8M0 scale per 32
    consecutive elements of the last axis.

    Returns ``(codes, scales)``: codes uint8 [..., D] (one E2M1 code per
    element, unpacked) and scale bytes uint8 [..., D/32] (= e + 127).
    """
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    assert D % 32 == 0
    xb = x.astype(np.float64).reshape(x.shape[:-1] + (D // 32, 32))
    e = e8m0_exponent(np.max(np.abs(xb), axis=-1), emax_elem=2)   # E2M1 emax = 2
    v = np.ldexp(xb, -e[..., None])                                # exact scaling
    codes = e2m1_round_code(v).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def hadamard_rotate(x: np.ndarray) -> np.ndarray:
    """Data-free rotation of each row of float32 ``x[..., D]`` (D a power of
    two) by the orthonormal Walsh-Hadamard matrix H/sqrt(D), Sylvester order
    (reading R34): the fast transform in place, stages h = 1, 2, 4, ..., D/2,
    each pair (j, j+h) in ascending j becoming (a+b, a-b), every sum rounded to
    fp32; then one fp32 multiply by fl32(1/sqrt(D)).

    The pages name rotation as the main alternative to promotion: it spreads
    outlier channels over every element of a block before MXFP4.  Applied to
    both Q and K it leaves QK^T unchanged in exact arithmetic."""
    y = np.array(x, dtype=np.float32, copy=True)
    D = y.shape[-1]
    assert D & (D - 1) == 0
    h = 1
    while h < D:
        yb = y.reshape(y.shape[:-1] + (D // (2 * h), 2, h))
        a = yb[..., 0, :].copy()
        b = yb[..., 1, :].copy()
        yb[..., 0, :] = (a + b).astype(np.float32)
        yb[..., 1, :] = (a - b).astype(np.float32)
        y = yb.reshape(y.shape)
        h *= 2
    return (y * np.float32(1.0 / np.sqrt(D))).astype(np.float32)


def dequantize_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E2M1(code) * 2**(scale-127), float64 (exact)."""
    codes = np.asarray(codes)
    D = codes.shape[-1]
    v = e2m1_value(codes).reshape(codes.shape[:-1] + (D // 32, 32))
    e = np.asarray(scales, dtype=np.int64) - 127
    return np.ldexp(v, e[..., None]).reshape(codes.shape)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Element 2k -> bits 0-3 and element 2k+1 -> bits 4-7 of byte k (R4)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 15) | ((c[..., 1::2] & 15) << 4)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


# --------------------------------------------------------------------------
# MXFP8 for V: blocks of 32 along the key axis (reading R5)
# --------------------------------------------------------------------------


def quantize_mxfp8_keys(v: np.ndarray):
    """Quantise float32 ``v[..., N, D]`` to MXFP8 E4M3 with one E8M0 scale per
    32 consecutive keys of each head_dim column (PV contracts over keys).

    Returns ``(codes_t, scales_t)`` in the key-contiguous layout the library
    writes: codes uint8 [..., D, N] and scale bytes uint8 [..., D, N/32].
    """
    v = np.asarray(v, dtype=np.float32)
    N, D = v.shape[-2], v.shape[-1]
    assert N % 32 == 0
    vt = np.swapaxes(v, -1, -2).astype(np.float64)            # [..., D, N]
    vb = vt.reshape(vt.shape[:-1] + (N // 32, 32))
    e = e8m0_exponent(np.max(np.abs(vb), axis=-1), emax_elem=8)  # E4M3 emax = 8
    codes = e4m3_round_code(np.ldexp(vb, -e[..., None])).reshape(vt.shape)
    return codes, (e + 127).astype(np.uint8)


def dequantize_mxfp8_keys(codes_t: np.ndarray, scales_t: np.ndarray) -> np.ndarray:
    """Inverse of :func:`quantize_mxfp8_keys`; returns float64 [..., N, D]."""
    codes_t = np.asarray(codes_t)
    N = codes_t.shape[-1]
    val = e4m3_value(codes_t).reshape(codes_t.shape[:-1] + (N // 32, 32))
    e = np.asarray(scales_t, dtype=np.int64) - 127
    vt = np.ldexp(val, e[..., None]).reshape(codes_t.shape)
    return np.swapaxes(vt, -1, -2)


# --------------------------------------------------------------------------
# fp16
# --------------------------------------------------------------------------


def round_f16(x: np.ndarray) -> np.ndarray:
    """Round to IEEE binary16, nearest-even (numpy's cast is correctly rounded;
    pinned by a brute-force test)."""
    return np.asarray(x).astype(np.float16)


# --------------------------------------------------------------------------
# INT4 asymmetric, 32-element groups along head_dim (decode cache, R19)
# --------------------------------------------------------------------------


def quantize_int4_g32(x: np.ndarray):
    """Asymmetric 4-bit quantisation of float32 ``x[..., D]`` per group of 32.

    s = fp16(fl32(fl32(max - min) / 15)), z = fp16(min),
    code = clamp(round_half_even(fl32(fl32(x - z) / s)), 0, 15)  (0 if s == 0).
    Returns codes uint8 [..., D] (unpacked), scale and zero float16 [..., D/32].
    """
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    assert D % 32 == 0
    xb = x.reshape(x.shape[:-1] + (D // 32, 32))
    mn = np.min(xb, axis=-1)
    mx = np.max(xb, axis=-1)
    s32 = np.float32(mx - mn) / np.float32(15.0)          # two fp32 roundings
    s = s32.astype(np.float16)
    z = mn.astype(np.float16)
    s_f = s.astype(np.float32)[..., None]
    z_f = z.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (xb - z_f) / s_f                               # fp32 ops, correctly rounded
    q = np.where(s_f == 0, np.float32(0), q)
    code = np.clip(np.rint(q), 0, 15).astype(np.uint8)     # rint: half to even
    return code.reshape(x.shape), s, z


def dequantize_int4_g32(codes, scale, zero) -> np.ndarray:
    """x_hat = fl32(code * s + z): the product is exact in fp32, so one rounding."""
    codes = np.asarray(codes)
    D = codes.shape[-1]
    c = codes.astype(np.float64).reshape(codes.shape[:-1] + (D // 32, 32))
    s = np.asarray(scale, dtype=np.float16).astype(np.float64)[..., None]
    z = np.asarray(zero, dtype=np.float16).astype(np.float64)[..., None]
    return (c * s + z).astype(np.float32).reshape(codes.shape)


# --------------------------------------------------------------------------
# exactly rounded fp32 fused multiply-add
# --------------------------------------------------------------------------


def fma_f32(a, b, c) -> np.ndarray:
    """Return fl32(a*b + c) with a single round-to-nearest-even, for float32
    inputs.  a*b is exact in float64; the sum is split exactly into s + err
    (Knuth's TwoSum), and the one case where rounding s alone would differ
    (s exactly halfway between two float32 values while err != 0) is fixed."""
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    b = np.asarray(b, dtype=np.float32).astype(np.float64)
    c = np.asarray(c, dtype=np.float32).astype(np.float64)
    with np.errstate(invalid="ignore"):
        p = a * b
        s = p + c
        bb = s - p
        err = (p - (s - bb)) + (c - bb)
        r = s.astype(np.float32)
        r64 = r.astype(np.float64)
        up = np.nextafter(r, np.float32(np.inf))
        dn = np.nextafter(r, np.float32(-np.inf))
        other = np.where(r64 > s, dn, up)
        o64 = other.astype(np.float64)
        half = (r64 + o64) * 0.5
        finite = np.isfinite(s)
        tie = finite & (half == s) & (err != 0) & (r64 != s)
        toward_other = np.sign(err) == np.sign(o64 - s)
        out = np.where(tie & toward_other, other, r)
    return np.asarray(out, dtype=np.float32)


# --------------------------------------------------------------------------
# P quantisation for low-bit tiles (readings R13-R15, R17)
# --------------------------------------------------------------------------

#: 1.5 * 2**12: a float32 in [2**12, 2**13) has a spacing of exactly 2**-11, so
#: adding it rounds the softmax exponent onto the 2**-11 grid in one step
P_GRID_MAGIC = np.float32(6144.0)
#: the exponent is offset by +8 so that E4M3 codes use the range up to 2**8
P_EXP_OFFSET = 8


def p_exponent_grid(s: np.ndarray, c: np.float32, m: np.ndarray) -> np.ndarray:
    """Exponent of P for a low-bit tile, on the 2**-11 grid (R14, R15):

        x_q = fl32(s*c + (6144 + 8 - m)) - 6144

    one fused multiply-add rounds s*c - m + 8 to the nearest multiple of 2**-11
    (ties to even); the subtraction is exact.  ``m`` is the integer-snapped
    running maximum (float32, integral).  Masked scores (-inf) give -inf.
    """
    s = np.asarray(s, dtype=np.float32)
    m = np.asarray(m, dtype=np.float32)
    off = (P_GRID_MAGIC + np.float32(P_EXP_OFFSET)) - m      # exact: integers < 2**24
    t = fma_f32(s, c, off)
    with np.errstate(invalid="ignore"):
        return np.where(np.isneginf(s), np.float32(-np.inf), t - P_GRID_MAGIC).astype(np.float32)


def p_e4m3_code(xq: np.ndarray) -> np.ndarray:
    """E4M3 code of 2**xq (xq <= 8 on the 2**-11 grid, or -inf), nearest-even.

    float64 exp2 of a grid point is within 1e-16 relative of the real 2**xq,
    and no grid point lies within 1e-6 relative of an E4M3 midpoint except
    xq = -10 (2**-10 is itself the midpoint between 0 and 2**-9, an exact tie
    that exp2 reproduces exactly); this is pinned against 40-digit decimal
    arithmetic over every grid point in tests/test_oracle_formats.py.
    """
    xq = np.asarray(xq, dtype=np.float64)
    return e4m3_round_code(np.exp2(xq))
