"""Pins for the oracle's mixed-precision attention (CPU only)."""

import math
from fractions import Fraction

import numpy as np
import pytest

import mxq_inputs
from oracle import attention as A
from oracle import formats as F
from oracle import select as S


def _inputs(N=256, D=64, Hq=2, Hkv=1, seed=0, n_valid=None, scale_q=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Hq, N, D)).astype(np.float32) * np.float32(scale_q)
    k = rng.standard_normal((1, Hkv, N, D)).astype(np.float32)
    v = rng.standard_normal((1, Hkv, N, D)).astype(np.float32)
    nv = N if n_valid is None else n_valid
    for t in (q, k, v):
        t[:, :, nv:] = 0
    return F.f32_to_bf16_bits(q), F.f32_to_bf16_bits(k), F.f32_to_bf16_bits(v), nv


def _full_mask(N, Bq, Bk, Hq):
    n_qt, n_kt = N // Bq, N // Bk
    m = np.zeros((1, Hq, n_qt, (n_kt + 31) // 32), dtype=np.uint32)
    for j in range(n_kt):
        m[..., j // 32] |= np.uint32(1 << (j % 32))
    return m


def test_lowbit_scores_are_exactly_rounded():
    q, k, v, nv = _inputs(N=64, D=64, Hq=1, seed=1)
    ops = A.prepare_operands(q, k, v, nv)
    s = A._exact_lowbit_scores(ops["q_hat"][0, 0], ops["k_hat"][0, 0], ops["q_exp"][0, 0], ops["k_exp"][0, 0])
    qc, qs = F.quantize_mxfp4(F.bf16_bits_to_f32(q)[0, 0])
    kc, ks = F.quantize_mxfp4(F.bf16_bits_to_f32(k)[0, 0])
    for r in range(0, 64, 7):
        for c in range(0, 64, 5):
            exact = Fraction(0)
            for d in range(64):
                a = Fraction(float(F.e2m1_value(qc[r, d]))) * Fraction(2) ** (int(qs[r, d // 32]) - 127)
                b = Fraction(float(F.e2m1_value(kc[c, d]))) * Fraction(2) ** (int(ks[c, d // 32]) - 127)
                exact += a * b
            f = np.float32(float(exact))
            # float(Fraction) is correctly rounded to double; check the fp32 rounding by neighbours
            cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
            best = min(cands, key=lambda z: (abs(Fraction(float(z)) - exact), int(np.array(z).view(np.uint32)) & 1))
            assert s[r, c] == best


def _fraction_score(qc, qs, kc, ks, r, c):
    exact = Fraction(0)
    for d in range(qc.shape[-1]):
        a = Fraction(float(F.e2m1_value(qc[r, d]))) * Fraction(2) ** (int(qs[r, d // 32]) - 127)
        b = Fraction(float(F.e2m1_value(kc[c, d]))) * Fraction(2) ** (int(ks[c, d // 32]) - 127)
        exact += a * b
    return exact


def _is_rounding_of(z, exact):
    f = np.float32(z)
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda w: (abs(Fraction(float(w)) - exact), int(np.array(w).view(np.uint32)) & 1))
    return f == best


@pytest.mark.parametrize("zero_side", ["q", "k"])
def test_all_zero_block_is_left_out_of_the_spread(zero_side):
    """A head_dim block whose q (or k) elements are all zero has E8M0 0 (2^-127)
    and contributes exactly 0, so a huge exponent on the other side of that
    block must not trip the exactness guard; the scores stay exactly rounded."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 1, 64, 128)).astype(np.float32)
    k = rng.standard_normal((1, 1, 64, 128)).astype(np.float32)
    if zero_side == "q":
        q[..., 32:64] = 0.0
        k[..., 32:64] *= np.float32(2.0 ** 60)  # spread ~187 if the zero block counted
    else:
        k[..., 64:96] = 0.0
        q[..., 64:96] *= np.float32(2.0 ** 60)
    qb, kb = F.f32_to_bf16_bits(q), F.f32_to_bf16_bits(k)
    ops = A.prepare_operands(qb, kb, kb, 64)
    s = A._exact_lowbit_scores(ops["q_hat"][0, 0], ops["k_hat"][0, 0], ops["q_exp"][0, 0], ops["k_exp"][0, 0])
    qc, qs = F.quantize_mxfp4(F.bf16_bits_to_f32(qb)[0, 0])
    kc, ks = F.quantize_mxfp4(F.bf16_bits_to_f32(kb)[0, 0])
    for r, c in ((0, 0), (5, 17), (63, 40), (31, 2)):
        assert _is_rounding_of(s[r, c], _fraction_score(qc, qs, kc, ks, r, c))


def test_spread_beyond_38_raises_and_20_is_exact():
    """Nonzero blocks whose exponents differ by more than 38 bits are refused
    (the float64 sum could round); a spread of about 20 (K block x2^12, Q
    block x2^-8) still gives exactly rounded scores."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 1, 64, 128)).astype(np.float32)
    k = rng.standard_normal((1, 1, 64, 128)).astype(np.float32)
    k_big = k.copy()
    k_big[..., 32:64] *= np.float32(2.0 ** 45)
    qb, kb = F.f32_to_bf16_bits(q), F.f32_to_bf16_bits(k_big)
    ops = A.prepare_operands(qb, kb, kb, 64)
    with pytest.raises(ValueError):
        A._exact_lowbit_scores(ops["q_hat"][0, 0], ops["k_hat"][0, 0], ops["q_exp"][0, 0], ops["k_exp"][0, 0])
    q2, k2 = q.copy(), k.copy()
    k2[..., 32:64] *= np.float32(2.0 ** 12)
    q2[..., 64:96] *= np.float32(2.0 ** -8)
    qb, kb = F.f32_to_bf16_bits(q2), F.f32_to_bf16_bits(k2)
    ops = A.prepare_operands(qb, kb, kb, 64)
    e = ops["q_exp"][0, 0][:, None, :] + ops["k_exp"][0, 0][None, :, :]
    assert int((e.max(-1) - e.min(-1)).max()) > 18
    s = A._exact_lowbit_scores(ops["q_hat"][0, 0], ops["k_hat"][0, 0], ops["q_exp"][0, 0], ops["k_exp"][0, 0])
    qc, qs = F.quantize_mxfp4(F.bf16_bits_to_f32(qb)[0, 0])
    kc, ks = F.quantize_mxfp4(F.bf16_bits_to_f32(kb)[0, 0])
    for r, c in ((0, 0), (7, 9), (63, 63), (20, 50)):
        assert _is_rounding_of(s[r, c], _fraction_score(qc, qs, kc, ks, r, c))


@pytest.mark.parametrize("causal", [False, True])
def test_all_fp16_mode_near_exact_softmax(causal):
    """P rounded to fp16 (relative error <= 2**-11) and S rounded to fp32 bound
    the difference to exact softmax attention: |out - exact| <= 2**-10 *
    max|v - exact| (+ fp32 noise)."""
    q, k, v, nv = _inputs(N=256, D=64, Hq=2, Hkv=1, seed=2)
    out, _ = A.attn_mixed_ref(q, k, v, nv, 64, 64, causal, mode=A.MODE_ALL_FP16)
    ex = A.attn_exact_ref(q, k, v, nv, causal)
    vmax = np.abs(F.bf16_bits_to_f32(v)).max()
    err = np.abs(out - ex).max()
    assert err <= 2.0 ** -10 * 2 * vmax * 1.001 + 1e-5
    assert err > 0  # P really is rounded


def test_mode_extremes_equal_mask_extremes():
    q, k, v, nv = _inputs(N=256, D=64, Hq=2, Hkv=1, seed=3)
    N, Bq, Bk = 256, 64, 64
    empty = np.zeros((1, 2, 4, 1), dtype=np.uint32)
    full = _full_mask(N, Bq, Bk, 2)
    a0, l0 = A.attn_mixed_ref(q, k, v, nv, Bq, Bk, True, mask=empty)
    b0, m0 = A.attn_mixed_ref(q, k, v, nv, Bq, Bk, True, mode=A.MODE_ALL_LOWBIT)
    a1, l1 = A.attn_mixed_ref(q, k, v, nv, Bq, Bk, True, mask=full)
    b1, m1 = A.attn_mixed_ref(q, k, v, nv, Bq, Bk, True, mode=A.MODE_ALL_FP16)
    assert np.array_equal(a0, b0) and np.array_equal(l0, m0)
    assert np.array_equal(a1, b1) and np.array_equal(l1, m1)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_zero_queries_give_mean_of_values(mode):
    """Q = 0: every score is 0, every P is exactly 1 (2**8 * 2**-8 in E4M3, or
    1 in fp16), so each row is the mean of its valid dequantised V rows."""
    N, D = 256, 64
    q, k, v, nv = _inputs(N=N, D=D, Hq=1, Hkv=1, seed=4)
    q[:] = 0
    rng = np.random.default_rng(0)
    mask = rng.integers(0, 16, size=(1, 1, 4, 1)).astype(np.uint32)
    out, lse = A.attn_mixed_ref(q, k, v, nv, 64, 64, True, mask=mask, mode=mode)
    ops = A.prepare_operands(q, k, v, nv)
    for r in range(0, N, 9):
        i = r // 64
        rows = []
        for t in range(r + 1):
            j = t // 64
            prom = mode == 2 or (mode == 0 and (int(mask[0, 0, i, 0]) >> j) & 1)
            rows.append(ops["v16"][0, 0, t] if prom else ops["v8"][0, 0, t])
        want = np.mean(rows, axis=0)
        assert np.allclose(out[0, 0, r], want, rtol=0, atol=1e-6)
        assert abs(lse[0, 0, r] - math.log(r + 1)) < 1e-5


def test_single_valid_key_returns_its_value():
    q, k, v, nv = _inputs(N=128, D=64, Hq=1, Hkv=1, seed=5, n_valid=1)
    for mode in (1, 2):
        out, _ = A.attn_mixed_ref(q, k, v, nv, 64, 64, False, mode=mode)
        ops = A.prepare_operands(q, k, v, nv)
        want = ops["v8"][0, 0, 0] if mode == 1 else ops["v16"][0, 0, 0]
        assert np.array_equal(out[0, 0, 0], want.astype(np.float32))
        assert np.all(out[0, 0, 1:] == 0)


def test_constant_values_are_reproduced_exactly():
    """l sums the same quantised P that weights V, so a constant V row comes back."""
    q, k, v, nv = _inputs(N=256, D=64, Hq=2, Hkv=1, seed=6, scale_q=3.0)
    u = np.random.default_rng(1).standard_normal(64).astype(np.float32)
    v[:] = F.f32_to_bf16_bits(np.broadcast_to(u, (1, 1, 256, 64)))
    rng = np.random.default_rng(2)
    mask = rng.integers(0, 16, size=(1, 2, 4, 1)).astype(np.uint32)
    out, _ = A.attn_mixed_ref(q, k, v, nv, 64, 64, True, mask=mask)
    ops = A.prepare_operands(q, k, v, nv)
    # MXFP8 and fp16 copies of a constant column agree here only if both are exact;
    # compare per row with the source tiles actually used
    for h in range(2):
        for r in range(256):
            i = r // 64
            used = set()
            for j in range(r // 64 + 1):
                used.add("v16" if (int(mask[0, h, i, 0]) >> j) & 1 else "v8")
            if len(used) == 1:
                want = ops[used.pop()][0, 0, 0]
                assert np.allclose(out[0, h, r], want, rtol=2e-7, atol=0)


def test_dominant_key_takes_all_weight():
    N, D = 128, 64
    q, k, v, nv = _inputs(N=N, D=D, Hq=1, Hkv=1, seed=7)
    qf = F.bf16_bits_to_f32(q)
    kf = F.bf16_bits_to_f32(k)
    kf[0, 0, 37] = qf[0, 0, 100] * 16   # key 37 dominates row 100 by a huge margin
    k = F.f32_to_bf16_bits(kf)
    for mode in (1, 2):
        out, _ = A.attn_mixed_ref(q, k, v, nv, 64, 64, False, mode=mode)
        ops = A.prepare_operands(q, k, v, nv)
        want = ops["v8" if mode == 1 else "v16"][0, 0, 37]
        assert np.array_equal(out[0, 0, 100], want.astype(np.float32))


def test_two_pass_equals_streaming_online_softmax():
    """A streaming implementation (one tile at a time, rescaling O and l by
    2**(m_old - m_new) when the reference grows) gives the two-pass result."""
    q, k, v, nv = _inputs(N=256, D=64, Hq=1, Hkv=1, seed=8, scale_q=2.0)
    Bq = Bk = 64
    rng = np.random.default_rng(3)
    mask = rng.integers(0, 16, size=(1, 1, 4, 1)).astype(np.uint32)
    out, lse = A.attn_mixed_ref(q, k, v, nv, Bq, Bk, True, mask=mask)
    ops = A.prepare_operands(q, k, v, nv)
    c = A.softmax_scale_log2(64)
    for i in range(4):
        rows = np.arange(i * Bq, (i + 1) * Bq)
        m = np.full(Bq, -np.inf)
        O = np.zeros((Bq, 64))
        L = np.zeros(Bq)
        for j in range(i + 1):
            cols = np.arange(j * Bk, (j + 1) * Bk)
            prom = (int(mask[0, 0, i, 0]) >> j) & 1
            if prom:
                s = (ops["q"][0, 0][rows] @ ops["k"][0, 0][cols].T).astype(np.float32)
            else:
                s = (ops["q_hat"][0, 0][rows] @ ops["k_hat"][0, 0][cols].T).astype(np.float32)
            s = np.where(cols[None, :] <= rows[:, None], s, np.float32(-np.inf))
            t = np.ceil((s.max(axis=1).astype(np.float64) * float(c)).astype(np.float32)).astype(np.float64)
            m_new = np.maximum(m, t)
            f = np.where(np.isfinite(m), np.exp2(m - m_new), 0.0)
            O *= f[:, None]
            L *= f
            m = m_new
            if prom:
                x = F.fma_f32(s, c, (-m).astype(np.float32)[:, None]).astype(np.float64)
                p = np.exp2(x).astype(np.float16).astype(np.float64)
                vv = ops["v16"][0, 0][cols]
            else:
                xq = F.p_exponent_grid(s, c, m.astype(np.float32)[:, None])
                p = F.e4m3_value(F.p_e4m3_code(xq)) / 256.0
                vv = ops["v8"][0, 0][cols]
            O += p @ vv
            L += p.sum(axis=1)
        assert np.allclose(out[0, 0, rows], O / L[:, None], rtol=1e-6, atol=1e-7)
        assert np.allclose(lse[0, 0, rows], math.log(2) * (m + np.log2(L)), rtol=1e-6)


def test_lowbit_error_is_fp4_sized_and_fp16_tiles_reduce_it():
    """Sanity on the method: low-bit attention differs from exact attention at
    FP4-like levels, and promoting every tile brings it to fp16 levels."""
    q, k, v, nv = _inputs(N=256, D=64, Hq=2, Hkv=1, seed=9)
    ex = A.attn_exact_ref(q, k, v, nv, True)
    lo, _ = A.attn_mixed_ref(q, k, v, nv, 64, 64, True, mode=A.MODE_ALL_LOWBIT)
    hi, _ = A.attn_mixed_ref(q, k, v, nv, 64, 64, True, mode=A.MODE_ALL_FP16)
    e_lo = np.sqrt(np.mean((lo - ex) ** 2))
    e_hi = np.sqrt(np.mean((hi - ex) ** 2))
    assert 1e-3 < e_lo < 0.3
    assert e_hi < e_lo / 20


def test_tiny_config_runs_end_to_end():
    cfg = mxq_inputs.make_prefill("tiny")
    mask, nfp, _ = S.select_blocks(cfg["q"], cfg["k"], cfg["n_valid"], cfg["Bq"], cfg["Bk"], cfg["causal"],
                                   cfg["topk"], cfg["ratio_num"], cfg["ratio_den"], cfg["sink_tiles"],
                                   cfg["local_tiles"])
    out, lse = A.attn_mixed_ref(cfg["q"], cfg["k"], cfg["v"], cfg["n_valid"], cfg["Bq"], cfg["Bk"],
                                cfg["causal"], mask=mask)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert int(nfp.sum()) == 8
