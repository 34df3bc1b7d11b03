"""Mixed-precision block-scaled attention, tile-ordered two-pass (test infrastructure).

ThriftAttention (abstract): the selected query-key blocks are computed in FP16
and the remaining blocks in FP4, and both paths are merged through online
softmax into a single output.  The "Attention Quantization" topic page
(overview) notes that softmax amplifies small quantisation errors, so the
softmax itself stays in full precision and only the matmul operands are
quantised.  Readings R7 and R12-R18 fix the open points:

* low-bit tiles: S = fl32(exact q_hat . k_hat) over MXFP4-dequantised Q and K;
  FP16 tiles: S = fl32(exact q . k) over the bf16 inputs (bf16 -> fp16 is exact);
* running reference m_j = max over tiles j' <= j (ascending) of
  ceil(fl32(rowmax(S_j') * c)), an integer in log2 units, c = fl32(scale*log2 e);
* low-bit tiles: P = E4M3(2**x_q) * 2**-8 with x_q the 2**-11-grid exponent of
  ``formats.p_exponent_grid``; V is the MXFP8 (E4M3, 32 keys per scale) copy;
* FP16 tiles: P = fp16(2**x), x = fl32(S*c - m) (one rounding); V = fp16(V);
* row sum l accumulates the same quantised P that multiplies V, so each output
  row is a convex combination of its V rows;
* O and l are rescaled by 2**(m_old - m_new) (exact) whenever m grows;
  out = O / l, lse = ln2 * (m + log2 l);
* vertical-line tokens (HyQuant, summary and abstract; readings R29, R30): the
  keys of a line list form one more FP16 tile that comes first in the
  reference order, and they are left out of every key tile, so each key is
  counted once, at FP16 if it is a line.

"Two-pass" here means: pass 1 computes every tile's running reference m_j,
pass 2 computes every tile's P against its own m_j and sums the rescaled
contributions.  In exact arithmetic this is the same number the one-pass
online algorithm produces, because every rescale factor is a power of two.
"""

from __future__ import annotations

import math

import numpy as np

from .formats import (
    bf16_bits_to_f32,
    hadamard_rotate,
    quantize_mxfp4,
    dequantize_mxfp4,
    quantize_mxfp8_keys,
    dequantize_mxfp8_keys,
    e4m3_value,
    fma_f32,
    p_exponent_grid,
    p_e4m3_code,
)
from .select import tile_sets, mask_to_sets, used_lines

LOG2E = 1.4426950408889634  # log2(e) in double precision

MODE_MIXED, MODE_ALL_LOWBIT, MODE_ALL_FP16 = 0, 1, 2


def softmax_scale_log2(D: int, softmax_scale=None) -> np.float32:
    """c = fl32(scale * log2 e), the product taken in double (R13).  A scale
    <= 0 or None means 1/sqrt(D)."""
    if softmax_scale is None or float(softmax_scale) <= 0.0:
        sc = 1.0 / math.sqrt(float(D))
    else:
        sc = float(np.float32(softmax_scale))
    return np.float32(sc * LOG2E)


def _zero_padding_rows(x: np.ndarray, n_valid: int) -> np.ndarray:
    x = x.copy()
    x[..., n_valid:, :] = 0.0
    return x


def prepare_operands(q_bits, k_bits, v_bits, n_valid, rotate=False):
    """Every operand form the attention needs, as float64 arrays (exact).
    With ``rotate`` the MXFP4 operands are those of Q and K rotated by the
    Walsh-Hadamard matrix (R34); FP16 tiles keep the unrotated bf16 values
    (the rotation is orthonormal, so both estimate the same QK^T)."""
    qf = _zero_padding_rows(bf16_bits_to_f32(q_bits), n_valid)
    kf = _zero_padding_rows(bf16_bits_to_f32(k_bits), n_valid)
    vf = _zero_padding_rows(bf16_bits_to_f32(v_bits), n_valid)
    qc, qs = quantize_mxfp4(hadamard_rotate(qf) if rotate else qf)
    kc, ks = quantize_mxfp4(hadamard_rotate(kf) if rotate else kf)
    vc, vs = quantize_mxfp8_keys(vf)
    return dict(
        q=qf.astype(np.float64), k=kf.astype(np.float64),
        q_hat=dequantize_mxfp4(qc, qs), k_hat=dequantize_mxfp4(kc, ks),
        q_exp=qs.astype(np.int64) - 127, k_exp=ks.astype(np.int64) - 127,
        v8=dequantize_mxfp8_keys(vc, vs),
        v16=vf.astype(np.float16).astype(np.float64),
    )


def _exact_lowbit_scores(q_hat, k_hat, q_exp, k_exp):
    """fl32 of the exact dot products of MXFP4-dequantised rows.

    Every product is exact in float64 and is a multiple of 2**(Eq+Ek-2) with
    |block sum| < 2**13; when the per-pair spread of Eq+Ek over the D/32
    blocks is at most 38 bits, every float64 partial sum is exact whatever the
    summation order, so the one rounding to fp32 is the exact rounding.  A
    block whose q or k elements are all zero contributes exactly 0 whatever its
    exponent, so it is left out of the spread."""
    nb = q_exp.shape[-1]
    nzq = np.any(q_hat.reshape(q_hat.shape[0], nb, -1) != 0, axis=-1)
    nzk = np.any(k_hat.reshape(k_hat.shape[0], nb, -1) != 0, axis=-1)

    def own_spread(e, nz):  # spread of one side's exponents over its nonzero blocks
        hi = np.where(nz, e, np.iinfo(np.int64).min).max(axis=-1)
        lo = np.where(nz, e, np.iinfo(np.int64).max).min(axis=-1)
        return np.where(nz.any(axis=-1), hi - lo, 0)

    # a pair's spread is at most the sum of both sides' own spreads; only when
    # that bound is over 38 is the pairwise spread computed
    if q_exp.size and k_exp.size and int(own_spread(q_exp, nzq).max()) + int(own_spread(k_exp, nzk).max()) > 38:
        live = nzq[:, None, :] & nzk[None, :, :]
        e = q_exp[:, None, :] + k_exp[None, :, :]
        hi = np.where(live, e, np.iinfo(np.int64).min).max(axis=-1)
        lo = np.where(live, e, np.iinfo(np.int64).max).min(axis=-1)
        spread = np.where(live.any(axis=-1), hi - lo, 0)
        if int(spread.max()) > 38:
            raise ValueError("block-scale spread too large for the exact float64 sum")
    return (q_hat @ k_hat.T).astype(np.float32)


def attn_mixed_ref(q_bits, k_bits, v_bits, n_valid, Bq, Bk, causal, mask=None,
                   mode=MODE_MIXED, softmax_scale=None, heads=None, qtiles=None,
                   ops=None, lines=None, rotate=False):
    """Reference mixed-precision attention.

    q_bits [B,Hq,N,D], k_bits/v_bits [B,Hkv,N,D] (bf16 bit patterns); mask u32
    [B,Hq,n_qt,ceil(n_kt/32)] (MIXED mode); lines int32 [B,Hq,n_lines] or None
    (vertical-line keys, in every mode).  ``heads`` (list of (b, hq)) and
    ``qtiles`` (list of query-tile indices) restrict the work to a sample; rows
    not computed are NaN.  Returns (out f32 [B,Hq,N,D], lse f32 [B,Hq,N]).
    """
    B, Hq, N, D = q_bits.shape
    Hkv = k_bits.shape[1]
    G = Hq // Hkv
    n_qt, n_kt = N // Bq, N // Bk
    c = softmax_scale_log2(D, softmax_scale)
    if ops is None:
        ops = prepare_operands(q_bits, k_bits, v_bits, n_valid, rotate=rotate)
    out = np.full((B, Hq, N, D), np.nan, dtype=np.float32)
    lse = np.full((B, Hq, N), np.nan, dtype=np.float32)
    sets = tile_sets(n_valid, N, Bq, Bk, causal, 0, 0)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    if qtiles is None:
        qtiles = list(range(n_qt))
    keys = np.arange(N)
    for (b, h) in heads:
        kv = h // G
        for i in qtiles:
            qs = i * Bq
            rows = np.arange(qs, qs + Bq)
            if qs >= n_valid:
                out[b, h, rows] = 0.0
                lse[b, h, rows] = -np.inf
                continue
            valid_tiles = sets[i][0]
            if mode == MODE_ALL_FP16:
                promoted = set(valid_tiles)
            elif mode == MODE_ALL_LOWBIT:
                promoted = set()
            else:
                promoted = set(mask_to_sets(mask[b, h, i], n_kt))
            nk = (max(valid_tiles) + 1) * Bk
            s_low = _exact_lowbit_scores(ops["q_hat"][b, h, rows], ops["k_hat"][b, kv, :nk],
                                         ops["q_exp"][b, h, rows], ops["k_exp"][b, kv, :nk])
            s_hi = (ops["q"][b, h, rows] @ ops["k"][b, kv, :nk].T).astype(np.float32)
            ok = keys[None, :nk] < n_valid
            if causal:
                ok = ok & (keys[None, :nk] <= rows[:, None])
            ok = ok & (rows[:, None] < n_valid)
            lk = used_lines(lines[b, h], n_valid) if lines is not None else []
            lk = np.asarray(lk, dtype=np.int64)
            ok_line = (rows[:, None] < n_valid) & np.ones((Bq, lk.size), dtype=bool)
            if causal:
                ok_line = ok_line & (lk[None, :] <= rows[:, None])
            ok[:, lk[lk < nk]] = False  # a line key leaves its tile
            # ---- pass 1: running integer reference per tile (ascending j),
            # the line tile first
            m_run = np.full(Bq, -np.inf, dtype=np.float32)
            m_tile = {}
            s_tile = {}
            if lk.size:
                s = (ops["q"][b, h, rows] @ ops["k"][b, kv, lk].T).astype(np.float32)
                s = np.where(ok_line, s, np.float32(-np.inf)).astype(np.float32)
                with np.errstate(invalid="ignore", over="ignore"):
                    t = np.ceil((s.max(axis=1).astype(np.float64) * np.float64(c)).astype(np.float32))
                m_run = np.maximum(m_run, t).astype(np.float32)
                m_tile["lines"] = m_run.copy()
                s_tile["lines"] = s
            for j in valid_tiles:
                cols = slice(j * Bk, (j + 1) * Bk)
                s = np.where(j in promoted, s_hi[:, cols], s_low[:, cols])
                s = np.where(ok[:, cols], s, np.float32(-np.inf)).astype(np.float32)
                rmax = s.max(axis=1)
                with np.errstate(invalid="ignore", over="ignore"):
                    t = np.ceil((rmax.astype(np.float64) * np.float64(c)).astype(np.float32))
                m_run = np.maximum(m_run, t).astype(np.float32)
                m_tile[j] = m_run.copy()
                s_tile[j] = s
            m_fin = m_run
            # ---- pass 2: P per tile against its own reference, rescaled sums
            O = np.zeros((Bq, D))
            L = np.zeros(Bq)
            for j in list(m_tile):  # the line tile (if any), then key tiles ascending
                s = s_tile[j]
                m = m_tile[j]
                live = np.isfinite(m)
                m_safe = np.where(live, m, np.float32(0))
                if j == "lines" or j in promoted:
                    x = fma_f32(s, c, -m_safe[:, None])
                    with np.errstate(over="ignore"):
                        p = np.exp2(x.astype(np.float64)).astype(np.float16).astype(np.float64)
                    vv = ops["v16"][b, kv, lk] if j == "lines" else ops["v16"][b, kv, j * Bk:(j + 1) * Bk]
                else:
                    xq = p_exponent_grid(s, c, m_safe[:, None])
                    p = e4m3_value(p_e4m3_code(xq)) * 2.0 ** -8
                    vv = ops["v8"][b, kv, j * Bk:(j + 1) * Bk]
                p = np.where(live[:, None], p, 0.0)
                f = np.where(live, np.exp2((m_safe - np.where(np.isfinite(m_fin), m_fin, 0)).astype(np.float64)), 0.0)
                O += f[:, None] * (p @ vv)
                L += f * p.sum(axis=1)
            with np.errstate(invalid="ignore", divide="ignore"):
                o = O / L[:, None]
                ls = math.log(2.0) * (m_fin.astype(np.float64) + np.log2(L))
            rv = rows < n_valid
            out[b, h, rows] = np.where(rv[:, None], o, 0.0).astype(np.float32)
            lse[b, h, rows] = np.where(rv, ls, -np.inf).astype(np.float32)
    return out, lse


def attn_exact_ref(q_bits, k_bits, v_bits, n_valid, causal, softmax_scale=None, heads=None,
                   rows=None):
    """Unquantised softmax attention in float64 over the bf16 inputs (used to
    pin the FP16 path and as the quality reference)."""
    B, Hq, N, D = q_bits.shape
    Hkv = k_bits.shape[1]
    G = Hq // Hkv
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    k = bf16_bits_to_f32(k_bits).astype(np.float64)
    v = bf16_bits_to_f32(v_bits).astype(np.float64)
    if softmax_scale is None or float(softmax_scale) <= 0:
        sc = 1.0 / math.sqrt(D)
    else:
        sc = float(np.float32(softmax_scale))
    out = np.full((B, Hq, N, D), np.nan)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    if rows is None:
        rows = np.arange(N)
    rows = np.asarray(rows)
    for (b, h) in heads:
        s = (q[b, h, rows] @ k[b, h // G, :n_valid].T) * sc
        ok = np.ones_like(s, dtype=bool)
        if causal:
            ok = np.arange(n_valid)[None, :] <= rows[:, None]
        s = np.where(ok, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        o = (p @ v[b, h // G, :n_valid]) / p.sum(axis=1, keepdims=True)
        out[b, h, rows] = np.where((rows < n_valid)[:, None], o, 0.0)
    return out
