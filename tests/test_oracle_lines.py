"""Pins for the oracle's vertical-line tokens: selection and attention (CPU only).

HyQuant (summary and abstract) keeps a few vertical-line tokens in high
precision.  These tests fix the oracle's selection against brute force on
inputs whose arithmetic is exact, special cases and planted lines, and its
attention against exact softmax attention and closed forms.
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import formats as F
from oracle import select as S


def _bits(x):
    return F.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _brute_lines(q, k, n_valid, Bq, n_lines, sink, heads):
    """Float64 brute force: probe = mean over valid query tiles (and heads) of
    the tile row means; rank remaining valid keys by (-score, index)."""
    n_vt = -(-n_valid // Bq)
    means = []
    for h in heads:
        for i in range(n_vt):
            rows = q[h, i * Bq:min((i + 1) * Bq, n_valid)].astype(np.float64)
            means.append(rows.mean(axis=0))
    probe = np.mean(means, axis=0)
    v = k[:n_valid].astype(np.float64) @ probe
    s = min(sink, n_valid, n_lines)
    cand = np.arange(s, n_valid)
    order = cand[np.lexsort((cand, -v[s:]))]
    chosen = sorted(list(range(s)) + list(order[:max(0, min(n_lines - s, cand.size))]))
    return chosen + [-1] * (n_lines - len(chosen))


@pytest.mark.parametrize("shared", [False, True])
def test_selection_matches_brute_force_on_exact_inputs(shared):
    # small integers: tile means with power-of-two row counts, the probe and
    # every score are exact in fp32, so fp32 and float64 rank identically
    # (ties included, which integer data produces plenty of)
    rng = np.random.default_rng(3)
    B, Hq, Hkv, N, D, Bq = 1, 4, 2, 128, 64, 32
    n_valid = 96
    q = rng.integers(-3, 4, size=(B, Hq, N, D)).astype(np.float32)
    k = rng.integers(-3, 4, size=(B, Hkv, N, D)).astype(np.float32)
    for n_lines, sink in ((8, 1), (16, 0), (5, 3)):
        lines, scores = S.select_lines(_bits(q), _bits(k), n_valid, Bq, n_lines, sink, group_shared=shared)
        G = Hq // Hkv
        for h in range(Hq):
            kv = h // G
            heads = list(range(kv * G, (kv + 1) * G)) if shared else [h]
            want = _brute_lines(q[0], k[0, kv], n_valid, Bq, n_lines, sink, heads)
            assert lines[0, h].tolist() == want, (h, n_lines, sink)
        assert np.all(np.isneginf(scores[..., n_valid:]))


def test_zero_keys_pick_the_lowest_indices():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 2, 128, 64)).astype(np.float32)
    k = np.zeros((1, 1, 128, 64), dtype=np.float32)
    lines, scores = S.select_lines(_bits(q), _bits(k), 120, 64, 6, 2)
    assert np.all(scores[..., :120] == 0)
    assert lines[0, 0].tolist() == [0, 1, 2, 3, 4, 5]


def test_short_sequences_pad_with_minus_one():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 128, 64)).astype(np.float32)
    k = rng.standard_normal((1, 1, 128, 64)).astype(np.float32)
    lines, _ = S.select_lines(_bits(q), _bits(k), 5, 64, 8, 1)
    assert lines[0, 0].tolist() == [0, 1, 2, 3, 4, -1, -1, -1]
    lines, _ = S.select_lines(_bits(q), _bits(k), 5, 64, 2, 4)   # sinks beyond the budget
    assert lines[0, 0].tolist() == [0, 1]


def test_planted_vertical_line_is_found():
    # every query shares a component along u; key 77 points along u, so all
    # queries attend to it: a vertical line in the attention map
    rng = np.random.default_rng(6)
    N, D = 256, 64
    u = rng.standard_normal(D).astype(np.float32)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((1, 4, N, D)).astype(np.float32) + 2.0 * u
    k = rng.standard_normal((1, 1, N, D)).astype(np.float32)
    k[0, 0, 77] = 6.0 * u
    for shared in (False, True):
        lines, scores = S.select_lines(_bits(q), _bits(k), 200, 64, 4, 1, group_shared=shared)
        for h in range(4):
            assert 0 in lines[0, h] and 77 in lines[0, h]
            assert int(np.argmax(scores[0, h])) == 77
    lines, _ = S.select_lines(_bits(q), _bits(k), 200, 64, 4, 1, group_shared=True)
    assert all(lines[0, h].tolist() == lines[0, 0].tolist() for h in range(4))


def test_used_lines_rule():
    assert S.used_lines(np.array([3, 3, 1, 200, 7, -1]), 100) == [3]
    assert S.used_lines(np.array([-1, 2, 5, 99, 100]), 100) == [2, 5, 99]
    assert S.used_lines(np.array([], dtype=np.int32), 10) == []


# ------------------------------------------------------------------ attention
def _inputs(N=128, D=64, Hq=2, Hkv=1, seed=0, n_valid=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Hq, N, D)).astype(np.float32)
    k = rng.standard_normal((1, Hkv, N, D)).astype(np.float32)
    v = rng.standard_normal((1, Hkv, N, D)).astype(np.float32)
    nv = N if n_valid is None else n_valid
    for t in (q, k, v):
        t[:, :, nv:] = 0
    return _bits(q), _bits(k), _bits(v), nv


@pytest.mark.parametrize("causal", [False, True])
def test_lines_covering_every_key_give_fp16_attention(causal):
    # all-low-bit mode, but every valid key is a line: the whole row runs in
    # FP16 and must match exact softmax attention to FP16 accuracy; without the
    # lines the same call carries the low-bit error
    q, k, v, nv = _inputs(N=128, D=64, Hq=2, seed=11, n_valid=16)
    lines = np.tile(np.arange(16, dtype=np.int32), (1, 2, 1))
    exact = A.attn_exact_ref(q, k, v, nv, causal)
    out, lse = A.attn_mixed_ref(q, k, v, nv, 64, 64, causal, mode=A.MODE_ALL_LOWBIT, lines=lines)
    low, _ = A.attn_mixed_ref(q, k, v, nv, 64, 64, causal, mode=A.MODE_ALL_LOWBIT)
    assert np.max(np.abs(out - exact)) < 3e-3
    assert np.max(np.abs(low - exact)) > 2e-2
    assert np.all(out[:, :, nv:] == 0) and np.all(np.isneginf(lse[:, :, nv:]))


def test_lines_in_fp16_mode_are_counted_once():
    q, k, v, nv = _inputs(N=256, D=64, Hq=2, seed=12, n_valid=230)
    lines = np.array([[[0, 5, 64, 65, 131, 229, -1, -1], [3, 200, 201, -1, -1, -1, -1, -1]]], dtype=np.int32)
    exact = A.attn_exact_ref(q, k, v, nv, True)
    out, _ = A.attn_mixed_ref(q, k, v, nv, 64, 64, True, mode=A.MODE_ALL_FP16, lines=lines)
    assert np.max(np.abs(out - exact)) < 3e-3


def test_empty_and_ignored_lines_change_nothing():
    q, k, v, nv = _inputs(N=256, D=64, Hq=2, seed=13, n_valid=250)
    mask, _, _ = S.select_blocks(q, k, nv, 64, 64, True, 1, 0, 1, 1, 1)
    base, base_lse = A.attn_mixed_ref(q, k, v, nv, 64, 64, True, mask=mask)
    empty = np.full((1, 2, 4), -1, dtype=np.int32)
    out, lse = A.attn_mixed_ref(q, k, v, nv, 64, 64, True, mask=mask, lines=empty)
    assert np.array_equal(out, base) and np.array_equal(lse, base_lse)
    messy = np.array([[[40, 40, 7, 300], [40, -1, -1, -1]]], dtype=np.int32)
    clean = np.array([[[40, -1, -1, -1], [40, -1, -1, -1]]], dtype=np.int32)
    lowbit = dict(mode=A.MODE_ALL_LOWBIT)
    a, _ = A.attn_mixed_ref(q, k, v, nv, 64, 64, True, lines=messy, **lowbit)
    b, _ = A.attn_mixed_ref(q, k, v, nv, 64, 64, True, lines=clean, **lowbit)
    c, _ = A.attn_mixed_ref(q, k, v, nv, 64, 64, True, **lowbit)
    assert np.array_equal(a, b)
    assert not np.array_equal(b[:, :, 40:nv], c[:, :, 40:nv])  # the line is seen from row 40 on
    assert np.array_equal(b[:, :, :40], c[:, :, :40])


def test_zero_queries_average_the_right_value_rows():
    # Q = 0: every score is 0, so every P is exactly 1 (E4M3 and fp16 alike)
    # and each row is the plain mean of its keys' values, lines taken from the
    # fp16 copy of V and the rest from the MXFP8 copy
    N, D, nv = 128, 64, 120
    _, k, v, _ = _inputs(N=N, D=D, Hq=1, seed=14, n_valid=nv)
    q = np.zeros((1, 1, N, D), dtype=np.uint16)
    lines = np.array([[[0, 9, 70, 119]]], dtype=np.int32)
    out, _ = A.attn_mixed_ref(q, k, v, nv, 64, 64, False, mode=A.MODE_ALL_LOWBIT, lines=lines)
    vf = F.bf16_bits_to_f32(v)[0, 0]
    vc, vs = F.quantize_mxfp8_keys(vf)
    v8 = F.dequantize_mxfp8_keys(vc, vs)
    rowsum = v8[:nv].sum(axis=0)
    for j in lines[0, 0]:
        rowsum += np.float64(np.float16(vf[j])) - v8[j]
    want = rowsum / nv
    assert np.max(np.abs(out[0, 0, :nv] - want[None, :])) < 1e-6
    # causal: row r averages keys 0..r
    outc, _ = A.attn_mixed_ref(q, k, v, nv, 64, 64, True, mode=A.MODE_ALL_LOWBIT, lines=lines)
    for r in (0, 8, 9, 69, 70, 100, 119):
        vals = [np.float64(np.float16(vf[j])) if j in lines[0, 0] else v8[j] for j in range(r + 1)]
        assert np.max(np.abs(outc[0, 0, r] - np.mean(vals, axis=0))) < 1e-6, r


def test_constant_values_stay_constant_with_lines():
    q, k, _, nv = _inputs(N=256, D=64, Hq=2, seed=15, n_valid=256)
    v = _bits(np.full((1, 1, 256, 64), 0.75, dtype=np.float32))
    lines = np.array([[[0, 100, 255, -1], [17, -1, -1, -1]]], dtype=np.int32)
    mask, _, _ = S.select_blocks(q, k, nv, 64, 64, True, 1, 0, 1, 1, 1)
    out, _ = A.attn_mixed_ref(q, k, v, nv, 64, 64, True, mask=mask, lines=lines)
    assert np.max(np.abs(out - 0.75)) < 1e-6
