"""Pins for the oracle's quantised-KV decode attention (CPU only)."""

import math

import numpy as np
import pytest

import mxq_inputs
from oracle import decode as Dm
from oracle import formats as F


def _small(B=3, L=512, Hq=8, Hkv=2, D=64, seed=0, lens=None):
    cfg = dict(B=B, L=L, Hq=Hq, Hkv=Hkv, D=D, n_sink=16, n_recent=32, seed=seed)
    if lens is not None:
        cfg["seq_len"] = lens
    return mxq_inputs.make_decode(cfg, threads=2)


def _softmax_attn(q, K, V, sc):
    s = (q @ K.T) * sc
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def test_all_fp16_cache_equals_exact_attention():
    """n_sink + n_recent >= len: every token comes from the fp16 copies."""
    d = _small(lens=[40, 48, 10])
    cache = Dm.build_kv_cache_ref(d["k"], d["v"], d["seq_len"], 16, 32)
    out = Dm.attn_decode_ref(d["q"], cache, d["seq_len"], 16, 32)
    qf = F.bf16_bits_to_f32(d["q"]).astype(np.float64)
    kf = F.bf16_bits_to_f32(d["k"]).astype(np.float16).astype(np.float64)
    vf = F.bf16_bits_to_f32(d["v"]).astype(np.float16).astype(np.float64)
    for b in range(3):
        n = int(d["seq_len"][b])
        for h in range(8):
            want = _softmax_attn(qf[b, h], kf[b, h // 4, :n], vf[b, h // 4, :n], 1 / 8.0)
            assert np.allclose(out[b, h], want, rtol=1e-12, atol=1e-12)


def test_mixed_cache_token_by_token():
    """Independent per-token loop: fp16 for the first n_sink and last n_recent
    tokens, x_hat = fl32(code*s + z) elsewhere."""
    d = _small(lens=[512, 300, 49])
    cache = Dm.build_kv_cache_ref(d["k"], d["v"], d["seq_len"], 16, 32)
    out = Dm.attn_decode_ref(d["q"], cache, d["seq_len"], 16, 32)
    qf = F.bf16_bits_to_f32(d["q"]).astype(np.float64)
    kb = F.bf16_bits_to_f32(d["k"])
    vb = F.bf16_bits_to_f32(d["v"])
    for b in range(3):
        n = int(d["seq_len"][b])
        for hk in range(2):
            K = np.zeros((n, 64))
            V = np.zeros((n, 64))
            for t in range(n):
                if t < 16 or t >= n - 32:
                    K[t] = kb[b, hk, t].astype(np.float16)
                    V[t] = vb[b, hk, t].astype(np.float16)
                else:
                    for X, src in ((K, kb), (V, vb)):
                        row = src[b, hk, t]
                        for g in range(2):
                            grp = row[32 * g:32 * g + 32]
                            s = np.float16(np.float32(np.float32(grp.max() - grp.min())) / np.float32(15))
                            z = np.float16(grp.min())
                            for e in range(32):
                                if s == 0:
                                    code = 0
                                else:
                                    code = int(np.clip(np.rint(np.float32(np.float32(grp[e] - np.float32(z)) / np.float32(s))), 0, 15))
                                X[t, 32 * g + e] = np.float32(np.float32(code) * np.float32(s) + np.float32(z))
            for hq in range(hk * 4, hk * 4 + 4):
                want = _softmax_attn(qf[b, hq], K, V, 1 / 8.0)
                assert np.allclose(out[b, hq], want, rtol=1e-12, atol=1e-12)


def test_decode_quantisation_error_is_small():
    d = _small(B=2, L=1024, lens=[1024, 777])
    cache = Dm.build_kv_cache_ref(d["k"], d["v"], d["seq_len"], 16, 32)
    out = Dm.attn_decode_ref(d["q"], cache, d["seq_len"], 16, 32)
    qf = F.bf16_bits_to_f32(d["q"]).astype(np.float64)
    kf = F.bf16_bits_to_f32(d["k"]).astype(np.float64)
    vf = F.bf16_bits_to_f32(d["v"]).astype(np.float64)
    errs = []
    for b in range(2):
        n = int(d["seq_len"][b])
        for h in range(8):
            errs.append(np.abs(out[b, h] - _softmax_attn(qf[b, h], kf[b, h // 4, :n], vf[b, h // 4, :n], 1 / 8.0)).max())
    # 4-bit codes over a 32-wide group: small but visible error
    assert 1e-4 < max(errs) < 0.1


def test_recent_rows_hold_the_last_tokens():
    d = _small(lens=[100, 33, 512])
    cache = Dm.build_kv_cache_ref(d["k"], d["v"], d["seq_len"], 16, 32)
    kb = F.bf16_bits_to_f32(d["k"])
    for b, n in enumerate([100, 33, 512]):
        for r in range(32):
            t = n - 32 + r
            assert np.array_equal(cache["k_recent"][b, :, r], kb[b, :, t].astype(np.float16))


# ------------------------------------------------------------ cache append
def _fp16_exact(bits):
    """Zero every bf16 value below fp16's normal range, so that every value is
    exact in fp16 (bf16's 8-bit significand fits fp16's 11 bits)."""
    x = F.bf16_bits_to_f32(bits)
    x = np.where(np.abs(x) < 2.0 ** -14, np.float32(0), x)
    return F.f32_to_bf16_bits(x)


def _grow(d, lens0, steps, n_sink, n_recent):
    """Build the cache at lens0 from K/V with every later position zeroed (the
    future is unknown), then append `steps` tokens per sequence from K/V."""
    k, v = d["k"].copy(), d["v"].copy()
    lens0 = np.asarray(lens0, dtype=np.int32)
    for b in range(k.shape[0]):
        k[b, :, lens0[b]:] = 0
        v[b, :, lens0[b]:] = 0
    cache = Dm.build_kv_cache_ref(k, v, lens0, n_sink, n_recent)
    lens = lens0
    for _ in range(steps):
        kn = np.stack([d["k"][b, :, lens[b]] for b in range(len(lens))])
        vn = np.stack([d["v"][b, :, lens[b]] for b in range(len(lens))])
        cache, lens = Dm.append_kv_ref(cache, lens, kn, vn, n_sink, n_recent)
    return cache, lens


@pytest.mark.parametrize("n_sink,n_recent,lens0", [(16, 32, [100, 40, 5]), (0, 32, [64, 33, 1]),
                                                    (16, 0, [100, 17, 3])])
def test_append_equals_rebuild_on_fp16_exact_inputs(n_sink, n_recent, lens0):
    """Appending tokens one at a time gives the cache a build at the final
    length gives, wherever decode reads it, and the same decode output."""
    d = _small(B=3, L=256, Hq=8, Hkv=2, D=64, seed=7)
    d["k"], d["v"] = _fp16_exact(d["k"]), _fp16_exact(d["v"])
    steps = 60
    cache, lens = _grow(d, lens0, steps, n_sink, n_recent)
    assert np.array_equal(lens, np.asarray(lens0) + steps)
    ref = Dm.build_kv_cache_ref(d["k"], d["v"], lens, n_sink, n_recent)
    for which in ("k", "v"):
        assert np.array_equal(cache[which + "_sink"], ref[which + "_sink"])
        assert np.array_equal(cache[which + "_recent"], ref[which + "_recent"])
        for b in range(3):
            lo, hi = n_sink, int(lens[b]) - n_recent  # the INT4 region decode reads
            for name in ("_codes", "_scale", "_zero"):
                assert np.array_equal(cache[which + name][b, :, lo:hi], ref[which + name][b, :, lo:hi])
    out = Dm.attn_decode_ref(d["q"], cache, lens, n_sink, n_recent)
    want = Dm.attn_decode_ref(d["q"], ref, lens, n_sink, n_recent)
    assert np.array_equal(out, want)


def test_append_window_holds_the_last_tokens():
    d = _small(B=2, L=128, Hq=4, Hkv=1, D=64, seed=8)
    cache, lens = _grow(d, [50, 7], 9, 4, 8)
    kf = F.bf16_bits_to_f32(d["k"]).astype(np.float16)
    for b in range(2):
        n = int(lens[b])
        for r in range(8):
            t = n - 8 + r
            if t >= 0:
                assert np.array_equal(cache["k_recent"][b, 0, r], kf[b, 0, t])
    assert np.array_equal(cache["k_sink"][1, 0, :4], kf[1, 0, :4])


# ------------------------------------------------------- vertical lines in decode
def test_lines_over_the_whole_int4_region_give_fp16_attention():
    """With every token of the INT4 region listed as a line, decode reads
    every token in fp16: exact softmax attention over fp16 K and V."""
    d = _small(B=2, L=128, Hq=8, Hkv=2, D=64, seed=21, lens=[60, 44])
    lines = np.full((2, 2, 16), -1, dtype=np.int32)
    lines[0, :, :12] = np.arange(16, 28)          # INT4 region [16, 60 - 32) = 12 tokens
    lines[1, :] = [-1, 3, 16, 20, 5] + [-1] * 11  # [16, 12): empty; entries ignored
    cache = Dm.build_kv_cache_ref(d["k"], d["v"], d["seq_len"], 16, 32, lines=lines)
    out = Dm.attn_decode_ref(d["q"], cache, d["seq_len"], 16, 32)
    qf = F.bf16_bits_to_f32(d["q"]).astype(np.float64)
    kf = F.bf16_bits_to_f32(d["k"]).astype(np.float16).astype(np.float64)
    vf = F.bf16_bits_to_f32(d["v"]).astype(np.float16).astype(np.float64)
    for b in range(2):
        n = int(d["seq_len"][b])
        for h in range(8):
            want = _softmax_attn(qf[b, h], kf[b, h // 4, :n], vf[b, h // 4, :n], 1 / 8.0)
            assert np.allclose(out[b, h], want, rtol=1e-12, atol=1e-12)


def test_lines_outside_the_int4_region_change_nothing():
    d = _small(B=2, L=256, Hq=8, Hkv=2, D=64, seed=22, lens=[256, 100])
    plain = Dm.build_kv_cache_ref(d["k"], d["v"], d["seq_len"], 16, 32)
    lines = np.array([[[0, 15, 224, 255, 300, -1]] * 2, [[5, 68, 99, 99, 7, -3]] * 2], dtype=np.int32)
    withl = Dm.build_kv_cache_ref(d["k"], d["v"], d["seq_len"], 16, 32, lines=lines)
    assert np.array_equal(Dm.attn_decode_ref(d["q"], plain, d["seq_len"], 16, 32),
                          Dm.attn_decode_ref(d["q"], withl, d["seq_len"], 16, 32))
    assert [t for _, t in Dm.used_decode_lines(lines[1, 0], 100, 16, 32)] == []
    assert Dm.used_decode_lines(np.array([40, 40, 20, 50, -1]), 100, 16, 32) == [(0, 40), (3, 50)]


def test_a_heavy_token_kept_as_a_line_cuts_the_error():
    """A token whose key lines up with every query carries most of the
    attention; quantised to 4 bits it drags the output, kept in fp16 as a
    line it does not (HyQuant's point, in decode)."""
    d = _small(B=1, L=512, Hq=4, Hkv=1, D=64, seed=23, lens=[512])
    q = F.bf16_bits_to_f32(d["q"])
    k = F.bf16_bits_to_f32(d["k"]).copy()
    k[0, 0, 200] = 3.0 * q[0].mean(axis=0) / np.linalg.norm(q[0].mean(axis=0)) * 8.0
    k[0, 0, 200, :8] += 37.0  # an outlier the 4-bit group cannot hold finely
    kb = F.f32_to_bf16_bits(k)
    lines = np.array([[[200] + [-1] * 15]], dtype=np.int32)
    exact = np.stack([_softmax_attn(q[0, h].astype(np.float64), F.bf16_bits_to_f32(kb)[0, 0].astype(np.float64),
                                    F.bf16_bits_to_f32(d["v"])[0, 0].astype(np.float64), 1 / 8.0) for h in range(4)])
    e_plain = np.abs(Dm.attn_decode_ref(d["q"], Dm.build_kv_cache_ref(kb, d["v"], d["seq_len"], 16, 32),
                                        d["seq_len"], 16, 32)[0] - exact).max()
    e_line = np.abs(Dm.attn_decode_ref(d["q"], Dm.build_kv_cache_ref(kb, d["v"], d["seq_len"], 16, 32, lines=lines),
                                       d["seq_len"], 16, 32)[0] - exact).max()
    assert e_line < 0.5 * e_plain, (e_line, e_plain)


def test_prefill_lines_choose_the_decode_lines():
    """Reading R36: the vertical lines the prefill finds for a kv group
    (group-shared probe, R31) become the decode cache's fp16 line tokens.  A
    key that lines up with the direction the prompt's queries share (plus a
    head_dim outlier 4 bits cannot hold) is found by the prefill selection,
    and decoding a query of the same kind with it as a line cuts the error."""
    from oracle import select as S

    rng = np.random.default_rng(31)
    Hq, Hkv, L, D = 4, 1, 512, 64
    G = Hq // Hkv
    common = rng.standard_normal(D).astype(np.float32)
    qp = (rng.standard_normal((1, Hq, L, D)) * 0.5 + common).astype(np.float32)   # the prompt's queries
    k = rng.standard_normal((1, Hkv, L, D)).astype(np.float32)
    v = rng.standard_normal((1, Hkv, L, D)).astype(np.float32)
    k[0, 0, 300] = 6.0 * common / np.linalg.norm(common) * np.sqrt(D) / 4.0
    k[0, 0, 300, :8] += 37.0
    qb, kb, vb = F.f32_to_bf16_bits(qp), F.f32_to_bf16_bits(k), F.f32_to_bf16_bits(v)
    lines_hq, _ = S.select_lines(qb, kb, L, 64, 16, 1, group_shared=True)
    assert all(np.array_equal(lines_hq[0, h], lines_hq[0, 0]) for h in range(G))
    assert 300 in lines_hq[0, 0] and lines_hq[0, 0, 0] == 0  # the planted key, after the sink token
    lines = lines_hq[:, ::G]  # the kv group's list
    qd = F.f32_to_bf16_bits((rng.standard_normal((1, Hq, D)) * 0.5 + common).astype(np.float32))
    lens = np.array([L], dtype=np.int32)
    exact = np.stack([_softmax_attn(F.bf16_bits_to_f32(qd)[0, h].astype(np.float64),
                                    F.bf16_bits_to_f32(kb)[0, 0].astype(np.float64),
                                    F.bf16_bits_to_f32(vb)[0, 0].astype(np.float64), 1 / 8.0) for h in range(Hq)])
    e_plain = np.abs(Dm.attn_decode_ref(qd, Dm.build_kv_cache_ref(kb, vb, lens, 16, 32), lens, 16, 32)[0]
                     - exact).max()
    e_line = np.abs(Dm.attn_decode_ref(qd, Dm.build_kv_cache_ref(kb, vb, lens, 16, 32, lines=lines), lens, 16, 32)[0]
                    - exact).max()
    assert e_line < 0.5 * e_plain, (e_line, e_plain)
