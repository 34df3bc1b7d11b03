"""Pins for the oracle's quantised-KV decode attention (CPU only)."""

import math

import numpy as np

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
