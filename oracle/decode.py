"""Decode attention over a 4-bit group-scaled KV cache (test infrastructure).

HyQuant (summary, abstract): in decode the same hybrid principle is applied to
KV-cache compression, and KV dequantisation is fused with the attention
computation.  The NOVA-KV abstract (third page) states why this path is
bandwidth-bound: each decode step reads the whole KV cache, and loading it
takes longer than computing attention over it.  Readings (R19, R20,
R23): keys/values are stored as asymmetric 4-bit codes with an fp16 scale and
zero per 32 elements of head_dim; the first ``n_sink`` tokens and the last
``n_recent`` tokens of each sequence stay in fp16 (the high-precision
vertical-line and local-window tokens); query heads use kv head hq // G.

The reference is plain softmax attention in float64 over the dequantised
cache; P is not quantised on this path.
"""

from __future__ import annotations

import math

import numpy as np

from .formats import bf16_bits_to_f32, quantize_int4_g32, dequantize_int4_g32


def build_kv_cache_ref(k_bits, v_bits, seq_len, n_sink, n_recent, lines=None):
    """Quantise a bf16 cache [B,Hkv,L,D].

    Returns dict with k_codes/v_codes uint8 [B,Hkv,L,D] (unpacked), k_scale,
    k_zero, v_scale, v_zero float16 [B,Hkv,L,D/32], k_sink/v_sink float16
    [B,Hkv,n_sink,D] (tokens 0..n_sink-1) and k_recent/v_recent float16
    [B,Hkv,n_recent,D] (row r holds token len_b - n_recent + r; rows whose
    token would be negative are zero).  With ``lines`` (int32 [B,Hkv,n]), also
    lines and k_lines/v_lines float16 [B,Hkv,n,D]: the fp16 rows of the listed
    tokens (zero rows for entries outside [0, L))."""
    k = bf16_bits_to_f32(k_bits)
    v = bf16_bits_to_f32(v_bits)
    B, Hkv, L, D = k.shape
    kc, ksc, kz = quantize_int4_g32(k)
    vc, vsc, vz = quantize_int4_g32(v)
    k_sink = k[:, :, :n_sink].astype(np.float16)
    v_sink = v[:, :, :n_sink].astype(np.float16)
    k_rec = np.zeros((B, Hkv, n_recent, D), dtype=np.float16)
    v_rec = np.zeros((B, Hkv, n_recent, D), dtype=np.float16)
    for b in range(B):
        n = int(seq_len[b])
        for r in range(n_recent):
            t = n - n_recent + r
            if 0 <= t < L:
                k_rec[b, :, r] = k[b, :, t].astype(np.float16)
                v_rec[b, :, r] = v[b, :, t].astype(np.float16)
    out = dict(k_codes=kc, k_scale=ksc, k_zero=kz, v_codes=vc, v_scale=vsc, v_zero=vz,
               k_sink=k_sink, v_sink=v_sink, k_recent=k_rec, v_recent=v_rec)
    if lines is not None:
        lines = np.asarray(lines, dtype=np.int32)
        kl = np.zeros(lines.shape + (D,), dtype=np.float16)
        vl = np.zeros(lines.shape + (D,), dtype=np.float16)
        for b in range(B):
            for h in range(Hkv):
                for e, t in enumerate(lines[b, h]):
                    if 0 <= t < L:
                        kl[b, h, e] = k[b, h, t].astype(np.float16)
                        vl[b, h, e] = v[b, h, t].astype(np.float16)
        out.update(lines=lines.copy(), k_lines=kl, v_lines=vl)
    return out


def used_decode_lines(row, n, n_sink, n_recent):
    """(entry, token) pairs of one line list that decode reads from the fp16
    line rows (reading R33): an entry counts when its token lies in the INT4
    region [n_sink, n - n_recent) and exceeds every earlier entry of the row;
    tokens in the sink or the window are fp16 already."""
    out, top = [], -1
    for e, t in enumerate(int(x) for x in row):
        if n_sink <= t < n - n_recent and t > top:
            out.append((e, t))
        top = max(top, t)
    return out


def cache_rows(cache, b, h, n, n_sink, n_recent, which):
    """Dequantised key (which='k') or value rows 0..n-1 of sequence b, kv head h,
    float64 [n, D]: fp16 for t < n_sink or t >= n - n_recent, and for the
    cache's vertical-line tokens if it has them; INT4 otherwise."""
    codes = cache[which + "_codes"][b, h, :n]
    rows = dequantize_int4_g32(codes, cache[which + "_scale"][b, h, :n],
                               cache[which + "_zero"][b, h, :n]).astype(np.float64)
    t = np.arange(n)
    sink = t < n_sink
    rows[sink] = cache[which + "_sink"][b, h, t[sink]].astype(np.float64)
    rec = (t >= n - n_recent) & ~sink
    r_idx = t[rec] - (n - n_recent)
    rows[rec] = cache[which + "_recent"][b, h, r_idx].astype(np.float64)
    if "lines" in cache:  # vertical-line tokens kept in fp16 (R33)
        for e, tok in used_decode_lines(cache["lines"][b, h], n, n_sink, n_recent):
            rows[tok] = cache[which + "_lines"][b, h, e].astype(np.float64)
    return rows


def attn_decode_ref(q_bits, cache, seq_len, n_sink, n_recent, softmax_scale=None, seqs=None):
    """out float64 [B,Hq,D]: softmax(q . k_hat * scale) @ v_hat per query head.
    ``seqs`` restricts the work to some sequences (others are NaN)."""
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    B, Hq, D = q.shape
    Hkv = cache["k_codes"].shape[1]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if (softmax_scale is None or softmax_scale <= 0) else float(np.float32(softmax_scale))
    out = np.full((B, Hq, D), np.nan)
    for b in (range(B) if seqs is None else seqs):
        n = int(seq_len[b])
        for h in range(Hkv):
            kk = cache_rows(cache, b, h, n, n_sink, n_recent, "k")
            vv = cache_rows(cache, b, h, n, n_sink, n_recent, "v")
            qq = q[b, h * G:(h + 1) * G]
            s = (qq @ kk.T) * sc
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[b, h * G:(h + 1) * G] = (p @ vv) / p.sum(axis=1, keepdims=True)
    return out


def append_kv_ref(cache, seq_len, k_new_bits, v_new_bits, n_sink, n_recent):
    """One decode step's cache update (reading R32), on copies of the inputs.

    HyQuant (summary, abstract) applies its hybrid principle to KV-cache
    compression in decode: the recent window stays in full precision and the
    rest is low-bit.  As the sequence grows, token t = seq_len[b] (k_new,
    v_new bf16 [B,Hkv,D]) enters the fp16 window as its last row and the
    window's first row, token t - n_recent, leaves it: unless it is a sink
    token (t - n_recent < n_sink) it is quantised to INT4 (R19) from its fp16
    copy at position t - n_recent.  With n_recent = 0 the new token itself is
    quantised, from its fp16 rounding.  A token t < n_sink is also written to
    the sink copy.  seq_len[b] grows by one.  Returns (cache, seq_len)."""
    c = {name: arr.copy() for name, arr in cache.items()}
    lens = np.asarray(seq_len, dtype=np.int32).copy()
    kn = bf16_bits_to_f32(k_new_bits).astype(np.float16)
    vn = bf16_bits_to_f32(v_new_bits).astype(np.float16)
    B = kn.shape[0]
    for b in range(B):
        t = int(lens[b])
        t_old = t - n_recent
        for which, new in (("k", kn), ("v", vn)):
            rec = c[which + "_recent"]
            leaving = rec[b, :, 0] if n_recent > 0 else new[b]
            if t_old >= n_sink and t_old >= 0:
                codes, sc, z = quantize_int4_g32(leaving.astype(np.float32))
                c[which + "_codes"][b, :, t_old] = codes
                c[which + "_scale"][b, :, t_old] = sc
                c[which + "_zero"][b, :, t_old] = z
            if n_recent > 0:
                rec[b, :, :-1] = rec[b, :, 1:].copy()
                rec[b, :, -1] = new[b]
            if t < n_sink:
                c[which + "_sink"][b, :, t] = new[b]
        lens[b] = t + 1
    return c, lens
