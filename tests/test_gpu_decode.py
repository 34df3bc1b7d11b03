"""GPU parity: attn_quantkv_decode against the oracle (max-abs <= 5e-3)."""

import numpy as np
import pytest

from gpu_helpers import bf16_dev, gpu_or_skip
import mxq_inputs
from oracle import decode as Dm

pytestmark = pytest.mark.gpu

TOL = 5e-3
# The PV contraction takes the weights p*s in fp16 (relative rounding at most
# 2^-11 each); over thousands of tokens these roundings average out and leave
# errors near 1e-4 against the float64 oracle.  This tighter bound catches a
# structural mistake (a wrong token, group or scale) long before TOL would.
TIGHT = 1e-3


def _run(mxq, d, n_sink, n_recent, num_splits=0):
    import torch

    k, v, q = bf16_dev(d["k"]), bf16_dev(d["v"]), bf16_dev(d["q"])
    lens = d["seq_len"]
    B = len(lens)
    if n_recent > 0:
        krec = torch.stack([k[b, :, lens[b] - n_recent:lens[b]] for b in range(B)])
        vrec = torch.stack([v[b, :, lens[b] - n_recent:lens[b]] for b in range(B)])
    else:
        krec = vrec = None
    cache = mxq.build_quant_kv_cache(k, v, torch.from_numpy(lens).to("cuda:0"), n_sink, n_recent, krec, vrec)
    out = mxq.attn_quantkv_decode(q, cache, d["Hkv"], int(lens.max()), num_splits=num_splits)
    return out.cpu().numpy(), cache


@pytest.mark.parametrize("num_splits", [0, 1, 3, 16])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_small_ragged(num_splits, G):
    mxq = gpu_or_skip()
    Hkv = 2
    lens = [1000, 257, 193, 64 + 128 + 5]
    d = mxq_inputs.make_decode(dict(B=4, L=1024, Hq=Hkv * G, Hkv=Hkv, D=128, n_sink=64, n_recent=128, seed=9,
                                    seq_len=lens), threads=4)
    out, _ = _run(mxq, d, 64, 128, num_splits)
    ref = Dm.attn_decode_ref(d["q"], Dm.build_kv_cache_ref(d["k"], d["v"], d["seq_len"], 64, 128),
                             d["seq_len"], 64, 128)
    err = np.abs(out - ref).max()
    assert err <= TOL, err
    assert err <= TIGHT, f"rounding-level error expected: {err}"


@pytest.mark.parametrize("n_sink, lens", [(0, [1, 2, 31, 33, 1024]), (64, [1, 10, 64, 65, 1024])])
def test_degenerate_lengths(n_sink, lens):
    """A single cached token, lengths below one 32-token block and below the
    sink, exactly the sink, and the full cache: every split but the ones that
    hold tokens is empty for the short sequences."""
    mxq = gpu_or_skip()
    d = mxq_inputs.make_decode(dict(B=len(lens), L=1024, Hq=8, Hkv=2, D=128, n_sink=n_sink, n_recent=0, seed=13,
                                    seq_len=lens), threads=4)
    for num_splits in (0, 16):
        out, _ = _run(mxq, d, n_sink, 0, num_splits)
        ref = Dm.attn_decode_ref(d["q"], Dm.build_kv_cache_ref(d["k"], d["v"], d["seq_len"], n_sink, 0),
                                 d["seq_len"], n_sink, 0)
        err = np.abs(out - ref).max()
        assert np.isfinite(out).all()
        # with a handful of tokens the fp16 roundings of p*s do not average
        # out: one token's relative 2^-11 on a value near 4 is about 2e-3, so
        # only the parity bar applies here, not TIGHT
        assert err <= TOL, (num_splits, err)


def test_all_fp16_and_no_fp16_regions():
    mxq = gpu_or_skip()
    d = mxq_inputs.make_decode(dict(B=2, L=256, Hq=8, Hkv=2, D=128, n_sink=64, n_recent=128, seed=3,
                                    seq_len=[150, 192]), threads=2)
    out, _ = _run(mxq, d, 64, 128)      # every token in the fp16 copies
    ref = Dm.attn_decode_ref(d["q"], Dm.build_kv_cache_ref(d["k"], d["v"], d["seq_len"], 64, 128), d["seq_len"], 64, 128)
    assert np.abs(out - ref).max() <= 1e-4  # fp16 tokens: plain fp32 arithmetic
    out0, _ = _run(mxq, d, 0, 0)         # every token INT4
    ref0 = Dm.attn_decode_ref(d["q"], Dm.build_kv_cache_ref(d["k"], d["v"], d["seq_len"], 0, 0), d["seq_len"], 0, 0)
    assert np.abs(out0 - ref0).max() <= TIGHT


def test_cache_build_matches_oracle():
    mxq = gpu_or_skip()
    from gpu_helpers import u8, u16
    from oracle.formats import pack_nibbles

    d = mxq_inputs.make_decode(dict(B=2, L=512, Hq=8, Hkv=2, D=128, n_sink=64, n_recent=128, seed=5,
                                    seq_len=[512, 400]), threads=2)
    _, cache = _run(mxq, d, 64, 128)
    ref = Dm.build_kv_cache_ref(d["k"], d["v"], d["seq_len"], 64, 128)
    assert np.array_equal(u8(cache.k_codes), pack_nibbles(ref["k_codes"]))
    assert np.array_equal(u8(cache.v_codes), pack_nibbles(ref["v_codes"]))
    assert np.array_equal(u16(cache.k_scale), ref["k_scale"].view(np.uint16))
    assert np.array_equal(u16(cache.v_zero), ref["v_zero"].view(np.uint16))
    assert np.array_equal(u16(cache.k_sink), ref["k_sink"].view(np.uint16))
    assert np.array_equal(u16(cache.v_recent), ref["v_recent"].view(np.uint16))


def test_decode_workload_shape_sampled():
    """The decode workload's per-sequence shape (32768 cached tokens, Hq=32,
    Hkv=8, D=128) for 4 sequences; the oracle checks 2 of them."""
    mxq = gpu_or_skip()
    d = mxq_inputs.make_decode("decode", seqs=range(4), B=4)
    out, _ = _run(mxq, d, 64, 128)
    sub = dict(d, k=d["k"][:2], v=d["v"][:2])
    ref = Dm.attn_decode_ref(d["q"][:2], Dm.build_kv_cache_ref(sub["k"], sub["v"], d["seq_len"][:2], 64, 128),
                             d["seq_len"][:2], 64, 128)
    err = np.abs(out[:2] - ref).max()
    assert err <= TOL, err
    print(f"decode full-length max-abs {err:.3e}")


def test_error_paths():
    mxq = gpu_or_skip()
    import torch

    d = mxq_inputs.make_decode(dict(B=1, L=256, Hq=16, Hkv=2, D=128, n_sink=0, n_recent=0, seed=1), threads=1)
    k, v, q = bf16_dev(d["k"]), bf16_dev(d["v"]), bf16_dev(d["q"])
    cache = mxq.build_quant_kv_cache(k, v, torch.tensor([256], dtype=torch.int32, device="cuda:0"), 0, 0)
    with pytest.raises(mxq.MxqError) as ei:        # G = 8 is not built
        mxq.attn_quantkv_decode(q, cache, 2, 256)
    assert ei.value.status == mxq.MXQ_EUNSUPPORTED
    with pytest.raises(mxq.MxqError) as ei:        # max_seq_len above the cache capacity
        mxq.attn_quantkv_decode(q[:, :8].contiguous(), cache, 4, 4096)
    assert ei.value.status == mxq.MXQ_EINVAL


def _host_cache(cache):
    from gpu_helpers import u8, u16

    out = {}
    for n in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero", "k_sink", "v_sink", "k_recent",
              "v_recent"):
        t = getattr(cache, n)
        out[n] = None if t is None else (u8(t) if n.endswith("codes") else u16(t))
    return out


@pytest.mark.parametrize("n_sink,n_recent", [(64, 128), (16, 0)])
def test_append_bit_exact_then_decode(n_sink, n_recent):
    """attn_quantkv_append against the oracle's append, step by step from the
    same cache: every array bit-exact after 24 steps (window moves, tokens
    leaving it re-quantised, sink writes for a short sequence), then decode
    over the grown cache against the oracle."""
    mxq = gpu_or_skip()
    import torch
    from oracle.formats import pack_nibbles

    lens0 = np.array([300, 150, 40], dtype=np.int32)
    d = mxq_inputs.make_decode(dict(B=3, L=512, Hq=8, Hkv=2, D=128, n_sink=n_sink, n_recent=n_recent, seed=11,
                                    seq_len=list(lens0)), threads=3)
    k0, v0 = d["k"].copy(), d["v"].copy()
    for b in range(3):  # the future is unknown when the cache is built
        k0[b, :, lens0[b]:] = 0
        v0[b, :, lens0[b]:] = 0
    krec = vrec = None
    if n_recent:
        krec = np.zeros((3, 2, n_recent, 128), dtype=np.uint16)
        vrec = np.zeros_like(krec)
        for b in range(3):
            for r in range(n_recent):
                t = lens0[b] - n_recent + r
                if t >= 0:
                    krec[b, :, r], vrec[b, :, r] = k0[b, :, t], v0[b, :, t]
        krec, vrec = bf16_dev(krec), bf16_dev(vrec)
    seq = torch.from_numpy(lens0.copy()).to("cuda:0")
    cache = mxq.build_quant_kv_cache(bf16_dev(k0), bf16_dev(v0), seq, n_sink, n_recent, krec, vrec)
    ref = Dm.build_kv_cache_ref(k0, v0, lens0, n_sink, n_recent)
    lens = lens0
    for _ in range(24):
        kn = np.stack([d["k"][b, :, lens[b]] for b in range(3)])
        vn = np.stack([d["v"][b, :, lens[b]] for b in range(3)])
        mxq.attn_quantkv_append(cache, bf16_dev(kn), bf16_dev(vn))
        ref, lens = Dm.append_kv_ref(ref, lens, kn, vn, n_sink, n_recent)
    got = _host_cache(cache)
    assert np.array_equal(seq.cpu().numpy(), lens)
    for which in ("k", "v"):
        assert np.array_equal(got[which + "_codes"], pack_nibbles(ref[which + "_codes"])), which
        for name in ("_scale", "_zero", "_sink", "_recent"):
            if got[which + name] is None:  # no copy kept (n_recent = 0)
                assert ref[which + name].size == 0
                continue
            assert np.array_equal(got[which + name], ref[which + name].view(np.uint16)), which + name
    out = mxq.attn_quantkv_decode(bf16_dev(d["q"]), cache, 2, int(lens.max())).cpu().numpy()
    want = Dm.attn_decode_ref(d["q"], ref, lens, n_sink, n_recent)
    assert np.abs(out - want).max() <= TIGHT


def test_append_leaves_out_of_range_sequences_alone():
    mxq = gpu_or_skip()
    import torch

    d = mxq_inputs.make_decode(dict(B=2, L=128, Hq=4, Hkv=1, D=128, n_sink=4, n_recent=8, seed=12,
                                    seq_len=[128, 60]), threads=2)
    krec = bf16_dev(np.stack([d["k"][b, :, d["seq_len"][b] - 8:d["seq_len"][b]] for b in range(2)]))
    vrec = bf16_dev(np.stack([d["v"][b, :, d["seq_len"][b] - 8:d["seq_len"][b]] for b in range(2)]))
    seq = torch.from_numpy(d["seq_len"].copy()).to("cuda:0")
    cache = mxq.build_quant_kv_cache(bf16_dev(d["k"]), bf16_dev(d["v"]), seq, 4, 8, krec, vrec)
    before = _host_cache(cache)
    kn = bf16_dev(d["k"][:, :, 0].copy())
    mxq.attn_quantkv_append(cache, kn, kn)
    after = _host_cache(cache)
    assert seq.cpu().numpy().tolist() == [128, 61]   # sequence 0 is full (L_cap = 128)
    assert np.array_equal(after["k_recent"][0], before["k_recent"][0])
    assert not np.array_equal(after["k_recent"][1], before["k_recent"][1])


def _gather_lines(x, lines):
    """bf16 bits [B,Hkv,L,D] -> the rows of the listed tokens [B,Hkv,n,D] (zero rows for entries outside [0, L))."""
    B, H, L, D = x.shape
    out = np.zeros(lines.shape + (D,), dtype=x.dtype)
    for b in range(B):
        for h in range(H):
            for e, t in enumerate(lines[b, h]):
                if 0 <= t < L:
                    out[b, h, e] = x[b, h, t]
    return out


def _run_lines(mxq, d, n_sink, n_recent, lines, num_splits=0):
    import torch

    k, v, q = bf16_dev(d["k"]), bf16_dev(d["v"]), bf16_dev(d["q"])
    lens = d["seq_len"]
    krec = torch.stack([k[b, :, lens[b] - n_recent:lens[b]] for b in range(len(lens))])
    vrec = torch.stack([v[b, :, lens[b] - n_recent:lens[b]] for b in range(len(lens))])
    lt = torch.from_numpy(lines).to("cuda:0")
    cache = mxq.build_quant_kv_cache(k, v, torch.from_numpy(lens).to("cuda:0"), n_sink, n_recent, krec, vrec,
                                     lines=lt, k_line_rows=bf16_dev(_gather_lines(d["k"], lines)),
                                     v_line_rows=bf16_dev(_gather_lines(d["v"], lines)))
    return mxq.attn_quantkv_decode(q, cache, d["Hkv"], int(lens.max()), num_splits=num_splits).cpu().numpy()


@pytest.mark.parametrize("num_splits", [0, 3, 16])
@pytest.mark.parametrize("G", [1, 4])
def test_decode_with_lines(num_splits, G):
    """Line tokens spread over the INT4 region (block edges, several splits),
    in the sink and the window (ignored) and in messy lists."""
    mxq = gpu_or_skip()
    Hkv = 2
    lens = [1000, 400, 64 + 128 + 40]
    d = mxq_inputs.make_decode(dict(B=3, L=1024, Hq=Hkv * G, Hkv=Hkv, D=128, n_sink=64, n_recent=128, seed=31,
                                    seq_len=lens), threads=3)
    rng = np.random.default_rng(31)
    lines = np.full((3, Hkv, 16), -1, dtype=np.int32)
    for b in range(3):
        for h in range(Hkv):
            picks = np.sort(rng.choice(np.arange(64, lens[b] - 128), size=min(10, lens[b] - 192), replace=False))
            row = list(picks) + [5, lens[b] - 3, 63, 64, 95, 96][: 16 - len(picks)]
            lines[b, h, :len(row)] = row
    lines[0, 0, :6] = [64, 95, 96, 127, 128, 200]  # block edges
    lines[1, 1, :5] = [300, 300, 200, 310, -1]     # a repeat and an out-of-order entry
    out = _run_lines(mxq, d, 64, 128, lines, num_splits)
    cache = Dm.build_kv_cache_ref(d["k"], d["v"], d["seq_len"], 64, 128, lines=lines)
    ref = Dm.attn_decode_ref(d["q"], cache, d["seq_len"], 64, 128)
    err = np.abs(out - ref).max()
    assert err <= TIGHT, err


def test_decode_heavy_token_as_a_line():
    """A planted heavy token: its 4-bit codes drag decode far from exact
    attention; kept as a line, the GPU result is close to exact."""
    mxq = gpu_or_skip()
    from oracle import formats as F

    d = mxq_inputs.make_decode(dict(B=1, L=2048, Hq=4, Hkv=1, D=128, n_sink=64, n_recent=128, seed=32,
                                    seq_len=[2048]), threads=1)
    q = F.bf16_bits_to_f32(d["q"])
    k = F.bf16_bits_to_f32(d["k"]).copy()
    u = q[0].mean(axis=0)
    k[0, 0, 1000] = 3.0 * u / np.linalg.norm(u) * 11.3
    k[0, 0, 1000, :8] += 37.0
    d["k"] = F.f32_to_bf16_bits(k)
    lines = np.array([[[1000] + [-1] * 15]], dtype=np.int32)
    out = _run_lines(mxq, d, 64, 128, lines)
    kf = F.bf16_bits_to_f32(d["k"]).astype(np.float64)[0, 0]
    vf = F.bf16_bits_to_f32(d["v"]).astype(np.float64)[0, 0]
    exact = []
    for h in range(4):
        s = kf @ q[0, h].astype(np.float64) / np.sqrt(128.0)
        p = np.exp(s - s.max())
        exact.append(p @ vf / p.sum())
    exact = np.stack(exact)
    plain, _ = _run(mxq, d, 64, 128)
    e_line, e_plain = np.abs(out[0] - exact).max(), np.abs(plain[0] - exact).max()
    assert e_line < 0.2 * e_plain, (e_line, e_plain)


def test_decode_lines_from_the_prefill_selection():
    """Reading R36: the prefill's group-shared vertical lines become the
    decode cache's fp16 line tokens (mxq_kv_lines_from_prefill): lists and
    fp16 rows bit-exact against the oracle, decode within the bound."""
    mxq = gpu_or_skip()
    import torch
    from gpu_helpers import u16
    from oracle import select as S

    B, Hq, Hkv, L, D = 2, 8, 2, 1024, 128
    G = Hq // Hkv
    rng = np.random.default_rng(36)
    common = rng.standard_normal((B, Hkv, 1, D)).astype(np.float32)
    qp = (rng.standard_normal((B, Hq, L, D)) * 0.5 + np.repeat(common, G, axis=1)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    k[:, :, 700] += 4.0 * common[:, :, 0]
    from oracle.formats import f32_to_bf16_bits
    qb, kb, vb = f32_to_bf16_bits(qp), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    qd_bits = f32_to_bf16_bits(rng.standard_normal((B, Hq, D)).astype(np.float32))
    lens = np.array([L, 900], dtype=np.int32)
    qg, kg, vg, qdg = bf16_dev(qb), bf16_dev(kb), bf16_dev(vb), bf16_dev(qd_bits)
    shape = mxq.Shape(B, Hq, Hkv, L, L, D, 64, 64, True)
    lines_hq, _ = mxq.attn_select_lines(qg, kg, shape, 16, 1, group_shared=True)
    lines, kl, vl = mxq.kv_lines_from_prefill(lines_hq, kg, vg)
    r_hq, _ = S.select_lines(qb, kb, L, 64, 16, 1, group_shared=True)
    r_lines = np.ascontiguousarray(r_hq[:, ::G])
    assert np.array_equal(lines.cpu().numpy(), r_lines)
    ref = Dm.build_kv_cache_ref(kb, vb, lens, 64, 128, lines=r_lines)
    assert np.array_equal(u16(kl), ref["k_lines"].view(np.uint16))
    assert np.array_equal(u16(vl), ref["v_lines"].view(np.uint16))
    krec = torch.stack([kg[b, :, lens[b] - 128:lens[b]] for b in range(B)])
    vrec = torch.stack([vg[b, :, lens[b] - 128:lens[b]] for b in range(B)])
    base = mxq.build_quant_kv_cache(kg, vg, torch.from_numpy(lens).to("cuda:0"), 64, 128, krec, vrec)
    cache = mxq.QuantKVCache(base.k_codes, base.v_codes, base.k_scale, base.k_zero, base.v_scale, base.v_zero,
                             base.k_sink, base.v_sink, base.k_recent, base.v_recent, base.seq_len, 64, 128,
                             lines, kl, vl)
    out = mxq.attn_quantkv_decode(qdg, cache, Hkv, int(lens.max())).cpu().numpy()
    oref = Dm.attn_decode_ref(qd_bits, ref, lens, 64, 128)
    err = np.abs(out - oref).max()
    assert err <= TIGHT, err
