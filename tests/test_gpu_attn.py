"""GPU parity: attn_mixed_fwd against the oracle (max-abs <= 5e-3, fp32 out)."""

import numpy as np
import pytest

from gpu_helpers import bf16_dev, gpu_or_skip, poison_lds, u32
import mxq_inputs
from oracle import attention as A
from oracle import select as S
from oracle.formats import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

TOL = 5e-3  # max-abs on outputs, unit-variance V, fp32 accumulation and output


def _shape(mxq, cfg):
    return mxq.Shape(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["n_valid"], cfg["D"], cfg["Bq"], cfg["Bk"],
                     cfg["causal"])


def _gpu_prefill(mxq, cfg, mode=0, mask=None, out_dtype=0, with_lines=False):
    q, k, v = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
    shape = _shape(mxq, cfg)
    lines = None
    if with_lines:
        lines, _ = mxq.attn_select_lines(q, k, shape, cfg["n_lines"], cfg["sink_tokens"])
    ops = mxq.prepare_prefill(q, k, v, cfg["n_valid"], mode, lines=with_lines)
    if mode == mxq.MXQ_MIXED and mask is None:
        mask, _, _ = mxq.attn_select_blocks(q, k, shape, topk=cfg["topk"], ratio=(cfg["ratio_num"], cfg["ratio_den"]),
                                            sink_tiles=cfg["sink_tiles"], local_tiles=cfg["local_tiles"])
    elif mask is not None:
        import torch
        mask = torch.from_numpy(np.ascontiguousarray(mask).view(np.int32)).to("cuda:0")
    out, lse = mxq.attn_mixed_fwd(ops, mask, shape, mode=mode, out_dtype=out_dtype, lines=lines)
    res = (out.float().cpu().numpy(), lse.cpu().numpy(), (u32(mask) if mask is not None else None))
    return res + (lines.cpu().numpy(),) if with_lines else res


def _check(out, lse, ro, rl, rows=None):
    if rows is not None:
        out, lse, ro, rl = out[..., rows, :], lse[..., rows], ro[..., rows, :], rl[..., rows]
    err = np.abs(out - ro)
    assert np.all(np.isfinite(out))
    assert err.max() <= TOL, f"max-abs {err.max():.3e}"
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - rl[fin]).max() <= TOL
    return float(err.max())


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_tiny_all_modes(mode):
    mxq = gpu_or_skip()
    cfg = mxq_inputs.make_prefill("tiny")
    out, lse, mask = _gpu_prefill(mxq, cfg, mode)
    rm = None
    if mode == 0:
        rm, _, _ = S.select_blocks(cfg["q"], cfg["k"], cfg["n_valid"], cfg["Bq"], cfg["Bk"], cfg["causal"],
                                   cfg["topk"], cfg["ratio_num"], cfg["ratio_den"], cfg["sink_tiles"],
                                   cfg["local_tiles"])
        assert np.array_equal(mask, rm)
    ro, rl = A.attn_mixed_ref(cfg["q"], cfg["k"], cfg["v"], cfg["n_valid"], cfg["Bq"], cfg["Bk"], cfg["causal"],
                              mask=rm, mode=mode)
    _check(out, lse, ro, rl)


CASES = [
    # D, Bq, causal, N, n_valid, Hq, Hkv
    (64, 64, True, 512, 512, 2, 1),
    (64, 128, False, 512, 389, 4, 2),
    (128, 64, True, 384, 333, 4, 4),
    (128, 128, True, 512, 500, 4, 1),
    (128, 128, False, 256, 256, 2, 2),
    # N <= 256 runs the short-sequence kernel: causal, ragged, one chunk
    (64, 128, True, 256, 250, 4, 2),
    (128, 64, True, 256, 130, 2, 1),
    (64, 64, True, 128, 100, 2, 1),
    (128, 128, False, 128, 77, 2, 2),
    # one valid row and key (the smallest input the host accepts), both kernels
    (64, 64, False, 128, 1, 2, 1),
    (128, 128, True, 384, 1, 2, 2),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_shapes_modes_ragged(case, mode):
    mxq = gpu_or_skip()
    D, Bq, causal, N, nv, Hq, Hkv = case
    rng = np.random.default_rng(D + Bq + N + nv)
    q = rng.standard_normal((1, Hq, N, D)).astype(np.float32) * 1.5
    k = rng.standard_normal((1, Hkv, N, D)).astype(np.float32)
    v = rng.standard_normal((1, Hkv, N, D)).astype(np.float32)
    k[:, :, 0] *= 8  # a sink key
    for t in (q, k, v):
        t[:, :, nv:] = 0
    n_qt, n_kt = N // Bq, N // 64
    mask = rng.integers(0, 2 ** 31, size=(1, Hq, n_qt, (n_kt + 31) // 32)).astype(np.uint32)
    mask &= np.uint32((1 << n_kt) - 1) if n_kt < 32 else np.uint32(0xFFFFFFFF)
    cfg = dict(B=1, Hq=Hq, Hkv=Hkv, N=N, n_valid=nv, D=D, Bq=Bq, Bk=64, causal=causal,
               q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v))
    out, lse, _ = _gpu_prefill(mxq, cfg, mode, mask=mask if mode == 0 else None)
    ro, rl = A.attn_mixed_ref(cfg["q"], cfg["k"], cfg["v"], nv, Bq, 64, causal, mask=mask, mode=mode)
    _check(out, lse, ro, rl)
    assert np.all(out[:, :, nv:] == 0) and np.all(np.isneginf(lse[:, :, nv:]))


def test_llama8b_full_size_sampled():
    """The Llama-8B-shaped causal workload at full size; the oracle computes a
    sample of (head, query tile) pairs, spread over the key range."""
    mxq = gpu_or_skip()
    cfg = mxq_inputs.make_prefill("llama8b")
    out, lse, mask = _gpu_prefill(mxq, cfg, 0)
    G = cfg["Hq"] // cfg["Hkv"]
    worst = 0.0
    for h in (0, 13, 31):
        kv = h // G
        sub_q, sub_k, sub_v = cfg["q"][:, h:h + 1], cfg["k"][:, kv:kv + 1], cfg["v"][:, kv:kv + 1]
        rm, _, _ = S.select_blocks(sub_q, sub_k, cfg["n_valid"], cfg["Bq"], cfg["Bk"], True, cfg["topk"],
                                   cfg["ratio_num"], cfg["ratio_den"], cfg["sink_tiles"], cfg["local_tiles"])
        assert np.array_equal(mask[:, h:h + 1], rm), f"head {h}: mask differs"
        ops = A.prepare_operands(sub_q, sub_k, sub_v, cfg["n_valid"])
        tiles = [0, 1, 17, 40, 63]
        ro, rl = A.attn_mixed_ref(sub_q, sub_k, sub_v, cfg["n_valid"], cfg["Bq"], cfg["Bk"], True,
                                  mask=rm, qtiles=tiles, ops=ops)
        rows = np.concatenate([np.arange(t * 128, (t + 1) * 128) for t in tiles])
        worst = max(worst, _check(out[:, h:h + 1], lse[:, h:h + 1], ro, rl, rows=rows))
    print(f"llama8b sampled max-abs {worst:.3e}")


def test_vit_batch_sampled():
    """ViT-shaped batch: the CLS token is a one-token vertical line, every
    tile low-bit."""
    mxq = gpu_or_skip()
    cfg = mxq_inputs.make_prefill("vit", B=8)
    out, lse, mask, lines = _gpu_prefill(mxq, cfg, 0, with_lines=True)
    assert not mask.any() and np.all(lines[..., 0] == 0)
    rlines, _ = S.select_lines(cfg["q"], cfg["k"], cfg["n_valid"], cfg["Bq"], cfg["n_lines"], cfg["sink_tokens"])
    assert np.array_equal(lines, rlines)
    for b, h in ((0, 0), (3, 7), (7, 11)):
        ro, rl = A.attn_mixed_ref(cfg["q"][b:b + 1, h:h + 1], cfg["k"][b:b + 1, h:h + 1], cfg["v"][b:b + 1, h:h + 1],
                                  cfg["n_valid"], 64, 64, False, mask=np.zeros_like(mask[b:b + 1, h:h + 1]),
                                  lines=rlines[b:b + 1, h:h + 1])
        _check(out[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], ro, rl)


def test_vit_full_batch_sampled():
    """The ViT-shaped workload at its full batch (512 x 12 heads, 197 of 256
    tokens, CLS as a line) in the benchmark's launch configuration: lines
    bit-exact for sampled heads and their outputs within 5e-3."""
    mxq = gpu_or_skip()
    import torch

    cfg = mxq_inputs.make_prefill("vit")
    q, k, v = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
    shape = _shape(mxq, cfg)
    pipe = mxq.PrefillPipeline(shape, topk=cfg["topk"], ratio=(cfg["ratio_num"], cfg["ratio_den"]),
                               sink_tiles=cfg["sink_tiles"], local_tiles=cfg["local_tiles"], n_lines=cfg["n_lines"],
                               sink_tokens=cfg["sink_tokens"], out_dtype=mxq.MXQ_OUT_F32)
    out_t, lse_t = pipe(q, k, v)
    torch.cuda.synchronize()
    out, lse = out_t.cpu().numpy(), lse_t.cpu().numpy()
    lines, mask = pipe.lines.cpu().numpy(), u32(pipe.mask)
    assert not mask.any()
    for b, h in ((0, 0), (137, 5), (300, 11), (511, 6)):
        sq, sk, sv = cfg["q"][b:b + 1, h:h + 1], cfg["k"][b:b + 1, h:h + 1], cfg["v"][b:b + 1, h:h + 1]
        rl_, _ = S.select_lines(sq, sk, cfg["n_valid"], cfg["Bq"], cfg["n_lines"], cfg["sink_tokens"])
        assert np.array_equal(lines[b:b + 1, h:h + 1], rl_)
        ro, rl = A.attn_mixed_ref(sq, sk, sv, cfg["n_valid"], 64, 64, False, mask=np.zeros_like(mask[b:b + 1, h:h + 1]),
                                  lines=rl_)
        _check(out[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], ro, rl)


def test_deterministic_and_bf16_output():
    mxq = gpu_or_skip()
    cfg = mxq_inputs.make_prefill("tiny")
    o1, l1, _ = _gpu_prefill(mxq, cfg, 0)
    o2, l2, _ = _gpu_prefill(mxq, cfg, 0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    ob, _, _ = _gpu_prefill(mxq, cfg, 0, out_dtype=1)
    # the bf16 output is the fp32 result rounded to nearest, ties to even
    assert np.array_equal(f32_to_bf16_bits(ob), f32_to_bf16_bits(o1))
    assert np.array_equal(ob, bf16_bits_to_f32(f32_to_bf16_bits(o1)))
    # the same for the short-sequence kernel
    cfg = mxq_inputs.make_prefill("vit", B=2)
    o1, _, _ = _gpu_prefill(mxq, cfg, 0)
    ob, _, _ = _gpu_prefill(mxq, cfg, 0, out_dtype=1)
    assert np.array_equal(ob, bf16_bits_to_f32(f32_to_bf16_bits(o1)))


def test_error_paths():
    mxq = gpu_or_skip()
    import torch

    cfg = mxq_inputs.make_prefill("tiny")
    q, k, v = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
    shape = _shape(mxq, cfg)
    ops = mxq.prepare_prefill(q, k, v, cfg["n_valid"])
    with pytest.raises(mxq.MxqError) as ei:          # MIXED without a mask
        mxq.attn_mixed_fwd(ops, None, shape)
    assert ei.value.status == mxq.MXQ_EINVAL
    bad = mxq.Shape(1, 2, 2, 256, 256, 96, 64, 64, False)  # unsupported head_dim
    with pytest.raises(mxq.MxqError) as ei:
        mxq.attn_mixed_fwd(ops, torch.zeros(1, dtype=torch.int32, device="cuda:0"), bad)
    assert ei.value.status == mxq.MXQ_EUNSUPPORTED


@pytest.mark.parametrize("mode", [0, 1])
def test_rotated_lowbit_operands(mode):
    """Q/K rotated by the Walsh-Hadamard matrix before MXFP4 (the pages'
    alternative to promotion), on the outlier recipe, against the oracle."""
    mxq = gpu_or_skip()
    import torch

    cfg = mxq_inputs.make_prefill("llama8b", N=1024, n_valid=1000, Hq=4, Hkv=1, B=1)
    q, k, v = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
    shape = _shape(mxq, cfg)
    ops = mxq.prepare_prefill(q, k, v, cfg["n_valid"], mode, rotate=True)
    mask = None
    if mode == 0:
        mask, _, _ = mxq.attn_select_blocks(q, k, shape, topk=-1, ratio=(5, 100), sink_tiles=1, local_tiles=1)
    out, lse = mxq.attn_mixed_fwd(ops, mask, shape, mode=mode)
    rm = None
    if mode == 0:
        rm, _, _ = S.select_blocks(cfg["q"], cfg["k"], cfg["n_valid"], 128, 64, True, -1, 5, 100, 1, 1)
        assert np.array_equal(u32(mask), rm)
    ro, rl = A.attn_mixed_ref(cfg["q"], cfg["k"], cfg["v"], cfg["n_valid"], 128, 64, True,
                              mask=rm, mode=mode, rotate=True)
    _check(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)


def test_prefill_pipeline_matches_the_sequential_calls():
    """PrefillPipeline (selection on a second stream) gives bit-identical
    results to the calls made one after another, over repeated steps."""
    mxq = gpu_or_skip()
    import torch

    for name, over in (("llama8b", dict(N=2048, n_valid=2000, Hq=8, Hkv=2)), ("vit", dict(B=4))):
        cfg = mxq_inputs.make_prefill(name, **over)
        q, k, v = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
        shape = _shape(mxq, cfg)
        pipe = mxq.PrefillPipeline(shape, topk=cfg["topk"], ratio=(cfg["ratio_num"], cfg["ratio_den"]),
                                   sink_tiles=cfg["sink_tiles"], local_tiles=cfg["local_tiles"],
                                   n_lines=cfg["n_lines"], sink_tokens=cfg["sink_tokens"], out_dtype=mxq.MXQ_OUT_F32)
        mask, _, _ = mxq.attn_select_blocks(q, k, shape, topk=cfg["topk"], ratio=(cfg["ratio_num"], cfg["ratio_den"]),
                                            sink_tiles=cfg["sink_tiles"], local_tiles=cfg["local_tiles"])
        lines = mxq.attn_select_lines(q, k, shape, cfg["n_lines"], cfg["sink_tokens"])[0] if cfg["n_lines"] else None
        ops = mxq.prepare_prefill(q, k, v, cfg["n_valid"], lines=lines is not None)
        ref, ref_lse = mxq.attn_mixed_fwd(ops, mask, shape, lines=lines)
        for _ in range(3):
            out, lse = pipe(q, k, v)
            torch.cuda.synchronize()
            assert torch.equal(out, ref) and torch.equal(lse, ref_lse), name


def test_prefill_pipeline_group_heads():
    """PrefillPipeline with group_heads (one mask and one line list per kv
    group, the attention launched per kv group) equals the calls made one
    after another with group-shared selection and the per-head launch, bit
    for bit, over repeated steps (both chains: tiles chosen by score on one
    stream, and lines on the two-stream step)."""
    mxq = gpu_or_skip()
    import torch

    for over in (dict(N=2048, n_valid=2000, Hq=8, Hkv=2, n_lines=0), dict(N=1024, n_valid=1024, Hq=8, Hkv=4, n_lines=8)):
        n_lines = over.pop("n_lines")
        cfg = mxq_inputs.make_prefill("llama8b", **over)
        q, k, v = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
        shape = _shape(mxq, cfg)
        sel = dict(topk=cfg["topk"], ratio=(cfg["ratio_num"], cfg["ratio_den"]), sink_tiles=cfg["sink_tiles"],
                   local_tiles=cfg["local_tiles"])
        grouped = mxq.PrefillPipeline(shape, n_lines=n_lines, sink_tokens=1, out_dtype=mxq.MXQ_OUT_F32,
                                      group_shared=True, group_heads=True, **sel)
        mask, _, _ = mxq.attn_select_blocks(q, k, shape, group_shared=True, **sel)
        lines = mxq.attn_select_lines(q, k, shape, n_lines, 1, group_shared=True)[0] if n_lines else None
        ops = mxq.prepare_prefill(q, k, v, cfg["n_valid"], lines=lines is not None)
        ref, ref_lse = mxq.attn_mixed_fwd(ops, mask, shape, lines=lines)
        for _ in range(3):
            out, lse = grouped(q, k, v)
            torch.cuda.synchronize()
            assert torch.equal(out, ref) and torch.equal(lse, ref_lse), over


def test_long32k_full_size_sampled():
    """The long-context causal workload at full size (N = 32768, 5% + sink +
    4-tile window) in the launch configuration the benchmark times (the fused
    quantiser with tile means, selection on the means, attention), with fp32
    output for parity: masks bit-exact for sampled heads, and the first, a
    middle and the last query tiles (256 key chunks) within 5e-3."""
    mxq = gpu_or_skip()
    import torch

    cfg = mxq_inputs.make_prefill("long32k")
    q, k, v = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
    shape = _shape(mxq, cfg)
    pipe = mxq.PrefillPipeline(shape, topk=cfg["topk"], ratio=(cfg["ratio_num"], cfg["ratio_den"]),
                               sink_tiles=cfg["sink_tiles"], local_tiles=cfg["local_tiles"],
                               out_dtype=mxq.MXQ_OUT_F32)
    assert pipe.fused
    out_t, lse_t = pipe(q, k, v)
    torch.cuda.synchronize()
    out, lse, mask = out_t.cpu().numpy(), lse_t.cpu().numpy(), u32(pipe.mask)
    del q, k, v
    G = cfg["Hq"] // cfg["Hkv"]
    tiles = [0, 127, 200, 255]
    rows = np.concatenate([np.arange(t * 128, (t + 1) * 128) for t in tiles])
    worst = 0.0
    for h in (0, 13, 31):
        kv = h // G
        sub_q, sub_k, sub_v = cfg["q"][:, h:h + 1], cfg["k"][:, kv:kv + 1], cfg["v"][:, kv:kv + 1]
        rm, _, _ = S.select_blocks(sub_q, sub_k, cfg["n_valid"], cfg["Bq"], cfg["Bk"], True, cfg["topk"],
                                   cfg["ratio_num"], cfg["ratio_den"], cfg["sink_tiles"], cfg["local_tiles"])
        assert np.array_equal(mask[:, h:h + 1], rm), f"head {h}: mask differs"
        ops = A.prepare_operands(sub_q, sub_k, sub_v, cfg["n_valid"])
        ro, rl = A.attn_mixed_ref(sub_q, sub_k, sub_v, cfg["n_valid"], cfg["Bq"], cfg["Bk"], True,
                                  mask=rm, qtiles=tiles, ops=ops)
        worst = max(worst, _check(out[:, h:h + 1], lse[:, h:h + 1], ro, rl, rows=rows))
    print(f"long32k sampled max-abs {worst:.3e}")


@pytest.mark.parametrize("mode", [0, 1])
def test_block_exponent_spread_above_18(mode):
    """A pair's block-exponent spread above 18 bits: K's head_dim block 1 is
    scaled by 2^12 and Q's block 2 by 2^-8 (spread about 20), with a softmax
    scale of 2^-13 that keeps the logits near unit size, so every block still
    shapes P.  The FP4 MFMA's scores must still give outputs within 5e-3 of
    the oracle's exactly rounded ones."""
    mxq = gpu_or_skip()
    rng = np.random.default_rng(77)
    N, nv, Hq, Hkv, D = 512, 500, 4, 1, 128
    q = rng.standard_normal((1, Hq, N, D)).astype(np.float32)
    k = rng.standard_normal((1, Hkv, N, D)).astype(np.float32)
    v = rng.standard_normal((1, Hkv, N, D)).astype(np.float32)
    k[..., 32:64] *= np.float32(2.0 ** 12)
    q[..., 64:96] *= np.float32(2.0 ** -8)
    for t in (q, k, v):
        t[:, :, nv:] = 0
    cfg = dict(B=1, Hq=Hq, Hkv=Hkv, N=N, n_valid=nv, D=D, Bq=128, Bk=64, causal=True,
               q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v))
    ops_ref = A.prepare_operands(cfg["q"], cfg["k"], cfg["v"], nv)
    e = ops_ref["q_exp"][0, 0][:nv, None, :] + ops_ref["k_exp"][0, 0][None, :nv, :]
    assert int((e.max(-1) - e.min(-1)).max()) > 18
    scale = 2.0 ** -13
    qd, kd, vd = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
    shape = _shape(mxq, cfg)
    ops = mxq.prepare_prefill(qd, kd, vd, nv, mode)
    mask = None
    if mode == 0:
        mask, _, _ = mxq.attn_select_blocks(qd, kd, shape, topk=1, ratio=(0, 1), sink_tiles=0, local_tiles=1)
    out, lse = mxq.attn_mixed_fwd(ops, mask, shape, softmax_scale=scale, mode=mode)
    rm = None
    if mode == 0:
        rm, _, _ = S.select_blocks(cfg["q"], cfg["k"], nv, 128, 64, True, 1, 0, 1, 0, 1)
        assert np.array_equal(u32(mask), rm)
    ro, rl = A.attn_mixed_ref(cfg["q"], cfg["k"], cfg["v"], nv, 128, 64, True, mask=rm, mode=mode,
                              softmax_scale=scale, ops=ops_ref)
    err = _check(out.cpu().numpy(), lse.cpu().numpy(), ro, rl)
    print(f"spread > 18, mode {mode}: max-abs {err:.3e}")


@pytest.mark.parametrize("word", [0xFFFFFFFF, 0x7F7F7F7F])
def test_stale_lds_does_not_reach_the_output(word):
    """LDS is not cleared between kernels: fill every CU's LDS with E4M3 / E8M0
    NaN bytes right before the attention kernel (same stream).  Buffers the
    first pipeline step reads before any copy has filled them must not let a
    NaN into O (0 * NaN is NaN): outputs stay finite and within 5e-3."""
    mxq = gpu_or_skip()
    import torch

    cases = [mxq_inputs.make_prefill("tiny"),
             mxq_inputs.make_prefill("llama8b", N=1024, n_valid=1000, Hq=4, Hkv=1),
             mxq_inputs.make_prefill("vit", B=2)]
    for cfg in cases:
        lines_on = cfg["n_lines"] > 0
        q, k, v = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
        shape = _shape(mxq, cfg)
        lines = mxq.attn_select_lines(q, k, shape, cfg["n_lines"], cfg["sink_tokens"])[0] if lines_on else None
        rlines = None
        if lines_on:
            rlines, _ = S.select_lines(cfg["q"], cfg["k"], cfg["n_valid"], cfg["Bq"], cfg["n_lines"],
                                       cfg["sink_tokens"])
            assert np.array_equal(lines.cpu().numpy(), rlines)
        for mode in (0, 1):
            ops = mxq.prepare_prefill(q, k, v, cfg["n_valid"], mode, lines=lines_on)
            mask = None
            if mode == 0:
                mask, _, _ = mxq.attn_select_blocks(q, k, shape, topk=cfg["topk"],
                                                    ratio=(cfg["ratio_num"], cfg["ratio_den"]),
                                                    sink_tiles=cfg["sink_tiles"], local_tiles=cfg["local_tiles"])
            rm = None
            if mode == 0:
                rm, _, _ = S.select_blocks(cfg["q"], cfg["k"], cfg["n_valid"], cfg["Bq"], cfg["Bk"], cfg["causal"],
                                           cfg["topk"], cfg["ratio_num"], cfg["ratio_den"], cfg["sink_tiles"],
                                           cfg["local_tiles"])
                assert np.array_equal(u32(mask), rm)
            torch.cuda.synchronize()
            poison_lds(word)
            out, lse = mxq.attn_mixed_fwd(ops, mask, shape, mode=mode, lines=lines)
            torch.cuda.synchronize()
            hs = [(0, 0), (cfg["B"] - 1, cfg["Hq"] - 1)]
            for b, h in hs:
                kv = h // (cfg["Hq"] // cfg["Hkv"])
                ro, rl = A.attn_mixed_ref(cfg["q"][b:b + 1, h:h + 1], cfg["k"][b:b + 1, kv:kv + 1],
                                          cfg["v"][b:b + 1, kv:kv + 1], cfg["n_valid"], cfg["Bq"], cfg["Bk"],
                                          cfg["causal"], mask=rm[b:b + 1, h:h + 1] if rm is not None else None,
                                          mode=mode, lines=rlines[b:b + 1, h:h + 1] if lines_on else None)
                _check(out.cpu().numpy()[b:b + 1, h:h + 1], lse.cpu().numpy()[b:b + 1, h:h + 1], ro, rl)
            assert torch.isfinite(out).all()


def test_largest_key_axis_sampled():
    """The largest key axis the host accepts (2048 key tiles, N = 131072) with a
    ragged tail: 1024 chunks per row at the end, 64 mask words per row.  Masks
    bit-exact for both heads; the first, a middle and the last query tile of
    head 1 within 5e-3."""
    mxq = gpu_or_skip()
    import torch

    cfg = mxq_inputs.make_prefill("long32k", N=131072, n_valid=131072 - 37, Hq=2, Hkv=1)
    q, k, v = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
    shape = _shape(mxq, cfg)
    pipe = mxq.PrefillPipeline(shape, topk=cfg["topk"], ratio=(cfg["ratio_num"], cfg["ratio_den"]),
                               sink_tiles=cfg["sink_tiles"], local_tiles=cfg["local_tiles"],
                               out_dtype=mxq.MXQ_OUT_F32)
    out_t, lse_t = pipe(q, k, v)
    torch.cuda.synchronize()
    out, lse, mask = out_t.cpu().numpy(), lse_t.cpu().numpy(), u32(pipe.mask)
    del q, k, v
    last = (cfg["n_valid"] - 1) // 128
    tiles = [0, 512, last]
    rows = np.concatenate([np.arange(t * 128, (t + 1) * 128) for t in tiles])
    for h in (0, 1):
        sub_q, sub_k, sub_v = cfg["q"][:, h:h + 1], cfg["k"], cfg["v"]
        rm, _, _ = S.select_blocks(sub_q, sub_k, cfg["n_valid"], cfg["Bq"], cfg["Bk"], True, cfg["topk"],
                                   cfg["ratio_num"], cfg["ratio_den"], cfg["sink_tiles"], cfg["local_tiles"])
        assert np.array_equal(mask[:, h:h + 1], rm), f"head {h}: mask differs"
    ops = A.prepare_operands(sub_q, sub_k, sub_v, cfg["n_valid"])
    ro, rl = A.attn_mixed_ref(sub_q, sub_k, sub_v, cfg["n_valid"], cfg["Bq"], cfg["Bk"], True,
                              mask=rm, qtiles=tiles, ops=ops)
    _check(out[:, 1:2], lse[:, 1:2], ro, rl, rows=rows)


GROUP_CASES = [
    # D, Bq, causal, N, n_valid, Hq, Hkv, n_lines, sink_tiles
    (128, 128, True, 768, 700, 8, 2, 0, 1),    # G = 4, 32 rows per head and workgroup
    (64, 64, False, 512, 450, 4, 2, 0, 1),     # G = 2, 64 rows per head
    (128, 64, True, 512, 333, 4, 1, 0, 1),     # G = 4, 64-row selection tiles
    (128, 128, True, 1024, 1024, 8, 4, 4, 1),  # G = 2 with shared vertical lines
    (64, 128, True, 1024, 1000, 8, 2, 6, 1),   # G = 4, head_dim 64, lines, ragged
    # 64-row selection tiles, no forced sink tile, no padding: a 128-row
    # workgroup of the per-head launch spans two mask rows, so it can take
    # the masked path for chunks that the grouped launch runs unmasked
    (128, 64, True, 1024, 1024, 4, 2, 0, 0),
    (64, 64, False, 768, 768, 8, 2, 0, 0),
]


@pytest.mark.parametrize("case", GROUP_CASES)
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_group_heads_equal_the_per_head_kernel(case, mode):
    """One workgroup serving the G query heads of a kv group (MXQ_GROUP_HEADS)
    under masks and line lists shared by the group (selection with
    group_shared): outputs and lse bit-identical to the per-head kernel, whose
    rows do the same arithmetic; then the first head against the oracle."""
    mxq = gpu_or_skip()
    import torch

    D, Bq, causal, N, nv, Hq, Hkv, n_lines, sink_tiles = case
    rng = np.random.default_rng(D + N + nv + Hq)
    q = rng.standard_normal((1, Hq, N, D)).astype(np.float32) * 1.5
    k = rng.standard_normal((1, Hkv, N, D)).astype(np.float32)
    v = rng.standard_normal((1, Hkv, N, D)).astype(np.float32)
    k[:, :, 0] *= 8
    for t in (q, k, v):
        t[:, :, nv:] = 0
    qb, kb, vb = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    qd, kd, vd = bf16_dev(qb), bf16_dev(kb), bf16_dev(vb)
    shape = mxq.Shape(1, Hq, Hkv, N, nv, D, Bq, 64, causal)
    mask = None
    if mode == mxq.MXQ_MIXED:
        mask, _, _ = mxq.attn_select_blocks(qd, kd, shape, topk=-1, ratio=(10, 100), sink_tiles=sink_tiles,
                                            local_tiles=1, group_shared=True)
    lines = mxq.attn_select_lines(qd, kd, shape, n_lines, 1, group_shared=True)[0] if n_lines else None
    ops = mxq.prepare_prefill(qd, kd, vd, nv, mode, lines=bool(n_lines))
    o1, l1 = mxq.attn_mixed_fwd(ops, mask, shape, mode=mode, lines=lines)
    o2, l2 = mxq.attn_mixed_fwd(ops, mask, shape, mode=mode, lines=lines, group_heads=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    # the first and last heads against the oracle, each with its own mask row
    # and line list (the shared ones)
    G = Hq // Hkv
    for h in (0, Hq - 1):
        hs = slice(h, h + 1)
        ks = slice(h // G, h // G + 1)
        rm = u32(mask)[:, hs] if mask is not None else None
        rlines = lines.cpu().numpy()[:, hs] if lines is not None else None
        ro, rl = A.attn_mixed_ref(qb[:, hs], kb[:, ks], vb[:, ks], nv, Bq, 64, causal, mask=rm, mode=mode,
                                  lines=rlines)
        _check(o2.cpu().numpy()[:, hs], l2.cpu().numpy()[:, hs], ro, rl)


def test_group_heads_host_checks():
    mxq = gpu_or_skip()
    import torch

    q = torch.zeros((1, 2, 512, 128), dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros((1, 2, 512, 128), dtype=torch.bfloat16, device="cuda:0")
    ops = mxq.prepare_prefill(q, k, k, 512, mxq.MXQ_ALL_LOWBIT)
    with pytest.raises(mxq.MxqError, match="GROUP_HEADS"):  # G = 1
        mxq.attn_mixed_fwd(ops, None, mxq.Shape(1, 2, 2, 512, 512, 128, 128, 64, True), mode=mxq.MXQ_ALL_LOWBIT,
                           group_heads=True)
    q2 = torch.zeros((1, 4, 256, 128), dtype=torch.bfloat16, device="cuda:0")
    k2 = torch.zeros((1, 2, 256, 128), dtype=torch.bfloat16, device="cuda:0")
    ops2 = mxq.prepare_prefill(q2, k2, k2, 256, mxq.MXQ_ALL_LOWBIT)
    with pytest.raises(mxq.MxqError, match="GROUP_HEADS"):  # N <= 256
        mxq.attn_mixed_fwd(ops2, None, mxq.Shape(1, 4, 2, 256, 256, 128, 128, 64, True), mode=mxq.MXQ_ALL_LOWBIT,
                           group_heads=True)
