"""GPU parity: attn_mixed_fwd against the oracle (max-abs <= 5e-3, fp32 out)."""

import numpy as np
import pytest

from gpu_helpers import bf16_dev, gpu_or_skip, u32
import mxq_inputs
from oracle import attention as A
from oracle import select as S
from oracle.formats import f32_to_bf16_bits

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
        ops = A.prepare_operands(sub_q, sub_k, sub_v, cfg["n_valid"])
        tiles = [0, 1, 17, 40, 63]
        ro, rl = A.attn_mixed_ref(sub_q, sub_k, sub_v, cfg["n_valid"], cfg["Bq"], cfg["Bk"], True,
                                  mask=mask[:, h:h + 1], qtiles=tiles, ops=ops)
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
    for b, h in ((0, 0), (3, 7), (7, 11)):
        ro, rl = A.attn_mixed_ref(cfg["q"][b:b + 1, h:h + 1], cfg["k"][b:b + 1, h:h + 1], cfg["v"][b:b + 1, h:h + 1],
                                  cfg["n_valid"], 64, 64, False, mask=mask[b:b + 1, h:h + 1],
                                  lines=lines[b:b + 1, h:h + 1])
        _check(out[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], ro, rl)


def test_deterministic_and_bf16_output():
    mxq = gpu_or_skip()
    cfg = mxq_inputs.make_prefill("tiny")
    o1, l1, _ = _gpu_prefill(mxq, cfg, 0)
    o2, l2, _ = _gpu_prefill(mxq, cfg, 0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    ob, _, _ = _gpu_prefill(mxq, cfg, 0, out_dtype=1)
    # bf16 store of the same fp32 result: relative error <= 2^-9
    assert np.all(np.abs(ob - o1) <= np.abs(o1) * 2.0 ** -8 + 1e-30)


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
    ro, rl = A.attn_mixed_ref(cfg["q"], cfg["k"], cfg["v"], cfg["n_valid"], 128, 64, True,
                              mask=u32(mask) if mask is not None else None, mode=mode, rotate=True)
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
