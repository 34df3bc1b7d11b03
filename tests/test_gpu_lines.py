"""GPU parity for vertical-line tokens (HyQuant, summary and abstract):
attn_select_lines bit-exact against the oracle, and attn_mixed_fwd with lines
within max-abs 5e-3 of the oracle."""

import numpy as np
import pytest

from gpu_helpers import bf16_dev, gpu_or_skip, u32
import mxq_inputs
from oracle import attention as A
from oracle import select as S
from oracle.formats import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

TOL = 5e-3


def _inputs(B, Hq, Hkv, N, D, nv, seed, plant=()):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    u = rng.standard_normal(D).astype(np.float32)
    u /= np.linalg.norm(u)
    q += 1.5 * u                      # a shared query direction ...
    for j in plant:                   # ... that planted keys line up with
        k[:, :, j] = 5.0 * u + 0.3 * k[:, :, j]
    k[:, :, 0] *= 6.0                 # a large-norm sink key
    for t in (q, k, v):
        t[:, :, nv:] = 0
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


SELECT_CASES = [
    # B, Hq, Hkv, N, D, n_valid, Bq, n_lines, sink, shared
    (1, 4, 2, 512, 64, 500, 64, 8, 1, False),
    (1, 4, 2, 512, 64, 500, 64, 8, 1, True),
    (2, 4, 1, 1024, 128, 1000, 128, 16, 0, False),
    (2, 8, 2, 640, 128, 577, 128, 16, 3, True),
    (1, 2, 2, 128, 64, 5, 64, 8, 1, False),       # fewer valid keys than lines
    (3, 3, 3, 256, 64, 197, 64, 1, 1, False),     # ViT-shaped: the CLS token only
]


@pytest.mark.parametrize("case", SELECT_CASES)
def test_select_lines_bit_exact(case):
    mxq = gpu_or_skip()
    B, Hq, Hkv, N, D, nv, Bq, n_lines, sink, shared = case
    q, k, _ = _inputs(B, Hq, Hkv, N, D, nv, seed=N + D + n_lines, plant=(7, N // 3, nv - 1))
    shape = mxq.Shape(B, Hq, Hkv, N, nv, D, Bq, 64, True)
    lines, scores = mxq.attn_select_lines(bf16_dev(q), bf16_dev(k), shape, n_lines, sink, group_shared=shared,
                                          want_scores=True)
    rl, rs = S.select_lines(q, k, nv, Bq, n_lines, sink, group_shared=shared)
    assert np.array_equal(scores.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(lines.cpu().numpy(), rl)


def test_select_lines_llama8b_full_size():
    mxq = gpu_or_skip()
    cfg = mxq_inputs.make_prefill("llama8b")
    shape = mxq.Shape(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["n_valid"], cfg["D"], cfg["Bq"], cfg["Bk"],
                      cfg["causal"])
    q, k = bf16_dev(cfg["q"]), bf16_dev(cfg["k"])
    for shared in (False, True):
        lines, _ = mxq.attn_select_lines(q, k, shape, 16, 1, group_shared=shared)
        rl, _ = S.select_lines(cfg["q"], cfg["k"], cfg["n_valid"], cfg["Bq"], 16, 1, group_shared=shared)
        assert np.array_equal(lines.cpu().numpy(), rl)


def _run(mxq, q, k, v, shape, mode, mask, lines_np):
    import torch

    ops = mxq.prepare_prefill(bf16_dev(q), bf16_dev(k), bf16_dev(v), shape.n_valid, mode, lines=True)
    mask_t = torch.from_numpy(np.ascontiguousarray(mask).view(np.int32)).to("cuda:0") if mask is not None else None
    lines_t = torch.from_numpy(np.ascontiguousarray(lines_np, dtype=np.int32)).to("cuda:0")
    out, lse = mxq.attn_mixed_fwd(ops, mask_t, shape, mode=mode, lines=lines_t)
    return out.cpu().numpy(), lse.cpu().numpy()


def _check(out, lse, ro, rl):
    err = np.abs(out - ro)
    assert np.all(np.isfinite(out))
    assert err.max() <= TOL, f"max-abs {err.max():.3e}"
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - rl[fin]).max() <= TOL


ATTN_CASES = [
    # D, Bq, causal, N, n_valid, Hq, Hkv, n_lines, sink
    (64, 64, True, 512, 500, 2, 1, 8, 1),
    (64, 128, False, 384, 300, 4, 2, 16, 2),
    (128, 128, True, 768, 768, 4, 1, 16, 1),
    (128, 64, False, 256, 197, 2, 2, 1, 1),
]


@pytest.mark.parametrize("case", ATTN_CASES)
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_attention_with_lines(case, mode):
    mxq = gpu_or_skip()
    D, Bq, causal, N, nv, Hq, Hkv, n_lines, sink = case
    q, k, v = _inputs(1, Hq, Hkv, N, D, nv, seed=D + N + nv + mode, plant=(3, 130, 131, nv - 2))
    shape = mxq.Shape(1, Hq, Hkv, N, nv, D, Bq, 64, causal)
    lines, _ = S.select_lines(q, k, nv, Bq, n_lines, sink)
    mask = None
    if mode == 0:
        mask, _, _ = S.select_blocks(q, k, nv, Bq, 64, causal, -1, 10, 100, 1, 1)
    out, lse = _run(mxq, q, k, v, shape, mode, mask, lines)
    ro, rl = A.attn_mixed_ref(q, k, v, nv, Bq, 64, causal, mask=mask, mode=mode, lines=lines)
    _check(out, lse, ro, rl)
    assert np.all(out[:, :, nv:] == 0) and np.all(np.isneginf(lse[:, :, nv:]))


def test_line_list_rule_and_spread_lines():
    """Lines in every 128-key chunk (no chunk takes the fast path), and a messy
    list: repeats, out-of-order and out-of-range entries are ignored."""
    mxq = gpu_or_skip()
    N, nv, D = 1024, 1000, 128
    q, k, v = _inputs(1, 2, 1, N, D, nv, seed=21)
    shape = mxq.Shape(1, 2, 1, N, nv, D, 128, 64, True)
    spread = np.array([[list(range(0, 1024, 128)) + [5, 1001, -1, 999, 999, 4000, 2000, -7]] * 2], dtype=np.int32)
    spread[0, 1] = [40, 40, 39, 900, 1100, 950, -1, -1, 960, 961, 962, 963, 964, 2, 1, 0]
    mask, _, _ = S.select_blocks(q, k, nv, 128, 64, True, -1, 5, 100, 1, 1)
    out, lse = _run(mxq, q, k, v, shape, 0, mask, spread)
    ro, rl = A.attn_mixed_ref(q, k, v, nv, 128, 64, True, mask=mask, lines=spread)
    _check(out, lse, ro, rl)


def test_llama8b_with_lines_sampled():
    """Full-size Llama-8B-shaped causal prefill with 16 lines per head (the
    sink token forced) on top of the 5% tiles; sampled (head, query tile)
    pairs against the oracle."""
    mxq = gpu_or_skip()
    import torch

    cfg = mxq_inputs.make_prefill("llama8b")
    shape = mxq.Shape(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["n_valid"], cfg["D"], cfg["Bq"], cfg["Bk"],
                      cfg["causal"])
    q, k, v = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
    mask, _, _ = mxq.attn_select_blocks(q, k, shape, topk=-1, ratio=(5, 100), sink_tiles=1, local_tiles=1)
    lines, _ = mxq.attn_select_lines(q, k, shape, 16, 1)
    ops = mxq.prepare_prefill(q, k, v, cfg["n_valid"])
    out, lse = mxq.attn_mixed_fwd(ops, mask, shape, lines=lines)
    out, lse, mask, lines = out.cpu().numpy(), lse.cpu().numpy(), u32(mask), lines.cpu().numpy()
    torch.cuda.synchronize()
    G = cfg["Hq"] // cfg["Hkv"]
    for h in (0, 21):
        kv = h // G
        sub_q, sub_k, sub_v = cfg["q"][:, h:h + 1], cfg["k"][:, kv:kv + 1], cfg["v"][:, kv:kv + 1]
        rm, _, _ = S.select_blocks(sub_q, sub_k, cfg["n_valid"], 128, 64, True, -1, 5, 100, 1, 1)
        rlines, _ = S.select_lines(sub_q, sub_k, cfg["n_valid"], 128, 16, 1)
        assert np.array_equal(mask[:, h:h + 1], rm) and np.array_equal(lines[:, h:h + 1], rlines)
        tiles = [0, 9, 40, 63]
        ro, rl = A.attn_mixed_ref(sub_q, sub_k, sub_v, cfg["n_valid"], 128, 64, True, mask=rm,
                                  qtiles=tiles, lines=rlines)
        rows = np.concatenate([np.arange(t * 128, (t + 1) * 128) for t in tiles])
        _check(out[:, h:h + 1][..., rows, :], lse[:, h:h + 1][..., rows], ro[..., rows, :], rl[..., rows])


# Lists with no room for a scored key (n_lines <= sink_tokens) or no key left to
# score (n_valid <= sink_tokens): without a score request the library writes the
# first keys directly; the lists must equal the oracle's and the scored path's.
SINK_ONLY_CASES = [
    # B, Hq, Hkv, N, D, n_valid, Bq, n_lines, sink
    (3, 3, 3, 256, 64, 197, 64, 1, 1),      # ViT-shaped: the CLS token only
    (2, 4, 2, 512, 128, 500, 128, 4, 6),    # more sink tokens than lines
    (1, 2, 2, 128, 64, 3, 64, 8, 5),        # fewer valid keys than sink tokens
]


@pytest.mark.parametrize("case", SINK_ONLY_CASES)
def test_select_lines_sink_only_without_scores(case):
    mxq = gpu_or_skip()
    B, Hq, Hkv, N, D, nv, Bq, n_lines, sink = case
    q, k, _ = _inputs(B, Hq, Hkv, N, D, nv, seed=N + n_lines + sink)
    shape = mxq.Shape(B, Hq, Hkv, N, nv, D, Bq, 64, False)
    lines, scores = mxq.attn_select_lines(bf16_dev(q), bf16_dev(k), shape, n_lines, sink)
    assert scores is None
    rl, _ = S.select_lines(q, k, nv, Bq, n_lines, sink)
    assert np.array_equal(lines.cpu().numpy(), rl)
    scored, _ = mxq.attn_select_lines(bf16_dev(q), bf16_dev(k), shape, n_lines, sink, want_scores=True)
    assert np.array_equal(scored.cpu().numpy(), rl)


@pytest.mark.parametrize("case", [
    # D, Bq, causal, N, n_valid, Hq, Hkv, n_lines, sink
    (64, 64, False, 256, 197, 3, 3, 1, 1),       # the short-sequence kernel, ViT-shaped
    (128, 128, False, 256, 200, 2, 1, 4, 1),
    (64, 64, True, 512, 500, 2, 1, 8, 1),        # the pipelined kernel
    (128, 128, True, 768, 700, 4, 2, 16, 2),
])
def test_lines_with_bf16_v_when_nothing_is_promoted(case):
    """A step whose mask promotes no tile needs no fp16 copy of V: the line
    keys' V values come from bf16 V, rounded to fp16 in the kernel.  The
    output equals the one computed with the fp16 copy bit for bit, and the
    oracle within the tolerance (values in fp16's subnormal range included)."""
    mxq = gpu_or_skip()
    import torch

    D, Bq, causal, N, nv, Hq, Hkv, n_lines, sink = case
    q, k, v = _inputs(1, Hq, Hkv, N, D, nv, seed=7 * N + D, plant=(2, nv // 2))
    # tiny values at the line keys: their fp16 rounding goes through subnormals
    vf = bf16_bits_to_f32(v)
    vf[:, :, 0, :4] = [3e-5, -7.1e-6, 2.9e-8, 6.0e-8]
    vf[:, :, nv // 2, :2] = [1.3e-7, -5.5e-6]
    v = f32_to_bf16_bits(vf)
    shape = mxq.Shape(1, Hq, Hkv, N, nv, D, Bq, 64, causal)
    lines, _ = S.select_lines(q, k, nv, Bq, n_lines, sink)
    mask, _, _ = S.select_blocks(q, k, nv, Bq, 64, causal, 0, 0, 1, 0, 0)
    assert not np.any(mask)
    mask_t = torch.from_numpy(np.ascontiguousarray(mask).view(np.int32)).to("cuda:0")
    lines_t = torch.from_numpy(np.ascontiguousarray(lines, dtype=np.int32)).to("cuda:0")
    qd, kd, vd = bf16_dev(q), bf16_dev(k), bf16_dev(v)
    outs = []
    for promoted in (True, False):
        ops = mxq.prepare_prefill(qd, kd, vd, nv, 0, lines=True, promoted=promoted)
        assert (ops.v_f16t is None) == (not promoted)
        out, lse = mxq.attn_mixed_fwd(ops, mask_t, shape, mode=0, lines=lines_t)
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    (o1, l1), (o2, l2) = outs
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))
    ro, rl = A.attn_mixed_ref(q, k, v, nv, Bq, 64, causal, mask=mask, mode=0, lines=lines)
    _check(o2, l2, ro, rl)
