"""GPU parity: attn_select_blocks masks, counts and scores are bit-exact."""

import numpy as np
import torch
import pytest

from gpu_helpers import bf16_dev, gpu_or_skip, u32
import mxq_inputs
from oracle import select as S
from oracle.formats import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def _run(mxq, cfg, want_scores=True):
    shape = mxq.Shape(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["n_valid"], cfg["D"], cfg["Bq"],
                      cfg["Bk"], cfg["causal"])
    mask, nfp, sc = mxq.attn_select_blocks(bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), shape, topk=cfg["topk"],
                                           ratio=(cfg["ratio_num"], cfg["ratio_den"]),
                                           sink_tiles=cfg["sink_tiles"], local_tiles=cfg["local_tiles"],
                                           want_scores=want_scores)
    return u32(mask), nfp.cpu().numpy(), (sc.cpu().numpy() if sc is not None else None)


def _ref(cfg):
    return S.select_blocks(cfg["q"], cfg["k"], cfg["n_valid"], cfg["Bq"], cfg["Bk"], cfg["causal"], cfg["topk"],
                           cfg["ratio_num"], cfg["ratio_den"], cfg["sink_tiles"], cfg["local_tiles"])


@pytest.mark.parametrize("name", ["tiny", "llama8b", "vit"])
def test_configured_workloads_bit_exact(name):
    mxq = gpu_or_skip()
    # vit: a 16-image batch of the same recipe (images are independent)
    cfg = mxq_inputs.make_prefill(name, **({"B": 16} if name == "vit" else {}))
    mask, nfp, sc = _run(mxq, cfg)
    rm, rn, rs = _ref(cfg)
    assert np.array_equal(sc.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(mask, rm)
    assert np.array_equal(nfp, rn)


def test_long32k_counts_and_sampled_rows():
    mxq = gpu_or_skip()
    cfg = mxq_inputs.make_prefill("long32k")
    mask, nfp, _ = _run(mxq, cfg, want_scores=False)
    assert int(nfp.sum()) == 32 * 4933
    # full oracle on 4 of the 32 heads (one per kv group pair)
    for h in (0, 9, 18, 31):
        sub = dict(cfg, q=cfg["q"][:, h:h + 1], k=cfg["k"][:, h // 4:h // 4 + 1], Hq=1, Hkv=1)
        rm, rn, _ = _ref(sub)
        assert np.array_equal(mask[:, h:h + 1], rm)


@pytest.mark.parametrize("causal", [False, True])
def test_ragged_gqa_and_constructed_ties(causal):
    mxq = gpu_or_skip()
    rng = np.random.default_rng(4)
    N, D = 1024, 64
    q = rng.standard_normal((2, 4, N, D)).astype(np.float32)
    k = rng.standard_normal((2, 2, N, D)).astype(np.float32)
    k[:, :, 256:512] = k[:, :, 0:256]          # repeated key tiles -> equal scores
    k[1] = np.round(k[1])                       # coarse values -> more ties
    q[1] = 1.0
    cfg = dict(B=2, Hq=4, Hkv=2, N=N, n_valid=1000, D=D, Bq=128, Bk=64, causal=causal, topk=-1,
               ratio_num=30, ratio_den=100, sink_tiles=1, local_tiles=2,
               q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k))
    mask, nfp, sc = _run(mxq, cfg)
    rm, rn, rs = _ref(cfg)
    assert np.array_equal(sc.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(mask, rm)
    assert np.array_equal(nfp, rn)


@pytest.mark.parametrize("B,Hq,Hkv,N,Bq,heuristic", [(4, 64, 16, 1152, 128, 0), (1, 8, 2, 65664, 128, 0),
                                                     (3, 64, 16, 1152, 64, 1)])
def test_row_groups_ragged_and_wide(B, Hq, Hkv, N, Bq, heuristic):
    """A workgroup scores and selects up to 8 query tiles of one head: 8 when a
    score row fits 4 KB of LDS and the launch keeps at least 512 workgroups.
    Shapes that run those groups with a partial last one: 9 query tiles (8 +
    1), 513 tiles of 1026 key tiles each (7 per group: 73 x 7 + 2), 18 tiles
    under the max-pooled heuristic (8 + 8 + 2).  Scores, masks and counts
    bit-exact."""
    mxq = gpu_or_skip()
    rng = np.random.default_rng(N + Bq + Hq)
    nv = N - 64 - 3
    q = rng.standard_normal((B, Hq, N, 64)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, 64)).astype(np.float32)
    q[:, :, nv:] = 0
    k[:, :, nv:] = 0
    qb, kb = f32_to_bf16_bits(q), f32_to_bf16_bits(k)
    del q, k
    shape = mxq.Shape(B, Hq, Hkv, N, nv, 64, Bq, 64, True)
    mask, nfp, sc = mxq.attn_select_blocks(bf16_dev(qb), bf16_dev(kb), shape, topk=-1, ratio=(5, 100),
                                           sink_tiles=1, local_tiles=2, want_scores=True, heuristic=heuristic)
    rm, rn, rs = S.select_blocks(qb, kb, nv, Bq, 64, True, -1, 5, 100, 1, 2,
                                 heuristic="maxkey" if heuristic else "mean")
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(u32(mask), rm)
    assert np.array_equal(nfp.cpu().numpy(), rn)


def test_deterministic():
    mxq = gpu_or_skip()
    cfg = mxq_inputs.make_prefill("llama8b")
    a = _run(mxq, cfg)
    b = _run(mxq, cfg)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


# A zero budget (topk = 0, or a ratio of 0) chooses only the forced tiles: without
# a score request the library skips the tile means and scores.  Masks and counts
# must equal the oracle's and the scored path's.
ZERO_BUDGET_CASES = [
    # B, Hq, Hkv, N, D, n_valid, Bq, causal, topk, ratio_num, sink_tiles, local_tiles
    (2, 4, 2, 1024, 128, 1000, 128, True, 0, 5, 1, 1),
    (3, 6, 6, 256, 64, 197, 64, False, -1, 0, 0, 0),     # ViT-shaped: nothing promoted
    (1, 4, 1, 640, 64, 577, 64, True, -1, 0, 2, 3),
    (1, 2, 2, 512, 128, 130, 128, False, 0, 0, 1, 0),
]


@pytest.mark.parametrize("case", ZERO_BUDGET_CASES)
def test_zero_budget_without_scores(case):
    mxq = gpu_or_skip()
    B, Hq, Hkv, N, D, nv, Bq, causal, topk, rnum, sink, local = case
    rng = np.random.default_rng(N + nv + Hq)
    q = rng.standard_normal((B, Hq, N, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    q[:, :, nv:] = 0
    k[:, :, nv:] = 0
    cfg = dict(B=B, Hq=Hq, Hkv=Hkv, N=N, n_valid=nv, D=D, Bq=Bq, Bk=64, causal=causal, topk=topk,
               ratio_num=rnum, ratio_den=100, sink_tiles=sink, local_tiles=local,
               q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k))
    mask, nfp, sc = _run(mxq, cfg, want_scores=False)
    assert sc is None
    rm, rn, _ = _ref(cfg)
    assert np.array_equal(mask, rm)
    assert np.array_equal(nfp, rn)
    mask2, nfp2, _ = _run(mxq, cfg, want_scores=True)
    assert np.array_equal(mask2, rm)
    assert np.array_equal(nfp2, rn)


# mxq_prefill_operands_means: the quantiser's tile means equal the oracle's (bit
# for bit), and selecting from them equals attn_select_blocks on the same inputs.
MEANS_CASES = [
    ("llama8b", {}),
    ("tiny", {}),
    ("vit", {"B": 8}),
]


@pytest.mark.parametrize("name,over", MEANS_CASES)
def test_select_from_fused_means(name, over):
    mxq = gpu_or_skip()
    cfg = mxq_inputs.make_prefill(name, **over)
    shape = mxq.Shape(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["n_valid"], cfg["D"], cfg["Bq"],
                      cfg["Bk"], cfg["causal"])
    q, k, v = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
    ops, qm, km = mxq.prepare_prefill_means(q, k, v, shape)
    rqm, rkm = S.pooled_means(cfg["q"], cfg["k"], cfg["n_valid"], cfg["Bq"], cfg["Bk"])
    assert np.array_equal(qm.cpu().numpy().view(np.uint32), rqm.view(np.uint32))
    assert np.array_equal(km.cpu().numpy().transpose(0, 1, 3, 2).view(np.uint32), rkm.view(np.uint32))
    ref = mxq.prepare_prefill(q, k, v, cfg["n_valid"])
    for f in ("q_codes", "q_scales", "k_codes", "k_scales", "v_codes", "v_scales", "v_f16t"):
        assert torch.equal(getattr(ops, f), getattr(ref, f)), f
    topk, ratio = cfg["topk"], (cfg["ratio_num"], cfg["ratio_den"])
    if topk == 0 or (topk < 0 and ratio[0] == 0):
        topk, ratio = -1, (5, 100)  # a budget that needs the scores
    m1, n1, s1 = mxq.attn_select_blocks_means(qm, km, shape, topk=topk, ratio=ratio, sink_tiles=cfg["sink_tiles"],
                                              local_tiles=cfg["local_tiles"], want_scores=True)
    m2, n2, s2 = mxq.attn_select_blocks(q, k, shape, topk=topk, ratio=ratio, sink_tiles=cfg["sink_tiles"],
                                        local_tiles=cfg["local_tiles"], want_scores=True)
    assert torch.equal(m1, m2) and torch.equal(n1, n2)
    assert np.array_equal(s1.cpu().numpy().view(np.uint32), s2.cpu().numpy().view(np.uint32))
    rm, rn, rs = S.select_blocks(cfg["q"], cfg["k"], cfg["n_valid"], cfg["Bq"], cfg["Bk"], cfg["causal"], topk,
                                 ratio[0], ratio[1], cfg["sink_tiles"], cfg["local_tiles"])
    assert np.array_equal(u32(m1), rm)


def test_fused_means_ragged_gqa():
    mxq = gpu_or_skip()
    rng = np.random.default_rng(11)
    B, Hq, Hkv, N, D, nv = 2, 6, 2, 640, 64, 577
    q = rng.standard_normal((B, Hq, N, D)).astype(np.float32) * 2
    k = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, N, D)).astype(np.float32)
    for t in (q, k, v):
        t[:, :, nv:] = 0
    qb, kb, vb = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    for Bq in (64, 128):
        shape = mxq.Shape(B, Hq, Hkv, N, nv, D, Bq, 64, True)
        ops, qm, km = mxq.prepare_prefill_means(bf16_dev(qb), bf16_dev(kb), bf16_dev(vb), shape)
        rqm, rkm = S.pooled_means(qb, kb, nv, Bq, 64)
        assert np.array_equal(qm.cpu().numpy().view(np.uint32), rqm.view(np.uint32))
        assert np.array_equal(km.cpu().numpy().transpose(0, 1, 3, 2).view(np.uint32), rkm.view(np.uint32))


@pytest.mark.parametrize("fused", [False, True])
def test_group_shared_masks_bit_exact(fused):
    """One mask per kv group (reading R35), from bf16 Q/K and from the fused
    quantiser's tile means: bit-exact against the oracle, every head of a
    group identical; and the attention on it within 5e-3."""
    mxq = gpu_or_skip()
    from oracle import attention as A

    cfg = mxq_inputs.make_prefill("llama8b", N=2048, n_valid=2000, Hq=8, Hkv=2)
    q, k, v = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
    shape = mxq.Shape(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["n_valid"], cfg["D"], cfg["Bq"], cfg["Bk"],
                      cfg["causal"])
    if fused:
        ops, qm, km = mxq.prepare_prefill_means(q, k, v, shape)
        mask, nfp, sc = mxq.attn_select_blocks_means(qm, km, shape, topk=-1, ratio=(10, 100), sink_tiles=1,
                                                     local_tiles=1, want_scores=True, group_shared=True)
    else:
        ops = mxq.prepare_prefill(q, k, v, cfg["n_valid"])
        mask, nfp, sc = mxq.attn_select_blocks(q, k, shape, topk=-1, ratio=(10, 100), sink_tiles=1, local_tiles=1,
                                               want_scores=True, group_shared=True)
    rm, rn, rs = S.select_blocks(cfg["q"], cfg["k"], cfg["n_valid"], cfg["Bq"], cfg["Bk"], True, -1, 10, 100, 1, 1,
                                 group_shared=True)
    got = u32(mask)
    assert np.array_equal(got, rm) and np.array_equal(nfp.cpu().numpy(), rn)
    assert np.array_equal(sc.cpu().numpy(), rs)
    for h in range(1, 4):
        assert np.array_equal(got[:, h], got[:, 0]) and np.array_equal(got[:, 4 + h], got[:, 4])
    out, lse = mxq.attn_mixed_fwd(ops, mask, shape)
    for h in (0, 5):
        kv = h // 4
        ro, rl = A.attn_mixed_ref(cfg["q"][:, h:h + 1], cfg["k"][:, kv:kv + 1], cfg["v"][:, kv:kv + 1],
                                  cfg["n_valid"], 128, 64, True, mask=rm[:, h:h + 1], qtiles=[0, 7, 15])
        rows = np.concatenate([np.arange(t * 128, (t + 1) * 128) for t in (0, 7, 15)])
        o = out.cpu().numpy()[:, h:h + 1][..., rows, :]
        assert np.abs(o - ro[..., rows, :]).max() <= 5e-3


def test_maxkey_heuristic_bit_exact():
    """Max-pooled key logits (reading R37): scores, masks and counts bit-exact
    against the oracle (causal, ragged, GQA), and the means-only entry point
    refuses the heuristic."""
    mxq = gpu_or_skip()
    cfg = mxq_inputs.make_prefill("llama8b", N=1024, n_valid=1000, Hq=8, Hkv=2)
    q, k = bf16_dev(cfg["q"]), bf16_dev(cfg["k"])
    shape = mxq.Shape(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["n_valid"], cfg["D"], cfg["Bq"], cfg["Bk"],
                      cfg["causal"])
    for want_scores in (True, False):
        mask, nfp, sc = mxq.attn_select_blocks(q, k, shape, topk=-1, ratio=(10, 100), sink_tiles=1, local_tiles=1,
                                               want_scores=want_scores, heuristic=1)
        rm, rn, rs = S.select_blocks(cfg["q"], cfg["k"], cfg["n_valid"], cfg["Bq"], cfg["Bk"], True, -1, 10, 100,
                                     1, 1, heuristic="maxkey")
        assert np.array_equal(u32(mask), rm) and np.array_equal(nfp.cpu().numpy(), rn)
        if want_scores:
            assert np.array_equal(sc.cpu().numpy(), rs)
    ops, qm, km = mxq.prepare_prefill_means(q, k, bf16_dev(cfg["v"]), shape)
    sp = mxq.SelectParams(-1, 10, 100, 1, 1, 0, 1)
    st = mxq.load_library().attn_select_blocks_means(mxq._ptr(qm), mxq._ptr(km), mxq.ctypes.byref(shape.c()),
                                                     mxq.ctypes.byref(sp), mxq._ptr(mask), None, None, mxq._stream())
    assert st == mxq.MXQ_EUNSUPPORTED
