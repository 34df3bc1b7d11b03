"""GPU: the quality properties behind the promotion curve (bench.py --only quality).

Against exact softmax attention in float64 (numpy, on the host):
  - all-FP16 mode is exact up to fp16 P rounding and fp32 accumulation;
  - all-low-bit mode carries a visible MXFP4/FP8 error;
  - with a large-norm sink key, promoting the forced sink and window tiles
    (ThriftAttention's tiles in FP16, HyQuant's sink and local tiles) removes
    most of that error, and the 5% selection on top does not add to it.
"""

import math

import numpy as np
import pytest

from gpu_helpers import bf16_dev, gpu_or_skip
import mxq_inputs

pytestmark = pytest.mark.gpu


def _bits_to_f64(b):
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _exact(cfg, rows):
    """float64 softmax attention of the sampled rows, [Hq, rows, D]."""
    q, k, v = _bits_to_f64(cfg["q"])[0], _bits_to_f64(cfg["k"])[0], _bits_to_f64(cfg["v"])[0]
    G = cfg["Hq"] // cfg["Hkv"]
    out = []
    for h in range(cfg["Hq"]):
        s = q[h, rows] @ k[h // G].T / math.sqrt(cfg["D"])
        if cfg["causal"]:
            s = np.where(np.arange(cfg["N"])[None, :] > rows[:, None], -np.inf, s)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out.append((p / p.sum(axis=1, keepdims=True)) @ v[h // G])
    return np.stack(out)


def _rel(got, ref):
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def test_promotion_curve_properties():
    mxq = gpu_or_skip()
    cfg = mxq_inputs.make_prefill("llama8b", Hq=4, Hkv=1, N=1024, n_valid=1024, outliers=False)  # sink key x8
    rows = np.linspace(64, cfg["N"] - 1, 24).round().astype(np.int64)
    ref = _exact(cfg, rows)
    q, k, v = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
    shape = mxq.Shape(1, cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["N"], cfg["D"], cfg["Bq"], cfg["Bk"], cfg["causal"])
    ops = mxq.prepare_prefill(q, k, v, cfg["N"])

    def run(mode, ratio_num=None):
        mask = None
        if mode == mxq.MXQ_MIXED:
            mask, _, _ = mxq.attn_select_blocks(q, k, shape, topk=-1, ratio=(ratio_num, 100),
                                                sink_tiles=cfg["sink_tiles"], local_tiles=cfg["local_tiles"])
        out, _ = mxq.attn_mixed_fwd(ops, mask, shape, mode=mode, out_dtype=mxq.MXQ_OUT_F32)
        return out.cpu().numpy()[0][:, rows].astype(np.float64)

    e_fp16 = _rel(run(mxq.MXQ_ALL_FP16), ref)
    e_low = _rel(run(mxq.MXQ_ALL_LOWBIT), ref)
    e_forced = _rel(run(mxq.MXQ_MIXED, 0), ref)
    e_5 = _rel(run(mxq.MXQ_MIXED, 5), ref)
    assert e_fp16 < 1e-3, e_fp16
    assert e_low > 20 * e_fp16, (e_low, e_fp16)
    assert e_forced < 0.25 * e_low, (e_forced, e_low)
    assert e_5 <= e_forced * 1.05, (e_5, e_forced)


def test_rotation_helps_where_promotion_cannot():
    """Outlier channels x20 in Q and K: a few promoted tiles barely help (the
    near-argmax keys are spread over every tile), while rotating Q and K by the
    Walsh-Hadamard matrix before MXFP4 spreads the outliers over each block
    and cuts the all-low-bit error severalfold."""
    mxq = gpu_or_skip()
    cfg = mxq_inputs.make_prefill("llama8b", Hq=4, Hkv=1, N=1024, n_valid=1024)
    rows = np.linspace(64, cfg["N"] - 1, 24).round().astype(np.int64)
    ref = _exact(cfg, rows)
    q, k, v = bf16_dev(cfg["q"]), bf16_dev(cfg["k"]), bf16_dev(cfg["v"])
    shape = mxq.Shape(1, cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["N"], cfg["D"], cfg["Bq"], cfg["Bk"], cfg["causal"])

    def run(rotate):
        ops = mxq.prepare_prefill(q, k, v, cfg["N"], mode=mxq.MXQ_ALL_LOWBIT, rotate=rotate)
        out, _ = mxq.attn_mixed_fwd(ops, None, shape, mode=mxq.MXQ_ALL_LOWBIT, out_dtype=mxq.MXQ_OUT_F32)
        return out.cpu().numpy()[0][:, rows].astype(np.float64)

    e_plain, e_rot = _rel(run(False), ref), _rel(run(True), ref)
    assert e_rot < 0.6 * e_plain, (e_rot, e_plain)
