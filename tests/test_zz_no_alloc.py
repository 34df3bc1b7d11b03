"""attn_quantkv_decode_noalloc, the allocation-free decode entry point (for
callers that cannot allocate: graph capture, serving loops): through the C
ABI it gives the workspace entry point's output bit for bit, on two calls in a
row with the second one smaller (the fixed per-GPU array keeps the first
call's contents), and refuses requests beyond its fixed size."""

import numpy as np
import pytest

from gpu_helpers import bf16_dev, gpu_or_skip
import mxq_inputs
from oracle import decode as Dm

pytestmark = pytest.mark.gpu


def _cache(mxq, d, n_sink=64, n_recent=128, lines=None):
    import torch

    k, v, q = bf16_dev(d["k"]), bf16_dev(d["v"]), bf16_dev(d["q"])
    lens = d["seq_len"]
    B = len(lens)
    krec = torch.stack([k[b, :, lens[b] - n_recent:lens[b]] for b in range(B)])
    vrec = torch.stack([v[b, :, lens[b] - n_recent:lens[b]] for b in range(B)])
    cache = mxq.build_quant_kv_cache(k, v, torch.from_numpy(lens).to("cuda:0"), n_sink, n_recent, krec, vrec)
    return q, cache


def test_noalloc_matches_workspace_entry_point_twice_then_smaller():
    mxq = gpu_or_skip()
    import torch

    big = mxq_inputs.make_decode(dict(B=6, L=8192, Hq=32, Hkv=8, D=128, n_sink=64, n_recent=128, seed=21,
                                      seq_len=[8192, 5000, 8000, 333, 4096, 7777]), threads=4)
    small = mxq_inputs.make_decode(dict(B=3, L=2048, Hq=16, Hkv=4, D=128, n_sink=64, n_recent=128, seed=22,
                                        seq_len=[2048, 1500, 700]), threads=3)
    for d, splits in ((big, 0), (small, 3)):
        q, cache = _cache(mxq, d)
        maxlen = int(d["seq_len"].max())
        ref = mxq.attn_quantkv_decode(q, cache, d["Hkv"], maxlen, num_splits=splits)
        out = torch.full_like(ref, float("nan"))
        got = mxq.attn_quantkv_decode_noalloc(q, cache, d["Hkv"], maxlen, num_splits=splits, out=out)
        torch.cuda.synchronize()
        assert got is out
        assert torch.equal(out, ref), float((out - ref).abs().max())
        # and the oracle's bar, on the sequences the oracle computes quickly
        oref = Dm.attn_decode_ref(d["q"], Dm.build_kv_cache_ref(d["k"], d["v"], d["seq_len"], 64, 128),
                                  d["seq_len"], 64, 128, seqs=[len(d["seq_len"]) - 1])
        b = len(d["seq_len"]) - 1
        assert np.abs(out.cpu().numpy()[b] - oref[b]).max() <= 5e-3


def test_noalloc_rejects_requests_beyond_its_scratch():
    mxq = gpu_or_skip()
    import torch

    d = mxq_inputs.make_decode(dict(B=2, L=1024, Hq=8, Hkv=2, D=128, n_sink=64, n_recent=128, seed=23,
                                    seq_len=[1024, 900]), threads=2)
    q, cache = _cache(mxq, d)
    need = mxq.load_library().attn_quantkv_decode_workspace(2, 8, 128, 4096, 1024)
    assert need > mxq.DECODE_SCRATCH_BYTES
    out = torch.zeros((2, 8, 128), dtype=torch.float32, device="cuda:0")
    with pytest.raises(mxq.MxqError) as ei:
        mxq.attn_quantkv_decode_noalloc(q, cache, 2, 1024, num_splits=4096, out=out)
    assert ei.value.status == mxq.MXQ_EINVAL and b"scratch" in mxq.load_library().mxq_last_error()
    torch.cuda.synchronize()
    assert not out.any()  # nothing was launched
