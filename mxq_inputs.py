"""Seeded synthetic inputs for the mixed-precision attention workloads.

This module only draws random numbers and rounds them to bf16; it holds none
of the method's arithmetic.  Both the CPU oracle's callers and the GPU path's
callers take their inputs from here, so the two sides see identical bits.

The workloads stand in for the long-context benchmarks and model families the
ThriftAttention abstract evaluates on, and for the ViT-style attention
workloads of the QFlash abstract; no dataset or trained weight is used.

Recipe (numpy PCG64 ``default_rng``):

* prefill: Q [B,Hq,N,D], K [B,Hkv,N,D], V [B,Hkv,N,D] drawn N(0,1) in that
  order; then, when ``outliers`` is set, for each kv head 4 distinct head_dim
  channels are drawn and Q (all query heads of that group) and K are scaled by
  20 on them; when ``sink`` is set, key 0 of every kv head is scaled by it;
  rows >= n_valid are zero; finally every value is rounded to bf16 (nearest,
  ties to even).
* decode: q [B,Hq,D] from ``default_rng([seed, 1_000_000])``; sequence b's K
  then V [Hkv,L,D] from ``default_rng([seed, b])``, N(0,1), rounded to bf16.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

PREFILL_CONFIGS = {
    # B=1, H=2, N=256, d=64, non-causal, 64x64 tiles, top-1 FP16 key tile per query tile
    "tiny": dict(B=1, Hq=2, Hkv=2, N=256, n_valid=256, D=64, causal=False, Bq=64, Bk=64,
                 topk=1, ratio_num=0, ratio_den=1, sink_tiles=0, local_tiles=0, n_lines=0, sink_tokens=0,
                 outliers=False, sink=None, seed=1),
    # Llama-8B-shaped causal prefill, GQA 4:1, 128x64 tiles, 5% + sink column + 1-tile window
    "llama8b": dict(B=1, Hq=32, Hkv=8, N=8192, n_valid=8192, D=128, causal=True, Bq=128, Bk=64,
                    topk=-1, ratio_num=5, ratio_den=100, sink_tiles=1, local_tiles=1, n_lines=0, sink_tokens=0,
                    outliers=True, sink=8.0, seed=2),
    # long-context causal prefill, 5% + sink + 4-tile window
    "long32k": dict(B=1, Hq=32, Hkv=8, N=32768, n_valid=32768, D=128, causal=True, Bq=128, Bk=64,
                    topk=-1, ratio_num=5, ratio_den=100, sink_tiles=1, local_tiles=4, n_lines=0, sink_tokens=0,
                    outliers=True, sink=8.0, seed=3),
    # ViT-B/16-shaped: batch 512, 12 heads, 197 tokens padded to 256; the CLS
    # token's key column is kept FP16 as a one-token vertical line, no FP16 tile
    "vit": dict(B=512, Hq=12, Hkv=12, N=256, n_valid=197, D=64, causal=False, Bq=64, Bk=64,
                topk=0, ratio_num=0, ratio_den=1, sink_tiles=0, local_tiles=0, n_lines=1, sink_tokens=1,
                outliers=False, sink=None, seed=5),
}

DECODE_CONFIGS = {
    # 64 sequences x 32768 cached tokens, Hq=32, Hkv=8, d=128, fp16 first 64 / last 128 tokens
    "decode": dict(B=64, L=32768, Hq=32, Hkv=8, D=128, n_sink=64, n_recent=128, seed=4),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def make_prefill(cfg: dict | str, **override):
    """Return dict(q, k, v) of bf16 bit arrays plus the config fields."""
    if isinstance(cfg, str):
        cfg = PREFILL_CONFIGS[cfg]
    cfg = dict(cfg, **override)
    B, Hq, Hkv, N, D = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["D"]
    G = Hq // Hkv
    rng = np.random.default_rng(cfg["seed"])
    q = rng.standard_normal((B, Hq, N, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, N, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, N, D), dtype=np.float32)
    if cfg.get("outliers"):
        for h in range(Hkv):
            ch = rng.choice(D, size=4, replace=False)
            q[:, h * G:(h + 1) * G, :, ch] *= np.float32(20.0)
            k[:, h, :, ch] *= np.float32(20.0)
    if cfg.get("sink"):
        k[:, :, 0, :] *= np.float32(cfg["sink"])
    nv = cfg["n_valid"]
    q[:, :, nv:, :] = 0
    k[:, :, nv:, :] = 0
    v[:, :, nv:, :] = 0
    out = dict(cfg)
    out.update(q=to_bf16_bits(q), k=to_bf16_bits(k), v=to_bf16_bits(v))
    return out


def _decode_seq(seed, b, Hkv, L, D):
    rng = np.random.default_rng([seed, b])
    k = to_bf16_bits(rng.standard_normal((Hkv, L, D), dtype=np.float32))
    v = to_bf16_bits(rng.standard_normal((Hkv, L, D), dtype=np.float32))
    return k, v


def make_decode(cfg: dict | str, seqs=None, threads=None, **override):
    """Return dict(q [B,Hq,D], k/v [nb,Hkv,L,D] bf16 bits, seq_len [B]).

    ``seqs`` picks which sequences' K/V are generated (all by default); each
    sequence has its own generator, so any subset is reproducible alone."""
    if isinstance(cfg, str):
        cfg = DECODE_CONFIGS[cfg]
    cfg = dict(cfg, **override)
    B, L, Hq, Hkv, D = cfg["B"], cfg["L"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    seqs = list(range(B)) if seqs is None else list(seqs)
    rq = np.random.default_rng([cfg["seed"], 1_000_000])
    q = to_bf16_bits(rq.standard_normal((B, Hq, D), dtype=np.float32))
    k = np.empty((len(seqs), Hkv, L, D), dtype=np.uint16)
    v = np.empty((len(seqs), Hkv, L, D), dtype=np.uint16)
    nthreads = threads or min(16, len(os.sched_getaffinity(0)))

    def fill(idx):
        k[idx], v[idx] = _decode_seq(cfg["seed"], seqs[idx], Hkv, L, D)

    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(fill, range(len(seqs))))
    seq_len = np.asarray(cfg.get("seq_len", [L] * B), dtype=np.int32)
    out = dict(cfg)
    out.update(q=q, k=k, v=v, seq_len=seq_len, seqs=seqs)
    return out
