"""Benchmark of the mixed-precision block-scaled attention hot path on one MI355X.

One step = the whole prefill path on one batch: MXFP4 quantisation of Q and K
(with the tile means the selection scores), MXFP8 quantisation of V (blocks
along keys) and its fp16 copy, block selection (5% of tiles plus the sink
column and local window), and the fused mixed-precision attention pass, as one
chain on the caller's stream (PrefillPipeline).  Inputs are bf16 tensors
already resident in HBM when the timed region starts.

The headline workload is the long-context causal prefill (B=1, Hq=32, Hkv=8,
N=32768, D=128, 5% + sink + 4-tile window), the largest single-GPU
configuration.  The JSON line reports effective attention TFLOP/s of the step
(4*D per valid query-key pair per head, divided by the step time), the
roofline of the dominant kernel (attn_mixed_fwd, timed with HIP events on the
stream it runs on) against the precision-weighted MFMA peak, the CPU oracle
timed on a bounded sample across the host's cores, and two extra legs: the
Llama-8B-shaped prefill (N=8192), the ViT-shaped batch (512 x 12 heads x 197
tokens, the short-sequence kernel) and the quantised-KV decode step (KV-read
GB/s against HBM peak).

Warm-up, the same rule for every leg: W untimed steps, then more until at
least 100 ms of the same step have run, so that the GPU clocks are steady
before timing (fewer read a few percent slow after the idle input upload).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--no-decode] [--no-extra]
                       [--only prefill|decode|copy|quality]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Published MI355X dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_FP16 = 2516.6
PEAK_FP8 = 5033.2
PEAK_FP4 = 10066.4
PEAK_HBM = 8000.0
METRIC = "effective attention TFLOPS @5% FP16 tiles (prefill); KV-read GB/s (decode)"


def recorded_traffic(kernel, workload):
    """HBM bytes per launch recorded by rocprofv3 FETCH_SIZE / WRITE_SIZE passes
    (profiles/hbm_traffic.json, entry "kernel/workload"), or None when the
    kernel's sources have changed since the counters were taken."""
    import hashlib

    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))[f"{kernel}/{workload}"]
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except (OSError, KeyError, ValueError):
        return None
    return rec["bytes"] if h.hexdigest() == rec["source_sha256"] else None


def warm(fn, steps, min_ms=100.0):
    """The warm-up rule of every leg: ``steps`` untimed calls, then more, in
    rounds of ``max(steps, 1)``, until at least ``min_ms`` of them have run
    (GPU clocks settle).  Returns the number of calls made."""
    import torch

    t0 = time.perf_counter()
    n = 0
    for _ in range(steps):
        fn()
        n += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(max(steps, 1)):
            fn()
            n += 1
        torch.cuda.synchronize()
    return n


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _bf16(t_np, dev):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(t_np).view(np.int16)).view(torch.bfloat16).to(dev)


def pair_counts(cfg, mask_np, lines_np=None):
    """Valid (query, key) pairs per head summed over heads, and how many of them
    run in FP16: those in FP16 tiles (read back from the selection mask) plus
    those of vertical-line keys that sit in low-bit tiles."""
    import numpy as np

    N, nv, Bq, Bk, causal = cfg["N"], cfg["n_valid"], cfg["Bq"], cfg["Bk"], cfg["causal"]
    n_qt, n_kt = N // Bq, N // Bk
    # pairs[i, j]: valid pairs inside tile (i, j); per valid row r, key tile j
    # holds min(max(r + 1 - j*Bk, 0), keys of j) valid keys when causal
    q = np.arange(nv)
    k0 = np.arange(n_kt) * Bk
    width = np.clip(nv - k0, 0, Bk)
    if causal:
        per_row = np.minimum(np.clip(q[:, None] + 1 - k0[None, :], 0, None), width[None, :])
    else:
        per_row = np.broadcast_to(width[None, :], (nv, n_kt))
    pairs = np.zeros((n_qt, n_kt), dtype=np.int64)
    np.add.at(pairs, q // Bq, per_row.astype(np.int64))
    bits = np.unpackbits(mask_np.view(np.uint8).reshape(mask_np.shape[:-1] + (-1,)), axis=-1, bitorder="little")
    bits = bits[..., :n_kt].astype(bool)  # [B, Hq, n_qt, n_kt]
    heads = mask_np.shape[0] * mask_np.shape[1]
    total = int(pairs.sum()) * heads
    fp16 = int((bits * pairs[None, None]).sum())
    if lines_np is not None:
        for b in range(lines_np.shape[0]):
            for h in range(lines_np.shape[1]):
                top = -1
                for key in (int(x) for x in lines_np[b, h]):
                    used = 0 <= key < nv and key > top
                    top = max(top, key)
                    if not used:
                        continue
                    j = key // Bk
                    for i in range(n_qt):
                        rows = q[(q >= i * Bq) & (q < (i + 1) * Bq)]
                        if rows.size and not bits[b, h, i, j]:
                            fp16 += int((rows >= key).sum()) if causal else int(rows.size)
    return total, fp16


def roofline_peak(D, total_pairs, fp16_pairs):
    """Precision-weighted MFMA peak: FP16 pairs at the FP16 peak; low-bit pairs
    split evenly between the FP4 QK^T and the FP8 PV contractions."""
    f_all = 4.0 * D * total_pairs
    f16 = 4.0 * D * fp16_pairs
    flow = f_all - f16
    t_roof = f16 / (PEAK_FP16 * 1e12) + flow * (0.5 / (PEAK_FP4 * 1e12) + 0.5 / (PEAK_FP8 * 1e12))
    return f_all / t_roof / 1e12, t_roof


def bench_prefill(args, dev, workload):
    """Time the prefill step (PrefillPipeline) of one workload; the attention
    kernel is bracketed by HIP events on the stream it is launched on."""
    import numpy as np
    import torch

    import bit_mixed_precision_mxq_amd as mxq
    import mxq_inputs

    cfg = mxq_inputs.make_prefill(workload)
    q, k, v = _bf16(cfg["q"], dev), _bf16(cfg["k"], dev), _bf16(cfg["v"], dev)
    shape = mxq.Shape(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["N"], cfg["n_valid"], cfg["D"], cfg["Bq"], cfg["Bk"],
                      cfg["causal"])
    n_lines = cfg.get("n_lines", 0)
    # one workgroup per kv group where the launch supports it (G = 2 or 4, N > 256)
    group_heads = args.group_heads and cfg["Hq"] // cfg["Hkv"] in (2, 4) and cfg["N"] > 256
    pipe = mxq.PrefillPipeline(shape, topk=cfg["topk"], ratio=(cfg["ratio_num"], cfg["ratio_den"]),
                               sink_tiles=cfg["sink_tiles"], local_tiles=cfg["local_tiles"], n_lines=n_lines,
                               sink_tokens=cfg.get("sink_tokens", 0), out_dtype=mxq.MXQ_OUT_BF16, device=dev,
                               group_shared=args.group_shared or group_heads, group_heads=group_heads)
    ev_a0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_a1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    def step(i=None):
        pipe(q, k, v, events=None if i is None else (ev_a0[i], ev_a1[i]))

    n_warm = warm(step, args.warmup)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    attn_ms = sum(a.elapsed_time(b) for a, b in zip(ev_a0, ev_a1)) / args.steps
    mask_np = pipe.mask.cpu().numpy().view(np.uint32)
    lines_np = pipe.lines.cpu().numpy() if pipe.lines is not None else None
    total, fp16 = pair_counts(cfg, mask_np, lines_np)
    flops = 4.0 * cfg["D"] * total
    peak_eff, t_roof = roofline_peak(cfg["D"], total, fp16)
    achieved = flops / (attn_ms * 1e-3) / 1e12
    res = dict(
        workload=workload, cfg=cfg, ms_step=ms_step, attn_ms=attn_ms, flops=flops, total_pairs=total,
        fp16_pairs=fp16, tflops_step=flops / (ms_step * 1e-3) / 1e12, tflops_attn=achieved, peak_eff=peak_eff,
        t_roof_ms=t_roof * 1e3, warmup_calls=n_warm,
        group="heads" if group_heads else ("shared" if args.group_shared or args.group_heads else None),
    )
    log(f"prefill {workload}: step {ms_step:.3f} ms, attn {attn_ms:.3f} ms, "
        f"{res['tflops_step']:.1f} TFLOP/s step, {achieved:.1f} TFLOP/s attn, "
        f"fp16 pairs {fp16 / total:.4f}, roofline {t_roof * 1e3:.3f} ms ({peak_eff:.0f} TFLOP/s eff peak), "
        f"frac {achieved / peak_eff:.4f}, {n_warm} warm-up steps")
    del q, k, v, pipe
    torch.cuda.empty_cache()
    return res


def workload_text(name, cfg):
    return (f"{name}: B={cfg['B']} Hq={cfg['Hq']} Hkv={cfg['Hkv']} N={cfg['N']} n_valid={cfg['n_valid']} "
            f"D={cfg['D']} {'causal' if cfg['causal'] else 'non-causal'}, {cfg['Bq']}x{cfg['Bk']} tiles, FP16 = top "
            f"{('k=' + str(cfg['topk'])) if cfg['topk'] >= 0 else str(cfg['ratio_num']) + '%'}"
            f" + sink {cfg['sink_tiles']} + window {cfg['local_tiles']}"
            + (f", {cfg['n_lines']} vertical-line token(s) incl. {cfg['sink_tokens']} sink/CLS"
               if cfg.get("n_lines", 0) else ""))


def quality_sweep(args, dev):
    """Synthetic quality/speed curve of the promotion fraction.

    For the Llama-8B-shaped shapes at N = 8K, 16K and 32K, under three input
    recipes (the workload's: outlier channels x20 and a sink key x8; the sink
    key alone; plain N(0,1)), and FP16 fractions from none (all low-bit) through the forced
    sink and window tiles alone, 1, 2, 5, 10 and 20% (plus the forced tiles),
    to all FP16: the error of attn_mixed_fwd (fp32 output) against exact
    softmax attention computed in float64 by torch on sampled query rows, the
    kernel time, and the share of the all-low-bit-to-all-FP16 error gap each
    fraction recovers, (e_lowbit - e) / (e_lowbit - e_fp16).  Two more rows
    put the pages' alternative beside promotion: Q and K rotated by the
    Walsh-Hadamard matrix before MXFP4, all low-bit and with 5% promoted.  The
    pages report this quantity on real models and benchmarks; here it is
    measured on seeded synthetic inputs only."""
    import numpy as np
    import torch

    import bit_mixed_precision_mxq_amd as mxq
    import mxq_inputs

    sizes = [int(x) for x in args.quality_n.split(",")]
    recipes = {"outliers+sink": {}, "sink": dict(outliers=False), "plain": dict(outliers=False, sink=None)}
    fracs = [("lowbit", None), ("forced", 0), ("1%", 1), ("2%", 2), ("5%", 5), ("10%", 10), ("20%", 20), ("fp16", None),
             ("lowbit+rot", None), ("5%+rot", 5), ("5%+shared", 5), ("5%+maxkey", 5)]
    rows_per_head = 16
    results = []
    for recipe, N in [(r, n) for r in recipes for n in sizes]:
        base = "llama8b" if N <= 8192 else "long32k"
        cfg = mxq_inputs.make_prefill(base, N=N, n_valid=N, **recipes[recipe])
        B, Hq, Hkv, D = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"]
        G = Hq // Hkv
        q, k, v = _bf16(cfg["q"], dev), _bf16(cfg["k"], dev), _bf16(cfg["v"], dev)
        shape = mxq.Shape(B, Hq, Hkv, N, N, D, cfg["Bq"], cfg["Bk"], cfg["causal"])
        # sampled rows: evenly spread over the sequence, the last row included
        rows = torch.linspace(N - 1, N / rows_per_head, rows_per_head, device=dev).round().long().flip(0)
        scale = 1.0 / math.sqrt(D)
        exact = []
        for h in range(Hq):
            qd = q[0, h, rows].double()
            kd, vd = k[0, h // G].double(), v[0, h // G].double()
            sc = (qd @ kd.T) * scale
            if cfg["causal"]:
                sc = sc.masked_fill(torch.arange(N, device=dev)[None, :] > rows[:, None], float("-inf"))
            exact.append(torch.softmax(sc, dim=-1) @ vd)
        exact = torch.stack(exact)  # [Hq, rows, D]
        ops_mixed = mxq.prepare_prefill(q, k, v, N, mode=mxq.MXQ_MIXED)
        ops_rot = mxq.prepare_prefill(q, k, v, N, mode=mxq.MXQ_MIXED, rotate=True)
        ws = mxq.select_workspace(shape, dev)
        errs = {}
        for label, pct in fracs:
            base_label = label.replace("+rot", "").replace("+shared", "").replace("+maxkey", "")
            ops_use = ops_rot if label.endswith("+rot") else ops_mixed
            mode = (mxq.MXQ_ALL_LOWBIT if base_label == "lowbit" else mxq.MXQ_ALL_FP16 if base_label == "fp16"
                    else mxq.MXQ_MIXED)
            mask = None
            fp16_frac = 0.0 if base_label == "lowbit" else 1.0
            if mode == mxq.MXQ_MIXED:
                mask, _, _ = mxq.attn_select_blocks(q, k, shape, topk=-1, ratio=(pct, 100),
                                                    sink_tiles=cfg["sink_tiles"], local_tiles=cfg["local_tiles"],
                                                    workspace=ws, group_shared=label.endswith("+shared"),
                                                    heuristic=1 if label.endswith("+maxkey") else 0)
                total, fp16 = pair_counts(cfg, mask.cpu().numpy().view(np.uint32))
                fp16_frac = fp16 / total
            out = torch.empty((B, Hq, N, D), dtype=torch.float32, device=dev)
            call = lambda: mxq.attn_mixed_fwd(ops_use, mask, shape, mode=mode, out_dtype=mxq.MXQ_OUT_F32,
                                              out=out, want_lse=False)
            for _ in range(5):
                call()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(10):
                call()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            got = out[0][:, rows].double()
            diff = got - exact
            rel = float(diff.norm() / exact.norm())
            mabs = float(diff.abs().max())
            errs[label] = rel
            results.append(dict(recipe=recipe, N=N, fp16=label, fp16_pair_fraction=round(fp16_frac, 5), rel_l2=rel, max_abs=mabs,
                                attn_ms=round(ms, 4)))
            log(f"quality {recipe} N={N} {label:7s} fp16 pairs {fp16_frac:.4f}: rel L2 {rel:.3e}, max abs {mabs:.3e}, "
                f"attn {ms:.3f} ms")
        gap = errs["lowbit"] - errs["fp16"]
        for r in results:
            if r["N"] == N and r["recipe"] == recipe:
                r["gap_recovered"] = round((errs["lowbit"] - r["rel_l2"]) / gap, 4) if gap > 0 else None
        del q, k, v, ops_mixed, ops_rot, out
        torch.cuda.empty_cache()
    print(json.dumps({"quality_sweep": results, "rows_sampled_per_head": rows_per_head,
                      "reference": "float64 softmax attention (torch) on the sampled rows",
                      "data": "synthetic (seeded N(0,1) bf16; outlier channels and sink key as in the recipe)"}),
          flush=True)


def bench_decode(args, dev):
    import numpy as np
    import torch

    import bit_mixed_precision_mxq_amd as mxq
    import mxq_inputs

    t_gen = time.perf_counter()
    d = mxq_inputs.make_decode("decode")
    log(f"decode inputs generated in {time.perf_counter() - t_gen:.1f} s")
    B, Hq, Hkv, D, L = d["B"], d["Hq"], d["Hkv"], d["D"], d["L"]
    n_sink, n_recent = d["n_sink"], d["n_recent"]
    lens = d["seq_len"]
    # build the cache on the GPU one sequence at a time (bounded device memory)
    kc = torch.empty((B, Hkv, L, D // 2), dtype=torch.uint8, device=dev)
    vc = torch.empty_like(kc)
    ks = torch.empty((B, Hkv, L, D // 32), dtype=torch.float16, device=dev)
    kz, vs, vz = torch.empty_like(ks), torch.empty_like(ks), torch.empty_like(ks)
    k_sink = torch.empty((B, Hkv, n_sink, D), dtype=torch.float16, device=dev)
    v_sink = torch.empty_like(k_sink)
    k_rec = torch.empty((B, Hkv, n_recent, D), dtype=torch.float16, device=dev)
    v_rec = torch.empty_like(k_rec)
    # vertical-line tokens (optional): evenly spread over the INT4 region
    n_lines = args.decode_lines
    lines_np = None
    if n_lines:
        lines_np = np.zeros((B, Hkv, n_lines), dtype=np.int32)
        for b in range(B):
            lo, hi = n_sink, int(lens[b]) - n_recent
            lines_np[b, :] = np.linspace(lo, hi - 1, n_lines).round().astype(np.int32)
        k_ln = torch.empty((B, Hkv, n_lines, D), dtype=torch.bfloat16, device=dev)
        v_ln = torch.empty_like(k_ln)
    for b in range(B):
        kb = _bf16(d["k"][b:b + 1], dev)
        vb = _bf16(d["v"][b:b + 1], dev)
        if n_lines:
            idx = torch.from_numpy(lines_np[b]).long().to(dev)  # [Hkv, n_lines]
            for h in range(Hkv):
                k_ln[b, h] = kb[0, h, idx[h]]
                v_ln[b, h] = vb[0, h, idx[h]]
        c = mxq.build_quant_kv_cache(kb, vb, torch.tensor([int(lens[b])], dtype=torch.int32, device=dev), n_sink,
                                     n_recent, kb[:, :, lens[b] - n_recent:lens[b]], vb[:, :, lens[b] - n_recent:lens[b]])
        kc[b], vc[b], ks[b], kz[b], vs[b], vz[b] = c.k_codes[0], c.v_codes[0], c.k_scale[0], c.k_zero[0], c.v_scale[0], c.v_zero[0]
        k_sink[b], v_sink[b], k_rec[b], v_rec[b] = c.k_sink[0], c.v_sink[0], c.k_recent[0], c.v_recent[0]
    del d["k"], d["v"]
    cache = mxq.QuantKVCache(kc, vc, ks, kz, vs, vz, k_sink, v_sink, k_rec, v_rec,
                             torch.from_numpy(lens).to(dev), n_sink, n_recent)
    line_cache = None
    if n_lines:
        k_lf, _, _ = mxq.mxq_quantize(k_ln, mxq.MXQ_FP16, mxq.MXQ_AXIS_D)
        v_lf, _, _ = mxq.mxq_quantize(v_ln, mxq.MXQ_FP16, mxq.MXQ_AXIS_D)
        line_cache = mxq.QuantKVCache(kc, vc, ks, kz, vs, vz, k_sink, v_sink, k_rec, v_rec, cache.seq_len, n_sink,
                                      n_recent, torch.from_numpy(lines_np).to(dev), k_lf, v_lf)
    q = _bf16(d["q"], dev)
    ws = mxq.decode_workspace(B, Hq, D, 0, int(lens.max()), dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    n_warm = warm(lambda: mxq.attn_quantkv_decode(q, cache, Hkv, int(lens.max()), workspace=ws, out=out),
                  args.warmup)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        mxq.attn_quantkv_decode(q, cache, Hkv, int(lens.max()), workspace=ws, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # bytes the step must read: INT4 codes + fp16 scale/zero for the quantised
    # tokens, fp16 rows for the sink/recent tokens, q, and the output written
    n_fp = n_sink + n_recent
    n_q = lens.astype(np.int64) - n_fp
    per_tok_q = 2 * (D // 2 + 2 * 2 * (D // 32))
    per_tok_f = 2 * D * 2
    byts = int((n_q * per_tok_q + n_fp * per_tok_f).sum()) * Hkv + B * Hq * D * 2 + B * Hq * D * 4
    gbs = byts / (ms * 1e-3) / 1e9
    log(f"decode: {ms:.4f} ms/step, {byts / 1e9:.4f} GB, {gbs:.0f} GB/s ({gbs / PEAK_HBM:.3f} of HBM peak)")
    lines_ms = None
    if line_cache is not None:
        warm(lambda: mxq.attn_quantkv_decode(q, line_cache, Hkv, int(lens.max()), workspace=ws, out=out),
             args.warmup)
        e0.record()
        for _ in range(args.steps):
            mxq.attn_quantkv_decode(q, line_cache, Hkv, int(lens.max()), workspace=ws, out=out)
        e1.record()
        torch.cuda.synchronize()
        lines_ms = e0.elapsed_time(e1) / args.steps
        log(f"decode with {n_lines} vertical-line tokens per kv head: {lines_ms:.4f} ms/step")
    # the step's cache update: one new token per sequence enters the fp16
    # window, the token leaving it is quantised.  Timed on the same arrays with
    # the lengths pulled back so that every append has room (contents differ
    # from the timed decode's from here on; nothing reads them afterwards).
    # (the warm-up rule runs at most about 100 ms of appends, far fewer than
    # the room of 8192 tokens made here)
    n_app = 8192
    seq = torch.from_numpy(lens - n_app).to(dev)
    app_cache = mxq.QuantKVCache(kc, vc, ks, kz, vs, vz, k_sink, v_sink, k_rec, v_rec, seq, n_sink, n_recent)
    g = torch.Generator(device=dev).manual_seed(4)
    kn = torch.randn((B, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((B, Hkv, D), generator=g, device=dev).to(torch.bfloat16)
    n_warm_app = warm(lambda: mxq.attn_quantkv_append(app_cache, kn, vn), args.warmup)
    assert n_warm_app + args.steps <= n_app
    e0.record()
    for _ in range(args.steps):
        mxq.attn_quantkv_append(app_cache, kn, vn)
    e1.record()
    torch.cuda.synchronize()
    app_ms = e0.elapsed_time(e1) / args.steps
    assert int(seq[0]) == int(lens[0]) - n_app + n_warm_app + args.steps
    # bytes per append: the window read and written (K and V), the leaving
    # token's fp16 row read and its codes, scales and zeros written, the new rows
    app_bytes = B * Hkv * 2 * (2 * n_recent * D * 2 + D * 2 + D // 2 + 2 * 2 * (D // 32) + D * 2)
    log(f"append: {app_ms * 1e3:.1f} us/step, {app_bytes / 1e6:.1f} MB, "
        f"{app_bytes / (app_ms * 1e-3) / 1e9:.0f} GB/s")
    return dict(ms=ms, bytes=byts, gbs=gbs, append_ms=app_ms, append_bytes=app_bytes, lines_ms=lines_ms,
                n_lines=n_lines, warmup_calls=n_warm)


# ---------------------------------------------------------------- CPU baseline
# The oracle (test infrastructure, never tuned for speed) timed on the host's
# cores on a bounded sample of the same workloads.  Workers come from a pool
# forked before the GPU is initialised; each runs single-threaded numpy.


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _oracle_prefill_worker(task):
    """One query head of a prefill workload: its tile selection, the quantised
    operands (a1-a3), then the mixed attention of the given query tiles until
    the time budget runs out.  Returns (valid pairs done, tiles done)."""
    import numpy as np

    import oracle
    from oracle import attention as A

    sub, cfg, tiles, budget_s = task
    t0 = time.perf_counter()
    mask, _, _ = oracle.select_blocks(sub["q"], sub["k"], cfg["n_valid"], cfg["Bq"], cfg["Bk"], cfg["causal"],
                                      cfg["topk"], cfg["ratio_num"], cfg["ratio_den"], cfg["sink_tiles"],
                                      cfg["local_tiles"])
    lines = None
    if cfg.get("n_lines", 0):
        lines, _ = oracle.select_lines(sub["q"], sub["k"], cfg["n_valid"], cfg["Bq"], cfg["n_lines"],
                                       cfg["sink_tokens"])
    ops = A.prepare_operands(sub["q"], sub["k"], sub["v"], cfg["n_valid"])
    pairs = done = 0
    for i in tiles:
        if time.perf_counter() - t0 >= budget_s:
            break
        A.attn_mixed_ref(sub["q"], sub["k"], sub["v"], cfg["n_valid"], cfg["Bq"], cfg["Bk"], cfg["causal"],
                         mask=mask, qtiles=[int(i)], ops=ops, lines=lines)
        r = np.arange(i * cfg["Bq"], min((i + 1) * cfg["Bq"], cfg["n_valid"]))
        pairs += int(np.minimum(r + 1, cfg["n_valid"]).sum()) if cfg["causal"] else r.size * cfg["n_valid"]
        done += 1
    return pairs, done


def cpu_baseline_prefill(pool, n_workers, pre, seconds):
    """Each worker takes one (batch, query head), chosen at random with a fixed
    seed, and its query tiles in a random order; the rate is the valid pairs
    done by all workers over the wall time of the pool, and the whole step's
    CPU time is extrapolated linearly by valid-pair count."""
    import numpy as np

    cfg = pre["cfg"]
    G = cfg["Hq"] // cfg["Hkv"]
    n_qt = cfg["N"] // cfg["Bq"]
    rng = np.random.default_rng(1234)
    heads = [(b, h) for b in range(cfg["B"]) for h in range(cfg["Hq"])]
    pick = rng.permutation(len(heads))[:n_workers]
    small = {k: v for k, v in cfg.items() if k not in ("q", "k", "v")}
    tasks = []
    for idx in pick:
        b, h = heads[idx]
        kv = slice(h // G, h // G + 1)
        sub = dict(q=cfg["q"][b:b + 1, h:h + 1].copy(), k=cfg["k"][b:b + 1, kv].copy(),
                   v=cfg["v"][b:b + 1, kv].copy())
        tasks.append((sub, small, rng.permutation(n_qt), seconds))
    t0 = time.perf_counter()
    res = pool.map(_oracle_prefill_worker, tasks, chunksize=1)
    dt = time.perf_counter() - t0
    pairs = sum(r[0] for r in res)
    tiles = sum(r[1] for r in res)
    flops = 4.0 * cfg["D"] * pairs
    est_s = pre["total_pairs"] / (pairs / dt)
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=n_workers, kind="oracle",
                sample=f"{pre['workload']}: {len(tasks)} (batch, query head) pairs, one per worker, each its "
                       f"selection, quantised operands and the mixed attention of randomly ordered query tiles "
                       f"for {seconds:.0f} s: {tiles} query tiles, {pairs} of {pre['total_pairs']} valid pairs, "
                       f"{dt:.1f} s wall on {n_workers} single-threaded processes; the whole step extrapolated "
                       f"linearly by valid-pair count",
                extrapolated_step_s=round(est_s, 1))


def _oracle_decode_worker(task):
    """Decode step of the oracle for one sequence: the INT4 cache of each kv
    head is built (untimed, the cache build is off the step) and the decode
    attention over it timed, kv head by kv head, until the budget runs out.
    Returns (cache bytes processed, timed seconds)."""
    import mxq_inputs
    from oracle import decode as Dd

    name, b, budget_s = task
    d = mxq_inputs.make_decode(name, seqs=[b], threads=1)
    Hq, Hkv, D = d["Hq"], d["Hkv"], d["D"]
    G = Hq // Hkv
    n_sink, n_recent = d["n_sink"], d["n_recent"]
    lens = d["seq_len"][b:b + 1]
    n = int(lens[0])
    per_head = (n - n_sink - n_recent) * 2 * (D // 2 + 2 * 2 * (D // 32)) + (n_sink + n_recent) * 2 * D * 2
    t_busy = 0.0
    byts = 0
    for h in range(Hkv):
        if t_busy >= budget_s:
            break
        cache = Dd.build_kv_cache_ref(d["k"][:, h:h + 1], d["v"][:, h:h + 1], lens, n_sink, n_recent)
        t0 = time.perf_counter()
        Dd.attn_decode_ref(d["q"][b:b + 1, h * G:(h + 1) * G], cache, lens, n_sink, n_recent)
        t_busy += time.perf_counter() - t0
        byts += per_head
    return byts, t_busy


def cpu_baseline_decode(pool, n_workers, dec, seconds):
    """Each worker takes one sequence (the first n_workers) and times the
    oracle's decode attention over its cache, kv head by kv head; the rate is
    the sum of the workers' rates (they run at the same time)."""
    tasks = [("decode", b, seconds) for b in range(n_workers)]
    t0 = time.perf_counter()
    res = pool.map(_oracle_decode_worker, tasks, chunksize=1)
    dt = time.perf_counter() - t0
    rate = sum(r[0] / r[1] for r in res if r[1] > 0) / 1e9
    byts = sum(r[0] for r in res)
    return dict(value=round(rate, 4), unit="GB/s", cores=n_workers, kind="oracle",
                sample=f"decode: sequences 0..{n_workers - 1}, one per worker, the oracle's decode attention "
                       f"over the INT4 + fp16 cache of each kv head (cache build untimed): {byts / 1e9:.3f} GB "
                       f"of cache processed, {dt:.1f} s wall on {n_workers} single-threaded processes; the "
                       f"whole step ({dec['bytes'] / 1e9:.4f} GB) would take {dec['bytes'] / 1e9 / rate:.1f} s")


def copy_calibration(dev, mib=256, reps=3):
    """A plain device-to-device copy of `mib` MiB, the known-size reference that
    scales hardware byte counters (FETCH_SIZE, WRITE_SIZE) to HBM bytes."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert torch.equal(dst[-4:], src[-4:])
    print(json.dumps({"copy_calibration_bytes": n * 4, "reps": reps}), flush=True)


def prefill_summary(pre, with_traffic):
    """The prefill leg's numbers for the JSON line."""
    cfg = pre["cfg"]
    scored = cfg["topk"] > 0 or (cfg["topk"] < 0 and cfg["ratio_num"] > 0)
    promoted = scored or cfg["sink_tiles"] > 0 or cfg["local_tiles"] > 0
    return {
        "config": {
            "workload": workload_text(pre["workload"], cfg),
            "step": "quantize Q,K (MXFP4" + (", with tile means" if scored else "") + "), V (MXFP8"
                    + (" + fp16 copy" if promoted else "") + ") -> select tiles"
                    + (" and lines" if cfg.get("n_lines", 0) else "")
                    + (" (one mask per kv group)" if pre.get("group") else "") + " -> fused mixed attention"
                    + ("" if promoted else " (line V from bf16 V)")
                    + (" (one workgroup per kv group)" if pre.get("group") == "heads" else ""),
            "fp16_pair_fraction": round(pre["fp16_pairs"] / pre["total_pairs"], 5),
            "attn_ms": round(pre["attn_ms"], 4),
            "attn_tflops": round(pre["tflops_attn"], 2),
            "warmup_calls": pre["warmup_calls"],
        },
        "roofline": {
            "bound": "mfma", "kernel": "attn_mixed_fwd",
            "achieved": round(pre["tflops_attn"], 2), "peak": round(pre["peak_eff"], 1), "unit": "TFLOP/s",
            "frac": round(pre["tflops_attn"] / pre["peak_eff"], 4),
            # the recorded counters are those of the default per-head launch
            "traffic": recorded_traffic("attn_mixed_fwd", pre["workload"])
                       if with_traffic and not pre.get("group") else None,
            "peak_note": "precision-weighted: FP16 pairs at 2516.6, low-bit pairs half at FP4 10066.4 (QK^T) "
                         "and half at FP8 5033.2 (PV); achieved = 4*D*valid pairs / attention kernel time",
        },
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long32k", choices=["tiny", "llama8b", "long32k", "vit"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the Llama-8B-shaped and ViT-shaped prefill legs")
    ap.add_argument("--only", choices=["prefill", "decode", "copy", "quality"], default=None,
                    help="copy: a plain device copy of a known size, the reference for HBM byte counters; "
                         "quality: the synthetic error/speed curve over the FP16 fraction")
    ap.add_argument("--quality-n", default="8192,16384,32768", help="sequence lengths of the quality sweep")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="wall-time budget of each CPU-baseline leg")
    ap.add_argument("--group-shared", action="store_true",
                    help="prefill with one tile mask per kv group (the G query heads share it)")
    ap.add_argument("--group-heads", action="store_true",
                    help="prefill with shared masks and one attention workgroup per kv group (implies --group-shared)")
    ap.add_argument("--decode-lines", type=int, default=0,
                    help="also time decode with this many vertical-line tokens (fp16) per kv head, at most 16")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU; each (batch, kv head) is independent, so more GPUs "
              "would shard heads with no communication, but that path is not built. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    # the CPU baseline's worker processes are forked before anything touches
    # the GPU (they never do); at most 16 workers, the host share of one GPU
    pool = None
    n_workers = 0
    want_cpu = not args.no_cpu_baseline and args.only not in ("copy", "quality")
    if want_cpu:
        import multiprocessing as mp

        n_workers = max(1, min(len(os.sched_getaffinity(0)), 16))
        pool = mp.get_context("fork").Pool(n_workers, initializer=_pool_init)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    import bit_mixed_precision_mxq_amd as mxq

    if args.only == "copy":
        copy_calibration(dev)
        return
    mxq.load_library()
    if args.only == "quality":
        quality_sweep(args, dev)
        return
    pre = dec = None
    extras = {}
    if args.only != "decode":
        pre = bench_prefill(args, dev, args.workload)
        if not args.no_extra and args.only is None:
            for name in ("llama8b", "vit"):
                if name == args.workload:
                    continue
                extras[name] = bench_prefill(args, dev, name)
                for key in ("q", "k", "v"):  # only the headline's inputs feed the CPU baseline
                    extras[name]["cfg"].pop(key)
    if args.only != "prefill" and not args.no_decode:
        dec = bench_decode(args, dev)
    cpu = cpu_dec = None
    if pool is not None:
        if pre is not None:
            cpu = cpu_baseline_prefill(pool, n_workers, pre, args.cpu_seconds)
            log(f"cpu baseline (prefill): {cpu['value']:.6f} TFLOP/s ({cpu['sample']})")
        if dec is not None:
            cpu_dec = cpu_baseline_decode(pool, n_workers, dec, args.cpu_seconds * 2 / 3)
            log(f"cpu baseline (decode): {cpu_dec['value']:.4f} GB/s ({cpu_dec['sample']})")
        pool.close()
        pool.join()
    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "data": "synthetic (seeded N(0,1) bf16; outlier channels and "
            "sink key as in the workload recipe)"}
    if pre is not None:
        summ = prefill_summary(pre, with_traffic=True)
        line.update(value=round(pre["tflops_step"], 3), unit="TFLOP/s", ms_per_step=round(pre["ms_step"], 4),
                    dtype="mxfp4 QK^T + fp8 PV, fp16 on selected tiles, fp32 accumulate", config=summ["config"],
                    roofline=summ["roofline"])
    for name, extra in extras.items():
        summ = prefill_summary(extra, with_traffic=True)
        line[name] = dict(value=round(extra["tflops_step"], 3), unit="TFLOP/s",
                          ms_per_step=round(extra["ms_step"], 4), **summ)
    if dec is not None:
        dline = {"value": round(dec["gbs"], 1), "unit": "GB/s", "ms_per_step": round(dec["ms"], 5),
                 "workload": "decode: 64 seqs x 32768 cached tokens, Hq=32 Hkv=8 D=128, INT4-G32 KV + fp16 "
                             "first 64 / last 128 tokens",
                 "warmup_calls": dec["warmup_calls"],
                 "roofline": {"bound": "hbm", "kernel": "attn_quantkv_decode", "achieved": round(dec["gbs"], 1),
                              "peak": PEAK_HBM, "unit": "GB/s", "frac": round(dec["gbs"] / PEAK_HBM, 4),
                              "traffic": recorded_traffic("attn_quantkv_decode", "decode")},
                 "append": {"ms_per_step": round(dec["append_ms"], 5), "bytes": dec["append_bytes"],
                            "gbs": round(dec["append_bytes"] / (dec["append_ms"] * 1e-3) / 1e9, 1),
                            "what": "attn_quantkv_append: one token per sequence into the fp16 window, the "
                                    "leaving token quantised to INT4"}}
        if dec["lines_ms"] is not None:
            dline["with_lines"] = {"n_lines": dec["n_lines"], "ms_per_step": round(dec["lines_ms"], 5)}
        if cpu_dec is not None:
            dline["cpu_baseline"] = cpu_dec
        line["decode"] = dline
        if pre is None:
            line.update(value=dline["value"], unit="GB/s", ms_per_step=dline["ms_per_step"], dtype="int4 KV, fp32",
                        config={"workload": dline["workload"]}, roofline=dline["roofline"])
            cpu = cpu_dec
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
