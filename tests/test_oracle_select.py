"""Pins for the oracle's block selection (CPU only)."""

import os

import numpy as np

import mxq_inputs
from oracle import select as S
from oracle import formats as F
from oracle.formats import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_counts():
    out = {}
    with open(os.path.join(GOLDEN, "tile_counts.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                name, *vals = line.split()
                out[name] = tuple(int(v) for v in vals)
    return out


def _closed_form_counts(N, Bq, Bk, causal, n_valid, sink, w, topk, num, den):
    """Independent count formulas (interval arithmetic, no set building)."""
    n_qt = N // Bq
    tv = tf = tk = 0
    for i in range(n_qt):
        qs = i * Bq
        if qs >= n_valid:
            continue
        qe = min(qs + Bq, n_valid) - 1
        last = (qe // Bk) if causal else (n_valid - 1) // Bk
        nvalid = last + 1
        ns = min(sink, nvalid)                      # sink tiles [0, ns)
        if w >= 1:
            lo_t = max(0, (qs - (w - 1) * Bk) // Bk)
            hi_t = min(last, qe // Bk)
            nloc = hi_t - lo_t + 1                  # window tiles [lo_t, hi_t]
            both = max(0, min(hi_t, ns - 1) - lo_t + 1)
            forced = nloc + ns - both
        else:
            forced = ns
        k = topk if topk >= 0 else -((-num * nvalid) // den)
        tv += nvalid
        tf += forced
        tk += min(k, nvalid - forced)
    return tv, tf, tk, tf + tk


def test_tile_count_closed_forms_match_golden():
    gold = _golden_counts()
    for name, cfg in mxq_inputs.PREFILL_CONFIGS.items():
        got = _closed_form_counts(cfg["N"], cfg["Bq"], cfg["Bk"], cfg["causal"], cfg["n_valid"],
                                  cfg["sink_tiles"], cfg["local_tiles"], cfg["topk"],
                                  cfg["ratio_num"], cfg["ratio_den"])
        assert got == gold[name], (name, got, gold[name])


def test_oracle_selection_counts_match_closed_forms():
    gold = _golden_counts()
    rng = np.random.default_rng(0)
    for name, cfg in mxq_inputs.PREFILL_CONFIGS.items():
        N, D = cfg["N"], 32
        q = f32_to_bf16_bits(rng.standard_normal((1, 1, N, D)).astype(np.float32))
        k = f32_to_bf16_bits(rng.standard_normal((1, 1, N, D)).astype(np.float32))
        sets = S.tile_sets(cfg["n_valid"], N, cfg["Bq"], cfg["Bk"], cfg["causal"],
                           cfg["sink_tiles"], cfg["local_tiles"])
        assert sum(len(v) for v, _ in sets) == gold[name][0]
        assert sum(len(f) for _, f in sets) == gold[name][1]
        mask, nfp, _ = S.select_blocks(q, k, cfg["n_valid"], cfg["Bq"], cfg["Bk"], cfg["causal"],
                                       cfg["topk"], cfg["ratio_num"], cfg["ratio_den"],
                                       cfg["sink_tiles"], cfg["local_tiles"])
        assert int(nfp.sum()) == gold[name][3], name
        bits = sum(bin(int(w)).count("1") for w in mask.ravel())
        assert bits == gold[name][3]


def test_local_window_is_w_tiles_when_square():
    # Bq == Bk: the window is exactly the diagonal tile and the w-1 before it
    sets = S.tile_sets(1024, 1024, 64, 64, True, 0, 3)
    for i, (valid, forced) in enumerate(sets):
        assert forced == list(range(max(0, i - 2), i + 1))
    # Bq = 2*Bk, w = 1: both diagonal key tiles (the diagonal band)
    sets = S.tile_sets(1024, 1024, 128, 64, True, 0, 1)
    for i, (valid, forced) in enumerate(sets):
        assert forced == [2 * i, 2 * i + 1]


def test_tile_means_and_scores_against_float32_loops():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((256, 8)).astype(np.float32) * 5
    xb = S.bf16_bits_to_f32(f32_to_bf16_bits(x))
    m = S._tile_means(xb, 150, 64)   # tiles: 64 rows, 64 rows, 22 rows valid, 0 valid (pad to 256)
    # plain loops, one element at a time in float32
    for t in range(3):
        for d in range(8):
            acc = np.float32(0)
            n = 0
            for r in range(t * 64, min(t * 64 + 64, 150)):
                acc = np.float32(acc + xb[r, d])
                n += 1
            assert m[t, d] == np.float32(acc / np.float32(n))
    sc = S.tile_scores(m[:3], m[:3])
    for i in range(3):
        for j in range(3):
            acc = np.float32(0)
            for d in range(8):
                acc = np.float32(acc + np.float32(m[i, d] * m[j, d]))
            assert sc[i, j] == acc


def _check_topk_property(scores_row, cand, chosen, k):
    """Selected candidates dominate unselected ones: score strictly higher, or
    equal score with a lower tile index (the tie rule)."""
    assert len(chosen) == k
    rest = [j for j in cand if j not in chosen]
    for a in chosen:
        for b in rest:
            sa, sb = scores_row[a], scores_row[b]
            assert sa > sb or (sa == sb and a < b)


def test_topk_dominance_property_random_and_ties():
    rng = np.random.default_rng(2)
    N, D = 1024, 16
    for trial in range(4):
        qf = rng.standard_normal((1, 2, N, D)).astype(np.float32)
        kf = rng.standard_normal((1, 1, N, D)).astype(np.float32)
        if trial == 3:
            kf[:] = np.round(kf)  # coarse values make equal scores likely
            qf[:] = 1.0
        q, k = f32_to_bf16_bits(qf), f32_to_bf16_bits(kf)
        mask, nfp, scores = S.select_blocks(q, k, N, 64, 64, True, -1, 20, 100, 1, 1)
        sets = S.tile_sets(N, N, 64, 64, True, 1, 1)
        for h in range(2):
            for i, (valid, forced) in enumerate(sets):
                chosen = set(S.mask_to_sets(mask[0, h, i], N // 64))
                assert set(forced) <= chosen
                cand = [j for j in valid if j not in forced]
                kk = S.budget(-1, 20, 100, len(valid), len(cand))
                _check_topk_property(scores[0, h, i], cand, chosen - set(forced), kk)


def test_zero_keys_pick_lowest_index_candidates():
    N, D = 512, 16
    rng = np.random.default_rng(3)
    q = f32_to_bf16_bits(rng.standard_normal((1, 1, N, D)).astype(np.float32))
    k = np.zeros((1, 1, N, D), dtype=np.uint16)
    mask, _, scores = S.select_blocks(q, k, N, 64, 64, False, 2, 0, 1, 1, 0)
    assert np.all(scores == 0)
    for i in range(N // 64):
        assert S.mask_to_sets(mask[0, 0, i], 8) == [0, 1, 2]   # sink 0 + lowest two candidates


# ---- one mask per kv group (reading R35)
def _small_int_bits(shape, seed, lo=-3, hi=4):
    """bf16 bits of small integers: every fp32 sum and product of the tile
    means below stays exact, so float64 arithmetic is the exact reference."""
    rng = np.random.default_rng(seed)
    x = rng.integers(lo, hi, size=shape).astype(np.float32)
    return F.f32_to_bf16_bits(x)


def test_group_shared_equals_per_head_when_g_is_1():
    q = _small_int_bits((1, 3, 256, 64), 1)
    k = _small_int_bits((1, 3, 256, 64), 2)
    a = S.select_blocks(q, k, 250, 64, 64, True, -1, 20, 100, 1, 1)
    b = S.select_blocks(q, k, 250, 64, 64, True, -1, 20, 100, 1, 1, group_shared=True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_group_shared_brute_force_and_identical_rows():
    """G = 4: every head of a group gets the same mask row; the shared scores
    equal the float64 dot product of the exact mean of the G heads' tile
    means with the key tile means (tile means of 64 rows of small integers
    are multiples of 1/64: every fp32 step is exact), and the chosen tiles are
    a brute-force sort by (-score, index) of the candidates."""
    B, Hq, Hkv, N, D, Bq, Bk = 1, 8, 2, 512, 64, 64, 64
    q = _small_int_bits((B, Hq, N, D), 3)
    k = _small_int_bits((B, Hkv, N, D), 4)
    mask, nfp, sc = S.select_blocks(q, k, N, Bq, Bk, False, 2, 0, 1, 0, 0, group_shared=True)
    qf = F.bf16_bits_to_f32(q).astype(np.float64)
    kf = F.bf16_bits_to_f32(k).astype(np.float64)
    n_t = N // Bq
    for g in range(Hkv):
        for h in range(g * 4, g * 4 + 4):
            assert np.array_equal(mask[0, h], mask[0, g * 4]) and np.array_equal(sc[0, h], sc[0, g * 4])
        qbar = qf[0, g * 4:g * 4 + 4].reshape(4, n_t, Bq, D).mean(axis=2).mean(axis=0)  # [n_t, D]
        kbar = kf[0, g].reshape(n_t, Bk, D).mean(axis=1)
        exact = qbar @ kbar.T
        assert np.array_equal(sc[0, g * 4].astype(np.float64), exact)
        for i in range(n_t):
            order = sorted(range(n_t), key=lambda j: (-exact[i, j], j))[:2]
            assert S.mask_to_sets(mask[0, g * 4, i], n_t) == sorted(order)


def test_group_shared_differs_from_per_head_in_general():
    q = F.f32_to_bf16_bits(np.random.default_rng(5).standard_normal((1, 4, 512, 64)).astype(np.float32))
    k = F.f32_to_bf16_bits(np.random.default_rng(6).standard_normal((1, 1, 512, 64)).astype(np.float32))
    per_head, _, _ = S.select_blocks(q, k, 512, 64, 64, False, 1, 0, 1, 0, 0)
    shared, _, _ = S.select_blocks(q, k, 512, 64, 64, False, 1, 0, 1, 0, 0, group_shared=True)
    assert not np.array_equal(per_head, shared)
    assert all(np.array_equal(shared[0, h], shared[0, 0]) for h in range(4))


# ---- max-pooled key logits (reading R37)
def test_maxkey_scores_brute_force():
    """Small-integer inputs: every fp32 step is exact, so the score is the
    float64 maximum over each tile's valid keys of (exact query-tile mean) .
    key; -inf for a tile with no valid key."""
    B, Hq, Hkv, N, D, Bq, Bk, nv = 1, 2, 1, 384, 64, 64, 64, 288  # a 32-row tile: its mean is exact
    q = _small_int_bits((B, Hq, N, D), 7)
    k = _small_int_bits((B, Hkv, N, D), 8)
    _, _, sc = S.select_blocks(q, k, nv, Bq, Bk, False, 1, 0, 1, 0, 0, heuristic="maxkey")
    qf = F.bf16_bits_to_f32(q).astype(np.float64)
    kf = F.bf16_bits_to_f32(k).astype(np.float64)
    for h in range(Hq):
        for i in range(N // Bq):
            rows = [r for r in range(i * Bq, (i + 1) * Bq) if r < nv]
            if not rows:
                continue
            qbar = qf[0, h, rows].mean(axis=0)
            for j in range(N // Bk):
                keys = [c for c in range(j * Bk, (j + 1) * Bk) if c < nv]
                want = max(qbar @ kf[0, 0, c] for c in keys) if keys else -np.inf
                assert sc[0, h, i, j] == want


def test_maxkey_finds_one_strong_key_that_the_mean_dilutes():
    """A single key aligned with the queries' shared direction, in an
    otherwise ordinary tile: its tile tops the max-pooled scores, while the
    mean over the tile's 64 keys dilutes it below tiles of mildly aligned keys."""
    rng = np.random.default_rng(9)
    N, D = 1024, 64
    common = rng.standard_normal(D).astype(np.float32)
    q = (rng.standard_normal((1, 1, N, D)) + common).astype(np.float32)
    k = rng.standard_normal((1, 1, N, D)).astype(np.float32)
    k[0, 0, 64 * 5:64 * 6] += 0.3 * common      # tile 5: every key a little aligned
    k[0, 0, 64 * 11 + 17] = 8.0 * common        # tile 11: one strong key
    qb, kb = f32_to_bf16_bits(q), f32_to_bf16_bits(k)
    mean_mask, _, mean_sc = S.select_blocks(qb, kb, N, 64, 64, False, 1, 0, 1, 0, 0)
    max_mask, _, max_sc = S.select_blocks(qb, kb, N, 64, 64, False, 1, 0, 1, 0, 0, heuristic="maxkey")
    assert all(S.mask_to_sets(max_mask[0, 0, i], 16) == [11] for i in range(16))
    assert all(S.mask_to_sets(mean_mask[0, 0, i], 16) == [5] for i in range(16))
