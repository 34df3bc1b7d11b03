"""Block selection: which query-key tiles run in FP16 (test infrastructure).

ThriftAttention (abstract): "a heuristic rapidly selects a small number of
important query-key block pairs for FP16 precision"; the error matters most
for the most important query-key interactions.  HyQuant (summary, abstract):
vertical-line tokens and a local sliding window are kept in full precision.
The pages give no formula; the readings used here (R8-R11) are:

* importance estimate s_ij = mean(Q over query tile i) . mean(K over key tile j)
  (the logit of the tile means), fp32 with a fixed operation order;
* forced tiles: key tiles j < sink_tiles (the sink column) and the local
  window, i.e. the key tiles meeting rows [qs - (w-1)*Bk, qe] of the query
  tile (its diagonal tiles plus w-1 tiles before them);
* budget per query tile k_i = topk, or ceil(num*|V_i|/den) in integers,
  capped at the number of non-forced candidates; candidates ordered by
  descending score, ties to the lower tile index;
* optionally one mask per kv group (R35, after HyQuant's vertical-line
  signals shared by the query heads of a group): the G heads' tile means are
  averaged (fp32 sum in head order, one division by G) and scored as above;
* optionally max-pooled key logits (R37): a tile's score is the largest logit
  of the query-tile mean against the tile's individual keys.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f32


def tile_sets(n_valid, N, Bq, Bk, causal, sink_tiles, local_tiles):
    """Per query tile i: (valid key tiles V_i, forced tiles F_i), as sorted lists.

    Query tiles with qs >= n_valid get empty sets (their rows output 0)."""
    n_qt, n_kt = N // Bq, N // Bk
    out = []
    for i in range(n_qt):
        qs = i * Bq
        if qs >= n_valid:
            out.append(([], []))
            continue
        qe = min(qs + Bq, n_valid) - 1
        valid = [j for j in range(n_kt) if j * Bk < n_valid and (not causal or j * Bk <= qe)]
        lo = qs - (local_tiles - 1) * Bk
        forced = []
        for j in valid:
            sink = j < sink_tiles
            local = local_tiles >= 1 and (j + 1) * Bk - 1 >= lo and j * Bk <= qe
            if sink or local:
                forced.append(j)
        out.append((valid, forced))
    return out


def _tile_means(x: np.ndarray, n_valid: int, T: int) -> np.ndarray:
    """fp32 mean over each tile of T rows of x[N, D] (rows >= n_valid excluded):
    sequential fp32 sum in ascending row order, then one fp32 division by the
    row count.  Tiles with no valid row give zeros."""
    N, D = x.shape
    nt = N // T
    xt = x.reshape(nt, T, D)
    acc = np.zeros((nt, D), dtype=np.float32)
    cnt = np.zeros(nt, dtype=np.float32)
    rows = np.arange(N).reshape(nt, T)
    for r in range(T):
        ok = rows[:, r] < n_valid
        acc = np.where(ok[:, None], (acc + xt[:, r, :]).astype(np.float32), acc)
        cnt = cnt + ok.astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        mean = (acc / np.where(cnt == 0, np.float32(1), cnt)[:, None]).astype(np.float32)
    return np.where(cnt[:, None] == 0, np.float32(0), mean)


def pooled_means(q_bits, k_bits, n_valid, Bq, Bk):
    """Tile means of Q per query head [B,Hq,n_qt,D] and of K per kv head
    [B,Hkv,n_kt,D], float32 (reading R8)."""
    q = bf16_bits_to_f32(q_bits)
    k = bf16_bits_to_f32(k_bits)
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    qm = np.stack([np.stack([_tile_means(q[b, h], n_valid, Bq) for h in range(Hq)]) for b in range(B)])
    km = np.stack([np.stack([_tile_means(k[b, h], n_valid, Bk) for h in range(Hkv)]) for b in range(B)])
    return qm, km


def tile_scores(qm: np.ndarray, km: np.ndarray) -> np.ndarray:
    """s[i, j] for one head: acc = fl32(acc + fl32(qm[i,d]*km[j,d])) for d
    ascending, starting from +0 (no fused multiply-add)."""
    n_qt, D = qm.shape
    n_kt = km.shape[0]
    acc = np.zeros((n_qt, n_kt), dtype=np.float32)
    for d in range(D):
        prod = (qm[:, d][:, None] * km[:, d][None, :]).astype(np.float32)
        acc = (acc + prod).astype(np.float32)
    return acc


def tile_scores_maxkey(qm: np.ndarray, k_rows: np.ndarray, n_valid: int, Bk: int) -> np.ndarray:
    """Max-pooled key logits (reading R37): s[i, j] = the largest, over the
    valid keys of key tile j, of qm[i] . k_key with the arithmetic of
    ``tile_scores`` (fl32 products, fl32 sums, d ascending, from +0); -inf for
    a tile with no valid key.  Unlike the mean-pooled key tile, one strong key
    keeps its full weight in the score of its tile."""
    n_qt, D = qm.shape
    N = k_rows.shape[0]
    acc = np.zeros((n_qt, N), dtype=np.float32)
    for d in range(D):
        prod = (qm[:, d][:, None] * k_rows[:, d][None, :]).astype(np.float32)
        acc = (acc + prod).astype(np.float32)
    acc[:, n_valid:] = -np.inf
    return acc.reshape(n_qt, N // Bk, Bk).max(axis=2)


def budget(topk, ratio_num, ratio_den, n_valid_tiles, n_candidates):
    """k_i (reading R9): topk if topk >= 0, else ceil(num*|V_i|/den) computed
    in integers; never more than the number of candidates."""
    if topk >= 0:
        k = topk
    else:
        k = -((-ratio_num * n_valid_tiles) // ratio_den)
    return min(k, n_candidates)


def group_tile_means(qm_heads: np.ndarray) -> np.ndarray:
    """Shared query-tile means of one kv group (reading R35): the G heads' tile
    means [G, n_qt, D] summed in fp32 head by head (ascending), then one fp32
    division by G."""
    acc = np.zeros(qm_heads.shape[1:], dtype=np.float32)
    for h in range(qm_heads.shape[0]):
        acc = (acc + qm_heads[h]).astype(np.float32)
    return (acc / np.float32(qm_heads.shape[0])).astype(np.float32)


def select_blocks(q_bits, k_bits, n_valid, Bq, Bk, causal, topk, ratio_num, ratio_den,
                  sink_tiles, local_tiles, group_shared=False, heuristic="mean"):
    """Return (mask u32 [B,Hq,n_qt,ceil(n_kt/32)], n_fp16 i32 [B,Hq,n_qt],
    scores f32 [B,Hq,n_qt,n_kt]).  Bit j%32 of word j//32 is set when key tile
    j runs in FP16 for that query tile.  Scores are given for every tile pair
    (also non-candidates) for inspection.  With ``group_shared`` (reading R35)
    the G query heads of a kv group score with their shared tile means
    (``group_tile_means``) and so share one mask.  ``heuristic`` "maxkey"
    scores with the max-pooled key logits (R37) instead of the key tile means."""
    B, Hq, N, D = q_bits.shape
    Hkv = k_bits.shape[1]
    G = Hq // Hkv
    n_qt, n_kt = N // Bq, N // Bk
    nw = (n_kt + 31) // 32
    sets = tile_sets(n_valid, N, Bq, Bk, causal, sink_tiles, local_tiles)
    qm, km = pooled_means(q_bits, k_bits, n_valid, Bq, Bk)
    if heuristic == "maxkey":
        kf = bf16_bits_to_f32(k_bits).copy()
        kf[..., n_valid:, :] = 0.0
    mask = np.zeros((B, Hq, n_qt, nw), dtype=np.uint32)
    nfp = np.zeros((B, Hq, n_qt), dtype=np.int32)
    scores = np.zeros((B, Hq, n_qt, n_kt), dtype=np.float32)
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            qh = group_tile_means(qm[b, kv * G:(kv + 1) * G]) if group_shared else qm[b, h]
            s = tile_scores(qh, km[b, kv]) if heuristic == "mean" else tile_scores_maxkey(qh, kf[b, kv], n_valid, Bk)
            scores[b, h] = s
            for i in range(n_qt):
                valid, forced = sets[i]
                fset = set(forced)
                cand = [j for j in valid if j not in fset]
                k = budget(topk, ratio_num, ratio_den, len(valid), len(cand))
                # descending score; equal scores keep ascending tile index (stable sort)
                order = sorted(cand, key=lambda j: (-float(s[i, j]), j))
                chosen = set(forced) | set(order[:k])
                for j in chosen:
                    mask[b, h, i, j // 32] |= np.uint32(1) << np.uint32(j % 32)
                nfp[b, h, i] = len(chosen)
    return mask, nfp, scores


def mask_to_sets(mask_row: np.ndarray, n_kt: int):
    """Promoted tile indices of one mask row (u32 words)."""
    return [j for j in range(n_kt) if (int(mask_row[j // 32]) >> (j % 32)) & 1]


# ---------------------------------------------------------------- vertical lines
# HyQuant (summary and abstract): besides a local window, a small set of
# "vertical-line" tokens -- key positions that queries across the whole
# sequence attend to -- stays in full precision, found from cheap
# attention-pattern signals.  The pages give no formula; the readings are:
#
# * probe vector of a head (R28): the mean of its valid query tiles' means,
#   i.e. sum over query tiles i ascending (tiles with a valid row) of the fp32
#   tile mean, one fp32 division by the tile count.  With group sharing (R31)
#   the sum runs over the G query heads of the kv group (head ascending, then
#   tile ascending) and is divided once by G times the tile count;
# * line score of key j: v_j = probe . k_j with the arithmetic of the tile
#   scores (fl32 product, fl32 sum, d ascending, from +0);
# * lines: the first min(sink_tokens, n_valid) keys (attention sink / CLS
#   token), then the top (n_lines - sinks) remaining valid keys by descending
#   score, ties to the lower index; listed ascending, padded with -1.


def line_probe(qm_heads: np.ndarray, n_valid: int, Bq: int) -> np.ndarray:
    """qm_heads: tile means [G', n_qt, D] of the heads that share the probe."""
    n_vt = -(-n_valid // Bq)  # query tiles holding at least one valid row
    acc = np.zeros(qm_heads.shape[-1], dtype=np.float32)
    for h in range(qm_heads.shape[0]):
        for i in range(n_vt):
            acc = (acc + qm_heads[h, i]).astype(np.float32)
    return (acc / np.float32(qm_heads.shape[0] * n_vt)).astype(np.float32)


def line_scores(probe: np.ndarray, k_rows: np.ndarray) -> np.ndarray:
    """v_j for every row of k_rows [N, D] (fp32): sequential, never fused."""
    acc = np.zeros(k_rows.shape[0], dtype=np.float32)
    for d in range(k_rows.shape[1]):
        acc = (acc + (k_rows[:, d] * probe[d]).astype(np.float32)).astype(np.float32)
    return acc


def choose_lines(v: np.ndarray, n_valid: int, n_lines: int, sink_tokens: int) -> np.ndarray:
    """Ascending line list (int32 [n_lines], -1 padded) from scores v [N]."""
    s = min(sink_tokens, n_valid, n_lines)
    cand = list(range(s, n_valid))
    k = min(n_lines - s, len(cand))
    order = sorted(cand, key=lambda j: (-float(v[j]), j))
    chosen = sorted(list(range(s)) + order[:k])
    out = np.full(n_lines, -1, dtype=np.int32)
    out[:len(chosen)] = chosen
    return out


def select_lines(q_bits, k_bits, n_valid, Bq, n_lines, sink_tokens, group_shared=False):
    """Return (lines int32 [B,Hq,n_lines], scores f32 [B,Hq,N]); scores of keys
    j >= n_valid are -inf (they are never lines)."""
    B, Hq, N, D = q_bits.shape
    Hkv = k_bits.shape[1]
    G = Hq // Hkv
    q = bf16_bits_to_f32(q_bits)
    k = bf16_bits_to_f32(k_bits)
    lines = np.full((B, Hq, n_lines), -1, dtype=np.int32)
    scores = np.full((B, Hq, N), -np.inf, dtype=np.float32)
    for b in range(B):
        qm = np.stack([_tile_means(q[b, h], n_valid, Bq) for h in range(Hq)])
        for h in range(Hq):
            kv = h // G
            heads = qm[kv * G:(kv + 1) * G] if group_shared else qm[h:h + 1]
            probe = line_probe(heads, n_valid, Bq)
            kr = k[b, kv].copy()
            kr[n_valid:] = 0.0
            v = line_scores(probe, kr)
            v[n_valid:] = -np.inf
            scores[b, h] = v
            lines[b, h] = choose_lines(v, n_valid, n_lines, sink_tokens)
    return lines, scores


def used_lines(row: np.ndarray, n_valid: int):
    """Keys of one line list that take part (reading R30): an entry counts when
    0 <= key < n_valid and it exceeds every earlier entry; anything else (the
    -1 padding, duplicates, out-of-order or out-of-range values) is ignored."""
    out, top = [], -1
    for key in (int(x) for x in row):
        if 0 <= key < n_valid and key > top:
            out.append(key)
        top = max(top, key)
    return out
