"""Query preparation, score estimator and decode attention (oracle, float64).

TurboQuant article §六: the query is rotated (q Pi^T) and sketched (q S^T)
once per query; the score of a cached key is the MSE part plus the QJL part,
the scores become logits and go through softmax over the dequantised values.

The oracle deliberately evaluates the score in the *dequantised-key* form
(§五: <y, x~_mse> + ||r|| sqrt(pi/2)/m <S^T signs, y>) -- it rebuilds k^ in
the original space and takes <q, k^> -- so it shares no algebra with a
query-side implementation.  Softmax is the textbook two-pass form with the
maximum subtracted; logits are score / sqrt(d) unless another scale is given.
GQA: query head hq reads kv head hq // (Hq / Hkv).
"""
from __future__ import annotations

import numpy as np

from .keys import dequantize_keys
from .values import dequantize_values


def prepare_query(q, rotation, sketch, w: int):
    """q [n, d] -> (q_rot = Pi q [n, d] or None for w == 0, q_sk = S q [n, m])."""
    q = np.asarray(q, dtype=np.float64)
    S = np.asarray(sketch, dtype=np.float64)
    q_sk = q @ S.T
    if w == 0:
        return None, q_sk
    Pi = np.asarray(rotation, dtype=np.float64)
    return q @ Pi.T, q_sk


def scores(q, key_rows, rotation, sketch, centroids, w: int):
    """<q_h, k^_t> for queries q [G, d] against dequantised keys; [G, T]."""
    idx, bits, norm, rnorm = key_rows
    k_hat = dequantize_keys(idx, bits, norm, rnorm, rotation, sketch, centroids, w)
    return np.asarray(q, dtype=np.float64) @ k_hat.T


def softmax_attention(s, v_hat, softmax_scale: float):
    """Two-pass softmax over tokens; s [G, T], v_hat [T, d] -> out [G, d]."""
    logits = np.asarray(s, dtype=np.float64) * softmax_scale
    mx = np.max(logits, axis=1, keepdims=True)
    e = np.exp(logits - mx)
    p = e / np.sum(e, axis=1, keepdims=True)
    return p @ np.asarray(v_hat, dtype=np.float64)


def decode_slot(q, key_rows, value_rows, rotation, sketch, centroids, w: int,
                softmax_scale=None, group: int = 32):
    """Decode attention of the G query heads that share one KV slot.

    q [G, d]; key_rows = (idx, bits, norm, rnorm); value_rows = (codes, scale, vmin).
    Returns (scores [G, T], out [G, d])."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[1]
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(d)
    s = scores(q, key_rows, rotation, sketch, centroids, w)
    v_hat = dequantize_values(*value_rows, group=group)
    return s, softmax_attention(s, v_hat, softmax_scale)


def decode_slot_window(q, key_rows, value_rows, k_win, v_win, rotation, sketch, centroids, w: int,
                       softmax_scale=None, group: int = 32):
    """Decode attention over the compressed history and a recent-token window.

    TurboQuant article §六: the most recent tokens are kept at full precision in
    a ring buffer and the compressed path serves the older history; attention
    covers both.  The window's scores are the exact <q, k> and its values are
    the stored ones; the history's are the estimator and the dequantised
    values; one softmax runs over all of them (the order of tokens does not
    matter).  key_rows / value_rows may hold 0 tokens (no history yet) and the
    window may be empty.  Returns (window scores [G, W], out [G, d])."""
    q = np.asarray(q, dtype=np.float64)
    G, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(d)
    k_win = np.asarray(k_win, dtype=np.float64).reshape(-1, d)
    v_win = np.asarray(v_win, dtype=np.float64).reshape(-1, d)
    s_win = q @ k_win.T
    n_hist = len(key_rows[2])
    if n_hist > 0:
        s_hist = scores(q, key_rows, rotation, sketch, centroids, w)
        v_hist = dequantize_values(*value_rows, group=group)
    else:
        s_hist, v_hist = np.zeros((G, 0)), np.zeros((0, d))
    s = np.concatenate([s_hist, s_win], axis=1)
    v = np.concatenate([v_hist, v_win], axis=0)
    if s.shape[1] == 0:
        return s_win, np.zeros((G, d))
    return s_win, softmax_attention(s, v, softmax_scale)


def selection_query(q):
    """QUOKA article §1 (pre-aggregation over the KV heads, cosine scoring): the
    G query heads that share a KV head are reduced to one selection query, the
    sum of their unit vectors, so that <q_sel, k>/||k|| is the sum of the heads'
    cosine similarities with k times 1/||k|| -- a ranking by the group's mean
    cosine.  q [G, d] -> [d] (float64); a zero head contributes nothing."""
    q = np.asarray(q, dtype=np.float64)
    n = np.linalg.norm(q, axis=1, keepdims=True)
    u = np.divide(q, n, out=np.zeros_like(q), where=n > 0)
    return u.sum(axis=0)


def select_top_k(q, key_rows, rotation, sketch, centroids, w: int, budget: int):
    """QUOKA article §1 (dynamic top-K KV selection): the `budget` cached tokens
    with the largest cosine score cos_t = <q_sel, k^_t> / ||k_t|| (k^ the
    dequantised key, ||k_t|| its stored norm; 0 for a zero key), ties to the
    lower token index.  Returns the chosen token indices in increasing order
    and the cosine scores [T]."""
    q_sel = selection_query(q)
    norm = np.asarray(key_rows[2], dtype=np.float64)
    T = norm.shape[0]
    s = scores(q_sel[None, :], key_rows, rotation, sketch, centroids, w)[0] if T else np.zeros(0)
    cos = np.divide(s, norm, out=np.zeros_like(s), where=norm > 0)
    k = min(int(budget), T)
    order = np.argsort(-cos, kind="stable")[:k]
    return np.sort(order), cos


def decode_slot_top_k(q, key_rows, value_rows, rotation, sketch, centroids, w: int, budget: int,
                      softmax_scale=None, group: int = 32):
    """Decode attention of the G query heads of one KV slot over the QUOKA
    selection of at most `budget` tokens only.  Returns (chosen indices, out [G, d])."""
    sel, _ = select_top_k(q, key_rows, rotation, sketch, centroids, w, budget)
    sub_k = tuple(np.asarray(a)[sel] for a in key_rows)
    sub_v = _value_rows_subset(value_rows, sel)
    q = np.asarray(q, dtype=np.float64)
    if sel.size == 0:
        return sel, np.zeros_like(q)
    _, out = decode_slot(q, sub_k, sub_v, rotation, sketch, centroids, w, softmax_scale, group)
    return sel, out


def _value_rows_subset(value_rows, sel):
    codes, scale, vmin = value_rows
    return (np.asarray(codes)[sel], np.asarray(scale)[sel], np.asarray(vmin)[sel])


def select_top_k_blocks(q, key_rows, rotation, sketch, centroids, w: int, budget: int, block: int = 32):
    """QUOKA's dynamic top-K selection taken at the granularity of contiguous
    KV blocks (QUOKA article §2, the cache organised as contiguous memory
    blocks; a reading: the article ranks keys).  Tokens are grouped into
    consecutive blocks of `block` rows (the last one ragged); a block ranks by
    the largest cosine score cos_t (select_top_k) of its tokens, and the
    min(ceil(budget / block), number of blocks) blocks with the largest ranks
    are chosen, ties to the lower block.  Returns (chosen block indices in
    increasing order, the block ranks)."""
    _, cos = select_top_k(q, key_rows, rotation, sketch, centroids, w, 1)
    T = cos.shape[0]
    n_blk = (T + block - 1) // block
    rank = np.array([cos[b * block:(b + 1) * block].max() for b in range(n_blk)], dtype=np.float64)
    nb = max(1, min((int(budget) + block - 1) // block, n_blk)) if n_blk else 0
    order = np.argsort(-rank, kind="stable")[:nb]
    return np.sort(order), rank


def decode_slot_top_k_blocks(q, key_rows, value_rows, rotation, sketch, centroids, w: int, budget: int,
                             softmax_scale=None, group: int = 32, block: int = 32):
    """Decode attention of the G query heads of one KV slot over every token of
    the chosen blocks (select_top_k_blocks).  Returns (chosen blocks, out [G, d])."""
    blocks, _ = select_top_k_blocks(q, key_rows, rotation, sketch, centroids, w, budget, block)
    T = np.asarray(key_rows[2]).shape[0]
    rows = np.array([t for b in blocks for t in range(b * block, min((b + 1) * block, T))], dtype=np.int64)
    q = np.asarray(q, dtype=np.float64)
    if rows.size == 0:
        return blocks, np.zeros_like(q)
    sub_k = tuple(np.asarray(a)[rows] for a in key_rows)
    sub_v = _value_rows_subset(value_rows, rows)
    _, out = decode_slot(q, sub_k, sub_v, rotation, sketch, centroids, w, softmax_scale, group)
    return blocks, out
