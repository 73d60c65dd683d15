"""Brute-force attention with pure-Python loops — oracle self-check (tiny inputs).

Written independently of the vectorised oracle: nested lists, ``math.fsum``
for every sum, no numpy. Used only to pin ``oracle.attention`` on tiny cases
(a handful of keys, head_dim <= 8).
"""
from __future__ import annotations

import math


def brute_attention_row(q, keys, values, scale):
    """One query row against lists of key/value rows. Returns (out, lse)."""
    if not keys:
        return [0.0] * len(q), -math.inf
    scores = [scale * math.fsum(qd * kd for qd, kd in zip(q, k)) for k in keys]
    top = max(scores)
    weights = [math.exp(s - top) for s in scores]
    total = math.fsum(weights)
    out = [math.fsum(w * v[d] for w, v in zip(weights, values)) / total
           for d in range(len(values[0]))]
    return out, top + math.log(total)


def brute_paged(q_rows, pool, kv_indptr, kv_indices, last_page_len, page_size, request_of_row,
                visible_of_row, num_qo_heads, num_kv_heads, scale):
    """Attention for every (row, head) with explicit page walking.

    ``pool[page][kv][slot][head][d]`` nested lists of floats (kv 0 = K, 1 = V);
    ``q_rows[row][head][d]``. Row r belongs to request ``request_of_row[r]``
    and sees its first ``visible_of_row[r]`` tokens.
    """
    group = num_qo_heads // num_kv_heads
    out, lse = [], []
    for r, qr in enumerate(q_rows):
        b = request_of_row[r]
        n = kv_indptr[b + 1] - kv_indptr[b]
        kv_len = 0 if n == 0 else (n - 1) * page_size + last_page_len[b]
        vis = max(0, min(kv_len, visible_of_row[r]))
        row_out, row_lse = [], []
        for h in range(num_qo_heads):
            hk = h // group
            keys, vals = [], []
            for t in range(vis):
                page = kv_indices[kv_indptr[b] + t // page_size]
                slot = t % page_size
                keys.append(pool[page][0][slot][hk])
                vals.append(pool[page][1][slot][hk])
            o, s = brute_attention_row(qr[h], keys, vals, scale)
            row_out.append(o)
            row_lse.append(s)
        out.append(row_out)
        lse.append(row_lse)
    return out, lse
