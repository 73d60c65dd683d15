"""Log-sum-exp merge of attention states — oracle (test infrastructure only).

[Guide, "Cascade attention for shared prefixes"] names merge_state and
merge_states as the operation that combines attention computed over disjoint
parts of a request's keys. The pages give only the name; the formula below
is the unique combination for which merging the states of any split of the
key set equals attention over the whole set (pinned by that property in the
tests):

    s   = log(sum_c exp(s_c))
    v   = sum_c exp(s_c - s) * v_c

A state with ``s = -inf`` (no keys) is the identity; merging only such
states gives ``(0, -inf)``.
"""
from __future__ import annotations

import numpy as np


def merge_state(v_a, s_a, v_b, s_b):
    """Merge two states: ``v_* [..., D]`` float64, ``s_* [...]`` (natural-log LSE)."""
    v_a = np.asarray(v_a, np.float64)
    v_b = np.asarray(v_b, np.float64)
    s_a = np.asarray(s_a, np.float64)
    s_b = np.asarray(s_b, np.float64)
    return merge_states(np.stack([v_a, v_b], axis=-2), np.stack([s_a, s_b], axis=-1))


def merge_states(v, s):
    """Merge k states along the state axis.

    ``v``: ``[..., k, D]``; ``s``: ``[..., k]``. Returns ``(v [..., D], s [...])``.
    """
    v = np.asarray(v, np.float64)
    s = np.asarray(s, np.float64)
    m = s.max(axis=-1)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    w = np.where(np.isneginf(s), 0.0, np.exp(s - m_safe[..., None]))
    tot = w.sum(axis=-1)
    tot_safe = np.where(live, tot, 1.0)
    out_v = (w[..., None] * v).sum(axis=-2) / tot_safe[..., None]
    out_v = np.where(live[..., None], out_v, 0.0)
    out_s = np.where(live, m_safe + np.log(tot_safe), -np.inf)
    return out_v, out_s
