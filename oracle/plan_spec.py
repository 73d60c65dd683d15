"""Split-KV work plan, reference procedure — oracle (test infrastructure only).

[Guide, "What FlashInfer is", idea 3] and [DeepDive, "The Architecture,
Unpacked" and "It In Action", step 1]: requests of very different lengths are
cut into tiles that are spread evenly over the compute units; the launch
shape is fixed while the tile assignment changes from step to step, so a
captured graph stays valid. The pages give no algorithm, so this module fixes
one integer-only procedure; the library's planner must produce exactly the
same tile list (bit-exact), and the attention result does not depend on the
choice.

Units. A *q tile* is a run of at most ``qo_tile`` query rows of one request
(``qo_tile = 1`` for decode: one row per request). Its visible key count is
``vis = kv_len`` (decode / non-causal) or ``min(kv_len, kv_len - qo_len + i1)``
(causal, ``i1`` = request-relative end of the tile's rows). Its cost in
page-units is ``vis_pages = ceil(vis / page_size)``.

Procedure:

1. ``units = num_kv_heads * sum(vis_pages)`` over all q tiles.
2. ``target = num_cu * tiles_per_cu``;
   ``P = max(min_chunk_pages, ceil(units / target))`` pages per chunk.
3. Each q tile is split into ``C = max(1, ceil(vis_pages / P))`` chunks;
   chunk c covers keys ``[c*P*ps, min((c+1)*P*ps, vis))``.
4. Q tiles are visited in order (request, tile). A tile with ``C > 1`` gets
   ``C * rows`` partial slots starting at the running count ``base``; the
   state of row r for chunk c goes to slot ``base + (r - q_begin)*C + c``,
   and every such row gets a merge entry ``(r, base + (r - q_begin)*C, C)``.
5. Tiles are emitted in order (request, q tile, chunk, kv head) as
   ``[b, kv_head, q_begin, q_end, tok_begin, tok_end, slot0, C]`` with
   ``slot0 = base + c`` (or -1 when ``C == 1``), then stably sorted by
   descending cost ``(tok_end - tok_begin) * (q_end - q_begin)`` so that
   in-order dispatch starts the longest tiles first.
6. More tiles, slots or merge entries than the capacities is an error.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

SUPPORTED_HEAD_DIM = (128,)
SUPPORTED_PAGE_SIZE = (16,)
SUPPORTED_GROUP = (1, 2, 4, 8)


class PlanSpecError(Exception):
    """``code`` is one of "INVALID", "UNSUPPORTED", "CAPACITY"."""

    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def default_knobs(num_kv_heads: int, max_batch: int, max_qo_tokens: int, is_append: bool,
                  num_cu: int = 0, tiles_per_cu: int = 0, min_chunk_pages: int = 0,
                  qo_tile: int = 0, max_tiles: int = 0, max_partials: int = 0,
                  max_merge: int = 0) -> dict:
    """Fill zero knobs with defaults; capacities are the worst case of the procedure."""
    num_cu = num_cu or 256
    tiles_per_cu = tiles_per_cu or (2 if is_append else 8)
    min_chunk_pages = min_chunk_pages or 1
    qo_tile = (qo_tile or 32) if is_append else 1
    target = num_cu * tiles_per_cu
    n_qtiles = (max_batch + _cdiv(max_qo_tokens, qo_tile)) if is_append else max_batch
    max_tiles = max_tiles or (target + num_kv_heads * n_qtiles)
    max_partials = max_partials or (2 * qo_tile * _cdiv(target, num_kv_heads))
    max_merge = max_merge or (qo_tile * _cdiv(target, num_kv_heads))
    return dict(num_cu=num_cu, tiles_per_cu=tiles_per_cu, min_chunk_pages=min_chunk_pages,
                qo_tile=qo_tile, max_tiles=max_tiles, max_partials=max_partials,
                max_merge=max_merge)


def validate(kv_indptr, kv_lens, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
             max_batch, qo_indptr=None, causal=False, max_qo_tokens=0):
    if batch < 0 or batch > max_batch:
        raise PlanSpecError("INVALID", "batch out of range")
    if num_kv_heads <= 0 or num_qo_heads <= 0 or num_qo_heads % num_kv_heads:
        raise PlanSpecError("INVALID", "num_qo_heads must be a positive multiple of num_kv_heads")
    if head_dim not in SUPPORTED_HEAD_DIM or page_size not in SUPPORTED_PAGE_SIZE:
        raise PlanSpecError("UNSUPPORTED", "head_dim/page_size")
    if num_qo_heads // num_kv_heads not in SUPPORTED_GROUP:
        raise PlanSpecError("UNSUPPORTED", "group size")
    if kv_indptr[0] != 0:
        raise PlanSpecError("INVALID", "kv_indptr[0] != 0")
    for b in range(batch):
        n = int(kv_indptr[b + 1]) - int(kv_indptr[b])
        L = int(kv_lens[b])
        if n < 0:
            raise PlanSpecError("INVALID", "kv_indptr not monotone")
        if n == 0:
            if L != 0:
                raise PlanSpecError("INVALID", "kv_len > 0 with no pages")
        elif not ((n - 1) * page_size < L <= n * page_size):
            raise PlanSpecError("INVALID", "kv_len inconsistent with page count")
    if qo_indptr is not None:
        if qo_indptr[0] != 0:
            raise PlanSpecError("INVALID", "qo_indptr[0] != 0")
        for b in range(batch):
            ql = int(qo_indptr[b + 1]) - int(qo_indptr[b])
            if ql < 0:
                raise PlanSpecError("INVALID", "qo_indptr not monotone")
            if causal and ql > int(kv_lens[b]):
                raise PlanSpecError("INVALID", "causal qo_len exceeds kv_len")
        if int(qo_indptr[batch]) > max_qo_tokens:
            raise PlanSpecError("INVALID", "too many query rows for max_qo_tokens")


def plan_spec(kv_indptr: Sequence[int], kv_lens: Sequence[int], batch: int,
              num_qo_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
              max_batch: int, qo_indptr: Optional[Sequence[int]] = None, causal: bool = False,
              max_qo_tokens: int = 0, **knobs) -> dict:
    """Reference plan. Returns tiles ``int32 [n, 8]``, merge ``int32 [m, 4]`` and scalars."""
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    is_append = qo_indptr is not None
    validate(kv_indptr, kv_lens, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
             max_batch, None if qo_indptr is None else np.asarray(qo_indptr, np.int64), causal,
             max_qo_tokens)
    k = default_knobs(num_kv_heads, max_batch, max_qo_tokens, is_append, **knobs)
    ps = page_size
    qtiles = []                     # (b, q_begin, q_end, vis)
    for b in range(batch):
        L = int(kv_lens[b])
        if not is_append:
            qtiles.append((b, b, b + 1, L))
            continue
        r0, r1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        ql = r1 - r0
        for t0 in range(0, ql, k["qo_tile"]):
            t1 = min(ql, t0 + k["qo_tile"])
            vis = min(L, L - ql + t1) if causal else L
            qtiles.append((b, r0 + t0, r0 + t1, vis))
    units = num_kv_heads * sum(_cdiv(v, ps) for (_, _, _, v) in qtiles)
    target = k["num_cu"] * k["tiles_per_cu"]
    P = max(k["min_chunk_pages"], _cdiv(units, target))
    tiles, merge = [], []
    slots = 0
    for (b, q0, q1, vis) in qtiles:
        C = max(1, _cdiv(_cdiv(vis, ps), P))
        base = -1
        if C > 1:
            base = slots
            slots += C * (q1 - q0)
            for r in range(q0, q1):
                merge.append((r, base + (r - q0) * C, C, 0))
        for c in range(C):
            t0 = c * P * ps
            t1 = min((c + 1) * P * ps, vis)
            for h in range(num_kv_heads):
                tiles.append((b, h, q0, q1, t0, t1, base + c if C > 1 else -1, C))
    order = sorted(range(len(tiles)),
                   key=lambda i: -((tiles[i][5] - tiles[i][4]) * (tiles[i][3] - tiles[i][2])))
    tiles = [tiles[i] for i in order]
    if len(tiles) > k["max_tiles"]:
        raise PlanSpecError("CAPACITY", "too many tiles")
    if slots > k["max_partials"]:
        raise PlanSpecError("CAPACITY", "too many partial slots")
    if len(merge) > k["max_merge"]:
        raise PlanSpecError("CAPACITY", "too many merge rows")
    return dict(
        tiles=np.asarray(tiles, dtype=np.int32).reshape(-1, 8),
        merge=np.asarray(merge, dtype=np.int32).reshape(-1, 4),
        chunk_pages=P, target=target, num_slots=slots, knobs=k,
    )
