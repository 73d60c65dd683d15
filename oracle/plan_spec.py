"""Split-KV work plan, reference procedure — oracle (test infrastructure only).

[Guide, "What FlashInfer is", idea 3] and [DeepDive, "The Architecture,
Unpacked", "It In Action" step 1 and "Why This Design Works"]: requests of
very different lengths are cut into pieces spread evenly over the GPU; the
launch shape is fixed while the assignment changes from step to step, so a
captured graph stays valid. The pages give no algorithm, so this module fixes
one integer-only procedure per mode; the library's planner must produce the
same arrays bit for bit, and the attention result does not depend on the
choice.

A *unit* is one kv head of one q tile. A q tile is one request in decode, or
up to ``qo_tile`` query rows of one request in append; its visible key count
is ``vis = kv_len`` (decode, non-causal) or ``min(kv_len, kv_len - qo_len +
i1)`` (causal; ``i1`` = request-relative end of its rows), and its cost in
pages is ``ceil(vis / page_size)``. Units are ordered (q tile, kv head).

Decode — static work lists, balanced by dealing pieces largest first:

1. ``S = num_cu * tiles_per_cu`` worker waves; ``NS = max(1, S *
   pieces_per_worker // num_kv_heads)`` bins (``pieces_per_worker`` defaults
   to ``PIECES_PER_WORKER``). A piece costs its pages plus ``c0`` =
   ``PIECE_COST_PAGES`` (8 for an E4M3 pool, else 4): the set-up and
   epilogue of a piece, in pages of streaming time.
2. ``N`` = total pages of the requests (``n_b = ceil(kv_len_b / ps)``);
   piece size ``Q = min(MAX_PIECE_PAGES, max(1, min_chunk_pages,
   ceil((N + c0 * batch) / NS)))``, the bins' mean cost.
3. Request b splits into ``C_b = max(1, ceil(n_b / Q))`` pieces; piece i
   covers pages ``[i Q, min((i+1) Q, n_b))`` (a request with no pages is one
   empty piece).
4. Pieces, in descending pages (stable on (b, i)), are dealt to the NS bins,
   each to the bin with the least cost so far (lowest index on ties); a bin
   keeps its pieces in dealing order.
5. Requests with ``C_b > 1`` get ``C_b`` partial slots per kv head (request
   order, running count ``base_b``; kv head h owns ``base_b + h C_b ..``);
   piece i of unit (b, h) writes slot ``base_b + h C_b + i``; ``base = slot
   = -1`` when ``C_b == 1``. Merge entry per split unit: ``(b, kv_head,
   base_b + h C_b, C_b)``, in (request, kv head) order.
6. Work list ``j = bin * num_kv_heads + h`` is bin ``bin``'s pieces for kv
   head h, as tiles ``[b, h, kv_indptr[b], unit base, key0, key1, slot,
   C_b]`` (keys clipped to kv_len); it runs on wave ``j mod S``. The tile
   list is wave-major (a wave's lists in increasing j) and ``worker_ptr[w]
   .. worker_ptr[w+1]-1`` are wave w's tiles. The num_kv_heads waves of a bin
   read the kv heads of the same pages, i.e. whole token rows, at about the
   same time.

Append — uniform chunks:

1. ``target = num_cu * tiles_per_cu``; ``units = num_kv_heads * sum(cost)``;
   ``P = max(min_chunk_pages, ceil(units / target))`` pages per chunk.
2. Each q tile splits into ``C = max(1, ceil(cost / P))`` chunks; chunk c
   covers keys ``[c P ps, min((c+1) P ps, vis))``.
3. Units with ``C > 1`` get ``C * rows`` slots (unit order, running count
   ``base``); chunk c of the unit writes row r to slot
   ``base + c*rows + (r - q0)``. Merge entry per split unit:
   ``(q0, kv_head, base, C)``.
4. Tiles ``[b, kv_head, q0, q1, key0, key1, slot0, C]`` with
   ``slot0 = base + c*rows`` (-1 when ``C == 1``) are emitted in order
   (request, q tile, kv head, chunk); a tile's cost is
   ``(key1 - key0) * (q1 - q0)``.
5. XCD bins. A *group* is one (request, kv head): all its q tiles and
   chunks read the same keys. Groups, in descending total cost (stable on
   ``b * num_kv_heads + kv_head``), are dealt to ``XCD_BINS`` (8) bins, each
   to the bin with the least total cost so far (lowest bin on ties). The
   tile list is bin 0, bin 1, ...; inside a bin, groups in dealing order and
   each group's tiles by descending cost (stable on emission order);
   ``worker_ptr[0..8]`` are the bin offsets. The GPU hands workgroups to
   its 8 XCDs round-robin and workgroup i runs bin ``i mod 8``, so a group's
   tiles run together on one XCD and share its L2.

More tiles, slots or merge entries than the capacities is an error.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

SUPPORTED_HEAD_DIM = (128,)
SUPPORTED_PAGE_SIZE = (16,)
SUPPORTED_GROUP = (1, 2, 4, 8)
MAX_PIECE_PAGES = 128
XCD_BINS = 8
APPEND_COLS = 256  # query columns of an append tile (G heads x APPEND_COLS / G rows)
PIECES_PER_WORKER = 1
PIECE_COST_PAGES = {"16-bit": 4, "e4m3": 8}


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
                  max_merge: int = 0, pieces_per_worker: int = 0, group: int = 1) -> dict:
    """Fill zero knobs with defaults; capacities are the worst case of the procedure.

    An append q tile holds at most ``APPEND_COLS / group`` rows (the library's
    tiles have APPEND_COLS query columns = group heads x rows); that is also
    the default."""
    num_cu = num_cu or 256
    pieces_per_worker = 0 if is_append else (pieces_per_worker or PIECES_PER_WORKER)
    tiles_per_cu = tiles_per_cu or (2 if is_append else 4)
    min_chunk_pages = min_chunk_pages or 1
    qo_tile = (qo_tile or APPEND_COLS // group) if is_append else 1
    if is_append and qo_tile > APPEND_COLS // group:
        raise PlanSpecError("UNSUPPORTED", "qo_tile larger than APPEND_COLS / group")
    target = num_cu * tiles_per_cu
    if is_append:
        n_qtiles = max_batch + _cdiv(max_qo_tokens, qo_tile)
        max_tiles = max_tiles or (target + num_kv_heads * n_qtiles)
        max_partials = max_partials or (2 * qo_tile * target)
        max_merge = max_merge or target
    else:
        units = max_batch * num_kv_heads
        max_tiles = max_tiles or (pieces_per_worker * target + units)
        max_partials = max_partials or (pieces_per_worker * target + units)
        max_merge = max_merge or units
    return dict(num_cu=num_cu, tiles_per_cu=tiles_per_cu, min_chunk_pages=min_chunk_pages,
                qo_tile=qo_tile, max_tiles=max_tiles, max_partials=max_partials,
                max_merge=max_merge, pieces_per_worker=pieces_per_worker)


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


def _decode_plan(kv_indptr, kv_lens, batch, Hkv, ps, k, c0):
    S = k["num_cu"] * k["tiles_per_cu"]
    NS = max(1, S * k["pieces_per_worker"] // Hkv)
    n = [_cdiv(int(kv_lens[b]), ps) for b in range(batch)]
    Q = min(MAX_PIECE_PAGES, max(1, k["min_chunk_pages"], _cdiv(sum(n) + c0 * batch, NS)))
    pieces, C = [], []                      # (b, first page, end page, i)
    for b in range(batch):
        C.append(max(1, _cdiv(n[b], Q)))
        for i in range(C[b]):
            pieces.append((b, i * Q, min((i + 1) * Q, n[b]), i))
    dealt = sorted(range(len(pieces)), key=lambda x: -(pieces[x][2] - pieces[x][1]))
    cost, bins = [0] * NS, [[] for _ in range(NS)]
    for x in dealt:
        j = min(range(NS), key=lambda y: (cost[y], y))
        bins[j].append(x)
        cost[j] += pieces[x][2] - pieces[x][1] + c0
    base, merge, slots = {}, [], 0
    for b in range(batch):
        base[b] = -1
        if C[b] > 1:
            base[b] = slots
            merge += [(b, h, slots + h * C[b], C[b]) for h in range(Hkv)]
            slots += C[b] * Hkv
    tiles, wptr = [], []
    for w in range(S):
        wptr.append(len(tiles))
        for j in range(w, NS * Hkv, S):
            sg, h = divmod(j, Hkv)
            for x in bins[sg]:
                b, p0, p1, i = pieces[x]
                ub = base[b] + h * C[b] if base[b] >= 0 else -1
                tiles.append((b, h, int(kv_indptr[b]), ub, p0 * ps, min(p1 * ps, int(kv_lens[b])),
                              ub + i if ub >= 0 else -1, C[b]))
    wptr.append(len(tiles))
    return tiles, merge, slots, wptr, Q


def _append_plan(kv_lens, batch, Hkv, ps, qo_indptr, causal, k):
    qtiles = []                         # (b, q0, q1, vis)
    for b in range(batch):
        L = int(kv_lens[b])
        r0, r1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        ql = r1 - r0
        for t0 in range(0, ql, k["qo_tile"]):
            t1 = min(ql, t0 + k["qo_tile"])
            vis = min(L, L - ql + t1) if causal else L
            qtiles.append((b, r0 + t0, r0 + t1, vis))
    units = Hkv * sum(_cdiv(v, ps) for (_, _, _, v) in qtiles)
    target = k["num_cu"] * k["tiles_per_cu"]
    P = max(k["min_chunk_pages"], _cdiv(units, target))
    tiles, merge, slots = [], [], 0
    for (b, q0, q1, vis) in qtiles:
        C = max(1, _cdiv(_cdiv(vis, ps), P))
        rows = q1 - q0
        for h in range(Hkv):
            base = -1
            if C > 1:
                base = slots
                slots += C * rows
                merge.append((q0, h, base, C))
            for c in range(C):
                t0 = c * P * ps
                t1 = min((c + 1) * P * ps, vis)
                tiles.append((b, h, q0, q1, t0, t1, base + c * rows if C > 1 else -1, C))
    cost = [(t[5] - t[4]) * (t[3] - t[2]) for t in tiles]
    ngroups = batch * Hkv
    gcost = [0] * ngroups
    for t, c in zip(tiles, cost):
        gcost[t[0] * Hkv + t[1]] += c
    bin_of, seq_of, bcost = [0] * ngroups, [0] * ngroups, [0] * XCD_BINS
    for n, g in enumerate(sorted(range(ngroups), key=lambda g: -gcost[g])):
        x = min(range(XCD_BINS), key=lambda j: bcost[j])
        bin_of[g], seq_of[g] = x, n
        bcost[x] += gcost[g]
    gid = [t[0] * Hkv + t[1] for t in tiles]
    order = sorted(range(len(tiles)), key=lambda i: (bin_of[gid[i]], seq_of[gid[i]], -cost[i]))
    counts = [0] * XCD_BINS
    for i in order:
        counts[bin_of[gid[i]]] += 1
    wptr = [0]
    for x in range(XCD_BINS):
        wptr.append(wptr[-1] + counts[x])
    return [tiles[i] for i in order], merge, slots, wptr, P


def plan_spec(kv_indptr: Sequence[int], kv_lens: Sequence[int], batch: int,
              num_qo_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
              max_batch: int, qo_indptr: Optional[Sequence[int]] = None, causal: bool = False,
              max_qo_tokens: int = 0, kv_dtype: Optional[str] = None, **knobs) -> dict:
    """Reference plan: tiles ``int32 [n, 8]``, merge ``int32 [m, 4]``, worker_ptr
    ``int32 [S+1]`` (decode: worker waves; append: the 8 XCD bins) and scalars.
    ``kv_dtype="e4m3"`` plans a decode over an FP8 pool (another piece cost)."""
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    is_append = qo_indptr is not None
    validate(kv_indptr, kv_lens, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
             max_batch, None if qo_indptr is None else np.asarray(qo_indptr, np.int64), causal,
             max_qo_tokens)
    k = default_knobs(num_kv_heads, max_batch, max_qo_tokens, is_append,
                      group=num_qo_heads // num_kv_heads, **knobs)
    if is_append:
        tiles, merge, slots, wptr, P = _append_plan(kv_lens, batch, num_kv_heads, page_size,
                                                    np.asarray(qo_indptr, np.int64), causal, k)
    else:
        c0 = PIECE_COST_PAGES["e4m3" if kv_dtype == "e4m3" else "16-bit"]
        tiles, merge, slots, wptr, P = _decode_plan(kv_indptr, kv_lens, batch, num_kv_heads,
                                                    page_size, k, c0)
    if len(tiles) > k["max_tiles"]:
        raise PlanSpecError("CAPACITY", "too many tiles")
    if slots > k["max_partials"]:
        raise PlanSpecError("CAPACITY", "too many partial slots")
    if len(merge) > k["max_merge"]:
        raise PlanSpecError("CAPACITY", "too many merge entries")
    return dict(
        tiles=np.asarray(tiles, dtype=np.int32).reshape(-1, 8),
        merge=np.asarray(merge, dtype=np.int32).reshape(-1, 4),
        worker_ptr=None if wptr is None else np.asarray(wptr, dtype=np.int32),
        chunk_pages=P, target=k["num_cu"] * k["tiles_per_cu"], num_slots=slots, knobs=k,
    )
