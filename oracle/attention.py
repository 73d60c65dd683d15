"""fp64 attention over a paged KV cache — oracle (test infrastructure only).

Definitions followed:

* Page table [DeepDive, "Snippet One: Paged KV-Cache Attention and MLA"]: the
  KV cache lives in fixed-size pages of a pool; each request owns a list of
  page ids, flattened as CSR (``kv_indptr``/``kv_indices``), and
  ``last_page_len`` says how many tokens fill its last page. Reading taken:
  ``kv_len = (n_pages - 1) * page_size + last_page_len`` (0 for a request
  with no pages), token ``t`` lives in page ``indices[indptr[b] + t // ps]``
  at slot ``t % ps``, NHD layout ``[pages, (K,V), ps, kv_heads, head_dim]``.
* Attention [Guide, "What FlashInfer is" (block-sparse KV format);
  DeepDive intro (fused FlashAttention-style attention)]: for query row q of
  head h, ``s_j = scale * <q, k_j>`` over the visible keys of kv head
  ``h // G`` (G = q heads per kv head), ``out = sum_j softmax(s)_j v_j`` and
  ``lse = log(sum_j exp(s_j))`` (natural log). The pages do not print the
  formula; this is the textbook scaled-dot-product attention, with
  ``scale = 1/sqrt(head_dim)`` unless given. An empty key set gives
  ``out = 0``, ``lse = -inf``.
* Causal append [Guide, "Features (from the repository README)": decode,
  prefill and append kernels]: request b has ``qo_len`` new rows that are
  already in its pages; row i sits at absolute position
  ``kv_len - qo_len + i`` and sees keys ``j <= position`` (bottom-right
  alignment, the reading under which decode is the qo_len = 1 case).
* Cascade [Guide, "Cascade attention for shared prefixes"]: attention over a
  shared prefix, attention over each private suffix, combined by
  merge_state; equal to attention over prefix ++ suffix.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .fp8 import e4m3_value
from .merge import merge_state


def upcast(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored bf16/fp16 bit patterns (or E4M3 byte codes,
    unscaled) to float64."""
    if dtype == "e4m3":
        return e4m3_value(bits)
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def request_pages(kv_indptr: np.ndarray, kv_indices: np.ndarray, b: int) -> np.ndarray:
    """Page ids of request b, in logical order (CSR row b)."""
    return np.asarray(kv_indices[int(kv_indptr[b]): int(kv_indptr[b + 1])])


def request_kv_len(kv_indptr: np.ndarray, last_page_len: np.ndarray, page_size: int,
                   b: int) -> int:
    """Number of valid tokens of request b: full pages plus the last page's fill."""
    n = int(kv_indptr[b + 1]) - int(kv_indptr[b])
    if n == 0:
        return 0
    return (n - 1) * page_size + int(last_page_len[b])


def gather_request_kv(pool: np.ndarray, dtype: str, kv_indptr, kv_indices, last_page_len,
                      page_size: int, b: int, k_scale: float = 1.0, v_scale: float = 1.0):
    """K and V of request b as float64 ``[kv_len, kv_heads, head_dim]``.

    Token t is read from page ``pages[t // page_size]`` at slot
    ``t % page_size``; slots past ``last_page_len`` are never touched. The
    stored values are multiplied by the per-tensor scales (1 for 16-bit
    pools; see ``oracle.fp8`` for the FP8 reading).
    """
    pages = request_pages(kv_indptr, kv_indices, b)
    L = request_kv_len(kv_indptr, last_page_len, page_size, b)
    t = np.arange(L)
    page_of_token = pages[t // page_size]
    slot_of_token = t % page_size
    K = k_scale * upcast(pool[page_of_token, 0, slot_of_token], dtype)
    V = v_scale * upcast(pool[page_of_token, 1, slot_of_token], dtype)
    return K, V


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           visible: Optional[Sequence[int]] = None):
    """Scaled-dot-product attention with a per-row count of visible keys.

    q: ``[R, Hq, D]`` float64; K, V: ``[L, Hkv, D]`` float64. Row r sees keys
    ``0 .. visible[r]-1`` (all L keys when ``visible`` is None). Query head h
    reads kv head ``h // (Hq // Hkv)``. Returns ``out [R, Hq, D]`` and
    ``lse [R, Hq]`` (natural log); rows with no visible key get 0 and -inf.
    """
    R, Hq, D = q.shape
    L, Hkv, _ = K.shape
    if Hq % Hkv:
        raise ValueError("num_qo_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    vis = np.full(R, L, dtype=np.int64) if visible is None else np.asarray(visible, np.int64)
    vis = np.clip(vis, 0, L)
    out = np.zeros((R, Hq, D), dtype=np.float64)
    lse = np.full((R, Hq), -np.inf, dtype=np.float64)
    if L == 0:
        return out, lse
    keymask = np.arange(L)[None, :] < vis[:, None]            # [R, L]
    live = vis > 0
    for h in range(Hq):
        hk = h // G
        S = scale * (q[:, h, :] @ K[:, hk, :].T)               # [R, L]
        S = np.where(keymask, S, -np.inf)
        m = S.max(axis=1)
        m_safe = np.where(live, m, 0.0)
        W = np.exp(S - m_safe[:, None])                        # masked -> exp(-inf) = 0
        l = W.sum(axis=1)
        o = W @ V[:, hk, :]
        out[live, h, :] = o[live] / l[live, None]
        lse[live, h] = m[live] + np.log(l[live])
    return out, lse


def decode(q_bits: np.ndarray, pool: np.ndarray, dtype: str, kv_indptr, kv_indices,
           last_page_len, page_size: int, scale: Optional[float] = None,
           requests: Optional[Sequence[int]] = None, kv_dtype: Optional[str] = None,
           k_scale: float = 1.0, v_scale: float = 1.0):
    """Decode: one query row per request over its paged KV.

    ``dtype`` is the query type; the pool holds ``kv_dtype`` (default: the
    same), scaled by ``k_scale`` / ``v_scale``. Returns ``out [n, Hq, D]``,
    ``lse [n, Hq]`` for the requested rows (all requests by default, in
    order).
    """
    D = q_bits.shape[-1]
    scale = default_scale(D) if scale is None else scale
    kv_dtype = dtype if kv_dtype is None else kv_dtype
    reqs = range(q_bits.shape[0]) if requests is None else list(requests)
    outs, lses = [], []
    for b in reqs:
        K, V = gather_request_kv(pool, kv_dtype, kv_indptr, kv_indices, last_page_len, page_size,
                                 b, k_scale, v_scale)
        o, s = attend(upcast(q_bits[b: b + 1], dtype), K, V, scale)
        outs.append(o[0])
        lses.append(s[0])
    return np.stack(outs), np.stack(lses)


def append(q_bits: np.ndarray, qo_indptr, pool: np.ndarray, dtype: str, kv_indptr, kv_indices,
           last_page_len, page_size: int, causal: bool = True, scale: Optional[float] = None,
           rows: Optional[Sequence[int]] = None):
    """Append/prefill: request b's rows ``qo_indptr[b]..qo_indptr[b+1]-1``.

    With ``causal`` the row i of request b (i counted from its first new row)
    sees keys ``0 .. kv_len - qo_len + i`` inclusive; otherwise all kv_len
    keys. Returns ``out``/``lse`` for the listed rows of the packed q (all
    rows by default, in order).
    """
    return _append_rows(q_bits, qo_indptr, dtype, lambda b: gather_request_kv(
        pool, dtype, kv_indptr, kv_indices, last_page_len, page_size, b), causal, scale, rows)


def ragged_request_kv(k_bits: np.ndarray, v_bits: np.ndarray, dtype: str, kv_offsets, b: int,
                      k_scale: float = 1.0, v_scale: float = 1.0):
    """K and V of request b of a ragged cache as float64 ``[kv_len, kv_heads, head_dim]``.

    [Guide, "What FlashInfer is", idea 1]: a ragged tensor holds each
    request's keys as consecutive rows; request b owns rows
    ``kv_offsets[b] .. kv_offsets[b+1]-1`` of ``[rows, kv_heads, head_dim]``.
    """
    r0, r1 = int(kv_offsets[b]), int(kv_offsets[b + 1])
    return k_scale * upcast(k_bits[r0:r1], dtype), v_scale * upcast(v_bits[r0:r1], dtype)


def decode_ragged(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, dtype: str,
                  kv_offsets, scale: Optional[float] = None,
                  requests: Optional[Sequence[int]] = None, kv_dtype: Optional[str] = None,
                  k_scale: float = 1.0, v_scale: float = 1.0):
    """Decode over a ragged cache (one query row per request); a single
    request over one contiguous K / V ([DeepDive, "Snippet One"]: the
    single-sequence decode) is ``kv_offsets = [0, kv_len]``."""
    D = q_bits.shape[-1]
    scale = default_scale(D) if scale is None else scale
    kv_dtype = dtype if kv_dtype is None else kv_dtype
    reqs = range(q_bits.shape[0]) if requests is None else list(requests)
    outs, lses = [], []
    for b in reqs:
        K, V = ragged_request_kv(k_bits, v_bits, kv_dtype, kv_offsets, b, k_scale, v_scale)
        o, s = attend(upcast(q_bits[b: b + 1], dtype), K, V, scale)
        outs.append(o[0])
        lses.append(s[0])
    return np.stack(outs), np.stack(lses)


def append_ragged(q_bits: np.ndarray, qo_indptr, k_bits: np.ndarray, v_bits: np.ndarray,
                  dtype: str, kv_offsets, causal: bool = True, scale: Optional[float] = None,
                  rows: Optional[Sequence[int]] = None):
    """Append/prefill over a ragged cache; rows and masking as ``append``."""
    return _append_rows(q_bits, qo_indptr, dtype, lambda b: ragged_request_kv(
        k_bits, v_bits, dtype, kv_offsets, b), causal, scale, rows)


def block_sparse(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, dtype: str,
                 block_indptr, block_indices, row_offsets, col_offsets,
                 scale: Optional[float] = None):
    """Block-sparse attention ([Windows] "Core Features", Attention Kernels:
    block-sparse and variable block-sparse patterns). Query rows
    ``row_offsets[i] .. row_offsets[i+1]-1`` (row block i) attend, without a
    mask inside the blocks, to the keys of column blocks
    ``block_indices[block_indptr[i] .. block_indptr[i+1]-1]``; column block j
    is key rows ``col_offsets[j] .. col_offsets[j+1]-1``. Returns out / lse for
    every query row."""
    D = q_bits.shape[-1]
    scale = default_scale(D) if scale is None else scale
    row_offsets = np.asarray(row_offsets)
    outs, lses = [], []
    for i in range(row_offsets.shape[0] - 1):
        rows = []
        for n in range(int(block_indptr[i]), int(block_indptr[i + 1])):
            j = int(block_indices[n])
            rows.extend(range(int(col_offsets[j]), int(col_offsets[j + 1])))
        K = upcast(k_bits[rows], dtype)
        V = upcast(v_bits[rows], dtype)
        r0, r1 = int(row_offsets[i]), int(row_offsets[i + 1])
        o, s = attend(upcast(q_bits[r0:r1], dtype), K, V, scale)
        outs.append(o)
        lses.append(s)
    return np.concatenate(outs), np.concatenate(lses)


def _append_rows(q_bits, qo_indptr, dtype, kv_of, causal, scale, rows):
    """Rows of ``append`` / ``append_ragged``; ``kv_of(b)`` gives request b's K, V."""
    D = q_bits.shape[-1]
    scale = default_scale(D) if scale is None else scale
    qo_indptr = np.asarray(qo_indptr)
    B = qo_indptr.shape[0] - 1
    want = range(int(qo_indptr[-1])) if rows is None else list(rows)
    by_req = {}
    for r in want:
        b = int(np.searchsorted(qo_indptr, r, side="right") - 1)
        by_req.setdefault(b, []).append(r)
    res = {}
    for b in range(B):
        if b not in by_req:
            continue
        K, V = kv_of(b)
        L = K.shape[0]
        qo_len = int(qo_indptr[b + 1] - qo_indptr[b])
        rs = by_req[b]
        i = np.asarray(rs) - int(qo_indptr[b])
        vis = (L - qo_len + i + 1) if causal else np.full(len(rs), L)
        o, s = attend(upcast(q_bits[rs], dtype), K, V, scale, vis)
        for k, r in enumerate(rs):
            res[r] = (o[k], s[k])
    return (np.stack([res[r][0] for r in want]), np.stack([res[r][1] for r in want]))


def _prefix_kv(pool, dtype, prefix_indptr, prefix_indices, prefix_last_page_len, page_size):
    return gather_request_kv(pool, dtype, prefix_indptr, prefix_indices, prefix_last_page_len,
                             page_size, 0)


def cascade(q_bits, pool, dtype, prefix_indptr, prefix_indices, prefix_last_page_len,
            kv_indptr, kv_indices, last_page_len, page_size, scale=None, requests=None):
    """Shared-prefix pass + per-request suffix pass, combined by merge_state."""
    D = q_bits.shape[-1]
    scale = default_scale(D) if scale is None else scale
    reqs = list(range(q_bits.shape[0])) if requests is None else list(requests)
    Kp, Vp = _prefix_kv(pool, dtype, prefix_indptr, prefix_indices, prefix_last_page_len,
                        page_size)
    q = upcast(q_bits[reqs], dtype)
    o_p, s_p = attend(q, Kp, Vp, scale)
    o_s, s_s = decode(q_bits, pool, dtype, kv_indptr, kv_indices, last_page_len, page_size,
                      scale, requests=reqs)
    return merge_state(o_p, s_p, o_s, s_s)


def cascade_direct(q_bits, pool, dtype, prefix_indptr, prefix_indices, prefix_last_page_len,
                   kv_indptr, kv_indices, last_page_len, page_size, scale=None, requests=None):
    """The same result computed in one pass over prefix ++ suffix."""
    D = q_bits.shape[-1]
    scale = default_scale(D) if scale is None else scale
    reqs = list(range(q_bits.shape[0])) if requests is None else list(requests)
    Kp, Vp = _prefix_kv(pool, dtype, prefix_indptr, prefix_indices, prefix_last_page_len,
                        page_size)
    outs, lses = [], []
    for b in reqs:
        Ks, Vs = gather_request_kv(pool, dtype, kv_indptr, kv_indices, last_page_len,
                                   page_size, b)
        o, s = attend(upcast(q_bits[b: b + 1], dtype), np.concatenate([Kp, Ks]),
                      np.concatenate([Vp, Vs]), scale)
        outs.append(o[0])
        lses.append(s[0])
    return np.stack(outs), np.stack(lses)
