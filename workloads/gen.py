"""Seeded generators for the paged-KV workloads.

Everything here is input preparation: lengths, a page table in CSR form
(``kv_indptr`` / ``kv_indices`` / ``last_page_len``), a page pool and the
queries, stored as 16-bit floating-point bit patterns (or, for an FP8 pool,
E4M3 byte codes with one scale per tensor). There is no attention
arithmetic in this module.

Layout of the pool (the combined K/V pool shown in the page "FlashInfer: The
Attention Kernel Library That Proves the Bottleneck ...", section "Snippet
One: Paged KV-Cache Attention and MLA"): ``[num_pages, 2, page_size,
num_kv_heads, head_dim]``, index 0 of the second axis is K, index 1 is V,
tokens-major inside a page (the NHD layout).

Draw order for a workload with seed ``s`` (``numpy.random.default_rng(s)``):
lengths -> positions of long requests -> page permutation -> Q -> K pool ->
V pool. Normal values are drawn as float32 (``standard_normal(dtype=float32)``)
in chunks of 1024 pages and rounded to the storage type with
round-to-nearest-even.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

CONFIG_NAMES = {
    1: "single-request decode, 32/32 heads, kv 2048, fp16",
    2: "batched GQA decode, batch 64, 32/8 heads, kv U[512,4096], bf16",
    3: "skewed decode, batch 128 (4 x 32768 + 124 log-normal), 32/8 heads, bf16",
    4: "cascade, batch 256, 16384-token shared prefix + suffix U[256,1024], 32/8 heads, bf16",
    5: "causal append, batch 16 x 512 new tokens onto 4096 cached, 32/8 heads, bf16",
}

_NAN_BITS = {"bf16": 0x7FC0, "fp16": 0x7E00, "e4m3": 0x7F}
_PAGE_CHUNK = 1024

# Per-tensor scales of FP8 (E4M3) pools: stored code c stands for
# scale * e4m3(c). With these, N(0,1) draws up to 8 (K) and 6 (V) standard
# deviations map inside the format's finite range (|code value| <= 448);
# the rare draw beyond saturates there.
FP8_K_SCALE = 8.0 / 448.0
FP8_V_SCALE = 6.0 / 448.0
_E4M3_MAX = 448.0


def to_storage_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to bf16/fp16 (nearest-even) and return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    if dtype != "bf16":
        raise ValueError(f"unknown storage dtype {dtype!r}")
    u = x.view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = np.uint16(_NAN_BITS["bf16"])
    return r


def to_e4m3_codes(x: np.ndarray, scale: float) -> np.ndarray:
    """Quantise float32 values to E4M3 byte codes of ``x / scale``
    (round to nearest even, saturating at +-448), via torch's float8 cast."""
    import torch

    y = np.clip(np.asarray(x, dtype=np.float32) / np.float32(scale), -_E4M3_MAX, _E4M3_MAX)
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def csr_from_page_lists(page_lists: Sequence[Sequence[int]]):
    """Flatten per-request page lists into (indptr, indices), both int32."""
    counts = [len(p) for p in page_lists]
    indptr = np.zeros(len(page_lists) + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(counts, dtype=np.int64)
    if sum(counts):
        indices = np.concatenate([np.asarray(p, dtype=np.int32) for p in page_lists])
    else:
        indices = np.zeros(0, dtype=np.int32)
    return indptr, indices.astype(np.int32)


def _pages_for(kv_len: int, page_size: int) -> int:
    return -(-int(kv_len) // page_size)


def _last_page_len(kv_len: int, page_size: int) -> int:
    n = _pages_for(kv_len, page_size)
    return 0 if n == 0 else int(kv_len) - (n - 1) * page_size


@dataclass
class Workload:
    name: str
    dtype: str
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_lens: np.ndarray            # int32 [B]
    kv_indptr: np.ndarray          # int32 [B+1]
    kv_indices: np.ndarray         # int32 [nnz_pages]
    last_page_len: np.ndarray      # int32 [B]
    qo_indptr: Optional[np.ndarray]  # int32 [B+1]; None = decode (one row per request)
    causal: bool
    pool: np.ndarray               # uint16 [P, 2, ps, Hkv, D] (uint8 codes for e4m3)
    q: np.ndarray                  # uint16 [rows, Hq, D]
    seed: int
    mode: str = "bench"
    kv_dtype: Optional[str] = None  # pool storage type when it differs from dtype ("e4m3")
    k_scale: float = 1.0            # per-tensor scales of an e4m3 pool
    v_scale: float = 1.0
    # shared prefix (cascade); one extra "request" whose pages every request shares
    prefix_len: int = 0
    prefix_indptr: Optional[np.ndarray] = None
    prefix_indices: Optional[np.ndarray] = None
    prefix_last_page_len: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.kv_lens.shape[0])

    @property
    def rows(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.pool.shape[0])

    @property
    def qo_lens(self) -> np.ndarray:
        if self.qo_indptr is None:
            return np.ones(self.batch, dtype=np.int32)
        return np.diff(self.qo_indptr).astype(np.int32)

    def manifest(self) -> dict:
        """Lengths, page table and SHA-256 of the stored bytes."""
        h = hashlib.sha256()
        h.update(self.pool.tobytes())
        hq = hashlib.sha256(self.q.tobytes()).hexdigest()
        return {
            "name": self.name,
            "seed": self.seed,
            "kv_lens_sum": int(self.kv_lens.sum()),
            "kv_indices_sha256": hashlib.sha256(self.kv_indices.tobytes()).hexdigest(),
            "pool_sha256": h.hexdigest(),
            "q_sha256": hq,
        }


def _fill_normal_pool(rng, pool: np.ndarray, which: int, dtype: str) -> None:
    P, _, ps, hkv, d = pool.shape
    for p0 in range(0, P, _PAGE_CHUNK):
        p1 = min(P, p0 + _PAGE_CHUNK)
        x = rng.standard_normal((p1 - p0, ps, hkv, d), dtype=np.float32)
        if dtype == "e4m3":
            pool[p0:p1, which] = to_e4m3_codes(x, FP8_K_SCALE if which == 0 else FP8_V_SCALE)
        else:
            pool[p0:p1, which] = to_storage_bits(x, dtype)


def _poison_tails(pool, page_tables, page_size, dtype):
    """Test mode: slots past last_page_len of each last page hold NaN."""
    nan = pool.dtype.type(_NAN_BITS[dtype])
    for indptr, indices, last in page_tables:
        for b in range(len(indptr) - 1):
            n = indptr[b + 1] - indptr[b]
            if n == 0:
                continue
            lp = int(last[b])
            if lp < page_size:
                pool[indices[indptr[b + 1] - 1], :, lp:] = nan


def make_workload(
    kv_lens: Sequence[int],
    num_qo_heads: int,
    num_kv_heads: int,
    dtype: str,
    seed: int,
    rng: Optional[np.random.Generator] = None,
    qo_lens: Optional[Sequence[int]] = None,
    causal: bool = True,
    head_dim: int = 128,
    page_size: int = 16,
    mode: str = "bench",
    extra_pages: int = 0,
    name: str = "custom",
    kv_dtype: Optional[str] = None,
) -> Workload:
    """Lay out a paged KV cache for the given lengths and draw Q, K, V.

    ``rng`` continues a generator that already drew the lengths; if None a
    fresh ``default_rng(seed)`` is used. ``qo_lens=None`` means decode (one
    query row per request). With ``mode="test"`` unused tail slots and the
    ``extra_pages`` unreferenced pool pages hold NaN. ``kv_dtype="e4m3"``
    stores the pool as E4M3 codes with the scales FP8_K_SCALE / FP8_V_SCALE
    (the same normal draws, quantised); q stays in ``dtype``.
    """
    kvt = dtype if kv_dtype is None else kv_dtype
    if rng is None:
        rng = np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    B = kv_lens.shape[0]
    n_pages = np.array([_pages_for(L, page_size) for L in kv_lens], dtype=np.int64)
    total = int(n_pages.sum())
    P = total + int(extra_pages)
    perm = rng.permutation(P).astype(np.int32)
    lists, off = [], 0
    for b in range(B):
        lists.append(perm[off: off + n_pages[b]])
        off += int(n_pages[b])
    kv_indptr, kv_indices = csr_from_page_lists(lists)
    last = np.array([_last_page_len(L, page_size) for L in kv_lens], dtype=np.int32)

    if qo_lens is None:
        qo_indptr = None
        rows = B
    else:
        qo_lens = np.asarray(qo_lens, dtype=np.int32)
        if qo_lens.shape[0] != B or np.any(qo_lens > kv_lens) or np.any(qo_lens < 0):
            raise ValueError("qo_lens must be per-request and not exceed kv_lens")
        qo_indptr = np.zeros(B + 1, dtype=np.int32)
        qo_indptr[1:] = np.cumsum(qo_lens)
        rows = int(qo_indptr[-1])

    qf = rng.standard_normal((rows, num_qo_heads, head_dim), dtype=np.float32)
    q = to_storage_bits(qf, dtype)
    pool = np.empty((P, 2, page_size, num_kv_heads, head_dim),
                    dtype=np.uint8 if kvt == "e4m3" else np.uint16)
    _fill_normal_pool(rng, pool, 0, kvt)
    _fill_normal_pool(rng, pool, 1, kvt)
    if mode == "test":
        _poison_tails(pool, [(kv_indptr, kv_indices, last)], page_size, kvt)
        if extra_pages:
            unref = perm[total:]
            pool[unref] = pool.dtype.type(_NAN_BITS[kvt])
    fp8 = kvt == "e4m3"
    return Workload(
        name=name, dtype=dtype, num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, page_size=page_size, kv_lens=kv_lens, kv_indptr=kv_indptr,
        kv_indices=kv_indices, last_page_len=last, qo_indptr=qo_indptr, causal=causal,
        pool=pool, q=q, seed=seed, mode=mode, kv_dtype=kv_dtype if fp8 else None,
        k_scale=FP8_K_SCALE if fp8 else 1.0, v_scale=FP8_V_SCALE if fp8 else 1.0,
    )


def make_cascade(
    prefix_len: int,
    suffix_lens: Sequence[int],
    num_qo_heads: int,
    num_kv_heads: int,
    dtype: str,
    seed: int,
    rng: Optional[np.random.Generator] = None,
    head_dim: int = 128,
    page_size: int = 16,
    mode: str = "bench",
    name: str = "cascade",
) -> Workload:
    """Decode batch whose requests share one prefix stored once in the pool.

    ``prefix_len`` must be a whole number of pages. ``kv_indptr`` etc. describe
    each request's private suffix; ``prefix_*`` describe the shared prefix as a
    one-request page table. Request b attends to prefix ++ suffix_b.
    """
    if prefix_len % page_size:
        raise ValueError("prefix_len must be a multiple of page_size")
    if rng is None:
        rng = np.random.default_rng(seed)
    suffix_lens = np.asarray(suffix_lens, dtype=np.int32)
    B = suffix_lens.shape[0]
    npre = prefix_len // page_size
    n_suf = np.array([_pages_for(L, page_size) for L in suffix_lens], dtype=np.int64)
    P = npre + int(n_suf.sum())
    perm = rng.permutation(P).astype(np.int32)
    prefix_indptr, prefix_indices = csr_from_page_lists([perm[:npre]])
    prefix_last = np.array([_last_page_len(prefix_len, page_size)], dtype=np.int32)
    lists, off = [], npre
    for b in range(B):
        lists.append(perm[off: off + n_suf[b]])
        off += int(n_suf[b])
    kv_indptr, kv_indices = csr_from_page_lists(lists)
    last = np.array([_last_page_len(L, page_size) for L in suffix_lens], dtype=np.int32)
    qf = rng.standard_normal((B, num_qo_heads, head_dim), dtype=np.float32)
    q = to_storage_bits(qf, dtype)
    pool = np.empty((P, 2, page_size, num_kv_heads, head_dim), dtype=np.uint16)
    _fill_normal_pool(rng, pool, 0, dtype)
    _fill_normal_pool(rng, pool, 1, dtype)
    if mode == "test":
        _poison_tails(pool, [(kv_indptr, kv_indices, last)], page_size, dtype)
    return Workload(
        name=name, dtype=dtype, num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, page_size=page_size, kv_lens=suffix_lens, kv_indptr=kv_indptr,
        kv_indices=kv_indices, last_page_len=last, qo_indptr=None, causal=False,
        pool=pool, q=q, seed=seed, mode=mode, prefix_len=prefix_len,
        prefix_indptr=prefix_indptr, prefix_indices=prefix_indices,
        prefix_last_page_len=prefix_last,
    )


@dataclass
class RaggedWorkload:
    """A ragged KV cache: request b's keys are rows kv_offsets[b] ..
    kv_offsets[b+1]-1 of k / v ``[rows, num_kv_heads, head_dim]`` (stored bits;
    E4M3 codes with ``kv_dtype="e4m3"``). Test mode appends ``pad_rows`` NaN
    rows after the last request."""
    dtype: str
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    kv_lens: np.ndarray            # int32 [B]
    kv_offsets: np.ndarray         # int32 [B+1]
    qo_indptr: Optional[np.ndarray]
    causal: bool
    k: np.ndarray                  # [rows + pad_rows, Hkv, D]
    v: np.ndarray
    q: np.ndarray                  # uint16 [rows_q, Hq, D]
    seed: int
    kv_dtype: Optional[str] = None
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def batch(self) -> int:
        return int(self.kv_lens.shape[0])

    @property
    def rows(self) -> int:
        return int(self.q.shape[0])


def make_ragged(kv_lens: Sequence[int], num_qo_heads: int, num_kv_heads: int, dtype: str,
                seed: int, qo_lens: Optional[Sequence[int]] = None, causal: bool = True,
                head_dim: int = 128, mode: str = "bench", pad_rows: int = 0,
                kv_dtype: Optional[str] = None) -> RaggedWorkload:
    """Draw a ragged KV cache for the given lengths: Q, then K rows, then V
    rows, N(0,1) as float32 rounded to the storage type (E4M3 with the FP8
    scales when ``kv_dtype="e4m3"``). ``qo_lens=None`` means decode."""
    rng = np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    B = kv_lens.shape[0]
    kv_offsets = np.zeros(B + 1, dtype=np.int32)
    kv_offsets[1:] = np.cumsum(kv_lens)
    total = int(kv_offsets[-1])
    if qo_lens is None:
        qo_indptr, rows = None, B
    else:
        qo_lens = np.asarray(qo_lens, dtype=np.int32)
        if qo_lens.shape[0] != B or np.any(qo_lens > kv_lens) or np.any(qo_lens < 0):
            raise ValueError("qo_lens must be per-request and not exceed kv_lens")
        qo_indptr = np.zeros(B + 1, dtype=np.int32)
        qo_indptr[1:] = np.cumsum(qo_lens)
        rows = int(qo_indptr[-1])
    q = to_storage_bits(rng.standard_normal((rows, num_qo_heads, head_dim), dtype=np.float32),
                        dtype)
    kvt = dtype if kv_dtype is None else kv_dtype
    fp8 = kvt == "e4m3"
    shape = (total + pad_rows, num_kv_heads, head_dim)
    kv = []
    for which in range(2):
        x = rng.standard_normal((total, num_kv_heads, head_dim), dtype=np.float32)
        arr = np.empty(shape, dtype=np.uint8 if fp8 else np.uint16)
        if fp8:
            arr[:total] = to_e4m3_codes(x, FP8_K_SCALE if which == 0 else FP8_V_SCALE)
        else:
            arr[:total] = to_storage_bits(x, kvt)
        arr[total:] = _NAN_BITS[kvt] if mode == "test" else 0
        kv.append(arr)
    return RaggedWorkload(
        dtype=dtype, num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        kv_lens=kv_lens, kv_offsets=kv_offsets, qo_indptr=qo_indptr, causal=causal, k=kv[0],
        v=kv[1], q=q, seed=seed, kv_dtype=kv_dtype if fp8 else None,
        k_scale=FP8_K_SCALE if fp8 else 1.0, v_scale=FP8_V_SCALE if fp8 else 1.0)


@dataclass
class BlockSparseWorkload:
    """A block-sparse pattern over contiguous q [rows, Hq, D] and k / v [keys,
    Hkv, D] (stored bits): row block i is q rows row_offsets[i] ..
    row_offsets[i+1]-1 and attends to column blocks block_indices[
    block_indptr[i] .. block_indptr[i+1]-1]; column block j is key rows
    col_offsets[j] .. col_offsets[j+1]-1. Test mode appends NaN key rows."""
    dtype: str
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    row_offsets: np.ndarray
    col_offsets: np.ndarray
    block_indptr: np.ndarray
    block_indices: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    seed: int


def make_block_sparse(row_sizes: Sequence[int], col_sizes: Sequence[int], density: float,
                      num_qo_heads: int, num_kv_heads: int, dtype: str, seed: int,
                      head_dim: int = 128, mode: str = "bench", pad_rows: int = 0,
                      empty_rows: Sequence[int] = ()) -> BlockSparseWorkload:
    """Draw a pattern (each column block kept with probability ``density``,
    increasing per row block; the listed row blocks keep none), then Q, K, V
    as N(0,1) rounded to the storage type. Column blocks other than a row
    block's last must be whole pages (16 rows): sizes are the caller's."""
    rng = np.random.default_rng(seed)
    row_offsets = np.concatenate([[0], np.cumsum(row_sizes)]).astype(np.int32)
    col_offsets = np.concatenate([[0], np.cumsum(col_sizes)]).astype(np.int32)
    nrb, ncb = len(row_sizes), len(col_sizes)
    keep = rng.random((nrb, ncb)) < density
    for i in empty_rows:
        keep[i] = False
    block_indices = np.concatenate([np.nonzero(keep[i])[0] for i in range(nrb)] +
                                   [np.zeros(0, np.int64)]).astype(np.int32)
    block_indptr = np.concatenate([[0], np.cumsum(keep.sum(axis=1))]).astype(np.int32)
    M, N = int(row_offsets[-1]), int(col_offsets[-1])
    q = to_storage_bits(rng.standard_normal((M, num_qo_heads, head_dim), dtype=np.float32), dtype)
    kv = []
    for _ in range(2):
        arr = np.empty((N + pad_rows, num_kv_heads, head_dim), np.uint16)
        arr[:N] = to_storage_bits(rng.standard_normal((N, num_kv_heads, head_dim),
                                                      dtype=np.float32), dtype)
        arr[N:] = _NAN_BITS[dtype] if mode == "test" else 0
        kv.append(arr)
    return BlockSparseWorkload(dtype=dtype, num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
                               head_dim=head_dim, row_offsets=row_offsets, col_offsets=col_offsets,
                               block_indptr=block_indptr, block_indices=block_indices, q=q,
                               k=kv[0], v=kv[1], seed=seed)


def config_lengths(k: int, rng: np.random.Generator) -> dict:
    """Draw the lengths of config k (the first draws of its generator)."""
    if k == 1:
        return dict(kv_lens=np.array([2048]))
    if k == 2:
        return dict(kv_lens=rng.integers(512, 4097, size=64))
    if k == 3:
        z = rng.standard_normal(124)
        short = np.clip(np.round(512.0 * np.exp(z)), 16, 8192).astype(np.int64)
        lens = np.concatenate([np.full(4, 32768, dtype=np.int64), short])
        order = rng.permutation(128)
        return dict(kv_lens=lens[order])
    if k == 4:
        return dict(prefix_len=16384, suffix_lens=rng.integers(256, 1025, size=256))
    if k == 5:
        return dict(kv_lens=np.full(16, 4608), qo_lens=np.full(16, 512))
    raise ValueError(f"no config {k}")


def make_config(k: int, seed: Optional[int] = None, mode: str = "bench",
                kv_dtype: Optional[str] = None) -> Workload:
    """The five benchmark workloads (seed defaults to the config number).

    ``kv_dtype="e4m3"`` gives the batch-64 and batch-128 decodes with an FP8 pool
    (same lengths, page table and draws; q stays bf16)."""
    if seed is None:
        seed = k
    if kv_dtype is not None and k not in (2, 3):
        raise ValueError("an FP8 pool is defined for the batch-64 and batch-128 decodes only")
    rng = np.random.default_rng(seed)
    name = f"config{k}" + ("" if kv_dtype is None else f"_{kv_dtype}")
    ln = config_lengths(k, rng)
    if k == 1:
        return make_workload(ln["kv_lens"], 32, 32, "fp16", seed, rng=rng, mode=mode, name=name)
    if k in (2, 3):
        return make_workload(ln["kv_lens"], 32, 8, "bf16", seed, rng=rng, mode=mode, name=name,
                             kv_dtype=kv_dtype)
    if k == 4:
        return make_cascade(ln["prefix_len"], ln["suffix_lens"], 32, 8, "bf16", seed, rng=rng,
                            mode=mode, name=name)
    return make_workload(ln["kv_lens"], 32, 8, "bf16", seed, rng=rng, qo_lens=ln["qo_lens"],
                         causal=True, mode=mode, name=name)
