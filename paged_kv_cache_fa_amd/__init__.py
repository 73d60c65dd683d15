"""Paged-KV attention for AMD Instinct MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI in ``include/fa.h`` (``libpkfa.so``, built
from ``csrc/`` by ``build.py``). It only marshals arguments: every step of the
computation runs in the library's HIP kernels. Device buffers are torch
tensors (used for memory and streams only); there is no CPU fallback — if the
library is missing, the import of any entry point raises.

Entry points (same names as the C ABI): ``workspace_size``, ``plan`` /
``plan_ragged`` (return a ``Plan``), ``decode``, ``decode_noalloc``, ``decode_scaled``,
``decode_ragged``, ``append``, ``append_ragged``, ``pod``, ``cascade``, ``merge_state``,
``merge_states``, ``block_sparse_pages``; and ``single_decode_with_kv_cache`` /
``block_sparse_attention``, which plan and run a one-request decode over a
contiguous K / V and a block-sparse pattern.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from . import _lib
from ._lib import (FA_BF16, FA_E4M3, FA_F16, FA_F32, FA_MODE_APPEND, FA_MODE_DECODE,  # noqa: F401
                   FAError, Geometry, PlanStats, PlanT, check, load)

_DTYPE_CODES = {"bf16": FA_BF16, "fp16": FA_F16, "fp32": FA_F32, "e4m3": FA_E4M3}


def _torch():
    import torch
    return torch


def dtype_code(dt) -> int:
    """Map "bf16"/"fp16"/"fp32"/"e4m3" or a torch dtype to the ABI dtype code."""
    if isinstance(dt, str):
        return _DTYPE_CODES[dt]
    torch = _torch()
    return {torch.bfloat16: FA_BF16, torch.float16: FA_F16, torch.float32: FA_F32,
            torch.float8_e4m3fn: FA_E4M3}[dt]


def geometry(mode: str, dtype, max_batch: int, num_qo_heads: int, num_kv_heads: int,
             head_dim: int = 128, page_size: int = 16, max_qo_tokens: int = 0,
             **knobs) -> Geometry:
    g = Geometry()
    g.mode = FA_MODE_APPEND if mode == "append" else FA_MODE_DECODE
    g.dtype = dtype_code(dtype)
    g.max_batch = max_batch
    g.max_qo_tokens = max_qo_tokens
    g.num_qo_heads = num_qo_heads
    g.num_kv_heads = num_kv_heads
    g.head_dim = head_dim
    g.page_size = page_size
    for k, v in knobs.items():
        if k == "kv_dtype":
            v = 0 if v is None else dtype_code(v)
        setattr(g, k, int(v))
    return g


def workspace_size(geom: Geometry):
    """(host_bytes, device_bytes) for a geometry."""
    lib = load()
    h, d = ctypes.c_size_t(), ctypes.c_size_t()
    check(lib.fa_workspace_size(ctypes.byref(geom), ctypes.byref(h), ctypes.byref(d)))
    return h.value, d.value


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        torch = _torch()
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    return stream if isinstance(stream, int) else stream.cuda_stream


def _i32(a) -> np.ndarray:
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


class Plan:
    """A plan object plus its host and device workspaces.

    ``device=None`` plans on the host only (inspectable, not runnable). The
    host workspace is pinned memory when a GPU is used.
    """

    def __init__(self, geom: Geometry, device=None):
        lib = load()
        self.geom = geom
        self.device = device
        self._plan = PlanT()
        hb, db = workspace_size(geom)
        self.host_bytes, self.dev_bytes = hb, db
        if device is None:
            self.host_ws = np.zeros(hb, dtype=np.uint8)
            self.dev_ws = None
        else:
            torch = _torch()
            self.host_ws = torch.empty(hb, dtype=torch.uint8, pin_memory=True)
            self.dev_ws = torch.empty(db + 256, dtype=torch.uint8, device=device)
            off = (-self.dev_ws.data_ptr()) % 256
            self.dev_ws = self.dev_ws[off: off + db]
        self._lib = lib
        self._keep = None

    def plan(self, kv_indptr, kv_lens, qo_indptr=None, causal: bool = False, stream=None):
        kv_indptr, kv_lens, qo_indptr = _i32(kv_indptr), _i32(kv_lens), _i32(qo_indptr)
        self._keep = (kv_indptr, kv_lens, qo_indptr)
        batch = int(kv_lens.shape[0])
        check(self._lib.fa_plan(ctypes.byref(self._plan), ctypes.byref(self.geom),
                                _ptr(kv_indptr), _ptr(kv_lens), batch,
                                _ptr(qo_indptr) if qo_indptr is not None else None, int(causal),
                                _ptr(self.host_ws), self.host_bytes,
                                _ptr(self.dev_ws) if self.dev_ws is not None else None,
                                self.dev_bytes if self.dev_ws is not None else 0,
                                _stream(stream) if self.dev_ws is not None else None))
        return self

    def plan_ragged(self, kv_offsets, qo_indptr=None, causal: bool = False, stream=None):
        """Plan over a ragged KV cache: request b's keys are rows kv_offsets[b] ..
        kv_offsets[b+1]-1 (see fa_plan_ragged)."""
        kv_offsets, qo_indptr = _i32(kv_offsets), _i32(qo_indptr)
        self._keep = (kv_offsets, qo_indptr)
        batch = int(kv_offsets.shape[0]) - 1
        check(self._lib.fa_plan_ragged(ctypes.byref(self._plan), ctypes.byref(self.geom),
                                       _ptr(kv_offsets), batch,
                                       _ptr(qo_indptr) if qo_indptr is not None else None,
                                       int(causal), _ptr(self.host_ws), self.host_bytes,
                                       _ptr(self.dev_ws) if self.dev_ws is not None else None,
                                       self.dev_bytes if self.dev_ws is not None else 0,
                                       _stream(stream) if self.dev_ws is not None else None))
        return self

    def info(self) -> PlanStats:
        st = PlanStats()
        check(self._lib.fa_plan_info(ctypes.byref(self._plan), ctypes.byref(st)))
        return st

    def tiles(self, with_workers: bool = False):
        """Host copies of the current plan: (tiles int32 [n, 8], merge int32 [m, 4])
        and, with ``with_workers``, worker_ptr int32 [workers+1] (decode: worker
        waves; append: the 8 XCD bins)."""
        tp, mp, wp = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
        nt, nm, nw = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        check(self._lib.fa_plan_tiles(ctypes.byref(self._plan), ctypes.byref(tp),
                                      ctypes.byref(nt), ctypes.byref(mp), ctypes.byref(nm),
                                      ctypes.byref(wp), ctypes.byref(nw)))

        def arr(ptr, n):
            if n == 0:
                return np.zeros(0, np.int32)
            return np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ctypes.c_int32)),
                                         shape=(n,)).copy()
        t = arr(tp, nt.value * 8).reshape(-1, 8)
        m = arr(mp, nm.value * 4).reshape(-1, 4)
        if not with_workers:
            return t, m
        w = arr(wp, nw.value + 1) if nw.value else None
        return t, m, w

    def __del__(self):
        try:
            self._lib.fa_plan_destroy(ctypes.byref(self._plan))
        except Exception:
            pass


def plan(geom: Geometry, kv_indptr, kv_lens, qo_indptr=None, causal: bool = False,
         device=None, stream=None) -> Plan:
    """Build a plan (and upload it when ``device`` is given)."""
    return Plan(geom, device).plan(kv_indptr, kv_lens, qo_indptr, causal, stream)


def plan_ragged(geom: Geometry, kv_offsets, qo_indptr=None, causal: bool = False, device=None,
                stream=None) -> Plan:
    """Build a ragged-KV plan (and upload it when ``device`` is given)."""
    return Plan(geom, device).plan_ragged(kv_offsets, qo_indptr, causal, stream)


def _alloc_out(q, out, lse, rows, heads):
    torch = _torch()
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(rows, heads, dtype=torch.float32, device=q.device)
    return out, lse


def decode(p: Plan, q, k_pages, v_pages, page_stride: int, token_stride: int, head_stride: int,
           kv_indices, kv_indptr, last_page_len, sm_scale: float = 0.0, out=None, lse=None,
           stream=None):
    """Batched paged decode (see fa_decode). Returns (out, lse)."""
    out, lse = _alloc_out(q, out, lse, q.shape[0], q.shape[1])
    check(p._lib.fa_decode(ctypes.byref(p._plan), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                           page_stride, token_stride, head_stride, _ptr(kv_indices),
                           _ptr(kv_indptr), _ptr(last_page_len), float(sm_scale), _ptr(out),
                           _ptr(lse), _stream(stream)))
    return out, lse


def decode_noalloc(geom: Geometry, kv_indptr_h, kv_lens_h, q, k_pages, v_pages, page_stride: int,
                   token_stride: int, head_stride: int, kv_indices, kv_indptr, last_page_len,
                   sm_scale: float = 0.0, out=None, lse=None, stream=None):
    """fa_plan + fa_decode in one call with the library's static per-GPU
    workspaces (see fa_decode_noalloc): no workspace is passed and nothing is
    allocated by the library. Returns (out, lse)."""
    lib = load()
    ip, lens = _i32(kv_indptr_h), _i32(kv_lens_h)
    out, lse = _alloc_out(q, out, lse, q.shape[0], q.shape[1])
    check(lib.fa_decode_noalloc(ctypes.byref(geom), _ptr(ip), _ptr(lens), int(lens.shape[0]),
                                _ptr(q), _ptr(k_pages), _ptr(v_pages), page_stride, token_stride,
                                head_stride, _ptr(kv_indices), _ptr(kv_indptr),
                                _ptr(last_page_len), float(sm_scale), _ptr(out), _ptr(lse),
                                _stream(stream)))
    return out, lse


def decode_scaled(p: Plan, q, k_pages, v_pages, page_stride: int, token_stride: int,
                  head_stride: int, kv_indices, kv_indptr, last_page_len, sm_scale: float = 0.0,
                  k_scale: float = 1.0, v_scale: float = 1.0, out=None, lse=None, stream=None):
    """Paged decode with per-tensor K/V scales, e.g. over an E4M3 page pool
    (see fa_decode_scaled; strides count pool elements, bytes for E4M3).
    Returns (out, lse)."""
    out, lse = _alloc_out(q, out, lse, q.shape[0], q.shape[1])
    check(p._lib.fa_decode_scaled(ctypes.byref(p._plan), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                  page_stride, token_stride, head_stride, _ptr(kv_indices),
                                  _ptr(kv_indptr), _ptr(last_page_len), float(sm_scale),
                                  float(k_scale), float(v_scale), _ptr(out), _ptr(lse),
                                  _stream(stream)))
    return out, lse


def decode_ragged(p: Plan, q, k, v, token_stride: int, head_stride: int, kv_offsets=None,
                  sm_scale: float = 0.0, k_scale: float = 1.0, v_scale: float = 1.0, out=None,
                  lse=None, stream=None):
    """Decode over a ragged KV cache (see fa_decode_ragged); ``kv_offsets`` is a
    device int32 tensor or None for the plan's copy. Returns (out, lse)."""
    out, lse = _alloc_out(q, out, lse, q.shape[0], q.shape[1])
    check(p._lib.fa_decode_ragged(ctypes.byref(p._plan), _ptr(q), _ptr(k), _ptr(v), token_stride,
                                  head_stride, _ptr(kv_offsets), float(sm_scale), float(k_scale),
                                  float(v_scale), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def append_ragged(p: Plan, q, qo_indptr, k, v, token_stride: int, head_stride: int,
                  kv_offsets=None, sm_scale: float = 0.0, out=None, lse=None, stream=None):
    """Append / prefill over a ragged KV cache (see fa_append_ragged). Returns (out, lse)."""
    out, lse = _alloc_out(q, out, lse, q.shape[0], q.shape[1])
    check(p._lib.fa_append_ragged(ctypes.byref(p._plan), _ptr(q), _ptr(qo_indptr), _ptr(k),
                                  _ptr(v), token_stride, head_stride, _ptr(kv_offsets),
                                  float(sm_scale), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def single_decode_with_kv_cache(q, k, v, sm_scale: float = 0.0, k_scale: float = 1.0,
                                v_scale: float = 1.0, return_lse: bool = False, **knobs):
    """One query row per q head against a contiguous K / V of one request.

    q [num_qo_heads, head_dim], k / v [kv_len, num_kv_heads, head_dim] (16-bit,
    or uint8 E4M3 codes with their scales). Plans a batch-1 ragged decode
    (workspaces allocated here, as torch tensors) and runs it: every step is
    the library's. Returns out [num_qo_heads, head_dim] (and lse [num_qo_heads])."""
    torch = _torch()
    L, hkv, d = k.shape
    kvd = "e4m3" if k.dtype in (torch.uint8, torch.float8_e4m3fn) else None
    g = geometry("decode", q.dtype, 1, q.shape[0], hkv, head_dim=d, kv_dtype=kvd, **knobs)
    p = Plan(g, device=q.device).plan_ragged(np.array([0, L], dtype=np.int32))
    out, lse = decode_ragged(p, q.reshape(1, *q.shape), k, v, k.stride(0), k.stride(1),
                             sm_scale=sm_scale, k_scale=k_scale, v_scale=v_scale)
    out = out.reshape(q.shape)
    return (out, lse.reshape(-1)) if return_lse else out


def block_sparse_pages(block_indptr, block_indices, col_offsets, page_size: int = 16):
    """Row-id page table of a block-sparse pattern (see fa_block_sparse_pages):
    returns (kv_indptr, kv_indices, last_page_len, kv_lens) as int32 arrays."""
    lib = load()
    bi, bx, co = _i32(block_indptr), _i32(block_indices), _i32(col_offsets)
    nrb, ncb = int(bi.shape[0]) - 1, int(co.shape[0]) - 1
    kv_indptr = np.zeros(nrb + 1, np.int32)
    last = np.zeros(max(nrb, 1), np.int32)
    lens = np.zeros(max(nrb, 1), np.int32)
    n = ctypes.c_int64()
    bxp = _ptr(bx) if bx.size else None
    st = lib.fa_block_sparse_pages(_ptr(bi), bxp, nrb, _ptr(co), ncb, page_size, _ptr(kv_indptr),
                                   None, 0, _ptr(last), _ptr(lens), ctypes.byref(n))
    if st not in (0, _lib.FA_ERR_CAPACITY):
        check(st)
    kv_indices = np.zeros(max(n.value, 1), np.int32)
    check(lib.fa_block_sparse_pages(_ptr(bi), bxp, nrb, _ptr(co), ncb, page_size,
                                    _ptr(kv_indptr), _ptr(kv_indices), kv_indices.shape[0],
                                    _ptr(last), _ptr(lens), ctypes.byref(n)))
    return kv_indptr, kv_indices[: n.value], last[:nrb], lens[:nrb]


def block_sparse_attention(q, k, v, block_indptr, block_indices, row_offsets, col_offsets,
                           sm_scale: float = 0.0, **knobs):
    """Block-sparse attention: query rows row_offsets[i] .. row_offsets[i+1]-1
    (row block i) attend to the keys of their column blocks (see
    fa_block_sparse_pages). q [rows, Hq, D], k / v [keys, Hkv, D]. Builds the
    page table and a plan (workspaces allocated here, as torch tensors) and
    runs fa_decode (one query row per block) or fa_append (non-causal).
    Returns (out, lse)."""
    torch = _torch()
    kv_indptr, kv_indices, last, lens = block_sparse_pages(block_indptr, block_indices,
                                                           col_offsets)
    ro = _i32(row_offsets)
    nrb = int(ro.shape[0]) - 1
    dev = q.device
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    ts, hs = k.stride(0), k.stride(1)
    if np.all(np.diff(ro) == 1):
        g = geometry("decode", q.dtype, max(nrb, 1), q.shape[1], k.shape[1], **knobs)
        p = Plan(g, device=dev).plan(kv_indptr, lens)
        return decode(p, q, k, v, ts, ts, hs, t(kv_indices), t(kv_indptr), t(last),
                      sm_scale=sm_scale)
    g = geometry("append", q.dtype, max(nrb, 1), q.shape[1], k.shape[1],
                 max_qo_tokens=max(int(ro[-1]), 1), **knobs)
    p = Plan(g, device=dev).plan(kv_indptr, lens, ro, False)
    return append(p, q, t(ro), k, v, ts, ts, hs, t(kv_indices), t(kv_indptr), t(last),
                  sm_scale=sm_scale)


def append(p: Plan, q, qo_indptr, k_pages, v_pages, page_stride: int, token_stride: int,
           head_stride: int, kv_indices, kv_indptr, last_page_len, sm_scale: float = 0.0,
           out=None, lse=None, stream=None):
    """Append / prefill over the paged cache (see fa_append). Returns (out, lse)."""
    out, lse = _alloc_out(q, out, lse, q.shape[0], q.shape[1])
    check(p._lib.fa_append(ctypes.byref(p._plan), _ptr(q), _ptr(qo_indptr), _ptr(k_pages),
                           _ptr(v_pages), page_stride, token_stride, head_stride,
                           _ptr(kv_indices), _ptr(kv_indptr), _ptr(last_page_len),
                           float(sm_scale), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def pod(prefill_plan: Plan, q_p, qo_indptr_p, kv_indices_p, kv_indptr_p, last_page_len_p,
        decode_plan: Plan, q_d, kv_indices_d, kv_indptr_d, last_page_len_d, k_pages, v_pages,
        page_stride: int, token_stride: int, head_stride: int, sm_scale: float = 0.0,
        out_p=None, lse_p=None, out_d=None, lse_d=None, stream=None):
    """Prefill and decode requests of a mixed batch in one launch (see fa_pod).
    Returns ((out_p, lse_p), (out_d, lse_d))."""
    out_p, lse_p = _alloc_out(q_p, out_p, lse_p, q_p.shape[0], q_p.shape[1])
    out_d, lse_d = _alloc_out(q_d, out_d, lse_d, q_d.shape[0], q_d.shape[1])
    check(prefill_plan._lib.fa_pod(
        ctypes.byref(prefill_plan._plan), _ptr(q_p), _ptr(qo_indptr_p), _ptr(kv_indices_p),
        _ptr(kv_indptr_p), _ptr(last_page_len_p), _ptr(out_p), _ptr(lse_p),
        ctypes.byref(decode_plan._plan), _ptr(q_d), _ptr(kv_indices_d), _ptr(kv_indptr_d),
        _ptr(last_page_len_d), _ptr(out_d), _ptr(lse_d), _ptr(k_pages), _ptr(v_pages),
        page_stride, token_stride, head_stride, float(sm_scale), _stream(stream)))
    return (out_p, lse_p), (out_d, lse_d)


def cascade(prefix_plan: Plan, suffix_plan: Plan, q, k_pages, v_pages, page_stride: int,
            token_stride: int, head_stride: int, prefix_qo_indptr, prefix_indices, prefix_indptr,
            prefix_last_page_len, kv_indices, kv_indptr, last_page_len, sm_scale: float = 0.0,
            states=None, out=None, lse=None, stream=None, side_stream=None, suffix_stream=None):
    """Cascade attention over one shared prefix (see fa_cascade). ``states`` is
    (prefix_out, prefix_lse, suffix_out, suffix_lse) scratch, allocated if None;
    ``side_stream`` / ``suffix_stream`` (torch streams or handles) run the
    prefix pass / the suffix decode, forked from and joined back to ``stream``.
    Returns (out, lse)."""
    torch = _torch()
    B, H = q.shape[0], q.shape[1]
    if states is None:
        states = (torch.empty_like(q), torch.empty(B, H, dtype=torch.float32, device=q.device),
                  torch.empty_like(q), torch.empty(B, H, dtype=torch.float32, device=q.device))
    out, lse = _alloc_out(q, out, lse, B, H)
    po, pl_, so, sl = states
    side = None if side_stream is None else _stream(side_stream)
    suf = None if suffix_stream is None else _stream(suffix_stream)
    check(prefix_plan._lib.fa_cascade(
        ctypes.byref(prefix_plan._plan), ctypes.byref(suffix_plan._plan), _ptr(q), _ptr(k_pages),
        _ptr(v_pages), page_stride, token_stride, head_stride, _ptr(prefix_qo_indptr),
        _ptr(prefix_indices), _ptr(prefix_indptr), _ptr(prefix_last_page_len), _ptr(kv_indices),
        _ptr(kv_indptr), _ptr(last_page_len), float(sm_scale), _ptr(po), _ptr(pl_), _ptr(so),
        _ptr(sl), _ptr(out), _ptr(lse), _stream(stream), side, suf))
    return out, lse


def merge_state(v_a, s_a, v_b, s_b, v_out=None, s_out=None, stream=None):
    """Merge two states [n, heads, D] / [n, heads] (see fa_merge_state)."""
    torch = _torch()
    n, heads, d = v_a.shape
    if v_out is None:
        v_out = torch.empty_like(v_a)
    if s_out is None:
        s_out = torch.empty_like(s_a)
    check(load().fa_merge_state(_ptr(v_a), _ptr(s_a), _ptr(v_b), _ptr(s_b), _ptr(v_out),
                                _ptr(s_out), n, heads, d, dtype_code(v_a.dtype), _stream(stream)))
    return v_out, s_out


def merge_states(v, s, v_out=None, s_out=None, stream=None):
    """Merge k states per row: v [n, k, heads, D], s [n, k, heads] (see fa_merge_states)."""
    torch = _torch()
    n, k, heads, d = v.shape
    if v_out is None:
        v_out = torch.empty(n, heads, d, dtype=v.dtype, device=v.device)
    if s_out is None:
        s_out = torch.empty(n, heads, dtype=torch.float32, device=v.device)
    check(load().fa_merge_states(_ptr(v), _ptr(s), n, k, heads, d, dtype_code(v.dtype),
                                 _ptr(v_out), _ptr(s_out), _stream(stream)))
    return v_out, s_out


def probe_stream_read(src, flag, workgroups: int = 4096, stream=None):
    """Read all of the device tensor ``src`` once (see fa_probe_stream_read): a
    plain streaming read to compare the decode's bandwidth with. ``flag`` is a
    4-byte device tensor the probe may write."""
    nbytes = src.numel() * src.element_size()
    check(load().fa_probe_stream_read(_ptr(src), nbytes, _ptr(flag), workgroups, _stream(stream)))
