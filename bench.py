"""Benchmark: paged-KV attention hot path on one MI355X.

Headline (the JSON ``value``): batched paged decode, batch 64, GQA 32 q / 8 kv
heads, head_dim 128, bf16, page 16, kv_len uniform in [512, 4096], pages
scattered by a seeded permutation. One step = the host plan (balanced
split-KV work list, uploaded to the device workspace) + the decode kernel
(which also merges split requests). ``value`` is the achieved algorithmic
HBM bandwidth of the step in GB/s: bytes of the valid K/V of every request,
plus q, out and lse, divided by the wall time per step.

Reported alongside in the same JSON line:
  * ``batch128``: the skewed batch-128 decode (4 x 32768 + 124 log-normal);
  * ``cascade``: batch 256 sharing a 16384-token prefix (prefix pass on MFMA +
    suffix decode + merge_state), as HBM GB/s with the prefix counted once;
    ``no_cascade_decode`` times the same batch as one plain decode whose
    requests each read the prefix pages (17.9 GB), for the speedup;
  * ``append``: causal append of 16 x 512 rows onto 4096 cached tokens, as
    MFMA utilisation (584.2 GFLOP of unmasked work per step);
  * ``fp8``: the batch-64 decode with an E4M3 page pool (per-tensor scales,
    bf16 q / out), as HBM GB/s with one byte per K/V element;
  * ``ragged``: the batch-64 decode over a ragged (contiguous-row) KV cache;
  * ``single``: the single-request decode (32 heads, kv_len 2048, fp16) over a
    contiguous K / V;
  * ``ragged`` and ``single`` also give ``graph_ms_per_call``: the median time
    per call of a captured hipGraph of back-to-back run calls over the
    rotating K/V copies (plan excluded). The single-request step is bound by
    the host (binding + plan), and its HIP events then time the host's
    submission gap rather than the kernel;
  * ``bsr``: block-sparse prefill, 4096 query rows x 16384 keys in 64 x 64
    blocks, a quarter of the blocks kept, as MFMA utilisation;
  * ``pod``: a mixed batch over one pool, the causal append of 16 x 512 rows
    plus the batch-64 decode, in one fa_pod launch against the two
    kernels back to back;
  * ``roofline``: the decode kernel against the 8 TB/s HBM peak (kernel time
    from HIP timing events around each launch on its stream, created without
    the system-scope fence), with HBM traffic from
    rocprofv3 counters when the stored counter summary matches the current
    kernel source (a graph of back-to-back calls measured slower per call:
    it adds the launch gaps); ``host_plan_us`` is the host cost of one
    fa_plan call;
  * ``roofline.attainable_GB/s``: a plain streaming read of 1 GiB on the same
    device (fa_probe_stream_read, best launch size), and the decode kernel's
    bandwidth as a fraction of it;
  * ``cpu_baseline``: the fp64 numpy oracle on the host cores.

Inputs are synthetic (seeded N(0,1)), resident in HBM before the timed
region; steps rotate over enough copies of the page pool (>= 1 GiB in total)
that the 256 MB Infinity Cache cannot hold them.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2516.6  # bf16 dense: 256 CU x 4096 FLOP/clk x 2.4 GHz
METRIC = "paged decode achieved HBM GB/s (% of peak) and tokens/sec at batch 64/128"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_batch64_hbm_counters.txt")


def kv_bytes(lens, hkv, d=128, elt=2) -> int:
    return int(np.asarray(lens, np.int64).sum()) * hkv * d * 2 * elt


def io_bytes(rows, hq, d=128, elt=2) -> int:
    return rows * hq * d * elt * 2 + rows * hq * 4


def algorithmic_bytes(wl) -> int:
    """Valid K/V bytes of every request (a shared prefix once) plus q, out, lse."""
    elt = 1 if wl.kv_dtype == "e4m3" else 2
    b = kv_bytes(wl.kv_lens, wl.num_kv_heads, elt=elt) + io_bytes(wl.rows, wl.num_qo_heads)
    if wl.prefix_len:
        b += kv_bytes([wl.prefix_len], wl.num_kv_heads)
    return b


def no_cascade_view(wl):
    """The cascade batch as a plain decode: every request's page list is the
    shared prefix's pages followed by its own (same pool, same q)."""
    import dataclasses
    ps = wl.page_size
    pre = wl.prefix_indices[wl.prefix_indptr[0]:wl.prefix_indptr[1]]
    lists = [np.concatenate([pre, wl.kv_indices[wl.kv_indptr[b]:wl.kv_indptr[b + 1]]])
             for b in range(wl.batch)]
    indptr = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    assert wl.prefix_len % ps == 0  # the prefix fills whole pages, so the last page is the suffix's
    return dataclasses.replace(wl, kv_lens=(wl.kv_lens + wl.prefix_len).astype(np.int32),
                               kv_indptr=indptr, kv_indices=np.concatenate(lists).astype(np.int32),
                               prefix_len=0, prefix_indptr=None, prefix_indices=None,
                               prefix_last_page_len=None)


def append_flops(wl) -> float:
    """4 * head_dim FLOPs per unmasked (query row, key) pair and query head."""
    pairs = 0
    for b in range(wl.batch):
        ql = int(wl.qo_indptr[b + 1] - wl.qo_indptr[b])
        L = int(wl.kv_lens[b])
        if wl.causal:
            pairs += sum(L - ql + i + 1 for i in range(ql))
        else:
            pairs += ql * L
    return float(pairs) * wl.num_qo_heads * 4 * wl.head_dim


def _dev(wl, device, min_rotation_bytes):
    import torch
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[wl.dtype]
    if wl.kv_dtype == "e4m3":
        pool = torch.from_numpy(wl.pool).to(device)
    else:
        pool = torch.from_numpy(wl.pool.view(np.int16)).to(device).view(dt)
    copies = max(1, math.ceil(min_rotation_bytes / max(1, pool.numel() * pool.element_size())))
    pools = [pool] + [pool.clone() for _ in range(copies - 1)]
    q = torch.from_numpy(wl.q.view(np.int16)).to(device).view(dt)
    _, _, ps, hkv, d = wl.pool.shape
    return pools, q, (2 * ps * hkv * d, hkv * d, d)


def _i32(a, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


class HipEvent:
    """A HIP timing event recorded on torch's current stream, created with
    hipEventDisableSystemFence, the flag HIP documents for timing the commands
    between two events without a system-scope cache write-back at each record.
    Measured around the batch-64 decode launch: 106 us against 105 us in
    rocprofv3's kernel trace, where torch's timing events gave 112 us and
    lengthened the step by 3 us."""

    _hip = None
    FLAGS = 0x20000000

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            import torch  # noqa: F401  (loads the HIP runtime that torch and libpkfa share)
            hip = ctypes.CDLL("libamdhip64.so.7")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipEvent._hip = hip
        self.ev = ctypes.c_void_p()
        self._destroy = HipEvent._hip.hipEventDestroy
        self._check(HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), self.FLAGS),
                    "hipEventCreateWithFlags")

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def record(self):
        import torch
        self._check(HipEvent._hip.hipEventRecord(self.ev, torch.cuda.current_stream().cuda_stream),
                    "hipEventRecord")

    def elapsed_time(self, end: "HipEvent") -> float:
        import ctypes
        ms = ctypes.c_float()
        self._check(HipEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev),
                    "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        if getattr(self, "ev", None):
            self._destroy(self.ev)


class Timed:
    """Run steps; time the whole step (torch events around all steps) and one named
    kernel call per step (HIP timing events around it, on its stream)."""

    def run(self, steps: int, warmup: int):
        import torch
        for i in range(warmup):
            self.step(i, None)
        torch.cuda.synchronize()
        kev = [(HipEvent(), HipEvent()) for _ in range(steps)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for i in range(steps):
            self.step(warmup + i, kev[i])
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps, float(np.mean([a.elapsed_time(b) for a, b in kev]))

    def graph_call_ms(self, calls: int, replays: int = 20) -> float:
        """Median time per run call of a captured hipGraph of `calls` back-to-back run
        calls over the rotating input copies (the plan is made once, before capture)."""
        import torch
        self.step(0, None)  # plan + one eager call
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(calls):
                    self.run_call(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(replays):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / calls)
        del g
        return float(np.median(ts))


class DecodeBench(Timed):
    def __init__(self, wl, device="cuda", min_rotation_bytes=1 << 30, **knobs):
        import torch
        import paged_kv_cache_fa_amd as fa
        self.fa, self.wl = fa, wl
        self.pools, self.q, self.strides = _dev(wl, device, min_rotation_bytes)
        self.kv_indptr = _i32(wl.kv_indptr, device)
        self.kv_indices = _i32(wl.kv_indices, device)
        self.last = _i32(wl.last_page_len, device)
        geom = fa.geometry("decode", wl.dtype, wl.batch, wl.num_qo_heads, wl.num_kv_heads,
                           kv_dtype=wl.kv_dtype, **knobs)
        self.plan = fa.Plan(geom, device=device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(wl.rows, wl.num_qo_heads, dtype=torch.float32, device=device)
        self.indptr_h = np.ascontiguousarray(wl.kv_indptr)
        self.lens_h = np.ascontiguousarray(wl.kv_lens.astype(np.int32))

    def step(self, i: int, ev=None):
        self.plan.plan(self.indptr_h, self.lens_h)
        if ev is not None:
            ev[0].record()
        self.run_call(i)
        if ev is not None:
            ev[1].record()

    def run_call(self, i: int):
        pool = self.pools[i % len(self.pools)]
        args = (self.plan, self.q, pool[:, 0], pool[:, 1], *self.strides, self.kv_indices,
                self.kv_indptr, self.last)
        if self.wl.kv_dtype is None:
            self.fa.decode(*args, out=self.out, lse=self.lse)
        else:
            self.fa.decode_scaled(*args, k_scale=self.wl.k_scale, v_scale=self.wl.v_scale,
                                  out=self.out, lse=self.lse)


def attainable_read_gbs(nbytes: int = 1 << 30, launches: int = 10) -> dict:
    """HBM bandwidth of a plain streaming read on this device (the library's
    fa_probe_stream_read over a 1 GiB buffer, 4x the Infinity Cache), the best
    median over a few launch sizes, each launch timed with HIP events."""
    import torch
    import paged_kv_cache_fa_amd as fa
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    best = (0.0, 0)
    for wg in (512, 1024, 2048, 4096, 8192):
        for _ in range(3):
            fa.probe_stream_read(src, flag, wg)
        ev = [(HipEvent(), HipEvent()) for _ in range(launches)]
        for a, b in ev:
            a.record()
            fa.probe_stream_read(src, flag, wg)
            b.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        best = max(best, (nbytes / (ms * 1e-3) / 1e9, wg))
    del src, flag
    torch.cuda.empty_cache()
    return {"GB/s": round(best[0], 1), "workgroups": best[1]}


def plan_us(b: DecodeBench, n: int = 200) -> float:
    """Host time of one fa_plan call (build + enqueue of the upload)."""
    import torch
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(n):
        b.plan.plan(b.indptr_h, b.lens_h)
    dt = (time.perf_counter() - t) / n
    torch.cuda.synchronize()
    return dt * 1e6


class RaggedDecodeBench(Timed):
    """Decode over a ragged KV cache (rows of K / V in request order)."""

    def __init__(self, rw, device="cuda", min_rotation_bytes=1 << 30, **knobs):
        import torch
        import paged_kv_cache_fa_amd as fa
        self.fa, self.rw = fa, rw
        dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[rw.dtype]
        k = torch.from_numpy(rw.k.view(np.int16)).to(device).view(dt)
        v = torch.from_numpy(rw.v.view(np.int16)).to(device).view(dt)
        copies = max(1, math.ceil(min_rotation_bytes / (2 * k.numel() * 2)))
        self.kv = [(k, v)] + [(k.clone(), v.clone()) for _ in range(copies - 1)]
        self.q = torch.from_numpy(rw.q.view(np.int16)).to(device).view(dt)
        self.offs = _i32(rw.kv_offsets, device)
        self.offs_h = np.ascontiguousarray(rw.kv_offsets, dtype=np.int32)
        geom = fa.geometry("decode", rw.dtype, rw.batch, rw.num_qo_heads, rw.num_kv_heads, **knobs)
        self.plan = fa.Plan(geom, device=device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(rw.rows, rw.num_qo_heads, dtype=torch.float32, device=device)

    def step(self, i: int, ev=None):
        self.plan.plan_ragged(self.offs_h)
        if ev is not None:
            ev[0].record()
        self.run_call(i)
        if ev is not None:
            ev[1].record()

    def run_call(self, i: int):
        k, v = self.kv[i % len(self.kv)]
        self.fa.decode_ragged(self.plan, self.q, k, v, k.stride(0), k.stride(1), self.offs,
                              out=self.out, lse=self.lse)


def ragged_bytes(rw) -> int:
    return kv_bytes(rw.kv_lens, rw.num_kv_heads) + io_bytes(rw.rows, rw.num_qo_heads)


class BlockSparseBench(Timed):
    """Block-sparse attention: the pattern's page table is built once (a
    static pattern); every step re-plans and runs the append kernel."""

    def __init__(self, bw, device="cuda"):
        import torch
        import paged_kv_cache_fa_amd as fa
        self.fa, self.bw = fa, bw
        dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[bw.dtype]
        t = lambda a: torch.from_numpy(a.view(np.int16)).to(device).view(dt)
        self.q, self.k, self.v = t(bw.q), t(bw.k), t(bw.v)
        ip, ix, last, lens = fa.block_sparse_pages(bw.block_indptr, bw.block_indices,
                                                   bw.col_offsets)
        self.ip_h, self.lens_h, self.ro_h = ip, lens, np.ascontiguousarray(bw.row_offsets)
        self.ip, self.ix, self.last = _i32(ip, device), _i32(ix, device), _i32(last, device)
        self.ro = _i32(bw.row_offsets, device)
        nrb = len(bw.row_offsets) - 1
        geom = fa.geometry("append", bw.dtype, nrb, bw.num_qo_heads, bw.num_kv_heads,
                           max_qo_tokens=int(bw.row_offsets[-1]))
        self.plan = fa.Plan(geom, device=device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[0], bw.num_qo_heads, dtype=torch.float32,
                               device=device)
        self.flops = float((np.diff(bw.row_offsets) * lens).sum()) * bw.num_qo_heads * 4 * 128

    def step(self, i: int, ev=None):
        self.plan.plan(self.ip_h, self.lens_h, self.ro_h, False)
        if ev is not None:
            ev[0].record()
        ts, hs = self.k.stride(0), self.k.stride(1)
        self.fa.append(self.plan, self.q, self.ro, self.k, self.v, ts, ts, hs, self.ix, self.ip,
                       self.last, out=self.out, lse=self.lse)
        if ev is not None:
            ev[1].record()


class PodBench(Timed):
    """A mixed batch (prefill / append requests + decode requests, one pool):
    fa_pod, or fa_append then fa_decode when ``separate``."""

    def __init__(self, wl, n_prefill, device="cuda", separate=False):
        import torch
        import paged_kv_cache_fa_amd as fa
        self.fa, self.wl, self.separate = fa, wl, separate
        self.pools, q, self.strides = _dev(wl, device, 1 << 30)
        ip, ix, last, qo = wl.kv_indptr, wl.kv_indices, wl.last_page_len, wl.qo_indptr
        k = int(ip[n_prefill])
        self.nrows_p = int(qo[n_prefill])
        self.q_p, self.q_d = q[: self.nrows_p], q[self.nrows_p:]
        self.pre_h = (np.ascontiguousarray(ip[: n_prefill + 1]), wl.kv_lens[:n_prefill].copy(),
                      np.ascontiguousarray(qo[: n_prefill + 1]))
        self.dec_h = ((ip[n_prefill:] - k).astype(np.int32), wl.kv_lens[n_prefill:].copy())
        self.ptabs = (_i32(ix[:k], device), _i32(ip[: n_prefill + 1], device),
                      _i32(last[:n_prefill], device))
        self.dtabs = (_i32(ix[k:], device), _i32(self.dec_h[0], device),
                      _i32(last[n_prefill:], device))
        self.qo = _i32(qo[: n_prefill + 1], device)
        gp = fa.geometry("append", wl.dtype, n_prefill, wl.num_qo_heads, wl.num_kv_heads,
                         max_qo_tokens=self.nrows_p)
        gd = fa.geometry("decode", wl.dtype, wl.batch - n_prefill, wl.num_qo_heads,
                         wl.num_kv_heads)
        self.pp, self.dp = fa.Plan(gp, device=device), fa.Plan(gd, device=device)
        self.out_p = torch.empty_like(self.q_p)
        self.out_d = torch.empty_like(self.q_d)
        mk = lambda n: torch.empty(n, wl.num_qo_heads, dtype=torch.float32, device=device)
        self.lse_p, self.lse_d = mk(self.nrows_p), mk(self.q_d.shape[0])

    def step(self, i: int, ev=None):
        fa = self.fa
        pool = self.pools[i % len(self.pools)]
        k, v = pool[:, 0], pool[:, 1]
        self.pp.plan(*self.pre_h, True)
        self.dp.plan(*self.dec_h)
        if ev is not None:
            ev[0].record()
        if self.separate:
            fa.append(self.pp, self.q_p, self.qo, k, v, *self.strides, *self.ptabs,
                      out=self.out_p, lse=self.lse_p)
            fa.decode(self.dp, self.q_d, k, v, *self.strides, *self.dtabs, out=self.out_d,
                      lse=self.lse_d)
        else:
            fa.pod(self.pp, self.q_p, self.qo, *self.ptabs, self.dp, self.q_d, *self.dtabs, k, v,
                   *self.strides, out_p=self.out_p, lse_p=self.lse_p, out_d=self.out_d,
                   lse_d=self.lse_d)
        if ev is not None:
            ev[1].record()


class AppendBench(Timed):
    def __init__(self, wl, device="cuda", min_rotation_bytes=1 << 30, **knobs):
        import torch
        import paged_kv_cache_fa_amd as fa
        self.fa, self.wl = fa, wl
        self.pools, self.q, self.strides = _dev(wl, device, min_rotation_bytes)
        self.kv_indptr = _i32(wl.kv_indptr, device)
        self.kv_indices = _i32(wl.kv_indices, device)
        self.last = _i32(wl.last_page_len, device)
        self.qo_indptr = _i32(wl.qo_indptr, device)
        geom = fa.geometry("append", wl.dtype, wl.batch, wl.num_qo_heads, wl.num_kv_heads,
                           max_qo_tokens=wl.rows, **knobs)
        self.plan = fa.Plan(geom, device=device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(wl.rows, wl.num_qo_heads, dtype=torch.float32, device=device)

    def step(self, i: int, ev=None):
        wl = self.wl
        pool = self.pools[i % len(self.pools)]
        self.plan.plan(wl.kv_indptr, wl.kv_lens, wl.qo_indptr, wl.causal)
        if ev is not None:
            ev[0].record()
        self.fa.append(self.plan, self.q, self.qo_indptr, pool[:, 0], pool[:, 1], *self.strides,
                       self.kv_indices, self.kv_indptr, self.last, out=self.out, lse=self.lse)
        if ev is not None:
            ev[1].record()


class CascadeBench(Timed):
    """One fa_cascade call: the suffix decode (HBM), the prefix pass
    (non-causal append over the shared prefix, MFMA) and the combine kernel;
    the kernel time is the whole call."""

    def __init__(self, wl, device="cuda", min_rotation_bytes=1 << 30, prefix_knobs=None,
                 suffix_knobs=None):
        import torch
        import paged_kv_cache_fa_amd as fa
        self.fa, self.wl = fa, wl
        B = wl.batch
        self.pools, self.q, self.strides = _dev(wl, device, min_rotation_bytes)
        self.kv_indptr = _i32(wl.kv_indptr, device)
        self.kv_indices = _i32(wl.kv_indices, device)
        self.last = _i32(wl.last_page_len, device)
        self.p_indptr = _i32(wl.prefix_indptr, device)
        self.p_indices = _i32(wl.prefix_indices, device)
        self.p_last = _i32(wl.prefix_last_page_len, device)
        self.qo = _i32([0, B], device)
        gp = fa.geometry("append", wl.dtype, 1, wl.num_qo_heads, wl.num_kv_heads, max_qo_tokens=B,
                         **(prefix_knobs or {}))
        gs = fa.geometry("decode", wl.dtype, B, wl.num_qo_heads, wl.num_kv_heads,
                         **(suffix_knobs or {}))
        self.pplan = fa.Plan(gp, device=device)
        self.splan = fa.Plan(gs, device=device)
        mk = lambda: (torch.empty_like(self.q),
                      torch.empty(B, wl.num_qo_heads, dtype=torch.float32, device=device))
        self.op, self.lp = mk()
        self.os, self.ls = mk()
        self.out, self.lse = mk()
        # One stream: measured on MI355X, running the prefix pass on a side
        # stream beside the suffix decode is slower (they compete for each
        # CU's registers and caches) than running the two back to back.
        self.side = None

    def step(self, i: int, ev=None):
        wl, fa = self.wl, self.fa
        pool = self.pools[i % len(self.pools)]
        k, v = pool[:, 0], pool[:, 1]
        self.pplan.plan(wl.prefix_indptr, [wl.prefix_len], [0, wl.batch], False)
        self.splan.plan(wl.kv_indptr, wl.kv_lens)
        if ev is not None:
            ev[0].record()
        fa.cascade(self.pplan, self.splan, self.q, k, v, *self.strides, self.qo, self.p_indices,
                   self.p_indptr, self.p_last, self.kv_indices, self.kv_indptr, self.last,
                   states=(self.op, self.lp, self.os, self.ls), out=self.out, lse=self.lse,
                   side_stream=self.side)
        if ev is not None:
            ev[1].record()


KERNEL_SOURCES = ("decode.hip", "decode_dev.h", "device_common.h", "kernels.h")


def kernel_source_sha256() -> str:
    """SHA-256 over the decode kernel's source files, in a fixed order."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "paged_kv_cache_fa_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def stored_traffic(kernel_src: str = ""):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    fields = {}
    for line in open(COUNTERS_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, min_seconds: float = 10.0) -> dict:
    """The fp64 oracle on the host cores, repeated over the batch for >= min_seconds."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    per_tok = wl.num_kv_heads * wl.head_dim * 2 * 2
    done_bytes, done_req, t_used, passes = 0, 0, 0.0, 0
    while t_used < min_seconds and passes < 20:
        for b in range(wl.batch):
            t = time.perf_counter()
            oracle.decode(wl.q, wl.pool, wl.dtype, wl.kv_indptr, wl.kv_indices, wl.last_page_len,
                          wl.page_size, requests=[b])
            t_used += time.perf_counter() - t
            done_bytes += int(wl.kv_lens[b]) * per_tok + io_bytes(1, wl.num_qo_heads)
            done_req += 1
        passes += 1
    return {"value": round(done_bytes / t_used / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle over all {wl.batch} requests of the same workload, "
                      f"{passes} pass(es): {done_req / t_used:.1f} requests/s "
                      f"({done_req / t_used * 1:.1f} tokens/s), {t_used:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="decode workload for the headline (1-3)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true", help="skip batch128/cascade/append")
    ap.add_argument("--parts", default="batch128,cascade,append,fp8,ragged,single,bsr,pod",
                    help="comma list of the secondary workloads to run after the headline")
    ap.add_argument("--knob", action="append", default=[], help="decode plan knob name=value")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one plain 1 GiB device copy first (scales rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path (requests "
              "or kv heads would shard across GPUs with no exchange; long sequences by key "
              "range, with an all-gather of partial states and a local merge).", file=sys.stderr)
        sys.exit(2)
    import torch
    from workloads import CONFIG_NAMES, config_lengths, make_config
    knobs = {k: int(v) for k, v in (s.split("=") for s in args.knob)}
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    wl = make_config(args.config)
    b = DecodeBench(wl, **knobs)
    step_ms, kernel_ms = b.run(args.steps, args.warmup)
    host_plan_us = plan_us(b)
    att = attainable_read_gbs()
    nbytes = algorithmic_bytes(wl)
    gbs = nbytes / (step_ms * 1e-3) / 1e9
    kgbs = nbytes / (kernel_ms * 1e-3) / 1e9
    st = b.plan.info()
    traffic = stored_traffic()
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": CONFIG_NAMES[args.config],
                   "batch": wl.batch, "num_qo_heads": wl.num_qo_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "page_size": wl.page_size, "kv_tokens": int(wl.kv_lens.sum()),
                   "algorithmic_bytes": nbytes, "pool_copies": len(b.pools),
                   "tiles": st.num_tiles, "split_units": st.num_merge,
                   "workers": st.num_workers, "piece_pages": st.chunk_pages},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(wl.batch / (step_ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(kgbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "decode_kernel (one fa_decode call)",
                     "kernel_ms": round(kernel_ms, 5), "algorithmic_bytes": nbytes,
                     "attainable_GB/s": att["GB/s"],
                     "frac_of_attainable": round(kgbs / att["GB/s"], 4)},
        "host_plan_us": round(host_plan_us, 1),
    }
    del b
    torch.cuda.empty_cache()
    parts = set() if args.only_headline else set(filter(None, args.parts.split(",")))
    if "batch128" in parts:
        w3 = make_config(3)
        b3 = DecodeBench(w3, **knobs)
        s3, k3 = b3.run(args.steps, args.warmup)
        n3 = algorithmic_bytes(w3)
        line["batch128"] = {"workload": CONFIG_NAMES[3],
                            "GB/s": round(n3 / (s3 * 1e-3) / 1e9, 2),
                            "pct_of_hbm_peak": round(100 * n3 / (s3 * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                            "tokens_per_s": round(128 / (s3 * 1e-3), 1),
                            "ms_per_step": round(s3, 5), "kernel_ms": round(k3, 5)}
        del b3, w3
        torch.cuda.empty_cache()
    if "cascade" in parts:
        w4 = make_config(4)
        b4 = CascadeBench(w4)
        s4, k4 = b4.run(max(5, args.steps // 2), max(2, args.warmup // 2))
        n4 = algorithmic_bytes(w4)
        line["cascade"] = {"workload": CONFIG_NAMES[4],
                           "GB/s": round(n4 / (s4 * 1e-3) / 1e9, 2),
                           "pct_of_hbm_peak": round(100 * n4 / (s4 * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                           "tokens_per_s": round(256 / (s4 * 1e-3), 1),
                           "ms_per_step": round(s4, 5), "kernel_ms": round(k4, 5),
                           "algorithmic_bytes": n4}
        del b4
        torch.cuda.empty_cache()
        # context: the same batch as one plain decode (each request re-reads the prefix)
        wn = no_cascade_view(w4)
        bn = DecodeBench(wn, max_tiles=40000, max_partials=40000, max_merge=4096)
        sn, kn = bn.run(5, 2)
        nn = algorithmic_bytes(wn)
        # (its re-read prefix pages mostly come from the 256 MB Infinity Cache, so this
        # effective rate is not an HBM figure)
        line["cascade"]["no_cascade_decode"] = {
            "kernel_ms": round(kn, 5), "ms_per_step": round(sn, 5), "algorithmic_bytes": nn,
            "effective_GB/s": round(nn / (kn * 1e-3) / 1e9, 2)}
        line["cascade"]["speedup_over_no_cascade"] = round(kn / k4, 2)
        del bn, wn, w4
        torch.cuda.empty_cache()
    if "append" in parts:
        w5 = make_config(5)
        b5 = AppendBench(w5)
        s5, k5 = b5.run(max(5, args.steps // 2), max(2, args.warmup // 2))
        f5 = append_flops(w5)
        line["append"] = {"workload": CONFIG_NAMES[5],
                          "TFLOP/s": round(f5 / (k5 * 1e-3) / 1e12, 1),
                          "mfma_utilisation": round(f5 / (k5 * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
                          "flops": f5, "kernel_ms": round(k5, 5), "ms_per_step": round(s5, 5),
                          "tokens_per_s": round(w5.rows / (s5 * 1e-3), 1)}
        del b5, w5
        torch.cuda.empty_cache()
    if "fp8" in parts:
        w8 = make_config(2, kv_dtype="e4m3")
        b8 = DecodeBench(w8, **knobs)
        s8, k8 = b8.run(args.steps, args.warmup)
        n8 = algorithmic_bytes(w8)
        line["fp8"] = {"workload": f"{CONFIG_NAMES[2]}, K/V pages in E4M3",
                       "kv_dtype": "e4m3", "k_scale": w8.k_scale, "v_scale": w8.v_scale,
                       "GB/s": round(n8 / (s8 * 1e-3) / 1e9, 2),
                       "pct_of_hbm_peak": round(100 * n8 / (s8 * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                       "kernel_GB/s": round(n8 / (k8 * 1e-3) / 1e9, 2),
                       "kernel_frac": round(n8 / (k8 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "tokens_per_s": round(w8.batch / (s8 * 1e-3), 1),
                       "ms_per_step": round(s8, 5), "kernel_ms": round(k8, 5),
                       "algorithmic_bytes": n8}
        del b8, w8
        torch.cuda.empty_cache()
    from workloads import make_ragged
    for part, k in (("ragged", 2), ("single", 1)):
        if part not in parts:
            continue
        wk = make_config(k)
        rw = make_ragged(wk.kv_lens, wk.num_qo_heads, wk.num_kv_heads, wk.dtype, seed=k)
        br = RaggedDecodeBench(rw, **knobs)
        sr, kr = br.run(args.steps, args.warmup)
        gr = br.graph_call_ms(len(br.kv))
        nr = ragged_bytes(rw)
        line[part] = {"workload": f"{CONFIG_NAMES[k]}, ragged (contiguous) K/V",
                      "GB/s": round(nr / (sr * 1e-3) / 1e9, 2),
                      "pct_of_hbm_peak": round(100 * nr / (sr * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                      "kernel_GB/s": round(nr / (kr * 1e-3) / 1e9, 2),
                      "tokens_per_s": round(rw.batch / (sr * 1e-3), 1),
                      "ms_per_step": round(sr, 5), "kernel_ms": round(kr, 5),
                      "graph_ms_per_call": round(gr, 5),
                      "graph_GB/s": round(nr / (gr * 1e-3) / 1e9, 2),
                      "algorithmic_bytes": nr, "kv_copies": len(br.kv)}
        del br, rw, wk
        torch.cuda.empty_cache()
    if "bsr" in parts:
        from workloads import make_block_sparse
        bw = make_block_sparse([64] * 64, [64] * 256, 0.25, 32, 8, "bf16", seed=7)
        bb = BlockSparseBench(bw)
        sb, kb = bb.run(max(5, args.steps // 2), max(2, args.warmup // 2))
        line["bsr"] = {"workload": "block-sparse prefill: 4096 query rows x 16384 keys, 64 x 64 "
                                   "blocks, 25% kept (seeded), 32/8 heads, bf16",
                       "TFLOP/s": round(bb.flops / (kb * 1e-3) / 1e12, 1),
                       "mfma_utilisation": round(bb.flops / (kb * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS,
                                                 4),
                       "flops": bb.flops, "kernel_ms": round(kb, 5), "ms_per_step": round(sb, 5),
                       "blocks_kept": int(len(bw.block_indices))}
        del bb, bw
        torch.cuda.empty_cache()
    if "pod" in parts:
        from workloads import make_workload
        r5, r2 = np.random.default_rng(5), np.random.default_rng(2)
        l5, l2 = config_lengths(5, r5), config_lengths(2, r2)
        lens = np.concatenate([l5["kv_lens"], l2["kv_lens"]])
        qo = np.concatenate([l5["qo_lens"], np.ones(len(l2["kv_lens"]), np.int64)])
        wm = make_workload(lens, 32, 8, "bf16", 52, qo_lens=qo, causal=True, name="mixed")
        n_pre = len(l5["kv_lens"])
        res = {}
        for sep in (False, True):
            pb = PodBench(wm, n_pre, separate=sep)
            sp, kp = pb.run(max(5, args.steps // 2), max(2, args.warmup // 2))
            res[sep] = (sp, kp)
            del pb
            torch.cuda.empty_cache()
        f5 = append_flops(make_config(5))
        line["pod"] = {"workload": "mixed batch over one pool: causal append (16 x 512 rows onto "
                                   "4096) + GQA decode (batch 64, kv U[512,4096]), 32/8 heads, bf16",
                       "kernel_ms": round(res[False][1], 5),
                       "separate_kernels_ms": round(res[True][1], 5),
                       "speedup": round(res[True][1] / res[False][1], 3),
                       "ms_per_step": round(res[False][0], 5),
                       "tokens_per_s": round((wm.rows) / (res[False][0] * 1e-3), 1),
                       "append_flops": f5}
        del wm
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
