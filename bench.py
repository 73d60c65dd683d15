"""Benchmark: paged-KV attention hot path on one MI355X.

Headline (the JSON ``value``): batched paged decode, batch 64, GQA 32 q / 8 kv
heads, head_dim 128, bf16, page 16, kv_len uniform in [512, 4096], pages
scattered by a seeded permutation. One step = the host plan (balanced
split-KV work list, uploaded to the device workspace) + the decode kernel
(which also merges split requests), steps back to back with nothing else
queued between them. ``value`` is the achieved algorithmic HBM bandwidth of
the step in GB/s: bytes of the valid K/V of every request, plus q, out and
lse, divided by the wall time per step.

Every line reports a ``roofline`` block for its dominant kernel: its
algorithmic bytes (or FLOPs) per run call over the call's time measured with
HIP timing events on the launch stream (each call re-planned first, outside
the events), against the 8 TB/s HBM or the 2.5 PFLOP/s bf16 MFMA peak, with
``traffic`` (HBM bytes per call from rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled
by a 1 GiB copy) when ``profiles/<line>_hbm_counters.txt`` was taken on this
line and on the current kernel sources. Decode lines also give the timing
protocol for a run call alone, ``graph_ms_per_call``: one hipGraph of R
back-to-back calls over the rotating pool copies, median of 20 replays / R.

Lines after the headline:
  * ``single``: the single-request decode (one request, 32/32 heads, 2048
    tokens in 128 pages under a seeded permutation, fp16), a graph of 32 back-to-back
    calls over 32 pool copies (its eager step is bound by the host);
  * ``batch128``: the skewed batch-128 decode (4 x 32768 + 124 log-normal);
  * ``cascade``: batch 256 sharing a 16384-token prefix (one fa_cascade call:
    prefix pass on MFMA + suffix decode + merge), HBM GB/s with the prefix
    counted once; its roofline times the call in a graph of back-to-back
    calls (eagerly the GPU finishes a call before the host has queued the
    next); ``no_cascade_decode`` times the same batch as one plain
    decode whose requests each re-read the prefix pages (17.9 GB);
  * ``append``: causal append of 16 x 512 rows onto 4096 cached tokens, MFMA
    utilisation (584.2 GFLOP of unmasked work per call);
  * ``fp8``: the batch-64 decode over an E4M3 page pool (per-tensor scales);
  * ``ragged`` / ``single_ragged``: the batch-64 and single-request decodes
    over a ragged (contiguous) K/V;
  * ``bsr``: block-sparse prefill, 4096 x 16384 in 64 x 64 blocks, 25% kept;
  * ``pod``: causal append + batch-64 decode in one fa_pod launch against the
    two kernels back to back;
  * ``groups``: the batch-64 decode lengths at GQA group sizes 1, 2, 4, 8
    (16-bit and E4M3 pools), the decode call alone;
  * ``host_plan_us`` (the host cost of one fa_plan), the streaming-read ceiling
    ``roofline.attainable_GB/s`` (fa_probe_stream_read over 1 GiB) and
    ``cpu_baseline`` (the fp64 numpy oracle on the host cores).

``--profile LINE`` runs only one line's run call (for rocprofv3 kernel-trace and
counter runs) and ``--profile LINE --summarize DIR`` turns that run's CSV output
into the text summaries kept under profiles/.

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
N_XCD, N_CU, N_SIMD = 8, 256, 1024
METRIC = "paged decode achieved HBM GB/s (% of peak) and tokens/sec at batch 64/128"


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


def _dev(wl, device, min_rotation_bytes, min_copies=1):
    """Device copies of the pool (enough copies to rotate over min_rotation_bytes,
    at least min_copies), q and the pool strides."""
    import torch
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[wl.dtype]
    if wl.kv_dtype == "e4m3":
        pool = torch.from_numpy(wl.pool).to(device)
    else:
        pool = torch.from_numpy(wl.pool.view(np.int16)).to(device).view(dt)
    copies = max(min_copies,
                 math.ceil(min_rotation_bytes / max(1, pool.numel() * pool.element_size())))
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
    """Timing of one workload line. A bench object provides ``replan()`` (the
    host plan + its upload, on torch's current stream) and ``run_call(i)``
    (the run calls of one step over input copy i)."""

    def step(self, i: int):
        self.replan()
        self.run_call(i)

    def warm(self, warmup: int) -> int:
        """Untimed steps before a timed run: at least one per rotated input
        copy (the first launch over a copy is slow, a one-time cost)."""
        return max(warmup, len(getattr(self, "pools", ())))

    def steps_ms(self, steps: int, warmup: int) -> float:
        """Whole steps (re-plan + run), back to back with nothing else queued
        between them: torch events around all steps, mean per step."""
        import torch
        warmup = self.warm(warmup)
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(steps):
            self.step(warmup + i)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def kernel_ms(self, launches: int, warmup: int = 2) -> float:
        """The run calls alone: each step re-plans, then HIP timing events on
        the launch stream bracket its run calls; mean over the launches."""
        import torch
        warmup = self.warm(warmup)
        for i in range(warmup):
            self.step(i)
        ev = [(HipEvent(), HipEvent()) for _ in range(launches)]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(ev):
            self.replan()
            a.record()
            self.run_call(warmup + i)
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev]))

    def graph_ms(self, calls: int, replays: int = 20) -> float:
        """The timing protocol for a run call alone: one hipGraph of `calls`
        back-to-back run calls over the rotating input copies (plan made once,
        before capture), replayed `replays` times; median time per call."""
        import torch
        self.step(0)
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
    """fa_plan + fa_decode (fa_decode_scaled for an E4M3 pool) over a paged pool."""

    def __init__(self, wl, device="cuda", min_rotation_bytes=1 << 30, min_copies=1, **knobs):
        import torch
        import paged_kv_cache_fa_amd as fa
        self.fa, self.wl = fa, wl
        self.pools, self.q, self.strides = _dev(wl, device, min_rotation_bytes, min_copies)
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

    def replan(self):
        self.plan.plan(self.indptr_h, self.lens_h)

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
        b.replan()
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

    def replan(self):
        self.plan.plan_ragged(self.offs_h)

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

    def replan(self):
        self.plan.plan(self.ip_h, self.lens_h, self.ro_h, False)

    def run_call(self, i: int):
        ts, hs = self.k.stride(0), self.k.stride(1)
        self.fa.append(self.plan, self.q, self.ro, self.k, self.v, ts, ts, hs, self.ix, self.ip,
                       self.last, out=self.out, lse=self.lse)


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
        # both forms take the append kernel's default q tiles (256 / G rows),
        # which fa_pod runs in the append kernel's workgroup shape
        gp = fa.geometry("append", wl.dtype, n_prefill, wl.num_qo_heads, wl.num_kv_heads,
                         max_qo_tokens=self.nrows_p)
        gd = fa.geometry("decode", wl.dtype, wl.batch - n_prefill, wl.num_qo_heads,
                         wl.num_kv_heads)
        self.pp, self.dp = fa.Plan(gp, device=device), fa.Plan(gd, device=device)
        self.out_p = torch.empty_like(self.q_p)
        self.out_d = torch.empty_like(self.q_d)
        mk = lambda n: torch.empty(n, wl.num_qo_heads, dtype=torch.float32, device=device)
        self.lse_p, self.lse_d = mk(self.nrows_p), mk(self.q_d.shape[0])

    def replan(self):
        self.pp.plan(*self.pre_h, True)
        self.dp.plan(*self.dec_h)

    def run_call(self, i: int):
        fa = self.fa
        pool = self.pools[i % len(self.pools)]
        k, v = pool[:, 0], pool[:, 1]
        if self.separate:
            fa.append(self.pp, self.q_p, self.qo, k, v, *self.strides, *self.ptabs,
                      out=self.out_p, lse=self.lse_p)
            fa.decode(self.dp, self.q_d, k, v, *self.strides, *self.dtabs, out=self.out_d,
                      lse=self.lse_d)
        else:
            fa.pod(self.pp, self.q_p, self.qo, *self.ptabs, self.dp, self.q_d, *self.dtabs, k, v,
                   *self.strides, out_p=self.out_p, lse_p=self.lse_p, out_d=self.out_d,
                   lse_d=self.lse_d)


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

    def replan(self):
        wl = self.wl
        self.plan.plan(wl.kv_indptr, wl.kv_lens, wl.qo_indptr, wl.causal)

    def run_call(self, i: int):
        pool = self.pools[i % len(self.pools)]
        self.fa.append(self.plan, self.q, self.qo_indptr, pool[:, 0], pool[:, 1], *self.strides,
                       self.kv_indices, self.kv_indptr, self.last, out=self.out, lse=self.lse)


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
        # prefix q tiles of the append default (256 / G rows) in the one-launch
        # kernel's wide form: the suffix decode's 8-wave workgroups hold 128
        # CUs, so the prefix is planned as one round of tiles for the other 128
        pk = {"num_cu": 128, "tiles_per_cu": 1, **(prefix_knobs or {})}
        gp = fa.geometry("append", wl.dtype, 1, wl.num_qo_heads, wl.num_kv_heads, max_qo_tokens=B,
                         **pk)
        gs = fa.geometry("decode", wl.dtype, B, wl.num_qo_heads, wl.num_kv_heads,
                         **(suffix_knobs or {}))
        self.pplan = fa.Plan(gp, device=device)
        self.splan = fa.Plan(gs, device=device)
        mk = lambda: (torch.empty_like(self.q),
                      torch.empty(B, wl.num_qo_heads, dtype=torch.float32, device=device))
        self.op, self.lp = mk()
        self.os, self.ls = mk()
        self.out, self.lse = mk()

    def replan(self):
        wl = self.wl
        self.pplan.plan(wl.prefix_indptr, [wl.prefix_len], [0, wl.batch], False)
        self.splan.plan(wl.kv_indptr, wl.kv_lens)

    def run_call(self, i: int):
        # one stream: measured on MI355X, running the prefix pass on a side
        # stream beside the suffix decode is slower than the one-kernel form
        pool = self.pools[i % len(self.pools)]
        k, v = pool[:, 0], pool[:, 1]
        self.fa.cascade(self.pplan, self.splan, self.q, k, v, *self.strides, self.qo,
                        self.p_indices, self.p_indptr, self.p_last, self.kv_indices,
                        self.kv_indptr, self.last, states=(self.op, self.lp, self.os, self.ls),
                        out=self.out, lse=self.lse)


# --- stored rocprofv3 counter summaries ---------------------------------------------------------

# kernel sources whose hash keys a stored counter summary, per line
KERNEL_SOURCES = {
    "decode": ("decode.hip", "decode_dev.h", "device_common.h", "kernels.h"),
    "cascade": ("pod.hip", "append_dev.h", "decode_dev.h", "merge.hip", "device_common.h",
                "kernels.h"),
    "append": ("append.hip", "append_dev.h", "device_common.h", "kernels.h"),
}
LINE_KERNEL = {"decode_batch64": "decode", "decode_batch128": "decode",
               "decode_fp8_batch64": "decode", "decode_single_kv2048": "decode",
               "cascade_batch256": "cascade", "append_causal_batch16": "append"}


def kernel_source_sha256(kind: str = "decode") -> str:
    """SHA-256 over the source files of a line's kernels, in a fixed order."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        h.update(open(os.path.join(ROOT, "paged_kv_cache_fa_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def counters_file(line: str) -> str:
    return os.path.join(ROOT, "profiles", f"{line}_hbm_counters.txt")


def stored_traffic(line: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled) from the committed
    counter summary of this line, if it was taken on this workload and on the
    current kernel sources; else None."""
    path = counters_file(line)
    if not os.path.exists(path):
        return None
    fields = {}
    for text in open(path):
        if ":" in text and not text.startswith("#"):
            k, v = text.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("line") != line or \
            fields.get("kernel_source_sha256") != kernel_source_sha256(LINE_KERNEL[line]):
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


def hbm_roofline(line, nbytes, kernel_ms, kernel_name, **extra) -> dict:
    gbs = nbytes / (kernel_ms * 1e-3) / 1e9
    r = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": stored_traffic(line),
         "kernel": kernel_name, "kernel_ms": round(kernel_ms, 5), "algorithmic_bytes": nbytes}
    r.update(extra)
    return r


def mfma_roofline(flops, kernel_ms, kernel_name, **extra) -> dict:
    tf = flops / (kernel_ms * 1e-3) / 1e12
    r = {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
         "frac": round(tf / MFMA_PEAK_TFLOPS, 4), "traffic": None, "kernel": kernel_name,
         "kernel_ms": round(kernel_ms, 5), "algorithmic_flops": flops}
    r.update(extra)
    return r


# --- workload lines -------------------------------------------------------------------------------

def line_decode(k, steps, warmup, kv_dtype=None, knobs=None):
    """A batched paged decode (batch 64 or the skewed batch 128, or batch 64
    over an E4M3 pool):
    whole steps (re-plan + decode), the decode call alone with HIP events, and
    the graph protocol (R back-to-back calls over the rotating pool copies)."""
    from workloads import CONFIG_NAMES, make_config
    wl = make_config(k, kv_dtype=kv_dtype) if kv_dtype else make_config(k)
    b = DecodeBench(wl, **(knobs or {}))
    step_ms = b.steps_ms(steps, warmup)
    kern_ms = b.kernel_ms(steps)
    graph_ms = b.graph_ms(len(b.pools))
    nbytes = algorithmic_bytes(wl)
    st = b.plan.info()
    line = "decode_fp8_batch64" if kv_dtype else {2: "decode_batch64", 3: "decode_batch128"}[k]
    res = {"workload": CONFIG_NAMES[k] + (", K/V pages in E4M3" if kv_dtype else ""),
           "GB/s": round(nbytes / (step_ms * 1e-3) / 1e9, 2),
           "pct_of_hbm_peak": round(100 * nbytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
           "tokens_per_s": round(wl.batch / (step_ms * 1e-3), 1),
           "ms_per_step": round(step_ms, 5),
           "roofline": hbm_roofline(line, nbytes, kern_ms, "decode_kernel (one fa_decode call)",
                                    graph_ms_per_call=round(graph_ms, 5),
                                    graph_frac=round(nbytes / (graph_ms * 1e-3) / 1e9 /
                                                     HBM_PEAK_GBS, 4)),
           "plan": {"tiles": st.num_tiles, "split_units": st.num_merge,
                    "workers": st.num_workers, "piece_pages": st.chunk_pages},
           "pool_copies": len(b.pools), "kv_tokens": int(wl.kv_lens.sum())}
    if kv_dtype:
        res.update(kv_dtype=kv_dtype, k_scale=wl.k_scale, v_scale=wl.v_scale)
    return res, b, wl


def line_single(steps, warmup):
    """The single-request decode: one request, q [32, 128] fp16, K/V of 2048 tokens
    x 32 kv heads in 128 pages of 16 tokens under a seeded random page
    permutation; a graph of 32 back-to-back fa_decode calls over 32 pool
    copies (the timing protocol), and the eager step for context."""
    from workloads import CONFIG_NAMES, make_config
    wl = make_config(1)
    b = DecodeBench(wl, min_copies=32)
    graph_ms = b.graph_ms(len(b.pools))
    step_ms = b.steps_ms(steps, warmup)
    kern_ms = b.kernel_ms(steps)
    nbytes = algorithmic_bytes(wl)
    st = b.plan.info()
    return {"workload": CONFIG_NAMES[1] + ", 128 pages in a seeded permutation",
            "GB/s": round(nbytes / (graph_ms * 1e-3) / 1e9, 2),
            "pct_of_hbm_peak": round(100 * nbytes / (graph_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "tokens_per_s": round(1 / (graph_ms * 1e-3), 1),
            "graph_ms_per_call": round(graph_ms, 5), "eager_ms_per_step": round(step_ms, 5),
            "roofline": hbm_roofline("decode_single_kv2048", nbytes, graph_ms,
                                     "decode_kernel (graph of 32 back-to-back fa_decode calls)",
                                     event_kernel_ms=round(kern_ms, 5)),
            "plan": {"tiles": st.num_tiles, "split_units": st.num_merge,
                     "piece_pages": st.chunk_pages},
            "pool_copies": len(b.pools)}


def line_cascade(steps, warmup):
    from workloads import CONFIG_NAMES, make_config
    w4 = make_config(4)
    b4 = CascadeBench(w4)
    n = max(5, steps // 2)
    step_ms = b4.steps_ms(n, max(2, warmup // 2))
    # the run call from a graph of back-to-back calls: eagerly, the GPU
    # finishes a call before the host has queued the next one's launches
    kern_ms = b4.graph_ms(2 * len(b4.pools))
    n4 = algorithmic_bytes(w4)
    res = {"workload": CONFIG_NAMES[4],
           "GB/s": round(n4 / (step_ms * 1e-3) / 1e9, 2),
           "pct_of_hbm_peak": round(100 * n4 / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
           "tokens_per_s": round(w4.batch / (step_ms * 1e-3), 1),
           "ms_per_step": round(step_ms, 5),
           "roofline": hbm_roofline("cascade_batch256", n4, kern_ms,
                                    "pod_kernel + cascade_merge_kernel (one fa_cascade call)")}
    del b4
    import torch
    torch.cuda.empty_cache()
    # context: the same batch as one plain decode (each request re-reads the prefix)
    wn = no_cascade_view(w4)
    bn = DecodeBench(wn, max_tiles=40000, max_partials=40000, max_merge=4096)
    kn = bn.kernel_ms(5)
    nn = algorithmic_bytes(wn)
    # (its re-read prefix pages mostly come from the 256 MB Infinity Cache, so this
    # effective rate is not an HBM figure)
    res["no_cascade_decode"] = {"kernel_ms": round(kn, 5), "algorithmic_bytes": nn,
                                "effective_GB/s": round(nn / (kn * 1e-3) / 1e9, 2)}
    res["speedup_over_no_cascade"] = round(kn / kern_ms, 2)
    return res


def line_append(steps, warmup):
    from workloads import CONFIG_NAMES, make_config
    w5 = make_config(5)
    b5 = AppendBench(w5)
    n = max(5, steps // 2)
    step_ms = b5.steps_ms(n, max(2, warmup // 2))
    kern_ms = b5.kernel_ms(n)
    f5 = append_flops(w5)
    return {"workload": CONFIG_NAMES[5],
            "TFLOP/s": round(f5 / (step_ms * 1e-3) / 1e12, 1),
            "tokens_per_s": round(w5.rows / (step_ms * 1e-3), 1),
            "ms_per_step": round(step_ms, 5),
            "roofline": mfma_roofline(f5, kern_ms, "append_kernel (one fa_append call)",
                                      algorithmic_bytes=algorithmic_bytes(w5))}


def line_ragged(k, steps, warmup):
    from workloads import CONFIG_NAMES, make_config, make_ragged
    wk = make_config(k)
    rw = make_ragged(wk.kv_lens, wk.num_qo_heads, wk.num_kv_heads, wk.dtype, seed=k)
    br = RaggedDecodeBench(rw)
    sr = br.steps_ms(steps, warmup)
    kr = br.kernel_ms(steps)
    gr = br.graph_ms(len(br.kv))
    nr = ragged_bytes(rw)
    return {"workload": f"{CONFIG_NAMES[k]}, ragged (contiguous) K/V",
            "GB/s": round(nr / (sr * 1e-3) / 1e9, 2), "ms_per_step": round(sr, 5),
            "kernel_ms": round(kr, 5), "kernel_GB/s": round(nr / (kr * 1e-3) / 1e9, 2),
            "graph_ms_per_call": round(gr, 5), "graph_GB/s": round(nr / (gr * 1e-3) / 1e9, 2),
            "algorithmic_bytes": nr, "kv_copies": len(br.kv)}


def line_bsr(steps, warmup):
    from workloads import make_block_sparse
    bw = make_block_sparse([64] * 64, [64] * 256, 0.25, 32, 8, "bf16", seed=7)
    bb = BlockSparseBench(bw)
    n = max(5, steps // 2)
    sb = bb.steps_ms(n, max(2, warmup // 2))
    kb = bb.kernel_ms(n)
    return {"workload": "block-sparse prefill: 4096 query rows x 16384 keys, 64 x 64 blocks, "
                        "25% kept (seeded), 32/8 heads, bf16",
            "ms_per_step": round(sb, 5), "blocks_kept": int(len(bw.block_indices)),
            "roofline": mfma_roofline(bb.flops, kb, "append_kernel (one fa_append call)")}


def line_groups(steps, warmup):
    """The batch-64 decode lengths at every GQA group size (8 kv heads, 8 to 64
    q heads; 16-bit and E4M3 pools): the decode call alone, HIP events after a
    re-plan, one line per group size and pool type. G <= 2 runs the VALU
    path, G >= 4 the matrix-core path."""
    import torch
    from workloads import config_lengths, make_workload
    lens = config_lengths(2, np.random.default_rng(2))["kv_lens"]
    res = {}
    for kvd in (None, "e4m3"):
        for g in (1, 2, 4, 8):
            wl = make_workload(lens, 8 * g, 8, "bf16", 2, kv_dtype=kvd)
            b = DecodeBench(wl)
            k = b.kernel_ms(max(10, steps // 2), warmup=3)
            n = algorithmic_bytes(wl)
            res[f"{kvd or 'bf16'}_G{g}"] = {"kernel_ms": round(k, 5),
                                           "GB/s": round(n / (k * 1e-3) / 1e9, 1),
                                           "frac": round(n / (k * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            del b, wl
            torch.cuda.empty_cache()
    return {"workload": "batch-64 decode lengths (kv U[512,4096], seed 2), 8 kv heads, "
                        "G = 1, 2, 4, 8 query heads per kv head, bf16 q", "lines": res}


def line_pod(steps, warmup):
    import torch
    from workloads import config_lengths, make_config, make_workload
    r5, r2 = np.random.default_rng(5), np.random.default_rng(2)
    l5, l2 = config_lengths(5, r5), config_lengths(2, r2)
    lens = np.concatenate([l5["kv_lens"], l2["kv_lens"]])
    qo = np.concatenate([l5["qo_lens"], np.ones(len(l2["kv_lens"]), np.int64)])
    wm = make_workload(lens, 32, 8, "bf16", 52, qo_lens=qo, causal=True, name="mixed")
    n_pre = len(l5["kv_lens"])
    res = {}
    n = max(5, steps // 2)
    for sep in (False, True):
        pb = PodBench(wm, n_pre, separate=sep)
        res[sep] = (pb.steps_ms(n, max(2, warmup // 2)), pb.kernel_ms(n))
        del pb
        torch.cuda.empty_cache()
    f5 = append_flops(make_config(5))
    return {"workload": "mixed batch over one pool: causal append (16 x 512 rows onto 4096) + "
                        "GQA decode (batch 64, kv U[512,4096]), 32/8 heads, bf16",
            "kernel_ms": round(res[False][1], 5), "separate_kernels_ms": round(res[True][1], 5),
            "speedup": round(res[True][1] / res[False][1], 3),
            "ms_per_step": round(res[False][0], 5),
            "tokens_per_s": round(wm.rows / (res[False][0] * 1e-3), 1), "append_flops": f5}


# --- profiling support ----------------------------------------------------------------------------

PROFILE_LINES = ("decode_batch64", "decode_batch128", "decode_fp8_batch64",
                 "decode_single_kv2048", "cascade_batch256", "append_causal_batch16")


def profile_line(line: str, steps: int, warmup: int, copy_probe: bool):
    """Run one line's run call `warmup + steps` times, each after a re-plan (as
    the roofline timing does), and nothing else (plus an optional plain 1 GiB
    device copy first, whose byte counters scale the kernel's), for a
    rocprofv3 kernel-trace or counter run."""
    import torch
    from workloads import make_config
    if copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    mk = {"decode_batch64": lambda: DecodeBench(make_config(2)),
          "decode_batch128": lambda: DecodeBench(make_config(3)),
          "decode_fp8_batch64": lambda: DecodeBench(make_config(2, kv_dtype="e4m3")),
          "decode_single_kv2048": lambda: DecodeBench(make_config(1), min_copies=32),
          "cascade_batch256": lambda: CascadeBench(make_config(4)),
          "append_causal_batch16": lambda: AppendBench(make_config(5))}[line]
    b = mk()
    torch.cuda.synchronize()
    for i in range(warmup + steps):
        b.replan()       # as in the roofline timing: every run call is re-planned first
        b.run_call(i)
    torch.cuda.synchronize()
    print(f"profiled {line}: {warmup} + {steps} run calls", flush=True)


def line_work(line: str):
    """(algorithmic bytes, algorithmic FLOPs) of one run call of a line."""
    from workloads import make_config
    k = {"decode_batch64": 2, "decode_batch128": 3, "decode_fp8_batch64": 2,
         "decode_single_kv2048": 1, "cascade_batch256": 4, "append_causal_batch16": 5}[line]
    wl = make_config(k, kv_dtype="e4m3") if line == "decode_fp8_batch64" else make_config(k)
    return algorithmic_bytes(wl), (append_flops(wl) if k == 5 else None)


def is_path_kernel(name: str) -> bool:
    """A kernel of the attention path (not the plan upload, nor a runtime or
    torch kernel)."""
    return "pkfa::" in name and "upload_kernel" not in name and "stream_read" not in name


def summarize(line: str, run_dir: str, command: str, warmup: int) -> str:
    """Text summary of rocprofv3 runs of `--profile line` (kernel trace and / or
    counters, CSV output under the comma-separated directories run_dir), for
    profiles/."""
    import csv
    import glob
    import re
    out = [f"# rocprofv3 summary: {line} (one MI355X, gfx950)", f"# command: {command}",
           f"line: {line}"]
    nbytes, flops = line_work(line)
    dirs = run_dir.split(",")
    traces = [f for d in dirs for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"),
                                                 recursive=True)]
    counters = [f for d in dirs for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"),
                                                   recursive=True)]
    totals = {}
    short = lambda n: re.sub(r"\(.*", "", re.sub(r"^(void )?pkfa::\(anonymous namespace\)::", "", n))
    if traces:
        rows = sorted(csv.DictReader(open(traces[0])), key=lambda r: int(r["Start_Timestamp"]))
        by = {}
        for r in rows:
            by.setdefault(r["Kernel_Name"], []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        for name, ds in by.items():
            if not is_path_kernel(name):
                continue
            ds = ds[warmup:] if len(ds) > warmup else ds
            out.append(f"kernel: {short(name)}  launches {len(ds)}  avg_us {np.mean(ds):.2f}  "
                       f"min_us {np.min(ds):.2f}  max_us {np.max(ds):.2f}")
        main_k = [n for n in by if is_path_kernel(n)]
        # the run call's time: all its kernels per call (cascade: two kernels)
        per_call = sum(np.mean(by[n][warmup:] if len(by[n]) > warmup else by[n]) for n in main_k)
        out.append(f"run_call_avg_us: {per_call:.2f}")
        if flops:
            out.append(f"algorithmic_flops_per_call: {flops:.0f}")
            tf = flops / (per_call * 1e-6) / 1e12
            out.append(f"achieved: {tf:.1f} TFLOP/s = {tf / MFMA_PEAK_TFLOPS:.4f} of "
                       f"{MFMA_PEAK_TFLOPS} TFLOP/s bf16 dense MFMA peak")
        else:
            gbs = nbytes / (per_call * 1e-6) / 1e9
            out.append(f"algorithmic_bytes_per_call: {nbytes}")
            out.append(f"achieved: {gbs:.1f} GB/s = {gbs / HBM_PEAK_GBS:.4f} of "
                       f"{HBM_PEAK_GBS:.0f} GB/s HBM peak")
    for path in counters:
        rows = list(csv.DictReader(open(path)))
        per = {}
        for r in rows:
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            per.setdefault(key, {}).setdefault(r["Counter_Name"], 0.0)
            per[key][r["Counter_Name"]] += float(r["Counter_Value"])
        copies = [v for (d, n), v in sorted(per.items()) if n == "__amd_rocclr_copyBuffer"
                  and max(v.values()) > 1e5]
        mine = [(d, n, v) for (d, n), v in sorted(per.items()) if is_path_kernel(n)]
        mine = mine[warmup * (2 if line == "cascade_batch256" else 1):]
        names = sorted({c for _, _, v in mine for c in v})
        for c in names:
            by_k = {}
            for _, n, v in mine:
                if c in v:
                    by_k.setdefault(short(n), []).append(v[c])
            for kname, vals in by_k.items():
                out.append(f"counter {c} {kname}: mean {np.mean(vals):.0f} over {len(vals)} "
                           f"dispatches")
        def per_call(counter):
            # sum over the call's kernels of each kernel's mean per dispatch
            by_name = {}
            for _, n, v in mine:
                if counter in v:
                    by_name.setdefault(n, []).append(v[counter])
            return sum(np.mean(x) for x in by_name.values()) if by_name else None

        fetch, write = per_call("FETCH_SIZE"), per_call("WRITE_SIZE")
        if copies and (fetch is not None or write is not None):
            c = copies[0]
            kib = 1 << 20  # the probe copies 1 GiB = 1048576 KiB
            if fetch is not None and "FETCH_SIZE" in c:
                f_scale = kib / c["FETCH_SIZE"]
                out.append(f"fetch_scale (1 GiB copy: {c['FETCH_SIZE']:.0f} KiB read): {f_scale:.4f}")
                out.append(f"fetch_bytes_per_call: {fetch * f_scale * 1024:.0f}")
                totals["fetch"] = fetch * f_scale * 1024
            if write is not None and "WRITE_SIZE" in c:
                w_scale = kib / c["WRITE_SIZE"]
                out.append(f"write_scale (1 GiB copy: {c['WRITE_SIZE']:.0f} KiB written): {w_scale:.4f}")
                out.append(f"write_bytes_per_call: {write * w_scale * 1024:.0f}")
                totals["write"] = write * w_scale * 1024
        # MFMA occupancy of the dominant kernel: busy cycles of the matrix units
        # over (GPU-active cycles of one XCD x 1024 SIMDs); GRBM_GUI_ACTIVE is
        # summed over the 8 XCDs, and its cycles over the dispatch's duration give
        # the clock the kernel actually ran at
        busy = [v for _, n, v in mine if "SQ_VALU_MFMA_BUSY_CYCLES" in v and "GRBM_GUI_ACTIVE" in v]
        if busy:
            act = np.mean([v["GRBM_GUI_ACTIVE"] for v in busy]) / N_XCD
            mb = np.mean([v["SQ_VALU_MFMA_BUSY_CYCLES"] for v in busy])
            out.append(f"mfma_busy_frac (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE/{N_XCD} x "
                       f"{N_SIMD} SIMDs)): {mb / (act * N_SIMD):.4f}")
            spans = {int(r["Dispatch_Id"]): (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9
                     for r in rows}
            durs = [spans[d] for d, n, v in mine
                    if "SQ_VALU_MFMA_BUSY_CYCLES" in v and "GRBM_GUI_ACTIVE" in v]
            if durs:
                out.append(f"active_clock_GHz (GRBM_GUI_ACTIVE/{N_XCD} over the dispatch time "
                           f"under counter collection): {act / np.mean(durs) / 1e9:.3f}")
            if "SQ_BUSY_CU_CYCLES" in busy[0]:
                cu = np.mean([v["SQ_BUSY_CU_CYCLES"] for v in busy])
                out.append(f"cu_busy_frac (SQ_BUSY_CU_CYCLES / (GRBM_GUI_ACTIVE/{N_XCD} x "
                           f"{N_CU} CUs)): {cu / (act * N_CU):.4f}")
    if "fetch" in totals and "write" in totals:
        hbm = totals["fetch"] + totals["write"]
        out.append(f"hbm_bytes_per_launch: {hbm:.0f}")
        out.append(f"algorithmic_bytes_per_launch: {nbytes}")
        out.append(f"traffic_over_algorithmic: {hbm / nbytes:.4f}")
    out.append(f"kernel_source_sha256: {kernel_source_sha256(LINE_KERNEL[line])}")
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true", help="skip the secondary lines")
    ap.add_argument("--parts",
                    default="single,batch128,cascade,append,fp8,ragged,single_ragged,bsr,pod,groups",
                    help="comma list of the secondary lines to run after the headline")
    ap.add_argument("--knob", action="append", default=[], help="decode plan knob name=value")
    ap.add_argument("--profile", choices=PROFILE_LINES,
                    help="run only this line's run call (for rocprofv3), print no JSON")
    ap.add_argument("--copy-probe", action="store_true",
                    help="with --profile: one plain 1 GiB device copy first (scales byte counters)")
    ap.add_argument("--summarize", metavar="DIRS",
                    help="with --profile: print a text summary of the rocprofv3 output in DIRS "
                         "(comma-separated)")
    ap.add_argument("--command", default="", help="with --summarize: the command that made DIR")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path (requests "
              "or kv heads would shard across GPUs with no exchange; long sequences by key "
              "range, with an all-gather of partial states and a local merge).", file=sys.stderr)
        sys.exit(2)
    if args.profile and args.summarize:
        sys.stdout.write(summarize(args.profile, args.summarize, args.command, args.warmup))
        return
    import torch
    if args.profile:
        profile_line(args.profile, args.steps, args.warmup, args.copy_probe)
        return
    from workloads import CONFIG_NAMES
    knobs = {k: int(v) for k, v in (s.split("=") for s in args.knob)}

    head, b, wl = line_decode(2, args.steps, args.warmup, knobs=knobs)
    host_plan_us = plan_us(b)
    del b
    torch.cuda.empty_cache()
    att = attainable_read_gbs()
    rl = head["roofline"]
    rl["attainable_GB/s"] = att["GB/s"]
    rl["frac_of_attainable"] = round(rl["achieved"] / att["GB/s"], 4)
    nbytes = rl["algorithmic_bytes"]
    step_ms = head["ms_per_step"]
    line = {
        "metric": METRIC,
        "value": head["GB/s"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": CONFIG_NAMES[2], "batch": wl.batch,
                   "num_qo_heads": wl.num_qo_heads, "num_kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "page_size": wl.page_size,
                   "kv_tokens": head["kv_tokens"], "algorithmic_bytes": nbytes,
                   "pool_copies": head["pool_copies"], **head["plan"]},
        "pct_of_hbm_peak": head["pct_of_hbm_peak"],
        "tokens_per_s": head["tokens_per_s"],
        "roofline": rl,
        "host_plan_us": round(host_plan_us, 1),
    }
    parts = set() if args.only_headline else set(filter(None, args.parts.split(",")))
    runners = [("single", lambda: line_single(args.steps, args.warmup)),
               ("batch128", lambda: line_decode(3, args.steps, args.warmup, knobs=knobs)[0]),
               ("cascade", lambda: line_cascade(args.steps, args.warmup)),
               ("append", lambda: line_append(args.steps, args.warmup)),
               ("fp8", lambda: line_decode(2, args.steps, args.warmup, kv_dtype="e4m3",
                                           knobs=knobs)[0]),
               ("ragged", lambda: line_ragged(2, args.steps, args.warmup)),
               ("single_ragged", lambda: line_ragged(1, args.steps, args.warmup)),
               ("bsr", lambda: line_bsr(args.steps, args.warmup)),
               ("pod", lambda: line_pod(args.steps, args.warmup)),
               ("groups", lambda: line_groups(args.steps, args.warmup))]
    for name, fn in runners:
        if name in parts:
            line[name] = fn()
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
