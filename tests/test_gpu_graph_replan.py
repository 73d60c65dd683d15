"""A captured run call stays valid across re-plans ([DeepDive] "Snippet One": the
plan is made before capture and a new plan with new lengths keeps the captured
launch; "The Architecture, Unpacked": static launch shape, dynamic tile
assignment).

Each test captures one run call into a graph on stream ``s`` over fixed device
buffers (pool, q, page tables, outputs), then for a sequence of workloads with
new lengths: copies the workload's bytes into those buffers, re-plans on ``s``
(same geometry and workspaces), replays the graph on ``s`` and compares every
row with the fp64 oracle over that workload. The upload of a re-plan and the
replay are ordered by the stream itself.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle  # noqa: E402
from gpu_util import assert_close, to_f64, torch_dtype  # noqa: E402
from workloads import make_cascade, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu


class Slots:
    """Device buffers sized for the largest of a list of workloads; a workload's
    stored bytes are copied into their leading parts."""

    def __init__(self, wls, prefix=False):
        import torch
        w0 = wls[0]
        self.fp8 = w0.kv_dtype == "e4m3"
        self.dt = torch_dtype(w0.dtype)
        P = max(w.pool.shape[0] for w in wls)
        shape = (P,) + w0.pool.shape[1:]
        self.pool = torch.zeros(shape, dtype=torch.uint8 if self.fp8 else self.dt, device="cuda")
        rows = max(w.q.shape[0] for w in wls)
        self.q = torch.zeros((rows,) + w0.q.shape[1:], dtype=self.dt, device="cuda")
        self.out = torch.zeros_like(self.q)
        self.lse = torch.zeros(rows, w0.num_qo_heads, dtype=torch.float32, device="cuda")
        i32 = lambda n: torch.zeros(max(n, 1), dtype=torch.int32, device="cuda")
        self.kv_indices = i32(max(len(w.kv_indices) for w in wls))
        self.kv_indptr = i32(max(len(w.kv_indptr) for w in wls))
        self.last = i32(max(len(w.last_page_len) for w in wls))
        self.qo = i32(max(len(w.kv_indptr) for w in wls))
        if prefix:
            self.p_indices = i32(max(len(w.prefix_indices) for w in wls))
            self.p_indptr = i32(2)
            self.p_last = i32(1)
            self.p_qo = i32(2)
            B = rows
            self.states = (torch.zeros_like(self.q), torch.zeros(B, w0.num_qo_heads,
                                                                 dtype=torch.float32,
                                                                 device="cuda"),
                           torch.zeros_like(self.q), torch.zeros(B, w0.num_qo_heads,
                                                                 dtype=torch.float32,
                                                                 device="cuda"))
        _, _, ps, hkv, d = w0.pool.shape
        self.strides = (2 * ps * hkv * d, hkv * d, d)

    def load(self, wl):
        import torch

        def put(dst, a):
            a = np.ascontiguousarray(a, dtype=np.int32)
            dst[: a.shape[0]].copy_(torch.from_numpy(a).cuda())

        self.pool.zero_()
        src = torch.from_numpy(wl.pool if self.fp8 else wl.pool.view(np.int16))
        self.pool[: wl.pool.shape[0]].copy_(src.cuda().view(self.pool.dtype))
        self.q[: wl.q.shape[0]].copy_(torch.from_numpy(wl.q.view(np.int16)).cuda().view(self.dt))
        self.out.fill_(7)
        self.lse.fill_(7)
        for dst in (self.kv_indices, self.kv_indptr, self.last, self.qo):
            dst.zero_()
        put(self.kv_indices, wl.kv_indices)
        put(self.kv_indptr, wl.kv_indptr)
        put(self.last, wl.last_page_len)
        if wl.qo_indptr is not None:
            put(self.qo, wl.qo_indptr)
        if wl.prefix_indptr is not None:
            put(self.p_indices, wl.prefix_indices)
            put(self.p_indptr, wl.prefix_indptr)
            put(self.p_last, wl.prefix_last_page_len)
            put(self.p_qo, np.array([0, wl.batch], np.int32))
        torch.cuda.synchronize()

    @property
    def k(self):
        return self.pool[:, 0]

    @property
    def v(self):
        return self.pool[:, 1]


def _replay_check(s, g, replan, slots, wls, ref_of, rows_of):
    """For each workload: load, re-plan on s, replay on s, compare with the oracle."""
    import torch
    for rep, wl in enumerate(wls):
        print(f"[graph re-plan] step {rep}: lens {list(wl.kv_lens)[:6]}", flush=True)
        slots.load(wl)
        replan(wl)
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        n = rows_of(wl)
        ref = ref_of(wl)
        e = assert_close(to_f64(slots.out[:n]), to_f64(slots.lse[:n]), *ref,
                         what=f"replay {rep} lens {list(wl.kv_lens)[:6]}")
        print(f"   max-abs out {e[0]:.3g} lse {e[1]:.3g}", flush=True)


def _capture(s, fn):
    import torch
    with torch.cuda.stream(s):
        fn()  # eager warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("kv_dtype", [None, "e4m3"])
def test_decode_graph_replan(kv_dtype):
    """Paged decode (16-bit or E4M3 pool): new lengths, a smaller batch and a
    split / unsplit change between replays."""
    import torch
    import paged_kv_cache_fa_amd as fa
    mk = lambda lens, seed: make_workload(lens, 32, 8, "bf16", seed, mode="test",
                                          kv_dtype=kv_dtype)
    wls = [mk([300, 1000, 17, 4000, 1], 21), mk([4000, 5, 2500, 640, 3000], 22),
           mk([16, 2, 33], 23), mk([1, 9000, 64, 100, 0], 24)]
    slots = Slots(wls)
    s = torch.cuda.Stream()
    geom = fa.geometry("decode", "bf16", 5, 32, 8, num_cu=16, tiles_per_cu=4, kv_dtype=kv_dtype)
    plan = fa.Plan(geom, device="cuda")
    plan.plan(wls[0].kv_indptr, wls[0].kv_lens, stream=s)
    torch.cuda.synchronize()
    args = lambda: (plan, slots.q, slots.k, slots.v, *slots.strides, slots.kv_indices,
                    slots.kv_indptr, slots.last)
    if kv_dtype is None:
        run = lambda: fa.decode(*args(), out=slots.out, lse=slots.lse, stream=s)
    else:
        run = lambda: fa.decode_scaled(*args(), k_scale=wls[0].k_scale, v_scale=wls[0].v_scale,
                                       out=slots.out, lse=slots.lse, stream=s)
    slots.load(wls[0])
    g = _capture(s, run)

    def ref_of(wl):
        return oracle.decode(wl.q, wl.pool, wl.dtype, wl.kv_indptr, wl.kv_indices,
                             wl.last_page_len, wl.page_size, kv_dtype=wl.kv_dtype,
                             k_scale=wl.k_scale, v_scale=wl.v_scale)

    _replay_check(s, g, lambda wl: plan.plan(wl.kv_indptr, wl.kv_lens, stream=s), slots,
                  wls * 2, ref_of, lambda wl: wl.batch)


def test_append_graph_replan_causal_switch():
    """Append: new lengths and query counts, and the mask switched between causal
    and non-causal by the re-plan alone (the kernel reads it from the plan)."""
    import torch
    import paged_kv_cache_fa_amd as fa
    cases = [([700, 130, 64], [100, 64, 1], True), ([2048, 33], [256, 33], False),
             ([5, 500, 16, 1000], [5, 70, 16, 3], True), ([900, 10], [128, 10], False)]
    wls = [make_workload(l, 32, 8, "bf16", 31 + i, qo_lens=q, causal=c, mode="test")
           for i, (l, q, c) in enumerate(cases)]
    slots = Slots(wls)
    s = torch.cuda.Stream()
    rows = max(w.rows for w in wls)
    geom = fa.geometry("append", "bf16", 4, 32, 8, max_qo_tokens=rows, num_cu=8, tiles_per_cu=4)
    plan = fa.Plan(geom, device="cuda")
    replan = lambda wl: plan.plan(wl.kv_indptr, wl.kv_lens, wl.qo_indptr, wl.causal, stream=s)
    replan(wls[0])
    torch.cuda.synchronize()
    slots.load(wls[0])
    run = lambda: fa.append(plan, slots.q, slots.qo, slots.k, slots.v, *slots.strides,
                            slots.kv_indices, slots.kv_indptr, slots.last, out=slots.out,
                            lse=slots.lse, stream=s)
    g = _capture(s, run)

    def ref_of(wl):
        return oracle.append(wl.q, wl.qo_indptr, wl.pool, wl.dtype, wl.kv_indptr,
                             wl.kv_indices, wl.last_page_len, wl.page_size, causal=wl.causal)

    _replay_check(s, g, replan, slots, wls * 2, ref_of, lambda wl: wl.rows)


@pytest.mark.parametrize("qo_tile", [32, 64])
def test_cascade_graph_replan(qo_tile):
    """fa_cascade (one kernel for both passes, in its shared or wide form, + the
    combine): new suffix lengths, a new prefix length (split into chunks or
    not) and a smaller batch."""
    import torch
    import paged_kv_cache_fa_amd as fa
    wls = [make_cascade(512, [5, 16, 17, 300, 1, 64], 32, 8, "bf16", 41, mode="test"),
           make_cascade(96, [900, 0, 3, 40, 2, 7], 32, 8, "bf16", 42, mode="test"),
           make_cascade(2048, [33, 1, 250], 32, 8, "bf16", 43, mode="test")]
    slots = Slots(wls, prefix=True)
    s = torch.cuda.Stream()
    B = max(w.batch for w in wls)
    gp = fa.geometry("append", "bf16", 1, 32, 8, max_qo_tokens=B, num_cu=8, qo_tile=qo_tile)
    pplan = fa.Plan(gp, device="cuda")
    splan = fa.Plan(fa.geometry("decode", "bf16", B, 32, 8, num_cu=8), device="cuda")

    def replan(wl):
        pplan.plan(wl.prefix_indptr, [wl.prefix_len], [0, wl.batch], False, stream=s)
        splan.plan(wl.kv_indptr, wl.kv_lens, stream=s)

    replan(wls[0])
    torch.cuda.synchronize()
    slots.load(wls[0])
    run = lambda: fa.cascade(pplan, splan, slots.q, slots.k, slots.v, *slots.strides, slots.p_qo,
                             slots.p_indices, slots.p_indptr, slots.p_last, slots.kv_indices,
                             slots.kv_indptr, slots.last, states=slots.states, out=slots.out,
                             lse=slots.lse, stream=s)
    g = _capture(s, run)

    def ref_of(wl):
        return oracle.cascade(wl.q, wl.pool, wl.dtype, wl.prefix_indptr, wl.prefix_indices,
                              wl.prefix_last_page_len, wl.kv_indptr, wl.kv_indices,
                              wl.last_page_len, wl.page_size)

    _replay_check(s, g, replan, slots, wls * 2, ref_of, lambda wl: wl.batch)
