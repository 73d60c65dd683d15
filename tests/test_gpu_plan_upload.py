"""The plan's trip to the device ([Guide] "What FlashInfer is", idea 3: a plan
per step, a static launch; [DeepDive] "It In Action": plan, then run).

* Back-to-back re-plans on one plan object with no synchronisation between
  steps: each fa_plan must wait until the previous copy has read the pinned
  host image before rewriting it. Two workloads alternate over 8 steps, each
  step's decode writes its own output, and every output is compared with the
  oracle at the end: a plan overwritten too early would pair a workload's page
  table with the other workload's tiles.
* A pageable (not pinned) host workspace takes the hipMemcpyAsync path; its
  results must be the bits of the pinned path.
"""
import ctypes
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from gpu_util import DevWorkload, assert_close, decode_geometry, oracle_decode, to_f64  # noqa: E402
from workloads import make_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def test_back_to_back_replans_alternating_workloads():
    import torch
    import paged_kv_cache_fa_amd as fa
    wa = make_workload([300, 4000, 17, 1000, 2500, 64], 32, 8, "bf16", 61, mode="test")
    wb = make_workload([4000, 5, 2600, 700, 1, 3000], 32, 8, "bf16", 62, mode="test")
    da, db = DevWorkload(wa), DevWorkload(wb)
    plan = fa.Plan(decode_geometry(wa, num_cu=32, tiles_per_cu=4), device="cuda")
    outs = []
    for step in range(8):
        wl, dw = (wa, da) if step % 2 == 0 else (wb, db)
        plan.plan(wl.kv_indptr, wl.kv_lens)
        out, lse = fa.decode(plan, dw.q, dw.k, dw.v, *dw.strides, dw.kv_indices, dw.kv_indptr,
                             dw.last_page_len)
        outs.append((wl, out, lse))
    torch.cuda.synchronize()
    refs = {id(wa): oracle_decode(wa), id(wb): oracle_decode(wb)}
    for step, (wl, out, lse) in enumerate(outs):
        e = assert_close(to_f64(out), to_f64(lse), *refs[id(wl)], what=f"step {step}")
        print(f"[back-to-back re-plan] step {step} max-abs out {e[0]:.3g} lse {e[1]:.3g}",
              flush=True)


def test_pageable_host_workspace_matches_pinned():
    import torch
    import paged_kv_cache_fa_amd as fa
    from paged_kv_cache_fa_amd import _lib
    lib = fa.load()
    wl = make_workload([700, 33, 2000, 5, 4096], 32, 8, "bf16", 63, mode="test")
    dw = DevWorkload(wl)
    geom = decode_geometry(wl, num_cu=16, tiles_per_cu=4)
    pinned = fa.Plan(geom, device="cuda").plan(wl.kv_indptr, wl.kv_lens)
    ref_o, ref_l = fa.decode(pinned, dw.q, dw.k, dw.v, *dw.strides, dw.kv_indices, dw.kv_indptr,
                             dw.last_page_len)
    hb, dbytes = fa.workspace_size(geom)
    host_ws = np.zeros(hb, dtype=np.uint8)                        # pageable
    dev_ws = torch.empty(dbytes, dtype=torch.uint8, device="cuda")
    raw = _lib.PlanT()
    ip = np.ascontiguousarray(wl.kv_indptr, dtype=np.int32)
    lens = np.ascontiguousarray(wl.kv_lens, dtype=np.int32)
    try:
        for rep in range(3):                                      # re-plans wait on the copy's event
            st = lib.fa_plan(ctypes.byref(raw), ctypes.byref(geom), ip.ctypes.data, lens.ctypes.data,
                             wl.batch, None, 0, host_ws.ctypes.data, hb, dev_ws.data_ptr(), dbytes,
                             fa._stream(None))
            assert st == 0, lib.fa_last_error()
            out = torch.full_like(ref_o, 7)
            lse = torch.full_like(ref_l, 7)
            st = lib.fa_decode(ctypes.byref(raw), dw.q.data_ptr(), dw.k.data_ptr(), dw.v.data_ptr(),
                               *dw.strides, dw.kv_indices.data_ptr(), dw.kv_indptr.data_ptr(),
                               dw.last_page_len.data_ptr(), 0.0, out.data_ptr(), lse.data_ptr(),
                               fa._stream(None))
            assert st == 0, lib.fa_last_error()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"rep {rep}"
    finally:
        lib.fa_plan_destroy(ctypes.byref(raw))
    assert_close(to_f64(ref_o), to_f64(ref_l), *oracle_decode(wl), what="pinned path")
