"""fa_decode_noalloc (plan + decode with the library's static per-GPU
workspaces, no allocation) against the existing entry points fa_plan +
fa_decode with caller-owned workspaces: two calls in a row on the same GPU,
the second with a smaller batch, must give the same bits (same plan, same
kernel), and both must match the fp64 oracle. A geometry whose workspace
exceeds the static arrays is refused with FA_ERR_CAPACITY before any work."""
import ctypes
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from gpu_util import DevWorkload, assert_close, oracle_decode, run_decode, to_f64  # noqa: E402
from workloads import make_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def _noalloc(geom, wl, dw, out, lse):
    """fa_decode_noalloc through the binding (status checked by the caller)."""
    import paged_kv_cache_fa_amd as fa
    lib = fa.load()
    ip = np.ascontiguousarray(wl.kv_indptr, dtype=np.int32)
    lens = np.ascontiguousarray(wl.kv_lens, dtype=np.int32)
    return lib.fa_decode_noalloc(ctypes.byref(geom), ip.ctypes.data, lens.ctypes.data, wl.batch,
                                 dw.q.data_ptr(), dw.k.data_ptr(), dw.v.data_ptr(), *dw.strides,
                                 dw.kv_indices.data_ptr(), dw.kv_indptr.data_ptr(),
                                 dw.last_page_len.data_ptr(), 0.0, out.data_ptr(),
                                 lse.data_ptr(), fa._stream(None))


def test_decode_noalloc_matches_fa_decode_two_calls():
    import torch
    import paged_kv_cache_fa_amd as fa
    lib = fa.load()
    rng = np.random.default_rng(77)
    cases = [(list(rng.integers(512, 4097, size=64)), 32, 8, "bf16", 71),   # the batch-64 shape
             ([1, 17, 300, 0, 1000, 16, 33, 2049], 32, 8, "bf16", 72)]      # then a smaller one
    for lens, hq, hkv, dtype, seed in cases:
        print(f"[noalloc] batch {len(lens)} seed {seed}", flush=True)
        wl = make_workload(lens, hq, hkv, dtype, seed, mode="test", extra_pages=2)
        dw = DevWorkload(wl)
        geom = fa.geometry("decode", dtype, wl.batch, hq, hkv)
        _, ref_o, ref_l = run_decode(dw)                   # fa_plan + fa_decode, own workspaces
        out = torch.full_like(ref_o, 7)
        lse = torch.full_like(ref_l, 7)
        st = _noalloc(geom, wl, dw, out, lse)
        assert st == 0, lib.fa_last_error()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"batch {wl.batch}"
        e = assert_close(to_f64(out), to_f64(lse), *oracle_decode(wl), what=f"noalloc {wl.batch}")
        # the Python binding reaches the same entry point
        o2, l2 = fa.decode_noalloc(geom, wl.kv_indptr, wl.kv_lens, dw.q, dw.k, dw.v, *dw.strides,
                                   dw.kv_indices, dw.kv_indptr, dw.last_page_len)
        torch.cuda.synchronize()
        assert torch.equal(o2, ref_o) and torch.equal(l2, ref_l)
        print(f"   bit-identical to fa_decode; oracle max-abs out {e[0]:.3g} lse {e[1]:.3g}",
              flush=True)


def test_decode_noalloc_refuses_oversized_geometry():
    import torch
    import paged_kv_cache_fa_amd as fa
    lib = fa.load()
    wl = make_workload([16], 32, 8, "bf16", 1)
    dw = DevWorkload(wl)
    out = torch.empty_like(dw.q)
    lse = torch.empty(1, 32, dtype=torch.float32, device="cuda")
    big = fa.geometry("decode", "bf16", 4096, 32, 8)      # workspace far beyond the static arrays
    st = _noalloc(big, wl, dw, out, lse)
    assert st == fa._lib.FA_ERR_CAPACITY and b"static" in lib.fa_last_error()
