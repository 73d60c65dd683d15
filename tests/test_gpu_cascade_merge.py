"""GPU parity: merge_state / merge_states kernels and the cascade path."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle  # noqa: E402
from gpu_util import (DevWorkload, assert_close, oracle_cascade, run_cascade,  # noqa: E402
                      to_f64, torch_dtype)
from workloads import make_cascade, make_config, to_storage_bits  # noqa: E402

pytestmark = pytest.mark.gpu


def _states(rng, shape, dtype, empty_frac=0.1):
    import torch
    v = rng.standard_normal(shape + (128,)).astype(np.float32)
    s = (rng.standard_normal(shape) * 3).astype(np.float32)
    s[rng.random(shape) < empty_frac] = -np.inf
    if dtype == "fp32":
        vt = torch.from_numpy(v).cuda()
        v64 = v.astype(np.float64)
    else:
        bits = to_storage_bits(v, dtype)
        vt = torch.from_numpy(bits.view(np.int16)).cuda().view(torch_dtype(dtype))
        v64 = oracle.upcast(bits, dtype)
    return vt, torch.from_numpy(s).cuda(), v64, s.astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_merge_state(dtype):
    import paged_kv_cache_fa_amd as fa
    rng = np.random.default_rng(1)
    va, sa, va64, sa64 = _states(rng, (37, 8), dtype)
    vb, sb, vb64, sb64 = _states(rng, (37, 8), dtype)
    sb[0, 0] = -np.inf
    sa[0, 0] = -np.inf          # both empty -> (0, -inf)
    sa64[0, 0] = sb64[0, 0] = -np.inf
    vo, so = fa.merge_state(va, sa, vb, sb)
    ro, rs = oracle.merge_state(va64, sa64, vb64, sb64)
    tol = 2e-2 if dtype != "fp32" else 1e-5
    assert_close(to_f64(vo), so.cpu().numpy().astype(np.float64), ro, rs, out_tol=tol,
                 what=f"merge_state {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("k", [1, 3, 17])
def test_merge_states(dtype, k):
    import paged_kv_cache_fa_amd as fa
    rng = np.random.default_rng(k)
    v, s, v64, s64 = _states(rng, (23, k, 4), dtype)
    vo, so = fa.merge_states(v, s)
    ro, rs = oracle.merge_states(np.moveaxis(v64, 1, 2), np.moveaxis(s64, 1, 2))
    tol = 2e-2 if dtype != "fp32" else 1e-5
    assert_close(to_f64(vo), so.cpu().numpy().astype(np.float64), ro, rs, out_tol=tol,
                 what=f"merge_states {dtype} k={k}")


@pytest.mark.parametrize("k", [3, 17])
def test_merge_states_ignores_empty_values(k):
    """A state with lse = -inf leaves the merge as it is, whatever its values
    hold (NaN here): the same bits as with finite values in those states."""
    import torch
    import paged_kv_cache_fa_amd as fa
    rng = np.random.default_rng(40 + k)
    v, s, _, _ = _states(rng, (23, k, 4), "fp32", empty_frac=0.3)
    v_nan = v.clone()
    v_nan[torch.isinf(s)] = float("nan")
    vo, so = fa.merge_states(v, s)
    vn, sn = fa.merge_states(v_nan, s)
    torch.cuda.synchronize()
    assert torch.equal(vo, vn) and torch.equal(so, sn)
    assert bool(torch.isfinite(vo).all())


def test_merge_recovers_unsplit_attention():
    """Two decode passes over disjoint halves of each request's keys, merged on
    the GPU, equal the oracle over the whole request."""
    import torch
    import paged_kv_cache_fa_amd as fa
    from workloads import make_workload
    from gpu_util import run_decode, oracle_decode
    lens = [640, 1024, 48]
    wl = make_workload(lens, 32, 8, "bf16", 17, mode="test")
    # first half: pages [0, n/2), second half: the rest, as two page tables
    halves = []
    for part in (0, 1):
        lists, L2 = [], []
        for b, L in enumerate(lens):
            pages = wl.kv_indices[wl.kv_indptr[b]: wl.kv_indptr[b + 1]]
            n = len(pages)
            cut = n // 2
            sel = pages[:cut] if part == 0 else pages[cut:]
            lists.append(sel)
            L2.append(cut * 16 if part == 0 else L - cut * 16)
        import copy
        w2 = copy.copy(wl)
        w2.kv_indptr = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
        w2.kv_indices = np.concatenate(lists).astype(np.int32)
        w2.kv_lens = np.array(L2, np.int32)
        w2.last_page_len = np.array([0 if x == 0 else x - 16 * ((x - 1) // 16) for x in L2],
                                    np.int32)
        dw = DevWorkload(w2)
        _, o, l_ = run_decode(dw)
        halves.append((o, l_))
    out, lse = fa.merge_state(halves[0][0], halves[0][1], halves[1][0], halves[1][1])
    ref = oracle_decode(wl)
    assert_close(to_f64(out), lse.cpu().numpy().astype(np.float64), *ref, what="split+merge")


# the prefix plan's q tile picks the one-launch kernel's shape: 128 / G rows
# share each CU with a decode workgroup, 256 / G (the default) take whole CUs
FORMS = {"shared": {"qo_tile": 32}, "wide": {}}


@pytest.mark.parametrize("form", sorted(FORMS))
def test_cascade_small(form):
    wl = make_cascade(256, [5, 16, 17, 300, 1], 32, 8, "bf16", 21, mode="test")
    dw = DevWorkload(wl)
    out, lse, _ = run_cascade(dw, prefix={"num_cu": 4, **FORMS[form]}, suffix={"num_cu": 4})
    ref = oracle_cascade(wl)
    assert_close(to_f64(out), to_f64(lse), *ref, what="cascade small")
    direct = oracle.cascade_direct(wl.q, wl.pool, wl.dtype, wl.prefix_indptr, wl.prefix_indices,
                                   wl.prefix_last_page_len, wl.kv_indptr, wl.kv_indices,
                                   wl.last_page_len, wl.page_size)
    assert_close(to_f64(out), to_f64(lse), *direct, what="cascade vs direct")


@pytest.mark.parametrize("form", sorted(FORMS))
@pytest.mark.parametrize("prefix_len,num_cu", [(512, 8), (96, 1), (2048, 64)])
def test_cascade_call(prefix_len, num_cu, form):
    """fa_cascade matches the oracle whether the prefix pass splits its keys
    (chunk partials merged with the suffix in the combine kernel) or not, and
    gives the same bits serially and with the passes forked onto other streams."""
    import torch
    wl = make_cascade(prefix_len, [5, 16, 17, 300, 1, 64, 900, 0], 32, 8, "bf16", 22,
                      mode="test")
    dw = DevWorkload(wl)
    _, _, plans = run_cascade(dw, prefix={"num_cu": num_cu, **FORMS[form]}, suffix={"num_cu": 8})
    print(f"[cascade] prefix {prefix_len} {form}: {plans[0].info().num_merge} split units",
          flush=True)
    o1, l1, _ = run_cascade(dw, *plans, fused=True)
    o1, l1 = o1.clone(), l1.clone()
    o2, l2, _ = run_cascade(dw, *plans, fused=True, side_stream=torch.cuda.Stream())
    o2, l2 = o2.clone(), l2.clone()
    o3, l3, _ = run_cascade(dw, *plans, fused=True, side_stream=torch.cuda.Stream(),
                            suffix_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    assert_close(to_f64(o1), to_f64(l1), *oracle_cascade(wl), what="fa_cascade")


@pytest.mark.parametrize("forked,form", [(True, "wide"), (False, "wide"), (False, "shared")])
def test_cascade_graph_capture_with_side_stream(forked, form):
    """fa_cascade captures into one graph, with the fork/join of a side stream
    or as the one-kernel form; replays (with eager work and synchronisation
    between them) reproduce the eager bits."""
    import torch
    import paged_kv_cache_fa_amd as fa
    wl = make_cascade(256, [40, 3, 700], 32, 8, "bf16", 23, mode="test")
    dw = DevWorkload(wl)
    _, _, plans = run_cascade(dw, prefix={"num_cu": 8, **FORMS[form]}, suffix={"num_cu": 8})
    ref_o, ref_l, _ = run_cascade(dw, *plans, fused=True)  # eager fa_cascade
    ref_o, ref_l = ref_o.clone(), ref_l.clone()
    assert plans[0].info().num_merge > 0  # the prefix chunks go through the combine kernel
    B, H = wl.batch, wl.num_qo_heads
    qo = torch.tensor([0, B], dtype=torch.int32, device="cuda")
    states = (torch.empty_like(dw.q), torch.empty(B, H, dtype=torch.float32, device="cuda"),
              torch.empty_like(dw.q), torch.empty(B, H, dtype=torch.float32, device="cuda"))
    out = torch.empty_like(dw.q)
    lse = torch.empty(B, H, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream() if forked else None
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        fa.cascade(plans[0], plans[1], dw.q, dw.k, dw.v, *dw.strides, qo, dw.prefix_indices,
                   dw.prefix_indptr, dw.prefix_last_page_len, dw.kv_indices, dw.kv_indptr,
                   dw.last_page_len, states=states, out=out, lse=lse, side_stream=side)
    for i in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {i}"


_FULL = {}


def _full_cascade():
    if not _FULL:
        print("[cascade batch 256] generating", flush=True)
        wl = make_config(4, mode="test")
        _FULL["wl"], _FULL["dw"] = wl, DevWorkload(wl)
        _FULL["ref"] = oracle_cascade(wl)
    return _FULL["wl"], _FULL["dw"], _FULL["ref"]


@pytest.mark.parametrize("form,knobs", [("wide", {"num_cu": 128, "tiles_per_cu": 1}),
                                        ("shared", {"qo_tile": 32})])
def test_cascade_batch256_full_size(form, knobs):
    """The batch-256 cascade (16384-token shared prefix) as one fa_cascade
    call on one stream (both passes in one kernel), in the launch
    configuration the benchmark times (wide: 64-row prefix tiles, one round
    of 128) and in the shared form; the same bits with the prefix pass forked onto a
    side stream."""
    import torch
    wl, dw, ref = _full_cascade()
    out, lse, plans = run_cascade(dw, fused=True, prefix=knobs)
    out, lse = out.clone(), lse.clone()
    o2, l2, _ = run_cascade(dw, *plans, fused=True, side_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    print(f"[cascade batch 256 {form}] prefix tiles {plans[0].info().num_tiles} suffix tiles "
          f"{plans[1].info().num_tiles}", flush=True)
    e = assert_close(to_f64(out), to_f64(lse), *ref, what=f"cascade batch 256 {form}")
    print(f"[cascade batch 256 {form}] all {wl.batch} requests: max-abs out {e[0]:.3g} "
          f"lse {e[1]:.3g}", flush=True)


def test_cascade_equals_decode_over_prefix_and_suffix():
    """fa_cascade against fa_decode over each request's whole page list (the
    shared prefix's pages, then its own): the two paths, and the oracle's
    direct attention over prefix ++ suffix, agree within the tolerances."""
    import dataclasses
    from gpu_util import run_decode
    wl = make_cascade(512, [5, 16, 17, 300, 1, 64, 0, 33], 32, 8, "bf16", 23, mode="test")
    dw = DevWorkload(wl)
    out_c, lse_c, _ = run_cascade(dw, fused=True, prefix={"num_cu": 8}, suffix={"num_cu": 8})
    pre = wl.prefix_indices[wl.prefix_indptr[0]:wl.prefix_indptr[1]]
    lists = [np.concatenate([pre, wl.kv_indices[wl.kv_indptr[b]:wl.kv_indptr[b + 1]]])
             for b in range(wl.batch)]
    indptr = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    whole = dataclasses.replace(
        wl, kv_lens=(wl.kv_lens + wl.prefix_len).astype(np.int32), kv_indptr=indptr,
        kv_indices=np.concatenate(lists).astype(np.int32), last_page_len=wl.last_page_len.copy(),
        prefix_len=0, prefix_indptr=None, prefix_indices=None, prefix_last_page_len=None)
    # a suffix of 0 tokens leaves the prefix's full last page as the request's last page
    whole.last_page_len[wl.kv_lens == 0] = 16
    _, out_d, lse_d = run_decode(DevWorkload(whole), num_cu=8)
    direct = oracle.cascade_direct(wl.q, wl.pool, wl.dtype, wl.prefix_indptr, wl.prefix_indices,
                                   wl.prefix_last_page_len, wl.kv_indptr, wl.kv_indices,
                                   wl.last_page_len, wl.page_size)
    assert_close(to_f64(out_c), to_f64(lse_c), *direct, what="cascade vs direct")
    assert_close(to_f64(out_d), to_f64(lse_d), *direct, what="decode over prefix ++ suffix")
    assert_close(to_f64(out_c), to_f64(lse_c), to_f64(out_d), to_f64(lse_d),
                 what="cascade vs decode")


def test_cascade_wide_prefix_tiles():
    """A prefix plan with q tiles of 256 / G positions (the planner's default
    for append) runs the one-launch kernel's wide form; same results as the
    oracle."""
    wl = make_cascade(512, [5, 16, 300, 0, 900], 32, 8, "bf16", 24, mode="test")
    dw = DevWorkload(wl)
    out, lse, plans = run_cascade(dw, fused=True, prefix={"qo_tile": 64, "num_cu": 8},
                                  suffix={"num_cu": 8})
    assert plans[0].info().resolved.qo_tile == 64
    assert_close(to_f64(out), to_f64(lse), *oracle_cascade(wl), what="cascade wide tiles")


@pytest.mark.parametrize("qo_tile", [32, 16])
def test_cascade_group8(qo_tile):
    """Eight query heads per kv head: prefix tiles of 32 rows run the one-kernel
    wide form; tiles of 16 rows (the shared form's, not built for G = 8) run
    the suffix decode and the append kernel in order; then the combine."""
    wl = make_cascade(704, [5, 16, 300, 0, 33], 32, 4, "bf16", 25, mode="test")
    dw = DevWorkload(wl)
    out, lse, plans = run_cascade(dw, fused=True, prefix={"qo_tile": qo_tile, "num_cu": 8},
                                  suffix={"num_cu": 8})
    assert plans[0].info().num_merge > 0
    assert_close(to_f64(out), to_f64(lse), *oracle_cascade(wl), what="cascade G = 8")
