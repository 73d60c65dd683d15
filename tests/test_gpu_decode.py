"""GPU parity for paged decode against the fp64 oracle (through the C ABI)."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle_pins  # noqa: E402
from gpu_util import (DevWorkload, assert_close, oracle_decode, run_decode,  # noqa: E402
                      to_f64)
from workloads import CONFIG_NAMES, make_config, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def _case(lens, hq, hkv, dtype, seed, **kw):
    print(f"[decode case] lens={list(lens)[:8]}.. B={len(lens)} hq={hq} hkv={hkv} {dtype} "
          f"seed={seed} {kw}", flush=True)
    wl = make_workload(lens, hq, hkv, dtype, seed, mode="test", extra_pages=3)
    dw = DevWorkload(wl)
    plan, out, lse = run_decode(dw, **kw)
    ref = oracle_decode(wl)
    return assert_close(to_f64(out), to_f64(lse), *ref, what=str(lens)[:40]), plan


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_ragged_small(dtype, group):
    lens = [1, 15, 16, 17, 31, 33, 100, 257, 0, 513]
    hkv = 2
    _case(lens, hkv * group, hkv, dtype, 100 + group)


@pytest.mark.parametrize("tiles_per_cu,min_chunk", [(1, 1), (64, 1), (8, 3)])
def test_split_kv_paths(tiles_per_cu, min_chunk):
    """Force many splits (tiny chunks) and no splits; both must match."""
    lens = [1, 40, 300, 1000, 2049, 16]
    (e_out, e_lse), plan = _case(lens, 16, 4, "bf16", 7, num_cu=4, tiles_per_cu=tiles_per_cu,
                                 min_chunk_pages=min_chunk)
    st = plan.info()
    print("tiles", st.num_tiles, "merge rows", st.num_merge, "chunk pages", st.chunk_pages)


def test_identity_bit_exact_and_poison():
    """One-hot keys select one token per (request, kv head); out equals its V row bitwise."""
    import torch
    for dtype in ("bf16", "fp16"):
        for choose in ("first", "boundary", "last", "random"):
            wl, chosen = oracle_pins.identity_workload(dtype, choose=choose)
            print(f"[identity] {dtype} {choose}", flush=True)
            dw = DevWorkload(wl)
            for knobs in ({}, dict(num_cu=2, tiles_per_cu=16)):
                _, out, lse = run_decode(dw, **knobs)
                o = to_f64(out)
                assert np.isfinite(o).all()
                G = wl.num_qo_heads // wl.num_kv_heads
                for (b, hk), (page, slot) in chosen.items():
                    for h in range(hk * G, (hk + 1) * G):
                        expect = np.zeros(wl.head_dim)
                        expect[:4] = (page // 256, page % 256, slot, hk)
                        assert np.array_equal(o[b, h], expect), (dtype, choose, b, h, o[b, h, :4])
            torch.cuda.synchronize()


def test_count_lse_is_log_kv_len():
    lens = [1, 15, 16, 17, 31, 32, 33, 100, 0, 4097]
    wl = make_workload(lens, 8, 2, "bf16", 5, mode="test", extra_pages=2)
    wl.q[:] = 0
    dw = DevWorkload(wl)
    _, out, lse = run_decode(dw, num_cu=3, tiles_per_cu=5)
    l = to_f64(lse)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.isneginf(l[b]).all()
        else:
            assert np.max(np.abs(l[b] - np.log(L))) < 1e-5, (b, L, l[b])


def test_determinism():
    import torch
    wl = make_workload([700, 33, 2000, 5], 32, 8, "bf16", 9, mode="test")
    dw = DevWorkload(wl)
    plan, o1, l1 = run_decode(dw, num_cu=8, tiles_per_cu=4)
    o1, l1 = o1.clone(), l1.clone()
    _, o2, l2 = run_decode(dw, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("k", [1, 2, 3])
def test_benchmark_decode_workloads_full_size(k):
    print(f"[{CONFIG_NAMES[k]}] generating", flush=True)
    wl = make_config(k, mode="test")
    dw = DevWorkload(wl)
    plan, out, lse = run_decode(dw)
    st = plan.info()
    print(f"[{CONFIG_NAMES[k]}] tiles {st.num_tiles} merge {st.num_merge} P {st.chunk_pages}", flush=True)
    ref = oracle_decode(wl)
    e = assert_close(to_f64(out), to_f64(lse), *ref, what=CONFIG_NAMES[k])
    print(f"[{CONFIG_NAMES[k]}] max-abs out {e[0]:.3g} lse {e[1]:.3g}", flush=True)


@pytest.mark.parametrize("kv_dtype", [None, "e4m3"])
def test_group8_batch64_full_size(kv_dtype):
    """GQA group 8 (64 q / 8 kv heads) on the batch-64 lengths, every row: the
    group size whose scores run on the matrix cores."""
    from workloads import config_lengths
    lens = config_lengths(2, np.random.default_rng(2))["kv_lens"]
    print(f"[group 8 batch 64 {kv_dtype}] generating", flush=True)
    wl = make_workload(lens, 64, 8, "bf16", 12, mode="test", kv_dtype=kv_dtype)
    dw = DevWorkload(wl)
    plan, out, lse = run_decode(dw)
    e = assert_close(to_f64(out), to_f64(lse), *oracle_decode(wl), what=f"group 8 {kv_dtype}")
    print(f"[group 8 batch 64 {kv_dtype}] max-abs out {e[0]:.3g} lse {e[1]:.3g}", flush=True)


def test_graph_static_replan():
    """Capture decode once, re-plan with new lengths (same geometry), replay."""
    import torch
    import paged_kv_cache_fa_amd as fa
    from gpu_util import decode_geometry
    lens_a = [300, 1000, 17, 4000]
    lens_b = [4000, 5, 2500, 640]
    wa = make_workload(lens_a, 32, 8, "bf16", 21, mode="test", extra_pages=300)
    wb = make_workload(lens_b, 32, 8, "bf16", 22, mode="test", extra_pages=0)
    # one pool big enough for both; b's tables point into the same buffer
    P = max(wa.num_pages, wb.num_pages)
    assert wa.num_pages == P and wb.num_pages <= P
    dw = DevWorkload(wa)
    geom = decode_geometry(wa, num_cu=16, tiles_per_cu=4)
    plan = fa.Plan(geom, device="cuda").plan(wa.kv_indptr, wa.kv_lens)
    cap = 2 * P
    ind_buf = torch.zeros(cap, dtype=torch.int32, device="cuda")
    ind_buf[: len(wa.kv_indices)] = dw.kv_indices
    indptr_buf = dw.kv_indptr.clone()
    last_buf = dw.last_page_len.clone()
    q_buf = dw.q.clone()
    out = torch.empty_like(q_buf)
    lse = torch.empty(q_buf.shape[0], q_buf.shape[1], dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fa.decode(plan, q_buf, dw.k, dw.v, *dw.strides, ind_buf, indptr_buf, last_buf, out=out,
                  lse=lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fa.decode(plan, q_buf, dw.k, dw.v, *dw.strides, ind_buf, indptr_buf, last_buf, out=out,
                  lse=lse)
    for rep in range(3):
        for wl_ in (wa, wb):
            # new lengths: rewrite page tables in place, re-plan outside capture, replay
            pool_np = wa.pool.copy()
            pool_np[: wl_.num_pages] = wl_.pool
            dw.pool.copy_(torch.from_numpy(pool_np.view(np.int16)).cuda().view(dw.pool.dtype))
            ind_buf.zero_()
            ind_buf[: len(wl_.kv_indices)] = torch.from_numpy(wl_.kv_indices).cuda()
            indptr_buf.copy_(torch.from_numpy(wl_.kv_indptr).cuda())
            last_buf.copy_(torch.from_numpy(wl_.last_page_len).cuda())
            q_buf.copy_(torch.from_numpy(wl_.q.view(np.int16)).cuda().view(q_buf.dtype))
            torch.cuda.synchronize()
            # the upload and the replay are ordered by stream s
            plan.plan(wl_.kv_indptr, wl_.kv_lens, stream=s)
            with torch.cuda.stream(s):
                g.replay()
            torch.cuda.synchronize()
            wref = wl_
            wref_pool = pool_np
            import oracle
            ref = oracle.decode(wref.q, wref_pool, wref.dtype, wref.kv_indptr, wref.kv_indices,
                                wref.last_page_len, wref.page_size)
            assert_close(to_f64(out), to_f64(lse), *ref, what=f"replay {rep} {wl_.kv_lens}")


def test_plan_refuses_capture():
    import torch
    import paged_kv_cache_fa_amd as fa
    from gpu_util import decode_geometry
    wl = make_workload([40], 8, 2, "bf16", 1)
    plan = fa.Plan(decode_geometry(wl), device="cuda")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(fa.FAError) as e:
        with torch.cuda.graph(g, stream=s):
            plan.plan(wl.kv_indptr, wl.kv_lens, stream=s)
    assert e.value.code == "CAPTURING"
