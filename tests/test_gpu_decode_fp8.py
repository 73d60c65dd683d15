"""GPU parity for decode over an FP8 (E4M3) page pool with per-tensor scales,
against the fp64 oracle (through the C ABI: fa_decode_scaled / fa_decode)."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from gpu_util import (DevWorkload, assert_close, decode_geometry, oracle_decode,  # noqa: E402
                      run_decode, to_f64)
from workloads import CONFIG_NAMES, make_config, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def _wl(lens, hq, hkv, dtype, seed, extra_pages=3):
    print(f"[fp8 decode case] lens={list(lens)[:8]}.. B={len(lens)} hq={hq} hkv={hkv} q {dtype} "
          f"seed={seed}", flush=True)
    return make_workload(lens, hq, hkv, dtype, seed, mode="test", extra_pages=extra_pages,
                         kv_dtype="e4m3")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_fp8_ragged_small(dtype, group):
    """Ragged tails (NaN codes past last_page_len), empty requests, unreferenced
    NaN pages; q in bf16 or fp16."""
    lens = [1, 15, 16, 17, 31, 33, 100, 257, 0, 513]
    wl = _wl(lens, 2 * group, 2, dtype, 300 + group)
    dw = DevWorkload(wl)
    _, out, lse = run_decode(dw)
    e = assert_close(to_f64(out), to_f64(lse), *oracle_decode(wl), what=f"fp8 G={group}")
    print(f"  max-abs out {e[0]:.3g} lse {e[1]:.3g}", flush=True)


@pytest.mark.parametrize("tiles_per_cu,min_chunk", [(1, 1), (64, 1), (8, 3)])
def test_fp8_split_kv_paths(tiles_per_cu, min_chunk):
    """Many pieces per unit (in-kernel merge of partial states) and none."""
    lens = [1, 40, 300, 1000, 2049, 16]
    wl = _wl(lens, 16, 4, "bf16", 17)
    dw = DevWorkload(wl)
    plan, out, lse = run_decode(dw, num_cu=4, tiles_per_cu=tiles_per_cu, min_chunk_pages=min_chunk)
    st = plan.info()
    print(f"  tiles {st.num_tiles} merge {st.num_merge} pieces {st.chunk_pages}", flush=True)
    assert_close(to_f64(out), to_f64(lse), *oracle_decode(wl), what="fp8 split")


def test_fp8_scale_invariances():
    """Power-of-two scales are exact in fp32: k_scale = 2^a gives the bits of
    sm_scale * 2^a with k_scale 1; v_scale = 2^b gives 2^b * out (bf16 output
    rounding commutes with a power of two away from overflow and underflow).
    fa_decode on an E4M3 plan is fa_decode_scaled with both scales 1."""
    import torch
    import paged_kv_cache_fa_amd as fa
    wl = _wl([5, 100, 2000, 0, 64], 16, 4, "bf16", 23)
    dw = DevWorkload(wl)
    plan = fa.Plan(decode_geometry(wl, num_cu=8, tiles_per_cu=4), device="cuda")
    plan.plan(wl.kv_indptr, wl.kv_lens)
    args = (plan, dw.q, dw.k, dw.v, *dw.strides, dw.kv_indices, dw.kv_indptr, dw.last_page_len)
    sm = 1 / np.sqrt(128)
    o1, l1 = fa.decode_scaled(*args, sm_scale=sm, k_scale=0.25, v_scale=1.0)
    o2, l2 = fa.decode_scaled(*args, sm_scale=sm * 0.25, k_scale=1.0, v_scale=1.0)
    o3, l3 = fa.decode_scaled(*args, sm_scale=sm * 0.25, k_scale=1.0, v_scale=8.0)
    o4, l4 = fa.decode(*args, sm_scale=sm * 0.25)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, o2 * 8) and torch.equal(l3, l2)
    assert torch.equal(o4, o2) and torch.equal(l4, l2)


@pytest.mark.parametrize("k", [2, 3])
def test_fp8_configs_full_size(k):
    """The batch-64 and skewed batch-128 decode workloads with E4M3 pools."""
    print(f"[fp8 config {k}] generating", flush=True)
    wl = make_config(k, mode="test", kv_dtype="e4m3")
    dw = DevWorkload(wl)
    plan, out, lse = run_decode(dw)
    st = plan.info()
    print(f"[fp8 {CONFIG_NAMES[k]}] tiles {st.num_tiles} merge {st.num_merge} P {st.chunk_pages}",
          flush=True)
    e = assert_close(to_f64(out), to_f64(lse), *oracle_decode(wl), what=f"fp8 config {k}")
    print(f"[fp8 config {k}] max-abs out {e[0]:.3g} lse {e[1]:.3g}", flush=True)


def test_fp8_graph_replay():
    """A captured fa_decode_scaled replays to the eager result, with eager work
    and synchronisation between the replays."""
    import torch
    import paged_kv_cache_fa_amd as fa
    wl = _wl([700, 33, 2000, 5, 4096, 1], 32, 8, "bf16", 29, extra_pages=0)
    dw = DevWorkload(wl)
    plan = fa.Plan(decode_geometry(wl, num_cu=16, tiles_per_cu=4), device="cuda")
    plan.plan(wl.kv_indptr, wl.kv_lens)
    args = (plan, dw.q, dw.k, dw.v, *dw.strides, dw.kv_indices, dw.kv_indptr, dw.last_page_len)
    kw = dict(k_scale=wl.k_scale, v_scale=wl.v_scale)
    ref_o, ref_l = fa.decode_scaled(*args, **kw)
    ref_o, ref_l = ref_o.clone(), ref_l.clone()
    out = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_l)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fa.decode_scaled(*args, out=out, lse=lse, stream=s, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fa.decode_scaled(*args, out=out, lse=lse, stream=s, **kw)
    for rep in range(4):
        out.fill_(7)
        lse.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"
    assert_close(to_f64(ref_o), to_f64(ref_l), *oracle_decode(wl), what="fp8 graph")


def test_fp8_argument_errors():
    """Strides that are not 16-byte steps, bad scales, and a cascade over an
    FP8 suffix plan are refused before any launch."""
    import torch
    import paged_kv_cache_fa_amd as fa
    wl = _wl([40, 7], 8, 2, "bf16", 31)
    dw = DevWorkload(wl)
    plan = fa.Plan(decode_geometry(wl), device="cuda").plan(wl.kv_indptr, wl.kv_lens)
    tail = (dw.kv_indices, dw.kv_indptr, dw.last_page_len)
    ps, ts, hs = dw.strides
    for bad in ((ps, ts + 8, hs), (ps + 8, ts, hs), (ps, ts, hs + 8)):
        with pytest.raises(fa.FAError) as e:
            fa.decode_scaled(plan, dw.q, dw.k, dw.v, *bad, *tail)
        assert e.value.code == "INVALID"
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("nan"), 1.0), (1.0, float("inf"))):
        with pytest.raises(fa.FAError) as e:
            fa.decode_scaled(plan, dw.q, dw.k, dw.v, *dw.strides, *tail, k_scale=ks, v_scale=vs)
        assert e.value.code == "INVALID"
    B = wl.batch
    pg = fa.geometry("append", "bf16", 1, wl.num_qo_heads, wl.num_kv_heads, max_qo_tokens=B)
    pre = fa.Plan(pg, device="cuda").plan([0, 1], [16], [0, B], False)
    qo = torch.tensor([0, B], dtype=torch.int32, device="cuda")
    one = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    # pages read through 16-bit strides would stay inside this buffer
    room = torch.zeros(4 * dw.pool.numel(), dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.cascade(pre, plan, dw.q, room, room[ps:], *dw.strides, qo, dw.kv_indices[:1] * 0, one,
                   dw.last_page_len[:1], *tail)
    assert e.value.code == "INVALID"
    torch.cuda.synchronize()
