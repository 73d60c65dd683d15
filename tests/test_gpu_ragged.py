"""GPU parity for ragged (contiguous) KV caches and the single-request decode,
against the fp64 oracle (through the C ABI: fa_plan_ragged, fa_decode_ragged,
fa_append_ragged)."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle  # noqa: E402
from gpu_util import assert_close, to_f64  # noqa: E402
from workloads import make_ragged  # noqa: E402

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 31, 33, 100, 257, 0, 513]


def _dev(rw):
    """Device copies of a ragged workload (K / V with their NaN pad rows)."""
    import torch
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[rw.dtype]

    def kv(a):
        if rw.kv_dtype == "e4m3":
            return torch.from_numpy(a).cuda()
        return torch.from_numpy(a.view(np.int16)).cuda().view(dt)
    q = torch.from_numpy(rw.q.view(np.int16)).cuda().view(dt)
    return q, kv(rw.k), kv(rw.v), torch.from_numpy(rw.kv_offsets).cuda()


def _decode(rw, use_device_offsets=True, **knobs):
    import paged_kv_cache_fa_amd as fa
    q, k, v, offs = _dev(rw)
    g = fa.geometry("decode", rw.dtype, max(rw.batch, 1), rw.num_qo_heads, rw.num_kv_heads,
                    kv_dtype=rw.kv_dtype, **knobs)
    p = fa.plan_ragged(g, rw.kv_offsets, device="cuda")
    out, lse = fa.decode_ragged(p, q, k, v, k.stride(0), k.stride(1),
                                offs if use_device_offsets else None, k_scale=rw.k_scale,
                                v_scale=rw.v_scale)
    return p, out, lse


def _oracle_decode(rw):
    return oracle.decode_ragged(rw.q, rw.k, rw.v, rw.dtype, rw.kv_offsets, kv_dtype=rw.kv_dtype,
                                k_scale=rw.k_scale, v_scale=rw.v_scale)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_ragged_decode_small(dtype, group):
    print(f"[ragged decode] {dtype} G={group}", flush=True)
    rw = make_ragged(LENS, 2 * group, 2, dtype, 400 + group, mode="test", pad_rows=40)
    _, out, lse = _decode(rw)
    e = assert_close(to_f64(out), to_f64(lse), *_oracle_decode(rw), what=f"ragged G={group}")
    print(f"  max-abs out {e[0]:.3g} lse {e[1]:.3g}", flush=True)


@pytest.mark.parametrize("knobs", [dict(num_cu=4, tiles_per_cu=64),
                                   dict(num_cu=2, tiles_per_cu=1, max_tiles=64),
                                   dict(num_cu=8, tiles_per_cu=4, min_chunk_pages=3)])
def test_ragged_decode_split_paths(knobs):
    print(f"[ragged split] {knobs}", flush=True)
    rw = make_ragged([1, 40, 300, 1000, 2049, 16], 16, 4, "bf16", 17, mode="test", pad_rows=20)
    p, out, lse = _decode(rw, use_device_offsets=False, **knobs)
    st = p.info()
    print(f"  tiles {st.num_tiles} merge {st.num_merge} Q {st.chunk_pages}", flush=True)
    assert_close(to_f64(out), to_f64(lse), *_oracle_decode(rw), what="ragged split")


def test_ragged_count_catches_overreads():
    """q = 0: lse = ln kv_len exactly (to fp32), so one row read past a
    request's end (the next request's first row) would show."""
    rw = make_ragged(LENS, 8, 2, "bf16", 5, mode="test", pad_rows=16)
    rw.q[:] = 0
    _, _, lse = _decode(rw, num_cu=3, tiles_per_cu=5)
    lg = to_f64(lse)
    for b, L in enumerate(LENS):
        if L == 0:
            assert np.isneginf(lg[b]).all()
        else:
            assert np.max(np.abs(lg[b] - np.log(L))) < 1e-5, (b, L, lg[b])


def test_ragged_decode_e4m3():
    rw = make_ragged(LENS, 16, 4, "bf16", 7, mode="test", pad_rows=16, kv_dtype="e4m3")
    _, out, lse = _decode(rw)
    assert_close(to_f64(out), to_f64(lse), *_oracle_decode(rw), what="ragged e4m3")


def test_ragged_equals_paged_bitwise():
    """Requests whose rows start on 16-row boundaries read through a paged
    view of the same memory (page = 16 rows, identity page lists) give the
    same bits: one plan, one kernel, the same values in the same order."""
    import torch
    import paged_kv_cache_fa_amd as fa
    lens = [32, 48, 16, 37]
    rw = make_ragged(lens, 32, 8, "bf16", 11, mode="test", pad_rows=11)
    q, k, v, offs = _dev(rw)
    _, out_r, lse_r = _decode(rw)
    n = [-(-L // 16) for L in lens]
    first = [int(o) // 16 for o in rw.kv_offsets[:-1]]
    indptr = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    indices = np.concatenate([np.arange(f, f + m) for f, m in zip(first, n)]).astype(np.int32)
    last = np.array([L - 16 * (m - 1) for L, m in zip(lens, n)], np.int32)
    g = fa.geometry("decode", "bf16", 4, 32, 8)
    p = fa.plan(g, indptr, np.asarray(lens, np.int32), device="cuda")
    ts, hs = k.stride(0), k.stride(1)
    out_p, lse_p = fa.decode(p, q, k, v, 16 * ts, ts, hs, torch.from_numpy(indices).cuda(),
                             torch.from_numpy(indptr).cuda(), torch.from_numpy(last).cuda())
    torch.cuda.synchronize()
    assert torch.equal(out_r, out_p) and torch.equal(lse_r, lse_p)


@pytest.mark.parametrize("causal", [True, False])
def test_ragged_append(causal):
    import paged_kv_cache_fa_amd as fa
    lens = [5, 40, 300, 17, 0, 129]
    qo = [5, 9, 300, 1, 0, 64] if causal else [3, 40, 70, 17, 0, 1]
    print(f"[ragged append] causal={causal}", flush=True)
    rw = make_ragged(lens, 16, 4, "bf16", 23, qo_lens=qo, causal=causal, mode="test",
                     pad_rows=16)
    q, k, v, offs = _dev(rw)
    import torch
    g = fa.geometry("append", "bf16", rw.batch, 16, 4, max_qo_tokens=rw.rows, num_cu=8)
    p = fa.plan_ragged(g, rw.kv_offsets, rw.qo_indptr, causal, device="cuda")
    out, lse = fa.append_ragged(p, q, torch.from_numpy(rw.qo_indptr).cuda(), k, v, k.stride(0),
                                k.stride(1), offs)
    ref = oracle.append_ragged(rw.q, rw.qo_indptr, rw.k, rw.v, "bf16", rw.kv_offsets,
                               causal=causal)
    e = assert_close(to_f64(out), to_f64(lse), *ref, what=f"ragged append causal={causal}")
    print(f"  max-abs out {e[0]:.3g} lse {e[1]:.3g}", flush=True)


@pytest.mark.parametrize("kv_len", [2048, 2047, 1])
def test_single_decode_with_kv_cache(kv_len):
    """One request, q [32, 128] fp16 and a contiguous K / V [kv_len, 32, 128]
    fp16 (the single-request decode shape), through the one-call helper."""
    import torch
    import paged_kv_cache_fa_amd as fa
    rw = make_ragged([kv_len], 32, 32, "fp16", 1, mode="test", pad_rows=16)
    q, k, v, _ = _dev(rw)
    # the views end at kv_len; the NaN rows after them catch any read past it
    out, lse = fa.single_decode_with_kv_cache(q[0], k[:kv_len], v[:kv_len], return_lse=True)
    torch.cuda.synchronize()
    ro, rl = _oracle_decode(rw)
    assert_close(to_f64(out)[None], to_f64(lse)[None], ro, rl, what=f"single kv_len={kv_len}")


def test_ragged_graph_replay_and_errors():
    """A captured ragged decode (offsets from the plan's workspace copy)
    replays to the eager bits after a re-plan with new lengths of the same
    geometry; paged calls refuse a ragged plan and ragged calls a paged one."""
    import torch
    import paged_kv_cache_fa_amd as fa
    lens_a, lens_b = [300, 17, 1000, 0], [5, 900, 33, 400]
    ra = make_ragged(lens_a, 32, 8, "bf16", 31, mode="test", pad_rows=8)
    rb = make_ragged(lens_b, 32, 8, "bf16", 32, mode="test", pad_rows=8)
    rows = max(ra.k.shape[0], rb.k.shape[0])
    q, k, v, _ = _dev(ra)
    kbuf = torch.zeros(rows, 8, 128, dtype=torch.bfloat16, device="cuda")
    vbuf = torch.zeros_like(kbuf)
    g = fa.geometry("decode", "bf16", 4, 32, 8, num_cu=16, tiles_per_cu=4)
    p = fa.plan_ragged(g, ra.kv_offsets, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(4, 32, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()

    def load(rw):
        qq, kk, vv, _ = _dev(rw)
        kbuf.zero_()
        vbuf.zero_()
        kbuf[: kk.shape[0]] = kk
        vbuf[: vv.shape[0]] = vv
        q.copy_(qq)
        torch.cuda.synchronize()
    load(ra)
    with torch.cuda.stream(s):
        fa.decode_ragged(p, q, kbuf, vbuf, kbuf.stride(0), kbuf.stride(1), None, out=out,
                         lse=lse, stream=s)
    torch.cuda.synchronize()
    g_ = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_, stream=s):
        fa.decode_ragged(p, q, kbuf, vbuf, kbuf.stride(0), kbuf.stride(1), None, out=out,
                         lse=lse, stream=s)
    for rep in range(2):
        for rw in (ra, rb):
            load(rw)
            p.plan_ragged(rw.kv_offsets, stream=s)
            torch.cuda.synchronize()
            g_.replay()
            torch.cuda.synchronize()
            assert_close(to_f64(out), to_f64(lse), *_oracle_decode(rw), what=f"replay {rep}")
    # mode mismatches are refused before any launch (the tables given would
    # keep every read in bounds and make every piece read nothing even so)
    pp = fa.plan(g, np.array([0, 1], np.int32), np.array([16], np.int32), device="cuda")
    one = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.decode_ragged(pp, q[:1], kbuf, vbuf, kbuf.stride(0), kbuf.stride(1), one)
    assert e.value.code == "INVALID"
    zeros = torch.zeros(4096, dtype=torch.int32, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.decode(p, q, kbuf, vbuf, 16 * kbuf.stride(0), kbuf.stride(0), kbuf.stride(1),
                  zeros, zeros[:5], zeros[:4])
    assert e.value.code == "INVALID"
    torch.cuda.synchronize()
