"""GPU parity for a mixed batch in one launch (fa_pod): prefill / append
requests and decode requests over one page pool give the bits of fa_append and
fa_decode run separately, and match the fp64 oracle."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle  # noqa: E402
from gpu_util import assert_close, to_f64, torch_dtype  # noqa: E402
from workloads import make_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def split_mixed(wl, n_prefill):
    """CSR tables of the first n_prefill requests and of the rest."""
    ip, ix, last, qo = wl.kv_indptr, wl.kv_indices, wl.last_page_len, wl.qo_indptr
    k = int(ip[n_prefill])
    pre = dict(kv_indptr=ip[: n_prefill + 1].copy(), kv_indices=ix[:k].copy(),
               last=last[:n_prefill].copy(), kv_lens=wl.kv_lens[:n_prefill].copy(),
               qo_indptr=qo[: n_prefill + 1].copy())
    dec = dict(kv_indptr=(ip[n_prefill:] - k).astype(np.int32), kv_indices=ix[k:].copy(),
               last=last[n_prefill:].copy(), kv_lens=wl.kv_lens[n_prefill:].copy())
    return pre, dec, int(qo[n_prefill])


@pytest.mark.parametrize("group,causal,wide", [(4, True, False), (1, False, False),
                                               (2, True, False), (4, True, True),
                                               (1, False, True), (2, False, True),
                                               (8, True, True), (8, False, True)])
def test_pod_mixed_batch(group, causal, wide):
    """Both launch shapes: prefill tiles of 128 / G rows (decode and append
    workgroups share each CU) and of 256 / G rows (the append kernel's
    workgroups, one role per CU at a time; the only shape for G = 8)."""
    pre_lens, pre_qo = [300, 64, 1000], [300, 17, 128] if causal else [40, 17, 128]
    dec_lens = [1, 15, 16, 17, 33, 257, 5, 900, 2000, 48]
    _pod_case(group, causal, wide, pre_lens, pre_qo, dec_lens, 80 + group)


@pytest.mark.parametrize("group,wide", [(4, False), (4, True), (8, True)])
def test_pod_empty_requests(group, wide):
    """Prefill requests with no query rows (one with no cached tokens either)
    beside ordinary ones and short decode requests, in each launch shape."""
    _pod_case(group, True, wide, [300, 64, 500, 0], [0, 17, 0, 0], [1, 5, 2, 900, 16, 1],
              90 + group)


def _pod_case(group, causal, wide, pre_lens, pre_qo, dec_lens, seed):
    import torch
    import paged_kv_cache_fa_amd as fa
    hkv = 4
    print(f"[pod] G={group} causal={causal} wide={wide} prefill {pre_lens} rows {pre_qo} "
          f"decode {dec_lens}", flush=True)
    wl = make_workload(pre_lens + dec_lens, hkv * group, hkv, "bf16", seed,
                       qo_lens=pre_qo + [1] * len(dec_lens), causal=causal, mode="test",
                       extra_pages=3)
    pre, dec, nrows_p = split_mixed(wl, len(pre_lens))
    dt = torch_dtype("bf16")
    pool = torch.from_numpy(wl.pool.view(np.int16)).cuda().view(dt)
    q = torch.from_numpy(wl.q.view(np.int16)).cuda().view(dt)
    q_p, q_d = q[:nrows_p], q[nrows_p:]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    _, _, ps, hk, d = wl.pool.shape
    strides = (2 * ps * hk * d, hk * d, d)
    k, v = pool[:, 0], pool[:, 1]
    gp = fa.geometry("append", "bf16", len(pre_lens), hkv * group, hkv,
                     max_qo_tokens=max(nrows_p, 1), num_cu=32,
                     qo_tile=(256 if wide else 128) // group)
    gd = fa.geometry("decode", "bf16", len(dec_lens), hkv * group, hkv, num_cu=32)
    pp = fa.plan(gp, pre["kv_indptr"], pre["kv_lens"], pre["qo_indptr"], causal, device="cuda")
    dp = fa.plan(gd, dec["kv_indptr"], dec["kv_lens"], device="cuda")
    ptabs = (t(pre["kv_indices"]), t(pre["kv_indptr"]), t(pre["last"]))
    dtabs = (t(dec["kv_indices"]), t(dec["kv_indptr"]), t(dec["last"]))
    (op, lp), (od, ld) = fa.pod(pp, q_p, t(pre["qo_indptr"]), *ptabs, dp, q_d, *dtabs, k, v,
                                *strides)
    op, lp, od, ld = op.clone(), lp.clone(), od.clone(), ld.clone()
    rp_o, rp_l = fa.append(pp, q_p, t(pre["qo_indptr"]), k, v, *strides, *ptabs)
    rd_o, rd_l = fa.decode(dp, q_d, k, v, *strides, *dtabs)
    torch.cuda.synchronize()
    assert torch.equal(op, rp_o) and torch.equal(lp, rp_l), "prefill part differs from fa_append"
    assert torch.equal(od, rd_o) and torch.equal(ld, rd_l), "decode part differs from fa_decode"
    ref_p = oracle.append(wl.q[:nrows_p], pre["qo_indptr"], wl.pool, "bf16", pre["kv_indptr"],
                          pre["kv_indices"], pre["last"], 16, causal=causal)
    assert_close(to_f64(op), to_f64(lp), *ref_p, what="pod prefill")
    ref_d = oracle.decode(wl.q[nrows_p:], wl.pool, "bf16", dec["kv_indptr"], dec["kv_indices"],
                          dec["last"], 16)
    assert_close(to_f64(od), to_f64(ld), *ref_d, what="pod decode")


def test_pod_refuses_group_8_shared_shape():
    """With 8 query heads per kv head fa_pod runs only the wide shape: prefill
    tiles of at most 128 / G = 16 rows are refused."""
    import torch
    import paged_kv_cache_fa_amd as fa
    wl = make_workload([300, 40], 32, 4, "bf16", 3, qo_lens=[100, 1], causal=True, mode="test")
    pre, dec, nrows_p = split_mixed(wl, 1)
    gp = fa.geometry("append", "bf16", 1, 32, 4, max_qo_tokens=nrows_p, qo_tile=16)
    gd = fa.geometry("decode", "bf16", 1, 32, 4)
    pp = fa.plan(gp, pre["kv_indptr"], pre["kv_lens"], pre["qo_indptr"], True, device="cuda")
    dp = fa.plan(gd, dec["kv_indptr"], dec["kv_lens"], device="cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    pool = torch.zeros(wl.pool.shape, dtype=torch.bfloat16, device="cuda")
    q = torch.zeros(wl.q.shape, dtype=torch.bfloat16, device="cuda")
    _, _, ps, hk, d = wl.pool.shape
    with pytest.raises(fa.FAError) as e:
        fa.pod(pp, q[:nrows_p], t(pre["qo_indptr"]), t(pre["kv_indices"]), t(pre["kv_indptr"]),
               t(pre["last"]), dp, q[nrows_p:], t(dec["kv_indices"]), t(dec["kv_indptr"]),
               t(dec["last"]), pool[:, 0], pool[:, 1], 2 * ps * hk * d, hk * d, d)
    assert e.value.code == "INVALID"
