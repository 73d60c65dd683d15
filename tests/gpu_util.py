"""Helpers for GPU tests: upload a seeded workload, run the library, compare."""
from __future__ import annotations

import numpy as np

import oracle
import paged_kv_cache_fa_amd as fa

OUT_TOL = 2e-2     # max-abs on out (16-bit outputs, fp32 accumulation)
LSE_TOL = 1e-3     # max-abs on lse (natural log)


def torch_dtype(name):
    import torch
    return {"bf16": torch.bfloat16, "fp16": torch.float16}[name]


class DevWorkload:
    """Device copies of a workload's stored bytes (pool, q, page tables)."""

    def __init__(self, wl, device="cuda"):
        import torch
        self.wl = wl
        dt = torch_dtype(wl.dtype)
        self.device = device
        if wl.kv_dtype == "e4m3":  # E4M3 codes, one byte per element
            self.pool = torch.from_numpy(wl.pool).to(device)
        else:
            self.pool = torch.from_numpy(wl.pool.view(np.int16)).to(device).view(dt)
        self.q = torch.from_numpy(wl.q.view(np.int16)).to(device).view(dt)
        self.kv_indptr = torch.from_numpy(wl.kv_indptr).to(device)
        self.kv_indices = torch.from_numpy(wl.kv_indices).to(device)
        self.last_page_len = torch.from_numpy(wl.last_page_len).to(device)
        self.qo_indptr = (torch.from_numpy(wl.qo_indptr).to(device)
                          if wl.qo_indptr is not None else None)
        if wl.prefix_indptr is not None:
            self.prefix_indptr = torch.from_numpy(wl.prefix_indptr).to(device)
            self.prefix_indices = torch.from_numpy(wl.prefix_indices).to(device)
            self.prefix_last_page_len = torch.from_numpy(wl.prefix_last_page_len).to(device)
        _, _, ps, hkv, d = wl.pool.shape
        self.strides = (2 * ps * hkv * d, hkv * d, d)

    @property
    def k(self):
        return self.pool[:, 0]

    @property
    def v(self):
        return self.pool[:, 1]


def decode_geometry(wl, **knobs):
    if wl.kv_dtype is not None:
        knobs.setdefault("kv_dtype", wl.kv_dtype)
    return fa.geometry("decode", wl.dtype, max(wl.batch, 1), wl.num_qo_heads, wl.num_kv_heads,
                       **knobs)


def run_decode(dw: DevWorkload, plan=None, out=None, lse=None, **knobs):
    """fa_decode, or fa_decode_scaled with the workload's scales for an FP8 pool."""
    wl = dw.wl
    if plan is None:
        plan = fa.Plan(decode_geometry(wl, **knobs), device=dw.device)
        plan.plan(wl.kv_indptr, wl.kv_lens)
    args = (plan, dw.q, dw.k, dw.v, *dw.strides, dw.kv_indices, dw.kv_indptr, dw.last_page_len)
    if wl.kv_dtype is not None:
        out, lse = fa.decode_scaled(*args, k_scale=wl.k_scale, v_scale=wl.v_scale, out=out,
                                    lse=lse)
    else:
        out, lse = fa.decode(*args, out=out, lse=lse)
    return plan, out, lse


def to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def oracle_decode(wl, requests=None):
    return oracle.decode(wl.q, wl.pool, wl.dtype, wl.kv_indptr, wl.kv_indices, wl.last_page_len,
                         wl.page_size, requests=requests, kv_dtype=wl.kv_dtype,
                         k_scale=wl.k_scale, v_scale=wl.v_scale)


def assert_close(out, lse, ref_out, ref_lse, out_tol=OUT_TOL, lse_tol=LSE_TOL, what=""):
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    assert np.array_equal(np.isneginf(lse), np.isneginf(ref_lse)), f"{what}: -inf pattern"
    e_out = float(np.max(np.abs(out - ref_out))) if out.size else 0.0
    fin = np.isfinite(ref_lse)
    e_lse = float(np.max(np.abs(lse[fin] - ref_lse[fin]))) if fin.any() else 0.0
    assert e_out <= out_tol, f"{what}: out max-abs {e_out} > {out_tol}"
    assert e_lse <= lse_tol, f"{what}: lse max-abs {e_lse} > {lse_tol}"
    return e_out, e_lse


def append_geometry(wl, **knobs):
    return fa.geometry("append", wl.dtype, max(wl.batch, 1), wl.num_qo_heads, wl.num_kv_heads,
                       max_qo_tokens=max(wl.rows, 1), **knobs)


def run_append(dw: DevWorkload, plan=None, out=None, lse=None, **knobs):
    wl = dw.wl
    if plan is None:
        plan = fa.Plan(append_geometry(wl, **knobs), device=dw.device)
        plan.plan(wl.kv_indptr, wl.kv_lens, wl.qo_indptr, wl.causal)
    out, lse = fa.append(plan, dw.q, dw.qo_indptr, dw.k, dw.v, *dw.strides, dw.kv_indices,
                         dw.kv_indptr, dw.last_page_len, out=out, lse=lse)
    return plan, out, lse


def oracle_append(wl, rows=None):
    return oracle.append(wl.q, wl.qo_indptr, wl.pool, wl.dtype, wl.kv_indptr, wl.kv_indices,
                         wl.last_page_len, wl.page_size, causal=wl.causal, rows=rows)


def run_cascade(dw: DevWorkload, prefix_plan=None, suffix_plan=None, fused=False,
                side_stream=None, suffix_stream=None, **knobs):
    """Shared-prefix pass (non-causal append of every request's query over the
    prefix) + private-suffix decode + merge_state, as three calls or as one
    fa_cascade call (optionally with the prefix pass on ``side_stream``).
    Returns (out, lse, plans)."""
    import torch
    wl = dw.wl
    B = wl.batch
    if prefix_plan is None:
        # the append geometry's default q tile (256 / G rows: the one-launch
        # kernel's wide form); {"qo_tile": 128 // G} picks its shared form
        pk = dict(knobs.get("prefix", {}))
        g = fa.geometry("append", wl.dtype, 1, wl.num_qo_heads, wl.num_kv_heads,
                        max_qo_tokens=B, **pk)
        prefix_plan = fa.Plan(g, device=dw.device)
        prefix_plan.plan(wl.prefix_indptr, [wl.prefix_len], [0, B], False)
    if suffix_plan is None:
        suffix_plan = fa.Plan(decode_geometry(wl, **knobs.get("suffix", {})), device=dw.device)
        suffix_plan.plan(wl.kv_indptr, wl.kv_lens)
    qo = torch.tensor([0, B], dtype=torch.int32, device=dw.device)
    if fused:
        out, lse = fa.cascade(prefix_plan, suffix_plan, dw.q, dw.k, dw.v, *dw.strides, qo,
                              dw.prefix_indices, dw.prefix_indptr, dw.prefix_last_page_len,
                              dw.kv_indices, dw.kv_indptr, dw.last_page_len,
                              side_stream=side_stream, suffix_stream=suffix_stream)
        return out, lse, (prefix_plan, suffix_plan)
    o_p, l_p = fa.append(prefix_plan, dw.q, qo, dw.k, dw.v, *dw.strides, dw.prefix_indices,
                         dw.prefix_indptr, dw.prefix_last_page_len)
    o_s, l_s = fa.decode(suffix_plan, dw.q, dw.k, dw.v, *dw.strides, dw.kv_indices, dw.kv_indptr,
                         dw.last_page_len)
    out, lse = fa.merge_state(o_p, l_p, o_s, l_s)
    return out, lse, (prefix_plan, suffix_plan)


def oracle_cascade(wl, requests=None):
    return oracle.cascade(wl.q, wl.pool, wl.dtype, wl.prefix_indptr, wl.prefix_indices,
                          wl.prefix_last_page_len, wl.kv_indptr, wl.kv_indices, wl.last_page_len,
                          wl.page_size, requests=requests)
