"""Benchmark: paged decode HBM throughput on one MI355X.

One step = one pass of the decode hot path over one batch: the host plan
(split-KV tiles, uploaded to the device workspace) followed by the decode
kernel and the log-sum-exp merge of split requests. The headline workload is
batch 64 with GQA (32 q / 8 kv heads, head_dim 128, bf16, page 16, kv_len
uniform in [512, 4096], pages scattered by a seeded permutation); the batch-128
skewed workload (4 x 32768 + 124 log-normal lengths) is reported alongside.

Inputs are synthetic (seeded N(0,1)), already resident in HBM before the timed
region; steps rotate over enough copies of the page pool (>= 1 GiB in total)
that the 256 MB Infinity Cache cannot serve them.

Prints one JSON line. ``value`` is the achieved algorithmic HBM bandwidth in
GB/s of the whole step (bytes of valid K/V + q + out + lse, divided by the
wall time per step).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode achieved HBM GB/s (% of peak) and tokens/sec at batch 64/128"


def algorithmic_bytes(wl) -> int:
    """Valid K/V bytes of every request plus q, out and lse."""
    elt = 2
    kv = int(wl.kv_lens.astype(np.int64).sum()) * wl.num_kv_heads * wl.head_dim * 2 * elt
    q = wl.rows * wl.num_qo_heads * wl.head_dim * elt
    return kv + 2 * q + wl.rows * wl.num_qo_heads * 4


class DecodeBench:
    def __init__(self, wl, device="cuda", min_rotation_bytes=1 << 30, **knobs):
        import torch
        import paged_kv_cache_fa_amd as fa
        self.fa = fa
        self.wl = wl
        dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[wl.dtype]
        pool = torch.from_numpy(wl.pool.view(np.int16)).to(device).view(dt)
        copies = max(1, math.ceil(min_rotation_bytes / max(1, pool.numel() * 2)))
        self.pools = [pool] + [pool.clone() for _ in range(copies - 1)]
        self.q = torch.from_numpy(wl.q.view(np.int16)).to(device).view(dt)
        self.kv_indptr = torch.from_numpy(wl.kv_indptr).to(device)
        self.kv_indices = torch.from_numpy(wl.kv_indices).to(device)
        self.last = torch.from_numpy(wl.last_page_len).to(device)
        _, _, ps, hkv, d = wl.pool.shape
        self.strides = (2 * ps * hkv * d, hkv * d, d)
        geom = fa.geometry("decode", wl.dtype, wl.batch, wl.num_qo_heads, wl.num_kv_heads, **knobs)
        self.plan = fa.Plan(geom, device=device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(wl.rows, wl.num_qo_heads, dtype=torch.float32, device=device)
        self.indptr_h = np.ascontiguousarray(wl.kv_indptr)
        self.lens_h = np.ascontiguousarray(wl.kv_lens.astype(np.int32))

    def step(self, i: int, ev=None):
        pool = self.pools[i % len(self.pools)]
        self.plan.plan(self.indptr_h, self.lens_h)
        if ev is not None:
            ev[0].record()
        self.fa.decode(self.plan, self.q, pool[:, 0], pool[:, 1], *self.strides, self.kv_indices,
                       self.kv_indptr, self.last, out=self.out, lse=self.lse)
        if ev is not None:
            ev[1].record()

    def run(self, steps: int, warmup: int):
        import torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for i in range(steps):
            self.step(warmup + i, kev[i])
        t1.record()
        torch.cuda.synchronize()
        step_ms = t0.elapsed_time(t1) / steps
        kernel_ms = float(np.mean([a.elapsed_time(b) for a, b in kev]))
        return step_ms, kernel_ms


def cpu_baseline(wl, budget_s: float = 15.0) -> dict:
    """The fp64 oracle on the host cores over a bounded sample of requests."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        cores = 1
    reqs, t_used, done_bytes = [], 0.0, 0
    per_tok = wl.num_kv_heads * wl.head_dim * 2 * 2
    t_start = time.perf_counter()
    for b in range(wl.batch):
        t = time.perf_counter()
        oracle.decode(wl.q, wl.pool, wl.dtype, wl.kv_indptr, wl.kv_indices, wl.last_page_len,
                      wl.page_size, requests=[b])
        t_used += time.perf_counter() - t
        reqs.append(b)
        done_bytes += int(wl.kv_lens[b]) * per_tok + wl.num_qo_heads * wl.head_dim * 2 * 2
        if time.perf_counter() - t_start > budget_s:
            break
    return {"value": round(done_bytes / t_used / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"fp64 numpy oracle over requests 0..{len(reqs) - 1} of {wl.batch} "
                      f"({len(reqs) / t_used:.2f} requests/s, {t_used:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="2 = batch 64 (headline), 3 = batch 128")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batch128", action="store_true")
    ap.add_argument("--knob", action="append", default=[], help="plan knob name=value")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(see DESIGN.md for how it would shard).", file=sys.stderr)
        sys.exit(2)
    import torch
    from workloads import CONFIG_NAMES, make_config
    knobs = {k: int(v) for k, v in (s.split("=") for s in args.knob)}

    wl = make_config(args.config)
    b = DecodeBench(wl, **knobs)
    step_ms, kernel_ms = b.run(args.steps, args.warmup)
    nbytes = algorithmic_bytes(wl)
    gbs = nbytes / (step_ms * 1e-3) / 1e9
    kgbs = nbytes / (kernel_ms * 1e-3) / 1e9
    st = b.plan.info()
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"config{args.config}: {CONFIG_NAMES[args.config]}",
                   "batch": wl.batch, "num_qo_heads": wl.num_qo_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "page_size": wl.page_size, "kv_tokens": int(wl.kv_lens.sum()),
                   "algorithmic_bytes": nbytes, "pool_copies": len(b.pools),
                   "tiles": st.num_tiles, "merge_rows": st.num_merge,
                   "chunk_pages": st.chunk_pages},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(wl.batch / (step_ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(kgbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_kernel + merge_partials_kernel (one fa_decode call)",
                     "kernel_ms": round(kernel_ms, 5)},
    }
    del b
    torch.cuda.empty_cache()
    if args.config == 2 and not args.no_batch128:
        wl3 = make_config(3)
        b3 = DecodeBench(wl3, **knobs)
        s3, k3 = b3.run(args.steps, args.warmup)
        n3 = algorithmic_bytes(wl3)
        line["batch128"] = {"workload": f"config3: {CONFIG_NAMES[3]}",
                            "GB/s": round(n3 / (s3 * 1e-3) / 1e9, 2),
                            "pct_of_hbm_peak": round(100 * n3 / (s3 * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                            "tokens_per_s": round(128 / (s3 * 1e-3), 1),
                            "ms_per_step": round(s3, 5), "kernel_ms": round(k3, 5)}
        del b3, wl3
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
