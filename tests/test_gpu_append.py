"""GPU parity for causal / non-causal append (MFMA) against the fp64 oracle."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from gpu_util import (DevWorkload, assert_close, oracle_append, run_append,  # noqa: E402
                      to_f64)
from workloads import make_config, make_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def _case(lens, qo, hq, hkv, dtype, seed, causal=True, **knobs):
    print(f"[append case] lens={lens} qo={qo} hq={hq} hkv={hkv} {dtype} causal={causal} "
          f"{knobs}", flush=True)
    wl = make_workload(lens, hq, hkv, dtype, seed, qo_lens=qo, causal=causal, mode="test",
                       extra_pages=2)
    dw = DevWorkload(wl)
    plan, out, lse = run_append(dw, **knobs)
    ref = oracle_append(wl)
    e = assert_close(to_f64(out), to_f64(lse), *ref, what=f"append {lens} {qo}")
    st = plan.info()
    print(f"   tiles {st.num_tiles} splits {st.num_merge} chunk {st.chunk_pages} err {e}",
          flush=True)
    return plan


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_causal_ragged(dtype, group):
    # partial q tiles, kv not a multiple of 16 or 64, pure prefill, qo_len 1
    lens = [37, 100, 64, 257, 5, 130]
    qo = [37, 33, 1, 70, 5, 64]
    _case(lens, qo, 2 * group, 2, dtype, 40 + group)


@pytest.mark.parametrize("num_cu,tiles_per_cu", [(1, 1), (2, 4), (64, 8)])
def test_split_chunks(num_cu, tiles_per_cu):
    lens = [700, 1000, 130]
    qo = [40, 100, 64]
    _case(lens, qo, 32, 8, "bf16", 7, num_cu=num_cu, tiles_per_cu=tiles_per_cu)


@pytest.mark.parametrize("group,dtype,lens,qo,num_cu,tiles_per_cu", [
    (1, "fp16", [3000, 130], [70, 9], 64, 8),    # over a hundred chunks per tile
    (2, "bf16", [900], [900], 16, 8),            # causal prefill: early rows see empty chunks
    (8, "bf16", [1500, 40], [33, 40], 32, 8),    # one partial tile of 32 columns per request
    (4, "fp16", [2500], [200], 8, 4),            # a ragged last tile (200 = 3 x 64 + 8)
])
def test_split_chunks_groups(group, dtype, lens, qo, num_cu, tiles_per_cu):
    # the last workgroup of a split merges the chunks: every group size, chunk
    # counts past the merge's batch of 8, rows with no visible key in a chunk
    plan = _case(lens, qo, 2 * group, 2, dtype, 60 + group, num_cu=num_cu,
                 tiles_per_cu=tiles_per_cu)
    assert plan.info().num_merge > 0


@pytest.mark.parametrize("causal", [False, True])
def test_prefix_style_non_causal(causal):
    # many query rows against one long request (the shared-prefix pass shape)
    _case([2048], [256], 32, 8, "bf16", 9, causal=causal, num_cu=4, tiles_per_cu=8)


def test_zero_query_rows_and_empty():
    lens = [64, 16, 50]
    qo = [0, 16, 0]
    _case(lens, qo, 8, 2, "bf16", 11)


def test_determinism():
    import torch
    wl = make_workload([700, 300], 32, 8, "bf16", 3, qo_lens=[100, 300], causal=True,
                       mode="test")
    dw = DevWorkload(wl)
    plan, o1, l1 = run_append(dw, num_cu=4, tiles_per_cu=4)
    o1, l1 = o1.clone(), l1.clone()
    _, o2, l2 = run_append(dw, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_causal_append_batch16_full_size_all_rows():
    """The batch-16 causal append (512 new rows onto 4096 cached, 32/8 heads,
    bf16) in the launch configuration the benchmark times, every one of its
    8192 query rows and 32 heads against the oracle."""
    print("[causal append batch 16 x 512] generating", flush=True)
    wl = make_config(5, mode="test")
    dw = DevWorkload(wl)
    plan, out, lse = run_append(dw)
    st = plan.info()
    print(f"[causal append batch 16 x 512] tiles {st.num_tiles} splits {st.num_merge}", flush=True)
    ref = oracle_append(wl)
    e = assert_close(to_f64(out), to_f64(lse), *ref, what="causal append batch 16 x 512")
    print(f"[causal append batch 16 x 512] all {wl.rows} rows: max-abs out {e[0]:.3g} "
          f"lse {e[1]:.3g}", flush=True)
