"""Plant plausible mistakes in copies of oracle functions; some pin must fail.

Every mutation here is applied on the CPU to the oracle only (monkeypatched
for the duration of one test) and shows that the pins are strong enough to
catch a dropped term, a wrong index or a wrong sign.
"""
import math
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle.attention as OA  # noqa: E402
import oracle.merge as OM  # noqa: E402
import oracle_pins as P  # noqa: E402

_attend = OA.attend


def _attend_gqa_mod(q, K, V, scale, visible=None):
    """Mistake: q head h reads kv head h % Hkv instead of h // G."""
    R, Hq, D = q.shape
    Hkv = K.shape[1]
    perm = [(h % Hkv) * (Hq // Hkv) + h // Hkv for h in range(Hq)]
    out, lse = _attend(q[:, perm, :], K, V, scale, visible)
    inv = np.argsort(perm)
    return out[:, inv, :], lse[:, inv]


def _attend_scale_1_over_d(q, K, V, scale, visible=None):
    """Mistake: scale 1/D where the caller asked for 1/sqrt(D)."""
    D = q.shape[-1]
    if abs(scale - 1 / math.sqrt(D)) < 1e-15:
        scale = 1.0 / D
    return _attend(q, K, V, scale, visible)


def _attend_drop_last(q, K, V, scale, visible=None):
    """Mistake: the last visible key is dropped."""
    L = K.shape[0]
    vis = np.full(q.shape[0], L) if visible is None else np.asarray(visible)
    return _attend(q, K, V, scale, np.maximum(vis - 1, 0))


def _attend_log2(q, K, V, scale, visible=None):
    """Mistake: base-2 log-sum-exp."""
    out, lse = _attend(q, K, V, scale, visible)
    return out, lse / math.log(2)


def _kv_len_off_by_one(kv_indptr, last_page_len, page_size, b):
    n = int(kv_indptr[b + 1]) - int(kv_indptr[b])
    return 0 if n == 0 else n * page_size - page_size + int(last_page_len[b]) - 1


def _kv_len_full_pages(kv_indptr, last_page_len, page_size, b):
    return (int(kv_indptr[b + 1]) - int(kv_indptr[b])) * page_size


_merge_states = OM.merge_states


def _merge_wrong_sign(v, s):
    out_v, out_s = _merge_states(v, -np.asarray(s))
    return out_v, -out_s


def _merge_no_norm(v, s):
    v = np.asarray(v); s = np.asarray(s)
    m = s.max(axis=-1)
    w = np.exp(s - m[..., None])
    return (w[..., None] * v).sum(axis=-2), m + np.log(w.sum(axis=-1))


import oracle.fp8 as OF  # noqa: E402

_e4m3 = OF.e4m3_value


def _e4m3_bias8(codes):
    """Mistake: exponent bias 8 (the E5M2-style or off-by-one bias)."""
    return _e4m3(codes) / 2.0


def _e4m3_no_subnormals(codes):
    """Mistake: exponent field 0 read as a normal number."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    v = _e4m3(codes)
    sub = ((c >> 3) & 0xF) == 0
    m = (c & 7).astype(np.float64)
    return np.where(sub, np.where(c >> 7, -1.0, 1.0) * (1 + m / 8) * 2.0 ** -7, v)


def _e4m3_fnuz_nan(codes):
    """Mistake: the FNUZ variant's NaN at 0x80 and no NaN at S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8)
    v = _e4m3(np.where((c & 0x7F) == 0x7F, c & 0xFE, c))
    v = np.where((c & 0x7F) == 0x7F, np.where(c >> 7, -480.0, 480.0), v)
    return np.where(c == 0x80, np.nan, v)


_gather = OA.gather_request_kv


def _gather_swapped_scales(pool, dtype, kv_indptr, kv_indices, last_page_len, page_size, b,
                           k_scale=1.0, v_scale=1.0):
    """Mistake: K multiplied by v_scale and V by k_scale."""
    return _gather(pool, dtype, kv_indptr, kv_indices, last_page_len, page_size, b, v_scale,
                   k_scale)


_ragged_kv = OA.ragged_request_kv


def _ragged_shifted(k_bits, v_bits, dtype, kv_offsets, b, k_scale=1.0, v_scale=1.0):
    """Mistake: request b's rows taken one row late."""
    off = np.asarray(kv_offsets).copy()
    off[b] += 1
    off[b + 1] += 1
    return _ragged_kv(k_bits, v_bits, dtype, off, b, k_scale, v_scale)


_attend_raw = OA.attend


def _block_sparse_extra_key(q_bits, k_bits, v_bits, dtype, block_indptr, block_indices,
                            row_offsets, col_offsets, scale=None):
    """Mistake: each column block reaches one key row too far."""
    co = np.asarray(col_offsets).copy()
    co[1:] = np.minimum(co[1:] + 1, co[-1])
    return _block_sparse(q_bits, k_bits, v_bits, dtype, block_indptr, block_indices, row_offsets,
                         co, scale)


_block_sparse = OA.block_sparse


def _run_all():
    for chk in P.ALL_CHECKS:
        chk()


MUTATIONS = [
    ("gqa_mod", OA, "attend", _attend_gqa_mod),
    ("scale_1_over_d", OA, "attend", _attend_scale_1_over_d),
    ("drop_last_key", OA, "attend", _attend_drop_last),
    ("log2_lse", OA, "attend", _attend_log2),
    ("kv_len_off_by_one", OA, "request_kv_len", _kv_len_off_by_one),
    ("kv_len_ignores_last_page_len", OA, "request_kv_len", _kv_len_full_pages),
    ("merge_wrong_sign", OM, "merge_states", _merge_wrong_sign),
    ("merge_no_normalisation", OM, "merge_states", _merge_no_norm),
    ("e4m3_bias_8", OA, "e4m3_value", _e4m3_bias8),
    ("e4m3_no_subnormals", OA, "e4m3_value", _e4m3_no_subnormals),
    ("e4m3_fnuz_nan", OA, "e4m3_value", _e4m3_fnuz_nan),
    ("fp8_scales_swapped", OA, "gather_request_kv", _gather_swapped_scales),
    ("ragged_rows_shifted", OA, "ragged_request_kv", _ragged_shifted),
    ("block_sparse_extra_key", OA, "block_sparse", _block_sparse_extra_key),
]


@pytest.mark.parametrize("name,mod,attr,fn", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, mod, attr, fn):
    monkeypatch.setattr(mod, attr, fn)
    with pytest.raises(AssertionError):
        _run_all()


def test_causal_offset_mutation_is_caught(monkeypatch):
    """Mistake: top-left causal alignment (row i sees keys 0..i)."""
    real_append = OA.append

    def top_left(q_bits, qo_indptr, pool, dtype, kv_indptr, kv_indices, last_page_len,
                 page_size, causal=True, scale=None, rows=None):
        if not causal:
            return real_append(q_bits, qo_indptr, pool, dtype, kv_indptr, kv_indices,
                               last_page_len, page_size, False, scale, rows)
        # shift the cache away: pretend every request's kv_len equals its qo_len
        outs = []
        D = q_bits.shape[-1]
        sc = 1 / math.sqrt(D) if scale is None else scale
        B = len(qo_indptr) - 1
        for b in range(B):
            K, V = OA.gather_request_kv(pool, dtype, kv_indptr, kv_indices, last_page_len,
                                        page_size, b)
            r0, r1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
            vis = np.arange(1, r1 - r0 + 1)
            outs.append(_attend(OA.upcast(q_bits[r0:r1], dtype), K, V, sc, vis))
        return (np.concatenate([o[0] for o in outs]), np.concatenate([o[1] for o in outs]))

    monkeypatch.setattr(OA, "append", top_left)
    with pytest.raises(AssertionError):
        P.check_causal_prefill()
        P.check_brute_append()
