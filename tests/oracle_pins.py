"""Pins for the fp64 oracle: closed forms, identity cases, brute force, invariants.

Each ``check_*`` raises AssertionError when the oracle disagrees with what the
mathematics or the pages fix. The checks look the oracle functions up at call
time (``oracle.attention.attend`` etc.), so tests/test_oracle_mutations.py can
plant a mistake in a copy of one function and confirm that a check fails.
"""
from __future__ import annotations

import math

import numpy as np

import oracle.attention as OA
import oracle.merge as OM
from oracle.brute import brute_paged
from workloads import csr_from_page_lists, make_workload, to_storage_bits

TOL = 1e-12


def _close(a, b, tol=TOL):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    same_inf = np.isneginf(a) == np.isneginf(b)
    assert same_inf.all(), "-inf pattern differs"
    fin = ~np.isneginf(a)
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]))
        assert err <= tol, f"max abs err {err} > {tol}"


def _pool_from_float(K, V, dtype):
    """K, V float arrays [P, ps, Hkv, D] -> stored pool bits [P, 2, ps, Hkv, D]."""
    return np.stack([to_storage_bits(K, dtype), to_storage_bits(V, dtype)], axis=1)


# ---------------------------------------------------------------- closed forms
def check_single_token(seed=0):
    rng = np.random.default_rng(seed)
    D, Hq = 16, 4
    q = rng.standard_normal((3, Hq, D))
    K = rng.standard_normal((1, 2, D))
    V = rng.standard_normal((1, 2, D))
    scale = 0.37
    out, lse = OA.attend(q, K, V, scale)
    for h in range(Hq):
        hk = h // 2
        _close(out[:, h, :], np.repeat(V[0:1, hk, :], 3, axis=0))
        _close(lse[:, h], scale * (q[:, h, :] @ K[0, hk, :]))


def check_identical_keys(seed=1):
    rng = np.random.default_rng(seed)
    L, D = 37, 8
    k = rng.standard_normal(D)
    K = np.tile(k, (L, 1, 1))
    V = rng.standard_normal((L, 1, D))
    q = rng.standard_normal((2, 1, D))
    out, lse = OA.attend(q, K, V, 0.5)
    _close(out[:, 0, :], np.tile(V[:, 0, :].mean(axis=0), (2, 1)))
    _close(lse[:, 0], 0.5 * (q[:, 0, :] @ k) + math.log(L))


def check_q_zero_and_v_ones(seed=2):
    rng = np.random.default_rng(seed)
    L, D = 50, 8
    K = rng.standard_normal((L, 1, D))
    V = rng.standard_normal((L, 1, D))
    out, lse = OA.attend(np.zeros((1, 1, D)), K, V, 1.0)
    _close(out[0, 0], V[:, 0, :].mean(axis=0))
    _close(lse[0, 0], math.log(L))
    q = rng.standard_normal((4, 1, D)) * 3
    out1, _ = OA.attend(q, K, np.ones((L, 1, D)), 1.0)
    _close(out1, np.ones_like(out1), 1e-14)           # weights sum to one


def check_scale_default():
    """head_dim 128: q = 2 e0, k = 3 e0, one key -> lse = 6 / sqrt(128)."""
    D = 128
    q = np.zeros((1, 1, D)); q[0, 0, 0] = 2.0
    K = np.zeros((1, 1, D)); K[0, 0, 0] = 3.0
    V = np.ones((1, 1, D))
    _, lse = OA.attend(q, K, V, OA.default_scale(D))
    _close(lse[0, 0], 0.5303300858899106, 1e-15)


def check_gqa_map(seed=3):
    """8 q heads over 2 kv heads: heads 0-3 read kv head 0, heads 4-7 kv head 1."""
    rng = np.random.default_rng(seed)
    D, L = 8, 5
    K = np.zeros((L, 2, D)); K[:, 0, 0] = 1.0; K[:, 1, 0] = -2.0
    V = np.zeros((L, 2, D)); V[:, 0, :] = 10.0; V[:, 1, :] = 20.0
    q = rng.standard_normal((1, 8, D))
    out, lse = OA.attend(q, K, V, 1.0)
    for h in range(8):
        hk = h // 4
        _close(out[0, h], np.full(D, 10.0 * (hk + 1)))
        _close(lse[0, h], q[0, h, 0] * K[0, hk, 0] + math.log(L))


# ---------------------------------------------------------- paged structures
def identity_workload(dtype="bf16", lens=(1, 16, 17, 40, 33), Hq=8, Hkv=2, seed=11,
                      choose="random", extra_pages=3):
    """One-hot keys: per (request, kv head) one chosen token has k[0] = 64.

    q = 32 e0 for every head, so the chosen key scores 2048/sqrt(128) = 181
    above every other key and takes the whole weight. V of (page, slot, head)
    encodes (page // 256, page % 256, slot, head) as exact small integers.
    Unused tail slots and unreferenced pages hold NaN.
    """
    wl = make_workload(list(lens), Hq, Hkv, dtype, seed, mode="test", extra_pages=extra_pages)
    rng = np.random.default_rng(seed + 1000)
    ps, D = wl.page_size, wl.head_dim
    P = wl.num_pages
    nan_mask = np.isnan(OA.upcast(wl.pool, dtype))
    K = np.zeros((P, ps, Hkv, D), np.float32)
    V = np.zeros((P, ps, Hkv, D), np.float32)
    pg = np.arange(P)[:, None, None]
    sl = np.arange(ps)[None, :, None]
    hd = np.arange(Hkv)[None, None, :]
    V[..., 0] = pg // 256
    V[..., 1] = pg % 256
    V[..., 2] = sl
    V[..., 3] = hd
    chosen = {}
    for b, L in enumerate(lens):
        pages = wl.kv_indices[wl.kv_indptr[b]: wl.kv_indptr[b + 1]]
        for h in range(Hkv):
            if L == 0:
                continue
            if choose == "first":
                t = 0
            elif choose == "last":
                t = L - 1
            elif choose == "boundary":
                t = min(L - 1, ps)
            else:
                t = int(rng.integers(0, L))
            K[pages[t // ps], t % ps, h, 0] = 64.0
            chosen[(b, h)] = (int(pages[t // ps]), t % ps)
    pool = _pool_from_float(K, V, dtype)
    pool[nan_mask] = wl.pool[nan_mask]            # keep the NaN poison
    wl.pool = pool
    q = np.zeros((len(lens), Hq, D), np.float32)
    q[:, :, 0] = 32.0
    wl.q = to_storage_bits(q, dtype)
    return wl, chosen


def check_identity_gather(dtype="bf16", choose="random"):
    wl, chosen = identity_workload(dtype, choose=choose)
    out, lse = OA.decode(wl.q, wl.pool, dtype, wl.kv_indptr, wl.kv_indices, wl.last_page_len,
                         wl.page_size)
    G = wl.num_qo_heads // wl.num_kv_heads
    assert np.isfinite(out).all(), "NaN reached the output (read past kv_len?)"
    for (b, hk), (page, slot) in chosen.items():
        for h in range(hk * G, (hk + 1) * G):
            expect = np.zeros(wl.head_dim)
            expect[:4] = (page // 256, page % 256, slot, hk)
            assert np.max(np.abs(out[b, h] - expect)) < 1e-50, (b, h, out[b, h, :4], expect[:4])


def check_count(dtype="bf16", lens=(1, 15, 16, 17, 31, 32, 33, 100, 0)):
    """q = 0 -> lse = ln(kv_len) exactly; the NaN tails must stay unread."""
    wl = make_workload(list(lens), 4, 2, dtype, 21, mode="test", extra_pages=2)
    wl.q = np.zeros_like(wl.q)
    out, lse = OA.decode(wl.q, wl.pool, dtype, wl.kv_indptr, wl.kv_indices, wl.last_page_len,
                         wl.page_size)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.isneginf(lse[b]).all() and (out[b] == 0).all()
        else:
            assert np.all(np.abs(lse[b] - math.log(L)) <= 1e-13), (b, L, lse[b])
            assert np.isfinite(out[b]).all()


def _tiny_paged(dtype, lens, qo_lens, Hq, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    ps = 4
    n = [-(-L // ps) for L in lens]
    P = sum(n) + 2
    perm = rng.permutation(P)
    lists, off = [], 0
    for k in n:
        lists.append(list(perm[off: off + k]))
        off += k
    indptr, indices = csr_from_page_lists(lists)
    last = np.array([0 if k == 0 else L - (k - 1) * ps for L, k in zip(lens, n)], np.int32)
    K = rng.standard_normal((P, ps, Hkv, D)).astype(np.float32)
    V = rng.standard_normal((P, ps, Hkv, D)).astype(np.float32)
    pool = _pool_from_float(K, V, dtype)
    rows = sum(qo_lens)
    q = to_storage_bits(rng.standard_normal((rows, Hq, D)).astype(np.float32), dtype)
    return pool, indptr, indices, last, ps, q


def _to_lists(pool_bits, dtype):
    return OA.upcast(pool_bits, dtype).tolist()


def check_brute_decode(dtype="bf16", seed=5):
    lens = [0, 1, 3, 4, 5, 9]
    Hq, Hkv, D = 4, 2, 6
    pool, indptr, indices, last, ps, q = _tiny_paged(dtype, lens, [1] * len(lens), Hq, Hkv, D,
                                                     seed)
    scale = 1 / math.sqrt(D)
    out, lse = OA.decode(q, pool, dtype, indptr, indices, last, ps)
    bo, bl = brute_paged(OA.upcast(q, dtype).tolist(), _to_lists(pool, dtype), indptr.tolist(),
                         indices.tolist(), last.tolist(), ps, list(range(len(lens))),
                         [10 ** 9] * len(lens), Hq, Hkv, scale)
    _close(out, np.array(bo))
    _close(lse, np.array(bl))


def check_brute_append(dtype="bf16", seed=6, causal=True):
    lens = [5, 9, 4, 7]
    qo = [2, 9, 1, 3]
    Hq, Hkv, D = 4, 1, 5
    pool, indptr, indices, last, ps, q = _tiny_paged(dtype, lens, qo, Hq, Hkv, D, seed)
    qo_indptr = np.concatenate([[0], np.cumsum(qo)]).astype(np.int32)
    scale = 1 / math.sqrt(D)
    out, lse = OA.append(q, qo_indptr, pool, dtype, indptr, indices, last, ps, causal=causal)
    req, vis = [], []
    for b in range(len(lens)):
        for i in range(qo[b]):
            req.append(b)
            # position of the i-th new row, counted from the start of the sequence
            vis.append(lens[b] - qo[b] + i + 1 if causal else lens[b])
    bo, bl = brute_paged(OA.upcast(q, dtype).tolist(), _to_lists(pool, dtype), indptr.tolist(),
                         indices.tolist(), last.tolist(), ps, req, vis, Hq, Hkv, scale)
    _close(out, np.array(bo))
    _close(lse, np.array(bl))


def check_causal_prefill(dtype="bf16", seed=7):
    """qo_len == kv_len: row 0 sees only key 0 (out = v_0, lse = s_00); the
    last row sees every key (equals decode of that row)."""
    L = 37
    wl = make_workload([L], 4, 2, dtype, seed, qo_lens=[L], causal=True, mode="test")
    out, lse = OA.append(wl.q, wl.qo_indptr, wl.pool, dtype, wl.kv_indptr, wl.kv_indices,
                         wl.last_page_len, wl.page_size, causal=True)
    K, V = OA.gather_request_kv(wl.pool, dtype, wl.kv_indptr, wl.kv_indices, wl.last_page_len,
                                wl.page_size, 0)
    q = OA.upcast(wl.q, dtype)
    scale = 1 / math.sqrt(wl.head_dim)
    for h in range(4):
        hk = h // 2
        _close(out[0, h], V[0, hk])
        _close(lse[0, h], scale * float(q[0, h] @ K[0, hk]))
    dq = wl.q[L - 1: L]
    od, sd = OA.decode(dq, wl.pool, dtype, wl.kv_indptr, wl.kv_indices, wl.last_page_len,
                       wl.page_size)
    _close(out[L - 1], od[0])
    _close(lse[L - 1], sd[0])
    # with a cache: request of 30 tokens, the last 6 new; the first new row
    # sees 25 keys, i.e. equals attention over the first 25 tokens.
    wl2 = make_workload([30], 4, 2, dtype, seed + 1, qo_lens=[6], causal=True, mode="test")
    o2, s2 = OA.append(wl2.q, wl2.qo_indptr, wl2.pool, dtype, wl2.kv_indptr, wl2.kv_indices,
                       wl2.last_page_len, wl2.page_size, causal=True)
    K2, V2 = OA.gather_request_kv(wl2.pool, dtype, wl2.kv_indptr, wl2.kv_indices,
                                  wl2.last_page_len, wl2.page_size, 0)
    q2 = OA.upcast(wl2.q, dtype)
    for i in (0, 5):
        n_vis = 25 + i
        S = scale * (q2[i, 0] @ K2[:n_vis, 0].T)
        w = np.exp(S - S.max())
        _close(o2[i, 0], (w @ V2[:n_vis, 0]) / w.sum(), 1e-12)
        _close(s2[i, 0], S.max() + math.log(w.sum()), 1e-12)


def check_permutation_invariance(dtype="bf16", seed=8):
    wl = make_workload([33, 64, 7], 8, 2, dtype, seed, mode="test", extra_pages=4)
    a = OA.decode(wl.q, wl.pool, dtype, wl.kv_indptr, wl.kv_indices, wl.last_page_len,
                  wl.page_size)
    rng = np.random.default_rng(seed + 7)
    perm = rng.permutation(wl.num_pages)          # new physical slot of page p is perm[p]
    pool2 = np.empty_like(wl.pool)
    pool2[perm] = wl.pool
    idx2 = perm[wl.kv_indices].astype(np.int32)
    b = OA.decode(wl.q, pool2, dtype, wl.kv_indptr, idx2, wl.last_page_len, wl.page_size)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- merge / cascade
def check_merge_split(seed=9):
    rng = np.random.default_rng(seed)
    L, D, Hq, Hkv = 41, 8, 4, 2
    K = rng.standard_normal((L, Hkv, D))
    V = rng.standard_normal((L, Hkv, D))
    q = rng.standard_normal((3, Hq, D))
    whole_o, whole_s = OA.attend(q, K, V, 0.3)
    for cuts in ([0, 41], [0, 20, 41], [0, 1, 2, 40, 41], [0, 0, 10, 10, 41], [0, 7, 13, 29, 41]):
        parts = [OA.attend(q, K[a:b], V[a:b], 0.3) for a, b in zip(cuts[:-1], cuts[1:])]
        vo = np.stack([p[0] for p in parts], axis=2)       # [R, Hq, k, D]
        so = np.stack([p[1] for p in parts], axis=2)       # [R, Hq, k]
        mo, ms = OM.merge_states(vo, so)
        _close(mo, whole_o)
        _close(ms, whole_s)
        if len(parts) == 2:
            mo2, ms2 = OM.merge_state(parts[0][0], parts[0][1], parts[1][0], parts[1][1])
            _close(mo2, whole_o)
            _close(ms2, whole_s)


def check_merge_algebra(seed=10):
    rng = np.random.default_rng(seed)
    shp = (5, 3)
    v = [rng.standard_normal(shp + (4,)) for _ in range(3)]
    s = [rng.standard_normal(shp) * 4 for _ in range(3)]
    ab = OM.merge_state(v[0], s[0], v[1], s[1])
    ab_c = OM.merge_state(ab[0], ab[1], v[2], s[2])
    bc = OM.merge_state(v[1], s[1], v[2], s[2])
    a_bc = OM.merge_state(v[0], s[0], bc[0], bc[1])
    _close(ab_c[0], a_bc[0]); _close(ab_c[1], a_bc[1])
    ba = OM.merge_state(v[1], s[1], v[0], s[0])
    _close(ab[0], ba[0]); _close(ab[1], ba[1])
    ninf = np.full(shp, -np.inf)
    ident = OM.merge_state(v[0], s[0], np.zeros_like(v[0]), ninf)
    _close(ident[0], v[0]); _close(ident[1], s[0])
    empty = OM.merge_state(v[0], ninf, v[1], ninf)
    assert np.isneginf(empty[1]).all() and (empty[0] == 0).all()
    # two equal states: lse grows by ln 2, value unchanged
    same = OM.merge_state(v[0], s[0], v[0], s[0])
    _close(same[0], v[0]); _close(same[1], s[0] + math.log(2))


def check_cascade(dtype="bf16", seed=12):
    from workloads import make_cascade
    wl = make_cascade(64, [5, 16, 17, 40], 8, 2, dtype, seed, mode="test")
    args = (wl.q, wl.pool, dtype, wl.prefix_indptr, wl.prefix_indices, wl.prefix_last_page_len,
            wl.kv_indptr, wl.kv_indices, wl.last_page_len, wl.page_size)
    a = OA.cascade(*args)
    b = OA.cascade_direct(*args)
    _close(a[0], b[0]); _close(a[1], b[1])


# ---------------------------------------------------------------- FP8 (E4M3) KV
# Values fixed by the OCP 8-bit floating-point definition of E4M3 (bias 7,
# 3 mantissa bits, subnormals at exponent field 0, no infinities, NaN at
# S.1111.111), worked out by hand.
E4M3_SPOT = {
    0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
    0x3C: 1.5, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0,
}


def _torch_e4m3(codes):
    """Codes -> float64 through torch's float8_e4m3fn (not the oracle's code)."""
    import torch

    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def check_e4m3_definition():
    codes = np.arange(256, dtype=np.uint8)
    v = OA.upcast(codes, "e4m3")
    for c, want in E4M3_SPOT.items():
        assert v[c] == want, f"code {c:#04x}: {v[c]} != {want}"
    assert math.copysign(1.0, v[0x80]) < 0 and v[0x80] == 0.0, "0x80 must be -0"
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]), "S.1111.111 must be NaN"
    assert np.all(np.diff(v[:127]) > 0), "codes 0..126 must increase"
    assert np.array_equal(v[128:255], -v[:127]), "sign bit must negate"
    ref = _torch_e4m3(codes)
    fin = ~np.isnan(ref)
    assert np.array_equal(v[fin], ref[fin]), "differs from torch float8_e4m3fn"


def _fp8_tiny(seed):
    from workloads import make_workload

    return make_workload([0, 1, 15, 16, 17, 40], 4, 2, "bf16", seed, head_dim=16, page_size=4,
                         mode="test", extra_pages=2, kv_dtype="e4m3")


def check_fp8_scale_placement(seed=41):
    """s_j is linear in k (k_scale joins sm_scale); out is linear in v and the
    lse does not see v_scale."""
    wl = _fp8_tiny(seed)
    args = (wl.q, wl.pool, "bf16", wl.kv_indptr, wl.kv_indices, wl.last_page_len, wl.page_size)
    sm, a, b = 0.3, 0.05, 0.07
    o1, s1 = OA.decode(*args, scale=sm, kv_dtype="e4m3", k_scale=a, v_scale=b)
    o0, s0 = OA.decode(*args, scale=sm * a, kv_dtype="e4m3")
    _close(o1, b * o0)
    _close(s1, s0)


def check_brute_decode_fp8(seed=42):
    """Uniform random codes (subnormals to +-448, NaN codes excluded) decoded by
    torch, scaled, and attended by the pure-Python brute force."""
    rng = np.random.default_rng(seed)
    lens = [0, 1, 3, 4, 5, 9]
    Hq, Hkv, D, ps = 4, 2, 6, 4
    n = [-(-L // ps) for L in lens]
    P = sum(n) + 1
    perm = rng.permutation(P)
    lists, off = [], 0
    for k in n:
        lists.append(list(perm[off: off + k]))
        off += k
    indptr, indices = csr_from_page_lists(lists)
    last = np.array([0 if k == 0 else L - (k - 1) * ps for L, k in zip(lens, n)], np.int32)
    pool = rng.integers(0, 256, size=(P, 2, ps, Hkv, D)).astype(np.uint8)
    pool[(pool & 0x7F) == 0x7F] = 0x3A  # no NaN codes
    q = to_storage_bits(rng.standard_normal((len(lens), Hq, D)).astype(np.float32), "bf16")
    ks, vs, sm = 1.0 / 56.0, 3.0 / 224.0, 1 / math.sqrt(D)
    out, lse = OA.decode(q, pool, "bf16", indptr, indices, last, ps, kv_dtype="e4m3",
                         k_scale=ks, v_scale=vs)
    vals = _torch_e4m3(pool)
    vals[:, 0] *= ks
    vals[:, 1] *= vs
    bo, bl = brute_paged(OA.upcast(q, "bf16").tolist(), vals.tolist(), indptr.tolist(),
                         indices.tolist(), last.tolist(), ps, list(range(len(lens))),
                         [10 ** 9] * len(lens), Hq, Hkv, sm)
    _close(out, np.array(bo))
    _close(lse, np.array(bl))


# ---------------------------------------------------------------- ragged KV
def check_brute_ragged(seed=43):
    """Ragged decode and causal / non-causal append against the pure-Python
    brute force over explicit row slices (q heads 4, kv heads 2)."""
    from oracle.brute import brute_attention_row
    from workloads import make_ragged
    lens, qo = [0, 1, 3, 5, 9], [0, 1, 2, 5, 3]
    Hq, Hkv, D = 4, 2, 6
    for causal in (True, False):
        rw = make_ragged(lens, Hq, Hkv, "bf16", seed, qo_lens=qo, causal=causal, head_dim=D)
        sc = 1 / math.sqrt(D)
        K, V = OA.upcast(rw.k, "bf16").tolist(), OA.upcast(rw.v, "bf16").tolist()
        Q = OA.upcast(rw.q, "bf16").tolist()
        out, lse = OA.append_ragged(rw.q, rw.qo_indptr, rw.k, rw.v, "bf16", rw.kv_offsets,
                                    causal=causal)
        r = 0
        for b, L in enumerate(lens):
            o0 = int(rw.kv_offsets[b])
            for i in range(qo[b]):
                vis = L - qo[b] + i + 1 if causal else L
                for h in range(Hq):
                    keys = [K[o0 + t][h // 2] for t in range(vis)]
                    vals = [V[o0 + t][h // 2] for t in range(vis)]
                    bo, bl = brute_attention_row(Q[r][h], keys, vals, sc)
                    _close(out[r, h], np.array(bo))
                    _close([lse[r, h]], [bl])
                r += 1
    dw = make_ragged(lens, Hq, Hkv, "bf16", seed + 1, head_dim=D)
    out, lse = OA.decode_ragged(dw.q, dw.k, dw.v, "bf16", dw.kv_offsets)
    K, V = OA.upcast(dw.k, "bf16").tolist(), OA.upcast(dw.v, "bf16").tolist()
    Q = OA.upcast(dw.q, "bf16").tolist()
    for b, L in enumerate(lens):
        o0 = int(dw.kv_offsets[b])
        for h in range(Hq):
            bo, bl = brute_attention_row(Q[b][h], [K[o0 + t][h // 2] for t in range(L)],
                                         [V[o0 + t][h // 2] for t in range(L)], 1 / math.sqrt(D))
            _close(out[b, h], np.array(bo))
            _close([lse[b, h]], [bl])


# ---------------------------------------------------------------- block-sparse
def check_brute_block_sparse(seed=44):
    """Variable block-sparse attention against the pure-Python brute force
    over an explicit dense mask (row blocks of 1-3 rows, column blocks of
    2-4 keys, an empty row block)."""
    from oracle.brute import brute_attention_row
    from workloads import make_block_sparse
    bw = make_block_sparse([2, 1, 3, 2], [3, 2, 4, 2, 3], 0.5, 4, 2, "bf16", seed, head_dim=6,
                           empty_rows=[1])
    out, lse = OA.block_sparse(bw.q, bw.k, bw.v, "bf16", bw.block_indptr, bw.block_indices,
                               bw.row_offsets, bw.col_offsets)
    Q, K, V = (OA.upcast(x, "bf16").tolist() for x in (bw.q, bw.k, bw.v))
    N = int(bw.col_offsets[-1])
    for i in range(4):
        sel = set(bw.block_indices[bw.block_indptr[i]:bw.block_indptr[i + 1]].tolist())
        # dense mask: key t is visible iff its column block is selected
        visible = [t for t in range(N)
                   if int(np.searchsorted(bw.col_offsets, t, side="right") - 1) in sel]
        for r in range(int(bw.row_offsets[i]), int(bw.row_offsets[i + 1])):
            for h in range(4):
                bo, bl = brute_attention_row(Q[r][h], [K[t][h // 2] for t in visible],
                                             [V[t][h // 2] for t in visible], 1 / math.sqrt(6))
                _close(out[r, h], np.array(bo))
                _close([lse[r, h]], [bl])


ALL_CHECKS = [
    check_single_token, check_identical_keys, check_q_zero_and_v_ones, check_scale_default,
    check_gqa_map, check_identity_gather, check_count, check_brute_decode, check_brute_append,
    check_causal_prefill, check_permutation_invariance, check_merge_split, check_merge_algebra,
    check_cascade, check_e4m3_definition, check_fp8_scale_placement, check_brute_decode_fp8,
    check_brute_ragged, check_brute_block_sparse,
]
