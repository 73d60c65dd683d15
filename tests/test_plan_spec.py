"""The reference plan procedure: a hand-worked example and invariants."""
import numpy as np
import pytest

from oracle.plan_spec import PlanSpecError, plan_spec
from workloads import config_lengths


def _indptr(lens, ps=16):
    n = [-(-int(L) // ps) for L in lens]
    return np.concatenate([[0], np.cumsum(n)]).astype(np.int64)


def test_hand_worked_decode_plan():
    # Three requests of 4, 2, 5 full pages (the page lists of the worked CSR
    # example), 2 kv heads; piece cost c0 = 4 pages. 16 workers -> NS = 8 bins;
    # N = 11 pages, Q = ceil((11 + 4*3) / 8) = 3: request 0 -> [0,3) [3,4),
    # request 1 -> [0,2), request 2 -> [0,3) [3,5). Dealt largest first
    # (stable): (0,[0,3)) bin 0, (2,[0,3)) bin 1, (1,[0,2)) bin 2, (2,[3,5))
    # bin 3, (0,[3,4)) bin 4. List j = bin*2 + head runs on wave j. Requests 0
    # and 2 are split: head h of request 0 owns slots 2h, 2h+1; of request 2,
    # 4+2h, 5+2h. Field 2 is the request's first page in kv_indices (0, 4, 6).
    lens = [64, 32, 80]
    p = plan_spec(_indptr(lens), lens, 3, 2, 2, 128, 16, max_batch=3, num_cu=4, tiles_per_cu=4)
    assert p["tiles"].tolist() == [
        [0, 0, 0, 0, 0, 48, 0, 2], [0, 1, 0, 2, 0, 48, 2, 2],       # bin 0
        [2, 0, 6, 4, 0, 48, 4, 2], [2, 1, 6, 6, 0, 48, 6, 2],       # bin 1
        [1, 0, 4, -1, 0, 32, -1, 1], [1, 1, 4, -1, 0, 32, -1, 1],   # bin 2
        [2, 0, 6, 4, 48, 80, 5, 2], [2, 1, 6, 6, 48, 80, 7, 2],     # bin 3
        [0, 0, 0, 0, 48, 64, 1, 2], [0, 1, 0, 2, 48, 64, 3, 2],     # bin 4
    ]
    assert p["worker_ptr"].tolist() == list(range(11)) + [10] * 6
    assert p["merge"].tolist() == [[0, 0, 0, 2], [0, 1, 2, 2], [2, 0, 4, 2], [2, 1, 6, 2]]
    assert p["num_slots"] == 8 and p["chunk_pages"] == 3
    # 8 workers -> 4 bins, Q = ceil(23 / 4) = 6: no request is split; dealt
    # 5, 4, 2 pages to bins 0, 1, 2 (waves 0-1, 2-3, 4-5)
    p = plan_spec(_indptr(lens), lens, 3, 2, 2, 128, 16, max_batch=3, num_cu=2, tiles_per_cu=4)
    assert p["num_slots"] == 0 and p["merge"].shape == (0, 4) and p["chunk_pages"] == 6
    assert p["tiles"].tolist() == [
        [2, 0, 6, -1, 0, 80, -1, 1], [2, 1, 6, -1, 0, 80, -1, 1],
        [0, 0, 0, -1, 0, 64, -1, 1], [0, 1, 0, -1, 0, 64, -1, 1],
        [1, 0, 4, -1, 0, 32, -1, 1], [1, 1, 4, -1, 0, 32, -1, 1],
    ]
    assert p["worker_ptr"].tolist() == [0, 1, 2, 3, 4, 5, 6, 6, 6]
    # one worker: one bin; the wave runs list 0 (head 0) then list 1 (head 1)
    p = plan_spec(_indptr(lens), lens, 3, 2, 2, 128, 16, max_batch=3, num_cu=1, tiles_per_cu=1)
    assert p["tiles"][:, :2].tolist() == [[2, 0], [0, 0], [1, 0], [2, 1], [0, 1], [1, 1]]
    assert p["worker_ptr"].tolist() == [0, 6]
    # an E4M3 pool: c0 = 8 -> Q = ceil((11 + 24) / 8) = 5, no split
    p = plan_spec(_indptr(lens), lens, 3, 2, 2, 128, 16, max_batch=3, num_cu=4, tiles_per_cu=4,
                  kv_dtype="e4m3")
    assert p["chunk_pages"] == 5 and p["num_slots"] == 0


def test_hand_worked_append_plan():
    # one request, kv 40, 40 new rows (pure prefill), qo_tile 16, causal:
    # q tiles rows [0,16) vis 16, [16,32) vis 32, [32,40) vis 40 -> 1+2+3 = 6 pages;
    # 1 kv head, target 4 -> P = 2 pages: C = 1, 1, 2; the split unit has 8 rows.
    p = plan_spec([0, 3], [40], 1, 4, 1, 128, 16, max_batch=1, qo_indptr=[0, 40], causal=True,
                  max_qo_tokens=40, num_cu=1, tiles_per_cu=4, qo_tile=16)
    assert p["chunk_pages"] == 2
    assert p["tiles"].tolist() == [
        [0, 0, 16, 32, 0, 32, -1, 1],
        [0, 0, 0, 16, 0, 16, -1, 1],
        [0, 0, 32, 40, 0, 32, 0, 2],
        [0, 0, 32, 40, 32, 40, 8, 2],
    ]
    assert p["num_slots"] == 16
    assert p["worker_ptr"].tolist() == [0, 4, 4, 4, 4, 4, 4, 4, 4]  # one group: all in bin 0
    assert p["merge"].tolist() == [[32, 0, 0, 2]]


def test_hand_worked_append_xcd_bins():
    # 2 requests x 2 kv heads (G = 1), non-causal, qo_tile 16: request 0 has 16
    # rows over 32 keys, request 1 16 rows over 16 keys. target 64 -> P = 1 page:
    # request 0 splits in 2 chunks (slots: head 0 base 0, head 1 base 32).
    # Group costs (0,0) 512, (0,1) 512, (1,0) 256, (1,1) 256 are dealt to bins
    # 0, 1, 2, 3 (each to the least-loaded bin, lowest index first).
    p = plan_spec([0, 2, 3], [32, 16], 2, 2, 2, 128, 16, max_batch=2, qo_indptr=[0, 16, 32],
                  causal=False, max_qo_tokens=32, num_cu=1, tiles_per_cu=64, qo_tile=16)
    assert p["chunk_pages"] == 1
    assert p["tiles"].tolist() == [
        [0, 0, 0, 16, 0, 16, 0, 2],
        [0, 0, 0, 16, 16, 32, 16, 2],
        [0, 1, 0, 16, 0, 16, 32, 2],
        [0, 1, 0, 16, 16, 32, 48, 2],
        [1, 0, 16, 32, 0, 16, -1, 1],
        [1, 1, 16, 32, 0, 16, -1, 1],
    ]
    assert p["worker_ptr"].tolist() == [0, 2, 4, 5, 6, 6, 6, 6, 6]
    assert p["merge"].tolist() == [[0, 0, 0, 2], [0, 1, 32, 2]]
    assert p["num_slots"] == 64


def _pages(k0, k1, ps=16):
    return -(-k1 // ps) - k0 // ps


def check_decode_invariants(p, lens, Hkv, ps=16, c0=4):
    tiles, wptr, Q = p["tiles"], p["worker_ptr"], p["chunk_pages"]
    S = p["target"]
    assert len(wptr) == S + 1 and wptr[0] == 0 and wptr[-1] == len(tiles)
    assert np.all(np.diff(wptr) >= 0)
    NS = max(1, S * p["knobs"]["pieces_per_worker"] // Hkv)
    if NS * Hkv <= S:
        # wave s*Hkv + h runs bin s for head h: the Hkv waves of a bin run the
        # same pieces; the pieces of a bin come in non-increasing pages; the
        # bins' costs (pages + c0 per piece) are within one piece of each other
        bcost = []
        for sg in range(NS):
            lists = [tiles[wptr[sg * Hkv + h]:wptr[sg * Hkv + h + 1]] for h in range(Hkv)]
            for h, lst in enumerate(lists):
                assert (lst[:, 1] == h).all()
                assert (lst[:, [0, 4, 5]] == lists[0][:, [0, 4, 5]]).all()
            pg = [_pages(t[4], t[5], ps) for t in lists[0].tolist()]
            assert all(x >= y for x, y in zip(pg, pg[1:])), "bin not in dealing order"
            bcost.append(sum(pg) + c0 * len(pg))
        assert wptr[NS * Hkv] == len(tiles), "waves past the bins hold tiles"
        if len(tiles):
            assert max(bcost) - min(bcost) <= Q + c0, "bins out of balance"
    by_unit = {}
    for t in tiles.tolist():
        by_unit.setdefault((t[0], t[1]), []).append(t)
    assert sorted(by_unit) == [(b, h) for b in range(len(lens)) for h in range(Hkv)]
    slots = set()
    for (b, h), parts in by_unit.items():
        parts.sort(key=lambda t: t[4] if t[6] < 0 else t[6])
        L = int(lens[b])
        n = -(-L // ps)
        C = len(parts)
        assert C == max(1, -(-n // Q)), "piece count"
        assert parts[0][4] == 0 and parts[-1][5] == L
        for a, c in zip(parts[:-1], parts[1:]):
            assert a[5] == c[4] and c[4] % ps == 0
        sizes = [_pages(t[4], t[5], ps) for t in parts]
        assert all(x == Q for x in sizes[:-1]) and sizes[-1] <= Q  # full pieces, then the rest
        for i, t in enumerate(parts):
            assert t[2] == sum(-(-int(x) // ps) for x in lens[:b]) and t[7] == C
            if C == 1:
                assert t[3] == -1 and t[6] == -1
            else:
                assert t[6] == t[3] + i
                slots.add(t[6])
    assert slots == set(range(p["num_slots"]))


def check_append_invariants(p, lens, Hkv, qo_indptr, causal, ps=16):
    tiles = p["tiles"]
    cost = (tiles[:, 5] - tiles[:, 4]).astype(np.int64) * (tiles[:, 3] - tiles[:, 2])
    # XCD bins: bin offsets, each (request, kv head) group contiguous in one
    # bin with its tiles in descending cost, and the greedy balance bound
    wptr = p["worker_ptr"]
    assert len(wptr) == 9 and wptr[0] == 0 and wptr[-1] == len(tiles)
    assert np.all(np.diff(wptr) >= 0)
    seen, bcost, gcost = set(), [0] * 8, {}
    for x in range(8):
        prev = None
        for i in range(wptr[x], wptr[x + 1]):
            g = (int(tiles[i, 0]), int(tiles[i, 1]))
            if g != prev:
                assert g not in seen, "group split across runs or bins"
                seen.add(g)
            else:
                assert cost[i] <= cost[i - 1], "group tiles not in descending cost"
            prev = g
            bcost[x] += int(cost[i])
            gcost[g] = gcost.get(g, 0) + int(cost[i])
    if gcost:
        assert max(bcost) - min(bcost) <= max(gcost.values()), "bins out of balance"
    assert np.all(tiles[:, 4] % ps == 0), "chunk begin not page aligned"
    cover = {}
    for b, h, q0, q1, t0, t1, s0, C in tiles.tolist():
        cover.setdefault((b, h, q0, q1), []).append((t0, t1, s0, C))
    rows_seen = {}
    used = set()
    for (b, h, q0, q1), parts in cover.items():
        parts.sort()
        L = int(lens[b])
        ql = qo_indptr[b + 1] - qo_indptr[b]
        vis = min(L, L - ql + (q1 - qo_indptr[b])) if causal else L
        assert parts[0][0] == 0 and parts[-1][1] == max(vis, 0)
        for (a0, a1, _, _), (b0, b1, _, _) in zip(parts[:-1], parts[1:]):
            assert a1 == b0, "chunks must tile the key range"
        C = parts[0][3]
        assert len(parts) == C and all(x[3] == C for x in parts)
        if C == 1:
            assert parts[0][2] == -1
        else:
            for c, x in enumerate(parts):
                assert x[2] == parts[0][2] + c * (q1 - q0)
                for r in range(q1 - q0):
                    assert x[2] + r not in used
                    used.add(x[2] + r)
        for r in range(q0, q1):
            rows_seen[(r, h)] = rows_seen.get((r, h), 0) + 1
    for r in range(int(qo_indptr[-1])):
        for h in range(Hkv):
            assert rows_seen.get((r, h), 0) == 1, "each (row, kv head) in exactly one q tile"
    assert used == set(range(p["num_slots"]))


@pytest.mark.parametrize("k", [1, 2, 3])
def test_decode_configs(k):
    lens = config_lengths(k, np.random.default_rng(k))["kv_lens"]
    Hkv = 32 if k == 1 else 8
    p = plan_spec(_indptr(lens), lens, len(lens), 32, Hkv, 128, 16, max_batch=len(lens))
    check_decode_invariants(p, lens, Hkv)
    assert len(p["tiles"]) <= p["knobs"]["max_tiles"]


def test_append_batch16_and_cascade_prefix():
    lens = [4608] * 16
    qo = np.concatenate([[0], np.cumsum([512] * 16)])
    p = plan_spec(_indptr(lens), lens, 16, 32, 8, 128, 16, max_batch=16, qo_indptr=qo,
                  causal=True, max_qo_tokens=8192)
    check_append_invariants(p, lens, 8, qo, True)
    # q tiles of 256 / G = 64 rows: 8 per (request, kv head), no key split
    assert p["num_slots"] == 0 and len(p["tiles"]) == 16 * 8 * 8
    p = plan_spec([0, 1024], [16384], 1, 32, 8, 128, 16, max_batch=1, qo_indptr=[0, 256],
                  causal=False, max_qo_tokens=256)
    check_append_invariants(p, [16384], 8, [0, 256], False)
    # 4 q tiles x 8 kv heads x 1024 pages over 512 tiles: chunks of 64 pages
    assert p["chunk_pages"] == 64 and len(p["tiles"]) == 512


def test_random_geometries():
    rng = np.random.default_rng(0)
    for it in range(300):
        B = int(rng.integers(0, 9))
        lens = rng.integers(0, 300, size=B)
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8]))
        knobs = dict(num_cu=int(rng.integers(1, 9)), tiles_per_cu=int(rng.integers(1, 5)),
                     min_chunk_pages=int(rng.integers(1, 4)))
        if it % 2:
            p = plan_spec(_indptr(lens), lens, B, G * Hkv, Hkv, 128, 16, max_batch=max(B, 1),
                          pieces_per_worker=int(rng.integers(1, 5)), **knobs)
            check_decode_invariants(p, lens, Hkv)
        else:
            ql = np.minimum(rng.integers(0, 70, size=B), lens)
            qo = np.concatenate([[0], np.cumsum(ql)]).astype(np.int64)
            causal = bool(rng.integers(0, 2))
            qt = min(int(rng.choice([8, 16, 32, 64])), 256 // G)
            p = plan_spec(_indptr(lens), lens, B, G * Hkv, Hkv, 128, 16, max_batch=max(B, 1),
                          qo_indptr=qo, causal=causal, max_qo_tokens=max(int(qo[-1]), 1),
                          qo_tile=qt, **knobs)
            check_append_invariants(p, lens, Hkv, qo, causal)


@pytest.mark.parametrize("bad,code", [
    (dict(lens=[33], indptr=[0, 2]), "INVALID"),      # 33 tokens need 3 pages
    (dict(lens=[32], indptr=[0, 3]), "INVALID"),      # 3 pages but only 32 tokens
    (dict(lens=[5], indptr=[0, 0]), "INVALID"),       # tokens without pages
    (dict(lens=[16], indptr=[1, 2]), "INVALID"),      # indptr must start at 0
    (dict(Hq=12, Hkv=8), "INVALID"),                  # non-integer group
    (dict(D=64), "UNSUPPORTED"),
    (dict(Hq=48, Hkv=3), "UNSUPPORTED"),              # group 16
    (dict(max_batch=0), "INVALID"),
])
def test_errors(bad, code):
    args = dict(lens=[16], indptr=[0, 1], Hq=8, Hkv=2, D=128, max_batch=1)
    args.update(bad)
    with pytest.raises(PlanSpecError) as e:
        plan_spec(args["indptr"], args["lens"], len(args["lens"]), args["Hq"], args["Hkv"],
                  args["D"], 16, max_batch=args["max_batch"])
    assert e.value.code == code


def test_capacity_error():
    lens = [160] * 4
    with pytest.raises(PlanSpecError) as e:
        plan_spec(_indptr(lens), lens, 4, 8, 8, 128, 16, max_batch=4, max_tiles=16, num_cu=64)
    assert e.value.code == "CAPACITY"
