"""The seeded generator: storage rounding, page-table layout, config recipes."""
import json
import os

import numpy as np
import pytest

import oracle.attention as OA
from workloads import config_lengths, csr_from_page_lists, make_cascade, make_workload, to_storage_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, -2.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -7, 3.0e38, np.inf, -0.0],
                 np.float32)
    bits = to_storage_bits(x, "bf16")
    # 1+2^-8 is halfway between 1.0 and 1.0078125 -> even (1.0); 1+3*2^-8 -> 1.015625
    assert bits.tolist() == [0x3F80, 0xC000, 0x3F80, 0x3F82, 0x3F81, 0x7F62, 0x7F80, 0x8000]
    assert OA.upcast(bits, "bf16")[:5].tolist() == [1.0, -2.0, 1.0, 1.015625, 1.0078125]


def test_fp16_round_to_nearest_even():
    x = np.array([1.0, 1 + 2 ** -11, 1 + 3 * 2 ** -11, 65504.0, 1 / 3], np.float32)
    bits = to_storage_bits(x, "fp16")
    assert bits.tolist()[:4] == [0x3C00, 0x3C00, 0x3C02, 0x7BFF]
    assert OA.upcast(bits, "fp16")[4] == 0.333251953125


def test_csr_example_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "csr_example.json")))
    indptr, indices = csr_from_page_lists(g["page_lists"])
    assert indptr.tolist() == g["kv_indptr"] and indices.tolist() == g["kv_indices"]
    for b, pl in enumerate(g["page_lists"]):
        assert OA.request_pages(indptr, indices, b).tolist() == pl
        assert OA.request_kv_len(indptr, g["last_page_len_reading"], g["page_size"], b) == \
            g["kv_lens_reading"][b]


def test_layout_and_last_page_len():
    wl = make_workload([1, 16, 17, 0, 40], 4, 2, "bf16", 3, mode="test", extra_pages=2)
    assert wl.kv_indptr.tolist() == [0, 1, 2, 4, 4, 7]
    assert wl.last_page_len.tolist() == [1, 16, 1, 0, 8]
    assert wl.pool.shape == (9, 2, 16, 2, 128) and wl.q.shape == (5, 4, 128)
    assert sorted(wl.kv_indices.tolist() + []) == sorted(set(wl.kv_indices.tolist()))
    # poison: the tail of request 0's only page, all unreferenced pages
    p0 = wl.kv_indices[0]
    assert (wl.pool[p0, :, 1:] == 0x7FC0).all() and not (wl.pool[p0, :, 0] == 0x7FC0).any()
    unref = sorted(set(range(9)) - set(wl.kv_indices.tolist()))
    assert len(unref) == 2 and (wl.pool[unref] == 0x7FC0).all()


def test_determinism_and_seed():
    a = make_workload([40, 9], 8, 2, "bf16", 5)
    b = make_workload([40, 9], 8, 2, "bf16", 5)
    c = make_workload([40, 9], 8, 2, "bf16", 6)
    assert a.manifest() == b.manifest() and a.manifest() != c.manifest()


def test_cascade_layout():
    wl = make_cascade(64, [5, 16, 17], 8, 2, "bf16", 1)
    assert wl.prefix_indptr.tolist() == [0, 4] and wl.prefix_last_page_len.tolist() == [16]
    allp = sorted(wl.prefix_indices.tolist() + wl.kv_indices.tolist())
    assert allp == list(range(wl.num_pages))


def test_config_length_recipes():
    r = config_lengths(2, np.random.default_rng(2))["kv_lens"]
    assert r.shape == (64,) and r.min() >= 512 and r.max() <= 4096
    r = config_lengths(3, np.random.default_rng(3))["kv_lens"]
    assert r.shape == (128,) and (r == 32768).sum() == 4
    short = r[r != 32768]
    assert short.min() >= 16 and short.max() <= 8192 and 300 < np.median(short) < 800
    c4 = config_lengths(4, np.random.default_rng(4))
    assert c4["prefix_len"] == 16384 and c4["suffix_lens"].min() >= 256
    assert c4["suffix_lens"].max() <= 1024
    c5 = config_lengths(5, np.random.default_rng(5))
    assert (c5["kv_lens"] == 4608).all() and (c5["qo_lens"] == 512).all()


def test_normal_statistics():
    wl = make_workload([4096], 8, 8, "bf16", 0)
    v = OA.upcast(wl.pool, "bf16")
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01
