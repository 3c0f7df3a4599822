"""Pins for the oracle's routing and packing (CPU only)."""

import json
import os

import numpy as np
import pytest

import oracle
from oracle.routing import DEV_CAPACITY, DEV_ID_RANGE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _golden():
    with open(GOLDEN, encoding="utf-8") as f:
        return json.load(f)


def test_worked_example_unaligned():
    g = _golden()
    ids = np.array(g["topk_ids"], dtype=np.int32)
    r = oracle.route(ids, g["E"], "contiguous", align=1)
    assert r["counts"].tolist() == g["expected_counts"]
    u = g["unaligned"]
    assert r["m_packed"] == u["m_packed"]
    assert r["m_indices"][:u["m_packed"]].tolist() == u["m_indices"]
    assert r["output_index"].tolist() == u["output_index"]
    x = np.array(g["x"], dtype=np.int64)
    packed = oracle.pack_rows(x, r["output_index"], r["rows_cap"])
    assert np.array_equal(packed[:10], x[u["packed_token_of_row"]])


def test_worked_example_aligned_128():
    g = _golden()
    ids = np.array(g["topk_ids"], dtype=np.int32)
    r = oracle.route(ids, g["E"], "contiguous", align=128)
    a = g["aligned128"]
    assert r["counts"].tolist() == g["expected_counts"]
    assert r["m_packed"] == a["m_packed"]
    assert r["seg_offsets"][:4].tolist() == a["segment_starts"]
    exp_m = []
    for e, n in a["m_indices_runs"]:
        exp_m += [e] * n
    assert r["m_indices"][:a["m_packed"]].tolist() == exp_m
    assert (r["m_indices"][a["m_packed"]:] == -1).all()
    assert r["output_index"].tolist() == a["output_index"]
    x = np.array(g["x"], dtype=np.int64)
    packed = oracle.pack_rows(x, r["output_index"], r["rows_cap"], fill=-999)
    for start, toks in a["valid_rows"].items():
        s = int(start)
        assert np.array_equal(packed[s:s + len(toks)], x[toks])
        assert (packed[s + len(toks):s + 128] == -999).all()  # padding rows never written


def _check_invariants(ids, E, layout, align, max_m, r):
    flat = ids.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    oi = r["output_index"].reshape(-1)
    # independent formulation: stable sort of valid assignments by expert id
    order = np.argsort(np.where(valid, flat, E + 1), kind="stable")
    rank = np.empty(flat.size, dtype=np.int64)
    seen = {}
    for i in order:
        if not valid[i]:
            continue
        e = flat[i]
        rank[i] = seen.get(e, 0)
        seen[e] = rank[i] + 1
    for i in range(flat.size):
        if not valid[i]:
            assert oi[i] == -1
            continue
        e = flat[i]
        if layout == "masked":
            if rank[i] >= max_m:
                assert oi[i] == -1
                continue
            assert oi[i] == e * max_m + rank[i]
        else:
            assert oi[i] == r["seg_offsets"][e] + rank[i]
        assert r["m_indices"][oi[i]] == e
    used = oi[oi >= 0]
    assert np.unique(used).size == used.size
    if layout == "contiguous":
        so = r["seg_offsets"]
        assert (np.diff(so) >= 0).all() and (so % align == 0).all()
        tot = np.bincount(flat[valid], minlength=E)
        assert np.array_equal(r["counts"], tot)
        assert np.array_equal(np.diff(so), -(-tot // align) * align)
        assert r["m_packed"] <= r["rows_cap"]


@pytest.mark.parametrize("seed", range(4))
def test_routing_invariants_random(seed):
    rng = np.random.default_rng(seed)
    T, k, E = int(rng.integers(1, 60)), int(rng.integers(1, 5)), int(rng.integers(1, 20))
    ids = rng.integers(-2, E + 2, size=(T, k)).astype(np.int32)
    r = oracle.route(ids, E, "contiguous", align=16)
    _check_invariants(ids, E, "contiguous", 16, 0, r)
    assert bool(r["status"] & DEV_ID_RANGE) == bool((ids >= E).any())
    rm = oracle.route(ids, E, "masked", max_m=3)
    _check_invariants(ids, E, "masked", 0, 3, rm)
    cnt = np.bincount(ids[(ids >= 0) & (ids < E)], minlength=E)
    assert bool(rm["status"] & DEV_CAPACITY) == bool((cnt > 3).any())
    assert np.array_equal(rm["counts"], np.minimum(cnt, 3))


def test_routing_empty_and_all_invalid():
    ids = np.full((4, 2), -1, dtype=np.int32)
    r = oracle.route(ids, 8, "contiguous", align=128)
    assert r["m_packed"] == 0 and (r["counts"] == 0).all() and (r["output_index"] == -1).all()
    assert (r["m_indices"] == -1).all()
    r2 = oracle.route(np.zeros((0, 2), np.int32), 8, "contiguous", align=128)
    assert r2["m_packed"] == 0


def test_packed_rows_cap_is_an_upper_bound():
    rng = np.random.default_rng(7)
    for _ in range(50):
        T, k, E = int(rng.integers(1, 40)), int(rng.integers(1, 9)), int(rng.integers(1, 300))
        ids = rng.integers(0, E, size=(T, k))
        r = oracle.route(ids, E, "contiguous", align=128)
        assert r["m_packed"] <= oracle.packed_rows_cap(T, k, E, 128)
