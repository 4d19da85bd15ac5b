"""Pins for the oracle's routing, histogram/offsets and permutation."""
import json
import os

import numpy as np
import pytest
import scipy.special

from oracle import brute, routing
from workloads import generate, get_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_tiny_routing():
    d = json.load(open(os.path.join(GOLDEN, "layer_tiny.json")))
    lg = np.array(d["logits"], dtype=np.float32)
    for c in d["cases"]:
        ids, w = routing.route_topk(lg, c["k"], c["num_valid_rows"])
        assert ids.tolist() == c["ids"]
        np.testing.assert_allclose(w, np.array(c["w"]), rtol=1e-6, atol=0)
        off, sr, rp = routing.build_offsets(ids.reshape(-1), 2)
        assert off.tolist() == c["offsets"]
        assert sr.tolist() == c["sorted_rows"]
        assert rp.tolist() == c["row_pos"]


def test_ties_go_to_lower_expert_and_signed_zero():
    lg = np.array([[1.0, 3.0, 2.0, 3.0], [0.0, -0.0, 0.0, 5.0], [-0.0, 0.0, -1.0, -1.0]],
                  dtype=np.float32)
    ids, _ = routing.route_topk(lg, 2)
    assert ids.tolist() == [[1, 3], [3, 0], [0, 1]]


@pytest.mark.parametrize("T,E,k", [(33, 8, 2), (17, 5, 5), (40, 64, 8), (9, 130, 16), (50, 1, 1)])
@pytest.mark.parametrize("ties", [False, True])
def test_route_matches_full_sort(T, E, k, ties):
    rng = np.random.default_rng(T * 1000 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if ties:
        lg = np.round(lg * 2) / 2          # many equal logits
    for renorm in (True, False):
        ids, w = routing.route_topk(lg, k, renormalize=renorm)
        ids_b, w_b = brute.route_by_sort(lg, k, renormalize=renorm)
        assert np.array_equal(ids, ids_b)
        np.testing.assert_allclose(w, w_b, rtol=1e-6, atol=0)


def test_weights_closed_forms():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((100, 16)).astype(np.float32)
    ids, w = routing.route_topk(lg, 1)
    assert np.all(w == 1.0)                                  # softmax over one logit
    ids, w = routing.route_topk(lg, 4)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)                   # slots in descending logit order
    ids, w = routing.route_topk(lg, 4, renormalize=False)
    full = scipy.special.softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(full, ids, 1), rtol=1e-6)


def test_valid_rows_make_sentinels():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((10, 8)).astype(np.float32)
    ids, w = routing.route_topk(lg, 3, num_valid_rows=7)
    assert np.all(ids.reshape(-1)[7:] == 8) and np.all(w.reshape(-1)[7:] == 0)
    assert np.all(ids.reshape(-1)[:7] < 8)


def _check_permutation(ids, E, off, sr, rp):
    R = ids.size
    key = np.where((ids >= 0) & (ids < E), ids, E)
    assert sorted(sr.tolist()) == list(range(R))                     # bijection
    assert np.array_equal(rp[sr], np.arange(R))
    assert off[0] == 0 and np.all(np.diff(off) >= 0)
    assert off[E] == np.count_nonzero(key < E)
    for e in range(E):
        seg = sr[off[e]:off[e + 1]]
        assert np.all(key[seg] == e)
        assert np.all(np.diff(seg) > 0)                               # stable
    tail = sr[off[E]:]
    assert np.all(key[tail] == E) and np.all(np.diff(tail) > 0)


@pytest.mark.parametrize("R,E", [(1, 1), (100, 3), (1000, 8), (4096, 129), (5000, 1024)])
def test_offsets_and_permutation_brute(R, E):
    rng = np.random.default_rng(R + E)
    ids = rng.integers(0, E + 1, R)
    ids[rng.random(R) < 0.05] = -3                                    # invalid -> sentinel
    ids[rng.random(R) < 0.05] = E + 7
    off, sr, rp = routing.build_offsets(ids, E)
    # brute-force histogram with a Python loop
    cnt = [0] * E
    for i in ids.tolist():
        if 0 <= i < E:
            cnt[i] += 1
    acc, ref = 0, [0]
    for c in cnt:
        acc += c
        ref.append(acc)
    assert off.tolist() == ref
    _check_permutation(ids, E, off, sr, rp)


def test_empty_experts_and_all_sentinel():
    ids = np.array([2, 2, 2, 5, 5])
    off, sr, rp = routing.build_offsets(ids, 5)
    assert off.tolist() == [0, 0, 0, 3, 3, 3]
    assert sr.tolist() == [0, 1, 2, 3, 4]
    off, sr, rp = routing.build_offsets(np.full(7, 4), 4)
    assert off.tolist() == [0] * 5 and sr.tolist() == list(range(7))


def test_sentinel_sweep_offsets_match_pages():
    d = json.load(open(os.path.join(GOLDEN, "sentinel_sweep_offsets.json")))
    for c in d["cases"]:
        cfg = get_config(c["workload"])
        inp = generate(cfg, "cpu")
        ids, _ = routing.route_topk(inp.logits.numpy(), cfg.k, cfg.num_valid_rows)
        off, sr, rp = routing.build_offsets(ids.reshape(-1), cfg.E)
        assert cfg.R == 16384
        assert int(off[cfg.E]) == c["offsets_last"]
        assert np.count_nonzero(np.diff(off) > 0) == cfg.E          # every expert touched
        _check_permutation(ids.reshape(-1), cfg.E, off, sr, rp)
