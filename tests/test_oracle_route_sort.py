"""Pins for the oracle's routing and sort (CPU only).

Routing follows the StepFun page's "Renormalize top-k" stage; the sort follows
the grouped-GEMM page's offs / m_indptr convention and the StepFun page's
expanded_idx_to_permuted_idx output. Each check ties the oracle to something
other than itself: a different library routine, brute force, a hand-worked
fixture or an invariant.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_logits(T, E, seed, integer=False):
    g = np.random.default_rng(seed)
    if integer:  # many exact ties
        return g.integers(-2, 3, size=(T, E)).astype(np.float32)
    return g.standard_normal((T, E), dtype=np.float32)


@pytest.mark.parametrize("T,E,k,integer", [(64, 8, 2, False), (64, 8, 2, True), (32, 256, 8, False),
                                           (40, 64, 8, True), (17, 5, 5, False), (9, 16, 1, True)])
def test_route_ids_match_stable_argsort(T, E, k, integer):
    lg = _rand_logits(T, E, 3, integer)
    ids, _ = O.route(lg, k)
    # numpy's stable sort of the negated logits keeps the lower id first on ties
    ref = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(ids, ref)


def test_route_negative_zero_ties_with_positive_zero():
    lg = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], dtype=np.float32)
    ids, w = O.route(lg, 2)
    np.testing.assert_array_equal(ids, [[0, 1], [0, 1]])
    np.testing.assert_array_equal(w, 0.5)


def test_route_selected_set_is_brute_force_max_sum():
    lg = _rand_logits(50, 7, 11)
    k = 3
    ids, _ = O.route(lg, k)
    for t in range(lg.shape[0]):
        best = max(itertools.combinations(range(7), k), key=lambda c: sum(float(lg[t, j]) for j in c))
        assert set(ids[t].tolist()) == set(best)
        # slots in descending logit order
        assert all(lg[t, ids[t, s]] >= lg[t, ids[t, s + 1]] for s in range(k - 1))


@pytest.mark.parametrize("E,k", [(8, 2), (256, 8), (64, 8), (6, 6)])
def test_route_weights_equal_full_softmax_renormalized(E, k):
    lg = _rand_logits(128, E, 5) * np.float32(3.0)
    ids, w = O.route(lg, k)
    p = torch.softmax(torch.from_numpy(lg.astype(np.float64)), dim=1).numpy()
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    ref = sel / sel.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, ref, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    if k == E:  # renormalising over every expert is the plain softmax
        np.testing.assert_allclose(np.take_along_axis(p, ids.astype(np.int64), 1), w, rtol=1e-12)


def test_route_k1_weight_is_exactly_one_and_large_logits_are_finite():
    lg = _rand_logits(33, 12, 2) * np.float32(1000.0)
    ids, w = O.route(lg, 1)
    np.testing.assert_array_equal(w, 1.0)
    np.testing.assert_array_equal(ids[:, 0], np.argmax(lg, axis=1))
    _, w4 = O.route(lg, 4)
    assert np.all(np.isfinite(w4))


def test_route_golden_closed_forms():
    with open(os.path.join(GOLDEN, "route_renormalize.json")) as f:
        fx = json.load(f)
    for c in fx["cases"]:
        lg = np.log(np.array(c["log_of"], dtype=np.float64)).astype(np.float32)[None, :]
        ids, w = O.route(lg, c["top_k"])
        assert ids[0].tolist() == c["ids"]
        ref = np.array(c["weights_num"], dtype=np.float64) / c["weights_den"]
        # the logits are float32 roundings of ln(a): relative error <= 2^-24 * |ln a| each
        np.testing.assert_allclose(w[0], ref, rtol=1e-6)


# --------------------------------------------------------------------------- sort
def _sort_ref_library(ids, E, L, off):
    flat = ids.reshape(-1).astype(np.int64)
    loc = flat - off
    ok = (flat >= 0) & (flat < E) & (loc >= 0) & (loc < L)
    key = np.where(ok, loc, L)
    order = np.argsort(key, kind="stable")
    n = int(ok.sum())
    counts = np.bincount(key[ok], minlength=L)
    return order[:n], np.cumsum(counts), ok


@pytest.mark.parametrize("T,k,E,L,off", [(32, 2, 8, 8, 0), (4096, 2, 8, 8, 0), (512, 8, 256, 32, 64),
                                         (300, 8, 64, 64, 0), (1, 1, 4, 4, 0), (0, 8, 256, 32, 64),
                                         (257, 3, 10, 3, 7)])
def test_sort_matches_library_stable_argsort(T, k, E, L, off):
    g = np.random.default_rng(T + k)
    ids = g.integers(-1, E + 2, size=(T, k)).astype(np.int32)  # includes invalid ids
    r = O.sort_routes(ids, E, L, off)
    p2e_ref, offs_ref, ok = _sort_ref_library(ids, E, L, off)
    np.testing.assert_array_equal(r["p2e"], p2e_ref)
    np.testing.assert_array_equal(r["offs"], offs_ref)
    np.testing.assert_array_equal(r["m_indptr"], np.concatenate([[0], offs_ref]))
    assert r["n_local"] == int(ok.sum())
    e2p = r["e2p"]
    # invariants: foreign -> -1; e2p is a bijection of local routes onto [0, n)
    np.testing.assert_array_equal(e2p < 0, ~ok)
    np.testing.assert_array_equal(np.sort(e2p[ok]), np.arange(r["n_local"]))
    np.testing.assert_array_equal(e2p[r["p2e"]], np.arange(r["n_local"]))
    loc = O.local_expert(ids, E, L, off)
    for e in range(L):
        s, f = (0 if e == 0 else r["offs"][e - 1]), r["offs"][e]
        members = r["p2e"][s:f]
        assert np.all(np.diff(members) > 0)      # stable: ascending expanded index
        assert np.all(loc[members] == e)


def test_sort_golden_worked_examples():
    with open(os.path.join(GOLDEN, "sort_worked.json")) as f:
        fx = json.load(f)
    for c in fx["cases"]:
        r = O.sort_routes(np.array(c["topk_ids"], dtype=np.int32), c["num_experts"],
                          c["num_local"], c["local_offset"])
        for key in ("offs", "m_indptr", "e2p", "p2e"):
            assert r[key].tolist() == c[key], key
        assert r["n_local"] == c["n_local"]
