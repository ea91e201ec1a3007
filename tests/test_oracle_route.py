"""Pins for the oracle's routing step (top-k selection + renormalised softmax).

The pages ("Expert parallelism", "Adding an implementation") fix only the
outputs: per token, the selected experts' ids and routing weights.  The rule
is softmax top-k with ties to the lower expert index.  These tests pin the
oracle to brute force and to closed forms that do not depend on how the
oracle computes: a plain sort, the two-expert logistic form, equal logits,
and invariances.
"""
import math

import numpy as np
import pytest

import oracle


def brute_force_topk(row, k):
    # a plain sort by (larger logit first, then lower index)
    return sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:k]


def test_selection_matches_sort_with_ties():
    rng = np.random.default_rng(1234)
    values = np.array([-1.0, 0.0, -0.0, 1.0, 0.5, -0.5], dtype=np.float32)
    n_cases = 0
    for _ in range(600):
        T = int(rng.integers(1, 17))
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        logits = values[rng.integers(0, len(values), size=(T, E))]
        idx, _ = oracle.route(logits, k)
        for t in range(T):
            assert list(idx[t]) == brute_force_topk(logits[t], k), (logits[t], k)
            n_cases += 1
    assert n_cases > 1000


def test_selection_matches_sort_random_wide():
    rng = np.random.default_rng(7)
    for E, k in [(16, 2), (128, 4), (256, 8), (256, 256), (37, 5)]:
        logits = rng.standard_normal((32, E)).astype(np.float32)
        # force some exact ties
        logits[:, E // 2] = logits[:, 0]
        idx, _ = oracle.route(logits, k)
        for t in range(32):
            assert list(idx[t]) == brute_force_topk(logits[t], k)


def test_negative_zero_ties_positive_zero():
    logits = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], dtype=np.float32)
    idx, w = oracle.route(logits, 2)
    assert idx.tolist() == [[0, 1], [0, 1]]
    assert np.all(w == 0.5)


def test_all_equal_logits():
    for E in (1, 3, 8, 128):
        for k in sorted({1, min(2, E), max(1, E // 2), E}):
            logits = np.full((5, E), 0.25, dtype=np.float32)
            idx, w = oracle.route(logits, k)
            assert idx.tolist() == [list(range(k))] * 5
            np.testing.assert_allclose(w, 1.0 / k, rtol=1e-15, atol=0)


def test_k1_weight_is_exactly_one():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((200, 16)).astype(np.float32) * 10
    _, w = oracle.route(logits, 1)
    assert np.all(w == 1.0)


def test_k2_is_logistic_of_logit_gap():
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((300, 16)).astype(np.float32) * 3
    idx, w = oracle.route(logits, 2)
    for t in range(300):
        l0 = float(logits[t, idx[t, 0]])
        l1 = float(logits[t, idx[t, 1]])
        w0 = 1.0 / (1.0 + math.exp(l1 - l0))
        assert abs(w[t, 0] - w0) <= 1e-15
        assert abs(w[t, 1] - (1.0 - w0)) <= 1e-15


def test_worked_example():
    # logits (1, 2, 3, 0), k = 2: experts 2 then 1, weights e/(e+1) and 1/(e+1)
    idx, w = oracle.route(np.array([[1.0, 2.0, 3.0, 0.0]], dtype=np.float32), 2)
    assert idx.tolist() == [[2, 1]]
    assert abs(w[0, 0] - math.e / (math.e + 1)) < 1e-15
    assert abs(w[0, 1] - 1 / (math.e + 1)) < 1e-15


def test_weights_are_softmax_over_selected():
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((100, 32)).astype(np.float32) * 4
    for k in (1, 3, 8, 32):
        idx, w = oracle.route(logits, k)
        for t in range(0, 100, 7):
            sel = [float(logits[t, e]) for e in idx[t]]
            z = sum(math.exp(v) for v in sel)
            ref = [math.exp(v) / z for v in sel]
            assert max(abs(a - b) for a, b in zip(w[t], ref)) < 1e-14


def test_weights_sum_to_one_and_descend():
    rng = np.random.default_rng(13)
    logits = rng.standard_normal((500, 64)).astype(np.float32) * 5
    for k in (2, 4, 16):
        _, w = oracle.route(logits, k)
        assert np.max(np.abs(w.sum(axis=1) - 1.0)) < 1e-14
        assert np.all(np.diff(w, axis=1) <= 0)
        assert np.all(w > 0)


def test_shift_invariance():
    rng = np.random.default_rng(17)
    # logits on a 2^-10 grid within +-8: adding an integer <= 64 is exact in float32
    logits = (rng.integers(-8 * 1024, 8 * 1024, size=(64, 16)) / 1024.0).astype(np.float32)
    idx0, w0 = oracle.route(logits, 4)
    for shift in (-64, -3, 1, 64):
        shifted = (logits + np.float32(shift)).astype(np.float32)
        assert np.array_equal(shifted - np.float32(shift), logits)
        idx1, w1 = oracle.route(shifted, 4)
        assert np.array_equal(idx0, idx1)
        assert np.max(np.abs(w0 - w1)) < 1e-12


def test_permuting_experts_permutes_selection():
    rng = np.random.default_rng(19)
    logits = rng.standard_normal((50, 12)).astype(np.float32)  # no ties (continuous draw)
    perm = rng.permutation(12)
    idx0, w0 = oracle.route(logits, 3)
    idx1, w1 = oracle.route(logits[:, perm], 3)
    # column c of the permuted logits is expert perm[c]
    assert np.array_equal(perm[idx1], idx0)
    assert np.max(np.abs(w0 - w1)) < 1e-15


def test_invalid_arguments():
    logits = np.zeros((2, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.route(logits, 5)
    with pytest.raises(ValueError):
        oracle.route(logits, 0)


def test_empty_batch():
    idx, w = oracle.route(np.zeros((0, 8), dtype=np.float32), 2)
    assert idx.shape == (0, 2) and w.shape == (0, 2)
