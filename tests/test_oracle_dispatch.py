"""Pins for the oracle's dispatch step (pairs grouped by expert, stable).

"Expert parallelism", "Token dispatch": each (token, expert) pair goes to the
owner of its expert, which runs its experts on the rows it received.  On one
device: a stable grouping of pairs by expert.  Pinned against a plain
stable sort and against the invariants the grouping must satisfy.
"""
import numpy as np
import pytest

import oracle


def brute_force(pair_expert, k, E):
    P = len(pair_expert)
    order = sorted([p for p in range(P) if pair_expert[p] >= 0], key=lambda p: pair_expert[p])
    counts = [sum(1 for p in range(P) if pair_expert[p] == e) for e in range(E)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    pair_row = [-1] * P
    for r, p in enumerate(order):
        pair_row[p] = r
    return offsets, pair_row, [p // k for p in order]


def check_invariants(pe, k, E, offsets, pair_row, row_token):
    P = len(pe)
    live = pe >= 0
    assert offsets[0] == 0 and offsets[E] == int(live.sum())
    assert np.all(np.diff(offsets) >= 0)
    assert np.array_equal(np.diff(offsets), np.bincount(pe[live], minlength=E))
    # bijection of live pairs onto rows
    rows = pair_row[live]
    assert np.array_equal(np.sort(rows), np.arange(offsets[E]))
    assert np.all(pair_row[~live] == -1)
    # each row maps back to its token, and sits in its expert's block
    p_live = np.nonzero(live)[0]
    assert np.array_equal(row_token[rows], p_live // k)
    for e in range(E):
        ps = p_live[(rows >= offsets[e]) & (rows < offsets[e + 1])]
        assert np.all(pe[ps] == e)
        # stable: rows of an expert in increasing pair order
        assert np.all(np.diff(pair_row[ps]) > 0)


def test_brute_force_tiny():
    rng = np.random.default_rng(21)
    for _ in range(400):
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, 4))
        T = int(rng.integers(0, 12))
        pe = rng.integers(-1, E, size=T * k).astype(np.int32)
        offsets, pair_row, row_token = oracle.dispatch(pe, k, E)
        o2, pr2, rt2 = brute_force(pe.tolist(), k, E)
        assert offsets.tolist() == o2
        assert pair_row.tolist() == pr2
        assert row_token.tolist() == rt2
        check_invariants(pe, k, E, offsets, pair_row, row_token)


def test_invariants_large():
    rng = np.random.default_rng(22)
    for T, k, E in [(8192, 4, 128), (4096, 2, 16), (33, 3, 256)]:
        pe = rng.integers(0, E, size=T * k).astype(np.int32)
        pe[rng.random(T * k) < 0.1] = -1
        check_invariants(pe, k, E, *oracle.dispatch(pe, k, E))


def test_all_to_one_expert_and_all_masked():
    pe = np.full(40, 3, dtype=np.int32)
    offsets, pair_row, row_token = oracle.dispatch(pe, 2, 5)
    assert offsets.tolist() == [0, 0, 0, 0, 40, 40]
    assert pair_row.tolist() == list(range(40))
    assert row_token.tolist() == [p // 2 for p in range(40)]
    offsets, pair_row, row_token = oracle.dispatch(np.full(10, -1, dtype=np.int32), 1, 4)
    assert offsets.tolist() == [0] * 5 and np.all(pair_row == -1) and row_token.size == 0


def test_counts_sum_to_pairs_for_routed_batch():
    rng = np.random.default_rng(23)
    logits = rng.standard_normal((1000, 16)).astype(np.float32)
    idx, _ = oracle.route(logits, 2)
    offsets, _, _ = oracle.dispatch(idx.reshape(-1), 2, 16)
    assert offsets[-1] == 2000


def test_out_of_range_expert_is_an_error():
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([0, 4], dtype=np.int32), 1, 4)
    with pytest.raises(ValueError):
        oracle.dispatch(np.array([0, -2], dtype=np.int32), 1, 4)


def test_empty():
    offsets, pair_row, row_token = oracle.dispatch(np.zeros(0, dtype=np.int32), 2, 4)
    assert offsets.tolist() == [0] * 5 and pair_row.size == 0 and row_token.size == 0
