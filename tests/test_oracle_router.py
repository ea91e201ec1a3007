"""Pins for the oracle's router projection (logits = x @ W_r^T, W_r [E, d]).

The pages name the router module (a model's gate linear layer, mlp.gate /
mlp.router, "Expert parallelism") but print no formula; the plainest reading
is a bias-free linear layer whose weight is [E, d].  These tests pin the
oracle to what that definition fixes independently of how it is computed: a
brute-force loop, one-hot rows selecting weight columns, exact power-of-two
scaling, linearity over a split of the hidden dimension, and the bfloat16
inputs expanding exactly.
"""
import numpy as np

import oracle
import workloads


def test_matches_brute_force_loop():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(5, 7)).astype(np.float32)
    w = rng.normal(size=(4, 7)).astype(np.float32)
    got = oracle.router_logits(x, w)
    for t in range(5):
        for e in range(4):
            ref = 0.0
            for c in range(7):
                ref += float(x[t, c]) * float(w[e, c])
            assert abs(got[t, e] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_one_hot_rows_pick_weight_columns():
    rng = np.random.default_rng(4)
    w = rng.normal(size=(6, 32)).astype(np.float32)
    x = np.zeros((32, 32), dtype=np.float32)
    x[np.arange(32), np.arange(32)] = 1.0
    # token c is the unit vector along hidden unit c: its logits are column c of W_r
    assert np.array_equal(oracle.router_logits(x, w), w.T.astype(np.float64))


def test_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(9, 64)).astype(np.float32)
    w = rng.normal(size=(8, 64)).astype(np.float32)
    base = oracle.router_logits(x, w)
    assert np.array_equal(oracle.router_logits(x * np.float32(4), w), 4 * base)
    assert np.array_equal(oracle.router_logits(x, w * np.float32(0.5)), 0.5 * base)


def test_split_of_hidden_dimension_adds():
    rng = np.random.default_rng(6)
    x = rng.normal(size=(10, 48)).astype(np.float32)
    w = rng.normal(size=(5, 48)).astype(np.float32)
    full = oracle.router_logits(x, w)
    parts = oracle.router_logits(x[:, :20], w[:, :20]) + oracle.router_logits(x[:, 20:], w[:, 20:])
    assert np.allclose(full, parts, rtol=0, atol=1e-12)


def test_bf16_inputs_expand_exactly():
    rng = np.random.default_rng(8)
    xf = rng.normal(size=(6, 16)).astype(np.float32)
    wf = rng.normal(size=(3, 16)).astype(np.float32)
    xb, wb = workloads.bf16_bits(xf), workloads.bf16_bits(wf)
    # the same values as float32 arrays give the same float64 logits
    xe = (xb.astype(np.uint32) << 16).view(np.float32)
    we = (wb.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(oracle.router_logits(xb, wb), oracle.router_logits(xe, we))


def test_zero_row_gives_zero_logits_and_index_order():
    w = np.ones((4, 8), dtype=np.float32)
    x = np.zeros((2, 8), dtype=np.float32)
    logits = oracle.router_logits(x, w)
    assert np.all(logits == 0)
    # all-equal logits: the lower expert indices win (the routing rule)
    idx, wts = oracle.route(logits.astype(np.float32), 2)
    assert idx.tolist() == [[0, 1], [0, 1]] and np.all(wts == 0.5)
