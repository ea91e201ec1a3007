"""Pins for the oracle's expert feed-forward and combine.

Sources: "Tensor parallelism for inference", "Packed strategies" (packed
gate/up weight [E, hidden, 2I], applied as hidden @ W, split with the gate
half first); "Expert parallelism", "Token dispatch" (routing-weighted sum of
the experts' outputs); SwiGLU per the benchmark definition.

Each test pins something a plausible mistake would break:
  * a worked example with one-hot inputs (orientation of both weights,
    gate/up order, the SiLU formula) against math.exp;
  * scaling laws that hold exactly in floating point (up half and down
    weight are linear; the gate half is not);
  * zero rows give zero outputs;
  * identical experts make the output independent of routing;
  * linearity of the combine over the k slots;
  * the masked dense formulation ("all_reduce" expert parallelism) via
    numpy matmul, and the large-gate limit where SiLU is the identity;
  * splitting experts into blocks and summing the masked block outputs
    (expert-parallel ranks) reproduces the whole layer;
  * bf16 and f32 inputs holding the same values give identical results.
"""
import math

import numpy as np
import pytest

import oracle
from workloads import bf16_bits, make_custom, to_float32


def silu(z):
    return z / (1.0 + math.exp(-z))


def small_case(T=6, d=8, E=4, k=2, I=5, seed=0):
    inp = make_custom(T=T, d=d, E=E, k=k, I=I, dtype="f32", seed=seed, logits="normal")
    # larger weights than the workloads use, so that SiLU is well inside its nonlinear range
    return inp.x, inp.logits, inp.w_gate_up * 50, inp.w_down * 50


def test_worked_example_one_hot():
    # d = 2, I = 1, E = 2.  Token 0 is (0, 1), token 1 is (1, 0).
    x = np.array([[0.0, 1.0], [1.0, 0.0]], dtype=np.float32)
    wgu = np.array([[[5.0, 7.0], [2.0, 3.0]],       # expert 0: rows c, columns (gate, up)
                    [[1.0, -1.0], [-2.0, 4.0]]],    # expert 1
                   dtype=np.float32)
    wd = np.array([[[0.5, -1.0]], [[2.0, 0.25]]], dtype=np.float32)   # [E, I=1, d=2]
    idx = np.array([[0], [1]], dtype=np.int32)
    w = np.array([[1.0], [1.0]])
    out = oracle.moe_tokens(x, idx, w, wgu, wd)
    # token 0 through expert 0: gate = W[0][1][0] = 2, up = W[0][1][1] = 3
    h0 = silu(2.0) * 3.0
    # token 1 through expert 1: gate = W[1][0][0] = 1, up = W[1][0][1] = -1
    h1 = silu(1.0) * -1.0
    ref = np.array([[h0 * 0.5, h0 * -1.0], [h1 * 2.0, h1 * 0.25]])
    np.testing.assert_allclose(out, ref, rtol=1e-15, atol=0)
    # both tokens through both experts with weights 0.75 / 0.25
    idx2 = np.array([[0, 1], [1, 0]], dtype=np.int32)
    w2 = np.array([[0.75, 0.25], [0.75, 0.25]])
    out2 = oracle.moe_tokens(x, idx2, w2, wgu, wd)
    h0b = silu(-2.0) * 4.0     # token 0 through expert 1
    h1b = silu(5.0) * 7.0      # token 1 through expert 0
    ref2 = np.array([[0.75 * h0 * 0.5 + 0.25 * h0b * 2.0, 0.75 * h0 * -1.0 + 0.25 * h0b * 0.25],
                     [0.75 * h1 * 2.0 + 0.25 * h1b * 0.5, 0.75 * h1 * 0.25 + 0.25 * h1b * -1.0]])
    np.testing.assert_allclose(out2, ref2, rtol=1e-15, atol=1e-300)


def test_scaling_up_half_and_down_is_exact_gate_is_not():
    x, logits, wgu, wd = small_case()
    idx, w = oracle.route(logits, 2)
    base = oracle.moe_tokens(x, idx, w, wgu, wd)
    I = wd.shape[1]
    wgu_up2 = wgu.copy()
    wgu_up2[:, :, I:] *= 2
    assert np.array_equal(oracle.moe_tokens(x, idx, w, wgu_up2, wd), 2 * base)
    assert np.array_equal(oracle.moe_tokens(x, idx, w, wgu, wd * 2), 2 * base)
    wgu_g2 = wgu.copy()
    wgu_g2[:, :, :I] *= 2
    out_g2 = oracle.moe_tokens(x, idx, w, wgu_g2, wd)
    assert not np.allclose(out_g2, 2 * base, rtol=1e-3)


def test_zero_row_gives_zero_output():
    x, logits, wgu, wd = small_case()
    x = x.copy()
    x[2] = 0.0
    idx, w = oracle.route(logits, 2)
    out = oracle.moe_tokens(x, idx, w, wgu, wd)
    assert np.all(out[2] == 0.0)
    assert np.all(np.abs(out[[0, 1, 3]]).sum(axis=1) > 0)


def test_identical_experts_ignore_routing():
    x, logits, wgu, wd = small_case(E=5)
    wgu = np.repeat(wgu[:1], 5, axis=0)
    wd = np.repeat(wd[:1], 5, axis=0)
    single = oracle.moe_tokens(x, np.zeros((x.shape[0], 1), np.int32), np.ones((x.shape[0], 1)), wgu, wd)
    for k in (1, 2, 5):
        idx, w = oracle.route(logits, k)
        out = oracle.moe_tokens(x, idx, w, wgu, wd)
        np.testing.assert_allclose(out, single, rtol=1e-13, atol=1e-15)


def test_k_equals_e_uniform_is_mean_of_experts():
    x, _, wgu, wd = small_case(E=4)
    T = x.shape[0]
    idx, w = oracle.route(np.zeros((T, 4), np.float32), 4)
    assert np.all(w == 0.25)
    out = oracle.moe_tokens(x, idx, w, wgu, wd)
    each = [oracle.moe_tokens(x, np.full((T, 1), e, np.int32), np.ones((T, 1)), wgu, wd) for e in range(4)]
    np.testing.assert_allclose(out, sum(each) / 4, rtol=1e-13, atol=1e-15)


def test_combine_is_linear_over_slots():
    x, logits, wgu, wd = small_case()
    T = x.shape[0]
    idx, w = oracle.route(logits, 2)
    out, y = oracle.moe_tokens(x, idx, w, wgu, wd, want_y=True)
    for j in range(2):
        yj = oracle.moe_tokens(x, idx[:, j:j + 1], np.ones((T, 1)), wgu, wd)
        assert np.array_equal(y[:, j], yj)
    np.testing.assert_allclose(out, w[:, :1] * y[:, 0] + w[:, 1:] * y[:, 1], rtol=1e-15, atol=1e-300)


def dense_masked(x, idx, w, wgu, wd):
    """Every expert on every token, weighted by a dense [T, E] matrix that is
    zero off the selected experts (the masked "all_reduce" formulation)."""
    xd = to_float32(x).astype(np.float64)
    wgu = to_float32(wgu).astype(np.float64)
    wd = to_float32(wd).astype(np.float64)
    T = xd.shape[0]
    E, _, two_i = wgu.shape
    I = two_i // 2
    M = np.zeros((T, E))
    for t in range(T):
        for j in range(idx.shape[1]):
            if idx[t, j] >= 0:
                M[t, idx[t, j]] += w[t, j]
    out = np.zeros_like(xd)
    for e in range(E):
        gu = xd @ wgu[e]
        g, u = gu[:, :I], gu[:, I:]
        out += M[:, e:e + 1] * (((g / (1 + np.exp(-g))) * u) @ wd[e])
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dense_masked_formulation(dtype):
    inp = make_custom(T=40, d=64, E=8, k=3, I=48, dtype=dtype, seed=31, logits="normal")
    idx, w = oracle.route(inp.logits, 3)
    out = oracle.moe_tokens(inp.x, idx, w, inp.w_gate_up, inp.w_down)
    ref = dense_masked(inp.x, idx, w, inp.w_gate_up, inp.w_down)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-14)


def test_large_gate_limit_is_bilinear():
    # gate pre-activations >= 40: silu(g) == g in double, so the expert is
    # ((x Wg) * (x Wu)) Wd, a plain matmul chain
    rng = np.random.default_rng(41)
    T, d, I, E = 5, 6, 4, 2
    x = np.abs(rng.standard_normal((T, d))).astype(np.float32) + 1
    wgu = rng.standard_normal((E, d, 2 * I)).astype(np.float32)
    wgu[:, :, :I] = np.abs(wgu[:, :, :I]) + 10.0
    wd = rng.standard_normal((E, I, d)).astype(np.float32)
    idx = np.array([[0, 1]] * T, dtype=np.int32)
    w = np.array([[0.6, 0.4]] * T)
    out = oracle.moe_tokens(x, idx, w, wgu, wd)
    xd = x.astype(np.float64)
    ref = np.zeros((T, d))
    for j, e in enumerate((0, 1)):
        g = xd @ wgu[e, :, :I].astype(np.float64)
        assert g.min() >= 40
        u = xd @ wgu[e, :, I:].astype(np.float64)
        ref += w[:, j:j + 1] * ((g * u) @ wd[e].astype(np.float64))
    np.testing.assert_allclose(out, ref, rtol=1e-12)


def test_expert_blocks_sum_to_whole_layer():
    # ranks r = 0..3 each own experts [4r, 4r+4) ("Expert parallelism",
    # "How the sizes combine"); pairs on other ranks are masked with -1
    inp = make_custom(T=24, d=32, E=16, k=4, I=24, dtype="bf16", seed=43, logits="uniform")
    idx, w = oracle.route(inp.logits, 4)
    full = oracle.moe_tokens(inp.x, idx, w, inp.w_gate_up, inp.w_down)
    total = np.zeros_like(full)
    for r in range(4):
        local = np.where((idx >= 4 * r) & (idx < 4 * r + 4), idx, -1).astype(np.int32)
        total += oracle.moe_tokens(inp.x, local, w, inp.w_gate_up, inp.w_down)
    np.testing.assert_allclose(total, full, rtol=1e-13, atol=1e-16)


def test_bf16_and_f32_storage_agree():
    inp = make_custom(T=10, d=16, E=3, k=2, I=8, dtype="bf16", seed=47, logits="normal")
    idx, w = oracle.route(inp.logits, 2)
    a = oracle.moe_tokens(inp.x, idx, w, inp.w_gate_up, inp.w_down)
    b = oracle.moe_tokens(to_float32(inp.x), idx, w, to_float32(inp.w_gate_up), to_float32(inp.w_down))
    assert np.array_equal(a, b)
    # the decode is exact: round trip through bf16_bits is the identity on bf16 values
    assert np.array_equal(bf16_bits(to_float32(inp.x)), inp.x)


def test_thread_count_and_token_order_do_not_matter():
    inp = make_custom(T=37, d=16, E=5, k=2, I=8, dtype="bf16", seed=53, logits="normal")
    idx, w = oracle.route(inp.logits, 2)
    a = oracle.moe_tokens(inp.x, idx, w, inp.w_gate_up, inp.w_down, nthreads=1)
    b = oracle.moe_tokens(inp.x, idx, w, inp.w_gate_up, inp.w_down, nthreads=7)
    assert np.array_equal(a, b)
    sel = np.array([30, 2, 2, 17])
    c = oracle.moe_tokens(inp.x, idx, w, inp.w_gate_up, inp.w_down, tokens=sel)
    assert np.array_equal(c, a[sel])


def test_masked_pairs_contribute_nothing():
    x, logits, wgu, wd = small_case()
    idx, w = oracle.route(logits, 2)
    masked = idx.copy()
    masked[:, 1] = -1
    out = oracle.moe_tokens(x, masked, w, wgu, wd)
    only0 = oracle.moe_tokens(x, idx[:, :1], w[:, :1], wgu, wd)
    assert np.array_equal(out, only0)
    allmasked = oracle.moe_tokens(x, np.full_like(idx, -1), w, wgu, wd)
    assert np.all(allmasked == 0)


def test_forward_wires_the_steps():
    inp = make_custom(T=20, d=16, E=6, k=2, I=8, dtype="bf16", seed=59, logits="normal_bias")
    res = oracle.forward(inp.x, inp.w_gate_up, inp.w_down, 2, logits=inp.logits, want_y=True)
    idx, w = oracle.route(inp.logits, 2)
    assert np.array_equal(res["idx"], idx)
    off, pr, rt = oracle.dispatch(idx.reshape(-1), 2, 6)
    assert np.array_equal(res["offsets"], off) and np.array_equal(res["pair_row"], pr)
    assert np.array_equal(res["row_token"], rt)
    np.testing.assert_array_equal(res["out"], oracle.moe_tokens(inp.x, idx, w, inp.w_gate_up, inp.w_down))


def test_combine_step_matches_layer():
    # rows placed in expert order by the dispatch, then combined on their own,
    # give the layer's output
    inp = make_custom(T=30, d=16, E=5, k=3, I=8, dtype="f32", seed=61, logits="normal")
    res = oracle.forward(inp.x, inp.w_gate_up, inp.w_down, 3, logits=inp.logits, want_y=True)
    P = 30 * 3
    y_perm = np.zeros((P, 16), dtype=np.float32)
    pr = res["pair_row"]
    for p in range(P):
        y_perm[pr[p]] = res["y_pair"][p // 3, p % 3]
    out = oracle.combine(y_perm, pr, res["w"], 30, 3)
    ref = oracle.combine(y_perm.astype(np.float64).astype(np.float32), pr, res["w"], 30, 3)
    assert np.array_equal(out, ref)
    # y_perm holds the expert outputs rounded to float32; the layer keeps doubles
    np.testing.assert_allclose(out, res["out"], rtol=1e-6, atol=1e-9)
