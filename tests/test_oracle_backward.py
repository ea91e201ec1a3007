"""Pins of the oracle's backward pass (``oracle.backward``) that do not re-type it.

- Central finite differences of L = <dout, out>, with the forward taken from
  the oracle's C forward (independent code), on tiny cases whose inputs and
  steps are exact in float32, for every input that has a gradient: x, the
  gate/up and down weights, the routing weights and the logits.
- Exact consequences of degree-one homogeneity (Euler): the output is linear
  in the down weights, in the up half of the gate/up weights and in the
  routing weights, so <dW, W> = <dout, out> for each of them.
- Invariants: the renormalised softmax ignores a common shift of a token's
  logits, so each token's logit gradient sums to zero; k = 1 gives weight 1
  whatever the logits, so no logit gradient; masked pairs and experts without
  rows get exactly zero.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def grid(rng, shape, step, lim):
    """float32 values on a grid of ``step`` within +-lim (every value and
    every value +- a smaller power of two is exact in float32)."""
    return (np.round(rng.uniform(-lim, lim, size=shape) / step) * step).astype(np.float32)


def tiny_case(seed, T=5, d=8, E=3, k=2, I=4):
    rng = np.random.default_rng(seed)
    x = grid(rng, (T, d), 2.0 ** -4, 2.0)
    wgu = grid(rng, (E, d, 2 * I), 2.0 ** -8, 0.5)
    wd = grid(rng, (E, I, d), 2.0 ** -8, 0.5)
    # logits spaced at least 2^-3 apart within a token: no selection changes
    # under the 2^-12 steps below
    logits = np.stack([rng.permutation(E).astype(np.float32) * 0.25 + grid(rng, (1,), 2.0 ** -4, 0.5)[0]
                       for _ in range(T)])
    dout = rng.normal(size=(T, d))
    return x, wgu, wd, logits.astype(np.float32), dout


def loss(x, wgu, wd, k, dout, logits=None, idx=None, w=None):
    if logits is not None:
        idx, w = oracle.route(logits, k)
    out = oracle.moe_tokens(x, idx, w, wgu, wd, nthreads=1)
    return float(np.sum(dout * out))


def fd_check(array, grad, f, h, rtol):
    """Central differences over every entry of ``array`` (perturbed in place)."""
    num = np.zeros(array.shape)
    flat = array.reshape(-1)
    for i in range(flat.size):
        v = flat[i]
        flat[i] = v + h
        lp = f()
        flat[i] = v - h
        lm = f()
        flat[i] = v
        num.reshape(-1)[i] = (lp - lm) / (2 * h)
    scale = np.max(np.abs(num))
    assert scale > 0
    err = np.max(np.abs(num - grad))
    assert err <= rtol * scale, (err, scale)


@pytest.mark.parametrize("seed", [1, 2])
def test_finite_differences_all_inputs(seed):
    x, wgu, wd, logits, dout = tiny_case(seed)
    k = 2
    g = oracle.backward(x, wgu, wd, k, dout, logits=logits)
    f = lambda: loss(x, wgu, wd, k, dout, logits=logits)
    h = 2.0 ** -12
    fd_check(x, g["dx"], f, h, 1e-5)
    fd_check(wgu, g["dw_gate_up"], f, h, 1e-5)
    fd_check(wd, g["dw_down"], f, h, 1e-8)      # linear: differences are exact up to rounding
    fd_check(logits, g["dlogits"], f, h, 1e-5)


def test_finite_differences_routing_weights_given_pairs():
    x, wgu, wd, _, dout = tiny_case(3, T=6, E=4, k=3)
    rng = np.random.default_rng(4)
    idx = np.stack([rng.permutation(4)[:3] for _ in range(6)]).astype(np.int32)
    idx[2, 1] = -1  # a masked pair
    w = rng.uniform(0.1, 1.0, size=(6, 3))
    g = oracle.backward(x, wgu, wd, 3, dout, pair_expert=idx, pair_w=w)
    f = lambda: loss(x, wgu, wd, 3, dout, idx=idx, w=w)
    fd_check(w, g["dw"], f, 2.0 ** -10, 1e-8)   # out is linear in the weights
    assert g["dw"][2, 1] == 0.0
    fd_check(x, g["dx"], f, 2.0 ** -12, 1e-5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_degree_one_homogeneity(dtype):
    inp = workloads.make_custom(T=50, d=32, E=6, k=2, I=24, dtype=dtype, seed=7, logits="normal")
    dout = np.random.default_rng(8).normal(size=(50, 32))
    g = oracle.backward(inp.x, inp.w_gate_up, inp.w_down, 2, dout, logits=inp.logits)
    out = oracle.forward(inp.x, inp.w_gate_up, inp.w_down, 2, logits=inp.logits)["out"]
    ref = float(np.sum(dout * out))
    wgu = workloads.to_float32(inp.w_gate_up).astype(np.float64)
    wd = workloads.to_float32(inp.w_down).astype(np.float64)
    I = 24
    assert np.isclose(np.sum(g["dw_down"] * wd), ref, rtol=1e-10, atol=0)
    assert np.isclose(np.sum(g["dw_gate_up"][:, :, I:] * wgu[:, :, I:]), ref, rtol=1e-10, atol=0)
    assert np.isclose(np.sum(g["dw"] * g["w"]), ref, rtol=1e-10, atol=0)
    # the gate half is not homogeneous of degree one (SiLU): the same sum differs
    assert not np.isclose(np.sum(g["dw_gate_up"][:, :, :I] * wgu[:, :, :I]), ref, rtol=1e-3)


def test_logit_gradient_invariants():
    inp = workloads.make_custom(T=40, d=16, E=8, k=3, I=16, dtype="f32", seed=9, logits="normal")
    dout = np.random.default_rng(10).normal(size=(40, 16))
    g = oracle.backward(inp.x, inp.w_gate_up, inp.w_down, 3, dout, logits=inp.logits)
    assert np.max(np.abs(g["dlogits"].sum(axis=1))) < 1e-12
    # experts not selected get nothing
    sel = np.zeros((40, 8), dtype=bool)
    np.put_along_axis(sel, g["idx"].astype(np.int64), True, axis=1)
    assert np.all(g["dlogits"][~sel] == 0)
    g1 = oracle.backward(inp.x, inp.w_gate_up, inp.w_down, 1, dout, logits=inp.logits)
    assert np.all(g1["dlogits"] == 0)


def test_empty_expert_and_zero_upstream():
    inp = workloads.make_custom(T=30, d=16, E=5, k=1, I=8, dtype="f32", seed=11, logits="normal")
    inp.logits[:, 3] -= 100.0  # expert 3 never selected
    dout = np.random.default_rng(12).normal(size=(30, 16))
    g = oracle.backward(inp.x, inp.w_gate_up, inp.w_down, 1, dout, logits=inp.logits)
    assert np.all(g["dw_gate_up"][3] == 0) and np.all(g["dw_down"][3] == 0)
    z = oracle.backward(inp.x, inp.w_gate_up, inp.w_down, 1, np.zeros((30, 16)), logits=inp.logits)
    for key in ("dx", "dw_gate_up", "dw_down", "dw", "dlogits"):
        assert np.all(z[key] == 0), key
