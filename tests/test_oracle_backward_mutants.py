"""The backward oracle's pins catch plausible mistakes in its chain rule.

Each case plants one mistake in a copy of ``oracle.backward`` (its source,
re-executed in the oracle module's namespace), swaps it in, and runs the
backward pins (finite differences against the oracle's independent C
forward, degree-one homogeneity, the logit-gradient invariants, exact zeros):
at least one pin must fail.  The real function is restored after.  CPU only.
"""
import inspect
import textwrap

import pytest

import oracle
import test_oracle_backward as pins

MUTANTS = {
    # SiLU's derivative loses its second term
    "silu_derivative_dropped_term": ("dg = dh * u * s * (1.0 + g * (1.0 - s))", "dg = dh * u * s"),
    # du misses the gate's value
    "du_without_gate": ("du = dh * g * s", "du = dh * s"),
    # the gate and up halves of the weight gradient swapped
    "swapped_gate_up_gradients": ("dwgu[e][:, :I] = xe.T @ dg\n        dwgu[e][:, I:] = xe.T @ du",
                                  "dwgu[e][:, :I] = xe.T @ du\n        dwgu[e][:, I:] = xe.T @ dg"),
    # the routing weight not applied to the expert's upstream gradient
    "routing_weight_dropped": ("dy = w[tt, jj][:, None] * dO[tt]", "dy = dO[tt]"),
    # the down weight's gradient taken against the pre-activation
    "down_gradient_from_gate": ("dwd[e] = h.T @ dy", "dwd[e] = g.T @ dy"),
    # dx only through the gate half
    "dx_misses_up_path": ("dg @ Wgu[e][:, :I].T + du @ Wgu[e][:, I:].T", "dg @ Wgu[e][:, :I].T"),
    # a token's pairs overwrite instead of adding up
    "dx_overwritten_per_expert": ("np.add.at(dx, tt, dg @ Wgu[e][:, :I].T + du @ Wgu[e][:, I:].T)",
                                  "dx[tt] = dg @ Wgu[e][:, :I].T + du @ Wgu[e][:, I:].T"),
    # the routing weight's gradient scaled by the weight itself
    "routing_gradient_scaled": ("dw[tt, jj] = np.sum(dO[tt] * y, axis=1)",
                                "dw[tt, jj] = np.sum(dO[tt] * y, axis=1) * w[tt, jj]"),
    # the renormalised softmax's Jacobian loses its coupling term
    "softmax_jacobian_dropped_term": ("w * (dw - inner)", "w * dw"),
}


def _pins():
    return [
        ("finite_differences[1]", lambda: pins.test_finite_differences_all_inputs(1)),
        ("finite_differences_routing_weights", pins.test_finite_differences_routing_weights_given_pairs),
        ("homogeneity[f32]", lambda: pins.test_degree_one_homogeneity("f32")),
        ("homogeneity[bf16]", lambda: pins.test_degree_one_homogeneity("bf16")),
        ("logit_invariants", pins.test_logit_gradient_invariants),
        ("empty_expert_zero_upstream", pins.test_empty_expert_and_zero_upstream),
    ]


def _mutated_backward(before, after):
    src = textwrap.dedent(inspect.getsource(oracle.backward))
    assert src.count(before) == 1, f"mutation site not found: {before}"
    ns = dict(vars(oracle))
    exec(compile(src.replace(before, after), "<mutant>", "exec"), ns)
    return ns["backward"]


def test_pins_pass_on_the_real_backward():
    for _, fn in _pins():
        fn()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_backward_mutant(name, monkeypatch):
    monkeypatch.setattr(oracle, "backward", _mutated_backward(*MUTANTS[name]))
    caught = []
    for pin_name, fn in _pins():
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin_name)
    assert caught, f"no pin caught the planted mistake {name}"
