"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a temporary copy of the oracle's C source
(swapped gate/up halves, a flipped SiLU sign, the wrong tie-break, missing
renormalisation, an unstable grouping, a dropped slot, a misread weight
orientation, a wrong bfloat16 decode, the wrong token index), builds it,
swaps it in for the real library and runs the pin tests against it: at least
one pin must fail.  Runs on the CPU only; the real oracle is restored after.
"""
import contextlib
import ctypes
import os

import pytest

import oracle
import test_oracle_dispatch as pins_dispatch
import test_oracle_ffn as pins_ffn
import test_oracle_route as pins_route

MUTANTS = {
    "gate_reads_up_half": ("s->g[i] += xc * s->wrow[i];", "s->g[i] += xc * s->wrow[I + i];"),
    "up_reads_gate_half": ("s->u[i] += xc * s->wrow[I + i];", "s->u[i] += xc * s->wrow[i];"),
    "silu_sign": ("gi / (1.0 + exp(-gi))", "gi / (1.0 + exp(gi))"),
    "ties_to_higher_index": ("(la == lb && a < b)", "(la == lb && a > b)"),
    "no_renormalisation": ("w[t * k + j] = prob[idx[t * k + j]] / s;", "w[t * k + j] = prob[idx[t * k + j]];"),
    "unstable_grouping": ("for (int64_t p = 0; p < P; ++p) {\n    int32_t e = pair_expert[p];",
                          "for (int64_t p = P - 1; p >= 0; --p) {\n    int32_t e = pair_expert[p];"),
    "drops_last_slot": ("for (int32_t j = 0; j < k; ++j) {\n      const int32_t e = jb->idx[t * k + j];",
                        "for (int32_t j = 0; j < k - (k > 1); ++j) {\n      const int32_t e = jb->idx[t * k + j];"),
    "down_weight_row_misread": ("((int64_t)e * I + i) * d, d, s->wrow);", "((int64_t)e * I + 0) * d, d, s->wrow);"),
    "bf16_decode_shift": ("<< 16;", "<< 15;"),
    "row_token_is_pair": ("row_token[r] = (int32_t)(p / k);", "row_token[r] = (int32_t)p;"),
    "weights_of_wrong_slot": ("for (int32_t o = 0; o < d; ++o) acc[o] += wj * s.y[o];",
                              "for (int32_t o = 0; o < d; ++o) acc[o] += jb->w[t * k] * s.y[o];"),
}


def _pins():
    fns = []
    for mod in (pins_route, pins_dispatch, pins_ffn):
        for name in sorted(dir(mod)):
            if not name.startswith("test_"):
                continue
            f = getattr(mod, name)
            if name == "test_dense_masked_formulation":
                fns += [(name + "[f32]", lambda f=f: f("f32")), (name + "[bf16]", lambda f=f: f("bf16"))]
            else:
                fns.append((name, f))
    return fns


@contextlib.contextmanager
def swapped_library(path):
    old = oracle._lib
    oracle._lib = oracle._bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        oracle._lib = old


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(oracle.SRC_PATH).read()
    before, after = MUTANTS[name]
    assert src.count(before) >= 1, f"mutation site for {name} not found"
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(before, after, 1))
    lib = oracle.build(str(mutated), str(tmp_path / f"lib_{name}.so"))
    caught = []
    with swapped_library(lib):
        for pin_name, fn in _pins():
            try:
                fn()
            except (AssertionError, ValueError):
                caught.append(pin_name)
    assert caught, f"no pin caught the planted mistake {name}"
    os.remove(lib)
