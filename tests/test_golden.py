"""The oracle still reproduces its stored outputs for the tiny workload.

tests/golden/tiny_f32.json was written by tests/golden/make_golden.py, which
calls only the oracle and the input generator; a change here means the
oracle's arithmetic changed."""
import json
import os

import numpy as np

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_f32.json")


def test_tiny_golden():
    doc = json.load(open(GOLDEN))
    inp = workloads.make("tiny_f32")
    res = oracle.forward(inp.x, inp.w_gate_up, inp.w_down, inp.k, logits=inp.logits)
    assert res["idx"].tolist() == doc["topk_idx"]
    assert res["offsets"].tolist() == doc["expert_offsets"]
    assert res["row_token"].tolist() == doc["row_token"]
    np.testing.assert_allclose(res["w"], np.array(doc["topk_w"]), rtol=1e-15, atol=0)
    for t, row in doc["out_rows"].items():
        np.testing.assert_allclose(res["out"][int(t)], np.array(row), rtol=1e-13, atol=1e-17)
    assert abs(np.abs(res["out"]).sum() - doc["out_abs_sum"]) <= 1e-12 * doc["out_abs_sum"]
