"""Writes tests/golden/tiny_f32.json from the CPU oracle (and the seeded
input generator) only.  Rerun after a deliberate change to the oracle's
arithmetic, and say in the commit which passage justifies the change.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    inp = workloads.make("tiny_f32")
    res = oracle.forward(inp.x, inp.w_gate_up, inp.w_down, inp.k, logits=inp.logits)
    doc = {
        "what": "oracle outputs for the tiny_f32 workload (T=64, d=128, E=8, k=2, I=256, float32, seed 1)",
        "source": "Hugging Face Transformers docs, 'Expert parallelism' (Token dispatch; Adding an "
                  "implementation) and 'Tensor parallelism for inference' (Packed strategies); "
                  "softmax top-k, ties to the lower expert index, SwiGLU",
        "written_by": "tests/golden/make_golden.py (calls oracle/ and workloads/ only)",
        "topk_idx": res["idx"].tolist(),
        "topk_w": [[float(f"{v:.17g}") for v in row] for row in res["w"]],
        "expert_offsets": res["offsets"].tolist(),
        "row_token": res["row_token"].tolist(),
        "out_rows": {str(t): [float(f"{v:.17g}") for v in res["out"][t]] for t in (0, 1, 31, 63)},
        "out_abs_sum": float(f"{abs(res['out']).sum():.17g}"),
    }
    with open(os.path.join(HERE, "tiny_f32.json"), "w") as f:
        json.dump(doc, f, indent=0)
        f.write("\n")


if __name__ == "__main__":
    main()
