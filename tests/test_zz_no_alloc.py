"""moe_forward_noalloc: the layer with the library's static scratch instead of
a workspace, for callers that cannot allocate.  Two calls in a row on one
GPU, the second with a smaller input (the scratch keeps the first call's
contents), each equal to moe_forward with a workspace bit for bit, outputs
starting as NaN so that a row left unwritten shows; the small call also
against the oracle.  Collected last (test_zz_*): a failure here hides no
other test."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import TOL, check_outputs, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tre():
    import torch
    assert torch.cuda.is_available(), "the GPU tests need an MI355X"
    import token_routing_expert_amd as m
    m.load()
    return m


def _case(tre, inp, given_pairs):
    import torch
    T, d, E, k, I = inp.T, inp.d, inp.E, inp.k, inp.I
    x, wgu, wd = to_device(inp.x), to_device(inp.w_gate_up), to_device(inp.w_down)
    assert tre.moe_forward_workspace_size(T, d, E, k, I, tre.MOE_BF16) <= tre.noalloc_scratch_bytes()
    outs = {}
    for mode in ("noalloc", "workspace"):
        out = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        offs = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
        prow = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
        rtok = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
        if given_pairs:
            idx = to_device(inp.pair_expert.reshape(T, k))
            w = to_device(inp.pair_w.reshape(T, k))
            lg = None
        else:
            idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
            w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
            lg = to_device(inp.logits)
        if mode == "noalloc":
            tre.moe_forward_noalloc(x, wgu, wd, k, out, idx, w, logits=lg, expert_offsets=offs, row_token=rtok,
                                    pair_row=prow)
        else:
            ws = torch.full((tre.moe_forward_workspace_size(T, d, E, k, I, tre.MOE_BF16),), 0xFF,
                            dtype=torch.uint8, device="cuda")
            tre.moe_forward(x, wgu, wd, k, logits=lg, topk_idx=idx, topk_w=w, out=out, expert_offsets=offs,
                            row_token=rtok, pair_row=prow, workspace=ws)
        torch.cuda.synchronize()
        outs[mode] = {"out": to_host(out), "idx": to_host(idx), "w": to_host(w), "offsets": to_host(offs),
                      "pair_row": to_host(prow), "row_token": to_host(rtok)}
    a, b = outs["noalloc"], outs["workspace"]
    n = int(a["offsets"][-1])
    for key in ("out", "idx", "w", "offsets", "pair_row"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key
    assert np.array_equal(a["row_token"][:n], b["row_token"][:n])
    print(f"  noalloc T={T} d={d} E={E} k={k} I={I}: equal to moe_forward bit for bit", flush=True)
    return a


def test_noalloc_two_calls_second_smaller(tre):
    # the first call: 256-row tiles, routing from logits, k = 2
    big = workloads.make_custom(T=2048, d=512, E=16, k=2, I=1408, dtype="bf16", seed=81, logits="normal_bias")
    _case(tre, big, given_pairs=False)
    # the second, smaller: given pairs, one per token, some dropped (-1); few
    # rows, so the down projection splits its k-stages and writes the output
    # rows itself -- scratch regions the first call left full of its own data
    small = workloads.make_custom(T=48, d=512, E=16, k=1, I=1408, dtype="bf16", seed=82, logits=None,
                                  zero_experts=3)
    small.pair_expert[::5] = -1
    got = _case(tre, small, given_pairs=True)
    ref = oracle.moe_tokens(small.x, small.pair_expert.reshape(48, 1), small.pair_w.reshape(48, 1).astype(np.float64),
                            small.w_gate_up, small.w_down)
    live = small.pair_expert >= 0
    check_outputs(got["out"][live], ref[live], TOL["bf16"], label="noalloc small call vs the oracle")
    assert not np.any(got["out"][~live])


def test_noalloc_refuses_more_than_its_scratch(tre):
    import torch
    T, d, E, k, I = 8192, 1024, 16, 2, 2048
    assert tre.moe_forward_workspace_size(T, d, E, k, I, tre.MOE_BF16) > tre.noalloc_scratch_bytes()
    x = torch.zeros((T, d), dtype=torch.bfloat16, device="cuda")
    wgu = torch.zeros((E, d, 2 * I), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((E, I, d), dtype=torch.bfloat16, device="cuda")
    out = torch.full((T, d), 3.0, dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    w = torch.ones((T, k), dtype=torch.float32, device="cuda")
    with pytest.raises(tre.MoeError) as err:
        tre.moe_forward_noalloc(x, wgu, wd, k, out, idx, w)
    assert err.value.status == 3   # MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)   # nothing was enqueued
