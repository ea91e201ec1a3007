"""The seeded input generators: reproducible, right shapes, right recipes."""
import numpy as np

import workloads
from workloads import bf16_bits, make, make_custom, to_float32, zipf_counts


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -2.5, 0.0, -0.0],
                 dtype=np.float32)
    bits = bf16_bits(f)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even (1.0);
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even (1 + 2^-6)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000, 0x8000]
    assert np.array_equal(to_float32(bits)[[0, 4]], np.array([1.0, -2.5], np.float32))


def test_seeded_reproducible_and_distinct():
    a = make_custom(T=16, d=32, E=4, k=2, I=8, seed=9)
    b = make_custom(T=16, d=32, E=4, k=2, I=8, seed=9)
    c = make_custom(T=16, d=32, E=4, k=2, I=8, seed=10)
    for f in ("x", "w_gate_up", "w_down", "logits"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
        assert not np.array_equal(getattr(a, f), getattr(c, f))


def test_tiny_config_shapes_and_logits():
    inp = make("tiny_f32")
    assert inp.x.shape == (64, 128) and inp.x.dtype == np.float32
    assert inp.w_gate_up.shape == (8, 128, 512) and inp.w_down.shape == (8, 256, 128)
    assert inp.logits.shape == (64, 8) and inp.logits.dtype == np.float32
    assert 0.015 < inp.w_gate_up.std() < 0.025


def test_small_config_skewed_logits():
    inp = make("small_bf16", weights=False)
    assert inp.x.dtype == np.uint16 and inp.x.shape == (4096, 1024)
    col_means = inp.logits.mean(axis=0)
    # per-expert bias ~ N(0, 0.5): column means spread far more than N(0,1)/sqrt(T) noise
    assert col_means.std() > 0.2


def test_uniform_logits_grid():
    inp = make_custom(T=64, d=32, E=128, k=4, I=32, logits="uniform", weights=False)
    lg = inp.logits.astype(np.float64)
    assert lg.min() >= 0 and lg.max() < 1
    assert np.all(lg * 2**24 == np.floor(lg * 2**24))


def test_zipf_counts_recipe():
    counts = zipf_counts(32768, 16, 1.1, 3, seed=4)
    assert counts.sum() == 32768
    assert (counts == 0).sum() == 3
    nz = np.sort(counts[counts > 0])[::-1]
    assert nz.size == 13
    # shares follow rank^-1.1 within one row of rounding
    share = np.arange(1, 14, dtype=np.float64) ** -1.1
    quota = 32768 * share / share.sum()
    assert np.all(np.abs(nz - quota) < 1.0)


def test_ep_rank_share_pairs():
    inp = make("ep_rank_share", weights=False)
    assert inp.logits is None and inp.k == 1
    assert inp.pair_expert.shape == (32768,) and inp.pair_expert.dtype == np.int32
    counts = np.bincount(inp.pair_expert, minlength=16)
    assert np.array_equal(counts, zipf_counts(32768, 16, 1.1, 3, seed=4))
    assert inp.pair_w.dtype == np.float32
    assert inp.pair_w.min() > 0 and inp.pair_w.max() <= 1
    # shuffled: not sorted by expert
    assert np.any(np.diff(inp.pair_expert) < 0)


def test_config_table_matches_definition():
    c = workloads.CONFIGS
    assert (c["large_e128"]["T"], c["large_e128"]["d"], c["large_e128"]["E"], c["large_e128"]["k"],
            c["large_e128"]["I"]) == (8192, 2880, 128, 4, 2880)
    assert (c["decode"]["T"], c["decode"]["d"], c["decode"]["E"], c["decode"]["k"],
            c["decode"]["I"]) == (64, 5120, 16, 1, 8192)
    assert workloads.ORDER[1] == "small_bf16"


def test_router_weight_layout():
    # the gate linear layer's weight [E, d]: its transpose is the W_r [d, E]
    # that the tiny workload's logits were drawn with
    inp = make("tiny_f32", weights=False)
    wr = workloads.router_weight(inp)
    assert wr.shape == (inp.E, inp.d) and wr.dtype == np.float32 and wr.flags.c_contiguous
    lg = (inp.x.astype(np.float64) @ wr.astype(np.float64).T).astype(np.float32)
    assert np.array_equal(lg, inp.logits)
    big = workloads.router_weight("large_e128")
    assert big.shape == (128, 2880) and big.dtype == np.uint16
    assert 0.015 < float(np.std(to_float32(big))) < 0.025
