"""Seeded synthetic inputs for one mixture-of-experts layer's forward pass.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Both the CPU oracle and the GPU path receive exactly the
arrays produced here: bfloat16 tensors as uint16 bit patterns (rounded from
float32 to nearest-even), float32 tensors as float32.

Named workloads (sizes fixed by the benchmark definition; distributions where
unstated are the plainest choice and are recorded in the recipe text):

  tiny_f32        T=64, d=128, E=8, k=2, I=256, float32.  x ~ N(0,1);
                  router weight W_r [d,E] ~ N(0,0.02), logits = x @ W_r taken
                  in float64 and stored as float32; expert weights ~ N(0,0.02).
  small_bf16      T=4096, d=1024, E=16, k=2, I=2816, bfloat16.  logits =
                  N(0,1) + b_e with a per-expert bias b_e ~ N(0,0.5), so the
                  expert load is skewed; weights ~ N(0,0.02); x ~ N(0,1).
  large_e128      T=8192, d=2880, E=128, k=4, I=2880, bfloat16.  logits
                  U[0,1) (float32 on a 2^-24 grid); weights ~ N(0,0.02).
  ep_rank_share   one expert-parallel rank's received rows: 32768 rows, 16
                  local experts, d=I=2880, bfloat16, k=1 (one pair per row,
                  token = row).  Per-expert counts follow Zipf(1.1) over a
                  seeded ranking of the experts; the three lowest-ranked
                  experts get no rows; the remaining 32768 rows are
                  apportioned by largest remainder; rows are shuffled.
                  Routing weights U(0,1] float32.  No logits.
  decode          T=64, d=5120, E=16, k=1, I=8192, bfloat16.  logits N(0,1).

Every tensor is drawn from ``numpy.random.default_rng([seed, tag, part])``
(PCG64), so each expert's weights can be drawn independently (in parallel).
"""
from __future__ import annotations

import dataclasses
import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# tags: one stream per tensor role
_TAG_X, _TAG_LOGITS, _TAG_BIAS, _TAG_ROUTER, _TAG_WGU, _TAG_WD, _TAG_PAIRS = range(1, 8)

CONFIGS = {
    "tiny_f32": dict(T=64, d=128, E=8, k=2, I=256, dtype="f32", seed=1, logits="router"),
    "small_bf16": dict(T=4096, d=1024, E=16, k=2, I=2816, dtype="bf16", seed=2, logits="normal_bias"),
    "large_e128": dict(T=8192, d=2880, E=128, k=4, I=2880, dtype="bf16", seed=3, logits="uniform"),
    "ep_rank_share": dict(T=32768, d=2880, E=16, k=1, I=2880, dtype="bf16", seed=4, logits=None,
                          zipf_s=1.1, zero_experts=3),
    "decode": dict(T=64, d=5120, E=16, k=1, I=8192, dtype="bf16", seed=5, logits="normal"),
}
ORDER = ["tiny_f32", "small_bf16", "large_e128", "ep_rank_share", "decode"]

WEIGHT_STD = 0.02
BIAS_STD = 0.5


@dataclasses.dataclass
class Inputs:
    name: str
    T: int
    d: int
    E: int
    k: int
    I: int
    dtype: str                     # "f32" or "bf16"
    x: np.ndarray                  # [T, d] float32 or uint16 (bf16 bits)
    w_gate_up: np.ndarray | None   # [E, d, 2I]
    w_down: np.ndarray | None      # [E, I, d]
    logits: np.ndarray | None      # [T, E] float32, or None for given pairs
    pair_expert: np.ndarray | None = None  # [T*k] int32 (given pairs only)
    pair_w: np.ndarray | None = None       # [T*k] float32 (given pairs only)

    @property
    def P(self) -> int:
        return self.T * self.k


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def _rng(seed: int, tag: int, part: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, tag, part])


def _threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def _normal(seed, tag, part, shape, std=1.0) -> np.ndarray:
    a = _rng(seed, tag, part).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _expert_weights(seed: int, tag: int, E: int, shape, dtype: str) -> np.ndarray:
    """[E, *shape] weights ~ N(0, 0.02), each expert from its own stream.

    The values are those of ``_normal`` followed by ``bf16_bits`` (same draws,
    same rounding); each worker thread reuses its own scratch buffers, so the
    many-gigabyte workloads do not fault in fresh temporaries per expert."""
    out = np.empty((E,) + tuple(shape), dtype=np.float32 if dtype == "f32" else np.uint16)
    n = int(np.prod(shape))
    local = threading.local()

    def one(e):
        if dtype == "f32":
            _rng(seed, tag, e).standard_normal(dtype=np.float32, out=out[e])
            out[e] *= np.float32(WEIGHT_STD)
            return
        if getattr(local, "f", None) is None:
            local.f = np.empty(n, dtype=np.float32)
            local.t = np.empty(n, dtype=np.uint32)
        f, t = local.f, local.t
        _rng(seed, tag, e).standard_normal(dtype=np.float32, out=f)
        f *= np.float32(WEIGHT_STD)
        u = f.view(np.uint32)
        # round to nearest even, as bf16_bits: (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        np.right_shift(u, 16, out=t)
        np.bitwise_and(t, 1, out=t)
        t += np.uint32(0x7FFF)
        u += t
        np.right_shift(u, 16, out=u)
        out[e].reshape(-1)[:] = u

    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(one, range(E)))
    return out


def zipf_counts(n_rows: int, E: int, s: float, zero_experts: int, seed: int) -> np.ndarray:
    """Per-expert row counts: a seeded ranking of the experts, Zipf(s) shares by
    rank, the lowest ``zero_experts`` ranks get nothing, and n_rows is split by
    largest remainder (equal remainders: lower expert index first)."""
    rng = _rng(seed, _TAG_PAIRS, 0)
    rank = rng.permutation(E) + 1                  # rank of expert e, 1..E
    share = rank.astype(np.float64) ** (-s)
    share[rank > E - zero_experts] = 0.0
    quota = n_rows * share / share.sum()
    counts = np.floor(quota).astype(np.int64)
    rest = n_rows - int(counts.sum())
    frac = quota - counts
    order = sorted(range(E), key=lambda e: (-frac[e], e))
    for e in order[:rest]:
        counts[e] += 1
    return counts


def make(name: str, weights: bool = True, seed: int | None = None) -> Inputs:
    """Draw the named workload.  ``weights=False`` skips the expert weights
    (useful for routing/permutation-only checks of the large workloads)."""
    cfg = dict(CONFIGS[name])
    if seed is not None:
        cfg["seed"] = seed
    return make_custom(name=name, **cfg, weights=weights)


def make_custom(T: int, d: int, E: int, k: int, I: int, dtype: str = "bf16", seed: int = 0,
                logits: str | None = "normal", name: str = "custom", weights: bool = True,
                zipf_s: float = 1.1, zero_experts: int = 0) -> Inputs:
    """Draw a workload of any shape.

    logits: "normal" N(0,1); "normal_bias" N(0,1) + per-expert N(0,0.5) bias;
    "uniform" U[0,1); "router" x @ W_r with W_r ~ N(0,0.02) (float64 product
    stored as float32); None: given pairs (k=1 rows with Zipf counts, see
    ``zipf_counts``, and U(0,1] weights).
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    xf = _normal(seed, _TAG_X, 0, (T, d))
    x = xf if dtype == "f32" else bf16_bits(xf)
    lg = pe = pw = None
    if logits == "normal":
        lg = _normal(seed, _TAG_LOGITS, 0, (T, E))
    elif logits == "normal_bias":
        bias = _normal(seed, _TAG_BIAS, 0, (E,), BIAS_STD)
        lg = _normal(seed, _TAG_LOGITS, 0, (T, E)) + bias[None, :]
    elif logits == "uniform":
        lg = _rng(seed, _TAG_LOGITS, 0).random((T, E), dtype=np.float32)
    elif logits == "router":
        wr = _normal(seed, _TAG_ROUTER, 0, (d, E), WEIGHT_STD)
        lg = (xf.astype(np.float64) @ wr.astype(np.float64)).astype(np.float32)
    elif logits is None:
        if k != 1:
            raise ValueError("given pairs are drawn one per row (k=1)")
        counts = zipf_counts(T, E, zipf_s, zero_experts, seed)
        rows = np.repeat(np.arange(E, dtype=np.int32), counts)
        rng = _rng(seed, _TAG_PAIRS, 1)
        pe = rows[rng.permutation(T)].astype(np.int32)
        pw = (np.float32(1.0) - rng.random(T, dtype=np.float32)).astype(np.float32)
    else:
        raise ValueError(logits)
    wgu = wd = None
    if weights:
        wgu = _expert_weights(seed, _TAG_WGU, E, (d, 2 * I), dtype)
        wd = _expert_weights(seed, _TAG_WD, E, (I, d), dtype)
    return Inputs(name=name, T=T, d=d, E=E, k=k, I=I, dtype=dtype, x=x, w_gate_up=wgu, w_down=wd,
                  logits=lg, pair_expert=pe, pair_w=pw)


def router_weight(name_or_inputs, seed: int | None = None) -> np.ndarray:
    """The router (gate linear layer) weight of a workload, laid out as that
    layer stores it: [E, d], N(0, 0.02), in the workload's element type.  It
    is the transpose of the W_r [d, E] that the "router" logits recipe draws
    (same stream), so on tiny_f32 x @ W_r reproduces the workload's logits."""
    inp = name_or_inputs if isinstance(name_or_inputs, Inputs) else make(name_or_inputs, weights=False)
    cfg_seed = CONFIGS[inp.name]["seed"] if inp.name in CONFIGS else 0
    wr = _normal(cfg_seed if seed is None else seed, _TAG_ROUTER, 0, (inp.d, inp.E), WEIGHT_STD)
    wt = np.ascontiguousarray(wr.T)
    return wt if inp.dtype == "f32" else bf16_bits(wt)


def to_float32(a: np.ndarray) -> np.ndarray:
    """Decode an array of either element type to float32 (bf16 bits are exact in float32)."""
    if a.dtype == np.float32:
        return a
    return (a.astype(np.uint32) << 16).view(np.float32)
