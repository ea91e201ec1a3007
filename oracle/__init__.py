"""CPU oracle for one mixture-of-experts layer's forward pass.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(the HIP library and its binding) never imports it, and it imports nothing
from the product path.

The arithmetic lives in ``moe_oracle.c`` (plain C, double precision); this
module builds it with gcc, loads it with ctypes and marshals numpy arrays.
Array conventions: ``x`` and the expert weights are either ``float32`` arrays
or ``uint16`` arrays of bfloat16 bit patterns; logits are ``float32``.

Steps and the passages they follow (Hugging Face Transformers docs):
  router     "Expert parallelism", introduction (a router sends each token to
             its experts) and "Token dispatch" (the router module, mlp.gate /
             mlp.router): logits = x @ W_r^T with the linear layer's weight
             W_r [E, d], no bias.
  route      "Expert parallelism", "Adding an implementation" (top_k_index,
             top_k_weights); softmax top-k, ties to the lower expert index.
  dispatch   "Expert parallelism", "Token dispatch": pairs grouped by expert,
             stable in pair order.
  experts    "Tensor parallelism for inference", "Packed strategies": packed
             gate/up weight [E, d, 2I], hidden @ W, gate half first; SwiGLU.
  combine    "Expert parallelism", "Token dispatch": routing-weighted sum.
  backward   "Expert parallelism", "Adding an implementation" (gradients, the
             routing weights' included, must reach every rank that holds
             tokens) and "Combining with FSDP2" (an expert's gradient sums
             over every batch it served; an expert that received no tokens
             still takes part, with a zero gradient): the chain rule through
             the steps above, in float64 (``backward``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC_PATH = os.path.join(_HERE, "moe_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1

_lib = None


def build(src: str = SRC_PATH, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile the oracle's C source into a shared library (gcc, -O2, no
    fast-math, no FMA contraction; ``extra_flags`` for instrumented builds)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off", *extra_flags,
           src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # TRE_ORACLE_LIB: another build of the same source (the sanitizer test
    # runs the pins against an instrumented copy)
    path = os.environ.get("TRE_ORACLE_LIB", LIB_PATH)
    if path == LIB_PATH and not os.path.exists(LIB_PATH):
        build()
    _lib = _bind(ctypes.CDLL(path))
    return _lib


def _bind(lib):
    """Declare the C signatures on a loaded copy of the oracle library."""
    p = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.oracle_route.argtypes = [p, i64, i32, i32, p, p]
    lib.oracle_route.restype = ctypes.c_int
    lib.oracle_dispatch.argtypes = [p, i64, i32, i32, p, p, p]
    lib.oracle_dispatch.restype = ctypes.c_int
    lib.oracle_moe_tokens.argtypes = [p, ctypes.c_int, i64, i32, i32, i32, i32, p, p, p, p, p, i64,
                                      ctypes.c_int, p, p]
    lib.oracle_moe_tokens.restype = ctypes.c_int
    return lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"expected float32 or uint16 (bfloat16 bits), got {a.dtype}")


# At most this many threads: on a shared multi-GPU host one GPU's job is
# given a share of 16 CPUs, whatever the machine's total.
THREAD_CAP = 16


def default_threads() -> int:
    """The CPUs this process may run on, capped at THREAD_CAP."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, THREAD_CAP))


def _f64(a: np.ndarray) -> np.ndarray:
    """float32 or bfloat16 bits -> float64 (exact)."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """Router projection: ``logits[t, e] = sum_c x[t, c] * w_router[e, c]`` in
    float64 from the exact input values (``x`` [T, d], ``w_router`` [E, d], both
    float32 or both bfloat16 bits).  The router is the model's gate linear layer
    ("Expert parallelism", introduction; module mlp.gate / mlp.router in "Token
    dispatch"); its output feeds the top-k selection as ``route`` takes it."""
    if x.dtype != w_router.dtype:
        raise TypeError("x and w_router must share one element type")
    if x.shape[1] != w_router.shape[1]:
        raise ValueError(f"shape mismatch: x {x.shape}, w_router {w_router.shape}")
    return _f64(x) @ _f64(w_router).T


def route(logits: np.ndarray, k: int):
    """Top-k selection and renormalised softmax weights.

    Returns ``(idx int32 [T, k], w float64 [T, k])``; slot 0 holds the largest logit.
    """
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    rc = _load().oracle_route(_ptr(logits), T, E, k, _ptr(idx), _ptr(w))
    if rc != 0:
        raise ValueError(f"oracle_route failed ({rc}): T={T} E={E} k={k}")
    return idx, w


def dispatch(pair_expert: np.ndarray, k: int, E: int):
    """Stable grouping of pairs by expert.

    ``pair_expert`` [P] holds the expert of pair p = t*k + j, or -1.
    Returns ``(offsets [E+1], pair_row [P], row_token [offsets[E]])`` (int32).
    """
    pe = np.ascontiguousarray(pair_expert, dtype=np.int32).reshape(-1)
    P = pe.shape[0]
    offsets = np.empty(E + 1, dtype=np.int32)
    pair_row = np.empty(P, dtype=np.int32)
    row_token = np.empty(P, dtype=np.int32)
    rc = _load().oracle_dispatch(_ptr(pe), P, k, E, _ptr(offsets), _ptr(pair_row), _ptr(row_token))
    if rc != 0:
        raise ValueError(f"oracle_dispatch failed ({rc}): P={P} k={k} E={E}")
    return offsets, pair_row, row_token[: offsets[E]].copy()


def permute_rows(x: np.ndarray, row_token: np.ndarray) -> np.ndarray:
    """Expert-ordered copy of the token rows: row r is x[row_token[r]] (a pure byte move)."""
    return x[np.asarray(row_token, dtype=np.int64)]


def moe_tokens(x: np.ndarray, idx: np.ndarray, w: np.ndarray, w_gate_up: np.ndarray,
               w_down: np.ndarray, tokens=None, nthreads: int | None = None, want_y: bool = False):
    """Experts + combine for the listed tokens (all tokens when ``tokens`` is None).

    ``out[n] = sum_j w[t, j] * FFN_{idx[t, j]}(x[t])`` for ``t = tokens[n]``, float64.
    With ``want_y`` also returns ``y_pair [n, k, d]`` = FFN_{idx[t, j]}(x[t]).
    """
    dt = _dtype_code(x)
    if _dtype_code(w_gate_up) != dt or _dtype_code(w_down) != dt:
        raise TypeError("x and expert weights must share one element type")
    x = np.ascontiguousarray(x)
    w_gate_up = np.ascontiguousarray(w_gate_up)
    w_down = np.ascontiguousarray(w_down)
    T, d = x.shape
    E, d2, two_i = w_gate_up.shape
    I = two_i // 2
    if d2 != d or two_i != 2 * I or w_down.shape != (E, I, d):
        raise ValueError(f"shape mismatch: x {x.shape}, w_gate_up {w_gate_up.shape}, w_down {w_down.shape}")
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(T, -1)
    k = idx.shape[1]
    w = np.ascontiguousarray(w, dtype=np.float64).reshape(T, k)
    if tokens is None:
        tokens = np.arange(T, dtype=np.int64)
    tokens = np.ascontiguousarray(tokens, dtype=np.int64).reshape(-1)
    n = tokens.shape[0]
    out = np.empty((n, d), dtype=np.float64)
    y = np.empty((n, k, d), dtype=np.float64) if want_y else None
    rc = _load().oracle_moe_tokens(_ptr(x), dt, T, d, E, k, I, _ptr(idx), _ptr(w), _ptr(w_gate_up),
                                   _ptr(w_down), _ptr(tokens), n, nthreads or default_threads(),
                                   _ptr(out), _ptr(y) if want_y else None)
    if rc != 0:
        raise ValueError(f"oracle_moe_tokens failed ({rc})")
    return (out, y) if want_y else out


def forward(x: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray, k: int, logits=None,
            pair_expert=None, pair_w=None, tokens=None, nthreads: int | None = None,
            want_y: bool = False) -> dict:
    """The whole layer: route (when ``logits`` is given; otherwise the pairs are
    given as ``pair_expert``/``pair_w``), dispatch, experts, combine.

    Returns a dict with ``idx, w, offsets, pair_row, row_token, out`` (and
    ``y_pair`` with ``want_y``); ``out`` covers ``tokens`` (default: all).
    """
    T = x.shape[0]
    E = w_gate_up.shape[0]
    if logits is not None:
        idx, w = route(logits, k)
    else:
        idx = np.asarray(pair_expert, dtype=np.int32).reshape(T, k)
        w = np.asarray(pair_w, dtype=np.float64).reshape(T, k)
    offsets, pair_row, row_token = dispatch(idx.reshape(-1), k, E)
    res = dict(idx=idx, w=w, offsets=offsets, pair_row=pair_row, row_token=row_token)
    r = moe_tokens(x, idx, w, w_gate_up, w_down, tokens=tokens, nthreads=nthreads, want_y=want_y)
    if want_y:
        res["out"], res["y_pair"] = r
    else:
        res["out"] = r
    return res


def combine(y_perm: np.ndarray, pair_row: np.ndarray, pair_w: np.ndarray, T: int, k: int) -> np.ndarray:
    """The combine step on its own, for given expert-ordered rows: for each
    token t, the sum over slots j (ascending) with a row of
    ``pair_w[t*k+j] * y_perm[pair_row[t*k+j]]``, in float64.  ``y_perm`` is
    float32 or bf16 bits."""
    y = y_perm.astype(np.float64) if y_perm.dtype == np.float32 else \
        (y_perm.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    pair_row = np.asarray(pair_row).reshape(-1)
    pair_w = np.asarray(pair_w, dtype=np.float64).reshape(-1)
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            r = int(pair_row[t * k + j])
            if 0 <= r < y.shape[0]:
                out[t] += pair_w[t * k + j] * y[r]
    return out


def _expand(a: np.ndarray) -> np.ndarray:
    """float64 copy of a float32 array or of bfloat16 bits (both exact)."""
    return _f64(a)


def backward(x: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray, k: int, dout: np.ndarray,
             logits=None, pair_expert=None, pair_w=None) -> dict:
    """Gradients of the layer's output, contracted with ``dout`` [T, d]: the
    chain rule through combine, down projection, SwiGLU, gate/up projection
    and (with ``logits``) the renormalised softmax, in float64 with one
    matmul per expert.  The top-k selection itself is piecewise constant and
    passes no gradient.

    For pair p = (t, j) with expert e, row x_t, weight w_p:
      g = x_t Wg_e, u = x_t Wu_e, s = sigmoid(g), h = g s u, y_p = h Wd_e
      out_t = sum_j w_p y_p
    so, with dy_p = w_p dout_t:
      dw_p   = <dout_t, y_p>
      dh     = dy_p Wd_e^T,            dWd_e  += h^T dy_p
      dg     = dh u s (1 + g (1 - s)), du = dh g s
      dx_t  += dg Wg_e^T + du Wu_e^T,  dWg_e += x_t^T dg, dWu_e += x_t^T du
    and, when the weights come from logits (w_j = softmax of the selected
    logits), dlogit_{t, e_j} = w_j (dw_j - sum_i w_i dw_i), zero for experts
    not selected.

    Pairs with expert -1 are skipped.  Returns a dict of float64 arrays
    ``dx [T, d], dw_gate_up [E, d, 2I], dw_down [E, I, d], dw [T, k]`` and
    ``dlogits [T, E]`` (when ``logits`` is given), plus ``idx`` and ``w``.
    """
    X = _expand(x)
    Wgu = _expand(w_gate_up)
    Wd = _expand(w_down)
    dO = np.asarray(dout, dtype=np.float64)
    T, d = X.shape
    E, _, two_i = Wgu.shape
    I = two_i // 2
    if logits is not None:
        idx, w = route(logits, k)
    else:
        idx = np.asarray(pair_expert, dtype=np.int32).reshape(T, k)
        w = np.asarray(pair_w, dtype=np.float64).reshape(T, k)
    dx = np.zeros((T, d))
    dwgu = np.zeros((E, d, 2 * I))
    dwd = np.zeros((E, I, d))
    dw = np.zeros((T, k))
    for e in range(E):
        tt, jj = np.nonzero(idx == e)  # the pairs of expert e (t ascending, then j)
        if tt.size == 0:
            continue
        xe = X[tt]
        g = xe @ Wgu[e][:, :I]
        u = xe @ Wgu[e][:, I:]
        s = 1.0 / (1.0 + np.exp(-g))
        h = g * s * u
        y = h @ Wd[e]
        dw[tt, jj] = np.sum(dO[tt] * y, axis=1)
        dy = w[tt, jj][:, None] * dO[tt]
        dh = dy @ Wd[e].T
        dwd[e] = h.T @ dy
        dg = dh * u * s * (1.0 + g * (1.0 - s))
        du = dh * g * s
        dwgu[e][:, :I] = xe.T @ dg
        dwgu[e][:, I:] = xe.T @ du
        np.add.at(dx, tt, dg @ Wgu[e][:, :I].T + du @ Wgu[e][:, I:].T)
    res = dict(idx=idx, w=w, dx=dx, dw_gate_up=dwgu, dw_down=dwd, dw=dw)
    if logits is not None:
        dl = np.zeros((T, E))
        inner = np.sum(w * dw, axis=1, keepdims=True)
        np.put_along_axis(dl, idx.astype(np.int64), w * (dw - inner), axis=1)
        res["dlogits"] = dl
    return res
