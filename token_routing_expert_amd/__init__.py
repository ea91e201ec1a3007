"""MI355X (gfx950) mixture-of-experts layer forward: a thin Python binding.

The work runs in the HIP library ``libmoe.so`` (C ABI in ``include/moe.h``);
this module only marshals arguments: it checks tensor shapes, dtypes and
devices, passes raw device pointers and the current HIP stream, and turns a
non-zero status into an exception.  torch supplies device memory and
streams.  There is no fallback: without the built library every call raises.

Functions carry the C entry points' names:
  moe_route_topk    top-k + renormalised softmax routing
  moe_permute       pairs grouped by expert, token rows moved to expert order
  moe_grouped_ffn   each expert's SwiGLU feed-forward on its rows
  moe_gate_up_swiglu / moe_down_proj   its two halves
  moe_combine       routing-weighted sum back to token order
  moe_forward       the whole layer
  moe_tile_weights / moe_forward_tiled   the layer on column-tiled weights
"""
from __future__ import annotations

import ctypes
import os
import re

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmoe.so")
DEBUG_LIB_PATH = os.path.join(PKG_DIR, "libmoe_debug.so")   # the same entry points, device checks compiled in
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "moe.h")

MOE_F32 = 0
MOE_BF16 = 1
STATUS = {0: "MOE_OK", 1: "MOE_ERR_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _lib.moe_status_string(status).decode() if _lib is not None else ""
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")


def exported_symbols() -> list[str]:
    """Names of the functions include/moe.h declares."""
    text = open(HEADER_PATH).read()
    return re.findall(r"^(?:moe_status|size_t|const char\*)\s+(moe_\w+)\s*\(", text, flags=re.M)


def open_library(path: str):
    """ctypes handle of a built library at `path` with every entry point's
    signature declared (libmoe.so, or its device-checked twin
    libmoe_debug.so, which has the same entry points)."""
    lib = ctypes.CDLL(path)
    p, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    st = ctypes.c_int
    sig = {
        "moe_status_string": ([st], ctypes.c_char_p),
        "moe_route_topk": ([p, i32, i32, i32, p, p, p], st),
        "moe_route_project": ([p, p, st, i32, i32, i32, i32, p, p, p, p], st),
        "moe_permute_workspace_size": ([i32, i32, i32], sz),
        "moe_permute": ([p, st, i32, i32, i32, p, i32, p, p, p, p, p, sz, p], st),
        "moe_grouped_ffn_workspace_size": ([i32, i32, i32, i32, st], sz),
        "moe_grouped_ffn": ([p, p, i32, i32, i32, i32, p, p, st, p, p, sz, p], st),
        "moe_gate_up_swiglu": ([p, p, i32, i32, i32, i32, p, st, p, i32, p, p], st),
        "moe_down_proj": ([p, p, i32, i32, i32, i32, p, st, p, p], st),
        "moe_combine": ([p, i32, p, p, i32, i32, i32, st, p, p], st),
        "moe_forward_workspace_size": ([i32, i32, i32, i32, i32, st], sz),
        "moe_forward": ([p, p, i32, i32, i32, i32, i32, p, p, st, p, p, p, p, p, p, p, sz, p], st),
        "moe_backward_workspace_size": ([i32, i32, i32, i32, i32, st], sz),
        "moe_backward": ([p, p, i32, i32, i32, i32, i32, p, p, st, p, p, p, p, p, p, p, p, i32, p, sz, p], st),
        "moe_forward_train": ([p, p, i32, i32, i32, i32, i32, p, p, st, p, p, p, p, sz, p], st),
        "moe_forward_noalloc": ([p, p, i32, i32, i32, i32, i32, p, p, st, p, p, p, p, p, p, p], st),
        "moe_tile_weights": ([p, p, i32, i32, i32, st, p, p, p], st),
        "moe_forward_tiled": ([p, p, i32, i32, i32, i32, i32, p, p, st, p, p, p, p, p, p, p, sz, p], st),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


def load(build_if_missing: bool = True):
    """Load libmoe.so (building it first when it does not exist yet)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise RuntimeError(f"{LIB_PATH} is not built")
        from . import build as _build
        _build.build()
    _lib = open_library(LIB_PATH)
    return _lib


# ---- marshalling helpers ----------------------------------------------------------

def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"element type must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the MoE library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status)


def _expect(t, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def _empty(shape, dtype, like):
    return _torch().empty(shape, dtype=dtype, device=like.device)


def _workspace(nbytes, like, workspace):
    torch = _torch()
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                             f"{nbytes} needed")
        return workspace
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=like.device)


# ---- entry points --------------------------------------------------------------------

def moe_route_topk(logits, k: int, topk_idx=None, topk_w=None, stream=None):
    """logits [T, E] float32 -> (topk_idx [T, k] int32, topk_w [T, k] float32)."""
    torch = _torch()
    lib = load()
    T, E = logits.shape
    topk_idx = _empty((T, k), torch.int32, logits) if topk_idx is None else topk_idx
    topk_w = _empty((T, k), torch.float32, logits) if topk_w is None else topk_w
    _expect(logits, torch.float32, (T, E), "logits")
    _expect(topk_idx, torch.int32, (T, k), "topk_idx")
    _expect(topk_w, torch.float32, (T, k), "topk_w")
    _check("moe_route_topk", lib.moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_idx), _ptr(topk_w),
                                                _stream(stream)))
    return topk_idx, topk_w


def moe_route_project(x, w_router, k: int, want_logits: bool = False, logits=None, topk_idx=None, topk_w=None,
                      stream=None):
    """logits = x @ w_router^T (x [T, d], w_router [E, d], float32 accumulation), then
    top-k routing -> (topk_idx [T, k] int32, topk_w [T, k] float32), plus the logits
    [T, E] float32 when ``want_logits`` (or when ``logits`` is given)."""
    torch = _torch()
    lib = load()
    T, d = x.shape
    E, d2 = w_router.shape
    _expect(w_router, x.dtype, (E, d), "w_router")
    topk_idx = _empty((T, k), torch.int32, x) if topk_idx is None else topk_idx
    topk_w = _empty((T, k), torch.float32, x) if topk_w is None else topk_w
    _expect(topk_idx, torch.int32, (T, k), "topk_idx")
    _expect(topk_w, torch.float32, (T, k), "topk_w")
    if logits is None and want_logits:
        logits = _empty((T, E), torch.float32, x)
    if logits is not None:
        _expect(logits, torch.float32, (T, E), "logits")
    _check("moe_route_project", lib.moe_route_project(_ptr(x), _ptr(w_router), _dt(x), T, d, E, k, _ptr(logits),
                                                      _ptr(topk_idx), _ptr(topk_w), _stream(stream)))
    return (topk_idx, topk_w, logits) if logits is not None else (topk_idx, topk_w)


def moe_permute(x, pair_expert, k: int, E: int, x_perm=None, row_token=None, pair_row=None,
                expert_offsets=None, workspace=None, stream=None, move_rows: bool = True):
    """Group pairs by expert and move token rows.

    x [T, d]; pair_expert [T*k] (or [T, k]) int32 -> (x_perm [T*k, d], row_token [T*k],
    pair_row [T*k], expert_offsets [E+1]).  With ``move_rows=False`` only the index
    arrays are built and x_perm is None."""
    torch = _torch()
    lib = load()
    T, d = x.shape
    P = T * k
    pe = pair_expert.reshape(-1)
    _expect(pe, torch.int32, (P,), "pair_expert")
    if not move_rows:
        x_perm = None
    elif x_perm is None:
        x_perm = _empty((P, d), x.dtype, x)
    row_token = _empty((P,), torch.int32, x) if row_token is None else row_token
    pair_row = _empty((P,), torch.int32, x) if pair_row is None else pair_row
    expert_offsets = _empty((E + 1,), torch.int32, x) if expert_offsets is None else expert_offsets
    if x_perm is not None:
        _expect(x_perm, x.dtype, (P, d), "x_perm")
    _expect(row_token, torch.int32, (P,), "row_token")
    _expect(pair_row, torch.int32, (P,), "pair_row")
    _expect(expert_offsets, torch.int32, (E + 1,), "expert_offsets")
    nbytes = lib.moe_permute_workspace_size(T, k, E)
    ws = _workspace(nbytes, x, workspace)
    _check("moe_permute", lib.moe_permute(_ptr(x), _dt(x), T, d, k, _ptr(pe), E, _ptr(x_perm), _ptr(row_token),
                                          _ptr(pair_row), _ptr(expert_offsets), _ptr(ws), nbytes, _stream(stream)))
    return x_perm, row_token, pair_row, expert_offsets


def moe_grouped_ffn(x_perm, expert_offsets, w_gate_up, w_down, y_perm=None, workspace=None, stream=None):
    """x_perm [R, d] rows grouped by expert_offsets [E+1]; w_gate_up [E, d, 2I]; w_down [E, I, d]
    -> y_perm [R, d]."""
    torch = _torch()
    lib = load()
    R, d = x_perm.shape
    E, d2, two_i = w_gate_up.shape
    I = two_i // 2
    if d2 != d or two_i != 2 * I:
        raise ValueError(f"w_gate_up {tuple(w_gate_up.shape)} does not match d={d}")
    _expect(w_gate_up, x_perm.dtype, (E, d, 2 * I), "w_gate_up")
    _expect(w_down, x_perm.dtype, (E, I, d), "w_down")
    _expect(expert_offsets, torch.int32, (E + 1,), "expert_offsets")
    y_perm = _empty((R, d), x_perm.dtype, x_perm) if y_perm is None else y_perm
    _expect(y_perm, x_perm.dtype, (R, d), "y_perm")
    dt = _dt(x_perm)
    nbytes = lib.moe_grouped_ffn_workspace_size(R, E, d, I, dt)
    ws = _workspace(nbytes, x_perm, workspace)
    _check("moe_grouped_ffn", lib.moe_grouped_ffn(_ptr(x_perm), _ptr(expert_offsets), R, E, d, I, _ptr(w_gate_up),
                                                  _ptr(w_down), dt, _ptr(y_perm), _ptr(ws), nbytes,
                                                  _stream(stream)))
    return y_perm


def moe_gate_up_swiglu(x, expert_offsets, w_gate_up, h=None, row_token=None, max_rows=None, stream=None):
    """h[r] = silu(a_r @ Wgu[e][:, :I]) * (a_r @ Wgu[e][:, I:]) -> h [R, I].

    Without ``row_token``, ``x`` is the expert-ordered x_perm [R, d] and a_r = x[r].
    With ``row_token`` [R] (as moe_permute writes it), ``x`` is the token batch and
    a_r = x[row_token[r]]; R = ``max_rows`` (default len(row_token))."""
    torch = _torch()
    lib = load()
    x_rows, d = x.shape
    if row_token is None:
        R = x_rows
    else:
        R = int(max_rows if max_rows is not None else row_token.shape[0])
        _expect(row_token, torch.int32, (row_token.shape[0],), "row_token")
        if row_token.shape[0] < R:
            raise ValueError("row_token holds fewer rows than max_rows")
    E, d2, two_i = w_gate_up.shape
    I = two_i // 2
    _expect(w_gate_up, x.dtype, (E, d, 2 * I), "w_gate_up")
    _expect(expert_offsets, torch.int32, (E + 1,), "expert_offsets")
    h = _empty((R, I), x.dtype, x) if h is None else h
    _expect(h, x.dtype, (R, I), "h")
    _check("moe_gate_up_swiglu", lib.moe_gate_up_swiglu(_ptr(x), _ptr(expert_offsets), R, E, d, I, _ptr(w_gate_up),
                                                        _dt(x), _ptr(row_token), x_rows, _ptr(h), _stream(stream)))
    return h


def moe_down_proj(h, expert_offsets, w_down, y_perm=None, stream=None):
    """y_perm[r] = h[r] @ Wd[e] -> y_perm [R, d]."""
    torch = _torch()
    lib = load()
    R, I = h.shape
    E, I2, d = w_down.shape
    _expect(w_down, h.dtype, (E, I, d), "w_down")
    _expect(expert_offsets, torch.int32, (E + 1,), "expert_offsets")
    y_perm = _empty((R, d), h.dtype, h) if y_perm is None else y_perm
    _expect(y_perm, h.dtype, (R, d), "y_perm")
    _check("moe_down_proj", lib.moe_down_proj(_ptr(h), _ptr(expert_offsets), R, E, d, I, _ptr(w_down), _dt(h),
                                              _ptr(y_perm), _stream(stream)))
    return y_perm


def moe_combine(y_perm, pair_row, pair_w, T: int, k: int, out=None, stream=None):
    """out[t] = sum_j pair_w[t*k+j] * y_perm[pair_row[t*k+j]] -> out [T, d]."""
    torch = _torch()
    lib = load()
    R, d = y_perm.shape
    pr = pair_row.reshape(-1)
    pw = pair_w.reshape(-1)
    _expect(pr, torch.int32, (T * k,), "pair_row")
    _expect(pw, torch.float32, (T * k,), "pair_w")
    out = _empty((T, d), y_perm.dtype, y_perm) if out is None else out
    _expect(out, y_perm.dtype, (T, d), "out")
    _check("moe_combine", lib.moe_combine(_ptr(y_perm), R, _ptr(pr), _ptr(pw), T, k, d, _dt(y_perm), _ptr(out),
                                          _stream(stream)))
    return out


def moe_forward_workspace_size(T: int, d: int, E: int, k: int, I: int, dtype) -> int:
    return int(load().moe_forward_workspace_size(T, d, E, k, I, dtype))


def moe_forward(x, w_gate_up, w_down, k: int, logits=None, topk_idx=None, topk_w=None, out=None,
                expert_offsets=None, row_token=None, pair_row=None, workspace=None, stream=None, _tiled=False):
    """The whole layer.  With ``logits`` [T, E] the layer routes first (topk_idx / topk_w are
    outputs); without, ``topk_idx`` / ``topk_w`` [T, k] are the given pairs.
    Returns (out [T, d], topk_idx, topk_w)."""
    torch = _torch()
    lib = load()
    T, d = x.shape
    E, d2, two_i = w_gate_up.shape
    I = two_i // 2
    if d2 != d or two_i != 2 * I:
        raise ValueError(f"w_gate_up {tuple(w_gate_up.shape)} does not match d={d}")
    _expect(w_gate_up, x.dtype, (E, d, 2 * I), "w_gate_up")
    _expect(w_down, x.dtype, (E, I, d), "w_down")
    if logits is not None:
        _expect(logits, torch.float32, (T, E), "logits")
        topk_idx = _empty((T, k), torch.int32, x) if topk_idx is None else topk_idx
        topk_w = _empty((T, k), torch.float32, x) if topk_w is None else topk_w
    elif topk_idx is None or topk_w is None:
        raise ValueError("without logits, topk_idx and topk_w must be given")
    _expect(topk_idx.reshape(T, k), torch.int32, (T, k), "topk_idx")
    _expect(topk_w.reshape(T, k), torch.float32, (T, k), "topk_w")
    out = _empty((T, d), x.dtype, x) if out is None else out
    _expect(out, x.dtype, (T, d), "out")
    for name, t, n in (("expert_offsets", expert_offsets, E + 1), ("row_token", row_token, T * k),
                       ("pair_row", pair_row, T * k)):
        if t is not None:
            _expect(t, torch.int32, (n,), name)
    dt = _dt(x)
    nbytes = lib.moe_forward_workspace_size(T, d, E, k, I, dt)
    ws = _workspace(nbytes, x, workspace)
    fn, name = (lib.moe_forward_tiled, "moe_forward_tiled") if _tiled else (lib.moe_forward, "moe_forward")
    _check(name, fn(_ptr(x), _ptr(logits), T, d, E, k, I, _ptr(w_gate_up), _ptr(w_down), dt, _ptr(topk_idx),
                    _ptr(topk_w), _ptr(expert_offsets), _ptr(row_token), _ptr(pair_row), _ptr(out), _ptr(ws), nbytes,
                    _stream(stream)))
    return out, topk_idx, topk_w


def moe_tile_weights(w_gate_up, w_down, stream=None):
    """The expert weights in the column-tiled layout (include/moe.h): new
    tensors of the same shapes, for moe_forward_tiled.  bf16 only."""
    torch = _torch()
    lib = load()
    E, d, two_i = w_gate_up.shape
    I = two_i // 2
    if two_i != 2 * I:
        raise ValueError(f"w_gate_up {tuple(w_gate_up.shape)}: the last dimension is 2I")
    _expect(w_down, w_gate_up.dtype, (E, I, d), "w_down")
    wgu_t, wd_t = torch.empty_like(w_gate_up), torch.empty_like(w_down)
    _check("moe_tile_weights", lib.moe_tile_weights(_ptr(w_gate_up), _ptr(w_down), E, d, I, _dt(w_gate_up),
                                                    _ptr(wgu_t), _ptr(wd_t), _stream(stream)))
    return wgu_t, wd_t


def moe_forward_tiled(x, w_gate_up_tiled, w_down_tiled, k: int, **kw):
    """moe_forward on weights from moe_tile_weights (same arguments and results)."""
    return moe_forward(x, w_gate_up_tiled, w_down_tiled, k, _tiled=True, **kw)


def noalloc_scratch_bytes() -> int:
    """MOE_NOALLOC_SCRATCH_BYTES of include/moe.h: the scratch moe_forward_noalloc has."""
    m = re.search(r"#define\s+MOE_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", open(HEADER_PATH).read())
    return int(m.group(1)) << int(m.group(2))


def moe_forward_noalloc(x, w_gate_up, w_down, k: int, out, topk_idx, topk_w, logits=None, expert_offsets=None,
                        row_token=None, pair_row=None, stream=None):
    """The whole layer as moe_forward computes it, with the library's static
    scratch instead of a workspace: nothing is allocated, so every output
    (out [T, d], topk_idx / topk_w [T, k]) must be given.  Calls that overlap
    on one GPU race.  Returns (out, topk_idx, topk_w)."""
    torch = _torch()
    lib = load()
    T, d = x.shape
    E, d2, two_i = w_gate_up.shape
    I = two_i // 2
    if d2 != d or two_i != 2 * I:
        raise ValueError(f"w_gate_up {tuple(w_gate_up.shape)} does not match d={d}")
    _expect(w_gate_up, x.dtype, (E, d, 2 * I), "w_gate_up")
    _expect(w_down, x.dtype, (E, I, d), "w_down")
    if logits is not None:
        _expect(logits, torch.float32, (T, E), "logits")
    _expect(topk_idx.reshape(T, k), torch.int32, (T, k), "topk_idx")
    _expect(topk_w.reshape(T, k), torch.float32, (T, k), "topk_w")
    _expect(out, x.dtype, (T, d), "out")
    for name, t, n in (("expert_offsets", expert_offsets, E + 1), ("row_token", row_token, T * k),
                       ("pair_row", pair_row, T * k)):
        if t is not None:
            _expect(t, torch.int32, (n,), name)
    _check("moe_forward_noalloc",
           lib.moe_forward_noalloc(_ptr(x), _ptr(logits), T, d, E, k, I, _ptr(w_gate_up), _ptr(w_down), _dt(x),
                                   _ptr(topk_idx), _ptr(topk_w), _ptr(expert_offsets), _ptr(row_token),
                                   _ptr(pair_row), _ptr(out), _stream(stream)))
    return out, topk_idx, topk_w


def moe_backward_workspace_size(T: int, d: int, E: int, k: int, I: int, dtype) -> int:
    return int(load().moe_backward_workspace_size(T, d, E, k, I, dtype))


def moe_forward_train(x, w_gate_up, w_down, k: int, logits=None, topk_idx=None, topk_w=None, out=None,
                      workspace=None, stream=None):
    """The forward of a training step (bf16 or float32): ``out`` as moe_forward computes it, and
    the intermediates the backward needs kept in ``workspace`` (a backward-sized
    buffer, allocated when None).  Returns (out, topk_idx, topk_w, workspace); pass
    the same topk arrays and workspace to ``moe_backward(..., recompute=False)``."""
    torch = _torch()
    lib = load()
    T, d = x.shape
    E, d2, two_i = w_gate_up.shape
    I = two_i // 2
    if d2 != d or two_i != 2 * I:
        raise ValueError(f"w_gate_up {tuple(w_gate_up.shape)} does not match d={d}")
    _expect(w_gate_up, x.dtype, (E, d, 2 * I), "w_gate_up")
    _expect(w_down, x.dtype, (E, I, d), "w_down")
    if logits is not None:
        _expect(logits, torch.float32, (T, E), "logits")
        topk_idx = _empty((T, k), torch.int32, x) if topk_idx is None else topk_idx
        topk_w = _empty((T, k), torch.float32, x) if topk_w is None else topk_w
    elif topk_idx is None or topk_w is None:
        raise ValueError("without logits, topk_idx and topk_w must be given")
    _expect(topk_idx.reshape(T, k), torch.int32, (T, k), "topk_idx")
    _expect(topk_w.reshape(T, k), torch.float32, (T, k), "topk_w")
    out = _empty((T, d), x.dtype, x) if out is None else out
    _expect(out, x.dtype, (T, d), "out")
    dt = _dt(x)
    nbytes = lib.moe_backward_workspace_size(T, d, E, k, I, dt)
    ws = _workspace(nbytes, x, workspace)
    _check("moe_forward_train", lib.moe_forward_train(_ptr(x), _ptr(logits), T, d, E, k, I, _ptr(w_gate_up),
                                                      _ptr(w_down), dt, _ptr(topk_idx), _ptr(topk_w), _ptr(out),
                                                      _ptr(ws), nbytes, _stream(stream)))
    return out, topk_idx, topk_w, ws


def moe_backward(x, w_gate_up, w_down, k: int, dout, logits=None, topk_idx=None, topk_w=None,
                 want_dlogits: bool = True, workspace=None, recompute: bool = True, stream=None):
    """Gradients of <dout, moe_forward(x, ...)> (bf16 or float32).  With ``logits`` the layer
    routes first (topk_idx / topk_w are outputs, and dlogits is returned when
    ``want_dlogits``); without, ``topk_idx`` / ``topk_w`` are the given pairs.
    ``recompute=False`` uses what moe_forward_train left in ``workspace`` (pass its
    topk arrays too) instead of recomputing the forward.
    Returns a dict with dx, dw_gate_up, dw_down, dtopk_w, topk_idx, topk_w and
    (with logits) dlogits."""
    if not recompute and (workspace is None or topk_idx is None or topk_w is None):
        raise ValueError("recompute=False needs the workspace and topk arrays of moe_forward_train")
    torch = _torch()
    lib = load()
    T, d = x.shape
    E, d2, two_i = w_gate_up.shape
    I = two_i // 2
    if d2 != d or two_i != 2 * I:
        raise ValueError(f"w_gate_up {tuple(w_gate_up.shape)} does not match d={d}")
    _expect(w_gate_up, x.dtype, (E, d, 2 * I), "w_gate_up")
    _expect(w_down, x.dtype, (E, I, d), "w_down")
    _expect(dout, x.dtype, (T, d), "dout")
    if logits is not None:
        _expect(logits, torch.float32, (T, E), "logits")
        topk_idx = _empty((T, k), torch.int32, x) if topk_idx is None else topk_idx
        topk_w = _empty((T, k), torch.float32, x) if topk_w is None else topk_w
    elif topk_idx is None or topk_w is None:
        raise ValueError("without logits, topk_idx and topk_w must be given")
    _expect(topk_idx.reshape(T, k), torch.int32, (T, k), "topk_idx")
    _expect(topk_w.reshape(T, k), torch.float32, (T, k), "topk_w")
    dx = _empty((T, d), x.dtype, x)
    dwgu = _empty((E, d, 2 * I), x.dtype, x)
    dwd = _empty((E, I, d), x.dtype, x)
    dtw = _empty((T, k), torch.float32, x)
    dlg = _empty((T, E), torch.float32, x) if (logits is not None and want_dlogits) else None
    dt = _dt(x)
    nbytes = lib.moe_backward_workspace_size(T, d, E, k, I, dt)
    ws = _workspace(nbytes, x, workspace)
    _check("moe_backward", lib.moe_backward(_ptr(x), _ptr(logits), T, d, E, k, I, _ptr(w_gate_up), _ptr(w_down), dt,
                                            _ptr(topk_idx), _ptr(topk_w), _ptr(dout), _ptr(dx), _ptr(dwgu),
                                            _ptr(dwd), _ptr(dtw), _ptr(dlg), 1 if recompute else 0, _ptr(ws),
                                            nbytes, _stream(stream)))
    res = dict(dx=dx, dw_gate_up=dwgu, dw_down=dwd, dtopk_w=dtw, topk_idx=topk_idx, topk_w=topk_w)
    if dlg is not None:
        res["dlogits"] = dlg
    return res
