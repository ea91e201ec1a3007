"""The C-ABI library: it loads, exports what include/moe.h declares, and its
host-side validation rejects bad arguments before touching the GPU.

Every call here returns from the host checks, so no kernel is launched and no
GPU is needed."""
import ctypes

import pytest

import token_routing_expert_amd as tre

P = ctypes.c_void_p
FAKE = P(256)  # never dereferenced: every call below fails validation or has nothing to do


@pytest.fixture(scope="module")
def lib():
    return tre.load()


def test_exports_every_declared_symbol(lib):
    names = tre.exported_symbols()
    assert set(names) == {
        "moe_status_string", "moe_route_topk", "moe_permute_workspace_size", "moe_permute",
        "moe_grouped_ffn_workspace_size", "moe_grouped_ffn", "moe_combine",
        "moe_forward_workspace_size", "moe_forward", "moe_gate_up_swiglu", "moe_down_proj", "moe_route_project",
        "moe_backward_workspace_size", "moe_backward", "moe_forward_train", "moe_forward_noalloc",
        "moe_tile_weights", "moe_forward_tiled"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(5):
        assert lib.moe_status_string(s)
    assert lib.moe_status_string(99) == b"unknown status"


def test_route_validation(lib):
    f = lib.moe_route_topk
    assert f(FAKE, 4, 8, 9, FAKE, FAKE, None) == 1          # k > E
    assert f(FAKE, 4, 8, 0, FAKE, FAKE, None) == 1          # k < 1
    assert f(FAKE, -1, 8, 2, FAKE, FAKE, None) == 1         # T < 0
    assert f(FAKE, 4, 257, 2, FAKE, FAKE, None) == 2        # E > 256
    assert f(FAKE, 4, 0, 1, FAKE, FAKE, None) == 1          # E < 1
    assert f(None, 4, 8, 2, FAKE, FAKE, None) == 1          # NULL logits
    assert f(None, 0, 8, 2, None, None, None) == 0          # T == 0: nothing to do


def test_permute_validation(lib):
    f = lib.moe_permute
    ws = lib.moe_permute_workspace_size(100, 2, 16)
    assert ws >= 2 * 16 * 4 and ws % 256 == 0
    assert lib.moe_permute_workspace_size(-1, 2, 16) == 0
    args = [FAKE, 1, 100, 128, 2, FAKE, 16, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None]
    assert f(*args[:3], 96, *args[4:]) == 2                          # d % 64
    assert f(*args[:6], 300, *args[7:]) == 2                         # E > 256
    assert f(*args[:1], 7, *args[2:]) == 1                           # bad dtype
    assert f(*args[:12], ws - 1, None) == 3                          # small workspace
    assert f(*args[:5], None, *args[6:]) == 1                        # NULL pair_expert
    assert f(None, *args[1:]) == 1                                   # rows to move but no x
    assert f(FAKE, 1, 0, 128, 2, None, 16, None, None, None, FAKE, None, 0, None) == 0   # T == 0


def test_grouped_ffn_validation(lib):
    f = lib.moe_grouped_ffn
    n = lib.moe_grouped_ffn_workspace_size(1000, 16, 1024, 2816, 1)
    assert n >= 1000 * 2816 * 2
    assert lib.moe_grouped_ffn_workspace_size(1000, 16, 1024, 2816, 0) >= 1000 * 2816 * 4
    base = [FAKE, FAKE, 1000, 16, 1024, 2816, FAKE, FAKE, 1, FAKE, FAKE, n, None]
    assert f(*base[:5], 2800, *base[6:]) == 2                        # I % 64
    assert f(*base[:4], 1000, *base[5:]) == 2                        # d % 64
    assert f(*base[:11], n - 1, None) == 3
    assert f(*base[:6], None, *base[7:]) == 1                        # NULL weights
    assert f(*base[:2], 0, *base[3:]) == 0                           # no rows
    assert f(*base[:2], -5, *base[3:]) == 1


def test_combine_validation(lib):
    f = lib.moe_combine
    assert f(FAKE, 10, FAKE, FAKE, 5, 2, 100, 1, FAKE, None) == 2    # d % 64
    assert f(FAKE, 10, FAKE, FAKE, 5, 0, 128, 1, FAKE, None) == 1    # k < 1
    assert f(FAKE, 10, None, FAKE, 5, 2, 128, 1, FAKE, None) == 1    # NULL pair_row
    assert f(None, 0, None, None, 0, 2, 128, 1, None, None) == 0     # T == 0


def test_forward_validation(lib):
    f = lib.moe_forward
    n = lib.moe_forward_workspace_size(64, 128, 8, 2, 256, 0)
    assert n > 0
    base = [FAKE, FAKE, 64, 128, 8, 2, 256, FAKE, FAKE, 0, FAKE, FAKE, None, None, None, FAKE, FAKE, n, None]
    assert f(*base[:5], 9, *base[6:]) == 1                           # routed k > E
    assert f(*base[:17], n - 1, None) == 3
    assert f(*base[:6], 100, *base[7:]) == 2                         # I % 64
    assert f(*base[:4], 300, *base[5:]) == 2                         # E > 256
    assert f(*base[:15], None, *base[16:]) == 1                      # NULL out
    assert f(*base[:2], 0, *base[3:]) == 0                           # T == 0
    # workspace grows with the batch
    assert lib.moe_forward_workspace_size(128, 128, 8, 2, 256, 0) > n


def test_ffn_halves_validation(lib):
    f = lib.moe_down_proj
    assert f(FAKE, FAKE, 100, 8, 128, 96, FAKE, 1, FAKE, None) == 2     # I % 64
    assert f(FAKE, FAKE, 100, 0, 128, 128, FAKE, 1, FAKE, None) == 1    # E < 1
    assert f(FAKE, FAKE, 100, 8, 128, 128, None, 1, FAKE, None) == 1    # NULL weight
    assert f(FAKE, FAKE, 100, 8, 128, 128, FAKE, 5, FAKE, None) == 1    # bad dtype
    assert f(None, None, 0, 8, 128, 128, None, 1, None, None) == 0      # no rows
    g = lib.moe_gate_up_swiglu
    assert g(FAKE, FAKE, 100, 8, 128, 96, FAKE, 1, None, 0, FAKE, None) == 2       # I % 64
    assert g(FAKE, FAKE, 100, 0, 128, 128, FAKE, 1, None, 0, FAKE, None) == 1      # E < 1
    assert g(FAKE, FAKE, 100, 8, 128, 128, None, 1, None, 0, FAKE, None) == 1      # NULL weight
    assert g(FAKE, FAKE, 100, 8, 128, 128, FAKE, 0, FAKE, 50, FAKE, None) == 2     # gather is bf16 only
    assert g(FAKE, FAKE, 100, 8, 128, 128, FAKE, 1, FAKE, -1, FAKE, None) == 1     # x_rows < 0
    assert g(FAKE, FAKE, 100, 8, 1024, 128, FAKE, 1, FAKE, 1 << 20, FAKE, None) == 2  # x too large for gathering
    assert g(None, None, 0, 8, 128, 128, None, 1, None, 0, None, None) == 0        # no rows


def test_route_project_validation(lib):
    f = lib.moe_route_project
    assert f(FAKE, FAKE, 1, 10, 128, 8, 9, None, FAKE, FAKE, None) == 1     # k > E
    assert f(FAKE, FAKE, 1, 10, 128, 300, 2, None, FAKE, FAKE, None) == 2   # E > 256
    assert f(FAKE, FAKE, 1, 10, 96, 8, 2, None, FAKE, FAKE, None) == 2      # d % 64
    assert f(FAKE, FAKE, 7, 10, 128, 8, 2, None, FAKE, FAKE, None) == 1     # bad dtype
    assert f(FAKE, None, 1, 10, 128, 8, 2, None, FAKE, FAKE, None) == 1     # NULL router weight
    assert f(FAKE, FAKE, 1, 10, 128, 8, 2, None, None, FAKE, None) == 1     # NULL topk_idx
    assert f(None, None, 1, 0, 128, 8, 2, None, None, None, None) == 0      # T == 0
    assert f(FAKE, FAKE, 1, 10, 1 << 22, 8, 2, None, FAKE, FAKE, None) == 2  # d >= 2^22


def test_backward_validation(lib):
    f = lib.moe_backward

    def call(x=FAKE, logits=FAKE, T=10, d=128, E=8, k=2, I=64, dt=1, dout=FAKE, dlogits=FAKE, ws=FAKE,
             ws_bytes=0, recompute=1):
        return f(x, logits, T, d, E, k, I, FAKE, FAKE, dt, FAKE, FAKE, dout, FAKE, FAKE, FAKE, FAKE, dlogits,
                 recompute, ws, ws_bytes, None)
    assert call(dt=0) == 3                    # float32: supported, and the workspace is too small
    assert call(dt=5) == 1                    # bad dtype
    assert call(k=9) == 1                     # k > E with logits
    assert call(E=300) == 2                   # E > 256
    assert call(d=96) == 2                    # d % 64
    assert call(I=100) == 2                   # I % 64
    assert call(logits=None) == 1             # dlogits without logits
    assert call(dout=None) == 1               # NULL upstream gradient
    assert call(x=None) == 1
    assert call(ws_bytes=1024) == 3           # workspace too small
    assert call(recompute=2) == 1             # recompute is 0 or 1
    need = lib.moe_backward_workspace_size(10, 128, 8, 2, 64, 1)
    assert call(ws=None, ws_bytes=need) == 3  # no workspace
    # float32: its seven row buffers (x, y, dy, dx rows; h; g | u and their gradient), 4 bytes an element
    assert lib.moe_backward_workspace_size(10, 128, 8, 2, 64, 0) >= 20 * 4 * (4 * 128 + 64 + 2 * 2 * 64)
    assert lib.moe_backward_workspace_size(10, 128, 8, 2, 64, 7) == 0      # no such dtype
    assert need > lib.moe_forward_workspace_size(10, 128, 8, 2, 64, 1)
    assert lib.moe_backward_workspace_size(20, 128, 8, 2, 64, 1) > need


def test_weight_size_limit(lib):
    # one expert's gate/up weight 4*d*I bytes must stay below 2 GiB
    assert lib.moe_down_proj(FAKE, FAKE, 100, 2, 32768, 16384, FAKE, 1, FAKE, None) == 2


def test_forward_train_validation(lib):
    f = lib.moe_forward_train

    def call(x=FAKE, logits=FAKE, T=10, d=128, E=8, k=2, I=64, dt=1, out=FAKE, ws=FAKE, ws_bytes=0):
        return f(x, logits, T, d, E, k, I, FAKE, FAKE, dt, FAKE, FAKE, out, ws, ws_bytes, None)
    assert call(dt=0) == 3                    # float32: supported, and the workspace is too small
    assert call(dt=5) == 1                    # bad dtype
    assert call(k=9) == 1                     # k > E with logits
    assert call(d=96) == 2                    # d % 64
    assert call(out=None) == 1
    assert call(ws_bytes=64) == 3             # needs the backward-sized workspace
    assert call(T=0, x=None, out=None) == 0   # empty batch


def test_forward_noalloc_validation(lib):
    # the layer without a workspace refuses what its static scratch cannot
    # hold before anything is looked up or enqueued, and validates like
    # moe_forward
    f = lib.moe_forward_noalloc
    cap = tre.noalloc_scratch_bytes()
    T, d, E, k, I = 8192, 1024, 16, 2, 2048
    assert lib.moe_forward_workspace_size(T, d, E, k, I, 1) > cap
    big = [FAKE, FAKE, T, d, E, k, I, FAKE, FAKE, 1, FAKE, FAKE, None, None, None, FAKE, None]
    assert f(*big) == 3                                              # more than the scratch
    assert f(*big[:3], 1000, *big[4:]) == 2                          # d % 64
    assert f(*big[:4], 300, *big[5:]) == 2                           # E > 256
    assert f(*big[:9], 7, *big[10:]) == 1                            # bad dtype


def test_device_checked_library_has_the_same_entry_points():
    # libmoe_debug.so: the same kernels with the device-side contract checks
    # compiled in; built beside libmoe.so
    import os
    if not os.path.exists(tre.DEBUG_LIB_PATH):
        from token_routing_expert_amd import build as tre_build
        tre_build.build(debug=True)
    dbg = tre.open_library(tre.DEBUG_LIB_PATH)
    for n in tre.exported_symbols():
        assert hasattr(dbg, n), n
    # host validation is shared: the same refusals, nothing launched
    assert dbg.moe_route_topk(FAKE, 4, 8, 9, FAKE, FAKE, None) == 1
    assert dbg.moe_forward_workspace_size(100, 128, 8, 2, 256, 1) == tre.load().moe_forward_workspace_size(
        100, 128, 8, 2, 256, 1)


def test_tile_weights_validation(lib):
    f = lib.moe_tile_weights
    assert f(FAKE, FAKE, 8, 128, 256, 0, FAKE, FAKE, None) == 2     # float32: bf16 only
    assert f(FAKE, FAKE, 8, 96, 256, 1, FAKE, FAKE, None) == 2      # d % 64
    assert f(FAKE, FAKE, 300, 128, 256, 1, FAKE, FAKE, None) == 2   # E > 256
    assert f(FAKE, FAKE, 0, 128, 256, 1, FAKE, FAKE, None) == 1     # E < 1
    assert f(FAKE, FAKE, 8, 128, 256, 5, FAKE, FAKE, None) == 1     # bad dtype
    assert f(FAKE, None, 8, 128, 256, 1, FAKE, FAKE, None) == 1     # NULL weight
    assert f(FAKE, FAKE, 8, 128, 256, 1, FAKE, None, None) == 1     # NULL output
    g = lib.moe_forward_tiled
    assert g(FAKE, None, 4, 128, 8, 2, 256, FAKE, FAKE, 0, FAKE, FAKE, None, None, None, FAKE, FAKE, 1 << 20,
             None) == 2                                               # float32: bf16 only
    assert g(FAKE, None, 0, 128, 8, 2, 256, FAKE, FAKE, 1, FAKE, FAKE, None, None, None, FAKE, None, 0,
             None) == 0                                               # T == 0: nothing to do
