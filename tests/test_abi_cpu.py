"""The C-ABI library loads, exports every symbol include/hstu.h declares,
and rejects bad host-side arguments before touching a device (no GPU
needed: these calls return before any HIP work)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "hstu.h")).read()
    return sorted(set(re.findall(r"\b(hstu_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    from hstu_jagged_pointwise_attn_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from hstu_jagged_pointwise_attn_amd import build
        build.build()
    return _lib


def test_every_declared_symbol_is_exported(L):
    lib = L.lib()
    names = _declared()
    assert "hstu_attn_fwd" in names and "hstu_attn_bwd" in names and "hstu_mfalcon_score" in names
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.SIGNATURES, n


def test_version(L):
    assert L.lib().hstu_version().decode().count(".") == 2


def _problem(L, **kw):
    p = L.Problem()
    p.B, p.H, p.d, p.dtype = 2, 2, 64, L.HSTU_BF16
    p.total_tokens, p.max_len, p.n_max = 10, 8, 8
    p.offsets = ctypes.c_void_p(0x1000)  # never dereferenced by the host checks
    p.norm, p.eps, p.n_groups = L.HSTU_NORM_LN, 1e-5, 1
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _ws(L, p, op=0):
    n = ctypes.c_size_t(0)
    st = L.lib().hstu_workspace_size(ctypes.byref(p), op, 0, 0, 0, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    ({}, 0),
    ({"d": 48}, 2),
    ({"d": 256}, 2),
    ({"B": -1}, 1),
    ({"H": 0}, 1),
    ({"dtype": 7}, 1),
    ({"n_max": 0}, 1),
    ({"offsets": None}, 1),
    ({"norm": 5}, 1),
    ({"eps": 0.0}, 1),
    ({"norm": 2}, 1),               # GLN without token_group
    ({"total_tokens": -3}, 1),
    ({"max_len": 2_000_000}, 2),
    ({"B": 100000}, 2),
    ({"H": 64, "d": 128}, 2),        # D = 8192 wider than the norm kernel supports
    ({"mask_flags": 2}, 1),          # unknown mask bit
    ({"mask_flags": 1}, 1),          # timestamp filter without timestamps
    ({"mask_flags": 1, "timestamps": ctypes.c_void_p(0x2000)}, 0),
])
def test_workspace_size_validation(L, kw, status):
    st, n = _ws(L, _problem(L, **kw))
    assert st == status, L.lib().hstu_last_error()
    if status == 0:
        assert n > 0 and n % 256 == 0
    else:
        assert L.lib().hstu_last_error()


def test_fwd_rejects_null_and_small_workspace(L):
    p = _problem(L)
    lib = L.lib()
    dummy = ctypes.c_void_p(0x2000)
    args = [dummy] * 8
    st = lib.hstu_attn_fwd(ctypes.byref(p), *args[:6], dummy, dummy, None, 0, None)
    assert st == L.HSTU_ERR_WORKSPACE
    st = lib.hstu_attn_fwd(ctypes.byref(p), *args[:6], dummy, dummy, ctypes.c_void_p(0x10000), 16, None)
    assert st == L.HSTU_ERR_WORKSPACE
    st = lib.hstu_attn_fwd(ctypes.byref(p), None, *args[:5], dummy, dummy, ctypes.c_void_p(0x10000), 1 << 30, None)
    assert st == L.HSTU_ERR_INVALID_ARG
    st = lib.hstu_attn_fwd(ctypes.byref(p), *args[:6], dummy, dummy, ctypes.c_void_p(0x10010), 1 << 30, None)
    assert st == L.HSTU_ERR_INVALID_ARG  # misaligned workspace


def test_attention_rejects_misaligned_arrays(L):
    """Every dense array is moved in 16-byte vectors: a pointer off a 16-byte
    boundary is refused before anything is enqueued."""
    lib = L.lib()
    dummy, odd = ctypes.c_void_p(0x2000), ctypes.c_void_p(0x2008)
    ws = ctypes.c_void_p(0x10000)
    p = _problem(L)
    for i in range(6):
        args = [dummy] * 6
        args[i] = odd
        assert lib.hstu_attn_fwd(ctypes.byref(p), *args, dummy, dummy, ws, 1 << 30, None) == L.HSTU_ERR_INVALID_ARG
    for i in range(10):
        args = [dummy] * 10
        args[i] = odd
        st = lib.hstu_attn_bwd(ctypes.byref(p), *args[:5], dummy, dummy, *args[5:], None, None, None, None,
                               ws, 1 << 30, None)
        assert st == L.HSTU_ERR_INVALID_ARG
    q = _problem(L, norm=L.HSTU_NORM_LN, eps=1e-5, gamma=odd)
    assert lib.hstu_attn_fwd(ctypes.byref(q), *([dummy] * 8), ws, 1 << 30, None) == L.HSTU_ERR_INVALID_ARG
    c = _problem(L)
    for i in range(8):
        args = [dummy] * 8          # K_cache, V_cache, then Qc, Kc, Vc, Uc, then Yc, Oc
        args[i] = odd
        st = lib.hstu_mfalcon_score(ctypes.byref(c), dummy, 16, 8, args[0], args[1], None, *args[2:6], 0,
                                    args[6], args[7], dummy, dummy, ws, 1 << 30, None)
        assert st == L.HSTU_ERR_INVALID_ARG


def test_mfalcon_rejects_prefix_and_cand_len(L):
    p = _problem(L, prefix_len=ctypes.c_void_p(0x3000))
    n = ctypes.c_size_t(0)
    lib = L.lib()
    dummy = ctypes.c_void_p(0x2000)
    st = lib.hstu_mfalcon_score(ctypes.byref(p), dummy, 16, 8, *([dummy] * 7), 0, *([dummy] * 5), 1 << 20, None)
    assert st == L.HSTU_ERR_INVALID_ARG
    p = _problem(L)
    st = lib.hstu_mfalcon_score(ctypes.byref(p), dummy, 16, 8, dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                -1, *([dummy] * 5), 1 << 20, None)
    assert st == L.HSTU_ERR_INVALID_ARG
    del n


def _weights(L, dm=16, **kw):
    w = L.LayerWeights()
    w.d_model, w.W1, w.W2 = dm, ctypes.c_void_p(0x4000), ctypes.c_void_p(0x8000)
    for k, v in kw.items():
        setattr(w, k, v)
    return w


def test_layer_workspace_size(L):
    p = _problem(L)
    lib = L.lib()
    n = ctypes.c_size_t(0)
    assert lib.hstu_layer_workspace_size(ctypes.byref(p), 16, L.HSTU_OP_FWD, ctypes.byref(n)) == 0
    _, core = _ws(L, p, L.HSTU_OP_FWD)
    T, D = p.total_tokens, p.H * p.d
    assert n.value >= core + 4 * T * D * 2 + (64 << 20) and n.value % 256 == 0
    nb = ctypes.c_size_t(0)
    assert lib.hstu_layer_workspace_size(ctypes.byref(p), 16, L.HSTU_OP_BWD, ctypes.byref(nb)) == 0
    assert nb.value > n.value
    for dm, op in ((0, L.HSTU_OP_FWD), (70000, L.HSTU_OP_FWD), (16, L.HSTU_OP_MFALCON)):
        assert lib.hstu_layer_workspace_size(ctypes.byref(p), dm, op, ctypes.byref(n)) == L.HSTU_ERR_INVALID_ARG


def test_layer_entry_points_reject_bad_arguments(L):
    p = _problem(L)
    lib = L.lib()
    dummy = ctypes.c_void_p(0x2000)
    big = ctypes.c_void_p(0x100000)
    fwd = lambda w, X=dummy, ws=big, n=1 << 40: lib.hstu_layer_fwd(
        ctypes.byref(p), None if w is None else ctypes.byref(w), X, dummy, dummy, None, dummy, dummy, dummy, dummy,
        ws, n, None)
    assert fwd(None) == L.HSTU_ERR_INVALID_ARG
    assert fwd(_weights(L, dm=0)) == L.HSTU_ERR_INVALID_ARG
    assert fwd(_weights(L, W1=None)) == L.HSTU_ERR_INVALID_ARG
    assert fwd(_weights(L, W2=ctypes.c_void_p(0x8004))) == L.HSTU_ERR_INVALID_ARG  # misaligned weight
    assert fwd(_weights(L), X=ctypes.c_void_p(0x2002)) == L.HSTU_ERR_INVALID_ARG   # misaligned X
    assert fwd(_weights(L), X=None) == L.HSTU_ERR_INVALID_ARG
    assert fwd(_weights(L), n=1024) == L.HSTU_ERR_WORKSPACE
    w = _weights(L)
    bwd = lambda dW1, n=1 << 40: lib.hstu_layer_bwd(
        ctypes.byref(p), ctypes.byref(w), dummy, dummy, None, *([dummy] * 5), dummy, dW1, None, dummy, None, None,
        None, None, None, big, n, None)
    assert bwd(None) == L.HSTU_ERR_INVALID_ARG
    assert bwd(ctypes.c_void_p(0x2004)) == L.HSTU_ERR_INVALID_ARG  # misaligned dW1
    assert bwd(dummy, n=1024) == L.HSTU_ERR_WORKSPACE


def test_stack_entry_points_reject_bad_arguments(L):
    p = _problem(L)
    lib = L.lib()
    dummy = ctypes.c_void_p(0x2000)
    n = ctypes.c_size_t(0)
    assert lib.hstu_stack_workspace_size(ctypes.byref(p), 16, L.HSTU_OP_FWD, 0, 0, 0, ctypes.byref(n)) == 0
    assert n.value % 256 == 0 and n.value > (64 << 20)
    assert lib.hstu_stack_workspace_size(ctypes.byref(p), 16, L.HSTU_OP_BWD, 0, 0, 0,
                                         ctypes.byref(n)) == L.HSTU_ERR_INVALID_ARG
    layers = (L.StackLayer * 2)()
    for i in range(2):
        layers[i].w = _weights(L)
        layers[i].K_cache = layers[i].V_cache = ctypes.c_void_p(0x10000)
    big = ctypes.c_void_p(0x100000)
    hist = lambda nl, lay: lib.hstu_stack_history(ctypes.byref(p), nl, lay, dummy, None, big, 1 << 40, None)
    assert hist(0, layers) == L.HSTU_ERR_INVALID_ARG
    assert hist(65, layers) == L.HSTU_ERR_INVALID_ARG
    assert hist(2, None) == L.HSTU_ERR_INVALID_ARG
    layers[1].w = _weights(L, dm=32)  # d_model differs between layers
    assert hist(2, layers) == L.HSTU_ERR_INVALID_ARG
    layers[1].w = _weights(L)
    layers[1].rab_p = ctypes.c_void_p(0x3000)  # the problem has n_pos = 0
    assert hist(2, layers) == L.HSTU_ERR_INVALID_ARG
    layers[1].rab_p = None
    layers[0].K_cache = ctypes.c_void_p(0x10008)  # misaligned cache
    assert hist(2, layers) == L.HSTU_ERR_INVALID_ARG
    layers[0].K_cache = ctypes.c_void_p(0x10000)
    assert lib.hstu_stack_history(ctypes.byref(p), 2, layers, dummy, None, big, 1024, None) == L.HSTU_ERR_WORKSPACE
    g = ctypes.c_void_p(0)
    assert lib.hstu_stack_score_capture(ctypes.byref(p), 2, layers, dummy, 16, 8, None, 0, dummy, dummy, big, 1 << 40,
                                        None) == L.HSTU_ERR_INVALID_ARG
    assert lib.hstu_graph_launch(None, None) == L.HSTU_ERR_INVALID_ARG
    assert lib.hstu_graph_destroy(None) == L.HSTU_ERR_INVALID_ARG
    del g


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with a message before
    touching a device or importing the library."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_static_forward_rejects_oversized_problem(L):
    """hstu_attn_fwd_static refuses, before any GPU work, a problem whose
    schedule does not fit the static scratch."""
    lib = L.lib()
    cap = lib.hstu_static_scratch_bytes()
    assert cap == 4 << 20
    p = _problem(L, B=8192, total_tokens=100_000_000, max_len=65536)
    dummy = ctypes.c_void_p(0x1000)
    st = lib.hstu_attn_fwd_static(ctypes.byref(p), *([dummy] * 8), None)
    assert st == L.HSTU_ERR_WORKSPACE
    assert b"static scratch" in lib.hstu_last_error()


def test_tile_order_switch(L):
    """hstu_set_tile_order (host only): returns the previous order and
    rejects unknown ones without changing the setting."""
    f = L.lib().hstu_set_tile_order
    assert f(1) == 0
    assert f(7) == -1
    assert f(0) == 1
    assert f(0) == 0
