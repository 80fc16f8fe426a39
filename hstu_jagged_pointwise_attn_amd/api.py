"""Torch-facing binding of libhstu.so: argument checking and marshalling only.

Every step of the computation runs in the library's HIP kernels; torch only
provides device memory and the current stream. Functions mirror the C entry
points of include/hstu.h (hstu_attn_fwd, hstu_attn_bwd, hstu_mfalcon_score,
hstu_schedule_export, hstu_get_device_status).
"""
from __future__ import annotations

import ctypes
from types import SimpleNamespace
from typing import Optional

import numpy as np
import torch

from . import _lib as L
from ._lib import (HSTU_BF16, HSTU_F32, HSTU_NORM_GLN, HSTU_NORM_LN, HSTU_NORM_NONE,  # noqa: F401
                   HSTU_OP_BWD, HSTU_OP_FWD, HSTU_OP_MFALCON, HSTUError)

_DTYPES = {torch.bfloat16: HSTU_BF16, torch.float32: HSTU_F32}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, device=None, numel=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if device is not None and (t.device.type != device.type or
                               (device.index is not None and t.device.index != device.index)):
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def workspace(nbytes: int, device) -> torch.Tensor:
    """A 256-byte aligned uint8 device buffer of at least nbytes."""
    raw = torch.empty(int(nbytes) + 256, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 256
    return raw[off:off + int(nbytes)]


def problem(offsets: torch.Tensor, *, H: int, d: int, dtype: torch.dtype, total_tokens: int,
            max_len: int, n_max: int, prefix_len=None, cand_len=None, timestamps=None, rab_p=None,
            rab_t=None, norm=HSTU_NORM_LN, eps=1e-5, token_group=None, n_groups=1, gamma=None,
            beta=None, time_filter=False):
    """Build the hstu_problem_t of a jagged batch (device tensors; host scalars).
    time_filter sets HSTU_MASK_CAND_TIME_FILTER."""
    dev = offsets.device
    B = offsets.numel() - 1
    _need(offsets, "offsets", torch.int32, dev)
    _need(prefix_len, "prefix_len", torch.int32, dev, B)
    _need(cand_len, "cand_len", torch.int32, dev, B)
    _need(timestamps, "timestamps", torch.int64, dev, total_tokens)
    _need(rab_p, "rab_p", torch.float32, dev)
    _need(rab_t, "rab_t", torch.float32, dev)
    _need(token_group, "token_group", torch.uint8, dev, total_tokens)
    G = n_groups if norm == HSTU_NORM_GLN else 1
    _need(gamma, "gamma", torch.float32, dev, G * H * d)
    _need(beta, "beta", torch.float32, dev, G * H * d)
    if dtype not in _DTYPES:
        raise TypeError(f"dtype {dtype} not supported (bfloat16, float32)")
    p = L.Problem()
    p.B, p.H, p.d, p.dtype = B, H, d, _DTYPES[dtype]
    p.total_tokens, p.max_len, p.n_max = int(total_tokens), int(max_len), int(n_max)
    p.offsets, p.prefix_len, p.cand_len, p.timestamps = (
        _ptr(offsets), _ptr(prefix_len), _ptr(cand_len), _ptr(timestamps))
    p.rab_p, p.rab_t = _ptr(rab_p), _ptr(rab_t)
    p.n_pos = 0 if rab_p is None else rab_p.numel()
    p.n_tb = 0 if rab_t is None else rab_t.numel()
    p.norm, p.eps = int(norm), float(eps)
    p.token_group, p.n_groups = _ptr(token_group), int(n_groups)
    p.gamma, p.beta = _ptr(gamma), _ptr(beta)
    p.mask_flags = L.HSTU_MASK_CAND_TIME_FILTER if time_filter else 0
    # keep the tensors alive as long as the struct
    p._keep = (offsets, prefix_len, cand_len, timestamps, rab_p, rab_t, token_group, gamma, beta)
    return p


def workspace_size(p, op, microbatch=0, hist_max_len=0, hist_tokens=0) -> int:
    n = ctypes.c_size_t(0)
    L.check(L.lib().hstu_workspace_size(ctypes.byref(p), op, microbatch, hist_max_len, hist_tokens,
                                        ctypes.byref(n)))
    return int(n.value)


def tile_shape(p, op=HSTU_OP_FWD):
    bm, bn = ctypes.c_int32(0), ctypes.c_int32(0)
    L.check(L.lib().hstu_tile_shape(ctypes.byref(p), op, ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def attn_fwd(p, Q, K, V, U, *, Y=None, O=None, mean=None, rstd=None, ws=None, stream=None):
    """hstu_attn_fwd. Q/K/V/U: [T, H, d] in the problem's dtype. Returns a
    namespace with Y, O ([T, H*d]), mean, rstd ([T] fp32) and ws."""
    T, D = p.total_tokens, p.H * p.d
    dev = Q.device
    dt = Q.dtype
    for t, n in ((Q, "Q"), (K, "K"), (V, "V"), (U, "U")):
        _need(t, n, dt, dev, T * D)
    if _DTYPES.get(dt) != p.dtype:
        raise TypeError("tensor dtype differs from the problem's dtype")
    Y = torch.empty(T, D, dtype=dt, device=dev) if Y is None else Y
    O = torch.empty(T, D, dtype=dt, device=dev) if O is None else O
    mean = torch.empty(T, dtype=torch.float32, device=dev) if mean is None else mean
    rstd = torch.empty(T, dtype=torch.float32, device=dev) if rstd is None else rstd
    for t, n in ((Y, "Y"), (O, "O")):
        _need(t, n, dt, dev, T * D)
    _need(mean, "mean", torch.float32, dev, T)
    _need(rstd, "rstd", torch.float32, dev, T)
    if ws is None:
        ws = workspace(workspace_size(p, HSTU_OP_FWD), dev)
    L.check(L.lib().hstu_attn_fwd(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(U), _ptr(Y), _ptr(O),
                                  _ptr(mean), _ptr(rstd), _ptr(ws), ws.numel(), _stream(stream)))
    return SimpleNamespace(Y=Y, O=O, mean=mean, rstd=rstd, ws=ws)


def attn_fwd_static(p, Q, K, V, U, *, Y=None, O=None, mean=None, rstd=None, stream=None):
    """hstu_attn_fwd_static: hstu_attn_fwd with the library's static device
    scratch instead of a workspace (no allocation inside the library). The
    outputs are allocated here unless given. Returns a namespace with Y, O,
    mean and rstd."""
    T, D = p.total_tokens, p.H * p.d
    dev, dt = Q.device, Q.dtype
    for t, n in ((Q, "Q"), (K, "K"), (V, "V"), (U, "U")):
        _need(t, n, dt, dev, T * D)
    if _DTYPES.get(dt) != p.dtype:
        raise TypeError("tensor dtype differs from the problem's dtype")
    Y = torch.empty(T, D, dtype=dt, device=dev) if Y is None else Y
    O = torch.empty(T, D, dtype=dt, device=dev) if O is None else O
    mean = torch.empty(T, dtype=torch.float32, device=dev) if mean is None else mean
    rstd = torch.empty(T, dtype=torch.float32, device=dev) if rstd is None else rstd
    for t, n in ((Y, "Y"), (O, "O")):
        _need(t, n, dt, dev, T * D)
    _need(mean, "mean", torch.float32, dev, T)
    _need(rstd, "rstd", torch.float32, dev, T)
    L.check(L.lib().hstu_attn_fwd_static(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(U), _ptr(Y), _ptr(O),
                                         _ptr(mean), _ptr(rstd), _stream(stream)))
    return SimpleNamespace(Y=Y, O=O, mean=mean, rstd=rstd)


def static_scratch_bytes() -> int:
    return int(L.lib().hstu_static_scratch_bytes())


def attn_bwd(p, Q, K, V, U, O, mean, rstd, dY, *, dQ=None, dK=None, dV=None, dU=None, d_rab_p=None,
             d_rab_t=None, d_gamma=None, d_beta=None, want_affine=True, ws=None, stream=None):
    """hstu_attn_bwd. Returns a namespace with dQ, dK, dV, dU ([T, H, d]),
    d_rab_p, d_rab_t, d_gamma, d_beta (fp32, None when not applicable)."""
    T, D = p.total_tokens, p.H * p.d
    dev, dt = Q.device, Q.dtype
    for t, n in ((Q, "Q"), (K, "K"), (V, "V"), (U, "U"), (O, "O"), (dY, "dY")):
        _need(t, n, dt, dev, T * D)
    _need(mean, "mean", torch.float32, dev, T)
    _need(rstd, "rstd", torch.float32, dev, T)
    shape = (T, p.H, p.d)
    dQ = torch.empty(shape, dtype=dt, device=dev) if dQ is None else dQ
    dK = torch.empty(shape, dtype=dt, device=dev) if dK is None else dK
    dV = torch.empty(shape, dtype=dt, device=dev) if dV is None else dV
    dU = torch.empty(shape, dtype=dt, device=dev) if dU is None else dU
    if p.rab_p and d_rab_p is None:
        d_rab_p = torch.empty(p.n_pos, dtype=torch.float32, device=dev)
    if p.rab_t and d_rab_t is None:
        d_rab_t = torch.empty(p.n_tb, dtype=torch.float32, device=dev)
    G = p.n_groups if p.norm == HSTU_NORM_GLN else 1
    if want_affine and p.gamma and d_gamma is None:
        d_gamma = torch.empty(G, D, dtype=torch.float32, device=dev)
    if want_affine and p.beta and d_beta is None:
        d_beta = torch.empty(G, D, dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(workspace_size(p, HSTU_OP_BWD), dev)
    L.check(L.lib().hstu_attn_bwd(ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(U), _ptr(O), _ptr(mean),
                                  _ptr(rstd), _ptr(dY), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dU),
                                  _ptr(d_rab_p), _ptr(d_rab_t), _ptr(d_gamma), _ptr(d_beta), _ptr(ws),
                                  ws.numel(), _stream(stream)))
    return SimpleNamespace(dQ=dQ, dK=dK, dV=dV, dU=dU, d_rab_p=d_rab_p, d_rab_t=d_rab_t, d_gamma=d_gamma,
                           d_beta=d_beta, ws=ws)


class HSTUAttnFn(torch.autograd.Function):
    """hstu_attn_fwd / hstu_attn_bwd as one autograd node.

    apply(p, Q, K, V, U, rab_p, rab_t, gamma, beta) -> Y [T, H*d]. `p` is the
    problem built by problem(); rab_p, rab_t, gamma and beta must be the very
    tensors `p` was built with (or None), so that their gradients land on
    them. The forward keeps O, mean and rstd for the backward; the backward
    calls hstu_attn_bwd once with the incoming dY (made contiguous) and hands
    back dQ, dK, dV, dU and the table / affine gradients. Timestamps, offsets
    and segment lengths take no gradient."""

    @staticmethod
    def forward(ctx, p, Q, K, V, U, rab_p=None, rab_t=None, gamma=None, beta=None):
        for t, name, field in ((rab_p, "rab_p", p.rab_p), (rab_t, "rab_t", p.rab_t), (gamma, "gamma", p.gamma),
                               (beta, "beta", p.beta)):
            if (t.data_ptr() if t is not None else None) != field:
                raise ValueError(f"{name} is not the tensor the problem was built with")
        out = attn_fwd(p, Q, K, V, U)
        ctx.p = p
        ctx.save_for_backward(Q, K, V, U, out.O, out.mean, out.rstd)
        ctx.want_affine = gamma is not None or beta is not None
        ctx.affine_shapes = (None if gamma is None else gamma.shape, None if beta is None else beta.shape)
        return out.Y

    @staticmethod
    def backward(ctx, dY):
        Q, K, V, U, O, mean, rstd = ctx.saved_tensors
        g = attn_bwd(ctx.p, Q, K, V, U, O, mean, rstd, dY.contiguous(), want_affine=ctx.want_affine)
        gs, bs = ctx.affine_shapes
        return (None, g.dQ, g.dK, g.dV, g.dU, g.d_rab_p, g.d_rab_t,
                g.d_gamma.view(gs) if g.d_gamma is not None else None,
                g.d_beta.view(bs) if g.d_beta is not None else None)


def hstu_attention(offsets, Q, K, V, U, *, max_len, n_max, prefix_len=None, cand_len=None, timestamps=None,
                   rab_p=None, rab_t=None, norm=HSTU_NORM_LN, eps=1e-5, token_group=None, n_groups=1, gamma=None,
                   beta=None, time_filter=False):
    """Y = Norm(A V) * U of a jagged batch through HSTUAttnFn (differentiable
    in Q, K, V, U, rab_p, rab_t, gamma, beta). Q/K/V/U: [T, H, d] device
    tensors of one dtype; the other arguments as for problem()."""
    T, H, d = Q.shape
    p = problem(offsets, H=H, d=d, dtype=Q.dtype, total_tokens=T, max_len=max_len, n_max=n_max,
                prefix_len=prefix_len, cand_len=cand_len, timestamps=timestamps, rab_p=rab_p, rab_t=rab_t,
                norm=norm, eps=eps, token_group=token_group, n_groups=n_groups, gamma=gamma, beta=beta,
                time_filter=time_filter)
    return HSTUAttnFn.apply(p, Q, K, V, U, rab_p, rab_t, gamma, beta)


def mfalcon_score(cand_p, hist_offsets, hist_tokens, hist_max_len, K_cache, V_cache, Qc, Kc, Vc, Uc, *,
                  hist_ts=None, microbatch=0, Yc=None, Oc=None, mean=None, rstd=None, ws=None, stream=None):
    """hstu_mfalcon_score. cand_p describes the candidates (offsets over Tc
    candidate tokens). Returns a namespace with Yc, Oc, mean, rstd, ws."""
    Tc, D = cand_p.total_tokens, cand_p.H * cand_p.d
    dev, dt = Qc.device, Qc.dtype
    for t, n in ((Qc, "Qc"), (Kc, "Kc"), (Vc, "Vc"), (Uc, "Uc")):
        _need(t, n, dt, dev, Tc * D)
    for t, n in ((K_cache, "K_cache"), (V_cache, "V_cache")):
        _need(t, n, dt, dev, int(hist_tokens) * D)
    _need(hist_offsets, "hist_offsets", torch.int32, dev, cand_p.B + 1)
    _need(hist_ts, "hist_ts", torch.int64, dev, int(hist_tokens))
    Yc = torch.empty(Tc, D, dtype=dt, device=dev) if Yc is None else Yc
    Oc = torch.empty(Tc, D, dtype=dt, device=dev) if Oc is None else Oc
    mean = torch.empty(Tc, dtype=torch.float32, device=dev) if mean is None else mean
    rstd = torch.empty(Tc, dtype=torch.float32, device=dev) if rstd is None else rstd
    if ws is None:
        ws = workspace(workspace_size(cand_p, HSTU_OP_MFALCON, microbatch, hist_max_len, hist_tokens), dev)
    L.check(L.lib().hstu_mfalcon_score(
        ctypes.byref(cand_p), _ptr(hist_offsets), int(hist_tokens), int(hist_max_len), _ptr(K_cache),
        _ptr(V_cache), _ptr(hist_ts), _ptr(Qc), _ptr(Kc), _ptr(Vc), _ptr(Uc), int(microbatch), _ptr(Yc),
        _ptr(Oc), _ptr(mean), _ptr(rstd), _ptr(ws), ws.numel(), _stream(stream)))
    return SimpleNamespace(Y=Yc, O=Oc, mean=mean, rstd=rstd, ws=ws)


def schedule_export(p, op=HSTU_OP_FWD, hist_offsets=None, hist_tokens=0, hist_max_len=0, microbatch=0,
                    stream=None):
    """Run only the tile scheduler and return (qtile_off [B+1], tiles [N, 4])
    as numpy int32 arrays; tiles rows are {b, row0, nk, nf | nrows << 16} in
    execution order. Synchronises the stream."""
    dev = torch.device("cuda", torch.cuda.current_device())
    ws = workspace(workspace_size(p, op, microbatch, hist_max_len, hist_tokens), dev)
    qoff = np.zeros(p.B + 1, dtype=np.int32)
    cap = 1 << 20
    tiles = np.zeros((cap, 4), dtype=np.int32)
    count = ctypes.c_int64(0)
    L.check(L.lib().hstu_schedule_export(
        ctypes.byref(p), op, _ptr(hist_offsets), int(hist_tokens), int(hist_max_len), int(microbatch),
        _ptr(ws), ws.numel(), _stream(stream), ctypes.c_void_p(qoff.ctypes.data),
        ctypes.c_void_p(tiles.ctypes.data), cap, ctypes.byref(count)))
    return qoff, tiles[:count.value].copy()


def device_status(ws, stream=None) -> int:
    """hstu_get_device_status: HSTU_DEV_* bits left by the last call on ws."""
    v = ctypes.c_int32(0)
    L.check(L.lib().hstu_get_device_status(_ptr(ws), _stream(stream), ctypes.byref(v)))
    return int(v.value)


def kernel_timing(enable: bool) -> None:
    """hstu_kernel_timing: bracket every library kernel launch with HIP events."""
    L.check(L.lib().hstu_kernel_timing(1 if enable else 0))


def set_inline_schedule(enable: bool) -> bool:
    """hstu_set_inline_schedule: whether small forwards build their tiles
    inside the attention kernel (default) instead of launching the scheduler.
    Returns the previous setting."""
    return bool(L.lib().hstu_set_inline_schedule(1 if enable else 0))


def set_fused_projection(enable: bool) -> bool:
    """hstu_set_fused_projection: whether the bf16 training forward runs f1
    as the library's own GEMM with the SiLU split epilogue (default) or as a
    library GEMM followed by a separate SiLU split pass. Returns the previous
    setting."""
    return bool(L.lib().hstu_set_fused_projection(1 if enable else 0))


HSTU_TILE_ORDER_LONGEST = 0
HSTU_TILE_ORDER_BY_SEQUENCE = 1


def set_tile_order(order: int) -> int:
    """hstu_set_tile_order: the scheduler's work-list order (longest record
    first, or by sequence). Returns the previous order."""
    prev = int(L.lib().hstu_set_tile_order(int(order)))
    if prev < 0:
        raise ValueError(f"unknown tile order {order}")
    return prev


def kernel_timing_read(kernel: int):
    """hstu_kernel_timing_read: (total milliseconds, launches) of one kernel id."""
    ms, n = ctypes.c_double(0), ctypes.c_int64(0)
    L.check(L.lib().hstu_kernel_timing_read(int(kernel), ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)


# ------------------------------------------------------------ batch preparation

def stochastic_length(offsets: torch.Tensor, keys: torch.Tensor, cap: int, max_len: int, stream=None):
    """hstu_stochastic_length. offsets int32 [B+1], keys int32/uint32 bits
    [T] on the device. Returns (new_offsets int32 [B+1], gather_idx int32 [T],
    status int32 [1]); the first new_offsets[B] entries of gather_idx are
    valid."""
    dev = offsets.device
    B = offsets.numel() - 1
    T = keys.numel()
    _need(offsets, "offsets", torch.int32, dev)
    if keys.dtype not in (torch.int32, torch.uint32):
        raise TypeError("keys must be 32-bit")
    new_off = torch.empty(B + 1, dtype=torch.int32, device=dev)
    idx = torch.empty(max(T, 1), dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    L.check(L.lib().hstu_stochastic_length(_ptr(offsets), B, T, int(max_len), int(cap), _ptr(keys), _ptr(new_off),
                                           _ptr(idx), _ptr(status), _stream(stream)))
    return new_off, idx, status


def gather_rows(src: torch.Tensor, idx: torch.Tensor, n: int, stream=None):
    """hstu_gather_rows: rows src[idx[r]] for r < n of a dense [rows, ...] tensor."""
    dev = src.device
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    row_bytes = src[0].numel() * src.element_size() if src.shape[0] else src.element_size()
    dst = torch.empty((int(n),) + tuple(src.shape[1:]), dtype=src.dtype, device=dev)
    L.check(L.lib().hstu_gather_rows(_ptr(src), _ptr(idx), int(n), int(row_bytes), _ptr(dst), _stream(stream)))
    return dst


def balance_bins(offsets: torch.Tensor, n_bins: int, cost_kind=L.HSTU_COST_TOKENS, stream=None):
    """hstu_balance_bins. Returns (bin int32 [B], bin_cost int64 [n_bins])."""
    dev = offsets.device
    B = offsets.numel() - 1
    _need(offsets, "offsets", torch.int32, dev)
    b = torch.empty(max(B, 1), dtype=torch.int32, device=dev)
    cost = torch.empty(n_bins, dtype=torch.int64, device=dev)
    L.check(L.lib().hstu_balance_bins(_ptr(offsets), B, int(n_bins), int(cost_kind), _ptr(b), _ptr(cost),
                                      _stream(stream)))
    return b[:B], cost


def layer_weights(W1: torch.Tensor, W2: torch.Tensor, b1=None, b2=None):
    """The hstu_layer_weights_t of W1 [d_model, 4D], W2 [D, d_model] (the
    problem's dtype) and the optional fp32 biases b1 [4D], b2 [d_model]."""
    dm = W1.shape[0]
    dev = W1.device
    _need(W1, "W1", None, dev)
    _need(W2, "W2", W1.dtype, dev, W1.shape[1] // 4 * dm)
    _need(b1, "b1", torch.float32, dev, W1.shape[1])
    _need(b2, "b2", torch.float32, dev, dm)
    w = L.LayerWeights()
    w.d_model = int(dm)
    w.W1, w.W2, w.b1, w.b2 = _ptr(W1), _ptr(W2), _ptr(b1), _ptr(b2)
    w._keep = (W1, W2, b1, b2)
    return w


def layer_workspace_size(p, d_model: int, op) -> int:
    n = ctypes.c_size_t(0)
    L.check(L.lib().hstu_layer_workspace_size(ctypes.byref(p), int(d_model), op, ctypes.byref(n)))
    return int(n.value)


def layer_fwd(p, w, X, *, Out=None, Z=None, UVQK=None, save_act=False, keep_z=True, Y=None, O=None, mean=None,
              rstd=None, ws=None, stream=None):
    """hstu_layer_fwd. X: [T, d_model]. Returns a namespace with Out
    [T, d_model] and the saved Z [T, 4D] (None when keep_z is false and no Z
    is given: the inference form, SiLU in the f1 GEMMs' epilogue), Y, O
    [T, D], mean, rstd, ws, and UVQK [4, T, D] (the activations, kept for the
    backward) when save_act is set or UVQK is given (else None)."""
    T, D, dm = p.total_tokens, p.H * p.d, w.d_model
    dev, dt = X.device, X.dtype
    if _DTYPES.get(dt) != p.dtype:
        raise TypeError("tensor dtype differs from the problem's dtype")
    _need(X, "X", dt, dev, T * dm)
    Out = torch.empty(T, dm, dtype=dt, device=dev) if Out is None else Out
    if Z is None and keep_z:
        Z = torch.empty(T, 4 * D, dtype=dt, device=dev)
    if UVQK is None and save_act:
        UVQK = torch.empty(4, T, D, dtype=dt, device=dev)
    _need(UVQK, "UVQK", dt, dev, 4 * T * D)
    Y = torch.empty(T, D, dtype=dt, device=dev) if Y is None else Y
    O = torch.empty(T, D, dtype=dt, device=dev) if O is None else O
    mean = torch.empty(T, dtype=torch.float32, device=dev) if mean is None else mean
    rstd = torch.empty(T, dtype=torch.float32, device=dev) if rstd is None else rstd
    for t, n, k in ((Out, "Out", T * dm), (Z, "Z", T * 4 * D), (Y, "Y", T * D), (O, "O", T * D)):
        _need(t, n, dt, dev, k)
    _need(mean, "mean", torch.float32, dev, T)
    _need(rstd, "rstd", torch.float32, dev, T)
    if ws is None:
        ws = workspace(layer_workspace_size(p, dm, HSTU_OP_FWD), dev)
    L.check(L.lib().hstu_layer_fwd(ctypes.byref(p), ctypes.byref(w), _ptr(X), _ptr(Out), _ptr(Z), _ptr(UVQK), _ptr(Y),
                                   _ptr(O), _ptr(mean), _ptr(rstd), _ptr(ws), ws.numel(), _stream(stream)))
    return SimpleNamespace(Out=Out, Z=Z, UVQK=UVQK, Y=Y, O=O, mean=mean, rstd=rstd, ws=ws)


def layer_bwd(p, w, X, f, dOut, *, dX=None, dW1=None, db1=None, dW2=None, db2=None, d_rab_p=None, d_rab_t=None,
              d_gamma=None, d_beta=None, want_bias=True, want_affine=True, ws=None, stream=None):
    """hstu_layer_bwd. f: the namespace layer_fwd returned (Z, UVQK, Y, O,
    mean, rstd; UVQK may be None). Returns a namespace with dX and the fp32 dW1, db1, dW2, db2,
    d_rab_p, d_rab_t, d_gamma, d_beta (None when not applicable)."""
    T, D, dm = p.total_tokens, p.H * p.d, w.d_model
    dev, dt = X.device, X.dtype
    _need(X, "X", dt, dev, T * dm)
    _need(dOut, "dOut", dt, dev, T * dm)
    f32 = dict(dtype=torch.float32, device=dev)
    dX = torch.empty(T, dm, dtype=dt, device=dev) if dX is None else dX
    dW1 = torch.empty(dm, 4 * D, **f32) if dW1 is None else dW1
    dW2 = torch.empty(D, dm, **f32) if dW2 is None else dW2
    if want_bias:
        db1 = torch.empty(4 * D, **f32) if db1 is None else db1
        db2 = torch.empty(dm, **f32) if db2 is None else db2
    _need(dX, "dX", dt, dev, T * dm)
    _need(dW1, "dW1", torch.float32, dev, dm * 4 * D)
    _need(dW2, "dW2", torch.float32, dev, D * dm)
    _need(db1, "db1", torch.float32, dev, 4 * D)
    _need(db2, "db2", torch.float32, dev, dm)
    if p.rab_p and d_rab_p is None:
        d_rab_p = torch.empty(p.n_pos, **f32)
    if p.rab_t and d_rab_t is None:
        d_rab_t = torch.empty(p.n_tb, **f32)
    G = p.n_groups if p.norm == HSTU_NORM_GLN else 1
    if want_affine and p.gamma and d_gamma is None:
        d_gamma = torch.empty(G, D, **f32)
    if want_affine and p.beta and d_beta is None:
        d_beta = torch.empty(G, D, **f32)
    if ws is None:
        ws = workspace(layer_workspace_size(p, dm, HSTU_OP_BWD), dev)
    L.check(L.lib().hstu_layer_bwd(
        ctypes.byref(p), ctypes.byref(w), _ptr(X), _ptr(f.Z), _ptr(getattr(f, "UVQK", None)), _ptr(f.Y), _ptr(f.O),
        _ptr(f.mean), _ptr(f.rstd),
        _ptr(dOut), _ptr(dX), _ptr(dW1), _ptr(db1), _ptr(dW2), _ptr(db2), _ptr(d_rab_p), _ptr(d_rab_t),
        _ptr(d_gamma), _ptr(d_beta), _ptr(ws), ws.numel(), _stream(stream)))
    return SimpleNamespace(dX=dX, dW1=dW1, db1=db1, dW2=dW2, db2=db2, d_rab_p=d_rab_p, d_rab_t=d_rab_t,
                           d_gamma=d_gamma, d_beta=d_beta, ws=ws)


def stack_layers(layers, H, d, dtype, device, K_caches=None, V_caches=None, hist_tokens=0):
    """The hstu_stack_layer_t array of a list of per-layer dicts (W1, W2 in
    dtype; optional fp32 b1, b2, rab_p, rab_t, gamma, beta; device tensors).
    K/V caches ([Th, H, d] each per layer) are allocated when not given.
    Returns (ctypes array, K_caches, V_caches)."""
    n = len(layers)
    arr = (L.StackLayer * n)()
    Ks = K_caches or [torch.empty(hist_tokens, H, d, dtype=dtype, device=device) for _ in range(n)]
    Vs = V_caches or [torch.empty(hist_tokens, H, d, dtype=dtype, device=device) for _ in range(n)]
    keep = []
    for i, lay in enumerate(layers):
        w = layer_weights(lay["W1"], lay["W2"], lay.get("b1"), lay.get("b2"))
        arr[i].w = w
        for name in ("rab_p", "rab_t", "gamma", "beta"):
            t = lay.get(name)
            _need(t, name, torch.float32, device)
            setattr(arr[i], name, _ptr(t))
        _need(Ks[i], "K_cache", dtype, device, hist_tokens * H * d)
        _need(Vs[i], "V_cache", dtype, device, hist_tokens * H * d)
        arr[i].K_cache, arr[i].V_cache = _ptr(Ks[i]), _ptr(Vs[i])
        keep.append((w, lay))
    arr._keep = (keep, Ks, Vs)
    return arr, Ks, Vs


def stack_workspace_size(p, d_model, op, microbatch=0, hist_max_len=0, hist_tokens=0) -> int:
    n = ctypes.c_size_t(0)
    L.check(L.lib().hstu_stack_workspace_size(ctypes.byref(p), int(d_model), op, int(microbatch), int(hist_max_len),
                                              int(hist_tokens), ctypes.byref(n)))
    return int(n.value)


def stack_history(hist_p, layers, X, *, Out=None, ws=None, stream=None):
    """hstu_stack_history. layers: the array from stack_layers. Returns a
    namespace with Out ([Th, d_model], the last layer's output) and ws."""
    dm = layers[0].w.d_model
    T, dev, dt = hist_p.total_tokens, X.device, X.dtype
    _need(X, "X", dt, dev, T * dm)
    Out = torch.empty(T, dm, dtype=dt, device=dev) if Out is None else Out
    _need(Out, "Out", dt, dev, T * dm)
    if ws is None:
        ws = workspace(stack_workspace_size(hist_p, dm, HSTU_OP_FWD), dev)
    L.check(L.lib().hstu_stack_history(ctypes.byref(hist_p), len(layers), layers, _ptr(X), _ptr(Out), _ptr(ws),
                                       ws.numel(), _stream(stream)))
    return SimpleNamespace(Out=Out, ws=ws)


def _stack_score_args(cand_p, layers, hist_offsets, hist_tokens, hist_max_len, hist_ts, microbatch, Xc, Out, ws):
    dm = layers[0].w.d_model
    T, dev, dt = cand_p.total_tokens, Xc.device, Xc.dtype
    _need(Xc, "Xc", dt, dev, T * dm)
    _need(hist_offsets, "hist_offsets", torch.int32, dev, cand_p.B + 1)
    _need(hist_ts, "hist_ts", torch.int64, dev, int(hist_tokens))
    Out = torch.empty(T, dm, dtype=dt, device=dev) if Out is None else Out
    _need(Out, "Out", dt, dev, T * dm)
    if ws is None:
        ws = workspace(stack_workspace_size(cand_p, dm, HSTU_OP_MFALCON, microbatch, hist_max_len, hist_tokens), dev)
    args = (ctypes.byref(cand_p), len(layers), layers, _ptr(hist_offsets), int(hist_tokens), int(hist_max_len),
            _ptr(hist_ts), int(microbatch), _ptr(Xc), _ptr(Out), _ptr(ws), ws.numel())
    return args, Out, ws


def stack_score(cand_p, layers, hist_offsets, hist_tokens, hist_max_len, Xc, *, hist_ts=None, microbatch=0,
                Out=None, ws=None, stream=None):
    """hstu_stack_score. Returns a namespace with Out ([Tc, d_model]) and ws."""
    args, Out, ws = _stack_score_args(cand_p, layers, hist_offsets, hist_tokens, hist_max_len, hist_ts, microbatch,
                                      Xc, Out, ws)
    L.check(L.lib().hstu_stack_score(*args, _stream(stream)))
    return SimpleNamespace(Out=Out, ws=ws)


class Graph:
    """An executable HIP graph of one hstu_stack_score call
    (hstu_stack_score_capture); launch() replays it, the graph is freed
    with the object. Keeps the captured buffers alive."""

    def __init__(self, handle, keep):
        self._h = handle
        self._keep = keep

    def launch(self, stream=None):
        L.check(L.lib().hstu_graph_launch(self._h, _stream(stream)))

    def __del__(self):
        if getattr(self, "_h", None):
            L.lib().hstu_graph_destroy(self._h)
            self._h = None


def stack_score_capture(cand_p, layers, hist_offsets, hist_tokens, hist_max_len, Xc, *, hist_ts=None,
                        microbatch=0, Out=None, ws=None):
    """hstu_stack_score_capture. Returns (Graph, namespace with Out and ws)."""
    args, Out, ws = _stack_score_args(cand_p, layers, hist_offsets, hist_tokens, hist_max_len, hist_ts, microbatch,
                                      Xc, Out, ws)
    h = ctypes.c_void_p(0)
    L.check(L.lib().hstu_stack_score_capture(*args, ctypes.byref(h)))
    return Graph(h, (cand_p, layers, hist_offsets, hist_ts, Xc, Out, ws)), SimpleNamespace(Out=Out, ws=ws)
