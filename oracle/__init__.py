"""CPU oracle for HSTU jagged pointwise attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It wraps ``oracle.c`` (plain fp64 loops,
OpenMP over (sequence, head)) through ctypes and adds small pieces of pure
Python: the tile schedule built from the brute-force tile classifier, and the
two orders of the query tiles (longest first, and by sequence).

Everything here takes numpy arrays; floating-point inputs are converted to
float64 (bf16 and fp32 values are represented exactly). Nothing here imports
the HIP package, and the HIP package never imports this one.

What is pinned and how is described in the header of ``oracle.c``. Every
function below has a pin in the CPU test suite; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

NORM_NONE, NORM_LN, NORM_GLN = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall", "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = ctypes.CDLL(_LIB_PATH)
        _lib.oracle_time_bucket.restype = ctypes.c_int
        _lib.oracle_time_bucket.argtypes = [ctypes.c_int64, ctypes.c_int]
        _lib.oracle_visible.restype = ctypes.c_int
        _lib.oracle_visible.argtypes = [ctypes.c_int] * 5
        _lib.oracle_classify_tiles.restype = ctypes.c_int
        _lib.oracle_classify_tiles.argtypes = [ctypes.c_int] * 7 + [ctypes.c_void_p]
        _lib.oracle_classify_tiles_tf.restype = ctypes.c_int
        _lib.oracle_classify_tiles_tf.argtypes = [ctypes.c_int] * 8 + [ctypes.c_void_p]
        for name in ("oracle_fwd", "oracle_bwd", "oracle_mfalcon"):
            getattr(_lib, name).restype = ctypes.c_int
    return _lib


def _p(a):
    """Pointer of a numpy array, or NULL for None."""
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _f64(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _i64(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _u8(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.uint8))


def _threads(nthreads):
    return int(nthreads) if nthreads else (os.cpu_count() or 1)


def time_bucket(dt: int, n_tb: int) -> int:
    return int(_load().oracle_time_bucket(int(dt), int(n_tb)))


def visible(i: int, j: int, L: int, P: int, C: int) -> bool:
    return bool(_load().oracle_visible(int(i), int(j), int(L), int(P), int(C)))


def fwd(offsets, Q, K, V, U, *, H, d, prefix_len=None, cand_len=None, ts=None, rab_p=None,
        rab_t=None, n_max=1.0, norm=NORM_LN, eps=1e-5, group=None, n_groups=1, gamma=None,
        beta=None, row_sel=None, time_filter=False, nthreads=0):
    """Forward pass. Q/K/V/U: [T, H, d] (any float dtype). Returns dict with
    Y, O ([T, H*d] float64), mean, rstd ([T] float64). time_filter: MTGR's
    timestamp filter (a candidate sees a causal-segment key only if the key
    is strictly earlier)."""
    lib = _load()
    offsets = _i32(offsets)
    B = len(offsets) - 1
    T = int(offsets[-1])
    D = H * d
    Q, K, V, U = (_f64(x).reshape(T, D) for x in (Q, K, V, U))
    rp, rt = _f64(rab_p), _f64(rab_t)
    gm, bt = _f64(gamma), _f64(beta)
    Y = np.zeros((T, D)); O = np.zeros((T, D)); mean = np.zeros(T); rstd = np.zeros(T)
    pl, cl, ts_, grp, sel = _i32(prefix_len), _i32(cand_len), _i64(ts), _u8(group), _u8(row_sel)
    rc = lib.oracle_fwd(
        ctypes.c_int(B), ctypes.c_int(H), ctypes.c_int(d), _p(offsets), _p(pl), _p(cl),
        _p(Q), _p(K), _p(V), _p(U), _p(ts_),
        _p(rp), ctypes.c_int(0 if rp is None else len(rp)),
        _p(rt), ctypes.c_int(0 if rt is None else len(rt)),
        ctypes.c_double(n_max), ctypes.c_int(norm), ctypes.c_double(eps),
        _p(grp), ctypes.c_int(n_groups), _p(gm), _p(bt), _p(sel),
        _p(Y), _p(O), _p(mean), _p(rstd), ctypes.c_int(int(bool(time_filter))),
        ctypes.c_int(_threads(nthreads)))
    if rc != 0:
        raise ValueError(f"oracle_fwd rejected its input (code {rc})")
    return {"Y": Y, "O": O, "mean": mean, "rstd": rstd}


def bwd(offsets, Q, K, V, U, dY, *, H, d, prefix_len=None, cand_len=None, ts=None, rab_p=None,
        rab_t=None, n_max=1.0, norm=NORM_LN, eps=1e-5, group=None, n_groups=1, gamma=None,
        beta=None, time_filter=False, nthreads=0):
    """Backward pass (recomputes the forward). Returns dict with dQ, dK, dV,
    dU ([T, H*d]), drab_p, drab_t, dgamma, dbeta (None when not applicable),
    and drab_p_abs / drab_t_abs: the sums of |dS| that enter each rab entry."""
    lib = _load()
    offsets = _i32(offsets)
    B = len(offsets) - 1
    T = int(offsets[-1])
    D = H * d
    Q, K, V, U, dY = (_f64(x).reshape(T, D) for x in (Q, K, V, U, dY))
    rp, rt = _f64(rab_p), _f64(rab_t)
    gm, bt = _f64(gamma), _f64(beta)
    G = n_groups if norm == NORM_GLN else 1
    dQ, dK, dV, dU = (np.zeros((T, D)) for _ in range(4))
    drp = np.zeros(len(rp)) if rp is not None else None
    drt = np.zeros(len(rt)) if rt is not None else None
    dgm = np.zeros((G, D)) if gm is not None else None
    dbt = np.zeros((G, D)) if bt is not None else None
    drpa = np.zeros(len(rp)) if rp is not None else None
    drta = np.zeros(len(rt)) if rt is not None else None
    pl, cl, ts_, grp = _i32(prefix_len), _i32(cand_len), _i64(ts), _u8(group)
    rc = lib.oracle_bwd(
        ctypes.c_int(B), ctypes.c_int(H), ctypes.c_int(d), _p(offsets), _p(pl), _p(cl),
        _p(Q), _p(K), _p(V), _p(U), _p(ts_),
        _p(rp), ctypes.c_int(0 if rp is None else len(rp)),
        _p(rt), ctypes.c_int(0 if rt is None else len(rt)),
        ctypes.c_double(n_max), ctypes.c_int(norm), ctypes.c_double(eps),
        _p(grp), ctypes.c_int(n_groups), _p(gm), _p(bt), _p(dY),
        _p(dQ), _p(dK), _p(dV), _p(dU), _p(drp), _p(drt), _p(dgm), _p(dbt), _p(drpa), _p(drta),
        ctypes.c_int(int(bool(time_filter))), ctypes.c_int(_threads(nthreads)))
    if rc != 0:
        raise ValueError(f"oracle_bwd rejected its input (code {rc})")
    return {"dQ": dQ, "dK": dK, "dV": dV, "dU": dU, "drab_p": drp, "drab_t": drt,
            "dgamma": dgm, "dbeta": dbt, "drab_p_abs": drpa, "drab_t_abs": drta}


def mfalcon(hist_offsets, cand_offsets, K_cache, V_cache, Qc, Kc, Vc, Uc, *, H, d, hist_ts=None,
            cand_ts=None, rab_p=None, rab_t=None, n_max=1.0, norm=NORM_LN, eps=1e-5,
            cand_group=None, n_groups=1, gamma=None, beta=None, time_filter=False, nthreads=0):
    """M-FALCON scoring of candidates against cached history K/V. Returns dict
    with Y, O ([Tc, H*d]), mean, rstd ([Tc])."""
    lib = _load()
    ho, co = _i32(hist_offsets), _i32(cand_offsets)
    B = len(co) - 1
    Th, Tc = int(ho[-1]), int(co[-1])
    D = H * d
    Kh, Vh = (_f64(x).reshape(Th, D) for x in (K_cache, V_cache))
    Qc, Kc, Vc, Uc = (_f64(x).reshape(Tc, D) for x in (Qc, Kc, Vc, Uc))
    rp, rt = _f64(rab_p), _f64(rab_t)
    gm, bt = _f64(gamma), _f64(beta)
    Y = np.zeros((Tc, D)); O = np.zeros((Tc, D)); mean = np.zeros(Tc); rstd = np.zeros(Tc)
    hts, cts, grp = _i64(hist_ts), _i64(cand_ts), _u8(cand_group)
    rc = lib.oracle_mfalcon(
        ctypes.c_int(B), ctypes.c_int(H), ctypes.c_int(d), _p(ho), _p(co), _p(Kh), _p(Vh), _p(hts),
        _p(Qc), _p(Kc), _p(Vc), _p(Uc), _p(cts),
        _p(rp), ctypes.c_int(0 if rp is None else len(rp)),
        _p(rt), ctypes.c_int(0 if rt is None else len(rt)),
        ctypes.c_double(n_max), ctypes.c_int(norm), ctypes.c_double(eps),
        _p(grp), ctypes.c_int(n_groups), _p(gm), _p(bt),
        _p(Y), _p(O), _p(mean), _p(rstd), ctypes.c_int(int(bool(time_filter))),
        ctypes.c_int(_threads(nthreads)))
    if rc != 0:
        raise ValueError(f"oracle_mfalcon rejected its input (code {rc})")
    return {"Y": Y, "O": O, "mean": mean, "rstd": rstd}


def classify_tiles(L, P, C, r0, nrows, BN, nkt, time_filter=False):
    """Brute-force kinds (0 absent, 1 partial, 2 full) of key tiles [0, nkt)
    for query rows [r0, r0+nrows) of a frame (L, P, C). With time_filter, a
    (candidate row, causal key) pair makes its tile present but not full."""
    kind = np.zeros(max(nkt, 1), dtype=np.int8)
    _load().oracle_classify_tiles_tf(int(L), int(P), int(C), int(r0), int(nrows), int(BN), int(nkt),
                                     int(bool(time_filter)), ctypes.c_void_p(kind.ctypes.data))
    return kind[:nkt]


def _qtile_entry(b, frame_L, P, C, frame_r0, nrows, BN, local_row0, time_filter=False):
    nkt = -(-frame_L // BN)
    kinds = classify_tiles(frame_L, P, C, frame_r0, nrows, BN, nkt, time_filter)
    return {"b": b, "row0": local_row0, "nrows": nrows, "kinds": kinds}


def schedule(offsets, BM, BN, prefix_len=None, cand_len=None, time_filter=False):
    """Query-tile schedule of the attention forward: one entry per query tile
    (sequence b, first row row0, row count nrows, kinds of its key tiles),
    canonical order (b, row0) ascending."""
    offsets = np.asarray(offsets, dtype=np.int64)
    out = []
    for b in range(len(offsets) - 1):
        L = int(offsets[b + 1] - offsets[b])
        P = int(prefix_len[b]) if prefix_len is not None else 0
        C = int(cand_len[b]) if cand_len is not None else 0
        for r0 in range(0, L, BM):
            out.append(_qtile_entry(b, L, P, C, r0, min(BM, L - r0), BN, r0, time_filter))
    return out


def schedule_mfalcon(hist_offsets, cand_offsets, BM, BN, microbatch, time_filter=False):
    """Query-tile schedule of M-FALCON scoring: the candidates of user b are
    cut into microbatches of `microbatch` candidates (0 = one microbatch), and
    each microbatch into query tiles of at most BM rows. Row indices are local
    candidate indices; the tiles are classified in the frame
    [history | candidates] with the candidate tail as the only segment."""
    ho = np.asarray(hist_offsets, dtype=np.int64)
    co = np.asarray(cand_offsets, dtype=np.int64)
    out = []
    for b in range(len(co) - 1):
        n = int(ho[b + 1] - ho[b])
        m = int(co[b + 1] - co[b])
        mb = microbatch if microbatch > 0 else max(m, 1)
        for s in range(0, m, mb):
            e = min(m, s + mb)
            for r0 in range(s, e, BM):
                nrows = min(BM, e - r0)
                out.append(_qtile_entry(b, n + m, 0, m, n + r0, nrows, BN, r0, time_filter))
    return out


def lpt_order(entries):
    """Longest-processing-time order: by number of present key tiles,
    descending; ties keep the canonical order."""
    return sorted(range(len(entries)), key=lambda g: (-int(np.count_nonzero(entries[g]["kinds"])), g))


def sequence_order(entries):
    """The by-sequence order of a query-tile schedule: whole sequences by
    their longest tile (present key tiles), descending; within a sequence its
    tiles longest first; sequences of equal length later-index first (the
    tile index breaks every tie, descending)."""
    nk = [int(np.count_nonzero(e["kinds"])) for e in entries]
    seq_len = {}
    for g, e in enumerate(entries):
        seq_len[e["b"]] = max(seq_len.get(e["b"], 0), nk[g])
    return sorted(range(len(entries)), key=lambda g: (-seq_len[entries[g]["b"]], -g))


def stochastic_length(offsets, keys, cap):
    """Stochastic Length (HSTU blog, section 3.4): a sequence longer than cap
    keeps the cap tokens with the smallest (key, index), in their order;
    shorter ones are kept whole. Returns (new_offsets, gather_idx) as int64
    arrays (gather_idx holds input token indices)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.uint32)
    new_off = [0]
    idx = []
    for b in range(len(offsets) - 1):
        s, e = int(offsets[b]), int(offsets[b + 1])
        toks = list(range(s, e))
        if len(toks) > cap:
            ranked = sorted(toks, key=lambda t: (int(keys[t]), t))
            toks = sorted(ranked[:cap])
        idx.extend(toks)
        new_off.append(new_off[-1] + len(toks))
    return np.array(new_off, dtype=np.int64), np.array(idx, dtype=np.int64)


def balance_bins(lengths, n_bins, cost_kind=0):
    """Work-balanced batching (MTGR deep read, section 2): sequences in order
    of decreasing cost (ties by index) each go to the bin with the smallest
    cost so far (ties to the lowest bin). cost_kind 0: L, 1: L * L. Returns
    (bin per sequence, cost per bin)."""
    cost = [int(L) if cost_kind == 0 else int(L) * int(L) for L in lengths]
    order = sorted(range(len(cost)), key=lambda b: (-cost[b], b))
    load = [0] * n_bins
    out = [0] * len(cost)
    for b in order:
        best = min(range(n_bins), key=lambda k: (load[k], k))
        out[b] = best
        load[best] += cost[b]
    return np.array(out, dtype=np.int64), np.array(load, dtype=np.int64)


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _silu_grad(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def layer_fwd(offsets, X, W1, W2, *, H, d, b1=None, b2=None, **attn):
    """One HSTU layer (HSTU blog, section 3, the layer formula): the input
    projection f1(X) = X W1 + b1 of width 4D, phi1 = SiLU, its column blocks
    taken as U, V, Q, K in that order, the attention core (``fwd`` above,
    keyword arguments passed through) and the output projection
    f2(Y) = Y W2 + b2 of Y = Norm(A V) * U. X: [T, d_model], W1: [d_model, 4D],
    W2: [D, d_model]. Returns dict with Out, Z (the pre-activation f1(X)), the
    split U, V, Q, K and the core's Y, O, mean, rstd."""
    D = H * d
    X, W1, W2 = _f64(X), _f64(W1), _f64(W2)
    Z = X @ W1
    if b1 is not None:
        Z = Z + _f64(b1)
    A = _silu(Z)
    U, V, Q, K = (A[:, i * D:(i + 1) * D] for i in range(4))
    core = fwd(offsets, Q, K, V, U, H=H, d=d, **attn)
    Out = core["Y"] @ W2
    if b2 is not None:
        Out = Out + _f64(b2)
    return {"Out": Out, "Z": Z, "U": U, "V": V, "Q": Q, "K": K, **core}


def layer_bwd(offsets, X, W1, W2, dOut, *, H, d, b1=None, b2=None, **attn):
    """Backward of ``layer_fwd`` by the chain rule through its steps: the
    output projection (dY = dOut W2^T, dW2 = Y^T dOut, db2 = column sums of
    dOut), the attention core (``bwd`` above), SiLU (dZ = [dU | dV | dQ | dK]
    * SiLU'(Z)) and the input projection (dW1 = X^T dZ, db1 = column sums of
    dZ, dX = dZ W1^T). Returns dict with dX, dW1, db1, dW2, db2, dZ and the
    core's drab_p, drab_t, dgamma, dbeta."""
    f = layer_fwd(offsets, X, W1, W2, H=H, d=d, b1=b1, b2=b2, **attn)
    X, W1, W2, dOut = _f64(X), _f64(W1), _f64(W2), _f64(dOut)
    attn = {k: v for k, v in attn.items() if k not in ("row_sel",)}
    dY = dOut @ W2.T
    g = bwd(offsets, f["Q"], f["K"], f["V"], f["U"], dY, H=H, d=d, **attn)
    dZ = np.concatenate([g["dU"], g["dV"], g["dQ"], g["dK"]], axis=1) * _silu_grad(f["Z"])
    return {"dX": dZ @ W1.T, "dW1": X.T @ dZ, "db1": dZ.sum(0), "dW2": f["Y"].T @ dOut,
            "db2": dOut.sum(0), "dZ": dZ, "dY": dY, "drab_p": g["drab_p"], "drab_t": g["drab_t"],
            "dgamma": g["dgamma"], "dbeta": g["dbeta"]}


def mfalcon_stack(hist_offsets, cand_offsets, X_hist, X_cand, layers, *, H, d, hist_ts=None, cand_ts=None,
                  hist_group=None, cand_group=None, n_groups=1, n_max=1.0, norm=NORM_LN, eps=1e-5,
                  time_filter=False):
    """Candidate scoring through a stack of HSTU layers (HSTU blog, sections
    4.2 and 4.3: a user's history and its candidates form one sequence, every
    candidate sees the whole history and itself, none sees another). Plain
    definition, without any cache: for each user the sequence [history |
    candidates] runs through every layer (``layer_fwd`` with P = 0 and
    C = number of candidates), each layer's output feeding the next.
    layers: list of dicts with W1, W2 and optionally b1, b2, rab_p, rab_t,
    gamma, beta. Returns dict with Out (candidate rows of the last layer,
    [Tc, d_model]) and Out_hist (history rows, [Th, d_model])."""
    ho = np.asarray(hist_offsets, dtype=np.int64)
    co = np.asarray(cand_offsets, dtype=np.int64)
    B = len(co) - 1
    Xh, Xc = _f64(X_hist), _f64(X_cand)
    rows_h, rows_c, lens, cands = [], [], [], []
    pos = 0
    for b in range(B):
        n, m = int(ho[b + 1] - ho[b]), int(co[b + 1] - co[b])
        rows_h.append(np.arange(pos, pos + n))
        rows_c.append(np.arange(pos + n, pos + n + m))
        lens.append(n + m)
        cands.append(m)
        pos += n + m
    rh = np.concatenate(rows_h) if rows_h else np.zeros(0, np.int64)
    rc = np.concatenate(rows_c) if rows_c else np.zeros(0, np.int64)
    X = np.zeros((pos, Xh.shape[1] if Xh.ndim == 2 else Xc.shape[1]))
    X[rh] = Xh
    X[rc] = Xc

    def interleave(a_h, a_c, dtype):
        if a_h is None:
            return None
        out = np.zeros(pos, dtype=dtype)
        out[rh] = np.asarray(a_h)
        out[rc] = np.asarray(a_c)
        return out

    ts = interleave(hist_ts, cand_ts, np.int64)
    grp = interleave(hist_group, cand_group, np.uint8)
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    for lay in layers:
        X = layer_fwd(offsets, X, lay["W1"], lay["W2"], H=H, d=d, b1=lay.get("b1"), b2=lay.get("b2"),
                      cand_len=np.asarray(cands, np.int32), ts=ts, rab_p=lay.get("rab_p"), rab_t=lay.get("rab_t"),
                      n_max=n_max, norm=norm, eps=eps, group=grp, n_groups=n_groups, gamma=lay.get("gamma"),
                      beta=lay.get("beta"), time_filter=time_filter)["Out"]
    return {"Out": X[rc], "Out_hist": X[rh]}
