"""Pins of the CPU oracle against things other than itself: hand-typed mask
and schedule fixtures, integer bucket boundaries, the L = 1 closed form,
torch library routines for the dense special cases, exact invariants, torch
autograd and central finite differences for the backward."""
import math
import os

import numpy as np
import pytest
import torch

from hstu_jagged_pointwise_attn_amd import synth
from tests import dense_torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_blocks(name):
    lines = [l.rstrip("\n") for l in open(os.path.join(GOLDEN, name))]
    return [l for l in lines if l and not l.startswith("#")]


def _masks():
    out, lines, k = [], _read_blocks("masks.txt"), 0
    while k < len(lines):
        l = lines[k]
        if l.startswith("mask"):
            kv = dict(x.split("=") for x in l.split()[1:])
            L, P, C = int(kv["L"]), int(kv["P"]), int(kv["C"])
            rows = lines[k + 1:k + 1 + L]
            assert lines[k + 1 + L] == "end"
            out.append((L, P, C, np.array([[int(c) for c in r] for r in rows])))
            k += L + 2
        else:
            k += 1
    return out


def _positions():
    out = []
    for l in _read_blocks("masks.txt"):
        if l.startswith("pos"):
            head, vals = l.split(":")
            kv = dict(x.split("=") for x in head.split()[1:])
            out.append((int(kv["L"]), int(kv["C"]), [int(v) for v in vals.split()]))
    return out


# ------------------------------------------------------------------ masks

@pytest.mark.parametrize("case", _masks(), ids=lambda c: f"L{c[0]}P{c[1]}C{c[2]}")
def test_visibility_matches_hand_fixture(oracle_mod, case):
    L, P, C, expected = case
    got = np.array([[int(oracle_mod.visible(i, j, L, P, C)) for j in range(L)] for i in range(L)])
    np.testing.assert_array_equal(got, expected)
    np.testing.assert_array_equal(dense_torch.block_mask(L, P, C).int().numpy(), expected)


@pytest.mark.parametrize("case", _positions(), ids=lambda c: f"L{c[0]}C{c[1]}")
def test_positions_read_out_through_rab_p(oracle_mod, case):
    """With Q = 0, V = identity, N_max = 1, no norm and U = 1, the output
    matrix is the attention matrix itself: O[i, j] = SiLU(rab_p[|pos i - pos j|])
    on visible pairs. Distinct rab_p entries make each position readable."""
    L, C, pos = case
    P = 0
    n_pos = 16
    rab_p = np.array([0.25 * k - 1.0 for k in range(n_pos)])
    Q = np.zeros((L, 1, L)); K = np.random.default_rng(0).normal(size=(L, 1, L))
    V = np.eye(L).reshape(L, 1, L); U = np.ones((L, 1, L))
    r = oracle_mod.fwd([0, L], Q, K, V, U, H=1, d=L, cand_len=[C], prefix_len=[P], rab_p=rab_p,
                       n_max=1.0, norm=oracle_mod.NORM_NONE)
    for i in range(L):
        for j in range(L):
            vis = oracle_mod.visible(i, j, L, P, C)
            x = rab_p[min(abs(pos[i] - pos[j]), n_pos - 1)]
            want = x / (1 + math.exp(-x)) if vis else 0.0
            assert r["O"][i, j] == pytest.approx(want, rel=1e-15, abs=0)


# ------------------------------------------------------------------ buckets

def test_time_bucket_integer_boundaries(oracle_mod):
    for n_tb in (16, 128):
        cases = [0, 1, -1]
        for k in range(1, 63):
            cases += [2 ** k - 1, 2 ** k, 2 ** k + 1, -(2 ** k - 1), -(2 ** k), -(2 ** k + 1)]
        for dt in cases:
            want = min(n_tb - 1, max(1, abs(dt)).bit_length() - 1)
            assert oracle_mod.time_bucket(dt, n_tb) == want, (dt, n_tb)


def test_time_bucket_frexp_agrees(oracle_mod):
    dts = torch.tensor([0, 1, 2, 3, 4, 7, 8, 3599, 3600, 86399, 86400, -5, -(2 ** 40)], dtype=torch.int64)
    got = [oracle_mod.time_bucket(int(x), 128) for x in dts]
    assert got == dense_torch.bucket(dts, 128).tolist()


# ------------------------------------------------------------------ forward

def test_single_token_closed_form(oracle_mod):
    """L = 1: y = LN(SiLU(q.k + rab_p[0] + rab_t[0]) v / N_max) * u over all heads."""
    rng = np.random.default_rng(1)
    H, d = 2, 4
    q, k, v, u = (rng.normal(size=(1, H, d)) for _ in range(4))
    rab_p, rab_t = np.array([0.3, -1.0]), np.array([-0.2, 5.0])
    r = oracle_mod.fwd([0, 1], q, k, v, u, H=H, d=d, ts=[123], rab_p=rab_p, rab_t=rab_t,
                       n_max=2.0, norm=oracle_mod.NORM_LN, eps=1e-5)
    x = []
    for h in range(H):
        s = float(np.dot(q[0, h], k[0, h])) + 0.3 - 0.2
        a = s / (1 + math.exp(-s)) / 2.0
        x += [a * float(vv) for vv in v[0, h]]
    mu = sum(x) / len(x)
    var = sum((t - mu) ** 2 for t in x) / len(x)
    y = [(t - mu) / math.sqrt(var + 1e-5) * float(uu) for t, uu in zip(x, u.reshape(-1))]
    np.testing.assert_allclose(r["Y"][0], y, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["O"][0], x, rtol=1e-13, atol=0)


def _torch_inputs(p):
    f = lambda t: t.double().clone()
    return f(p.Q), f(p.K), f(p.V), f(p.U)


def _dense_opts(p):
    return dict(H=p.H, d=p.d, prefix_len=p.prefix_len, cand_len=p.cand_len, ts=p.ts,
                rab_p=None if p.rab_p is None else torch.tensor(p.rab_p, dtype=torch.float64),
                rab_t=None if p.rab_t is None else torch.tensor(p.rab_t, dtype=torch.float64),
                n_max=float(p.n_max), norm=p.norm, eps=p.eps, group=p.group,
                gamma=None if p.gamma is None else torch.tensor(p.gamma, dtype=torch.float64),
                beta=None if p.beta is None else torch.tensor(p.beta, dtype=torch.float64),
                time_filter=p.time_filter)


def _oracle_opts(p):
    return dict(H=p.H, d=p.d, prefix_len=p.prefix_len, cand_len=p.cand_len, ts=p.ts, rab_p=p.rab_p,
                rab_t=p.rab_t, n_max=p.n_max, norm=p.norm, eps=p.eps, group=p.group,
                n_groups=p.n_groups, gamma=p.gamma, beta=p.beta, time_filter=p.time_filter)


def _small_problems():
    """Small problems covering every mask kind, rab on/off, the norms."""
    out = []
    out.append(synth.custom("causal_rab", [5, 17, 1, 30], H=2, d=8, dtype=torch.float32, wid=11,
                            std=0.5, n_max=4, norm=synth.NORM_LN, n_pos=12, n_tb=8, rab_std=0.5))
    L = np.array([12, 20, 7, 9])
    P = np.array([3, 5, 0, 9]); C = np.array([4, 6, 7, 0])
    grp = np.concatenate([np.minimum(np.arange(l) * 3 // max(l, 1), 2) for l in L])
    out.append(synth.custom("mtgr_gln", L, H=3, d=4, dtype=torch.float32, wid=12, std=0.7, n_max=2,
                            norm=synth.NORM_GLN, prefix_len=P, cand_len=C, group=grp, n_groups=3,
                            gamma_std=0.3, beta_std=0.3, n_pos=8, n_tb=6, rab_std=0.4))
    out.append(synth.custom("none_norm", [6, 0, 11], H=1, d=16, dtype=torch.bfloat16, wid=13,
                            std=0.5, n_max=1, norm=synth.NORM_NONE, cand_len=[2, 0, 5]))
    return out


@pytest.mark.parametrize("p", _small_problems(), ids=lambda p: p.name)
def test_forward_matches_torch_library_dense(oracle_mod, p):
    Q, K, V, U = _torch_inputs(p)
    Yd, Od = dense_torch.forward(p.offsets, Q, K, V, U, **_dense_opts(p))
    r = oracle_mod.fwd(p.offsets, p.Q.double().numpy(), p.K.double().numpy(), p.V.double().numpy(),
                       p.U.double().numpy(), **_oracle_opts(p))
    np.testing.assert_allclose(r["O"], Od.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(r["Y"], Yd.numpy(), rtol=1e-10, atol=1e-12)


def test_zero_queries_give_zero_output(oracle_mod):
    """Q = 0 with zero rab: S = 0, SiLU(0) = 0, so O = 0 and Y = beta * U."""
    p = synth.custom("zq", [9, 4, 13], H=2, d=8, dtype=torch.float32, wid=14, std=1.0, n_max=3,
                     norm=synth.NORM_LN, beta_std=1.0, gamma_std=1.0, cand_len=[3, 0, 5],
                     n_pos=10, n_tb=5)
    p.rab_p[:] = 0
    p.rab_t[:] = 0
    Q = np.zeros((p.T, p.H, p.d))
    r = oracle_mod.fwd(p.offsets, Q, p.K.numpy(), p.V.numpy(), p.U.numpy(), **_oracle_opts(p))
    assert np.all(r["O"] == 0.0)
    np.testing.assert_array_equal(r["Y"], p.beta[0][None, :] * p.U.double().numpy().reshape(p.T, -1))


def test_masked_pairs_contribute_exactly_zero(oracle_mod):
    """Perturbing K/V of keys a row cannot see leaves that row bit-identical."""
    L = np.array([10, 16])
    P = np.array([2, 4]); C = np.array([3, 5])
    p = synth.custom("mz", L, H=2, d=8, dtype=torch.float32, wid=15, std=0.5, n_max=4,
                     norm=synth.NORM_NONE, prefix_len=P, cand_len=C, n_pos=8, n_tb=4)
    base = oracle_mod.fwd(p.offsets, p.Q.numpy(), p.K.numpy(), p.V.numpy(), p.U.numpy(), **_oracle_opts(p))
    for b in range(2):
        s, Lb, Pb, Cb = int(p.offsets[b]), int(L[b]), int(P[b]), int(C[b])
        for j in range(Lb):
            K2, V2 = p.K.numpy().copy(), p.V.numpy().copy()
            K2[s + j] += 3.0
            V2[s + j] -= 7.0
            r = oracle_mod.fwd(p.offsets, p.Q.numpy(), K2, V2, p.U.numpy(), **_oracle_opts(p))
            for i in range(Lb):
                if not oracle_mod.visible(i, j, Lb, Pb, Cb):
                    np.testing.assert_array_equal(r["O"][s + i], base["O"][s + i])
                    np.testing.assert_array_equal(r["Y"][s + i], base["Y"][s + i])


def test_none_norm_scales_exactly_with_power_of_two_nmax(oracle_mod):
    p = synth.custom("sc", [7, 12], H=2, d=8, dtype=torch.float32, wid=16, std=0.5, n_max=1,
                     norm=synth.NORM_NONE, n_pos=6, n_tb=4, cand_len=[2, 3])
    a = oracle_mod.fwd(p.offsets, p.Q.numpy(), p.K.numpy(), p.V.numpy(), p.U.numpy(),
                       **{**_oracle_opts(p), "n_max": 1})
    b = oracle_mod.fwd(p.offsets, p.Q.numpy(), p.K.numpy(), p.V.numpy(), p.U.numpy(),
                       **{**_oracle_opts(p), "n_max": 8})
    np.testing.assert_array_equal(a["O"] / 8.0, b["O"])


# ------------------------------------------------------------------ M-FALCON

def _mf_small(with_rab=True, users=3, n=37, m=19, H=2, d=8):
    mf = synth.mfalcon_bf16(users=users, n_hist=n, m_cand=m, microbatch=5, H=H, d=d, with_rab=with_rab)
    if with_rab:
        mf.rab_p = mf.rab_p[:64].copy()
    return mf


def _mf_oracle(oracle_mod, mf, cand_rows=None, cand_offsets=None):
    f = lambda t: t.double().numpy()
    sel = slice(None) if cand_rows is None else cand_rows
    cts = None if mf.cand_ts is None else mf.cand_ts[sel]
    return oracle_mod.mfalcon(mf.hist_offsets, mf.cand_offsets if cand_offsets is None else cand_offsets,
                              f(mf.K_cache), f(mf.V_cache), f(mf.Qc)[sel], f(mf.Kc)[sel], f(mf.Vc)[sel],
                              f(mf.Uc)[sel], H=mf.H, d=mf.d, hist_ts=mf.hist_ts, cand_ts=cts,
                              rab_p=mf.rab_p, rab_t=mf.rab_t, n_max=mf.n_max, norm=mf.norm, eps=mf.eps,
                              time_filter=mf.time_filter)


@pytest.mark.parametrize("time_filter", [False, True])
def test_mfalcon_cached_equals_full_pass(oracle_mod, time_filter):
    """Scoring against cached history K/V equals the candidate rows of one
    full pass over [history | candidates] with the candidate mask."""
    mf = _mf_small()
    if time_filter:
        # candidate times among the history times, so the filter bites
        rng = np.random.default_rng(5)
        for b in range(mf.B):
            hs, he, cs, ce = mf.hist_offsets[b], mf.hist_offsets[b + 1], mf.cand_offsets[b], mf.cand_offsets[b + 1]
            mf.cand_ts[cs:ce] = mf.hist_ts[rng.integers(hs, he, size=ce - cs)] + rng.integers(0, 2, size=ce - cs)
        mf.time_filter = True
    got = _mf_oracle(oracle_mod, mf)
    ho, co = mf.hist_offsets, mf.cand_offsets
    f = lambda t: t.double().numpy()
    Qs, Ks, Vs, Us, ts, lengths, cand = [], [], [], [], [], [], []
    for b in range(mf.B):
        hs, he, cs, ce = ho[b], ho[b + 1], co[b], co[b + 1]
        Qs += [f(mf.Q_hist)[hs:he], f(mf.Qc)[cs:ce]]
        Ks += [f(mf.K_cache)[hs:he], f(mf.Kc)[cs:ce]]
        Vs += [f(mf.V_cache)[hs:he], f(mf.Vc)[cs:ce]]
        Us += [f(mf.U_hist)[hs:he], f(mf.Uc)[cs:ce]]
        ts += [mf.hist_ts[hs:he], mf.cand_ts[cs:ce]]
        lengths.append(he - hs + ce - cs)
        cand.append(ce - cs)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    full = oracle_mod.fwd(off, np.concatenate(Qs), np.concatenate(Ks), np.concatenate(Vs),
                          np.concatenate(Us), H=mf.H, d=mf.d, cand_len=cand, ts=np.concatenate(ts),
                          rab_p=mf.rab_p, rab_t=mf.rab_t, n_max=mf.n_max, norm=mf.norm, eps=mf.eps,
                          time_filter=time_filter)
    rows = np.concatenate([np.arange(off[b + 1] - cand[b], off[b + 1]) for b in range(mf.B)])
    np.testing.assert_array_equal(got["Y"], full["Y"][rows])
    np.testing.assert_array_equal(got["O"], full["O"][rows])


def test_mfalcon_microbatches_equal_one_pass(oracle_mod):
    mf = _mf_small()
    full = _mf_oracle(oracle_mod, mf)
    co = mf.cand_offsets
    for mb in (1, 4, 7):
        for start in range(0, int(np.max(np.diff(co))), mb):
            rows, counts = [], []
            for b in range(mf.B):
                s, e = co[b] + start, min(co[b + 1], co[b] + start + mb)
                rows += list(range(s, max(s, e)))
                counts.append(max(0, e - s))
            sub_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
            r = _mf_oracle(oracle_mod, mf, cand_rows=np.array(rows), cand_offsets=sub_off)
            np.testing.assert_array_equal(r["Y"], full["Y"][rows])


def test_mfalcon_candidate_permutation_permutes_outputs(oracle_mod):
    mf = _mf_small()
    base = _mf_oracle(oracle_mod, mf)
    rng = np.random.default_rng(5)
    perm = np.concatenate([mf.cand_offsets[b] + rng.permutation(mf.cand_offsets[b + 1] - mf.cand_offsets[b])
                           for b in range(mf.B)])
    r = _mf_oracle(oracle_mod, mf, cand_rows=perm)
    np.testing.assert_array_equal(r["Y"], base["Y"][perm])


# ------------------------------------------------------------------ backward

def _grad_problems():
    out = []
    out.append(synth.custom("g_causal", [6, 11, 1], H=2, d=4, dtype=torch.float32, wid=21, std=0.6,
                            n_max=2, norm=synth.NORM_LN, n_pos=8, n_tb=6, rab_std=0.5,
                            gamma_std=0.3, beta_std=0.3, with_dy=True))
    L = np.array([9, 13])
    grp = np.concatenate([np.arange(l) % 3 for l in L])
    out.append(synth.custom("g_mtgr", L, H=2, d=4, dtype=torch.float32, wid=22, std=0.6, n_max=1,
                            norm=synth.NORM_GLN, prefix_len=[3, 4], cand_len=[2, 5], group=grp,
                            n_groups=3, gamma_std=0.3, beta_std=0.3, n_pos=8, n_tb=6, rab_std=0.5,
                            with_dy=True))
    out.append(synth.custom("g_none", [7, 5], H=1, d=8, dtype=torch.float32, wid=23, std=0.6, n_max=3,
                            norm=synth.NORM_NONE, cand_len=[3, 0], with_dy=True))
    return out


@pytest.mark.parametrize("p", _grad_problems(), ids=lambda p: p.name)
def test_backward_matches_torch_autograd(oracle_mod, p):
    Q, K, V, U = (t.requires_grad_(True) for t in _torch_inputs(p))
    opts = _dense_opts(p)
    params = [opts[k] for k in ("rab_p", "rab_t", "gamma", "beta") if opts[k] is not None]
    for t in params:
        t.requires_grad_(True)
    Y, _ = dense_torch.forward(p.offsets, Q, K, V, U, **opts)
    (Y * p.dY.double()).sum().backward()
    r = oracle_mod.bwd(p.offsets, p.Q.numpy(), p.K.numpy(), p.V.numpy(), p.U.numpy(), p.dY.numpy(),
                       **_oracle_opts(p))
    T, D = p.T, p.H * p.d
    for name, t in (("dQ", Q), ("dK", K), ("dV", V), ("dU", U)):
        np.testing.assert_allclose(r[name], t.grad.reshape(T, D).numpy(), rtol=1e-9, atol=1e-12, err_msg=name)
    for name, key in (("drab_p", "rab_p"), ("drab_t", "rab_t"), ("dgamma", "gamma"), ("dbeta", "beta")):
        if opts[key] is not None:
            np.testing.assert_allclose(r[name], opts[key].grad.numpy(), rtol=1e-9, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("p", _grad_problems(), ids=lambda p: p.name)
def test_backward_matches_central_differences_of_forward(oracle_mod, p):
    """<grad, delta> against (f(x + h delta) - f(x - h delta)) / 2h with
    f = sum(Y * dY) evaluated by oracle_fwd itself."""
    base = {k: v for k, v in dict(Q=p.Q.numpy(), K=p.K.numpy(), V=p.V.numpy(), U=p.U.numpy()).items()}
    base = {k: np.asarray(v, dtype=np.float64) for k, v in base.items()}
    extra = {k: np.asarray(getattr(p, k), dtype=np.float64) for k in ("rab_p", "rab_t", "gamma", "beta")
             if getattr(p, k) is not None}
    dY = p.dY.double().numpy()
    opts = _oracle_opts(p)

    def f(vals):
        o = dict(opts)
        for k in extra:
            o[k] = vals[k]
        return float((oracle_mod.fwd(p.offsets, vals["Q"], vals["K"], vals["V"], vals["U"], **o)["Y"] * dY).sum())

    g = oracle_mod.bwd(p.offsets, base["Q"], base["K"], base["V"], base["U"], dY, **opts)
    gname = {"Q": "dQ", "K": "dK", "V": "dV", "U": "dU", "rab_p": "drab_p", "rab_t": "drab_t",
             "gamma": "dgamma", "beta": "dbeta"}
    rng = np.random.default_rng(3)
    allv = {**base, **extra}
    h = 1e-5
    for k in allv:
        for _ in range(2):
            delta = rng.normal(size=allv[k].shape)
            plus = {**allv, k: allv[k] + h * delta}
            minus = {**allv, k: allv[k] - h * delta}
            fd = (f(plus) - f(minus)) / (2 * h)
            an = float((g[gname[k]].reshape(delta.shape) * delta).sum())
            assert an == pytest.approx(fd, rel=1e-6, abs=1e-9), k


@pytest.mark.parametrize("p", _grad_problems(), ids=lambda p: p.name)
def test_backward_identities(oracle_mod, p):
    """<Q, dQ> = <K, dK> per (sequence, head); sum(drab_p) = sum(drab_t);
    LN backward makes every token's dO sum to zero (checked through dQ/dK
    indirectly via the first identity)."""
    r = oracle_mod.bwd(p.offsets, p.Q.numpy(), p.K.numpy(), p.V.numpy(), p.U.numpy(), p.dY.numpy(),
                       **_oracle_opts(p))
    T, H, d = p.T, p.H, p.d
    Q = p.Q.double().numpy().reshape(T, H, d); K = p.K.double().numpy().reshape(T, H, d)
    dQ = r["dQ"].reshape(T, H, d); dK = r["dK"].reshape(T, H, d)
    for b in range(p.B):
        s, e = p.offsets[b], p.offsets[b + 1]
        for h in range(H):
            a = float((Q[s:e, h] * dQ[s:e, h]).sum()); c = float((K[s:e, h] * dK[s:e, h]).sum())
            assert a == pytest.approx(c, rel=1e-10, abs=1e-13)
    if r["drab_p"] is not None and r["drab_t"] is not None:
        assert r["drab_p"].sum() == pytest.approx(r["drab_t"].sum(), rel=1e-10, abs=1e-13)


# ------------------------------------------------------------------ schedule

def _schedule_fixture():
    lines = _read_blocks("schedule.txt")
    out, k = [], 0
    while k < len(lines):
        head = lines[k].split()
        k += 1
        rows = []
        while lines[k] != "end":
            rows.append([int(x) for x in lines[k].split()])
            k += 1
        k += 1
        out.append((head[0], [int(x) for x in head[1:]], rows))
    return out


@pytest.mark.parametrize("case", _schedule_fixture(), ids=lambda c: c[0] + "_" + "_".join(map(str, c[1])))
def test_schedule_matches_hand_fixture(oracle_mod, case):
    kind, args, rows = case
    if kind == "attn":
        L, P, C, BM, BN = args
        got = oracle_mod.schedule([0, L], BM, BN, prefix_len=[P], cand_len=[C])
    else:
        n, m, mb, BM, BN = args
        got = oracle_mod.schedule_mfalcon([0, n], [0, m], BM, BN, mb)
    assert len(got) == len(rows)
    for e, want in zip(got, rows):
        assert [e["row0"], e["nrows"]] + list(map(int, e["kinds"])) == want


def _hi(i, L, P, C):
    """Exclusive end of the keys row i carries (a prefix of the sequence)."""
    E = L - C
    return P if i < P else (i + 1 if i < E else E)


@pytest.mark.parametrize("seed", range(4))
def test_schedule_tiles_form_prefixes(oracle_mod, seed):
    """The brute-force classification always yields present tiles [0, nk) and
    FULL tiles [0, nf) with nk = ceil(hi(last row)/BN), nf = floor(hi(first row)/BN)."""
    rng = np.random.default_rng(seed)
    for _ in range(30):
        L = int(rng.integers(1, 300))
        P = int(rng.integers(0, L + 1))
        C = int(rng.integers(0, L - P + 1))
        BM, BN = int(rng.choice([16, 32, 64, 128])), int(rng.choice([16, 32, 64]))
        for e in oracle_mod.schedule([0, L], BM, BN, prefix_len=[P], cand_len=[C]):
            k = list(map(int, e["kinds"]))
            nk = sum(1 for x in k if x)
            nf = sum(1 for x in k if x == 2)
            assert all(x != 0 for x in k[:nk]) and all(x == 0 for x in k[nk:])
            assert all(x == 2 for x in k[:nf]) and all(x == 1 for x in k[nf:nk])
            r0, r1 = e["row0"], e["row0"] + e["nrows"] - 1
            assert nk == -(-_hi(r1, L, P, C) // BN)
            assert nf == _hi(r0, L, P, C) // BN


def test_lpt_order_is_stable_longest_first(oracle_mod):
    ent = oracle_mod.schedule([0, 130, 300, 301], 64, 64)
    order = oracle_mod.lpt_order(ent)
    nks = [int(np.count_nonzero(ent[g]["kinds"])) for g in order]
    assert nks == sorted(nks, reverse=True)
    for a, b in zip(order, order[1:]):
        if nks[order.index(a)] == nks[order.index(b)]:
            assert a < b


def test_sequence_order_groups_sequences_longest_first(oracle_mod):
    # lengths in key tiles of 64: 3, 1, 3, 5 (the last sequence's last tile
    # sees 5 key tiles), plus an empty sequence
    ent = oracle_mod.schedule([0, 130, 150, 150, 330, 600], 64, 64)
    order = oracle_mod.sequence_order(ent)
    assert sorted(order) == list(range(len(ent)))
    seqs = [ent[g]["b"] for g in order]
    # each sequence's tiles are contiguous
    runs = [b for i, b in enumerate(seqs) if i == 0 or seqs[i - 1] != b]
    assert len(runs) == len(set(runs))
    # hand-computed: sequence 4 (5 key tiles) first, then 3 and 0 (3 each;
    # the later index first), then 1; within a sequence the longest tile first
    assert runs == [4, 3, 0, 1]
    for b in runs:
        rows = [ent[g]["row0"] for g in order if ent[g]["b"] == b]
        assert rows == sorted(rows, reverse=True)


# ------------------------------------------------------------------ inputs

def test_stochastic_length_cap_matches_page():
    for l in _read_blocks("stochastic_length.txt"):
        n, alpha, cap = l.split()
        assert synth.stochastic_length_cap(int(n), float(alpha)) == int(cap)


def test_generators_are_deterministic():
    a, b = synth.tiny_fp32(), synth.tiny_fp32()
    assert np.array_equal(a.offsets, b.offsets)
    assert torch.equal(a.Q, b.Q) and np.array_equal(a.ts, b.ts)
    t = synth.train_bf16(False)
    assert abs(t.lengths.mean() - 776) < 150
    lit = synth.train_bf16(True)
    assert lit.lengths.max() <= 776


@pytest.mark.parametrize("p", _grad_problems()[:2], ids=lambda p: p.name)
def test_rab_gradient_absolute_mass(oracle_mod, p):
    """drab_*_abs are sums of |dS|: they bound |drab_*| entrywise, both
    tables see the same total mass (each visible pair hits one entry of
    each), and with dY = 0 everything is zero."""
    r = oracle_mod.bwd(p.offsets, p.Q.numpy(), p.K.numpy(), p.V.numpy(), p.U.numpy(), p.dY.numpy(),
                       **_oracle_opts(p))
    assert np.all(r["drab_p_abs"] >= np.abs(r["drab_p"]) - 1e-12)
    assert np.all(r["drab_t_abs"] >= np.abs(r["drab_t"]) - 1e-12)
    assert r["drab_p_abs"].sum() == pytest.approx(r["drab_t_abs"].sum(), rel=1e-12)
    # a single visible pair: L = 1, the mass is |dS| of that pair in entry 0
    q = synth.custom("one", [1], H=1, d=4, dtype=torch.float32, wid=61, std=0.7, n_max=1,
                     norm=synth.NORM_NONE, n_pos=3, n_tb=3, with_dy=True)
    o = oracle_mod.bwd(q.offsets, q.Q.numpy(), q.K.numpy(), q.V.numpy(), q.U.numpy(), q.dY.numpy(),
                       **_oracle_opts(q))
    assert o["drab_p_abs"][0] == pytest.approx(abs(o["drab_p"][0]), rel=1e-14)
    assert np.all(o["drab_p_abs"][1:] == 0)
    z = oracle_mod.bwd(p.offsets, p.Q.numpy(), p.K.numpy(), p.V.numpy(), p.U.numpy(),
                       np.zeros_like(p.dY.numpy()), **_oracle_opts(p))
    assert np.all(z["drab_p_abs"] == 0) and np.all(z["drab_t_abs"] == 0)


# ------------------------------------------------- MTGR timestamp filter

def _filter_problems():
    """Hybrid-mask problems whose candidates carry times interleaved with the
    real-time tokens' times, with the timestamp filter on."""
    L = np.array([14, 20, 9, 12])
    P = np.array([3, 5, 0, 4]); C = np.array([5, 6, 4, 0])
    a = synth.custom("tf_ln", L, H=2, d=4, dtype=torch.float32, wid=61, std=0.7, n_max=2,
                     norm=synth.NORM_LN, prefix_len=P, cand_len=C, n_pos=8, n_tb=6, rab_std=0.4,
                     gamma_std=0.3, beta_std=0.3, with_dy=True)
    b = synth.custom("tf_norab", L, H=1, d=8, dtype=torch.float32, wid=62, std=0.7, n_max=1,
                     norm=synth.NORM_NONE, prefix_len=P, cand_len=C, with_dy=True)
    out = []
    for p, seed in ((a, 71), (b, 72)):
        synth.interleave_candidate_times(p, seed)
        p.time_filter = True
        out.append(p)
    return out


def test_interleaved_times_exercise_the_filter():
    """The fixtures have candidates that see some real-time tokens and not
    others, including equal timestamps."""
    for p in _filter_problems():
        seen = hidden = equal = 0
        for b in range(p.B):
            s = int(p.offsets[b]); L = int(p.lengths[b])
            P, C = int(p.prefix_len[b]), int(p.cand_len[b])
            E = L - C
            for i in range(E, L):
                for j in range(P, E):
                    if p.ts[s + j] < p.ts[s + i]:
                        seen += 1
                    else:
                        hidden += 1
                    equal += int(p.ts[s + j] == p.ts[s + i])
        assert seen > 0 and hidden > 0 and equal > 0


@pytest.mark.parametrize("p", _filter_problems(), ids=lambda p: p.name)
def test_time_filter_forward_matches_torch_dense(oracle_mod, p):
    Q, K, V, U = _torch_inputs(p)
    Yd, Od = dense_torch.forward(p.offsets, Q, K, V, U, **_dense_opts(p))
    r = oracle_mod.fwd(p.offsets, p.Q.double().numpy(), p.K.double().numpy(), p.V.double().numpy(),
                       p.U.double().numpy(), **_oracle_opts(p))
    np.testing.assert_allclose(r["O"], Od.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(r["Y"], Yd.numpy(), rtol=1e-10, atol=1e-12)
    # and the filter changes the candidate rows
    q = dict(_oracle_opts(p), time_filter=False)
    r0 = oracle_mod.fwd(p.offsets, p.Q.double().numpy(), p.K.double().numpy(), p.V.double().numpy(),
                        p.U.double().numpy(), **q)
    assert not np.array_equal(r0["O"], r["O"])


@pytest.mark.parametrize("p", _filter_problems(), ids=lambda p: p.name)
def test_time_filter_backward_matches_torch_autograd(oracle_mod, p):
    Q, K, V, U = (t.requires_grad_(True) for t in _torch_inputs(p))
    opts = _dense_opts(p)
    params = [opts[k] for k in ("rab_p", "rab_t", "gamma", "beta") if opts[k] is not None]
    for t in params:
        t.requires_grad_(True)
    Y, _ = dense_torch.forward(p.offsets, Q, K, V, U, **opts)
    (Y * p.dY.double()).sum().backward()
    r = oracle_mod.bwd(p.offsets, p.Q.numpy(), p.K.numpy(), p.V.numpy(), p.U.numpy(), p.dY.numpy(),
                       **_oracle_opts(p))
    T, D = p.T, p.H * p.d
    for name, t in (("dQ", Q), ("dK", K), ("dV", V), ("dU", U)):
        np.testing.assert_allclose(r[name], t.grad.reshape(T, D).numpy(), rtol=1e-9, atol=1e-12, err_msg=name)
    for name, key in (("drab_p", "rab_p"), ("drab_t", "rab_t"), ("dgamma", "gamma"), ("dbeta", "beta")):
        if opts[key] is not None:
            np.testing.assert_allclose(r[name], opts[key].grad.numpy(), rtol=1e-9, atol=1e-12, err_msg=name)


def test_time_filter_hides_exactly_the_later_keys(oracle_mod):
    """Perturbing a real-time key leaves a candidate row bit-identical exactly
    when the key is not strictly earlier than the candidate (equal times hide
    the key), and changes it otherwise."""
    p = _filter_problems()[1]
    base = oracle_mod.fwd(p.offsets, p.Q.numpy(), p.K.numpy(), p.V.numpy(), p.U.numpy(), **_oracle_opts(p))
    for b in range(p.B):
        s = int(p.offsets[b]); L = int(p.lengths[b])
        P, C = int(p.prefix_len[b]), int(p.cand_len[b])
        E = L - C
        for j in range(P, E):
            V2 = p.V.numpy().copy()
            V2[s + j] += 5.0
            r = oracle_mod.fwd(p.offsets, p.Q.numpy(), p.K.numpy(), V2, p.U.numpy(), **_oracle_opts(p))
            for i in range(E, L):
                same = np.array_equal(r["O"][s + i], base["O"][s + i])
                assert same == (not p.ts[s + j] < p.ts[s + i]), (b, i, j)


def test_time_filter_is_inert_when_real_time_is_earlier(oracle_mod):
    """Timestamps increasing along each sequence (candidates last): every
    real-time token is earlier than every candidate unless their times tie,
    so with strictly increasing times the filter changes nothing."""
    L = np.array([11, 15]); P = np.array([2, 3]); C = np.array([3, 4])
    p = synth.custom("tf_inert", L, H=2, d=4, dtype=torch.float32, wid=63, std=0.7, n_max=2,
                     norm=synth.NORM_LN, prefix_len=P, cand_len=C, n_pos=8, n_tb=6)
    p.ts = np.concatenate([1_000_000 + 10 * np.arange(l) for l in L]).astype(np.int64)
    a = oracle_mod.fwd(p.offsets, p.Q.numpy(), p.K.numpy(), p.V.numpy(), p.U.numpy(), **_oracle_opts(p))
    p.time_filter = True
    b = oracle_mod.fwd(p.offsets, p.Q.numpy(), p.K.numpy(), p.V.numpy(), p.U.numpy(), **_oracle_opts(p))
    np.testing.assert_array_equal(a["Y"], b["Y"])


def test_time_filter_schedule_marks_candidate_causal_tiles_partial(oracle_mod):
    """With the filter a tile holding (candidate row, causal key) pairs is
    present and never full; without it such a tile can be full."""
    L, P, C, BN = 40, 8, 16, 8
    E = L - C
    plain = oracle_mod.classify_tiles(L, P, C, E, C, BN, L // BN)
    filt = oracle_mod.classify_tiles(L, P, C, E, C, BN, L // BN, time_filter=True)
    # keys [0, 8) prefix: full either way; [8, 24) causal: full -> partial; the
    # candidate tail carries only self pairs, which are added outside the tiles
    assert list(plain) == [2, 2, 2, 0, 0]
    assert list(filt) == [2, 1, 1, 0, 0]


# ------------------------------------------- batch preparation (SL, bins)

def test_stochastic_length_special_cases(oracle_mod):
    off = np.array([0, 5, 5, 17, 20])
    T = 20
    # cap at least every length: identity
    no, idx = oracle_mod.stochastic_length(off, np.zeros(T, np.uint32), 12)
    np.testing.assert_array_equal(no, off)
    np.testing.assert_array_equal(idx, np.arange(T))
    # increasing keys keep the first cap tokens, decreasing keys the last cap
    no, idx = oracle_mod.stochastic_length(off, np.arange(T, dtype=np.uint32), 4)
    np.testing.assert_array_equal(no, [0, 4, 4, 8, 11])
    np.testing.assert_array_equal(idx, [0, 1, 2, 3, 5, 6, 7, 8, 17, 18, 19])
    no, idx = oracle_mod.stochastic_length(off, (100 - np.arange(T)).astype(np.uint32), 4)
    np.testing.assert_array_equal(idx, [1, 2, 3, 4, 13, 14, 15, 16, 17, 18, 19])
    # equal keys: ties go by index, so the first cap are kept
    no, idx = oracle_mod.stochastic_length(off, np.full(T, 7, np.uint32), 2)
    np.testing.assert_array_equal(idx, [0, 1, 5, 6, 17, 18])


def test_stochastic_length_is_uniform(oracle_mod):
    """With independent uniform keys every token of a long sequence is kept
    with probability cap / L (checked to a few standard errors), and the kept
    tokens keep their order."""
    L, cap, trials = 40, 10, 3000
    rng = np.random.default_rng(11)
    hits = np.zeros(L)
    for _ in range(trials):
        keys = rng.integers(0, 2 ** 32, size=L, dtype=np.uint64).astype(np.uint32)
        no, idx = oracle_mod.stochastic_length([0, L], keys, cap)
        assert no[-1] == cap and np.all(np.diff(idx) > 0)
        hits[idx] += 1
    p = cap / L
    se = np.sqrt(p * (1 - p) / trials)
    assert np.all(np.abs(hits / trials - p) < 5 * se)


def test_balance_bins_hand_fixture(oracle_mod):
    # lengths 5, 3, 3, 2 into 2 bins: 5 -> 0, 3 -> 1, 3 -> 1, 2 -> 0
    b, c = oracle_mod.balance_bins([3, 5, 2, 3], 2)
    np.testing.assert_array_equal(b, [1, 0, 0, 1])
    np.testing.assert_array_equal(c, [7, 6])
    # attention cost: 25 -> 0, 9 -> 1, 9 -> 1, 4 -> 1 (loads 25 | 9, 18, 22)
    b, c = oracle_mod.balance_bins([3, 5, 2, 3], 2, cost_kind=1)
    np.testing.assert_array_equal(b, [1, 0, 1, 1])
    np.testing.assert_array_equal(c, [25, 22])


def test_balance_bins_within_graham_bound(oracle_mod):
    """Longest-first greedy is within (4/3 - 1/(3m)) of the best makespan,
    found here by brute force on small inputs; costs are conserved."""
    import itertools
    rng = np.random.default_rng(12)
    for _ in range(30):
        n, m = int(rng.integers(3, 8)), int(rng.integers(2, 4))
        lengths = rng.integers(1, 50, size=n)
        b, c = oracle_mod.balance_bins(lengths, m)
        assert c.sum() == lengths.sum()
        for k in range(m):
            assert c[k] == lengths[b == k].sum()
        best = min(max(sum(int(lengths[i]) for i in range(n) if a[i] == k) for k in range(m))
                   for a in itertools.product(range(m), repeat=n))
        assert c.max() <= (4.0 / 3.0 - 1.0 / (3 * m)) * best + 1e-9


# ------------------------------------------------------------------ full layer

def _layer_problems():
    """Small layers with d_model != D (a transposed weight cannot go
    unnoticed) over the backward pins' attention problems."""
    out = []
    for i, p in enumerate(_grad_problems()):
        out.append(synth.with_layer(p, d_model=[6, 11, 5][i], wid=70 + i, x_std=0.8, w_std=0.4,
                                    bias_std=None if i == 2 else 0.3))
    return out


def _torch_layer(lp, X, W1, b1, W2, b2, opts):
    """The layer out of torch library routines: matmul, F.silu, torch.split
    into U, V, Q, K, the dense attention above, matmul."""
    p = lp.core
    D = p.H * p.d
    Z = X @ W1 + (b1 if b1 is not None else 0.0)
    U, V, Q, K = (t.reshape(p.T, p.H, p.d) for t in torch.split(torch.nn.functional.silu(Z), D, dim=1))
    Y, _ = dense_torch.forward(p.offsets, Q, K, V, U, **opts)
    return Y @ W2 + (b2 if b2 is not None else 0.0)


def _layer_np(lp):
    f = lambda t: None if t is None else np.asarray(t.double().numpy() if torch.is_tensor(t) else t, np.float64)
    return f(lp.X), f(lp.W1), f(lp.b1), f(lp.W2), f(lp.b2), f(lp.dOut)


@pytest.mark.parametrize("lp", _layer_problems(), ids=lambda lp: lp.name)
def test_layer_matches_torch_autograd(oracle_mod, lp):
    p = lp.core
    X, W1, b1, W2, b2, dOut = _layer_np(lp)
    leaves = {k: (None if v is None else torch.tensor(v, requires_grad=True))
              for k, v in dict(X=X, W1=W1, b1=b1, W2=W2, b2=b2).items()}
    opts = _dense_opts(p)
    params = {k: opts[k] for k in ("rab_p", "rab_t", "gamma", "beta") if opts[k] is not None}
    for t in params.values():
        t.requires_grad_(True)
    Out = _torch_layer(lp, leaves["X"], leaves["W1"], leaves["b1"], leaves["W2"], leaves["b2"], opts)
    (Out * torch.tensor(dOut)).sum().backward()
    f = oracle_mod.layer_fwd(p.offsets, X, W1, W2, b1=b1, b2=b2, **_oracle_opts(p))
    np.testing.assert_allclose(f["Out"], Out.detach().numpy(), rtol=1e-10, atol=1e-12)
    g = oracle_mod.layer_bwd(p.offsets, X, W1, W2, dOut, b1=b1, b2=b2, **_oracle_opts(p))
    for name, key in (("dX", "X"), ("dW1", "W1"), ("db1", "b1"), ("dW2", "W2"), ("db2", "b2")):
        if leaves[key] is not None:
            np.testing.assert_allclose(g[name], leaves[key].grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)
    for name, key in (("drab_p", "rab_p"), ("drab_t", "rab_t"), ("dgamma", "gamma"), ("dbeta", "beta")):
        if key in params:
            np.testing.assert_allclose(g[name], params[key].grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)


@pytest.mark.parametrize("lp", _layer_problems()[:2], ids=lambda lp: lp.name)
def test_layer_backward_matches_central_differences(oracle_mod, lp):
    """<grad, delta> against central differences of sum(Out * dOut) from
    layer_fwd itself, for every layer parameter and the input."""
    p = lp.core
    X, W1, b1, W2, b2, dOut = _layer_np(lp)
    vals = {k: v for k, v in dict(X=X, W1=W1, b1=b1, W2=W2, b2=b2).items() if v is not None}
    opts = _oracle_opts(p)

    def f(v):
        return float((oracle_mod.layer_fwd(p.offsets, v["X"], v["W1"], v["W2"], b1=v.get("b1"),
                                           b2=v.get("b2"), **opts)["Out"] * dOut).sum())

    g = oracle_mod.layer_bwd(p.offsets, X, W1, W2, dOut, b1=b1, b2=b2, **opts)
    rng = np.random.default_rng(5)
    h = 1e-5
    for k in vals:
        delta = rng.normal(size=vals[k].shape)
        fd = (f({**vals, k: vals[k] + h * delta}) - f({**vals, k: vals[k] - h * delta})) / (2 * h)
        an = float((g["d" + k] * delta).sum())
        assert an == pytest.approx(fd, rel=1e-6, abs=1e-9), k


def test_layer_with_block_identity_weights_is_the_core(oracle_mod):
    """W1 = [a_u I | a_v I | a_q I | a_k I] (d_model = D), no biases and
    W2 = I make the layer the attention core on Q = SiLU(a_q X) and so on:
    pins the order of the split and where each block goes. The SiLU here is
    torch's."""
    p = _grad_problems()[0]
    D = p.H * p.d
    lp = synth.with_layer(p, wid=77, x_std=1.0, bias_std=None)
    X = lp.X.double().numpy()
    scales = dict(u=0.5, v=-1.25, q=2.0, k=0.75)
    W1 = np.concatenate([s * np.eye(D) for s in scales.values()], axis=1)
    f = oracle_mod.layer_fwd(p.offsets, X, W1, np.eye(D), **_oracle_opts(p))
    act = {k: torch.nn.functional.silu(torch.tensor(s * X)).numpy() for k, s in scales.items()}
    core = oracle_mod.fwd(p.offsets, act["q"], act["k"], act["v"], act["u"], **_oracle_opts(p))
    for name, want in (("Q", act["q"]), ("K", act["k"]), ("V", act["v"]), ("U", act["u"])):
        np.testing.assert_allclose(f[name], want, rtol=1e-14, atol=1e-300, err_msg=name)
    np.testing.assert_allclose(f["Out"], core["Y"], rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ layer stack, M-FALCON

def _stack_small(**kw):
    args = dict(n_layers=2, H=2, d=4, d_model=6, dtype=torch.float32, wid=140, x_std=1.0, w_std=0.4,
                bias_std=0.3, n_pos=16, n_tb=8, rab_std=0.3, gamma_std=0.3, beta_std=0.3)
    args.update(kw)
    return synth.stack_custom("stack_small", [7, 0, 12], [3, 2, 5], **args)


def _stack_run(oracle_mod, sp, hist_rows=None, cand_rows=None):
    """oracle.mfalcon_stack on sp, optionally restricted to some history or
    candidate rows (per-user counts recomputed)."""
    def sel(offsets, rows):
        off = np.asarray(offsets, np.int64)
        if rows is None:
            return off, np.arange(off[-1])
        rows = np.asarray(sorted(rows), np.int64)
        counts = [int(((rows >= off[b]) & (rows < off[b + 1])).sum()) for b in range(len(off) - 1)]
        return np.concatenate([[0], np.cumsum(counts)]), rows
    ho, hr = sel(sp.hist_offsets, hist_rows)
    co, cr = sel(sp.cand_offsets, cand_rows)
    f = lambda t: t.double().numpy()
    return oracle_mod.mfalcon_stack(
        ho, co, f(sp.X_hist)[hr], f(sp.X_cand)[cr], sp.layers, H=sp.H, d=sp.d,
        hist_ts=None if sp.hist_ts is None else sp.hist_ts[hr], cand_ts=None if sp.cand_ts is None else sp.cand_ts[cr],
        n_max=sp.n_max, norm=sp.norm, eps=sp.eps, time_filter=sp.time_filter), cr


def test_stack_history_rows_ignore_candidates(oracle_mod):
    sp = _stack_small()
    full, _ = _stack_run(oracle_mod, sp)
    none, _ = _stack_run(oracle_mod, sp, cand_rows=[])
    np.testing.assert_allclose(full["Out_hist"], none["Out_hist"], rtol=1e-12, atol=1e-14)


def test_stack_candidates_ignore_each_other(oracle_mod):
    sp = _stack_small()
    full, _ = _stack_run(oracle_mod, sp)
    keep = [r for r in range(int(sp.cand_offsets[-1])) if r not in (1, 5, 6)]
    part, cr = _stack_run(oracle_mod, sp, cand_rows=keep)
    np.testing.assert_allclose(part["Out"], full["Out"][cr], rtol=1e-12, atol=1e-14)


def test_stack_cached_layers_equal_full_pass(oracle_mod):
    """Layer by layer with per-layer history K/V caches (layer_fwd over the
    histories alone) and oracle.mfalcon for the candidates equals the full
    pass over [history | candidates]: the history K/V of every layer is all a
    candidate needs."""
    for tf in (False, True):
        sp = _stack_small()
        sp.time_filter = tf
        ref, _ = _stack_run(oracle_mod, sp)
        D = sp.H * sp.d
        Xh, Xc = sp.X_hist.double().numpy(), sp.X_cand.double().numpy()
        for lay in sp.layers:
            h = oracle_mod.layer_fwd(sp.hist_offsets, Xh, lay["W1"], lay["W2"], H=sp.H, d=sp.d, b1=lay.get("b1"),
                                     b2=lay.get("b2"), ts=sp.hist_ts, rab_p=lay.get("rab_p"), rab_t=lay.get("rab_t"),
                                     n_max=sp.n_max, norm=sp.norm, eps=sp.eps, gamma=lay.get("gamma"),
                                     beta=lay.get("beta"))
            Zc = Xc @ np.asarray(lay["W1"].double()) + lay["b1"]
            A = torch.nn.functional.silu(torch.tensor(Zc)).numpy()
            Uc, Vc, Qc, Kc = (A[:, i * D:(i + 1) * D] for i in range(4))
            m = oracle_mod.mfalcon(sp.hist_offsets, sp.cand_offsets, h["K"], h["V"], Qc, Kc, Vc, Uc, H=sp.H, d=sp.d,
                                   hist_ts=sp.hist_ts, cand_ts=sp.cand_ts, rab_p=lay.get("rab_p"),
                                   rab_t=lay.get("rab_t"), n_max=sp.n_max, norm=sp.norm, eps=sp.eps,
                                   gamma=lay.get("gamma"), beta=lay.get("beta"), time_filter=tf)
            Xc = m["Y"] @ np.asarray(lay["W2"].double()) + lay["b2"]
            Xh = h["Out"]
        np.testing.assert_allclose(Xc, ref["Out"], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(Xh, ref["Out_hist"], rtol=1e-10, atol=1e-12)


def test_stack_candidate_permutation_permutes_outputs(oracle_mod):
    sp = _stack_small()
    ref, _ = _stack_run(oracle_mod, sp)
    perm = np.arange(int(sp.cand_offsets[-1]))
    perm[5:10] = perm[5:10][::-1]  # reverse the last user's candidates
    sp2 = _stack_small()
    sp2.X_cand = sp.X_cand[torch.from_numpy(perm)]
    sp2.cand_ts = sp.cand_ts[perm]
    got, _ = _stack_run(oracle_mod, sp2)
    np.testing.assert_allclose(got["Out"], ref["Out"][perm], rtol=1e-12, atol=1e-14)
