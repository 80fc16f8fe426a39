"""GPU parity of the backward pass (hstu_attn_bwd through the C ABI) against
the CPU oracle's gradients."""
import numpy as np
import pytest
import torch

import oracle
from hstu_jagged_pointwise_attn_amd import api, device, synth
from tests.common import oracle_bwd, oracle_fwd, rel_l2, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)


def _say(*a):
    print(*a, flush=True)


def _problems():
    ps = []
    ps.append(synth.custom("f32_causal_rab", [70, 1, 129, 64], H=2, d=32, dtype=torch.float32, wid=51, std=0.4,
                           n_max=8, norm=synth.NORM_LN, n_pos=100, n_tb=12, rab_std=0.3, gamma_std=0.3,
                           beta_std=0.3, with_dy=True))
    L = np.array([150, 40, 133, 7])
    P = np.array([100, 0, 60, 3]); C = np.array([30, 40, 33, 2])
    grp = np.concatenate([np.minimum(np.arange(l) * 3 // l, 2) for l in L])
    ps.append(synth.custom("f32_mtgr_gln", L, H=2, d=64, dtype=torch.float32, wid=52, std=0.4, n_max=16,
                           norm=synth.NORM_GLN, prefix_len=P, cand_len=C, group=grp, n_groups=3, gamma_std=0.3,
                           beta_std=0.3, n_pos=64, n_tb=10, rab_std=0.3, with_dy=True))
    ps.append(synth.custom("bf16_causal_rab", [300, 1, 129, 64, 0, 257], H=2, d=128, wid=53, std=0.3, n_max=64,
                           norm=synth.NORM_LN, n_pos=300, n_tb=20, rab_std=0.3, with_dy=True))
    ps.append(synth.custom("bf16_mtgr_gln", L, H=3, d=64, wid=54, std=0.3, n_max=300, norm=synth.NORM_GLN,
                           prefix_len=P, cand_len=C, group=grp, n_groups=3, gamma_std=0.3, beta_std=0.3,
                           n_pos=64, n_tb=12, rab_std=0.3, with_dy=True))
    ps.append(synth.custom("bf16_none_cand_d32", [200, 65, 3], H=4, d=32, wid=55, std=0.5, n_max=8,
                           norm=synth.NORM_NONE, cand_len=[20, 0, 3], n_pos=40, rab_std=0.3, with_dy=True))
    ps.append(synth.custom("bf16_ln_active", [190, 77], H=2, d=128, wid=56, std=1.0, qk_std=0.1, n_max=1,
                           norm=synth.NORM_LN, gamma_std=0.5, beta_std=0.5, n_tb=16, rab_std=0.3, with_dy=True))
    return ps


def _run(p, ns=None):
    ns = ns or device.upload(p)
    f = device.run_fwd(ns)
    g = api.attn_bwd(ns.problem, ns.Q, ns.K, ns.V, ns.U, f.O, f.mean, f.rstd, ns.dY)
    torch.cuda.synchronize()
    return ns, f, g


def mass_rel(got, ref, mass):
    """||got - ref|| / ||mass||: the error of a sum of many cancelling terms
    measured against the sum of their magnitudes (a diagnostic printed next
    to the plain relative error)."""
    got = np.asarray(got, np.float64).reshape(-1)
    den = np.linalg.norm(np.asarray(mass, np.float64).reshape(-1))
    return np.linalg.norm(got - np.asarray(ref).reshape(-1)) / den if den else np.linalg.norm(got - ref)


def kappa(ref, mass):
    """Cancellation factor ||sum |dS| per entry|| / ||d rab||: how much larger
    the magnitudes summed into a rab gradient are than the gradient itself."""
    r = np.linalg.norm(np.asarray(ref, np.float64))
    return np.linalg.norm(np.asarray(mass, np.float64)) / r if r else np.inf


# (problem, gradient) pairs whose plain relative error cannot reach the bf16
# bound with bf16 operands: the gradient is a sum over ~60k pairs that cancels
# by a factor above 1000, so the 2^-9 relative rounding of dO (the dP
# product's bf16 operand) and of the forward's attention weights (the A.V
# product's bf16 operand) each exceed 1e-2 of it on their own (a CPU
# emulation of those two roundings alone gives 1.0e-2 and 5.8e-3). For these
# the test asserts the mass-relative error at the bf16 bound and that the
# cancellation factor really is above 1000; the plain error is printed.
ILL_CONDITIONED = {("bf16_mtgr_gln", "drab_t"): 1000.0}


def _compare(p, g, ref, rows=None, what=("dQ", "dK", "dV", "dU"), extra=True):
    """Plain relative L2 error per gradient (the rab gradients also print
    their mass-relative error, "<name>~", and cancellation factor)."""
    T, D = p.T, p.H * p.d
    errs = {}
    for name in what:
        got = getattr(g, name).float().cpu().numpy().reshape(T, D)
        want = ref[name]
        if rows is not None:
            got, want = got[rows], want[rows]
        errs[name] = rel_l2(got, want)
    if extra:
        for name, gname in (("dgamma", "d_gamma"), ("dbeta", "d_beta")):
            if ref[name] is not None and getattr(g, gname) is not None:
                errs[name] = rel_l2(getattr(g, gname).cpu().numpy(), ref[name])
        for name, gname in (("drab_p", "d_rab_p"), ("drab_t", "d_rab_t")):
            if ref[name] is not None and getattr(g, gname) is not None:
                got = getattr(g, gname).cpu().numpy()
                errs[name] = rel_l2(got, ref[name])
                errs["(diag) " + name + "~"] = mass_rel(got, ref[name], ref[name + "_abs"])
                errs["(diag) " + name + " kappa"] = kappa(ref[name], ref[name + "_abs"])
    return errs


def check_errs(p, errs):
    """Every gradient within the dtype's bound in plain relative L2, except
    the listed ill-conditioned rab gradients (see ILL_CONDITIONED)."""
    for k, v in errs.items():
        if k.startswith("(diag)"):
            continue
        bound = ILL_CONDITIONED.get((p.name, k))
        if bound is not None:
            assert errs["(diag) " + k + " kappa"] >= bound, (k, errs["(diag) " + k + " kappa"])
            assert errs["(diag) " + k + "~"] <= tol(p), (k, errs["(diag) " + k + "~"])
            continue
        assert v <= tol(p), (k, v)


@pytest.mark.parametrize("p", _problems(), ids=lambda p: p.name)
def test_bwd_matches_oracle_small(p):
    _say("bwd", p.name, p.dtype, p.offsets.tolist())
    ns, f, g = _run(p)
    assert api.device_status(g.ws) == 0
    ref = oracle_bwd(p)
    errs = _compare(p, g, ref)
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    check_errs(p, errs)


def _subsample_seqs(p):
    """argmin L, argmax L and the two sequences nearest the median (ties by index)."""
    lens = p.lengths
    order = np.argsort(np.abs(lens - np.median(lens)), kind="stable")
    picks = [int(np.argmin(lens)), int(np.argmax(lens))]
    for s in order:
        if int(s) not in picks:
            picks.append(int(s))
        if len(picks) == 4:
            break
    return sorted(picks)


def test_bwd_long_full_size_on_subsample():
    """The long-sequence workload at full size on the GPU; dQ, dK, dV, dU of
    four sequences against the oracle run on those sequences (a sequence's
    gradients depend on that sequence only), and d rab from a GPU run on the
    same four-sequence sub-batch (the tables' gradients sum over the batch)."""
    p = synth.long_bf16()
    seqs = _subsample_seqs(p)
    _say("bwd long: B", p.B, "T", p.T, "subsample", seqs, "lengths", p.lengths[seqs].tolist())
    ns, f, g = _run(p)
    assert api.device_status(g.ws) == 0
    sub = synth.subbatch(p, seqs)
    ref = oracle_bwd(sub)
    rows = np.concatenate([np.arange(p.offsets[s], p.offsets[s + 1]) for s in seqs])
    T, D = p.T, p.H * p.d
    errs = {}
    for name in ("dQ", "dK", "dV", "dU"):
        got = getattr(g, name).float().cpu().numpy().reshape(T, D)[rows]
        errs[name] = rel_l2(got, ref[name])
    _, _, gs = _run(sub)
    for name, gname in (("drab_p", "d_rab_p"), ("drab_t", "d_rab_t")):
        errs[name] = rel_l2(getattr(gs, gname).cpu().numpy(), ref[name])
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= 1e-2, (k, v)


def test_bwd_gradient_identity_on_gpu():
    """<Q, dQ> = <K, dK> per (sequence, head): both equal sum dS_ij q_i.k_j."""
    p = synth.custom("ident", [180, 90], H=2, d=64, dtype=torch.float32, wid=57, std=0.5, n_max=4,
                     norm=synth.NORM_LN, cand_len=[30, 10], n_pos=64, n_tb=8, with_dy=True)
    ns, f, g = _run(p)
    Q = p.Q.double().numpy(); K = p.K.double().numpy()
    dQ = g.dQ.double().cpu().numpy(); dK = g.dK.double().cpu().numpy()
    for b in range(p.B):
        s, e = p.offsets[b], p.offsets[b + 1]
        for h in range(p.H):
            a1 = (Q[s:e, h] * dQ[s:e, h]).sum()
            a2 = (K[s:e, h] * dK[s:e, h]).sum()
            assert a1 == pytest.approx(a2, rel=1e-4, abs=1e-9)


def test_autograd_function_matches_oracle():
    """api.hstu_attention (HSTUAttnFn: hstu_attn_fwd in the forward,
    hstu_attn_bwd in the backward) under torch.autograd: Y and the gradients
    of Q, K, V, U, both rab tables and the Group LayerNorm affine against the
    oracle."""
    L = np.array([150, 40, 133, 7])
    P = np.array([100, 0, 60, 3]); C = np.array([30, 40, 33, 2])
    grp = np.concatenate([np.minimum(np.arange(l) * 3 // l, 2) for l in L])
    for dtype in (torch.float32, torch.bfloat16):
        p = synth.custom(f"autograd_{dtype}", L, H=2, d=64, dtype=dtype, wid=58, std=0.4, n_max=16,
                         norm=synth.NORM_GLN, prefix_len=P, cand_len=C, group=grp, n_groups=3, gamma_std=0.3,
                         beta_std=0.3, n_pos=200, n_tb=24, rab_std=0.3, with_dy=True)
        ns = device.upload(p)
        leaves = {k: getattr(ns, k).clone().requires_grad_(True) for k in ("Q", "K", "V", "U")}
        tabs = {k: getattr(ns, k).clone().requires_grad_(True) for k in ("rab_p", "rab_t", "gamma", "beta")}
        Y = api.hstu_attention(ns.offsets, leaves["Q"], leaves["K"], leaves["V"], leaves["U"], max_len=p.max_len,
                               n_max=p.n_max, prefix_len=ns.prefix_len, cand_len=ns.cand_len, timestamps=ns.ts,
                               norm=p.norm, eps=p.eps, token_group=ns.group, n_groups=p.n_groups, **tabs)
        Y.backward(ns.dY)
        torch.cuda.synchronize()
        ref = oracle_bwd(p)
        fref = oracle_fwd(p)
        T, D = p.T, p.H * p.d
        errs = {"Y": rel_l2(Y.detach(), fref["Y"])}
        for name in ("Q", "K", "V", "U"):
            errs["d" + name] = rel_l2(leaves[name].grad.float().cpu().numpy().reshape(T, D), ref["d" + name])
        for name, rname in (("rab_p", "drab_p"), ("rab_t", "drab_t"), ("gamma", "dgamma"), ("beta", "dbeta")):
            errs[rname] = rel_l2(tabs[name].grad.cpu().numpy(), ref[rname])
        _say(f"autograd {dtype}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        for k, v in errs.items():
            assert v <= tol(p), (k, v)
