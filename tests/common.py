"""Helpers shared by the tests: oracle calls on generated problems, error metrics."""
import numpy as np
import torch

import oracle


def f64(t):
    return None if t is None else (t.detach().double().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float64))


def oracle_opts(p):
    return dict(H=p.H, d=p.d, prefix_len=p.prefix_len, cand_len=p.cand_len, ts=p.ts, rab_p=p.rab_p,
                rab_t=p.rab_t, n_max=p.n_max, norm=p.norm, eps=p.eps, group=p.group,
                n_groups=p.n_groups, gamma=p.gamma, beta=p.beta, time_filter=p.time_filter)


def oracle_fwd(p, row_sel=None, Q=None, K=None, V=None, U=None):
    return oracle.fwd(p.offsets, f64(p.Q if Q is None else Q), f64(p.K if K is None else K),
                      f64(p.V if V is None else V), f64(p.U if U is None else U), row_sel=row_sel,
                      **oracle_opts(p))


def oracle_bwd(p):
    return oracle.bwd(p.offsets, f64(p.Q), f64(p.K), f64(p.V), f64(p.U), f64(p.dY), **oracle_opts(p))


def oracle_mfalcon(mf):
    return oracle.mfalcon(mf.hist_offsets, mf.cand_offsets, f64(mf.K_cache), f64(mf.V_cache), f64(mf.Qc),
                          f64(mf.Kc), f64(mf.Vc), f64(mf.Uc), H=mf.H, d=mf.d, hist_ts=mf.hist_ts,
                          cand_ts=mf.cand_ts, rab_p=mf.rab_p, rab_t=mf.rab_t, n_max=mf.n_max, norm=mf.norm,
                          eps=mf.eps, cand_group=mf.cand_group, n_groups=mf.n_groups, gamma=mf.gamma,
                          beta=mf.beta, time_filter=mf.time_filter)


def rel_l2(got, ref):
    got = f64(got).reshape(-1)
    ref = f64(ref).reshape(-1)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0:
        return num
    return num / den


# Tolerances on relative L2 error: bf16 inputs with fp32 accumulation, and
# the fp32 path.
TOL_BF16 = 1e-2
TOL_F32 = 1e-5


def tol(p):
    return TOL_F32 if p.dtype == torch.float32 else TOL_BF16


def oracle_layer_fwd(lp):
    p = lp.core
    return oracle.layer_fwd(p.offsets, f64(lp.X), f64(lp.W1), f64(lp.W2), b1=f64(lp.b1), b2=f64(lp.b2),
                            **oracle_opts(p))


def oracle_layer_bwd(lp):
    p = lp.core
    return oracle.layer_bwd(p.offsets, f64(lp.X), f64(lp.W1), f64(lp.W2), f64(lp.dOut), b1=f64(lp.b1),
                            b2=f64(lp.b2), **oracle_opts(p))


def f64_layers(layers):
    """Per-layer dicts with every tensor as a float64 numpy array (the
    oracle takes numpy; bf16 weights are represented exactly)."""
    return [{k: f64(v) for k, v in lay.items()} for lay in layers]
