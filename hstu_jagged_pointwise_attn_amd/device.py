"""Upload generated problems (``synth``) to the GPU and describe them to the
library. Marshalling only: no arithmetic of the method happens here."""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import torch

from . import api


def _t(a, dtype, dev):
    return None if a is None else torch.as_tensor(np.ascontiguousarray(a)).to(dtype).to(dev)


def upload(p, device="cuda", with_grad_inputs=False):
    """Device tensors and the hstu_problem_t of a synth.Problem."""
    dev = torch.device(device)
    offsets = _t(p.offsets, torch.int32, dev)
    ns = SimpleNamespace(src=p, device=dev)
    ns.offsets = offsets
    ns.prefix_len = _t(p.prefix_len, torch.int32, dev)
    ns.cand_len = _t(p.cand_len, torch.int32, dev)
    ns.ts = _t(p.ts, torch.int64, dev)
    ns.rab_p = _t(p.rab_p, torch.float32, dev)
    ns.rab_t = _t(p.rab_t, torch.float32, dev)
    ns.group = _t(p.group, torch.uint8, dev)
    ns.gamma = _t(p.gamma, torch.float32, dev)
    ns.beta = _t(p.beta, torch.float32, dev)
    ns.Q, ns.K, ns.V, ns.U = (x.contiguous().to(dev) for x in (p.Q, p.K, p.V, p.U))
    ns.dY = None if p.dY is None else p.dY.contiguous().to(dev)
    ns.problem = api.problem(
        offsets, H=p.H, d=p.d, dtype=p.dtype, total_tokens=p.T, max_len=p.max_len, n_max=p.n_max,
        prefix_len=ns.prefix_len, cand_len=ns.cand_len, timestamps=ns.ts, rab_p=ns.rab_p,
        rab_t=ns.rab_t, norm=p.norm, eps=p.eps, token_group=ns.group, n_groups=p.n_groups,
        gamma=ns.gamma, beta=ns.beta, time_filter=p.time_filter)
    return ns


def upload_mfalcon(mf, device="cuda"):
    """Device tensors and the candidate hstu_problem_t of a synth.MFalconProblem."""
    dev = torch.device(device)
    ns = SimpleNamespace(src=mf, device=dev)
    ns.hist_offsets = _t(mf.hist_offsets, torch.int32, dev)
    ns.cand_offsets = _t(mf.cand_offsets, torch.int32, dev)
    ns.hist_ts = _t(mf.hist_ts, torch.int64, dev)
    ns.cand_ts = _t(mf.cand_ts, torch.int64, dev)
    ns.rab_p = _t(mf.rab_p, torch.float32, dev)
    ns.rab_t = _t(mf.rab_t, torch.float32, dev)
    ns.group = _t(mf.cand_group, torch.uint8, dev)
    ns.gamma = _t(mf.gamma, torch.float32, dev)
    ns.beta = _t(mf.beta, torch.float32, dev)
    for name in ("K_cache", "V_cache", "Qc", "Kc", "Vc", "Uc"):
        setattr(ns, name, getattr(mf, name).contiguous().to(dev))
    ns.hist_tokens = int(mf.hist_offsets[-1])
    ns.hist_max_len = int(np.diff(mf.hist_offsets).max()) if mf.B else 0
    cand_max = int(np.diff(mf.cand_offsets).max()) if mf.B else 0
    ns.problem = api.problem(
        ns.cand_offsets, H=mf.H, d=mf.d, dtype=mf.dtype, total_tokens=int(mf.cand_offsets[-1]),
        max_len=cand_max, n_max=mf.n_max, timestamps=ns.cand_ts, rab_p=ns.rab_p, rab_t=ns.rab_t,
        norm=mf.norm, eps=mf.eps, token_group=ns.group, n_groups=mf.n_groups, gamma=ns.gamma,
        beta=ns.beta, time_filter=mf.time_filter)
    return ns


def run_fwd(ns, **kw):
    return api.attn_fwd(ns.problem, ns.Q, ns.K, ns.V, ns.U, **kw)


def run_mfalcon(ns, microbatch=None, **kw):
    mb = ns.src.microbatch if microbatch is None else microbatch
    return api.mfalcon_score(ns.problem, ns.hist_offsets, ns.hist_tokens, ns.hist_max_len, ns.K_cache,
                             ns.V_cache, ns.Qc, ns.Kc, ns.Vc, ns.Uc, hist_ts=ns.hist_ts, microbatch=mb, **kw)


def upload_layer(lp, device="cuda"):
    """Device tensors of a synth.LayerProblem: the core problem (upload), X,
    the weights and dOut, and the hstu_layer_weights_t."""
    ns = upload(lp.core, device)
    dev = ns.device
    ns.layer = lp
    ns.X = lp.X.contiguous().to(dev)
    ns.W1 = lp.W1.contiguous().to(dev)
    ns.W2 = lp.W2.contiguous().to(dev)
    ns.b1 = _t(lp.b1, torch.float32, dev)
    ns.b2 = _t(lp.b2, torch.float32, dev)
    ns.dOut = None if lp.dOut is None else lp.dOut.contiguous().to(dev)
    ns.weights = api.layer_weights(ns.W1, ns.W2, ns.b1, ns.b2)
    return ns


def run_layer_fwd(ns, **kw):
    return api.layer_fwd(ns.problem, ns.weights, ns.X, **kw)


def run_layer_bwd(ns, f, **kw):
    return api.layer_bwd(ns.problem, ns.weights, ns.X, f, ns.dOut, **kw)


def upload_stack(sp, device="cuda"):
    """Device tensors of a synth.StackProblem: the history and candidate
    problems, the layer array with its K/V caches, X_hist and X_cand."""
    dev = torch.device(device)
    ns = SimpleNamespace(src=sp, device=dev)
    ns.hist_offsets = _t(sp.hist_offsets, torch.int32, dev)
    ns.cand_offsets = _t(sp.cand_offsets, torch.int32, dev)
    ns.hist_ts = _t(sp.hist_ts, torch.int64, dev)
    ns.cand_ts = _t(sp.cand_ts, torch.int64, dev)
    ns.hist_group = _t(sp.hist_group, torch.uint8, dev)
    ns.cand_group = _t(sp.cand_group, torch.uint8, dev)
    ns.hist_tokens = int(sp.hist_offsets[-1])
    ns.hist_max_len = int(np.diff(sp.hist_offsets).max()) if sp.B else 0
    cand_max = int(np.diff(sp.cand_offsets).max()) if sp.B else 0
    n_pos = max([len(l["rab_p"]) for l in sp.layers if "rab_p" in l] or [0])
    n_tb = max([len(l["rab_t"]) for l in sp.layers if "rab_t" in l] or [0])
    ns.layer_tensors = []
    for lay in sp.layers:
        t = {"W1": lay["W1"].contiguous().to(dev), "W2": lay["W2"].contiguous().to(dev)}
        for k in ("b1", "b2", "rab_p", "rab_t", "gamma", "beta"):
            if k in lay:
                t[k] = _t(lay[k], torch.float32, dev)
        ns.layer_tensors.append(t)
    ns.layers, ns.K_caches, ns.V_caches = api.stack_layers(ns.layer_tensors, sp.H, sp.d, sp.dtype, dev,
                                                           hist_tokens=ns.hist_tokens)
    ns.X_hist = sp.X_hist.contiguous().to(dev)
    ns.X_cand = sp.X_cand.contiguous().to(dev)

    def prob(offsets, T, max_len, ts, group, time_filter):
        p = api.problem(offsets, H=sp.H, d=sp.d, dtype=sp.dtype, total_tokens=T, max_len=max_len, n_max=sp.n_max,
                        timestamps=ts, norm=sp.norm, eps=sp.eps, token_group=group, n_groups=sp.n_groups,
                        time_filter=time_filter)
        p.n_pos, p.n_tb = n_pos, n_tb
        return p

    ns.hist_problem = prob(ns.hist_offsets, ns.hist_tokens, ns.hist_max_len, ns.hist_ts, ns.hist_group, False)
    ns.cand_problem = prob(ns.cand_offsets, int(sp.cand_offsets[-1]), cand_max, ns.cand_ts, ns.cand_group,
                           sp.time_filter)
    return ns


def run_stack_history(ns, **kw):
    return api.stack_history(ns.hist_problem, ns.layers, ns.X_hist, **kw)


def run_stack_score(ns, Xc=None, microbatch=None, **kw):
    mb = ns.src.microbatch if microbatch is None else microbatch
    return api.stack_score(ns.cand_problem, ns.layers, ns.hist_offsets, ns.hist_tokens, ns.hist_max_len,
                           ns.X_cand if Xc is None else Xc, hist_ts=ns.hist_ts, microbatch=mb, **kw)
