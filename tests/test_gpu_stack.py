"""GPU parity of multi-layer M-FALCON serving (hstu_stack_history /
hstu_stack_score / hstu_stack_score_capture through the C ABI) against the
oracle's plain full pass over [history | candidates] (oracle.mfalcon_stack)."""
import numpy as np
import pytest
import torch

import oracle
from hstu_jagged_pointwise_attn_amd import api, device, synth
from tests.common import f64_layers, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)


def _say(*a):
    print(*a, flush=True)


def _tol(sp):
    # bf16: the single-layer bound 1e-2 per layer of the stack (first-order error terms add up)
    return 1e-5 if sp.dtype == torch.float32 else 1e-2 * len(sp.layers)


def _stacks():
    out = []
    out.append(synth.stack_custom("S_f32_rab_ln", [70, 0, 129, 33], [12, 5, 40, 1], n_layers=2, H=2, d=32,
                                  d_model=48, dtype=torch.float32, wid=150, microbatch=16, x_std=1.0, w_std=0.1,
                                  bias_std=0.2, n_pos=256, n_tb=16, rab_std=0.3, gamma_std=0.3, beta_std=0.3))
    out.append(synth.stack_custom("S_bf16_gln_rab", [300, 64, 1, 129], [33, 64, 7, 100], n_layers=3, H=2, d=64,
                                  wid=151, microbatch=32, norm=synth.NORM_GLN, x_std=1.0, w_std=0.05, bias_std=0.2,
                                  n_pos=512, n_tb=20, rab_std=0.3, gamma_std=0.3, beta_std=0.3))
    out.append(synth.stack_custom("S_bf16_d128_norab", [200, 257], [130, 64], n_layers=2, H=4, d=128, wid=152,
                                  microbatch=64, x_std=1.0, w_std=0.03, bias_std=0.2))
    sp = synth.stack_custom("S_bf16_time_filter", [150, 90], [40, 25], n_layers=2, H=2, d=64, wid=153, microbatch=16,
                            x_std=1.0, w_std=0.05, bias_std=0.2, n_tb=16, rab_std=0.3, with_ts=True)
    # candidates at times inside the history, so the filter hides part of it
    rng = np.random.default_rng(5)
    for b in range(sp.B):
        hs, he = int(sp.hist_offsets[b]), int(sp.hist_offsets[b + 1])
        cs, ce = int(sp.cand_offsets[b]), int(sp.cand_offsets[b + 1])
        sp.cand_ts[cs:ce] = sp.hist_ts[hs:he][rng.integers(0, he - hs, ce - cs)] + rng.integers(0, 2, ce - cs)
    sp.time_filter = True
    out.append(sp)
    return out


def _oracle(sp, Xc=None):
    f = lambda t: t.double().numpy()
    return oracle.mfalcon_stack(sp.hist_offsets, sp.cand_offsets, f(sp.X_hist), f(sp.X_cand if Xc is None else Xc),
                                f64_layers(sp.layers), H=sp.H, d=sp.d, hist_ts=sp.hist_ts, cand_ts=sp.cand_ts,
                                hist_group=sp.hist_group, cand_group=sp.cand_group, n_groups=sp.n_groups,
                                n_max=sp.n_max, norm=sp.norm, eps=sp.eps, time_filter=sp.time_filter)


@pytest.mark.parametrize("sp", _stacks(), ids=lambda sp: sp.name)
def test_stack_matches_full_pass_oracle(sp):
    _say("stack", sp.name, sp.dtype, "layers", len(sp.layers), "hist", np.diff(sp.hist_offsets).tolist(),
         "cand", np.diff(sp.cand_offsets).tolist())
    ns = device.upload_stack(sp)
    h = device.run_stack_history(ns)
    s = device.run_stack_score(ns)
    torch.cuda.synchronize()
    assert api.device_status(h.ws) == 0 and api.device_status(s.ws) == 0
    ref = _oracle(sp)
    errs = {"Out": rel_l2(s.Out.float().cpu().numpy(), ref["Out"]),
            "Out_hist": rel_l2(h.Out.float().cpu().numpy(), ref["Out_hist"])}
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= _tol(sp), (k, v)
    # the microbatch does not change the result, bit for bit
    s0 = device.run_stack_score(ns, microbatch=0)
    torch.cuda.synchronize()
    assert torch.equal(s0.Out, s.Out)


def test_stack_caches_serve_a_second_request():
    """Caches built once serve a second candidate set of the same users."""
    sp = _stacks()[1]
    ns = device.upload_stack(sp)
    device.run_stack_history(ns)
    first = device.run_stack_score(ns)
    sp2 = synth.stack_custom("S_bf16_gln_rab", [300, 64, 1, 129], [33, 64, 7, 100], n_layers=3, H=2, d=64, wid=151,
                             microbatch=32, norm=synth.NORM_GLN, x_std=1.0, w_std=0.05, bias_std=0.2, n_pos=512,
                             n_tb=20, rab_std=0.3, gamma_std=0.3, beta_std=0.3, x_cand_seed=1)
    second = device.run_stack_score(ns, Xc=sp2.X_cand.to(ns.device))
    torch.cuda.synchronize()
    for got, Xc in ((first.Out, sp.X_cand), (second.Out, sp2.X_cand)):
        e = rel_l2(got.float().cpu().numpy(), _oracle(sp, Xc)["Out"])
        _say(f"  request err={e:.2e}")
        assert e <= _tol(sp)


def test_stack_graph_replays_match_eager():
    """A captured hstu_stack_score replayed with new candidate features in the
    same buffer, with eager work in between, equals the eager call on the same
    input every time (and the oracle)."""
    sp = _stacks()[2]
    ns = device.upload_stack(sp)
    device.run_stack_history(ns)
    Xc = ns.X_cand.clone()
    eager = device.run_stack_score(ns, Xc=Xc)   # also settles the GEMM algorithm choices
    torch.cuda.synchronize()
    graph, gout = api.stack_score_capture(ns.cand_problem, ns.layers, ns.hist_offsets, ns.hist_tokens,
                                          ns.hist_max_len, Xc, hist_ts=ns.hist_ts, microbatch=sp.microbatch)
    for r in range(4):
        new = synth.stack_custom("S_bf16_d128_norab", [200, 257], [130, 64], n_layers=2, H=4, d=128, wid=152,
                                 microbatch=64, x_std=1.0, w_std=0.03, bias_std=0.2, x_cand_seed=r + 2).X_cand
        Xc.copy_(new.to(ns.device))
        graph.launch()
        torch.cuda.synchronize()
        want = device.run_stack_score(ns, Xc=Xc.clone())
        torch.cuda.synchronize()
        _say(f"  replay {r}: equal={torch.equal(gout.Out, want.Out)}")
        assert torch.equal(gout.Out, want.Out)
        if r == 0:
            e = rel_l2(gout.Out.float().cpu().numpy(), _oracle(sp, new)["Out"])
            _say(f"  replay 0 vs oracle {e:.2e}")
            assert e <= _tol(sp)
    del graph
    assert torch.isfinite(eager.Out.float()).all()


def test_stack_full_shape_on_one_user():
    """The 3-layer M-FALCON serving shape (16 users x 2048 history x 1024
    candidates, d_model = D = 1024) at full size; one user's candidate rows
    against the oracle's full pass over that user alone (a user's rows depend
    only on that user)."""
    sp = synth.mfalcon_stack_bf16()
    ns = device.upload_stack(sp)
    device.run_stack_history(ns)
    s = device.run_stack_score(ns)
    torch.cuda.synchronize()
    assert api.device_status(s.ws) == 0
    u = 5
    hs, he = int(sp.hist_offsets[u]), int(sp.hist_offsets[u + 1])
    cs, ce = int(sp.cand_offsets[u]), int(sp.cand_offsets[u + 1])
    f = lambda t: t.double().numpy()
    ref = oracle.mfalcon_stack([0, he - hs], [0, ce - cs], f(sp.X_hist[hs:he]), f(sp.X_cand[cs:ce]),
                               f64_layers(sp.layers),
                               H=sp.H, d=sp.d, n_max=sp.n_max, norm=sp.norm, eps=sp.eps)
    e = rel_l2(s.Out[cs:ce].float().cpu().numpy(), ref["Out"])
    _say(f"  user {u}: err={e:.2e}")
    assert e <= _tol(sp)
