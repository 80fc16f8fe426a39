"""Run-to-run reproducibility of the HIP path.

The forward has no atomics and a fixed tile order, so two runs on the same
inputs must agree bit for bit, also when other work ran in between (a
different cache state) and when the second run goes on another stream. In
the backward dQ, dK, dV and dU are each written by exactly one workgroup, so
they must be bit-identical too. The rab and affine gradients are sums that
workgroups add into with atomics in whatever order they finish: for them the
test asserts only that two runs agree far inside the parity tolerance."""
import numpy as np
import pytest
import torch

from hstu_jagged_pointwise_attn_amd import api, device, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _problems():
    L = np.array([150, 40, 133, 7, 600])
    P = np.array([100, 0, 60, 3, 300]); C = np.array([30, 40, 33, 2, 100])
    grp = np.concatenate([np.minimum(np.arange(l) * 3 // l, 2) for l in L])
    return [
        synth.custom("det_bf16_causal_rab", [300, 1, 129, 64, 0, 257, 1500], H=4, d=128, wid=71, std=0.3,
                     n_max=64, norm=synth.NORM_LN, n_pos=300, n_tb=20, rab_std=0.3, with_dy=True),
        synth.custom("det_bf16_mtgr_gln", L, H=3, d=64, wid=72, std=0.3, n_max=300, norm=synth.NORM_GLN,
                     prefix_len=P, cand_len=C, group=grp, n_groups=3, gamma_std=0.3, beta_std=0.3,
                     n_pos=64, n_tb=12, rab_std=0.3, with_dy=True),
        synth.custom("det_f32_causal_rab", [70, 1, 129, 64, 400], H=2, d=32, dtype=torch.float32, wid=73, std=0.4,
                     n_max=8, norm=synth.NORM_LN, n_pos=100, n_tb=12, rab_std=0.3, gamma_std=0.3, beta_std=0.3,
                     with_dy=True),
    ]


def _rel(a, b):
    a = a.double(); b = b.double()
    n = torch.linalg.norm(b)
    return float(torch.linalg.norm(a - b) / n) if n > 0 else float(torch.linalg.norm(a - b))


def _fwd_bwd(ns):
    f = device.run_fwd(ns)
    g = api.attn_bwd(ns.problem, ns.Q, ns.K, ns.V, ns.U, f.O, f.mean, f.rstd, ns.dY)
    return f, g


@pytest.mark.parametrize("p", _problems(), ids=lambda p: p.name)
def test_forward_and_backward_reproduce(p):
    print(f"[determinism] {p.name} T={p.T} H={p.H} d={p.d}", flush=True)
    ns = device.upload(p)
    f1, g1 = _fwd_bwd(ns)
    torch.cuda.synchronize()
    # Other work in between: a large write that evicts the caches.
    junk = torch.empty(64 << 20, dtype=torch.float32, device="cuda")
    junk.fill_(1.0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f2, g2 = _fwd_bwd(ns)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del junk
    for name in ("O", "Y", "mean", "rstd"):
        assert torch.equal(getattr(f1, name), getattr(f2, name)), f"forward {name} differs between runs"
    for name in ("dQ", "dK", "dV", "dU"):
        assert torch.equal(getattr(g1, name), getattr(g2, name)), f"{name} differs between runs"
    bound = 1e-6 if p.dtype == torch.float32 else 1e-4
    for name in ("d_rab_p", "d_rab_t", "d_gamma", "d_beta"):
        a, b = getattr(g1, name), getattr(g2, name)
        if a is None:
            continue
        r = _rel(a, b)
        print(f"  {name}: run-to-run rel {r:.2e}", flush=True)
        assert r <= bound, f"{name} run-to-run rel {r:.2e} > {bound:.0e}"
