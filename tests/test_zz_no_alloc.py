"""hstu_attn_fwd_static (the forward with the library's static device
scratch, for callers that cannot allocate) through the C ABI against
hstu_attn_fwd with a caller workspace: two calls in a row, the second on a
smaller problem, then the first again; outputs bit-identical (the same
kernels run on the same inputs) and within the oracle bound."""
import numpy as np
import pytest
import torch

import oracle
from hstu_jagged_pointwise_attn_amd import api, device, synth
from tests.common import oracle_fwd, rel_l2, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)


def _problems():
    big = synth.custom("static_big", [700, 3, 129, 1000, 64, 0, 333], H=4, d=128, wid=401, std=0.3, n_max=1000,
                       prefix_len=[100, 0, 0, 200, 10, 0, 0], cand_len=[50, 1, 20, 100, 0, 0, 33], n_pos=1024,
                       n_tb=32, rab_std=0.3, gamma_std=0.3, beta_std=0.3)
    small = synth.custom("static_small", [90, 17], H=2, d=64, wid=402, std=0.3, n_max=90, n_pos=128, n_tb=16,
                         rab_std=0.3)
    return big, small


def _check(p, ns):
    ref = device.run_fwd(ns)
    got = api.attn_fwd_static(ns.problem, ns.Q, ns.K, ns.V, ns.U)
    torch.cuda.synchronize()
    for name in ("Y", "O", "mean", "rstd"):
        assert torch.equal(getattr(got, name), getattr(ref, name)), name
    o = oracle_fwd(p)
    ey, eo = rel_l2(got.Y, o["Y"]), rel_l2(got.O, o["O"])
    print(f"static {p.name}: Y {ey:.2e} O {eo:.2e}", flush=True)
    assert ey <= tol(p) and eo <= tol(p)
    return got


def test_static_forward_two_calls_then_first_again():
    big, small = _problems()
    nb, ns = device.upload(big), device.upload(small)
    print("static scratch bytes", api.static_scratch_bytes(), "need", api.workspace_size(nb.problem, api.HSTU_OP_FWD),
          flush=True)
    g1 = _check(big, nb)
    _check(small, ns)
    g3 = api.attn_fwd_static(nb.problem, nb.Q, nb.K, nb.V, nb.U)
    torch.cuda.synchronize()
    assert torch.equal(g1.Y, g3.Y) and torch.equal(g1.O, g3.O)
