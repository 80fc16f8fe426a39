"""Seeded random problems against the CPU oracle, forward and backward: jagged
lengths (empty, single-token, tile-boundary and ragged), static prefixes and
candidate suffixes, H, d, dtype, rab tables, norm kind and the timestamp
filter drawn per case. Each case prints its seed and shape first."""
import numpy as np
import pytest
import torch

import oracle
from hstu_jagged_pointwise_attn_amd import api, device, synth
from tests.common import oracle_bwd, oracle_fwd, rel_l2, tol
from tests.test_gpu_bwd import _compare, _run, check_errs

pytestmark = pytest.mark.gpu

N_CASES = 16


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 7))
    lengths = rng.choice([0, 1, 2, 63, 64, 65, 127, 128, 129, 200, 300], size=B)
    P = np.array([int(rng.integers(0, l + 1)) if rng.random() < 0.4 else 0 for l in lengths])
    C = np.array([int(rng.integers(0, l - p + 1)) if rng.random() < 0.5 else 0 for l, p in zip(lengths, P)])
    H = int(rng.choice([1, 2, 3, 4]))
    d = int(rng.choice([32, 64, 128]))
    dtype = torch.float32 if rng.random() < 0.25 else torch.bfloat16
    norm = int(rng.choice([synth.NORM_NONE, synth.NORM_LN, synth.NORM_GLN]))
    use_p, use_t = rng.random() < 0.6, rng.random() < 0.6
    kw = {}
    if norm == synth.NORM_GLN:
        kw = dict(group=rng.integers(0, 3, size=int(lengths.sum())).astype(np.uint8), n_groups=3,
                  gamma_std=0.3, beta_std=0.3)
    elif norm == synth.NORM_LN and rng.random() < 0.5:
        kw = dict(gamma_std=0.3, beta_std=0.3)
    p = synth.custom(f"rand{seed}", lengths, H=H, d=d, dtype=dtype, wid=2000 + seed, std=0.3,
                     n_max=int(max(1, lengths.max())), norm=norm, prefix_len=P, cand_len=C,
                     n_pos=int(rng.choice([8, 64, 512])) if use_p else 0,
                     n_tb=int(rng.choice([4, 16, 40])) if use_t else 0, rab_std=0.3, with_dy=True, **kw)
    if use_t and C.sum() > 0 and rng.random() < 0.5:
        synth.interleave_candidate_times(p, seed)
        p.time_filter = True
    return p


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_problem_fwd_bwd(seed):
    p = _case(seed)
    print(f"random seed {seed}: lengths {p.lengths.tolist()} P {p.prefix_len.tolist()} C {p.cand_len.tolist()} "
          f"H {p.H} d {p.d} {p.dtype} norm {p.norm} rab_p {p.rab_p is not None} rab_t {p.rab_t is not None} "
          f"filter {p.time_filter}", flush=True)
    if p.T == 0:
        ns = device.upload(p)
        device.run_fwd(ns)
        torch.cuda.synchronize()
        return
    _, f, g = _run(p)
    assert api.device_status(f.ws) == 0 and api.device_status(g.ws) == 0
    ref = oracle_fwd(p)
    eo, ey = rel_l2(f.O, ref["O"]), rel_l2(f.Y, ref["Y"])
    errs = _compare(p, g, oracle_bwd(p))
    print(f"  O={eo:.2e} Y={ey:.2e} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert eo <= tol(p) and ey <= tol(p)
    check_errs(p, errs)
