"""GPU parity at the edges of what the library accepts: the widest rows
(H*d = 4096 in bf16, 2048 in fp32, the norm kernels' largest register
tiles), the most sequences per call (8192) and one long sequence with many
key tiles, forward and backward, against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from hstu_jagged_pointwise_attn_amd import api, device, synth
from tests.common import oracle_bwd, oracle_fwd, rel_l2, tol
from tests.test_gpu_bwd import _compare, _run, check_errs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)


def _say(*a):
    print(*a, flush=True)


def _wide():
    grp = np.concatenate([np.arange(l) % 3 for l in (150, 70, 1)]).astype(np.uint8)
    return [
        synth.custom("wide_bf16_h32_d128", [150, 70, 1], H=32, d=128, wid=161, std=0.3, n_max=150,
                     norm=synth.NORM_GLN, group=grp, n_groups=3, gamma_std=0.3, beta_std=0.3,
                     n_pos=160, n_tb=16, rab_std=0.3, with_dy=True),
        synth.custom("wide_f32_h16_d128", [90, 33], H=16, d=128, dtype=torch.float32, wid=162, std=0.3,
                     n_max=90, norm=synth.NORM_LN, gamma_std=0.3, n_pos=90, n_tb=8, rab_std=0.3, with_dy=True),
    ]


@pytest.mark.parametrize("p", _wide(), ids=lambda p: p.name)
def test_widest_rows_fwd_bwd(p):
    _say("limits", p.name, p.offsets.tolist())
    _, f, g = _run(p)
    assert api.device_status(f.ws) == 0 and api.device_status(g.ws) == 0
    ref = oracle_fwd(p)
    assert rel_l2(f.O, ref["O"]) <= tol(p) and rel_l2(f.Y, ref["Y"]) <= tol(p)
    errs = _compare(p, g, oracle_bwd(p))
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    check_errs(p, errs)


def test_most_sequences_per_call():
    rng = np.random.default_rng(163)
    lengths = rng.integers(0, 5, size=8192)
    lengths[rng.integers(0, 8192, size=8)] = 200   # a few longer ones among them
    cand = np.minimum(lengths, rng.integers(0, 3, size=8192))
    p = synth.custom("max_seqs", lengths, H=2, d=64, wid=164, std=0.5, n_max=200, cand_len=cand,
                     n_pos=256, n_tb=8, rab_std=0.3)
    _say("limits max_seqs T", p.T)
    ns = device.upload(p)
    out = device.run_fwd(ns)
    torch.cuda.synchronize()
    assert api.device_status(out.ws) == 0
    ref = oracle_fwd(p)
    assert rel_l2(out.O, ref["O"]) <= tol(p) and rel_l2(out.Y, ref["Y"]) <= tol(p)


def test_one_long_sequence_sampled_rows():
    p = synth.custom("long_one", [12000, 5], H=1, d=32, wid=165, std=0.3, n_max=12000, n_pos=12000,
                     n_tb=32, rab_std=0.3)
    ns = device.upload(p)
    out = device.run_fwd(ns)
    torch.cuda.synchronize()
    assert api.device_status(out.ws) == 0
    sel = np.zeros(p.T, dtype=np.uint8)
    sel[[0, 1, 63, 64, 4095, 6000, 11998, 11999, 12000, 12004]] = 1
    rows = np.flatnonzero(sel)
    ref = oracle_fwd(p, row_sel=sel)
    eo = rel_l2(out.O.float().cpu().numpy()[rows], ref["O"][rows])
    ey = rel_l2(out.Y.float().cpu().numpy()[rows], ref["Y"][rows])
    _say(f"  rel_l2 O={eo:.2e} Y={ey:.2e}")
    assert eo <= tol(p) and ey <= tol(p)
