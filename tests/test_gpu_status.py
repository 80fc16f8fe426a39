"""GPU tests of the device-side precondition flags (HSTU_DEV_TOO_LONG,
HSTU_DEV_BAD_TIMESTAMPS) and of the backward's key-major schedule beyond the
scheduler's sort capacity, through the C ABI against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from hstu_jagged_pointwise_attn_amd import _lib, api, device, synth
from tests.common import oracle_bwd, oracle_fwd, rel_l2, tol
from tests.test_gpu_bwd import _compare, check_errs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)


def _say(*a):
    print(*a, flush=True)


def _rows(p, seqs):
    return np.concatenate([np.arange(p.offsets[s], p.offsets[s + 1]) for s in seqs])


def _fwd_bwd(p, ns=None):
    ns = ns or device.upload(p)
    f = device.run_fwd(ns)
    fs = api.device_status(f.ws)
    g = api.attn_bwd(ns.problem, ns.Q, ns.K, ns.V, ns.U, f.O, f.mean, f.rstd, ns.dY)
    bs = api.device_status(g.ws)
    torch.cuda.synchronize()
    return f, g, fs, bs


def test_too_long_flag_and_other_sequences():
    """A sequence longer than max_len raises HSTU_DEV_TOO_LONG and is treated
    as empty; the other sequences are computed as usual."""
    p = synth.custom("too_long", [100, 300, 64], H=2, d=64, wid=301, std=0.3, n_max=300, n_pos=320, n_tb=16,
                     rab_std=0.3, with_dy=True)
    ns = device.upload(p)
    ns.problem.max_len = 200   # sequence 1 (300 tokens) is longer
    f, g, fs, bs = _fwd_bwd(p, ns)
    _say("too_long: status fwd", fs, "bwd", bs)
    assert fs & _lib.HSTU_DEV_TOO_LONG and bs & _lib.HSTU_DEV_TOO_LONG
    good = [0, 2]
    sub = synth.subbatch(p, good)
    rows = _rows(p, good)
    ref = oracle_fwd(sub)
    D = p.H * p.d
    ey = rel_l2(f.Y.float().cpu().numpy()[rows], ref["Y"])
    rb = oracle_bwd(sub)
    errs = {"Y": ey}
    for name in ("dQ", "dK", "dV", "dU"):
        errs[name] = rel_l2(getattr(g, name).float().cpu().numpy().reshape(p.T, D)[rows], rb[name])
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= tol(p), (k, v)


def _with_times(p, b, t):
    ts = p.ts.copy()
    s, e = int(p.offsets[b]), int(p.offsets[b + 1])
    ts[s:e] = t
    p.ts = ts
    return p


def test_bad_timestamps_wide_span():
    """A sequence whose timestamps span 5e9 s raises HSTU_DEV_BAD_TIMESTAMPS in
    the forward and the backward; the other sequences are unaffected."""
    p = synth.custom("bad_ts", [150, 250, 90], H=2, d=64, wid=302, std=0.3, n_max=250, n_pos=256, n_tb=40,
                     rab_std=0.3, with_dy=True)
    _with_times(p, 1, 1_700_000_000 + np.arange(250, dtype=np.int64) * 20_000_000)
    f, g, fs, bs = _fwd_bwd(p)
    _say("bad_ts: status fwd", fs, "bwd", bs)
    assert fs & _lib.HSTU_DEV_BAD_TIMESTAMPS and bs & _lib.HSTU_DEV_BAD_TIMESTAMPS
    good = [0, 2]
    rows = _rows(p, good)
    sub = synth.subbatch(p, good)
    ref = oracle_fwd(sub)
    ey = rel_l2(f.Y.float().cpu().numpy()[rows], ref["Y"])
    _say(f"  Y (other sequences) {ey:.2e}")
    assert ey <= tol(p)


def test_bad_timestamps_key_major_pass():
    """A span between 2^31 and 2^32 s that every query tile of the forward
    and the dQ pass represents exactly (each time within 2^31 of its tile's
    first row), but that the key-major dK/dV pass (times relative to a key
    tile's first key) cannot: the forward is exact and clean, the backward
    raises HSTU_DEV_BAD_TIMESTAMPS."""
    p = synth.custom("span_2p31", [200, 60], H=1, d=64, wid=303, std=0.3, n_max=200, n_pos=256, n_tb=40,
                     rab_std=0.3, with_dy=True)
    t = np.empty(200, np.int64)
    t[:128] = 1_000 + np.arange(128) * 10
    t[128:] = 2_100_000_000 + np.arange(72) * 1_000_000   # last row 2.171e9 s after the first
    _with_times(p, 0, t)
    f, g, fs, bs = _fwd_bwd(p)
    _say("span_2p31: status fwd", fs, "bwd", bs)
    assert fs == 0
    assert bs & _lib.HSTU_DEV_BAD_TIMESTAMPS
    ref = oracle_fwd(p)
    eo = rel_l2(f.O, ref["O"])
    _say(f"  O {eo:.2e}")
    assert eo <= tol(p)


def test_bwd_key_schedule_over_sort_cap():
    """4000 sequences of 140 tokens: 12000 key tiles of 64 in the backward's
    key-major pass, more than the scheduler sorts (canonical order), and 8000
    query tiles; all gradients against the oracle."""
    lengths = np.full(4000, 140)
    p = synth.custom("many_key_tiles", lengths, H=1, d=32, wid=304, std=0.3, n_max=140, n_pos=160, n_tb=16,
                     rab_std=0.3, with_dy=True)
    _say("many_key_tiles T", p.T)
    f, g, fs, bs = _fwd_bwd(p)
    assert fs == 0 and bs == 0
    errs = _compare(p, g, oracle_bwd(p))
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    check_errs(p, errs)
