"""Small forwards whose attention workgroups build their own tiles (no
scheduler launch) against the same forwards with the scheduler kernel, and
against the CPU oracle; status bits through both paths."""
import numpy as np
import pytest
import torch

import oracle
from hstu_jagged_pointwise_attn_amd import _lib, api, device, synth
from tests.common import oracle_fwd, rel_l2, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    yield
    api.set_inline_schedule(True)


def _say(*a):
    print(*a, flush=True)


def _problems():
    L = np.array([150, 40, 133, 7, 0, 300])
    P = np.array([100, 0, 60, 3, 0, 50]); C = np.array([30, 40, 33, 2, 0, 64])
    grp = np.concatenate([np.minimum(np.arange(l) * 3 // max(l, 1), 2) for l in L]).astype(np.int64)
    ps = [
        synth.tiny_fp32(),
        synth.custom("inl_bf16_causal_rab", [300, 1, 129, 64, 0, 257], H=2, d=128, wid=81, std=0.3, n_max=64,
                     n_pos=300, n_tb=20, rab_std=0.3),
        synth.custom("inl_bf16_mtgr_gln", L, H=3, d=64, wid=82, std=0.3, n_max=300, norm=synth.NORM_GLN,
                     prefix_len=P, cand_len=C, group=grp, n_groups=3, gamma_std=0.3, beta_std=0.3, n_pos=64,
                     n_tb=12, rab_std=0.3),
        synth.custom("inl_bf16_d32_none", [200, 65, 3], H=4, d=32, wid=83, std=0.5, n_max=8,
                     norm=synth.NORM_NONE, cand_len=[20, 0, 3], n_pos=40, rab_std=0.3),
        synth.custom("inl_f32_mtgr", L, H=2, d=64, dtype=torch.float32, wid=84, std=0.4, n_max=16,
                     norm=synth.NORM_GLN, prefix_len=P, cand_len=C, group=grp, n_groups=3, gamma_std=0.3,
                     beta_std=0.3, n_pos=64, n_tb=10, rab_std=0.3),
        synth.custom("inl_seqs_256", np.random.default_rng(85).integers(0, 40, 256), H=2, d=64, wid=85, std=0.3,
                     n_max=64, n_pos=64, n_tb=16, rab_std=0.3),
    ]
    tf = synth.custom("inl_bf16_time_filter", L, H=2, d=64, wid=86, std=0.3, n_max=300, prefix_len=P, cand_len=C,
                      n_pos=64, n_tb=12, rab_std=0.3)
    tf = synth.interleave_candidate_times(tf, seed=86)
    tf.time_filter = True
    ps.append(tf)
    return ps


def _sched_launches(fn):
    api.kernel_timing(True)
    out = fn()
    torch.cuda.synchronize()
    _, n = api.kernel_timing_read(_lib.HSTU_KERNEL_SCHED)
    api.kernel_timing(False)
    return out, n


@pytest.mark.parametrize("p", _problems(), ids=lambda p: p.name)
def test_inline_tiles_match_scheduled_and_oracle(p):
    _say(f"[inline] {p.name} B={p.B} T={p.T} H={p.H} d={p.d}")
    ns = device.upload(p)
    api.set_inline_schedule(True)
    a, n_inl = _sched_launches(lambda: device.run_fwd(ns))
    sa = api.device_status(a.ws)
    api.set_inline_schedule(False)
    b, n_sch = _sched_launches(lambda: device.run_fwd(ns))
    sb = api.device_status(b.ws)
    api.set_inline_schedule(True)
    _say(f"  scheduler launches: inline {n_inl}, scheduled {n_sch}; status {sa} / {sb}")
    assert n_inl == 0 and n_sch == 1
    assert sa == sb == 0
    for name in ("O", "Y", "mean", "rstd"):
        assert torch.equal(getattr(a, name), getattr(b, name)), f"{name} differs between the two paths"
    ref = oracle_fwd(p)
    eo, ey = rel_l2(a.O, ref["O"]), rel_l2(a.Y, ref["Y"])
    _say(f"  O {eo:.2e} Y {ey:.2e}")
    assert eo <= tol(p) and ey <= tol(p)


def test_inline_status_bits_and_their_lifetime():
    """TOO_LONG and BAD_TIMESTAMPS come out of the inline path as out of the
    scheduled one, and a clean call on the same workspace clears them."""
    p = synth.custom("inl_flags", [150, 250, 90], H=2, d=64, wid=87, std=0.3, n_max=250, n_pos=256, n_tb=40,
                     rab_std=0.3)
    ts = p.ts.copy()
    ts[150:400] = 1_700_000_000 + np.arange(250, dtype=np.int64) * 20_000_000   # a 5e9 s span
    bad = synth.custom("inl_flags", [150, 250, 90], H=2, d=64, wid=87, std=0.3, n_max=250, n_pos=256, n_tb=40,
                       rab_std=0.3)
    bad.ts = ts
    ns_good, ns_bad = device.upload(p), device.upload(bad)
    for inline in (True, False):
        api.set_inline_schedule(inline)
        f = device.run_fwd(ns_bad)
        s_bad = api.device_status(f.ws)
        device.run_fwd(ns_good, ws=f.ws)
        s_good = api.device_status(f.ws)
        ns_good.problem.max_len = 200
        device.run_fwd(ns_good, ws=f.ws)
        s_long = api.device_status(f.ws)
        ns_good.problem.max_len = p.max_len
        device.run_fwd(ns_good, ws=f.ws)
        s_clean = api.device_status(f.ws)
        _say(f"  inline={inline}: bad ts {s_bad}, then clean {s_good}, too long {s_long}, clean {s_clean}")
        assert s_bad == _lib.HSTU_DEV_BAD_TIMESTAMPS
        assert s_good == 0 and s_clean == 0
        assert s_long == _lib.HSTU_DEV_TOO_LONG
    api.set_inline_schedule(True)
