"""GPU parity of MTGR's timestamp-filtered candidate mask (hstu_problem_t
mask_flags = HSTU_MASK_CAND_TIME_FILTER: a candidate sees a key of the causal
segment only if the key is strictly earlier) against the CPU oracle, forward,
backward, schedule and M-FALCON, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from hstu_jagged_pointwise_attn_amd import api, device, synth
from tests.common import oracle_bwd, oracle_fwd, oracle_mfalcon, rel_l2, tol
from tests.test_gpu_bwd import _compare, check_errs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)


def _say(*a):
    print(*a, flush=True)


def _filtered(p, seed):
    synth.interleave_candidate_times(p, seed)
    p.time_filter = True
    return p


def _problems():
    L = np.array([150, 40, 333, 7, 200])
    P = np.array([100, 0, 200, 3, 0]); C = np.array([30, 40, 60, 2, 70])
    grp = np.concatenate([np.minimum(np.arange(l) * 4 // l, 3) for l in L])
    ps = [
        synth.custom("tf_bf16_rab_gln", L, H=3, d=64, wid=81, std=0.3, n_max=300, norm=synth.NORM_GLN,
                     prefix_len=P, cand_len=C, group=grp, n_groups=4, gamma_std=0.3, beta_std=0.3,
                     n_pos=64, n_tb=12, rab_std=0.3, with_dy=True),
        synth.custom("tf_bf16_times_only_d128", L, H=2, d=128, wid=82, std=0.3, n_max=64,
                     norm=synth.NORM_LN, prefix_len=P, cand_len=C, n_pos=300, rab_std=0.3, with_dy=True),
        synth.custom("tf_f32_rab", L, H=2, d=32, dtype=torch.float32, wid=83, std=0.4, n_max=16,
                     norm=synth.NORM_LN, prefix_len=P, cand_len=C, n_pos=64, n_tb=10, rab_std=0.3,
                     with_dy=True),
    ]
    return [_filtered(p, 90 + i) for i, p in enumerate(ps)]


@pytest.mark.parametrize("p", _problems(), ids=lambda p: p.name)
def test_filter_fwd_matches_oracle(p):
    _say("filter fwd", p.name, p.offsets.tolist())
    ns = device.upload(p)
    out = device.run_fwd(ns)
    torch.cuda.synchronize()
    assert api.device_status(out.ws) == 0
    ref = oracle_fwd(p)
    eo, ey = rel_l2(out.O, ref["O"]), rel_l2(out.Y, ref["Y"])
    _say(f"  rel_l2 O={eo:.2e} Y={ey:.2e}")
    assert eo <= tol(p) and ey <= tol(p)
    # the filter matters for these inputs: the unfiltered oracle is far off
    p.time_filter = False
    e_off = rel_l2(out.O, oracle_fwd(p)["O"])
    p.time_filter = True
    _say(f"  vs unfiltered oracle: {e_off:.2e}")
    assert e_off > 10 * tol(p)


def test_filter_schedule_bit_exact():
    p = _problems()[0]
    ns = device.upload(p)
    BM, BN = api.tile_shape(ns.problem)
    qoff, tiles = api.schedule_export(ns.problem)
    entries = oracle.schedule(p.offsets, BM, BN, prefix_len=p.prefix_len, cand_len=p.cand_len,
                              time_filter=True)
    order = oracle.lpt_order(entries)
    exp = []
    for g in order:
        e = entries[g]
        k = e["kinds"]
        nk = int(np.count_nonzero(k))
        nf = int(np.count_nonzero(k == 2))
        exp.append((e["b"], e["row0"], nk, nf, e["nrows"]))
    got = [(int(t[0]), int(t[1]), int(t[2]), int(t[3]) & 0xffff, int(t[3]) >> 16) for t in tiles]
    assert got == exp


def test_filter_hidden_keys_contribute_exactly_zero_on_gpu():
    """Perturbing V of a real-time token leaves bit-identical every candidate
    row that the filter hides it from."""
    p = _problems()[1]
    ns = device.upload(p)
    base = device.run_fwd(ns).O.clone()
    V2 = p.V.clone()
    hidden = np.zeros(p.T, dtype=bool)
    changed_keys = []
    for b in range(p.B):
        s = int(p.offsets[b]); Lb = int(p.lengths[b])
        P, C = int(p.prefix_len[b]), int(p.cand_len[b])
        E = Lb - C
        for j in range(max(P, E - 3), E):   # the latest real-time tokens
            V2[s + j] += 3.0
            changed_keys.append(s + j)
    ns.V = V2.to(ns.V.device)
    out = device.run_fwd(ns).O
    torch.cuda.synchronize()
    for b in range(p.B):
        s = int(p.offsets[b]); Lb = int(p.lengths[b])
        P, C = int(p.prefix_len[b]), int(p.cand_len[b])
        E = Lb - C
        ks = [j for j in changed_keys if s + P <= j < s + E]
        for i in range(E, Lb):
            if ks and all(not p.ts[j] < p.ts[s + i] for j in ks):
                hidden[s + i] = True
    rows = np.nonzero(hidden)[0]
    _say("candidate rows that see none of the perturbed keys:", len(rows))
    assert len(rows) > 0
    assert torch.equal(out[rows].cpu(), base[rows].cpu())


def test_filter_mfalcon_matches_oracle():
    mf = synth.mfalcon_bf16(users=3, n_hist=333, m_cand=150, microbatch=64, H=2, d=128, with_rab=True)
    mf.rab_p = mf.rab_p[:400].copy()
    rng = np.random.default_rng(7)
    for b in range(mf.B):
        hs, he, cs, ce = mf.hist_offsets[b], mf.hist_offsets[b + 1], mf.cand_offsets[b], mf.cand_offsets[b + 1]
        mf.cand_ts[cs:ce] = mf.hist_ts[rng.integers(hs, he, size=ce - cs)] + rng.integers(0, 2, size=ce - cs)
    mf.time_filter = True
    ns = device.upload_mfalcon(mf)
    out = device.run_mfalcon(ns)
    torch.cuda.synchronize()
    assert api.device_status(out.ws) == 0
    ref = oracle_mfalcon(mf)
    eo, ey = rel_l2(out.O, ref["O"]), rel_l2(out.Y, ref["Y"])
    _say(f"filter mfalcon rel_l2 O={eo:.2e} Y={ey:.2e}")
    assert eo <= 1e-2 and ey <= 1e-2


@pytest.mark.parametrize("p", _problems(), ids=lambda p: p.name)
def test_filter_bwd_matches_oracle(p):
    _say("filter bwd", p.name)
    ns = device.upload(p)
    f = device.run_fwd(ns)
    g = api.attn_bwd(ns.problem, ns.Q, ns.K, ns.V, ns.U, f.O, f.mean, f.rstd, ns.dY)
    torch.cuda.synchronize()
    assert api.device_status(g.ws) == 0
    ref = oracle_bwd(p)
    errs = _compare(p, g, ref)
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    check_errs(p, errs)
