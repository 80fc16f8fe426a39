"""GPU parity of the forward path, the tile scheduler and M-FALCON scoring
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from hstu_jagged_pointwise_attn_amd import api, device, synth
from tests.common import oracle_fwd, oracle_mfalcon, rel_l2, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ problems

def _small_problems():
    ps = []
    ps.append(synth.tiny_fp32())
    ps.append(synth.custom("causal_rab_bf16", [300, 1, 129, 64, 0, 257], H=2, d=128, wid=31, std=0.3,
                           n_max=64, n_pos=300, n_tb=20, rab_std=0.3))
    L = np.array([150, 40, 333, 7])
    P = np.array([100, 0, 200, 3]); C = np.array([30, 40, 60, 2])
    grp = np.concatenate([np.minimum(np.arange(l) * 4 // l, 3) for l in L])
    ps.append(synth.custom("mtgr_small", L, H=3, d=64, wid=32, std=0.3, n_max=300, norm=synth.NORM_GLN,
                           prefix_len=P, cand_len=C, group=grp, n_groups=4, gamma_std=0.3, beta_std=0.3,
                           n_pos=64, n_tb=12, rab_std=0.3))
    ps.append(synth.custom("none_norm_d32", [200, 65, 3], H=4, d=32, wid=33, std=0.5, n_max=8,
                           norm=synth.NORM_NONE, cand_len=[20, 0, 3]))
    ps.append(synth.custom("ln_active", [190, 77], H=2, d=128, wid=34, std=1.0, qk_std=0.1, n_max=1,
                           norm=synth.NORM_LN, gamma_std=0.5, beta_std=0.5))
    ps.append(synth.custom("f32_mtgr", [70, 130], H=2, d=64, dtype=torch.float32, wid=35, std=0.3,
                           n_max=16, prefix_len=[20, 50], cand_len=[10, 30], n_pos=32, n_tb=8,
                           rab_std=0.3))
    ps.append(synth.custom("f32_d128", [90, 3, 64], H=1, d=128, dtype=torch.float32, wid=36, std=0.3,
                           n_max=4, norm=synth.NORM_LN, n_pos=16, n_tb=8))
    return ps


@pytest.mark.parametrize("p", _small_problems(), ids=lambda p: p.name)
def test_fwd_matches_oracle_small(p):
    _say("fwd", p.name, p.dtype, p.offsets.tolist())
    ns = device.upload(p)
    out = device.run_fwd(ns)
    torch.cuda.synchronize()
    assert api.device_status(out.ws) == 0
    ref = oracle_fwd(p)
    eo, ey = rel_l2(out.O, ref["O"]), rel_l2(out.Y, ref["Y"])
    _say(f"  rel_l2 O={eo:.2e} Y={ey:.2e}")
    assert eo <= tol(p) and ey <= tol(p)
    if p.norm != synth.NORM_NONE:
        assert rel_l2(out.mean, ref["mean"]) <= max(tol(p), 1e-3)
        assert rel_l2(out.rstd, ref["rstd"]) <= tol(p)


def _sample_rows(p, n=96, seed=0):
    rng = np.random.default_rng(seed)
    lens = p.lengths
    off = p.offsets
    rows = set()
    for b in (int(np.argmax(lens)), int(np.argmin(lens))):
        if lens[b]:
            rows.update([off[b], off[b] + lens[b] // 2, off[b + 1] - 1])
    rows.update(rng.integers(0, p.T, size=n).tolist())
    sel = np.zeros(p.T, dtype=np.uint8)
    sel[sorted(rows)] = 1
    return sel


@pytest.mark.parametrize("name", ["train", "train_literal", "mtgr", "long"])
def test_fwd_full_size_sampled_rows(name):
    p = synth.WORKLOADS[name]()
    _say("fwd full", name, "B", p.B, "T", p.T, "max", p.max_len)
    ns = device.upload(p)
    out = device.run_fwd(ns)
    torch.cuda.synchronize()
    assert api.device_status(out.ws) == 0
    sel = _sample_rows(p)
    ref = oracle_fwd(p, row_sel=sel)
    rows = np.nonzero(sel)[0]
    eo = rel_l2(out.O.float().cpu().numpy()[rows], ref["O"][rows])
    ey = rel_l2(out.Y.float().cpu().numpy()[rows], ref["Y"][rows])
    _say(f"  rows {len(rows)} rel_l2 O={eo:.2e} Y={ey:.2e}")
    assert eo <= tol(p) and ey <= tol(p)


# ------------------------------------------------------------------ scheduler

def _expected_tiles(entries):
    order = oracle.lpt_order(entries) if len(entries) <= 8192 else list(range(len(entries)))
    out = []
    for g in order:
        k = entries[g]["kinds"]
        nk = int(np.count_nonzero(k))
        nf = int(np.count_nonzero(k == 2))
        out.append((entries[g]["b"], entries[g]["row0"], nk, nf, entries[g]["nrows"]))
    return out


def _got_tiles(tiles):
    return [(int(t[0]), int(t[1]), int(t[2]), int(t[3]) & 0xFFFF, int(t[3]) >> 16) for t in tiles]


def _many_tiles(n_seqs, seed, lo=1, hi=400):
    """Many short sequences: the longest-first order of a few thousand query
    tiles (several sort keys per thread in the scheduler's sort); with
    lengths of 129..500 and 4000 sequences, more query tiles (about 11.6k)
    than the scheduler sorts, so it keeps the canonical order."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi, size=n_seqs)
    return synth.custom(f"many_tiles_{n_seqs}", lengths, H=1, d=32, wid=seed, std=0.3, n_max=hi)


@pytest.mark.parametrize("name", ["tiny_fp32", "causal_rab_bf16", "mtgr_small", "train", "mtgr", "long",
                                  "many_tiles_900", "many_tiles_1500", "many_tiles_3500", "over_sort_cap_4000"])
def test_schedule_bit_exact(name):
    if name.startswith("over_sort_cap_"):
        n = int(name.rsplit("_", 1)[1])
        p = _many_tiles(n, 171, lo=129, hi=501)
    elif name.startswith("many_tiles_"):
        n = int(name.rsplit("_", 1)[1])
        p = _many_tiles(n, 170 + n % 97)
    else:
        p = synth.WORKLOADS[name]() if name in synth.WORKLOADS else {q.name: q for q in _small_problems()}[name]
    print("schedule", name, "B", p.B, flush=True)
    ns = device.upload(p)
    BM, BN = api.tile_shape(ns.problem)
    qoff, tiles = api.schedule_export(ns.problem)
    entries = oracle.schedule(p.offsets, BM, BN, prefix_len=p.prefix_len, cand_len=p.cand_len)
    if name.startswith("over_sort_cap_"):
        assert len(entries) > 8192, len(entries)
    counts = np.bincount([e["b"] for e in entries], minlength=p.B)
    np.testing.assert_array_equal(qoff, np.concatenate([[0], np.cumsum(counts)]))
    assert _got_tiles(tiles) == _expected_tiles(entries)


@pytest.mark.parametrize("microbatch,m_cand", [(0, 200), (256, 200), (100, 200), (1, 20), (1, 3000)])
def test_schedule_mfalcon_bit_exact(microbatch, m_cand):
    """(1, 3000): one candidate per microbatch, 9000 query tiles, more than
    the scheduler sorts."""
    mf = synth.mfalcon_bf16(users=3, n_hist=300, m_cand=m_cand, microbatch=microbatch, H=2, d=64)
    ns = device.upload_mfalcon(mf)
    BM, BN = api.tile_shape(ns.problem, api.HSTU_OP_MFALCON)
    qoff, tiles = api.schedule_export(ns.problem, api.HSTU_OP_MFALCON, ns.hist_offsets, ns.hist_tokens,
                                      ns.hist_max_len, microbatch)
    entries = oracle.schedule_mfalcon(mf.hist_offsets, mf.cand_offsets, BM, BN, microbatch)
    assert _got_tiles(tiles) == _expected_tiles(entries)


# ------------------------------------------------------------------ M-FALCON

def test_mfalcon_matches_oracle_small():
    mf = synth.mfalcon_bf16(users=3, n_hist=333, m_cand=150, microbatch=64, H=2, d=128, with_rab=True)
    mf.rab_p = mf.rab_p[:400].copy()
    ns = device.upload_mfalcon(mf)
    out = device.run_mfalcon(ns)
    torch.cuda.synchronize()
    assert api.device_status(out.ws) == 0
    ref = oracle_mfalcon(mf)
    eo, ey = rel_l2(out.O, ref["O"]), rel_l2(out.Y, ref["Y"])
    _say(f"mfalcon small rel_l2 O={eo:.2e} Y={ey:.2e}")
    assert eo <= 1e-2 and ey <= 1e-2


def test_mfalcon_full_size_two_users():
    """The full 16-user workload on the GPU; users 0 and 15 against the oracle."""
    mf = synth.mfalcon_bf16()
    ns = device.upload_mfalcon(mf)
    out = device.run_mfalcon(ns)
    torch.cuda.synchronize()
    assert api.device_status(out.ws) == 0
    users = [0, mf.B - 1]
    ho, co = mf.hist_offsets, mf.cand_offsets
    hrows = np.concatenate([np.arange(ho[u], ho[u + 1]) for u in users])
    crows = np.concatenate([np.arange(co[u], co[u + 1]) for u in users])
    sub = synth.MFalconProblem(
        name="mf_sub", dtype=mf.dtype, H=mf.H, d=mf.d,
        hist_offsets=np.concatenate([[0], np.cumsum([ho[u + 1] - ho[u] for u in users])]).astype(np.int32),
        cand_offsets=np.concatenate([[0], np.cumsum([co[u + 1] - co[u] for u in users])]).astype(np.int32),
        K_cache=mf.K_cache[hrows], V_cache=mf.V_cache[hrows], Qc=mf.Qc[crows], Kc=mf.Kc[crows],
        Vc=mf.Vc[crows], Uc=mf.Uc[crows], n_max=mf.n_max, microbatch=mf.microbatch, norm=mf.norm, eps=mf.eps)
    ref = oracle_mfalcon(sub)
    ey = rel_l2(out.Y.float().cpu().numpy()[crows], ref["Y"])
    eo = rel_l2(out.O.float().cpu().numpy()[crows], ref["O"])
    _say(f"mfalcon full rel_l2 O={eo:.2e} Y={ey:.2e}")
    assert eo <= 1e-2 and ey <= 1e-2


def test_mfalcon_microbatching_is_exact():
    mf = synth.mfalcon_bf16(users=4, n_hist=500, m_cand=300, microbatch=0, H=2, d=128, with_rab=True)
    ns = device.upload_mfalcon(mf)
    base = device.run_mfalcon(ns, microbatch=0)
    for mb in (256, 100, 37, 1):
        r = device.run_mfalcon(ns, microbatch=mb)
        torch.cuda.synchronize()
        assert torch.equal(r.Y, base.Y), mb
        assert torch.equal(r.O, base.O), mb


def test_mfalcon_candidate_permutation_permutes_outputs():
    mf = synth.mfalcon_bf16(users=3, n_hist=400, m_cand=200, microbatch=64, H=2, d=128, with_rab=True)
    ns = device.upload_mfalcon(mf)
    base = device.run_mfalcon(ns)
    rng = np.random.default_rng(7)
    perm = np.concatenate([mf.cand_offsets[b] + rng.permutation(mf.cand_offsets[b + 1] - mf.cand_offsets[b])
                           for b in range(mf.B)])
    pt = torch.from_numpy(perm).to(ns.device)
    for name in ("Qc", "Kc", "Vc", "Uc"):
        setattr(ns, name, getattr(ns, name)[pt].contiguous())
    ns.cand_ts = ns.cand_ts[pt].contiguous()
    ns.problem.timestamps = api._ptr(ns.cand_ts)
    r = device.run_mfalcon(ns)
    torch.cuda.synchronize()
    assert torch.equal(r.Y, base.Y[pt])


def test_mfalcon_cached_equals_full_pass_on_gpu():
    mf = synth.mfalcon_bf16(users=3, n_hist=257, m_cand=190, microbatch=64, H=2, d=128, with_rab=True)
    ns = device.upload_mfalcon(mf)
    cached = device.run_mfalcon(ns)
    ho, co = mf.hist_offsets, mf.cand_offsets
    cat = lambda a, b: torch.cat(sum([[a[ho[u]:ho[u + 1]], b[co[u]:co[u + 1]]] for u in range(mf.B)], []))
    full = synth.Problem(
        name="mf_full", dtype=mf.dtype, H=mf.H, d=mf.d,
        offsets=np.concatenate([[0], np.cumsum(np.diff(ho) + np.diff(co))]).astype(np.int32),
        Q=cat(mf.Q_hist, mf.Qc), K=cat(mf.K_cache, mf.Kc), V=cat(mf.V_cache, mf.Vc), U=cat(mf.U_hist, mf.Uc),
        n_max=mf.n_max, norm=mf.norm, eps=mf.eps, cand_len=np.diff(co).astype(np.int32),
        ts=np.concatenate(sum([[mf.hist_ts[ho[u]:ho[u + 1]], mf.cand_ts[co[u]:co[u + 1]]] for u in range(mf.B)], [])),
        rab_p=mf.rab_p, rab_t=mf.rab_t)
    fns = device.upload(full)
    fo = device.run_fwd(fns)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(full.offsets[u + 1] - (co[u + 1] - co[u]), full.offsets[u + 1])
                           for u in range(mf.B)])
    rt = torch.from_numpy(rows).to(fns.device)
    assert torch.equal(cached.O, fo.O[rt])
    assert torch.equal(cached.Y, fo.Y[rt])


# ------------------------------------------------------------------ invariants

def test_masked_pairs_contribute_exactly_zero_on_gpu():
    """Perturb the K/V of a candidate key and of a causal key that shares its
    tile with rows that see it; rows that see neither must be bit-identical."""
    p = synth.custom("mz", [200, 130], H=2, d=128, wid=41, std=0.3, n_max=8, prefix_len=[60, 0],
                     cand_len=[50, 30], n_pos=256, n_tb=16)
    ns = device.upload(p)
    base = device.run_fwd(ns)
    keys = {0: [170, 120], 1: [110, 50]}   # local key indices per sequence
    K2, V2 = ns.K.clone(), ns.V.clone()
    for b, ks in keys.items():
        for k in ks:
            K2[p.offsets[b] + k] = K2[p.offsets[b] + k] * 3 + 1
            V2[p.offsets[b] + k] = V2[p.offsets[b] + k] * -5 + 2
    r = api.attn_fwd(ns.problem, ns.Q, K2, V2, ns.U)
    torch.cuda.synchronize()
    checked = 0
    for b, ks in keys.items():
        s, e = int(p.offsets[b]), int(p.offsets[b + 1])
        L, P, C = e - s, int(p.prefix_len[b]), int(p.cand_len[b])
        for i in range(L):
            if all(i != k and not oracle.visible(i, k, L, P, C) for k in ks):
                assert torch.equal(r.O[s + i], base.O[s + i]), (b, i)
                checked += 1
    assert checked > 100


def test_zero_queries_give_beta_times_u():
    p = synth.custom("zq", [150, 70], H=2, d=128, wid=42, std=0.5, n_max=8, norm=synth.NORM_LN, gamma_std=1.0,
                     beta_std=1.0, cand_len=[20, 5])
    p.Q = torch.zeros_like(p.Q)
    ns = device.upload(p)
    out = device.run_fwd(ns)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.O) == 0
    want = (torch.from_numpy(p.beta[0]).to(ns.device)[None, :] * ns.U.float().reshape(p.T, -1)).to(p.dtype)
    assert torch.equal(out.Y, want)


def test_empty_and_degenerate_batches():
    for lengths in ([0], [0, 0, 5, 0], [1], [1, 1, 1]):
        p = synth.custom("deg", lengths, H=2, d=64, wid=43, std=0.5, n_max=4, cand_len=[min(1, l) for l in lengths])
        ns = device.upload(p)
        out = device.run_fwd(ns)
        torch.cuda.synchronize()
        assert api.device_status(out.ws) == 0
        if p.T:
            ref = oracle_fwd(p)
            assert rel_l2(out.Y, ref["Y"]) <= 1e-2
    p = synth.custom("empty", [], H=2, d=64, wid=44, std=0.5, n_max=4)
    ns = device.upload(p)
    device.run_fwd(ns)
    torch.cuda.synchronize()


def test_device_status_flags_bad_inputs():
    p = synth.custom("bad", [50, 60, 70], H=1, d=64, wid=45, std=0.5, n_max=4, prefix_len=[10, 50, 0],
                     cand_len=[5, 20, 0], norm=synth.NORM_GLN, group=np.zeros(180, np.uint8), n_groups=2)
    p.group[100] = 7
    ns = device.upload(p)
    out = device.run_fwd(ns)
    st = api.device_status(out.ws)
    assert st & api.L.HSTU_DEV_BAD_SEGMENTS  # sequence 1 has P + C > L
    assert st & api.L.HSTU_DEV_BAD_GROUP
    # the other sequences are still computed correctly
    ref = oracle.fwd(p.offsets[[0, 1]], p.Q[:50].double().numpy(), p.K[:50].double().numpy(),
                     p.V[:50].double().numpy(), p.U[:50].double().numpy(), H=1, d=64, prefix_len=[10],
                     cand_len=[5], n_max=4, norm=synth.NORM_GLN, group=np.zeros(50, np.uint8), n_groups=2)
    assert rel_l2(out.Y[:50], ref["Y"]) <= 1e-2
