"""GPU parity of the full HSTU layer (hstu_layer_fwd / hstu_layer_bwd through
the C ABI: the projections f1, f2 around the attention core) against the CPU
oracle's layer_fwd / layer_bwd."""
import numpy as np
import pytest
import torch

import oracle
from hstu_jagged_pointwise_attn_amd import api, device, synth
from tests.common import oracle_layer_bwd, oracle_layer_fwd, rel_l2, tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)


def _say(*a):
    print(*a, flush=True)


def _layers():
    out = []
    p = synth.custom("L_f32_causal_rab", [70, 1, 129, 64], H=2, d=32, dtype=torch.float32, wid=81, std=0.4,
                     n_max=8, norm=synth.NORM_LN, n_pos=100, n_tb=12, rab_std=0.3, gamma_std=0.3, beta_std=0.3)
    out.append(synth.with_layer(p, d_model=40, wid=91, x_std=1.0, w_std=0.1, bias_std=0.2))
    L = np.array([150, 40, 133, 7])
    P = np.array([100, 0, 60, 3]); C = np.array([30, 40, 33, 2])
    grp = np.concatenate([np.minimum(np.arange(l) * 3 // l, 2) for l in L])
    p = synth.custom("L_bf16_mtgr_gln", L, H=3, d=64, wid=82, n_max=300, norm=synth.NORM_GLN, prefix_len=P,
                     cand_len=C, group=grp, n_groups=3, gamma_std=0.3, beta_std=0.3, n_pos=64, n_tb=12,
                     rab_std=0.3)
    out.append(synth.with_layer(p, d_model=96, wid=92, x_std=1.0, w_std=0.1, bias_std=0.2))
    p = synth.custom("L_bf16_causal_d128", [300, 1, 129, 64, 0, 257], H=2, d=128, wid=83, n_max=64,
                     norm=synth.NORM_LN, n_pos=300, n_tb=20, rab_std=0.3)
    out.append(synth.with_layer(p, wid=93, x_std=1.0, w_std=0.05, bias_std=0.2))
    p = synth.custom("L_bf16_none_cand_d32_nobias", [200, 65, 3], H=4, d=32, wid=84, n_max=8,
                     norm=synth.NORM_NONE, cand_len=[20, 0, 3], n_pos=40, rab_std=0.3)
    out.append(synth.with_layer(p, d_model=100, wid=94, x_std=1.0, w_std=0.1, bias_std=None))
    p = synth.custom("L_bf16_time_filter", [160, 90], H=2, d=64, wid=85, n_max=32, norm=synth.NORM_LN,
                     prefix_len=[40, 10], cand_len=[50, 30], n_tb=16, rab_std=0.3)
    p.time_filter = True
    synth.interleave_candidate_times(p, seed=7)
    out.append(synth.with_layer(p, d_model=64, wid=95, x_std=1.0, w_std=0.1, bias_std=0.2))
    # 2103 tokens: the weight gradients split the tokens into 4 chunks of 525 and a remainder of 3
    p = synth.custom("L_bf16_split_remainder", [1000, 1103], H=2, d=64, wid=88, n_max=128, norm=synth.NORM_LN,
                     n_pos=256, n_tb=16, rab_std=0.3)
    out.append(synth.with_layer(p, d_model=128, wid=98, x_std=1.0, w_std=0.1, bias_std=0.2))
    return out


def _check_fwd(lp, f, ref, rows=None):
    errs = {}
    for name, got in (("Out", f.Out), ("Z", f.Z), ("Y", f.Y), ("O", f.O)):
        g = got.float().cpu().numpy()
        r = ref[name]
        if rows is not None:
            g, r = g[rows], r[rows]
        errs[name] = rel_l2(g, r)
    return errs


def _cases():
    ls = _layers()
    # the activations recomputed from Z in the backward, and (two cases) kept from the forward
    return [(lp, False) for lp in ls] + [(ls[0], True), (ls[1], True)]


@pytest.mark.parametrize("lp,save", _cases(), ids=lambda v: v.name if hasattr(v, "name") else f"save{int(v)}")
def test_layer_fwd_bwd_match_oracle(lp, save):
    _say("layer", lp.name, lp.core.dtype, "d_model", lp.d_model, "save_act", save, lp.core.offsets.tolist())
    ns = device.upload_layer(lp)
    f = device.run_layer_fwd(ns, save_act=save)
    assert (f.UVQK is not None) == save
    g = device.run_layer_bwd(ns, f)
    torch.cuda.synchronize()
    assert api.device_status(f.ws) == 0 and api.device_status(g.ws) == 0
    ref = oracle_layer_fwd(lp)
    errs = _check_fwd(lp, f, ref)
    rb = oracle_layer_bwd(lp)
    for name in ("dX", "dW1", "db1", "dW2", "db2"):
        got = getattr(g, name)
        if got is None or rb[name] is None or lp.b1 is None and name == "db1" or lp.b2 is None and name == "db2":
            continue
        errs[name] = rel_l2(got.float().cpu().numpy(), rb[name])
    for name, gname in (("dgamma", "d_gamma"), ("dbeta", "d_beta")):
        if rb[name] is not None and getattr(g, gname) is not None:
            errs[name] = rel_l2(getattr(g, gname).cpu().numpy(), rb[name])
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= tol(lp.core), (k, v)


@pytest.mark.parametrize("lp", _layers()[:4], ids=lambda v: v.name)
def test_layer_inference_form_without_z(lp):
    """Z = NULL: f1 as four GEMMs with the SiLU in their epilogue (U, V, Q, K
    rounded once); Out, Y and O match the oracle and the Z form."""
    _say("layer inference", lp.name)
    ns = device.upload_layer(lp)
    fz = device.run_layer_fwd(ns)
    fi = device.run_layer_fwd(ns, keep_z=False)
    torch.cuda.synchronize()
    assert fi.Z is None and api.device_status(fi.ws) == 0
    ref = oracle_layer_fwd(lp)
    for name in ("Out", "Y", "O"):
        got = getattr(fi, name)
        e_ref = rel_l2(got.float().cpu().numpy(), ref[name])
        e_z = rel_l2(got.float().cpu().numpy(), getattr(fz, name).float().cpu().numpy())
        _say(f"  {name}: vs oracle {e_ref:.2e}, vs the Z form {e_z:.2e}")
        assert e_ref <= tol(lp.core) and e_z <= tol(lp.core), name


def _fused_cases():
    out = [lp for lp in _layers() if lp.core.dtype == torch.bfloat16 and lp.d_model % 8 == 0]
    # d_model 72: a K tail of 8 columns; 3 heads x 32: column blocks that
    # straddle the 256-column tiles and a partial column tile (4D = 384);
    # 300 tokens: a partial token tile
    p = synth.custom("L_bf16_ktail", [180, 120], H=3, d=32, wid=89, n_max=32, norm=synth.NORM_LN, n_pos=64,
                     rab_std=0.3)
    out.append(synth.with_layer(p, d_model=72, wid=99, x_std=1.0, w_std=0.1, bias_std=0.2))
    return out


@pytest.mark.parametrize("lp", _fused_cases(), ids=lambda v: v.name)
def test_layer_fused_projection_matches_split_form(lp):
    """f1 as the library's own GEMM with the SiLU split epilogue against the
    library GEMM + separate SiLU pass: Z agrees to bf16 rounding, each of
    U, V, Q, K is SiLU of the stored Z (computed here in fp32, one bf16
    rounding apart), and the layer's outputs match the oracle either way;
    likewise the backward with SiLU' applied by the kernels that produce
    dU, dV, dQ, dK against the separate SiLU' pass."""
    _say("layer fused f1", lp.name, "d_model", lp.d_model, "D", lp.core.H * lp.core.d, "T", lp.T)
    ns = device.upload_layer(lp)
    prev = api.set_fused_projection(True)
    try:
        ff = device.run_layer_fwd(ns, save_act=True)
        gf = device.run_layer_bwd(ns, ff)
        api.set_fused_projection(False)
        fs = device.run_layer_fwd(ns, save_act=True)
        gs = device.run_layer_bwd(ns, fs)
    finally:
        api.set_fused_projection(prev)
    torch.cuda.synchronize()
    assert api.device_status(gf.ws) == 0 and api.device_status(gs.ws) == 0
    ref = oracle_layer_fwd(lp)
    rb = oracle_layer_bwd(lp)
    # backward: fused (the attention and norm kernels write dZ with SiLU')
    # and split (a separate SiLU' pass), both against the oracle
    for name, g in (("fused", gf), ("split", gs)):
        errs = {}
        for k in ("dX", "dW1", "db1", "dW2", "db2"):
            got = getattr(g, k)
            if got is None or rb[k] is None or (lp.b1 is None and k == "db1") or (lp.b2 is None and k == "db2"):
                continue
            errs[k] = rel_l2(got.float().cpu().numpy(), rb[k])
        _say(f"  {name} backward: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        for k, v in errs.items():
            assert v <= tol(lp.core), (name, k, v)
    D = lp.core.H * lp.core.d
    for name, f in (("fused", ff), ("split", fs)):
        errs = _check_fwd(lp, f, ref)
        z = f.Z.float()
        silu = (z * torch.sigmoid(z)).to(torch.bfloat16).float()
        act = f.UVQK.float().reshape(4, lp.T, D)
        for blk in range(4):
            got = act[blk]
            want = silu[:, blk * D:(blk + 1) * D]
            bad = (got - want).abs() > 2.0 ** -7 * want.abs() + 1e-6
            assert int(bad.sum()) == 0, (name, blk, int(bad.sum()))
        _say(f"  {name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        for k, v in errs.items():
            assert v <= tol(lp.core), (name, k, v)
    dz = (ff.Z.float() - fs.Z.float()).abs()
    assert rel_l2(ff.Z.float().cpu().numpy(), fs.Z.float().cpu().numpy()) <= 2e-3
    assert float(dz.max()) <= 2.0 ** -6 * float(fs.Z.float().abs().max())


def test_layer_bias_gradients_without_bias_inputs_are_column_sums():
    """With b1 = b2 = None the layer still returns db1, db2 (the gradients a
    zero bias would get): they must equal the column sums of dZ and dOut."""
    lp = _layers()[3]
    ns = device.upload_layer(lp)
    f = device.run_layer_fwd(ns)
    g = device.run_layer_bwd(ns, f)
    rb = oracle_layer_bwd(lp)
    assert rel_l2(g.db1.cpu().numpy(), rb["dZ"].sum(0)) <= 1e-2
    assert rel_l2(g.db2.cpu().numpy(), lp.dOut.double().numpy().sum(0)) <= 1e-3


def test_layer_empty_batch():
    """T = 0: nothing to project; the weight and bias gradients are zero."""
    p = synth.custom("L_empty", [0, 0], H=2, d=64, wid=86, n_max=4, norm=synth.NORM_LN)
    lp = synth.with_layer(p, d_model=32, wid=96)
    ns = device.upload_layer(lp)
    f = device.run_layer_fwd(ns)
    g = device.run_layer_bwd(ns, f)
    torch.cuda.synchronize()
    for t in (g.dW1, g.dW2, g.db1, g.db2):
        assert torch.count_nonzero(t).item() == 0


def _subsample_seqs(lens):
    order = np.argsort(np.abs(lens - np.median(lens)), kind="stable")
    picks = [int(np.argmin(lens)), int(np.argmax(lens))]
    for s in order:
        if int(s) not in picks:
            picks.append(int(s))
        if len(picks) == 4:
            break
    return sorted(picks)


def _sub_layer(lp, seqs):
    """The layer problem restricted to sequences seqs (same weights)."""
    core = synth.subbatch(lp.core, seqs)
    off = lp.core.offsets.astype(np.int64)
    rows = torch.from_numpy(np.concatenate([np.arange(off[s], off[s + 1]) for s in seqs]))
    return synth.LayerProblem(core=core, d_model=lp.d_model, X=lp.X.index_select(0, rows), W1=lp.W1, W2=lp.W2,
                              b1=lp.b1, b2=lp.b2, dOut=lp.dOut.index_select(0, rows)), rows.numpy()


def test_layer_train_full_size_on_subsample():
    """The training-shape layer (128 sequences, D = d_model = 512) at full size:
    Out and dX of four sequences against the oracle on those sequences (rows
    depend only on their own sequence), and the weight gradients of a GPU run
    on that four-sequence sub-batch against the oracle on it."""
    lp = synth.layer_train_bf16()
    seqs = _subsample_seqs(lp.core.lengths)
    _say("layer train: T", lp.T, "subsample", seqs, "lengths", lp.core.lengths[seqs].tolist())
    ns = device.upload_layer(lp)
    f = device.run_layer_fwd(ns)
    g = device.run_layer_bwd(ns, f)
    torch.cuda.synchronize()
    assert api.device_status(f.ws) == 0 and api.device_status(g.ws) == 0
    sub, rows = _sub_layer(lp, seqs)
    ref = oracle_layer_fwd(sub)
    rb = oracle_layer_bwd(sub)
    errs = {"Out": rel_l2(f.Out.float().cpu().numpy()[rows], ref["Out"]),
            "dX": rel_l2(g.dX.float().cpu().numpy()[rows], rb["dX"])}
    nsub = device.upload_layer(sub)
    fs = device.run_layer_fwd(nsub)
    gs = device.run_layer_bwd(nsub, fs)
    for name in ("dW1", "db1", "dW2", "db2"):
        errs[name] = rel_l2(getattr(gs, name).cpu().numpy(), rb[name])
    _say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= 1e-2, (k, v)


def test_layer_reuses_gemm_choice_across_token_counts():
    """Two batches whose token counts differ but round to the same size class
    (the GEMM algorithm cache is keyed by it): the second call runs the
    algorithm chosen for the first; both must match the oracle."""
    for i, lens in enumerate(([500, 300], [400, 450, 20])):
        p = synth.custom(f"L_bucket_{i}", lens, H=2, d=64, wid=87 + i, n_max=64, norm=synth.NORM_LN, n_pos=64,
                         rab_std=0.3)
        lp = synth.with_layer(p, d_model=128, wid=97 + i, x_std=1.0, w_std=0.1, bias_std=0.2)
        ns = device.upload_layer(lp)
        f = device.run_layer_fwd(ns)
        g = device.run_layer_bwd(ns, f)
        ref = oracle_layer_fwd(lp)
        rb = oracle_layer_bwd(lp)
        errs = {"Out": rel_l2(f.Out.float().cpu().numpy(), ref["Out"])}
        for name in ("dX", "dW1", "db1", "dW2", "db2"):
            errs[name] = rel_l2(getattr(g, name).float().cpu().numpy(), rb[name])
        _say(f"  T={lp.T} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        for k, v in errs.items():
            assert v <= 1e-2, (k, v)
