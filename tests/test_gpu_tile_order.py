"""The by-sequence work-list order (hstu_set_tile_order): the scheduler's list
bit for bit against the oracle's order, and forward and backward results
identical to those of the default longest-first order."""
import numpy as np
import pytest
import torch

import oracle
from hstu_jagged_pointwise_attn_amd import api, device, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    yield
    api.set_tile_order(api.HSTU_TILE_ORDER_LONGEST)


def _say(*a):
    print(*a, flush=True)


def _small():
    L = np.array([150, 40, 133, 7, 0, 300])
    P = np.array([100, 0, 60, 3, 0, 50]); C = np.array([30, 40, 33, 2, 0, 64])
    return [
        synth.custom("ord_causal", [300, 1, 129, 64, 0, 257, 1500], H=2, d=64, wid=91, std=0.3, n_max=64,
                     n_pos=300, n_tb=20, rab_std=0.3, with_dy=True),
        synth.custom("ord_mtgr", L, H=2, d=64, wid=92, std=0.3, n_max=300, prefix_len=P, cand_len=C,
                     n_pos=64, n_tb=12, rab_std=0.3, with_dy=True),
    ]


def _tiles(entries, order):
    out = []
    for g in order:
        k = entries[g]["kinds"]
        out.append((entries[g]["b"], entries[g]["row0"], int(np.count_nonzero(k)), int(np.count_nonzero(k == 2)),
                    entries[g]["nrows"]))
    return out


def _got(tiles):
    return [(int(t[0]), int(t[1]), int(t[2]), int(t[3]) & 0xFFFF, int(t[3]) >> 16) for t in tiles]


@pytest.mark.parametrize("name", ["ord_causal", "ord_mtgr", "train", "mtgr", "long"])
def test_schedule_by_sequence_bit_exact(name):
    p = synth.WORKLOADS[name]() if name in synth.WORKLOADS else {q.name: q for q in _small()}[name]
    _say(f"[order] schedule {name} B={p.B}")
    ns = device.upload(p)
    BM, BN = api.tile_shape(ns.problem)
    prev = api.set_tile_order(api.HSTU_TILE_ORDER_BY_SEQUENCE)
    try:
        qoff, tiles = api.schedule_export(ns.problem)
    finally:
        api.set_tile_order(prev)
    entries = oracle.schedule(p.offsets, BM, BN, prefix_len=p.prefix_len, cand_len=p.cand_len)
    counts = np.bincount([e["b"] for e in entries], minlength=p.B)
    np.testing.assert_array_equal(qoff, np.concatenate([[0], np.cumsum(counts)]))
    assert _got(tiles) == _tiles(entries, oracle.sequence_order(entries))


def _run(ns):
    f = device.run_fwd(ns)
    g = api.attn_bwd(ns.problem, ns.Q, ns.K, ns.V, ns.U, f.O, f.mean, f.rstd, ns.dY)
    torch.cuda.synchronize()
    return f, g


def _rel(a, b):
    a, b = a.double(), b.double()
    n = torch.linalg.norm(b)
    return float(torch.linalg.norm(a - b) / n) if n > 0 else float(torch.linalg.norm(a - b))


@pytest.mark.parametrize("idx", [0, 1])
def test_results_do_not_depend_on_the_order(idx):
    """Large enough (inline schedule off) that both passes run the scheduler's lists."""
    p = _small()[idx]
    _say(f"[order] results {p.name}")
    ns = device.upload(p)
    inl = api.set_inline_schedule(False)
    try:
        api.set_tile_order(api.HSTU_TILE_ORDER_LONGEST)
        f1, g1 = _run(ns)
        api.set_tile_order(api.HSTU_TILE_ORDER_BY_SEQUENCE)
        f2, g2 = _run(ns)
    finally:
        api.set_tile_order(api.HSTU_TILE_ORDER_LONGEST)
        api.set_inline_schedule(inl)
    for name in ("O", "Y", "mean", "rstd"):
        assert torch.equal(getattr(f1, name), getattr(f2, name)), name
    for name in ("dQ", "dK", "dV", "dU"):
        assert torch.equal(getattr(g1, name), getattr(g2, name)), name
    for name in ("d_rab_p", "d_rab_t"):
        r = _rel(getattr(g1, name), getattr(g2, name))
        _say(f"  {name}: {r:.2e}")
        assert r <= 1e-4, (name, r)
