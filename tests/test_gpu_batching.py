"""GPU parity of the batch-preparation entry points (Stochastic Length,
row gather, work-balanced bins) against the CPU oracle, bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from hstu_jagged_pointwise_attn_amd import _lib, api, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _keys(T, seed):
    return np.random.default_rng(seed).integers(0, 2 ** 32, size=T, dtype=np.uint64).astype(np.uint32)


@pytest.mark.parametrize("case", ["train_sl776", "long_sl2048", "ties", "short_only", "empty_seqs"])
def test_stochastic_length_bit_exact(case):
    if case == "train_sl776":
        lengths = synth._train_lengths(2, False)
        cap = synth.stochastic_length_cap(4096, 1.6)
        keys = _keys(int(lengths.sum()), 1)
    elif case == "long_sl2048":
        z = np.random.default_rng(5).standard_normal(32)
        lengths = np.clip(np.round(2048.0 * np.exp2(z)), 256, 8192).astype(np.int64)
        cap, keys = 2048, _keys(int(lengths.sum()), 2)
    elif case == "ties":
        lengths = np.array([300, 1000, 77, 2500])
        cap = 100
        keys = (np.random.default_rng(3).integers(0, 4, size=int(lengths.sum()))).astype(np.uint32)
    elif case == "short_only":
        lengths = np.array([5, 9, 1])
        cap, keys = 50, _keys(15, 4)
    else:
        lengths = np.array([0, 400, 0, 0, 3, 0])
        cap, keys = 64, _keys(403, 6)
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    print("SL", case, "B", len(lengths), "T", off[-1], "cap", cap, flush=True)
    d_off = torch.from_numpy(off).cuda()
    d_keys = torch.from_numpy(keys.view(np.int32)).cuda()
    new_off, idx, status = api.stochastic_length(d_off, d_keys, cap, int(lengths.max()))
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref_off, ref_idx = oracle.stochastic_length(off, keys, cap)
    np.testing.assert_array_equal(new_off.cpu().numpy(), ref_off)
    n = int(ref_off[-1])
    np.testing.assert_array_equal(idx[:n].cpu().numpy(), ref_idx)


def test_gather_rows_after_stochastic_length():
    p = synth.custom("g", [900, 30, 1200], H=2, d=64, wid=41, std=0.5)
    T = p.T
    keys = _keys(T, 7)
    d_off = torch.from_numpy(p.offsets).cuda()
    new_off, idx, status = api.stochastic_length(d_off, torch.from_numpy(keys.view(np.int32)).cuda(), 256,
                                                 p.max_len)
    n = int(new_off[-1].item())
    Q = p.Q.cuda()
    got = api.gather_rows(Q, idx, n)
    ts = torch.from_numpy(np.arange(T, dtype=np.int64) * 10).cuda()
    got_ts = api.gather_rows(ts, idx, n)
    torch.cuda.synchronize()
    _, ref_idx = oracle.stochastic_length(p.offsets, keys, 256)
    assert torch.equal(got.cpu(), p.Q[torch.from_numpy(ref_idx)])
    np.testing.assert_array_equal(got_ts.cpu().numpy(), ref_idx * 10)


def test_stochastic_length_flags_bad_offsets():
    off = torch.tensor([0, 10, 5, 20], dtype=torch.int32, device="cuda")  # decreasing
    keys = torch.zeros(20, dtype=torch.int32, device="cuda")
    new_off, idx, status = api.stochastic_length(off, keys, 4, 64)
    torch.cuda.synchronize()
    assert int(status.item()) & _lib.HSTU_DEV_BAD_OFFSETS
    assert int(new_off[-1].item()) == 0


@pytest.mark.parametrize("n_bins,cost", [(8, _lib.HSTU_COST_TOKENS), (8, _lib.HSTU_COST_ATTENTION),
                                         (3, _lib.HSTU_COST_TOKENS), (64, _lib.HSTU_COST_ATTENTION),
                                         (1, _lib.HSTU_COST_TOKENS), (9, _lib.HSTU_COST_ATTENTION),
                                         (16, _lib.HSTU_COST_TOKENS), (17, _lib.HSTU_COST_ATTENTION),
                                         (32, _lib.HSTU_COST_TOKENS), (33, _lib.HSTU_COST_TOKENS)])
def test_balance_bins_bit_exact(n_bins, cost):
    lengths = np.concatenate([synth._train_lengths(2, False), synth._train_lengths(2, True)])  # 256 seqs
    lengths[::17] = 0
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    b, c = api.balance_bins(torch.from_numpy(off).cuda(), n_bins, cost)
    torch.cuda.synchronize()
    rb, rc = oracle.balance_bins(lengths, n_bins, cost)
    np.testing.assert_array_equal(b.cpu().numpy(), rb)
    np.testing.assert_array_equal(c.cpu().numpy(), rc)
