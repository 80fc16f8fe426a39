"""Host-side pieces of bench.py: the closed-form pair count behind the useful
FLOPs of the metric, and the rule that a stored traffic figure is used only
while its kernel's sources are unchanged."""
import json
import os
import shutil

import numpy as np
import pytest

import bench
import oracle


@pytest.fixture(scope="module", autouse=True)
def _oracle():
    oracle.build(force=False)


def _brute(L, P, C):
    return sum(oracle.visible(i, j, L, P, C) for i in range(L) for j in range(L))


@pytest.mark.parametrize("L,P,C", [(0, 0, 0), (1, 0, 0), (1, 0, 1), (1, 1, 0), (7, 0, 0), (7, 7, 0), (7, 0, 7),
                                   (9, 3, 2), (16, 16, 0), (12, 0, 5), (12, 4, 8)])
def test_visible_pairs_edge_cases(L, P, C):
    """The closed form equals the per-pair count of the oracle's mask (the
    pages' causal / hybrid static-causal-candidate mask, self pairs included)."""
    assert bench.visible_pairs([L], [P], [C]) == _brute(L, P, C)


def test_visible_pairs_random_batches():
    rng = np.random.default_rng(7)
    for _ in range(20):
        B = int(rng.integers(1, 6))
        L = rng.integers(0, 40, size=B)
        P = np.array([rng.integers(0, l + 1) for l in L])
        C = np.array([rng.integers(0, l - p + 1) for l, p in zip(L, P)])
        want = sum(_brute(int(l), int(p), int(c)) for l, p, c in zip(L, P, C))
        assert bench.visible_pairs(L, P, C) == want
        # plain causal when neither segment is given
        assert bench.visible_pairs(L) == sum(int(l) * (int(l) + 1) // 2 for l in L)


def test_traffic_figure_follows_the_kernel_sources(tmp_path, monkeypatch):
    """A stored per-launch byte count is returned while the hash of the kernel's
    sources matches the one recorded with it, and None once a source changes
    or the entry is missing."""
    csrc = tmp_path / "hstu_jagged_pointwise_attn_amd" / "csrc"
    csrc.mkdir(parents=True)
    src = os.path.join(bench.ROOT, "hstu_jagged_pointwise_attn_amd", "csrc")
    for name in set(sum(bench.KERNEL_SOURCES.values(), [])):
        shutil.copy(os.path.join(src, name), csrc / name)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    h = bench.kernel_source_hash("attn_bwd_dkdv")
    (tmp_path / "profiles" / "traffic.json").write_text(
        json.dumps({"long": {"attn_bwd_dkdv": {"source_hash": h, "bytes_per_launch": 1234}}}))
    assert bench.traffic_from_profiles("long", "attn_bwd_dkdv") == 1234
    assert bench.traffic_from_profiles("long", "attn_fwd") is None
    assert bench.traffic_from_profiles("train", "attn_bwd_dkdv") is None
    with open(csrc / "attn_bwd.hip", "a") as f:
        f.write("\n// changed\n")
    assert bench.kernel_source_hash("attn_bwd_dkdv") != h
    assert bench.traffic_from_profiles("long", "attn_bwd_dkdv") is None
