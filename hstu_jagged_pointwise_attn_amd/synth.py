"""Seeded synthetic inputs for HSTU jagged pointwise attention.

This module holds the input recipes only (length distributions, value
distributions, timestamps, segment sizes) and none of the method's
arithmetic. Both the HIP path and the CPU oracle are fed from it.

The pages measure on proprietary logs (Meituan delivery logs, Meta production
traffic); these generators stand in for them with the shapes the pages give:
skewed, long-tailed sequence lengths (HSTU page, section 3.4 "Stochastic
Length"; MTGR page section 3, contribution 3), lengths up to 3k/4096, model
widths 512/768/1024, and MTGR's per-user [static | history | real-time |
candidates] layout (fmread.com MTGR report, section 三.1).

Every array is drawn from numpy's PCG64 with seed = 1000 * workload_id +
tensor_id, so a workload is reproducible bit for bit. Floating tensors are
drawn in fp32 and rounded to bf16 (round-to-nearest-even, torch's cast) for
bf16 workloads.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

NORM_NONE, NORM_LN, NORM_GLN = 0, 1, 2

# Tensor ids for seeding.
_LEN, _TS, _Q, _K, _V, _U, _RP, _RT, _GAMMA, _DY, _KC, _VC, _QC, _UC, _CTS, _SEG = range(16)
_X, _W1, _B1, _W2, _B2, _DOUT = range(16, 22)


@dataclass
class Problem:
    """One batch of jagged sequences plus every operand of the attention core."""
    name: str
    dtype: torch.dtype
    H: int
    d: int
    offsets: np.ndarray                  # int32 [B+1]
    Q: torch.Tensor                      # [T, H, d]
    K: torch.Tensor
    V: torch.Tensor
    U: torch.Tensor
    n_max: int
    norm: int = NORM_LN
    eps: float = 1e-5
    prefix_len: Optional[np.ndarray] = None   # int32 [B]
    cand_len: Optional[np.ndarray] = None     # int32 [B]
    ts: Optional[np.ndarray] = None           # int64 [T]
    rab_p: Optional[np.ndarray] = None        # float32 [n_pos]
    rab_t: Optional[np.ndarray] = None        # float32 [n_tb]
    group: Optional[np.ndarray] = None        # uint8 [T]
    n_groups: int = 1
    gamma: Optional[np.ndarray] = None        # float32 [n_groups, D]
    beta: Optional[np.ndarray] = None
    dY: Optional[torch.Tensor] = None         # [T, H*d]
    time_filter: bool = False                 # candidates see causal keys only if strictly earlier
    extra: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return len(self.offsets) - 1

    @property
    def T(self) -> int:
        return int(self.offsets[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.offsets)

    @property
    def max_len(self) -> int:
        return int(self.lengths.max()) if self.B else 0


@dataclass
class MFalconProblem:
    """Candidates of B users scored against each user's cached history K/V."""
    name: str
    dtype: torch.dtype
    H: int
    d: int
    hist_offsets: np.ndarray             # int32 [B+1]
    cand_offsets: np.ndarray             # int32 [B+1]
    K_cache: torch.Tensor                # [Th, H, d]
    V_cache: torch.Tensor
    Qc: torch.Tensor                     # [Tc, H, d]
    Kc: torch.Tensor
    Vc: torch.Tensor
    Uc: torch.Tensor
    n_max: int
    microbatch: int
    norm: int = NORM_LN
    eps: float = 1e-5
    hist_ts: Optional[np.ndarray] = None
    cand_ts: Optional[np.ndarray] = None
    rab_p: Optional[np.ndarray] = None
    rab_t: Optional[np.ndarray] = None
    cand_group: Optional[np.ndarray] = None
    n_groups: int = 1
    gamma: Optional[np.ndarray] = None
    beta: Optional[np.ndarray] = None
    Q_hist: Optional[torch.Tensor] = None   # history queries, used only for a full-pass check
    U_hist: Optional[torch.Tensor] = None
    time_filter: bool = False               # candidates see history keys only if strictly earlier

    @property
    def B(self) -> int:
        return len(self.cand_offsets) - 1


def _rng(wid: int, tid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * wid + tid))


def _normal(wid, tid, shape, std, dtype):
    a = _rng(wid, tid).standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return torch.from_numpy(a).to(dtype)


def truncated_pareto(rng, shape_a, lo, hi, n):
    """Inverse-CDF draws of a Pareto(shape_a) truncated to [lo, hi], floored."""
    u = rng.random(n)
    r = (lo / hi) ** shape_a
    x = lo / (1.0 - u * (1.0 - r)) ** (1.0 / shape_a)
    return np.clip(np.floor(x), lo, hi).astype(np.int64)


def truncated_pareto_mean(shape_a, lo, hi):
    a = shape_a
    norm = 1.0 - (lo / hi) ** a
    return a * lo ** a * (lo ** (1 - a) - hi ** (1 - a)) / ((a - 1) * norm)


def pareto_lo_for_mean(shape_a, hi, mean):
    """The lower bound lo of a Pareto(shape_a) truncated to [lo, hi] whose mean is `mean`."""
    a, b = 1.0, float(hi)
    for _ in range(200):
        m = 0.5 * (a + b)
        if truncated_pareto_mean(shape_a, m, hi) < mean:
            a = m
        else:
            b = m
    return 0.5 * (a + b)


def stochastic_length_cap(max_len: int, alpha: float) -> int:
    """Stochastic Length keeps at most max_len^(alpha/2) tokens of a sequence
    (HSTU page, section 3.4: alpha = 1.6 takes 4096 to about 776)."""
    return int(math.floor(max_len ** (alpha / 2.0)))


def _timestamps(wid, lengths, mean_gap=3600.0):
    """int64 seconds: per-sequence base 1.7e9 + U{0..1e6}, gaps floor(Exp(mean_gap))
    (zero gaps allowed), so timestamps are non-decreasing within a sequence."""
    rng = _rng(wid, _TS)
    out = []
    for L in lengths:
        base = 1_700_000_000 + int(rng.integers(0, 1_000_001))
        gaps = np.floor(rng.exponential(mean_gap, size=int(L))).astype(np.int64)
        if L:
            gaps[0] = 0
        out.append(base + np.cumsum(gaps))
    return np.concatenate(out).astype(np.int64) if out else np.zeros(0, np.int64)


def _offsets(lengths):
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    off[1:] = np.cumsum(lengths)
    assert off[-1] < 2 ** 31
    return off.astype(np.int32)


def custom(name, lengths, *, H, d, dtype=torch.bfloat16, wid=99, std=0.02, n_max=None,
           norm=NORM_LN, eps=1e-5, prefix_len=None, cand_len=None, n_pos=0, n_tb=0,
           rab_std=0.02, group=None, n_groups=1, gamma_std=None, beta_std=None, with_dy=False,
           qk_std=None) -> Problem:
    """A problem with the given lengths and options (used by tests and by the
    named workloads below)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    off = _offsets(lengths)
    T = int(off[-1])
    D = H * d
    qs = std if qk_std is None else qk_std
    Q = _normal(wid, _Q, (T, H, d), qs, dtype)
    K = _normal(wid, _K, (T, H, d), qs, dtype)
    V = _normal(wid, _V, (T, H, d), std, dtype)
    U = _normal(wid, _U, (T, H, d), std, dtype)
    ts = _timestamps(wid, lengths) if n_tb else None
    rab_p = (_rng(wid, _RP).standard_normal(n_pos, dtype=np.float32) * np.float32(rab_std)
             if n_pos else None)
    rab_t = (_rng(wid, _RT).standard_normal(n_tb, dtype=np.float32) * np.float32(rab_std)
             if n_tb else None)
    G = n_groups if norm == NORM_GLN else 1
    gamma = beta = None
    if gamma_std is not None:
        gamma = (1.0 + _rng(wid, _GAMMA).standard_normal((G, D), dtype=np.float32)
                 * np.float32(gamma_std)).astype(np.float32)
    if beta_std is not None:
        beta = (_rng(wid, _GAMMA + 100).standard_normal((G, D), dtype=np.float32)
                * np.float32(beta_std)).astype(np.float32)
    dY = _normal(wid, _DY, (T, D), 1.0, dtype) if with_dy else None
    return Problem(
        name=name, dtype=dtype, H=H, d=d, offsets=off, Q=Q, K=K, V=V, U=U,
        n_max=int(n_max if n_max is not None else max(int(lengths.max()) if len(lengths) else 1, 1)),
        norm=norm, eps=eps,
        prefix_len=None if prefix_len is None else np.asarray(prefix_len, np.int32),
        cand_len=None if cand_len is None else np.asarray(cand_len, np.int32),
        ts=ts, rab_p=rab_p, rab_t=rab_t,
        group=None if group is None else np.asarray(group, np.uint8), n_groups=n_groups,
        gamma=gamma, beta=beta, dY=dY)


def interleave_candidate_times(p: Problem, seed: int) -> Problem:
    """Give each candidate a timestamp drawn among the times of its sequence's
    causal segment (half of them exactly equal to one, the rest one second
    after one), so that under the timestamp filter candidates see different
    prefixes of the real-time tokens. Sequences without a causal segment keep
    their times. Creates timestamps if the problem has none."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ts = p.ts.copy() if p.ts is not None else _timestamps(seed % 1000, p.lengths)
    for b in range(p.B):
        s, e = int(p.offsets[b]), int(p.offsets[b + 1])
        P = int(p.prefix_len[b]) if p.prefix_len is not None else 0
        C = int(p.cand_len[b]) if p.cand_len is not None else 0
        E = e - s - C
        if C == 0 or E <= P:
            continue
        src = ts[s + P:s + E]
        pick = src[rng.integers(0, len(src), size=C)] + rng.integers(0, 2, size=C)
        ts[s + E:e] = pick
    p.ts = ts
    return p


# ---------------------------------------------------------------- workloads

def tiny_fp32() -> Problem:
    """4 jagged sequences of U{8..64} tokens, 2 heads, d = 32, fp32, causal,
    rab_p (64 positions) and rab_t (16 log2-second buckets), LN, N_max = 64."""
    wid = 1
    lengths = _rng(wid, _LEN).integers(8, 65, size=4)
    return custom("tiny_fp32", lengths, H=2, d=32, dtype=torch.float32, wid=wid, std=0.1,
                  n_max=64, norm=NORM_LN, n_pos=64, n_tb=16, rab_std=0.02)


def _train_lengths(wid, literal: bool, B=128):
    rng = _rng(wid, _LEN)
    if literal:
        raw = truncated_pareto(rng, 1.2, 16, 4096, B)
        return np.minimum(raw, stochastic_length_cap(4096, 1.6))
    lo = pareto_lo_for_mean(1.2, 4096, 776.0)
    return truncated_pareto(rng, 1.2, lo, 4096, B)


def train_bf16(literal: bool = False) -> Problem:
    """HSTU training shape: 128 jagged sequences, 4 heads, d = 128, bf16,
    causal, rab_p (4096 positions), rab_t (128 log buckets), LN, N_max = 4096.
    Default lengths: truncated Pareto(1.2) on [lo, 4096] with lo solved for a
    mean of 776 tokens. literal=True: Pareto(1.2) on [16, 4096] capped at the
    Stochastic Length budget 4096^0.8 = 776 (mean about 60)."""
    wid = 2
    lengths = _train_lengths(wid, literal)
    p = custom("train_literal" if literal else "train", lengths, H=4, d=128, wid=wid, std=0.02,
               n_max=4096, norm=NORM_LN, n_pos=4096, n_tb=128, rab_std=0.02)
    return p


def mtgr_bf16(B=64) -> Problem:
    """MTGR hybrid mask: per user 16 static tokens + history (truncated
    Pareto(1.2) on [64, 3000]) + U{0..64} real-time tokens + U{32..200}
    candidates. Static and history form the bidirectional prefix, real-time
    tokens are causal, candidates see the prefix, the real-time tokens and
    themselves. 6 heads, d = 128, Group LayerNorm over 4 token groups
    (static, history, real-time, candidate), no rab, N_max = 3280."""
    wid = 3
    rng = _rng(wid, _SEG)
    hist = truncated_pareto(rng, 1.2, 64, 3000, B)
    rt = rng.integers(0, 65, size=B)
    cand = rng.integers(32, 201, size=B)
    static = np.full(B, 16)
    lengths = static + hist + rt + cand
    group = np.concatenate([
        np.concatenate([np.zeros(16), np.ones(h), np.full(r, 2), np.full(c, 3)])
        for h, r, c in zip(hist, rt, cand)]).astype(np.uint8)
    p = custom("mtgr", lengths, H=6, d=128, wid=wid, std=0.02, n_max=3280, norm=NORM_GLN,
               prefix_len=static + hist, cand_len=cand, group=group, n_groups=4, gamma_std=0.1)
    p.beta = np.zeros_like(p.gamma)
    return p


def mfalcon_bf16(users=16, n_hist=2048, m_cand=1024, microbatch=256, H=8, d=128,
                 with_rab=False) -> MFalconProblem:
    """M-FALCON ranking: 16 users, each with n = 2048 history tokens whose K/V
    are cached and m = 1024 candidates scored in microbatches of 256; 8 heads,
    d = 128, LN, no rab, N_max = n + m. Candidate timestamps are the last
    history timestamp plus floor(Exp(3600))."""
    wid = 4
    dtype = torch.bfloat16
    hist_len = np.full(users, n_hist)
    cand_len = np.full(users, m_cand)
    ho, co = _offsets(hist_len), _offsets(cand_len)
    Th, Tc = int(ho[-1]), int(co[-1])
    std = 0.02
    hts = _timestamps(wid, hist_len)
    rng = _rng(wid, _CTS)
    last = hts[ho[1:] - 1] if n_hist > 0 else np.full(users, 1_700_000_000, np.int64)
    cts = np.concatenate([
        last[b] + np.floor(rng.exponential(3600.0, size=m_cand)).astype(np.int64)
        for b in range(users)]) if Tc else np.zeros(0, np.int64)
    n_pos = n_tb = 0
    rab_p = rab_t = None
    if with_rab:
        n_pos, n_tb = 4096, 128
        rab_p = _rng(wid, _RP).standard_normal(n_pos, dtype=np.float32) * np.float32(0.02)
        rab_t = _rng(wid, _RT).standard_normal(n_tb, dtype=np.float32) * np.float32(0.02)
    return MFalconProblem(
        name="mfalcon", dtype=dtype, H=H, d=d, hist_offsets=ho, cand_offsets=co,
        K_cache=_normal(wid, _KC, (Th, H, d), std, dtype),
        V_cache=_normal(wid, _VC, (Th, H, d), std, dtype),
        Qc=_normal(wid, _QC, (Tc, H, d), std, dtype),
        Kc=_normal(wid, _K, (Tc, H, d), std, dtype),
        Vc=_normal(wid, _V, (Tc, H, d), std, dtype),
        Uc=_normal(wid, _UC, (Tc, H, d), std, dtype),
        n_max=n_hist + m_cand, microbatch=microbatch, norm=NORM_LN,
        hist_ts=hts if with_rab else None, cand_ts=cts if with_rab else None,
        rab_p=rab_p, rab_t=rab_t,
        Q_hist=_normal(wid, _Q, (Th, H, d), std, dtype),
        U_hist=_normal(wid, _U, (Th, H, d), std, dtype))


def long_bf16(B=32) -> Problem:
    """Long sequences, forward and backward: 32 sequences with lengths
    round(2048 * 2^Z) clipped to [256, 8192] (lognormal, median 2048,
    sigma = ln 2); 8 heads, d = 128, causal, rab_p (8192 positions), rab_t
    (128 buckets), LN, N_max = 8192, dY ~ N(0, 1)."""
    wid = 5
    z = _rng(wid, _LEN).standard_normal(B)
    lengths = np.clip(np.round(2048.0 * np.exp2(z)), 256, 8192).astype(np.int64)
    return custom("long", lengths, H=8, d=128, wid=wid, std=0.02, n_max=8192, norm=NORM_LN,
                  n_pos=8192, n_tb=128, rab_std=0.02, with_dy=True)


WORKLOADS = {
    "tiny_fp32": tiny_fp32,
    "train": lambda: train_bf16(False),
    "train_literal": lambda: train_bf16(True),
    "mtgr": mtgr_bf16,
    "mfalcon": mfalcon_bf16,
    "long": long_bf16,
}


def subbatch(p: Problem, seqs) -> Problem:
    """The sub-batch made of sequences `seqs` (in that order) of problem p."""
    seqs = [int(s) for s in seqs]
    off = p.offsets.astype(np.int64)
    rows = np.concatenate([np.arange(off[s], off[s + 1]) for s in seqs]) if seqs else np.zeros(0, np.int64)
    idx = torch.from_numpy(rows)
    lengths = np.array([off[s + 1] - off[s] for s in seqs], dtype=np.int64)

    def sel(t):
        return None if t is None else t.index_select(0, idx)

    def sel_np(a):
        return None if a is None else a[rows]

    def seq_np(a):
        return None if a is None else np.asarray(a)[seqs]

    return Problem(
        name=p.name + "_sub", dtype=p.dtype, H=p.H, d=p.d, offsets=_offsets(lengths),
        Q=sel(p.Q), K=sel(p.K), V=sel(p.V), U=sel(p.U), n_max=p.n_max, norm=p.norm, eps=p.eps,
        prefix_len=seq_np(p.prefix_len), cand_len=seq_np(p.cand_len), ts=sel_np(p.ts),
        rab_p=p.rab_p, rab_t=p.rab_t, group=sel_np(p.group), n_groups=p.n_groups,
        gamma=p.gamma, beta=p.beta, dY=sel(p.dY))


@dataclass
class LayerProblem:
    """A full HSTU layer: the attention problem `core` (its masks, rab, norm
    and sizes; its Q/K/V/U are not used, the layer makes its own from X)
    plus the layer input X [T, d_model], the projections W1 [d_model, 4D],
    b1 [4D], W2 [D, d_model], b2 [d_model] and the output gradient dOut."""
    core: Problem
    d_model: int
    X: torch.Tensor
    W1: torch.Tensor
    W2: torch.Tensor
    b1: Optional[np.ndarray]
    b2: Optional[np.ndarray]
    dOut: Optional[torch.Tensor]

    @property
    def name(self) -> str:
        return self.core.name

    @property
    def T(self) -> int:
        return self.core.T


def with_layer(p: Problem, d_model: Optional[int] = None, wid: int = 60, x_std=1.0, w_std=0.02,
               bias_std: Optional[float] = 0.02, with_dout=True) -> LayerProblem:
    """Layer inputs around problem p: X ~ N(0, x_std) and the weights
    ~ N(0, w_std) in p's dtype (0.02 is the pages' initialisation scale for
    the workloads' tensors), fp32 biases ~ N(0, bias_std) (None: no biases),
    dOut ~ N(0, 1). d_model defaults to D = H * d."""
    D = p.H * p.d
    dm = D if d_model is None else int(d_model)
    T = p.T
    b1 = b2 = None
    if bias_std is not None:
        b1 = _rng(wid, _B1).standard_normal(4 * D, dtype=np.float32) * np.float32(bias_std)
        b2 = _rng(wid, _B2).standard_normal(dm, dtype=np.float32) * np.float32(bias_std)
    return LayerProblem(
        core=p, d_model=dm, X=_normal(wid, _X, (T, dm), x_std, p.dtype),
        W1=_normal(wid, _W1, (dm, 4 * D), w_std, p.dtype), W2=_normal(wid, _W2, (D, dm), w_std, p.dtype),
        b1=b1, b2=b2, dOut=_normal(wid, _DOUT, (T, dm), 1.0, p.dtype) if with_dout else None)


def layer_train_bf16() -> LayerProblem:
    """The training shape (train_bf16) as one full layer: d_model = D = 512,
    projection biases on."""
    return with_layer(train_bf16(False), wid=62)


def layer_long_bf16() -> LayerProblem:
    """The long-sequence shape (long_bf16) as one full layer: d_model = D = 1024."""
    return with_layer(long_bf16(), wid=65)


@dataclass
class StackProblem:
    """Candidates of B users scored through a stack of HSTU layers against the
    users' histories (M-FALCON over several layers). X_hist [Th, d_model] and
    X_cand [Tc, d_model] are the first layer's inputs; `layers` holds one dict
    per layer with W1 [d_model, 4D], W2 [D, d_model] (the problem's dtype),
    fp32 b1, b2, and optional fp32 rab_p, rab_t, gamma, beta."""
    name: str
    dtype: torch.dtype
    H: int
    d: int
    d_model: int
    hist_offsets: np.ndarray
    cand_offsets: np.ndarray
    X_hist: torch.Tensor
    X_cand: torch.Tensor
    layers: list
    n_max: int
    microbatch: int
    norm: int = NORM_LN
    eps: float = 1e-5
    hist_ts: Optional[np.ndarray] = None
    cand_ts: Optional[np.ndarray] = None
    hist_group: Optional[np.ndarray] = None
    cand_group: Optional[np.ndarray] = None
    n_groups: int = 1
    time_filter: bool = False

    @property
    def B(self) -> int:
        return len(self.cand_offsets) - 1


def stack_custom(name, hist_len, cand_len, *, n_layers, H, d, d_model=None, dtype=torch.bfloat16, wid=120,
                 microbatch=0, n_max=None, norm=NORM_LN, x_std=1.0, w_std=0.02, bias_std=0.02, n_pos=0, n_tb=0,
                 rab_std=0.02, gamma_std=None, beta_std=None, n_groups=1, with_ts=None, x_cand_seed=0) -> StackProblem:
    """A stack problem with the given history and candidate counts per user.
    Timestamps: per-user history times as for the attention workloads and
    candidate times = last history time + floor(Exp(3600)) (made when rab_t
    is on or with_ts is set). GLN groups: history tokens group 0, candidates
    group 1 (n_groups = 2). x_cand_seed varies the candidates' inputs only
    (a new request against the same histories)."""
    hist_len = np.asarray(hist_len, dtype=np.int64)
    cand_len = np.asarray(cand_len, dtype=np.int64)
    B = len(hist_len)
    D = H * d
    dm = D if d_model is None else int(d_model)
    ho, co = _offsets(hist_len), _offsets(cand_len)
    Th, Tc = int(ho[-1]), int(co[-1])
    hts = cts = None
    if n_tb or with_ts:
        hts = _timestamps(wid, hist_len)
        rng = _rng(wid, _CTS)
        base = np.array([hts[ho[b + 1] - 1] if hist_len[b] else 1_700_000_000 for b in range(B)], np.int64)
        cts = (np.concatenate([base[b] + np.floor(rng.exponential(3600.0, size=int(cand_len[b]))).astype(np.int64)
                               for b in range(B)]) if Tc else np.zeros(0, np.int64))
    G = 2 if norm == NORM_GLN else 1
    layers = []
    for l in range(n_layers):
        lw = 1000 * wid + 50 * l  # per-layer seeds
        lay = {"W1": _normal(lw, _W1, (dm, 4 * D), w_std, dtype), "W2": _normal(lw, _W2, (D, dm), w_std, dtype)}
        if bias_std is not None:
            lay["b1"] = _rng(lw, _B1).standard_normal(4 * D, dtype=np.float32) * np.float32(bias_std)
            lay["b2"] = _rng(lw, _B2).standard_normal(dm, dtype=np.float32) * np.float32(bias_std)
        if n_pos:
            lay["rab_p"] = _rng(lw, _RP).standard_normal(n_pos, dtype=np.float32) * np.float32(rab_std)
        if n_tb:
            lay["rab_t"] = _rng(lw, _RT).standard_normal(n_tb, dtype=np.float32) * np.float32(rab_std)
        if gamma_std is not None:
            lay["gamma"] = (1.0 + _rng(lw, _GAMMA).standard_normal((G, D), dtype=np.float32)
                            * np.float32(gamma_std)).astype(np.float32)
        if beta_std is not None:
            lay["beta"] = (_rng(lw, _GAMMA + 100).standard_normal((G, D), dtype=np.float32)
                           * np.float32(beta_std)).astype(np.float32)
        layers.append(lay)
    return StackProblem(
        name=name, dtype=dtype, H=H, d=d, d_model=dm, hist_offsets=ho, cand_offsets=co,
        X_hist=_normal(wid, _X, (Th, dm), x_std, dtype),
        X_cand=_normal(wid + 7919 * x_cand_seed, _DOUT, (Tc, dm), x_std, dtype),
        layers=layers, n_max=int(n_max if n_max is not None else max(int((hist_len + cand_len).max()) if B else 1, 1)),
        microbatch=microbatch, norm=norm, hist_ts=hts, cand_ts=cts,
        hist_group=np.zeros(Th, np.uint8) if norm == NORM_GLN else None,
        cand_group=np.ones(Tc, np.uint8) if norm == NORM_GLN else None, n_groups=G)


def mfalcon_stack_bf16(n_layers=3) -> StackProblem:
    """The M-FALCON ranking shape (16 users x 2048 history tokens x 1024
    candidates, microbatch 256, 8 heads, d = 128, LN, no rab, N_max 3072)
    through a stack of 3 layers (MTGR-Small's depth) with d_model = D = 1024."""
    return stack_custom("mfalcon_stack", np.full(16, 2048), np.full(16, 1024), n_layers=n_layers, H=8, d=128,
                        wid=130, microbatch=256, n_max=3072)
