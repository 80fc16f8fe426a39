"""A dense formulation of HSTU pointwise attention out of torch library
routines, used only to pin the oracle (never to check the HIP path).

It is built differently from the oracle's per-pair loops on purpose: masks
are assembled from blocks (ones / torch.tril / identity), the time bucket
comes from torch.frexp, SiLU from torch.nn.functional.silu, the contraction
from torch.matmul and the normalisation from torch.nn.functional.layer_norm.
Gradients come from torch.autograd, which derives them independently of the
oracle's hand-written backward.
"""
import torch
import torch.nn.functional as F


def block_mask(L, P, C):
    """[L, L] visibility: prefix block sees the prefix; causal block sees the
    prefix and its own lower triangle; candidates see everything before the
    candidate tail plus themselves (MTGR / M-FALCON masks)."""
    E = L - C
    m = torch.zeros(L, L, dtype=torch.bool)
    m[:, :P] = True                                   # prefix keys: visible to every row
    m[P:E, P:E] = torch.ones(E - P, E - P, dtype=torch.bool).tril()
    m[E:, P:E] = True                                 # candidates see the causal part
    m[E:, E:] = torch.eye(C, dtype=torch.bool)        # ... and only themselves in the tail
    return m


def positions(L, C):
    E = L - C
    return torch.cat([torch.arange(E), torch.full((C,), E)]).to(torch.int64)


def bucket(dt, n_tb):
    """floor(log2(max(1, |dt|))) clamped to n_tb - 1, via frexp."""
    a = dt.abs().clamp(min=1).to(torch.float64)
    _, e = torch.frexp(a)
    return (e.to(torch.int64) - 1).clamp(max=n_tb - 1)


def forward(offsets, Q, K, V, U, *, H, d, prefix_len=None, cand_len=None, ts=None, rab_p=None,
            rab_t=None, n_max=1.0, norm=1, eps=1e-5, group=None, gamma=None, beta=None,
            time_filter=False):
    """Q, K, V, U: float64 tensors [T, H, d] (may require grad); rab tables,
    gamma, beta: float64 tensors or None. Returns Y [T, H*d] and O [T, H*d].
    time_filter: the candidate block's view of the causal block is cut down to
    the keys with an earlier timestamp."""
    T = Q.shape[0]
    D = H * d
    outs = []
    for b in range(len(offsets) - 1):
        s, e = int(offsets[b]), int(offsets[b + 1])
        L = e - s
        P = int(prefix_len[b]) if prefix_len is not None else 0
        C = int(cand_len[b]) if cand_len is not None else 0
        if L == 0:
            continue
        mask = block_mask(L, P, C)
        if time_filter:
            E = L - C
            t = torch.as_tensor(ts[s:e], dtype=torch.int64)
            mask[E:, P:E] &= t[None, P:E] < t[E:, None]
        bias = torch.zeros(L, L, dtype=torch.float64)
        if rab_p is not None:
            pos = positions(L, C)
            idx = (pos[:, None] - pos[None, :]).abs().clamp(max=rab_p.shape[0] - 1)
            bias = bias + rab_p[idx]
        if rab_t is not None and ts is not None:
            t = torch.as_tensor(ts[s:e], dtype=torch.int64)
            bias = bias + rab_t[bucket(t[:, None] - t[None, :], rab_t.shape[0])]
        q = Q[s:e].transpose(0, 1)       # [H, L, d]
        k = K[s:e].transpose(0, 1)
        v = V[s:e].transpose(0, 1)
        S = torch.matmul(q, k.transpose(1, 2)) + bias
        A = torch.where(mask, F.silu(S), torch.zeros((), dtype=torch.float64)) / n_max
        outs.append(torch.matmul(A, v).transpose(0, 1).reshape(L, D))
    O = torch.cat(outs, 0) if outs else torch.zeros(0, D, dtype=torch.float64)
    Uf = U.reshape(T, D)
    if norm == 0:
        N = O
    else:
        N = F.layer_norm(O, (D,), eps=eps)
        if gamma is not None:
            g = torch.as_tensor(group, dtype=torch.int64) if group is not None else torch.zeros(T, dtype=torch.int64)
            N = N * gamma[g]
            if beta is not None:
                N = N + beta[g]
        elif beta is not None:
            g = torch.as_tensor(group, dtype=torch.int64) if group is not None else torch.zeros(T, dtype=torch.int64)
            N = N + beta[g]
    return N * Uf, O
