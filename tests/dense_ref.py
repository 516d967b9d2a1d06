"""Dense restatements of the method used to pin the oracle (test code only).

These build the *dense* picture -- an augmented key/value sequence [raw; level 1; ...; level L] and an
additive bias matrix that is -inf outside each query's entry set -- and hand it to torch's CPU fp64
``scaled_dot_product_attention`` and autograd.  They share no code with the oracle's C loops.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F


def pooled_levels_torch(x: torch.Tensor, block: int, levels: int):
    """Level l pooled tokens as a direct reshape-mean over B^l raw tokens (autograd-friendly)."""
    n, d = x.shape[-2], x.shape[-1]
    out = []
    for l in range(1, levels + 1):
        span = block ** l
        out.append(x.reshape(*x.shape[:-2], n // span, span, d).mean(dim=-2))
    return out


def level_offsets(n, block, levels):
    offs, o = [], 0
    for l in range(1, levels + 1):
        offs.append(o)
        o += n // block ** l
    return offs


def bias_matrix(idx_slice: np.ndarray, n: int, block: int, levels: int, enrich_levels: int,
                weights=None) -> np.ndarray:
    """[n, n + R] additive bias for one (b, h) slice.  weights[l-1] is the multiplicative weight of a
    level-l token (default B^l), entered as log(weight)."""
    offs = level_offsets(n, block, levels)
    R = sum(n // block ** l for l in range(1, levels + 1))
    if weights is None:
        weights = [float(block ** l) for l in range(1, levels + 1)]
    bias = np.full((n, n + R), -np.inf)
    for qi in range(n):
        i = qi // block
        for c in idx_slice[offs[0] + i]:
            if c >= 0:
                bias[qi, c * block:(c + 1) * block] = 0.0
        for l in range(1, min(enrich_levels, levels) + 1):
            a = i // block ** (l - 1)
            for j in idx_slice[offs[l - 1] + a]:
                if j >= 0:
                    bias[qi, n + offs[l - 1] + j] = math.log(weights[l - 1])
    return bias


def dense_forward(q, k, v, idx, block, levels, enrich_levels, scale, weights=None):
    """q, k, v: float64 torch [bh, n, d] (may require grad).  Returns (o, lse) via SDPA on the
    augmented sequence."""
    bh, n, d = q.shape
    outs, lses = [], []
    for s in range(bh):
        pk = pooled_levels_torch(k[s], block, levels)
        pv = pooled_levels_torch(v[s], block, levels)
        kk = torch.cat([k[s]] + pk, 0)
        vv = torch.cat([v[s]] + pv, 0)
        bias = torch.from_numpy(bias_matrix(idx[s], n, block, levels, enrich_levels, weights))
        o = F.scaled_dot_product_attention(q[s][None], kk[None], vv[None], attn_mask=bias[None],
                                           scale=scale)[0]
        logits = scale * q[s] @ kk.T + bias
        lses.append(torch.logsumexp(logits, dim=-1))
        outs.append(o)
    return torch.stack(outs), torch.stack(lses)


def exhaustive_topk(scores: np.ndarray, cand: np.ndarray, k: int) -> np.ndarray:
    """Top-k by full sort: score descending, candidate index ascending; returned ascending."""
    order = np.lexsort((cand, -scores))
    return np.sort(cand[order[:k]])
