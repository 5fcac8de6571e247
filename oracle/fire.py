"""fp64 oracle for the FIRE positional bias (functional interpolation for
relative positions).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The FAT5 report lists FIRE beside RoPE and ALiBi among the encodings its
kernels serve (note under "Noyau CUDA", citing Li et al., "Functional
Interpolation for Relative Positions Improves Long Context Transformers") but
prints no formula.  The reading taken here is that paper's definition, for
causal attention (key j at or before query i):

    psi(t)   = log(c t + 1)                       (natural log, c > 0)
    x_ij     = psi(i - j) / psi(max(L, i))        (L > 0 the threshold)
    bias_hij = f_theta(x_ij)_h = b2_h + sum_k w2_hk relu(w1_k x_ij + b1_k)

f_theta is a one-hidden-layer ReLU MLP from the scalar x to one value per
head (K hidden units).  The parameters theta = (w1 [K], b1 [K], w2 [H, K],
b2 [H], c, L) are all trained: the gradient flows into c and L through x.
For rows i < L the normaliser is psi(L), so the derivative with respect to L
is taken on those rows only (i >= L: max(L, i) = i does not depend on L).

Parameters travel as one flat vector, in this order:
    theta = [w1 (K), b1 (K), w2 (H*K, row h = w2[h*K:(h+1)*K]), b2 (H), c, L]

The bias is evaluated straight from this definition (hidden activations
materialised, a block of query rows at a time); its gradient is the chain
rule through the same steps.  Nothing is reformulated.
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 128


def theta_size(heads: int, hidden: int) -> int:
    return 2 * hidden + heads * hidden + heads + 2


def unpack(theta, heads: int, hidden: int):
    """theta -> (w1 [K], b1 [K], w2 [H, K], b2 [H], c, L) as float64."""
    t = np.asarray(theta, dtype=np.float64)
    assert t.shape == (theta_size(heads, hidden),), t.shape
    K, H = hidden, heads
    w1 = t[:K]
    b1 = t[K:2 * K]
    w2 = t[2 * K:2 * K + H * K].reshape(H, K)
    b2 = t[2 * K + H * K:2 * K + H * K + H]
    c, L = float(t[-2]), float(t[-1])
    return w1, b1, w2, b2, c, L


def fire_x(rows: np.ndarray, cols: np.ndarray, c: float, L: float) -> np.ndarray:
    """x_ij = log(c (i - j) + 1) / log(c max(L, i) + 1) for query rows `rows`
    and keys `cols`; entries with j > i (masked under causality) are 0."""
    i = np.asarray(rows, dtype=np.float64)[:, None]
    j = np.asarray(cols, dtype=np.float64)[None, :]
    d = np.maximum(i - j, 0.0)
    return np.log1p(c * d) / np.log1p(c * np.maximum(L, i))


def fire_mlp(x: np.ndarray, w1, b1, w2, b2) -> np.ndarray:
    """f_theta(x) for an array of x: returns [..., H]."""
    z = x[..., None] * w1 + b1
    return np.maximum(z, 0.0) @ w2.T + b2


def fire_bias(seqlen: int, theta, heads: int, hidden: int, head=None) -> np.ndarray:
    """The FIRE bias [H, S, S] (or the head's [S, S] when `head` is given);
    entries with key after query are 0 (the causal mask removes them)."""
    w1, b1, w2, b2, c, L = unpack(theta, heads, hidden)
    hs = range(heads) if head is None else [head]
    out = np.zeros((len(hs), seqlen, seqlen))
    cols = np.arange(seqlen)
    for r0 in range(0, seqlen, ROW_BLOCK):
        rows = np.arange(r0, min(seqlen, r0 + ROW_BLOCK))
        x = fire_x(rows, cols, c, L)
        f = fire_mlp(x, w1, b1, w2[list(hs)], b2[list(hs)])      # [rb, S, nh]
        vis = cols[None, :] <= rows[:, None]
        out[:, rows[0]:rows[-1] + 1, :] = np.where(vis[None], np.moveaxis(f, -1, 0), 0.0)
    return out if head is None else out[0]


def fire_theta_grad(dS: np.ndarray, head: int, theta, heads: int, hidden: int) -> np.ndarray:
    """Gradient of sum_ij dS_ij bias_hij with respect to theta, for one head's
    [S, S] gradient dS (dL/dS', zero at masked pairs).  Chain rule through
    the MLP and through x(c, L):

        dx/dc = (d / (c d + 1) - x m / (c m + 1)) / log(c m + 1),  m = max(L, i)
        dx/dL = -x c / ((c L + 1) log(c L + 1))   on rows i < L, else 0
    """
    w1, b1, w2, b2, c, L = unpack(theta, heads, hidden)
    K, H = hidden, heads
    S = dS.shape[0]
    g_w1 = np.zeros(K)
    g_b1 = np.zeros(K)
    g_w2 = np.zeros((H, K))
    g_b2 = np.zeros(H)
    g_c = 0.0
    g_L = 0.0
    cols = np.arange(S)
    for r0 in range(0, S, ROW_BLOCK):
        rows = np.arange(r0, min(S, r0 + ROW_BLOCK))
        g = np.where(cols[None, :] <= rows[:, None], dS[rows[0]:rows[-1] + 1], 0.0)
        x = fire_x(rows, cols, c, L)                          # [rb, S]
        z = x[..., None] * w1 + b1                            # [rb, S, K]
        a = np.maximum(z, 0.0)
        g_b2[head] += g.sum()
        g_w2[head] += np.einsum("rs,rsk->k", g, a)
        dz = g[..., None] * w2[head] * (z > 0)                # [rb, S, K]
        g_w1 += np.einsum("rsk,rs->k", dz, x)
        g_b1 += dz.sum(axis=(0, 1))
        dx = dz @ w1                                          # [rb, S]
        i = rows.astype(np.float64)[:, None]
        d = np.maximum(i - cols[None, :], 0.0)
        m = np.maximum(L, i)
        lnE = np.log1p(c * m)
        dxdc = (d / (c * d + 1.0) - x * m / (c * m + 1.0)) / lnE
        g_c += (dx * dxdc).sum()
        below = (i < L).astype(np.float64)
        dxdL = -x * c / ((c * L + 1.0) * np.log1p(c * L)) * below
        g_L += (dx * dxdL).sum()
    return np.concatenate([g_w1, g_b1, g_w2.ravel(), g_b2, [g_c, g_L]])
