"""fp64 NumPy oracle for the report's two other fused kernels: RMSNorm and the
cross-entropy loss with z-loss.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: FAT5 report, section on Triton kernels ("d'autres parties de
l'architecture ont été optimisées à l'aide de noyaux Triton ad hoc"): the
cross-entropy loss with the z-loss it cites (de Brébisson & Vincent, 2016)
and the RMSNorm layer it cites (Zhang & Sennrich, 2019); benchmarks under
"Torch vs Triton".  The pages print no formula for either; the readings:

* RMSNorm (the cited layer, as T5 uses it): no mean subtraction, no bias,
      y = x / sqrt(mean_j x_j^2 + eps) * w,
  per row of x [N, d], weight w [d].  The backward is its calculus:
      r = 1 / sqrt(mean x^2 + eps),  g = dy * w,
      dx = r g - x r^3 (sum_j g_j x_j) / d,   dw = sum over rows of dy x r.
* Cross-entropy with z-loss, per row of logits z [N, V] and label y:
      lse = log sum_v exp(z_v),  loss = lse - z_y + c lse^2,
  with c the z-loss coefficient; rows whose label is the ignore index (or
  outside [0, V)) have loss 0 and no gradient.  The mean over rows is the
  caller's.  Backward with dL/dloss = g per row:
      dz = g * (softmax(z) * (1 + 2 c lse) - onehot(y)).
"""
from __future__ import annotations

import numpy as np


def rmsnorm_fwd(x, w, eps):
    """x float64 [N, d], w [d] -> (y [N, d], rstd [N])."""
    x = np.asarray(x, dtype=np.float64)
    rstd = 1.0 / np.sqrt((x * x).mean(axis=1) + eps)
    return x * rstd[:, None] * np.asarray(w, dtype=np.float64)[None, :], rstd


def rmsnorm_bwd(x, w, dy, eps):
    """-> (dx [N, d], dw [d]) for loss gradient dy [N, d]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    d = x.shape[1]
    _, r = rmsnorm_fwd(x, w, eps)
    g = dy * w[None, :]
    c = (g * x).sum(axis=1) / d
    dx = r[:, None] * g - x * (r ** 3)[:, None] * c[:, None]
    dw = (dy * x * r[:, None]).sum(axis=0)
    return dx, dw


def _valid(y, V, ignore_index):
    y = np.asarray(y, dtype=np.int64)
    return (y != ignore_index) & (y >= 0) & (y < V)


def _lse(z):
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def cross_entropy_fwd(z, y, z_loss, ignore_index=-100):
    """z float64 [N, V], y int [N] -> (loss [N], lse [N])."""
    z = np.asarray(z, dtype=np.float64)
    N, V = z.shape
    ok = _valid(y, V, ignore_index)
    lse = _lse(z)
    zy = np.where(ok, z[np.arange(N), np.where(ok, y, 0)], 0.0)
    loss = np.where(ok, lse - zy + z_loss * lse * lse, 0.0)
    return loss, lse


def cross_entropy_bwd(z, y, dloss, z_loss, ignore_index=-100):
    """-> dz [N, V] for dL/dloss = dloss [N]."""
    z = np.asarray(z, dtype=np.float64)
    N, V = z.shape
    ok = _valid(y, V, ignore_index)
    lse = _lse(z)
    p = np.exp(z - lse[:, None])
    dz = p * (1.0 + 2.0 * z_loss * lse)[:, None]
    rows = np.nonzero(ok)[0]
    dz[rows, np.asarray(y)[rows]] -= 1.0
    dz *= np.asarray(dloss, dtype=np.float64)[:, None]
    dz[~ok] = 0.0
    return dz
