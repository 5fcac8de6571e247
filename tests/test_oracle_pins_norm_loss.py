"""Pins of the RMSNorm and cross-entropy (+ z-loss) oracle against PyTorch's
own fp64 routines with autograd, central finite differences, closed forms
and invariants (no GPU)."""
import math

import numpy as np
import pytest
import torch

import oracle


@pytest.mark.parametrize("N,d,eps", [(7, 16, 1e-6), (3, 33, 1e-2), (5, 512, 1e-5)])
def test_rmsnorm_against_torch_rms_norm_and_autograd(N, d, eps):
    rng = np.random.default_rng(N * d)
    x, dy = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    w = rng.normal(1.0, 0.3, d)
    y, rstd = oracle.rmsnorm_fwd(x, w, eps)
    dx, dw = oracle.rmsnorm_bwd(x, w, dy, eps)
    tx, tw = torch.tensor(x, requires_grad=True), torch.tensor(w, requires_grad=True)
    ty = torch.nn.functional.rms_norm(tx, (d,), weight=tw, eps=eps)
    ty.backward(torch.tensor(dy))
    np.testing.assert_allclose(y, ty.detach().numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=0, atol=1e-12)
    # rstd is the reciprocal root mean square, and normalised rows have unit RMS
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt((x * x).mean(1) + eps), rtol=1e-15)
    np.testing.assert_allclose(np.sqrt(((y / w) ** 2).mean(1) + eps * rstd ** 2), 1.0, rtol=1e-12)


def test_rmsnorm_finite_differences_and_scale_invariance():
    rng = np.random.default_rng(5)
    N, d, eps = 3, 9, 1e-6
    x, dy, w = rng.standard_normal((N, d)), rng.standard_normal((N, d)), rng.normal(1, .3, d)
    dx, dw = oracle.rmsnorm_bwd(x, w, dy, eps)

    def loss(x_, w_):
        return float((oracle.rmsnorm_fwd(x_, w_, eps)[0] * dy).sum())

    h = 1e-6
    num = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        a, b = x.copy(), x.copy()
        a[idx] += h
        b[idx] -= h
        num[idx] = (loss(a, w) - loss(b, w)) / (2 * h)
    np.testing.assert_allclose(dx, num, rtol=0, atol=1e-7)
    numw = np.array([(loss(x, w + h * e) - loss(x, w - h * e)) / (2 * h) for e in np.eye(d)])
    np.testing.assert_allclose(dw, numw, rtol=0, atol=1e-7)
    # with eps = 0 the output does not depend on the scale of a row, so the
    # row's gradient is orthogonal to the row
    dx0, _ = oracle.rmsnorm_bwd(x, w, dy, 0.0)
    np.testing.assert_allclose((dx0 * x).sum(1), 0.0, atol=1e-12)


@pytest.mark.parametrize("z_loss", [0.0, 1e-4, 0.05])
def test_cross_entropy_against_torch_and_autograd(z_loss):
    rng = np.random.default_rng(11)
    N, V = 9, 37
    z = 3.0 * rng.standard_normal((N, V))
    y = rng.integers(0, V, N)
    y[2] = -100          # ignore index
    y[5] = V + 3         # outside the vocabulary: also ignored
    g = rng.standard_normal(N)
    loss, lse = oracle.cross_entropy_fwd(z, y, z_loss)
    dz = oracle.cross_entropy_bwd(z, y, g, z_loss)

    tz = torch.tensor(z, requires_grad=True)
    ok = torch.tensor((y >= 0) & (y < V))
    ty = torch.tensor(np.where((y >= 0) & (y < V), y, -100))
    tl = torch.nn.functional.cross_entropy(tz, ty, reduction="none", ignore_index=-100)
    tlse = torch.logsumexp(tz, dim=1)
    tl = tl + z_loss * tlse ** 2 * ok
    tl.backward(torch.tensor(g))
    np.testing.assert_allclose(loss, tl.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, tlse.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dz, tz.grad.numpy(), rtol=0, atol=1e-12)


def test_cross_entropy_closed_forms_and_finite_differences():
    # uniform logits: lse = log V + z0, loss = log V (+ z-loss), gradient 1/V - onehot
    V, c = 10, 1e-3
    z = np.full((2, V), 0.5)
    loss, lse = oracle.cross_entropy_fwd(z, np.array([3, 0]), c)
    np.testing.assert_allclose(lse, math.log(V) + 0.5, rtol=1e-15)
    np.testing.assert_allclose(loss, math.log(V) + c * (math.log(V) + 0.5) ** 2, rtol=1e-14)
    dz = oracle.cross_entropy_bwd(z, np.array([3, 0]), np.ones(2), 0.0)
    ref = np.full((2, V), 1.0 / V)
    ref[0, 3] -= 1
    ref[1, 0] -= 1
    np.testing.assert_allclose(dz, ref, atol=1e-15)
    # each row's gradient sums to 2 c lse g (softmax sums to one)
    rng = np.random.default_rng(2)
    z = rng.standard_normal((4, 13))
    y = np.array([1, 12, 0, 7])
    g = rng.standard_normal(4)
    _, lse = oracle.cross_entropy_fwd(z, y, 0.01)
    dz = oracle.cross_entropy_bwd(z, y, g, 0.01)
    np.testing.assert_allclose(dz.sum(1), 2 * 0.01 * lse * g, atol=1e-13)
    h = 1e-6
    num = np.zeros_like(z)
    for idx in np.ndindex(z.shape):
        a, b = z.copy(), z.copy()
        a[idx] += h
        b[idx] -= h
        num[idx] = ((oracle.cross_entropy_fwd(a, y, 0.01)[0] * g).sum()
                    - (oracle.cross_entropy_fwd(b, y, 0.01)[0] * g).sum()) / (2 * h)
    np.testing.assert_allclose(dz, num, rtol=0, atol=1e-8)
