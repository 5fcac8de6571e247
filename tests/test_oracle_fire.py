"""Pins of the FIRE oracle (oracle.fire and the "fire" bias of
oracle.attention) against closed forms, brute force, invariants of the
definition, torch autograd and finite differences.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.attention import head_bwd, head_fwd
from oracle.fire import fire_bias, fire_theta_grad, fire_x, theta_size, unpack


def test_x_closed_form_values():
    # psi(t) = ln(c t + 1); x = psi(i - j) / psi(max(L, i)); hand-picked pairs
    c, L = 1.0, 4.0
    x = fire_x(np.arange(10), np.arange(10), c, L)
    assert x[2, 0] == pytest.approx(math.log(3) / math.log(5), rel=1e-15)
    assert x[8, 3] == pytest.approx(math.log(6) / math.log(9), rel=1e-15)
    assert x[3, 1] == pytest.approx(math.log(3) / math.log(5), rel=1e-15)
    assert x[0, 0] == 0.0 and x[7, 7] == 0.0
    assert x[9, 0] == pytest.approx(1.0, rel=1e-15)      # j = 0, i >= L: x = 1
    c, L = 0.25, 2.5
    x = fire_x(np.arange(6), np.arange(6), c, L)
    assert x[1, 0] == pytest.approx(math.log(1.25) / math.log(1.625), rel=1e-15)
    assert x[5, 2] == pytest.approx(math.log(1.75) / math.log(2.25), rel=1e-15)


def _theta(H, K, ws, bs, w2, b2, c, L):
    return np.concatenate([ws, bs, np.asarray(w2, float).ravel(), b2, [c, L]])


def test_identity_mlp_gives_x_brute_force():
    # one hidden unit, w1 = 1, b1 = 0, w2 = 1, b2 = 0: f(x) = relu(x) = x
    S, c, L = 23, 0.3, 7.5
    th = _theta(1, 1, [1.0], [0.0], [[1.0]], [0.0], c, L)
    b = fire_bias(S, th, 1, 1)[0]
    for i in range(S):
        for j in range(S):
            want = math.log(c * (i - j) + 1) / math.log(c * max(L, i) + 1) if j <= i else 0.0
            assert b[i, j] == pytest.approx(want, rel=1e-14, abs=1e-15)


def test_mlp_brute_force_small():
    H, K, S = 3, 5, 17
    th = synth.draw_fire_theta(11, H, K, c=0.7, threshold=6.0).astype(np.float64)
    w1, b1, w2, b2, c, L = unpack(th, H, K)
    b = fire_bias(S, th, H, K)
    for h in range(H):
        for i in range(S):
            for j in range(i + 1):
                x = math.log(c * (i - j) + 1) / math.log(c * max(L, i) + 1)
                f = b2[h] + sum(w2[h, k] * max(w1[k] * x + b1[k], 0.0) for k in range(K))
                assert b[h, i, j] == pytest.approx(f, rel=1e-13, abs=1e-14)


def test_invariants():
    H, K, S = 4, 16, 96
    th = synth.draw_fire_theta(3, H, K, c=0.2, threshold=40.0).astype(np.float64)
    w1, b1, w2, b2, c, L = unpack(th, H, K)
    b = fire_bias(S, th, H, K)
    f0 = b2 + w2 @ np.maximum(b1, 0.0)             # x = 0
    f1 = b2 + w2 @ np.maximum(w1 + b1, 0.0)        # x = 1
    for h in range(H):
        # diagonal: distance 0 gives x = 0
        assert np.allclose(np.diag(b[h]), f0[h], rtol=0, atol=1e-12)
        # rows below the threshold share the normaliser psi(L): Toeplitz
        for i in range(int(L) - 1):
            assert np.allclose(b[h, i + 1, 1:i + 2], b[h, i, :i + 1], rtol=0, atol=1e-12)
        # key 0 of a row at or past the threshold: x = 1
        assert np.allclose(b[h, int(math.ceil(L)):, 0], f1[h], rtol=0, atol=1e-12)
        # masked (key after query) entries are 0
        assert np.all(np.triu(b[h], 1) == 0.0)
    # x stays in [0, 1] for every visible pair
    x = fire_x(np.arange(S), np.arange(S), c, L)
    assert x.min() >= 0.0 and x.max() <= 1.0 + 1e-15


def _torch_fire_loss(th_t, dS, H, K):
    """sum_hij dS_hij f_theta(x_ij)_h in torch, for autograd."""
    S = dS.shape[-1]
    w1, b1 = th_t[:K], th_t[K:2 * K]
    w2 = th_t[2 * K:2 * K + H * K].reshape(H, K)
    b2 = th_t[2 * K + H * K:2 * K + H * K + H]
    c, L = th_t[-2], th_t[-1]
    i = torch.arange(S, dtype=torch.float64)[:, None]
    j = torch.arange(S, dtype=torch.float64)[None, :]
    d = torch.clamp(i - j, min=0.0)
    x = torch.log1p(c * d) / torch.log1p(c * torch.maximum(L.expand_as(i), i))
    f = torch.relu(x[..., None] * w1 + b1) @ w2.T + b2            # [S, S, H]
    vis = (j <= i).to(torch.float64)
    return (f.permute(2, 0, 1) * vis * dS).sum()


@pytest.mark.parametrize("c,L", [(0.1, 20.5), (1.3, 3.25), (0.5, 100.0)])
def test_theta_grad_against_torch_autograd(c, L):
    H, K, S = 3, 12, 48
    th = synth.draw_fire_theta(5, H, K, c=c, threshold=L).astype(np.float64)
    rng = np.random.default_rng(2)
    dS = np.tril(rng.standard_normal((H, S, S)))
    got = sum(fire_theta_grad(dS[h], h, th, H, K) for h in range(H))
    th_t = torch.tensor(th, requires_grad=True)
    _torch_fire_loss(th_t, torch.tensor(dS), H, K).backward()
    want = th_t.grad.numpy()
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10)


def test_theta_grad_finite_differences():
    H, K, S = 2, 6, 29
    th = synth.draw_fire_theta(8, H, K, c=0.4, threshold=9.5).astype(np.float64)
    rng = np.random.default_rng(4)
    dS = np.tril(rng.standard_normal((H, S, S)))

    def loss(t):
        b = fire_bias(S, t, H, K)
        return float((b * dS).sum())

    got = sum(fire_theta_grad(dS[h], h, th, H, K) for h in range(H))
    eps = 1e-6
    for idx in range(theta_size(H, K)):
        tp, tm = th.copy(), th.copy()
        tp[idx] += eps
        tm[idx] -= eps
        fd = (loss(tp) - loss(tm)) / (2 * eps)
        assert got[idx] == pytest.approx(fd, rel=1e-5, abs=1e-6), idx


def _attn_inputs(seed, S, D):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((S, D)) for _ in range(4))
    return q, k, v, do


def test_attention_with_fire_equals_dense_bias_mode():
    H, K, S, D = 2, 8, 40, 16
    th = synth.draw_fire_theta(6, H, K, c=0.3, threshold=12.0).astype(np.float64)
    q, k, v, do = _attn_inputs(1, S, D)
    for h in range(H):
        of, lf = head_fwd(q, k, v, h, scale=0.5, causal=True, bias="fire", fire=th,
                          fire_hidden=K)
        dense = fire_bias(S, th, H, K, head=h)
        od, ld = head_fwd(q, k, v, h, scale=0.5, causal=True, bias="dense", dense=dense)
        np.testing.assert_allclose(of, od, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lf, ld, rtol=0, atol=1e-13)
        _, _, _, dth = head_bwd(q, k, v, do, h, scale=0.5, causal=True, bias="fire", fire=th,
                                fire_hidden=K)
        _, _, _, dS = head_bwd(q, k, v, do, h, scale=0.5, causal=True, bias="dense", dense=dense)
        np.testing.assert_allclose(dth, fire_theta_grad(dS, h, th, H, K), rtol=1e-12, atol=1e-12)


def test_attention_theta_gradient_finite_differences():
    # loss = sum O * W + sum LSE * u over a batch of 2 and all heads; the
    # oracle's d(theta) against central differences of the whole forward
    B, S, H, D, K = 2, 21, 2, 8, 5
    th = synth.draw_fire_theta(9, H, K, c=0.6, threshold=7.5).astype(np.float64)
    rng = np.random.default_rng(7)
    q, k, v, W = (rng.standard_normal((B, S, H, D)) for _ in range(4))
    u = rng.standard_normal((B, H, S))
    kw = dict(scale=0.7, causal=True, bias="fire", fire_hidden=K)

    def loss(t):
        o, lse = oracle.attention_fwd(q, k, v, fire=t, **kw)
        return float((o * W).sum() + (lse * u).sum())

    _, _, _, dth = oracle.attention_bwd(q, k, v, W, dlse=u, fire=th, **kw)
    eps = 1e-6
    for idx in range(theta_size(H, K)):
        tp, tm = th.copy(), th.copy()
        tp[idx] += eps
        tm[idx] -= eps
        fd = (loss(tp) - loss(tm)) / (2 * eps)
        assert dth[idx] == pytest.approx(fd, rel=1e-5, abs=1e-7), idx


def test_fire_requires_causal():
    th = synth.draw_fire_theta(1, 1, 2).astype(np.float64)
    q, k, v, _ = _attn_inputs(0, 8, 4)
    with pytest.raises(ValueError):
        head_fwd(q, k, v, 0, causal=False, bias="fire", fire=th, fire_hidden=2)


def test_varlen_fire_equals_dense_slices():
    H, K, D = 2, 4, 8
    th = synth.draw_fire_theta(2, H, K, c=0.5, threshold=5.0).astype(np.float64)
    lens = [7, 1, 12]
    cu = np.concatenate([[0], np.cumsum(lens)])
    rng = np.random.default_rng(3)
    T = int(cu[-1])
    q, k, v, do = (rng.standard_normal((T, H, D)) for _ in range(4))
    kw = dict(scale=1.0, causal=True, bias="fire", fire=th, fire_hidden=K)
    o, lse = oracle.varlen_attention_fwd(q, k, v, cu, **kw)
    _, _, _, dth = oracle.varlen_attention_bwd(q, k, v, do, cu, **kw)
    want_dth = np.zeros_like(dth)
    for s in range(len(lens)):
        a, e = cu[s], cu[s + 1]
        od, ld = oracle.attention_fwd(q[None, a:e], k[None, a:e], v[None, a:e], **kw)
        np.testing.assert_allclose(o[a:e], od[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, a:e], ld[0], rtol=0, atol=1e-13)
        want_dth += oracle.attention_bwd(q[None, a:e], k[None, a:e], v[None, a:e],
                                         do[None, a:e], **kw)[3]
    np.testing.assert_allclose(dth, want_dth, rtol=1e-12, atol=1e-12)
