"""torch.compile through the attention custom ops on the GPU: a whole
forward-and-loss function traced as one graph (fullgraph=True, no break at
the kernels), whose outputs and gradients equal the eager ones bit for bit
(the same kernels run in both)."""
import numpy as np
import pytest
import torch

import synth
from helpers import bf16_tensor

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("attention_t5_relative_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _leaves(inp, table):
    q, k, v = (bf16_tensor(getattr(inp, n)).requires_grad_() for n in ("q", "k", "v"))
    t = torch.from_numpy(table).cuda().requires_grad_()
    return q, k, v, t


@pytest.mark.parametrize("causal", [True, False])
def test_compiled_dense_t5_equals_eager(causal):
    inp = synth.draw_dense(91, 2, 300, 3, 64)
    w = torch.randn(2, 300, 3, 64, device="cuda", generator=torch.Generator("cuda").manual_seed(1))

    def loss_fn(q, k, v, t):
        o, lse = fa.attention(q, k, v, bias=fa.T5Bias(t, 32, 128, not causal), causal=causal,
                              return_lse=True)
        return (o.float() * w).sum() + lse.sum() * 0.01

    runs = []
    for fn in (loss_fn, torch.compile(loss_fn, fullgraph=True, backend="aot_eager")):
        q, k, v, t = _leaves(inp, inp.table)
        loss = fn(q, k, v, t)
        loss.backward()
        torch.cuda.synchronize()
        runs.append([loss.detach()] + [x.grad for x in (q, k, v, t)])
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_compiled_packed_fire_equals_eager():
    lengths = np.array([5, 130, 64, 201])
    T, H, D, K = int(lengths.sum()), 2, 64, 8
    inp = synth.draw_varlen(92, T, H, D, lengths=lengths, with_table=False)
    theta = synth.draw_fire_theta(3, H, K, c=0.3, threshold=40.0)
    cu = torch.from_numpy(inp.cu_seqlens).cuda()

    def loss_fn(q, k, v, th):
        o = fa.varlen_attention(q, k, v, cu, int(lengths.max()), bias=fa.FireBias(th, K),
                                causal=True, scale=0.125)
        return o.float().square().sum()

    runs = []
    for fn in (loss_fn, torch.compile(loss_fn, fullgraph=True, backend="aot_eager")):
        q, k, v, th = _leaves(inp, theta)
        loss = fn(q, k, v, th)
        loss.backward()
        torch.cuda.synchronize()
        runs.append([loss.detach()] + [x.grad for x in (q, k, v, th)])
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_compiled_norm_and_loss_equal_eager():
    g = torch.Generator("cuda").manual_seed(5)
    x0 = torch.randn(256, 768, device="cuda", generator=g).to(torch.bfloat16)
    w0 = (1 + 0.25 * torch.randn(768, device="cuda", generator=g)).to(torch.bfloat16)
    proj = (torch.randn(768, 1000, device="cuda", generator=g) * 0.05).to(torch.bfloat16)
    labels = torch.randint(0, 1000, (256,), device="cuda", generator=g)
    labels[::7] = -100

    def loss_fn(x, w):
        h = fa.rms_norm(x, w)
        rows = fa.cross_entropy(h @ proj, labels, z_loss=1e-4)
        return rows.sum() / (labels != -100).sum()

    runs = []
    for fn in (loss_fn, torch.compile(loss_fn, fullgraph=True, backend="aot_eager")):
        x, w = x0.clone().requires_grad_(), w0.clone().requires_grad_()
        loss = fn(x, w)
        loss.backward()
        torch.cuda.synchronize()
        runs.append([loss.detach(), x.grad, w.grad])
    for a, b in zip(*runs):
        assert torch.equal(a, b)
