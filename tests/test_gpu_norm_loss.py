"""RMSNorm and cross-entropy with z-loss on the GPU (through the C ABI)
against the fp64 oracle on identical seeded inputs.

Bounds (per element): a bf16 output is the fp32 result rounded once (at most
half a bf16 ulp, 2^-9 relative) after fp32 arithmetic (a few fp32 ulps), so
|gpu - ref| <= 2^-8 |ref| plus a small absolute term for values that cancel;
fp32 outputs (rstd, dw, loss, lse) carry only fp32 rounding of their sums."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import bf16_tensor, to_f64

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("attention_t5_relative_amd")

BF16_REL = 2.0 ** -8


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def assert_bf16_close(got, ref, what, abs_scale):
    err = np.abs(got - ref)
    bound = BF16_REL * np.abs(ref) + 1e-5 * abs_scale
    assert np.isfinite(got).all(), f"{what}: non-finite"
    worst = float((err / bound).max()) if err.size else 0.0
    assert worst <= 1.0, f"{what}: error reaches {worst:.2f}x the bound (max err {err.max():.3e})"


def run_rms(x_bits, w_bits, dy_bits, eps, want_dw=True):
    x, w, dy = bf16_tensor(x_bits), bf16_tensor(w_bits), bf16_tensor(dy_bits)
    y = torch.empty_like(x)
    rstd = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
    fa.fa_rmsnorm_fwd(x, w, y, rstd, eps=eps)
    dx = torch.empty_like(x)
    dw = torch.full((x.shape[1],), float("nan"), device="cuda") if want_dw else None
    fa.fa_rmsnorm_bwd(x, w, rstd, dy, dx, dw, eps=eps)
    torch.cuda.synchronize()
    return (to_f64(y), rstd.cpu().numpy().astype(np.float64), to_f64(dx),
            None if dw is None else dw.cpu().numpy().astype(np.float64))


RMS_CASES = [(1, 8, 1e-6), (37, 64, 1e-6), (100, 512, 1e-5), (257, 768, 1e-6), (64, 520, 1e-6),
             (33, 4096, 1e-6), (5, 8192, 1e-2), (10000, 256, 1e-6)]


@pytest.mark.parametrize("rows,dim,eps", RMS_CASES, ids=lambda c: str(c))
def test_rmsnorm(rows, dim, eps):
    xb, wb, dyb = synth.draw_rmsnorm(rows * 7 + dim, rows, dim)
    y, rstd, dx, dw = run_rms(xb, wb, dyb, eps)
    x, w, dy = f64(xb), f64(wb), f64(dyb)
    ry, rr = oracle.rmsnorm_fwd(x, w, eps)
    rdx, rdw = oracle.rmsnorm_bwd(x, w, dy, eps)
    assert_bf16_close(y, ry, "y", np.abs(ry).max())
    np.testing.assert_allclose(rstd, rr, rtol=2e-6)
    assert_bf16_close(dx, rdx, "dx", np.abs(rdx).max())
    # dw: fp32 sums over rows; bound by the sum of magnitudes
    mag = (np.abs(dy * x) * rr[:, None]).sum(axis=0)
    assert (np.abs(dw - rdw) <= 1e-5 * mag + 1e-6).all(), np.abs(dw - rdw).max()


def test_rmsnorm_without_dw_and_empty():
    xb, wb, dyb = synth.draw_rmsnorm(3, 40, 128)
    _, _, dx, dw = run_rms(xb, wb, dyb, 1e-6, want_dw=False)
    assert dw is None
    rdx, _ = oracle.rmsnorm_bwd(f64(xb), f64(wb), f64(dyb), 1e-6)
    assert_bf16_close(dx, rdx, "dx", np.abs(rdx).max())
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    rstd = torch.empty(0, device="cuda")
    fa.fa_rmsnorm_fwd(x, w, x, rstd)
    dw = torch.full((64,), float("nan"), device="cuda")
    fa.fa_rmsnorm_bwd(x, w, rstd, x, x, dw)
    torch.cuda.synchronize()
    assert (dw == 0).all()


def run_ce(zb, y, g, z_loss, in_place=False, rows_out=None):
    z = bf16_tensor(zb)
    lab = torch.from_numpy(y).cuda()
    loss = torch.full((z.shape[0],), float("nan"), device="cuda")
    lse = torch.empty_like(loss)
    fa.fa_ce_fwd(z, lab, loss, lse, z_loss=z_loss)
    dz = z if in_place else torch.empty_like(z)
    fa.fa_ce_bwd(z, lab, lse, torch.from_numpy(g).cuda(), dz, z_loss=z_loss)
    torch.cuda.synchronize()
    if rows_out is not None:
        dz = dz[torch.from_numpy(rows_out).cuda()]
    return (loss.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            to_f64(dz))


CE_CASES = [(1, 8, 0.0), (37, 1000, 1e-4), (64, 32128, 1e-4), (5, 250112, 1e-4), (300, 4096, 0.0)]


@pytest.mark.parametrize("rows,vocab,z_loss", CE_CASES, ids=lambda c: str(c))
def test_cross_entropy(rows, vocab, z_loss):
    zb, y, g = synth.draw_cross_entropy(rows + vocab, rows, vocab)
    if rows > 3:
        y[1], y[2] = vocab + 5, -7      # outside the vocabulary: ignored
    loss, lse, dz = run_ce(zb, y, g, z_loss)
    z = f64(zb)
    rl, rlse = oracle.cross_entropy_fwd(z, y, z_loss)
    rdz = oracle.cross_entropy_bwd(z, y, g.astype(np.float64), z_loss)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=2e-5)
    tol = 2e-5 * (1 + 2 * z_loss * np.abs(rlse))
    assert (np.abs(loss - rl) <= tol).all(), np.abs(loss - rl).max()
    assert_bf16_close(dz, rdz, "dlogits", np.abs(g).max() * 1e-2)
    ignored = (y < 0) | (y >= vocab)
    assert (loss[ignored] == 0).all() and (dz[ignored] == 0).all()


def test_cross_entropy_backward_in_place():
    zb, y, g = synth.draw_cross_entropy(9, 50, 2048)
    loss, lse, dz = run_ce(zb, y, g, 1e-4, in_place=True)
    rdz = oracle.cross_entropy_bwd(f64(zb), y, g.astype(np.float64), 1e-4)
    assert_bf16_close(dz, rdz, "dlogits in place", np.abs(g).max() * 1e-2)


def test_autograd_wrappers():
    """rms_norm and cross_entropy as torch autograd functions; the caller
    takes the mean of the per-row losses over the non-ignored rows."""
    xb, wb, _ = synth.draw_rmsnorm(21, 16, 256)
    x = bf16_tensor(xb).requires_grad_(True)
    w = bf16_tensor(wb).requires_grad_(True)
    y = fa.rms_norm(x.view(4, 4, 256), w)
    assert y.shape == (4, 4, 256)
    zb, lab, _ = synth.draw_cross_entropy(22, 16, 256)
    logits = y.view(16, 256)
    rows = fa.cross_entropy(logits, torch.from_numpy(lab).cuda(), z_loss=1e-4)
    assert rows.shape == (16,) and rows.dtype == torch.float32
    loss = rows.sum() / int(((lab >= 0) & (lab < 256)).sum())
    loss.backward()
    # the same chain in fp64 autograd
    tx = torch.tensor(f64(xb), requires_grad=True)
    tw = torch.tensor(f64(wb), requires_grad=True)
    ty = torch.nn.functional.rms_norm(tx, (256,), weight=tw, eps=1e-6)
    tz = ty.to(torch.bfloat16).double()       # the same bf16 rounding of the logits
    ok = torch.tensor((lab >= 0) & (lab < 256))
    tl = torch.nn.functional.cross_entropy(tz, torch.tensor(lab).long(), ignore_index=-100,
                                           reduction="none") + 1e-4 * torch.logsumexp(tz, 1) ** 2 * ok
    (tl.sum() / ok.sum()).backward()
    assert abs(loss.item() - (tl.sum() / ok.sum()).item()) < 1e-3
    gx = x.grad.float().cpu().numpy().astype(np.float64)
    assert np.abs(gx - tx.grad.numpy()).max() <= 2e-2 * max(1.0, np.abs(tx.grad.numpy()).max())


# The shapes bench.py times: 32768 tokens (the causal decoder workload's
# B8 x S4096), model width 768 for RMSNorm and the T5 vocabulary (32128) for
# the loss.
RMS_BENCH = (32768, 768)
CE_BENCH = (32768, 32128)


def test_rmsnorm_bench_shape_all_rows():
    rows, dim = RMS_BENCH
    xb, wb, dyb = synth.draw_rmsnorm(1234, rows, dim)
    y, rstd, dx, dw = run_rms(xb, wb, dyb, 1e-6)
    x, w, dy = f64(xb), f64(wb), f64(dyb)
    ry, rr = oracle.rmsnorm_fwd(x, w, 1e-6)
    rdx, rdw = oracle.rmsnorm_bwd(x, w, dy, 1e-6)
    assert_bf16_close(y, ry, "y", np.abs(ry).max())
    assert_bf16_close(dx, rdx, "dx", np.abs(rdx).max())
    mag = (np.abs(dy * x) * rr[:, None]).sum(axis=0)
    assert (np.abs(dw - rdw) <= 1e-5 * mag + 1e-6).all()


def test_cross_entropy_bench_shape_sampled_rows():
    rows, vocab = CE_BENCH
    zb, y, g = synth.draw_cross_entropy(4321, rows, vocab)
    sample = np.sort(np.random.default_rng(0).choice(rows, 64, replace=False))
    loss, lse, dz = run_ce(zb, y, g, 1e-4, rows_out=sample)
    z = f64(zb[sample])
    rl, rlse = oracle.cross_entropy_fwd(z, y[sample], 1e-4)
    rdz = oracle.cross_entropy_bwd(z, y[sample], g[sample].astype(np.float64), 1e-4)
    assert (np.abs(lse[sample] - rlse) <= 2e-5).all()
    assert (np.abs(loss[sample] - rl) <= 2e-5 * (1 + 2e-4 * np.abs(rlse))).all()
    assert_bf16_close(dz, rdz, "dlogits", np.abs(g).max() * 1e-2)
    # every row: the loss is finite, ignored rows are exactly 0
    ignored = (y < 0) | (y >= vocab)
    assert np.isfinite(loss).all() and (loss[ignored] == 0).all()
