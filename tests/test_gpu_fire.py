"""FIRE bias on the GPU against the fp64 oracle: forward (O, LSE) and
backward (dQ, dK, dV and d(theta)), dense and packed, head_dim 64 and 128,
thresholds below and above the sequence length."""
import numpy as np
import pytest
import torch

import attention_t5_relative_amd as fa
import oracle
import synth
from helpers import (assert_grad, assert_lse, assert_o, bf16_tensor, log_margin, nan_like,
                     pmap, to_f64)

pytestmark = pytest.mark.gpu

# d(theta) gates.  The whole vector within 1e-2 of its Frobenius norm.  Each
# parameter group within 1e-2 of its own norm, or of 1e-3 of the whole
# vector's norm when the group's own gradient cancels to nearly zero: d(b2)
# is exactly 0 (a constant added to a head's scores leaves its softmax
# unchanged), and so is the constant part of any unit active on all of
# [0, 1]; there the fp32 sums leave only rounding noise.  c and L (scalars
# summed over every visible pair of every head) within 2e-2 of their own
# size plus 1e-3 of the largest entry.
THETA_REL = 1e-2
GROUP_FLOOR = 1e-3
SCALAR_REL, SCALAR_ABS = 2e-2, 1e-3


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _check_theta(got, ref, H, K, what):
    assert np.isfinite(got).all(), f"{what}: non-finite d(theta)"
    full = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref)) / full
    groups = {"w1": slice(0, K), "b1": slice(K, 2 * K), "w2": slice(2 * K, 2 * K + H * K),
              "b2": slice(2 * K + H * K, 2 * K + H * K + H)}
    out = {"theta": rel}
    msgs = []
    for name, sl in groups.items():
        e = float(np.linalg.norm(got[sl] - ref[sl]))
        scale_g = max(float(np.linalg.norm(ref[sl])), GROUP_FLOOR * full)
        out[name] = e / scale_g
        if e > THETA_REL * scale_g:
            msgs.append(f"d{name} error {e:.3e} vs norm {np.linalg.norm(ref[sl]):.3e}")
    big = float(np.abs(ref).max())
    for name, idx in (("c", -2), ("L", -1)):
        e = abs(float(got[idx] - ref[idx]))
        out[name] = e / (SCALAR_REL * abs(float(ref[idx])) + SCALAR_ABS * big)
        if e > SCALAR_REL * abs(float(ref[idx])) + SCALAR_ABS * big:
            msgs.append(f"d{name} {got[idx]:.6e} vs {ref[idx]:.6e}")
    assert rel <= THETA_REL and not msgs, (
        f"{what}: d(theta) relative error {rel:.3e}; " + "; ".join(msgs)
        + f"; dc {got[-2]:.6e}/{ref[-2]:.6e} dL {got[-1]:.6e}/{ref[-1]:.6e}")
    return out


DENSE = [
    # B, S, H, D, hidden, c, L, scale, seed
    (2, 300, 4, 64, 32, 0.1, 512.0, 0.125, 1),       # every row below L: one normaliser
    (1, 700, 3, 64, 32, 1.0, 100.0, 1.0, 2),         # rows past L: per-row normaliser
    (2, 257, 2, 128, 16, 0.5, 64.0, 128 ** -0.5, 3),
    (1, 200, 2, 64, 64, 2.0, 10.5, 0.125, 4),        # 64 hidden units, many kinks
    (1, 129, 5, 128, 1, 0.3, 7.0, 1.0, 5),           # one hidden unit
]


def _run_dense(B, S, H, D, K, c, L, scale, seed, backward=True):
    inp = synth.draw_dense(100 + seed, B, S, H, D, with_table=False)
    theta = synth.draw_fire_theta(seed, H, K, c=c, threshold=L)
    t = {n: bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do")}
    th = torch.from_numpy(theta).cuda()
    bias = fa.FireBias(th, K)
    o = nan_like(t["q"])
    lse = torch.full((B, H, S), float("nan"), device="cuda")
    fa.fa_fwd(t["q"], t["k"], t["v"], o, lse, scale=scale, causal=True, bias=bias)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = nan_like(t["q"]), nan_like(t["q"]), nan_like(t["q"])
        dth = torch.full_like(th, float("nan"))
        fa.fa_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], dq, dk, dv, dth, scale=scale,
                  causal=True, bias=bias)
        out.update(dq=dq, dk=dk, dv=dv, dtheta=dth)
    torch.cuda.synchronize()
    out = {k_: to_f64(v_) for k_, v_ in out.items()}
    kw = dict(scale=scale, causal=True, bias="fire", fire=theta.astype(np.float64),
              fire_hidden=K)
    f64 = {n: inp.f64(n) for n in ("q", "k", "v", "do")}
    return inp, theta, out, kw, f64


@pytest.mark.parametrize("case", DENSE, ids=[f"B{c[0]}S{c[1]}H{c[2]}D{c[3]}K{c[4]}"
                                              for c in DENSE])
def test_fire_dense_against_oracle(case):
    _need_gpu()
    B, S, H, D, K, c, L, scale, seed = case
    inp, theta, out, kw, f = _run_dense(*case)
    pairs = [(b, h) for b in range(B) for h in range(H)]

    def one(bh):
        b, h = bh
        o, lse = oracle.attention_fwd(f["q"], f["k"], f["v"], pairs=[bh], **kw)
        dq, dk, dv, dth = oracle.attention_bwd(f["q"], f["k"], f["v"], f["do"], pairs=[bh], **kw)
        return o[b, :, h], lse[b, h], dq[b, :, h], dk[b, :, h], dv[b, :, h], dth

    res = pmap(one, pairs)
    errs = {}
    dth_ref = np.zeros_like(res[0][5])
    for (b, h), (o, lse, dq, dk, dv, dth) in zip(pairs, res):
        tag = f"FIRE {case} b{b} h{h}"
        errs.setdefault("o", []).append(assert_o(out["o"][b, :, h], o, tag + " O")[0])
        errs.setdefault("lse", []).append(assert_lse(out["lse"][b, h], lse, tag + " LSE"))
        errs.setdefault("dq", []).append(assert_grad(out["dq"][b, :, h], dq, tag + " dQ")[0])
        errs.setdefault("dk", []).append(assert_grad(out["dk"][b, :, h], dk, tag + " dK")[0])
        errs.setdefault("dv", []).append(assert_grad(out["dv"][b, :, h], dv, tag + " dV")[0])
        dth_ref += dth
    te = _check_theta(out["dtheta"], dth_ref, H, K, f"FIRE {case}")
    log_margin(f"fire_dense_{case}", **{k_: max(v_) for k_, v_ in errs.items()},
               **{"dtheta_" + k_: v_ for k_, v_ in te.items()})


VARLEN = [
    # lengths, H, D, hidden, c, L, scale, seed
    ([5, 300, 1, 129, 64], 3, 64, 8, 0.3, 40.0, 0.125, 6),
    ([33, 200, 97], 2, 128, 32, 1.0, 16.0, 128 ** -0.5, 7),
]


@pytest.mark.parametrize("case", VARLEN, ids=["d64", "d128"])
def test_fire_varlen_against_oracle(case):
    _need_gpu()
    lens, H, D, K, c, L, scale, seed = case
    T = int(sum(lens))
    inp = synth.draw_varlen(200 + seed, T, H, D, lengths=np.array(lens), with_table=False)
    theta = synth.draw_fire_theta(seed, H, K, c=c, threshold=L)
    t = {n: bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do")}
    cu = torch.from_numpy(inp.cu_seqlens).cuda()
    th = torch.from_numpy(theta).cuda()
    bias = fa.FireBias(th, K)
    o = nan_like(t["q"])
    lse = torch.full((H, T), float("nan"), device="cuda")
    mx = max(lens)
    fa.fa_varlen_fwd(t["q"], t["k"], t["v"], o, lse, cu, mx, scale=scale, causal=True, bias=bias)
    dq, dk, dv = nan_like(t["q"]), nan_like(t["q"]), nan_like(t["q"])
    dth = torch.full_like(th, float("nan"))
    fa.fa_varlen_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], dq, dk, dv, cu, mx, dth,
                     scale=scale, causal=True, bias=bias)
    torch.cuda.synchronize()
    kw = dict(scale=scale, causal=True, bias="fire", fire=theta.astype(np.float64),
              fire_hidden=K)
    f = {n: inp.f64(n) for n in ("q", "k", "v", "do")}
    ro, rl = oracle.varlen_attention_fwd(f["q"], f["k"], f["v"], inp.cu_seqlens, **kw)
    rq, rk, rv, rth = oracle.varlen_attention_bwd(f["q"], f["k"], f["v"], f["do"],
                                                  inp.cu_seqlens, **kw)
    what = f"FIRE varlen {lens} D{D}"
    assert_o(to_f64(o), ro, what + " O")
    assert_lse(to_f64(lse), rl, what + " LSE")
    assert_grad(to_f64(dq), rq, what + " dQ")
    assert_grad(to_f64(dk), rk, what + " dK")
    assert_grad(to_f64(dv), rv, what + " dV")
    _check_theta(to_f64(dth), rth, H, K, what)


def test_fire_backward_deterministic():
    _need_gpu()
    B, S, H, D, K = 2, 333, 3, 64, 32
    inp = synth.draw_dense(77, B, S, H, D, with_table=False)
    theta = synth.draw_fire_theta(9, H, K, c=0.2, threshold=128.0)
    t = {n: bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do")}
    bias = fa.FireBias(torch.from_numpy(theta).cuda(), K)
    o = torch.empty_like(t["q"])
    lse = torch.empty((B, H, S), device="cuda")
    fa.fa_fwd(t["q"], t["k"], t["v"], o, lse, scale=0.125, causal=True, bias=bias)
    runs = []
    for _ in range(2):
        g = [torch.empty_like(t["q"]) for _ in range(3)] + [torch.empty_like(bias.theta)]
        fa.fa_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], *g, scale=0.125, causal=True,
                  bias=bias)
        runs.append(g)
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_fire_autograd_and_rope():
    # the autograd wrapper routes d(theta) to the parameter; RoPE combines
    _need_gpu()
    B, S, H, D, K = 1, 190, 2, 64, 8
    inp = synth.draw_dense(55, B, S, H, D, with_table=False)
    theta = synth.draw_fire_theta(10, H, K, c=0.7, threshold=50.0)
    q, k, v, do = (bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    th = torch.from_numpy(theta).cuda().requires_grad_(True)
    q.requires_grad_(True)
    o = fa.attention(q, k, v, bias=fa.FireBias(th, K), causal=True, scale=0.125,
                     rope_base=10000.0)
    o.backward(do)
    torch.cuda.synchronize()
    kw = dict(scale=0.125, causal=True, bias="fire", fire=theta.astype(np.float64),
              fire_hidden=K, rope_base=10000.0)
    f = {n: inp.f64(n) for n in ("q", "k", "v", "do")}
    ro, _ = oracle.attention_fwd(f["q"], f["k"], f["v"], **kw)
    rq, _, _, rth = oracle.attention_bwd(f["q"], f["k"], f["v"], f["do"], **kw)
    assert_o(to_f64(o), ro, "FIRE+RoPE O")
    assert_grad(to_f64(q.grad), rq, "FIRE+RoPE dQ")
    _check_theta(to_f64(th.grad), rth, H, K, "FIRE+RoPE")


def test_fire_full_length_batch_one():
    """The FIRE workload's length, heads and parameters (S 4096, H 12, D 64,
    32 hidden units, c 0.1, L 512, the same seeded draws) at batch 1: O, LSE,
    dQ, dK and dV of two heads, and d(theta), which sums over every head,
    against the oracle on all twelve pairs.  The kernels' grid differs from
    the batch-8 launch only in its size."""
    _need_gpu()
    c = synth.config_by_name("c3")
    B, S, H, D, K = 1, c.seqlen, c.heads, c.head_dim, 32
    inp = synth.draw_dense(c.seed, B, S, H, D, with_table=False)
    theta = synth.draw_fire_theta(c.seed, H, K, c=0.1, threshold=512.0)
    t = {n: bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do")}
    th = torch.from_numpy(theta).cuda()
    bias = fa.FireBias(th, K)
    o = nan_like(t["q"])
    lse = torch.full((B, H, S), float("nan"), device="cuda")
    fa.fa_fwd(t["q"], t["k"], t["v"], o, lse, scale=c.scale, causal=True, bias=bias)
    dq, dk, dv = nan_like(t["q"]), nan_like(t["q"]), nan_like(t["q"])
    dth = torch.full_like(th, float("nan"))
    fa.fa_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], dq, dk, dv, dth, scale=c.scale,
              causal=True, bias=bias)
    torch.cuda.synchronize()
    out = {k_: to_f64(v_) for k_, v_ in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items()}
    for name, arr in out.items():
        assert np.isfinite(arr).all(), f"{name}: elements not written or not finite"
    kw = dict(scale=c.scale, causal=True, bias="fire", fire=theta.astype(np.float64),
              fire_hidden=K)
    f = {n: inp.f64(n) for n in ("q", "k", "v", "do")}
    checked = (3, 10)

    def one(h):
        pair = [(0, h)]
        res = {}
        if h in checked:
            O, LSE = oracle.attention_fwd(f["q"], f["k"], f["v"], pairs=pair, **kw)
            res.update(o=O[0, :, h], lse=LSE[0, h])
        rq, rk, rv, rth = oracle.attention_bwd(f["q"], f["k"], f["v"], f["do"], pairs=pair, **kw)
        res.update(dq=rq[0, :, h], dk=rk[0, :, h], dv=rv[0, :, h], dth=rth)
        return res

    res = pmap(one, range(H), workers=12)
    for h in checked:
        r = res[h]
        tag = f"FIRE S{S} h{h}"
        assert_o(out["o"][0, :, h], r["o"], tag + " O")
        assert_lse(out["lse"][0, h], r["lse"], tag + " LSE")
        assert_grad(out["dq"][0, :, h], r["dq"], tag + " dQ")
        assert_grad(out["dk"][0, :, h], r["dk"], tag + " dK")
        assert_grad(out["dv"][0, :, h], r["dv"], tag + " dV")
    te = _check_theta(to_f64(dth), np.sum([r["dth"] for r in res], axis=0), H, K,
                      f"FIRE S{S}")
    log_margin(f"fire_full_length_b1", **{"dtheta_" + k_: v_ for k_, v_ in te.items()})
