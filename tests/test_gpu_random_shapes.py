"""Seeded random problems against the oracle, forward and backward, through
the dense and the packed entry points: head dims 64 and 128, lengths with
ragged tails and whole multiples of the 64-key tile, odd head and batch
counts, causal and bidirectional masks, T5 (random bucket geometries),
ALiBi or no bias, with and without RoPE, several scales; then dense bias
matrices (shared or per batch) and FIRE (random widths, c and thresholds).
The cases are drawn once from fixed seeds, so every run checks the same
problems; each compares every element of O, LSE, dQ, dK, dV and the bias
gradient under the gates of the other parity tests."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (assert_dtable, assert_grad, assert_lse, assert_o, bf16_tensor, nan_like,
                     oracle_kwargs, to_f64)

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("attention_t5_relative_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _geometry(rng):
    """A random valid T5 geometry: (num_buckets, max_distance, bidirectional)."""
    bidi = bool(rng.integers(0, 2))
    nb = int(rng.integers(2, 25)) * 2 if bidi else int(rng.integers(2, 49))
    nbp = nb // 2 if bidi else nb
    md = int(rng.integers(nbp // 2 + 1, 1025))
    return nb, md, bidi


def _common(rng):
    D = int(rng.choice([64, 128]))
    causal = bool(rng.integers(0, 2))
    kind = str(rng.choice(["t5", "t5", "t5", "alibi", "none"]))
    nb, md, bidi = _geometry(rng)
    rope = float(rng.choice([0.0, 0.0, 500.0, 10000.0])) or None
    scale = float(rng.choice([1.0, D ** -0.5, 0.3]))
    return D, causal, kind, nb, md, bidi, rope, scale


def _dense_cases(n=40, seed=20261):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        D, causal, kind, nb, md, bidi, rope, scale = _common(rng)
        form = int(rng.integers(0, 3))
        if form == 0:
            S = int(rng.integers(1, 700))
        elif form == 1:
            S = 64 * int(rng.integers(1, 10))
        else:
            S = 64 * int(rng.integers(1, 10)) + int(rng.choice([-1, 1]))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 6))
        out.append((B, S, H, D, causal, kind, nb, md, bidi, rope, scale))
    return out


def _varlen_cases(n=12, seed=20262):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        D, causal, kind, nb, md, bidi, rope, scale = _common(rng)
        lengths = tuple(int(x) for x in rng.integers(1, 400, size=int(rng.integers(2, 7))))
        H = int(rng.integers(1, 5))
        out.append((lengths, H, D, causal, kind, nb, md, bidi, rope, scale))
    return out


def _bias(kind, H, table, nb, md, bidi, slope_mult=1.0):
    if kind == "t5":
        return fa.T5Bias(torch.from_numpy(table).cuda(), nb, md, bidi), None
    if kind == "alibi":
        s = (synth.alibi_slope_values(H) * slope_mult).astype(np.float32)
        return fa.ALiBi(torch.from_numpy(s).cuda()), s.astype(np.float64)
    return None, None


def _dense_id(c):
    B, S, H, D, causal, kind, nb, md, bidi, rope, scale = c
    geo = f"{nb}x{md}{'bi' if bidi else ''}" if kind == "t5" else ""
    return f"b{B}s{S}h{H}d{D}-c{int(causal)}-{kind}{geo}-r{int(bool(rope))}"


@pytest.mark.parametrize("case", _dense_cases(), ids=_dense_id)
def test_random_dense_problem(case):
    B, S, H, D, causal, kind, nb, md, bidi, rope, scale = case
    inp = synth.draw_dense(5000 + S * 7 + H, B, S, H, D, num_buckets=nb)
    _check_dense(inp, case)


class _Scaled:
    """Inputs with q and k multiplied by 2^a (exact in bf16) and the T5 table
    by tmul: a softmax peaked far beyond the N(0, 1) draws."""

    def __init__(self, inp, a, tmul):
        f = 2.0 ** a
        for n in ("q", "k"):
            setattr(self, n, synth.bf16_round(synth.bf16_bits_to_f32(getattr(inp, n)) * f))
        self.v, self.do = inp.v, inp.do
        self.table = None if inp.table is None else (inp.table * tmul).astype(np.float32)

    def f64(self, name):
        return synth.bf16_bits_to_f32(getattr(self, name)).astype(np.float64)


PEAKED = [
    # B, S, H, D, causal, bias, nb, md, bidirectional, rope, scale, log2 of the q/k factor,
    # table factor, ALiBi slope factor
    (1, 300, 2, 64, True, "t5", 32, 128, False, None, 1.0, 2, 8.0, 1.0),
    (2, 257, 2, 128, False, "t5", 32, 128, True, None, 128 ** -0.5, 2, 4.0, 1.0),
    (1, 320, 3, 128, True, "alibi", 32, 128, False, None, 128 ** -0.5, 1, 1.0, 16.0),
    (1, 200, 2, 64, False, "none", 32, 128, False, 10000.0, 0.125, 2, 1.0, 1.0),
]


@pytest.mark.parametrize("case", PEAKED, ids=lambda c: f"{c[5]}-d{c[3]}-a{c[11]}")
def test_peaked_softmax(case):
    """Scores a few hundred log2 units apart (q, k amplified, large table
    values or slopes): nearly one-hot rows, exercising the running-max
    rescale, exponent underflow and the backward's exact D."""
    B, S, H, D, causal, kind, nb, md, bidi, rope, scale, a, tmul, smul = case
    base = synth.draw_dense(6100 + S, B, S, H, D, num_buckets=nb)
    _check_dense(_Scaled(base, a, tmul), case[:11], slope_mult=smul)


def _check_dense(inp, case, slope_mult=1.0):
    B, S, H, D, causal, kind, nb, md, bidi, rope, scale = case
    q, k, v, do = (bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    bias, slopes = _bias(kind, H, inp.table, nb, md, bidi, slope_mult)
    o = nan_like(q)
    lse = torch.full((B, H, S), float("nan"), device="cuda")
    fa.fa_fwd(q, k, v, o, lse, scale=scale, causal=causal, bias=bias, rope_base=rope or 0.0)
    dq, dk, dv = nan_like(q), nan_like(q), nan_like(q)
    dtable = torch.full((nb, H), float("nan"), device="cuda") if kind == "t5" else None
    fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, dtable, scale=scale, causal=causal, bias=bias,
              rope_base=rope or 0.0)
    torch.cuda.synchronize()
    kw = oracle_kwargs(kind, causal, scale, inp.table, slopes, nb, md, bidi, rope)
    args = (inp.f64("q"), inp.f64("k"), inp.f64("v"))
    o_ref, lse_ref = oracle.attention_fwd(*args, **kw)
    assert_o(to_f64(o), o_ref)
    assert_lse(lse.cpu().numpy().astype(np.float64), lse_ref)
    gq, gk, gv, gt = oracle.attention_bwd(*args, inp.f64("do"), **kw)
    assert_grad(to_f64(dq), gq, "dQ")
    assert_grad(to_f64(dk), gk, "dK")
    assert_grad(to_f64(dv), gv, "dV")
    if gt is not None:
        assert_dtable(dtable.cpu().numpy().astype(np.float64), gt)


def _varlen_id(c):
    lengths, H, D, causal, kind, nb, md, bidi, rope, scale = c
    return f"n{len(lengths)}t{sum(lengths)}h{H}d{D}-c{int(causal)}-{kind}-r{int(bool(rope))}"


@pytest.mark.parametrize("case", _varlen_cases(), ids=_varlen_id)
def test_random_packed_problem(case):
    lengths, H, D, causal, kind, nb, md, bidi, rope, scale = case
    lens = np.array(lengths)
    inp = synth.draw_varlen(7000 + int(lens.sum()), int(lens.sum()), H, D, lengths=lens,
                            num_buckets=nb)
    q, k, v, do = (bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    T = q.shape[0]
    cu = torch.from_numpy(inp.cu_seqlens).cuda()
    mx = int(lens.max())
    bias, slopes = _bias(kind, H, inp.table, nb, md, bidi)
    o = nan_like(q)
    lse = torch.full((H, T), float("nan"), device="cuda")
    fa.fa_varlen_fwd(q, k, v, o, lse, cu, mx, scale=scale, causal=causal, bias=bias,
                     rope_base=rope or 0.0)
    dq, dk, dv = nan_like(q), nan_like(q), nan_like(q)
    dtable = torch.full((nb, H), float("nan"), device="cuda") if kind == "t5" else None
    fa.fa_varlen_bwd(q, k, v, o, lse, do, dq, dk, dv, cu, mx, dtable, scale=scale,
                     causal=causal, bias=bias, rope_base=rope or 0.0)
    torch.cuda.synchronize()
    kw = oracle_kwargs(kind, causal, scale, inp.table, slopes, nb, md, bidi, rope)
    args = (inp.f64("q"), inp.f64("k"), inp.f64("v"))
    o_ref, lse_ref = oracle.varlen_attention_fwd(*args, inp.cu_seqlens, **kw)
    assert_o(to_f64(o), o_ref)
    assert_lse(lse.cpu().numpy().astype(np.float64), lse_ref)
    gq, gk, gv, gt = oracle.varlen_attention_bwd(*args, inp.f64("do"), inp.cu_seqlens, **kw)
    assert_grad(to_f64(dq), gq, "dQ")
    assert_grad(to_f64(dk), gk, "dK")
    assert_grad(to_f64(dv), gv, "dV")
    if gt is not None:
        assert_dtable(dtable.cpu().numpy().astype(np.float64), gt)


def _dense_bias_cases(n=8, seed=20263):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        S = int(rng.integers(1, 600))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        Bb = int(rng.choice([1, B]))
        scale = float(rng.choice([1.0, D ** -0.5]))
        rope = float(rng.choice([0.0, 0.0, 10000.0])) or None
        out.append((B, S, H, D, causal, Bb, scale, rope))
    return out


@pytest.mark.parametrize("case", _dense_bias_cases(), ids=lambda c: "b{}s{}h{}d{}-c{}-bb{}-r{}".format(
    c[0], c[1], c[2], c[3], int(c[4]), c[5], int(c[7] is not None)))
def test_random_dense_bias_problem(case):
    from test_gpu_dense_bias import assert_dbias, run_dense
    B, S, H, D, causal, Bb, scale, rope = case
    inp = synth.draw_dense(8000 + S, B, S, H, D, with_table=False)
    dense = synth.draw_dense_bias(9000 + S, Bb, H, S)
    out, kw = run_dense(inp, dense, causal=causal, scale=scale, rope_base=rope)
    args = (inp.f64("q"), inp.f64("k"), inp.f64("v"))
    O, LSE = oracle.attention_fwd(*args, **kw)
    assert_o(out["o"], O)
    assert_lse(out["lse"], LSE)
    gq, gk, gv, gb = oracle.attention_bwd(*args, inp.f64("do"), **kw)
    assert_grad(out["dq"], gq, "dQ")
    assert_grad(out["dk"], gk, "dK")
    assert_grad(out["dv"], gv, "dV")
    assert_dbias(out["dbias"], gb)


def _fire_cases(n=8, seed=20264):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 5))
        S = int(rng.integers(1, 600))
        D = int(rng.choice([64, 128]))
        K = (1, 3, 8, 16, 32, 64, 5, 48)[i % 8]
        c = float(np.round(rng.uniform(0.05, 2.0), 3))
        L = float(np.round(rng.uniform(2.0, 1000.0), 1))
        scale = float(rng.choice([1.0, D ** -0.5]))
        out.append((B, S, H, D, K, c, L, scale, 30 + i))
    return out


@pytest.mark.parametrize("case", _fire_cases(), ids=lambda c: "b{}s{}h{}d{}k{}".format(*c[:5]))
def test_random_fire_problem(case):
    from test_gpu_fire import _check_theta, _run_dense
    B, S, H, D, K, c, L, scale, seed = case
    inp, theta, out, kw, f = _run_dense(*case)
    O, LSE = oracle.attention_fwd(f["q"], f["k"], f["v"], **kw)
    assert_o(out["o"], O)
    assert_lse(out["lse"], LSE)
    gq, gk, gv, gth = oracle.attention_bwd(f["q"], f["k"], f["v"], f["do"], **kw)
    assert_grad(out["dq"], gq, "dQ")
    assert_grad(out["dk"], gk, "dK")
    assert_grad(out["dv"], gv, "dV")
    _check_theta(out["dtheta"], gth, H, K, f"FIRE {case}")
