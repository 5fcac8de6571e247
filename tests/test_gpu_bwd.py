"""Backward parity on the GPU: dQ, dK, dV and the T5 table gradient from the
HIP path (through the C ABI) against the fp64 oracle on identical seeded
inputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (assert_dtable, assert_grad, assert_o, bf16_tensor, check_exact_rotation,
                     log_margin, nan_like, norm_err, oracle_kwargs, to_f64)

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("attention_t5_relative_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _bias(kind, H, table, nb, md, bidirectional):
    if kind == "t5":
        return fa.T5Bias(torch.from_numpy(table).cuda(), nb, md, bidirectional), None
    if kind == "alibi":
        s = synth.alibi_slope_values(H)
        return fa.ALiBi(torch.from_numpy(s).cuda()), s.astype(np.float64)
    return None, None


def run_dense_bwd(inp, *, causal, kind, scale, bidirectional=True, rope_base=None, nb=32,
                  md=128, want_dtable=True, o_for_bwd=None):
    q, k, v, do = (bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    B, S, H, D = q.shape
    bias, slopes = _bias(kind, H, inp.table, nb, md, bidirectional)
    o = nan_like(q)
    lse = torch.full((B, H, S), float("nan"), device="cuda")
    fa.fa_fwd(q, k, v, o, lse, scale=scale, causal=causal, bias=bias, rope_base=rope_base or 0.0)
    dq, dk, dv = nan_like(q), nan_like(q), nan_like(q)
    dtable = (torch.full((nb, H), float("nan"), device="cuda")
              if (kind == "t5" and want_dtable) else None)
    o_in = o if o_for_bwd is None else o_for_bwd(o)
    fa.fa_bwd(q, k, v, o_in, lse, do, dq, dk, dv, dtable, scale=scale, causal=causal, bias=bias,
              rope_base=rope_base or 0.0)
    torch.cuda.synchronize()
    kw = oracle_kwargs(kind, causal, scale, inp.table, slopes, nb, md, bidirectional, rope_base)
    out = dict(o=to_f64(o), dq=to_f64(dq), dk=to_f64(dk), dv=to_f64(dv),
               dtable=None if dtable is None else dtable.cpu().numpy().astype(np.float64))
    return out, kw


SMALL = [
    # B, S, H, D, causal, bias, bidirectional, scale, rope
    (1, 1, 1, 64, False, "t5", True, 1.0, None),
    (2, 37, 3, 64, False, "t5", True, 1.0, None),
    (1, 200, 2, 64, True, "t5", False, 1.0, None),
    (2, 333, 2, 64, False, "t5", False, 0.5, None),
    (1, 300, 3, 128, True, "alibi", False, 0.125, None),
    (1, 257, 2, 128, False, "alibi", False, 0.125, None),
    (1, 300, 2, 128, True, "none", False, 0.088, 10000.0),
    (2, 190, 2, 64, False, "none", False, 0.3, None),
    (1, 260, 2, 64, True, "t5", False, 1.0, 500.0),
    (1, 129, 4, 128, False, "t5", True, 0.2, None),
    (1, 700, 1, 64, False, "t5", True, 1.0, None),
    (1, 520, 2, 128, True, "t5", False, 0.2, None),
    # B*H a multiple of 8: the grouped tile order (two and three pairs per group)
    (2, 300, 8, 64, True, "t5", False, 1.0, None),
    (4, 200, 12, 64, False, "t5", True, 1.0, None),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "b{}s{}h{}d{}-c{}-{}-bi{}-r{}".format(
    c[0], c[1], c[2], c[3], int(c[4]), c[5], int(c[6]), int(c[8] is not None)))
def test_backward_small(case):
    B, S, H, D, causal, kind, bidi, scale, rope = case
    inp = synth.draw_dense(300 + S, B, S, H, D)
    out, kw = run_dense_bwd(inp, causal=causal, kind=kind, scale=scale, bidirectional=bidi,
                            rope_base=rope)
    dq, dk, dv, dtab = oracle.attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"),
                                            inp.f64("do"), **kw)
    assert_grad(out["dq"], dq, "dQ")
    assert_grad(out["dk"], dk, "dK")
    assert_grad(out["dv"], dv, "dV")
    if dtab is not None:
        assert_dtable(out["dtable"], dtab)
        # sum over buckets of a head's gradient is zero (rows of dS sum to zero)
        assert np.abs(out["dtable"].sum(axis=0)).max() <= 1e-3 * np.abs(dtab).max() + 1e-4
    if rope is not None:
        # the exact rotation, without the reading's bf16 rounding of the
        # rotated q and k: the same gates
        g = oracle.attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do"),
                                 **dict(kw, rope_round=False))
        errs = {}
        for name, rd, ex in zip(("dq", "dk", "dv"), (dq, dk, dv), g[:3]):
            errs[name + "_kernel"], errs[name + "_reading"] = check_exact_rotation(
                out[name], rd, ex, name, scale, D, assert_grad)
        log_margin(f"backward small {case} vs exact rotation", **errs)


GEOMS = [
    # B, S, H, D, causal, bidirectional, num_buckets, max_distance
    (1, 300, 2, 64, False, True, 8, 16),
    (1, 300, 2, 64, True, False, 8, 16),
    (1, 260, 1, 128, True, True, 6, 10),
    (1, 1100, 1, 64, False, True, 32, 1024),
    (1, 1100, 1, 64, True, False, 32, 1024),
    (1, 400, 2, 128, False, False, 17, 300),
]


@pytest.mark.parametrize("case", GEOMS, ids=lambda c: "s{}d{}-c{}-bi{}-nb{}-md{}".format(
    c[1], c[3], int(c[4]), int(c[5]), c[6], c[7]))
def test_backward_t5_geometries(case):
    """Short and long saturation distances and odd bucket counts (the bias
    table's clamped per-lane base and the table-gradient bins)."""
    B, S, H, D, causal, bidi, nb, md = case
    inp = synth.draw_dense(11 * S + nb, B, S, H, D, num_buckets=nb)
    out, kw = run_dense_bwd(inp, causal=causal, kind="t5", scale=1.0, bidirectional=bidi,
                            nb=nb, md=md)
    dq, dk, dv, dtab = oracle.attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"),
                                            inp.f64("do"), **kw)
    assert_grad(out["dq"], dq, "dQ")
    assert_grad(out["dk"], dk, "dK")
    assert_grad(out["dv"], dv, "dV")
    assert_dtable(out["dtable"], dtab)


def test_backward_o_only_centres():
    """The backward reads O only as the centre dO.O of its D accumulation.
    With another O, dK, dV and the table gradient still meet the gate (D
    itself is summed in fp32 from the recomputed P); dQ keeps a bounded
    error (its B = sum P k enters as bf16 and is multiplied by D - dO.O, no
    longer small); a non-finite centre is replaced by 0, bit for bit."""
    inp = synth.draw_dense(77, 1, 300, 2, 64)
    ref = oracle.attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do"),
                               **oracle_kwargs("t5", True, 1.0, inp.table, None, 32, 128, False))
    runs = {}
    for kind, alter in (("zero", torch.zeros_like),
                        ("nan", lambda o: torch.full_like(o, float("nan"))),
                        ("scaled", lambda o: (o.float() * 1.25).to(o.dtype))):
        out, _ = run_dense_bwd(inp, causal=True, kind="t5", scale=1.0, bidirectional=False,
                               o_for_bwd=alter)
        runs[kind] = out
        dq, dk, dv, dtab = ref
        assert_grad(out["dk"], dk, f"dK ({kind} O)")
        assert_grad(out["dv"], dv, f"dV ({kind} O)")
        assert_dtable(out["dtable"], dtab, f"dtable ({kind} O)")
        assert np.isfinite(out["dq"]).all()
        assert norm_err(out["dq"], dq)[0] <= 0.25, f"dQ ({kind} O)"
    for name in ("dq", "dk", "dv", "dtable"):
        assert np.array_equal(runs["nan"][name], runs["zero"][name]), name


def run_varlen_bwd(inp, H, *, causal, scale, kind="t5", bidirectional=True, rope_base=None):
    q, k, v, do = (bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    T = q.shape[0]
    cu = torch.from_numpy(inp.cu_seqlens).cuda()
    bias, slopes = _bias(kind, H, inp.table, 32, 128, bidirectional)
    o = nan_like(q)
    lse = torch.full((H, T), float("nan"), device="cuda")
    mx = int(inp.lengths.max())
    fa.fa_varlen_fwd(q, k, v, o, lse, cu, mx, scale=scale, causal=causal, bias=bias,
                     rope_base=rope_base or 0.0)
    dq, dk, dv = nan_like(q), nan_like(q), nan_like(q)
    dtable = torch.full((32, H), float("nan"), device="cuda") if kind == "t5" else None
    fa.fa_varlen_bwd(q, k, v, o, lse, do, dq, dk, dv, cu, mx, dtable, scale=scale,
                     causal=causal, bias=bias, rope_base=rope_base or 0.0)
    torch.cuda.synchronize()
    kw = oracle_kwargs(kind, causal, scale, inp.table, slopes, 32, 128, bidirectional, rope_base)
    return dict(dq=to_f64(dq), dk=to_f64(dk), dv=to_f64(dv),
                dtable=None if dtable is None else dtable.cpu().numpy().astype(np.float64)), kw


@pytest.mark.parametrize("causal,kind,rope", [(False, "t5", None), (True, "t5", None),
                                              (True, "alibi", None), (False, "none", 1000.0)])
def test_varlen_backward_small(causal, kind, rope):
    lengths = np.array([1, 130, 17, 256, 64, 300, 5])
    inp = synth.draw_varlen(31, int(lengths.sum()), 3, 64, lengths=lengths)
    out, kw = run_varlen_bwd(inp, 3, causal=causal, scale=1.0 if kind == "t5" else 0.25,
                             kind=kind, bidirectional=not causal, rope_base=rope)
    dq, dk, dv, dtab = oracle.varlen_attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"),
                                                   inp.f64("do"), inp.cu_seqlens, **kw)
    assert_grad(out["dq"], dq, "dQ")
    assert_grad(out["dk"], dk, "dK")
    assert_grad(out["dv"], dv, "dV")
    if dtab is not None:
        assert_dtable(out["dtable"], dtab)


@pytest.mark.parametrize("causal,kind,rope", [(True, "alibi", None), (False, "none", 10000.0),
                                              (True, "t5", None)])
def test_varlen_backward_head_dim_128(causal, kind, rope):
    """Packed sequences at head_dim 128 (32-key dq tiles, V rows in LDS for
    the dkv kernel without a T5 bias)."""
    lengths = np.array([1, 130, 300, 64, 257, 33])
    inp = synth.draw_varlen(41, int(lengths.sum()), 2, 128, lengths=lengths)
    out, kw = run_varlen_bwd(inp, 2, causal=causal, scale=128 ** -0.5, kind=kind,
                             bidirectional=not causal, rope_base=rope)
    dq, dk, dv, dtab = oracle.varlen_attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"),
                                                   inp.f64("do"), inp.cu_seqlens, **kw)
    assert_grad(out["dq"], dq, "dQ")
    assert_grad(out["dk"], dk, "dK")
    assert_grad(out["dv"], dv, "dV")
    if dtab is not None:
        assert_dtable(out["dtable"], dtab)


@pytest.mark.parametrize("nseq", [2048, 2100])
def test_varlen_many_sequences(nseq):
    """Thousands of short sequences and a few long ones, three heads: the
    schedule ranks sequences by length up to 2048 of them and keeps index
    order beyond; both must cover every (sequence, head, tile) once."""
    rng = np.random.default_rng(nseq)
    lengths = rng.integers(1, 25, size=nseq)
    lengths[[5, nseq // 2, nseq - 1]] = [300, 129, 200]
    inp = synth.draw_varlen(nseq, int(lengths.sum()), 3, 64, lengths=lengths)
    out, kw = run_varlen_bwd(inp, 3, causal=True, scale=1.0, kind="t5", bidirectional=False)
    dq, dk, dv, dtab = oracle.varlen_attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"),
                                                   inp.f64("do"), inp.cu_seqlens, **kw)
    assert_grad(out["dq"], dq, "dQ")
    assert_grad(out["dk"], dk, "dK")
    assert_grad(out["dv"], dv, "dV")
    assert_dtable(out["dtable"], dtab)


def test_backward_deterministic():
    """No atomics anywhere: two runs give the same bits for every output."""
    inp = synth.draw_dense(77, 2, 300, 2, 64)
    a, _ = run_dense_bwd(inp, causal=True, kind="t5", scale=1.0, bidirectional=False)
    b, _ = run_dense_bwd(inp, causal=True, kind="t5", scale=1.0, bidirectional=False)
    for name in ("o", "dq", "dk", "dv", "dtable"):
        np.testing.assert_array_equal(a[name], b[name])


def test_dtable_optional_and_empty_problem():
    inp = synth.draw_dense(78, 1, 150, 2, 64)
    a, kw = run_dense_bwd(inp, causal=False, kind="t5", scale=1.0, want_dtable=False)
    assert a["dtable"] is None
    dq, dk, dv, _ = oracle.attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"),
                                         inp.f64("do"), **kw)
    assert_grad(a["dk"], dk, "dK")
    # an empty batch still overwrites the table gradient (with zeros)
    q = torch.empty((0, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((0, 2, 16), device="cuda")
    dtable = torch.full((32, 2), 5.0, device="cuda")
    bias = fa.T5Bias(torch.zeros(32, 2, device="cuda"), 32, 128, True)
    fa.fa_bwd(q, q, q, q, lse, q, q, q, q, dtable, bias=bias)
    torch.cuda.synchronize()
    assert float(dtable.abs().max()) == 0.0


def test_autograd_wrapper_matches_oracle():
    inp = synth.draw_dense(79, 1, 170, 2, 64)
    q, k, v, do = (bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    q.requires_grad_(True)
    k.requires_grad_(True)
    v.requires_grad_(True)
    table = torch.from_numpy(inp.table).cuda().requires_grad_(True)
    o = fa.attention(q, k, v, bias=fa.T5Bias(table, 32, 128, False), causal=True, scale=1.0)
    o.backward(do)
    torch.cuda.synchronize()
    kw = oracle_kwargs("t5", True, 1.0, inp.table, None, 32, 128, False, None)
    O, _ = oracle.attention_fwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), **kw)
    dq, dk, dv, dtab = oracle.attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"),
                                            inp.f64("do"), **kw)
    assert_o(to_f64(o), O)
    assert_grad(to_f64(q.grad), dq, "dQ")
    assert_grad(to_f64(k.grad), dk, "dK")
    assert_grad(to_f64(v.grad), dv, "dV")
    assert_dtable(table.grad.cpu().numpy().astype(np.float64), dtab)


@pytest.mark.parametrize("causal", [True, False])
def test_lse_gradient(causal):
    """A loss that uses the returned LSE: dlse adds dlse_i P_ij to dS_ij, in
    dQ, dK and the table gradient (dV does not depend on it)."""
    inp = synth.draw_dense(81, 2, 300, 3, 64)
    q, k, v, do = (bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    B, S, H, D = q.shape
    bias = fa.T5Bias(torch.from_numpy(inp.table).cuda(), 32, 128, not causal)
    o, lse = nan_like(q), torch.full((B, H, S), float("nan"), device="cuda")
    fa.fa_fwd(q, k, v, o, lse, causal=causal, bias=bias)
    dlse = torch.from_numpy(np.random.default_rng(5).standard_normal((B, H, S)).astype(
        np.float32)).cuda()
    dq, dk, dv = nan_like(q), nan_like(q), nan_like(q)
    dtable = torch.full((32, H), float("nan"), device="cuda")
    fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, dtable, dlse=dlse, causal=causal, bias=bias)
    torch.cuda.synchronize()
    kw = oracle_kwargs("t5", causal, 1.0, inp.table, None, 32, 128, not causal, None)
    g = oracle.attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do"),
                             dlse=dlse.cpu().numpy().astype(np.float64), **kw)
    for name, got, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), g[:3]):
        assert_grad(to_f64(got), ref, name)
    assert_dtable(dtable.cpu().numpy().astype(np.float64), g[3])


def test_lse_gradient_packed_and_autograd():
    """The packed backward with dlse, and the autograd wrapper with a loss
    that uses both outputs."""
    lengths = np.array([1, 130, 17, 256, 64])
    inp = synth.draw_varlen(83, int(lengths.sum()), 2, 64, lengths=lengths)
    q, k, v, do = (bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    T, H = q.shape[:2]
    cu = torch.from_numpy(inp.cu_seqlens).cuda()
    table = torch.from_numpy(inp.table).cuda()
    rng = np.random.default_rng(6)
    dlse = torch.from_numpy(rng.standard_normal((H, T)).astype(np.float32)).cuda()
    for t in (q, k, v):
        t.requires_grad_(True)
    table.requires_grad_(True)
    o, lse = fa.varlen_attention(q, k, v, cu, int(lengths.max()),
                                 bias=fa.T5Bias(table, 32, 128, True), return_lse=True)
    ((o.float() * do.float()).sum() + (lse * dlse).sum()).backward()
    torch.cuda.synchronize()
    kw = oracle_kwargs("t5", False, 1.0, inp.table, None, 32, 128, True, None)
    g = oracle.varlen_attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do"),
                                    inp.cu_seqlens, dlse=dlse.cpu().numpy().astype(np.float64),
                                    **kw)
    for name, got, ref in zip(("dQ", "dK", "dV"), (q.grad, k.grad, v.grad), g[:3]):
        assert_grad(to_f64(got), ref, name)
    assert_dtable(table.grad.cpu().numpy().astype(np.float64), g[3])
    # a loss of the LSE alone: dO is zero
    for t in (q, k, v, table):
        t.grad = None
    o, lse = fa.varlen_attention(q, k, v, cu, int(lengths.max()),
                                 bias=fa.T5Bias(table, 32, 128, True), return_lse=True)
    (lse * dlse).sum().backward()
    torch.cuda.synchronize()
    g = oracle.varlen_attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"),
                                    np.zeros_like(inp.f64("do")), inp.cu_seqlens,
                                    dlse=dlse.cpu().numpy().astype(np.float64), **kw)
    for name, got, ref in zip(("dQ", "dK"), (q.grad, k.grad), g[:2]):
        assert_grad(to_f64(got), ref, name + " (LSE loss only)")
    assert float(v.grad.abs().max()) == 0.0
