"""Dense bias matrix (the report's first kernel) on the GPU: O, LSE, dQ, dK,
dV and dL/dB from the HIP path (through the C ABI) against the fp64 oracle on
identical seeded inputs, and against the T5 mode with the T5 bias
materialised as a matrix."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (assert_dtable, assert_grad, assert_lse, assert_o, bf16_tensor, norm_err,
                     oracle_kwargs, to_f64)

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("attention_t5_relative_amd")

# dL/dB is written in fp32 (no bf16 rounding of the output): the error is
# that of fp32 P and dP, far below the bf16 gradient gate.
DBIAS_MAX, DBIAS_MEAN = 1e-3, 1e-5


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def run_dense(inp, dense_bits, *, causal, scale, rope_base=None, want_grad=True):
    q, k, v, do = (bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    B, S, H, D = q.shape
    bias = fa.DenseBias(bf16_tensor(dense_bits))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, scale=scale, causal=causal, bias=bias, rope_base=rope_base or 0.0)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dbias = (torch.full(dense_bits.shape, float("nan"), device="cuda") if want_grad else None)
    fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, dbias, scale=scale, causal=causal, bias=bias,
              rope_base=rope_base or 0.0)
    torch.cuda.synchronize()
    out = dict(o=to_f64(o), lse=lse.cpu().numpy().astype(np.float64), dq=to_f64(dq),
               dk=to_f64(dk), dv=to_f64(dv),
               dbias=None if dbias is None else dbias.cpu().numpy().astype(np.float64))
    kw = dict(scale=scale, causal=causal, bias="dense",
              dense=synth.bf16_bits_to_f32(dense_bits).astype(np.float64), rope_base=rope_base)
    return out, kw


def assert_dbias(got, ref, what="dbias"):
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    mx, mean = norm_err(got, ref)
    assert mx <= DBIAS_MAX and mean <= DBIAS_MEAN, f"{what}: normalised max {mx:.3e} mean {mean:.3e}"


CASES = [
    # B, S, H, D, causal, Bb, scale, rope
    (1, 37, 2, 64, False, 1, 1.0, None),
    (2, 200, 2, 64, True, 1, 1.0, None),      # shared matrix, B > 1: per-batch sum
    (2, 130, 2, 128, False, 2, 0.125, None),
    (2, 257, 3, 64, True, 2, 0.5, None),
    (1, 129, 2, 128, True, 1, 0.2, None),
    (3, 100, 1, 64, False, 1, 1.0, None),
    (1, 160, 2, 64, True, 1, 0.3, 10000.0),   # with RoPE
    (2, 150, 2, 64, True, 1, 0.3, 10000.0),   # RoPE and the batch sum of a shared matrix
    # the batch-sum kernel at head_dim 128 (64-row tiles, two per 128-row
    # super tile; a ragged last one), odd and even batch counts
    (3, 200, 2, 128, True, 1, 0.125, None),
    (2, 150, 2, 128, False, 1, 0.25, None),
    (5, 131, 1, 64, True, 1, 0.5, None),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}s{}h{}d{}-c{}-bb{}-r{}".format(
    c[0], c[1], c[2], c[3], int(c[4]), c[5], int(c[7] is not None)))
def test_dense_bias_small(case):
    B, S, H, D, causal, Bb, scale, rope = case
    inp = synth.draw_dense(500 + S, B, S, H, D, with_table=False)
    dense = synth.draw_dense_bias(600 + S, Bb, H, S)
    out, kw = run_dense(inp, dense, causal=causal, scale=scale, rope_base=rope)
    O, LSE = oracle.attention_fwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), **kw)
    assert_o(out["o"], O)
    assert_lse(out["lse"], LSE)
    dq, dk, dv, dbias = oracle.attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"),
                                             inp.f64("do"), **kw)
    assert_grad(out["dq"], dq, "dQ")
    assert_grad(out["dk"], dk, "dK")
    assert_grad(out["dv"], dv, "dV")
    assert_dbias(out["dbias"], dbias)
    if causal:   # masked pairs carry no gradient
        upper = np.triu(np.ones((S, S), dtype=bool), 1)
        assert (out["dbias"][:, :, upper] == 0).all()


@pytest.mark.parametrize("causal,bidir", [(False, True), (True, False)])
def test_dense_bias_matches_t5_mode(causal, bidir):
    """The T5 bias materialised as a bf16 matrix (table values exactly
    representable in bf16) gives the T5 mode's results, and dL/dB summed over
    each bucket's pairs gives its table gradient."""
    B, S, H, D, nb, md = 2, 300, 2, 64, 32, 128
    inp = synth.draw_dense(71, B, S, H, D)
    table = synth.bf16_bits_to_f32(synth.bf16_round(inp.table)).astype(np.float32)
    buckets = torch.empty((S, S), dtype=torch.int32, device="cuda")
    fa.fa_t5_buckets(S, S, nb, md, bidir, buckets)
    bk = buckets.cpu().numpy()
    dense = synth.bf16_round(table[bk].transpose(2, 0, 1)[None])   # exact: values are bf16
    out_d, _ = run_dense(inp, dense, causal=causal, scale=1.0)

    q, k, v, do = (bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    t5 = fa.T5Bias(torch.from_numpy(table).cuda(), nb, md, bidir)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, scale=1.0, causal=causal, bias=t5)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dtab = torch.empty((nb, H), device="cuda")
    fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, dtab, scale=1.0, causal=causal, bias=t5)
    torch.cuda.synchronize()
    assert_o(out_d["o"], to_f64(o), "O dense vs T5")
    assert_lse(out_d["lse"], lse.cpu().numpy().astype(np.float64), "LSE dense vs T5")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_grad(out_d[name], to_f64(t), f"{name} dense vs T5")
    per_bucket = np.stack([np.bincount(bk.ravel(), weights=out_d["dbias"][0, h].ravel(),
                                       minlength=nb) for h in range(H)], axis=1)
    assert_dtable(per_bucket, dtab.cpu().numpy().astype(np.float64), "dbias by bucket vs dtable")


def test_dense_bias_empty_batch_zeroes_shared_gradient():
    S, H, D = 16, 2, 64
    q = torch.empty((0, S, H, D), dtype=torch.bfloat16, device="cuda")
    bias = fa.DenseBias(torch.zeros((1, H, S, S), dtype=torch.bfloat16, device="cuda"))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((0, H, S), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, q, q, o, lse, bias=bias)
    dbias = torch.full((1, H, S, S), float("nan"), device="cuda")
    fa.fa_bwd(q, q, q, o, lse, q, dq, dk, dv, dbias, bias=bias)
    torch.cuda.synchronize()
    assert (dbias == 0).all()


def test_dense_bias_full_size_sampled_head():
    """The causal decoder workload's shape (B8 H12 S4096 D64) with one shared
    dense bias per head; the oracle computes every batch of head 3 (dL/dB of
    a shared matrix sums over the batch)."""
    c = synth.config_by_name("c3")
    inp = synth.draw_dense(c.seed, c.batch, c.seqlen, c.heads, c.head_dim, with_table=False)
    dense = synth.draw_dense_bias(c.seed + 100, 1, c.heads, c.seqlen)
    out, kw = run_dense(inp, dense, causal=True, scale=c.scale)
    h = 3
    pairs = [(b, h) for b in range(c.batch)]
    O, LSE = oracle.attention_fwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), pairs=pairs, **kw)
    assert_o(out["o"][:, :, h], O[:, :, h], "O[:,:,3]")
    dq, dk, dv, dbias = oracle.attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"),
                                             inp.f64("do"), pairs=pairs, **kw)
    assert_grad(out["dq"][:, :, h], dq[:, :, h], "dQ[:,:,3]")
    assert_grad(out["dk"][:, :, h], dk[:, :, h], "dK[:,:,3]")
    assert_grad(out["dv"][:, :, h], dv[:, :, h], "dV[:,:,3]")
    assert_dbias(out["dbias"][0, h], dbias[0, h], "dbias[0,3]")


@pytest.mark.parametrize("D", [64, 128])
def test_dense_bias_shared_gradient_deterministic(D):
    """The batch sum of a shared matrix's gradient runs in one fixed order:
    two backward calls give the same bits."""
    B, S, H = 4, 300, 2
    inp = synth.draw_dense(900 + D, B, S, H, D, with_table=False)
    dense = synth.draw_dense_bias(901 + D, 1, H, S)
    q, k, v, do = (bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    bias = fa.DenseBias(bf16_tensor(dense))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, o, lse, scale=0.125, causal=True, bias=bias)
    runs = []
    for _ in range(2):
        g = [torch.empty_like(q) for _ in range(3)]
        db = torch.full(dense.shape, float("nan"), device="cuda")
        fa.fa_bwd(q, k, v, o, lse, do, *g, db, scale=0.125, causal=True, bias=bias)
        runs.append(g + [db])
    torch.cuda.synchronize()
    assert torch.isfinite(runs[0][3]).all()
    for a, b in zip(*runs):
        assert torch.equal(a, b)
