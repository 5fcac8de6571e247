"""Forward parity on the GPU: the HIP path (through the C ABI) against the
fp64 oracle on identical seeded bf16 inputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (assert_lse, assert_o, bf16_tensor, check_exact_rotation, log_margin,
                     nan_like, oracle_kwargs, to_f64)

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("attention_t5_relative_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _bias_objs(kind, H, table, nb, md, bidirectional):
    if kind == "t5":
        return fa.T5Bias(torch.from_numpy(table).cuda(), nb, md, bidirectional), None
    if kind == "alibi":
        s = synth.alibi_slope_values(H)
        return fa.ALiBi(torch.from_numpy(s).cuda()), s.astype(np.float64)
    return None, None


def run_dense(inp, *, causal, kind, scale, bidirectional=True, nb=32, md=128, rope_base=None):
    q, k, v = (bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v"))
    B, S, H, D = q.shape
    bias, slopes = _bias_objs(kind, H, inp.table, nb, md, bidirectional)
    o = nan_like(q)
    lse = torch.full((B, H, S), float("nan"), device="cuda")
    fa.fa_fwd(q, k, v, o, lse, scale=scale, causal=causal, bias=bias,
              rope_base=rope_base or 0.0)
    torch.cuda.synchronize()
    kw = oracle_kwargs(kind, causal, scale, inp.table, slopes, nb, md, bidirectional, rope_base)
    return to_f64(o), lse.cpu().numpy().astype(np.float64), kw


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
    # B*H a multiple of 8: the grouped tile order (two and six pairs per group)
    (2, 300, 8, 64, True, "t5", False, 1.0, None),
    (4, 200, 12, 64, False, "t5", True, 1.0, None),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "b{}s{}h{}d{}-c{}-{}-bi{}-r{}".format(
    c[0], c[1], c[2], c[3], int(c[4]), c[5], int(c[6]), int(c[8] is not None)))
def test_forward_small(case):
    B, S, H, D, causal, kind, bidi, scale, rope = case
    inp = synth.draw_dense(100 + S, B, S, H, D, with_dout=False)
    o, lse, kw = run_dense(inp, causal=causal, kind=kind, scale=scale, bidirectional=bidi,
                           rope_base=rope)
    q64, k64 = inp.f64("q"), inp.f64("k")
    O, LSE = oracle.attention_fwd(q64, k64, inp.f64("v"), **kw)
    assert_o(o, O)
    assert_lse(lse, LSE)
    if rope is not None:
        # the exact rotation, without the reading's bf16 rounding of the
        # rotated q and k: the same gates
        O2, _ = oracle.attention_fwd(q64, k64, inp.f64("v"), **dict(kw, rope_round=False))
        e_k, e_r = check_exact_rotation(o, O, O2, "O", scale, D, assert_o)
        log_margin(f"forward small {case} vs exact rotation", o_kernel=e_k, o_reading=e_r)


# Other T5 geometries: a short saturation distance (most tiles saturated,
# the per-lane table base clamped on both sides), the largest one the
# kernels take, and an odd bucket count; causal and not, both head sizes.
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
def test_forward_t5_geometries(case):
    B, S, H, D, causal, bidi, nb, md = case
    inp = synth.draw_dense(7 * S + nb, B, S, H, D, num_buckets=nb, with_dout=False)
    o, lse, kw = run_dense(inp, causal=causal, kind="t5", scale=1.0, bidirectional=bidi,
                           nb=nb, md=md)
    O, LSE = oracle.attention_fwd(inp.f64("q"), inp.f64("k"), inp.f64("v"), **kw)
    assert_o(o, O)
    assert_lse(lse, LSE)


def _run_varlen(inp, H, D, *, causal, scale, kind="t5", bidirectional=True, rope_base=None):
    q, k, v = (bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v"))
    T = q.shape[0]
    cu = torch.from_numpy(inp.cu_seqlens).cuda()
    bias, slopes = _bias_objs(kind, H, inp.table, 32, 128, bidirectional)
    o = nan_like(q)
    lse = torch.full((H, T), float("nan"), device="cuda")
    fa.fa_varlen_fwd(q, k, v, o, lse, cu, int(inp.lengths.max()), scale=scale, causal=causal,
                     bias=bias, rope_base=rope_base or 0.0)
    torch.cuda.synchronize()
    kw = oracle_kwargs(kind, causal, scale, inp.table, slopes, 32, 128, bidirectional, rope_base)
    return to_f64(o), lse.cpu().numpy().astype(np.float64), kw


@pytest.mark.parametrize("causal,kind,rope", [(False, "t5", None), (True, "t5", None),
                                              (True, "alibi", None), (False, "none", 1000.0)])
def test_varlen_forward_small(causal, kind, rope):
    lengths = np.array([1, 130, 17, 256, 64, 300, 5])
    inp = synth.draw_varlen(21, int(lengths.sum()), 3, 64, lengths=lengths, with_dout=False)
    o, lse, kw = _run_varlen(inp, 3, 64, causal=causal, scale=1.0 if kind == "t5" else 0.25,
                             kind=kind, bidirectional=not causal, rope_base=rope)
    q64, k64 = inp.f64("q"), inp.f64("k")
    O, LSE = oracle.varlen_attention_fwd(q64, k64, inp.f64("v"), inp.cu_seqlens, **kw)
    assert_o(o, O)
    assert_lse(lse, LSE)
    # a length-1 sequence returns its own v, bit for bit
    np.testing.assert_array_equal(o[0], inp.f64("v")[0])


def test_varlen_isolation_bit_exact():
    lengths = np.array([70, 200, 33, 129])
    inp = synth.draw_varlen(5, int(lengths.sum()), 2, 64, lengths=lengths, with_dout=False)
    o1, _, _ = _run_varlen(inp, 2, 64, causal=False, scale=1.0)
    a, e = 70, 270
    k2, v2 = inp.k.copy(), inp.v.copy()
    rng = np.random.default_rng(0)
    k2[a:e] = synth.bf16_round(rng.standard_normal(k2[a:e].shape, dtype=np.float32))
    v2[a:e] = synth.bf16_round(rng.standard_normal(v2[a:e].shape, dtype=np.float32))
    inp.k, inp.v = k2, v2
    o2, _, _ = _run_varlen(inp, 2, 64, causal=False, scale=1.0)
    np.testing.assert_array_equal(o2[:a], o1[:a])
    np.testing.assert_array_equal(o2[e:], o1[e:])
    assert not np.array_equal(o2[a:e], o1[a:e])


def test_causal_first_row_is_v0_and_deterministic():
    inp = synth.draw_dense(9, 2, 300, 3, 64, with_dout=False)
    o1, lse1, _ = run_dense(inp, causal=True, kind="t5", scale=1.0, bidirectional=False)
    np.testing.assert_array_equal(o1[:, 0], inp.f64("v")[:, 0])
    o2, lse2, _ = run_dense(inp, causal=True, kind="t5", scale=1.0, bidirectional=False)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(lse1, lse2)


@pytest.mark.parametrize("nb,md,bidi", [(32, 128, True), (32, 128, False), (16, 64, True),
                                        (64, 512, False), (8, 20, True), (256, 1024, False)])
def test_t5_buckets_bit_exact(nb, md, bidi):
    n = 4096 if (nb, md) == (32, 128) else 1500
    out = torch.empty((n, n), dtype=torch.int32, device="cuda")
    fa.fa_t5_buckets(n, n, nb, md, bidi, out)
    torch.cuda.synchronize()
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.t5_bucket(j - i, nb, md, bidi))


def test_empty_inputs_are_no_ops():
    q = torch.empty((0, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((0, 2, 16), dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, q, q, torch.empty_like(q), lse)
    q = torch.empty((2, 0, 2, 64), dtype=torch.bfloat16, device="cuda")
    fa.fa_fwd(q, q, q, torch.empty_like(q), torch.empty((2, 2, 0), device="cuda"))
    torch.cuda.synchronize()
