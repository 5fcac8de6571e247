"""Pins for the fp64 oracle: each check compares it with something other than
itself (brute force in pure Python, exact integer arithmetic, a closed form,
a library routine, finite differences, or an invariant of the mathematics).

The pages print no worked example and no output values, so no pin comes from
stored numbers of the pages (tests/golden/README.md says so).
"""
import cmath
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.attention import head_bwd, head_fwd

# ---------------------------------------------------------------------------
# T5 buckets
# ---------------------------------------------------------------------------


def bucket_exact(rel: int, nb: int, md: int, bidirectional: bool) -> int:
    """T5 bucket decided by exact integer comparisons (no logarithm).

    For n >= me the bucket is me + k for the largest k < nb'-me with
    (n/me)^(nb'-me) >= (md/me)^k, i.e. n^L * me^k >= md^k * me^L, L = nb'-me;
    capped at nb'-1.
    """
    if bidirectional:
        nbp = nb // 2
        off = nbp if rel > 0 else 0
        n = abs(rel)
    else:
        nbp = nb
        off = 0
        n = max(-rel, 0)
    me = nbp // 2
    if n < me:
        return off + n
    L = nbp - me
    k = 0
    while k + 1 <= L and n ** L * me ** (k + 1) >= md ** (k + 1) * me ** L:
        k += 1
    return off + min(me + k, nbp - 1)


@pytest.mark.parametrize("nb,md", [(32, 128), (16, 64), (64, 256), (32, 512), (8, 20)])
@pytest.mark.parametrize("bidirectional", [True, False])
def test_t5_bucket_matches_exact_integer_evaluation(nb, md, bidirectional):
    rel = np.arange(-20000, 20000)
    got = oracle.t5_bucket(rel, nb, md, bidirectional)
    # the exact evaluation only depends on n and the side; tabulate it once
    want = np.empty_like(got)
    cache = {}
    for idx, r in enumerate(rel):
        key = (int(r) > 0, abs(int(r))) if bidirectional else max(-int(r), 0)
        if key not in cache:
            cache[key] = bucket_exact(int(r), nb, md, bidirectional)
        want[idx] = cache[key]
    np.testing.assert_array_equal(got, want)


# Threshold tables for 32 buckets, max distance 128: the first n of each
# bucket past the exact range, worked out by hand from the T5 formula with
# exact comparisons (e.g. bidirectional bucket 10 starts at n = 16 where
# ln(16/8)/ln(128/8)*8 = 2 exactly).
BIDIR_FIRST_N = {8: 8, 9: 12, 10: 16, 11: 23, 12: 32, 13: 46, 14: 64, 15: 91}
UNIDIR_FIRST_N = {16: 16, 17: 19, 18: 21, 19: 24, 20: 27, 21: 31, 22: 35, 23: 40, 24: 46,
                  25: 52, 26: 59, 27: 67, 28: 77, 29: 87, 30: 99, 31: 113}


def test_t5_bucket_closed_form_tables_32_128():
    n = np.arange(0, 5000)
    lo_side = oracle.t5_bucket(-n, 32, 128, True)      # key before the query
    hi_side = oracle.t5_bucket(n, 32, 128, True)       # key after the query
    uni = oracle.t5_bucket(-n, 32, 128, False)
    for t in range(8):
        assert lo_side[t] == t
    for b, first in BIDIR_FIRST_N.items():
        assert lo_side[first] == b and lo_side[first - 1] == b - 1
    assert np.all(lo_side[91:] == 15)
    # symmetry: the upper half mirrors the lower half, offset by 16 (n > 0)
    np.testing.assert_array_equal(hi_side[1:], lo_side[1:] + 16)
    assert hi_side[0] == 0
    for t in range(16):
        assert uni[t] == t
    for b, first in UNIDIR_FIRST_N.items():
        assert uni[first] == b and uni[first - 1] == b - 1
    assert np.all(uni[113:] == 31)
    # unidirectional: every key after the query maps to bucket 0
    assert np.all(oracle.t5_bucket(np.arange(1, 100), 32, 128, False) == 0)


# ---------------------------------------------------------------------------
# ALiBi, RoPE, bf16 rounding
# ---------------------------------------------------------------------------


def nearest_bf16(x: float) -> float:
    """Nearest bfloat16 value by brute force over the two candidates that
    bracket x (8 significant bits), ties to the even significand."""
    if x == 0.0:
        return 0.0
    e = math.floor(math.log2(abs(x)))
    # make sure 2^e <= |x| < 2^(e+1) despite log2 rounding
    while 2.0 ** e > abs(x):
        e -= 1
    while 2.0 ** (e + 1) <= abs(x):
        e += 1
    ulp = 2.0 ** (e - 7)
    lo = math.floor(abs(x) / ulp) * ulp
    hi = lo + ulp
    dlo, dhi = abs(x) - lo, hi - abs(x)
    if dlo < dhi or (dlo == dhi and int(round(lo / ulp)) % 2 == 0):
        r = lo
    else:
        r = hi
    return math.copysign(r, x)


def test_bf16_round_exact_matches_brute_force():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(20000) * 3.0,
                        # exact ties between neighbours: odd multiples of half an ulp
                        (np.arange(1, 2001) * 2 + 1) * 2.0 ** -9 + 1.0,
                        -(np.arange(1, 2001) * 2 + 1) * 2.0 ** -9 - 2.0])
    got = oracle.bf16_round_exact(x)
    want = np.array([nearest_bf16(float(v)) for v in x])
    np.testing.assert_array_equal(got, want)
    # fp32 inputs that are already bf16 values are unchanged
    b = synth.bf16_bits_to_f32(synth.bf16_round(rng.standard_normal(1000).astype(np.float32)))
    np.testing.assert_array_equal(oracle.bf16_round_exact(b.astype(np.float64)), b)


def test_alibi_slopes_closed_form():
    # for 8 heads the ALiBi paper's sequence is 1/2, 1/4, ..., 1/256
    np.testing.assert_array_equal(oracle.alibi_slopes(8), [2.0 ** -(i + 1) for i in range(8)])
    # for 16 heads it is 2^-0.5, 2^-1, ..., 2^-8
    np.testing.assert_allclose(oracle.alibi_slopes(16), [2.0 ** (-(i + 1) / 2) for i in range(16)],
                               rtol=0, atol=1e-15)
    # the inputs the long-context config hands to both sides agree with it
    np.testing.assert_allclose(synth.alibi_slope_values(16), oracle.alibi_slopes(16), rtol=1e-7)


def test_rope_matches_complex_multiplication():
    rng = np.random.default_rng(0)
    D, S, base = 16, 40, 10000.0
    x = rng.standard_normal((S, D))
    pos = np.arange(S) + 3
    got = oracle.rope_rotate(x, pos, base)
    for t in range(S):
        for p in range(D // 2):
            z = complex(x[t, 2 * p], x[t, 2 * p + 1]) * cmath.exp(1j * pos[t] * base ** (-2 * p / D))
            assert abs(got[t, 2 * p] - z.real) < 1e-12 and abs(got[t, 2 * p + 1] - z.imag) < 1e-12


def test_rope_properties():
    rng = np.random.default_rng(1)
    D, S = 32, 50
    q = rng.standard_normal((S, D))
    k = rng.standard_normal((S, D))
    pos = np.arange(S)
    # position 0 is the identity
    np.testing.assert_allclose(oracle.rope_rotate(q[:1], [0], 1e4), q[:1], atol=0)
    # rotations keep norms
    np.testing.assert_allclose(np.linalg.norm(oracle.rope_rotate(q, pos, 1e4), axis=1),
                               np.linalg.norm(q, axis=1), rtol=1e-13)
    # scores depend only on relative position
    s0 = oracle.rope_rotate(q, pos, 1e4) @ oracle.rope_rotate(k, pos, 1e4).T
    s7 = oracle.rope_rotate(q, pos + 7, 1e4) @ oracle.rope_rotate(k, pos + 7, 1e4).T
    np.testing.assert_allclose(s0, s7, atol=1e-10)
    # unrotate inverts rotate
    np.testing.assert_allclose(oracle.rope_unrotate(oracle.rope_rotate(q, pos, 1e4), pos, 1e4), q,
                               atol=1e-13)


# ---------------------------------------------------------------------------
# Forward against brute force in pure Python
# ---------------------------------------------------------------------------


def brute_force_head(q, k, v, head, *, scale, causal, bias, table, nb, md, bidirectional,
                     slopes, rope_base):
    """O and LSE of one head with Python loops, math.fsum and math.exp."""
    S, D = len(q), len(q[0])

    def rot(x, t):
        if rope_base is None:
            return list(x)
        out = []
        for p in range(D // 2):
            z = complex(x[2 * p], x[2 * p + 1]) * cmath.exp(1j * t * rope_base ** (-2 * p / D))
            out += [nearest_bf16(z.real), nearest_bf16(z.imag)]
        return out

    qr = [rot(q[i], i) for i in range(S)]
    kr = [rot(k[j], j) for j in range(S)]
    O, LSE = [], []
    for i in range(S):
        scores = []
        for j in range(S):
            if causal and j > i:
                continue
            s = scale * math.fsum(qr[i][d] * kr[j][d] for d in range(D))
            if bias == "t5":
                s += float(table[bucket_exact(j - i, nb, md, bidirectional)][head])
            elif bias == "alibi":
                s += -float(slopes[head]) * abs(i - j)
            scores.append((j, s))
        m = max(s for _, s in scores)
        z = math.fsum(math.exp(s - m) for _, s in scores)
        LSE.append(m + math.log(z))
        O.append([math.fsum(math.exp(s - m) / z * v[j][d] for j, s in scores) for d in range(D)])
    return np.array(O), np.array(LSE)


CASES = [
    dict(bias="t5", causal=False, bidirectional=True, scale=1.0, rope_base=None),
    dict(bias="t5", causal=True, bidirectional=False, scale=1.0, rope_base=None),
    dict(bias="t5", causal=False, bidirectional=False, scale=0.5, rope_base=None),
    dict(bias="alibi", causal=True, bidirectional=False, scale=0.3, rope_base=None),
    dict(bias="alibi", causal=False, bidirectional=False, scale=0.3, rope_base=None),
    dict(bias="none", causal=True, bidirectional=False, scale=0.4, rope_base=100.0),
    dict(bias="none", causal=False, bidirectional=False, scale=1.0, rope_base=None),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c['bias']}-causal{int(c['causal'])}"
                         f"-bi{int(c['bidirectional'])}-rope{int(c['rope_base'] is not None)}")
def test_forward_matches_brute_force(case):
    rng = np.random.default_rng(7)
    S, D, H, nb, md = 11, 4, 3, 8, 20
    q = rng.standard_normal((S, D))
    k = rng.standard_normal((S, D))
    v = rng.standard_normal((S, D))
    table = rng.normal(0, 0.5, (nb, H))
    slopes = oracle.alibi_slopes(H)
    for head in range(H):
        kw = dict(scale=case["scale"], causal=case["causal"], bias=case["bias"], table=table,
                  num_buckets=nb, max_distance=md, bidirectional=case["bidirectional"],
                  slopes=slopes, rope_base=case["rope_base"])
        O, lse = head_fwd(q, k, v, head, **kw)
        Ob, lseb = brute_force_head(q.tolist(), k.tolist(), v.tolist(), head,
                                    scale=case["scale"], causal=case["causal"], bias=case["bias"],
                                    table=table, nb=nb, md=md,
                                    bidirectional=case["bidirectional"], slopes=slopes,
                                    rope_base=case["rope_base"])
        np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lseb, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Forward and backward against PyTorch's own attention and autograd (fp64 CPU)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("causal,bidirectional", [(False, True), (True, False)])
def test_against_torch_sdpa_and_autograd(causal, bidirectional):
    rng = np.random.default_rng(11)
    B, S, H, D, nb, md = 2, 37, 3, 8, 32, 128
    q, k, v, do = (rng.standard_normal((B, S, H, D)) for _ in range(4))
    table = rng.normal(0, 0.5, (nb, H))
    kw = dict(scale=0.7, causal=causal, bias="t5", table=table, num_buckets=nb, max_distance=md,
              bidirectional=bidirectional)
    O, LSE = oracle.attention_fwd(q, k, v, **kw)
    dq, dk, dv, dtab = oracle.attention_bwd(q, k, v, do, **kw)

    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), requires_grad=True) for x in (q, k, v))
    # the additive bias as a dense [H, S, S] matrix, with its own gradient
    buckets = torch.tensor(np.stack([[bucket_exact(int(jj - ii), nb, md, bidirectional)
                                      for jj in range(S)] for ii in range(S)]))
    ttab = torch.tensor(table, requires_grad=True)
    bias = ttab[buckets].permute(2, 0, 1)  # [H, S, S]
    mask = bias
    if causal:
        mask = bias.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
    tO = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask[None],
                                                          scale=0.7)
    np.testing.assert_allclose(tO.detach().numpy().transpose(0, 2, 1, 3), O, atol=1e-12)
    tO.backward(torch.tensor(do.transpose(0, 2, 1, 3)))
    np.testing.assert_allclose(tq.grad.numpy().transpose(0, 2, 1, 3), dq, atol=1e-11)
    np.testing.assert_allclose(tk.grad.numpy().transpose(0, 2, 1, 3), dk, atol=1e-11)
    np.testing.assert_allclose(tv.grad.numpy().transpose(0, 2, 1, 3), dv, atol=1e-11)
    np.testing.assert_allclose(ttab.grad.numpy(), dtab, atol=1e-11)
    # LSE from torch's logsumexp of the biased scores
    s = torch.einsum("bhid,bhjd->bhij", tq.detach(), tk.detach()) * 0.7 + mask.detach()[None]
    np.testing.assert_allclose(torch.logsumexp(s, -1).numpy(), LSE, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_lse_gradient_against_torch_autograd(causal):
    """A loss that uses both O and LSE: the oracle's dq, dk, dv and table
    gradient with dlse against torch's autograd of a plain fp64 statement
    (scores, logsumexp, softmax, P V) written here without SDPA."""
    rng = np.random.default_rng(19)
    B, S, H, D, nb, md = 2, 29, 2, 8, 16, 40
    q, k, v, do = (rng.standard_normal((B, S, H, D)) for _ in range(4))
    dlse = rng.standard_normal((B, H, S))
    table = rng.normal(0, 0.5, (nb, H))
    kw = dict(scale=0.8, causal=causal, bias="t5", table=table, num_buckets=nb, max_distance=md,
              bidirectional=not causal)
    dq, dk, dv, dtab = oracle.attention_bwd(q, k, v, do, dlse=dlse, **kw)
    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), requires_grad=True) for x in (q, k, v))
    buckets = torch.tensor(np.stack([[bucket_exact(int(jj - ii), nb, md, not causal)
                                      for jj in range(S)] for ii in range(S)]))
    ttab = torch.tensor(table, requires_grad=True)
    s = tq @ tk.transpose(-1, -2) * 0.8 + ttab[buckets].permute(2, 0, 1)[None]
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
    lse = torch.logsumexp(s, -1)
    o = torch.softmax(s, -1) @ tv
    loss = (o * torch.tensor(do.transpose(0, 2, 1, 3))).sum() + (lse * torch.tensor(dlse)).sum()
    loss.backward()
    np.testing.assert_allclose(tq.grad.numpy().transpose(0, 2, 1, 3), dq, atol=1e-11)
    np.testing.assert_allclose(tk.grad.numpy().transpose(0, 2, 1, 3), dk, atol=1e-11)
    np.testing.assert_allclose(tv.grad.numpy().transpose(0, 2, 1, 3), dv, atol=1e-11)
    np.testing.assert_allclose(ttab.grad.numpy(), dtab, atol=1e-11)
    # with dlse the table gradient no longer sums to zero over buckets: it sums
    # to the total of dlse over the head's rows (each row of P sums to one)
    np.testing.assert_allclose(dtab.sum(axis=0), dlse.sum(axis=(0, 2)), atol=1e-11)


@pytest.mark.parametrize("Bb,causal", [(1, False), (2, True), (1, True)])
def test_dense_bias_against_torch_sdpa_and_autograd(Bb, causal):
    """Dense bias (kernel v1): O, LSE, dq, dk, dv and dBias against PyTorch's
    attention with the bias as attn_mask and its autograd gradient (summed
    over the batch by broadcasting when Bb == 1)."""
    rng = np.random.default_rng(13)
    B, S, H, D = 2, 23, 3, 8
    q, k, v, do = (rng.standard_normal((B, S, H, D)) for _ in range(4))
    dense = rng.standard_normal((Bb, H, S, S))
    kw = dict(scale=0.6, causal=causal, bias="dense", dense=dense)
    O, LSE = oracle.attention_fwd(q, k, v, **kw)
    dq, dk, dv, dbias = oracle.attention_bwd(q, k, v, do, **kw)
    assert dbias.shape == dense.shape

    tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), requires_grad=True) for x in (q, k, v))
    tb = torch.tensor(dense, requires_grad=True)
    mask = tb
    if causal:
        mask = tb.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
    tO = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.6)
    np.testing.assert_allclose(tO.detach().numpy().transpose(0, 2, 1, 3), O, atol=1e-12)
    tO.backward(torch.tensor(do.transpose(0, 2, 1, 3)))
    np.testing.assert_allclose(tq.grad.numpy().transpose(0, 2, 1, 3), dq, atol=1e-11)
    np.testing.assert_allclose(tk.grad.numpy().transpose(0, 2, 1, 3), dk, atol=1e-11)
    np.testing.assert_allclose(tv.grad.numpy().transpose(0, 2, 1, 3), dv, atol=1e-11)
    np.testing.assert_allclose(tb.grad.numpy(), dbias, atol=1e-11)
    s = torch.einsum("bhid,bhjd->bhij", tq.detach(), tk.detach()) * 0.6 + mask.detach()
    np.testing.assert_allclose(torch.logsumexp(s, -1).numpy(), LSE, atol=1e-12)


def test_dense_bias_reproduces_t5_mode():
    """The T5 bias materialised as a dense matrix gives the T5 results, and
    the dense gradient summed over each bucket's pairs is the table gradient."""
    rng = np.random.default_rng(17)
    B, S, H, D, nb, md = 2, 40, 2, 8, 16, 24
    q, k, v, do = (rng.standard_normal((B, S, H, D)) for _ in range(4))
    table = rng.normal(0, 0.5, (nb, H))
    for causal, bidir in ((False, True), (True, False)):
        t5 = dict(scale=1.0, causal=causal, bias="t5", table=table, num_buckets=nb,
                  max_distance=md, bidirectional=bidir)
        buckets = np.array([[bucket_exact(j - i, nb, md, bidir) for j in range(S)]
                            for i in range(S)])
        dense = table[buckets].transpose(2, 0, 1)[None]          # [1, H, S, S]
        dn = dict(scale=1.0, causal=causal, bias="dense", dense=dense)
        for a, b in zip(oracle.attention_fwd(q, k, v, **t5), oracle.attention_fwd(q, k, v, **dn)):
            np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)
        g5 = oracle.attention_bwd(q, k, v, do, **t5)
        gd = oracle.attention_bwd(q, k, v, do, **dn)
        for a, b in zip(g5[:3], gd[:3]):
            np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)
        per_bucket = np.stack([np.bincount(buckets.ravel(), weights=gd[3][0, h].ravel(),
                                           minlength=nb) for h in range(H)], axis=1)
        np.testing.assert_allclose(per_bucket, g5[3], rtol=0, atol=1e-11)


# ---------------------------------------------------------------------------
# Backward against central finite differences of the oracle forward
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c['bias']}-causal{int(c['causal'])}"
                         f"-bi{int(c['bidirectional'])}-rope{int(c['rope_base'] is not None)}")
def test_backward_matches_finite_differences(case):
    rng = np.random.default_rng(3)
    S, D, nb, md, head = 9, 6, 8, 20, 1
    q, k, v, do = (rng.standard_normal((S, D)) for _ in range(4))
    table = rng.normal(0, 0.5, (nb, 2))
    slopes = oracle.alibi_slopes(2)
    # a rounding step has no derivative: check the calculus with it switched off
    kw = dict(scale=case["scale"], causal=case["causal"], bias=case["bias"], table=table,
              num_buckets=nb, max_distance=md, bidirectional=case["bidirectional"],
              slopes=slopes, rope_base=case["rope_base"], rope_round=False)
    dlse = rng.standard_normal(S)
    dq, dk, dv, dtab = head_bwd(q, k, v, do, head, dlse=dlse, **kw)

    def loss(q_, k_, v_, table_):
        kw2 = dict(kw, table=table_)
        O, lse = head_fwd(q_, k_, v_, head, **kw2)
        return float((O * do).sum() + (lse * dlse).sum())

    h = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1, a2 = arr.copy(), arr.copy()
            a1[idx] += h
            a2[idx] -= h
            args1 = dict(q_=q, k_=k, v_=v, table_=table)
            args2 = dict(q_=q, k_=k, v_=v, table_=table)
            args1[name + "_"] = a1
            args2[name + "_"] = a2
            num[idx] = (loss(**args1) - loss(**args2)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=0, atol=2e-7 * max(1.0, np.abs(num).max()))
    if case["bias"] == "t5":
        num = np.zeros(nb)
        for b in range(nb):
            t1, t2 = table.copy(), table.copy()
            t1[b, head] += h
            t2[b, head] -= h
            num[b] = (loss(q, k, v, t1) - loss(q, k, v, t2)) / (2 * h)
        np.testing.assert_allclose(dtab, num, rtol=0, atol=2e-7 * max(1.0, np.abs(num).max()))


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------


def _small_inputs(seed=5, B=2, S=33, H=3, D=8):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, S, H, D)) for _ in range(4)] + [rng.normal(0, 0.5, (32, H))]


@pytest.mark.parametrize("causal,bidirectional", [(False, True), (True, False)])
def test_invariants(causal, bidirectional):
    q, k, v, do, table = _small_inputs()
    kw = dict(scale=1.0, causal=causal, bias="t5", table=table, num_buckets=32, max_distance=128,
              bidirectional=bidirectional)
    O, LSE = oracle.attention_fwd(q, k, v, **kw)
    dq, dk, dv, dtab = oracle.attention_bwd(q, k, v, do, **kw)
    # each O element is a convex combination of its column of V
    assert np.all(O <= v.max(axis=1, keepdims=True) + 1e-12)
    assert np.all(O >= v.min(axis=1, keepdims=True) - 1e-12)
    # sum over buckets of dTable is zero (rows of dS sum to zero)
    np.testing.assert_allclose(dtab.sum(axis=0), 0, atol=1e-10)
    # without RoPE, sum over keys of dK is zero; sum over keys of dV equals sum of dO
    np.testing.assert_allclose(dk.sum(axis=1), 0, atol=1e-10)
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), atol=1e-10)
    # adding a constant to every table entry of a head leaves O unchanged and shifts LSE
    t2 = table.copy()
    t2[:, 1] += 0.75
    O2, LSE2 = oracle.attention_fwd(q, k, v, **dict(kw, table=t2))
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(LSE2[:, 1] - LSE[:, 1], 0.75, atol=1e-12)
    np.testing.assert_allclose(LSE2[:, 0], LSE[:, 0], atol=0)
    # a zero table and ALiBi with slope zero both give plain attention
    Oz, _ = oracle.attention_fwd(q, k, v, **dict(kw, table=np.zeros_like(table)))
    Oa, _ = oracle.attention_fwd(q, k, v, scale=1.0, causal=causal, bias="alibi",
                                 slopes=np.zeros(3))
    On, _ = oracle.attention_fwd(q, k, v, scale=1.0, causal=causal, bias="none")
    np.testing.assert_allclose(Oz, On, atol=1e-12)
    np.testing.assert_allclose(Oa, On, atol=1e-12)
    if causal:
        # the first query sees only the first key
        np.testing.assert_array_equal(O[:, 0], v[:, 0])


def test_softmax_rows_sum_to_one_and_lse():
    q, k, v, do, table = _small_inputs(S=20)
    # V = identity columns recovers P itself; its rows must sum to one
    S = q.shape[1]
    eye = np.broadcast_to(np.eye(S)[None, :, None, :], (2, S, 3, S)).copy()
    for causal in (False, True):
        P, _ = oracle.attention_fwd(q, k, eye, scale=1.0, causal=causal, bias="t5", table=table,
                                    num_buckets=32, max_distance=128, bidirectional=not causal)
        np.testing.assert_allclose(P.sum(axis=-1), 1.0, atol=1e-13)
        assert np.all(P >= 0)


def test_fully_masked_row_guard():
    from oracle.attention import _softmax_rows
    s = np.array([[0.0, -np.inf], [-np.inf, -np.inf]])
    P, lse = _softmax_rows(s)
    np.testing.assert_array_equal(P, [[1.0, 0.0], [0.0, 0.0]])
    assert lse[0] == 0.0 and lse[1] == -np.inf


# ---------------------------------------------------------------------------
# Packed batches
# ---------------------------------------------------------------------------


def test_segment_ids_and_varlen_equals_dense_slices():
    lengths = np.array([5, 1, 17, 9])
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, D = int(lengths.sum()), 2, 8
    ids = oracle.segment_ids(cu, T)
    np.testing.assert_array_equal(ids, np.repeat(np.arange(4), lengths))
    rng = np.random.default_rng(9)
    q, k, v, do = (rng.standard_normal((T, H, D)) for _ in range(4))
    table = rng.normal(0, 0.5, (32, H))
    kw = dict(scale=1.0, causal=False, bias="t5", table=table, num_buckets=32, max_distance=128,
              bidirectional=True)
    O, LSE = oracle.varlen_attention_fwd(q, k, v, cu, **kw)
    dq, dk, dv, dtab = oracle.varlen_attention_bwd(q, k, v, do, cu, **kw)
    dt_sum = np.zeros_like(dtab)
    for s in range(4):
        a, e = cu[s], cu[s + 1]
        Od, Ld = oracle.attention_fwd(q[None, a:e], k[None, a:e], v[None, a:e], **kw)
        np.testing.assert_allclose(O[a:e], Od[0], atol=0)
        np.testing.assert_allclose(LSE[:, a:e], Ld[0], atol=0)
        g = oracle.attention_bwd(q[None, a:e], k[None, a:e], v[None, a:e], do[None, a:e], **kw)
        np.testing.assert_allclose(dq[a:e], g[0][0], atol=0)
        np.testing.assert_allclose(dk[a:e], g[1][0], atol=0)
        np.testing.assert_allclose(dv[a:e], g[2][0], atol=0)
        dt_sum += g[3]
    np.testing.assert_allclose(dtab, dt_sum, atol=1e-12)
    # a length-1 sequence returns its own v
    np.testing.assert_array_equal(O[5], v[5])


def test_varlen_isolation():
    lengths = np.array([7, 12, 4])
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, D = int(lengths.sum()), 2, 4
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((T, H, D)) for _ in range(3))
    kw = dict(scale=1.0, causal=False, bias="none")
    O, _ = oracle.varlen_attention_fwd(q, k, v, cu, **kw)
    k2, v2 = k.copy(), v.copy()
    k2[7:19] += 3.0
    v2[7:19] -= 1.0
    O2, _ = oracle.varlen_attention_fwd(q, k2, v2, cu, **kw)
    np.testing.assert_array_equal(O2[:7], O[:7])
    np.testing.assert_array_equal(O2[19:], O[19:])


# ---------------------------------------------------------------------------
# Input generator (shared with the GPU side)
# ---------------------------------------------------------------------------


def test_bf16_rounding_is_round_to_nearest_even():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -9, 1 + 3 * 2 ** -8, -2.5, 65504.0, 1e-40],
                 np.float32)
    got = synth.bf16_bits_to_f32(synth.bf16_round(x))
    want = np.array([1.0, 1.0, 1 + 2 ** -7, 1 + 2 ** -6, -2.5, 65536.0, 1e-40], np.float32)
    # 1e-40 is a float32 subnormal; its bf16 neighbour is the truncation/rounding of its bits
    want[-1] = synth.bf16_bits_to_f32(np.array([(np.float32(1e-40).view(np.uint32) + 0x7FFF
                                                 + ((np.float32(1e-40).view(np.uint32) >> 16) & 1))
                                                >> 16], np.uint16))[0]
    np.testing.assert_array_equal(got, want)
    # agreement with torch's own float32 -> bfloat16 conversion (round to nearest even)
    r = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    tb = torch.from_numpy(r).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.bf16_round(r), tb)


def test_varlen_lengths_recipe():
    for seed, (nseq, ssq) in {0: (50, 41242800), 4: (55, 48759550)}.items():
        L = synth.draw_varlen_lengths(np.random.default_rng(seed), 32768)
        assert L.sum() == 32768 and L.min() >= 16 and L.max() <= 4096
        assert len(L) == nseq and int((L ** 2).sum()) == ssq


@pytest.mark.parametrize("bias,causal,bidi", [("t5", True, False), ("t5", False, True),
                                              ("alibi", True, True), ("none", False, True)])
def test_sampled_rows_and_keys_equal_the_whole_head(bias, causal, bidi):
    # the row-by-row form for long sequences against the materialised head:
    # the same definitions on fewer rows, so the results agree to rounding
    from oracle.attention import head_bwd, head_fwd, head_sampled
    rng = np.random.default_rng(17)
    S, D, h = 70, 8, 1
    q, k, v, do = (rng.standard_normal((S, D)) for _ in range(4))
    table = rng.standard_normal((32, 2))
    slopes = np.array([0.5, 0.125])
    kw = dict(scale=0.7, causal=causal, bias=bias, table=table, num_buckets=32,
              max_distance=20, bidirectional=bidi, slopes=slopes)
    O, lse = head_fwd(q, k, v, h, **kw)
    dq, dk, dv, _ = head_bwd(q, k, v, do, h, **kw)
    rows = [0, 1, 33, 68, 69]
    keys = [40, 55, 69] if causal else [0, 21, 69]
    o_r, l_r, dq_r, dk_k, dv_k = oracle.head_sampled(q, k, v, do, h, rows, keys, **kw)
    np.testing.assert_allclose(o_r, O[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_r, lse[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq_r, dq[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk_k, dk[keys], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_k, dv[keys], rtol=0, atol=1e-12)
