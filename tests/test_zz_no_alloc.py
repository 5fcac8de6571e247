"""fa_bwd_noalloc, the backward that allocates nothing (its scratch is the
library's static device array), against fa_bwd with a caller workspace.

Both run the same kernels on the same inputs, so every output must agree bit
for bit.  Two calls in a row on one GPU, the second on a smaller problem:
the static scratch keeps the first call's contents, which the second must
not depend on.  Each call is also checked against the oracle under the
parity gates."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (assert_dtable, assert_grad, bf16_tensor, nan_like, oracle_kwargs, to_f64)

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("attention_t5_relative_amd")

# B, S, H, D, causal, bidirectional, scale: the first is the larger problem
CASES = [(2, 777, 6, 64, True, False, 1.0), (1, 300, 2, 64, False, True, 1.0)]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _run(case, seed):
    B, S, H, D, causal, bidi, scale = case
    inp = synth.draw_dense(seed, B, S, H, D)
    q, k, v, do = (bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    bias = fa.T5Bias(torch.from_numpy(inp.table).cuda(), 32, 128, bidi)
    o = nan_like(q)
    lse = torch.full((B, H, S), float("nan"), device="cuda")
    fa.fa_fwd(q, k, v, o, lse, scale=scale, causal=causal, bias=bias)
    outs = {}
    for name, call in (("noalloc", fa.fa_bwd_noalloc), ("workspace", fa.fa_bwd)):
        dq, dk, dv = nan_like(q), nan_like(q), nan_like(q)
        dtable = torch.full((32, H), float("nan"), device="cuda")
        call(q, k, v, o, lse, do, dq, dk, dv, dtable, scale=scale, causal=causal, bias=bias)
        torch.cuda.synchronize()
        outs[name] = {n: to_f64(t) for n, t in (("dq", dq), ("dk", dk), ("dv", dv),
                                                ("dtable", dtable))}
    kw = oracle_kwargs("t5", causal, scale, inp.table, None, 32, 128, bidi, None)
    return inp, outs, kw


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    for i, case in enumerate(CASES):
        print(f"[no-alloc] call {i}: B,S,H,D = {case[:4]}", flush=True)
        inp, outs, kw = _run(case, 500 + i)
        for n in ("dq", "dk", "dv", "dtable"):
            assert np.isfinite(outs["noalloc"][n]).all(), f"call {i} {n}: not all written"
            np.testing.assert_array_equal(outs["noalloc"][n], outs["workspace"][n],
                                          err_msg=f"call {i} {n}")
        dq, dk, dv, dtab = oracle.attention_bwd(inp.f64("q"), inp.f64("k"), inp.f64("v"),
                                                inp.f64("do"), **kw)
        assert_grad(outs["noalloc"]["dq"], dq, f"call {i} dQ")
        assert_grad(outs["noalloc"]["dk"], dk, f"call {i} dK")
        assert_grad(outs["noalloc"]["dv"], dv, f"call {i} dV")
        assert_dtable(outs["noalloc"]["dtable"], dtab, f"call {i} dtable")


def test_noalloc_rejects_problems_beyond_its_scratch():
    # RoPE needs rotated copies of q and k: far beyond the static scratch
    q = torch.zeros((1, 16384, 16, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 16, 16384), device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.fa_bwd_noalloc(q, q, q, q, lse, q, q, q, q, rope_base=10000.0, scale=0.1)
    assert e.value.status == -2 and "static scratch" in str(e.value)
