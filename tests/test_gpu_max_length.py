"""The longest sequence the library takes (65536 tokens) through the C ABI,
against the fp64 oracle on sampled outputs: its S x S score matrix (4.3G
pairs per head) is too large to materialise, so the oracle evaluates whole
rows of S' for the sampled query rows (O, LSE, dQ) and every row that sees
the sampled keys (dK, dV; keys near the end under the causal mask).  Every
output starts as NaN and must come back finite everywhere, and each head's
table gradient must sum to zero over its buckets (rows of P sum to one, so
the dS of a row sum to zero)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_grad, assert_lse, assert_o, bf16_tensor, log_margin, nan_like, to_f64

pytestmark = pytest.mark.gpu

fa = pytest.importorskip("attention_t5_relative_amd")

S_MAX = 65536


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def test_causal_t5_at_the_maximum_length():
    B, S, H, D, scale = 1, S_MAX, 2, 64, 1.0
    nb, md, bidi = 32, 128, False
    inp = synth.draw_dense(4242, B, S, H, D, num_buckets=nb)
    t = {n: bf16_tensor(getattr(inp, n)) for n in ("q", "k", "v", "do")}
    bias = fa.T5Bias(torch.from_numpy(inp.table).cuda(), nb, md, bidi)
    print(f"[max length] GPU launch B{B} S{S} H{H} D{D}", flush=True)
    o = nan_like(t["q"])
    lse = torch.full((B, H, S), float("nan"), device="cuda")
    fa.fa_fwd(t["q"], t["k"], t["v"], o, lse, scale=scale, causal=True, bias=bias)
    dq, dk, dv = nan_like(t["q"]), nan_like(t["q"]), nan_like(t["q"])
    dtable = torch.full((nb, H), float("nan"), device="cuda")
    fa.fa_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], dq, dk, dv, dtable, scale=scale,
              causal=True, bias=bias)
    torch.cuda.synchronize()
    out = {n: to_f64(x) for n, x in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv,
                                         dtable=dtable).items()}
    for name, arr in out.items():
        bad = int((~np.isfinite(arr)).sum())
        assert bad == 0, f"{name}: {bad} elements not written or not finite"

    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 4095, 4096, 32767, 32768,
                                      65534, 65535], rng.integers(0, S, 6)]))
    keys = np.unique(np.concatenate([[S - 64, S - 33, S - 32, S - 1], S - 64 + rng.integers(0, 64, 4)]))
    kw = dict(scale=scale, causal=True, bias="t5", table=inp.table.astype(np.float64),
              num_buckets=nb, max_distance=md, bidirectional=bidi)
    errs = {}
    for h in range(H):
        qh, kh, vh, doh = (np.ascontiguousarray(inp.f64(n)[0, :, h]) for n in ("q", "k", "v", "do"))
        O, LSE, dQ, dK, dV = oracle.head_sampled(qh, kh, vh, doh, h, rows, keys, **kw)
        tag = f"S{S} head {h}"
        errs[f"o_max_h{h}"] = assert_o(out["o"][0, rows, h], O, tag + " O rows")[0]
        errs[f"lse_max_h{h}"] = assert_lse(out["lse"][0, h, rows], LSE, tag + " LSE rows")
        errs[f"dq_max_h{h}"] = assert_grad(out["dq"][0, rows, h], dQ, tag + " dQ rows")[0]
        errs[f"dk_max_h{h}"] = assert_grad(out["dk"][0, keys, h], dK, tag + " dK keys")[0]
        errs[f"dv_max_h{h}"] = assert_grad(out["dv"][0, keys, h], dV, tag + " dV keys")[0]
        col = out["dtable"][:, h]
        rel = abs(col.sum()) / np.abs(col).sum()
        errs[f"dtable_zero_sum_h{h}"] = rel
        assert rel <= 1e-3, f"{tag}: table gradient sums to {col.sum():.3e} ({rel:.2e} of its size)"
    log_margin("max length S65536", **errs)
