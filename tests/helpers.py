"""Shared test helpers: moving synth inputs to torch, running the oracle on
the same values, and the error measures the parity gates use."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

# Parity gates (elementwise against the fp64 oracle):
#   O:           max |gpu - ref| <= 2e-2 and mean |gpu - ref| <= 2e-3
#   dQ, dK, dV:  e = |gpu - ref| / max(1, |ref|): max e <= 2e-2, mean e <= 2e-3
#   dtable:      ||gpu - ref||_F / ||ref||_F <= 1e-2
#   LSE:         max |gpu - ref| <= 1e-3 (fp32 output; error of fp32 score sums)
O_MAX, O_MEAN = 2e-2, 2e-3
G_MAX, G_MEAN = 2e-2, 2e-3
DTABLE_REL = 1e-2
LSE_MAX = 1e-3


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def abs_err(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got - ref)
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def norm_err(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got - ref) / np.maximum(1.0, np.abs(ref))
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def assert_o(got, ref, what="O"):
    mx, mean = abs_err(got, ref)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    assert mx <= O_MAX and mean <= O_MEAN, f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e}"
    return mx, mean


def assert_lse(got, ref, what="LSE", tol=None):
    """tol: scalar or per-row bound (default LSE_MAX)."""
    tol = LSE_MAX if tol is None else tol
    d = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    assert np.all(d <= tol), f"{what}: max-abs {d.max():.3e}, worst excess {(d - tol).max():.3e}"
    return float(d.max())


def assert_grad(got, ref, what):
    mx, mean = norm_err(got, ref)
    rmx, rmean = abs_err(got, ref)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    assert mx <= G_MAX and mean <= G_MEAN, (
        f"{what}: normalised max {mx:.3e} mean {mean:.3e} (raw max {rmx:.3e} mean {rmean:.3e})")
    return mx, mean


def assert_dtable(got, ref, what="dtable"):
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert rel <= DTABLE_REL, f"{what}: Frobenius relative error {rel:.3e}"
    return rel


def oracle_kwargs(bias, causal, scale, table=None, slopes=None, nb=32, md=128,
                  bidirectional=True, rope_base=None, rope_round=True):
    return dict(scale=scale, causal=causal, bias=bias, table=table, num_buckets=nb,
                max_distance=md, bidirectional=bidirectional, slopes=slopes,
                rope_base=rope_base, rope_round=rope_round)


def nan_like(t: torch.Tensor) -> torch.Tensor:
    """An output buffer pre-filled with NaN: any element a kernel fails to
    write stays NaN and fails the finiteness checks."""
    return torch.full_like(t, float("nan"))


def pmap(fn, items, workers=8):
    """fn over items on a thread pool (NumPy releases the GIL in its array
    work, so independent oracle heads run side by side); results in order."""
    from concurrent.futures import ThreadPoolExecutor
    items = list(items)
    if len(items) <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=min(workers, len(items))) as ex:
        return list(ex.map(fn, items))


def log_margin(what: str, **errs):
    """Append one line of measured errors to $FA_PARITY_LOG (if set)."""
    import json
    import os
    path = os.environ.get("FA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(dict(case=what, **{k: float(v) for k, v in errs.items()})) + "\n")


def check_exact_rotation(got, reading, exact, what, scale, head_dim, gate):
    """RoPE against the exact rotation (no bf16 rounding of the rotated q, k).

    `reading` is the oracle's result under the RoPE reading (rotated q, k
    rounded once to bf16), `exact` the oracle's result without the rounding,
    `gate` the assert_* function of the output.  At the usual softmax scale
    (at most 1/sqrt(D), as the long-context workload uses) the kernel must
    meet the output's own gate against the exact rotation.  At larger scales
    the rounding of the rotated operands is itself beyond the gate (scores
    of std 8 at scale 1, D 64), so the kernel must then stay within 1.25x
    the reading's own distance from the exact rotation (plus 1e-3).
    Returns (kernel max error, reading max error) against the exact result."""
    e_k = norm_err(got, exact)[0]
    e_r = norm_err(reading, exact)[0]
    if scale * np.sqrt(head_dim) <= 1.0 + 1e-6:
        gate(got, exact, f"{what} (exact rotation)")
    else:
        assert e_k <= 1.25 * e_r + 1e-3, (
            f"{what}: {e_k:.3e} from the exact rotation, the reading's own rounding {e_r:.3e}")
    return e_k, e_r
