"""Seeded input generators (no attention arithmetic here).

Recipe (the same for every consumer):

* ``numpy.random.default_rng(seed)``.
* Varlen configs draw the sequence lengths first (``draw_varlen_lengths``).
* Then q, k, v and dO are drawn, in that order, as float32 standard normals of
  shape ``[B, S, H, D]`` (``[T, H, D]`` for packed batches) and each is
  rounded once to bfloat16 with round-to-nearest-even.  Both sides consume
  those exact bfloat16 values.
* Then the T5 bias table is drawn as float32 ``normal(0, 0.5)`` of shape
  ``[num_buckets, H]``.
* FIRE parameters come from their own seeded draw (``draw_fire_theta``).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as ``uint16``.  Inputs here are finite
    normal draws, so no NaN handling is needed; infinities pass through.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    # bits + 0x7FFF + lsb stays below 2^32 for every non-NaN pattern (the
    # largest, -inf, is 0xFF800000)
    rounded = bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to the float32 values they encode (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def draw_varlen_lengths(rng: np.random.Generator, total: int, mu: float = 6.0,
                        sigma: float = 1.0, lo: int = 16, hi: int = 4096) -> np.ndarray:
    """Packed-batch sequence lengths that sum exactly to ``total``.

    Lengths are ``rint(lognormal(mu, sigma))`` clipped to ``[lo, hi]``, drawn
    one at a time until the running sum reaches ``total``; the last length is
    the remainder.  A remainder below ``lo`` is merged into the previous
    sequence, or, if that would exceed ``hi``, the previous sequence gives
    ``lo - r`` tokens to a last sequence of length ``lo``.
    """
    lens: list[int] = []
    acc = 0
    while acc < total:
        L = int(np.clip(np.rint(rng.lognormal(mu, sigma)), lo, hi))
        if acc + L >= total:
            r = total - acc
            if r < lo and lens:
                if lens[-1] + r <= hi:
                    lens[-1] += r
                else:
                    lens[-1] -= lo - r
                    lens.append(lo)
            else:
                lens.append(r)
            acc = total
        else:
            lens.append(L)
            acc += L
    out = np.asarray(lens, dtype=np.int64)
    assert out.sum() == total and out.min() >= min(lo, total) and out.max() <= hi
    return out


def alibi_slope_values(heads: int) -> np.ndarray:
    """The per-head ALiBi slope inputs the long-context config prescribes:
    ``2**(-8*h/heads)`` for ``h = 1..heads``, as float32."""
    h = np.arange(1, heads + 1, dtype=np.float64)
    return np.exp2(-8.0 * h / heads).astype(np.float32)


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return bf16_round(rng.standard_normal(size=shape, dtype=np.float32))


@dataclass
class DenseInputs:
    q: np.ndarray      # uint16 bf16 bits [B,S,H,D]
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray]
    table: Optional[np.ndarray]  # float32 [nb, H]

    def f64(self, name: str) -> np.ndarray:
        return bf16_bits_to_f32(getattr(self, name)).astype(np.float64)


@dataclass
class VarlenInputs:
    lengths: np.ndarray      # int64 [nseq]
    cu_seqlens: np.ndarray   # int32 [nseq+1]
    q: np.ndarray            # uint16 bf16 bits [T,H,D]
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray]
    table: Optional[np.ndarray]

    def f64(self, name: str) -> np.ndarray:
        return bf16_bits_to_f32(getattr(self, name)).astype(np.float64)


def draw_dense(seed: int, B: int, S: int, H: int, D: int, *, num_buckets: int = 32,
               with_dout: bool = True, with_table: bool = True) -> DenseInputs:
    rng = np.random.default_rng(seed)
    shape = (B, S, H, D)
    q = _normal_bf16(rng, shape)
    k = _normal_bf16(rng, shape)
    v = _normal_bf16(rng, shape)
    do = _normal_bf16(rng, shape) if with_dout else None
    table = (rng.normal(0.0, 0.5, size=(num_buckets, H)).astype(np.float32)
             if with_table else None)
    return DenseInputs(q, k, v, do, table)


def draw_dense_bias(seed: int, Bb: int, H: int, S: int, sigma: float = 1.0) -> np.ndarray:
    """A dense additive bias matrix [Bb, H, S, S] as bf16 bits: N(0, sigma)
    values rounded once to bfloat16 (row = query, column = key)."""
    rng = np.random.default_rng(seed)
    return bf16_round((sigma * rng.standard_normal(size=(Bb, H, S, S))).astype(np.float32))


def draw_rmsnorm(seed: int, rows: int, dim: int):
    """RMSNorm inputs as bf16 bits: x, dy ~ N(0, 1) [rows, dim] and the weight
    w ~ N(1, 0.25) [dim]."""
    rng = np.random.default_rng(seed)
    x = _normal_bf16(rng, (rows, dim))
    dy = _normal_bf16(rng, (rows, dim))
    w = bf16_round((1.0 + 0.25 * rng.standard_normal(dim)).astype(np.float32))
    return x, w, dy


def draw_cross_entropy(seed: int, rows: int, vocab: int, sigma: float = 3.0,
                       ignore_frac: float = 0.1, ignore_index: int = -100):
    """Cross-entropy inputs: logits ~ N(0, sigma) as bf16 bits [rows, vocab],
    int32 labels uniform over the vocabulary with a fraction set to the
    ignore index, and dL/dloss per row ~ U(0.5, 1.5) / rows (fp32)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((rows, vocab), dtype=np.float32)
    z *= np.float32(sigma)
    z = bf16_round(z)
    y = rng.integers(0, vocab, rows).astype(np.int32)
    y[rng.random(rows) < ignore_frac] = ignore_index
    g = (rng.uniform(0.5, 1.5, rows) / max(rows, 1)).astype(np.float32)
    return z, y, g


def draw_varlen(seed: int, total: int, H: int, D: int, *, num_buckets: int = 32,
                lengths: Optional[np.ndarray] = None, with_dout: bool = True,
                with_table: bool = True, mu: float = 6.0, sigma: float = 1.0,
                lo: int = 16, hi: int = 4096) -> VarlenInputs:
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = draw_varlen_lengths(rng, total, mu, sigma, lo, hi)
    lengths = np.asarray(lengths, dtype=np.int64)
    assert lengths.sum() == total
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    shape = (total, H, D)
    q = _normal_bf16(rng, shape)
    k = _normal_bf16(rng, shape)
    v = _normal_bf16(rng, shape)
    do = _normal_bf16(rng, shape) if with_dout else None
    table = (rng.normal(0.0, 0.5, size=(num_buckets, H)).astype(np.float32)
             if with_table else None)
    return VarlenInputs(lengths, cu, q, k, v, do, table)


def draw_fire_theta(seed: int, heads: int, hidden: int = 32, c: float = 0.1,
                    threshold: float = 512.0) -> np.ndarray:
    """FIRE parameters as one float32 vector [w1 (K), b1 (K), w2 (H*K), b2 (H),
    c, L]: w1 ~ N(0, 4), each hidden unit's kink -b1/w1 uniform on
    (-0.5, 1.5) (so about half of them fall inside the [0, 1] range of the
    normalised distance), w2 ~ N(0, 1/K), b2 ~ N(0, 0.25), then c and L as
    given."""
    rng = np.random.default_rng(seed)
    K = hidden
    w1 = 2.0 * rng.standard_normal(K)
    kink = rng.uniform(-0.5, 1.5, K)
    b1 = -w1 * kink
    w2 = rng.standard_normal((heads, K)) / np.sqrt(K)
    b2 = 0.5 * rng.standard_normal(heads)
    return np.concatenate([w1, b1, w2.ravel(), b2, [c, threshold]]).astype(np.float32)
