"""fp64 NumPy oracle for exact attention with T5 / ALiBi bias, RoPE and packing.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Every score matrix here is materialised in full, one (batch, head) pair (or one
packed sequence) at a time.  Nothing is tiled, fused or reordered beyond the
definitions below.

Definitions followed (FAT5 report, section "Noyau CUDA", kernel v2 forward):

    S  = scale * Q K^T                    (scores)
    S' = S + bias                         (bias from the per-head table T, or ALiBi)

and the report's first kernel, handed the bias matrix B itself (same
section, kernel v1): S' = S + B.
    P  = softmax(S') over keys            (row-wise)
    O  = P V

plus logsumexp per row, LSE_i = log sum_j exp(S'_ij), which a backward needs.

Readings taken where the pages are silent:

* T5 buckets: the pages name the T5 relative-position bias and its class but
  print no formula.  The T5 scheme is used: relative position r = j - i (key
  minus query).  Bidirectional: half of the buckets per side, keys after the
  query take the upper half, n = |r|.  Unidirectional: n = max(-r, 0).  With
  nb' buckets per side and me = nb'/2: n < me gives bucket n; otherwise
  me + floor(ln(n/me) / ln(md/me) * (nb' - me)), capped at nb' - 1.
* The bias is added to the scaled scores (the scale does not apply to it).
* ALiBi: bias = -m_h * |i - j|, slopes m_h = 2^(-8h/H) for h = 1..H
  (geometric sequence of the ALiBi paper, which the report links).
* RoPE: interleaved pairs (2p, 2p+1) rotated by angle t * base^(-2p/D), t the
  0-based position (local to each packed sequence); applied to q and k only.
  The report trains in full bf16 and its kernels take bf16 q and k from the
  positional-encoding classes, so the rotated q and k are bf16 tensors: the
  exact rotation is rounded once to bf16 (nearest, ties to even) before the
  scores.  Gradients flow through the rotation as if the rounding were the
  identity.
* Dense bias (kernel v1): the pages say only that the kernel loads B and
  adds it to S.  Read here as one [S, S] matrix per (batch, head), given as
  [Bb, H, S, S] with Bb = 1 (shared by the whole batch) or Bb = B; its
  gradient is dS, summed over the batch when Bb = 1.
* FIRE: the learned bias f_theta(psi(i - j) / psi(max(L, i))), causal
  attention only; the reading is in ``oracle.fire``.  Its gradient is the
  flat d(theta), summed over the batch and heads.
* Causal: key j is visible to query i iff j <= i.
* Packed batches: a query attends only keys of its own sequence; positions are
  local to the sequence.
* Backward (standard calculus of softmax attention, not printed on the pages):
      dP = dO V^T,  D_i = sum_j P_ij dP_ij,  dS = P * (dP - D),
      dV = P^T dO,  dQ = scale dS K,  dK = scale dS^T Q,
      dTable[b, h] = sum over batch and over pairs (i, j) with bucket b of dS_ij.
  With RoPE the gradients of the rotated q, k are mapped back by the inverse
  rotation.
* A row with every key masked gets O = 0 and LSE = -inf.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .fire import fire_bias, fire_theta_grad

# --------------------------------------------------------------------------
# Position encodings
# --------------------------------------------------------------------------


def t5_bucket(rel, num_buckets: int, max_distance: int, bidirectional: bool) -> np.ndarray:
    """T5 relative-position bucket of ``rel = key_pos - query_pos``.

    FAT5 report, "Noyau CUDA" (the bucket tensor T and the
    RelativePositionalEncoding class it links); the formula is the T5 scheme,
    evaluated in float64.
    """
    rel = np.asarray(rel, dtype=np.int64)
    nb = int(num_buckets)
    if bidirectional:
        nb //= 2
        offset = np.where(rel > 0, nb, 0).astype(np.int64)
        n = np.abs(rel)
    else:
        offset = np.zeros_like(rel)
        n = np.maximum(-rel, 0)
    me = nb // 2
    small = n < me
    nf = np.maximum(n, 1).astype(np.float64)
    large = me + np.floor(np.log(nf / me) / math.log(max_distance / me) * (nb - me))
    large = np.minimum(large.astype(np.int64), nb - 1)
    return offset + np.where(small, n, large)


def alibi_slopes(heads: int) -> np.ndarray:
    """ALiBi head slopes 2^(-8h/H), h = 1..H (the ALiBi paper's geometric
    sequence; the FAT5 report lists ALiBi among the supported encodings)."""
    h = np.arange(1, heads + 1, dtype=np.float64)
    return 2.0 ** (-8.0 * h / heads)


def _rope_angles(positions: np.ndarray, dim: int, base: float) -> np.ndarray:
    p = np.arange(dim // 2, dtype=np.float64)
    theta = base ** (-2.0 * p / dim)
    return np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]


def rope_rotate(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotate each interleaved pair (x[2p], x[2p+1]) of row t by angle
    t * base^(-2p/D).  x: [S, D] float64 (RoFormer rotary encoding, which the
    FAT5 report lists among the supported encodings)."""
    ang = _rope_angles(positions, x.shape[-1], base)
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[:, 0::2], x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = x0 * c - x1 * s
    out[:, 1::2] = x0 * s + x1 * c
    return out


def bf16_round_exact(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (8 significant bits),
    ties to even, in one rounding step: x = m * 2^e with 0.5 <= |m| < 1, so
    m * 2^8 rounded half-to-even by numpy gives the kept significand exactly.
    (Normal range only; the inputs here are O(1).)"""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 256.0), e - 8)


def rope_unrotate(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Inverse of :func:`rope_rotate` (rotation by the opposite angle); maps a
    gradient with respect to rotated rows back to the unrotated rows."""
    ang = _rope_angles(positions, x.shape[-1], base)
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[:, 0::2], x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = x0 * c + x1 * s
    out[:, 1::2] = -x0 * s + x1 * c
    return out


# --------------------------------------------------------------------------
# One (batch, head) or one packed sequence
# --------------------------------------------------------------------------


def bias_matrix(seqlen: int, head: int, *, bias: str, table=None, num_buckets: int = 32,
                max_distance: int = 128, bidirectional: bool = True,
                slopes=None, dense=None, fire=None,
                fire_hidden: int = 0) -> Optional[np.ndarray]:
    """Additive bias [S, S] (rows = query i, columns = key j) for one head, or
    None when there is no bias.  ``dense`` is the head's own [S, S] matrix
    (bias "dense"); ``fire`` the flat FIRE parameter vector with
    ``fire_hidden`` hidden units (bias "fire", see oracle.fire)."""
    if bias == "none":
        return None
    if bias == "dense":
        return np.asarray(dense, dtype=np.float64)
    if bias == "fire":
        K = int(fire_hidden)
        H = (len(fire) - 2 * K - 2) // (K + 1)
        return fire_bias(seqlen, fire, H, K, head=head)
    i = np.arange(seqlen)[:, None]
    j = np.arange(seqlen)[None, :]
    if bias == "t5":
        b = t5_bucket(j - i, num_buckets, max_distance, bidirectional)
        return np.asarray(table, dtype=np.float64)[b, head]
    if bias == "alibi":
        return -float(slopes[head]) * np.abs(i - j).astype(np.float64)
    raise ValueError(bias)


def _scores(qh, kh, head, *, scale, causal, bias, table, num_buckets, max_distance,
            bidirectional, slopes, rope_base, rope_round=True, dense=None, fire=None,
            fire_hidden=0):
    S = qh.shape[0]
    if bias == "fire" and not causal:
        raise ValueError("FIRE is defined for causal attention (key at or before the query)")
    pos = np.arange(S)
    if rope_base is not None:
        qh = rope_rotate(qh, pos, rope_base)
        kh = rope_rotate(kh, pos, rope_base)
        if rope_round:
            qh, kh = bf16_round_exact(qh), bf16_round_exact(kh)
    s = scale * (qh @ kh.T)
    bm = bias_matrix(S, head, bias=bias, table=table, num_buckets=num_buckets,
                     max_distance=max_distance, bidirectional=bidirectional, slopes=slopes,
                     dense=dense, fire=fire, fire_hidden=fire_hidden)
    if bm is not None:
        s = s + bm
    if causal:
        s = np.where(np.arange(S)[None, :] > np.arange(S)[:, None], -np.inf, s)
    return s, qh, kh


def _softmax_rows(s):
    m = s.max(axis=1)
    dead = ~np.isfinite(m)
    m_safe = np.where(dead, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        P = np.where(dead[:, None], 0.0, e / np.where(dead, 1.0, l)[:, None])
        lse = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, l)))
    return P, lse


def head_fwd(qh, kh, vh, head, *, scale=1.0, causal=False, bias="none", table=None,
             num_buckets=32, max_distance=128, bidirectional=True, slopes=None,
             rope_base=None, rope_round=True, dense=None, fire=None, fire_hidden=0):
    """Forward for one head: qh, kh, vh float64 [S, D] -> (O [S, D], LSE [S]).

    ``rope_round=False`` skips the bf16 rounding of the rotated q, k: the
    exact rotation (the finite-difference pin needs it, since a rounding step
    has no derivative; the GPU tests also measure the kernels against it)."""
    s, _, _ = _scores(qh, kh, head, scale=scale, causal=causal, bias=bias, table=table,
                      num_buckets=num_buckets, max_distance=max_distance,
                      bidirectional=bidirectional, slopes=slopes, rope_base=rope_base,
                      rope_round=rope_round, dense=dense, fire=fire, fire_hidden=fire_hidden)
    P, lse = _softmax_rows(s)
    return P @ vh, lse


def head_bwd(qh, kh, vh, doh, head, *, scale=1.0, causal=False, bias="none", table=None,
             num_buckets=32, max_distance=128, bidirectional=True, slopes=None,
             rope_base=None, rope_round=True, dense=None, fire=None, fire_hidden=0, dlse=None):
    """Backward for one head -> (dq, dk, dv [S, D], bias gradient): the bias
    gradient is dtable_h [num_buckets] for T5, dS [S, S] for a dense bias,
    this head's part of d(theta) (the flat FIRE vector) for FIRE, None
    otherwise.

    ``dlse`` [S] (optional) is the loss gradient with respect to the returned
    LSE.  LSE_i is the log-sum-exp of row i of S', whose derivative with
    respect to S'_ij is P_ij, so it adds dlse_i * P_ij to dS_ij."""
    S = qh.shape[0]
    s, qr, kr = _scores(qh, kh, head, scale=scale, causal=causal, bias=bias, table=table,
                        num_buckets=num_buckets, max_distance=max_distance,
                        bidirectional=bidirectional, slopes=slopes, rope_base=rope_base,
                        rope_round=rope_round, dense=dense, fire=fire, fire_hidden=fire_hidden)
    P, _ = _softmax_rows(s)
    dP = doh @ vh.T
    Drow = (P * dP).sum(axis=1)
    dS = P * (dP - Drow[:, None])
    if dlse is not None:
        dS = dS + P * np.asarray(dlse, dtype=np.float64)[:, None]
    dv = P.T @ doh
    dq = scale * (dS @ kr)
    dk = scale * (dS.T @ qr)
    if rope_base is not None:
        pos = np.arange(S)
        dq = rope_unrotate(dq, pos, rope_base)
        dk = rope_unrotate(dk, pos, rope_base)
    dtab = None
    if bias == "t5":
        i = np.arange(S)[:, None]
        j = np.arange(S)[None, :]
        b = t5_bucket(j - i, num_buckets, max_distance, bidirectional)
        dtab = np.bincount(b.ravel(), weights=dS.ravel(), minlength=num_buckets)
    if bias == "dense":
        dtab = dS
    if bias == "fire":
        K = int(fire_hidden)
        H = (len(fire) - 2 * K - 2) // (K + 1)
        dtab = fire_theta_grad(dS, head, fire, H, K)
    return dq, dk, dv, dtab


def head_sampled(qh, kh, vh, doh, head, rows, keys, *, scale=1.0, causal=False, bias="none",
                 table=None, num_buckets=32, max_distance=128, bidirectional=True,
                 slopes=None):
    """Selected outputs of one head, for sequences whose S x S score matrix
    is too large to hold: O, LSE and dQ at the query rows ``rows``, dK and
    dV at the keys ``keys``.  The definitions are those of head_fwd and
    head_bwd, evaluated on whole rows of S' only: a selected row needs its
    own row; a selected key j needs every row that sees it (rows j .. S-1
    under a causal mask, all rows otherwise), each with its own D_i.  T5,
    ALiBi or no bias, no RoPE.

    Returns (O [len(rows), D], LSE [len(rows)], dQ [len(rows), D],
    dK [len(keys), D], dV [len(keys), D])."""
    S = qh.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    j = np.arange(S)[None, :]

    def score_rows(ii):
        s = scale * (qh[ii] @ kh.T)
        rel = j - ii[:, None]
        if bias == "t5":
            s = s + np.asarray(table, dtype=np.float64)[
                t5_bucket(rel, num_buckets, max_distance, bidirectional), head]
        elif bias == "alibi":
            s = s - float(slopes[head]) * np.abs(rel).astype(np.float64)
        elif bias != "none":
            raise ValueError(bias)
        if causal:
            s = np.where(rel > 0, -np.inf, s)
        return s

    def grads(ii):
        P, lse = _softmax_rows(score_rows(ii))
        dP = doh[ii] @ vh.T
        Drow = (P * dP).sum(axis=1)
        return P, lse, P * (dP - Drow[:, None])

    P, lse, dS = grads(rows)
    O = P @ vh
    dq = scale * (dS @ kh)
    first = int(keys.min()) if (causal and keys.size) else 0
    seen = np.arange(first, S)
    Pk, _, dSk = grads(seen)
    dk = scale * (dSk[:, keys].T @ qh[seen])
    dv = Pk[:, keys].T @ doh[seen]
    return O, lse, dq, dk, dv


# --------------------------------------------------------------------------
# Dense batches [B, S, H, D]
# --------------------------------------------------------------------------


def _kw(kw):
    keys = ("scale", "causal", "bias", "table", "num_buckets", "max_distance",
            "bidirectional", "slopes", "rope_base", "rope_round", "fire", "fire_hidden")
    return {k: kw[k] for k in keys if k in kw}


def _head_kw(kw, b, h):
    """Per-head keyword arguments: a dense bias [Bb, H, S, S] is sliced to
    the head's own matrix (batch index 0 when Bb == 1)."""
    hk = _kw(kw)
    if kw.get("bias") == "dense":
        dense = kw["dense"]
        hk["dense"] = dense[b if dense.shape[0] > 1 else 0, h]
    return hk


def attention_fwd(q, k, v, pairs=None, **kw):
    """Dense forward.  q, k, v float64 [B, S, H, D].

    Returns O [B, S, H, D] and LSE [B, H, S].  With ``pairs`` (a list of
    (b, h)), only those heads are computed; the rest stay NaN.
    """
    B, S, H, _ = q.shape
    O = np.full((B, S, H, v.shape[-1]), np.nan)
    LSE = np.full((B, H, S), np.nan)
    todo = pairs if pairs is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        o, lse = head_fwd(q[b, :, h], k[b, :, h], v[b, :, h], h, **_head_kw(kw, b, h))
        O[b, :, h] = o
        LSE[b, h] = lse
    return O, LSE


def attention_bwd(q, k, v, do, pairs=None, dlse=None, **kw):
    """Dense backward.  Returns dq, dk, dv [B, S, H, D] and the bias
    gradient: dtable [nb, H] for T5, dbias [Bb, H, S, S] for a dense bias
    (summed over the batch when Bb == 1), None otherwise.  With ``pairs``,
    only those heads are computed (others NaN) and the bias gradient sums over
    the computed heads only.  ``dlse`` [B, H, S] (optional): the gradient with
    respect to the returned LSE."""
    B, S, H, D = q.shape
    dq = np.full(q.shape, np.nan)
    dk = np.full(q.shape, np.nan)
    dv = np.full(q.shape, np.nan)
    nb = kw.get("num_buckets", 32)
    dtable = None
    if kw.get("bias") == "t5":
        dtable = np.zeros((nb, H))
    elif kw.get("bias") == "dense":
        dtable = np.zeros(kw["dense"].shape)
    elif kw.get("bias") == "fire":
        dtable = np.zeros(len(kw["fire"]))
    todo = pairs if pairs is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        a, bb, c, dt = head_bwd(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], h,
                                dlse=None if dlse is None else dlse[b, h],
                                **_head_kw(kw, b, h))
        dq[b, :, h], dk[b, :, h], dv[b, :, h] = a, bb, c
        if kw.get("bias") == "t5":
            dtable[:, h] += dt
        elif kw.get("bias") == "dense":
            dtable[b if dtable.shape[0] > 1 else 0, h] += dt
        elif kw.get("bias") == "fire":
            dtable += dt
    return dq, dk, dv, dtable


# --------------------------------------------------------------------------
# Packed batches [T, H, D] with cu_seqlens
# --------------------------------------------------------------------------


def segment_ids(cu_seqlens, total: int) -> np.ndarray:
    """Sequence index of every packed token: the s with cu[s] <= t < cu[s+1]."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return np.searchsorted(cu, np.arange(total), side="right") - 1


def varlen_attention_fwd(q, k, v, cu_seqlens, seqs=None, heads=None, **kw):
    """Packed forward.  q, k, v float64 [T, H, D]; returns O [T, H, D] and
    LSE [H, T].  Each sequence is attended on its own, positions local.
    ``seqs``/``heads`` restrict the computed part (rest NaN)."""
    T, H, _ = q.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    O = np.full((T, H, v.shape[-1]), np.nan)
    LSE = np.full((H, T), np.nan)
    seqs = range(len(cu) - 1) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    for s in seqs:
        a, e = cu[s], cu[s + 1]
        if e == a:
            continue
        for h in heads:
            o, lse = head_fwd(q[a:e, h], k[a:e, h], v[a:e, h], h, **_kw(kw))
            O[a:e, h] = o
            LSE[h, a:e] = lse
    return O, LSE


def varlen_attention_bwd(q, k, v, do, cu_seqlens, seqs=None, heads=None, dlse=None, **kw):
    """Packed backward; ``dlse`` [H, T] (optional) as in attention_bwd."""
    T, H, D = q.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    dq = np.full(q.shape, np.nan)
    dk = np.full(q.shape, np.nan)
    dv = np.full(q.shape, np.nan)
    nb = kw.get("num_buckets", 32)
    dtable = np.zeros((nb, H)) if kw.get("bias") == "t5" else None
    if kw.get("bias") == "fire":
        dtable = np.zeros(len(kw["fire"]))
    seqs = range(len(cu) - 1) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    for s in seqs:
        a, e = cu[s], cu[s + 1]
        if e == a:
            continue
        for h in heads:
            r = head_bwd(q[a:e, h], k[a:e, h], v[a:e, h], do[a:e, h], h,
                         dlse=None if dlse is None else dlse[h, a:e], **_kw(kw))
            dq[a:e, h], dk[a:e, h], dv[a:e, h] = r[0], r[1], r[2]
            if kw.get("bias") == "fire":
                dtable += r[3]
            elif dtable is not None:
                dtable[:, h] += r[3]
    return dq, dk, dv, dtable
