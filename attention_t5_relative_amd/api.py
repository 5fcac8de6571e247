"""Python binding of libfat5attn with the C entry points' names.

Torch is plumbing here: it owns device memory and supplies the current HIP
stream.  Each function checks dtypes/shapes, fills the C params struct with
``data_ptr()`` values and calls the library; every step of the attention path
runs in the HIP kernels.  ``attention`` / ``varlen_attention`` wrap the pair
of calls as torch custom ops with autograd (torch.compile traces them as
single nodes).
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Union

import torch

from . import _lib
from ._lib import (FaBias, FaBwdParams, FaFwdParams, FaVarlenBwdParams, FaVarlenFwdParams,
                   check)


@dataclass
class T5Bias:
    """T5 bucketed relative-position bias: table fp32 [num_buckets, H]."""
    table: torch.Tensor
    num_buckets: int = 32
    max_distance: int = 128
    bidirectional: bool = True


@dataclass
class ALiBi:
    """ALiBi bias -slopes[h] * |i - j|: slopes fp32 [H]."""
    slopes: torch.Tensor


@dataclass
class DenseBias:
    """A dense additive bias matrix (the report's first kernel): bf16
    [Bb, H, S, S] with Bb = 1 (shared by the batch) or B; row = query,
    column = key."""
    matrix: torch.Tensor


@dataclass
class FireBias:
    """FIRE (causal attention only): theta fp32 [2K + H*K + H + 2] =
    [w1 (K), b1 (K), w2 (H*K), b2 (H), c, L] with K = hidden; the bias of query
    i, key j <= i is b2_h + sum_k w2_hk relu(w1_k x + b1_k),
    x = log(c (i - j) + 1) / log(c max(L, i) + 1)."""
    theta: torch.Tensor
    hidden: int = 32


def fire_theta_size(heads: int, hidden: int) -> int:
    return 2 * hidden + heads * hidden + heads + 2


BiasSpec = Optional[Union[T5Bias, ALiBi, DenseBias, FireBias]]


def alibi_slopes(heads: int, device=None) -> torch.Tensor:
    """ALiBi's geometric head slopes 2^(-8h/H), h = 1..H, as fp32."""
    h = torch.arange(1, heads + 1, dtype=torch.float64)
    return torch.exp2(-8.0 * h / heads).to(torch.float32).to(device)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _bias_struct(bias: BiasSpec, heads: int, device, batch: Optional[int] = None,
                 seqlen: Optional[int] = None) -> FaBias:
    b = FaBias()
    if bias is None:
        b.mode = _lib.FA_BIAS_NONE
    elif isinstance(bias, T5Bias):
        _need(bias.table, "bias.table", torch.float32, (bias.num_buckets, heads), device)
        b.mode = _lib.FA_BIAS_T5
        b.num_buckets = bias.num_buckets
        b.max_distance = bias.max_distance
        b.bidirectional = int(bool(bias.bidirectional))
        b.table = bias.table.data_ptr()
    elif isinstance(bias, ALiBi):
        _need(bias.slopes, "bias.slopes", torch.float32, (heads,), device)
        b.mode = _lib.FA_BIAS_ALIBI
        b.slopes = bias.slopes.data_ptr()
    elif isinstance(bias, DenseBias):
        if seqlen is None:
            raise ValueError("a dense bias matrix is for the dense entry points only")
        m = bias.matrix
        if m.dim() != 4 or m.shape[0] not in (1, batch):
            raise ValueError(f"bias.matrix must be [1 or {batch}, H, S, S]")
        _need(m, "bias.matrix", torch.bfloat16, (m.shape[0], heads, seqlen, seqlen), device)
        b.mode = _lib.FA_BIAS_DENSE
        b.dense = m.data_ptr()
        b.dense_batch = m.shape[0]
    elif isinstance(bias, FireBias):
        _need(bias.theta, "bias.theta", torch.float32, (fire_theta_size(heads, bias.hidden),),
              device)
        b.mode = _lib.FA_BIAS_FIRE
        b.table = bias.theta.data_ptr()
        b.fire_hidden = int(bias.hidden)
    else:
        raise TypeError("bias must be None, T5Bias, ALiBi, DenseBias or FireBias")
    return b


def _dbias_shape(bias: BiasSpec, heads: int):
    """Shape of the bias gradient fa_bwd writes (None when the mode has none)."""
    if isinstance(bias, T5Bias):
        return (bias.num_buckets, heads)
    if isinstance(bias, DenseBias):
        return tuple(bias.matrix.shape)
    if isinstance(bias, FireBias):
        return (fire_theta_size(heads, bias.hidden),)
    return None


def _fwd_params(q, k, v, o, lse, scale, causal, bias, rope_base) -> FaFwdParams:
    if q.dim() != 4:
        raise ValueError("dense q must be [B, S, H, D]")
    B, S, H, D = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _need(t, name, torch.bfloat16, (B, S, H, D), dev)
    _need(lse, "lse", torch.float32, (B, H, S), dev)
    p = FaFwdParams()
    p.batch, p.seqlen, p.heads, p.head_dim = B, S, H, D
    p.causal = int(bool(causal))
    p.scale = float(scale)
    p.rope_base = float(rope_base or 0.0)
    p.q, p.k, p.v, p.o, p.lse = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr()
    p.bias = _bias_struct(bias, H, dev, B, S)
    return p


def _varlen_params(q, k, v, o, lse, cu_seqlens, max_seqlen, scale, causal, bias,
                   rope_base) -> FaVarlenFwdParams:
    if q.dim() != 3:
        raise ValueError("packed q must be [T, H, D]")
    T, H, D = q.shape
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _need(t, name, torch.bfloat16, (T, H, D), dev)
    _need(lse, "lse", torch.float32, (H, T), dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
    p = FaVarlenFwdParams()
    p.nseq = cu_seqlens.numel() - 1
    p.total, p.max_seqlen, p.heads, p.head_dim = T, int(max_seqlen), H, D
    p.causal = int(bool(causal))
    p.scale = float(scale)
    p.rope_base = float(rope_base or 0.0)
    p.cu_seqlens = cu_seqlens.data_ptr()
    p.q, p.k, p.v, p.o, p.lse = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr()
    p.bias = _bias_struct(bias, H, dev)
    return p


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if nbytes == ctypes.c_size_t(-1).value:
        raise _lib.FaError(_lib.FA_ERR_INVALID, "workspace size")
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return workspace, workspace.numel() * workspace.element_size()


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------


def fa_fwd(q, k, v, o, lse, *, scale=1.0, causal=False, bias: BiasSpec = None, rope_base=0.0,
           workspace=None, stream=None) -> None:
    """Dense forward into o [B,S,H,D] bf16 and lse [B,H,S] fp32."""
    lib = _lib.load()
    p = _fwd_params(q, k, v, o, lse, scale, causal, bias, rope_base)
    ws, wsb = _workspace(lib.fa_fwd_workspace_size(ctypes.byref(p)), q.device, workspace)
    check(lib.fa_fwd(ctypes.byref(p), _ptr(ws), wsb, _stream(q.device, stream)), "fa_fwd")


def fa_varlen_fwd(q, k, v, o, lse, cu_seqlens, max_seqlen, *, scale=1.0, causal=False,
                  bias: BiasSpec = None, rope_base=0.0, workspace=None, stream=None) -> None:
    """Packed forward into o [T,H,D] bf16 and lse [H,T] fp32."""
    lib = _lib.load()
    p = _varlen_params(q, k, v, o, lse, cu_seqlens, max_seqlen, scale, causal, bias, rope_base)
    ws, wsb = _workspace(lib.fa_varlen_fwd_workspace_size(ctypes.byref(p)), q.device, workspace)
    check(lib.fa_varlen_fwd(ctypes.byref(p), _ptr(ws), wsb, _stream(q.device, stream)),
          "fa_varlen_fwd")


def _bwd_params(q, k, v, o, lse, dout, dq, dk, dv, dtable, dlse, scale, causal, bias,
                rope_base) -> FaBwdParams:
    p = FaBwdParams()
    p.f = _fwd_params(q, k, v, o, lse, scale, causal, bias, rope_base)
    for name, t in (("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _need(t, name, torch.bfloat16, q.shape, q.device)
    if dtable is not None:
        _need(dtable, "dtable", torch.float32, _dbias_shape(bias, q.shape[2]), q.device)
    if dlse is not None:
        _need(dlse, "dlse", torch.float32, lse.shape, q.device)
    p.dout, p.dq, p.dk, p.dv = dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    p.dtable = _ptr(dtable)
    p.dlse = _ptr(dlse)
    return p


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, dtable=None, *, dlse=None, scale=1.0,
           causal=False, bias: BiasSpec = None, rope_base=0.0, workspace=None,
           stream=None) -> None:
    """Dense backward into dq, dk, dv [B,S,H,D] bf16 and the bias gradient
    ``dtable``: fp32 [nb,H] for T5Bias, fp32 [Bb,H,S,S] for DenseBias, d(theta)
    for FireBias.
    ``dlse`` (optional, fp32 [B,H,S]) is the gradient with respect to lse."""
    lib = _lib.load()
    p = _bwd_params(q, k, v, o, lse, dout, dq, dk, dv, dtable, dlse, scale, causal, bias,
                    rope_base)
    ws, wsb = _workspace(lib.fa_bwd_workspace_size(ctypes.byref(p)), q.device, workspace)
    check(lib.fa_bwd(ctypes.byref(p), _ptr(ws), wsb, _stream(q.device, stream)), "fa_bwd")


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, dtable=None, *, dlse=None, scale=1.0,
                   causal=False, bias: BiasSpec = None, rope_base=0.0, stream=None) -> None:
    """fa_bwd with the library's static scratch instead of a workspace: the
    call allocates nothing (torch included)."""
    lib = _lib.load()
    p = _bwd_params(q, k, v, o, lse, dout, dq, dk, dv, dtable, dlse, scale, causal, bias,
                    rope_base)
    check(lib.fa_bwd_noalloc(ctypes.byref(p), _stream(q.device, stream)), "fa_bwd_noalloc")


def fa_varlen_bwd(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens, max_seqlen, dtable=None, *,
                  dlse=None, scale=1.0, causal=False, bias: BiasSpec = None, rope_base=0.0,
                  workspace=None, stream=None) -> None:
    """Packed backward into dq, dk, dv [T,H,D] bf16 and the bias gradient
    dtable (fp32 [nb,H] for T5Bias, d(theta) for FireBias); ``dlse``
    (optional, fp32 [H,T]) is the gradient with respect to lse."""
    lib = _lib.load()
    p = FaVarlenBwdParams()
    p.f = _varlen_params(q, k, v, o, lse, cu_seqlens, max_seqlen, scale, causal, bias, rope_base)
    for name, t in (("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _need(t, name, torch.bfloat16, q.shape, q.device)
    if dtable is not None:
        _need(dtable, "dtable", torch.float32, _dbias_shape(bias, q.shape[1]), q.device)
    if dlse is not None:
        _need(dlse, "dlse", torch.float32, lse.shape, q.device)
    p.dout, p.dq, p.dk, p.dv = dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    p.dtable = _ptr(dtable)
    p.dlse = _ptr(dlse)
    ws, wsb = _workspace(lib.fa_varlen_bwd_workspace_size(ctypes.byref(p)), q.device, workspace)
    check(lib.fa_varlen_bwd(ctypes.byref(p), _ptr(ws), wsb, _stream(q.device, stream)),
          "fa_varlen_bwd")


def fa_t5_buckets(qlen: int, klen: int, num_buckets: int, max_distance: int,
                  bidirectional: bool, out: torch.Tensor, stream=None) -> None:
    """Bucket index of every (query, key) pair into out int32 [qlen, klen]."""
    lib = _lib.load()
    _need(out, "out", torch.int32, (qlen, klen))
    check(lib.fa_t5_buckets(qlen, klen, num_buckets, max_distance, int(bool(bidirectional)),
                            out.data_ptr(), _stream(out.device, stream)), "fa_t5_buckets")


def fa_fwd_workspace_size(q, *, causal=False, scale=1.0, bias: BiasSpec = None,
                          rope_base=0.0) -> int:
    lib = _lib.load()
    B, S, H, D = q.shape
    o = q
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    p = _fwd_params(q, q, q, o, lse, scale, causal, bias, rope_base)
    return lib.fa_fwd_workspace_size(ctypes.byref(p))


# ---------------------------------------------------------------------------
# Autograd wrappers
# ---------------------------------------------------------------------------


def _output_grads(do, dlse, o):
    """The gradients autograd hands back for (O, LSE), either of which may be
    None when the loss does not use that output: a missing dO is zero, a
    missing dLSE is left out of the call."""
    do = torch.zeros_like(o) if do is None else do.to(o.dtype).contiguous()
    if dlse is not None:
        dlse = dlse.to(torch.float32).contiguous()
    return do, dlse


# The attention pair as torch custom ops (torch.library), so that
# torch.compile traces a call as one opaque node (no graph break) and
# autograd reaches the backward kernels.  The bias travels as its tensor plus
# plain scalars: kind 0 none, 1 T5, 2 ALiBi, 3 dense matrix, 4 FIRE.
_NO_BIAS, _T5, _ALIBI, _DENSE, _FIRE = 0, 1, 2, 3, 4


def _bias_fields(bias: BiasSpec):
    """(kind, tensor, num_buckets, max_distance, bidirectional, hidden)."""
    if isinstance(bias, T5Bias):
        return _T5, bias.table, bias.num_buckets, bias.max_distance, bool(bias.bidirectional), 0
    if isinstance(bias, ALiBi):
        return _ALIBI, bias.slopes, 0, 0, False, 0
    if isinstance(bias, DenseBias):
        return _DENSE, bias.matrix, 0, 0, False, 0
    if isinstance(bias, FireBias):
        return _FIRE, bias.theta, 0, 0, False, bias.hidden
    if bias is None:
        return _NO_BIAS, None, 0, 0, False, 0
    raise TypeError(f"unsupported bias {type(bias).__name__}")


def _bias_spec(kind, t, nb, md, bidi, hidden) -> BiasSpec:
    if kind == _T5:
        return T5Bias(t, nb, md, bidi)
    if kind == _ALIBI:
        return ALiBi(t)
    if kind == _DENSE:
        return DenseBias(t)
    if kind == _FIRE:
        return FireBias(t, hidden)
    return None


def _dbias_like(kind, t, device):
    """The bias-gradient buffer the kernels write (fp32), or an empty tensor
    when the bias has none."""
    if kind in (_T5, _FIRE):
        return torch.empty(t.shape, dtype=torch.float32, device=device)
    if kind == _DENSE:
        return torch.empty(t.shape, dtype=torch.float32, device=device)
    return torch.empty(0, dtype=torch.float32, device=device)


@torch.library.custom_op("fat5attn::attention_fwd", mutates_args=(), device_types="cuda")
def _attention_fwd_op(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      bias_t: Optional[torch.Tensor], kind: int, nb: int, md: int, bidi: bool,
                      hidden: int, scale: float, causal: bool,
                      rope_base: float) -> tuple[torch.Tensor, torch.Tensor]:
    B, S, H, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, scale=scale, causal=causal,
           bias=_bias_spec(kind, bias_t, nb, md, bidi, hidden), rope_base=rope_base)
    return o, lse


@_attention_fwd_op.register_fake
def _(q, k, v, bias_t, kind, nb, md, bidi, hidden, scale, causal, rope_base):
    B, S, H, D = q.shape
    return torch.empty_like(q), q.new_empty((B, H, S), dtype=torch.float32)


@torch.library.custom_op("fat5attn::attention_bwd", mutates_args=(), device_types="cuda")
def _attention_bwd_op(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                      lse: torch.Tensor, do: torch.Tensor, dlse: Optional[torch.Tensor],
                      bias_t: Optional[torch.Tensor], kind: int, nb: int, md: int, bidi: bool,
                      hidden: int, scale: float, causal: bool, rope_base: float,
                      want_dbias: bool) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor,
                                                 torch.Tensor]:
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dbias = (_dbias_like(kind, bias_t, q.device) if want_dbias
             else torch.empty(0, dtype=torch.float32, device=q.device))
    fa_bwd(q, k, v, o, lse, do, dq, dk, dv, dbias if dbias.numel() else None, dlse=dlse,
           scale=scale, causal=causal, bias=_bias_spec(kind, bias_t, nb, md, bidi, hidden),
           rope_base=rope_base)
    return dq, dk, dv, dbias


@_attention_bwd_op.register_fake
def _(q, k, v, o, lse, do, dlse, bias_t, kind, nb, md, bidi, hidden, scale, causal, rope_base,
      want_dbias):
    dbias = (_dbias_like(kind, bias_t, q.device) if want_dbias
             else q.new_empty((0,), dtype=torch.float32))
    return torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), dbias


def _attention_setup(ctx, inputs, output):
    q, k, v, bias_t, kind, nb, md, bidi, hidden, scale, causal, rope_base = inputs
    o, lse = output
    ctx.save_for_backward(q, k, v, o, lse, bias_t)
    ctx.cfg = (kind, nb, md, bidi, hidden, scale, causal, rope_base)


def _attention_backward(ctx, do, dlse):
    q, k, v, o, lse, bias_t = ctx.saved_tensors
    kind = ctx.cfg[0]
    want = bool(ctx.needs_input_grad[3]) and kind in (_T5, _DENSE, _FIRE)
    do, dlse = _output_grads(do, dlse, o)
    dq, dk, dv, dbias = _attention_bwd_op(q, k, v, o, lse, do, dlse, bias_t, *ctx.cfg, want)
    if not want:
        dbias = None
    elif kind == _DENSE:
        dbias = dbias.to(bias_t.dtype)   # a leaf's gradient keeps its dtype
    return dq, dk, dv, dbias, None, None, None, None, None, None, None, None


_attention_fwd_op.register_autograd(_attention_backward, setup_context=_attention_setup)


def attention(q, k, v, *, bias: BiasSpec = None, causal=False, scale=1.0, rope_base=0.0,
              return_lse=False):
    """Exact attention with optional T5 / ALiBi / FIRE / dense bias and RoPE;
    q, k, v [B,S,H,D] bf16.  Differentiable in q, k, v and the bias tensor
    (T5 table, dense matrix, FIRE theta), and traceable by torch.compile."""
    kind, t, nb, md, bidi, hidden = _bias_fields(bias)
    o, lse = _attention_fwd_op(q, k, v, t, kind, nb, md, bidi, hidden, float(scale),
                               bool(causal), float(rope_base))
    return (o, lse) if return_lse else o


@torch.library.custom_op("fat5attn::varlen_attention_fwd", mutates_args=(), device_types="cuda")
def _varlen_fwd_op(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                   max_seqlen: int, bias_t: Optional[torch.Tensor], kind: int, nb: int, md: int,
                   bidi: bool, hidden: int, scale: float, causal: bool,
                   rope_base: float) -> tuple[torch.Tensor, torch.Tensor]:
    T, H, D = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device)
    fa_varlen_fwd(q, k, v, o, lse, cu_seqlens, max_seqlen, scale=scale, causal=causal,
                  bias=_bias_spec(kind, bias_t, nb, md, bidi, hidden), rope_base=rope_base)
    return o, lse


@_varlen_fwd_op.register_fake
def _(q, k, v, cu_seqlens, max_seqlen, bias_t, kind, nb, md, bidi, hidden, scale, causal,
      rope_base):
    T, H, D = q.shape
    return torch.empty_like(q), q.new_empty((H, T), dtype=torch.float32)


@torch.library.custom_op("fat5attn::varlen_attention_bwd", mutates_args=(), device_types="cuda")
def _varlen_bwd_op(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                   lse: torch.Tensor, do: torch.Tensor, dlse: Optional[torch.Tensor],
                   cu_seqlens: torch.Tensor, max_seqlen: int, bias_t: Optional[torch.Tensor],
                   kind: int, nb: int, md: int, bidi: bool, hidden: int, scale: float,
                   causal: bool, rope_base: float,
                   want_dbias: bool) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor,
                                              torch.Tensor]:
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dbias = (_dbias_like(kind, bias_t, q.device) if want_dbias
             else torch.empty(0, dtype=torch.float32, device=q.device))
    fa_varlen_bwd(q, k, v, o, lse, do, dq, dk, dv, cu_seqlens, max_seqlen,
                  dbias if dbias.numel() else None, dlse=dlse, scale=scale, causal=causal,
                  bias=_bias_spec(kind, bias_t, nb, md, bidi, hidden), rope_base=rope_base)
    return dq, dk, dv, dbias


@_varlen_bwd_op.register_fake
def _(q, k, v, o, lse, do, dlse, cu_seqlens, max_seqlen, bias_t, kind, nb, md, bidi, hidden,
      scale, causal, rope_base, want_dbias):
    dbias = (_dbias_like(kind, bias_t, q.device) if want_dbias
             else q.new_empty((0,), dtype=torch.float32))
    return torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), dbias


def _varlen_setup(ctx, inputs, output):
    (q, k, v, cu_seqlens, max_seqlen, bias_t, kind, nb, md, bidi, hidden, scale, causal,
     rope_base) = inputs
    o, lse = output
    ctx.save_for_backward(q, k, v, o, lse, cu_seqlens, bias_t)
    ctx.max_seqlen = max_seqlen
    ctx.cfg = (kind, nb, md, bidi, hidden, scale, causal, rope_base)


def _varlen_backward(ctx, do, dlse):
    q, k, v, o, lse, cu, bias_t = ctx.saved_tensors
    kind = ctx.cfg[0]
    want = bool(ctx.needs_input_grad[5]) and kind in (_T5, _FIRE)
    do, dlse = _output_grads(do, dlse, o)
    dq, dk, dv, dbias = _varlen_bwd_op(q, k, v, o, lse, do, dlse, cu, ctx.max_seqlen, bias_t,
                                       *ctx.cfg, want)
    return (dq, dk, dv, None, None, dbias if want else None, None, None, None, None, None,
            None, None, None)


_varlen_fwd_op.register_autograd(_varlen_backward, setup_context=_varlen_setup)


def varlen_attention(q, k, v, cu_seqlens, max_seqlen, *, bias: BiasSpec = None, causal=False,
                     scale=1.0, rope_base=0.0, return_lse=False):
    """Packed attention; q, k, v [T,H,D] bf16, cu_seqlens int32 [nseq+1].
    Differentiable in q, k, v and the T5 table or FIRE theta, and traceable
    by torch.compile."""
    if isinstance(bias, DenseBias):
        raise ValueError("a dense bias matrix is for the dense entry points")
    kind, t, nb, md, bidi, hidden = _bias_fields(bias)
    o, lse = _varlen_fwd_op(q, k, v, cu_seqlens, int(max_seqlen), t, kind, nb, md, bidi, hidden,
                            float(scale), bool(causal), float(rope_base))
    return (o, lse) if return_lse else o


# ---------------------------------------------------------------------------
# RMSNorm and cross-entropy with z-loss (the report's two other fused kernels)
# ---------------------------------------------------------------------------


def _rms_params(x, w, y, rstd, eps) -> _lib.FaRmsnormFwdParams:
    if x.dim() != 2:
        raise ValueError("x must be [rows, dim]")
    rows, dim = x.shape
    _need(x, "x", torch.bfloat16, (rows, dim))
    _need(w, "w", torch.bfloat16, (dim,), x.device)
    _need(y, "y", torch.bfloat16, (rows, dim), x.device)
    _need(rstd, "rstd", torch.float32, (rows,), x.device)
    p = _lib.FaRmsnormFwdParams()
    p.rows, p.dim, p.eps = rows, dim, float(eps)
    p.x, p.w, p.y, p.rstd = x.data_ptr(), w.data_ptr(), y.data_ptr(), rstd.data_ptr()
    return p


def fa_rmsnorm_fwd(x, w, y, rstd, *, eps=1e-6, stream=None) -> None:
    """y = x / sqrt(mean x^2 + eps) * w into y [rows, dim] bf16, rstd [rows] fp32."""
    lib = _lib.load()
    p = _rms_params(x, w, y, rstd, eps)
    check(lib.fa_rmsnorm_fwd(ctypes.byref(p), _stream(x.device, stream)), "fa_rmsnorm_fwd")


def fa_rmsnorm_bwd(x, w, rstd, dy, dx, dw=None, *, eps=1e-6, workspace=None,
                   stream=None) -> None:
    """dx [rows, dim] bf16 and dw [dim] fp32 (optional) of RMSNorm."""
    lib = _lib.load()
    p = _lib.FaRmsnormBwdParams()
    p.f = _rms_params(x, w, x, rstd, eps)   # y is not read by the backward
    _need(dy, "dy", torch.bfloat16, x.shape, x.device)
    _need(dx, "dx", torch.bfloat16, x.shape, x.device)
    if dw is not None:
        _need(dw, "dw", torch.float32, (x.shape[1],), x.device)
    p.dy, p.dx, p.dw = dy.data_ptr(), dx.data_ptr(), _ptr(dw)
    ws, wsb = _workspace(lib.fa_rmsnorm_bwd_workspace_size(ctypes.byref(p)), x.device, workspace)
    check(lib.fa_rmsnorm_bwd(ctypes.byref(p), _ptr(ws), wsb, _stream(x.device, stream)),
          "fa_rmsnorm_bwd")


def _ce_params(logits, labels, loss, lse, z_loss, ignore_index) -> _lib.FaCeFwdParams:
    if logits.dim() != 2:
        raise ValueError("logits must be [rows, vocab]")
    rows, vocab = logits.shape
    _need(logits, "logits", torch.bfloat16, (rows, vocab))
    _need(labels, "labels", torch.int32, (rows,), logits.device)
    _need(loss, "loss", torch.float32, (rows,), logits.device)
    _need(lse, "lse", torch.float32, (rows,), logits.device)
    p = _lib.FaCeFwdParams()
    p.rows, p.vocab, p.z_loss, p.ignore_index = rows, vocab, float(z_loss), int(ignore_index)
    p.logits, p.labels = logits.data_ptr(), labels.data_ptr()
    p.loss, p.lse = loss.data_ptr(), lse.data_ptr()
    return p


def fa_ce_fwd(logits, labels, loss, lse, *, z_loss=0.0, ignore_index=-100, stream=None) -> None:
    """Per-row loss lse - z_y + z_loss lse^2 into loss [rows] and lse [rows] (fp32)."""
    lib = _lib.load()
    p = _ce_params(logits, labels, loss, lse, z_loss, ignore_index)
    check(lib.fa_ce_fwd(ctypes.byref(p), _stream(logits.device, stream)), "fa_ce_fwd")


def fa_ce_bwd(logits, labels, lse, dloss, dlogits, *, z_loss=0.0, ignore_index=-100,
              stream=None) -> None:
    """dlogits [rows, vocab] bf16 for dL/dloss = dloss [rows] (may be logits itself)."""
    lib = _lib.load()
    p = _lib.FaCeBwdParams()
    p.f = _ce_params(logits, labels, lse, lse, z_loss, ignore_index)   # loss is not read
    _need(dloss, "dloss", torch.float32, (logits.shape[0],), logits.device)
    _need(dlogits, "dlogits", torch.bfloat16, logits.shape, logits.device)
    p.dloss, p.dlogits = dloss.data_ptr(), dlogits.data_ptr()
    check(lib.fa_ce_bwd(ctypes.byref(p), _stream(logits.device, stream)), "fa_ce_bwd")


# RMSNorm and cross-entropy as torch custom ops with autograd as well.
@torch.library.custom_op("fat5attn::rms_norm_fwd", mutates_args=(), device_types="cuda")
def _rmsnorm_fwd_op(x: torch.Tensor, w: torch.Tensor,
                    eps: float) -> tuple[torch.Tensor, torch.Tensor]:
    y = torch.empty_like(x)
    rstd = torch.empty(x.shape[0], dtype=torch.float32, device=x.device)
    fa_rmsnorm_fwd(x, w, y, rstd, eps=eps)
    return y, rstd


@_rmsnorm_fwd_op.register_fake
def _(x, w, eps):
    return torch.empty_like(x), x.new_empty((x.shape[0],), dtype=torch.float32)


@torch.library.custom_op("fat5attn::rms_norm_bwd", mutates_args=(), device_types="cuda")
def _rmsnorm_bwd_op(x: torch.Tensor, w: torch.Tensor, rstd: torch.Tensor, dy: torch.Tensor,
                    eps: float, want_dw: bool) -> tuple[torch.Tensor, torch.Tensor]:
    dx = torch.empty_like(x)
    dw = torch.empty(w.shape if want_dw else (0,), dtype=torch.float32, device=w.device)
    fa_rmsnorm_bwd(x, w, rstd, dy, dx, dw if want_dw else None, eps=eps)
    return dx, dw


@_rmsnorm_bwd_op.register_fake
def _(x, w, rstd, dy, eps, want_dw):
    return torch.empty_like(x), w.new_empty(w.shape if want_dw else (0,), dtype=torch.float32)


def _rmsnorm_setup(ctx, inputs, output):
    x, w, eps = inputs
    ctx.save_for_backward(x, w, output[1])
    ctx.eps = eps


def _rmsnorm_backward(ctx, dy, drstd):
    x, w, rstd = ctx.saved_tensors
    want = bool(ctx.needs_input_grad[1])
    dx, dw = _rmsnorm_bwd_op(x, w, rstd, dy.contiguous(), ctx.eps, want)
    return dx, (dw.to(w.dtype) if want else None), None


_rmsnorm_fwd_op.register_autograd(_rmsnorm_backward, setup_context=_rmsnorm_setup)


def rms_norm(x, w, eps=1e-6):
    """RMSNorm over the last dimension of bf16 x (any leading shape), weight w [dim]."""
    shape = x.shape
    y, _ = _rmsnorm_fwd_op(x.reshape(-1, shape[-1]).contiguous(), w, float(eps))
    return y.reshape(shape)


@torch.library.custom_op("fat5attn::cross_entropy_fwd", mutates_args=(), device_types="cuda")
def _ce_fwd_op(logits: torch.Tensor, labels: torch.Tensor, z_loss: float,
               ignore_index: int) -> tuple[torch.Tensor, torch.Tensor]:
    rows = logits.shape[0]
    loss = torch.empty(rows, dtype=torch.float32, device=logits.device)
    lse = torch.empty_like(loss)
    fa_ce_fwd(logits, labels, loss, lse, z_loss=z_loss, ignore_index=ignore_index)
    return loss, lse


@_ce_fwd_op.register_fake
def _(logits, labels, z_loss, ignore_index):
    rows = logits.shape[0]
    return (logits.new_empty((rows,), dtype=torch.float32),
            logits.new_empty((rows,), dtype=torch.float32))


@torch.library.custom_op("fat5attn::cross_entropy_bwd", mutates_args=(), device_types="cuda")
def _ce_bwd_op(logits: torch.Tensor, labels: torch.Tensor, lse: torch.Tensor,
               dloss: torch.Tensor, z_loss: float, ignore_index: int) -> torch.Tensor:
    dlogits = torch.empty_like(logits)
    fa_ce_bwd(logits, labels, lse, dloss, dlogits, z_loss=z_loss, ignore_index=ignore_index)
    return dlogits


@_ce_bwd_op.register_fake
def _(logits, labels, lse, dloss, z_loss, ignore_index):
    return torch.empty_like(logits)


def _ce_setup(ctx, inputs, output):
    logits, labels, z_loss, ignore_index = inputs
    ctx.save_for_backward(logits, labels, output[1])
    ctx.z_loss, ctx.ignore_index = z_loss, ignore_index


def _ce_backward(ctx, dloss, dlse):
    logits, labels, lse = ctx.saved_tensors
    dlogits = _ce_bwd_op(logits, labels, lse, dloss.contiguous().float(), ctx.z_loss,
                         ctx.ignore_index)
    return dlogits, None, None, None


_ce_fwd_op.register_autograd(_ce_backward, setup_context=_ce_setup)


def cross_entropy(logits, labels, *, z_loss=0.0, ignore_index=-100):
    """Per-row cross-entropy with z-loss over bf16 logits [rows, vocab] and int
    labels [rows]: fp32 [rows], 0 for ignored rows.  Any reduction over the
    rows (a mean over the non-ignored ones, a sum) is the caller's, as in the
    C ABI: the kernels compute per-row losses and their gradients."""
    loss, _ = _ce_fwd_op(logits.contiguous(), labels.to(torch.int32).contiguous(),
                         float(z_loss), int(ignore_index))
    return loss
