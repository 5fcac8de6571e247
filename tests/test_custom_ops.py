"""The attention pair registered as torch custom ops (CPU): the four ops
exist and their fake implementations give the output shapes and dtypes the
kernels write, so torch.compile can trace a call without running it."""
import pytest
import torch

import attention_t5_relative_amd as fa  # noqa: F401  (registers the ops)


def _meta(*shape, dtype=torch.bfloat16):
    return torch.empty(*shape, dtype=dtype, device="meta")


@pytest.mark.parametrize("kind,bias_shape,nb", [(0, None, 0), (1, (32, 3), 32), (2, (3,), 0),
                                                 (3, (1, 3, 100, 100), 0), (4, (2 * 8 + 3 * 8 + 3 + 2,), 0)])
def test_dense_ops_fake_shapes(kind, bias_shape, nb):
    q = _meta(2, 100, 3, 64)
    t = None if bias_shape is None else _meta(*bias_shape, dtype=torch.float32)
    o, lse = torch.ops.fat5attn.attention_fwd(q, q, q, t, kind, nb, 128, False, 8, 1.0, True, 0.0)
    assert o.shape == q.shape and o.dtype == torch.bfloat16
    assert lse.shape == (2, 3, 100) and lse.dtype == torch.float32
    want = kind in (1, 3, 4)
    dq, dk, dv, db = torch.ops.fat5attn.attention_bwd(q, q, q, o, lse, o, None, t, kind, nb, 128,
                                                      False, 8, 1.0, True, 0.0, want)
    assert dq.shape == dk.shape == dv.shape == q.shape and dq.dtype == torch.bfloat16
    assert db.dtype == torch.float32
    assert db.shape == (tuple(bias_shape) if want else (0,))


def test_varlen_ops_fake_shapes():
    q = _meta(300, 4, 128)
    cu = torch.empty(4, dtype=torch.int32, device="meta")
    t = _meta(32, 4, dtype=torch.float32)
    o, lse = torch.ops.fat5attn.varlen_attention_fwd(q, q, q, cu, 200, t, 1, 32, 128, True, 0,
                                                     0.1, False, 0.0)
    assert o.shape == q.shape and lse.shape == (4, 300) and lse.dtype == torch.float32
    dq, dk, dv, db = torch.ops.fat5attn.varlen_attention_bwd(q, q, q, o, lse, o, None, cu, 200, t,
                                                             1, 32, 128, True, 0, 0.1, False, 0.0,
                                                             True)
    assert dq.shape == q.shape and db.shape == (32, 4)


def test_dense_bias_refused_by_packed_entry():
    q = _meta(10, 1, 64)
    with pytest.raises(ValueError):
        fa.varlen_attention(q, q, q, torch.zeros(2, dtype=torch.int32), 10,
                            bias=fa.DenseBias(_meta(1, 1, 10, 10)))


def test_norm_and_loss_ops_fake_shapes():
    x = _meta(64, 768)
    w = _meta(768)
    y, rstd = torch.ops.fat5attn.rms_norm_fwd(x, w, 1e-6)
    assert y.shape == x.shape and rstd.shape == (64,) and rstd.dtype == torch.float32
    dx, dw = torch.ops.fat5attn.rms_norm_bwd(x, w, rstd, y, 1e-6, True)
    assert dx.shape == x.shape and dw.shape == (768,) and dw.dtype == torch.float32
    logits = _meta(64, 1000)
    labels = torch.empty(64, dtype=torch.int32, device="meta")
    loss, lse = torch.ops.fat5attn.cross_entropy_fwd(logits, labels, 1e-4, -100)
    assert loss.shape == lse.shape == (64,) and loss.dtype == torch.float32
    dl = torch.ops.fat5attn.cross_entropy_bwd(logits, labels, lse, loss, 1e-4, -100)
    assert dl.shape == logits.shape and dl.dtype == torch.bfloat16
