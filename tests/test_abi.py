"""C-ABI checks that need no GPU: the library loads, exports every function
include/fat5attn.h declares, the ctypes structs match the C layout, and the
host-side argument checks return the documented status codes.  Nothing here
launches a kernel."""
import ctypes
import os
import re
import subprocess

import pytest

from attention_t5_relative_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fat5attn.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = header_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), set(names) ^ set(_lib.SIGNATURES)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa_[a-z0-9_]+)$", out, flags=re.M))
    assert set(names) <= exported


def test_kernel_timer_ids(lib):
    assert lib.fa_set_kernel_timer(_lib.FA_KERNEL_COUNT, None, None) == _lib.FA_ERR_INVALID
    assert lib.fa_set_kernel_timer(-1, None, None) == _lib.FA_ERR_INVALID
    assert _lib.FA_KERNEL_COUNT == 9
    for k in range(_lib.FA_KERNEL_COUNT):
        assert lib.fa_set_kernel_timer(k, None, None) == _lib.FA_OK


def test_status_strings_and_version(lib):
    assert lib.fa_status_str(0) == b"ok"
    assert lib.fa_status_str(-3) == b"workspace missing or too small"
    assert re.match(rb"^\d+\.\d+\.\d+$", lib.fa_version())


STRUCTS = {
    "fa_bias": (_lib.FaBias, ["mode", "num_buckets", "max_distance", "bidirectional", "table",
                              "slopes", "dense", "dense_batch", "fire_hidden"]),
    "fa_fwd_params": (_lib.FaFwdParams, ["batch", "seqlen", "heads", "head_dim", "causal",
                                         "scale", "rope_base", "reserved", "q", "k", "v", "o",
                                         "lse", "bias"]),
    "fa_bwd_params": (_lib.FaBwdParams, ["f", "dout", "dq", "dk", "dv", "dtable", "dlse"]),
    "fa_varlen_fwd_params": (_lib.FaVarlenFwdParams, ["nseq", "total", "max_seqlen", "heads",
                                                      "head_dim", "causal", "scale", "rope_base",
                                                      "cu_seqlens", "q", "k", "v", "o", "lse",
                                                      "bias"]),
    "fa_varlen_bwd_params": (_lib.FaVarlenBwdParams, ["f", "dout", "dq", "dk", "dv", "dtable",
                                                      "dlse"]),
    "fa_rmsnorm_fwd_params": (_lib.FaRmsnormFwdParams, ["rows", "dim", "eps", "reserved", "x",
                                                        "w", "y", "rstd"]),
    "fa_rmsnorm_bwd_params": (_lib.FaRmsnormBwdParams, ["f", "dy", "dx", "dw"]),
    "fa_ce_fwd_params": (_lib.FaCeFwdParams, ["rows", "vocab", "z_loss", "ignore_index",
                                              "logits", "labels", "loss", "lse"]),
    "fa_ce_bwd_params": (_lib.FaCeBwdParams, ["f", "dloss", "dlogits"]),
}


def test_ctypes_layout_matches_c_compiler(tmp_path):
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "fat5attn.h"',
             "int main(void) {"]
    for s, (_, fields) in STRUCTS.items():
        lines.append(f'printf("{s} %zu\\n", sizeof({s}));')
        for f in fields:
            lines.append(f'printf("{s}.{f} %zu\\n", offsetof({s}, {f}));')
    lines.append("return 0; }")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(c), "-o", str(exe)], check=True)
    got = dict(line.rsplit(" ", 1) for line in subprocess.run(
        [str(exe)], capture_output=True, text=True, check=True).stdout.split("\n") if line)
    for s, (cls, fields) in STRUCTS.items():
        assert int(got[s]) == ctypes.sizeof(cls), s
        for f in fields:
            assert int(got[f"{s}.{f}"]) == getattr(cls, f).offset, f"{s}.{f}"


def _dense(**kw):
    p = _lib.FaFwdParams()
    p.batch, p.seqlen, p.heads, p.head_dim = 2, 100, 3, 64
    p.causal, p.scale, p.rope_base = 0, 1.0, 0.0
    p.q = p.k = p.v = p.o = p.lse = 0x1000
    p.bias.mode = _lib.FA_BIAS_T5
    p.bias.num_buckets, p.bias.max_distance, p.bias.bidirectional = 32, 128, 1
    p.bias.table = 0x2000
    for k, v in kw.items():
        if k.startswith("bias_"):
            setattr(p.bias, k[5:], v)
        else:
            setattr(p, k, v)
    return p


@pytest.mark.parametrize("change,status", [
    ({}, _lib.FA_OK),
    ({"q": None}, _lib.FA_ERR_INVALID),
    ({"lse": None}, _lib.FA_ERR_INVALID),
    ({"batch": -1}, _lib.FA_ERR_INVALID),
    ({"heads": 0}, _lib.FA_ERR_INVALID),
    ({"head_dim": 96}, _lib.FA_ERR_UNSUPPORTED),
    ({"head_dim": 0}, _lib.FA_ERR_INVALID),
    ({"causal": 2}, _lib.FA_ERR_INVALID),
    ({"scale": float("nan")}, _lib.FA_ERR_INVALID),
    ({"scale": -1.0}, _lib.FA_ERR_UNSUPPORTED),
    ({"rope_base": -2.0}, _lib.FA_ERR_INVALID),
    ({"reserved": 1}, _lib.FA_ERR_INVALID),
    ({"seqlen": 70000}, _lib.FA_ERR_UNSUPPORTED),
    ({"bias_mode": 7}, _lib.FA_ERR_INVALID),
    ({"bias_table": None}, _lib.FA_ERR_INVALID),
    ({"bias_num_buckets": 31}, _lib.FA_ERR_UNSUPPORTED),
    ({"bias_num_buckets": 300}, _lib.FA_ERR_UNSUPPORTED),
    ({"bias_max_distance": 8}, _lib.FA_ERR_UNSUPPORTED),
    ({"bias_max_distance": 2048}, _lib.FA_ERR_UNSUPPORTED),
    ({"bias_bidirectional": 3}, _lib.FA_ERR_INVALID),
    ({"bias_mode": _lib.FA_BIAS_ALIBI}, _lib.FA_ERR_INVALID),   # slopes NULL
    ({"bias_mode": _lib.FA_BIAS_ALIBI, "bias_slopes": 0x3000}, _lib.FA_OK),
    ({"bias_mode": _lib.FA_BIAS_NONE, "bias_table": None}, _lib.FA_OK),
    ({"bias_bidirectional": 0, "bias_num_buckets": 31}, _lib.FA_OK),
    ({"bias_fire_hidden": 1}, _lib.FA_ERR_INVALID),    # only with FIRE
    # FIRE: theta in bias.table, causal only, 1..64 hidden units
    ({"bias_mode": _lib.FA_BIAS_FIRE, "bias_fire_hidden": 32, "causal": 1}, _lib.FA_OK),
    ({"bias_mode": _lib.FA_BIAS_FIRE, "bias_fire_hidden": 32, "causal": 0},
     _lib.FA_ERR_UNSUPPORTED),
    ({"bias_mode": _lib.FA_BIAS_FIRE, "bias_fire_hidden": 0, "causal": 1},
     _lib.FA_ERR_UNSUPPORTED),
    ({"bias_mode": _lib.FA_BIAS_FIRE, "bias_fire_hidden": 65, "causal": 1},
     _lib.FA_ERR_UNSUPPORTED),
    ({"bias_mode": _lib.FA_BIAS_FIRE, "bias_fire_hidden": 8, "causal": 1, "bias_table": None},
     _lib.FA_ERR_INVALID),
    ({"bias_mode": _lib.FA_BIAS_DENSE}, _lib.FA_ERR_INVALID),   # dense NULL
    ({"bias_mode": _lib.FA_BIAS_DENSE, "bias_dense": 0x6000, "bias_dense_batch": 1}, _lib.FA_OK),
    ({"bias_mode": _lib.FA_BIAS_DENSE, "bias_dense": 0x6000, "bias_dense_batch": 2}, _lib.FA_OK),
    ({"bias_mode": _lib.FA_BIAS_DENSE, "bias_dense": 0x6000, "bias_dense_batch": 3},
     _lib.FA_ERR_INVALID),
    ({"bias_mode": _lib.FA_BIAS_DENSE, "bias_dense": 0x6000, "bias_dense_batch": 0},
     _lib.FA_ERR_INVALID),
    ({"bias_mode": _lib.FA_BIAS_DENSE, "bias_dense": 0x6000, "bias_dense_batch": 1,
      "seqlen": 20000}, _lib.FA_ERR_UNSUPPORTED),
    # an empty batch with a dense bias: nothing is computed, but the backward
    # clears dense_batch * heads * seqlen^2 gradient floats, so those sizes are
    # still checked (pointers may be NULL)
    ({"bias_mode": _lib.FA_BIAS_DENSE, "bias_dense_batch": 1, "batch": 0, "q": None},
     _lib.FA_OK),
    ({"bias_mode": _lib.FA_BIAS_DENSE, "bias_dense_batch": 1, "batch": 0, "heads": -1},
     _lib.FA_ERR_INVALID),
    ({"bias_mode": _lib.FA_BIAS_DENSE, "bias_dense_batch": 1, "batch": 0, "seqlen": 20000},
     _lib.FA_ERR_UNSUPPORTED),
])
def test_dense_checks(lib, change, status):
    p = _dense(**change)
    assert lib.fa_check_fwd(ctypes.byref(p)) == status, lib.fa_last_error()
    if status != _lib.FA_OK:
        assert lib.fa_last_error() != b""
        assert lib.fa_fwd_workspace_size(ctypes.byref(p)) == ctypes.c_size_t(-1).value
        # the entry point refuses before touching the device
        assert lib.fa_fwd(ctypes.byref(p), None, 0, None) == status


def test_bwd_checks(lib):
    b = _lib.FaBwdParams()
    b.f = _dense()
    b.dout = b.dq = b.dk = b.dv = 0x4000
    assert lib.fa_check_bwd(ctypes.byref(b)) == _lib.FA_OK
    b.dk = None
    assert lib.fa_check_bwd(ctypes.byref(b)) == _lib.FA_ERR_INVALID
    assert lib.fa_bwd(ctypes.byref(b), None, 0, None) == _lib.FA_ERR_INVALID
    assert lib.fa_check_bwd(None) == _lib.FA_ERR_INVALID


def test_varlen_checks(lib):
    p = _lib.FaVarlenFwdParams()
    p.nseq, p.total, p.max_seqlen, p.heads, p.head_dim = 3, 300, 200, 4, 128
    p.scale = 0.1
    p.cu_seqlens = 0x5000
    p.q = p.k = p.v = p.o = p.lse = 0x1000
    assert lib.fa_check_varlen_fwd(ctypes.byref(p)) == _lib.FA_OK
    p.cu_seqlens = None
    assert lib.fa_check_varlen_fwd(ctypes.byref(p)) == _lib.FA_ERR_INVALID
    p.cu_seqlens = 0x5000
    p.nseq = -1
    assert lib.fa_check_varlen_fwd(ctypes.byref(p)) == _lib.FA_ERR_INVALID
    p.nseq = 3
    p.max_seqlen = 100000
    assert lib.fa_check_varlen_fwd(ctypes.byref(p)) == _lib.FA_ERR_UNSUPPORTED
    b = _lib.FaVarlenBwdParams()
    p.max_seqlen = 200
    b.f = p
    b.dout = b.dq = b.dk = b.dv = 0x4000
    assert lib.fa_check_varlen_bwd(ctypes.byref(b)) == _lib.FA_OK
    # a dense bias matrix belongs to the dense entry points
    p.bias.mode, p.bias.dense, p.bias.dense_batch = _lib.FA_BIAS_DENSE, 0x6000, 1
    assert lib.fa_check_varlen_fwd(ctypes.byref(p)) == _lib.FA_ERR_UNSUPPORTED


def test_workspace_sizes(lib):
    p = _dense()
    assert lib.fa_fwd_workspace_size(ctypes.byref(p)) == 0
    p.rope_base = 10000.0

    def a256(x):
        return (x + 255) // 256 * 256
    # the forward: a rotated copy of k and the fp64 (cos, sin) table [S, D/2] (q is
    # rotated in registers); each region 256-byte aligned
    one = 2 * 100 * 3 * 64 * 2
    table = 100 * 32 * 16
    assert lib.fa_fwd_workspace_size(ctypes.byref(p)) == a256(one) + a256(table)
    # a call that needs a workspace refuses without one
    assert lib.fa_fwd(ctypes.byref(p), None, 0, None) == _lib.FA_ERR_WORKSPACE
    # the backward: rotated copies of q and k, the table, -D and -lse/scale
    # (dQ and dK are turned back inside the kernels: no fp32 copies)
    b = _lib.FaBwdParams()
    b.f = p
    b.dout = b.dq = b.dk = b.dv = 0x4000
    delta = a256(2 * 2 * 100 * 3 * 4)
    assert lib.fa_bwd_workspace_size(ctypes.byref(b)) == 2 * a256(one) + a256(table) + delta


def test_fire_workspace(lib):
    """FIRE: the segment table (144 + 132 H floats) and the distance table
    (2 (S + 256) floats) in both workspaces; with d(theta) asked, the
    per-workgroup partials (325 rows per 128-key tile) and their per-head
    reduction (325 x H floats)."""
    def a256(x):
        return (x + 255) // 256 * 256
    p = _dense(bias_mode=_lib.FA_BIAS_FIRE, bias_fire_hidden=32, causal=1)
    B, S, H = p.batch, p.seqlen, p.heads
    tab = a256((144 + 132 * H) * 4) + a256(2 * (S + 256) * 4)
    assert lib.fa_fwd_workspace_size(ctypes.byref(p)) == tab
    b = _lib.FaBwdParams()
    b.f = p
    b.dout = b.dq = b.dk = b.dv = 0x4000
    delta = a256(2 * B * S * H * 4)
    assert lib.fa_bwd_workspace_size(ctypes.byref(b)) == delta + tab
    b.dtable = 0x7000
    parts = B * H * ((S + 127) // 128)
    assert lib.fa_bwd_workspace_size(ctypes.byref(b)) == (
        delta + a256(parts * 325 * 4) + tab + a256(325 * H * 4))


def test_dense_bias_gradient_workspace(lib):
    """The dense bias gradient needs no workspace of its own: a matrix shared
    by the batch (dense_batch 1, B > 1) is summed over the batch in
    registers, one matrix per batch is written in place."""
    def a256(x):
        return (x + 255) // 256 * 256
    b = _lib.FaBwdParams()
    b.f = _dense(bias_mode=_lib.FA_BIAS_DENSE, bias_dense=0x6000, bias_dense_batch=1)
    b.dout = b.dq = b.dk = b.dv = 0x4000
    B, S, H = b.f.batch, b.f.seqlen, b.f.heads
    delta = a256(2 * B * S * H * 4)   # -D and -lse/scale per row
    assert lib.fa_bwd_workspace_size(ctypes.byref(b)) == delta           # no gradient asked
    b.dtable = 0x7000
    assert lib.fa_bwd_workspace_size(ctypes.byref(b)) == delta
    b.f.bias.dense_batch = B
    assert lib.fa_bwd_workspace_size(ctypes.byref(b)) == delta


def test_t5_buckets_checks(lib):
    assert lib.fa_t5_buckets(4, 4, 33, 128, 1, 0x1000, None) == _lib.FA_ERR_UNSUPPORTED
    assert lib.fa_t5_buckets(-1, 4, 32, 128, 1, 0x1000, None) == _lib.FA_ERR_INVALID
    assert lib.fa_t5_buckets(4, 4, 32, 128, 1, None, None) == _lib.FA_ERR_INVALID
    assert lib.fa_t5_buckets(0, 0, 32, 128, 1, None, None) == _lib.FA_OK


def test_mfma_probe_checks(lib):
    flops = ctypes.c_double()
    assert lib.fa_mfma_probe(0, 0x1000, ctypes.byref(flops), None) == _lib.FA_ERR_INVALID
    assert lib.fa_mfma_probe((1 << 20) + 1, 0x1000, ctypes.byref(flops),
                             None) == _lib.FA_ERR_INVALID
    assert lib.fa_mfma_probe(10, None, ctypes.byref(flops), None) == _lib.FA_ERR_INVALID
    assert lib.fa_mfma_probe(10, 0x1000, None, None) == _lib.FA_ERR_INVALID


def test_rmsnorm_checks_and_workspace(lib):
    p = _lib.FaRmsnormBwdParams()
    p.f.rows, p.f.dim, p.f.eps = 100, 768, 1e-6
    p.f.x = p.f.w = p.f.y = p.f.rstd = 0x1000
    p.dy = p.dx = 0x2000
    assert lib.fa_rmsnorm_bwd_workspace_size(ctypes.byref(p)) == 0        # no dw: none
    p.dw = 0x3000
    assert lib.fa_rmsnorm_bwd_workspace_size(ctypes.byref(p)) == 25 * 768 * 4   # one row per wg
    for field, val, status in (("dim", 100, _lib.FA_ERR_UNSUPPORTED),
                               ("dim", 16384, _lib.FA_ERR_UNSUPPORTED),
                               ("dim", 0, _lib.FA_ERR_INVALID),
                               ("rows", -1, _lib.FA_ERR_INVALID),
                               ("eps", -1.0, _lib.FA_ERR_INVALID),
                               ("eps", float("inf"), _lib.FA_ERR_INVALID),
                               ("reserved", 1, _lib.FA_ERR_INVALID),
                               ("x", None, _lib.FA_ERR_INVALID)):
        q = _lib.FaRmsnormFwdParams.from_buffer_copy(p.f)
        setattr(q, field, val)
        assert lib.fa_rmsnorm_fwd(ctypes.byref(q), None) == status, (field, val)
        assert lib.fa_last_error() != b""
    p.dx = None
    assert lib.fa_rmsnorm_bwd(ctypes.byref(p), None, 0, None) == _lib.FA_ERR_INVALID
    p.dx = 0x2000
    # dw asked: the call refuses without its workspace
    assert lib.fa_rmsnorm_bwd(ctypes.byref(p), None, 0, None) == _lib.FA_ERR_WORKSPACE


def test_cross_entropy_checks(lib):
    p = _lib.FaCeBwdParams()
    p.f.rows, p.f.vocab, p.f.z_loss, p.f.ignore_index = 10, 32128, 1e-4, -100
    p.f.logits = p.f.labels = p.f.loss = p.f.lse = 0x1000
    for field, val, status in (("vocab", 1001, _lib.FA_ERR_UNSUPPORTED),
                               ("vocab", 0, _lib.FA_ERR_INVALID),
                               ("rows", -3, _lib.FA_ERR_INVALID),
                               ("z_loss", -1.0, _lib.FA_ERR_INVALID),
                               ("z_loss", float("nan"), _lib.FA_ERR_INVALID),
                               ("labels", None, _lib.FA_ERR_INVALID)):
        q = _lib.FaCeFwdParams.from_buffer_copy(p.f)
        setattr(q, field, val)
        assert lib.fa_ce_fwd(ctypes.byref(q), None) == status, (field, val)
    assert lib.fa_ce_bwd(ctypes.byref(p), None) == _lib.FA_ERR_INVALID   # dloss, dlogits NULL
    q = _lib.FaCeFwdParams.from_buffer_copy(p.f)
    q.rows = 0
    q.logits = q.labels = q.loss = q.lse = None
    assert lib.fa_ce_fwd(ctypes.byref(q), None) == _lib.FA_OK            # empty: nothing to do


def test_noalloc_backward_rejects_problems_beyond_its_scratch(lib):
    """The size check runs on the host before any HIP call: a RoPE backward
    (rotated q, k copies) needs far more than the static scratch."""
    p = _lib.FaBwdParams()
    f = p.f
    f.batch, f.seqlen, f.heads, f.head_dim, f.causal = 2, 16384, 16, 128, 1
    f.scale, f.rope_base = 0.088, 10000.0
    fake = 0x1000   # never dereferenced: the call returns before any launch
    f.q = f.k = f.v = f.o = f.lse = fake
    p.dout = p.dq = p.dk = p.dv = fake
    assert lib.fa_bwd_noalloc(ctypes.byref(p), None) == _lib.FA_ERR_UNSUPPORTED
    assert b"static scratch" in lib.fa_last_error()
    assert lib.fa_bwd_workspace_size(ctypes.byref(p)) > _lib.FA_BWD_NOALLOC_MAX_BYTES
