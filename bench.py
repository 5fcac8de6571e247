#!/usr/bin/env python
"""Benchmark of the attention hot path on one MI355X.

One step = forward + backward (dQ, dK, dV, table gradient) of causal decoder
self-attention with the unidirectional T5 bias: B8 H12 S4096 D64, 32 buckets,
max distance 128, scale 1.  Inputs are seeded synthetic bf16 N(0,1) tensors
resident in HBM before the timed region.

Prints ONE JSON line.  value = algorithmic TFLOP/s of the whole step with the
FlashAttention convention: forward 4*B*H*S^2*D/2 (causal), backward 2.5x the
forward (5 GEMMs); the backward's D sweep and the hi/lo splits are extra work
that is not counted.  "roofline" reports the dominant kernel (timed alone with
HIP events through the library's fa_set_kernel_timer hook, on the stream it
runs on) against the 2.5 PFLOP/s dense bf16 MFMA peak, credited with its share
of the step's count: forward 1.0x (S, PV), dK/dV kernel 2.0x (S, dP, dV, dK),
dQ kernel 0.5x (dQ), so the three shares sum to the step's 3.5x.  "cpu_baseline" times
the fp64 NumPy oracle on a bounded sample of the same workload on the host.

``--bias dense`` runs the same step with the report's first-kernel semantics
instead: a dense bf16 bias matrix [1, H, S, S] shared by the batch, and its
fp32 gradient, summed over the batch by a fourth kernel (timed beside the
three, outside the convention's shares).  Its roofline is the same MFMA one;
config.hbm_unique gives each kernel's least HBM bytes (every tensor and the
shared matrix once) and that rate, which stays far below 8 TB/s.

``--workload rmsnorm`` and ``--workload ce`` time the report's two other fused
kernels (RMSNorm, cross-entropy with z-loss) forward + backward on the same
32768 tokens (width 768; T5 vocabulary 32128); both are bound by HBM, so their
value is algorithmic GB/s (each tensor read or written once per pass).

``--workload encoder|varlen|alibi|rope`` time the other attention workloads
the same way (forward + backward, kernel times by HIP events), each on the
seeded draw its parity test uses: the bidirectional T5 encoder B16 H12 S1024
D64 (seed 2); 32768 packed tokens in 55 sequences of lognormal lengths (seed
4; 12 heads, D64, bidirectional T5); and the long-context causal B2 H16
S16384 D128 (seed 5) run with ALiBi or with RoPE; ``--workload fire`` the
causal decoder shape and draw with the FIRE bias (32 hidden units, c 0.1,
L 512) and its parameter gradient.  Their cpu_baseline times the oracle on a
few heads (one head at S16384 and for FIRE).

Every line reports the mean step over the K timed steps (ms_per_step, from
which value follows), the median, p10 and p90 of the single steps, and one
cold step run after 1 GiB has been written to evict the inputs from the
caches.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
                    [--bias t5|dense]
                    [--workload attention|rmsnorm|ce|encoder|varlen|alibi|rope|fire]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s (fraction of bf16 MFMA peak), T5-bias, seq 4096 d64"
METRIC_DENSE = ("attention fwd+bwd TFLOP/s, dense bias matrix (first-kernel semantics), "
                "seq 4096 d64")
PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_GBS = 8000.0           # MI355X HBM3E
B, S, H, D = 8, 4096, 12, 64
NB, MD = 32, 128
SEED = 3


def _hip():
    # the HIP runtime torch (and through it libfat5attn) already loaded: its
    # SONAME, so no second runtime copy enters the process
    lib = ctypes.CDLL("libamdhip64.so.7")
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return lib


def _event(hip):
    ev = ctypes.c_void_p()
    assert hip.hipEventCreate(ctypes.byref(ev)) == 0
    return ev


def _elapsed(hip, a, b) -> float:
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
    return ms.value


def run_timed(a, step, kernels, dev):
    """W untimed warm-up steps, then K steps timed with HIP events on the
    launch stream: the whole bracket (ms_per_step), each step on its own
    (median, p10, p90) and each kernel of `kernels` through the library's
    fa_set_kernel_timer hook.  Then one cold step: 1 GiB written first evicts
    the inputs from the 256 MB Infinity Cache and the L2s."""
    import numpy as np
    import torch

    from attention_t5_relative_amd import _lib
    lib = _lib.load()
    hip = _hip()
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = {n: [(_event(hip), _event(hip)) for _ in range(a.steps)] for n in kernels}
    marks = [_event(hip) for _ in range(a.steps + 1)]
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    torch.cuda.synchronize()
    hip.hipEventRecord(marks[0], stream)
    wall0 = time.perf_counter()
    for i in range(a.steps):
        for n, kid in kernels.items():
            lib.fa_set_kernel_timer(kid, evs[n][i][0], evs[n][i][1])
        step()
        hip.hipEventRecord(marks[i + 1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    for kid in kernels.values():
        lib.fa_set_kernel_timer(kid, None, None)
    steps_ms = np.array([_elapsed(hip, marks[i], marks[i + 1]) for i in range(a.steps)])
    res = {
        "ms_step": _elapsed(hip, marks[0], marks[-1]) / a.steps,
        "kernel_ms": {n: sum(_elapsed(hip, s0, s1) for s0, s1 in evs[n]) / a.steps
                      for n in kernels},
        "host_wall_ms": wall / a.steps * 1e3,
        "step_ms": {"median": round(float(np.median(steps_ms)), 4),
                    "p10": round(float(np.percentile(steps_ms, 10)), 4),
                    "p90": round(float(np.percentile(steps_ms, 90)), 4)},
    }
    scrub = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    c0, c1 = _event(hip), _event(hip)
    scrub.fill_(1.0)
    hip.hipEventRecord(c0, stream)
    step()
    hip.hipEventRecord(c1, stream)
    torch.cuda.synchronize()
    res["step_ms"]["cold_after_1GiB_scrub"] = round(_elapsed(hip, c0, c1), 4)
    del scrub
    return res


def mfma_probe(dev, iters=20000, reps=3):
    """The chip's sustained dense bf16 MFMA rate (TFLOP/s), measured by the
    library's probe kernel: best of `reps` timed calls after one warm-up."""
    import torch

    from attention_t5_relative_amd import _lib
    lib = _lib.load()
    hip = _hip()
    sink = torch.empty(_lib.FA_MFMA_PROBE_LANES, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    flops = ctypes.c_double()
    best = 0.0
    for r in range(reps + 1):
        e0, e1 = _event(hip), _event(hip)
        hip.hipEventRecord(e0, stream)
        st = lib.fa_mfma_probe(iters, ctypes.c_void_p(sink.data_ptr()), ctypes.byref(flops),
                               stream)
        if st != _lib.FA_OK:
            raise RuntimeError(f"fa_mfma_probe: {lib.fa_last_error().decode()}")
        hip.hipEventRecord(e1, stream)
        torch.cuda.synchronize()
        if r > 0:
            best = max(best, flops.value / (_elapsed(hip, e0, e1) * 1e-3) / 1e12)
    return best


def _traffic(kernel: str):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_c3_b8h12s4096d64_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    src = fields.get("source_sha256")
    cur = hashlib.sha256()
    for f in ("attention_t5_relative_amd/csrc/bwd.hip", "attention_t5_relative_amd/csrc/fwd.hip",
              "attention_t5_relative_amd/csrc/fa_device.h"):
        cur.update(open(os.path.join(ROOT, f), "rb").read())
    if src != cur.hexdigest():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, pairs, dense=None):
    """The fp64 oracle, as it stands, on `pairs` (batch, head) of the workload
    (with `dense`, the dense bias matrix [1, H, S, S] as float64)."""
    import oracle
    q, k, v, do = (inp.f64(n) for n in ("q", "k", "v", "do"))
    kw = dict(scale=1.0, causal=True, bias="t5", table=inp.table, num_buckets=NB,
              max_distance=MD, bidirectional=False)
    if dense is not None:
        kw = dict(scale=1.0, causal=True, bias="dense", dense=dense)
    work = [lambda: oracle.attention_fwd(q, k, v, pairs=pairs, **kw),
            lambda: oracle.attention_bwd(q, k, v, do, pairs=pairs, **kw)]
    flops = 3.5 * 4.0 * S * S * D / 2.0 * len(pairs)
    return _time_oracle(work, flops, f"{len(pairs)} of {B * H} (batch, head) pairs of the "
                                     "same workload")


NL_ROWS, RMS_DIM, CE_VOCAB, Z_LOSS = 32768, 768, 32128, 1e-4


def bench_norm_loss(a):
    """RMSNorm or cross-entropy (+ z-loss) forward + backward, GB/s."""
    import numpy as np
    import torch

    import attention_t5_relative_amd as fa
    import synth
    from attention_t5_relative_amd import _lib

    dev = torch.device("cuda:0")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(dev)

    N = NL_ROWS
    if a.workload == "rmsnorm":
        d = RMS_DIM
        xb, wb, dyb = synth.draw_rmsnorm(SEED, N, d)
        x, w, dy = up(xb), up(wb), up(dyb)
        y, dx = torch.empty_like(x), torch.empty_like(x)
        rstd = torch.empty(N, dtype=torch.float32, device=dev)
        dw = torch.empty(d, dtype=torch.float32, device=dev)
        lib = _lib.load()
        p = _lib.FaRmsnormBwdParams()
        p.f = fa.api._rms_params(x, w, y, rstd, 1e-6)
        p.dy, p.dx, p.dw = dy.data_ptr(), dx.data_ptr(), dw.data_ptr()
        ws = torch.empty(max(1, lib.fa_rmsnorm_bwd_workspace_size(ctypes.byref(p))),
                         dtype=torch.uint8, device=dev)

        def step():
            fa.fa_rmsnorm_fwd(x, w, y, rstd, eps=1e-6)
            fa.fa_rmsnorm_bwd(x, w, rstd, dy, dx, dw, eps=1e-6, workspace=ws)

        kernels = {"rmsnorm_fwd": _lib.FA_KERNEL_RMSNORM_FWD,
                   "rmsnorm_bwd": _lib.FA_KERNEL_RMSNORM_BWD}
        t = N * d * 2
        abytes = {"rmsnorm_fwd": 2 * t + 2 * d + 4 * N,          # x in, y out, w, rstd
                  "rmsnorm_bwd": 3 * t + 2 * d + 4 * N}          # x, dy in, dx out (dw partials extra)
        step_bytes = abytes["rmsnorm_fwd"] + abytes["rmsnorm_bwd"] + 4 * d
        metric = "rmsnorm fwd+bwd GB/s (algorithmic bytes), 32768 x 768 bf16"
        workload = ("RMSNorm (no mean, no bias, eps 1e-6) forward + backward (dx, dw) over "
                    "32768 rows x 768 bf16, weight bf16, dw fp32")
        cfg = {"rows": N, "dim": d}
    else:
        V = CE_VOCAB
        zb, yb, gb = synth.draw_cross_entropy(SEED, N, V)
        z = up(zb)
        lab = torch.from_numpy(yb).to(dev)
        g = torch.from_numpy(gb).to(dev)
        loss = torch.empty(N, dtype=torch.float32, device=dev)
        lse = torch.empty_like(loss)
        dz = torch.empty_like(z)
        del zb

        def step():
            fa.fa_ce_fwd(z, lab, loss, lse, z_loss=Z_LOSS)
            fa.fa_ce_bwd(z, lab, lse, g, dz, z_loss=Z_LOSS)

        kernels = {"ce_fwd": _lib.FA_KERNEL_CE_FWD, "ce_bwd": _lib.FA_KERNEL_CE_BWD}
        t = N * V * 2
        abytes = {"ce_fwd": t + 4 * N + 8 * N,            # logits, labels in; loss, lse out
                  "ce_bwd": 2 * t + 12 * N}                # logits in, dlogits out; labels, lse, dloss
        step_bytes = abytes["ce_fwd"] + abytes["ce_bwd"]
        metric = "cross-entropy + z-loss fwd+bwd GB/s (algorithmic bytes), 32768 x 32128 bf16"
        workload = ("per-row cross-entropy with z-loss 1e-4 forward + backward over 32768 rows "
                    "x 32128 bf16 logits (T5 vocabulary), 10% ignored labels")
        cfg = {"rows": N, "vocab": V, "z_loss": Z_LOSS}

    t = run_timed(a, step, kernels, dev)
    ms_step, kernel_ms = t["ms_step"], t["kernel_ms"]
    dom = dominant(kernel_ms)
    gbs = abytes[dom] / (kernel_ms[dom] * 1e-3) / 1e9
    value = step_bytes / (ms_step * 1e-3) / 1e9
    line = {
        "metric": metric, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": dict({"workload": workload, "parallelism": "none (one GPU)",
                        "kernel_ms": {n: round(v, 4) for n, v in kernel_ms.items()},
                        "step_ms": t["step_ms"],
                        "frac_of_hbm_peak": round(value / PEAK_GBS, 4)}, **cfg),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(gbs, 1), "peak": PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = norm_loss_cpu_baseline(a.workload)
    print(json.dumps(line), flush=True)
    return 0


def norm_loss_cpu_baseline(workload):
    """The fp64 oracle on a bounded sample of the rows, scaled to GB/s of the
    same algorithmic bytes per row."""
    import numpy as np
    import oracle
    import synth
    rows = NL_ROWS if workload == "rmsnorm" else 2048
    t0 = time.perf_counter()
    if workload == "rmsnorm":
        xb, wb, dyb = synth.draw_rmsnorm(SEED, rows, RMS_DIM)
        x, w, dy = (synth.bf16_bits_to_f32(b).astype(np.float64) for b in (xb, wb, dyb))
        t0 = time.perf_counter()
        oracle.rmsnorm_fwd(x, w, 1e-6)
        oracle.rmsnorm_bwd(x, w, dy, 1e-6)
        per_row = 10 * RMS_DIM + 8
    else:
        zb, yb, gb = synth.draw_cross_entropy(SEED, rows, CE_VOCAB)
        z = synth.bf16_bits_to_f32(zb).astype(np.float64)
        t0 = time.perf_counter()
        oracle.cross_entropy_fwd(z, yb, Z_LOSS)
        oracle.cross_entropy_bwd(z, yb, gb.astype(np.float64), Z_LOSS)
        per_row = 6 * CE_VOCAB + 24
    dt = time.perf_counter() - t0
    return {"value": round(rows * per_row / dt / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",   # element-wise NumPy: one thread
            "sample": f"{rows} of {NL_ROWS} rows of the same workload, fp64 NumPy on the host "
                      f"({dt:.2f} s); same algorithmic bytes per row as the GPU value"}


OTHER_ATTENTION = {"encoder": "c2", "varlen": "c4", "alibi": "c5a", "rope": "c5b", "fire": "c3"}
# FIRE side line: the causal decoder shape with the FIRE bias in place of T5
FIRE_HIDDEN, FIRE_C, FIRE_L = 32, 0.1, 512.0

# FlashAttention convention for a fwd+bwd step: the forward's two products
# count 1.0x, the backward's five 2.5x.  Per kernel the step's 3.5x is split
# so each product counts once: fwd S, PV = 1.0; dkv S, dP, dV, dK = 2.0; dq
# dQ = 0.5.  OWN_PRODUCTS credits each kernel with every product its outputs
# need (the dq kernel recomputes S and dP too): shown beside, never in value.
# The dense-bias batch sum and the FIRE gradient pass recompute S and dP
# (1.0x) for outputs the convention does not count: they have no share, so
# they are timed and listed but never the roofline's kernel.
CONVENTION = {"fwd": 1.0, "bwd_dq": 0.5, "bwd_dkv": 2.0}
OWN_PRODUCTS = {"fwd": 1.0, "bwd_dq": 1.5, "bwd_dkv": 2.0, "bwd_dbias_sum": 1.0, "bwd_fire": 1.0}


def dominant(kernel_ms, shares=None):
    """The slowest timed kernel; with ``shares``, the slowest of those that
    have a share of the step's flop count (the others are timed and listed
    only)."""
    names = [n for n in kernel_ms if shares is None or n in shares]
    return max(names, key=kernel_ms.get)


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 0) for i in threadpool_info()] or [0])
    except Exception:  # noqa: BLE001
        threads = 0
    return threads or (os.cpu_count() or 1)


def _time_oracle(work, flops, sample):
    """Run the oracle calls in `work` once on the host; TFLOP/s of the same
    algorithmic count as the GPU value."""
    threads = _oracle_threads()
    t0 = time.perf_counter()
    for fn in work:
        fn()
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{sample}, fwd+bwd in fp64 NumPy on the host ({dt:.1f} s); same "
                      f"algorithmic flop count per unit as the GPU value",
            "host": _host_info(threads)}


def _host_info(threads):
    model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(),
            "sched_affinity": len(os.sched_getaffinity(0)), "blas_threads": threads}


def _attention_line(a, metric, workload, shape, t, fwd_flops, traffic=None):
    """The JSON line of an attention fwd+bwd step from run_timed's result."""
    ms_step, kernel_ms = t["ms_step"], t["kernel_ms"]
    dom = dominant(kernel_ms, CONVENTION)

    def tf(share, n):
        return round(share * fwd_flops / (kernel_ms[n] * 1e-3) / 1e12, 2)

    achieved = tf(CONVENTION[dom], dom)
    value = 3.5 * fwd_flops / (ms_step * 1e-3) / 1e12
    probe = t.get("mfma_probe_tflops")
    extra = {}
    if probe:
        extra["mfma_probe"] = {"tflops": round(probe, 1),
                               "step_frac_of_probe": round(value / probe, 4),
                               "dominant_frac_of_probe": round(achieved / probe, 4)}
    return {
        "metric": metric, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": dict({"workload": workload, "parallelism": "none (one GPU)",
                        "frac_of_peak": round(value / PEAK_TFLOPS, 4),
                        "kernel_ms": {n: round(v, 4) for n, v in kernel_ms.items()},
                        "kernel_tflops_convention": {n: tf(CONVENTION[n], n) for n in kernel_ms
                                                     if n in CONVENTION},
                        "kernel_tflops_own_products": {n: tf(OWN_PRODUCTS[n], n)
                                                       for n in kernel_ms},
                        "step_ms": t["step_ms"],
                        "host_wall_ms_per_step": round(t["host_wall_ms"], 4)}, **extra, **shape),
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved,
                     "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": traffic},
        "cpu_baseline": None,
    }


def _attn_kernels(extra=()):
    from attention_t5_relative_amd import _lib
    ids = {"fwd": _lib.FA_KERNEL_FWD, "bwd_dq": _lib.FA_KERNEL_BWD_DQ,
           "bwd_dkv": _lib.FA_KERNEL_BWD_DKV, "bwd_dbias_sum": _lib.FA_KERNEL_BWD_DBIAS_SUM,
           "bwd_fire": _lib.FA_KERNEL_BWD_FIRE}
    return {n: ids[n] for n in ("fwd", "bwd_dq", "bwd_dkv") + tuple(extra)}


def bench_other_attention(a):
    """Forward + backward of one of the other attention workloads, on the
    same seeded draw its parity test uses; one JSON line."""
    import numpy as np
    import torch

    import attention_t5_relative_amd as fa
    import synth
    from attention_t5_relative_amd import _lib

    dev = torch.device("cuda:0")
    lib = _lib.load()
    c = synth.config_by_name(OTHER_ATTENTION[a.workload])

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(dev)

    H, Dh = c.heads, c.head_dim
    table = slopes = None
    fire = a.workload == "fire"
    if c.varlen_total:
        inp = synth.draw_varlen(c.seed, c.varlen_total, H, Dh, num_buckets=c.num_buckets)
        lens = inp.lengths
        cu = torch.from_numpy(inp.cu_seqlens).to(dev)
        T = int(lens.sum())
        q, k, v, do = (up(getattr(inp, n)) for n in ("q", "k", "v", "do"))
        table = torch.from_numpy(inp.table).to(dev)
        bias = fa.T5Bias(table, c.num_buckets, c.max_distance, c.bidirectional)
        dtable = torch.empty_like(table)
        o = torch.empty_like(q)
        lse = torch.empty((H, T), dtype=torch.float32, device=dev)
        mx = int(lens.max())
        fwd_flops = 4.0 * H * Dh * float((lens.astype(np.float64) ** 2).sum())
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        p = _lib.FaVarlenBwdParams()
        p.f = fa.api._varlen_params(q, k, v, o, lse, cu, mx, c.scale, c.causal, bias, 0.0)
        p.dout, p.dq, p.dk, p.dv, p.dtable = (do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                              dv.data_ptr(), dtable.data_ptr())
        wsb = torch.empty(max(1, lib.fa_varlen_bwd_workspace_size(ctypes.byref(p))),
                          dtype=torch.uint8, device=dev)

        def step():
            fa.fa_varlen_fwd(q, k, v, o, lse, cu, mx, scale=c.scale, causal=c.causal, bias=bias)
            fa.fa_varlen_bwd(q, k, v, o, lse, do, dq, dk, dv, cu, mx, dtable, scale=c.scale,
                             causal=c.causal, bias=bias, workspace=wsb)
        workload = (f"packed encoder self-attention fwd+bwd, {T} tokens in {len(lens)} "
                    "sequences (lognormal(6,1) lengths clipped to 16..4096, seed "
                    f"{c.seed}), H{H} D{Dh}, bidirectional T5 bias (32 buckets, max distance "
                    "128), scale 1")
        shape = {"tokens": T, "sequences": int(len(lens)), "heads": H, "head_dim": Dh,
                 "causal": c.causal}
    else:
        inp = synth.draw_dense(c.seed, c.batch, c.seqlen, H, Dh, num_buckets=c.num_buckets,
                               with_table=c.bias == "t5")
        q, k, v, do = (up(getattr(inp, n)) for n in ("q", "k", "v", "do"))
        Bq, Sq = c.batch, c.seqlen
        rope = c.rope_base or 0.0
        dtable = None
        if fire:
            theta = synth.draw_fire_theta(c.seed, H, FIRE_HIDDEN, c=FIRE_C, threshold=FIRE_L)
            table = torch.from_numpy(theta).to(dev)
            bias = fa.FireBias(table, FIRE_HIDDEN)
            dtable = torch.empty_like(table)
            workload = (f"causal decoder self-attention fwd+bwd with the FIRE bias (MLP "
                        f"{FIRE_HIDDEN} hidden units, c {FIRE_C}, L {FIRE_L:g}) and its "
                        f"parameter gradient, B{Bq} H{H} S{Sq} D{Dh}, scale 1")
        elif c.bias == "t5":
            table = torch.from_numpy(inp.table).to(dev)
            bias = fa.T5Bias(table, c.num_buckets, c.max_distance, c.bidirectional)
            dtable = torch.empty_like(table)
            workload = (f"encoder self-attention fwd+bwd, B{Bq} H{H} S{Sq} D{Dh}, "
                        "bidirectional T5 bias (32 buckets, max distance 128), scale 1")
        elif c.bias == "alibi":
            slopes = synth.alibi_slope_values(H)
            bias = fa.ALiBi(torch.from_numpy(slopes).to(dev))
            workload = (f"long-context causal attention fwd+bwd, B{Bq} H{H} S{Sq} D{Dh}, "
                        "ALiBi slopes 2^(-8h/16), scale 1/sqrt(128)")
        else:
            bias = None
            workload = (f"long-context causal attention fwd+bwd, B{Bq} H{H} S{Sq} D{Dh}, RoPE "
                        "base 10000 in the kernels, scale 1/sqrt(128)")
        o = torch.empty_like(q)
        lse = torch.empty((Bq, H, Sq), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        fwd_flops = 4.0 * Bq * H * Sq * Sq * Dh / (2.0 if c.causal else 1.0)
        p = _lib.FaBwdParams()
        p.f = fa.api._fwd_params(q, k, v, o, lse, c.scale, c.causal, bias, rope)
        p.dout, p.dq, p.dk, p.dv = do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
        p.dtable = None if dtable is None else dtable.data_ptr()
        wsb = torch.empty(max(1, lib.fa_bwd_workspace_size(ctypes.byref(p))), dtype=torch.uint8,
                          device=dev)

        def step():
            fa.fa_fwd(q, k, v, o, lse, scale=c.scale, causal=c.causal, bias=bias,
                      rope_base=rope)
            fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, dtable, scale=c.scale, causal=c.causal,
                      bias=bias, rope_base=rope, workspace=wsb)
        shape = {"batch": Bq, "heads": H, "seq_len": Sq, "head_dim": Dh, "causal": c.causal}

    t = run_timed(a, step, _attn_kernels(("bwd_fire",) if fire else ()), dev)
    t["mfma_probe_tflops"] = mfma_probe(dev)
    tag = f"{c.name} shape, FIRE bias" if fire else c.name
    line = _attention_line(a, f"attention fwd+bwd TFLOP/s, {a.workload} workload ({tag})",
                           workload, shape, t, fwd_flops)
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = other_cpu_baseline(c, inp, slopes,
                                                  theta if fire else None)
    print(json.dumps(line), flush=True)
    return 0


def other_cpu_baseline(c, inp, slopes, fire_theta=None):
    """The oracle on a bounded sample of one side workload: whole heads
    (dense) or whole sequences of a few heads (packed)."""
    import numpy as np
    import oracle
    kw = dict(scale=c.scale, causal=c.causal, bias=c.bias, num_buckets=c.num_buckets,
              max_distance=c.max_distance, bidirectional=c.bidirectional)
    if fire_theta is not None:
        kw["bias"] = "fire"
        kw["fire"] = fire_theta.astype(np.float64)
        kw["fire_hidden"] = FIRE_HIDDEN
    elif c.bias == "t5":
        kw["table"] = inp.table.astype(np.float64)
    if c.bias == "alibi":
        kw["slopes"] = slopes.astype(np.float64)
    if c.rope_base:
        kw["rope_base"] = c.rope_base
    f = {n: inp.f64(n) for n in ("q", "k", "v", "do")}
    if c.varlen_total:
        heads = [0, 5, 11]
        cu = inp.cu_seqlens
        work = [lambda: oracle.varlen_attention_fwd(f["q"], f["k"], f["v"], cu, heads=heads,
                                                    **kw),
                lambda: oracle.varlen_attention_bwd(f["q"], f["k"], f["v"], f["do"], cu,
                                                    heads=heads, **kw)]
        flops = 3.5 * 4.0 * c.head_dim * float((inp.lengths.astype(np.float64) ** 2).sum())
        return _time_oracle(work, flops * len(heads),
                            f"all {len(inp.lengths)} sequences of heads {heads} of {c.heads}")
    npairs = 1 if c.seqlen >= 16384 or fire_theta is not None else 48
    pairs = [(i % c.batch, (5 * i + 1) % c.heads) for i in range(npairs)]
    work = [lambda: oracle.attention_fwd(f["q"], f["k"], f["v"], pairs=pairs, **kw),
            lambda: oracle.attention_bwd(f["q"], f["k"], f["v"], f["do"], pairs=pairs, **kw)]
    flops = 3.5 * 4.0 * c.seqlen * c.seqlen * c.head_dim / (2.0 if c.causal else 1.0)
    return _time_oracle(work, flops * npairs,
                        f"{npairs} of {c.batch * c.heads} (batch, head) pairs {pairs[:4]}"
                        f"{'...' if npairs > 4 else ''} of the same workload")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-pairs", type=int, default=12)
    ap.add_argument("--bias", choices=("t5", "dense"), default="t5")
    ap.add_argument("--workload", choices=("attention", "rmsnorm", "ce") + tuple(OTHER_ATTENTION),
                    default="attention")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one device-to-device copy of this many MiB before the "
                         "timed steps (a known-size kernel to calibrate HBM byte counters)")
    a = ap.parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE {world}); "
              "this library has no multi-GPU path.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import attention_t5_relative_amd as fa
    import synth
    from attention_t5_relative_amd import _lib

    if a.workload in OTHER_ATTENTION:
        return bench_other_attention(a)
    if a.workload != "attention":
        return bench_norm_loss(a)

    dev = torch.device("cuda:0")
    inp = synth.draw_dense(SEED, B, S, H, D)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(dev)

    q, k, v, do = (up(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    dense_bits = None
    if a.bias == "dense":
        dense_bits = synth.draw_dense_bias(SEED + 100, 1, H, S)
        bias = fa.DenseBias(up(dense_bits))
        dtable = torch.empty((1, H, S, S), dtype=torch.float32, device=dev)
    else:
        table = torch.from_numpy(inp.table).to(dev)
        bias = fa.T5Bias(table, NB, MD, bidirectional=False)
        dtable = torch.empty_like(table)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)

    def step():
        fa.fa_fwd(q, k, v, o, lse, scale=1.0, causal=True, bias=bias)
        fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, dtable, scale=1.0, causal=True, bias=bias,
                  workspace=wsb)

    # workspace sized once, outside the timed region
    lib = _lib.load()
    p = _lib.FaBwdParams()
    p.f = fa.api._fwd_params(q, k, v, o, lse, 1.0, True, bias, 0.0)
    p.dout, p.dq, p.dk, p.dv, p.dtable = (do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                          dv.data_ptr(), dtable.data_ptr())
    wsb = torch.empty(lib.fa_bwd_workspace_size(ctypes.byref(p)), dtype=torch.uint8, device=dev)

    if a.copy_mib > 0:
        # one device-to-device copy of known size before the timed steps: the
        # byte counters of this kernel calibrate FETCH_SIZE / WRITE_SIZE
        src = torch.ones(a.copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    t = run_timed(a, step, _attn_kernels(("bwd_dbias_sum",) if a.bias == "dense" else ()), dev)
    t["mfma_probe_tflops"] = mfma_probe(dev)
    fwd_flops = 4.0 * B * H * S * S * D / 2.0
    shape = {"batch": B, "heads": H, "seq_len": S, "head_dim": D, "causal": True}
    if a.bias == "dense":
        workload = ("causal decoder self-attention fwd+bwd with a dense bf16 bias matrix "
                    "[1, H, S, S] shared by the batch and its fp32 gradient, B8 H12 S4096 D64, "
                    "scale 1")
        line = _attention_line(a, METRIC_DENSE, workload, shape, t, fwd_flops)
        # HBM side of each kernel: the bytes it must move at least (each bf16
        # tensor, the per-row LSE / D and the shared matrix [1, H, S, S]
        # read or written once; the batch sum writes the fp32 gradient of the
        # visible pairs once), and that over its time
        kernel_ms = t["kernel_ms"]
        t_bytes = B * S * H * D * 2
        rows = B * H * S * 4
        vis = H * S * (S + 1) / 2
        ubytes = {"fwd": 4 * t_bytes + rows + vis * 2,
                  "bwd_dq": 6 * t_bytes + 2 * rows + vis * 2,
                  "bwd_dkv": 6 * t_bytes + 2 * rows + vis * 2,
                  "bwd_dbias_sum": 4 * t_bytes + 2 * rows + vis * (2 + 4)}
        line["config"]["hbm_unique"] = {
            n: {"bytes": int(ubytes[n]),
                "gbs": round(ubytes[n] / (kernel_ms[n] * 1e-3) / 1e9, 1),
                "frac": round(ubytes[n] / (kernel_ms[n] * 1e-3) / 1e9 / PEAK_GBS, 4)}
            for n in kernel_ms}
    else:
        workload = ("causal decoder self-attention fwd+bwd with unidirectional T5 bias "
                    "(32 buckets, max distance 128), B8 H12 S4096 D64, scale 1")
        line = _attention_line(a, METRIC, workload, shape, t, fwd_flops)
        line["roofline"]["traffic"] = _traffic(line["roofline"]["kernel"])
    if not a.no_cpu_baseline:
        pairs = [(i % B, (5 * i + 1) % H) for i in range(min(a.cpu_pairs, B * H))]
        dense = None
        if dense_bits is not None:
            dense = synth.bf16_bits_to_f32(dense_bits).astype(np.float64)
        line["cpu_baseline"] = cpu_baseline(inp, pairs, dense)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
