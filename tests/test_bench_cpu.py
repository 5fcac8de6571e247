"""Host-side checks of bench.py: the one-GPU refusal and the FLOP credit
split.  No GPU is touched."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_convention_shares_sum_to_the_step():
    # FlashAttention convention: forward 2 products, backward 5, so the step
    # is 3.5x the forward; each product credited to exactly one kernel
    assert sum(bench.CONVENTION.values()) == 3.5
    assert bench.CONVENTION["fwd"] == 1.0
    assert bench.OWN_PRODUCTS["bwd_dq"] >= bench.CONVENTION["bwd_dq"]


def test_side_workloads_use_their_config_draws():
    import synth
    for name, prefix in bench.OTHER_ATTENTION.items():
        c = synth.config_by_name(prefix)
        assert c.backward, name
    c4 = synth.config_by_name(bench.OTHER_ATTENTION["varlen"])
    import numpy as np
    lens = synth.draw_varlen_lengths(np.random.default_rng(c4.seed), c4.varlen_total)
    assert len(lens) == 55


def test_dominant_kernel_and_attention_line_with_extra_kernels():
    # the dense-bias batch sum and the FIRE gradient pass are timed beside
    # the three attention kernels but have no convention share: they are
    # listed, never the roofline's kernel, even when the slowest
    import types
    km = {"fwd": 0.6, "bwd_dq": 0.8, "bwd_dkv": 1.0, "bwd_fire": 1.1}
    assert bench.dominant(km) == "bwd_fire"
    assert bench.dominant(km, bench.CONVENTION) == "bwd_dkv"
    assert bench.dominant({"rms_fwd": 0.02, "rms_bwd": 0.03}) == "rms_bwd"
    t = {"ms_step": 3.6, "kernel_ms": km, "host_wall_ms": 3.6,
         "step_ms": {"median": 3.6, "p10": 3.5, "p90": 3.7, "cold_after_1GiB_scrub": 3.9}}
    a = types.SimpleNamespace(steps=20, warmup=5)
    line = bench._attention_line(a, "m", "w", {"batch": 8}, t, fwd_flops=206.2e9)
    assert line["roofline"]["kernel"] == "bwd_dkv"
    assert "bwd_fire" not in line["config"]["kernel_tflops_convention"]
    assert "bwd_fire" in line["config"]["kernel_tflops_own_products"]
    assert line["value"] == round(3.5 * 206.2e9 / 3.6e-3 / 1e12, 2)
