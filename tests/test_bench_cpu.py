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
