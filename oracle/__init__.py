"""Oracle: a plain, slow, fp64 CPU statement of what the attention path computes.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or link anything in this package; only
the tests, the smoke check and the CPU-baseline leg of the benchmark do.  The
oracle shares no code, tables or constants with the HIP path: the one module
both sides use is ``synth``, which draws the seeded inputs and holds none of
the method's arithmetic.

Sources (the pages this method is described on):

* FAT5 report (CATIE, Albar & Bourdois), section "Noyau CUDA": the forward
  steps of the bias-extended flash attention.  Scores S are the product of Q
  and the transpose of K; S' is S plus a bias matrix (kernel v1) or a matrix
  filled from the per-head bucket tensor T (kernel v2); P is the softmax of S';
  O is P times V.
* Same report, "Vue d'ensemble de notre travail" and the positional-encoding
  note under "Noyau CUDA": the bias is the T5 relative-position bias; the same
  kernels also serve ALiBi and RoPE.
* Blog on DataCollatorWithFlattening and flash_attn_varlen_func: packed
  batches attend only within each example.
* FAT5 report, note under "Noyau CUDA": FIRE is among the encodings the
  kernels serve; its definition is taken from the FIRE paper the note cites
  (``oracle.fire``).
* FAT5 report, Triton-kernel section and "Torch vs Triton": the fused
  RMSNorm layer and cross-entropy loss with z-loss (``oracle.norm_loss``).

The pages print no formula for the T5 buckets, ALiBi or RoPE, no backward
equations and no worked numbers; the readings taken here are listed in the
module docstrings of ``oracle.attention``.  Every function is pinned by the
``-m "not gpu"`` tests (brute force, closed forms, finite differences,
invariants, library routines).
"""
from .attention import (  # noqa: F401
    t5_bucket,
    alibi_slopes,
    rope_rotate,
    rope_unrotate,
    bf16_round_exact,
    bias_matrix,
    head_sampled,
    attention_fwd,
    attention_bwd,
    varlen_attention_fwd,
    varlen_attention_bwd,
    segment_ids,
)
from .fire import (  # noqa: F401
    fire_bias,
    fire_theta_grad,
    fire_x,
    theta_size as fire_theta_size,
)
from .norm_loss import (  # noqa: F401
    cross_entropy_bwd,
    cross_entropy_fwd,
    rmsnorm_bwd,
    rmsnorm_fwd,
)
