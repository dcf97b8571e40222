"""Float64 CPU oracle for exact multi-head attention (test infrastructure only).

This package is the independent checker for the HIP path. Only the test
suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the library itself never does, and nothing here
imports the library. It shares no code with the HIP kernels.

Contents:
  attention.py  -- the plain definition, materialising the score matrix
                   (devpost "gpu-transformer-optimization", section 2.1,
                   ops (1)-(5)); full tensors and sampled rows.
  backward.py   -- the gradients dq, dk, dv of sum(dout * out) by the chain
                   rule on materialised matrices (rustingstudio
                   "brain/docs/baseline", "Fused attention", describes the
                   fused kernels they check).
  qkv.py        -- attention fed by its own QKV projection X W_qkv + b
                   (devpost "gpu-transformer-optimization", section 2.2).
  gate.py       -- the graded elementwise accuracy rule (devpost
                   "optimized-gpu-kernels-for-transformer-layers",
                   Inspiration; devpost "transformerkernel ... Tesla T4",
                   Inspiration).
"""

from .attention import attention, attention_rows, valid_mask, count_valid_pairs
from .backward import attention_backward
from .gate import gate, budget_fraction
from .qkv import qkv_attention, qkv_project

__all__ = [
    "attention",
    "attention_rows",
    "valid_mask",
    "count_valid_pairs",
    "attention_backward",
    "qkv_attention",
    "qkv_project",
    "gate",
    "budget_fraction",
]
