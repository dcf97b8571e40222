"""Plain float64 attention fed by its own QKV projection.

TEST INFRASTRUCTURE ONLY. Imported by tests/ and bench.py's cpu_baseline
leg; never by the library, and it imports nothing from it.

What it computes (devpost "gpu-transformer-optimization", section 2.2: one
projection against the column-concatenated weights, then attention on the
head slices of its output):

    [Q | K | V] = X W_qkv + b_qkv        X [B, S, D], W_qkv [D, 3D], b [3D]
    head h of Q, K, V: columns h*hd .. (h+1)*hd - 1 of each D-wide block
    out[:, :, h*hd:(h+1)*hd] = attention(Q_h, K_h, V_h)   (oracle.attention)

so out is [B, S, D], lse [B, H, S]. The projection is exact in float64; the
attention step is the pinned forward oracle.
"""

from __future__ import annotations

import numpy as np

from .attention import _as_f64, attention

__all__ = ["qkv_attention", "qkv_project"]


def qkv_project(x, w, b, H: int):
    """(q, k, v) as [B, H, S, hd] float64 arrays from X W + b."""
    x, w = _as_f64(x), _as_f64(w)
    B, S, D = x.shape
    if w.shape != (D, 3 * D) or D % H:
        raise ValueError(f"W must be [D, 3D] with H dividing D; got {w.shape}, H={H}")
    y = x @ w
    if b is not None:
        y = y + _as_f64(b).reshape(1, 1, 3 * D)
    hd = D // H
    heads = y.reshape(B, S, 3, H, hd).transpose(2, 0, 3, 1, 4)  # [3, B, H, S, hd]
    return heads[0], heads[1], heads[2]


def qkv_attention(x, w, b, H: int, causal: bool = False, key_len=None, threads: int = 1):
    """(out [B, S, D], lse [B, H, S]) in float64."""
    q, k, v = qkv_project(x, w, b, H)
    o, lse = attention(q, k, v, causal=causal, key_len=key_len, threads=threads)
    B, _, S, hd = o.shape
    return o.transpose(0, 2, 1, 3).reshape(B, S, H * hd), lse
