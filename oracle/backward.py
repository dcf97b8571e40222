"""Plain float64 gradients of exact attention (the backward pass).

TEST INFRASTRUCTURE ONLY. Imported by tests/ and bench.py's cpu_baseline
leg; never by the library, and it imports nothing from it.

With O = A V, A = softmax(S) over visible keys, S = Q K^T / sqrt(d_h) (the
forward definition, devpost "gpu-transformer-optimization", section 2.1),
and dO the gradient of a scalar loss with respect to O, the chain rule
through each op in reverse order gives

    dV = A^T dO                      (through O = A V)
    dA = dO V^T                      (same op, other operand)
    dS = A * (dA - rowsum(A * dA))   (through the row softmax; * elementwise)
    dQ = dS K / sqrt(d_h)            (through S = Q K^T / sqrt(d_h))
    dK = dS^T Q / sqrt(d_h)

Every step is written out on materialised [S, S] matrices, one (batch, head)
at a time. A masked pair has A = 0 and so dS = 0: keys past the key length
receive dK = dV = 0, and a row with no visible key contributes nothing.

The fused backward of rustingstudio "brain/docs/baseline" ("Fused
attention") rebuilds A from the stored log-sum-exp and takes the softmax
row term from dO and O instead of from A: rowsum(A * dA) = rowsum(dO * O)
because O = A V. The oracle keeps the A * dA form above; the identity is
checked by the tests, not used here.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import _as_f64, _key_lengths, valid_mask

__all__ = ["attention_backward"]


def _probs(s: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Row softmax of scaled scores over visible keys; rows with none are 0."""
    s = np.where(mask, s, -np.inf)
    has_key = mask.any(axis=-1)
    m = np.where(has_key, s.max(axis=-1, initial=-np.inf), 0.0)
    p = np.where(mask, np.exp(s - m[..., None]), 0.0)
    denom = np.where(has_key, p.sum(axis=-1), 1.0)
    return p / denom[..., None]


def _softmax_grad(a: np.ndarray, da: np.ndarray) -> np.ndarray:
    """dS from A and dA through the row softmax: A * (dA - rowsum(A * dA))."""
    return a * (da - (a * da).sum(axis=-1, keepdims=True))


def _operand_grads(ds, q, k, a, do, scale):
    """(dQ, dK, dV) through S = Q K^T * scale and O = A V."""
    dq = (ds @ k) * scale
    dk = (np.swapaxes(ds, -1, -2) @ q) * scale
    dv = np.swapaxes(a, -1, -2) @ do
    return dq, dk, dv


def attention_backward(q, k, v, dout, causal: bool = False, key_len=None,
                       heads_per_chunk: int = 256, threads: int = 1):
    """Gradients (dq, dk, dv) of sum(dout * attention(q, k, v)).

    Args:
      q, k, v, dout: [B, H, S, d_h] arrays or tensors, any float dtype
        (upcast exactly to float64).
      causal, key_len: the mask, as for attention().
      heads_per_chunk, threads: bound memory / run chunks of heads
        concurrently; the arithmetic per head is unchanged.
    Returns:
      (dq, dk, dv): float64 arrays [B, H, S, d_h].
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    if q.ndim != 4 or not (q.shape == k.shape == v.shape == do.shape):
        raise ValueError(f"q, k, v, dout must share a [B,H,S,d_h] shape: "
                         f"{q.shape} {k.shape} {v.shape} {do.shape}")
    B, H, S, D = q.shape
    kl = _key_lengths(key_len, B, S)
    scale = 1.0 / math.sqrt(D)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if B * H * S == 0:
        return dq, dk, dv
    heads_per_chunk = max(1, min(heads_per_chunk, (1 << 26) // (S * S)))
    bpc = max(1, heads_per_chunk // max(H, 1))
    jobs = []
    for L in np.unique(kl):
        bs = np.nonzero(kl == L)[0]
        for c0 in range(0, bs.shape[0], bpc):
            jobs.append((int(L), bs[c0:c0 + bpc]))

    def run(job):
        L, sel = job
        mask = valid_mask(S, L, causal)
        kk = k[sel].copy()
        vv = v[sel].copy()
        # padded key / value rows carry zero weight; zero them so that
        # whatever they hold (even NaN) cannot leak in through 0 * NaN
        kk[..., L:, :] = 0.0
        vv[..., L:, :] = 0.0
        qq, dd = q[sel], do[sel]
        a = _probs((qq @ np.swapaxes(kk, -1, -2)) * scale, mask)  # forward, again
        da = dd @ np.swapaxes(vv, -1, -2)                          # dA = dO V^T
        ds = _softmax_grad(a, da)                                  # through softmax
        dq[sel], dk[sel], dv[sel] = _operand_grads(ds, qq, kk, a, dd, scale)

    if threads > 1 and len(jobs) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(run, jobs))
    else:
        for job in jobs:
            run(job)
    return dq, dk, dv
