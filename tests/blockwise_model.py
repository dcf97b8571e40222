"""CPU model of the kernels' tile loop (test infrastructure).

The HIP kernels do not materialise the score matrix: each query tile walks the
key blocks in order and keeps a running row maximum m, running normaliser l
and unnormalised output O, rescaling both by exp(m_old - m_new) whenever the
maximum moves (devpost "gpu-transformer-optimization", section 2.1, the
running-max recurrence). Blocks entirely above the causal diagonal or past the
key length are skipped, not masked.

This module runs that loop in numpy so it can be compared with the
materialising oracle (they must agree to float64 rounding for every tile
size), and, with `emulate=True`, reproduces the kernels' precision choices
(fp32 scores and accumulators, exp2 with the scale folded into one multiply,
probabilities rounded to the input dtype before the P.V product, one rounding
of the output) to predict how much of the error budget the GPU should use.
It shares no code with the oracle or the kernels.
"""

from __future__ import annotations

import math

import numpy as np

LOG2E = 1.4426950408889634


def _round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    if dtype == "bf16x2":
        # split into a bfloat16 head and a bfloat16 remainder (two products)
        hi = _round_to(x, "bf16")
        return hi + _round_to((x - hi).astype(np.float32), "bf16")
    if dtype == "bf16":
        # round-to-nearest-even to bfloat16 via the float32 bit pattern
        b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
        b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
        return b.astype(np.uint32).view(np.float32)
    return x.astype(np.float32)


def running_max_attention(q, k, v, causal=False, key_len=None, BQ=64, PAIR=32,
                          emulate=False, dtype="f16", limit=65504.0, stats=None):
    """The loop with probabilities taken against the running max as it stands
    (no per-block maximum): each chunk of PAIR keys gets p = exp(s c - m); a
    row whose chunk has a probability above `limit` (the input dtype's range;
    the kernels detect it as a non-finite matrix-core row sum) or not finite
    moves m to the chunk's maximum, rescales O and l by exp(m_old - m_new),
    and redoes the chunk. m starts at a finite sentinel (-1e30) so the first
    visible keys of a row always take that path. Same return values as
    tiled_attention; `stats`, if a dict, receives the number of redone
    (row, chunk) pairs under "redo"."""
    q = np.asarray(q); k = np.asarray(k); v = np.asarray(v)
    B, H, S, D = q.shape
    kl = np.full(B, S) if key_len is None else np.clip(np.asarray(key_len).reshape(-1), 0, S)
    ft = np.float32 if emulate else np.float64
    c = ft(LOG2E / math.sqrt(D)) if emulate else 1.0 / math.sqrt(D)
    expf = (lambda x: np.exp2(x.astype(ft)).astype(ft)) if emulate else np.exp
    sentinel = ft(-1e30)
    out = np.zeros((B, H, S, D))
    lse = np.full((B, H, S), -np.inf)
    redo = 0
    with np.errstate(over="ignore", invalid="ignore"):
        for b in range(B):
            L = int(kl[b])
            for h in range(H):
                Q = q[b, h].astype(ft); K = k[b, h].astype(ft); V = v[b, h].astype(ft)
                for q0 in range(0, S, BQ):
                    q1 = min(S, q0 + BQ)
                    rows = np.arange(q0, q1)
                    kend = min(L, q1) if causal else L
                    m = np.full(q1 - q0, sentinel, dtype=ft)
                    l = np.zeros(q1 - q0, dtype=ft)
                    acc = np.zeros((q1 - q0, D), dtype=ft)
                    for k0 in range(0, kend, PAIR):
                        k1 = min(kend, k0 + PAIR)
                        s = (Q[q0:q1] @ K[k0:k1].T).astype(ft)
                        vis = np.ones((q1 - q0, k1 - k0), dtype=bool)
                        if causal:
                            vis &= np.arange(k0, k1)[None, :] <= rows[:, None]
                        s = np.where(vis, s, -np.inf).astype(ft)

                        def probs():
                            p = expf(s * c - m[:, None])
                            p = np.where(vis, p, 0).astype(ft)
                            return _round_to(p, dtype).astype(ft) if emulate else p

                        p = probs()
                        bad = ~np.all(np.isfinite(p) & (p <= limit), axis=1)
                        if bad.any():
                            redo += int(bad.sum())
                            m_new = np.where(bad, np.maximum(m, (s.max(axis=1) * c).astype(ft)), m).astype(ft)
                            alpha = expf(m - m_new)
                            acc = (alpha[:, None] * acc).astype(ft)
                            l = (alpha * l).astype(ft)
                            m = m_new
                            p = probs()
                        l = (l + p.sum(axis=1)).astype(ft)
                        acc = (acc + p @ V[k0:k1]).astype(ft)
                    has = l > 0
                    o = np.where(has[:, None], acc / np.where(has, l, 1)[:, None], 0)
                    if emulate:
                        o = _round_to(o.astype(np.float32), "bf16" if dtype == "bf16x2" else dtype)
                        lg = np.where(has, (m + np.log2(np.where(has, l, 1))) / LOG2E, -np.inf)
                    else:
                        lg = np.where(has, m + np.log(np.where(has, l, 1)), -np.inf)
                    out[b, h, q0:q1] = o
                    lse[b, h, q0:q1] = lg
    if stats is not None:
        stats["redo"] = redo
    return out, lse


def tiled_attention(q, k, v, causal=False, key_len=None, BQ=64, BK=64,
                    emulate=False, dtype="f16"):
    """Online-softmax attention over [B,H,S,D] arrays, one query tile at a time.

    emulate=False: float64 throughout (must equal the definition).
    emulate=True:  float32 arithmetic with the kernels' rounding points.
    Returns (out, lse) as float64 arrays.
    """
    q = np.asarray(q); k = np.asarray(k); v = np.asarray(v)
    B, H, S, D = q.shape
    kl = np.full(B, S) if key_len is None else np.clip(np.asarray(key_len).reshape(-1), 0, S)
    ft = np.float32 if emulate else np.float64
    c = (LOG2E / math.sqrt(D)) if emulate else (1.0 / math.sqrt(D))
    out = np.zeros((B, H, S, D))
    lse = np.full((B, H, S), -np.inf)
    for b in range(B):
        L = int(kl[b])
        for h in range(H):
            Q = q[b, h].astype(ft); K = k[b, h].astype(ft); V = v[b, h].astype(ft)
            for q0 in range(0, S, BQ):
                q1 = min(S, q0 + BQ)
                rows = np.arange(q0, q1)
                kend = min(L, q1) if causal else L     # keys this tile can see
                m = np.full(q1 - q0, -np.inf, dtype=ft)
                l = np.zeros(q1 - q0, dtype=ft)
                acc = np.zeros((q1 - q0, D), dtype=ft)
                for k0 in range(0, kend, BK):
                    k1 = min(kend, k0 + BK)
                    s = (Q[q0:q1] @ K[k0:k1].T).astype(ft)
                    cols = np.arange(k0, k1)
                    vis = np.ones((q1 - q0, k1 - k0), dtype=bool)
                    if causal:
                        vis &= cols[None, :] <= rows[:, None]
                    s = np.where(vis, s, -np.inf)
                    blk_max = s.max(axis=1)
                    m_new = np.maximum(m, blk_max * ft(c)) if emulate else np.maximum(m, blk_max * c)
                    m_use = np.where(np.isfinite(m_new), m_new, 0).astype(ft)
                    if emulate:
                        p = np.exp2((s * ft(c) - m_use[:, None]).astype(ft)).astype(ft)
                        alpha = np.exp2((m - m_use).astype(ft)).astype(ft)
                    else:
                        p = np.exp(s * c - m_use[:, None])
                        alpha = np.exp(m - m_use)
                    p = np.where(vis, p, 0).astype(ft)
                    alpha = np.where(np.isfinite(m), alpha, 0).astype(ft)
                    l = (alpha * l + p.sum(axis=1)).astype(ft)
                    pv = _round_to(p, dtype) if emulate else p
                    acc = (alpha[:, None] * acc + pv @ V[k0:k1]).astype(ft)
                    m = m_new.astype(ft)
                has = l > 0
                o = np.where(has[:, None], acc / np.where(has, l, 1)[:, None], 0)
                if emulate:
                    o = _round_to(o.astype(np.float32), "bf16" if dtype == "bf16x2" else dtype)
                    lg = np.where(has, (m + np.log2(np.where(has, l, 1))) / LOG2E, -np.inf)
                else:
                    lg = np.where(has, m + np.log(np.where(has, l, 1)), -np.inf)
                out[b, h, q0:q1] = o
                lse[b, h, q0:q1] = lg
    return out, lse
