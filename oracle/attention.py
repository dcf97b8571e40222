"""Plain float64 exact attention: the oracle the HIP path is checked against.

TEST INFRASTRUCTURE ONLY. Imported by tests/, __graft_entry__.smoke() and
the cpu_baseline leg of bench.py; never by the library.

What it computes is the textbook definition written out, one (batch, head)
at a time, with the whole score matrix materialised:

    (1) S = Q K^T            (2) S = S / sqrt(d_h)       (3) S = mask(S)
    (4) A = softmax(S) along the key axis                (5) O = A V

(devpost "gpu-transformer-optimization", section 2.1, ops (1)-(5)). The
online (running max / running sum) recurrence of the same section is what
the kernels use; that section states the recurrence reaches exactly this
result in exact arithmetic, so the oracle is the definition, not the
recurrence.

Readings of points the pages leave open (each repeated in the design notes):
  * mask = right-padded key length AND (optionally) causal: key j is visible
    to query i iff j < L_b and (not causal or j <= i). Padded query rows
    (i >= L_b) therefore attend to keys 0..L_b-1. Under causal masking rows
    i < L_b are identical to causal-only attention (the redundancy argument
    in the same section, "The mask trick").
  * the mask is additive -inf, so masked keys get exactly zero weight and
    padded K/V values (even NaN) never enter the result.
  * a row with no visible key (only possible when L_b == 0) has out = 0 and
    lse = -inf.
  * lse is the natural log of sum_j exp(scaled score), including the
    1/sqrt(d_h) scale; it is the per-row log-sum-exp a fused forward stores
    for its backward (rustingstudio "brain/docs/baseline", "Fused attention").
  * inputs are upcast exactly from their storage dtype to float64; all
    arithmetic is float64.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["attention", "attention_rows", "valid_mask", "count_valid_pairs"]


def _as_f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or torch tensor (any float dtype)."""
    if hasattr(x, "detach"):  # torch tensor, possibly on a device
        import torch
        x = x.detach()
        if x.is_cuda:
            x = x.cpu()
        x = x.to(dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _key_lengths(key_len, B: int, S: int) -> np.ndarray:
    """Per-batch valid key count, clamped to [0, S]; None means all S valid."""
    if key_len is None:
        return np.full(B, S, dtype=np.int64)
    if hasattr(key_len, "detach"):
        key_len = key_len.detach().cpu().numpy()
    kl = np.asarray(key_len, dtype=np.int64).reshape(-1)
    if kl.shape[0] != B:
        raise ValueError(f"key_len has {kl.shape[0]} entries, expected B={B}")
    return np.clip(kl, 0, S)


def valid_mask(S: int, L: int, causal: bool, rows=None) -> np.ndarray:
    """Boolean [n_rows, S]: True where query row i may attend to key j.

    Key j is visible iff j < L and (not causal or j <= i)
    (section 2.1, op (3): the causal / padding mask).
    """
    i = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(S)
    m = (j[None, :] < L) & np.ones((i.shape[0], 1), dtype=bool)
    if causal:
        m &= j[None, :] <= i[:, None]
    return m


def _softmax_rows(s: np.ndarray, mask: np.ndarray, v: np.ndarray):
    """Ops (3)-(5) on materialised scaled scores s [..., n, S] with v [..., S, D].

    Returns (out [..., n, D], lse [..., n]) in float64.
    """
    s = np.where(mask, s, -np.inf)                       # (3) additive -inf mask
    has_key = mask.any(axis=-1)
    m = np.where(has_key, s.max(axis=-1, initial=-np.inf), 0.0)
    p = np.exp(s - m[..., None])                         # (4) exp(s - rowmax)
    p = np.where(mask, p, 0.0)
    denom = p.sum(axis=-1)
    safe = np.where(has_key, denom, 1.0)
    out = (p @ v) / safe[..., None]                      # (5) A V, A = p / sum p
    out = np.where(has_key[..., None], out, 0.0)
    lse = np.where(has_key, m + np.log(safe), -np.inf)
    return out, lse


def attention(q, k, v, causal: bool = False, key_len=None, heads_per_chunk: int = 512,
              threads: int = 1):
    """Exact attention over [B, H, S, d_h] inputs.

    Args:
      q, k, v: arrays or tensors of shape [B, H, S, d_h], any float dtype.
      causal:  apply the causal mask (key j visible to query i only if j <= i).
      key_len: per-batch valid key count (length B) or None for all S valid.
      heads_per_chunk: how many (b, h) score matrices to materialise at once
        (further capped so one chunk's scores stay near 1 GB); only bounds
        memory, the arithmetic per head is unchanged.
      threads: independent chunks of heads evaluated concurrently (numpy
        releases the GIL); the arithmetic per head is unchanged.

    Returns:
      (out, lse): float64 arrays [B, H, S, d_h] and [B, H, S].
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q, k, v must share a [B,H,S,d_h] shape: {q.shape} {k.shape} {v.shape}")
    B, H, S, D = q.shape
    kl = _key_lengths(key_len, B, S)
    scale = 1.0 / math.sqrt(D)                           # (2) 1 / sqrt(d_h)
    out = np.zeros((B, H, S, D), dtype=np.float64)
    lse = np.full((B, H, S), -np.inf, dtype=np.float64)
    if B * H * S == 0:
        return out, lse
    # Batches sharing a key length share a mask; group them so one matmul call
    # covers many heads.
    heads_per_chunk = max(1, min(heads_per_chunk, (1 << 27) // (S * S)))
    bpc = max(1, heads_per_chunk // max(H, 1))
    jobs = []
    for L in np.unique(kl):
        bs = np.nonzero(kl == L)[0]
        for c0 in range(0, bs.shape[0], bpc):
            jobs.append((int(L), bs[c0:c0 + bpc]))

    def run(job):
        L, sel = job
        mask = valid_mask(S, L, causal)
        s = (q[sel] @ np.swapaxes(k[sel], -1, -2)) * scale        # (1), (2)
        # Padded value rows (j >= L) carry zero weight; zero them so that
        # whatever they hold (even NaN) cannot leak in through 0 * NaN.
        vv = v[sel].copy()
        vv[..., L:, :] = 0.0
        o, l = _softmax_rows(s, mask, vv)
        out[sel] = o
        lse[sel] = l

    if threads > 1 and len(jobs) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(run, jobs))
    else:
        for job in jobs:
            run(job)
    return out, lse


def attention_rows(q, k, v, rows, causal: bool = False, key_len=None):
    """Exact attention for selected query rows only.

    Args:
      q, k, v: [B, H, S, d_h] arrays or tensors (device tensors are copied
        back one head at a time, so only the heads named in `rows` move).
      rows: integer array [n, 3] of (b, h, i) triples.
    Returns:
      (out [n, d_h], lse [n]) in float64, in the order of `rows`.
    """
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    B, H, S, D = tuple(q.shape)
    kl = _key_lengths(key_len, B, S)
    scale = 1.0 / math.sqrt(D)
    out = np.zeros((rows.shape[0], D), dtype=np.float64)
    lse = np.full(rows.shape[0], -np.inf, dtype=np.float64)
    heads = {}
    for n, (b, h, i) in enumerate(rows):
        heads.setdefault((int(b), int(h)), []).append(n)
    for (b, h), idx in heads.items():
        idx = np.asarray(idx)
        ii = rows[idx, 2]
        L = int(kl[b])
        if hasattr(q, "detach"):
            import torch
            qi = _as_f64(q[b, h].index_select(0, torch.as_tensor(ii, device=q.device)))
        else:
            qi = _as_f64(np.asarray(q[b, h])[ii])
        kb = _as_f64(k[b, h])
        vb = _as_f64(v[b, h]).copy()
        vb[L:] = 0.0  # padded value rows carry zero weight (see attention())
        s = (qi @ kb.T) * scale
        mask = valid_mask(S, L, causal, rows=ii)
        o, l = _softmax_rows(s, mask, vb)
        out[idx] = o
        lse[idx] = l
    return out, lse


def count_valid_pairs(S: int, key_len, causal: bool, B: int, H: int) -> int:
    """Number of visible (query, key) pairs over all B*H heads (exact integers).

    Used for algorithmic FLOP counts: 4 * d_h * pairs (two matmuls, 2 flops per
    multiply-add).
    """
    kl = _key_lengths(key_len, B, S)
    total = 0
    for L in kl:
        L = int(L)
        if causal:
            # rows i < L see i+1 keys; rows i >= L see L keys
            total += L * (L + 1) // 2 + (S - L) * L
        else:
            total += S * L
    return total * H
