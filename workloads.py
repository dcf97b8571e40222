"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic: it only defines the workload
shapes and draws Q, K, V and key lengths from a seed. Both the HIP path's
tests / benchmark and the float64 oracle are fed from here, which is the one
thing the two sides share.

The pages measure on an organiser harness that draws synthetic tensors from a
fixed seed (devpost "gpu-transformer-optimization", "Development
environment"); that harness and its shape list are not available, so these
workloads, with their stated shapes and distributions, stand in for it.

Recipe (every workload): a torch CPU generator seeded with `seed` draws q, k,
v in that order as float32 N(0, 1) tensors of shape [B, H, S, d_h], each then
cast to the workload dtype with round-to-nearest-even; where the key lengths
are random they are drawn next, uniform on [lo, hi] inclusive. The long
workload (3.3e9 elements per tensor) is drawn by the device generator instead,
in the same order, and never exists on the host.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_backward_inputs", "make_qkv_inputs",
           "sample_rows"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: torch.dtype
    causal: bool
    # key lengths: None -> all S keys valid (NULL key_len pointer);
    # ("fixed", L) -> every batch has L valid keys;
    # ("uniform", lo, hi) -> per batch uniform on [lo, hi] inclusive.
    key_len: Optional[tuple]
    note: str = ""
    H_kv: Optional[int] = None  # key / value heads (grouped-query attention); None = H

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def elems(self) -> int:
        return self.B * self.H * self.S * self.D


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, 32, torch.float32, False, None,
                     "oracle-sized case: fp32, non-causal, all 64 keys valid"),
    "launch": Workload("launch", 1, 8, 128, 16, torch.float16, True, ("fixed", 128),
                       "launch-bound: B=1, d_model=128 in 8 heads of 16"),
    "bandwidth": Workload("bandwidth", 10000, 8, 128, 16, torch.float16, True, ("uniform", 64, 128),
                          "HBM-bound: 80000 short heads, right-padded key lengths"),
    "compute": Workload("compute", 16, 4, 1024, 256, torch.float16, False, ("fixed", 1024),
                        "MFMA-bound: d_model=1024 in 4 heads of 256"),
    "long": Workload("long", 32, 16, 100000, 64, torch.float16, True, ("fixed", 100000),
                     "long sequence: d_model=1024 in 16 heads of 64, S=100000"),
    # attention fed by its own QKV projection (devpost
    # "gpu-transformer-optimization", section 2.2): the launch- and HBM-bound
    # shapes above with x [B, S, d_model = H d_h] and W_qkv [d_model, 3 d_model]
    # in place of q, k, v
    "qkv_launch": Workload("qkv_launch", 1, 8, 128, 16, torch.float16, True, ("fixed", 128),
                           "fused QKV projection + attention: B=1, S=128, d_model=128, 8 heads"),
    "qkv_bandwidth": Workload("qkv_bandwidth", 10000, 8, 128, 16, torch.float16, True,
                              ("uniform", 64, 128),
                              "fused QKV projection + attention: B=10000, S=128, d_model=128, "
                              "8 heads, right-padded key lengths"),
    # the same with sixteen heads of 8 in d_model 128 (the pages' heads-of-8
    # cases, grouped two per 16-wide projection slice)
    "qkv_heads8": Workload("qkv_heads8", 10000, 16, 128, 8, torch.float16, True,
                           ("uniform", 64, 128),
                           "fused QKV projection + attention: B=10000, S=128, d_model=128, "
                           "16 heads of 8, right-padded key lengths"),
    # the training shape of the fused backward on rustingstudio
    # "brain/docs/baseline" ("Fused attention"): batch 4, sequence 1024,
    # 12 heads of 64, causal, bf16 (one key/value head per query head here)
    "bwd": Workload("bwd", 4, 12, 1024, 64, torch.bfloat16, True, None,
                    "backward: B=4, S=1024, 12 heads of 64, causal, bf16"),
    # the same with the page's 4 key / value heads (grouped-query attention)
    "bwd_gqa": Workload("bwd_gqa", 4, 12, 1024, 64, torch.bfloat16, True, None,
                        "backward: B=4, S=1024, 12 query / 4 key-value heads of 64, causal, bf16",
                        H_kv=4),
}


def _draw_key_len(w: Workload, gen: torch.Generator, device) -> Optional[torch.Tensor]:
    if w.key_len is None:
        return None
    kind = w.key_len[0]
    if kind == "fixed":
        return torch.full((w.B,), int(w.key_len[1]), dtype=torch.int32, device=device)
    if kind == "uniform":
        lo, hi = int(w.key_len[1]), int(w.key_len[2])
        return torch.randint(lo, hi + 1, (w.B,), generator=gen, dtype=torch.int32,
                             device=gen.device).to(device)
    raise ValueError(f"unknown key_len spec {w.key_len!r}")


def make_inputs(w: Workload, seed: int, device="cpu", gen_device: Optional[str] = None
                ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """Draw (q, k, v, key_len) for workload `w` from `seed`.

    gen_device: where the generator lives ("cpu" by default; the long workload
    uses the device generator, which must be "cuda"). Tensors are returned on
    `device`.
    """
    if gen_device is None:
        gen_device = "cuda" if w.name == "long" else "cpu"
    gen = torch.Generator(device=gen_device)
    gen.manual_seed(int(seed))
    shape = (w.B, w.H, w.S, w.D)
    out = []
    for _ in range(3):
        t = torch.randn(shape, generator=gen, dtype=torch.float32, device=gen_device)
        t = t.to(w.dtype)
        out.append(t.to(device))
        del t
    kl = _draw_key_len(w, gen, device)
    return out[0], out[1], out[2], kl


def make_backward_inputs(w: Workload, seed: int, device="cpu"):
    """(q, k, v, key_len, dout): q, k, v (k and v with H_kv heads when set),
    key lengths, then the output gradient dout, drawn in that order from one
    CPU generator, N(0, 1) in float32, cast to the workload dtype."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    shape = (w.B, w.H, w.S, w.D)
    kv_shape = (w.B, w.H_kv or w.H, w.S, w.D)
    qkv = [torch.randn(shp, generator=gen, dtype=torch.float32).to(w.dtype).to(device)
           for shp in (shape, kv_shape, kv_shape)]
    kl = _draw_key_len(w, gen, device)
    dout = torch.randn(shape, generator=gen, dtype=torch.float32).to(w.dtype).to(device)
    return qkv[0], qkv[1], qkv[2], kl, dout


def make_qkv_inputs(w: Workload, seed: int, device="cpu"):
    """(x, w_qkv, b_qkv, key_len) for the fused projection workloads: x
    [B, S, d_model] N(0, 1) (layer-normalised activations), then W_qkv
    [d_model, 3 d_model] and b_qkv [3 d_model] uniform on +-1/sqrt(d_model)
    (the default initialisation of a torch linear layer, the pages' randomly
    initialised weights), then the key lengths; float32 draws from one CPU
    generator, cast to the workload dtype."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    D = w.H * w.D
    a = 1.0 / np.sqrt(D)
    x = torch.randn((w.B, w.S, D), generator=gen, dtype=torch.float32)
    wq = (torch.rand((D, 3 * D), generator=gen, dtype=torch.float32) * 2 - 1) * a
    bq = (torch.rand((3 * D,), generator=gen, dtype=torch.float32) * 2 - 1) * a
    kl = _draw_key_len(w, gen, device)
    return (x.to(w.dtype).to(device), wq.to(w.dtype).to(device), bq.to(w.dtype).to(device), kl)


def sample_rows(B: int, H: int, S: int, n_rows: int, seed: int, tile: int = 128,
                n_heads: Optional[int] = None) -> np.ndarray:
    """Seeded (b, h, i) query-row sample for checking a long sequence row by row.

    The sample spans `n_heads` heads (default: one per batch, head drawn at
    random) and, in each, forced rows at the sequence ends and at tile edges
    plus uniform draws. Returns int64 [n, 3].
    """
    rng = np.random.Generator(np.random.PCG64(int(seed)))
    if n_heads is None:
        n_heads = B
    bs = np.arange(n_heads) % B
    hs = rng.integers(0, H, size=n_heads)
    per = max(1, n_rows // n_heads)
    forced = [0, 1, 2, tile - 1, tile, tile + 1, S // 2, S - tile - 1, S - tile,
              (S // tile) * tile - 1, (S // tile) * tile, S - 2, S - 1]
    forced = sorted({f for f in forced if 0 <= f < S})
    rows = []
    for n in range(n_heads):
        fr = forced if n % 4 == 0 else forced[:3] + forced[-3:]
        k = max(0, per - len(fr))
        rnd = rng.integers(0, S, size=k)
        for i in list(fr) + list(rnd):
            rows.append((bs[n], hs[n], i))
    rows = np.asarray(rows, dtype=np.int64)
    return rows[:max(n_rows, 1)] if rows.shape[0] > n_rows else rows
