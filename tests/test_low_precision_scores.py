"""Why the scores are not computed from 8-bit q and k (the INT8 Q K^T idea
the pages defer: devpost "transformerkernel-a-7-1x-transformer-layer-for-
the-tesla-t4", "What's next"): rounding q and k to fp8 e4m3 or int8 (per-row scales,
optionally with the key mean removed first) before an exact attention
breaks the graded accuracy rule by a wide margin, while the fp16 rounding
the kernels already apply stays inside it. CPU only, float64 oracle."""

import numpy as np
import pytest
import torch

import oracle

torch.manual_seed(0)


def _per_row(x, qmax, cast):
    sc = np.maximum(np.abs(x).max(axis=-1, keepdims=True) / qmax, 1e-30)
    return cast(x / sc) * sc


def _fp8(x):
    return _per_row(x, 448.0, lambda y: torch.from_numpy(y).float().to(torch.float8_e4m3fn)
                    .double().numpy())


def _int8(x):
    return _per_row(x, 127.0, lambda y: np.clip(np.round(y), -127, 127))


def _fp16(x):
    return torch.from_numpy(x).half().double().numpy()


def _budget(quant, smooth=False, seed=0):
    g = torch.Generator().manual_seed(seed)
    B, H, S, D = 1, 2, 512, 64
    q, k, v = (torch.randn(B, H, S, D, generator=g, dtype=torch.float64).numpy() for _ in range(3))
    ref, _ = oracle.attention(q, k, v, causal=True)
    kk = k - k.mean(axis=-2, keepdims=True) if smooth else k  # a per-row shift of the scores
    out, _ = oracle.attention(quant(q), quant(kk), v, causal=True)
    return oracle.budget_fraction(out, ref)


def test_fp16_scores_fit_the_budget():
    assert _budget(_fp16) < 0.5


@pytest.mark.parametrize("quant", [_fp8, _int8], ids=["fp8_e4m3", "int8"])
@pytest.mark.parametrize("smooth", [False, True])
def test_eight_bit_scores_break_the_budget(quant, smooth):
    assert _budget(quant, smooth) > 1.5
