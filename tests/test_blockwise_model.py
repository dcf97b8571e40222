"""The online-softmax tile loop (the method the kernels run) against the oracle.

Pins the method itself: for every tile size, partial tiles, causal block
skipping and key-length tails, the running-max recurrence reaches the
materialised definition to float64 rounding (devpost
"gpu-transformer-optimization", section 2.1: O_final / l_final equals
softmax(QK^T / sqrt(d_k)) V in exact arithmetic). With the kernels' precision
emulated, it also predicts how much of the error budget the GPU should use.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention, budget_fraction, gate
from blockwise_model import running_max_attention, tiled_attention


@pytest.mark.parametrize("BQ,BK", [(1, 1), (7, 16), (16, 32), (32, 7), (64, 64), (128, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_tile_loop_equals_definition(BQ, BK, causal):
    B, H, S, D = 2, 2, 100, 8          # 100 = partial last tile for every size above
    rng = np.random.default_rng(BQ * 1000 + BK)
    q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    kl = [100, 37]
    ref_o, ref_l = attention(q, k, v, causal=causal, key_len=kl)
    o, l = tiled_attention(q, k, v, causal=causal, key_len=kl, BQ=BQ, BK=BK)
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, ref_l, rtol=1e-12, atol=1e-12)


def test_tile_loop_empty_rows():
    q = k = v = np.ones((1, 1, 5, 4))
    o, l = tiled_attention(q, k, v, causal=True, key_len=[0], BQ=2, BK=2)
    assert (o == 0).all() and (l == -np.inf).all()


@pytest.mark.parametrize("dtype,limit", [("f16", 0.5), ("bf16x2", 0.5)])
def test_emulated_precision_budget(dtype, limit):
    """fp16 inputs with fp32 accumulation and fp16 probabilities should sit
    well inside the budget (the pages' rounding argument puts fp16 operand
    rounding at a relative 2^-11 against a 2e-2 rail); a budget fraction
    above 0.5 on these inputs would point at a bug, not at rounding."""
    B, H, S, D = 1, 4, 256, 64
    g = torch.Generator().manual_seed(0)
    td = torch.float16 if dtype == "f16" else torch.bfloat16
    # bf16 inputs keep probabilities as a bf16 head plus a bf16 remainder:
    # one bf16 rounding of p alone (2^-9 relative) uses most of the budget on
    # short causal rows (see test_single_bf16_probability_rounding_is_too_coarse)
    q, k, v = (torch.randn(B, H, S, D, generator=g).to(td).double().numpy() for _ in range(3))
    ref_o, ref_l = attention(q, k, v, causal=True)
    o, l = tiled_attention(q, k, v, causal=True, BQ=64, BK=64, emulate=True, dtype=dtype)
    frac = budget_fraction(o, ref_o)
    assert frac < limit, frac
    assert budget_fraction(l, ref_l) < 0.05
    assert gate(o, ref_o).all()


def test_single_bf16_probability_rounding_is_too_coarse():
    """Evidence for the split: rounding p once to bf16 before P.V leaves too
    little margin (worst element near the whole budget over a few seeds)."""
    worst = 0.0
    for seed in range(3):
        g = torch.Generator().manual_seed(seed)
        q, k, v = (torch.randn(1, 2, 256, 64, generator=g).bfloat16().double().numpy() for _ in range(3))
        ref_o, _ = attention(q, k, v, causal=True)
        o, _ = tiled_attention(q, k, v, causal=True, emulate=True, dtype="bf16")
        worst = max(worst, budget_fraction(o, ref_o))
    assert worst > 0.6


def _climbing(S, D, seed, step=14.0):
    """Scores climbing by `step` (natural units; x1.44 in log2 units) every
    32 keys: q = 1 along every axis, k_j = a_j / sqrt(D) along every axis."""
    rng = np.random.default_rng(seed)
    a = step * (np.arange(S) // 32) + 0.5 * rng.standard_normal(S)
    q = 1.0 + 0.05 * rng.standard_normal((1, 2, S, D))
    k = (a / math.sqrt(D))[None, None, :, None] + 0.05 * rng.standard_normal((1, 2, S, D))
    v = rng.standard_normal((1, 2, S, D))
    return q, k, v


@pytest.mark.parametrize("BQ,PAIR", [(1, 1), (16, 32), (64, 32), (33, 7)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("inputs", ["normal", "climbing"])
def test_running_max_loop_equals_definition(BQ, PAIR, causal, inputs):
    """Probabilities against the running max with an overflow check and
    recompute reach the definition to float64 rounding, also when the row
    maximum climbs past the limit at every chunk (redo on most chunks)."""
    B, H, S, D = 1, 2, 150, 8
    if inputs == "normal":
        rng = np.random.default_rng(BQ * 100 + PAIR)
        q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    else:
        q, k, v = _climbing(S, D, seed=PAIR)
    kl = [137]
    ref_o, ref_l = attention(q, k, v, causal=causal, key_len=kl)
    st = {}
    o, l = running_max_attention(q, k, v, causal=causal, key_len=kl, BQ=BQ, PAIR=PAIR, stats=st)
    np.testing.assert_allclose(o, ref_o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l, ref_l, rtol=1e-11, atol=1e-12)
    assert st["redo"] > 0  # at least the first visible keys of every row


def test_running_max_redoes_only_when_needed():
    """With N(0, 1) scores the running max from the first chunk holds (no
    redo after it); with scores climbing ~20 log2 units per 32 keys almost
    every chunk is redone."""
    B, H, S, D = 1, 2, 256, 64
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((B, H, S, D)) for _ in range(3))
    st = {}
    running_max_attention(q, k, v, BQ=64, PAIR=32, stats=st)
    assert st["redo"] == B * H * S  # each row once, at its first chunk
    q, k, v = _climbing(S, D, seed=1)
    st = {}
    running_max_attention(q, k, v, BQ=64, PAIR=32, stats=st)
    assert st["redo"] >= B * H * S * (S // 32 - 1)


@pytest.mark.parametrize("inputs", ["normal", "climbing"])
def test_running_max_emulated_precision_budget(inputs):
    """fp16 probabilities against a stale running max (values up to the fp16
    maximum keep their relative precision) stay well inside the budget."""
    B, H, S, D = 1, 2, 256, 64
    if inputs == "normal":
        g = torch.Generator().manual_seed(0)
        q, k, v = (torch.randn(B, H, S, D, generator=g).half().double().numpy() for _ in range(3))
    else:
        q, k, v = (torch.from_numpy(t).half().double().numpy() for t in _climbing(S, D, seed=2))
    ref_o, ref_l = attention(q, k, v, causal=True)
    o, l = running_max_attention(q, k, v, causal=True, BQ=64, PAIR=32, emulate=True, dtype="f16")
    assert budget_fraction(o, ref_o) < 0.5
    assert budget_fraction(l, ref_l) < 0.05
    assert gate(o, ref_o).all()


def test_running_max_bf16_needs_a_bound_not_just_a_finiteness_test():
    """bf16 probabilities only overflow at the fp32 range, so a check that
    only rejects infinite sums lets probabilities near 2^127 through while
    the running max is far behind, and O / l then overflow fp32 (scores
    spread over hundreds of log2 units: inputs scaled by 12). Bounding the
    probabilities by 2^21 (the kernels bound each 32-key pair's sum, which
    bounds every probability in it) keeps the result inside the rule."""
    B, H, S, D = 1, 2, 396, 128
    g = torch.Generator().manual_seed(144)
    q, k, v = (torch.randn(B, H, S, D, generator=g) for _ in range(3))
    q, k = (t * 12.0 for t in (q, k))
    q, k, v = (t.bfloat16().double().numpy() for t in (q, k, v))
    ref_o, ref_l = attention(q, k, v, causal=True)
    o, l = running_max_attention(q, k, v, causal=True, BQ=64, PAIR=32, emulate=True,
                                 dtype="bf16x2", limit=np.inf)
    assert not np.isfinite(o).all()
    o, l = running_max_attention(q, k, v, causal=True, BQ=64, PAIR=32, emulate=True,
                                 dtype="bf16x2", limit=2.0 ** 21)
    assert np.isfinite(o).all() and gate(o, ref_o).all() and gate(l, ref_l).all()
