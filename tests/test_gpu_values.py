"""GPU checks of exact properties of the definition that hold for every
variant, beyond the accuracy rule (devpost "gpu-transformer-optimization",
section 2.1: out = softmax(scores) V row by row).

* Uniform V returns V: every softmax row sums to 1, so with v_j = c for every
  key the output is c. A kernel that multiplies V by rounded probabilities
  but sums unrounded ones for the denominator misses this by up to one
  rounding of the weights; summing the same rounded weights it multiplies by
  gives c to fp32 rounding, which the final rounding to the input dtype
  removes: the output must equal c bit for bit.
* A non-finite value in V stays in its own output column: out[i, x] depends
  on column x of V only, so an Inf in V[j, x] (key j visible to every row)
  makes column x infinite and leaves every other column finite and within
  the rule. For bf16 inputs the probabilities enter the products as head +
  remainder pairs; where a remainder is exactly zero (a probability that
  bf16 holds exactly, such as the row maximum's 1), its product with the Inf
  is 0 * Inf = NaN, so there column x may come out NaN instead of +inf. The
  other columns are unaffected either way.
"""

import math

import pytest
import torch

import oracle
from gpu_helpers import check_full, run_gpu
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _variants(D, S):
    v = ["auto", "mfma", "mfma_small"]
    if S <= 128 and D <= 64:
        v.append("short")
    if D == 16:
        v.append("valu_d16")
    return v


_CASES = [(dt, D, S) for dt in ("f16", "bf16") for D in (8, 16, 32, 64, 128, 256)
          for S in (100, 128, 333)]


@pytest.mark.parametrize("dt,D,S", _CASES)
@pytest.mark.parametrize("causal", [False, True])
def test_uniform_v_is_returned_exactly(mha, dt, D, S, causal):
    w = Workload("uniform_v", 3, 2, S, D, _DT[dt], causal, ("uniform", 1, S))
    q, k, v, kl = make_inputs(w, seed=D + S)
    q = (q.float() * 2).to(_DT[dt])  # spread the weights
    for c in (0.3, -1.7, 1000.0):
        vc = torch.full_like(v, c)
        cval = vc.float()
        for variant in _variants(D, S):
            out, lse = run_gpu(mha, q, k, vc, kl, causal, variant)
            assert torch.equal(out.float(), cval), (
                f"{variant} {dt} D={D} S={S} causal={causal} c={c}: max |out - c| "
                f"{(out.float() - cval).abs().max().item():.3g}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("D,S", [(16, 128), (8, 128), (32, 128), (64, 100), (64, 300), (256, 200)])
def test_infinite_v_stays_in_its_column(mha, dt, D, S):
    """Non-causal, every key visible: V[b, h, j, x] = +inf for one key j per
    head. Column x of every row is +inf; all other columns pass the rule."""
    w = Workload("inf_v", 4, 2, S, D, _DT[dt], False, None)
    q, k, v, _ = make_inputs(w, seed=7 * D + S)
    x = D // 2 - 1
    v[:, :, S // 3, x] = math.inf
    for variant in _variants(D, S):
        out, lse = run_gpu(mha, q, k, v, None, False, variant)
        col = out[..., x]
        if dt == "f16":
            assert (col == math.inf).all(), f"{variant}: column {x} not +inf"
        else:
            assert (~torch.isfinite(col)).all(), f"{variant}: column {x} finite"
        rest = torch.cat([out[..., :x], out[..., x + 1:]], dim=-1)
        assert torch.isfinite(rest).all(), f"{variant}: the inf reached other columns"
        ro, rl = oracle.attention(q, k, v, causal=False)
        keep = [i for i in range(D) if i != x]
        assert oracle.gate(rest, ro[..., keep]).all(), f"{variant}: other columns fail the rule"
        assert oracle.gate(lse, rl).all(), f"{variant}: lse fails the rule"
