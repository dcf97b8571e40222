"""Pins for the float64 backward oracle, against things other than its own
chain-rule formulas: central finite differences of the (separately pinned)
forward oracle, float64 autograd of torch's CPU attention routine, exact
invariants of softmax attention, and planted mistakes that the pins must
catch. Nothing here touches a GPU."""

import importlib
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention, attention_backward

ob = importlib.import_module("oracle.backward")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _loss(q, k, v, do, causal, kl):
    out, _ = attention(q, k, v, causal=causal, key_len=kl)
    return float(np.sum(out * do))


def _finite_diff(q, k, v, do, causal, kl, h=1e-6):
    """Central differences of sum(dO * O) in every coordinate of q, k, v."""
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        it = np.nditer(g, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            x0 = args[which][idx]
            args[which][idx] = x0 + h
            lp = _loss(*args, do, causal, kl)
            args[which][idx] = x0 - h
            lm = _loss(*args, do, causal, kl)
            args[which][idx] = x0
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S,D,L", [(4, 3, 4), (5, 2, 3), (6, 4, 1)])
def test_matches_finite_differences(S, D, L, causal):
    q, k, v, do = (_rand((1, 2, S, D), 10 + t) for t in range(4))
    kl = [L]
    dq, dk, dv = attention_backward(q, k, v, do, causal=causal, key_len=kl)
    fq, fk, fv = _finite_diff(q, k, v, do, causal, kl)
    for name, a, b in (("dq", dq, fq), ("dk", dk, fk), ("dv", dv, fv)):
        assert np.allclose(a, b, rtol=1e-6, atol=1e-8), (name, np.abs(a - b).max())


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd_float64(causal):
    B, H, S, D = 2, 3, 17, 8
    q, k, v, do = (_rand((B, H, S, D), 20 + t) for t in range(4))
    kl = [17, 11]
    dq, dk, dv = attention_backward(q, k, v, do, causal=causal, key_len=kl)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = torch.zeros(B, 1, S, S, dtype=torch.bool)
    for b, L in enumerate(kl):
        mask[b, :, :, :L] = True
    if causal:
        mask &= torch.ones(S, S, dtype=torch.bool).tril()
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    out.backward(torch.tensor(do))
    assert np.allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(causal):
    """Shifting every key by the same vector leaves each softmax row, hence
    the output, unchanged: the key gradients sum to zero over the keys."""
    q, k, v, do = (_rand((2, 2, 9, 5), 30 + t) for t in range(4))
    _, dk, _ = attention_backward(q, k, v, do, causal=causal, key_len=[9, 6])
    assert np.abs(dk.sum(axis=2)).max() < 1e-12


def test_uniform_values_give_no_query_or_key_gradient():
    """With every value row equal the output is that row whatever Q and K
    are, so dQ = dK = 0 and dV_j = sum_i A_ij dO_i sums to sum_i dO_i."""
    q, k, do = (_rand((1, 2, 7, 4), 40 + t) for t in range(3))
    v = np.broadcast_to(_rand((1, 2, 1, 4), 44), (1, 2, 7, 4)).copy()
    dq, dk, dv = attention_backward(q, k, v, do, causal=True)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    assert np.allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)


def test_padding_gets_no_gradient_and_does_not_leak():
    q, k, v, do = (_rand((1, 1, 8, 4), 50 + t) for t in range(4))
    dq, dk, dv = attention_backward(q, k, v, do, causal=False, key_len=[5])
    assert np.all(dk[..., 5:, :] == 0) and np.all(dv[..., 5:, :] == 0)
    kp, vp = k.copy(), v.copy()
    kp[..., 5:, :] = np.nan
    vp[..., 5:, :] = np.inf
    pq, pk, pv = attention_backward(q, kp, vp, do, causal=False, key_len=[5])
    assert np.array_equal(pq, dq) and np.array_equal(pk, dk) and np.array_equal(pv, dv)


def test_linear_in_output_gradient():
    q, k, v, do = (_rand((1, 2, 6, 3), 60 + t) for t in range(4))
    g1 = attention_backward(q, k, v, do, causal=True)
    g2 = attention_backward(q, k, v, 2.5 * do, causal=True)
    g0 = attention_backward(q, k, v, 0 * do, causal=True)
    for a, b, z in zip(g1, g2, g0):
        assert np.allclose(2.5 * a, b, rtol=1e-13, atol=1e-14) and np.all(z == 0)


def test_empty_rows_and_single_key():
    q, k, v, do = (_rand((1, 1, 4, 2), 70 + t) for t in range(4))
    dq, dk, dv = attention_backward(q, k, v, do, key_len=[0])
    assert not dq.any() and not dk.any() and not dv.any()
    # one visible key: every row's output is v_0 whatever the scores are
    dq, dk, dv = attention_backward(q, k, v, do, key_len=[1])
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    assert np.allclose(dv[0, 0, 0], do[0, 0].sum(axis=0)) and not dv[0, 0, 1:].any()


def test_row_term_equals_rowsum_of_output_gradient_times_output():
    """rowsum(A * dA) = rowsum(dO * O): the identity that lets a fused
    backward take the softmax row term from dO and O."""
    q, k, v, do = (_rand((1, 2, 10, 6), 80 + t) for t in range(4))
    out, _ = attention(q, k, v, causal=True, key_len=[7])
    mask = oracle.valid_mask(10, 7, True)
    a = ob._probs((q @ np.swapaxes(k, -1, -2)) / math.sqrt(6), mask)
    vv = v.copy()
    vv[..., 7:, :] = 0
    da = do @ np.swapaxes(vv, -1, -2)
    assert np.allclose((a * da).sum(-1), (do * out).sum(-1), rtol=1e-12, atol=1e-13)


def test_finite_differences_catch_planted_mistakes(monkeypatch):
    """Each mistake is planted in the oracle itself; the finite-difference
    pin must reject every one of them."""
    q, k, v, do = (_rand((1, 1, 5, 3), 90 + t) for t in range(4))
    ref = _finite_diff(q, k, v, do, True, [4])

    def agrees():
        got = attention_backward(q, k, v, do, causal=True, key_len=[4])
        return all(np.allclose(a, b, rtol=1e-6, atol=1e-8) for a, b in zip(got, ref))

    assert agrees()
    sg, og, pr, vm = ob._softmax_grad, ob._operand_grads, ob._probs, ob.valid_mask
    planted = {
        # softmax Jacobian without its row term
        "row term": ("_softmax_grad", lambda a, da: a * da),
        # wrong sign of the row term
        "row sign": ("_softmax_grad", lambda a, da: a * (da + (a * da).sum(-1, keepdims=True))),
        # scale dropped from dQ and dK
        "scale": ("_operand_grads", lambda ds, q, k, a, do, c: og(ds, q, k, a, do, 1.0)),
        # dK without the transpose of dS
        "transpose": ("_operand_grads", lambda ds, q, k, a, do, c:
                      (og(ds, q, k, a, do, c)[0], (ds @ q) * c, og(ds, q, k, a, do, c)[2])),
        # dV from A instead of A^T
        "dv": ("_operand_grads", lambda ds, q, k, a, do, c:
               og(ds, q, k, a, do, c)[:2] + (a @ do,)),
        # probabilities not normalised
        "norm": ("_probs", lambda s, m: pr(s, m) * 1.5),
        # causal diagonal excluded
        "diagonal": ("valid_mask", lambda S, L, causal, rows=None:
                     vm(S, L, causal, rows) & ~np.eye(S, dtype=bool) | (np.arange(S) == 0)[None, :]),
    }
    for name, (attr, fn) in planted.items():
        monkeypatch.setattr(ob, attr, fn)
        assert not agrees(), name
        monkeypatch.undo()
    assert agrees()
