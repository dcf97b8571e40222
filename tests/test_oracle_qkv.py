"""Pins for the float64 QKV-projection oracle: the identity projection
reduces it to the (pinned) attention oracle on head slices of X, it agrees
with float64 torch (linear + scaled_dot_product_attention), bias shifts act
as the mathematics says, and planted mistakes fail. No GPU."""

import importlib

import numpy as np
import pytest
import torch

from oracle import attention, qkv_attention

oq = importlib.import_module("oracle.qkv")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_identity_projection_is_attention_on_head_slices():
    B, S, H, hd = 2, 9, 3, 4
    D = H * hd
    x = _rand((B, S, D), 1)
    w = np.concatenate([np.eye(D)] * 3, axis=1)
    out, lse = qkv_attention(x, w, None, H, causal=True, key_len=[9, 5])
    xh = x.reshape(B, S, H, hd).transpose(0, 2, 1, 3)
    ro, rl = attention(xh, xh, xh, causal=True, key_len=[9, 5])
    assert np.allclose(out, ro.transpose(0, 2, 1, 3).reshape(B, S, D), rtol=1e-14, atol=1e-14)
    assert np.allclose(lse, rl, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_float64(causal):
    B, S, H, hd = 2, 17, 4, 8
    D = H * hd
    x, w, b = _rand((B, S, D), 2), _rand((D, 3 * D), 3) / np.sqrt(D), _rand((3 * D,), 4)
    out, _ = qkv_attention(x, w, b, H, causal=causal)
    y = torch.nn.functional.linear(torch.tensor(x), torch.tensor(w).T, torch.tensor(b))
    q, k, v = (t.reshape(B, S, H, hd).transpose(1, 2) for t in y.split(D, dim=-1))
    ro = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    ro = ro.transpose(1, 2).reshape(B, S, D).numpy()
    assert np.allclose(out, ro, rtol=1e-12, atol=1e-12)


def test_bias_shifts():
    """A key bias shifts every score of a query row by the same amount
    (softmax unchanged); a value bias shifts each output row by itself."""
    B, S, H, hd = 1, 11, 2, 4
    D = H * hd
    x, w, b = _rand((B, S, D), 5), _rand((D, 3 * D), 6), _rand((3 * D,), 7)
    base, _ = qkv_attention(x, w, b, H, causal=True)
    bk = b.copy()
    bk[D:2 * D] += 3.0
    assert np.allclose(qkv_attention(x, w, bk, H, causal=True)[0], base, rtol=1e-12, atol=1e-12)
    bv = b.copy()
    delta = _rand((D,), 8)
    bv[2 * D:] += delta
    assert np.allclose(qkv_attention(x, w, bv, H, causal=True)[0], base + delta, rtol=1e-12,
                       atol=1e-12)


def test_planted_mistakes(monkeypatch):
    B, S, H, hd = 1, 6, 2, 3
    D = H * hd
    x, w, b = _rand((B, S, D), 9), _rand((D, 3 * D), 10), _rand((3 * D,), 11)
    y = torch.nn.functional.linear(torch.tensor(x), torch.tensor(w).T, torch.tensor(b))
    q, k, v = (t.reshape(B, S, H, hd).transpose(1, 2) for t in y.split(D, dim=-1))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v).transpose(1, 2).reshape(B, S, D)

    def agrees():
        return np.allclose(qkv_attention(x, w, b, H)[0], ref.numpy(), rtol=1e-10, atol=1e-10)

    assert agrees()
    orig = oq.qkv_project
    planted = {
        "q and k swapped": lambda *a: (lambda t: (t[1], t[0], t[2]))(orig(*a)),
        "heads split as [hd, H]": lambda x_, w_, b_, H_: tuple(
            t.transpose(0, 1, 3, 2).reshape(t.shape[0], t.shape[2], H_, -1).transpose(0, 2, 1, 3)
            for t in orig(x_, w_, b_, H_)),
        "bias dropped": lambda x_, w_, b_, H_: orig(x_, w_, None, H_),
    }
    for name, fn in planted.items():
        monkeypatch.setattr(oq, "qkv_project", fn)
        assert not agrees(), name
        monkeypatch.undo()
    assert agrees()
