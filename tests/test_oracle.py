"""Pins for the float64 oracle, against things other than the oracle itself.

Each test fixes the oracle to something the pages or the mathematics decide:
a hand-worked example, pure-Python brute force, a library routine for the
special case it covers, invariants and closed forms of softmax attention, and
planted mistakes that the pins must catch. Nothing here touches a GPU.
"""

import json
import math
import os
import types
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import importlib
oa = importlib.import_module("oracle.attention")
from oracle import attention, attention_rows, valid_mask, count_valid_pairs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------- brute force

def _brute(q, k, v, causal, L):
    """Pure-Python attention (no numpy arithmetic): math.exp, math.fsum.

    Direct transcription of the definition for one head: scaled dot products,
    visible keys j < L (and j <= i when causal), max-shifted softmax, weighted
    sum of value rows.
    """
    S, D = len(q), len(q[0])
    c = 1.0 / math.sqrt(D)
    outs, lses = [], []
    for i in range(S):
        vis = [j for j in range(S) if j < L and (not causal or j <= i)]
        if not vis:
            outs.append([0.0] * D)
            lses.append(-math.inf)
            continue
        s = {j: math.fsum(q[i][d] * k[j][d] for d in range(D)) * c for j in vis}
        m = max(s.values())
        w = {j: math.exp(s[j] - m) for j in vis}
        tot = math.fsum(w.values())
        outs.append([math.fsum(w[j] * v[j][d] for j in vis) / tot for d in range(D)])
        lses.append(m + math.log(tot))
    return outs, lses


@pytest.mark.parametrize("S", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("D", [1, 2, 3, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(S, D, causal):
    for L in sorted({0, 1, S // 2, S - 1, S}):
        if L < 0:
            continue
        seed = 1000 * S + 10 * D + L + (7 if causal else 0)
        q, k, v = (_rand((1, 1, S, D), seed + t) for t in range(3))
        out, lse = attention(q, k, v, causal=causal, key_len=[L])
        bo, bl = _brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), causal, L)
        np.testing.assert_allclose(out[0, 0], np.array(bo), rtol=1e-13, atol=1e-13)
        bl = np.array(bl)
        assert np.array_equal(np.isinf(lse[0, 0]), np.isinf(bl))
        fin = np.isfinite(bl)
        np.testing.assert_allclose(lse[0, 0][fin], bl[fin], rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------- hand-worked example

def test_worked_example_golden():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64)[None, None]
    k = np.array(g["k"], dtype=np.float64)[None, None]
    v = np.array(g["v"], dtype=np.float64)[None, None]
    tol = g["tolerance"]
    for case in g["cases"]:
        out, lse = attention(q, k, v, causal=case["causal"], key_len=[case["key_len"]])
        want = np.array([[float(Fraction(x)) for x in row] for row in case["out"]])
        np.testing.assert_allclose(out[0, 0], want, rtol=0, atol=tol)
        for i, n in enumerate(case["lse_of"]):
            if n == 0:
                assert lse[0, 0, i] == -np.inf
            else:
                assert abs(lse[0, 0, i] - math.log(n)) <= tol


# -------------------------------------------------- library routine special case

@pytest.mark.parametrize("shape", [(2, 3, 37, 16), (1, 2, 64, 32), (3, 1, 20, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(shape, causal):
    """CPU float64 scaled_dot_product_attention with a boolean mask is the same
    computation for every row that has at least one visible key."""
    B, H, S, D = shape
    q, k, v = (torch.from_numpy(_rand(shape, 11 + t)) for t in range(3))
    kl = np.array([S, max(1, S // 3), 1][:B])
    out, _ = attention(q, k, v, causal=causal, key_len=kl)
    mask = np.stack([valid_mask(S, int(L), causal) for L in kl])[:, None]  # [B,1,S,S]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=torch.from_numpy(mask)).numpy()
    has = mask.any(-1)[..., None] & np.ones((1, H, 1, 1), dtype=bool)
    np.testing.assert_allclose(np.where(has, out, 0), np.where(has, ref, 0), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ invariants

def _scores(q, k):
    return np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(q.shape[-1])


@pytest.mark.parametrize("causal", [False, True])
def test_probabilities_sum_to_one(causal):
    B, H, S, D = 2, 2, 33, 8
    q, k, v = (_rand((B, H, S, D), 20 + t) for t in range(3))
    kl = [S, 17]
    _, lse = attention(q, k, v, causal=causal, key_len=kl)
    s = _scores(q, k)
    for b, L in enumerate(kl):
        m = valid_mask(S, L, causal)
        p = np.where(m, np.exp(s[b] - lse[b][..., None]), 0.0)
        np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_values_return_the_value(causal):
    B, H, S, D = 2, 3, 29, 4
    q, k = _rand((B, H, S, D), 1), _rand((B, H, S, D), 2)
    c = np.array([0.5, -2.0, 3.25, 7.0])
    v = np.broadcast_to(c, (B, H, S, D)).copy()
    out, _ = attention(q, k, v, causal=causal, key_len=[S, 5])
    np.testing.assert_allclose(out, np.broadcast_to(c, out.shape), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_keys_give_mean_of_visible_values(causal):
    """K = 0 makes every visible score 0: uniform weights, lse = ln(#visible)."""
    B, H, S, D = 2, 2, 19, 5
    q, v = _rand((B, H, S, D), 3), _rand((B, H, S, D), 4)
    k = np.zeros((B, H, S, D))
    kl = [S, 7]
    out, lse = attention(q, k, v, causal=causal, key_len=kl)
    for b, L in enumerate(kl):
        for i in range(S):
            n = min(L, i + 1) if causal else L
            np.testing.assert_allclose(out[b, :, i], v[b, :, :n].mean(axis=1), rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse[b, :, i], math.log(n), rtol=0, atol=1e-13)


def test_single_key():
    q, k, v = (_rand((1, 3, 1, 6), 30 + t) for t in range(3))
    out, lse = attention(q, k, v)
    np.testing.assert_array_equal(out, v)
    np.testing.assert_allclose(lse[..., 0], (q * k).sum(-1)[..., 0] / math.sqrt(6), rtol=1e-14)


def test_causal_row0_is_v0_and_rows_are_prefix_attention():
    B, H, S, D = 1, 2, 24, 8
    q, k, v = (_rand((B, H, S, D), 40 + t) for t in range(3))
    out, lse = attention(q, k, v, causal=True)
    np.testing.assert_array_equal(out[:, :, 0], v[:, :, 0])
    for i in [1, 5, 23]:
        # non-causal attention of row i over the prefix K[0..i], V[0..i]
        qq = np.repeat(q[:, :, i:i + 1], i + 1, axis=2)
        o2, l2 = attention(qq, k[:, :, :i + 1], v[:, :, :i + 1], causal=False)
        np.testing.assert_allclose(out[:, :, i], o2[:, :, 0], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, i], l2[:, :, 0], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_key_len_is_truncation_and_padding_is_ignored(causal):
    B, H, S, D = 3, 2, 40, 8
    q, k, v = (_rand((B, H, S, D), 50 + t) for t in range(3))
    kl = [40, 13, 1]
    out, lse = attention(q, k, v, causal=causal, key_len=kl)
    # poison every padded key / value row: the result must not move
    kp, vp = k.copy(), v.copy()
    for b, L in enumerate(kl):
        kp[b, :, L:] = np.nan
        vp[b, :, L:] = np.inf
    out_p, lse_p = attention(q, kp, vp, causal=causal, key_len=kl)
    np.testing.assert_array_equal(out, out_p)
    np.testing.assert_array_equal(lse, lse_p)
    for b, L in enumerate(kl):
        # a row that sees keys 0..L-1 equals non-causal attention over the
        # truncated K[:L], V[:L] with no key-length argument at all
        rows = [i for i in (0, L - 1, L, S - 1) if 0 <= i < S and (not causal or i >= L - 1)]
        for i in rows:
            qq = np.repeat(q[b:b + 1, :, i:i + 1], L, axis=2)
            o2, l2 = attention(qq, k[b:b + 1, :, :L], v[b:b + 1, :, :L], causal=False)
            np.testing.assert_allclose(out[b, :, i], o2[0, :, 0], rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(lse[b, :, i], l2[0, :, 0], rtol=1e-13, atol=1e-13)


def test_causal_key_mask_is_redundant_for_valid_queries():
    """Under causal masking a valid query i < L only sees keys j <= i < L, so
    adding the key-length mask changes nothing for those rows (section 2.1,
    'The mask trick')."""
    B, H, S, D = 4, 2, 32, 8
    q, k, v = (_rand((B, H, S, D), 60 + t) for t in range(3))
    kl = [32, 20, 7, 1]
    both, lb = attention(q, k, v, causal=True, key_len=kl)
    causal_only, lc = attention(q, k, v, causal=True)
    for b, L in enumerate(kl):
        np.testing.assert_array_equal(both[b, :, :L], causal_only[b, :, :L])
        np.testing.assert_array_equal(lb[b, :, :L], lc[b, :, :L])
    # and the padded rows do differ (they see only L keys)
    assert not np.allclose(both[2, :, 7:], causal_only[2, :, 7:])


def test_permutation_equivariance():
    B, H, S, D = 2, 3, 21, 8
    q, k, v = (_rand((B, H, S, D), 70 + t) for t in range(3))
    out, lse = attention(q, k, v)
    rng = np.random.default_rng(0)
    pk = rng.permutation(S)
    o2, l2 = attention(q, k[:, :, pk], v[:, :, pk])  # joint key/value permutation
    np.testing.assert_allclose(o2, out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, lse, rtol=1e-13)
    pq = rng.permutation(S)
    o3, l3 = attention(q[:, :, pq], k, v)            # query permutation
    np.testing.assert_allclose(o3, out[:, :, pq], rtol=1e-13, atol=1e-14)
    pb, ph = rng.permutation(B), rng.permutation(H)  # (b, h) shuffle
    o4, l4 = attention(q[pb][:, ph], k[pb][:, ph], v[pb][:, ph])
    np.testing.assert_allclose(o4, out[pb][:, ph], rtol=1e-13, atol=1e-14)


def test_large_logits_are_near_one_hot():
    """Inputs scaled x30 give near one-hot rows: out ~ v at the argmax score,
    with no overflow because the row maximum is subtracted first."""
    B, H, S, D = 1, 2, 50, 16
    q, k, v = _rand((B, H, S, D), 80, 30.0), _rand((B, H, S, D), 81, 30.0), _rand((B, H, S, D), 82)
    out, lse = attention(q, k, v)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    s = _scores(q, k)
    arg = s.argmax(-1)
    pick = np.take_along_axis(v, arg[..., None], axis=2)
    srt = np.sort(s, axis=-1)
    clear = (srt[..., -1] - srt[..., -2]) > 40.0
    assert clear.mean() > 0.5
    np.testing.assert_allclose(out[clear], pick[clear], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[clear], srt[..., -1][clear], rtol=1e-14, atol=1e-12)


def test_rows_match_full_attention():
    B, H, S, D = 2, 3, 45, 8
    q, k, v = (_rand((B, H, S, D), 90 + t) for t in range(3))
    kl = [45, 30]
    for causal in (False, True):
        out, lse = attention(q, k, v, causal=causal, key_len=kl)
        rows = np.array([(0, 0, 0), (1, 2, 44), (1, 1, 29), (1, 1, 30), (0, 2, 17), (1, 0, 3)])
        ro, rl = attention_rows(q, k, v, rows, causal=causal, key_len=kl)
        np.testing.assert_allclose(ro, out[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(rl, lse[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=1e-13)
        # the same through torch tensors (how device tensors are read back)
        ro2, rl2 = attention_rows(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                  rows, causal=causal, key_len=torch.tensor(kl))
        np.testing.assert_array_equal(ro2, ro)


def test_valid_pair_count():
    for S, causal in [(128, True), (100, False), (37, True)]:
        kl = [S, 64, 1, 0, S // 2]
        want = sum(int(valid_mask(S, L, causal).sum()) for L in kl) * 3
        assert count_valid_pairs(S, kl, causal, B=len(kl), H=3) == want


def test_exact_upcast_from_half():
    x = torch.randn(1, 1, 8, 16).half()
    o1, _ = attention(x, x, x)
    o2, _ = attention(x.double().numpy(), x.double().numpy(), x.double().numpy())
    np.testing.assert_array_equal(o1, o2)


# ------------------------------------------------------------------ the rule

def test_gate_rule_boundaries():
    r = np.array([0.0, 0.0, 1.0, 1.0, 10.0, -10.0, 0.05, 0.2, 0.2])
    u = np.array([0.0019, 0.0021, 1.019, 1.021, 10.15, -10.25, 0.0519, 0.2039, 0.2041])
    ok = oracle.gate(u, r)
    assert ok.tolist() == [True, False, True, False, True, False, True, True, False]
    assert oracle.budget_fraction(np.array([0.001]), np.array([0.0])) == pytest.approx(0.5)
    assert oracle.budget_fraction(np.array([1.01]), np.array([1.0])) == pytest.approx(0.5)


def test_gate_nonfinite():
    r = np.array([1.0, -np.inf, -np.inf, 0.5])
    u = np.array([np.nan, -np.inf, 0.0, np.inf])
    assert oracle.gate(u, r).tolist() == [False, True, False, False]
    assert oracle.budget_fraction(u[1:2], r[1:2]) == 0.0
    assert oracle.budget_fraction(u, r) == np.inf


# ---------------------------------------------------------- planted mistakes

def _brute_agrees(seed=5):
    ok = True
    for causal in (False, True):
        for S, D, L in [(5, 3, 5), (6, 4, 3), (8, 2, 8)]:
            q, k, v = (_rand((1, 1, S, D), seed + t) for t in range(3))
            out, lse = attention(q, k, v, causal=causal, key_len=[L])
            bo, _ = _brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), causal, L)
            ok &= np.allclose(out[0, 0], np.array(bo), rtol=1e-12, atol=1e-12)
    return ok


def test_brute_force_catches_planted_mistakes(monkeypatch):
    assert _brute_agrees()

    # 1. causal diagonal excluded (j < i instead of j <= i)
    orig = oa.valid_mask

    def off_by_one(S, L, causal, rows=None):
        m = orig(S, L, causal, rows)
        if causal:
            i = np.arange(S) if rows is None else np.asarray(rows)
            m &= np.arange(S)[None, :] != i[:, None]
            m[:, 0] |= (L > 0)
        return m
    monkeypatch.setattr(oa, "valid_mask", off_by_one)
    assert not _brute_agrees()
    monkeypatch.setattr(oa, "valid_mask", orig)

    # 2. key length ignored
    monkeypatch.setattr(oa, "valid_mask", lambda S, L, causal, rows=None: orig(S, S, causal, rows))
    assert not _brute_agrees()
    monkeypatch.setattr(oa, "valid_mask", orig)

    # 3. 1/sqrt(d_h) scale dropped
    monkeypatch.setattr(oa, "math", types.SimpleNamespace(sqrt=lambda x: 1.0))
    assert not _brute_agrees()
    monkeypatch.setattr(oa, "math", math)

    # 4. softmax normaliser dropped / wrong sign in the exponent
    orig_sr = oa._softmax_rows

    def neg(s, mask, v):
        return orig_sr(-s, mask, v)
    monkeypatch.setattr(oa, "_softmax_rows", neg)
    assert not _brute_agrees()

    # 5. transposed score matrix (keys and queries swapped)
    def transposed(s, mask, v):
        return orig_sr(np.swapaxes(s, -1, -2), mask, v)
    monkeypatch.setattr(oa, "_softmax_rows", transposed)
    assert not _brute_agrees()
    monkeypatch.setattr(oa, "_softmax_rows", orig_sr)
    assert _brute_agrees()
