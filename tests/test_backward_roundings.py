"""Two roundings the backward kernels avoid, each shown to break the graded
accuracy rule (|u-r| <= 2e-3 or <= 2e-2 |r|) on inputs with large scores,
while the kernels' own arithmetic meets it. CPU only, float64, against the
pinned backward oracle; the gradients follow rustingstudio
"brain/docs/baseline", "Fused attention" (the row term and dS).

1. The softmax row term D_i = sum_j P_ij dP_ij equals dO_i . O_i for the
   exact output. Taking it from O rounded to fp16 or bf16 adds an error of
   about |dO| |O| 2^-11 (2^-8 for bf16) to D, and dQ_i = sum_j P_ij (dP_ij -
   D_i) k_j carries it as that error times sum_j P_ij k_j: where the softmax
   is peaked that sum is a whole key vector and nothing averages it away.
2. dS = P * (dP - D) rounded once to fp16 as a matrix-core operand: dP grows
   with d_h and the value scale, and where dQ or dK cancels to a small value
   the rounding errors of the few large dS terms stay; a head and a
   remainder, both fp16, carry dS to about 2^-22 instead.
3. P rounded once to fp16 for dV = P^T dO: with a peaked softmax each key's
   dV sums a few probabilities near 1 (over the query heads of a group too),
   and their 2^-12 relative rounding no longer averages out. P is split the
   same way.
"""

import math

import numpy as np
import pytest
import torch

import oracle

DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _peaked(dt):
    """B=3, H=9 query heads over 3 key / value heads, S=64, d_h=128, q and k
    scaled by 3 (scores of a few tens), inputs rounded to the dtype."""
    B, H, Hk, S, D = 3, 9, 3, 64, 128
    g = torch.Generator().manual_seed(158381)
    q = torch.randn(B, H, S, D, generator=g).mul(3.0).to(DT[dt])
    k = torch.randn(B, Hk, S, D, generator=g).mul(3.0).to(DT[dt])
    v = torch.randn(B, Hk, S, D, generator=g).to(DT[dt])
    do = torch.randn(B, H, S, D, generator=g).to(DT[dt])
    k, v = (t.repeat_interleave(H // Hk, dim=1) for t in (k, v))
    return tuple(t.double().numpy() for t in (q, k, v, do))


def _dq_given_row_term(q, k, v, do, row):
    """dQ through causal softmax attention with the row term supplied."""
    S, D = q.shape[-2:]
    sc = 1.0 / math.sqrt(D)
    s = np.where(np.tril(np.ones((S, S), bool)), (q @ np.swapaxes(k, -1, -2)) * sc, -np.inf)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    dp = do @ np.swapaxes(v, -1, -2)
    return (p * (dp - row[..., None])) @ k * sc


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_row_term_from_rounded_output_breaks_the_rule(dt):
    q, k, v, do = _peaked(dt)
    ref = oracle.attention_backward(q, k, v, do, causal=True)[0]
    out = oracle.attention(q, k, v, causal=True)[0]
    exact = _dq_given_row_term(q, k, v, do, (do * out).sum(-1))
    # the formula above is the oracle's dq when D is exact
    assert np.allclose(exact, ref, rtol=1e-9, atol=1e-9)
    rounded_out = torch.from_numpy(out).to(DT[dt]).double().numpy()
    from_rounded = _dq_given_row_term(q, k, v, do, (do * rounded_out).sum(-1))

    def as_dt(x):
        return torch.from_numpy(x).to(DT[dt]).double().numpy()

    # one rounding of the exact dq to the output dtype fits the rule;
    # the same rounding of dq built on D from the rounded output does not
    assert oracle.gate(as_dt(exact), ref).all()
    assert not oracle.gate(as_dt(from_rounded), ref).all()
    assert oracle.budget_fraction(as_dt(from_rounded), ref) > 1.5


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_row_term_from_the_fp32_output_meets_the_rule(dt):
    """The training pair's reading: D = dO . O32 with O32 the forward's output
    before its final rounding, built as the training forward builds it
    (unnormalised probabilities as a head and a remainder in the input dtype
    in the value product; fp32 accumulation; divided by the row sum of those
    pairs) and the backward's P rebuilt from lse = m + ln(that sum). On the
    peaked inputs where D from the rounded output misses the rule, dq and dk
    built on it stay inside with margin; with the probabilities rounded
    once (fp16), as the plain forward takes them, the margin shrinks to
    about half the budget here and random cases at this scale crossed it."""
    q, k, v, do = _peaked(dt)
    rq, rk, _ = oracle.attention_backward(q, k, v, do, causal=True)
    S, D = q.shape[-2:]
    sc = 1.0 / math.sqrt(D)
    s = np.where(np.tril(np.ones((S, S), bool)), (q @ np.swapaxes(k, -1, -2)) * sc, -np.inf)
    e = np.exp(s - s.max(axis=-1, keepdims=True))

    def as_dt(x):
        return torch.from_numpy(x).to(torch.float32).to(DT[dt]).double().numpy()

    def grads(pr):
        l = pr.sum(axis=-1, keepdims=True)
        o32 = torch.from_numpy((pr @ v) / l).float().double().numpy()
        p = e / l
        dp = do @ np.swapaxes(v, -1, -2)
        ds = p * (dp - (do * o32).sum(axis=-1, keepdims=True))
        return as_dt(ds @ k * sc), as_dt(np.swapaxes(ds, -1, -2) @ q * sc)

    head = as_dt(e)
    gq, gk = grads(head + as_dt(e - head))
    assert oracle.budget_fraction(gq, rq) < 0.25
    assert oracle.budget_fraction(gk, rk) < 0.25
    if dt == "f16":
        gq, gk = grads(head)
        assert 0.25 < oracle.budget_fraction(gq, rq) < 1.0


def _wide(seed=538493):
    """B=3, H=3, S=326, d_h=64, q and k scaled by 3, fp16, no mask."""
    B, H, S, D = 3, 3, 326, 64
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, S, D, generator=g).mul(3.0).half()
    k = torch.randn(B, H, S, D, generator=g).mul(3.0).half()
    v = torch.randn(B, H, S, D, generator=g).half()
    do = torch.randn(B, H, S, D, generator=g).half()
    return tuple(t.double().numpy() for t in (q, k, v, do))


def _f16(x):
    return torch.from_numpy(x).half().double().numpy()


def test_single_fp16_rounding_of_ds_breaks_the_rule():
    q, k, v, do = _wide()
    rq, rk, _ = oracle.attention_backward(q, k, v, do)
    S, D = q.shape[-2:]
    sc = 1.0 / math.sqrt(D)
    s = (q @ np.swapaxes(k, -1, -2)) * sc
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    dp = do @ np.swapaxes(v, -1, -2)
    ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))

    def grads(dsx):
        return _f16(dsx @ k * sc), _f16(np.swapaxes(dsx, -1, -2) @ q * sc)

    # exact dS: the oracle's gradients, one rounding to fp16 away
    for u, r in zip(grads(ds), (rq, rk)):
        assert oracle.gate(u, r).all()
    # dS rounded once: dQ misses the rule
    head = _f16(ds)
    gq, gk = grads(head)
    assert not oracle.gate(gq, rq).all()
    assert oracle.budget_fraction(gq, rq) > 1.1
    # head + remainder: back inside, with the exact dS's margin
    for u, r in zip(grads(head + _f16(ds - head)), (rq, rk)):
        assert oracle.budget_fraction(u, r) < 0.1


def test_single_fp16_rounding_of_p_breaks_the_rule_on_dv():
    """B=3, 9 query heads over 3 key / value heads, S=108, d_h=64, causal, q
    and k scaled by 3: dV of each key / value head summed over its group."""
    B, H, Hk, S, D = 3, 9, 3, 108, 64
    g = torch.Generator().manual_seed(221735)
    q = torch.randn(B, H, S, D, generator=g).mul(3.0).half()
    k = torch.randn(B, Hk, S, D, generator=g).mul(3.0).half()
    v = torch.randn(B, Hk, S, D, generator=g).half()
    do = torch.randn(B, H, S, D, generator=g).half()
    grp = H // Hk
    qn, dn = q.double().numpy(), do.double().numpy()
    kn, vn = (t.repeat_interleave(grp, dim=1).double().numpy() for t in (k, v))
    ref = oracle.attention_backward(qn, kn, vn, dn, causal=True)[2]
    ref = ref.reshape(B, Hk, grp, S, D).sum(axis=2)
    s = np.where(np.tril(np.ones((S, S), bool)),
                 (qn @ np.swapaxes(kn, -1, -2)) / math.sqrt(D), -np.inf)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)

    def dv(px):
        return _f16((np.swapaxes(px, -1, -2) @ dn).reshape(B, Hk, grp, S, D).sum(axis=2))

    assert oracle.gate(dv(p), ref).all()
    head = _f16(p)
    assert not oracle.gate(dv(head), ref).all()
    assert oracle.budget_fraction(dv(head + _f16(p - head)), ref) < 0.1


def test_fp32_score_arithmetic_is_the_limit_at_score_spread_64():
    """Where the backward stops meeting the rule, and why no kernel change
    fixes it: with q and k at 8 times unit variance (scores with a standard
    deviation of 64, d_h 32), the probabilities rebuilt from fp32 scores and
    an fp32 exponent argument alone (every other step exact) use most of the
    budget on dq. dq there is a near-cancelling sum, and an exponent argument
    of a few hundred carries an fp32 rounding of ~2^-16, i.e. that relative
    error in P. The kernels also accumulate the scores in fp32 and take an
    fp32 log-sum-exp from the forward, which goes past the rule: the
    backward's domain is scores of moderate spread (3 times unit variance, a
    spread of 9, passes with margin)."""
    B, H, Hk, S, D = 2, 8, 2, 618, 32
    g = torch.Generator().manual_seed(309842)
    q = torch.randn(B, H, S, D, generator=g).mul(8.0).bfloat16()
    k = torch.randn(B, Hk, S, D, generator=g).mul(8.0).bfloat16()
    v = torch.randn(B, Hk, S, D, generator=g).bfloat16()
    do = torch.randn(B, H, S, D, generator=g).bfloat16()
    grp = H // Hk
    qn, dn = q.double().numpy(), do.double().numpy()
    kn, vn = (t.repeat_interleave(grp, dim=1).double().numpy() for t in (k, v))
    ref = oracle.attention_backward(qn, kn, vn, dn)[0]
    sc = 1.0 / math.sqrt(D)
    s = qn @ np.swapaxes(kn, -1, -2)
    lse = s.max(axis=-1) * sc
    lse += np.log(np.exp(s * sc - lse[..., None]).sum(axis=-1))
    dp = dn @ np.swapaxes(vn, -1, -2)

    def dq(p):
        return (p * (dp - (p * dp).sum(axis=-1, keepdims=True))) @ kn * sc

    def bf16(x):
        return torch.from_numpy(x).bfloat16().double().numpy()

    exact = np.exp(s * sc - lse[..., None])
    c2 = np.float32(sc / math.log(2))
    arg = s.astype(np.float32) * c2 - (lse / math.log(2)).astype(np.float32)[..., None]
    p32 = np.exp2(arg.astype(np.float64))
    assert oracle.budget_fraction(bf16(dq(exact)), ref) < 0.3
    assert oracle.budget_fraction(bf16(dq(p32)), ref) > 0.7


def _dq_from_lse(q, k, v, do, lse, renormalise):
    """dQ as the backward kernels form it: P rebuilt from a stored lse,
    D = rowsum(P dP), optionally divided by rowsum(P)."""
    S, D = q.shape[-2:]
    sc = 1.0 / math.sqrt(D)
    s = np.where(np.tril(np.ones((S, S), bool)), (q @ np.swapaxes(k, -1, -2)) * sc, -np.inf)
    p = np.exp(s - lse[..., None])
    dp = do @ np.swapaxes(v, -1, -2)
    row = (p * dp).sum(-1)
    if renormalise:
        row = row / p.sum(-1)
    return (p * (dp - row[..., None])) @ k * sc


def test_lse_from_rounded_probabilities_needs_a_renormalised_row_term():
    """A forward that sums its fp16-rounded probabilities for the row sum
    (the same weights its numerator uses) stores an lse whose rebuilt
    probabilities sum to 1 only within that rounding (about 1e-4). The
    backward's row term D = rowsum(P dP) then leaves the rows of
    dS = P (dP - D) summing to (1 - rowsum P) D instead of 0, and dQ keeps a
    term D sum_j P_ij k_j; dividing D by rowsum(P) cancels it, leaving only a
    common factor. Case: B=1, H=2, S=273, d_h=16, causal, q and k scaled by
    3 and v by 3, fp16 inputs."""
    S, D = 273, 16
    g = torch.Generator().manual_seed(1005)
    q, k, v, do = (torch.randn(1, 2, S, D, generator=g) for _ in range(4))
    q, k, v = q * 3, k * 3, v * 3
    q, k, v, do = (t.half().double().numpy() for t in (q, k, v, do))
    ref = oracle.attention_backward(q, k, v, do, causal=True)[0]
    s = np.where(np.tril(np.ones((S, S), bool)), (q @ np.swapaxes(k, -1, -2)) / math.sqrt(D), -np.inf)
    m = s.max(-1, keepdims=True)
    p16 = torch.from_numpy(np.exp(s - m)).half().double().numpy()  # rounded probabilities
    lse_rounded = m[..., 0] + np.log(p16.sum(-1))
    lse_exact = m[..., 0] + np.log(np.exp(s - m).sum(-1))
    assert np.abs(lse_rounded - lse_exact).max() < 2e-3  # inside the rule for lse itself

    def as_f16(x):
        return torch.from_numpy(x).half().double().numpy()

    plain = _dq_from_lse(q, k, v, do, lse_rounded, renormalise=False)
    fixed = _dq_from_lse(q, k, v, do, lse_rounded, renormalise=True)
    assert oracle.budget_fraction(as_f16(plain), ref) > 1.0
    assert oracle.gate(as_f16(fixed), ref).all()
    assert oracle.budget_fraction(as_f16(fixed), ref) < 0.1
