"""Randomized parity against the float64 oracle: forward (every head size and
dtype, the automatic variant choice), backward (plain and grouped-query
heads) and the fused QKV projection, over random shapes, masks, key lengths
and input scales, under the graded rule |u-r| <= 2e-3 or <= 2e-2 |r|.

Each seed draws its cases (250 in the first test, 200 in the second) from
one generator; every case is seeded by its index. Input scales go beyond the pages' workloads on purpose: q and k up to
8 times unit variance in the forward (scores of a few hundred), 3 times in
the backward, projection weights up to twice the default initialisation
scale. These seeds found four precision problems that the fixed-shape tests
did not (the backward's row term and its dS and P roundings, the fused
projection's q and k rounding); each now has a test of its own."""

import random

import pytest
import torch

import exact_attention_mha_amd as mha_lib
import oracle
from gpu_helpers import THREADS
from oracle.qkv import qkv_attention as oracle_qkv

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
CASES_PER_SEED = 250


def _key_len(rng, B, S):
    if rng.random() < 0.4:
        return None
    return torch.tensor([rng.choice([S, 0, 1, rng.randint(0, S)]) for _ in range(B)],
                        dtype=torch.int32)


def _check(label, pairs):
    for name, u, r in pairs:
        ok = oracle.gate(u, r)
        assert ok.all(), f"{label} {name}: budget {oracle.budget_fraction(u, r):.3f}"


def _forward_case(mha, rng, g, causal, scale, case):
    D = rng.choice([8, 16, 32, 64, 128, 256])
    dt = rng.choice(["f16", "bf16", "f32"] if D != 8 else ["f16", "bf16"])
    S = rng.choice([rng.randint(1, 130), rng.randint(1, 600)])
    B, H = rng.randint(1, 4), rng.randint(1, 4)
    if dt == "f32":
        S = min(S, 200)
    q, k, v = (torch.randn(B, H, S, D, generator=g) for _ in range(3))
    q, k, v = (q * scale).to(DT[dt]), (k * scale).to(DT[dt]), v.to(DT[dt])
    kl = _key_len(rng, B, S)
    label = f"case {case} fwd B{B} H{H} S{S} D{D} {dt} causal={causal} scale={scale} kl={kl}"
    print(label, flush=True)
    out, lse = mha.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal,
                           key_len=None if kl is None else kl.cuda())
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, causal=causal, key_len=kl, threads=THREADS)
    _check(label, [("out", out.cpu(), ro), ("lse", lse.cpu(), rl)])


def _backward_case(mha, rng, g, causal, scale, case):
    D = rng.choice([16, 32, 64, 64, 128])
    dt = rng.choice(["f16", "bf16"])
    S, B, Hk = rng.randint(1, 400), rng.randint(1, 3), rng.randint(1, 3)
    H = Hk * rng.choice([1, 1, 2, 3])
    q = torch.randn(B, H, S, D, generator=g).mul(min(scale, 3.0)).to(DT[dt])
    k = torch.randn(B, Hk, S, D, generator=g).mul(min(scale, 3.0)).to(DT[dt])
    v = torch.randn(B, Hk, S, D, generator=g).to(DT[dt])
    do = torch.randn(B, H, S, D, generator=g).to(DT[dt])
    kl = _key_len(rng, B, S)
    label = f"case {case} bwd B{B} H{H}/{Hk} S{S} D{D} {dt} causal={causal} kl={kl}"
    print(label, flush=True)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    kld = None if kl is None else kl.cuda()
    out, lse = mha.forward(qd, kd, vd, causal=causal, key_len=kld)
    dq, dk, dv = mha.backward(qd, kd, vd, out, lse, dod, causal=causal, key_len=kld)
    torch.cuda.synchronize()
    grp = H // Hk
    ke, ve = (t.repeat_interleave(grp, dim=1) for t in (k, v))
    rq, rk, rv = oracle.attention_backward(q, ke, ve, do, causal=causal, key_len=kl,
                                           threads=THREADS)
    rk = rk.reshape(B, Hk, grp, S, D).sum(axis=2)
    rv = rv.reshape(B, Hk, grp, S, D).sum(axis=2)
    _check(label, [("dq", dq.cpu(), rq), ("dk", dk.cpu(), rk), ("dv", dv.cpu(), rv)])


def _qkv_case(mha, rng, g, causal, scale, case):
    hd = rng.choice([8, 16])
    H = rng.choice([2, 4, 8] if hd == 16 else [4, 8, 16])
    Dm = H * hd
    if Dm not in (32, 64, 128):
        return
    dt = rng.choice(["f16", "bf16"])
    S, B = rng.randint(1, 128), rng.randint(1, 40)
    x = torch.randn(B, S, Dm, generator=g).to(DT[dt])
    w = ((torch.rand(Dm, 3 * Dm, generator=g) * 2 - 1) / Dm ** 0.5 * min(scale, 2.0)).to(DT[dt])
    bias = (None if rng.random() < 0.3
            else ((torch.rand(3 * Dm, generator=g) * 2 - 1) / Dm ** 0.5).to(DT[dt]))
    kl = _key_len(rng, B, S)
    label = (f"case {case} qkv B{B} S{S} H{H}x{hd} {dt} causal={causal} scale={scale} "
             f"bias={bias is not None}")
    print(label, flush=True)
    out, lse = mha.qkv_attention(x.cuda(), w.cuda(), None if bias is None else bias.cuda(),
                                 n_heads=H, causal=causal,
                                 key_len=None if kl is None else kl.cuda(), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle_qkv(x, w, bias, H, causal=causal, key_len=kl, threads=THREADS)
    _check(label, [("out", out.cpu(), ro), ("lse", lse.cpu(), rl)])


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_randomized_parity(mha, seed):
    rng = random.Random(seed)
    run = {"fwd": _forward_case, "bwd": _backward_case, "qkv": _qkv_case}
    for case in range(CASES_PER_SEED):
        kind = rng.choice(["fwd", "fwd", "bwd", "qkv"])
        g = torch.Generator().manual_seed(case * 7919 + seed)
        causal = rng.random() < 0.5
        scale = rng.choice([1.0, 1.0, 3.0, 8.0])
        run[kind](mha, rng, g, causal, scale, case)


def _variant_case(mha, rng, g, causal, scale, case):
    variant = rng.choice(["mfma", "mfma_small", "short", "valu_d16", "mfma32", "f32"])
    if variant == "mfma32":  # a retired variant; drawn still, so the case stream stays the same
        variant = "mfma"
    D = rng.choice([8, 16, 32, 64, 128, 256])
    dt = rng.choice(["f16", "bf16", "f32"])
    S = rng.choice([rng.randint(1, 130), rng.randint(1, 700)])
    B, H = rng.randint(1, 3), rng.randint(1, 3)
    if dt == "f32":
        S = min(S, 200)
    q, k, v = (torch.randn(B, H, S, D, generator=g) for _ in range(3))
    q, k, v = (q * scale).to(DT[dt]), (k * scale).to(DT[dt]), v.to(DT[dt])
    kl = _key_len(rng, B, S)
    label = f"case {case} fwd {variant} B{B} H{H} S{S} D{D} {dt} causal={causal} scale={scale}"
    print(label, flush=True)
    try:
        out, lse = mha.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal,
                               key_len=None if kl is None else kl.cuda(), variant=variant)
    except mha_lib.MhaError as e:
        if e.status == 3:  # this variant does not run this dtype / head size
            return
        raise
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q, k, v, causal=causal, key_len=kl, threads=THREADS)
    _check(label, [("out", out.cpu(), ro), ("lse", lse.cpu(), rl)])


def _long_backward_case(mha, rng, g, causal, scale, case):
    D = rng.choice([16, 32, 64, 128, 256])
    dt = rng.choice(["f16", "bf16"])
    S = rng.randint(1, 700 if D <= 128 else 300)
    B, Hk = rng.randint(1, 2), rng.randint(1, 2)
    H = Hk * rng.choice([1, 2, 4])
    q = torch.randn(B, H, S, D, generator=g).mul(min(scale, 3.0)).to(DT[dt])
    k = torch.randn(B, Hk, S, D, generator=g).mul(min(scale, 3.0)).to(DT[dt])
    v = torch.randn(B, Hk, S, D, generator=g).to(DT[dt])
    do = torch.randn(B, H, S, D, generator=g).to(DT[dt])
    kl = _key_len(rng, B, S)
    label = f"case {case} bwd B{B} H{H}/{Hk} S{S} D{D} {dt} causal={causal} kl={kl}"
    print(label, flush=True)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    kld = None if kl is None else kl.cuda()
    out, lse = mha.forward(qd, kd, vd, causal=causal, key_len=kld)
    dq, dk, dv = mha.backward(qd, kd, vd, out, lse, dod, causal=causal, key_len=kld)
    torch.cuda.synchronize()
    grp = H // Hk
    ke, ve = (t.repeat_interleave(grp, dim=1) for t in (k, v))
    rq, rk, rv = oracle.attention_backward(q, ke, ve, do, causal=causal, key_len=kl,
                                           threads=THREADS)
    rk = rk.reshape(B, Hk, grp, S, D).sum(axis=2)
    rv = rv.reshape(B, Hk, grp, S, D).sum(axis=2)
    _check(label, [("dq", dq.cpu(), rq), ("dk", dk.cpu(), rk), ("dv", dv.cpu(), rv)])


def _strided_case(mha, rng, g, causal, scale, case):
    D = rng.choice([8, 16, 32, 64, 128, 256])
    dt = rng.choice(["f16", "bf16"])
    S, B, Hk = rng.randint(1, 600), rng.randint(1, 3), rng.randint(1, 3)
    H = Hk * rng.choice([1, 2, 3])
    qs = torch.randn(B, S, H, D, generator=g).mul(scale).to(DT[dt])
    ks = torch.randn(B, S, Hk, D, generator=g).mul(scale).to(DT[dt])
    vs = torch.randn(B, S, Hk, D, generator=g).to(DT[dt])
    kl = _key_len(rng, B, S)
    label = f"case {case} strided B{B} H{H}/{Hk} S{S} D{D} {dt} causal={causal} scale={scale}"
    print(label, flush=True)
    qd, kd, vd = (t.cuda().transpose(1, 2) for t in (qs, ks, vs))
    out = torch.empty(B, S, H, D, dtype=DT[dt], device="cuda")
    try:
        _, lse = mha.forward(qd, kd, vd, causal=causal, key_len=None if kl is None else kl.cuda(),
                             out=out.transpose(1, 2))
    except mha_lib.MhaError as e:
        if e.status == 3:  # a head size the strided entry point does not take
            return
        raise
    torch.cuda.synchronize()
    grp = H // Hk
    q = qs.transpose(1, 2).contiguous()
    k, v = (t.transpose(1, 2).repeat_interleave(grp, dim=1).contiguous() for t in (ks, vs))
    ro, rl = oracle.attention(q, k, v, causal=causal, key_len=kl, threads=THREADS)
    _check(label, [("out", out.transpose(1, 2).cpu(), ro), ("lse", lse.cpu(), rl)])


@pytest.mark.parametrize("seed", [1, 2])
def test_randomized_variants_layouts_long_backward(mha, seed):
    """Every forward variant forced (combinations a variant does not run are
    rejected by the library and skipped), [B, S, H, d_h] views with grouped
    heads, and the backward up to d_h 256 and S 700; q and k up to 3 times
    unit variance in the backward (scores of spread 9: beyond that fp32
    score arithmetic itself reaches the rule, as the CPU test of the
    backward roundings shows)."""
    rng = random.Random(1000 + seed)
    run = {"fwdv": _variant_case, "bwd": _long_backward_case, "strided": _strided_case}
    for case in range(200):
        kind = rng.choice(["fwdv", "fwdv", "bwd", "strided"])
        g = torch.Generator().manual_seed(case * 7919 + 1000 + seed)
        causal = rng.random() < 0.5
        scale = rng.choice([1.0, 1.0, 3.0, 8.0])
        run[kind](mha, rng, g, causal, scale, case)


def _training_case(mha, rng, g, causal, scale, case):
    """The training pair: mha_forward_train's fp32 output against the
    oracle's output, and mha_backward_train's gradients (row term from that
    output) against the oracle's, for plain and grouped-query heads."""
    D = rng.choice([16, 32, 64, 64, 128, 256])
    dt = rng.choice(["f16", "bf16"])
    S, B, Hk = rng.randint(1, 400), rng.randint(1, 3), rng.randint(1, 3)
    H = Hk * rng.choice([1, 1, 2, 3])
    q = torch.randn(B, H, S, D, generator=g).mul(min(scale, 3.0)).to(DT[dt])
    k = torch.randn(B, Hk, S, D, generator=g).mul(min(scale, 3.0)).to(DT[dt])
    v = torch.randn(B, Hk, S, D, generator=g).to(DT[dt])
    do = torch.randn(B, H, S, D, generator=g).to(DT[dt])
    kl = _key_len(rng, B, S)
    label = f"case {case} train B{B} H{H}/{Hk} S{S} D{D} {dt} causal={causal} kl={kl}"
    print(label, flush=True)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    kld = None if kl is None else kl.cuda()
    out, lse, out32 = mha.forward_train(qd, kd, vd, causal=causal, key_len=kld)
    dq, dk, dv = mha.backward_train(qd, kd, vd, out32, lse, dod, causal=causal, key_len=kld)
    torch.cuda.synchronize()
    grp = H // Hk
    ke, ve = (t.repeat_interleave(grp, dim=1) for t in (k, v))
    ro, rl = oracle.attention(q, ke, ve, causal=causal, key_len=kl, threads=THREADS)
    rq, rk, rv = oracle.attention_backward(q, ke, ve, do, causal=causal, key_len=kl,
                                           threads=THREADS)
    rk = rk.reshape(B, Hk, grp, S, D).sum(axis=2)
    rv = rv.reshape(B, Hk, grp, S, D).sum(axis=2)
    _check(label, [("out", out.cpu(), ro), ("out32", out32.cpu(), ro), ("lse", lse.cpu(), rl),
                   ("dq", dq.cpu(), rq), ("dk", dk.cpu(), rk), ("dv", dv.cpu(), rv)])


@pytest.mark.parametrize("seed", [11, 12])
def test_randomized_training_pair(mha, seed):
    rng = random.Random(seed)
    for case in range(100):
        g = torch.Generator().manual_seed(case * 7919 + seed)
        causal = rng.random() < 0.5
        scale = rng.choice([1.0, 1.0, 2.0, 3.0])
        _training_case(mha, rng, g, causal, scale, case)
