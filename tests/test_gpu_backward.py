"""GPU parity of the backward pass: dq, dk, dv from the HIP kernels (through
the C ABI binding, fed by the HIP forward's out and lse) against the float64
oracle's gradients of the same inputs, element by element, under the same
graded rule as the forward: |u-r| <= 2e-3 or |u-r| <= 2e-2 |r|."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import THREADS

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _inputs(B, H, S, D, dt, seed, key_len=None):
    g = torch.Generator().manual_seed(seed)
    q, k, v, do = (torch.randn(B, H, S, D, generator=g).to(DT[dt]) for _ in range(4))
    kl = None if key_len is None else torch.tensor(key_len, dtype=torch.int32)
    return q, k, v, do, kl


def _run(mha, q, k, v, do, kl, causal):
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    kld = None if kl is None else kl.cuda()
    out, lse = mha.forward(qd, kd, vd, causal=causal, key_len=kld)
    dq, dk, dv = mha.backward(qd, kd, vd, out, lse, dod, causal=causal, key_len=kld)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def _check(got, q, k, v, do, kl, causal, label):
    ref = oracle.attention_backward(q, k, v, do, causal=causal, key_len=kl, threads=THREADS)
    worst = []
    for name, u, r in zip(("dq", "dk", "dv"), got, ref):
        ok = oracle.gate(u, r)
        frac = oracle.budget_fraction(u, r)
        worst.append(frac)
        if not ok.all():
            bad = np.argwhere(~ok)[:5].tolist()
            raise AssertionError(f"{label}: {name}: {int((~ok).sum())} elements fail the rule "
                                 f"(budget {frac:.3f}); first {bad}")
    print(f"{label}: budget dq {worst[0]:.3f} dk {worst[1]:.3f} dv {worst[2]:.3f}", flush=True)
    return worst


SHAPES = [  # (B, H, S, D, key_len)
    (1, 2, 64, 64, None),
    (2, 2, 100, 32, [100, 37]),
    (1, 3, 17, 16, None),
    (2, 2, 130, 128, [130, 66]),
    (1, 2, 96, 256, [96]),
    (2, 1, 200, 64, [1, 200]),
]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:4])))
def test_backward_shapes(mha, shape, causal, dt):
    B, H, S, D, key_len = shape
    q, k, v, do, kl = _inputs(B, H, S, D, dt, 7, key_len)
    got = _run(mha, q, k, v, do, kl, causal)
    _check(got, q, k, v, do, kl, causal, f"{shape} causal={causal} {dt}")


@pytest.mark.parametrize("seed", range(10))
def test_backward_seeds(mha, seed):
    """The pages' backward workload shape reduced in batch (B=1, H=12,
    S=1024, d_h=64, causal, bf16; rustingstudio "brain/docs/baseline",
    "Fused attention"), over seeds."""
    q, k, v, do, kl = _inputs(1, 12, 1024, 64, "bf16", seed)
    got = _run(mha, q, k, v, do, kl, True)
    _check(got, q, k, v, do, kl, True, f"bwd B=1 H=12 S=1024 seed {seed}")


def test_backward_full_workload(mha):
    """B=4, H=12, S=1024, d_h=64, causal, bf16, every element."""
    q, k, v, do, kl = _inputs(4, 12, 1024, 64, "bf16", 0)
    got = _run(mha, q, k, v, do, kl, True)
    _check(got, q, k, v, do, kl, True, "bwd full workload")


def test_backward_edges(mha):
    # no visible key: every gradient is zero
    q, k, v, do, _ = _inputs(2, 2, 40, 64, "f16", 3)
    kl = torch.tensor([0, 40], dtype=torch.int32)
    dq, dk, dv = _run(mha, q, k, v, do, kl, True)
    assert not dq[0].any() and not dk[0].any() and not dv[0].any()
    _check((dq, dk, dv), q, k, v, do, kl, True, "key_len 0")
    # one row, one key
    q, k, v, do, _ = _inputs(1, 1, 1, 32, "f16", 4)
    got = _run(mha, q, k, v, do, None, False)
    _check(got, q, k, v, do, None, False, "S=1")


def test_backward_padding_never_read(mha):
    """NaN in padded key / value rows changes nothing; padded keys get zero."""
    q, k, v, do, _ = _inputs(1, 2, 90, 64, "f16", 5)
    kl = torch.tensor([50], dtype=torch.int32)
    base = _run(mha, q, k, v, do, kl, False)
    kp, vp = k.clone(), v.clone()
    kp[:, :, 50:] = float("nan")
    vp[:, :, 50:] = float("nan")
    pois = _run(mha, q, kp, vp, do, kl, False)
    for a, b in zip(base, pois):
        assert torch.equal(a, b)
    assert not base[1][:, :, 50:].any() and not base[2][:, :, 50:].any()
    _check(base, q, k, v, do, kl, False, "poisoned padding")


def test_backward_deterministic(mha):
    q, k, v, do, _ = _inputs(1, 2, 300, 64, "bf16", 6)
    a = _run(mha, q, k, v, do, None, True)
    b = _run(mha, q, k, v, do, None, True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_backward_row_term_workspace(mha, dt):
    """The workspace holds D = rowsum(P * dP), i.e. dout . O of the exact
    output (float64 oracle), to fp32 accumulation accuracy, for both dtypes."""
    q, k, v, do, _ = _inputs(1, 2, 300, 64, dt, 6)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    out, lse = mha.forward(qd, kd, vd, causal=True)
    delta = torch.empty(lse.shape, dtype=torch.float32, device="cuda")
    mha.backward(qd, kd, vd, out, lse, dod, causal=True, delta=delta)
    torch.cuda.synchronize()
    o64, _ = oracle.attention(q, k, v, causal=True)
    ref = (do.double().numpy() * o64).sum(-1)
    got = delta.cpu().double().numpy()
    assert np.allclose(got, ref, rtol=1e-4, atol=1e-4), np.abs(got - ref).max()


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 8, 2, 200, 64, [200, 77]), (1, 12, 4, 1024, 64, None),
                                   (1, 6, 1, 130, 128, [100]), (2, 4, 2, 64, 16, None)],
                         ids=lambda s: "x".join(map(str, s[:5])))
def test_backward_grouped_heads(mha, shape, causal, dt):
    """Grouped-query attention: the key / value gradients of a group, summed
    over its query heads, against the oracle's gradients of the repeated
    heads summed over each group (the chain rule through the repetition)."""
    B, H, Hk, S, D, key_len = shape
    g = torch.Generator().manual_seed(H * 100 + Hk)
    q = torch.randn(B, H, S, D, generator=g).to(DT[dt])
    k = torch.randn(B, Hk, S, D, generator=g).to(DT[dt])
    v = torch.randn(B, Hk, S, D, generator=g).to(DT[dt])
    do = torch.randn(B, H, S, D, generator=g).to(DT[dt])
    kl = None if key_len is None else torch.tensor(key_len, dtype=torch.int32)
    dq, dk, dv = _run(mha, q, k, v, do, kl, causal)
    grp = H // Hk
    ke, ve = (t.repeat_interleave(grp, dim=1) for t in (k, v))
    rq, rk, rv = oracle.attention_backward(q, ke, ve, do, causal=causal, key_len=kl,
                                           threads=THREADS)
    rk = rk.reshape(B, Hk, grp, S, D).sum(axis=2)
    rv = rv.reshape(B, Hk, grp, S, D).sum(axis=2)
    for name, u, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        ok = oracle.gate(u, r)
        assert ok.all(), (f"{shape} {dt} causal={causal} {name}: {int((~ok).sum())} fail, "
                          f"budget {oracle.budget_fraction(u, r):.3f}")
    print(f"grouped {shape} causal={causal} {dt}: budget dq {oracle.budget_fraction(dq, rq):.3f} "
          f"dk {oracle.budget_fraction(dk, rk):.3f} dv {oracle.budget_fraction(dv, rv):.3f}",
          flush=True)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("heads", [(9, 3), (3, 3)], ids=lambda h: f"H{h[0]}_Hkv{h[1]}")
def test_backward_peaked_softmax(mha, heads, dt):
    """Scores of a few tens (q and k scaled by 3, d_h 128, causal): the
    softmax is peaked, and a row term D taken from the output rounded to the
    input dtype misses the accuracy rule on dq by about three times for fp16
    (the CPU test of the backward roundings shows it); D accumulated as
    rowsum(P * dP) in fp32 meets it."""
    H, Hk = heads
    B, S, D = 3, 64, 128
    g = torch.Generator().manual_seed(158381)
    q = torch.randn(B, H, S, D, generator=g).mul(3.0).to(DT[dt])
    k = torch.randn(B, Hk, S, D, generator=g).mul(3.0).to(DT[dt])
    v = torch.randn(B, Hk, S, D, generator=g).to(DT[dt])
    do = torch.randn(B, H, S, D, generator=g).to(DT[dt])
    dq, dk, dv = _run(mha, q, k, v, do, None, True)
    grp = H // Hk
    ke, ve = (t.repeat_interleave(grp, dim=1) for t in (k, v))
    rq, rk, rv = oracle.attention_backward(q, ke, ve, do, causal=True, threads=THREADS)
    rk = rk.reshape(B, Hk, grp, S, D).sum(axis=2)
    rv = rv.reshape(B, Hk, grp, S, D).sum(axis=2)
    for name, u, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        ok = oracle.gate(u, r)
        assert ok.all(), (f"peaked {heads} {dt} {name}: {int((~ok).sum())} fail, "
                          f"budget {oracle.budget_fraction(u, r):.3f}")
    print(f"peaked {heads} {dt}: budget dq {oracle.budget_fraction(dq, rq):.3f} "
          f"dk {oracle.budget_fraction(dk, rk):.3f} dv {oracle.budget_fraction(dv, rv):.3f}",
          flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_large_ds_fp16(mha, causal):
    """q and k scaled by 3 at d_h 64 with unit values: dP reaches tens and dS
    several units, where a single fp16 rounding of dS misses the accuracy
    rule on dq (the CPU test of the backward roundings shows it); dS as an
    fp16 head and remainder meets it."""
    B, H, S, D = 3, 3, 326, 64
    g = torch.Generator().manual_seed(538493)
    q = torch.randn(B, H, S, D, generator=g).mul(3.0).half()
    k = torch.randn(B, H, S, D, generator=g).mul(3.0).half()
    v = torch.randn(B, H, S, D, generator=g).half()
    do = torch.randn(B, H, S, D, generator=g).half()
    got = _run(mha, q, k, v, do, None, causal)
    _check(got, q, k, v, do, None, causal, f"large dS fp16 causal={causal}")


def test_backward_peaked_dv_fp16(mha):
    """9 query heads over 3 key / value heads, S=108, d_h=64, causal, q and k
    scaled by 3: each key's dV sums a few probabilities near 1, where a single
    fp16 rounding of P misses the accuracy rule (the CPU test of the
    backward roundings shows it); P as an fp16 head and remainder meets it."""
    B, H, Hk, S, D = 3, 9, 3, 108, 64
    g = torch.Generator().manual_seed(221735)
    q = torch.randn(B, H, S, D, generator=g).mul(3.0).half()
    k = torch.randn(B, Hk, S, D, generator=g).mul(3.0).half()
    v = torch.randn(B, Hk, S, D, generator=g).half()
    do = torch.randn(B, H, S, D, generator=g).half()
    dq, dk, dv = _run(mha, q, k, v, do, None, True)
    grp = H // Hk
    ke, ve = (t.repeat_interleave(grp, dim=1) for t in (k, v))
    rq, rk, rv = oracle.attention_backward(q, ke, ve, do, causal=True, threads=THREADS)
    rk = rk.reshape(B, Hk, grp, S, D).sum(axis=2)
    rv = rv.reshape(B, Hk, grp, S, D).sum(axis=2)
    for name, u, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        ok = oracle.gate(u, r)
        assert ok.all(), (f"peaked dv {name}: {int((~ok).sum())} fail, "
                          f"budget {oracle.budget_fraction(u, r):.3f}")
    print(f"peaked dv fp16: budget dq {oracle.budget_fraction(dq, rq):.3f} "
          f"dk {oracle.budget_fraction(dk, rk):.3f} dv {oracle.budget_fraction(dv, rv):.3f}",
          flush=True)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("heads", [(4, 4), (8, 2)], ids=lambda h: f"H{h[0]}_Hkv{h[1]}")
def test_backward_graph_replays_match_eager(mha, heads, dt):
    """The backward (row pass, then one launch for both kinds of block; no
    memsets) captured in a HIP graph gives, on every replay, exactly the
    eager result. The output gradient changes in place between replays, and
    eager work and synchronisations run between them, so a replay cannot
    pass on stale outputs."""
    H, Hk = heads
    B, S, D = 2, 320, 64
    g = torch.Generator().manual_seed(H + Hk)
    q = torch.randn(B, H, S, D, generator=g).to(DT[dt]).cuda()
    k = torch.randn(B, Hk, S, D, generator=g).to(DT[dt]).cuda()
    v = torch.randn(B, Hk, S, D, generator=g).to(DT[dt]).cuda()
    do = torch.randn(B, H, S, D, generator=g).to(DT[dt]).cuda()
    out, lse = mha.forward(q, k, v, causal=True)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(lse.shape, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            mha.backward(q, k, v, out, lse, do, causal=True, dq=dq, dk=dk, dv=dv, delta=delta,
                         stream=cap)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(5)
    for rep in range(4):
        if rep:
            do.copy_(torch.randn(do.shape, generator=gen, device="cuda").to(do.dtype))
        ref = mha.backward(q, k, v, out, lse, do, causal=True)
        torch.cuda.synchronize()
        for t in (dq, dk, dv, delta):
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            assert torch.equal(a, b), f"replay {rep} {name}"
    grp = H // Hk
    qc, kc, vc, dc = (t.cpu() for t in (q, k, v, do))
    ke, ve = (t.repeat_interleave(grp, dim=1) for t in (kc, vc))
    rq, rk, rv = oracle.attention_backward(qc, ke, ve, dc, causal=True, threads=THREADS)
    rk = rk.reshape(B, Hk, grp, S, D).sum(axis=2)
    rv = rv.reshape(B, Hk, grp, S, D).sum(axis=2)
    for name, u, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        assert oracle.gate(u.cpu(), r).all(), f"graph {heads} {dt} {name}"
