"""GPU parity of mha_qkv_attention (attention fed by its own QKV projection,
d_h = 16, S <= 128) against the float64 oracle of the projection followed by
attention, under the graded rule |u-r| <= 2e-3 or |u-r| <= 2e-2 |r|, on the
same rounded inputs."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import THREADS
from workloads import WORKLOADS, make_qkv_inputs

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _inputs(B, S, H, dt, seed, key_len="random", bias=True, hd=16):
    w = WORKLOADS["qkv_bandwidth"].with_(B=B, S=S, H=H, D=hd, dtype=DT[dt],
                                         key_len=("uniform", 0, S) if key_len == "random"
                                         else key_len)
    x, wq, bq, kl = make_qkv_inputs(w, seed)
    return x, wq, (bq if bias else None), kl


def _run(mha, x, wq, bq, kl, H, causal):
    dev = [None if t is None else t.cuda() for t in (x, wq, bq, kl)]
    out, lse = mha.qkv_attention(dev[0], dev[1], dev[2], n_heads=H, causal=causal, key_len=dev[3])
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _check(out, lse, x, wq, bq, kl, H, causal, label, batches=None):
    if batches is not None:  # a sample of batch elements, computed one by one
        x, out, lse = x[batches], out[batches], lse[batches]
        kl = None if kl is None else kl[batches]
    ro, rl = oracle.qkv_attention(x, wq, bq, H, causal=causal, key_len=kl, threads=THREADS)
    ok_o, ok_l = oracle.gate(out, ro), oracle.gate(lse, rl)
    fo, fl = oracle.budget_fraction(out, ro), oracle.budget_fraction(lse, rl)
    if not (ok_o.all() and ok_l.all()):
        raise AssertionError(f"{label}: {int((~ok_o).sum())} out / {int((~ok_l).sum())} lse "
                             f"elements fail (budget out {fo:.3f}, lse {fl:.3f}); first bad "
                             f"{np.argwhere(~ok_o)[:5].tolist()}")
    print(f"{label}: budget out {fo:.3f} lse {fl:.3f}", flush=True)
    return fo, fl


CASES = [  # B, S, H
    (3, 128, 8),
    (2, 100, 8),   # ragged last tile
    (5, 17, 4),
    (4, 1, 2),
    (1, 64, 8),
    (700, 128, 8),  # more elements than workgroups: several per workgroup
    (1100, 77, 4),
]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_qkv_attention_shapes(mha, case, causal, dt):
    B, S, H = case
    x, wq, bq, kl = _inputs(B, S, H, dt, seed=B + S + H)
    out, lse = _run(mha, x, wq, bq, kl, H, causal)
    _check(out, lse, x, wq, bq, kl, H, causal, f"qkv {case} causal={causal} {dt}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_qkv_attention_no_bias_no_key_len(mha, dt):
    x, wq, _, _ = _inputs(6, 128, 8, dt, seed=1, key_len=None, bias=False)
    out, lse = _run(mha, x, wq, None, None, 8, True)
    _check(out, lse, x, wq, None, None, 8, True, f"no bias, all keys {dt}")


@pytest.mark.parametrize("name", ["qkv_launch", "qkv_bandwidth"])
def test_qkv_attention_workloads(mha, name):
    """The benchmark workloads at full size; the bandwidth one on a sample of
    300 batch elements (every element of those) plus every key length."""
    w = WORKLOADS[name]
    x, wq, bq, kl = make_qkv_inputs(w, seed=0)
    out, lse = _run(mha, x, wq, bq, kl, w.H, w.causal)
    batches = None
    if w.B > 300:
        rng = np.random.default_rng(0)
        batches = np.unique(np.concatenate([[0, w.B - 1], rng.choice(w.B, 298, replace=False)]))
    _check(out, lse, x, wq, bq, kl, w.H, w.causal, name, batches=batches)


def test_qkv_attention_edges(mha):
    # no visible key in some elements: out 0, lse -inf
    x, wq, bq, _ = _inputs(4, 40, 4, "f16", seed=3)
    kl = torch.tensor([0, 40, 0, 7], dtype=torch.int32)
    out, lse = _run(mha, x, wq, bq, kl, 4, True)
    assert not out[0].any() and not out[2].any()
    assert torch.isneginf(lse[0]).all() and torch.isneginf(lse[2]).all()
    _check(out, lse, x, wq, bq, kl, 4, True, "key_len 0")
    # key lengths past S clamp to S, negative to 0
    kl = torch.tensor([-3, 500, 40, 1], dtype=torch.int32)
    out, lse = _run(mha, x, wq, bq, kl, 4, False)
    _check(out, lse, x, wq, bq, kl.clamp(0, 40), 4, False, "clamped key_len")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_qkv_attention_hidden_rows_stay_local(mha, dt):
    """NaN in activation rows at or past the key length reaches only those
    rows' own outputs: the other rows are bitwise unchanged."""
    x, wq, bq, _ = _inputs(3, 128, 8, dt, seed=4)
    kl = torch.tensor([50, 128, 1], dtype=torch.int32)
    base_o, base_l = _run(mha, x, wq, bq, kl, 8, False)
    xp = x.clone()
    xp[0, 50:] = float("nan")
    xp[2, 1:] = float("nan")
    po, pl = _run(mha, xp, wq, bq, kl, 8, False)
    assert torch.equal(po[0, :50], base_o[0, :50]) and torch.equal(pl[0, :, :50], base_l[0, :, :50])
    assert torch.equal(po[1], base_o[1]) and torch.equal(po[2, :1], base_o[2, :1])
    assert torch.isnan(po[0, 50:]).all()
    _check(base_o, base_l, x, wq, bq, kl, 8, False, f"hidden rows {dt}")


def test_qkv_attention_deterministic_and_matches_unfused(mha):
    """Repeat calls give the same bits; the fused fp16 result agrees with the
    library's own unfused path (projection rounded to fp16, then forward on
    the head slices) to within 2e-3: the fused kernel keeps q and k as fp16
    pairs, so the two differ by the unfused path's rounding of q and k (about
    1e-3 at most here in a float64 model)."""
    x, wq, bq, kl = _inputs(64, 128, 8, "f16", seed=5)
    a = _run(mha, x, wq, bq, kl, 8, True)
    b = _run(mha, x, wq, bq, kl, 8, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    xd, wd, bd, kd = (t.cuda() for t in (x, wq, bq, kl))
    y = (xd.float() @ wd.float() + bd.float()).half()  # [B, S, 3D]
    q, k, v = (t.reshape(64, 128, 8, 16).transpose(1, 2) for t in y.split(128, dim=-1))
    out = torch.empty(64, 128, 8, 16, dtype=torch.float16, device="cuda").transpose(1, 2)
    mha.forward(q, k, v, causal=True, key_len=kd, out=out)
    torch.cuda.synchronize()
    ref = out.transpose(1, 2).reshape(64, 128, 128).cpu().float()
    assert (a[0].float() - ref).abs().max() <= 2e-3


CASES8 = [  # B, S, H with heads of 8 (d_model = 8 H)
    (3, 128, 16),   # sixteen heads of 8 in d_model 128 (the pages' heads-of-8 cases)
    (2, 100, 8),
    (5, 17, 4),
    (700, 128, 16),
]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES8, ids=lambda c: "x".join(map(str, c)))
def test_qkv_attention_heads_of_8(mha, case, causal, dt):
    """Two heads of 8 per 16-wide projection slice: each head's scores over
    its own columns, its own softmax, its own output columns and lse row."""
    B, S, H = case
    x, wq, bq, kl = _inputs(B, S, H, dt, seed=B + S + H + 1, hd=8)
    out, lse = _run(mha, x, wq, bq, kl, H, causal)
    _check(out, lse, x, wq, bq, kl, H, causal, f"qkv d8 {case} causal={causal} {dt}")


def test_qkv_attention_heads_of_8_hidden_rows(mha):
    x, wq, bq, _ = _inputs(2, 128, 16, "f16", seed=12, hd=8)
    kl = torch.tensor([70, 3], dtype=torch.int32)
    base_o, base_l = _run(mha, x, wq, bq, kl, 16, True)
    xp = x.clone()
    xp[0, 70:] = float("nan")
    xp[1, 3:] = float("inf")
    po, pl = _run(mha, xp, wq, bq, kl, 16, True)
    assert torch.equal(po[0, :70], base_o[0, :70]) and torch.equal(po[1, :3], base_o[1, :3])
    assert torch.equal(pl[0, :, :70], base_l[0, :, :70])
    _check(base_o, base_l, x, wq, bq, kl, 16, True, "d8 hidden rows")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("hd", [8, 16])
def test_qkv_attention_large_weights(mha, hd, dt):
    """Projection weights at three times the default initialisation scale:
    q and k rounded once to fp16 would miss the accuracy rule (the CPU test
    of the QKV roundings shows it); as head + remainder pairs they meet it."""
    H = 128 // hd
    x, wq, bq, kl = _inputs(8, 128, H, dt, seed=0, hd=hd)
    wq = wq * 3.0
    out, lse = _run(mha, x, wq, bq, kl, H, True)
    _check(out, lse, x, wq, bq, kl, H, True, f"qkv weights x3 d{hd} {dt}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("hd", [8, 16])
def test_qkv_graph_replays_match_eager(mha, hd, dt):
    """The fused kernel (persistent grid, double-buffered activation copies)
    captured in a HIP graph gives, on every replay, exactly the eager
    result; the activations change in place between replays, with eager
    work and synchronisations between them."""
    H = 128 // hd
    x, wq, bq, kl = (t.cuda() for t in _inputs(300, 128, H, dt, seed=21, hd=hd))
    out = torch.empty_like(x)
    lse = torch.empty(x.shape[0], H, x.shape[1], dtype=torch.float32, device="cuda")
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            mha.qkv_attention(x, wq, bq, n_heads=H, causal=True, key_len=kl, out=out, lse=lse,
                              stream=cap)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(9)
    for rep in range(4):
        if rep:
            x.copy_(torch.randn(x.shape, generator=gen, device="cuda").to(x.dtype))
        ref_o, ref_l = mha.qkv_attention(x, wq, bq, n_heads=H, causal=True, key_len=kl)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"
    _check(out.cpu(), lse.cpu(), x.cpu(), wq.cpu(), bq.cpu(), kl.cpu(), H, True,
           f"qkv graph d{hd} {dt}", batches=list(range(0, 300, 7)))
