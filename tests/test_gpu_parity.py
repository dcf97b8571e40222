"""GPU parity: the HIP path (through the C ABI binding) against the float64
oracle, element by element, under the accuracy rule |u-r| <= 2e-3 or
|u-r| <= 2e-2 |r| (devpost "optimized-gpu-kernels-for-transformer-layers",
Inspiration). Worst-element error grows with the number of elements checked
(devpost "transformerkernel ... Tesla T4", Challenges), so every workload is
run over many seeds."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (check_full, check_full_chunked, check_rows, run_gpu, to_dev, workload_case,
                         THREADS)
from workloads import WORKLOADS, make_inputs, sample_rows

pytestmark = pytest.mark.gpu


def _report(label, fracs):
    fo = max(f[0] for f in fracs)
    fl = max(f[1] for f in fracs)
    print(f"{label}: worst out budget {fo:.3f}, worst lse budget {fl:.4f}", flush=True)


# ---------------------------------------------------------------- workloads

@pytest.mark.parametrize("chunk", range(4))
def test_tiny_200_seeds(mha, chunk):
    w = WORKLOADS["tiny"]
    _report(f"tiny chunk {chunk}", [workload_case(mha, w, s) for s in range(50 * chunk, 50 * chunk + 50)])


@pytest.mark.parametrize("chunk", range(4))
def test_launch_200_seeds(mha, chunk):
    w = WORKLOADS["launch"]
    _report(f"launch chunk {chunk}", [workload_case(mha, w, s) for s in range(50 * chunk, 50 * chunk + 50)])


@pytest.mark.parametrize("variant", ["mfma", "mfma_small", "short", "valu_d16"])
def test_launch_every_variant(mha, variant):
    w = WORKLOADS["launch"]
    _report(f"launch {variant}", [workload_case(mha, w, s, variant) for s in range(20)])


@pytest.mark.parametrize("variant", ["auto", "mfma", "mfma_small", "short", "valu_d16"])
def test_bandwidth_shape_reduced_batch(mha, variant):
    """The bandwidth workload's per-head shape (S=128, d_h=16, causal, key
    lengths uniform on [64, 128]) at B=64, every element checked."""
    w = WORKLOADS["bandwidth"].with_(B=64)
    _report(f"bandwidth B=64 {variant}", [workload_case(mha, w, s, variant) for s in range(10)])


@pytest.mark.parametrize("chunk", range(5))
def test_bandwidth_full_size_every_element(mha, chunk):
    """The full B=10000 launch the benchmark times, 25 seeds (5 per chunk),
    every element of out and lse against the oracle: the pages report this
    shape failing only in the tail, under a 25-trial stress (devpost
    "transformerkernel ... Tesla T4", Challenges we ran into)."""
    w = WORKLOADS["bandwidth"]
    fr = []
    for seed in range(5 * chunk, 5 * chunk + 5):
        q, k, v, kl = make_inputs(w, seed)
        out, lse = run_gpu(mha, q, k, v, kl, w.causal)
        # row 0 of every head sees key 0 only: out = v_0 exactly
        torch.testing.assert_close(out[:, :, 0].float(), v[:, :, 0].float(), rtol=0, atol=0)
        fr.append(check_full_chunked(out, lse, q, k, v, kl, w.causal, f"bandwidth seed {seed}"))
        print(f"bandwidth full size seed {seed}: out budget {fr[-1][0]:.3f} lse budget {fr[-1][1]:.4f}",
              flush=True)
    _report(f"bandwidth full size, every element, seeds {5 * chunk}..{5 * chunk + 4}", fr)


@pytest.mark.parametrize("chunk", range(5))
def test_compute_25_seeds(mha, chunk):
    w = WORKLOADS["compute"]
    _report(f"compute chunk {chunk}", [workload_case(mha, w, s) for s in range(5 * chunk, 5 * chunk + 5)])


# ---------------------------------------------------------------- edge cases

_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def _variants_for(dt, D, S):
    if dt == "f32":
        return ["auto", "f32"]
    v = ["auto", "mfma", "mfma_small"]
    if S <= 128 and D <= 64:
        v.append("short")
    if D == 16:
        v.append("valu_d16")
    if D == 8:
        v = ["auto", "mfma", "mfma_small"] + (["short"] if S <= 128 else [])
    return v


# d_h = 8 takes fp16 / bf16 only (test_abi checks the error fp32 gets)
_DT_D = [(dt, D) for dt in ("f16", "bf16", "f32") for D in (8, 16, 32, 64, 128, 256)
         if not (dt == "f32" and D == 8)]


@pytest.mark.parametrize("dt,D", _DT_D)
@pytest.mark.parametrize("S", [1, 17, 65, 128, 200])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_shapes(mha, dt, D, S, causal):
    """Ragged and tiny sequences, every head size and dtype, key lengths
    {S, 0, 1, S//2 + 1} (0 = a batch with no visible key), every variant that
    accepts the shape."""
    from workloads import Workload
    B = 4
    w = Workload("edge", B, 3, S, D, _DT[dt], causal, None)
    q, k, v, _ = make_inputs(w, seed=S * 7 + D)
    kl = torch.tensor([S, 0, 1, S // 2 + 1], dtype=torch.int32)
    for variant in _variants_for(dt, D, S):
        out, lse = run_gpu(mha, q, k, v, kl, causal, variant)
        check_full(out, lse, q, k, v, kl, causal, f"{dt} D={D} S={S} causal={causal} {variant}")
        assert (out[1] == 0).all() and (lse[1] == -math.inf).all()


@pytest.mark.parametrize("variant", ["auto", "mfma", "mfma_small", "short", "valu_d16"])
def test_padded_keys_never_read(mha, variant):
    """NaN / Inf in padded K and V rows must not reach any output."""
    w = WORKLOADS["bandwidth"].with_(B=32)
    q, k, v, kl = make_inputs(w, 3)
    for b in range(w.B):
        k[b, :, int(kl[b]):] = float("nan")
        v[b, :, int(kl[b]):] = float("inf")
    out, lse = run_gpu(mha, q, k, v, kl, True, variant)
    assert torch.isfinite(out).all()
    check_full(out, lse, q, k, v, kl, True, f"poisoned padding {variant}")


@pytest.mark.parametrize("scale", [1e-3, 10.0, 30.0])
@pytest.mark.parametrize("D,S,dt", [(64, 300, "f16"), (256, 130, "f16"), (16, 128, "f16"),
                                    (128, 396, "bf16"), (64, 300, "bf16")])
def test_adversarial_input_scales(mha, scale, D, S, dt):
    """Scores spread over hundreds of log2 units: the running max is
    exceeded by huge margins (bf16 probabilities would stay finite in fp32
    far past the point where O overflows, so the overflow check must bound
    them, not just test for infinity)."""
    from workloads import Workload
    w = Workload("adv", 2, 2, S, D, _DT[dt], True, None)
    q, k, v, _ = make_inputs(w, 11)
    q = (q.float() * scale).to(_DT[dt])
    k = (k.float() * scale).to(_DT[dt])
    out, lse = run_gpu(mha, q, k, v, None, True)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    check_full(out, lse, q, k, v, None, True, f"scale {scale} D={D}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal,L", [(False, None), (True, None), (False, 650), (True, 650)])
def test_running_max_jumps(mha, dt, D, causal, L):
    """Scores that climb by about 20 log2 units every 32 keys, so a running
    max taken from earlier keys is exceeded past the fp16 range at every key
    pair, in the middle of blocks and across them (the general kernel's
    overflow check and recompute path). With q = 1 along every axis and
    k_j = a_j / sqrt(d_h) along every axis, q.k_j / sqrt(d_h) = a_j =
    14 floor(j / 32) (+ noise)."""
    B, H, S = 2, 2, 700
    g = torch.Generator().manual_seed(3)
    a = 14.0 * (torch.arange(S, dtype=torch.float64) // 32) + 0.5 * torch.randn(S, generator=g, dtype=torch.float64)
    q = 1.0 + 0.05 * torch.randn(B, H, S, D, generator=g, dtype=torch.float64)
    k = (a / math.sqrt(D))[:, None] + 0.05 * torch.randn(B, H, S, D, generator=g, dtype=torch.float64)
    v = torch.randn(B, H, S, D, generator=g, dtype=torch.float64)
    q, k, v = (t.to(_DT[dt]) for t in (q, k, v))
    kl = None if L is None else torch.full((B,), L, dtype=torch.int32)
    out, lse = run_gpu(mha, q, k, v, kl, causal, variant="mfma")
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    check_full(out, lse, q, k, v, kl, causal, f"climbing scores D={D} causal={causal} L={L}")


def test_deterministic(mha):
    w = WORKLOADS["compute"].with_(B=2)
    q, k, v, kl = make_inputs(w, 5)
    a = run_gpu(mha, q, k, v, kl, w.causal)
    b = run_gpu(mha, q, k, v, kl, w.causal)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_outputs_stay_inside_their_buffers(mha):
    """Guard bands before and after out / lse are never written."""
    B, H, S, D = 2, 3, 77, 64
    g = torch.Generator().manual_seed(0)
    q, k, v = (torch.randn(B, H, S, D, generator=g).half().cuda() for _ in range(3))
    n, nl = B * H * S * D, B * H * S
    pad = 4096
    buf = torch.full((pad + n + pad,), 7.0, dtype=torch.float16, device="cuda")
    lbuf = torch.full((pad + nl + pad,), 7.0, dtype=torch.float32, device="cuda")
    out = buf[pad:pad + n].view(B, H, S, D)
    lse = lbuf[pad:pad + nl].view(B, H, S)
    mha.forward(q, k, v, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert (buf[:pad] == 7).all() and (buf[pad + n:] == 7).all()
    assert (lbuf[:pad] == 7).all() and (lbuf[pad + nl:] == 7).all()
    check_full(out.cpu(), lse.cpu(), q.cpu(), k.cpu(), v.cpu(), None, True, "guard bands")


def test_without_lse_and_on_a_side_stream(mha):
    B, H, S, D = 1, 2, 300, 64
    g = torch.Generator().manual_seed(1)
    q, k, v = (torch.randn(B, H, S, D, generator=g).half().cuda() for _ in range(3))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, lse = mha.forward(q, k, v, causal=False, return_lse=False, stream=s)
    s.synchronize()
    assert lse is None
    ro, _ = oracle.attention(q.cpu(), k.cpu(), v.cpu())
    assert oracle.gate(out.cpu(), ro).all()


@pytest.mark.parametrize("wl,variant", [("launch", "auto"), ("launch", "mfma_small"),
                                        ("compute", "auto")])
def test_graph_replays_match_eager(mha, wl, variant):
    """The forward captured in a HIP graph (as the launch-bound benchmark
    replays it) gives, on every replay, exactly the eager result; eager work
    and synchronisations run between the replays, and the inputs change in
    place between replays so that a replay cannot pass on stale outputs."""
    w = WORKLOADS[wl].with_(B=min(WORKLOADS[wl].B, 2))
    q, k, v, kl = to_dev(*make_inputs(w, 11))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            mha.forward(q, k, v, causal=w.causal, key_len=kl, out=out, lse=lse,
                        variant=variant, stream=cap)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(3)
    for rep in range(4):
        if rep:
            q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(q.dtype))
        ref_o, ref_l = mha.forward(q, k, v, causal=w.causal, key_len=kl, variant=variant)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"
    check_full(out.cpu(), lse.cpu(), q.cpu(), k.cpu(), v.cpu(),
               None if kl is None else kl.cpu(), w.causal, f"graph {wl} {variant}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(64, 16, 128, ("uniform", 1, 128)), (2, 4, 1000, ("uniform", 1, 1000)),
                                   (1, 2, 4096, None)], ids=["short-b64-h16", "tiled-s1000", "tiled-s4096"])
def test_head_size_8(mha, dt, shape):
    """d_h = 8 heads (the pages' cases with sixteen heads of 8 in a
    d_model of 128) through the short and the tiled kernels, causal, every
    element against the oracle."""
    from workloads import Workload
    B, H, S, kl_spec = shape
    w = Workload("d8", B, H, S, 8, _DT[dt], True, kl_spec)
    q, k, v, kl = make_inputs(w, seed=S + H)
    for variant in (["auto", "mfma_small"] if S > 128 else ["auto", "mfma"]):
        out, lse = run_gpu(mha, q, k, v, kl, True, variant)
        check_full(out, lse, q, k, v, kl, True, f"d8 {shape} {dt} {variant}")


@pytest.mark.parametrize("D", [64, 128])
def test_pipelined_loop_graph_replays_match_eager(mha, D):
    """The software-pipelined loop (the general variant's default for fp16 at
    d_h 64 and 128; forced here, since a grid this small would otherwise take
    the small-grid configuration) captured in a HIP graph: every replay
    equals the eager call bit for bit, with q changed in place between
    replays."""
    from workloads import Workload
    w = Workload("pipe", 2, 4, 1500, D, torch.float16, True, ("uniform", 700, 1500))
    q, k, v, kl = to_dev(*make_inputs(w, 17))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            mha.forward(q, k, v, causal=True, key_len=kl, out=out, lse=lse, variant="mfma",
                        stream=cap)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(4)
    for rep in range(4):
        if rep:
            q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(q.dtype))
        ref_o, ref_l = mha.forward(q, k, v, causal=True, key_len=kl, variant="mfma")
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"
    check_full(out.cpu(), lse.cpu(), q.cpu(), k.cpu(), v.cpu(), kl.cpu(), True,
               f"pipelined graph D={D}")
