"""mha_backward_noalloc (the backward without a workspace argument, for
callers that cannot allocate) against mha_backward on the same inputs,
through the C ABI: bit-identical gradients on two calls in a row, the second
with a smaller problem (the static workspace keeps the first call's rows,
which the second must not read), and the gradients within the accuracy rule
of the float64 backward oracle (rustingstudio "brain/docs/baseline", "Fused
attention": the gradients of the fused backward)."""

import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _case(mha, B, H, S, D, dt, causal, key_len, seed):
    g = torch.Generator().manual_seed(seed)
    q, k, v, do = (torch.randn(B, H, S, D, generator=g).to(_DT[dt]) for _ in range(4))
    kl = None if key_len is None else torch.tensor(key_len, dtype=torch.int32)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    kld = None if kl is None else kl.cuda()
    out, lse = mha.forward(qd, kd, vd, causal=causal, key_len=kld)
    lib = mha.load()
    code = 1 if dt == "f16" else 2
    stream = torch.cuda.current_stream().cuda_stream
    ref = [torch.empty_like(qd) for _ in range(3)]
    delta = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    st = lib.mha_backward(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), dod.data_ptr(),
                          lse.data_ptr(), ref[0].data_ptr(), ref[1].data_ptr(), ref[2].data_ptr(),
                          delta.data_ptr(), B, H, S, D, int(causal),
                          None if kld is None else kld.data_ptr(), code, stream)
    assert st == 0
    got = [torch.full_like(qd, float("nan")) for _ in range(3)]
    st = lib.mha_backward_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(),
                                  dod.data_ptr(), lse.data_ptr(), got[0].data_ptr(), got[1].data_ptr(),
                                  got[2].data_ptr(), B, H, S, D, int(causal),
                                  None if kld is None else kld.data_ptr(), code, stream)
    assert st == 0, lib.mha_status_string(st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), f"{name}: the no-allocation entry point differs from mha_backward"
    refs = oracle.attention_backward(q, k, v, do, causal=causal, key_len=kl)
    for name, a, r in zip(("dq", "dk", "dv"), got, refs):
        ok = oracle.gate(a.cpu(), r)
        assert ok.all(), f"{name}: budget {oracle.budget_fraction(a.cpu(), r):.3f}"
    print(f"noalloc B{B} H{H} S{S} D{D} {dt} causal={causal}: equal to mha_backward, "
          + " ".join(f"{n} {oracle.budget_fraction(a.cpu(), r):.3f}"
                     for n, a, r in zip(("dq", "dk", "dv"), got, refs)), flush=True)


def test_noalloc_backward_two_calls_second_smaller(mha):
    _case(mha, B=2, H=4, S=700, D=64, dt="bf16", causal=True, key_len=[700, 513], seed=1)
    _case(mha, B=1, H=2, S=300, D=128, dt="f16", causal=False, key_len=[257], seed=2)


def test_noalloc_backward_rejects_too_many_rows(mha):
    lib = mha.load()
    B, H, S = mha.MAX_NOALLOC_ROWS // 1024 + 1, 1, 1024
    q = torch.empty(16, dtype=torch.float16, device="cuda")  # never read: rejected first
    p = q.data_ptr()
    st = lib.mha_backward_noalloc(p, p, p, p, p, p, p, p, p, B, H, S, 64, 1, None, 1, None)
    assert st == 6 and b"workspace" in lib.mha_status_string(st)
