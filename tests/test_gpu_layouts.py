"""GPU parity of mha_forward_strided: strided views ([B, S, H, d_h] tensors
seen as [B, H, S, d_h], slices of one fused QKV buffer, a strided output)
and grouped key / value heads, against the float64 oracle on contiguous
copies (key / value head h // (H / H_kv) repeated for every query head of
its group), under the same graded rule."""

import pytest
import torch

import oracle
from gpu_helpers import check_full

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _expand(t, H):
    """[B, H_kv, S, d] -> [B, H, S, d], repeating each head for its group."""
    return t.repeat_interleave(H // t.shape[1], dim=1).contiguous()


def _check(mha, q, k, v, kl, causal, label, out=None):
    o, lse = mha.forward(q, k, v, causal=causal, key_len=kl, out=out)
    torch.cuda.synchronize()
    H = q.shape[1]
    qc, kc, vc = q.cpu().contiguous(), _expand(k.cpu(), H), _expand(v.cpu(), H)
    kc_l = None if kl is None else kl.cpu()
    return check_full(o.cpu().contiguous(), lse.cpu(), qc, kc, vc, kc_l, causal, label)


CASES = [  # B, S, H, H_kv, D
    (2, 100, 4, 4, 64),
    (2, 300, 8, 2, 64),
    (1, 257, 6, 1, 128),
    (2, 130, 4, 2, 256),
    (3, 128, 8, 4, 16),    # d_h = 16, S <= 128: the short kernel
    (1, 1000, 12, 4, 64),  # grouped heads of the pages' training layer (12 query, 4 key/value)
    (2, 128, 16, 4, 8),    # d_h = 8, S <= 128: the short kernel
    (1, 300, 4, 2, 8),     # d_h = 8, tiled kernel
]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_bshd_views_and_grouped_heads(mha, case, causal, dt):
    """q, k, v and out all in [B, S, H, d_h] order, read through views."""
    B, S, H, Hk, D = case
    g = torch.Generator().manual_seed(B * 1000 + S)
    q = torch.randn(B, S, H, D, generator=g).to(DT[dt]).cuda().transpose(1, 2)
    k = torch.randn(B, S, Hk, D, generator=g).to(DT[dt]).cuda().transpose(1, 2)
    v = torch.randn(B, S, Hk, D, generator=g).to(DT[dt]).cuda().transpose(1, 2)
    kl = torch.randint(1, S + 1, (B,), generator=g, dtype=torch.int32).cuda()
    out = torch.empty(B, S, H, D, dtype=DT[dt], device="cuda").transpose(1, 2)
    _check(mha, q, k, v, kl, causal, f"bshd {case} causal={causal} {dt}", out=out)


@pytest.mark.parametrize("D", [16, 64, 128])
def test_fused_qkv_buffer(mha, D):
    """q, k, v as slices of one [B, S, 3, H, d_h] projection output."""
    B, S, H = 2, 120, 4
    g = torch.Generator().manual_seed(D)
    qkv = torch.randn(B, S, 3, H, D, generator=g).half().cuda()
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    _check(mha, q, k, v, None, True, f"fused qkv D={D}")


def test_strided_matches_contiguous_bitwise(mha):
    """The same data through views and through contiguous copies gives the
    same bits (the strided path only changes addressing)."""
    B, S, H, D = 2, 333, 4, 64
    g = torch.Generator().manual_seed(9)
    x = torch.randn(B, S, 3, H, D, generator=g).half().cuda()
    q, k, v = (x[:, :, i].transpose(1, 2) for i in range(3))
    a, la = mha.forward(q, k, v, causal=True)
    b, lb = mha.forward(q.contiguous(), k.contiguous(), v.contiguous(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_grouped_heads_equal_repeated_heads_bitwise(mha):
    B, S, H, Hk, D = 1, 500, 8, 2, 64
    g = torch.Generator().manual_seed(10)
    q = torch.randn(B, H, S, D, generator=g).half().cuda()
    k = torch.randn(B, Hk, S, D, generator=g).half().cuda()
    v = torch.randn(B, Hk, S, D, generator=g).half().cuda()
    a, la = mha.forward(q, k, v, causal=True)
    b, lb = mha.forward(q, _expand(k, H), _expand(v, H), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_strided_output_guard_bands(mha):
    """A strided output only writes its rows: the other heads' slots of a
    [B, S, H, d_h] buffer keep their contents."""
    B, S, H, D = 1, 70, 4, 64
    g = torch.Generator().manual_seed(11)
    q, k, v = (torch.randn(B, H, S, D, generator=g).half().cuda() for _ in range(3))
    buf = torch.full((B, S, H + 1, D), 7.0, dtype=torch.float16, device="cuda")
    out = buf[:, :, :H].transpose(1, 2)
    mha.forward(q, k, v, causal=False, out=out)
    torch.cuda.synchronize()
    assert (buf[:, :, H] == 7).all()
    ro, _ = oracle.attention(q.cpu(), k.cpu(), v.cpu())
    assert oracle.gate(out.cpu().contiguous(), ro).all()
