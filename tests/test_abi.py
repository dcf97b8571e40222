"""Host-side checks of the C ABI: the library loads on a machine without a GPU,
exports every function include/mha.h declares, and rejects invalid arguments
on the host before anything is enqueued (no kernel runs in these tests)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mha.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(mha_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for want in ("mha_forward", "mha_forward_variant", "mha_backward", "mha_select_variant",
                 "mha_status_string", "mha_variant_name", "mha_version"):
        assert want in names


def test_library_exports_every_declared_symbol(mha):
    lib = ctypes.CDLL(mha.library_path())
    for name in _declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def test_status_and_variant_strings(mha):
    lib = mha.load()
    assert lib.mha_status_string(0) == b"ok"
    for code in range(1, 7):
        assert lib.mha_status_string(code) not in (b"ok", b"unknown status")
    assert lib.mha_status_string(99) == b"unknown status"
    for name, code in mha.VARIANTS.items():
        assert lib.mha_variant_name(code).decode() == name
    assert lib.mha_version() >= 101


def _fwd(lib, q=0x1000, k=0x2000, v=0x3000, out=0x4000, lse=None, B=1, H=1, S=16, D=64,
         causal=0, key_len=None, dtype=1, variant=0):
    return lib.mha_forward_variant(q, k, v, out, lse, B, H, S, D, causal, key_len, dtype, None, variant)


def test_validation_codes(mha):
    lib = mha.load()
    assert _fwd(lib, q=None) == 1                 # MHA_ERR_NULL
    assert _fwd(lib, out=None) == 1
    assert _fwd(lib, B=-1) == 2                   # MHA_ERR_SHAPE
    assert _fwd(lib, S=-5) == 2
    assert _fwd(lib, D=0) == 2
    assert _fwd(lib, D=48) == 3                   # MHA_ERR_UNSUPPORTED head size
    assert _fwd(lib, D=8, dtype=0) == 3           # d_h = 8: fp16 / bf16 only
    assert _fwd(lib, D=4) == 3
    assert _fwd(lib, dtype=7) == 3
    assert _fwd(lib, variant=99) == 3
    assert _fwd(lib, variant=4, D=64) == 3        # VALU kernel is d_h = 16 only
    assert _fwd(lib, variant=1, dtype=1) == 3     # fp32 kernel needs fp32 inputs
    assert _fwd(lib, variant=2, dtype=0) == 3
    assert _fwd(lib, variant=5, S=129) == 3       # short kernel is S <= 128
    assert _fwd(lib, variant=5, D=128) == 3
    assert _fwd(lib, q=0x1008) == 4               # MHA_ERR_MISALIGNED
    assert _fwd(lib, lse=0x5002) == 4
    assert _fwd(lib, key_len=0x6001) == 4
    assert _fwd(lib, S=1 << 26, D=64) == 2        # S * d_h >= 2^31
    assert _fwd(lib, B=1 << 16, H=1 << 15) == 2   # B * H >= 2^31


def test_empty_problems_are_noops(mha):
    lib = mha.load()
    # zero-size calls return OK without touching the (bogus) pointers
    assert _fwd(lib, B=0) == 0
    assert _fwd(lib, H=0, q=None) == 0
    assert _fwd(lib, S=0) == 0


def test_variant_selection(mha):
    import torch
    sel = mha.select_variant
    assert sel(1, 2, 64, 32, False, torch.float32) == "f32"
    assert sel(1, 8, 128, 16, True, torch.float16) == "short"
    assert sel(1, 8, 512, 64, True, torch.float16) == "mfma_small"
    assert sel(10000, 8, 128, 16, True, torch.float16) == "short"
    assert sel(16, 4, 1024, 256, False, torch.float16) == "mfma"
    assert sel(32, 16, 100000, 64, True, torch.float16) == "mfma"
    # 16-row four-wave tiles: d_h 16 / 32, mid-size d_h 64, causal bf16 d_h 64
    assert sel(16, 16, 1024, 16, True, torch.float16) == "mfma_small"
    assert sel(16, 16, 2048, 32, False, torch.bfloat16) == "mfma_small"
    assert sel(4, 12, 1024, 64, True, torch.bfloat16) == "mfma_small"
    assert sel(16, 12, 1024, 64, True, torch.float16) == "mfma_small"
    assert sel(32, 16, 1024, 64, True, torch.bfloat16) == "mfma_small"
    assert sel(16, 16, 2048, 64, False, torch.bfloat16) == "mfma"
    assert sel(8, 16, 2048, 128, True, torch.float16) == "mfma"
    with pytest.raises(mha.MhaError):
        sel(1, 1, 16, 48, False, torch.float16)


def test_python_binding_rejects_cpu_tensors(mha):
    import torch
    x = torch.zeros(1, 1, 16, 16, dtype=torch.float16)
    with pytest.raises(ValueError):
        mha.forward(x, x, x)


def _bwd(lib, q=0x1000, k=0x2000, v=0x3000, out=0x4000, dout=0x5000, lse=0x6000, dq=0x7000,
         dk=0x8000, dv=0x9000, delta=0xa000, B=1, H=1, S=16, D=64, causal=0, key_len=None,
         dtype=1):
    return lib.mha_backward(q, k, v, out, dout, lse, dq, dk, dv, delta, B, H, S, D, causal,
                            key_len, dtype, None)


def test_backward_validation_codes(mha):
    lib = mha.load()
    assert _bwd(lib, dout=None) == 1
    assert _bwd(lib, lse=None) == 1
    assert _bwd(lib, delta=None) == 1
    assert _bwd(lib, dk=None) == 1
    assert _bwd(lib, S=-1) == 2
    assert _bwd(lib, S=1 << 26) == 2
    assert _bwd(lib, D=48) == 3
    assert _bwd(lib, dtype=0) == 3          # fp32 backward not provided
    assert _bwd(lib, dtype=5) == 3
    assert _bwd(lib, dv=0x9008) == 4
    assert _bwd(lib, out=0x4004) == 4
    assert _bwd(lib, delta=0xa002) == 4
    assert _bwd(lib, B=0) == 0              # empty: no-op
    assert _bwd(lib, S=0, dout=None) == 0


def _bwd_noalloc(lib, q=0x1000, k=0x2000, v=0x3000, out=0x4000, dout=0x5000, lse=0x6000, dq=0x7000,
                dk=0x8000, dv=0x9000, B=1, H=1, S=16, D=64, causal=0, key_len=None, dtype=1):
    return lib.mha_backward_noalloc(q, k, v, out, dout, lse, dq, dk, dv, B, H, S, D, causal,
                                    key_len, dtype, None)


def test_noalloc_backward_validation_codes(mha):
    """The no-allocation backward checks its arguments as mha_backward does,
    and rejects problems whose B * H * S rows exceed its static workspace
    before any HIP call (these run without a GPU)."""
    lib = mha.load()
    assert _bwd_noalloc(lib, dout=None) == 1
    assert _bwd_noalloc(lib, lse=None) == 1
    assert _bwd_noalloc(lib, dk=None) == 1
    assert _bwd_noalloc(lib, S=-1) == 2
    assert _bwd_noalloc(lib, D=48) == 3
    assert _bwd_noalloc(lib, D=8) == 3
    assert _bwd_noalloc(lib, dtype=0) == 3
    assert _bwd_noalloc(lib, dv=0x9008) == 4
    assert _bwd_noalloc(lib, B=0) == 0  # empty: no-op
    rows = mha.MAX_NOALLOC_ROWS
    assert _bwd_noalloc(lib, B=rows // 128 + 1, H=1, S=128) == 6
    assert _bwd_noalloc(lib, B=2048, H=64, S=128) == 6
    assert b"workspace" in lib.mha_status_string(6)
    header = open(HEADER).read()
    assert f"#define MHA_NOALLOC_MAX_ROWS {rows}" in header


def _strided(lib, strides=None, B=1, H=4, H_kv=2, S=16, D=64, dtype=1, q=0x1000):
    import ctypes
    if strides is None:
        strides = [H * S * D, S * D, D] * 4
    arr = (ctypes.c_int64 * 12)(*strides)
    return lib.mha_forward_strided(q, 0x2000, 0x3000, 0x4000, None, arr, B, H, H_kv, S, D, 0,
                                   None, dtype, None)


def test_strided_validation_codes(mha):
    lib = mha.load()
    assert _strided(lib, H_kv=3) == 2          # H_kv must divide H
    assert _strided(lib, H_kv=0) == 2
    assert _strided(lib, dtype=0) == 3         # fp16 / bf16 only
    assert _strided(lib, D=48) == 3
    assert _strided(lib, q=None) == 1
    s = [4 * 16 * 64, 16 * 64, 64] * 4
    bad = list(s); bad[2] = 32                 # row stride below d_h
    assert _strided(lib, bad) == 2
    bad = list(s); bad[5] = 68                 # k row stride not a multiple of 16 bytes
    assert _strided(lib, bad) == 4
    bad = list(s); bad[10] = -64               # negative head stride
    assert _strided(lib, bad) == 2
    bad = list(s); bad[8] = 1 << 27            # one head spans >= 2^31 bytes
    assert _strided(lib, bad) == 2
    assert _strided(lib, B=0) == 0


def test_grouped_backward_validation(mha):
    lib = mha.load()
    args = [0x1000 * i for i in range(1, 11)]
    assert lib.mha_backward_grouped(*args, 1, 4, 3, 16, 64, 0, None, 1, None) == 2  # 3 !| 4
    assert lib.mha_backward_grouped(*args, 1, 4, 0, 16, 64, 0, None, 1, None) == 2
    assert lib.mha_backward_grouped(*args, 1, 4, 2, 16, 64, 0, None, 0, None) == 3  # fp32
    assert lib.mha_backward_grouped(*args, 0, 4, 2, 16, 64, 0, None, 1, None) == 0  # empty


def _fwd_train(lib, q=0x1000, k=0x2000, v=0x3000, out=0x4000, lse=0x5000, out32=0x6000, B=1,
               H=2, H_kv=1, S=16, D=64, causal=0, key_len=None, dtype=1):
    return lib.mha_forward_train(q, k, v, out, lse, out32, B, H, H_kv, S, D, causal, key_len,
                                 dtype, None)


def test_forward_train_validation_codes(mha):
    """The training forward checks its arguments like mha_forward, and also
    needs lse and the fp32 output buffer (16-byte aligned); no kernel runs."""
    lib = mha.load()
    assert lib.mha_version() >= 107
    assert _fwd_train(lib, lse=None) == 1
    assert _fwd_train(lib, out32=None) == 1
    assert _fwd_train(lib, q=None) == 1
    assert _fwd_train(lib, out32=0x6004) == 4
    assert _fwd_train(lib, dtype=0) == 3          # fp32 inputs: no training path
    assert _fwd_train(lib, D=48) == 3
    assert _fwd_train(lib, S=-1) == 2
    assert _fwd_train(lib, S=1 << 23, D=64) == 2  # one head of out32 spans 2^31 bytes
    assert _fwd_train(lib, H_kv=3) == 2           # H_kv must divide H
    assert _fwd_train(lib, H_kv=0) == 2
    assert _fwd_train(lib, B=0, lse=None) == 0    # empty: no-op


def _bwd_train(lib, q=0x1000, k=0x2000, v=0x3000, out32=0x4000, dout=0x5000, lse=0x6000,
               dq=0x7000, dk=0x8000, dv=0x9000, delta=0xa000, B=1, H=2, H_kv=1, S=16, D=64,
               causal=0, key_len=None, dtype=1):
    return lib.mha_backward_train(q, k, v, out32, dout, lse, dq, dk, dv, delta, B, H, H_kv, S, D,
                                  causal, key_len, dtype, None)


def test_backward_train_validation_codes(mha):
    lib = mha.load()
    assert _bwd_train(lib, out32=None) == 1
    assert _bwd_train(lib, dout=None) == 1
    assert _bwd_train(lib, delta=None) == 1
    assert _bwd_train(lib, out32=0x4008) == 4
    assert _bwd_train(lib, H_kv=3) == 2
    assert _bwd_train(lib, D=8) == 3
    assert _bwd_train(lib, dtype=0) == 3
    assert _bwd_train(lib, B=0, out32=None) == 0  # empty: no-op


def _qkv(lib, x=0x1000, w=0x2000, b=None, out=0x4000, lse=None, B=2, S=128, D=128, H=8,
         causal=1, key_len=None, dtype=1):
    return lib.mha_qkv_attention(x, w, b, out, lse, B, S, D, H, causal, key_len, dtype, None)


def test_qkv_attention_validation(mha):
    lib = mha.load()
    assert lib.mha_version() >= 105
    assert _qkv(lib, x=None) == 1 and _qkv(lib, w=None) == 1 and _qkv(lib, out=None) == 1
    assert _qkv(lib, B=-1) == 2 and _qkv(lib, S=-1) == 2 and _qkv(lib, H=0) == 2
    assert _qkv(lib, D=100, H=8) == 2             # H does not divide d_model
    assert _qkv(lib, D=256, H=8) == 3             # d_h = 32: not this kernel
    assert _qkv(lib, D=256, H=16) == 3            # 16 heads
    assert _qkv(lib, D=96, H=6) == 3
    assert _qkv(lib, D=128, H=32) == 3            # d_h = 4
    assert _qkv(lib, D=96, H=12) == 3             # d_model 96
    assert _qkv(lib, D=128, H=16, B=0) == 0       # d_h = 8 accepted (empty: nothing launched)
    assert _qkv(lib, S=129) == 3                  # longer sequences: unfused path
    assert _qkv(lib, dtype=0) == 3 and _qkv(lib, dtype=9) == 3
    assert _qkv(lib, x=0x1008) == 4 and _qkv(lib, out=0x4004) == 4
    assert _qkv(lib, w=0x2001) == 4 and _qkv(lib, b=0x3001) == 4
    assert _qkv(lib, lse=0x5002) == 4 and _qkv(lib, key_len=0x6001) == 4
    assert _qkv(lib, B=0) == 0 and _qkv(lib, S=0) == 0  # empty: nothing launched
    assert _qkv(lib, B=0, x=None) == 0


def test_head_size_8(mha):
    lib = mha.load()
    assert lib.mha_select_variant(4, 16, 128, 8, 1, 1) == mha.VARIANTS["short"]
    assert lib.mha_select_variant(64, 16, 1000, 8, 1, 2) == mha.VARIANTS["mfma"]
    assert lib.mha_select_variant(2, 4, 1000, 8, 1, 2) == mha.VARIANTS["mfma_small"]
    assert lib.mha_select_variant(2, 4, 1000, 8, 1, 0) == -3  # fp32
    assert _fwd(lib, D=8, variant=mha.VARIANTS["valu_d16"]) == 3
    assert _fwd(lib, D=8, variant=6) == 3  # past the last variant
    args = [0x1000 * i for i in range(1, 11)]
    assert lib.mha_backward(*args, 1, 2, 16, 8, 0, None, 1, None) == 3  # no backward at d_h = 8
