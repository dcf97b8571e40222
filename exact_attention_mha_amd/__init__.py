"""Exact multi-head attention forward for MI355X (gfx950).

A thin ctypes binding over the C ABI in include/mha.h (libmha_gfx950.so).
PyTorch supplies device memory and the stream; every step of the attention
itself runs in the library's HIP kernels. There is no fallback: if the
library is not built, or the tensors are not on a GPU, calls raise.

    out, lse = forward(q, k, v, causal=True, key_len=lengths)

q, k, v: contiguous [B, H, S, d_h] tensors on the GPU (float32, float16 or
bfloat16), d_h in {8, 16, 32, 64, 128, 256} (8: fp16 / bf16 only); key_len: None or an int32 GPU
tensor [B] of right-padded key lengths. backward() gives dq, dk, dv;
qkv_attention() takes the activations and the QKV projection weights
instead of q, k, v, for short sequences of 16-wide heads. For training,
forward_train() also returns the output in fp32, from which backward_train()
takes the softmax row term with one pass over dout instead of a pass over the
keys.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "forward", "forward_train", "backward", "backward_train", "backward_noalloc",
    "qkv_attention", "load", "library_path",
    "library_built", "MAX_NOALLOC_ROWS",
    "select_variant", "VARIANTS", "DTYPES", "MhaError",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmha_gfx950.so"

# enum mha_variant (include/mha.h)
VARIANTS = {"auto": 0, "f32": 1, "mfma": 2, "mfma_small": 3, "valu_d16": 4, "short": 5}
_VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}
# enum mha_dtype
DTYPES = {"float32": 0, "float16": 1, "bfloat16": 2}

_lib = None


class MhaError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def library_built() -> bool:
    return os.path.exists(library_path())


def load() -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; build it with `python -m exact_attention_mha_amd.build` "
            "(or __graft_entry__.build()). There is no CPU fallback.")
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    args = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, vp, ctypes.c_int, vp]
    lib.mha_forward.argtypes = args
    lib.mha_forward.restype = ctypes.c_int
    lib.mha_forward_variant.argtypes = args + [ctypes.c_int]
    lib.mha_forward_variant.restype = ctypes.c_int
    lib.mha_forward_strided.argtypes = [vp] * 6 + [i64] * 5 + [ctypes.c_int, vp, ctypes.c_int, vp]
    lib.mha_forward_strided.restype = ctypes.c_int
    lib.mha_backward.argtypes = [vp] * 10 + [i64, i64, i64, i64, ctypes.c_int, vp, ctypes.c_int, vp]
    lib.mha_backward.restype = ctypes.c_int
    lib.mha_backward_grouped.argtypes = [vp] * 10 + [i64] * 5 + [ctypes.c_int, vp, ctypes.c_int, vp]
    lib.mha_backward_grouped.restype = ctypes.c_int
    lib.mha_backward_noalloc.argtypes = [vp] * 9 + [i64] * 4 + [ctypes.c_int, vp, ctypes.c_int, vp]
    lib.mha_backward_noalloc.restype = ctypes.c_int
    lib.mha_forward_train.argtypes = [vp] * 6 + [i64] * 5 + [ctypes.c_int, vp, ctypes.c_int, vp]
    lib.mha_forward_train.restype = ctypes.c_int
    lib.mha_backward_train.argtypes = [vp] * 10 + [i64] * 5 + [ctypes.c_int, vp, ctypes.c_int, vp]
    lib.mha_backward_train.restype = ctypes.c_int
    lib.mha_qkv_attention.argtypes = [vp] * 5 + [i64] * 4 + [ctypes.c_int, vp, ctypes.c_int, vp]
    lib.mha_qkv_attention.restype = ctypes.c_int
    lib.mha_select_variant.argtypes = [i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.mha_select_variant.restype = ctypes.c_int
    lib.mha_variant_name.argtypes = [ctypes.c_int]
    lib.mha_variant_name.restype = ctypes.c_char_p
    lib.mha_status_string.argtypes = [ctypes.c_int]
    lib.mha_status_string.restype = ctypes.c_char_p
    lib.mha_version.argtypes = []
    lib.mha_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _dtype_code(t) -> int:
    name = str(t.dtype).replace("torch.", "")
    if name not in DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32, float16 or bfloat16")
    return DTYPES[name]


def select_variant(B: int, H: int, S: int, d_h: int, causal: bool, dtype) -> str:
    """Name of the kernel variant mha_forward picks for these arguments."""
    lib = load()
    code = DTYPES[str(dtype).replace("torch.", "")] if not isinstance(dtype, int) else dtype
    v = lib.mha_select_variant(B, H, S, d_h, int(bool(causal)), code)
    if v < 0:
        raise MhaError("mha_select_variant", -v, lib.mha_status_string(-v).decode())
    return _VARIANT_NAMES.get(v, "unknown")


def forward(q, k, v, causal: bool = False, key_len=None, out=None, lse=None,
            return_lse: bool = True, variant: str = "auto", stream=None
            ) -> Tuple["torch.Tensor", Optional["torch.Tensor"]]:
    """softmax(Q K^T / sqrt(d_h) + mask) V on the GPU, plus per-row log-sum-exp.

    Args:
      q, k, v: [B, H, S, d_h] GPU tensors of one dtype (k and v may have
        H_kv heads, H_kv dividing H: grouped-query attention). Contiguous
        tensors take mha_forward; strided views (last dimension contiguous,
        e.g. [B, S, H, d_h] tensors transposed, or slices of a fused QKV
        buffer) and grouped heads take mha_forward_strided (fp16 / bf16).
      causal: key j visible to query i only if j <= i.
      key_len: None (all S keys valid) or an int32 GPU tensor [B].
      out: optional preallocated output (shape/dtype of q; may be a strided
        view whose last dimension is contiguous).
      lse: optional preallocated float32 [B, H, S]; ignored if return_lse is
        False and lse is None (then no lse is written).
      variant: kernel variant name (see VARIANTS); "auto" picks by regime.
      stream: a torch.cuda.Stream (default: the current stream).
    Returns:
      (out, lse) -- lse is None when return_lse is False and none was given.
    """
    import torch

    lib = load()
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError(f"q, k, v must be [B,H,S,d_h] / [B,H_kv,S,d_h] tensors, got "
                         f"{tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    B, H, S, D = q.shape
    H_kv = k.shape[1]
    if (k.shape[0], k.shape[2], k.shape[3]) != (B, S, D) or H_kv < 1 or H % H_kv:
        raise ValueError(f"k, v must be [B, H_kv, S, d_h] with H_kv dividing H={H}, got "
                         f"{tuple(k.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    dcode = _dtype_code(q)
    if out is None:
        out = torch.empty((B, H, S, D), dtype=q.dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda:
        raise ValueError("out must be a GPU tensor shaped and typed like q")
    if lse is None and return_lse:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, S) or lse.dtype != torch.float32
                            or not lse.is_contiguous() or not lse.is_cuda):
        raise ValueError("lse must be a contiguous float32 GPU tensor [B, H, S]")
    kl_ptr = None
    if key_len is not None:
        if (key_len.dtype != torch.int32 or key_len.shape != (B,) or not key_len.is_cuda
                or not key_len.is_contiguous()):
            raise ValueError("key_len must be a contiguous int32 GPU tensor [B]")
        kl_ptr = key_len.data_ptr()
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}; one of {sorted(VARIANTS)}")
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    plain = H_kv == H and all(t.is_contiguous() for t in (q, k, v, out))
    if not plain:
        if variant != "auto":
            raise ValueError("strided views and grouped heads take the automatic variant")
        for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
            if t.stride(3) != 1:
                raise ValueError(f"{name}: the d_h elements of a row must be contiguous")
        strides = (ctypes.c_int64 * 12)(*[x for t in (q, k, v, out) for x in t.stride()[:3]])
        status = lib.mha_forward_strided(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
            lse.data_ptr() if lse is not None else None, strides,
            B, H, H_kv, S, D, int(bool(causal)), kl_ptr, dcode, st.cuda_stream)
        if status != 0:
            raise MhaError("mha_forward_strided", status, lib.mha_status_string(status).decode())
        return out, lse
    status = lib.mha_forward_variant(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None,
        B, H, S, D, int(bool(causal)), kl_ptr, dcode, st.cuda_stream, VARIANTS[variant])
    if status != 0:
        raise MhaError("mha_forward", status, lib.mha_status_string(status).decode())
    return out, lse


def forward_train(q, k, v, causal: bool = False, key_len=None, out=None, lse=None,
                  out32=None, stream=None):
    """forward() that also writes the output in fp32 (mha_forward_train).

    Args as forward() (contiguous q and k, v with H or H_kv heads, H_kv
    dividing H; float16 or bfloat16); out32: optional preallocated contiguous
    float32 [B, H, S, d_h].
    Returns:
      (out, lse, out32) -- pass lse and out32 to backward_train().
    """
    import torch

    lib = load()
    B, H, S, D = q.shape
    H_kv = k.shape[1] if k.dim() == 4 else -1
    if H_kv < 1 or H % H_kv or k.shape != (B, H_kv, S, D) or v.shape != k.shape:
        raise ValueError(f"k, v must be [B, H_kv, S, d_h] with H_kv dividing H={H}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor of the dtype of q")
    dcode = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if out32 is None:
        out32 = torch.empty((B, H, S, D), dtype=torch.float32, device=q.device)
    for name, t, shp, dt in (("out", out, q.shape, q.dtype), ("lse", lse, (B, H, S), torch.float32),
                             ("out32", out32, q.shape, torch.float32)):
        if t.shape != shp or t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} GPU tensor of shape {tuple(shp)}")
    kl_ptr = _key_len_ptr(key_len, B)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    status = lib.mha_forward_train(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), out32.data_ptr(),
        B, H, H_kv, S, D, int(bool(causal)), kl_ptr, dcode, st.cuda_stream)
    if status != 0:
        raise MhaError("mha_forward_train", status, lib.mha_status_string(status).decode())
    return out, lse, out32


def _key_len_ptr(key_len, B):
    import torch

    if key_len is None:
        return None
    if (key_len.dtype != torch.int32 or key_len.shape != (B,) or not key_len.is_cuda
            or not key_len.is_contiguous()):
        raise ValueError("key_len must be a contiguous int32 GPU tensor [B]")
    return key_len.data_ptr()


def backward(q, k, v, out, lse, dout, causal: bool = False, key_len=None,
             dq=None, dk=None, dv=None, delta=None, stream=None):
    """Gradients (dq, dk, dv) of sum(dout * out) through the attention forward.

    Args:
      q, k, v, causal, key_len: exactly as passed to forward(); all
        contiguous here, k and v with H or H_kv (dividing H) heads.
      out, lse: forward()'s outputs for those inputs (lse is required; out
        is checked for shape and dtype but not read).
      dout: the output gradient, contiguous [B, H, S, d_h], dtype of q.
      dq, dk, dv: optional preallocated outputs shaped like q, k, v.
      delta: optional float32 [B, H, S] workspace; receives the row term
        rowsum(P * dP), i.e. rowsum(dout * O) for the exact output O.
      stream: a torch.cuda.Stream (default: the current stream).
    Returns:
      (dq, dk, dv).
    """
    return _backward(q, k, v, out, None, lse, dout, causal, key_len, dq, dk, dv, delta, stream)


def backward_train(q, k, v, out32, lse, dout, causal: bool = False, key_len=None,
                   dq=None, dk=None, dv=None, delta=None, stream=None):
    """backward() with the row term D = rowsum(dout * out32) taken from
    forward_train()'s fp32 output (mha_backward_train): one pass over dout
    and out32 replaces the pass over the keys. Other arguments as backward().
    Returns (dq, dk, dv)."""
    return _backward(q, k, v, None, out32, lse, dout, causal, key_len, dq, dk, dv, delta, stream)


def _backward(q, k, v, out, out32, lse, dout, causal, key_len, dq, dk, dv, delta, stream):
    import torch

    lib = load()
    B, H, S, D = q.shape
    H_kv = k.shape[1] if k.dim() == 4 else -1
    if H_kv < 1 or H % H_kv or k.shape != (B, H_kv, S, D) or v.shape != k.shape:
        raise ValueError(f"k, v must be [B, H_kv, S, d_h] with H_kv dividing H={H}")
    checks = [("q", q, q.shape), ("k", k, k.shape), ("v", v, k.shape), ("dout", dout, q.shape)]
    if out32 is None:
        checks.append(("out", out, q.shape))
    elif (out32.shape != q.shape or out32.dtype != torch.float32 or not out32.is_cuda
          or not out32.is_contiguous()):
        raise ValueError("out32 must be forward_train()'s contiguous float32 GPU tensor")
    for name, t, shp in checks:
        if t.shape != shp or t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor of shape {tuple(shp)} "
                             f"and the dtype of q")
    if (lse is None or lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_cuda
            or not lse.is_contiguous()):
        raise ValueError("lse must be forward()'s contiguous float32 GPU tensor [B, H, S]")
    dcode = _dtype_code(q)
    grads = []
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is None:
            t = torch.empty_like(like)
        elif (t.shape != like.shape or t.dtype != q.dtype or not t.is_cuda
              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor shaped like its input")
        grads.append(t)
    if delta is None:
        delta = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    elif (delta.shape != (B, H, S) or delta.dtype != torch.float32 or not delta.is_cuda
          or not delta.is_contiguous()):
        raise ValueError("delta must be a contiguous float32 GPU tensor [B, H, S]")
    kl_ptr = _key_len_ptr(key_len, B)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    fn = "mha_backward_grouped" if out32 is None else "mha_backward_train"
    status = getattr(lib, fn)(
        q.data_ptr(), k.data_ptr(), v.data_ptr(),
        out.data_ptr() if out32 is None else out32.data_ptr(), dout.data_ptr(),
        lse.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(),
        delta.data_ptr(), B, H, H_kv, S, D, int(bool(causal)), kl_ptr, dcode, st.cuda_stream)
    if status != 0:
        raise MhaError(fn, status, lib.mha_status_string(status).decode())
    return tuple(grads)


def backward_noalloc(q, k, v, out, lse, dout, dq, dk, dv, causal: bool = False, key_len=None,
                     stream=None):
    """backward() through mha_backward_noalloc: the row term goes through
    the library's static per-GPU workspace, so with dq, dk, dv preallocated
    nothing is allocated. Calls that overlap on one GPU share that workspace
    and must not be issued; B * H * S must not exceed MAX_NOALLOC_ROWS.
    k and v have H heads here. Returns (dq, dk, dv)."""
    import torch

    lib = load()
    B, H, S, D = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout),
                    ("dq", dq), ("dk", dk), ("dv", dv)):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor shaped and typed like q")
    if (lse is None or lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_cuda
            or not lse.is_contiguous()):
        raise ValueError("lse must be forward()'s contiguous float32 GPU tensor [B, H, S]")
    kl_ptr = None
    if key_len is not None:
        if (key_len.dtype != torch.int32 or key_len.shape != (B,) or not key_len.is_cuda
                or not key_len.is_contiguous()):
            raise ValueError("key_len must be a contiguous int32 GPU tensor [B]")
        kl_ptr = key_len.data_ptr()
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    status = lib.mha_backward_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, S, D, int(bool(causal)), kl_ptr,
        _dtype_code(q), st.cuda_stream)
    if status != 0:
        raise MhaError("mha_backward_noalloc", status, lib.mha_status_string(status).decode())
    return dq, dk, dv


MAX_NOALLOC_ROWS = 8388608  # MHA_NOALLOC_MAX_ROWS of include/mha.h


def qkv_attention(x, w_qkv, b_qkv=None, n_heads: int = 8, causal: bool = False, key_len=None,
                  out=None, lse=None, return_lse: bool = True, stream=None):
    """Attention of the head slices of x @ w_qkv + b_qkv, projected on chip.

    Args:
      x: contiguous [B, S, d_model] GPU tensor (float16 or bfloat16), S <= 128,
        d_model in {32, 64, 128}.
      w_qkv: contiguous [d_model, 3 d_model] (columns q | k | v), dtype of x.
      b_qkv: None or contiguous [3 d_model], dtype of x.
      n_heads: H, with head size d_model / H of 16 or 8.
      causal, key_len: as in forward().
      out: optional preallocated contiguous [B, S, d_model] output.
      lse: optional preallocated float32 [B, H, S].
    Returns:
      (out, lse) -- out[b, :, hd h : hd (h + 1)] is head h's attention output.
    """
    import torch

    lib = load()
    if x.dim() != 3:
        raise ValueError(f"x must be [B, S, d_model], got {tuple(x.shape)}")
    B, S, D = x.shape
    H = int(n_heads)
    if w_qkv.shape != (D, 3 * D) or (b_qkv is not None and b_qkv.shape != (3 * D,)):
        raise ValueError(f"w_qkv must be [{D}, {3 * D}] and b_qkv [{3 * D}]")
    for name, t in (("x", x), ("w_qkv", w_qkv), ("b_qkv", b_qkv)):
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous() or t.dtype != x.dtype:
            raise ValueError(f"{name} must be a contiguous GPU tensor of the dtype of x")
    dcode = _dtype_code(x)
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous GPU tensor shaped and typed like x")
    if lse is None and return_lse:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=x.device)
    if lse is not None and (lse.shape != (B, H, S) or lse.dtype != torch.float32
                            or not lse.is_contiguous() or not lse.is_cuda):
        raise ValueError("lse must be a contiguous float32 GPU tensor [B, H, S]")
    kl_ptr = None
    if key_len is not None:
        if (key_len.dtype != torch.int32 or key_len.shape != (B,) or not key_len.is_cuda
                or not key_len.is_contiguous()):
            raise ValueError("key_len must be a contiguous int32 GPU tensor [B]")
        kl_ptr = key_len.data_ptr()
    st = stream if stream is not None else torch.cuda.current_stream(x.device)
    status = lib.mha_qkv_attention(
        x.data_ptr(), w_qkv.data_ptr(), b_qkv.data_ptr() if b_qkv is not None else None,
        out.data_ptr(), lse.data_ptr() if lse is not None else None,
        B, S, D, H, int(bool(causal)), kl_ptr, dcode, st.cuda_stream)
    if status != 0:
        raise MhaError("mha_qkv_attention", status, lib.mha_status_string(status).decode())
    return out, lse
