// C ABI of the attention library: host-side validation, kernel choice and
// launch on the caller's stream. Declarations and the contract are in
// include/mha.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mha.h"
#include "launch.h"

// Row-term workspace of mha_backward_noalloc: one float per query row, for
// at most MHA_NOALLOC_MAX_ROWS rows. A file-scope device array, so every GPU
// the library runs on holds its own copy for the life of the process. Host
// code never uses this name as an address: the per-device address comes from
// hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) float scratch[MHA_NOALLOC_MAX_ROWS];

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool supported_d(int64_t d) { return d == 8 || d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

// Matrix-core tile choice (measured on MI355X over B, H, S, d_h, mask and
// dtype): 16-row tiles in four-wave workgroups for
//  * d_h 16 and 32 at every size measured,
//  * d_h 64 below ~8 workgroups per CU of 128-row tiles, and for causal
//    bf16 at any size (the general bf16 d_h 64 tile is the one without the
//    pipelined loop),
//  * any d_h with fewer than ~2 workgroups per CU of 128-row tiles;
// the general tiled kernels otherwise.
int choose_mfma(int64_t B, int64_t H, int64_t S, int64_t D, int causal, int dtype) {
  const int64_t wg128 = B * H * ((S + 127) / 128);
  if (D == 16 || D == 32) return MHA_VARIANT_MFMA_SMALL;
  if (D == 64 && (wg128 < 2048 || (dtype == MHA_BF16 && causal))) return MHA_VARIANT_MFMA_SMALL;
  if (wg128 < 512) return MHA_VARIANT_MFMA_SMALL;
  return MHA_VARIANT_MFMA;
}

// Static kernel choice by regime (dtype, d_h, sequence length, head count):
//  * fp32 inputs                         -> fp32 matrix-core kernel
//  * S <= 128 and d_h <= 16              -> one pass per head, no LDS (any
//                                           head count: few heads are split
//                                           over four waves each)
//  * S <= 128 and d_h <= 64, many heads  -> one pass per head, no rescaling
//  * otherwise                           -> matrix-core tiles (choose_mfma)
int choose(int64_t B, int64_t H, int64_t S, int64_t D, int causal, int dtype) {
  if (dtype == MHA_F32) return MHA_VARIANT_F32;
  const int64_t heads = B * H;
  if (S <= 128 && D <= 16) return MHA_VARIANT_SHORT;
  if (S <= 128 && D <= 64 && heads >= 512) return MHA_VARIANT_SHORT;
  return choose_mfma(B, H, S, D, causal, dtype);
}

int validate(const void* q, const void* k, const void* v, void* out, const float* lse,
             int64_t B, int64_t H, int64_t S, int64_t d_h, const int32_t* key_len, int dtype) {
  if (B < 0 || H < 0 || S < 0 || d_h <= 0) return MHA_ERR_SHAPE;
  if (dtype != MHA_F32 && dtype != MHA_F16 && dtype != MHA_BF16) return MHA_ERR_UNSUPPORTED;
  if (!supported_d(d_h) || (d_h == 8 && dtype == MHA_F32)) return MHA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || S == 0) return MHA_OK;
  if (!q || !k || !v || !out) return MHA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return MHA_ERR_MISALIGNED;
  if ((lse && !aligned(lse, 4)) || (key_len && !aligned(key_len, 4))) return MHA_ERR_MISALIGNED;
  const int64_t esize = dtype == MHA_F32 ? 4 : 2;
  if (S * d_h * esize >= (int64_t)1 << 31) return MHA_ERR_SHAPE;  // per-head byte offsets are 32-bit
  if (B * H >= (int64_t)1 << 31) return MHA_ERR_SHAPE;
  return MHA_OK;
}

bool variant_runs(int variant, int64_t S, int64_t D, int dtype) {
  switch (variant) {
    case MHA_VARIANT_F32: return dtype == MHA_F32;
    case MHA_VARIANT_MFMA:
    case MHA_VARIANT_MFMA_SMALL: return dtype != MHA_F32;
    case MHA_VARIANT_VALU_D16: return dtype != MHA_F32 && D == 16;
    case MHA_VARIANT_SHORT: return dtype != MHA_F32 && S <= 128 && D <= 64;
  }
  return false;
}

}  // namespace

extern "C" {

int mha_forward_variant(const void* q, const void* k, const void* v, void* out, float* lse,
                        int64_t B, int64_t H, int64_t S, int64_t d_h, int causal,
                        const int32_t* key_len, int dtype, void* stream, int variant) {
  const int st = validate(q, k, v, out, lse, B, H, S, d_h, key_len, dtype);
  if (st != MHA_OK) return st;
  if (variant < 0 || variant >= MHA_VARIANT_COUNT) return MHA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || S == 0) return MHA_OK;
  if (variant == MHA_VARIANT_AUTO) variant = choose(B, H, S, d_h, causal, dtype);
  if (!variant_runs(variant, S, d_h, dtype)) return MHA_ERR_UNSUPPORTED;

  mha::AttnParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.key_len = key_len;
  p.B = (int)B;
  p.H = (int)H;
  p.S = (int)S;
  p.D = (int)d_h;
  p.causal = causal ? 1 : 0;
  p.dtype = dtype;
  p.c_log2 = (float)(1.4426950408889634074 / sqrt((double)d_h));
  p.lay = mha::contiguous_layout((int)H, (int)S, (int)d_h);

  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipErrorInvalidValue;
  switch (variant) {
    case MHA_VARIANT_F32: e = mha::launch_f32(p, s); break;
    case MHA_VARIANT_MFMA: e = mha::launch_mfma(p, s); break;
    case MHA_VARIANT_MFMA_SMALL: e = mha::launch_mfma_small(p, s); break;
    case MHA_VARIANT_VALU_D16: e = mha::launch_valu_d16(p, s); break;
    case MHA_VARIANT_SHORT: e = d_h <= 16 ? mha::launch_short16(p, s) : mha::launch_short(p, s); break;
  }
  if (e == hipErrorInvalidConfiguration) return MHA_ERR_SHAPE;
  return e == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

int mha_forward_strided(const void* q, const void* k, const void* v, void* out, float* lse,
                        const int64_t* strides, int64_t B, int64_t H, int64_t H_kv, int64_t S,
                        int64_t d_h, int causal, const int32_t* key_len, int dtype, void* stream) {
  const int st = validate(q, k, v, out, lse, B, H, S, d_h, key_len, dtype);
  if (st != MHA_OK) return st;
  if (dtype == MHA_F32) return MHA_ERR_UNSUPPORTED;
  if (H_kv <= 0 || H % H_kv != 0) return H_kv < 0 ? MHA_ERR_SHAPE : (H == 0 ? MHA_OK : MHA_ERR_SHAPE);
  if (B == 0 || H == 0 || S == 0) return MHA_OK;
  if (!strides) return MHA_ERR_NULL;
  const int64_t esize = 2;
  for (int t = 0; t < 4; ++t) {
    const int64_t sb = strides[3 * t], sh = strides[3 * t + 1], ss = strides[3 * t + 2];
    if (sb < 0 || sh < 0 || ss < d_h) return MHA_ERR_SHAPE;
    if ((sb * esize) % 16 || (sh * esize) % 16 || (ss * esize) % 16) return MHA_ERR_MISALIGNED;
    if (((S - 1) * ss + d_h) * esize >= ((int64_t)1 << 31)) return MHA_ERR_SHAPE;
  }
  int variant = choose(B, H, S, d_h, causal, dtype);
  if (variant == MHA_VARIANT_SHORT && d_h > 16)  // the d_h 32/64 short kernel is contiguous only
    variant = choose_mfma(B, H, S, d_h, causal, dtype);

  mha::AttnParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.key_len = key_len;
  p.B = (int)B;
  p.H = (int)H;
  p.S = (int)S;
  p.D = (int)d_h;
  p.causal = causal ? 1 : 0;
  p.dtype = dtype;
  p.c_log2 = (float)(1.4426950408889634074 / sqrt((double)d_h));
  p.lay = mha::Layout{strides[0], strides[1], strides[3], strides[4], strides[6], strides[7],
                      strides[9], strides[10], (int)strides[2], (int)strides[5], (int)strides[8],
                      (int)strides[11], (int)(H / H_kv)};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipErrorInvalidValue;
  switch (variant) {
    case MHA_VARIANT_MFMA: e = mha::launch_mfma(p, s); break;
    case MHA_VARIANT_MFMA_SMALL: e = mha::launch_mfma_small(p, s); break;
    case MHA_VARIANT_SHORT: e = mha::launch_short16(p, s); break;
  }
  if (e == hipErrorInvalidConfiguration) return MHA_ERR_SHAPE;
  return e == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

int mha_forward(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
                int64_t H, int64_t S, int64_t d_h, int causal, const int32_t* key_len, int dtype,
                void* stream) {
  return mha_forward_variant(q, k, v, out, lse, B, H, S, d_h, causal, key_len, dtype, stream,
                             MHA_VARIANT_AUTO);
}

int mha_forward_train(const void* q, const void* k, const void* v, void* out, float* lse,
                      float* out32, int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t d_h,
                      int causal, const int32_t* key_len, int dtype, void* stream) {
  const int st = validate(q, k, v, out, lse, B, H, S, d_h, key_len, dtype);
  if (st != MHA_OK) return st;
  if (dtype == MHA_F32) return MHA_ERR_UNSUPPORTED;
  if (H_kv <= 0 || (H > 0 && H % H_kv != 0)) return MHA_ERR_SHAPE;
  if (B == 0 || H == 0 || S == 0) return MHA_OK;
  if (!lse || !out32) return MHA_ERR_NULL;
  if (!aligned(out32, 16)) return MHA_ERR_MISALIGNED;
  if (S * d_h * 4 >= (int64_t)1 << 31) return MHA_ERR_SHAPE;  // per-head fp32 byte offsets

  mha::AttnParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.out32 = out32;
  p.key_len = key_len;
  p.B = (int)B;
  p.H = (int)H;
  p.S = (int)S;
  p.D = (int)d_h;
  p.causal = causal ? 1 : 0;
  p.dtype = dtype;
  p.c_log2 = (float)(1.4426950408889634074 / sqrt((double)d_h));
  p.lay = mha::contiguous_layout((int)H, (int)S, (int)d_h);
  p.lay.k_b = p.lay.v_b = H_kv * S * d_h;  // k, v: contiguous [B, H_kv, S, d_h]
  p.lay.group = (int)(H / H_kv);
  // the matrix-core kernels (the only ones that write out32), with fp16
  // probabilities as head + remainder in the value product; the tiles are
  // bf16's, and so is the choice between them
  const bool small = choose_mfma(B, H, S, d_h, causal, MHA_BF16) == MHA_VARIANT_MFMA_SMALL;
  const hipError_t e = small ? mha::launch_mfma_small_train(p, (hipStream_t)stream)
                             : mha::launch_mfma_train(p, (hipStream_t)stream);
  if (e == hipErrorInvalidConfiguration) return MHA_ERR_SHAPE;
  return e == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

}  // extern "C"

namespace {

// mha_backward_grouped and mha_backward_train: `out` (not read) or `out32`
// (the row term's source) identifies the forward output.
int backward_impl(const void* q, const void* k, const void* v, const void* out,
                  const float* out32, const void* dout, const float* lse, void* dq, void* dk,
                  void* dv, float* delta, int64_t B, int64_t H, int64_t H_kv, int64_t S,
                  int64_t d_h, int causal, const int32_t* key_len, int dtype, void* stream) {
  int st = validate(q, k, v, dq, lse, B, H, S, d_h, key_len, dtype);
  if (st != MHA_OK) return st;
  if (dtype == MHA_F32 || d_h == 8) return MHA_ERR_UNSUPPORTED;
  if (H_kv <= 0 || (H > 0 && H % H_kv != 0)) return MHA_ERR_SHAPE;
  if (B == 0 || H == 0 || S == 0) return MHA_OK;
  if (!(out || out32) || !dout || !lse || !dk || !dv || !delta) return MHA_ERR_NULL;
  if ((out && !aligned(out, 16)) || (out32 && !aligned(out32, 16)) || !aligned(dout, 16) ||
      !aligned(dk, 16) || !aligned(dv, 16) || !aligned(delta, 4))
    return MHA_ERR_MISALIGNED;

  mha::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = delta;
  p.key_len = key_len;
  p.B = (int)B;
  p.H = (int)H;
  p.S = (int)S;
  p.D = (int)d_h;
  p.causal = causal ? 1 : 0;
  p.dtype = dtype;
  p.c_log2 = (float)(1.4426950408889634074 / sqrt((double)d_h));
  p.group = (int)(H / H_kv);
  p.out32 = out32;
  const hipError_t e = mha::launch_bwd(p, (hipStream_t)stream);
  if (e == hipErrorInvalidConfiguration) return MHA_ERR_SHAPE;
  return e == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

}  // namespace

extern "C" {

int mha_backward_grouped(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         float* delta, int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t d_h,
                         int causal, const int32_t* key_len, int dtype, void* stream) {
  return backward_impl(q, k, v, out, nullptr, dout, lse, dq, dk, dv, delta, B, H, H_kv, S, d_h,
                       causal, key_len, dtype, stream);
}

int mha_backward_train(const void* q, const void* k, const void* v, const float* out32,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       float* delta, int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t d_h,
                       int causal, const int32_t* key_len, int dtype, void* stream) {
  return backward_impl(q, k, v, nullptr, out32, dout, lse, dq, dk, dv, delta, B, H, H_kv, S, d_h,
                       causal, key_len, dtype, stream);
}

int mha_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, float* delta, int64_t B,
                 int64_t H, int64_t S, int64_t d_h, int causal, const int32_t* key_len, int dtype,
                 void* stream) {
  return mha_backward_grouped(q, k, v, out, dout, lse, dq, dk, dv, delta, B, H, H > 0 ? H : 1, S,
                              d_h, causal, key_len, dtype, stream);
}

}  // extern "C"

namespace {

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
float* noalloc_scratch(int* status) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = MHA_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *status = MHA_ERR_HIP;
      return nullptr;
    }
    addr[dev] = (float*)p;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

int mha_backward_noalloc(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int64_t B, int64_t H, int64_t S, int64_t d_h, int causal,
                         const int32_t* key_len, int dtype, void* stream) {
  // the same checks as mha_backward, then the row limit, all before any HIP call
  int st = validate(q, k, v, dq, lse, B, H, S, d_h, key_len, dtype);
  if (st != MHA_OK) return st;
  if (dtype == MHA_F32 || d_h == 8) return MHA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || S == 0) return MHA_OK;
  if (!out || !dout || !lse || !dk || !dv) return MHA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(dout, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return MHA_ERR_MISALIGNED;
  if (B * H * S > (int64_t)MHA_NOALLOC_MAX_ROWS) return MHA_ERR_WORKSPACE;
  st = MHA_OK;
  float* delta = noalloc_scratch(&st);
  if (!delta) return st;
  // every row of the workspace is written by the row pass before it is read
  return mha_backward_grouped(q, k, v, out, dout, lse, dq, dk, dv, delta, B, H, H, S, d_h, causal,
                              key_len, dtype, stream);
}

int mha_qkv_attention(const void* x, const void* w_qkv, const void* b_qkv, void* out, float* lse,
                      int64_t B, int64_t S, int64_t d_model, int64_t H, int causal,
                      const int32_t* key_len, int dtype, void* stream) {
  if (B < 0 || S < 0 || d_model <= 0 || H <= 0 || d_model % H) return MHA_ERR_SHAPE;
  if (dtype != MHA_F16 && dtype != MHA_BF16) return MHA_ERR_UNSUPPORTED;
  const int64_t hd = d_model / H;
  if ((hd != 16 && hd != 8) || (d_model != 32 && d_model != 64 && d_model != 128) || S > 128)
    return MHA_ERR_UNSUPPORTED;
  if (B == 0 || S == 0) return MHA_OK;
  if (!x || !w_qkv || !out) return MHA_ERR_NULL;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(w_qkv, 2) || (b_qkv && !aligned(b_qkv, 2)))
    return MHA_ERR_MISALIGNED;
  if ((lse && !aligned(lse, 4)) || (key_len && !aligned(key_len, 4))) return MHA_ERR_MISALIGNED;
  if (B * H >= ((int64_t)1 << 31)) return MHA_ERR_SHAPE;

  mha::QkvParams p;
  p.x = x;
  p.w = w_qkv;
  p.bias = b_qkv;
  p.out = out;
  p.lse = lse;
  p.key_len = key_len;
  p.B = (int)B;
  p.S = (int)S;
  p.H = (int)H;
  p.hd = (int)hd;
  p.causal = causal ? 1 : 0;
  p.dtype = dtype;
  p.c_log2 = (float)(1.4426950408889634074 / sqrt((double)hd));
  const hipError_t e = mha::launch_qkv16(p, (hipStream_t)stream);
  if (e == hipErrorInvalidConfiguration) return MHA_ERR_SHAPE;
  return e == hipSuccess ? MHA_OK : MHA_ERR_HIP;
}

int mha_select_variant(int64_t B, int64_t H, int64_t S, int64_t d_h, int causal, int dtype) {
  if (B < 0 || H < 0 || S < 0 || d_h <= 0) return -MHA_ERR_SHAPE;
  if (dtype != MHA_F32 && dtype != MHA_F16 && dtype != MHA_BF16) return -MHA_ERR_UNSUPPORTED;
  if (!supported_d(d_h) || (d_h == 8 && dtype == MHA_F32)) return -MHA_ERR_UNSUPPORTED;
  return choose(B, H, S, d_h, causal ? 1 : 0, dtype);
}

const char* mha_variant_name(int variant) {
  switch (variant) {
    case MHA_VARIANT_AUTO: return "auto";
    case MHA_VARIANT_F32: return "f32";
    case MHA_VARIANT_MFMA: return "mfma";
    case MHA_VARIANT_MFMA_SMALL: return "mfma_small";
    case MHA_VARIANT_VALU_D16: return "valu_d16";
    case MHA_VARIANT_SHORT: return "short";
  }
  return "unknown";
}

const char* mha_status_string(int status) {
  switch (status) {
    case MHA_OK: return "ok";
    case MHA_ERR_NULL: return "null pointer argument";
    case MHA_ERR_SHAPE: return "invalid or too large shape";
    case MHA_ERR_UNSUPPORTED: return "unsupported head size, dtype or variant";
    case MHA_ERR_MISALIGNED: return "misaligned pointer";
    case MHA_ERR_HIP: return "HIP kernel launch failed";
    case MHA_ERR_WORKSPACE:
      return "B * H * S exceeds the static row workspace of the no-allocation entry point "
             "(MHA_NOALLOC_MAX_ROWS)";
  }
  return "unknown status";
}

int mha_version(void) { return 107; }

}  // extern "C"
