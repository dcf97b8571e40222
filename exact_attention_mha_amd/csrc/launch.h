// Host-side launch interface between the C ABI (mha_api.cpp) and the kernel
// translation units. Each launcher validates nothing: the ABI layer has
// already checked pointers, sizes and alignment; a launcher returns
// hipErrorInvalidValue only when its kernel has no instantiation for the
// requested (dtype, d_h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mha {

// Where the rows of one (batch, head) start, per tensor: element offsets
// b * *_b + h * *_h (k / v use head h / group), and element strides *_s
// between consecutive rows; the d_h elements of a row are contiguous. The
// contiguous [B, H, S, d_h] layout is *_b = H*S*d_h, *_h = S*d_h,
// *_s = d_h, group = 1.
struct Layout {
  int64_t q_b, q_h, k_b, k_h, v_b, v_h, o_b, o_h;
  int q_s, k_s, v_s, o_s;
  int group;  // query heads per key/value head
};

inline Layout contiguous_layout(int H, int S, int D) {
  const int64_t hs = (int64_t)S * D, bs = (int64_t)H * hs;
  return Layout{bs, hs, bs, hs, bs, hs, bs, hs, D, D, D, D, 1};
}

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;              // nullable
  const int32_t* key_len;  // nullable
  int B, H, S, D;
  int causal;
  int dtype;               // enum mha_dtype
  float c_log2;            // log2(e) / sqrt(d_h)
  Layout lay;              // strides (contiguous unless from mha_forward_strided)
  float* out32 = nullptr;  // nullable: the output in fp32, contiguous [B, H, S, D]
                           // (matrix-core kernels only)
};

// Backward: dq, dk, dv of sum(dout * out); delta is the caller's float
// [B, H, S] workspace for the row term rowsum(P * dP) (= rowsum(dout * O) of
// the exact output; out itself is not read).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;
  const int32_t* key_len;  // nullable
  int B, H, S, D;
  int causal;
  int dtype;
  float c_log2;
  int group;               // query heads per key / value head (k, v, dk, dv have H / group)
  const float* out32 = nullptr;  // nullable: the forward's output in fp32 ([B, H, S, D]);
                                 // when given, D = rowsum(dout * out32) replaces the row pass
};

// Attention fed by its own QKV projection (d_h = hd in {8, 16}, S <= 128):
// x [B, S, hd H], w [hd H, 3 hd H] (columns q | k | v, head h at hd h within
// each), bias [3 hd H] or null, out [B, S, hd H], lse [B, H, S] or null; all
// contiguous.
struct QkvParams {
  const void* x;
  const void* w;
  const void* bias;        // nullable
  void* out;
  float* lse;              // nullable
  const int32_t* key_len;  // nullable
  int B, S, H, hd;
  int causal;
  int dtype;
  float c_log2;            // log2(e) / sqrt(hd)
};

hipError_t launch_bwd(const BwdParams& p, hipStream_t s);          // dq then dk/dv kernel

hipError_t launch_mfma(const AttnParams& p, hipStream_t s);        // general tiled, 16x16 products
hipError_t launch_mfma_small(const AttnParams& p, hipStream_t s);  // few rows per WG
// the same for the training forward (fp16 probabilities as head + remainder)
hipError_t launch_mfma_train(const AttnParams& p, hipStream_t s);
hipError_t launch_mfma_small_train(const AttnParams& p, hipStream_t s);
hipError_t launch_f32(const AttnParams& p, hipStream_t s);         // fp32 inputs
hipError_t launch_valu_d16(const AttnParams& p, hipStream_t s);    // d_h = 16 VALU
hipError_t launch_short(const AttnParams& p, hipStream_t s);       // S <= 128 one pass, d_h 32/64
hipError_t launch_short16(const AttnParams& p, hipStream_t s);     // S <= 128 one pass, d_h 16
hipError_t launch_qkv16(const QkvParams& p, hipStream_t s);        // projection + attention, d_h 16

}  // namespace mha
