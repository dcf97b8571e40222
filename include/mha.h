/*
 * mha.h -- C ABI of the gfx950 exact multi-head attention forward library.
 *
 * Computes, for every batch b and head h,
 *     out = softmax(Q K^T / sqrt(d_h) + mask) V
 * over [B, H, S, d_h] tensors, with an optional causal mask and right-padded
 * per-batch key lengths, plus the per-row log-sum-exp. The definition is the
 * textbook five-op attention (devpost "gpu-transformer-optimization",
 * section 2.1, ops (1)-(5)); the kernels evaluate it with the running-max /
 * running-sum recurrence of the same section, so the [B, H, S, S] score
 * tensor never reaches device memory.
 *
 * Mask: key j is visible to query row i iff j < L_b and, when causal,
 * j <= i, where L_b = key_len[b] clamped to [0, S] (or S when key_len is
 * NULL). Padded query rows (i >= L_b) still produce output: they attend to
 * keys 0..L_b-1. A row with no visible key (L_b == 0) gets out = 0 and
 * lse = -inf. Padded key/value rows (j >= L_b) are never read, so their
 * contents (even NaN) cannot affect any result.
 *
 * Precision: fp16 / bf16 inputs are multiplied on the matrix cores with fp32
 * accumulation; softmax arithmetic is fp32; out is rounded once to the input
 * dtype. fp32 inputs are computed in fp32 throughout.
 *
 * All functions are thread-safe and allocate no memory; the library keeps no
 * per-call state, except the static row workspace of mha_backward_noalloc
 * (see there for how calls sharing it must be ordered).
 */
#ifndef EXACT_ATTENTION_MHA_AMD_MHA_H
#define EXACT_ATTENTION_MHA_AMD_MHA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and out. */
enum mha_dtype {
  MHA_F32 = 0,
  MHA_F16 = 1,
  MHA_BF16 = 2
};

/* Return codes. Validation errors are detected on the host before anything
 * is enqueued; nothing is launched when a call returns an error. */
enum mha_status {
  MHA_OK = 0,
  MHA_ERR_NULL = 1,        /* a required pointer is NULL */
  MHA_ERR_SHAPE = 2,       /* negative size, or sizes beyond the per-head
                              byte / grid limits stated below */
  MHA_ERR_UNSUPPORTED = 3, /* d_h or dtype or variant not supported */
  MHA_ERR_MISALIGNED = 4,  /* q/k/v/out not 16-byte aligned, lse/key_len not
                              4-byte aligned */
  MHA_ERR_HIP = 5,         /* the kernel launch itself failed */
  MHA_ERR_WORKSPACE = 6    /* mha_backward_noalloc: B * H * S is larger than
                              its static workspace (MHA_NOALLOC_MAX_ROWS) */
};

/* Rows (B * H * S) that mha_backward_noalloc's static workspace holds:
 * one float each, 32 MiB per GPU. */
#define MHA_NOALLOC_MAX_ROWS 8388608

/* Kernel variants. MHA_VARIANT_AUTO picks by (dtype, d_h, causal, B*H, S);
 * the others force one kernel for A/B measurement and testing. Every variant
 * computes the same result to within the fp32 rounding of its own
 * accumulation order. */
enum mha_variant {
  MHA_VARIANT_AUTO = 0,
  MHA_VARIANT_F32 = 1,        /* fp32 inputs: fp32 matrix-core kernel        */
  MHA_VARIANT_MFMA = 2,       /* fp16/bf16 general tiled kernel, any d_h     */
  MHA_VARIANT_MFMA_SMALL = 3, /* fp16/bf16, 16-32 query rows per workgroup:
                                 more workgroups for launch-bound shapes     */
  MHA_VARIANT_VALU_D16 = 4,   /* fp16/bf16 d_h = 16 on the vector ALUs       */
  MHA_VARIANT_SHORT = 5,      /* fp16/bf16 d_h <= 64, S <= 128: one pass per
                                 head, no rescaling                          */
  MHA_VARIANT_COUNT = 6
};

/*
 * mha_forward -- enqueue one attention forward on `stream`.
 *
 *   q, k, v  device pointers, contiguous [B, H, S, d_h] of `dtype`,
 *            16-byte aligned. Read only.
 *   out      device pointer, contiguous [B, H, S, d_h] of `dtype`, 16-byte
 *            aligned. Written in full. Must not overlap q, k or v.
 *   lse      device pointer to contiguous fp32 [B, H, S] or NULL (not
 *            written). lse[b,h,i] = ln(sum over visible j of
 *            exp(q_i . k_j / sqrt(d_h))), -inf for rows with no visible key.
 *   B, H, S  batch, heads, sequence length (>= 0; any of them 0 is a no-op
 *            returning MHA_OK). One head must span fewer than 2^31 bytes
 *            (S * d_h * element size < 2^31) and the launch must fit a
 *            2^31-1 workgroup grid.
 *   d_h      head dimension: 16, 32, 64, 128 or 256; also 8 for fp16 / bf16
 *            (computed as a 16-wide head with zero columns 8..15).
 *   causal   non-zero: key j visible to row i only if j <= i.
 *   key_len  device pointer to int32[B] or NULL (all S keys valid). Values
 *            are clamped to [0, S] on the device (the host never reads them).
 *   dtype    enum mha_dtype.
 *   stream   hipStream_t to enqueue on; NULL = the null stream.
 *
 * Ownership: the caller allocates and owns every buffer and must keep them
 * alive until the stream has passed this call. The call is asynchronous:
 * device-side faults surface at the caller's next synchronisation.
 * Returns an enum mha_status code; no output is written on error.
 */
int mha_forward(const void* q, const void* k, const void* v, void* out, float* lse,
                int64_t B, int64_t H, int64_t S, int64_t d_h, int causal,
                const int32_t* key_len, int dtype, void* stream);

/* mha_forward with an explicit kernel variant (enum mha_variant). Returns
 * MHA_ERR_UNSUPPORTED when the variant cannot run this (dtype, d_h, S). */
int mha_forward_variant(const void* q, const void* k, const void* v, void* out, float* lse,
                        int64_t B, int64_t H, int64_t S, int64_t d_h, int causal,
                        const int32_t* key_len, int dtype, void* stream, int variant);

/*
 * mha_forward_train -- mha_forward that also keeps the output in fp32, for
 * the backward's row term (mha_backward_train).
 *
 * The fused backward of rustingstudio "brain/docs/baseline" ("Fused
 * attention") takes its softmax row term from dout and the forward output,
 * D = rowsum(dout * O). With O rounded to fp16 or bf16 that term is off by a
 * rounding of O, which dq and dk amplify where the softmax is peaked; the
 * output before that rounding (O / l in fp32, with the probabilities
 * entering the value product as a head and a remainder for both dtypes)
 * keeps it within the accuracy rule over the range of scores stated for
 * mha_backward, and lets the backward form D with one pass over dout and
 * out32 instead of a pass over the keys.
 *
 *   out32    device pointer, contiguous fp32 [B, H, S, d_h], 16-byte aligned;
 *            written in full (rows with no visible key get 0). Required.
 *   lse      required (the backward needs it).
 *   H_kv     key / value heads (>= 1, dividing H): k and v are contiguous
 *            [B, H_kv, S, d_h] and query head h uses head h / (H / H_kv), as
 *            in mha_forward_strided (H_kv = H: ordinary multi-head).
 *   other arguments as for mha_forward; dtype must be MHA_F16 or MHA_BF16.
 *
 * Runs the matrix-core kernels, chosen by size as mha_forward does for long
 * sequences. For bf16, out is identical to what mha_forward_variant writes
 * with MHA_VARIANT_MFMA or MHA_VARIANT_MFMA_SMALL; for fp16 the head and
 * remainder probabilities can move out by a rounding against mha_forward's
 * (out is always out32 rounded once). Returns MHA_ERR_UNSUPPORTED
 * for fp32 inputs, MHA_ERR_NULL without lse or out32, MHA_ERR_SHAPE when one
 * head of out32 spans 2^31 bytes or more or H_kv does not divide H. Ownership, asynchrony and error
 * behaviour as for mha_forward.
 */
int mha_forward_train(const void* q, const void* k, const void* v, void* out, float* lse,
                      float* out32, int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t d_h,
                      int causal, const int32_t* key_len, int dtype, void* stream);

/*
 * mha_forward_strided -- mha_forward over strided views, with grouped
 * key / value heads.
 *
 * Removes the head-split copies of a layer that keeps q, k, v in one fused
 * buffer or in [B, S, H, d_h] order: every tensor is indexed [b, h, i, d]
 * through element strides, and the d_h elements of a row are contiguous.
 *
 *   strides  host pointer to 12 int64: the (batch, head, row) element
 *            strides of q, k, v and out, in that order. Each must be
 *            >= 0 and a multiple of 16 bytes; row strides >= d_h; one
 *            head's rows must span < 2^31 bytes.
 *   H_kv     key / value heads (>= 1, dividing H): query head h uses key /
 *            value head h / (H / H_kv) (grouped-query attention; H_kv = H
 *            is ordinary multi-head attention). k and v are indexed with
 *            heads 0 .. H_kv - 1.
 *   lse      NULL or contiguous fp32 [B, H, S], as for mha_forward.
 *   other arguments as for mha_forward; dtype must be MHA_F16 or MHA_BF16.
 *
 * The rows of out written by one call must not overlap each other or any
 * input. Returns an enum mha_status code; MHA_ERR_MISALIGNED for a stride
 * or pointer that is not 16-byte aligned.
 */
int mha_forward_strided(const void* q, const void* k, const void* v, void* out, float* lse,
                        const int64_t* strides, int64_t B, int64_t H, int64_t H_kv, int64_t S,
                        int64_t d_h, int causal, const int32_t* key_len, int dtype, void* stream);

/*
 * mha_backward -- enqueue the gradients of the forward above on `stream`.
 *
 * Given the output gradient dout of a loss, writes dq, dk, dv: the
 * gradients of sum(dout * out) with respect to q, k and v, for the same
 * mask. Two kinds of work, as in the fused backward of rustingstudio
 * "brain/docs/baseline" ("Fused attention"): one per block of query rows
 * (dq), one per block of key rows (dk, dv); both rebuild the probabilities
 * from the forward's log-sum-exp, P = exp(q.k / sqrt(d_h) - lse). The
 * softmax row term D = rowsum(dout * O) is taken as rowsum(P * dP) /
 * rowsum(P), equal for the exact O and lse, accumulated in fp32 by a first
 * pass over the keys: D from the output rounded to fp16 or bf16 puts errors
 * beyond the accuracy rule into dq where the softmax is peaked, and the
 * division keeps the rows of dS summing to zero when lse is off by a
 * rounding (an lse from a row sum of rounded probabilities).
 *
 *   q, k, v      the forward's inputs (as for mha_forward). Read only.
 *   out, lse     the forward's outputs for exactly these inputs and mask
 *                (lse is required here). lse is read; out is checked
 *                (non-null, 16-byte aligned) but not read.
 *   dout         device pointer, [B, H, S, d_h] of `dtype`. Read only.
 *   dq, dk, dv   device pointers, [B, H, S, d_h] of `dtype`, 16-byte
 *                aligned; written in full (dk = dv = 0 for keys past the
 *                key length). Must not overlap any input.
 *   delta        caller-owned float workspace [B, H, S], 4-byte aligned;
 *                overwritten with D (it stays valid after the call; rows
 *                with no visible key get 0). Every row is written before
 *                it is read, so it needs no clearing.
 *   B .. dtype   as for mha_forward; dtype must be MHA_F16 or MHA_BF16
 *                (fp32 inputs and d_h = 8 return MHA_ERR_UNSUPPORTED).
 *
 * Precision: products on the matrix cores with fp32 accumulation; the
 * probabilities and dS enter them as a head and a remainder in the input
 * dtype (two products each); outputs rounded once to the input dtype. The
 * accuracy rule holds for scores of moderate spread (q and k up to about 3
 * times unit variance); far beyond that, fp32 score arithmetic itself
 * limits dq.
 * Ownership, asynchrony and error behaviour as for mha_forward.
 */
int mha_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, float* delta, int64_t B,
                 int64_t H, int64_t S, int64_t d_h, int causal, const int32_t* key_len, int dtype,
                 void* stream);

/*
 * mha_backward_noalloc -- mha_backward without the delta argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops, harnesses that forbid allocation). The row term goes
 * through a static device array of the library instead: MHA_NOALLOC_MAX_ROWS
 * floats (32 MiB) per GPU, held by each GPU the library runs on until the
 * process ends. Its device address is looked up once per device on the
 * first call (with that device current); the call allocates nothing and
 * makes no allocating library call.
 *
 * All calls on one GPU share that GPU's array, and each call overwrites the
 * rows it uses before reading them: calls that can overlap on one GPU (on
 * different streams, or from different host threads without ordering)
 * race on it and must not be issued. Calls ordered on one stream are safe.
 *
 * Arguments, results and precision as mha_backward (k, v, dk, dv with H
 * heads). Returns MHA_ERR_WORKSPACE, before anything is enqueued, when
 * B * H * S > MHA_NOALLOC_MAX_ROWS; MHA_ERR_HIP if the array's address
 * cannot be found.
 */
int mha_backward_noalloc(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int64_t B, int64_t H, int64_t S, int64_t d_h, int causal,
                         const int32_t* key_len, int dtype, void* stream);

/*
 * mha_backward_grouped -- mha_backward for grouped-query attention: q, out,
 * dout, dq are contiguous [B, H, S, d_h]; k, v, dk, dv are contiguous
 * [B, H_kv, S, d_h] (H_kv >= 1 dividing H; query head h uses key / value
 * head h / (H / H_kv), as in mha_forward_strided). The key / value
 * gradients are summed over the query heads of each group inside one
 * workgroup per key block, without atomics (rustingstudio
 * "brain/docs/baseline", "Fused attention": blocking the key-side kernel on
 * the key / value head). Other arguments and behaviour as mha_backward;
 * MHA_ERR_SHAPE if H_kv does not divide H.
 */
int mha_backward_grouped(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         float* delta, int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t d_h,
                         int causal, const int32_t* key_len, int dtype, void* stream);

/*
 * mha_backward_train -- mha_backward_grouped with the row term taken from
 * the fp32 output of mha_forward_train: D = rowsum(dout * out32) in fp32,
 * one pass over dout and out32 (rustingstudio "brain/docs/baseline",
 * "Fused attention": the row sum comes from dO and O), then the same dq and
 * dk / dv launch as mha_backward_grouped.
 *
 *   out32    the out32 of mha_forward_train for exactly these inputs and
 *            mask: device pointer, contiguous fp32 [B, H, S, d_h], 16-byte
 *            aligned. Read only.
 *   delta    caller-owned float workspace [B, H, S], 4-byte aligned;
 *            overwritten with D.
 *   other arguments as mha_backward_grouped (H_kv = H for ordinary
 *   multi-head attention).
 *
 * Precision as mha_backward: out32 is the exact output to fp32 rounding (the
 * training forward's probabilities enter its value product as a head and a
 * remainder for both dtypes). MHA_ERR_NULL without out32.
 */
int mha_backward_train(const void* q, const void* k, const void* v, const float* out32,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       float* delta, int64_t B, int64_t H, int64_t H_kv, int64_t S, int64_t d_h,
                       int causal, const int32_t* key_len, int dtype, void* stream);

/*
 * mha_qkv_attention -- attention fed by its own QKV projection, for short
 * sequences of 16- or 8-wide heads (devpost "gpu-transformer-optimization",
 * section 2.2: the fused QKV projection, and the fused QKV-attention program
 * used for S <= 128, with heads of 8 grouped in pairs per 16-wide product):
 *     [Q | K | V] = x W_qkv + b_qkv,   x [B, S, d_model], W_qkv [d_model, 3 d_model]
 *     head h of Q, K, V = columns hd h .. hd h + hd - 1 of the respective
 *                         d_model block, hd = d_model / H
 *     out[b, :, hd h .. hd h + hd - 1] = softmax(Q_h K_h^T / sqrt(hd) + mask) V_h
 * with the mask, lse and no-visible-key conventions of mha_forward
 * (key_len[b] clamps to [0, S]). q, k, v exist only on chip: the only
 * device-memory traffic is x, W_qkv, b_qkv in and out, lse out. Activation
 * rows at or past key_len[b] are query rows, but their keys and values are
 * hidden: their contents (even non-finite) reach only their own outputs.
 *
 *   x      contiguous [B, S, d_model], dtype; 16-byte aligned
 *   w_qkv  contiguous [d_model, 3 d_model], dtype (columns q | k | v); 2-byte aligned
 *   b_qkv  contiguous [3 d_model] in dtype, or NULL for no bias; 2-byte aligned
 *   out    contiguous [B, S, d_model], dtype; 16-byte aligned (may not alias x)
 *   lse    float [B, H, S] (natural log), or NULL; 4-byte aligned
 *   key_len  NULL or int32 [B] in device memory
 *   dtype  MHA_F16 or MHA_BF16
 *
 * Supported: d_model in {32, 64, 128} with hd = d_model / H in {8, 16}, and
 * 0 <= S <= 128; otherwise MHA_ERR_UNSUPPORTED (longer sequences or other
 * head sizes take a separate projection and mha_forward_strided);
 * MHA_ERR_SHAPE if H does not divide d_model. Precision: the projection
 * accumulates in fp32; q and k enter the score products as a head and a
 * remainder in the input dtype; v is rounded once for fp16 and carried as a
 * pair for bf16; attention as mha_forward. B == 0 or S == 0 launches
 * nothing.
 * Ownership, asynchrony and error behaviour as for mha_forward.
 */
int mha_qkv_attention(const void* x, const void* w_qkv, const void* b_qkv, void* out, float* lse,
                      int64_t B, int64_t S, int64_t d_model, int64_t H, int causal,
                      const int32_t* key_len, int dtype, void* stream);

/* The variant mha_forward would launch for these arguments (host-only, no
 * GPU call), or a negative mha_status code if the arguments are invalid. */
int mha_select_variant(int64_t B, int64_t H, int64_t S, int64_t d_h, int causal, int dtype);

/* Static name of a variant ("mfma", "valu_d16", ...) or "unknown". */
const char* mha_variant_name(int variant);

/* Static description of a status code. */
const char* mha_status_string(int status);

/* Library ABI version (major * 100 + minor); 101 adds mha_backward, 102
 * mha_forward_strided, 103 mha_backward_grouped, 104 mha_qkv_attention,
 * 105 d_h = 8 (mha_forward*, mha_qkv_attention), 106 mha_backward_noalloc,
 * 107 mha_forward_train and mha_backward_train. */
int mha_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_MHA_AMD_MHA_H */
