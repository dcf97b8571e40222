// Short-sequence attention forward for d_h = 16 heads (S <= 128), fp16/bf16;
// d_h = 8 heads run the same code as 16-wide heads with zero columns 8..15.
//
// The regime of many tiny heads (the bandwidth-bound shape: tens of thousands
// of heads of 128 rows x 16 columns) is decided by per-head overhead, so this
// kernel has none to spare: one wave owns one head (or, for launch-bound
// shapes with few heads, a balanced pair of 16-row query tiles of a head, or
// a single query tile),
// there is no LDS and no barrier, and every operand is loaded straight from
// memory in the layout the matrix cores consume:
//   * K rows and Q rows are the A / B operands of S^T = K Q^T
//     (16x16x16 MFMA): lane (g, c) reads 8 bytes, row c, columns 4g..4g+3;
//     16 lanes cover 512 contiguous bytes.
//   * V is read the same way and transposed through the wave's own slice of
//     LDS: each lane writes its 8 bytes (row c, columns 4g..4g+3) and the
//     LDS transpose read (ds_read_b64_tr_b16) returns, in lane (g, c),
//     column c of keys 4g..4g+3 -- the A-operand layout of O^T += V^T P^T.
//     Only the wave itself touches its slice, and its LDS operations complete
//     in issue order, so no barrier is needed; values pass through unchanged
//     (an Inf or NaN in V stays in its own column).
// A whole score row fits in registers, so each query tile takes a single
// pass: row maximum, exponentials, P.V, no rescaling (devpost
// "gpu-transformer-optimization", section 2.2: at S <= 128 the score row
// fits at once and no online softmax is needed). Only key tiles a query tile
// can see are computed: up to its own diagonal when causal, never past the
// key length. The row sum comes from a ones operand times the same rounded P
// as the numerator. Rows past S and keys past the key length are handled by
// the buffer range checks (reads as zero, stores dropped).
#include <utility>

#include "attn_common.h"
#include "launch.h"

namespace mha {

// At least two waves per SIMD: with that budget (<= 256 registers per lane)
// the compiler keeps matrix-core results in ordinary VGPRs, where the softmax
// reads them, instead of accumulation registers that need a copy per value.
// LDS: 8 key tiles x 16 rows x 32 bytes per wave, for the V transpose.
template <typename T, int D, int QPW, bool CAUSAL>
__global__ void __launch_bounds__(256, 2)
attn_fwd_short16(const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
                 T* __restrict__ Op, float* __restrict__ LSEp, const int32_t* __restrict__ key_len,
                 int BH, int H, int S, float c_log2, Layout lay) {
  constexpr bool causal = CAUSAL;
  typedef typename Vec<T>::x4 T4;
  // d_h = 16, or d_h = 8 run as a 16-wide head whose columns 8..15 are zero:
  // lane groups g = 2, 3 (those columns) load nothing and store nothing
  static_assert(D == 16 || D == 8, "head size");
  constexpr bool kHalf = D == 8;
  constexpr int RB = D * (int)sizeof(T);  // bytes per row
  constexpr int NT = 8;                    // 16-row tiles in S <= 128
  constexpr int PARTS = NT / QPW;          // waves per head
  constexpr bool kBf16 = __is_same(T, bf16_t);
  static_assert(QPW == 8 || QPW == 2 || QPW == 1,
                "whole head, a balanced tile pair or one tile per wave");

  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const bool gcol = !kHalf || g < 2;  // this lane group's four columns exist
  const int item = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  const int bh = item / PARTS, part = item - bh * PARTS;
  if (bh >= BH) return;  // wave-uniform; no barriers in this kernel
  const int b = bh / H, h = bh - b * H;
  const int L = clamp_len(key_len, b, S);
  // this head's rows in each tensor and the bytes between rows (a range of
  // n rows covers (n - 1) row strides plus one row; none when n = 0)
  const int RQ = lay.q_s * 2, RK = lay.k_s * 2, RV = lay.v_s * 2, RO = lay.o_s * 2;
  auto span = [](int n, int rs) { return n > 0 ? (uint32_t)((n - 1) * rs + RB) : 0u; };
  const rsrc_t rq = make_rsrc(Qp + b * lay.q_b + h * lay.q_h, span(S, RQ));
  const rsrc_t rk = make_rsrc(Kp + b * lay.k_b + (h / lay.group) * lay.k_h, span(L, RK));
  const rsrc_t rv = make_rsrc(Vp + b * lay.v_b + (h / lay.group) * lay.v_h, span(L, RV));
  const rsrc_t ro = make_rsrc(Op + b * lay.o_b + h * lay.o_h, span(S, RO));
  const rsrc_t rl = make_rsrc(LSEp + (int64_t)bh * S, (uint32_t)S * 4);

  // query tiles of this wave; with pairs, wave `part` takes tiles part and
  // 7-part, so every wave of a causal head does 9 key tiles of work; with
  // one tile per wave, wave `part` takes tile part
  int tile[QPW];
#pragma unroll
  for (int j = 0; j < QPW; ++j) tile[j] = QPW == NT ? j : (j == 0 ? part : NT - 1 - part);
  // key tiles the computation touches: none past the key length, none past
  // the last diagonal when causal
  int kt_need = (L + 15) >> 4;
  if (causal) {
    int tmax = 0;
#pragma unroll
    for (int j = 0; j < QPW; ++j) tmax = max(tmax, tile[j]);
    kt_need = min(kt_need, tmax + 1);
  }

  // ---- operands straight from memory (keys past L and rows past S read 0)
  T4 qf[QPW], kf[NT], vt[NT];
#pragma unroll
  for (int j = 0; j < QPW; ++j) qf[j] = buf_load8<T4>(rq, gcol ? (16 * tile[j] + c) * RQ + 8 * g : kOutOfRange, 0);
  T4 vraw[NT];
#pragma unroll
  for (int kt = 0; kt < NT; ++kt) {
    if (kt < kt_need) {
      kf[kt] = buf_load8<T4>(rk, gcol ? (16 * kt + c) * RK + 8 * g : kOutOfRange, 0);
      vraw[kt] = buf_load8<T4>(rv, gcol ? (16 * kt + c) * RV + 8 * g : kOutOfRange, 0);
    }
  }
  T4 ones;
#pragma unroll
  for (int e = 0; e < 4; ++e) ones[e] = to_t<T>(1.f);
  // V^T through this wave's LDS slice: tile kt holds keys 16kt..16kt+15 as
  // 16 rows of 16 elements (32 bytes). Lane (g, c) writes row c, columns
  // 4g..4g+3; the transpose read of lane (g, c) names row 4g + c/4, columns
  // 4(c%4)..4(c%4)+3 and receives column c of rows 4g..4g+3.
  __shared__ __attribute__((aligned(16))) T vlds[4][NT * 256];
  T* vw = vlds[threadIdx.x >> 6];
#pragma unroll
  for (int kt = 0; kt < NT; ++kt)
    if (kt < kt_need) *(T4*)(vw + kt * 256 + c * 16 + 4 * g) = vraw[kt];
#pragma unroll
  for (int kt = 0; kt < NT; ++kt)
    if (kt < kt_need)
      vt[kt] = __builtin_bit_cast(T4, lds_read_tr16(vw + kt * 256 + (4 * g + (c >> 2)) * 16 + 4 * (c & 3)));

  // Masks ride in the S^T accumulator: a product starts from 0 (visible) or
  // -inf (hidden), so hidden scores come out as -inf with no per-element
  // work. Register i of lane (g, c) in key tile kt is key 16kt + 4g + i of
  // row 16t + c. Key tiles at or past the key length's tile kL are never
  // computed except kL itself, which starts from `strad` (keys past L
  // hidden); the causal diagonal tile starts from `diag` (key <= row).
  const int kL = L >> 4;  // wave-uniform; L >= 1 below
  typedef AccK16T<T> AccT;  // accumulator of this dtype's K = 16 product

  // one query tile, with its index a compile-time constant so that every
  // register array is indexed statically; the key tiles it sees are
  // computed without per-element branches
  auto qtile = [&](auto J) {
    constexpr int j = decltype(J)::value;
    const int t = tile[j];
    if (16 * t >= S) return;  // wave-uniform
    const int row = 16 * t + c;
    if (L == 0) {  // no visible key
      buf_store8(zero_vec<T4>(), ro, gcol ? row * RO + 8 * g : kOutOfRange);
      if (LSEp) buf_store4(-INFINITY, rl, g == 0 ? row * 4 : kOutOfRange);
      return;
    }
    constexpr int NK = (QPW == NT && CAUSAL) ? j + 1 : NT;  // key tiles computed at most
    // last key tile with a visible key (wave-uniform)
    const int klast = min(CAUSAL ? t : NT - 1, (L - 1) >> 4);
    AccT s[NT];
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
      if (kt > klast) break;
      AccT init = AccT::zero();
      if (kt == kL || (CAUSAL && kt == t)) {  // wave-uniform: a tile with hidden keys
        const int lim = min(L - 1, CAUSAL && kt == t ? row : S) - 16 * kt - 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) init[i] = i <= lim ? 0.f : -INFINITY;
      }
      s[kt] = mfma_k16(kf[kt], qf[j], init);
      mx = max3(mx, s[kt][0], s[kt][1]);
      mx = max3(mx, s[kt][2], s[kt][3]);
    }
    const float m = group_max(mx) * c_log2;  // finite: key 0 is visible
    AccT o = AccT::zero(), lsum = AccT::zero();
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
      if (kt > klast) break;
      T4 pf, pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = fast_exp2(fmaf(s[kt][i], c_log2, -m));
        pf[i] = to_t<T>(pv);
        if constexpr (kBf16) pl[i] = to_t<T>(pv - to_f(pf[i]));
      }
      o = mfma_k16(vt[kt], pf, o);
      lsum = mfma_k16(ones, pf, lsum);
      if constexpr (kBf16) {
        o = mfma_k16(vt[kt], pl, o);
        lsum = mfma_k16(ones, pl, lsum);
      }
    }
    const float l = lsum[0];  // every row of the ones product holds the full sum
    const float inv = 1.f / l;
    T4 ov;
#pragma unroll
    for (int i = 0; i < 4; ++i) ov[i] = to_t<T>(o[i] * inv);
    buf_store8(ov, ro, gcol ? row * RO + 8 * g : kOutOfRange);  // O^T lane layout: row, columns 4g..4g+3
    if (LSEp) buf_store4((m + fast_log2(l)) * kLn2, rl, g == 0 ? row * 4 : kOutOfRange);
    __builtin_amdgcn_sched_barrier(0);  // keep query tiles from interleaving (register pressure)
  };
  [&]<int... J>(std::integer_sequence<int, J...>) {
    (qtile(std::integral_constant<int, J>{}), ...);
  }(std::make_integer_sequence<int, QPW>{});
}

template <typename T, int D, int QPW>
static hipError_t launch_one_short16(const AttnParams& p, hipStream_t s) {
  constexpr int PARTS = 8 / QPW;
  const int64_t waves = (int64_t)p.B * p.H * PARTS;
  const int64_t n_wg = (waves + 3) / 4;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (p.causal)
    hipLaunchKernelGGL((attn_fwd_short16<T, D, QPW, true>), dim3((unsigned)n_wg), dim3(256), 0, s,
                       (const T*)p.q, (const T*)p.k, (const T*)p.v, (T*)p.out, p.lse, p.key_len,
                       p.B * p.H, p.H, p.S, p.c_log2, p.lay);
  else
    hipLaunchKernelGGL((attn_fwd_short16<T, D, QPW, false>), dim3((unsigned)n_wg), dim3(256), 0, s,
                       (const T*)p.q, (const T*)p.k, (const T*)p.v, (T*)p.out, p.lse, p.key_len,
                       p.B * p.H, p.H, p.S, p.c_log2, p.lay);
  return hipGetLastError();
}

// Very few heads (at most one wave per SIMD even split 8 ways): one query
// tile per wave, so the longest wave computes 8 key tiles instead of a
// pair's 9 and loads only the key tiles its tile sees (3.69 -> 3.39 us per
// call for 8 heads); few heads: 4 waves per head on balanced tile pairs,
// which load fewer key tiles in all; many heads: one wave per head.
template <typename T, int D>
static hipError_t launch_short16_t(const AttnParams& p, hipStream_t s) {
  const int64_t bh = (int64_t)p.B * p.H;
  if (bh <= 128) return launch_one_short16<T, D, 1>(p, s);
  if (bh < 2048) return launch_one_short16<T, D, 2>(p, s);
  return launch_one_short16<T, D, 8>(p, s);
}

hipError_t launch_short16(const AttnParams& p, hipStream_t s) {
  if ((p.D != 16 && p.D != 8) || p.S > 128) return hipErrorInvalidValue;
  if (p.dtype == 1) return p.D == 16 ? launch_short16_t<f16_t, 16>(p, s) : launch_short16_t<f16_t, 8>(p, s);
  if (p.dtype == 2) return p.D == 16 ? launch_short16_t<bf16_t, 16>(p, s) : launch_short16_t<bf16_t, 8>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mha
