// Short-sequence fp16 / bf16 attention forward (S <= 128, d_h <= 64).
//
// When a whole row of scores fits on chip there is nothing to rescale: one
// pass computes the row maximum, the exponentials and the sum (devpost
// "gpu-transformer-optimization", section 2.2: at S <= 128 the score row fits
// at once and no online softmax is needed). One workgroup owns one
// (batch, head): it stages the head's visible K rows and transposed V rows in
// LDS once, and wave w computes query tiles w and 7-w, which balances the
// causal triangle (tile t needs t+1 key tiles) across the four waves.
// Every query tile computes only the key tiles it can see: up to its own
// diagonal when causal, never past the key length.
#include <type_traits>

#include "attn_common.h"
#include "launch.h"

namespace mha {

template <typename T, int D>
__global__ void __launch_bounds__(256)
attn_fwd_short(const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
               T* __restrict__ Op, float* __restrict__ LSEp, const int32_t* __restrict__ key_len,
               int H, int S, int causal, float c_log2) {
  typedef typename Vec<T>::x8 T8;
  typedef typename Vec<T>::x4 T4;
  constexpr int SK = 128;
  constexpr int KSTR = D + 8;
  constexpr int VSTR = SK + 8;
  constexpr int NDT = D / 16;
  constexpr int NKC = D >= 32 ? D / 32 : 1;
  constexpr int CPR = D / 8;
  constexpr bool kBf16 = __is_same(T, bf16_t);
  static_assert(D == 16 || D == 32 || D == 64, "short kernel head size");

  __shared__ __attribute__((aligned(16))) T Ks[SK * KSTR];
  __shared__ __attribute__((aligned(16))) T Vt[D * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;

  const uint32_t bh = xcd_logical_id(blockIdx.x, gridDim.x);
  const int b = (int)(bh / (uint32_t)H);
  const int L = clamp_len(key_len, b, S);
  const int64_t head = (int64_t)bh * S * D;
  const T* Qh = Qp + head;
  const T* Kh = Kp + head;
  const T* Vh = Vp + head;
  T* Oh = Op + head;

  // stage the visible key rows (rounded up to a 32-key pair, zero filled)
  const int nload = (L + 31) & ~31;
  for (int ch = tid; ch < nload * CPR; ch += 256) {
    const int r = ch / CPR, cc = ch - r * CPR;
    const T8 val = r < L ? *(const T8*)(Kh + r * D + cc * 8) : zero_vec<T8>();
    *(T8*)(Ks + r * KSTR + cc * 8) = val;
  }
  for (int ch = tid; ch < nload * CPR; ch += 256) {
    const int r = ch % nload, cc = ch / nload;
    const T8 val = r < L ? *(const T8*)(Vh + r * D + cc * 8) : zero_vec<T8>();
#pragma unroll
    for (int e = 0; e < 8; ++e) Vt[(cc * 8 + e) * VSTR + r] = val[e];
  }
  __syncthreads();

#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    const int t = half == 0 ? wave : 7 - wave;
    const int r0 = 16 * t;
    if (r0 >= S) continue;  // wave-uniform
    const int row = r0 + c;
    const int kv = causal ? min(L, r0 + 16) : L;  // keys this tile can see
    const int npair = (kv + 31) >> 5;

    T8 qf[NKC];
    T4 qf4;
    if constexpr (D == 16) {
      qf4 = row < S ? *(const T4*)(Qh + row * D + 4 * g) : zero_vec<T4>();
    } else {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
        qf[kc] = row < S ? *(const T8*)(Qh + row * D + 32 * kc + 8 * g) : zero_vec<T8>();
    }

    // scores come from K = 16 products at d_h = 16, K = 32 ones otherwise
    typedef std::conditional_t<D == 16, AccK16T<T>, AccK32> SAcc;
    SAcc s[8];
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      s[kt] = SAcc::zero();
      if (kt < 2 * npair) {
        const int krow = 32 * (kt >> 1) + 8 * (c >> 2) + 4 * (kt & 1) + (c & 3);
        if constexpr (D == 16) {
          const T4 kf = *(const T4*)(Ks + krow * KSTR + 4 * g);
          s[kt] = mfma_k16(kf, qf4, s[kt]);
        } else {
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc) {
            const T8 kf = *(const T8*)(Ks + krow * KSTR + 32 * kc + 8 * g);
            s[kt] = mfma_k32(kf, qf[kc], s[kt]);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 32 * (kt >> 1) + 8 * g + 4 * (kt & 1) + i;
          const bool ok = key < L && (!causal || key <= row);
          s[kt][i] = ok ? s[kt][i] : -INFINITY;
          mx = fmaxf(mx, s[kt][i]);
        }
      }
    }
    mx = group_max(mx);
    const float m = mx * c_log2;  // -inf only when the tile sees no key (L == 0)
    const float msafe = npair > 0 ? m : 0.f;
    float ls = 0.f;
    AccK32 o[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[dt] = AccK32::zero();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p < npair) {
        T8 pf, pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a0 = fast_exp2(fmaf(s[2 * p][i], c_log2, -msafe));
          const float a1 = fast_exp2(fmaf(s[2 * p + 1][i], c_log2, -msafe));
          pf[i] = to_t<T>(a0);
          pf[4 + i] = to_t<T>(a1);
          // the denominator sums the same rounded weights the numerator
          // multiplies V by (head + remainder for bf16)
          ls += to_f(pf[i]) + to_f(pf[4 + i]);
          if constexpr (kBf16) {
            pl[i] = to_t<T>(a0 - to_f(pf[i]));
            pl[4 + i] = to_t<T>(a1 - to_f(pf[4 + i]));
            ls += to_f(pl[i]) + to_f(pl[4 + i]);
          }
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const T8 vf = *(const T8*)(Vt + (16 * dt + c) * VSTR + 32 * p + 8 * g);
          o[dt] = mfma_k32(vf, pf, o[dt]);
          if constexpr (kBf16) o[dt] = mfma_k32(vf, pl, o[dt]);
        }
      }
    }
    const float l = group_sum(ls);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (row < S) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        T4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = to_t<T>(o[dt][i] * inv);
        *(T4*)(Oh + row * D + 16 * dt + 4 * g) = ov;
      }
      if (LSEp && g == 0)
        LSEp[(int64_t)bh * S + row] = l > 0.f ? (m + fast_log2(l)) * kLn2 : -INFINITY;
    }
  }
}

template <typename T, int D>
static hipError_t launch_one_short(const AttnParams& p, hipStream_t s) {
  const int64_t n_wg = (int64_t)p.B * p.H;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_short<T, D>), dim3((unsigned)n_wg), dim3(256), 0, s,
                     (const T*)p.q, (const T*)p.k, (const T*)p.v, (T*)p.out, p.lse, p.key_len,
                     p.H, p.S, p.causal, p.c_log2);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_short_t(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_one_short<T, 16>(p, s);
    case 32: return launch_one_short<T, 32>(p, s);
    case 64: return launch_one_short<T, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_short(const AttnParams& p, hipStream_t s) {
  if (p.S > 128) return hipErrorInvalidValue;
  if (p.dtype == 1) return launch_short_t<f16_t>(p, s);
  if (p.dtype == 2) return launch_short_t<bf16_t>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mha
