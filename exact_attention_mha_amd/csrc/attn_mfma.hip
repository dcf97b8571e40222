// General fp16 / bf16 attention forward on the gfx950 matrix cores.
//
// One workgroup owns one (batch, head) and a block of BQ = NW*NQT*16 query
// rows; each wave owns NQT 16-row query tiles whose Q fragments stay in
// registers. The workgroup walks key blocks of BK rows in order: K (row
// major) and V (transposed, so a lane reads 8 consecutive keys of one
// output column) are staged in LDS, then each wave computes
//     S^T = K Q^T            (16x16x32 MFMA, fp32 accumulate)
//     online softmax update  (running max m, running sum l, rescale O by
//                             exp2(m_old - m_new))
//     O^T += V^T P^T         (P rounded to the input dtype; bf16 uses a
//                             bf16 head + bf16 remainder, two products)
// following the running-max recurrence of devpost
// "gpu-transformer-optimization", section 2.1 ("The mechanism: online
// softmax"). Key blocks past the causal diagonal or the key length are
// skipped; only blocks that straddle either boundary are masked elementwise.
//
// Key order inside a 32-key pair: the two 16-key S^T tiles take keys
// 8*(r/4) + r%4 and 8*(r/4) + 4 + r%4 on their row r, so that lane group g
// ends up holding keys 8g..8g+7 of the pair, which is exactly the K index
// run of the P^T operand of the PV product and one 16-byte read of V^T.
#include "attn_common.h"
#include "launch.h"

namespace mha {

template <typename T, int D, int NQT, int NW, int BK>
__global__ void __launch_bounds__(NW * 64)
attn_fwd_mfma(const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
              T* __restrict__ Op, float* __restrict__ LSEp, const int32_t* __restrict__ key_len,
              int H, int S, int causal, int n_qblk, float c_log2) {
  typedef typename Vec<T>::x8 T8;
  typedef typename Vec<T>::x4 T4;
  constexpr int BQ = NW * NQT * 16;
  constexpr int KSTR = D + 8;   // padded LDS row strides (elements)
  constexpr int VSTR = BK + 8;
  constexpr int NDT = D / 16;   // output column tiles
  constexpr int NKT = BK / 16;  // key tiles per block
  constexpr int NKP = BK / 32;  // key pairs per block
  constexpr int NKC = D >= 32 ? D / 32 : 1;
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr bool kBf16 = __is_same(T, bf16_t);
  static_assert(BK % 32 == 0 && D % 16 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) T Ks[BK * KSTR];
  __shared__ __attribute__((aligned(16))) T Vt[D * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;

  const uint32_t logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const uint32_t bh = logical / (uint32_t)n_qblk;
  int qb = (int)(logical - bh * (uint32_t)n_qblk);
  if (causal) qb = n_qblk - 1 - qb;  // heaviest causal tiles are dispatched first
  const int b = (int)(bh / (uint32_t)H);
  const int L = clamp_len(key_len, b, S);
  const int64_t head = (int64_t)bh * S * D;
  const T* Qh = Qp + head;
  const T* Kh = Kp + head;
  const T* Vh = Vp + head;
  T* Oh = Op + head;

  const int q_start = qb * BQ;
  const int q_end = min(S, q_start + BQ);
  const int kend = causal ? min(L, q_end) : L;  // keys any row of the block sees
  const int nblk = (kend + BK - 1) / BK;
  const int wq0 = q_start + wave * NQT * 16;
  const bool wave_live = wq0 < S;
  const int kend_w = !wave_live ? 0 : (causal ? min(L, min(q_end, wq0 + NQT * 16)) : L);

  T8 qf[NQT][NKC];
  T4 qf4[NQT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    const int row = wq0 + 16 * t + c;
    if constexpr (D == 16) {
      qf4[t] = row < S ? *(const T4*)(Qh + row * D + 4 * g) : zero_vec<T4>();
    } else {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
        qf[t][kc] = row < S ? *(const T8*)(Qh + row * D + 32 * kc + 8 * g) : zero_vec<T8>();
    }
  }

  float m_run[NQT], l_run[NQT];
  f32x4 o[NQT][NDT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int kb = 0; kb < nblk; ++kb) {
    const int k0 = kb * BK;
    if (kb) __syncthreads();  // everyone is done reading the previous block
    // ---- stage K (row major) and V (transposed) into LDS; rows past kend
    //      are zero-filled and never read from memory
    for (int ch = tid; ch < BK * CPR; ch += NW * 64) {
      const int r = ch / CPR, cc = ch - r * CPR;
      const int key = k0 + r;
      const T8 val = key < kend ? *(const T8*)(Kh + key * D + cc * 8) : zero_vec<T8>();
      *(T8*)(Ks + r * KSTR + cc * 8) = val;
    }
    for (int ch = tid; ch < BK * CPR; ch += NW * 64) {
      const int r = ch % BK, cc = ch / BK;
      const int key = k0 + r;
      const T8 val = key < kend ? *(const T8*)(Vh + key * D + cc * 8) : zero_vec<T8>();
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[(cc * 8 + e) * VSTR + r] = val[e];
    }
    __syncthreads();
    if (k0 >= kend_w) continue;  // wave-uniform: block is past this wave's rows

    // ---- S^T = K Q^T for every key tile of the block
    f32x4 s[NQT][NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      const int krow = 32 * (kt >> 1) + 8 * (c >> 2) + 4 * (kt & 1) + (c & 3);
#pragma unroll
      for (int t = 0; t < NQT; ++t) s[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (D == 16) {
        const T4 kf = *(const T4*)(Ks + krow * KSTR + 4 * g);
#pragma unroll
        for (int t = 0; t < NQT; ++t) s[t][kt] = mfma_k16(kf, qf4[t], s[t][kt]);
      } else {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          const T8 kf = *(const T8*)(Ks + krow * KSTR + 32 * kc + 8 * g);
#pragma unroll
          for (int t = 0; t < NQT; ++t) s[t][kt] = mfma_k32(kf, qf[t][kc], s[t][kt]);
        }
      }
    }

    // ---- mask only blocks that straddle the key length or the diagonal
    const bool need_mask = (k0 + BK > L) || (causal && (k0 + BK - 1 > wq0));
    if (need_mask) {
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        const int row = wq0 + 16 * t + c;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = k0 + 32 * (kt >> 1) + 8 * g + 4 * (kt & 1) + i;
            const bool ok = key < L && (!causal || key <= row);
            if (!ok) s[t][kt][i] = -INFINITY;
          }
      }
    }

    // ---- online softmax update (exp2 domain, scale folded into one FMA)
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      float mx = s[t][0][0];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[t][kt][i]);
      mx = group_max(mx);  // finite: key 0 is visible to every row once L > 0
      const float m_new = fmaxf(m_run[t], mx * c_log2);
      const float alpha = fast_exp2(m_run[t] - m_new);
      m_run[t] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = fast_exp2(fmaf(s[t][kt][i], c_log2, -m_new));
          s[t][kt][i] = pv;
          ls += pv;
        }
      l_run[t] = fmaf(alpha, l_run[t], ls);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[t][dt] *= alpha;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int p = 0; p < NKP; ++p) {
      T8 pf[NQT], pl[NQT];
#pragma unroll
      for (int t = 0; t < NQT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a0 = s[t][2 * p][i], a1 = s[t][2 * p + 1][i];
          pf[t][i] = to_t<T>(a0);
          pf[t][4 + i] = to_t<T>(a1);
          if constexpr (kBf16) {
            pl[t][i] = to_t<T>(a0 - to_f(pf[t][i]));
            pl[t][4 + i] = to_t<T>(a1 - to_f(pf[t][4 + i]));
          }
        }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const T8 vf = *(const T8*)(Vt + (16 * dt + c) * VSTR + 32 * p + 8 * g);
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
          o[t][dt] = mfma_k32(vf, pf[t], o[t][dt]);
          if constexpr (kBf16) o[t][dt] = mfma_k32(vf, pl[t], o[t][dt]);
        }
      }
    }
  }

  // ---- epilogue: O / l rounded once to T; lse = ln(2) * (m + log2 l)
  if (wave_live) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      const float l = group_sum(l_run[t]);
      const int row = wq0 + 16 * t + c;
      const float inv = l > 0.f ? 1.f / l : 0.f;
      if (row < S) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          T4 ov;
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = to_t<T>(o[t][dt][i] * inv);
          *(T4*)(Oh + row * D + 16 * dt + 4 * g) = ov;
        }
        if (LSEp && g == 0)
          LSEp[(int64_t)bh * S + row] = l > 0.f ? (m_run[t] + fast_log2(l)) * kLn2 : -INFINITY;
      }
    }
  }
}

template <typename T, int D, int NQT, int NW, int BK>
static hipError_t launch_one(const AttnParams& p, hipStream_t s) {
  constexpr int BQ = NW * NQT * 16;
  const int n_qblk = (p.S + BQ - 1) / BQ;
  const int64_t n_wg = (int64_t)p.B * p.H * n_qblk;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_mfma<T, D, NQT, NW, BK>), dim3((unsigned)n_wg), dim3(NW * 64), 0, s,
                     (const T*)p.q, (const T*)p.k, (const T*)p.v, (T*)p.out, p.lse, p.key_len,
                     p.H, p.S, p.causal, n_qblk, p.c_log2);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_general(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_one<T, 16, 2, 4, 64>(p, s);
    case 32: return launch_one<T, 32, 2, 4, 64>(p, s);
    case 64: return launch_one<T, 64, 2, 4, 64>(p, s);
    case 128: return launch_one<T, 128, 2, 4, 64>(p, s);
    case 256: return launch_one<T, 256, 2, 4, 32>(p, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_small(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 16: return launch_one<T, 16, 1, 1, 64>(p, s);
    case 32: return launch_one<T, 32, 1, 1, 64>(p, s);
    case 64: return launch_one<T, 64, 1, 1, 64>(p, s);
    case 128: return launch_one<T, 128, 1, 1, 64>(p, s);
    case 256: return launch_one<T, 256, 1, 1, 32>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mfma(const AttnParams& p, hipStream_t s) {
  if (p.dtype == 1) return launch_general<f16_t>(p, s);
  if (p.dtype == 2) return launch_general<bf16_t>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_mfma_small(const AttnParams& p, hipStream_t s) {
  if (p.dtype == 1) return launch_small<f16_t>(p, s);
  if (p.dtype == 2) return launch_small<bf16_t>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mha
