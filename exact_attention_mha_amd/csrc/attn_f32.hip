// fp32 attention forward: the same tiled online-softmax loop as the fp16 /
// bf16 kernel, on the fp32 matrix-core product (16x16x4, exact fp32 inputs,
// fp32 accumulate), so fp32 inputs are never narrowed.
//
// Scores are computed transposed (S^T = K Q^T, devpost
// "gpu-transformer-optimization", section 2.1 ops (1)-(2)) and the softmax
// follows the running-max recurrence of the same section. With a K depth of
// 4 the PV product consumes one key per lane group per instruction, so V can
// stay row-major in LDS: lane (g, c) reads V[key 4g+i][column c], which is
// bank-conflict free without a transpose.
#include "attn_common.h"
#include "launch.h"

namespace mha {

template <int D, int NQT, int NW, int BK>
__global__ void __launch_bounds__(NW * 64)
attn_fwd_f32(const float* __restrict__ Qp, const float* __restrict__ Kp,
             const float* __restrict__ Vp, float* __restrict__ Op, float* __restrict__ LSEp,
             const int32_t* __restrict__ key_len, int H, int S, int causal, int n_qblk,
             float c_log2) {
  constexpr int BQ = NW * NQT * 16;
  constexpr int STR = D + 4;
  constexpr int NDT = D / 16;
  constexpr int NKT = BK / 16;
  constexpr int NKC = D / 16;
  constexpr int CPR = D / 4;  // 16-byte chunks per row
  static_assert(BK % 16 == 0 && D % 16 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) float Ks[BK * STR];
  __shared__ __attribute__((aligned(16))) float Vs[BK * STR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;

  const uint32_t logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const uint32_t bh = logical / (uint32_t)n_qblk;
  int qb = (int)(logical - bh * (uint32_t)n_qblk);
  if (causal) qb = n_qblk - 1 - qb;
  const int b = (int)(bh / (uint32_t)H);
  const int L = clamp_len(key_len, b, S);
  const int64_t head = (int64_t)bh * S * D;
  const float* Qh = Qp + head;
  const float* Kh = Kp + head;
  const float* Vh = Vp + head;
  float* Oh = Op + head;

  const int q_start = qb * BQ;
  const int q_end = min(S, q_start + BQ);
  const int kend = causal ? min(L, q_end) : L;
  const int nblk = (kend + BK - 1) / BK;
  const int wq0 = q_start + wave * NQT * 16;
  const bool wave_live = wq0 < S;
  const int kend_w = !wave_live ? 0 : (causal ? min(L, min(q_end, wq0 + NQT * 16)) : L);

  f32x4 qf[NQT][NKC];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    const int row = wq0 + 16 * t + c;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
      qf[t][kc] = row < S ? *(const f32x4*)(Qh + row * D + 16 * kc + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  float m_run[NQT], l_run[NQT];
  AccK4 o[NQT][NDT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[t][dt] = AccK4::zero();
  }

  for (int kb = 0; kb < nblk; ++kb) {
    const int k0 = kb * BK;
    if (kb) __syncthreads();
    for (int ch = tid; ch < BK * CPR; ch += NW * 64) {
      const int r = ch / CPR, cc = ch - r * CPR;
      const int key = k0 + r;
      const bool in = key < kend;
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      *(f32x4*)(Ks + r * STR + cc * 4) = in ? *(const f32x4*)(Kh + key * D + cc * 4) : zero;
      *(f32x4*)(Vs + r * STR + cc * 4) = in ? *(const f32x4*)(Vh + key * D + cc * 4) : zero;
    }
    __syncthreads();
    if (k0 >= kend_w) continue;

    AccK4 s[NQT][NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int t = 0; t < NQT; ++t) s[t][kt] = AccK4::zero();
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const f32x4 kf = *(const f32x4*)(Ks + (16 * kt + c) * STR + 16 * kc + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int t = 0; t < NQT; ++t) s[t][kt] = mfma_f32_k4(kf[e], qf[t][kc][e], s[t][kt]);
      }
    }

    const bool need_mask = (k0 + BK > L) || (causal && (k0 + BK - 1 > wq0));
    if (need_mask) {
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        const int row = wq0 + 16 * t + c;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = k0 + 16 * kt + 4 * g + i;
            const bool ok = key < L && (!causal || key <= row);
            if (!ok) s[t][kt][i] = -INFINITY;
          }
      }
    }

#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      float mx = s[t][0][0];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[t][kt][i]);
      mx = group_max(mx);
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

    // O^T += V^T P^T, one key per lane group per instruction
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const float vv = Vs[(16 * kt + 4 * g + i) * STR + 16 * dt + c];
#pragma unroll
          for (int t = 0; t < NQT; ++t) o[t][dt] = mfma_f32_k4(vv, s[t][kt][i], o[t][dt]);
        }
  }

  if (wave_live) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      const float l = group_sum(l_run[t]);
      const int row = wq0 + 16 * t + c;
      const float inv = l > 0.f ? 1.f / l : 0.f;
      if (row < S) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) *(f32x4*)(Oh + row * D + 16 * dt + 4 * g) = o[t][dt].vec() * inv;
        if (LSEp && g == 0)
          LSEp[(int64_t)bh * S + row] = l > 0.f ? (m_run[t] + fast_log2(l)) * kLn2 : -INFINITY;
      }
    }
  }
}

template <int D, int NQT, int NW, int BK>
static hipError_t launch_one_f32(const AttnParams& p, hipStream_t s) {
  constexpr int BQ = NW * NQT * 16;
  const int n_qblk = (p.S + BQ - 1) / BQ;
  const int64_t n_wg = (int64_t)p.B * p.H * n_qblk;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_f32<D, NQT, NW, BK>), dim3((unsigned)n_wg), dim3(NW * 64), 0, s,
                     (const float*)p.q, (const float*)p.k, (const float*)p.v, (float*)p.out, p.lse,
                     p.key_len, p.H, p.S, p.causal, n_qblk, p.c_log2);
  return hipGetLastError();
}

hipError_t launch_f32(const AttnParams& p, hipStream_t s) {
  if (p.dtype != 0) return hipErrorInvalidValue;
  switch (p.D) {
    case 16: return launch_one_f32<16, 1, 4, 32>(p, s);
    case 32: return launch_one_f32<32, 1, 4, 32>(p, s);
    case 64: return launch_one_f32<64, 1, 4, 32>(p, s);
    case 128: return launch_one_f32<128, 1, 4, 32>(p, s);
    case 256: return launch_one_f32<256, 1, 4, 16>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mha
