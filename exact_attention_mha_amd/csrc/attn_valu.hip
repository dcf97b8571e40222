// d_h = 16 attention forward on the vector ALUs (no matrix cores).
//
// One lane owns one query row: its 16 query values (pre-multiplied by
// log2(e)/sqrt(d_h)), its running max / sum and its 16 fp32 output
// accumulators all live in registers. The workgroup stages 64-key blocks of
// K and V in LDS as fp32; every lane reads the same key row, so the LDS reads
// are broadcasts. Per block a lane computes its 64 scores, takes their
// maximum once, rescales its state and accumulates p * v (running-max
// recurrence, devpost "gpu-transformer-optimization", section 2.1). The
// probabilities stay fp32 (no narrowing before the P.V product).
#include "attn_common.h"
#include "launch.h"

namespace mha {

template <typename T, int NW>
__global__ void __launch_bounds__(NW * 64)
attn_fwd_valu_d16(const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
                  T* __restrict__ Op, float* __restrict__ LSEp, const int32_t* __restrict__ key_len,
                  int H, int S, int causal, int n_qblk, float c_log2) {
  typedef typename Vec<T>::x8 T8;
  constexpr int D = 16;
  constexpr int BK = 64;
  constexpr int BQ = NW * 64;
  __shared__ __attribute__((aligned(16))) float Ks[BK * D];
  __shared__ __attribute__((aligned(16))) float Vs[BK * D];

  const int tid = threadIdx.x;
  const uint32_t logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const uint32_t bh = logical / (uint32_t)n_qblk;
  int qb = (int)(logical - bh * (uint32_t)n_qblk);
  if (causal) qb = n_qblk - 1 - qb;
  const int b = (int)(bh / (uint32_t)H);
  const int L = clamp_len(key_len, b, S);
  const int64_t head = (int64_t)bh * S * D;
  const T* Qh = Qp + head;
  const T* Kh = Kp + head;
  const T* Vh = Vp + head;
  T* Oh = Op + head;

  const int q_start = qb * BQ;
  const int q_end = min(S, q_start + BQ);
  const int kend = causal ? min(L, q_end) : L;
  const int nblk = (kend + BK - 1) / BK;
  const int row = q_start + tid;
  const int wrow0 = q_start + (tid & ~63);
  const int kend_w = wrow0 >= S ? 0 : (causal ? min(L, min(q_end, wrow0 + 64)) : L);
  const int kend_lane = causal ? min(L, row + 1) : L;

  float q[D];
  {
    T8 a = zero_vec<T8>(), bq = zero_vec<T8>();
    if (row < S) {
      a = *(const T8*)(Qh + row * D);
      bq = *(const T8*)(Qh + row * D + 8);
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      q[d] = to_f(a[d]) * c_log2;
      q[8 + d] = to_f(bq[d]) * c_log2;
    }
  }
  float m = -INFINITY, l = 0.f, o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = 0.f;

  for (int kb = 0; kb < nblk; ++kb) {
    const int k0 = kb * BK;
    if (kb) __syncthreads();
    for (int ch = tid; ch < BK * 2; ch += NW * 64) {
      const int r = ch >> 1, h = ch & 1;
      const int key = k0 + r;
      const T8 kv = key < kend ? *(const T8*)(Kh + key * D + 8 * h) : zero_vec<T8>();
      const T8 vv = key < kend ? *(const T8*)(Vh + key * D + 8 * h) : zero_vec<T8>();
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        Ks[r * D + 8 * h + e] = to_f(kv[e]);
        Vs[r * D + 8 * h + e] = to_f(vv[e]);
      }
    }
    __syncthreads();
    if (k0 >= kend_w) continue;

    float sv[BK];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(q[d], Ks[j * D + d], acc);
      sv[j] = (k0 + j < kend_lane) ? acc : -INFINITY;
      mx = fmaxf(mx, sv[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float msafe = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - msafe);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      const float p = fast_exp2(sv[j] - msafe);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, Vs[j * D + d], o[d]);
    }
    m = m_new;
  }

  if (row < S) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    T8 a, bo;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      a[d] = to_t<T>(o[d] * inv);
      bo[d] = to_t<T>(o[8 + d] * inv);
    }
    *(T8*)(Oh + row * D) = a;
    *(T8*)(Oh + row * D + 8) = bo;
    if (LSEp) LSEp[(int64_t)bh * S + row] = l > 0.f ? (m + fast_log2(l)) * kLn2 : -INFINITY;
  }
}

template <typename T, int NW>
static hipError_t launch_one_valu(const AttnParams& p, hipStream_t s) {
  constexpr int BQ = NW * 64;
  const int n_qblk = (p.S + BQ - 1) / BQ;
  const int64_t n_wg = (int64_t)p.B * p.H * n_qblk;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_valu_d16<T, NW>), dim3((unsigned)n_wg), dim3(NW * 64), 0, s,
                     (const T*)p.q, (const T*)p.k, (const T*)p.v, (T*)p.out, p.lse, p.key_len,
                     p.H, p.S, p.causal, n_qblk, p.c_log2);
  return hipGetLastError();
}

hipError_t launch_valu_d16(const AttnParams& p, hipStream_t s) {
  if (p.D != 16) return hipErrorInvalidValue;
  if (p.dtype == 1) return launch_one_valu<f16_t, 2>(p, s);
  if (p.dtype == 2) return launch_one_valu<bf16_t, 2>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mha
