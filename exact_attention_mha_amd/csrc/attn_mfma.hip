// General fp16 / bf16 attention forward on the gfx950 matrix cores.
//
// One workgroup owns one (batch, head) and a block of BQ = NW*NQT*16 query
// rows; each wave owns NQT 16-row query tiles whose Q fragments stay in
// registers. The workgroup walks key blocks of BK rows in order. K and V are
// staged row major in LDS, double buffered: the next block's global loads are
// issued before the current block's arithmetic and written to the other LDS
// buffer after it, so there is one barrier per block. Each wave computes
//     S^T = K Q^T            (16x16x32 MFMA, fp32 accumulate)
//     online softmax update  (running max m, running sum l, O rescaled by
//                             exp2(m_old - m_new))
//     O^T += V^T P^T         (V^T read with the LDS transpose read; P rounded
//                             to the input dtype, bf16 as head + remainder)
// following the running-max recurrence of devpost
// "gpu-transformer-optimization", section 2.1 ("The mechanism: online
// softmax"). The rescale is lazy: the running max only moves when a block's
// maximum exceeds it by more than 2^8 (probabilities then stay <= 256, which
// fp32 sums and fp16 probabilities hold without loss), so O is rarely
// touched; numerator and denominator always share the same max, so the
// result is the same quotient. Key blocks past the causal diagonal or the key
// length are skipped; only blocks that straddle either boundary are masked.
//
// Key order inside a 32-key pair: the two 16-key S^T tiles take keys
// 8*(r/4) + r%4 and 8*(r/4) + 4 + r%4 on their row r, so that lane group g
// holds keys 8g..8g+7 of the pair, which is the K index run of the P^T
// operand and of two transpose reads of V.
#include "attn_common.h"
#include "launch.h"

namespace mha {

constexpr float kRescaleSlack = 8.0f;  // log2 units: lazy rescale threshold

template <typename T, int D, int NQT, int NW, int BK>
__global__ void __launch_bounds__(NW * 64)
attn_fwd_mfma(const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
              T* __restrict__ Op, float* __restrict__ LSEp, const int32_t* __restrict__ key_len,
              int H, int S, int causal, int n_qblk, float c_log2) {
  typedef typename Vec<T>::x8 T8;
  typedef typename Vec<T>::x4 T4;
  constexpr int NT = NW * 64;
  constexpr int BQ = NW * NQT * 16;
  constexpr int STR = D + 8;        // padded LDS row stride (elements), K and V
  constexpr int TILE = BK * STR;    // one K or V block in LDS
  constexpr int NDT = D / 16;       // output column tiles
  constexpr int NKT = BK / 16;      // key tiles per block
  constexpr int NKP = BK / 32;      // key pairs per block
  constexpr int NKC = D >= 32 ? D / 32 : 1;
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int NCH = BK * CPR;     // chunks per block per tensor
  constexpr int CPT = (NCH + NT - 1) / NT;
  constexpr bool kBf16 = __is_same(T, bf16_t);
  static_assert(BK % 32 == 0 && D % 16 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) T smem[2 * 2 * TILE];  // [stage][K, V]

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

  // ---- global -> register prefetch of one K/V block, register -> LDS store
  T8 pk[CPT], pv[CPT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int ch = tid + j * NT;
      const int r = ch / CPR, cc = ch - r * CPR;
      const int key = k0 + r;
      const bool in = (NCH % NT == 0 || ch < NCH) && key < kend;
      pk[j] = in ? *(const T8*)(Kh + key * D + cc * 8) : zero_vec<T8>();
      pv[j] = in ? *(const T8*)(Vh + key * D + cc * 8) : zero_vec<T8>();
    }
  };
  auto lstore = [&](int st) {
    T* Ks = smem + st * 2 * TILE;
    T* Vs = Ks + TILE;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int ch = tid + j * NT;
      if (NCH % NT == 0 || ch < NCH) {
        const int r = ch / CPR, cc = ch - r * CPR;
        *(T8*)(Ks + r * STR + cc * 8) = pk[j];
        *(T8*)(Vs + r * STR + cc * 8) = pv[j];
      }
    }
  };

  if (nblk > 0) gload(0);

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

  if (nblk > 0) lstore(0);
  __syncthreads();

  for (int kb = 0; kb < nblk; ++kb) {
    const int k0 = kb * BK;
    const bool more = kb + 1 < nblk;
    if (more) gload(k0 + BK);  // in flight during this block's arithmetic

    if (k0 < kend_w) {  // wave-uniform: block overlaps this wave's rows
      const T* Ks = smem + (kb & 1) * 2 * TILE;
      const T* Vs = Ks + TILE;

      // ---- S^T = K Q^T
      f32x4 s[NQT][NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const int krow = 32 * (kt >> 1) + 8 * (c >> 2) + 4 * (kt & 1) + (c & 3);
#pragma unroll
        for (int t = 0; t < NQT; ++t) s[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (D == 16) {
          const T4 kf = *(const T4*)(Ks + krow * STR + 4 * g);
#pragma unroll
          for (int t = 0; t < NQT; ++t) s[t][kt] = mfma_k16(kf, qf4[t], s[t][kt]);
        } else {
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc) {
            const T8 kf = *(const T8*)(Ks + krow * STR + 32 * kc + 8 * g);
#pragma unroll
            for (int t = 0; t < NQT; ++t) s[t][kt] = mfma_k32(kf, qf[t][kc], s[t][kt]);
          }
        }
      }

      // ---- mask only blocks that straddle the key length or the diagonal
      if ((k0 + BK > L) || (causal && (k0 + BK - 1 > wq0))) {
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
          const int row = wq0 + 16 * t + c;
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = k0 + 32 * (kt >> 1) + 8 * g + 4 * (kt & 1) + i;
              const bool ok = key < L && (!causal || key <= row);
              s[t][kt][i] = ok ? s[t][kt][i] : -INFINITY;
            }
        }
      }

      // ---- block row maxima; move the running max only when it is exceeded
      //      by more than the slack (wave-uniform decision)
      float mb[NQT];
      bool grow = false;
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        float mx = s[t][0][0];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[t][kt][i]);
        mb[t] = group_max(mx) * c_log2;  // finite: key 0 is visible to every row
        grow |= mb[t] > m_run[t] + kRescaleSlack;
      }
      if (__any(grow)) {
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
          const float m_new = fmaxf(m_run[t], mb[t]);
          const float alpha = fast_exp2(m_run[t] - m_new);
          m_run[t] = m_new;
          l_run[t] *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[t][dt] *= alpha;
        }
      }

      // ---- P = exp2(S c - m); O^T += V^T P^T, one key pair at a time
#pragma unroll
      for (int p = 0; p < NKP; ++p) {
        T8 pf[NQT], pl[NQT];
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
          float ls = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a0 = fast_exp2(fmaf(s[t][2 * p][i], c_log2, -m_run[t]));
            const float a1 = fast_exp2(fmaf(s[t][2 * p + 1][i], c_log2, -m_run[t]));
            ls += a0 + a1;
            pf[t][i] = to_t<T>(a0);
            pf[t][4 + i] = to_t<T>(a1);
            if constexpr (kBf16) {
              pl[t][i] = to_t<T>(a0 - to_f(pf[t][i]));
              pl[t][4 + i] = to_t<T>(a1 - to_f(pf[t][4 + i]));
            }
          }
          l_run[t] += ls;
        }
        const T* vrow = Vs + (32 * p + 8 * g + (c >> 2)) * STR + 4 * (c & 3);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const i16x4 v0 = lds_read_tr16(vrow + 16 * dt);
          const i16x4 v1 = lds_read_tr16(vrow + 4 * STR + 16 * dt);
          const T8 vf = __builtin_bit_cast(
              T8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int t = 0; t < NQT; ++t) {
            o[t][dt] = mfma_k32(vf, pf[t], o[t][dt]);
            if constexpr (kBf16) o[t][dt] = mfma_k32(vf, pl[t], o[t][dt]);
          }
        }
      }
    }

    if (more) lstore((kb + 1) & 1);
    __syncthreads();
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

// Tile shapes (NQT query tiles per wave, NW waves, BK keys per block) per head
// size. Entry 0 is the default; the others are kept for A/B measurement and
// are selected with the MHA_TILE_CONFIG environment variable.
template <typename T>
static hipError_t launch_general(const AttnParams& p, hipStream_t s) {
  const int cfg = p.tile_cfg;
  switch (p.D) {
    case 16: return launch_one<T, 16, 2, 4, 64>(p, s);
    case 32: return launch_one<T, 32, 2, 4, 64>(p, s);
    case 64:
      if (cfg == 1) return launch_one<T, 64, 4, 4, 64>(p, s);
      if (cfg == 2) return launch_one<T, 64, 2, 4, 64>(p, s);
      if (cfg == 3) return launch_one<T, 64, 2, 8, 128>(p, s);
      return launch_one<T, 64, 2, 8, 64>(p, s);
    case 128:
      if (cfg == 1) return launch_one<T, 128, 2, 4, 64>(p, s);
      return launch_one<T, 128, 2, 8, 64>(p, s);
    case 256:
      if (cfg == 1) return launch_one<T, 256, 1, 8, 32>(p, s);
      if (cfg == 2) return launch_one<T, 256, 2, 8, 32>(p, s);
      if (cfg == 3) return launch_one<T, 256, 1, 4, 64>(p, s);
      return launch_one<T, 256, 2, 4, 32>(p, s);
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
