// General fp16 / bf16 attention forward on the gfx950 32x32x16 matrix cores,
// for d_h = 64, 128 and 256 (the mfma32 variant).
//
// On gfx950 one 32x32x16 product does twice the work of a 16x16x32 product
// in about the same issue time (measured in isolation: about 1.9 against
// 1.1-1.3 PFLOP/s fp16 on a full chip), so this kernel builds both attention
// products from 32x32 tiles. Within the whole kernel it measures no faster
// than the 16x16 kernel (its products run without overlapping the softmax
// work), so that one stays the default; this variant is kept selectable for
// measurement:
//     S^T = K Q^T      32 keys x 32 queries per tile, d_h / 16 products
//     O^T += V^T P^T   32 output columns x 32 queries, 16 keys per product
// with the running-max recurrence of devpost
// "gpu-transformer-optimization", section 2.1 ("The mechanism: online
// softmax"), the rescale taken lazily (only when a block's maximum exceeds
// the running maximum by more than 2^8).
//
// Lane layout (lane = 32 g + c): the 32x32 result of a product holds row
// 8J + 4g + i, column c in register 4J + i. Every lane owns one query column
// c of a score tile, so row maxima reduce inside the lane and across the
// lane pair (c, c + 32) only. Registers 8s .. 8s + 7 of a score tile are keys
// 16s + 8j + 4g + i (slot 4j + i), exactly the 16-key B operand of the P V
// product for key half s: probabilities need no shuffles.
//
// Work decomposition. A workgroup owns one (batch, head) and a block of
// NW * NQ * 32 query rows (each wave NQ tiles of 32 rows, Q held in
// registers as B operands); it walks the key blocks of BK rows in order. K
// and V blocks are copied from device memory straight into LDS by the
// buffer DMA path, NST stages deep, one barrier per block. Row sums are
// accumulated on the vector ALUs from the same rounded probabilities the
// P V products use.
//
// LDS layout, in natural key order:
//   * K rows padded to D + 8 elements: a K operand read (16 bytes of row c at
//     column 16kk + 8g) puts 16 consecutive rows on 16 distinct bank groups.
//   * V rows padded to D + 32 elements: the transposed reads of V
//     (ds_read_b64_tr_b16: lane j of a 16-lane group gets column j of a
//     4 x 16 block) touch 4 consecutive rows x 64 bytes per half wave, and a
//     row stride of 2D + 64 bytes puts those 4 rows on distinct 64-byte bank
//     groups.
// Pad slots and rows past the visible keys read as zero from out-of-range
// buffer offsets.
#include <utility>

#include "attn_common.h"
#include "launch.h"

namespace mha {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.f;
  return z;
}

constexpr float kRescaleSlack32 = 8.0f;  // log2 units: lazy rescale threshold

template <typename T, int D, int NQ, int NW, int BK, int NST>
__global__ void __launch_bounds__(NW * 64, NW == 4 ? 2 : 1)
attn_fwd_m32(const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
             T* __restrict__ Op, float* __restrict__ LSEp, const int32_t* __restrict__ key_len,
             int H, int S, int causal, int n_qblk, float c_log2, Layout lay) {
  typedef typename Vec<T>::x8 T8;
  typedef typename Vec<T>::x4 T4;
  constexpr int KSTR = D + 8, VSTR = D + 32;     // padded row strides (elements)
  constexpr int KSPR = KSTR / 8, VSPR = VSTR / 8;  // 16-byte slots per row
  constexpr int KNI = (BK * KSPR + 63) / 64;     // DMA instructions per K tile
  constexpr int VNI = (BK * VSPR + 63) / 64;     // ... per V tile
  constexpr int KTILE = KNI * 512, VTILE = VNI * 512;  // elements (whole instructions)
  constexpr int STAGE = KTILE + VTILE;
  constexpr int KIW = (KNI + NW - 1) / NW, VIW = (VNI + NW - 1) / NW;
  constexpr int MINW = KNI / NW + VNI / NW;      // copies every wave issues per block
  constexpr int NDT = D / 32;                    // output column tiles
  constexpr int NKT = BK / 32;                   // key tiles per block
  constexpr int NKS = D / 16;                    // K = 16 steps of S^T
  constexpr int ES = (int)sizeof(T);
  constexpr int BQ = NW * NQ * 32;
  constexpr bool kBf16 = __is_same(T, bf16_t);
  static_assert(BK % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(STAGE * ES * NST <= 160 * 1024, "LDS");
  constexpr int PF = NST - 1;  // blocks copied ahead
  // operand reads issued ahead of their products (fewer at d_h = 256, where
  // O and Q take most of the registers)
  constexpr int LAK = D == 256 ? 2 : 4, LAV = D == 256 ? 2 : 4;

  __shared__ __attribute__((aligned(16))) T smem[NST * STAGE];  // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, g = lane >> 5;

  const uint32_t logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const uint32_t bh = logical / (uint32_t)n_qblk;
  int qb = (int)(logical - bh * (uint32_t)n_qblk);
  if (causal) qb = n_qblk - 1 - qb;  // heaviest causal tiles are dispatched first
  const int b = (int)(bh / (uint32_t)H);
  const int h = (int)(bh - (uint32_t)b * (uint32_t)H);
  const int L = clamp_len(key_len, b, S);
  const T* Qh = Qp + b * lay.q_b + h * lay.q_h;
  const T* Kh = Kp + b * lay.k_b + (h / lay.group) * lay.k_h;
  const T* Vh = Vp + b * lay.v_b + (h / lay.group) * lay.v_h;
  T* Oh = Op + b * lay.o_b + h * lay.o_h;
  const int RQ = lay.q_s * ES, RK = lay.k_s * ES, RV = lay.v_s * ES, RO = lay.o_s * ES;
  auto span = [](int n, int rs) { return (uint32_t)((n - 1) * rs + D * ES); };

  const int q_start = qb * BQ;
  const int q_end = min(S, q_start + BQ);
  const int kend = causal ? min(L, q_end) : L;  // keys any row of the block sees
  const int nblk = (kend + BK - 1) / BK;
  const int wq0 = q_start + wave * NQ * 32;
  const bool wave_live = wq0 < S;
  const int kend_w = !wave_live ? 0 : (causal ? min(L, min(q_end, wq0 + NQ * 32)) : L);

  const rsrc_t ro = make_rsrc(Oh, span(S, RO));
  const rsrc_t rl = make_rsrc(LSEp + (int64_t)bh * S, (uint32_t)S * 4);

  if (nblk == 0) {  // no visible key (L == 0): out = 0, lse = -inf
    if (wave_live) {
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        const int row = wq0 + 32 * t + c;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int J = 0; J < 4; ++J)
            buf_store8(zero_vec<T4>(), ro, row * RO + (32 * dt + 8 * J + 4 * g) * ES);
        if (LSEp) buf_store4(-INFINITY, rl, g == 0 ? row * 4 : kOutOfRange);
      }
    }
    return;
  }

  // ---- per-lane DMA source offsets of this wave's slots (block relative)
  const rsrc_t rk = make_rsrc(Kh, span(kend, RK));
  const rsrc_t rv = make_rsrc(Vh, span(kend, RV));
  int koff[KIW], voff[VIW];
#pragma unroll
  for (int i = 0; i < KIW; ++i) {
    const int slot = (wave + i * NW) * 64 + lane;
    const int row = slot / KSPR, j = slot - row * KSPR;
    koff[i] = (row < BK && j < D / 8) ? row * RK + 16 * j : kOutOfRange;
  }
#pragma unroll
  for (int i = 0; i < VIW; ++i) {
    const int slot = (wave + i * NW) * 64 + lane;
    const int row = slot / VSPR, j = slot - row * VSPR;
    voff[i] = (row < BK && j < D / 8) ? row * RV + 16 * j : kOutOfRange;
  }
  auto dma_block = [&](int st, int k0) {
    T* Kst = smem + st * STAGE;
    T* Vst = Kst + KTILE;
#pragma unroll
    for (int i = 0; i < KIW; ++i) {
      const int inst = wave + i * NW;
      if (KNI % NW == 0 || inst < KNI) dma16(rk, Kst + inst * 512, koff[i], k0 * RK);
    }
#pragma unroll
    for (int i = 0; i < VIW; ++i) {
      const int inst = wave + i * NW;
      if (VNI % NW == 0 || inst < VNI) dma16(rv, Vst + inst * 512, voff[i], k0 * RV);
    }
  };

  // ---- Q fragments: B operands, lane (g, c) holds row c, columns
  //      16kk + 8g .. + 7 (rows past S read as zero)
  const rsrc_t rq = make_rsrc(Qh, span(S, RQ));
  T8 qf[NQ][NKS];
#pragma unroll
  for (int t = 0; t < NQ; ++t)
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk)
      qf[t][kk] = buf_load16<T8>(rq, (wq0 + 32 * t + c) * RQ + (16 * kk + 8 * g) * ES, 0);

  asm volatile("" ::: "memory");  // Q loads are issued (and so retire) before the copies
#pragma unroll
  for (int st = 0; st < PF; ++st) dma_block(st, st * BK);
  wait_vmem_keep<MINW * PF>();  // the older Q loads have landed
#pragma unroll
  for (int t = 0; t < NQ; ++t)
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) asm volatile("" : "+v"(qf[t][kk]));

  float m_run[NQ], l_run[NQ];  // running max (log2 units), this lane's share of the row sum
  f32x16 o[NQ][NDT];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    m_run[t] = -INFINITY;
    l_run[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[t][dt] = zero16();
  }

  // per-lane LDS byte addresses (stage 0): K operand row c at column 8g;
  // V transposed read: lanes 4r .. 4r + 3 of a 16-lane group supply row r
  // (key 4g + r) at columns 16 (c / 16) + 4 (c % 4)
  const uint32_t kaddr0 = lds_addr(smem) + (c * KSTR + 8 * g) * ES;
  const int j16 = c & 15;
  const uint32_t vaddr0 = lds_addr(smem + KTILE) +
                          ((4 * g + (j16 >> 2)) * VSTR + 16 * (c >> 4) + 4 * (j16 & 3)) * ES;

  // ---- the work on one key block, in three phases:
  //   scores  -- K operand reads and S^T = K Q^T
  //   softmax -- masks, block row max, lazy rescale, P = exp2(S c - m)
  //              rounded to T (bf16: head and remainder), row sums
  //   pv      -- V^T operand reads and O^T += V^T P^T
  auto scores = [&](int kb, f32x16 (&sc)[NQ][NKT]) {
    const uint32_t kaddr = kaddr0 + (uint32_t)((kb % NST) * STAGE * ES);
    static_for<NKT>([&](auto KT) {
      constexpr int kt = decltype(KT)::value;
#pragma unroll
      for (int t = 0; t < NQ; ++t) sc[t][kt] = zero16();
      constexpr int LA = NKS < LAK ? NKS : LAK;
      u32x4 kr[NKS];
      auto issue = [&](auto KK) {
        constexpr int kk = decltype(KK)::value;
        kr[kk] = lds_read_b128_asm<(32 * kt * KSTR + 16 * kk) * ES>(kaddr);
      };
      static_for<LA>(issue);
      static_for<NKS>([&](auto KK) {
        constexpr int kk = decltype(KK)::value;
        if constexpr (kk + LA < NKS) issue(std::integral_constant<int, kk + LA>{});
        constexpr int last = kk + LA < NKS ? kk + LA : NKS - 1;
        lgkm_wait1<last - kk>(kr[kk]);
        const T8 kf = __builtin_bit_cast(T8, kr[kk]);
#pragma unroll
        for (int t = 0; t < NQ; ++t) sc[t][kt] = mfma32(kf, qf[t][kk], sc[t][kt]);
      });
    });
  };
  auto softmax = [&](int kb, f32x16 (&sc)[NQ][NKT], T8 (&pf)[NQ][2 * NKT], T8 (&pl)[NQ][2 * NKT]) {
    const int k0 = kb * BK;
    // mask only blocks that straddle the key length or the diagonal:
    // register 4J + i of tile kt is key k0 + 32kt + 8J + 4g + i
    if ((k0 + BK > L) || (causal && (k0 + BK - 1 > wq0))) {
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        const int row = wq0 + 32 * t + c;
        const int lim = (causal ? min(L - 1, row) : L - 1) - k0 - 4 * g;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int off = 32 * kt + 8 * (v >> 2) + (v & 3);
            sc[t][kt][v] = off <= lim ? sc[t][kt][v] : -INFINITY;
          }
      }
    }
    // block row maxima; the running max moves only when exceeded by more
    // than the slack (wave-uniform decision)
    float mb[NQ];
    bool grow = false;
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      float mx = sc[t][0][0];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int v = 0; v < 16; v += 2) mx = max3(mx, sc[t][kt][v], sc[t][kt][v + 1]);
      mb[t] = xor32_pair_max(mx) * c_log2;  // finite: key 0 is visible to every row
      grow |= mb[t] > m_run[t] + kRescaleSlack32;
    }
    if (__any(grow)) {
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        const float m_new = fmaxf(m_run[t], mb[t]);
        const float alpha = fast_exp2(m_run[t] - m_new);
        m_run[t] = m_new;
        l_run[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[t][dt] *= alpha;
      }
    }
    // registers 8hs .. 8hs + 7 of tile kt: the B operand of key half 2kt + hs
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      float ls = 0.f;
#pragma unroll
      for (int kh = 0; kh < 2 * NKT; ++kh)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = fast_exp2(fmaf(sc[t][kh >> 1][8 * (kh & 1) + e], c_log2, -m_run[t]));
          pf[t][kh][e] = to_t<T>(a);
          ls += to_f(pf[t][kh][e]);  // the rounded weight the numerator uses
          if constexpr (kBf16) {
            pl[t][kh][e] = to_t<T>(a - to_f(pf[t][kh][e]));
            ls += to_f(pl[t][kh][e]);
          }
        }
      l_run[t] += ls;
    }
  };
  auto pv = [&](int kb, const T8 (&pf)[NQ][2 * NKT], const T8 (&pl)[NQ][2 * NKT]) {
    const uint32_t vaddr = vaddr0 + (uint32_t)((kb % NST) * STAGE * ES);
    static_for<NKT * 2>([&](auto KH) {
      constexpr int kh = decltype(KH)::value;
      constexpr int LA = NDT < LAV ? NDT : LAV;
      constexpr int rbase = 16 * kh;  // first key row of this half
      i16x4 va[NDT], vb[NDT];
      auto issue = [&](auto J) {
        constexpr int j = decltype(J)::value;
        va[j] = lds_read_tr16_asm<(rbase * VSTR + 32 * j) * ES>(vaddr);
        vb[j] = lds_read_tr16_asm<((rbase + 8) * VSTR + 32 * j) * ES>(vaddr);
      };
      static_for<LA>(issue);
      static_for<NDT>([&](auto DT) {
        constexpr int dt = decltype(DT)::value;
        if constexpr (dt + LA < NDT) issue(std::integral_constant<int, dt + LA>{});
        constexpr int last = dt + LA < NDT ? dt + LA : NDT - 1;
        lgkm_wait<2 * (last - dt)>(va[dt], vb[dt]);
        const T8 vf = __builtin_bit_cast(T8, __builtin_shufflevector(va[dt], vb[dt], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
          o[t][dt] = mfma32(vf, pf[t][kh], o[t][dt]);
          if constexpr (kBf16) o[t][dt] = mfma32(vf, pl[t][kh], o[t][dt]);
        }
      });
    });
  };

  const int nblk_w = (kend_w + BK - 1) / BK;  // blocks this wave's rows see
  for (int kb = 0; kb < nblk; ++kb) {
    // this wave's copies of block kb have landed (later blocks may still be
    // in flight); after the barrier everyone's have, and everyone is done
    // with block kb - 1, whose stage the next copy reuses
    if (PF == 1 || kb + PF - 1 >= nblk) wait_vmem();
    else wait_vmem_keep<MINW * (PF - 1)>();
    block_barrier();
    if (kb + PF < nblk) dma_block((kb + PF) % NST, (kb + PF) * BK);
    if (kb < nblk_w) {  // wave-uniform: past this wave's rows otherwise
      f32x16 s[NQ][NKT];
      T8 pf[NQ][2 * NKT], pl[NQ][2 * NKT];
      scores(kb, s);
      softmax(kb, s, pf, pl);
      pv(kb, pf, pl);
    }
  }

  // ---- epilogue: O / l rounded once to T; lse = ln(2) * (m + log2 l).
  //      Rows past S fall outside the store ranges and are dropped.
  if (wave_live) {
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      // the lane pair (c, c + 32) shares the row
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run[t]),
                                                      __float_as_uint(l_run[t]), false, false);
      const float l = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      const int row = wq0 + 32 * t + c;
      const float inv = __builtin_amdgcn_rcpf(l);  // l >= 1: the running max's own key gives 1
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          T4 ov;
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[i] = to_t<T>(o[t][dt][4 * J + i] * inv);
          buf_store8(ov, ro, row * RO + (32 * dt + 8 * J + 4 * g) * ES);
        }
      if (LSEp) buf_store4((m_run[t] + fast_log2(l)) * kLn2, rl, g == 0 ? row * 4 : kOutOfRange);
    }
  }
}

template <typename T, int D, int NQ, int NW, int BK, int NST = 2>
static hipError_t launch_m32_one(const AttnParams& p, hipStream_t s) {
  constexpr int BQ = NW * NQ * 32;
  const int n_qblk = (p.S + BQ - 1) / BQ;
  const int64_t n_wg = (int64_t)p.B * p.H * n_qblk;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_m32<T, D, NQ, NW, BK, NST>), dim3((unsigned)n_wg), dim3(NW * 64), 0, s,
                     (const T*)p.q, (const T*)p.k, (const T*)p.v, (T*)p.out, p.lse, p.key_len, p.H,
                     p.S, p.causal, n_qblk, p.c_log2, p.lay);
  return hipGetLastError();
}

// Tile shapes (NQ 32-row query tiles per wave, NW waves, BK keys per block,
// copy stages) per head size, the fastest of those measured.
template <typename T>
static hipError_t launch_m32_t(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 64: return launch_m32_one<T, 64, 2, 4, 64>(p, s);
    case 128: return launch_m32_one<T, 128, 1, 8, 64>(p, s);
    case 256: return launch_m32_one<T, 256, 1, 8, 32>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_m32(const AttnParams& p, hipStream_t s) {
  if (p.dtype == 1) return launch_m32_t<f16_t>(p, s);
  if (p.dtype == 2) return launch_m32_t<bf16_t>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mha
