// General fp16 / bf16 attention forward on the gfx950 matrix cores.
//
// One workgroup owns one (batch, head) and a block of BQ = NW*NQT*16 query
// rows; each wave owns NQT 16-row query tiles whose Q fragments stay in
// registers. The workgroup walks key blocks of BK rows in order. K and V
// blocks are copied from device memory straight into LDS by the buffer DMA
// path (no staging registers), double buffered: block kb+1 is in flight while
// block kb is consumed, with one barrier per block. Each wave computes
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
// quotient is unchanged. Key blocks past the causal diagonal or the key
// length are skipped; only blocks that straddle either boundary are masked.
// The row sum l can be accumulated on the matrix cores (a ones operand times
// the same rounded P as the numerator) instead of on the vector ALUs. With
// STALE the block maximum is not taken at all: probabilities use the running
// max as it stands, and each key pair's matrix-core row sums are checked for
// overflow of the dtype (the check and recompute of attn_fwd_pipe below; the
// pair's scores are still in registers, so a failing pair only needs its own
// maximum, a rescale and new probabilities).
//
// LDS layout. Rows are padded by one 16-byte slot (the DMA loads a zero
// there), and rows are permuted inside each 32-key pair so every read is
// bank-conflict free:
//  * S^T tile h of pair p reads, on its A-operand row c, key
//    8*(c/4) + 4h + c%4 of the pair (so lane group g ends up holding keys
//    8g..8g+7 of the pair, the K index run of the P^T operand). K is stored
//    in that read order: LDS row 16h + c holds that key, and one operand read
//    touches 16 consecutive padded rows.
//  * the two transpose reads of V for lane group g cover keys 8g+4s+r
//    (s = 0, 1; r = 0..3). V key 8g+4s+r is stored at LDS row
//    16*(g/2) + 8*(g%2) + 2r + s, so the 8 rows read together by a
//    32-lane half of the wave are all even or all odd rows.
// Rows past the visible key range and the pad slots come from out-of-range
// buffer offsets, which read as zero without touching memory.
#include <type_traits>

#include "attn_common.h"
#include "launch.h"

namespace mha {

constexpr float kRescaleSlack = 8.0f;  // log2 units: lazy rescale threshold
constexpr float kNoMaxStale = -1.0e30f;  // finite: exp2(s c - it) overflows, exp2(-inf) stays 0
// largest accepted row sum of one 32-key pair's rounded probabilities: above
// every sum of 32 finite fp16 values (32 * 65504 < 2^21), below any that
// holds an overflowed one; for bf16 it bounds each probability by 2^21
constexpr float kPairSumMax = 2097152.0f;

// key (within a 32-key pair) stored at LDS row rho of the K / V tile
__device__ __forceinline__ int k_key_of_row(int rho) {
  const int h = rho >> 4, c = rho & 15;
  return 8 * (c >> 2) + 4 * h + (c & 3);
}
__device__ __forceinline__ int v_key_of_row(int rho) {
  return 16 * (rho >> 4) + 8 * ((rho >> 3) & 1) + 4 * (rho & 1) + ((rho >> 1) & 3);
}

// Four-wave workgroups ask for two of them per CU (two waves per SIMD), which
// also keeps matrix-core results in ordinary VGPRs.
// SPLITP: fp16 probabilities enter the value product as a head and a
// remainder too (bf16 always does), for an output exact to fp32 rounding.
template <typename T, int D, int NQT, int NW, int BK, bool SUM_MFMA, int NST, bool STALE = false,
          bool SPLITP = false>
__global__ void __launch_bounds__(NW * 64, NW == 4 ? 2 : 1)
attn_fwd_mfma(const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
              T* __restrict__ Op, float* __restrict__ LSEp, float* __restrict__ O32p,
              const int32_t* __restrict__ key_len, int H, int S, int causal, int n_qblk,
              float c_log2, Layout lay) {
  typedef typename Vec<T>::x8 T8;
  typedef typename Vec<T>::x4 T4;
  constexpr int STR = D + 8;             // padded LDS row stride (elements)
  constexpr int SPR = D / 8 + 1;         // 16-byte slots per padded row
  constexpr int SLOTS = BK * SPR;        // slots per K or V tile
  constexpr int NI = (SLOTS + 63) / 64;  // DMA instructions per tile
  constexpr int TILE = NI * 64 * 8;      // elements per tile (whole DMA instructions)
  constexpr int NIW = (NI + NW - 1) / NW;
  // output column tiles; d_h = 8 runs as one 16-wide tile whose columns
  // 8..15 are zero (the LDS pad slot of each row holds zeros there, Q loads
  // and O stores of those columns are out of range)
  constexpr int NDT = D >= 16 ? D / 16 : 1;
  constexpr bool kHalf = D == 8;
  constexpr int NKT = BK / 16;           // key tiles per block
  constexpr int NKP = BK / 32;           // key pairs per block
  constexpr int NKC = D >= 32 ? D / 32 : 1;
  constexpr int ES = (int)sizeof(T);
  constexpr int BQ = NW * NQT * 16;
  constexpr bool kBf16 = __is_same(T, bf16_t) || SPLITP;  // probabilities as head + remainder
  static_assert(BK % 32 == 0 && (D % 16 == 0 || D == 8), "tile shape");

  __shared__ __attribute__((aligned(16))) T smem[NST * 2 * TILE];  // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;

  const uint32_t logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const uint32_t bh = logical / (uint32_t)n_qblk;
  int qb = (int)(logical - bh * (uint32_t)n_qblk);
  if (causal) qb = n_qblk - 1 - qb;  // heaviest causal tiles are dispatched first
  const int b = (int)(bh / (uint32_t)H);
  const int h = (int)(bh - (uint32_t)b * (uint32_t)H);
  const int L = clamp_len(key_len, b, S);
  // this head's rows in each tensor, and the bytes between consecutive rows
  const T* Qh = Qp + b * lay.q_b + h * lay.q_h;
  const T* Kh = Kp + b * lay.k_b + (h / lay.group) * lay.k_h;
  const T* Vh = Vp + b * lay.v_b + (h / lay.group) * lay.v_h;
  T* Oh = Op + b * lay.o_b + h * lay.o_h;
  const int RQ = lay.q_s * ES, RK = lay.k_s * ES, RV = lay.v_s * ES, RO = lay.o_s * ES;
  // byte range of n rows starting at a head's first row
  auto span = [](int n, int rs) { return (uint32_t)((n - 1) * rs + D * ES); };

  const int q_start = qb * BQ;
  const int q_end = min(S, q_start + BQ);
  const int kend = causal ? min(L, q_end) : L;  // keys any row of the block sees
  const int nblk = (kend + BK - 1) / BK;
  const int wq0 = q_start + wave * NQT * 16;
  const bool wave_live = wq0 < S;
  const int kend_w = !wave_live ? 0 : (causal ? min(L, min(q_end, wq0 + NQT * 16)) : L);

  const rsrc_t ro = make_rsrc(Oh, span(S, RO));
  const rsrc_t rl = make_rsrc(LSEp + (int64_t)bh * S, (uint32_t)S * 4);
  // fp32 copy of the output (training forward): contiguous [B, H, S, D]
  const rsrc_t r32 = make_rsrc(O32p + (int64_t)bh * S * D, (uint32_t)S * D * 4);

  if (nblk == 0) {  // no visible key (L == 0): out = 0, lse = -inf
    if (wave_live) {
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        const int row = wq0 + 16 * t + c;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          buf_store8(zero_vec<T4>(), ro, kHalf && g >= 2 ? kOutOfRange : row * RO + (16 * dt + 4 * g) * 2);
        if (O32p)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            buf_store16(f32x4{0.f, 0.f, 0.f, 0.f}, r32, kHalf && g >= 2 ? kOutOfRange : (row * D + 16 * dt + 4 * g) * 4);
        if (LSEp) buf_store4(-INFINITY, rl, g == 0 ? row * 4 : kOutOfRange);
      }
    }
    return;
  }

  // ---- per-lane DMA source offsets of this wave's slots (block relative)
  const rsrc_t rk = make_rsrc(Kh, span(kend, RK));
  const rsrc_t rv = make_rsrc(Vh, span(kend, RV));
  int koff[NIW], voff[NIW];
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    const int slot = (wave + i * NW) * 64 + lane;
    const int row = slot / SPR, j = slot - row * SPR;
    const bool live = slot < SLOTS && j < D / 8;
    const int base = 32 * (row >> 5);
    koff[i] = live ? (base + k_key_of_row(row & 31)) * RK + 16 * j : kOutOfRange;
    voff[i] = live ? (base + v_key_of_row(row & 31)) * RV + 16 * j : kOutOfRange;
  }
  auto dma_block = [&](int st, int k0) {
    T* Kst = smem + st * 2 * TILE;
    T* Vst = Kst + TILE;
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int inst = wave + i * NW;
      if (NI % NW == 0 || inst < NI) {  // wave-uniform
        dma16(rk, Kst + inst * 512, koff[i], k0 * RK);
        dma16(rv, Vst + inst * 512, voff[i], k0 * RV);
      }
    }
  };

  // ---- Q fragments (rows past S read as zero)
  const rsrc_t rq = make_rsrc(Qh, span(S, RQ));
  T8 qf[NQT][NKC];
  T4 qf4[NQT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    const int row = wq0 + 16 * t + c;
    if constexpr (D <= 16) {
      qf4[t] = buf_load8<T4>(rq, kHalf && g >= 2 ? kOutOfRange : row * RQ + 4 * g * 2, 0);
    } else {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) qf[t][kc] = buf_load16<T8>(rq, row * RQ + (32 * kc + 8 * g) * 2, 0);
    }
  }

  asm volatile("" ::: "memory");  // Q loads are issued (and so retire) before the copies
  // prologue copies; unconditional (blocks past the visible keys read as
  // zero) so the outstanding count below is fixed
#pragma unroll
  for (int st = 0; st < NST - 1; ++st) dma_block(st, st * BK);
  // the Q loads are older than every copy: this retires them before the loop
  wait_vmem_keep<2 * (NI / NW) * (NST - 1)>();
  // and this tells the compiler so: the fragments' last definition is now an
  // (empty) register-only instruction, not a pending load, so it adds no
  // load waits inside the loop
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    if constexpr (D <= 16) {
      asm volatile("" : "+v"(qf4[t]));
    } else {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) asm volatile("" : "+v"(qf[t][kc]));
    }
  }

  float m_run[NQT], l_run[NQT];
  AccK32 o[NQT][NDT], lsum[NQT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    m_run[t] = STALE ? kNoMaxStale : -INFINITY;
    l_run[t] = 0.f;
    lsum[t] = AccK32::zero();
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[t][dt] = AccK32::zero();
  }
  T8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = to_t<T>(1.f);

  // per-lane LDS operand offsets (elements)
  const int kread = c * STR + 8 * g;  // + (32p + 16h) * STR + 32kc
  const int kread16 = c * STR + 4 * g;
  const int vread = (16 * (g >> 1) + 8 * (g & 1) + 2 * (c >> 2)) * STR + 4 * (c & 3);  // + s*STR + 32p*STR + 16dt

  for (int kb = 0; kb < nblk; ++kb) {
    const int k0 = kb * BK;
    // this wave's copies of block kb have landed (later blocks may still be
    // in flight); after the barrier everyone's have, and everyone is done
    // with block kb-1, whose stage the next copy reuses
    // With NST - 2 later blocks issued, those may stay in flight (every wave
    // issues at least NI/NW copies per tile, so keeping that many per tile
    // outstanding never leaves one of block kb's); near the end fewer later
    // blocks exist and everything is waited for.
    if (NST == 2 || kb + NST - 2 >= nblk) wait_vmem();
    else wait_vmem_keep<2 * (NI / NW) * (NST - 2)>();
    block_barrier();
    if (kb + NST - 1 < nblk) dma_block((kb + NST - 1) % NST, k0 + (NST - 1) * BK);
    if (k0 >= kend_w) continue;  // wave-uniform: block is past this wave's rows

    const T* Ks = smem + (kb % NST) * 2 * TILE;
    const T* Vs = Ks + TILE;

    // ---- S^T = K Q^T
    // scores come from K = 16 products at d_h <= 16, K = 32 ones otherwise
    typedef std::conditional_t<(D <= 16), AccK16T<T>, AccK32> SAcc;
    SAcc s[NQT][NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      const int rbase = (32 * (kt >> 1) + 16 * (kt & 1)) * STR;
#pragma unroll
      for (int t = 0; t < NQT; ++t) s[t][kt] = SAcc::zero();
      if constexpr (D <= 16) {
        const T4 kf = *(const T4*)(Ks + rbase + kread16);
#pragma unroll
        for (int t = 0; t < NQT; ++t) s[t][kt] = mfma_k16(kf, qf4[t], s[t][kt]);
      }
    }
    if constexpr (D > 16) {
      // K fragments through inline asm, LAK reads ahead of their products
      // (compiler-visible reads were issued two at a time and waited for at
      // once, leaving the LDS latency exposed on every pair)
      constexpr int NKI = NKT * NKC;
      constexpr int LAK = NKI < 4 ? NKI : 4;
      const uint32_t kaddr = lds_addr(Ks + kread);
      u32x4 kfr[NKI];
      auto kissue = [&](auto I) {
        constexpr int i = decltype(I)::value;
        constexpr int kt = i / NKC, kc = i % NKC;
        kfr[i] = lds_read_b128_asm<((32 * (kt >> 1) + 16 * (kt & 1)) * STR + 32 * kc) * (int)sizeof(T)>(kaddr);
      };
      static_for<LAK>(kissue);
      static_for<NKI>([&](auto I) {
        constexpr int i = decltype(I)::value;
        constexpr int kt = i / NKC, kc = i % NKC;
        if constexpr (i + LAK < NKI) kissue(std::integral_constant<int, i + LAK>{});
        constexpr int last = i + LAK < NKI ? i + LAK : NKI - 1;
        lgkm_wait1<last - i>(kfr[i]);
        const T8 kf = __builtin_bit_cast(T8, kfr[i]);
#pragma unroll
        for (int t = 0; t < NQT; ++t) s[t][kt] = mfma_k32(kf, qf[t][kc], s[t][kt]);
      });
    }

    // ---- mask only blocks that straddle the key length or the diagonal:
    //      key k0 + 32p + 8g + 4h + i is visible to row r iff key < L and,
    //      when causal, key <= r
    if ((k0 + BK > L) || (causal && (k0 + BK - 1 > wq0))) {
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        const int row = wq0 + 16 * t + c;
        const int lim = (causal ? min(L - 1, row) : L - 1) - k0 - 8 * g;  // max visible offset
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int off = 32 * (kt >> 1) + 4 * (kt & 1) + i;
            s[t][kt][i] = off <= lim ? s[t][kt][i] : -INFINITY;
          }
      }
    }

    if constexpr (!STALE) {
      // ---- block row maxima; move the running max only when it is exceeded
      //      by more than the slack (wave-uniform decision)
      float mb[NQT];
      bool grow = false;
  #pragma unroll
      for (int t = 0; t < NQT; ++t) {
        float mx = s[t][0][0];
  #pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          mx = max3(mx, s[t][kt][0], s[t][kt][1]);
          mx = max3(mx, s[t][kt][2], s[t][kt][3]);
        }
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
          lsum[t] *= alpha;
  #pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[t][dt] *= alpha;
        }
      }
    }

    // ---- P = exp2(S c - m); O^T += V^T P^T, one key pair at a time. The
    //      V^T fragments are read LA column tiles ahead of their products.
    const uint32_t vaddr = lds_addr(Vs + vread);
    static_for<NKP>([&](auto P) {
      constexpr int p = decltype(P)::value;
      T8 pf[NQT], pl[NQT];
      // rounded probabilities of pair p for query tile t; returns the sum of
      // those rounded values (the weights the numerator uses)
      auto probs = [&](int t) {
        float ls = 0.f;
        if constexpr (kBf16) {
          float a[8];  // elements 0..3: key tile 2p, 4..7: key tile 2p + 1
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a[i] = fast_exp2(fmaf(s[t][2 * p][i], c_log2, -m_run[t]));
            a[4 + i] = fast_exp2(fmaf(s[t][2 * p + 1][i], c_log2, -m_run[t]));
          }
          // head + remainder, rounded two at a time
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t hi, lo;
            split2<T>(a[2 * w], a[2 * w + 1], hi, lo);
            set_word(pf[t], w, hi);
            set_word(pl[t], w, lo);
          }
          if constexpr (!SUM_MFMA && !STALE) {  // the rounded weights the numerator uses
#pragma unroll
            for (int i = 0; i < 8; ++i) ls += to_f(pf[t][i]) + to_f(pl[t][i]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a0 = fast_exp2(fmaf(s[t][2 * p][i], c_log2, -m_run[t]));
            const float a1 = fast_exp2(fmaf(s[t][2 * p + 1][i], c_log2, -m_run[t]));
            pf[t][i] = to_t<T>(a0);
            pf[t][4 + i] = to_t<T>(a1);
            if constexpr (!SUM_MFMA && !STALE) ls += to_f(pf[t][i]) + to_f(pf[t][4 + i]);
          }
        }
        return ls;
      };
      if constexpr (STALE) {
        // probabilities against the running max as it stands; the pair's
        // matrix-core row sums stay within kPairSumMax exactly when no fp16
        // probability overflowed (or was NaN). Otherwise move the max to the pair's maximum,
        // rescale, and redo the pair (its scores are still in registers).
        // row sums: every row of the ones product holds query c's sum, so
        // only element 0 is kept
        auto pair_sum = [&](int t) -> float {
          AccK32 a = mfma_k32(ones, pf[t], AccK32::zero());
          if constexpr (kBf16) a = mfma_k32(ones, pl[t], a);
          return a.vec()[0];
        };
        float ps[NQT];
        bool bad = false;
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
          probs(t);
          ps[t] = pair_sum(t);
        }
#pragma unroll
        for (int t = 0; t < NQT; ++t) bad |= !(ps[t] <= kPairSumMax);
        if (__any(bad)) {
#pragma unroll
          for (int t = 0; t < NQT; ++t) {
            float mx = max3(s[t][2 * p][0], s[t][2 * p][1], s[t][2 * p][2]);
            mx = max3(mx, s[t][2 * p][3], s[t][2 * p + 1][0]);
            mx = max3(mx, s[t][2 * p + 1][1], s[t][2 * p + 1][2]);
            mx = max2(mx, s[t][2 * p + 1][3]);
            const float m_new = max2(m_run[t], group_max(mx) * c_log2);
            const float alpha = fast_exp2(m_run[t] - m_new);
            m_run[t] = m_new;
            l_run[t] *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[t][dt] *= alpha;
            probs(t);
            ps[t] = pair_sum(t);
          }
        }
#pragma unroll
        for (int t = 0; t < NQT; ++t) l_run[t] += ps[t];
      } else {
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
          const float ls = probs(t);
          if constexpr (SUM_MFMA) {
            lsum[t] = mfma_k32(ones, pf[t], lsum[t]);
            if constexpr (kBf16) lsum[t] = mfma_k32(ones, pl[t], lsum[t]);
          } else {
            l_run[t] += ls;
          }
        }
      }
      constexpr int LA = NDT < 4 ? NDT : 4;
      i16x4 va[NDT], vb[NDT];
      auto issue = [&](auto J) {
        constexpr int j = decltype(J)::value;
        va[j] = lds_read_tr16_asm<(32 * p * STR + 16 * j) * (int)sizeof(T)>(vaddr);
        vb[j] = lds_read_tr16_asm<((32 * p + 1) * STR + 16 * j) * (int)sizeof(T)>(vaddr);
      };
      static_for<LA>(issue);
      static_for<NDT>([&](auto DT) {
        constexpr int dt = decltype(DT)::value;
        if constexpr (dt + LA < NDT) issue(std::integral_constant<int, dt + LA>{});
        constexpr int last = dt + LA < NDT ? dt + LA : NDT - 1;
        lgkm_wait<2 * (last - dt)>(va[dt], vb[dt]);  // reads issued after this tile's
        const T8 vf = __builtin_bit_cast(T8, __builtin_shufflevector(va[dt], vb[dt], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
          o[t][dt] = mfma_k32(vf, pf[t], o[t][dt]);
          if constexpr (kBf16) o[t][dt] = mfma_k32(vf, pl[t], o[t][dt]);
        }
      });
    });
  }

  // ---- epilogue: O / l rounded once to T; lse = ln(2) * (m + log2 l).
  //      Rows past S fall outside the store ranges and are dropped.
  if (wave_live) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      const float l = STALE ? l_run[t] : SUM_MFMA ? lsum[t][0] : group_sum(l_run[t]);
      const int row = wq0 + 16 * t + c;
      const float inv = 1.f / l;  // l >= 1: the running max's own key contributes 1
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        T4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = to_t<T>(o[t][dt][i] * inv);
        buf_store8(ov, ro, kHalf && g >= 2 ? kOutOfRange : row * RO + (16 * dt + 4 * g) * 2);
        if (O32p) buf_store16(o[t][dt].vec() * inv, r32, kHalf && g >= 2 ? kOutOfRange : (row * D + 16 * dt + 4 * g) * 4);
      }
      if (LSEp) buf_store4((m_run[t] + fast_log2(l)) * kLn2, rl, g == 0 ? row * 4 : kOutOfRange);
    }
  }
}

// ---------------------------------------------------------------------------
// Software-pipelined forward (fp16 / bf16, d_h >= 32). Same tiles, LDS layout
// and copies as attn_fwd_mfma; the loop differs in two ways.
//
// Probabilities of a key pair use the running max as it stands, without first
// taking the block's own maximum: p = exp2(s c - m) only has to be checked
// for size. The matrix-core row sum of the pair (ones times the rounded
// probabilities, which the denominator needs anyway) is checked against
// kPairSumMax = 2^21: a probability that overflowed fp16 (or is NaN) fails
// it, every sum of 32 finite fp16 probabilities passes, and for bf16 (whose
// probabilities only overflow at the fp32 range) it keeps every probability
// below 2^21, so O and l stay far from fp32 overflow. A pair that fails --
// the first visible keys of a row, or a row whose maximum jumped by more than
// about 16 (fp16) or 21 (bf16) log2 units -- recomputes its scores, moves the
// running max to their maximum, rescales O and l by exp2(m_old - m_new) and
// redoes its probabilities. Numerator and denominator always share one max,
// so the quotient is that of the online-softmax recurrence (devpost
// "gpu-transformer-optimization", section 2.1); rounded probabilities keep
// their relative precision at any magnitude below that bound.
//
// The loop is software pipelined: the step for key pair p of block kb issues,
// in one stretch of straight-line code,
//     the scores of pair p of block kb+1 (into the registers that pair p of
//     block kb releases),
//     the products O += V P of the previous pair (pair p-1 of block kb, or
//     the last pair of block kb-1), and
//     the exponentials of pair p of block kb,
// so the vector and transcendental work of the softmax has independent
// matrix-core work beside it. K of block kb+1 and V of block kb-1 are then
// resident with block kb, so the copies rotate over four LDS stages (block
// kb+2 in flight). All LDS reads go through inline asm with explicit
// lgkmcnt waits, counted over one stream of reads per step.
template <typename T, int D, int NQT, int NW, int BK, int MINB, bool SPLITP = false>
__global__ void __launch_bounds__(NW * 64, MINB)
attn_fwd_pipe(const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
              T* __restrict__ Op, float* __restrict__ LSEp, float* __restrict__ O32p,
              const int32_t* __restrict__ key_len, int H, int S, int causal, int n_qblk,
              float c_log2, Layout lay) {
  typedef typename Vec<T>::x8 T8;
  typedef typename Vec<T>::x4 T4;
  constexpr int NST = 4;
  constexpr int STR = D + 8;
  constexpr int SPR = D / 8 + 1;
  constexpr int SLOTS = BK * SPR;
  constexpr int NI = (SLOTS + 63) / 64;
  constexpr int TILE = NI * 64 * 8;
  constexpr int NIW = (NI + NW - 1) / NW;
  constexpr int NDT = D / 16;
  constexpr int NKP = BK / 32;
  constexpr int NKC = D / 32;
  constexpr int ES = (int)sizeof(T);
  constexpr int BQ = NW * NQT * 16;
  constexpr bool kBf16 = __is_same(T, bf16_t) || SPLITP;  // probabilities as head + remainder
  constexpr uint32_t kStage = 2 * TILE * ES;  // bytes per LDS stage (K tile, V tile)
  static_assert(BK % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(TILE * ES < 65536, "ds_read offsets within a tile");

  __shared__ __attribute__((aligned(16))) T smem[NST * 2 * TILE];  // [stage][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;

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
  const int kend = causal ? min(L, q_end) : L;
  const int nblk = (kend + BK - 1) / BK;
  const int wq0 = q_start + wave * NQT * 16;
  const bool wave_live = wq0 < S;
  const int kend_w = !wave_live ? 0 : (causal ? min(L, min(q_end, wq0 + NQT * 16)) : L);
  const int nblk_w = (kend_w + BK - 1) / BK;  // blocks this wave computes (wave-uniform)

  const rsrc_t ro = make_rsrc(Oh, span(S, RO));
  const rsrc_t rl = make_rsrc(LSEp + (int64_t)bh * S, (uint32_t)S * 4);
  // fp32 copy of the output (training forward): contiguous [B, H, S, D]
  const rsrc_t r32 = make_rsrc(O32p + (int64_t)bh * S * D, (uint32_t)S * D * 4);

  if (nblk == 0) {  // no visible key (L == 0): out = 0, lse = -inf
    if (wave_live) {
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        const int row = wq0 + 16 * t + c;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) buf_store8(zero_vec<T4>(), ro, row * RO + (16 * dt + 4 * g) * 2);
        if (O32p)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) buf_store16(f32x4{0.f, 0.f, 0.f, 0.f}, r32, (row * D + 16 * dt + 4 * g) * 4);
        if (LSEp) buf_store4(-INFINITY, rl, g == 0 ? row * 4 : kOutOfRange);
      }
    }
    return;
  }

  const rsrc_t rk = make_rsrc(Kh, span(kend, RK));
  const rsrc_t rv = make_rsrc(Vh, span(kend, RV));
  int koff[NIW], voff[NIW];
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    const int slot = (wave + i * NW) * 64 + lane;
    const int row = slot / SPR, j = slot - row * SPR;
    const bool live = slot < SLOTS && j < D / 8;
    const int base = 32 * (row >> 5);
    koff[i] = live ? (base + k_key_of_row(row & 31)) * RK + 16 * j : kOutOfRange;
    voff[i] = live ? (base + v_key_of_row(row & 31)) * RV + 16 * j : kOutOfRange;
  }
  auto dma_block = [&](int st, int k0) __attribute__((always_inline)) {
    T* Kst = smem + st * 2 * TILE;
    T* Vst = Kst + TILE;
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int inst = wave + i * NW;
      if (NI % NW == 0 || inst < NI) {  // wave-uniform
        dma16(rk, Kst + inst * 512, koff[i], k0 * RK);
        dma16(rv, Vst + inst * 512, voff[i], k0 * RV);
      }
    }
  };

  const rsrc_t rq = make_rsrc(Qh, span(S, RQ));
  T8 qf[NQT][NKC];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    const int row = wq0 + 16 * t + c;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) qf[t][kc] = buf_load16<T8>(rq, row * RQ + (32 * kc + 8 * g) * 2, 0);
  }
  asm volatile("" ::: "memory");
  dma_block(0, 0);
  dma_block(1, BK);
  wait_vmem_keep<2 * (NI / NW)>();  // Q and block 0 have landed
#pragma unroll
  for (int t = 0; t < NQT; ++t)
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) asm volatile("" : "+v"(qf[t][kc]));
  block_barrier();

  constexpr float kNoMax = -1.0e30f;  // finite: exp2(s c - kNoMax) overflows, exp2(-inf) stays 0
  float m_run[NQT], l_run[NQT];
  AccK32 o[NQT][NDT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    m_run[t] = kNoMax;
    l_run[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[t][dt] = AccK32::zero();
  }
  T8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = to_t<T>(1.f);
  const AccK32 zero4 = AccK32::zero();

  // LDS byte addresses of this lane's operands in stage 0
  const uint32_t kaddr0 = lds_addr(smem + c * STR + 8 * g);
  const uint32_t vaddr0 =
      lds_addr(smem + TILE + (16 * (g >> 1) + 8 * (g & 1) + 2 * (c >> 2)) * STR + 4 * (c & 3));

  // key k0 + 32p + 8g + 4h + i is visible to row r iff key < L and, when
  // causal, key <= r
  auto mask_pair = [&](int p, int k0, AccK32 (&sp)[NQT][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      const int row = wq0 + 16 * t + c;
      const int lim = (causal ? min(L - 1, row) : L - 1) - k0 - 32 * p - 8 * g;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) sp[t][hh][i] = 4 * hh + i <= lim ? sp[t][hh][i] : -INFINITY;
    }
  };
  // rounded probabilities of key tile hh of one pair for query tile t
  auto prob_unit = [&](int t, int hh, const AccK32 (&sp)[NQT][2], T8 (&pf)[NQT], T8 (&pl)[NQT])
      __attribute__((always_inline)) {
    if constexpr (kBf16) {
      // head + remainder, rounded two at a time: words 2hh, 2hh + 1
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = fast_exp2(fmaf(sp[t][hh][i], c_log2, -m_run[t]));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t hi, lo;
        split2<T>(a[2 * j], a[2 * j + 1], hi, lo);
        set_word(pf[t], 2 * hh + j, hi);
        set_word(pl[t], 2 * hh + j, lo);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) pf[t][4 * hh + i] = to_t<T>(fast_exp2(fmaf(sp[t][hh][i], c_log2, -m_run[t])));
    }
  };
  // row sum of one pair for query tile t on the matrix cores
  auto pair_sum = [&](int t, const T8 (&pf)[NQT], const T8 (&pl)[NQT]) __attribute__((always_inline)) {
    AccK32 a = mfma_k32(ones, pf[t], zero4);
    if constexpr (kBf16) a = mfma_k32(ones, pl[t], a);
    return a;
  };
  // true if any sum exceeds kPairSumMax or is NaN; ps takes query c's sum
  // (every row of the product holds it)
  auto check = [&](const AccK32 (&psv)[NQT], float (&ps)[NQT]) __attribute__((always_inline)) {
    bool bad = false;
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      ps[t] = psv[t][0];
      bad |= !(ps[t] <= kPairSumMax);
    }
    return bad;
  };
  auto no_work = [](auto) __attribute__((always_inline)) {};

  // One pipeline step's LDS stream: NVI items of V^T (two transposed reads
  // each; products O += V P with probabilities pp, pl of key pair PV) then
  // NKI items of K (one read each; scores of key pair PK into sp, key tile
  // j / NKC, depth chunk j % NKC). LA items are in flight ahead of their
  // products; LDS operations complete in issue order, so each item waits for
  // all but the reads issued after it. work(i) runs before item i's
  // products, and a scheduling fence closes each item, so the vector work
  // sits between the matrix-core products instead of in one run.
  auto stream = [&](auto PV, auto NVI_, auto PK, auto NKI_, uint32_t va_base, uint32_t ka_base,
                    const T8 (&pp)[NQT], const T8 (&pl)[NQT], AccK32 (&sp)[NQT][2], auto&& work)
      __attribute__((always_inline)) {
    constexpr int pv = decltype(PV)::value, pk = decltype(PK)::value;
    constexpr int NVI = decltype(NVI_)::value, NKI = decltype(NKI_)::value;
    constexpr int NIT = NVI + NKI;
    constexpr int LA = NIT < 4 ? NIT : 4;
    i16x4 va[NVI > 0 ? NVI : 1], vb[NVI > 0 ? NVI : 1];
    u32x4 kf[NKI > 0 ? NKI : 1];
    auto issue = [&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if constexpr (i < NVI) {
        va[i] = lds_read_tr16_asm<(32 * pv * STR + 16 * i) * ES>(va_base);
        vb[i] = lds_read_tr16_asm<((32 * pv + 1) * STR + 16 * i) * ES>(va_base);
      } else {
        constexpr int j = i - NVI;
        kf[j] = lds_read_b128_asm<((32 * pk + 16 * (j / NKC)) * STR + 32 * (j % NKC)) * ES>(ka_base);
      }
    };
    static_for<LA>(issue);
    static_for<NIT>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if constexpr (i + LA < NIT) issue(std::integral_constant<int, i + LA>{});
      work(I);
      constexpr int last = i + LA < NIT ? i + LA : NIT - 1;
      // LDS operations issued after item i: 2 per V item, 1 per K item
      constexpr int nv_after = (last < NVI ? last : NVI - 1) - (i < NVI ? i : NVI - 1);
      constexpr int nk_after = (last >= NVI ? last - NVI + 1 : 0) - (i >= NVI ? i - NVI + 1 : 0);
      constexpr int after = 2 * (nv_after > 0 ? nv_after : 0) + nk_after;
      static_assert(after >= 0 && after < 16, "lgkmcnt range");
      if constexpr (i < NVI) {
        lgkm_wait<after>(va[i], vb[i]);
        const T8 vf = __builtin_bit_cast(T8, __builtin_shufflevector(va[i], vb[i], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
          o[t][i] = mfma_k32(vf, pp[t], o[t][i]);
          if constexpr (kBf16) o[t][i] = mfma_k32(vf, pl[t], o[t][i]);
        }
      } else {
        constexpr int j = i - NVI;
        lgkm_wait1<after>(kf[j]);
        const T8 k8 = __builtin_bit_cast(T8, kf[j]);
#pragma unroll
        for (int t = 0; t < NQT; ++t)
          sp[t][j / NKC] = mfma_k32(k8, qf[t][j % NKC], j % NKC == 0 ? zero4 : sp[t][j / NKC]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto scores_pair = [&](auto P, uint32_t ka, AccK32 (&sp)[NQT][2]) __attribute__((always_inline)) {
    T8 dummy[NQT];
    stream(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, P,
           std::integral_constant<int, 2 * NKC>{}, 0u, ka, dummy, dummy, sp, no_work);
  };
  // a pair whose sums are not finite: recompute its scores, move the running
  // max to their maximum, rescale O and l, and redo its probabilities. One
  // query tile at a time, each K fragment read and waited for on its own, so
  // this rare path adds few live registers to the loop.
  auto redo = [&](auto P, uint32_t ka, int k0, bool edge, T8 (&pf)[NQT], T8 (&pl)[NQT], float (&ps)[NQT])
      __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    static_for<NQT>([&](auto TT) __attribute__((always_inline)) {
      constexpr int t = decltype(TT)::value;
      AccK32 sr[NQT][2];  // only row t is used
      static_for<2 * NKC>([&](auto J) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value;
        u32x4 kf = lds_read_b128_asm<((32 * p + 16 * (j / NKC)) * STR + 32 * (j % NKC)) * ES>(ka);
        lgkm_wait1<0>(kf);
        sr[t][j / NKC] = mfma_k32(__builtin_bit_cast(T8, kf), qf[t][j % NKC], j % NKC == 0 ? zero4 : sr[t][j / NKC]);
      });
      if (edge) {
        const int row = wq0 + 16 * t + c;
        const int lim = (causal ? min(L - 1, row) : L - 1) - k0 - 32 * p - 8 * g;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 4; ++i) sr[t][hh][i] = 4 * hh + i <= lim ? sr[t][hh][i] : -INFINITY;
      }
      float mx = max3(sr[t][0][0], sr[t][0][1], sr[t][0][2]);
      mx = max3(mx, sr[t][0][3], sr[t][1][0]);
      mx = max3(mx, sr[t][1][1], sr[t][1][2]);
      mx = max2(mx, sr[t][1][3]);
      const float m_new = max2(m_run[t], group_max(mx) * c_log2);
      const float alpha = fast_exp2(m_run[t] - m_new);
      m_run[t] = m_new;
      l_run[t] *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[t][dt] *= alpha;
      prob_unit(t, 0, sr, pf, pl);
      prob_unit(t, 1, sr, pf, pl);
      ps[t] = pair_sum(t, pf, pl)[0];
    });
  };

  AccK32 sc[NKP][NQT][2];       // scores of the current block, by key pair
  T8 pprev[NQT], plprev[NQT];  // probabilities of the previous pair
  if (nblk_w > 0) static_for<NKP>([&](auto P) { scores_pair(P, kaddr0, sc[decltype(P)::value]); });

  // one block: FIRST skips the products of the (nonexistent) previous pair
  auto block = [&](auto FIRST, int kb) __attribute__((always_inline)) {
    constexpr bool first = decltype(FIRST)::value;
    const int k0 = kb * BK;
    const uint32_t kcur = kaddr0 + (uint32_t)(kb % NST) * kStage;
    const uint32_t knext = kaddr0 + (uint32_t)((kb + 1) % NST) * kStage;
    const uint32_t vcur = vaddr0 + (uint32_t)(kb % NST) * kStage;
    const uint32_t vprev = vaddr0 + (uint32_t)((kb + NST - 1) % NST) * kStage;
    // only blocks that straddle the key length or the diagonal are masked
    const bool edge = (k0 + BK > L) || (causal && (k0 + BK - 1 > wq0));
    if (edge) static_for<NKP>([&](auto P) { mask_pair(decltype(P)::value, k0, sc[decltype(P)::value]); });
    static_for<NKP>([&](auto P) __attribute__((always_inline)) {
      constexpr int p = decltype(P)::value;
      constexpr int nvi = (first && p == 0) ? 0 : NDT;
      constexpr int NS = nvi + NKC + 1;  // slots whose work may still read the old scores
      constexpr int NU = 2 * NQT;        // work units (t, key tile), key tile 0 first
      T8 pf[NQT], pl[NQT];
      AccK32 psv[NQT];
      // unit u = (t, hh) reads key tile hh of the old scores, which the K
      // items of key tile hh overwrite (the first at slot nvi + NKC * hh):
      // tile-0 units go in slots <= nvi, tile-1 units in slots <= nvi + NKC
      auto work = [&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        static_for<NU>([&](auto U) __attribute__((always_inline)) {
          constexpr int u = decltype(U)::value;
          constexpr int t = u % NQT, hh = u / NQT;
          constexpr int slot = nvi == 0 ? 0 : u * NS / NU;
          static_assert(slot <= nvi + NKC * hh, "a unit must read its scores before they are overwritten");
          if constexpr (slot == i) {
            prob_unit(t, hh, sc[p], pf, pl);
            if constexpr (hh == 1) psv[t] = pair_sum(t, pf, pl);
          }
        });
      };
      // products of the previous pair, then the scores of pair p of block
      // kb+1 (past the wave's last block: unused) into the registers the
      // units release
      stream(std::integral_constant<int, p == 0 ? NKP - 1 : p - 1>{}, std::integral_constant<int, nvi>{},
             P, std::integral_constant<int, 2 * NKC>{}, p == 0 ? vprev : vcur, knext, pprev, plprev, sc[p],
             work);
      float ps[NQT];
      if (__any(check(psv, ps))) redo(P, kcur, k0, edge, pf, pl, ps);
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        l_run[t] += ps[t];
        pprev[t] = pf[t];
        if constexpr (kBf16) plprev[t] = pl[t];
      }
    });
    if (kb == nblk_w - 1) {  // the wave's last block: products of its last pair now
      AccK32 unused[NQT][2];
      stream(std::integral_constant<int, NKP - 1>{}, std::integral_constant<int, NDT>{},
             std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, vcur, 0u, pprev, plprev, unused,
             no_work);
    }
  };

  // block kb+1's copies (issued one block ago) have landed; after the
  // barrier everyone's have, and everyone is done with block kb-2, whose
  // stage the copy of block kb+2 reuses
  wait_vmem();
  block_barrier();
  if (2 < nblk) dma_block(2, 2 * BK);
  if (nblk_w > 0) block(std::true_type{}, 0);
  for (int kb = 1; kb < nblk; ++kb) {
    wait_vmem();
    block_barrier();
    if (kb + 2 < nblk) dma_block((kb + 2) % NST, (kb + 2) * BK);
    if (kb >= nblk_w) continue;  // wave-uniform: block is past this wave's rows
    block(std::false_type{}, kb);
  }

  // ---- epilogue: O / l rounded once to T; lse = ln(2) * (m + log2 l)
  if (wave_live) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      const float l = l_run[t];
      const int row = wq0 + 16 * t + c;
      const float inv = 1.f / l;  // l >= 1: the key that set the running max contributes 1
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        T4 ov;
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = to_t<T>(o[t][dt][i] * inv);
        buf_store8(ov, ro, row * RO + (16 * dt + 4 * g) * 2);
        if (O32p) buf_store16(o[t][dt].vec() * inv, r32, (row * D + 16 * dt + 4 * g) * 4);
      }
      if (LSEp) buf_store4((m_run[t] + fast_log2(l)) * kLn2, rl, g == 0 ? row * 4 : kOutOfRange);
    }
  }
}

template <typename T, int D, int NQT, int NW, int BK, bool SM, int NST = 2, bool STALE = false,
          bool SPLITP = false>
static hipError_t launch_one(const AttnParams& p, hipStream_t s) {
  constexpr int BQ = NW * NQT * 16;
  const int n_qblk = (p.S + BQ - 1) / BQ;
  const int64_t n_wg = (int64_t)p.B * p.H * n_qblk;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_mfma<T, D, NQT, NW, BK, SM, NST, STALE, SPLITP>), dim3((unsigned)n_wg), dim3(NW * 64), 0, s,
                     (const T*)p.q, (const T*)p.k, (const T*)p.v, (T*)p.out, p.lse, p.out32,
                     p.key_len, p.H, p.S, p.causal, n_qblk, p.c_log2, p.lay);
  return hipGetLastError();
}

template <typename T, int D, int NQT, int NW, int BK, int MINB, bool SPLITP = false>
static hipError_t launch_pipe(const AttnParams& p, hipStream_t s) {
  constexpr int BQ = NW * NQT * 16;
  const int n_qblk = (p.S + BQ - 1) / BQ;
  const int64_t n_wg = (int64_t)p.B * p.H * n_qblk;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_pipe<T, D, NQT, NW, BK, MINB, SPLITP>), dim3((unsigned)n_wg), dim3(NW * 64), 0, s,
                     (const T*)p.q, (const T*)p.k, (const T*)p.v, (T*)p.out, p.lse, p.out32,
                     p.key_len, p.H, p.S, p.causal, n_qblk, p.c_log2, p.lay);
  return hipGetLastError();
}

// Tile shapes (NQT query tiles per wave, NW waves, BK keys per block, row sum
// on the matrix cores) per head size.
template <typename T>
constexpr bool kBf16T = __is_same(T, bf16_t);

template <typename T>
static hipError_t launch_general(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 8: return launch_one<T, 8, 2, 4, 64, false>(p, s);
    case 16: return launch_one<T, 16, 2, 4, 64, false>(p, s);
    case 32: return launch_one<T, 32, 2, 4, 64, false>(p, s);
    case 64:
      // 4 waves of 64 query rows, two workgroups per CU; fp16 runs the
      // pipelined loop (bf16's head + remainder probabilities do not fit its
      // registers at this tile)
      if constexpr (kBf16T<T>) return launch_one<T, 64, 4, 4, 64, true>(p, s);
      else return launch_pipe<T, 64, 4, 4, 64, 2>(p, s);
    case 128:  // pipelined, 8 waves of 32 query rows
      return launch_pipe<T, 128, 2, 8, 64, 1>(p, s);
    case 256:  // fp16 takes probabilities against the running max with the
               // overflow check (bf16 spills with it)
      if constexpr (kBf16T<T>) return launch_one<T, 256, 2, 8, 32, true>(p, s);
      else return launch_one<T, 256, 2, 8, 32, true, 2, true>(p, s);
  }
  return hipErrorInvalidValue;
}

// 16-row query tiles, four waves sharing each K / V block (64 rows per
// workgroup), row sums on the matrix cores: for problems with too few rows
// to fill the chip with larger tiles, and (d_h <= 64) for causal problems,
// whose triangle the small tiles balance better.
template <typename T>
static hipError_t launch_small(const AttnParams& p, hipStream_t s) {
  switch (p.D) {
    case 8: return launch_one<T, 8, 1, 1, 64, false>(p, s);
    case 16: return launch_one<T, 16, 1, 4, 64, true>(p, s);
    case 32: return launch_one<T, 32, 1, 4, 64, true>(p, s);
    case 64: return launch_one<T, 64, 1, 4, 64, true>(p, s);
    case 128: return launch_one<T, 128, 1, 4, 64, true>(p, s);
    case 256: return launch_one<T, 256, 1, 4, 32, true>(p, s);
  }
  return hipErrorInvalidValue;
}

// The training forward's fp16 kernels: probabilities as head + remainder in
// the value product (the tiles bf16 uses, which carry the same pairs), so
// that the fp32 output the backward's row term comes from is exact to fp32
// rounding for both dtypes. bf16 runs its ordinary kernels.
static hipError_t launch_general_split(const AttnParams& p, hipStream_t s) {
  typedef f16_t T;
  switch (p.D) {
    case 8: return launch_one<T, 8, 2, 4, 64, false, 2, false, true>(p, s);
    case 16: return launch_one<T, 16, 2, 4, 64, false, 2, false, true>(p, s);
    case 32: return launch_one<T, 32, 2, 4, 64, false, 2, false, true>(p, s);
    case 64: return launch_one<T, 64, 4, 4, 64, true, 2, false, true>(p, s);
    case 128: return launch_pipe<T, 128, 2, 8, 64, 1, true>(p, s);
    case 256: return launch_one<T, 256, 2, 8, 32, true, 2, false, true>(p, s);
  }
  return hipErrorInvalidValue;
}
static hipError_t launch_small_split(const AttnParams& p, hipStream_t s) {
  typedef f16_t T;
  switch (p.D) {
    case 8: return launch_one<T, 8, 1, 1, 64, false, 2, false, true>(p, s);
    case 16: return launch_one<T, 16, 1, 4, 64, true, 2, false, true>(p, s);
    case 32: return launch_one<T, 32, 1, 4, 64, true, 2, false, true>(p, s);
    case 64: return launch_one<T, 64, 1, 4, 64, true, 2, false, true>(p, s);
    case 128: return launch_one<T, 128, 1, 4, 64, true, 2, false, true>(p, s);
    case 256: return launch_one<T, 256, 1, 4, 32, true, 2, false, true>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mfma_train(const AttnParams& p, hipStream_t s) {
  if (p.dtype == 1) return launch_general_split(p, s);
  if (p.dtype == 2) return launch_general<bf16_t>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_mfma_small_train(const AttnParams& p, hipStream_t s) {
  if (p.dtype == 1) return launch_small_split(p, s);
  if (p.dtype == 2) return launch_small<bf16_t>(p, s);
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
