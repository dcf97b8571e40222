// Attention backward on the gfx950 matrix cores (fp16 / bf16 inputs, fp32
// accumulation): dQ, dK, dV of sum(dO * O) for O = softmax(Q K^T / sqrt(d_h)
// + mask) V.
//
// Two kinds of work, as in the fused backward of rustingstudio
// "brain/docs/baseline" ("Fused attention"): the query gradient is complete
// inside a query tile and the key / value gradients inside a key tile, so
//   * the dq body walks key blocks for a block of query rows, and
//   * the dkv body walks query blocks for a block of key rows,
// and both rebuild the probabilities from the stored log-sum-exp instead of
// keeping them: P = exp(S / sqrt(d_h) - lse). With dP = dO V^T and the row
// term D = rowsum(dO * O) (equal to rowsum(P * dP) since O = P V),
//   dS = P * (dP - D),  dQ = dS K / sqrt(d_h),  dK = dS^T Q / sqrt(d_h),
//   dV = P^T dO.
// D goes through the caller's workspace: a first pass of the dq body
// (attn_bwd_dq) accumulates rowsum(P * dP) in fp32 and writes it, then one
// launch (attn_bwd_both) runs the dq body proper and the dkv body, both
// reading it. The forward's rounded output is not used for D.
//
// Products are formed transposed where that puts the contraction index in
// the operand registers directly (lane = 16g + c):
//   dq : S^T = K Q^T, dP^T = V dO^T (A operand: K / V rows from LDS,
//        B operand: Q / dO fragments in registers), dQ^T += K^T dS^T
//        (A operand: K read transposed from LDS, B operand: dS^T as the
//        S^T result tiles leave it).
//   dkv: S = Q K^T, dP = dO V^T (A: Q / dO rows from LDS, B: K / V fragments
//        in registers), dV^T += dO^T P and dK^T += Q^T dS (A: dO / Q read
//        transposed from LDS, B: P / dS as the result tiles leave them).
// P and dS are matrix-core operands in the input dtype, each split into a
// head and a remainder (two products). dP grows with d_h and the value
// scale, and where dQ or dK cancels to a small value a single fp16 rounding
// of dS (half an ulp, 2^-8, at |dS| near 8) already exceeds the accuracy
// rule; where the softmax is peaked, dV sums few probabilities near 1, and
// their single fp16 rounding (2^-12 relative) does too. bf16 needs both
// splits at any scale.
//
// A 32-row pair of an LDS operand block is read both as 16-row tiles (one
// 128-bit row read per lane) and transposed (ds_read_b64_tr_b16 over 4 rows
// per lane group). From d_h = 32 on, rows keep their order and each padded
// row holds d_h + 16 elements: the LDS bank-conflict counters read zero for
// both kinds of read in that layout (with d_h + 8, the row reads take two
// passes). At d_h = 16 row c of tile h of the pair is stored at LDS row
// 16h + 2(c % 8) + c / 8 of the pair, with d_h + 8 per row. In the
// contraction over a pair, k-slot 8g + 4h + i of lane group g stands for row
// 16h + 4g + i of the pair, in both operands.
#include <type_traits>

#include "attn_common.h"
#include "launch.h"

namespace mha {

// d_h = 16: LDS row (within a 32-row pair) of pair row x, and the pair row
// stored at LDS row r.
__device__ __forceinline__ int bwd_lds_row(int x) {
  const int c = x & 15;
  return (x & 16) + 2 * (c & 7) + (c >> 3);
}
__device__ __forceinline__ int bwd_row_at(int r) {
  const int cc = r & 15;
  return (r & 16) + 8 * (cc & 1) + (cc >> 1);
}

// Per-lane DMA slots of an operand block of NR rows x D columns in the
// padded LDS layout above: fills the source byte offsets (relative to the
// block's first row; kOutOfRange for pad slots) of this wave's slots.
template <typename T, int D, int NR, int NW>
struct BwdTile {
  static constexpr int STR = D >= 32 ? D + 16 : D + 8;
  static constexpr int SPR = STR / 8;
  static constexpr int SLOTS = NR * SPR;
  static constexpr int NI = (SLOTS + 63) / 64;
  static constexpr int ELEMS = NI * 64 * 8;  // whole DMA instructions
  static constexpr int NIW = (NI + NW - 1) / NW;
  static constexpr int RB = D * (int)sizeof(T);
  __device__ static void offsets(int wave, int lane, int (&off)[NIW]) {
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int slot = (wave + i * NW) * 64 + lane;
      const int row = slot / SPR, j = slot - row * SPR;
      const bool live = slot < SLOTS && j < D / 8;
      off[i] = live ? (D >= 32 ? row : 32 * (row >> 5) + bwd_row_at(row & 31)) * RB + 16 * j : kOutOfRange;
    }
  }
  __device__ static void copy(rsrc_t r, T* dst, const int (&off)[NIW], int wave, int soff) {
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int inst = wave + i * NW;
      if (NI % NW == 0 || inst < NI) dma16(r, dst + inst * 512, off[i], soff);
    }
  }
};

// ---------------------------------------------------------------- dq kernel
// MODE kRowPass: no dQ; D = rowsum(P * dP) / rowsum(P) accumulated over every
//   visible key in fp32 and written to the workspace. This equals dO . O of
//   the exact output; dO . O of the output rounded to fp16 or bf16 would put
//   an error of D times sum_j P_ij k_j into dQ, which rows whose softmax is
//   peaked or that see few keys do not average away (fp16, d_h 128, causal,
//   scores of a few tens: dQ off by three times the accuracy rule). The
//   division by rowsum(P) does the same for an lse that is off by a rounding.
// MODE kRowRead: dQ with D read from the workspace.
constexpr int kRowPass = 1, kRowRead = 2;

// The kernel bodies take their block index, the number of blocks of their
// kind and their LDS, so that one launch can run both kinds (below).
template <typename T, int D, int BK, int NW>
struct DqLds {
  static constexpr int BYTES = 2 * 2 * BwdTile<T, D, BK, NW>::ELEMS * (int)sizeof(T);
};

template <typename T, int D, int NQT, int NW, int BK, int MODE>
__device__ __forceinline__ void bwd_dq_body(
    uint32_t bh, int qb, T* __restrict__ smem, const T* __restrict__ Qp,
    const T* __restrict__ Kp, const T* __restrict__ Vp,
    const T* __restrict__ dOp, const float* __restrict__ LSEp, T* __restrict__ dQp,
    float* __restrict__ Dp, const int32_t* __restrict__ key_len, int H, int S, int causal,
    int n_qblk, float c_log2, float scale, int group) {
  typedef typename Vec<T>::x8 T8;
  typedef typename Vec<T>::x4 T4;
  typedef BwdTile<T, D, BK, NW> Tile;
  constexpr int STR = Tile::STR;
  constexpr int NDT = D / 16;
  constexpr int NKT = BK / 16;
  constexpr int NKP = BK / 32;
  constexpr int NKC = D >= 32 ? D / 32 : 1;
  constexpr int RB = D * (int)sizeof(T);
  constexpr int BQ = NW * NQT * 16;
  static_assert(BK % 32 == 0 && D % 16 == 0, "tile shape");

  // smem: [stage][K, V] tiles

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;

  // (batch, head) bh over B * H, query block qb
  const int b = (int)(bh / (uint32_t)H);
  const int L = clamp_len(key_len, b, S);
  const int64_t head = (int64_t)bh * S * D;
  // key / value head of this query head (grouped-query attention)
  const int hk = (int)(bh - (uint32_t)b * (uint32_t)H) / group;
  const int64_t head_kv = ((int64_t)b * (H / group) + hk) * S * D;
  const int q_start = qb * BQ;
  const int q_end = min(S, q_start + BQ);
  const int kend = causal ? min(L, q_end) : L;
  const int nblk = (kend + BK - 1) / BK;
  const int wq0 = q_start + wave * NQT * 16;
  const bool wave_live = wq0 < S;
  const int kend_w = !wave_live ? 0 : (causal ? min(L, min(q_end, wq0 + NQT * 16)) : L);

  const rsrc_t rq = make_rsrc(Qp + head, (uint32_t)S * RB);
  const rsrc_t rdo = make_rsrc(dOp + head, (uint32_t)S * RB);
  const rsrc_t rdq = make_rsrc(dQp + head, (uint32_t)S * RB);
  const rsrc_t rl = make_rsrc(LSEp + (int64_t)bh * S, (uint32_t)S * 4);
  const rsrc_t rd = make_rsrc(Dp + (int64_t)bh * S, (uint32_t)S * 4);

  // ---- Q and dO fragments (B operands, query column c), and the row term
  //      D of each of this wave's rows (read, or zeroed for the row pass)
  T8 qf[NQT][NKC], dof[NQT][NKC];
  T4 qf4[NQT], dof4[NQT];
  float drow[NQT], prow[NQT], nlse2[NQT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    const int row = wq0 + 16 * t + c;
    if constexpr (D == 16) {
      qf4[t] = buf_load8<T4>(rq, (row * D + 4 * g) * 2, 0);
      dof4[t] = buf_load8<T4>(rdo, (row * D + 4 * g) * 2, 0);
    } else {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        qf[t][kc] = buf_load16<T8>(rq, (row * D + 32 * kc + 8 * g) * 2, 0);
        dof[t][kc] = buf_load16<T8>(rdo, (row * D + 32 * kc + 8 * g) * 2, 0);
      }
    }
    if constexpr (MODE == kRowRead) {
      drow[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, row * 4, 0, 0));
    } else {
      drow[t] = 0.f;  // accumulates rowsum(P * dP) of this lane's keys
      prow[t] = 0.f;  // and rowsum(P)
    }
    const float lse = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, row * 4, 0, 0));
    nlse2[t] = -lse * kLog2e;
  }
  wait_vmem();

  AccK32 acc_dq[NQT][NDT];
#pragma unroll
  for (int t = 0; t < NQT; ++t)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc_dq[t][dt] = AccK32::zero();
  // dP^T accumulators start from -D of the lane's row (its query column),
  // so the products leave dP - D; the row pass accumulates from zero
  typedef std::conditional_t<D == 16, AccK16T<T>, AccK32> SAcc;  // K = 16 products at d_h = 16
  SAcc dp0[NQT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) dp0[t] = SAcc::fill(MODE == kRowRead ? -drow[t] : 0.f);

  if (nblk > 0) {
    const rsrc_t rk = make_rsrc(Kp + head_kv, (uint32_t)kend * RB);
    const rsrc_t rv = make_rsrc(Vp + head_kv, (uint32_t)kend * RB);
    int off[Tile::NIW];
    Tile::offsets(wave, lane, off);
    auto dma_block = [&](int st, int k0) {
      T* Kst = smem + st * 2 * Tile::ELEMS;
      Tile::copy(rk, Kst, off, wave, k0 * RB);
      Tile::copy(rv, Kst + Tile::ELEMS, off, wave, k0 * RB);
    };
    dma_block(0, 0);

    // per-lane LDS offsets (elements): tile row c of a pair (row reads), and
    // the transposed read of lane group g (rows 4g + c/4, column 4(c%4))
    const int rrow = (D >= 32 ? c : bwd_lds_row(c)) * STR;
    const int trow = (D >= 32 ? 4 * g + (c >> 2) : bwd_lds_row(4 * g + (c >> 2))) * STR + 4 * (c & 3);

    for (int kb = 0; kb < nblk; ++kb) {
      const int k0 = kb * BK;
      wait_vmem();
      block_barrier();
      if (kb + 1 < nblk) dma_block((kb + 1) & 1, k0 + BK);
      if (k0 >= kend_w) continue;  // wave-uniform

      const T* Ks = smem + (kb & 1) * 2 * Tile::ELEMS;
      const T* Vs = Ks + Tile::ELEMS;

      // S^T = K Q^T and dP^T - D = V dO^T - D; key 16kt + 4g + i of the
      // block in register i of lane (g, c)
      SAcc s[NQT][NKT], dp[NQT][NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const int rb = 16 * kt * STR + rrow;
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
          s[t][kt] = SAcc::zero();
          dp[t][kt] = dp0[t];
        }
        if constexpr (D == 16) {
          const T4 kf = *(const T4*)(Ks + rb + 4 * g);
          const T4 vf = *(const T4*)(Vs + rb + 4 * g);
#pragma unroll
          for (int t = 0; t < NQT; ++t) {
            s[t][kt] = mfma_k16(kf, qf4[t], s[t][kt]);
            dp[t][kt] = mfma_k16(vf, dof4[t], dp[t][kt]);
          }
        } else {
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc) {
            const T8 kf = *(const T8*)(Ks + rb + 32 * kc + 8 * g);
            const T8 vf = *(const T8*)(Vs + rb + 32 * kc + 8 * g);
#pragma unroll
            for (int t = 0; t < NQT; ++t) {
              s[t][kt] = mfma_k32(kf, qf[t][kc], s[t][kt]);
              dp[t][kt] = mfma_k32(vf, dof[t][kc], dp[t][kt]);
            }
          }
        }
      }

      // P = exp(S / sqrt(d) - lse) (0 for hidden pairs), dS = P (dP - D)
      // (dp already holds dP - D in the row read mode)
      const bool edge = (k0 + BK > L) || (causal && (k0 + BK - 1 > wq0));
      T8 dsf[NQT][NKP], dsl[NQT][NKP];
#pragma unroll
      for (int t = 0; t < NQT; ++t)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) s[t][kt][i] = fast_exp2(fmaf(s[t][kt][i], c_log2, nlse2[t]));
      // hidden pairs get P = 0, only in blocks that reach a boundary (the
      // empty asm keeps this a branch rather than a select on every element)
      if (edge) {
        asm volatile("");
#pragma unroll
        for (int t = 0; t < NQT; ++t) {
          const int row = wq0 + 16 * t + c;
          const int lim = (causal ? min(L - 1, row) : L - 1) - k0 - 4 * g;  // max visible key offset
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * kt + i > lim) s[t][kt][i] = 0.f;
        }
      }
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          if constexpr (MODE == kRowPass) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              drow[t] = fmaf(s[t][kt][i], dp[t][kt][i], drow[t]);
              prow[t] += s[t][kt][i];
            }
            continue;
          }
          // dS rounded two at a time as head + remainder: words
          // 2 (kt % 2), 2 (kt % 2) + 1 of the pair's operand
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int w = 2 * (kt & 1) + j;
            uint32_t dh, dlo;
            split2_prod<T>(s[t][kt][2 * j], dp[t][kt][2 * j], s[t][kt][2 * j + 1], dp[t][kt][2 * j + 1],
                           dh, dlo);
            set_word(dsf[t][kt >> 1], w, dh);
            set_word(dsl[t][kt >> 1], w, dlo);
          }
        }
      }

      // dQ^T += K^T dS^T, one key pair at a time
      if constexpr (MODE == kRowPass) continue;
      // (transposed reads through inline asm, LA column tiles ahead, so the
      // compiler does not make them wait for the next block's copy)
#pragma unroll
      for (int p = 0; p < NKP; ++p) {
        const uint32_t ka = lds_addr(Ks + 32 * p * STR + trow);
        constexpr int LA = NDT < 4 ? NDT : 4;
        i16x4 a0[NDT], a1[NDT];
        auto issue = [&](auto J) {
          constexpr int j = decltype(J)::value;
          a0[j] = lds_read_tr16_asm<16 * j * (int)sizeof(T)>(ka);
          a1[j] = lds_read_tr16_asm<(16 * STR + 16 * j) * (int)sizeof(T)>(ka);
        };
        static_for<LA>(issue);
        static_for<NDT>([&](auto DT) {
          constexpr int dt = decltype(DT)::value;
          if constexpr (dt + LA < NDT) issue(std::integral_constant<int, dt + LA>{});
          constexpr int last = dt + LA < NDT ? dt + LA : NDT - 1;
          lgkm_wait<2 * (last - dt)>(a0[dt], a1[dt]);
          const T8 kf = __builtin_bit_cast(T8, __builtin_shufflevector(a0[dt], a1[dt], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int t = 0; t < NQT; ++t) {
            acc_dq[t][dt] = mfma_k32(kf, dsf[t][p], acc_dq[t][dt]);
            acc_dq[t][dt] = mfma_k32(kf, dsl[t][p], acc_dq[t][dt]);
          }
        });
      }
    }
  }

  if constexpr (MODE == kRowPass) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      // D of the row's probabilities renormalised to sum 1: the stored lse
      // may come from a forward whose row sums were taken over rounded
      // probabilities, and then the rebuilt P sums to 1 only within that
      // rounding (about 1e-4 for fp16). With D / rowsum(P) the rows of
      // dS = P (dP - D) still sum to exactly zero, as the softmax's do, so no
      // term D * sum_j P_ij k_j is left uncancelled in dQ; what remains is a
      // common factor rowsum(P) on the row's dS.
      const float dsum = group_sum(drow[t]);
      const float psum = group_sum(prow[t]);
      const float dn = psum > 0.f ? dsum / psum : 0.f;  // no visible key: P = 0, D unused
      if (wave_live) buf_store4(dn, rd, g == 0 ? (wq0 + 16 * t + c) * 4 : kOutOfRange);
    }
    return;
  }

  // ---- dQ = dQ^T^T / sqrt(d): row c, columns 16dt + 4g .. 16dt + 4g + 3
  if (wave_live) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      const int row = wq0 + 16 * t + c;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        T4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = to_t<T>(acc_dq[t][dt][i] * scale);
        buf_store8(v, rdq, (row * D + 16 * dt + 4 * g) * 2);
      }
    }
  }
}

// --------------------------------------------------------------- dkv kernel
template <typename T, int D, int BQb, int NW>
struct DkvLds {
  static constexpr int TILE_BYTES = 2 * 2 * BwdTile<T, D, BQb, NW>::ELEMS * (int)sizeof(T);
  static constexpr int BYTES = TILE_BYTES + 2 * 2 * 64 * 4;  // + [stage][lse, D] rows
};

template <typename T, int D, int NKTW, int NW, int BQb>
__device__ __forceinline__ void bwd_dkv_body(
    uint32_t bh, int kb, T* __restrict__ smem, float* __restrict__ svec,
    const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
    const T* __restrict__ dOp, const float* __restrict__ LSEp, const float* __restrict__ Dp,
    T* __restrict__ dKp, T* __restrict__ dVp, const int32_t* __restrict__ key_len, int H, int S,
    int causal, int n_kblk, float c_log2, float scale, int group) {
  typedef typename Vec<T>::x8 T8;
  typedef typename Vec<T>::x4 T4;
  typedef BwdTile<T, D, BQb, NW> Tile;
  constexpr int STR = Tile::STR;
  constexpr int NDT = D / 16;
  constexpr int NQP = BQb / 32;  // query pairs per block
  constexpr int NKC = D >= 32 ? D / 32 : 1;
  constexpr int RB = D * (int)sizeof(T);
  constexpr int BKW = NW * NKTW * 16;  // keys per workgroup
  constexpr int ROWF = 64;             // floats in one row-vector stage (one DMA instruction)
  static_assert(BQb % 32 == 0 && BQb <= ROWF && D % 16 == 0, "tile shape");

  // smem: [stage][Q, dO] tiles; svec: [stage][lse, D] rows

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;

  // one workgroup per (batch, key / value head, key block); it walks the
  // query blocks of every query head of the group, so the key / value
  // gradients of grouped-query attention are complete without atomics
  // (batch, key / value head) bh over B * Hk, key block kb
  const int Hk = H / group;
  const int b = (int)(bh / (uint32_t)Hk);
  const int L = clamp_len(key_len, b, S);
  const int64_t head = (int64_t)bh * S * D;        // K, V, dK, dV
  const int64_t bhq0 = (int64_t)b * H + (int64_t)(bh - (uint32_t)b * (uint32_t)Hk) * group;
  const int k_start = kb * BKW;
  const int wk0 = k_start + wave * NKTW * 16;
  const rsrc_t rdk = make_rsrc(dKp + head, (uint32_t)S * RB);
  const rsrc_t rdv = make_rsrc(dVp + head, (uint32_t)S * RB);

  // queries that see any key of the workgroup: all when not causal, else
  // from its first visible key on; none past the key length
  const int q_lo = causal ? min(k_start, L) / BQb * BQb : 0;
  const int nblk = k_start >= L ? 0 : (S - q_lo + BQb - 1) / BQb;  // per query head

  // ---- K and V fragments (B operands, key column c) for this wave's tiles
  const rsrc_t rk = make_rsrc(Kp + head, (uint32_t)L * RB);
  const rsrc_t rv = make_rsrc(Vp + head, (uint32_t)L * RB);
  T8 kf[NKTW][NKC], vf[NKTW][NKC];
  T4 kf4[NKTW], vf4[NKTW];
#pragma unroll
  for (int t = 0; t < NKTW; ++t) {
    const int key = wk0 + 16 * t + c;
    if constexpr (D == 16) {
      kf4[t] = buf_load8<T4>(rk, (key * D + 4 * g) * 2, 0);
      vf4[t] = buf_load8<T4>(rv, (key * D + 4 * g) * 2, 0);
    } else {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        kf[t][kc] = buf_load16<T8>(rk, (key * D + 32 * kc + 8 * g) * 2, 0);
        vf[t][kc] = buf_load16<T8>(rv, (key * D + 32 * kc + 8 * g) * 2, 0);
      }
    }
  }
  wait_vmem();

  AccK32 adk[NKTW][NDT], adv[NKTW][NDT];
#pragma unroll
  for (int t = 0; t < NKTW; ++t)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) adk[t][dt] = adv[t][dt] = AccK32::zero();

  if (nblk > 0) {
    int off[Tile::NIW];
    Tile::offsets(wave, lane, off);
    // row vectors (lse, D of the block's rows): lane i of wave 0 copies one
    // float of each; lanes past the block (and rows past S) write zeros
    const int voff = lane < BQb ? 4 * lane : kOutOfRange;
    // iteration it covers query head j = it / nblk of the group, query
    // block it % nblk
    // the copies walk the iterations in order: (query head cj, block cqb)
    // of the next copy advance by one each time (no division per block),
    // and the buffer descriptors change only with the query head
    int cj = 0, cqb = 0;
    rsrc_t rq, rdo, rl, rd;
    auto set_head = [&](int j) {
      const int64_t hq = (bhq0 + j) * S * D, hr = (bhq0 + j) * S;
      rq = make_rsrc(Qp + hq, (uint32_t)S * RB);
      rdo = make_rsrc(dOp + hq, (uint32_t)S * RB);
      rl = make_rsrc(LSEp + hr, (uint32_t)S * 4);
      rd = make_rsrc(Dp + hr, (uint32_t)S * 4);
    };
    set_head(0);
    auto dma_next = [&](int st) {
      const int q0 = q_lo + cqb * BQb;
      T* Qst = smem + st * 2 * Tile::ELEMS;
      Tile::copy(rq, Qst, off, wave, q0 * RB);
      Tile::copy(rdo, Qst + Tile::ELEMS, off, wave, q0 * RB);
      if (wave == 0) {
        dma4(rl, svec + st * 2 * ROWF, voff, q0 * 4);
        dma4(rd, svec + st * 2 * ROWF + ROWF, voff, q0 * 4);
      }
      if (++cqb == nblk) {
        cqb = 0;
        if (++cj < group) set_head(cj);
      }
    };
    dma_next(0);

    const int rrow = (D >= 32 ? c : bwd_lds_row(c)) * STR;
    const int trow = (D >= 32 ? 4 * g + (c >> 2) : bwd_lds_row(4 * g + (c >> 2))) * STR + 4 * (c & 3);

    const int n_it = group * nblk;
    for (int it = 0, qb = 0; it < n_it; ++it, qb = qb + 1 == nblk ? 0 : qb + 1) {
      const int q0 = q_lo + qb * BQb;
      wait_vmem();
      block_barrier();
      if (it + 1 < n_it) dma_next((it + 1) & 1);

      const T* Qs = smem + (it & 1) * 2 * Tile::ELEMS;
      const T* dOs = Qs + Tile::ELEMS;
      const float* ls = svec + (it & 1) * 2 * ROWF;
      const float* ds = ls + ROWF;
      // a block needs masking if it reaches past S, or (causal) has a
      // query before some key of this wave
      const bool edge = (q0 + BQb > S) || (causal && q0 < wk0 + NKTW * 16 - 1) || (wk0 + NKTW * 16 > L);

#pragma unroll
      for (int p = 0; p < NQP; ++p) {
        // S = Q K^T and dP = dO V^T for the pair's two query tiles h:
        // register i of lane (g, c) is query 32p + 16h + 4g + i, key column c
        typedef std::conditional_t<D == 16, AccK16T<T>, AccK32> SAcc;  // as in the dq body
        SAcc s[2][NKTW], dp[2][NKTW];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int rb = (32 * p + 16 * h) * STR + rrow;
#pragma unroll
          for (int t = 0; t < NKTW; ++t) s[h][t] = dp[h][t] = SAcc::zero();
          if constexpr (D == 16) {
            const T4 qa = *(const T4*)(Qs + rb + 4 * g);
            const T4 da = *(const T4*)(dOs + rb + 4 * g);
#pragma unroll
            for (int t = 0; t < NKTW; ++t) {
              s[h][t] = mfma_k16(qa, kf4[t], s[h][t]);
              dp[h][t] = mfma_k16(da, vf4[t], dp[h][t]);
            }
          } else {
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
              const T8 qa = *(const T8*)(Qs + rb + 32 * kc + 8 * g);
              const T8 da = *(const T8*)(dOs + rb + 32 * kc + 8 * g);
#pragma unroll
              for (int t = 0; t < NKTW; ++t) {
                s[h][t] = mfma_k32(qa, kf[t][kc], s[h][t]);
                dp[h][t] = mfma_k32(da, vf[t][kc], dp[h][t]);
              }
            }
          }
        }
        // P and dS as B operands: k-slot 8g + 4h + i is query 32p + 16h + 4g + i
        T8 pf[NKTW], dsf[NKTW], pl[NKTW], dsl[NKTW];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int qr = 32 * p + 16 * h + 4 * g;  // block row of register 0
          const f32x4 lv = *(const f32x4*)(ls + qr);
          const f32x4 dv = *(const f32x4*)(ds + qr);
#pragma unroll
          for (int t = 0; t < NKTW; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) s[h][t][i] = fast_exp2(fmaf(s[h][t][i], c_log2, -lv[i] * kLog2e));
          // hidden pairs get P = 0, only in blocks that reach a boundary (the
          // empty asm keeps this a branch: if-converted, every element of
          // every block paid for the mask)
          if (edge) {
            asm volatile("");
#pragma unroll
            for (int t = 0; t < NKTW; ++t) {
              const int key = wk0 + 16 * t + c;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int q = q0 + qr + i;
                if (q >= S || key >= L || (causal && key > q)) s[h][t][i] = 0.f;
              }
            }
          }
          // rounded two at a time as head + remainder (one packed conversion
          // per pair): words 2h, 2h + 1 of each operand
#pragma unroll
          for (int t = 0; t < NKTW; ++t) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const float p0 = s[h][t][2 * j], p1 = s[h][t][2 * j + 1];
              uint32_t ph, plo, dh, dlo;
              split2<T>(p0, p1, ph, plo);
              split2_prod<T>(p0, dp[h][t][2 * j] - dv[2 * j], p1, dp[h][t][2 * j + 1] - dv[2 * j + 1], dh, dlo);
              set_word(pf[t], 2 * h + j, ph);
              set_word(pl[t], 2 * h + j, plo);
              set_word(dsf[t], 2 * h + j, dh);
              set_word(dsl[t], 2 * h + j, dlo);
            }
          }
        }
        // dV^T += dO^T P and dK^T += Q^T dS over the pair's 32 queries
        // (transposed reads through inline asm, LA column tiles ahead)
        const uint32_t oaddr = lds_addr(dOs + 32 * p * STR + trow);
        const uint32_t qaddr = lds_addr(Qs + 32 * p * STR + trow);
        constexpr int LA = NDT < 3 ? NDT : 3;
        i16x4 o0[NDT], o1[NDT], q0r[NDT], q1r[NDT];
        auto issue = [&](auto J) {
          constexpr int j = decltype(J)::value;
          o0[j] = lds_read_tr16_asm<16 * j * (int)sizeof(T)>(oaddr);
          o1[j] = lds_read_tr16_asm<(16 * STR + 16 * j) * (int)sizeof(T)>(oaddr);
          q0r[j] = lds_read_tr16_asm<16 * j * (int)sizeof(T)>(qaddr);
          q1r[j] = lds_read_tr16_asm<(16 * STR + 16 * j) * (int)sizeof(T)>(qaddr);
        };
        static_for<LA>(issue);
        static_for<NDT>([&](auto DT) {
          constexpr int dt = decltype(DT)::value;
          if constexpr (dt + LA < NDT) issue(std::integral_constant<int, dt + LA>{});
          constexpr int last = dt + LA < NDT ? dt + LA : NDT - 1;
          lgkm_wait<4 * (last - dt)>(o0[dt], o1[dt], q0r[dt], q1r[dt]);
          const T8 oa = __builtin_bit_cast(T8, __builtin_shufflevector(o0[dt], o1[dt], 0, 1, 2, 3, 4, 5, 6, 7));
          const T8 qa = __builtin_bit_cast(T8, __builtin_shufflevector(q0r[dt], q1r[dt], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int t = 0; t < NKTW; ++t) {
            adv[t][dt] = mfma_k32(oa, pf[t], adv[t][dt]);
            adk[t][dt] = mfma_k32(qa, dsf[t], adk[t][dt]);
            adv[t][dt] = mfma_k32(oa, pl[t], adv[t][dt]);
            adk[t][dt] = mfma_k32(qa, dsl[t], adk[t][dt]);
          }
        });
      }
    }
  }

  // ---- dK = (dK^T)^T / sqrt(d), dV = (dV^T)^T: key row c, columns
  //      16dt + 4g .. 16dt + 4g + 3 (zero for keys past the key length)
#pragma unroll
  for (int t = 0; t < NKTW; ++t) {
    const int key = wk0 + 16 * t + c;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      T4 vk, vv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vk[i] = to_t<T>(adk[t][dt][i] * scale);
        vv[i] = to_t<T>(adv[t][dt][i]);
      }
      buf_store8(vk, rdk, (key * D + 16 * dt + 4 * g) * 2);
      buf_store8(vv, rdv, (key * D + 16 * dt + 4 * g) * 2);
    }
  }
}

// ---------------------------------------------------------------- kernels
template <typename T, int D, int NQT, int NW, int BK, int MODE>
__global__ void __launch_bounds__(NW * 64, 2)
attn_bwd_dq(const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
            const T* __restrict__ dOp, const float* __restrict__ LSEp,
            T* __restrict__ dQp, float* __restrict__ Dp, const int32_t* __restrict__ key_len,
            int H, int S, int causal, int n_qblk, float c_log2, float scale, int group) {
  __shared__ __attribute__((aligned(16))) char lds[DqLds<T, D, BK, NW>::BYTES];
  const uint32_t logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const uint32_t bh = logical / (uint32_t)n_qblk;
  int qb = (int)(logical - bh * (uint32_t)n_qblk);
  if (causal) qb = n_qblk - 1 - qb;  // heaviest causal tiles first
  bwd_dq_body<T, D, NQT, NW, BK, MODE>(bh, qb, (T*)lds, Qp, Kp, Vp, dOp, LSEp,
                                       dQp, Dp, key_len, H, S, causal, n_qblk, c_log2, scale, group);
}

// Both kinds in one launch, once the row term D is in the workspace; the two
// kinds share the workgroup's LDS. Two orders of the workgroups:
//  * by level (causal multi-head problems of up to 4096 workgroups): level l holds key
//    block l of every key / value head (n_hk of them) and query block
//    n - 1 - l of every query head (n_hq), so the heaviest blocks of both
//    kinds start first and the lighter levels fill in behind them (a key
//    block's work falls with its index, a query block's grows with it);
//    item r of a level (n_hk + n_hq padded to a multiple of 8) runs on XCD
//    r % 8, so the blocks of one head share that XCD's L2 at every level.
//    Ordered by kind instead, every key block of such a problem is resident
//    before the first query block starts, and the heaviest query blocks
//    finish last.
//  * by kind (otherwise): the first n_kv_pad workgroups are key blocks (n_kv
//    live, padded to a multiple of 8), then the query blocks, each kind in
//    XCD-aware order (a head's blocks contiguous on one XCD), which larger
//    problems need for L2 reuse. With grouped heads a key block walks the
//    query blocks of every head of its group, so the key blocks are the
//    heavy kind and going first is already the better order.
template <typename T, int D, int NQT, int NW, int BK, int NKTW, int BQb>
__global__ void __launch_bounds__(NW * 64, 2)
attn_bwd_both(const T* __restrict__ Qp, const T* __restrict__ Kp, const T* __restrict__ Vp,
              const T* __restrict__ dOp, const float* __restrict__ LSEp, const float* __restrict__ Dp,
              T* __restrict__ dQp, T* __restrict__ dKp, T* __restrict__ dVp,
              const int32_t* __restrict__ key_len, int H, int S, int causal, int n_blk,
              uint32_t n_hk, uint32_t n_hq, uint32_t per_xcd, int by_level, float c_log2,
              float scale, int group) {
  typedef DkvLds<T, D, BQb, NW> KvLds;
  constexpr int BYTES = KvLds::BYTES > DqLds<T, D, BK, NW>::BYTES ? KvLds::BYTES
                                                                  : DqLds<T, D, BK, NW>::BYTES;
  __shared__ __attribute__((aligned(16))) char lds[BYTES];
  // wave-uniform: this workgroup's kind, head and block
  bool kv = false, live = true;
  uint32_t bh = 0;
  int blk = 0;
  if (by_level) {
    const uint32_t x = blockIdx.x & 7u, j = blockIdx.x >> 3;
    const uint32_t level = j / per_xcd;
    const uint32_t r = (j - level * per_xcd) * 8u + x;
    kv = r < n_hk;
    live = r < n_hk + n_hq;
    bh = kv ? r : r - n_hk;
    blk = kv ? (int)level : n_blk - 1 - (int)level;
  } else {
    const uint32_t n_kv = n_hk * (uint32_t)n_blk, n_kv_pad = (n_kv + 7u) & ~7u;
    kv = blockIdx.x < n_kv_pad;
    live = !kv || blockIdx.x < n_kv;
    const uint32_t logical = kv ? xcd_logical_id(blockIdx.x, n_kv)
                                : xcd_logical_id(blockIdx.x - n_kv_pad, n_hq * (uint32_t)n_blk);
    bh = logical / (uint32_t)n_blk;
    blk = (int)(logical - bh * (uint32_t)n_blk);
    if (!kv && causal) blk = n_blk - 1 - blk;  // heaviest causal tiles first
  }
  if (!live) return;
  if (kv) {
    bwd_dkv_body<T, D, NKTW, NW, BQb>(bh, blk, (T*)lds, (float*)(lds + KvLds::TILE_BYTES), Qp, Kp,
                                      Vp, dOp, LSEp, Dp, dKp, dVp, key_len, H, S, causal, n_blk,
                                      c_log2, scale, group);
  } else {
    bwd_dq_body<T, D, NQT, NW, BK, kRowRead>(bh, blk, (T*)lds, Qp, Kp, Vp, dOp, LSEp, dQp,
                                             const_cast<float*>(Dp), key_len, H, S, causal, n_blk,
                                             c_log2, scale, group);
  }
}

// Row term from the forward's fp32 output: D = rowsum(dO * O32) for every
// query row, in fp32. Each lane takes 8 consecutive columns of one row (a
// 16-byte dO load, two 16-byte O32 loads), D / 8 lanes per row, reduced
// across those lanes. Rows are contiguous over (batch, head, position).
template <typename T, int D>
__global__ void __launch_bounds__(256)
attn_bwd_rowdot(const T* __restrict__ dOp, const float* __restrict__ O32p, float* __restrict__ Dp,
                int64_t rows) {
  typedef typename Vec<T>::x8 T8;
  constexpr int LPR = D / 8;         // lanes per row
  constexpr int RPB = 256 / LPR;     // rows per workgroup
  static_assert(D % 8 == 0 && LPR <= 64, "row width");
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int col = 8 * (tid % LPR);
  float acc = 0.f;
  if (row < rows) {
    const T8 d = *(const T8*)(dOp + row * D + col);
    const f32x4 o0 = *(const f32x4*)(O32p + row * D + col);
    const f32x4 o1 = *(const f32x4*)(O32p + row * D + col + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(to_f(d[i]), o0[i], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(to_f(d[4 + i]), o1[i], acc);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && tid % LPR == 0) Dp[row] = acc;
}

template <typename T, int D>
static hipError_t launch_rowdot(const BwdParams& p, hipStream_t s) {
  constexpr int RPB = 256 / (D / 8);
  const int64_t rows = (int64_t)p.B * p.H * p.S;
  const int64_t nwg = (rows + RPB - 1) / RPB;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_bwd_rowdot<T, D>), dim3((unsigned)nwg), dim3(256), 0, s, (const T*)p.dout,
                     p.out32, p.delta, rows);
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers
template <typename T, int D, int NQT, int NW, int BK, int NKTW, int BQb>
static hipError_t launch_bwd_one(const BwdParams& p, hipStream_t s) {
  constexpr int BQ = NW * NQT * 16;
  constexpr int BKW = NW * NKTW * 16;
  const int n_qblk = (p.S + BQ - 1) / BQ;
  const int n_kblk = (p.S + BKW - 1) / BKW;
  const int64_t wq = (int64_t)p.B * p.H * n_qblk, wk = (int64_t)p.B * (p.H / p.group) * n_kblk;
  if (wq > 0x7fffffffLL || wk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float scale = 1.f / sqrtf((float)p.D);
  // the row pass (or, given the fp32 output, its dot product with dO)
  // writes D, then dQ and dK / dV run in one launch behind it
  hipError_t e;
  if (p.out32) {
    e = launch_rowdot<T, D>(p, s);
  } else {
    hipLaunchKernelGGL((attn_bwd_dq<T, D, NQT, NW, BK, kRowPass>), dim3((unsigned)wq), dim3(NW * 64), 0, s,
                       (const T*)p.q, (const T*)p.k, (const T*)p.v, (const T*)p.dout, p.lse,
                       (T*)p.dq, p.delta, p.key_len, p.H, p.S, p.causal, n_qblk, p.c_log2, scale, p.group);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  // one level per block index (key and query blocks are the same size)
  static_assert(BQ == BKW, "levels pair key block l with query block l");
  const int64_t n_hk = (int64_t)p.B * (p.H / p.group), n_hq = (int64_t)p.B * p.H;
  const int64_t per_xcd = (n_hk + n_hq + 7) / 8;
  const int by_level = p.causal && p.group == 1 && per_xcd * 8 * n_qblk <= 4096;
  const int64_t n_wg = by_level ? per_xcd * 8 * n_qblk : (wk + 7) / 8 * 8 + wq;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_bwd_both<T, D, NQT, NW, BK, NKTW, BQb>), dim3((unsigned)n_wg),
                     dim3(NW * 64), 0, s, (const T*)p.q, (const T*)p.k, (const T*)p.v,
                     (const T*)p.dout, p.lse, p.delta, (T*)p.dq, (T*)p.dk, (T*)p.dv, p.key_len,
                     p.H, p.S, p.causal, n_qblk, (uint32_t)n_hk, (uint32_t)n_hq,
                     (uint32_t)per_xcd, by_level, p.c_log2, scale, p.group);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t s) {
  switch (p.D) {
    // (query tiles per wave, waves, keys per block | key tiles per wave,
    // queries per block); one 16-row tile per wave doubles the workgroups,
    // which the training shape (B=4, H=12, S=1024) needs, at no cost on
    // larger problems
    case 16: return launch_bwd_one<T, 16, 1, 4, 64, 1, 64>(p, s);
    case 32: return launch_bwd_one<T, 32, 1, 4, 64, 1, 64>(p, s);
    case 64: return launch_bwd_one<T, 64, 1, 4, 64, 1, 64>(p, s);
    case 128: return launch_bwd_one<T, 128, 1, 4, 64, 1, 64>(p, s);
    case 256: return launch_bwd_one<T, 256, 1, 4, 32, 1, 32>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdParams& p, hipStream_t s) {
  if (p.dtype == 1) return launch_bwd_t<f16_t>(p, s);
  if (p.dtype == 2) return launch_bwd_t<bf16_t>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mha
