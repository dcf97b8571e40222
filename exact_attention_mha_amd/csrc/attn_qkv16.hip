// Attention fed by its own QKV projection, for d_h = 16 or 8 heads and
// S <= 128 (fp16 / bf16): out[b] = attention of the head slices of
// X[b] W_qkv + b_qkv,
// with the projected q, k, v never leaving the chip (devpost
// "gpu-transformer-optimization", section 2.2: the fused QKV-attention
// program reads the activations once and writes only the output).
//
// Work decomposition. A workgroup holds one wave per 16 projection columns
// (d_model / 16 waves: one head of 16, or two heads of 8, per wave) and
// walks over batch elements (persistent grid, one or two workgroups per CU).
// Each wave keeps its 48 weight columns in registers for the whole run,
// loaded once. With heads of 8 the projection uses all 16 columns of its
// products (the pages' heads-per-dot grouping, devpost
// "gpu-transformer-optimization", section 2.2); each head's scores then
// contract over its own columns only (the other head's columns of q are
// zero), and of the 16 output columns of each head's P V product only its
// own are kept. The [S, d_model] activation tile
// of a batch element is copied into LDS by buffer->LDS DMA (double-buffered,
// the next element's copy overlapping this element's attention) and read by
// every head.
//
// Layouts. With lane = 16 g + c, the three projections are arranged so that
// each result lands in exactly the register layout the attention products
// consume, with no shuffles:
//   * Q^T = W_q^T X^T and K^T = W_k^T X^T (A: weight columns, B: activation
//     rows) leave row 16t + c of Q / K, columns 4g..4g+3, in lane (g, c):
//     the B / A operands of S^T = K Q^T;
//   * V = X W_v (A: activation rows, B: weight columns) leaves V[16t + 4g + i]
//     [c] in register i of lane (g, c): the A operand (V^T) of O^T += V^T P^T.
// The activation fragment (row 16t + c, 8 columns from 32kk + 8g) is the B
// operand of the first two and the A operand of the third, so one LDS read
// feeds three matrix products. The weight fragments of all three have the
// same form: column c of the head's slice, rows 32kk + 8g .. 32kk + 8g + 7.
//
// Precision. The projections accumulate in fp32. q and k are kept as a
// head + remainder pair in the input dtype: an error of a few 2^-12 in a
// score moves every probability of its row by as much, and where an output
// is a small difference of large values (projection weights twice the
// default initialisation scale, heads of 8) a single fp16 rounding of q and
// k already exceeds the accuracy budget. v (and P) are rounded once for
// fp16; bf16 keeps them as pairs too, since one bf16 rounding of v alone
// exceeds the budget. The K = 32 products take a pair in their two halves:
//   S^T = [k_hi | k_lo] . [q_hi | q_hi] + [k_hi | k_lo] . [q_lo | q_lo],
//   bf16: O^T += [v_hi | v_lo] . [p_hi | p_hi] + [v_hi | v_lo] . [p_lo | p_lo].
// (A K = 16 product for k_hi . q_lo alone, accumulating onto the K = 32
// result, measured wrong on gfx950 with the wait states the compiler puts
// between the two shapes; every accumulator here sees one product shape.)
//
// Attention itself is the one-pass short-sequence form: a whole score row
// fits in registers (no online rescaling), masks ride in the accumulator's
// initial value (0 visible, -inf hidden), only key tiles a query tile can
// see are computed, and the row sum is a ones operand times the same rounded
// P as the numerator. Activation rows past S read zero from the
// range-checked copy and their stores are dropped; projected keys and values
// at or past the key length are zeroed, so whatever the activation rows there
// hold reaches only their own query outputs.
#include <type_traits>
#include <utility>

#include "attn_common.h"
#include "launch.h"

namespace mha {

template <typename T, int NH, int HPW, bool CAUSAL>
__global__ void __launch_bounds__(NH * 64, 2)
attn_qkv16(const T* __restrict__ Xp, const T* __restrict__ Wp, const T* __restrict__ bias,
           T* __restrict__ Op, float* __restrict__ LSEp, const int32_t* __restrict__ key_len,
           int B, int S, float c_log2) {
  typedef typename Vec<T>::x4 T4;
  typedef typename Vec<T>::x8 T8;
  constexpr int DM = 16 * NH;       // model width: 16 projection columns per wave
  constexpr int NHEAD = NH * HPW;   // heads (d_h = 16 / HPW)
  constexpr int RB = 2 * DM;        // bytes per activation / output row
  constexpr int NCH = RB / 16;      // 16-byte chunks per row
  constexpr int RPL = 16 / NCH;     // rows per 256-byte LDS line
  constexpr int NK = DM / 32;       // K = 32 steps of a projection
  constexpr int TB = 128 * RB;      // bytes of one [128, d_model] tile
  constexpr int NT = 8;             // 16-row tiles in S <= 128
  constexpr bool kSplit = __is_same(T, bf16_t);  // v and P as pairs too
  // a projected v tile: fp16 the rounded values, bf16 [head | remainder]
  // (k tiles are [head | remainder] for both)
  typedef std::conditional_t<kSplit, T8, T4> VT;
  static_assert(NH == 2 || NH == 4 || NH == 8, "d_model 32, 64 or 128");
  static_assert(HPW == 1 || HPW == 2, "one head of 16 or two heads of 8 per wave");
  static_assert(TB == 4 * NH * 1024, "four 1 KiB copies per wave fill a tile");
  __shared__ __attribute__((aligned(16))) char xs[2 * TB];

  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int h = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // this wave's head

  // LDS row r holds its 16-byte chunk q at chunk q ^ swz(r): the 16 lanes
  // that read one chunk index of 16 consecutive rows then cover all banks.
  auto swz = [](int r) { return (r / RPL) & (NCH - 1); };

  // ---- this head's weight columns and biases, once per workgroup ---------
  // wf[sec][kk] element e = W[32kk + 8g + e][sec * d_model + 16h + c]
  T8 wf[3][NK];
#pragma unroll
  for (int sec = 0; sec < 3; ++sec)
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        wf[sec][kk][e] = Wp[(size_t)(32 * kk + 8 * g + e) * (3 * DM) + sec * DM + 16 * h + c];
  AccK32 bq, bk, bv;  // biases: the projections' initial accumulators
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bq[i] = bias ? to_f(bias[16 * h + 4 * g + i]) : 0.f;       // Q^T row = dim 4g + i
    bk[i] = bias ? to_f(bias[DM + 16 * h + 4 * g + i]) : 0.f;  // K^T row = dim 4g + i
    bv[i] = bias ? to_f(bias[2 * DM + 16 * h + c]) : 0.f;      // V column = dim c
  }

  // Copy activation tile `bb` into stage `st`: instruction n of wave h fills
  // LDS bytes [1024 (h + NH n), +1024); each lane fetches the chunk that the
  // swizzle places at its 16 bytes. Rows past S read as zero.
  auto issue = [&](int bb, int st) {
    const rsrc_t rx = make_rsrc(Xp + (int64_t)bb * S * DM, (uint32_t)(S * RB));
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int base = 1024 * (h + NH * n);
      const int o = base + 16 * lane;
      const int r = o / RB, pc = (o % RB) / 16;
      dma16(rx, xs + st * TB + base, r * RB + 16 * (pc ^ swz(r)), 0);
    }
  };

  T4 ones4;
#pragma unroll
  for (int e = 0; e < 4; ++e) ones4[e] = to_t<T>(1.f);
  const T8 ones8 = __builtin_shufflevector(ones4, ones4, 0, 1, 2, 3, 4, 5, 6, 7);
  const AccK32 zero4 = AccK32::zero();
  const T4 zt4 = zero_vec<T4>();
  // Activation fragment kk of row 16j + c sits at xa[kk] + j * 16 * RB (the
  // swizzle of row 16j + c equals that of row c), so each tile's reads use
  // immediate offsets from NK per-lane addresses.
  const uint32_t x0 = lds_addr(xs) + c * RB;
  constexpr int TROW = 16 * RB;  // bytes of one 16-row tile

  // One projection over tile J: NK activation fragments read from LDS
  // (already issued into xf), each feeding the products the caller asks for.
  // PEND: LDS reads issued after these NK that may stay outstanding.
  auto project = [&](auto PEND, const T8 (&xf)[NK], bool with_q, bool with_kv, AccK32& aq,
                     AccK32& ak, AccK32& av) {
    constexpr int pend = decltype(PEND)::value;
    static_for<NK>([&](auto KK) {
      constexpr int kk = decltype(KK)::value;
      T8 x = xf[kk];
      lgkm_wait1<pend + NK - 1 - kk>(x);
      if (with_q) aq = mfma_k32(wf[0][kk], x, aq);
      if (with_kv) {
        ak = mfma_k32(wf[1][kk], x, ak);
        av = mfma_k32(x, wf[2][kk], av);
      }
    });
  };
  auto read_tile = [&](auto J, uint32_t st_off, T8 (&xf)[NK]) {
    constexpr int j = decltype(J)::value;
    static_for<NK>([&](auto KK) {
      constexpr int kk = decltype(KK)::value;
      const uint32_t a = x0 + st_off + 16 * ((4 * kk + g) ^ swz(c));
      xf[kk] = __builtin_bit_cast(T8, lds_read_b128_asm<j * TROW>(a));
    });
  };

  // causal diagonal tile: key 4g + i visible to query c iff 4g + i <= c
  AccK32 diag;
#pragma unroll
  for (int i = 0; i < 4; ++i) diag[i] = 4 * g + i <= c ? 0.f : -INFINITY;

  const int G = gridDim.x;
  int bb = blockIdx.x;  // the launcher sizes the grid to at most B
  issue(bb, 0);
  for (int it = 0; bb < B; ++it, bb += G) {
    const int st = it & 1;
    // This wave's copies of tile bb have landed: they were issued before the
    // (1 + HPW) * NT stores of the previous element, which may still be in
    // flight.
    // After the barrier every wave's copies have landed, and every wave is
    // done reading the other stage.
    if (it == 0)
      wait_vmem();
    else
      wait_vmem_keep<(1 + HPW) * NT>();
    block_barrier();
    // the next element's copy overlaps all of this element's work
    if (bb + G < B) issue(bb + G, st ^ 1);
    const uint32_t st_off = st * TB;
    const int L = clamp_len(key_len, bb, S);
    const int kt_need = (L + 15) >> 4;  // key tiles holding a visible key
    const int kL = L >> 4;              // the tile holding key L (if L % 16 != 0)
    const int vlim = L - 4 * g;
    // score offsets of tile kL: -inf on keys at or past L (register i of
    // lane (g, c) is key 16 kL + 4g + i)
    f32x4 mL;
#pragma unroll
    for (int i = 0; i < 4; ++i) mL[i] = 16 * kL + i >= vlim ? -INFINITY : 0.f;

    // ---- projection pass over the tiles: k and v for visible key tiles
    // (q is projected per query tile below, which keeps fewer registers live)
    T8 kf[NT];
    VT vt[NT];
    {
      T8 xf[2][NK];
      read_tile(std::integral_constant<int, 0>{}, st_off, xf[0]);
      static_for<NT>([&](auto J) {
        constexpr int j = decltype(J)::value;
        constexpr int pend = j + 1 < NT ? NK : 0;
        if constexpr (j + 1 < NT) read_tile(std::integral_constant<int, j + 1>{}, st_off, xf[(j + 1) & 1]);
        const bool with_kv = j < kt_need;
        AccK32 aq, ak = bk, av = bv;
        project(std::integral_constant<int, pend>{}, xf[j & 1], false, with_kv, aq, ak, av);
        // Keys at or past the key length are zeroed: their activation rows
        // are real query rows whose contents may be anything, and a hidden
        // score must stay exactly -inf (mask plus 0) and a hidden value
        // exactly 0 (it meets zero probabilities in the paired products).
        // Only the tile holding the key length has both kinds of rows; the
        // tiles past it were not projected (bias only, finite) and are never
        // read as keys.
        if (j == kL) {  // wave-uniform
          const bool krow_hidden = c >= L - 16 * j;  // K row 16j + c (A operand row)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ak[i] = krow_hidden ? 0.f : ak[i];
            av[i] = 16 * j + i >= vlim ? 0.f : av[i];  // V row 16j + 4g + i
          }
        }
        kf[j] = split4<T>(ak);
        if constexpr (kSplit) {
          vt[j] = split4<T>(av);
        } else {
          vt[j] = __builtin_bit_cast(T4, u32x2{pack2<T>(av[0], av[1]), pack2<T>(av[2], av[3])});
        }
        __builtin_amdgcn_sched_barrier(0);  // one tile at a time (register pressure)
      });
    }

    // ---- attention per query tile --------------------------------------
    // Every query tile issues exactly 1 + HPW stores (output, each head's
    // row lse), dropped where out of range, so each element ends with
    // (1 + HPW) * NT stores in flight.
    const rsrc_t ro = make_rsrc(Op + (int64_t)bb * S * DM, (uint32_t)(S * RB));
    rsrc_t rl[HPW];
#pragma unroll
    for (int j = 0; j < HPW; ++j)
      rl[j] = LSEp ? make_rsrc(LSEp + ((int64_t)bb * NHEAD + HPW * h + j) * S, (uint32_t)S * 4)
                   : make_rsrc(Op, 0u);
    // with two heads per wave, lane group g holds columns of head g / 2 (in
    // Q, K and the output), and V column c belongs to head c / 8
    const int gh = HPW == 2 ? g >> 1 : 0;
    auto qtile = [&](auto J) {
      constexpr int t = decltype(J)::value;
      const int row = 16 * t + c;
      const int ooff = row * RB + 32 * h + 8 * g;  // this wave's columns, lane g's four
      if (16 * t >= S || L == 0) {  // wave-uniform: no rows, or no visible key
        buf_store8(zt4, ro, 16 * t >= S ? kOutOfRange : ooff);
#pragma unroll
        for (int j = 0; j < HPW; ++j)
          buf_store4(-INFINITY, rl[j], (16 * t >= S || g != 2 * j) ? kOutOfRange : row * 4);
        return;
      }
      T4 q4, l4;  // this tile's q: head and remainder
      {
        T8 xf[NK];
        read_tile(J, st_off, xf);
        AccK32 aq = bq, ak, av;
        project(std::integral_constant<int, 0>{}, xf, true, false, aq, ak, av);
        const T8 ql = split4<T>(aq);
        q4 = __builtin_shufflevector(ql, ql, 0, 1, 2, 3);
        l4 = __builtin_shufflevector(ql, ql, 4, 5, 6, 7);
      }
      constexpr int NKT = CAUSAL ? t + 1 : NT;  // key tiles computed at most
      const int klast = min(CAUSAL ? t : NT - 1, (L - 1) >> 4);
      AccK32 o[HPW], lsum[HPW];
      float m[HPW];
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        // head j's scores: the other head's columns of q are zero, so the
        // 16-wide product contracts over head j's columns only
        const bool mine = gh == j;
        const T4 qm = mine ? q4 : zt4;
        const T8 qa = __builtin_shufflevector(qm, qm, 0, 1, 2, 3, 4, 5, 6, 7);
        const T4 lm = mine ? l4 : zt4;
        const T8 qb = __builtin_shufflevector(lm, lm, 0, 1, 2, 3, 4, 5, 6, 7);
        AccK32 sc[NT];
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          if (kt > klast) break;
          // the causal diagonal starts from its constant mask; the tile
          // holding the key length then adds its offsets
          const AccK32 init = (CAUSAL && kt == t) ? diag : zero4;
          sc[kt] = mfma_k32(kf[kt], qa, init);
          sc[kt] = mfma_k32(kf[kt], qb, sc[kt]);
          if (kt == kL) {  // wave-uniform
            // (a real branch: the empty volatile statement keeps the
            // compiler from turning this into an add and a select on every
            // tile)
            asm volatile("");
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[kt][i] += mL[i];
          }
          mx = max3(mx, sc[kt][0], sc[kt][1]);
          mx = max3(mx, sc[kt][2], sc[kt][3]);
        }
        m[j] = group_max(mx) * c_log2;  // finite: key 0 is visible
        auto probs = [&](const AccK32& sv, T4& hi, T4& lo) {
          AccK32 pv;
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(fmaf(sv[i], c_log2, -m[j]));
          if constexpr (kSplit) {
            const T8 pl = split4<T>(pv);
            hi = __builtin_shufflevector(pl, pl, 0, 1, 2, 3);
            lo = __builtin_shufflevector(pl, pl, 4, 5, 6, 7);
          } else {
            hi = __builtin_bit_cast(T4, u32x2{pack2<T>(pv[0], pv[1]), pack2<T>(pv[2], pv[3])});
          }
        };
        // all 16 value columns are multiplied; only head j's columns of
        // o[j] are kept below
        o[j] = zero4;
        lsum[j] = zero4;
        if constexpr (kSplit) {
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt) {
            if (kt > klast) break;
            T4 ph, pl;
            probs(sc[kt], ph, pl);
            o[j] = mfma_k32(vt[kt], __builtin_shufflevector(ph, ph, 0, 1, 2, 3, 4, 5, 6, 7), o[j]);
            o[j] = mfma_k32(vt[kt], __builtin_shufflevector(pl, pl, 0, 1, 2, 3, 4, 5, 6, 7), o[j]);
            lsum[j] = mfma_k32(ones8, __builtin_shufflevector(ph, pl, 0, 1, 2, 3, 4, 5, 6, 7), lsum[j]);
          }
        } else {
          // key tiles in pairs: one K = 32 product covers keys 16k0 + 4g + e
          // (slots e < 4) and 16k1 + 4g + e - 4 (slots e >= 4)
#pragma unroll
          for (int kp = 0; kp < (NKT + 1) / 2; ++kp) {
            const int k0 = 2 * kp, k1 = 2 * kp + 1;
            if (k0 > klast) break;
            T4 p0, p1 = zt4, unused;
            probs(sc[k0], p0, unused);
            if (k1 < NKT && k1 <= klast) probs(sc[k1], p1, unused);
            const T8 a = __builtin_shufflevector(vt[k0], vt[k1], 0, 1, 2, 3, 4, 5, 6, 7);
            const T8 pb = __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7);
            o[j] = mfma_k32(a, pb, o[j]);
            lsum[j] = mfma_k32(ones8, pb, lsum[j]);
          }
        }
      }
      // the O^T lane layout holds row `row`, columns 4g..4g+3: head gh's
      const AccK32 os = HPW == 2 && gh == 1 ? o[HPW - 1] : o[0];
      const float ls = HPW == 2 && gh == 1 ? lsum[HPW - 1][0] : lsum[0][0];  // every row holds the sum
      const float inv = __builtin_amdgcn_rcpf(ls);
      T4 ov;
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = to_t<T>(os[i] * inv);
      buf_store8(ov, ro, ooff);
#pragma unroll
      for (int j = 0; j < HPW; ++j)
        buf_store4((m[j] + fast_log2(lsum[j][0])) * kLn2, rl[j], g == 2 * j ? row * 4 : kOutOfRange);
      __builtin_amdgcn_sched_barrier(0);  // keep query tiles from interleaving (register pressure)
    };
    static_for<NT>(qtile);
  }
}

template <typename T, int NH, int HPW, bool C>
static hipError_t launch_qkv_t(const QkvParams& p, hipStream_t s) {
  auto kern = attn_qkv16<T, NH, HPW, C>;
  // persistent grid: as many workgroups as fit on the device at once
  static int per_cu[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (per_cu[dev] == 0) {
    int ncu = 0, occ = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidDevice;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, NH * 64, 0) != hipSuccess)
      return hipErrorInvalidConfiguration;
    per_cu[dev] = (ncu > 0 ? ncu : 1) * (occ > 0 ? occ : 1);
  }
  const int grid = p.B < per_cu[dev] ? p.B : per_cu[dev];
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NH * 64), 0, s, (const T*)p.x, (const T*)p.w,
                     (const T*)p.bias, (T*)p.out, p.lse, p.key_len, p.B, p.S, p.c_log2);
  return hipGetLastError();
}

template <typename T, int NH, int HPW>
static hipError_t launch_qkv_h(const QkvParams& p, hipStream_t s) {
  return p.causal ? launch_qkv_t<T, NH, HPW, true>(p, s) : launch_qkv_t<T, NH, HPW, false>(p, s);
}

// waves = d_model / 16; heads of 16 (one per wave) or of 8 (two per wave)
template <typename T>
static hipError_t launch_qkv_d(const QkvParams& p, hipStream_t s) {
  const int waves = p.H * p.hd / 16;
  if (p.hd == 16) {
    switch (waves) {
      case 2: return launch_qkv_h<T, 2, 1>(p, s);
      case 4: return launch_qkv_h<T, 4, 1>(p, s);
      case 8: return launch_qkv_h<T, 8, 1>(p, s);
    }
  } else if (p.hd == 8) {
    switch (waves) {
      case 2: return launch_qkv_h<T, 2, 2>(p, s);
      case 4: return launch_qkv_h<T, 4, 2>(p, s);
      case 8: return launch_qkv_h<T, 8, 2>(p, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_qkv16(const QkvParams& p, hipStream_t s) {
  if (p.S > 128 || p.B <= 0 || p.S <= 0) return hipErrorInvalidValue;
  if (p.dtype == 1) return launch_qkv_d<f16_t>(p, s);
  if (p.dtype == 2) return launch_qkv_d<bf16_t>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mha
