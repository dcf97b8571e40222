// Device-side helpers shared by the gfx950 attention kernels.
//
// Matrix-core conventions used throughout (64-lane wavefront, lane = 16*g + c,
// c = lane & 15, g = lane >> 4):
//   * a 16x16 fp32 MFMA result tile holds element (row 4g+i, col c) in
//     register i of lane (g, c);
//   * the A operand of a 16x16xK MFMA holds row c, and the B operand column c,
//     with the K index spread over (g, element); only the correspondence
//     between A and B matters, and every kernel fills both from the same
//     (g, element) -> k map.
// Scores are computed transposed, S^T = K Q^T (rows = keys, cols = queries),
// so every lane owns one query column: row max / sum reduce inside the lane
// and across the four lane groups only, and the probability tile P^T is
// already laid out as the B operand of O^T += V^T P^T.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>
#include <stdint.h>

namespace mha {

typedef _Float16 f16_t;
typedef __bf16 bf16_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.442695040888963407360f;

template <typename T> struct Vec;
template <> struct Vec<f16_t> { typedef f16x8 x8; typedef f16x4 x4; };
template <> struct Vec<bf16_t> { typedef bf16x8 x8; typedef bf16x4 x4; };

template <typename V> __device__ __forceinline__ V zero_vec();

// ---- matrix-core products (fp32 accumulate) ---------------------------------
// Every accumulator carries, in its type, the reduction depth K of the
// instruction shape that produces it: Acc<32> for 16x16x32, Acc<16> for the
// fp16 16x16x16 product, Acc<4> for the fp32 16x16x4 product. A product only
// takes an accumulator of its own shape, so the result of one shape cannot be
// fed to another shape as its accumulator by accident (on gfx950 a 16x16x32
// result used directly as the accumulator of a 16x16x16 product gave wrong
// sums); moving values between shapes takes an explicit element copy.
template <int K>
struct Acc {
  f32x4 v;
  // element access: reads give the float; writes go through a reference to
  // one lane of the vector. The reference lives only as long as the
  // accumulator: never keep one in an `auto` variable or return one (take
  // `float x = acc[i]`, or acc.vec()[i]).
  struct Ref {
    f32x4& v;
    int i;
    __device__ __forceinline__ operator float() const { return v[i]; }
    __device__ __forceinline__ Ref& operator=(float x) { v[i] = x; return *this; }
    __device__ __forceinline__ Ref& operator=(const Ref& r) { v[i] = (float)r; return *this; }
    __device__ __forceinline__ Ref& operator+=(float x) { v[i] += x; return *this; }
    __device__ __forceinline__ Ref& operator*=(float x) { v[i] *= x; return *this; }
  };
  __device__ __forceinline__ Ref operator[](int i) { return Ref{v, i}; }
  __device__ __forceinline__ float operator[](int i) const { return v[i]; }
  __device__ __forceinline__ Acc& operator*=(float a) {
    v *= a;
    return *this;
  }
  __device__ __forceinline__ f32x4 vec() const { return v; }
  static __device__ __forceinline__ Acc of(f32x4 x) { return Acc{x}; }
  static __device__ __forceinline__ Acc fill(float x) { return Acc{f32x4{x, x, x, x}}; }
  static __device__ __forceinline__ Acc zero() { return fill(0.f); }
};
typedef Acc<32> AccK32;  // v_mfma_f32_16x16x32_{f16,bf16}
typedef Acc<16> AccK16;  // v_mfma_f32_16x16x16_f16
typedef Acc<4> AccK4;    // v_mfma_f32_16x16x4_f32

__device__ __forceinline__ AccK32 mfma_k32(f16x8 a, f16x8 b, AccK32 c) {
  return AccK32::of(__builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c.vec(), 0, 0, 0));
}
__device__ __forceinline__ AccK32 mfma_k32(bf16x8 a, bf16x8 b, AccK32 c) {
  return AccK32::of(__builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c.vec(), 0, 0, 0));
}
__device__ __forceinline__ AccK16 mfma_k16(f16x4 a, f16x4 b, AccK16 c) {
  return AccK16::of(__builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c.vec(), 0, 0, 0));
}
// bf16 K=16 products go through the K=32 instruction with the upper half of
// both operands zero (the same sum: zero products add nothing), so their
// accumulator is a K=32 one.
__device__ __forceinline__ AccK32 mfma_k16(bf16x4 a, bf16x4 b, AccK32 c) {
  const bf16x8 a8 = __builtin_shufflevector(a, zero_vec<bf16x4>(), 0, 1, 2, 3, 4, 5, 6, 7);
  const bf16x8 b8 = __builtin_shufflevector(b, zero_vec<bf16x4>(), 0, 1, 2, 3, 4, 5, 6, 7);
  return AccK32::of(__builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, c.vec(), 0, 0, 0));
}
// the accumulator type of mfma_k16 for element type T
template <typename T> struct AccK16Of { typedef AccK16 type; };
template <> struct AccK16Of<bf16_t> { typedef AccK32 type; };
template <typename T> using AccK16T = typename AccK16Of<T>::type;
__device__ __forceinline__ AccK4 mfma_f32_k4(float a, float b, AccK4 c) {
  return AccK4::of(__builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c.vec(), 0, 0, 0));
}

// ---- LDS transpose read (gfx950 ds_read_b64_tr_b16) -------------------------
// Within each group of 16 lanes, lanes 4r..4r+3 each supply the address of 4
// consecutive 16-bit elements; together they form row r (16 elements) of a
// 4 x 16 tile. Lane j of the group receives column j: element j of rows
// 0, 1, 2, 3. Used to read V^T operands from a row-major V tile.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
}

// The same read issued through inline asm at LDS byte address addr + OFF.
// The compiler makes every LDS read it can see wait for all buffer->LDS
// copies in flight (s_waitcnt vmcnt(0)), including copies of later blocks
// into another stage, which would pull the copy latency into every block.
// It cannot see this one, so it adds no such wait -- and no wait for the
// result either: the caller orders each result with lgkm_wait<N>() before its
// first use. The caller also guarantees, by its own waits and barriers, that
// the copy which wrote the bytes read here has completed.
template <int OFF>
__device__ __forceinline__ i16x4 lds_read_tr16_asm(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  i16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
// s_waitcnt lgkmcnt(N): at most N LDS operations still outstanding. LDS
// operations complete in issue order, so the reads issued before the last N
// have landed. The two fragments pass through the instruction, which ties
// their uses to the wait.
template <int N>
__device__ __forceinline__ void lgkm_wait(i16x4& a, i16x4& b) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait(i16x4& a, i16x4& b, i16x4& c, i16x4& d) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "i"(N));
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1, so that loop
// indices are compile-time constants (static register indexing, immediate
// instruction offsets).
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
  }(std::make_integer_sequence<int, N>{});
}

// ---- buffer addressing -------------------------------------------------------
// Raw buffer resources carry a byte range; loads past it return zero without
// touching memory and stores past it are dropped. Kernels use this as the
// bounds check for ragged tails (rows past S, keys past the visible range).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
constexpr int kBufferWord3 = 0x00020000;  // raw (untyped) buffer, gfx9 family
constexpr int kOutOfRange = 0x7ffffff0;   // an offset past every range used here

// 16-byte LDS read at byte address addr + OFF through inline asm, for the
// same reason as lds_read_tr16_asm (no compiler wait for buffer->LDS copies
// into other stages); the caller orders the result with lgkm_wait1<N>.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read_b128_asm(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
// s_waitcnt lgkmcnt(N) tied to one value (see lgkm_wait).
template <int N, typename V>
__device__ __forceinline__ void lgkm_wait1(V& a) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "i"(N));
}

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, kBufferWord3);
}
template <typename V>
__device__ __forceinline__ V buf_load16(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
template <typename V>
__device__ __forceinline__ V buf_load8(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
template <typename V>
__device__ __forceinline__ void buf_store8(V v, rsrc_t r, int voff) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, voff, 0, 0);
}
__device__ __forceinline__ void buf_store16(f32x4 v, rsrc_t r, int voff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, 0, 0);
}
__device__ __forceinline__ void buf_store4(float v, rsrc_t r, int voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, voff, 0, 0);
}
// Asynchronous 16-byte-per-lane copy from a buffer straight into LDS: lane i's
// 16 bytes land at lds + 16*i (lds must be wave-uniform). Completion is
// tracked by the vector-memory counter.
__device__ __forceinline__ void dma16(rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, soff, 0, 0);
}
// The same with 4 bytes per lane: lane i's 4 bytes land at lds + 4*i.
__device__ __forceinline__ void dma4(rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                           voff, soff, 0, 0);
}
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left unconstrained)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }
// s_waitcnt vmcnt(N): at most N (the most recent) vector-memory operations
// still outstanding; vmcnt occupies bits [3:0] and [15:14] of the gfx9
// s_waitcnt immediate
template <int N>
__device__ __forceinline__ void wait_vmem_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// ---- transcendental helpers (single hardware instructions) ----------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// max(a, b, c) as IEEE 754-2019 maximum (NaN-propagating): one
// v_maximum3_f32. The fmaxf form (NaN-ignoring) needs an extra quieting
// instruction for every operand the compiler cannot prove canonical, which
// includes every matrix-core result. With either form a NaN score makes its
// row NaN (its exponential is NaN), as in the definition. Plain code, so
// the compiler inserts the wait states a read of a fresh matrix-core result
// needs.
__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// max(a, b), the same way.
__device__ __forceinline__ float max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Workgroup barrier without the release fence of __syncthreads (which would
// drain every outstanding global->LDS copy). Callers order their own copies
// with an explicit vmcnt wait before it; the memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// ---- cross-group reductions: lanes c, c+16, c+32, c+48 share a query ------
// v_permlane16_swap(x, x) yields, in its two results, the values of lanes
// i and i^16 (in some order) at every lane i; v_permlane32_swap likewise for
// i and i^32. Combining the pair reduces over the four lane groups on the
// vector ALU, with no LDS round trip.
__device__ __forceinline__ float xor16_pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float group_max(float x) { return xor32_pair_max(xor16_pair_max(x)); }
__device__ __forceinline__ float group_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- conversions -------------------------------------------------------------
template <typename T> __device__ __forceinline__ T to_t(float x);
template <> __device__ __forceinline__ f16_t to_t<f16_t>(float x) { return (f16_t)x; }
template <> __device__ __forceinline__ bf16_t to_t<bf16_t>(float x) { return (bf16_t)x; }

template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

// ---- pairs of floats rounded to 16-bit words (one packed conversion each) ----
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// (a, b) rounded to T, a in the low half
template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<f16_t>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}
template <> __device__ __forceinline__ uint32_t pack2<bf16_t>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// bf16 head + remainder of a pair: hi = (a, b) rounded to bf16, lo = the
// rounding errors (a - head_a, b - head_b) rounded to bf16 (exact
// subtractions: the heads are a's and b's leading bits)
__device__ __forceinline__ void split2_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack2<bf16_t>(a, b);
  const float ha = __builtin_bit_cast(float, hi << 16);
  const float hb = __builtin_bit_cast(float, hi & 0xffff0000u);
  lo = pack2<bf16_t>(a - ha, b - hb);
}
// a - (the fp16 number in the low / high half of h), in fp32: one
// mixed-precision FMA, (-1) * h + a, that widens h itself (the same value as
// widening h and subtracting)
__device__ __forceinline__ float sub_f16_lo(uint32_t h, float a) {
  float r;
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(a));
  return r;
}
__device__ __forceinline__ float sub_f16_hi(uint32_t h, float a) {
  float r;
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(a));
  return r;
}
// fp16 head + remainder of a pair, as above (a - head is exact in fp32 for
// |a| below the fp16 range)
__device__ __forceinline__ void split2_f16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack2<f16_t>(a, b);
  lo = pack2<f16_t>(sub_f16_lo(hi, a), sub_f16_hi(hi, b));
}
template <typename T> __device__ __forceinline__ void split2(float a, float b, uint32_t& hi,
                                                              uint32_t& lo) {
  if constexpr (__is_same(T, bf16_t)) split2_bf16(a, b, hi, lo);
  else split2_f16(a, b, hi, lo);
}
// head + remainder of two products pa * xa, pb * xb: the heads are the
// rounded products, the remainders come from one fused multiply-add each
// (pa * xa - head, compiled to a mixed-precision FMA for fp16), so they also
// carry the products' own fp32 rounding errors
template <typename T> __device__ __forceinline__ void split2_prod(float pa, float xa, float pb, float xb,
                                                                   uint32_t& hi, uint32_t& lo) {
  hi = pack2<T>(pa * xa, pb * xb);
  float ha, hb;
  if constexpr (__is_same(T, bf16_t)) {
    ha = __builtin_bit_cast(float, hi << 16);
    hb = __builtin_bit_cast(float, hi & 0xffff0000u);
  } else {
    const f32x2 h = __builtin_convertvector(__builtin_bit_cast(f16x2, hi), f32x2);
    ha = h[0];
    hb = h[1];
  }
  lo = pack2<T>(fmaf(pa, xa, -ha), fmaf(pb, xb, -hb));
}
// head + remainder of four values: elements 0-3 the heads, 4-7 the remainders
template <typename T> __device__ __forceinline__ typename Vec<T>::x8 split4(const AccK32& a) {
  uint32_t h0, l0, h1, l1;
  split2<T>(a[0], a[1], h0, l0);
  split2<T>(a[2], a[3], h1, l1);
  return __builtin_bit_cast(typename Vec<T>::x8, u32x4{h0, h1, l0, l1});
}
// word j of an 8 x 16-bit operand
template <typename V> __device__ __forceinline__ void set_word(V& v, int j, uint32_t w) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
  u[j] = w;
  v = __builtin_bit_cast(V, u);
}

template <typename V> __device__ __forceinline__ V zero_vec() {
  V z;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(V) / sizeof(z[0])); ++i) z[i] = 0;
  return z;
}

// Workgroup id -> logical tile id. Consecutive workgroup ids are dispatched
// round-robin over the 8 XCDs; this remap gives each XCD a contiguous range
// of logical tiles, so the query tiles of one head share that XCD's L2.
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t id, uint32_t n) {
  const uint32_t per = n >> 3, rem = n & 7u, x = id & 7u, j = id >> 3;
  return x * per + (x < rem ? x : rem) + j;
}

__device__ __forceinline__ int clamp_len(const int32_t* key_len, int b, int S) {
  if (!key_len) return S;
  int L = key_len[b];
  return L < 0 ? 0 : (L > S ? S : L);
}

}  // namespace mha
