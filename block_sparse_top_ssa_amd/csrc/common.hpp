// Shared device helpers for the SSA kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round-to-nearest-even float -> bf16 (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Two floats to packed bf16 (one v_cvt_pk_bf16_f32, nearest-even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}
// 2^x with the hardware v_exp_f32 (results below 2^-126 may flush to zero).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Element access for the two I/O types: float, or bf16 held as uint16_t bits.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPer16B = 4;
  __device__ static __forceinline__ void unpack(const u32x4& w, float* out) {
    out[0] = __uint_as_float(w[0]); out[1] = __uint_as_float(w[1]);
    out[2] = __uint_as_float(w[2]); out[3] = __uint_as_float(w[3]);
  }
  __device__ static __forceinline__ u32x4 pack(const float* in) {
    u32x4 w; w[0] = __float_as_uint(in[0]); w[1] = __float_as_uint(in[1]);
    w[2] = __float_as_uint(in[2]); w[3] = __float_as_uint(in[3]); return w;
  }
  __device__ static __forceinline__ float load1(const float* p) { return *p; }
  __device__ static __forceinline__ void store1(float* p, float x) { *p = x; }
};
template <> struct Elem<uint16_t> {
  static constexpr int kPer16B = 8;
  __device__ static __forceinline__ void unpack(const u32x4& w, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { out[2 * i] = lo_bf16(w[i]); out[2 * i + 1] = hi_bf16(w[i]); }
  }
  __device__ static __forceinline__ u32x4 pack(const float* in) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(in[2 * i], in[2 * i + 1]);
    return w;
  }
  __device__ static __forceinline__ float load1(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  __device__ static __forceinline__ void store1(uint16_t* p, float x) { *p = (uint16_t)f32_to_bf16_bits(x); }
};

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void store16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// Logical workgroup id such that consecutive logical ids run on the same XCD (the
// dispatcher hands workgroup i to XCD i % 8): XCD x gets logical ids
// [x*G/8, (x+1)*G/8) in order.  Identity when G is not a multiple of 8.
__device__ __forceinline__ int64_t xcd_logical(int64_t i, int64_t G) {
  if (G % 8) return i;
  return (i % 8) * (G / 8) + i / 8;
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
// Max over the four lanes l, l^16, l^32, l^48 (one per 16-lane row) with the gfx950
// row-swap permutes: VALU only, no LDS round trip.  Each swap exchanges alternate
// rows (16 or 32 lanes) between two copies of x, so the two results hold both
// partners of every pair.
__device__ __forceinline__ float max_over_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// Sum over the same four lanes, in the order (x0 + x1) + (x2 + x3) of their rows, which
// every lane of the group gets bit for bit.
__device__ __forceinline__ float sum_over_rows(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  lo = __shfl_xor(lo, m);
  hi = __shfl_xor(hi, m);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_u64(uint64_t x, int src) {
  uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  lo = __shfl(lo, src);
  hi = __shfl(hi, src);
  return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------- attention distance buckets
// Bucket of a block distance d = b_t - b_i: 0 for the own block, 1 + floor(log2 d) for
// d >= 1, the last of the kDistBuckets buckets also collecting everything beyond.
constexpr int kDistBuckets = 16;
__device__ __forceinline__ int dist_bucket(int d) {
  if (d <= 0) return 0;
  return min(32 - __clz(d), kDistBuckets - 1);  // 1 + floor(log2 d)
}

// ---------------------------------------------------------------- selection keys
// 64-bit key ordering candidates by (score descending, block index ascending):
// high word = order-preserving image of the float score (-0 folded onto +0),
// low word = 0xFFFFFFFF - j.  Key 0 is below every real candidate.
__device__ __forceinline__ uint32_t orderable_f32(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unorderable_f32(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
__device__ __forceinline__ uint64_t make_key(float score, int j) {
  return ((uint64_t)orderable_f32(score) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}
__device__ __forceinline__ int key_index(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }
__device__ __forceinline__ float key_score(uint64_t key) { return unorderable_f32((uint32_t)(key >> 32)); }

// ---------------------------------------------------------------- sparse rows that are full rows
// Whether one row's idx list keeps every block below its own block b_t: its valid
// entries (ascending, each in [0, b_t) and above the entry used before it -- the entries
// the sparse kernels use) number b_t.  The sparse stream of such a row is plain causal
// attention (paper sec. 3, p. 4: with every preceding block kept, nothing is dropped).
__device__ __forceinline__ bool row_keeps_all(const int32_t* __restrict__ ir, int topk, int bt) {
  if (bt > topk) return false;
  int prev = -1, kept = 0;
  for (int e = 0; e < topk; ++e) {
    const int j = ir[e];
    if (j > prev && j < bt) {
      prev = j;
      ++kept;
    }
  }
  return kept == bt;
}

}  // namespace ssa
