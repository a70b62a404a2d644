// Device helpers shared by the gfx950 kernels: vector types, bf16 packing, MFMA wrappers,
// wave-level reductions and searches.  Written for CDNA4 wave64 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lwm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ bf16 <-> f32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 p;
  p.x = (__bf16)lo;
  p.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

// acc + lo + hi of a packed bf16 pair (v_dot2_f32_bf16 against (1, 1)).  Takes the pair as a
// scalar word: feeding it an element of a vector through bit_cast has been lowered to the wrong
// register by this compiler.
__device__ __forceinline__ float sum_bf16x2(uint32_t pair, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x2 v;
  __builtin_memcpy(&v, &pair, sizeof(v));
  return __builtin_amdgcn_fdot2_f32_bf16(v, ones, acc, false);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// ------------------------------------------------------------------ MFMA
// D(32x32 f32) += A(32x16 bf16) * B(16x32 bf16).  Lane l holds A row (l % 32), k = 8*(l/32)..+7;
// B column (l % 32), same k; accumulator element i of lane l is row 8*(i/4) + 4*(l/32) + i%4,
// column l % 32.
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D(32x32 f32) += A(32x2 f32) * B(2x32 f32).  Lane l holds A row (l % 32), k = l/32.
__device__ __forceinline__ f32x16 mfma_32x32x2_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row of the 32x32 accumulator held by element i of a lane in half `h` (= lane / 32).
__device__ __forceinline__ constexpr int acc_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// ------------------------------------------------------------------ cross-lane
// Value held by lane (l ^ 32).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, kWave);
}

// max / sum of x over the lane pair (l, l ^ 32), in every lane.  v_permlane32_swap exchanges the
// two 32-lane halves between its two operands, so combining the two results pairs each lane with
// its partner, whichever half each operand ends up holding; no LDS round trip.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Integer min / max for 64-bit values (the generic overloads may go through double).
__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t imax64(int64_t a, int64_t b) { return a > b ? a : b; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ------------------------------------------------------------------ searches over segment ids
// First index p in [0, n) with a[p] >= value (n if none), for non-decreasing a.  Every lane
// of the wave must call it with the same arguments; all lanes return the same result.
// A 64-ary search: each round samples 64 evenly spaced positions and keeps the bracket.
__device__ inline int wave_lower_bound(const int32_t* __restrict__ a, int n, int32_t value) {
  const int lane = threadIdx.x & (kWave - 1);
  int lo = 0, hi = n;
  while (lo < hi) {
    const int span = hi - lo;
    const int step = (span + kWave - 1) / kWave;
    const int p = lo + lane * step;
    const bool valid = p < hi;
    const bool below = valid && (a[p] < value);
    const uint64_t below_mask = __ballot(below);
    const uint64_t valid_mask = __ballot(valid);
    const int cnt = __popcll(below_mask);
    const int nvalid = __popcll(valid_mask);
    if (cnt == 0) {
      hi = lo;
    } else {
      const int last_below = lo + (cnt - 1) * step;
      const int new_hi = (cnt < nvalid) ? (lo + cnt * step) : hi;
      lo = last_below + 1;
      hi = new_hi;
    }
  }
  return lo;
}

}  // namespace lwm
