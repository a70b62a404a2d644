// RoPE arithmetic shared by the standalone RoPE kernel and the attention kernels that rotate
// their operands in registers ("[论文解读] World Model on Million-Length Video And Language With
// Blockwise RingAttention", section 提出的方法: RoPE with theta scaled to the context length).
// One formula in one place, so a fused rotation gives the same bits as the standalone kernel.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace lwm {

// Cosine and sine of pos * inv_freq.  The angle is formed in double precision (at positions
// near 1e6 a single-precision angle would be off by about 0.06 rad) and reduced there to
// r = angle - k*pi/2 with |r| <= pi/4; sin r and cos r come from their Taylor series to degree
// 11 and 12 (truncation below 1e-11 on that interval), still in double, and are rounded to
// single precision once; the quadrant k mod 4 then permutes and negates them.  Straight-line
// code with no large-argument path, so it unrolls cheaply inside the attention kernels.
__device__ inline void rope_cos_sin(int64_t pos, double inv_freq, float& c, float& s) {
  const double ang = (double)pos * inv_freq;
  const double k = rint(ang * 0.6366197723675814);  // 2/pi
  double r = fma(-k, 1.5707963267948966, ang);      // pi/2, high part
  r = fma(-k, 6.123233995736766e-17, r);            // pi/2, low part
  const double r2 = r * r;
  const double sp =
      fma(r * r2,
          fma(r2, fma(r2, fma(r2, fma(r2, -1.0 / 39916800.0, 1.0 / 362880.0), -1.0 / 5040.0), 1.0 / 120.0), -1.0 / 6.0),
          r);
  const double cp =
      fma(r2,
          fma(r2,
              fma(r2, fma(r2, fma(r2, fma(r2, 1.0 / 479001600.0, -1.0 / 3628800.0), 1.0 / 40320.0), -1.0 / 720.0),
                  1.0 / 24.0),
              -0.5),
          1.0);
  const float sr = (float)sp, cr = (float)cp;
  const int q = (int)((int64_t)k & 3);  // angle = q*pi/2 + r (mod 2*pi)
  const float cq = (q & 1) ? sr : cr, sq = (q & 1) ? cr : sr;
  c = (q == 1 || q == 2) ? -cq : cq;
  s = (q >= 2) ? -sq : sq;
}

// The pair (a, b) rotated by the angle whose cosine and sine are c and s.
__device__ __forceinline__ void rope_rotate(float a, float b, float c, float s, float& ra, float& rb) {
  ra = __builtin_fmaf(a, c, -(b * s));
  rb = __builtin_fmaf(a, s, b * c);
}

// RoPE position of row r0 + lane % 32 of an operand with n rows whose segment ids are seg_row
// (non-decreasing): offset + row, or with `restart` offset + row - (first row of its segment).
// Every lane of the wave must call it with the same r0 (rows at or past n get some position).
__device__ inline int64_t rope_row_position(const int32_t* seg_row, int n, int r0, bool restart, int64_t offset) {
  const int c = threadIdx.x & 31;
  const int r = r0 + c;
  if (!restart || r0 >= n) return offset + r;
  const int rc = min(r, n - 1), rp = max(rc - 1, 0);  // both in [0, n)
  const int first0 = wave_lower_bound(seg_row, n, seg_row[r0]);  // start of the segment of row r0
  // rows of this wave (after r0) where a new segment begins; the nearest one at or before r is
  // the start of r's segment, else r shares row r0's segment
  const int32_t here = seg_row[rc], before = seg_row[rp];
  const bool starts = (c > 0) && (r < n) && (here != before);
  const uint32_t m = (uint32_t)__ballot(starts);
  const uint32_t upto = c == 31 ? m : (m & ((2u << c) - 1u));
  const int first = upto ? r0 + (31 - __clz(upto)) : first0;
  return offset + (r - first);
}

}  // namespace lwm

namespace lwm {

// Rotate one row held as eight bf16x8 MFMA operand fragments, fragment s = features
// 16s + 8h .. 16s + 8h + 7 (h = lane / 32), rounding the result to bf16 (nearest even) like the
// standalone kernel.  The frequency table is indexed per lane (h varies across the wave), so it is
// read with vector loads where it is used rather than held in scalar registers.
__device__ inline void rope_rotate_frags(bf16x8 (&x)[8], int64_t pos, const RopeFuse& r, int h) {
  u32x4 w[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) w[s] = as_u32x4(x[s]);
  if (r.layout == 0) {
    // pairs (i, i + 64): fragment s (< 4) with fragment s + 4, same element
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float a[2], b[2];
        a[0] = bf16_lo(w[s][k]); a[1] = bf16_hi(w[s][k]);
        b[0] = bf16_lo(w[s + 4][k]); b[1] = bf16_hi(w[s + 4][k]);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int i0 = 16 * s + 2 * k + e;  // frequency index for h = 0; h = 1 adds 8
          float c, sn;
          rope_cos_sin(pos, r.inv_freq[i0 + 8 * h], c, sn);
          rope_rotate(a[e], b[e], c, sn, a[e], b[e]);
        }
        w[s][k] = pack_bf16x2(a[0], a[1]);
        w[s + 4][k] = pack_bf16x2(b[0], b[1]);
      }
  } else {
    // pairs (2i, 2i + 1): the two halves of each 32-bit word
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float a = bf16_lo(w[s][k]), b = bf16_hi(w[s][k]);
        const int i0 = 8 * s + k;  // h = 1 adds 4
        float c, sn;
        rope_cos_sin(pos, r.inv_freq[i0 + 4 * h], c, sn);
        rope_rotate(a, b, c, sn, a, b);
        w[s][k] = pack_bf16x2(a, b);
      }
  }
#pragma unroll
  for (int s = 0; s < 8; ++s) x[s] = as_bf16x8(w[s]);
}

// Inverse rotation (by -angle) of a 32-row block held as 32x32 MFMA accumulators, acc[db]
// element i of lane l = feature db*32 + acc_row(i, l / 32) of row l % 32, in float32.
__device__ inline void rope_unrotate_acc(f32x16 (&acc)[4], int64_t pos, const RopeFuse& r, int h) {
  if (r.layout == 0) {
    // pairs (f, f + 64): acc[db] with acc[db + 2], same element
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int f0 = db * 32 + 8 * (i >> 2) + (i & 3);  // h = 1 adds 4
        float c, sn;
        rope_cos_sin(pos, r.inv_freq[f0 + 4 * h], c, sn);
        float x0, x1;
        rope_rotate(acc[db][i], acc[db + 2][i], c, -sn, x0, x1);
        acc[db][i] = x0;
        acc[db + 2][i] = x1;
      }
  } else {
    // pairs (f, f + 1), f even: elements i and i + 1 for i % 4 in {0, 2}
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const int i0 = db * 16 + 4 * (i >> 2) + ((i & 3) >> 1);  // (feature / 2) for h = 0; h = 1 adds 2
        float c, sn;
        rope_cos_sin(pos, r.inv_freq[i0 + 2 * h], c, sn);
        float x0, x1;
        rope_rotate(acc[db][i], acc[db][i + 1], c, -sn, x0, x1);
        acc[db][i] = x0;
        acc[db][i + 1] = x1;
      }
  }
}

}  // namespace lwm
