// Tile helpers shared by the attention kernels (forward, ring step, backward): LDS layouts of
// K/V/Q/dO tiles, workgroup ordering, visibility ranges and the LDS-staged row stores.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace lwm {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int D = kHeadDim;

// ---------------------------------------------------------------- direct-to-LDS tiles (CDNA4)
// A tile is R rows (keys or queries) x 128 bf16 features, row-major, one 256-byte row per key:
// exactly one row of the 64 x 4-byte LDS banks.  The sixteen 16-byte chunks of row r are stored
// at chunk c ^ swz16(r): the 16 rows read by one MFMA operand fetch (ds_read_b128) hit 16
// distinct chunk slots, and so do the 4 rows x 4 chunks read by one 32-lane half of a
// transposing read (ds_read_b64_tr_b16).
__device__ __forceinline__ int swz16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Buffer resource over [base, base + bytes): loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = (int)imax64(0, imin64(bytes, 0x7fffffff));  // a scalar: base and size are uniform
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// 16 bytes per lane from rsrc + voffset straight into LDS at lds_base + 16 * lane (the wave's
// 1 KB block); no registers involved.  lds_base must be wave-uniform.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds_base, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voffset, 0, 0, 0);
}
// 4 bytes per lane, LDS at lds_base + 4 * lane.
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t r, void* lds_base, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 4, voffset, 0, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Block-wide barrier that waits for nothing by itself: each wave first waits for exactly the
// loads and LDS reads it must see finished (__syncthreads also drains every load still in
// flight, including those of tiles further ahead).  The memory clobber keeps LDS accesses on
// their side of it.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }
// Wait until this wave's LDS reads (and other LGKM operations) have completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Wait until at most n (0, 1 or 2) later groups of L vector-memory operations are in flight.
template <int L>
__device__ __forceinline__ void wait_groups(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<L>(); break;
    default: wait_vmcnt<2 * L>(); break;
  }
}

// MFMA A operand "X^T" (32 features x 16 rows of X) read from a row-major swizzled tile with two
// transposing reads.  Lane l receives feature db*32 + l%32 of rows g*16 + 4*(l/32) + {0..3} and
// g*16 + 8 + 4*(l/32) + {0..3}: the row order of a 32x32 accumulator's lane half, so the B operand
// can be packed straight from accumulator registers.  `off` comes from tr_offsets().
__device__ __forceinline__ bf16x8 read_xt(const uint8_t* tile, int off_lo, int off_hi) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + off_lo));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + off_hi));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
// Byte offsets (within a tile, group g = 0) of this lane's two transposing reads for feature
// block db.  Within each 16-lane group, lane 4j + r points at row j, features 4r..4r+3 of its
// group's slice, so that lane 4r + c receives feature 4r + c of rows j = 0..3.
__device__ __forceinline__ void tr_offsets(int lane, int db, int& off_lo, int& off_hi) {
  const int gp = lane >> 4, j = (lane >> 2) & 3, r = lane & 3;
  const int col = db * 32 + 16 * (gp & 1) + 4 * r;  // first feature of this lane's 8 bytes
  const int chunk = col >> 3, sub = (col & 7) * 2;
  const int row_lo = 4 * (gp >> 1) + j, row_hi = row_lo + 8;
  off_lo = row_lo * 256 + ((chunk ^ swz16(row_lo)) << 4) + sub;
  off_hi = row_hi * 256 + ((chunk ^ swz16(row_hi)) << 4) + sub;
}

// ---------------------------------------------------------------- workgroup order
// Grid position -> (batch*head, tile).  `descending` numbers tiles from the last one (causal
// forward: the longest query tiles first); otherwise from the first (backward over keys: the
// earliest keys have the most queries).  When B*H is a multiple of 8, block ids congruent mod 8
// (dispatched to the same XCD) stay on their own (batch, head) pairs.  Head-major (`tile_major`
// false): an XCD walks one head's tiles in order, so its resident workgroups share that head's
// K/V in L2 and, under a causal mask, run longest first.  Tile-major: consecutive block ids take
// one tile of every (batch, head) before the next tile.  Used for packed rows, where a tile's work
// is its position inside its segment, not its index: dealing each tile to all heads at once
// spreads the long tiles of every segment over the launch instead of leaving some for its end.
__device__ __forceinline__ void map_block(int bid, int ntiles, int BH, bool descending, bool tile_major, int& bh,
                                          int& t) {
  int slot_t;
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3, per = BH >> 3;
    if (tile_major) {
      bh = (slot % per) * 8 + xcd;
      slot_t = slot / per;
    } else {
      bh = (slot / ntiles) * 8 + xcd;
      slot_t = slot % ntiles;
    }
  } else if (tile_major) {
    bh = bid % BH;
    slot_t = bid / BH;
  } else {
    bh = bid / ntiles;
    slot_t = bid % ntiles;
  }
  t = descending ? ntiles - 1 - slot_t : slot_t;
}

// True when the query and key sides share one segment-id array and one global offset under the
// causal mask (packed self-attention).  Then the segment of a query row reaches at least that row
// and the segment of a key starts no later than that key, so of each segment range one bound is
// already implied by the causal limit and only the other needs a search.
__device__ __forceinline__ bool causal_self_segments(const int32_t* seg_q, const int32_t* seg_k, int Lq, int Lk,
                                                     int64_t q_offset, int64_t k_offset, int causal) {
  return causal && seg_q == seg_k && Lq == Lk && q_offset == k_offset;
}

// Index range [lo, hi) of the rows of `other` (length n_other, segment ids seg_other) that can
// share a segment with rows whose ids run from s_first to s_last (ids non-decreasing).
__device__ inline void segment_range(const int32_t* seg_other, int n_other, int32_t s_first, int32_t s_last,
                                     int& lo, int& hi) {
  lo = wave_lower_bound(seg_other, n_other, s_first);
  hi = (s_last == INT32_MAX) ? n_other : wave_lower_bound(seg_other, n_other, s_last + 1);
}

// ---------------------------------------------------------------- LDS-staged row I/O
// A wave's 32x128 accumulator (one 32-row block of an output whose rows are the lanes' columns,
// features in the accumulator rows) is transposed through a wave-private LDS area so that global
// stores are whole 16-byte chunks of contiguous rows.  `stage` needs 32*128*4 bytes (fp32) or
// half of that (bf16).  Contains block-wide barriers: every wave of the block must call it.
__device__ inline void store_rows_bf16(uint8_t* stage, const f32x16 (&acc)[4], const float mul, uint16_t* gbase,
                                       int64_t row_stride, int rows_valid) {
  const int lane = threadIdx.x & 63, c32 = lane & 31, h32 = lane >> 5;
  u32x2* st2 = reinterpret_cast<u32x2*>(stage);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int chunk = db * 4 + g;  // features db*32 + 8g .. +7; this lane half holds 4 of them
      u32x2 w;
      w.x = pack_bf16x2(acc[db][g * 4 + 0] * mul, acc[db][g * 4 + 1] * mul);
      w.y = pack_bf16x2(acc[db][g * 4 + 2] * mul, acc[db][g * 4 + 3] * mul);
      st2[(c32 * 16 + (chunk ^ (c32 & 15))) * 2 + h32] = w;
    }
  __syncthreads();
  const u32x4* st4 = reinterpret_cast<const u32x4*>(stage);
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int r = it * 4 + (lane >> 4), c = lane & 15;
    if (r < rows_valid) *reinterpret_cast<u32x4*>(gbase + r * row_stride + c * 8) = st4[r * 16 + (c ^ (r & 15))];
  }
  __syncthreads();
}

__device__ inline void store_rows_f32(uint8_t* stage, const f32x16 (&acc)[4], const float mul, float* gbase,
                                      int64_t row_stride, int rows_valid) {
  const int lane = threadIdx.x & 63, c32 = lane & 31, h32 = lane >> 5;
  f32x4* st = reinterpret_cast<f32x4*>(stage);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int chunk = db * 8 + g * 2 + h32;
      f32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = acc[db][g * 4 + j] * mul;
      st[c32 * 32 + (chunk ^ (c32 & 31))] = w;
    }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int r = it * 2 + (lane >> 5), c = lane & 31;
    if (r < rows_valid) *reinterpret_cast<f32x4*>(gbase + r * row_stride + c * 4) = st[r * 32 + (c ^ (r & 31))];
  }
  __syncthreads();
}

__device__ inline void load_rows_f32(uint8_t* stage, f32x16 (&acc)[4], const float* gbase, int64_t row_stride,
                                     int rows_valid) {
  const int lane = threadIdx.x & 63, c32 = lane & 31, h32 = lane >> 5;
  f32x4* st = reinterpret_cast<f32x4*>(stage);
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int r = it * 2 + (lane >> 5), c = lane & 31;
    f32x4 w = {0.f, 0.f, 0.f, 0.f};
    if (r < rows_valid) w = *reinterpret_cast<const f32x4*>(gbase + r * row_stride + c * 4);
    st[r * 32 + (c ^ (r & 31))] = w;
  }
  __syncthreads();
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int chunk = db * 8 + g * 2 + h32;
      const f32x4 w = st[c32 * 32 + (chunk ^ (c32 & 31))];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[db][g * 4 + j] = w[j];
    }
  __syncthreads();
}

// gbase rows += acc * mul (32 fp32 rows, row stride in elements), staged through LDS both ways
// like load_rows_f32 / store_rows_f32.  Contains block-wide barriers: every wave must call it.
__device__ inline void add_rows_f32(uint8_t* stage, const f32x16 (&acc)[4], const float mul, float* gbase,
                                    int64_t row_stride, int rows_valid) {
  f32x16 t[4];
  load_rows_f32(stage, t, gbase, row_stride, rows_valid);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) t[db][i] = __builtin_fmaf(acc[db][i], mul, t[db][i]);
  store_rows_f32(stage, t, 1.f, gbase, row_stride, rows_valid);
}

// Pack 8 consecutive accumulator elements (u*8 .. u*8+7) into one bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 pack8(const f32x16& s, int u) {
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(s[u * 8 + 2 * j], s[u * 8 + 2 * j + 1]);
  return as_bf16x8(w);
}

}  // namespace lwm
