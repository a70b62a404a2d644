// Blockwise attention backward for gfx950 (bf16 operands, float32 accumulation).
//
// For the loss sum(dO * O) of the forward defined in include/lwm_attn.h (causal: "Inside Large
// World Model ...", section "Core Architecture"; packing: "LWM：突破 100 万 Token 的开源大模型",
// section 概述 (b); blockwise evaluation: the same page, section 配置参数), with
// P = exp(S - lse) recomputed from the forward's saved logsumexp:
//     delta_i = sum_d dO_id O_id
//     dV = P^T dO,   dP = dO V^T,   dS = P o (dP - delta),   dQ = scale dS K,   dK = scale dS^T Q.
//
// No atomics (the result is deterministic).  With room for it in the workspace the backward stores
// dS: the dK/dV kernel below also writes dS^T (bf16) and a dQ kernel forms dQ = scale dS K from it
// (five products in all); otherwise the dQ kernel recomputes S and dP itself (seven).  The two
// paths give the same bits.  Kernels:
//  * delta: one pass over dO and O (HBM-bound); also stores lse * log2(e) for the other two.
//  * dQ: a workgroup per 128-query tile walks the visible 64-key tiles like the forward does,
//    with scores transposed (S^T = K Q^T) so each lane owns one query: P^T and dS^T are formed in
//    registers and feed dQ^T += K^T dS^T directly; K^T operands come from the row-major K tile by
//    transposing LDS reads.
//  * dK/dV: a workgroup per 256-key tile (32 keys per wave, their K rows held in registers) walks
//    the visible 64-query tiles with scores in the other orientation (S = Q K^T, each lane owns one
//    key): P and dS feed dV^T += dO^T P and dK^T += Q^T dS directly; Q^T and dO^T operands come from
//    the row-major tiles by transposing LDS reads.
//  With fused RoPE (lwm_blockattn_bwd_rope) the dQ and dK/dV kernels rotate their float32 dQ', dK'
//  accumulators back by -angle just before the one rounding to bf16, so the stored gradients are
//  w.r.t. the pre-RoPE Q and K.
//  * dQ from the stored dS: a workgroup per 256-query tile streams K and dS^T tiles through LDS
//    and forms dQ^T += K^T dS^T only (bound by memory: two bytes of dS per visible pair).
//  Tiles travel HBM -> LDS by buffer loads that write LDS directly.  Neither path writes or
//  reduces a partial dQ through memory.

#include <cstddef>
#include <type_traits>

#include "attn_common.hpp"
#include "profile.hpp"
#include "rope_dev.hpp"

namespace lwm {
namespace {

constexpr int kTileBytes = 64 * 256;  // 64 rows x 128 bf16

// ------------------------------------------------------------------------------ delta
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams p) {
  const int64_t rows = (int64_t)p.B * p.Lq * p.H;
  const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  float acc = 0.f;
  int b = 0, i = 0, h = 0;
  if (r < rows) {
    h = (int)(r % p.H);
    const int64_t bi = r / p.H;
    i = (int)(bi % p.Lq);
    b = (int)(bi / p.Lq);
    const u32x4 x = *reinterpret_cast<const u32x4*>(p.dout + b * p.sdo.b + i * p.sdo.l + h * p.sdo.h + c * 8);
    const u32x4 y = *reinterpret_cast<const u32x4*>(p.o + b * p.so.b + i * p.so.l + h * p.so.h + c * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc += bf16_lo(x[j]) * bf16_lo(y[j]) + bf16_hi(x[j]) * bf16_hi(y[j]);
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (r < rows && c == 0) {
    const int64_t at = ((int64_t)b * p.H + h) * p.Lq + i;
    p.delta[at] = acc;
    // rows without any visible key: +inf makes exp2(s - lse2) = 0 for every score
    const float ls = p.lse[at];
    p.lse2[at] = ls == -INFINITY ? INFINITY : ls * kLog2e;
  }
}

// ------------------------------------------------------------------------------ dQ
// A wave's dQ^T accumulator (query rows wr0 + lane, features in the accumulator rows) out to
// memory: added into dq_acc (backward ring step, float32), or rotated back when RoPE is fused and
// rounded once to bf16.  Every wave of the workgroup calls it (the row helpers have block-wide
// barriers); `stage_w` is 16 KB of LDS of the wave's own, free by then.
__device__ __forceinline__ void dq_epilogue(const BwdParams& p, uint8_t* stage_w, f32x16 (&acc)[4], int b, int hh,
                                            int wr0, int h32, bool segs) {
  const int rows_valid = max(0, min(32, p.Lq - wr0));
  if (p.dq_acc) {  // backward ring step: dQ += this shard's share, in float32
    add_rows_f32(stage_w, acc, p.scale, p.dq_acc + b * p.sdqa.b + hh * p.sdqa.h + wr0 * p.sdqa.l, p.sdqa.l,
                 rows_valid);
  } else {
    if (p.rope.on) {  // dQ' -> dQ (inverse RoPE of the query rows) before the one rounding to bf16
      const bool restart = segs && p.rope.restart;
      const int64_t pos = rope_row_position(restart ? p.seg_q + (int64_t)b * p.Lq : nullptr, p.Lq, wr0, restart,
                                            p.rope.q_pos_offset);
      rope_unrotate_acc(acc, pos, p.rope, h32);
    }
    store_rows_bf16(stage_w, acc, p.scale, p.dq + b * p.sdq.b + hh * p.sdq.h + wr0 * p.sdq.l, p.sdq.l, rows_valid);
  }
}

struct SmemDq {
  uint8_t kv[2][2][kTileBytes];  // [stage][K, V] row-major swizzled
  int32_t seg[2][64];
};
static_assert(sizeof(SmemDq) >= kWaves * 32 * D * 4, "epilogue staging (float32 rows) must fit");

__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdParams p) {
  constexpr int MW = 32, BM = kWaves * MW, BN = 64;
  __shared__ __attribute__((aligned(1024))) SmemDq sm;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, h32 = lane >> 5;
  const int nqt = (p.Lq + BM - 1) / BM;
  int lbh, qt;
  const bool segs = p.seg_q != nullptr;
  map_block(blockIdx.x, nqt, p.bh_count, true, segs, lbh, qt);
  const int bh = p.bh0 + lbh;
  const int b = bh / p.H, hh = bh - b * p.H;
  const int q0 = qt * BM;
  const int qlast = min(q0 + BM, p.Lq) - 1;

  // the wave's rows first (Q, dO, lse, delta): their loads are in flight during the key-range search
  const int wr0 = q0 + w * MW, wr1 = min(wr0 + MW, p.Lq) - 1;
  const bool wave_rows = wr1 >= wr0;
  const int qrow = wr0 + c32;
  const int64_t gq = p.q_offset + qrow;
  const int64_t row_at = ((int64_t)b * p.H + hh) * p.Lq + qrow;
  const float lse2 = qrow < p.Lq ? p.lse2[row_at] : INFINITY;
  const float dlt = qrow < p.Lq ? p.delta[row_at] : 0.f;
  bf16x8 qreg[8], doreg[8];
  {
    const uint16_t* qg = p.q + b * p.sq.b + hh * p.sq.h + (int64_t)qrow * p.sq.l;
    const uint16_t* dg = p.dout + b * p.sdo.b + hh * p.sdo.h + (int64_t)qrow * p.sdo.l;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
      if (qrow < p.Lq) {
        a = *reinterpret_cast<const u32x4*>(qg + s * 16 + h32 * 8);
        c = *reinterpret_cast<const u32x4*>(dg + s * 16 + h32 * 8);
      }
      qreg[s] = as_bf16x8(a);
      doreg[s] = as_bf16x8(c);
    }
  }

  int kbeg = 0, kend = p.Lk;
  if (p.causal) kend = (int)imax64(0, imin64(kend, p.q_offset + qlast - p.k_offset + 1));
  if (segs) {
    const int32_t* segk = p.seg_k + (int64_t)b * p.Lk;
    if (causal_self_segments(p.seg_q, p.seg_k, p.Lq, p.Lk, p.q_offset, p.k_offset, p.causal)) {
      kbeg = max(kbeg, wave_lower_bound(segk, p.Lk, segk[q0]));  // the causal limit ends the range
    } else {
      int lo, hi;
      segment_range(segk, p.Lk, p.seg_q[(int64_t)b * p.Lq + q0], p.seg_q[(int64_t)b * p.Lq + qlast], lo, hi);
      kbeg = max(kbeg, lo);
      kend = min(kend, hi);
    }
  }
  const int t_begin = kbeg / BN;
  const int ntiles = (kend > kbeg) ? (kend + BN - 1) / BN - t_begin : 0;
  int32_t wseg0 = 0, wseg1 = 0;
  if (segs && wave_rows) {
    wseg0 = p.seg_q[(int64_t)b * p.Lq + wr0];
    wseg1 = p.seg_q[(int64_t)b * p.Lq + wr1];
  }
  const int32_t myseg = segs ? p.seg_q[(int64_t)b * p.Lq + min(qrow, p.Lq - 1)] : 0;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.k + b * p.sk.b + hh * p.sk.h);
  const uint8_t* vg = reinterpret_cast<const uint8_t*>(p.v + b * p.sv.b + hh * p.sv.h);
  const int64_t kl_bytes = p.sk.l * 2, vl_bytes = p.sv.l * 2;
  const int64_t k_extent = (int64_t)(p.Lk - 1) * kl_bytes + 256, v_extent = (int64_t)(p.Lk - 1) * vl_bytes + 256;
  const int32_t* segk_row = segs ? p.seg_k + (int64_t)b * p.Lk : nullptr;
  int ld_voff_k[4], ld_voff_v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = (w * 4 + r) * 4 + (lane >> 4);
    const int c = (lane & 15) ^ swz16(row);
    ld_voff_k[r] = (int)(row * kl_bytes) + c * 16;
    ld_voff_v[r] = (int)(row * vl_bytes) + c * 16;
  }
  auto issue = [&](int tile, int st) {
    const int k0 = tile * BN;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + k0 * kl_bytes, k_extent - k0 * kl_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + k0 * vl_bytes, v_extent - k0 * vl_bytes);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      load_lds16(rk, &sm.kv[st][0][(w * 4 + r) * 1024], ld_voff_k[r]);
      load_lds16(rv, &sm.kv[st][1][(w * 4 + r) * 1024], ld_voff_v[r]);
    }
    if (segs && w == 0) load_lds4(make_rsrc(segk_row + k0, (int64_t)(p.Lk - k0) * 4), &sm.seg[st][0], lane * 4);
  };
  // K / V row-major operand for feature step sd (+8192 for the second key block): the XOR swizzle
  // leaves bit 0 of an even chunk index alone, so the offset is a per-lane base plus
  // ((2*sd) ^ swizzle) * 16.  K^T operands for feature block db (+4096 per 16-key group) differ
  // from block 0's offsets by an XOR of db into chunk bits 2..3.
  const int rswz = swz16(c32 & 15);
  const int rbase = c32 * 256 + (((h32 ^ rswz) & 1) << 4);
  auto roff = [&](int sd) { return rbase + (((2 * sd) ^ (rswz & 14)) << 4); };
  int tlo0, thi0;
  tr_offsets(lane, 0, tlo0, thi0);

  if (ntiles > 0) issue(t_begin, 0);
  auto tile = [&](int st, int it) {
    const int k0 = (t_begin + it) * BN;
    wait_vmcnt<0>();
    __syncthreads();
    if (it + 1 < ntiles) issue(t_begin + it + 1, st ^ 1);
    const uint8_t* kt = sm.kv[st][0];
    const uint8_t* vt = sm.kv[st][1];
    bool active = wave_rows;
    bool need_mask = (k0 + BN > p.Lk) || (k0 < kbeg) || (k0 + BN > kend);
    if (p.causal) {
      active = active && (p.k_offset + k0 <= p.q_offset + wr1);
      need_mask = need_mask || (p.k_offset + k0 + BN - 1 > p.q_offset + wr0);
    }
    if (segs) {
      const int32_t ts0 = sm.seg[st][0], ts1 = sm.seg[st][min(BN, p.Lk - k0) - 1];
      active = active && !(ts1 < wseg0 || ts0 > wseg1);
      need_mask = need_mask || !(ts0 == ts1 && wseg0 == wseg1 && ts0 == wseg0);
    }
    if (!active) return;

    // S^T = K Q^T and dP^T = V dO^T, one key block at a time; operands read one step ahead
    bf16x8 dsb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
      bf16x8 fk[2], fv[2];
      fk[0] = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + kb * 8192 + roff(0)));
      fv[0] = as_bf16x8(*reinterpret_cast<const u32x4*>(vt + kb * 8192 + roff(0)));
#pragma unroll
      for (int sd = 0; sd < 8; ++sd) {
        if (sd + 1 < 8) {
          fk[(sd + 1) & 1] = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + kb * 8192 + roff(sd + 1)));
          fv[(sd + 1) & 1] = as_bf16x8(*reinterpret_cast<const u32x4*>(vt + kb * 8192 + roff(sd + 1)));
        }
        __builtin_amdgcn_sched_barrier(0);
        s = mfma_32x32x16(fk[sd & 1], qreg[sd], s);
        dp = mfma_32x32x16(fv[sd & 1], doreg[sd], dp);
        __builtin_amdgcn_sched_barrier(0);
      }
      // masked scores get exponent -inf (a select, not a branch): exp2(-inf) = 0
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = __builtin_fmaf(s[i], p.scale_log2, -lse2);
      if (need_mask) {
        // element i holds tile key kl = kb*32 + 8*(i/4) + 4*h32 + i%4, visible iff kl < lim (end of
        // the keys, causal limit) and its segment matches this lane's query
        int64_t lim64 = (int64_t)p.Lk - k0;
        if (p.causal) lim64 = imin64(lim64, gq - p.k_offset - k0 + 1);
        const int lim = (int)imax64(imin64(lim64, BN), 0) - kb * 32 - 4 * h32;
        const int32_t* segt = &sm.seg[st][kb * 32 + 4 * h32];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          i32x4 ks = {myseg, myseg, myseg, myseg};
          if (segs) ks = *reinterpret_cast<const i32x4*>(segt + 8 * g);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool vis = (8 * g + j < lim) & (ks[j] == myseg);
            x[4 * g + j] = vis ? x[4 * g + j] : -INFINITY;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = fast_exp2(x[i]) * (dp[i] - dlt);
      dsb[kb][0] = pack8(s, 0);
      dsb[kb][1] = pack8(s, 1);
    }
    // dQ^T += K^T dS^T (K^T operands by transposing reads, two ahead)
    {
      bf16x8 kf[3];
      auto kread = [&](int n) { return read_xt(kt + (n >> 2) * 4096, tlo0 ^ ((n & 3) << 6), thi0 ^ ((n & 3) << 6)); };
      kf[0] = kread(0);
      kf[1] = kread(1);
#pragma unroll
      for (int n = 0; n < 16; ++n) {  // n = 16-key group * 4 + feature block
        if (n + 2 < 16) kf[(n + 2) % 3] = kread(n + 2);
        __builtin_amdgcn_sched_barrier(0);
        const int g = n >> 2, db = n & 3;
        acc[db] = mfma_32x32x16(kf[n % 3], dsb[g >> 1][g & 1], acc[db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (int it = 0; it < ntiles; ++it) tile(it & 1, it);
  __syncthreads();
  dq_epilogue(p, reinterpret_cast<uint8_t*>(&sm) + w * (32 * D * 4), acc, b, hh, wr0, h32, segs);
}

// ------------------------------------------------------------------------------ dQ from stored dS
// When the dK/dV kernel has stored dS^T, dQ^T = scale K^T dS^T is one product over data already
// computed: a workgroup of 8 waves per 256-query tile walks the visible 64-key tiles, bringing
// the K tile and the matching 64 x 256 block of dS^T (rows = keys, queries along the row) into
// LDS by direct loads through a three-stage ring, two tiles ahead.  Both operands come out of LDS
// by transposing reads: K^T as in the dQ kernel above, and wave w's 32 queries of dS^T in the key
// order of a 32x32 accumulator's lane half.  The stored block holds dS for every pair the dK/dV
// kernel visited (zero where masked), not for pairs outside its ranges, so on tiles that need the
// mask every invisible pair is cleared before the product.  HBM-bound: two bytes of dS per
// visible pair are read once.
constexpr int kDsWaves = 8;
constexpr int kDsQueries = kDsWaves * 32;  // queries per workgroup
// Stored dS^T of one (batch, head) pair: blocks of 64 keys x 64 queries (8 KB), key block after
// key block, each the ds_ld / 64 query blocks in order, so the dK/dV kernel writes whole blocks
// per query tile and this kernel reads 32 KB in a row per key tile (plain rows of dS^T would
// scatter every write over as many rows).  Inside a block, 16-byte chunk j (queries 8j .. 8j + 7)
// of key r sits at byte j * 1024 + r * 16: one lane of the dK/dV kernel holds exactly such a chunk
// for its key (its LDS query rows are permuted by swap23 for that), so each of its stores is a
// whole 16-byte fragment and 32 lanes write 512 contiguous bytes.
constexpr int kDsBlock = 64;
constexpr int kDsBlockBytes = kDsBlock * kDsBlock * 2;
constexpr int kDsChunkBytes = kDsBlock * 16;  // one chunk of all 64 keys of a block
constexpr int kCachePolicyNT = 2;  // buffer instruction cache policy: non-temporal (gfx950 nt bit)
__device__ __forceinline__ int64_t ds_slot_bytes(const BwdParams& p) { return p.ds_slot_blocks * kDsBlockBytes; }
// Under the causal mask key block kb is seen by no query block before qlo(kb), so its row of
// blocks starts there; the rows follow each other without gaps.  Both in closed form (the same
// arithmetic as the host's workspace sizing).
__device__ __forceinline__ int64_t ds_qlo(const BwdParams& p, int64_t kb) {
  return imin64(imax64(kb + p.ds_shift, 0), p.ds_ld / kDsBlock);
}
// Blocks stored for key blocks 0 .. kb - 1.
__device__ __forceinline__ int64_t ds_row_start(const BwdParams& p, int64_t kb) {
  const int64_t nqb = p.ds_ld / kDsBlock, c = p.ds_shift;
  const int64_t a = imax64(0, -c), e = imax64(a, nqb - c);  // qlo = 0 below a, nqb from e on
  const int64_t m = imin64(imax64(kb, a), e);                // qlo = i + c for a <= i < m
  const int64_t lo_sum = (m - a) * c + (a + m - 1) * (m - a) / 2;
  return kb * nqb - (lo_sum + nqb * imax64(0, kb - e));
}
struct StageDs {
  uint8_t k[kTileBytes];                 // K rows, row-major swizzled
  uint8_t s[64 * kDsQueries * 2];        // dS^T rows (64 keys x 256 queries), 512 bytes per key
  int32_t seg[64];
};
template <int S>
using DsStage = std::integral_constant<int, S>;

__global__ __launch_bounds__(kDsWaves * kWave) void bwd_dq_ds_kernel(BwdParams p) {
  constexpr int MW = 32, BM = kDsQueries, BN = 64;
  __shared__ __attribute__((aligned(1024))) StageDs lds_s0;
  __shared__ __attribute__((aligned(1024))) StageDs lds_s1;
  __shared__ __attribute__((aligned(1024))) StageDs lds_s2;
  auto stage = [&](auto sc) __attribute__((always_inline)) -> StageDs& {
    if constexpr (decltype(sc)::value == 0) return lds_s0;
    else if constexpr (decltype(sc)::value == 1) return lds_s1;
    else return lds_s2;
  };
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, h32 = lane >> 5;
  const int nqt = (p.Lq + BM - 1) / BM;
  int lbh, qt;
  const bool segs = p.seg_q != nullptr;
  map_block(blockIdx.x, nqt, p.bh_count, true, segs, lbh, qt);
  const int bh = p.bh0 + lbh;
  const int b = bh / p.H, hh = bh - b * p.H;
  const int q0 = qt * BM;
  const int qlast = min(q0 + BM, p.Lq) - 1;
  const int wr0 = q0 + w * MW, wr1 = min(wr0 + MW, p.Lq) - 1;
  const bool wave_rows = wr1 >= wr0;
  const int64_t gq = p.q_offset + wr0 + c32;

  int kbeg = 0, kend = p.Lk;
  if (p.causal) kend = (int)imax64(0, imin64(kend, p.q_offset + qlast - p.k_offset + 1));
  if (segs) {
    const int32_t* segk = p.seg_k + (int64_t)b * p.Lk;
    if (causal_self_segments(p.seg_q, p.seg_k, p.Lq, p.Lk, p.q_offset, p.k_offset, p.causal)) {
      kbeg = max(kbeg, wave_lower_bound(segk, p.Lk, segk[q0]));
    } else {
      int lo, hi;
      segment_range(segk, p.Lk, p.seg_q[(int64_t)b * p.Lq + q0], p.seg_q[(int64_t)b * p.Lq + qlast], lo, hi);
      kbeg = max(kbeg, lo);
      kend = min(kend, hi);
    }
  }
  const int t_begin = kbeg / BN;
  const int ntiles = (kend > kbeg) ? (kend + BN - 1) / BN - t_begin : 0;
  int32_t wseg0 = 0, wseg1 = 0;
  if (segs && wave_rows) {
    wseg0 = p.seg_q[(int64_t)b * p.Lq + wr0];
    wseg1 = p.seg_q[(int64_t)b * p.Lq + wr1];
  }
  const int32_t myseg = segs ? p.seg_q[(int64_t)b * p.Lq + min(wr0 + c32, p.Lq - 1)] : 0;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  const uint8_t* kg = reinterpret_cast<const uint8_t*>(p.k + b * p.sk.b + hh * p.sk.h);
  const int64_t kl_bytes = p.sk.l * 2;
  const int64_t k_extent = (int64_t)(p.Lk - 1) * kl_bytes + 256;
  // this pair's dS^T blocks: the tile of keys k0.. is query blocks q0/64 .. + 3 of key block
  // k0/64, 32 KB in a row, of which those before the row's first stored block are not read
  const uint8_t* sg = reinterpret_cast<const uint8_t*>(p.ds) + (int64_t)lbh * ds_slot_bytes(p);
  const int64_t nqb = p.ds_ld / kDsBlock;
  const int32_t* segk_row = segs ? p.seg_k + (int64_t)b * p.Lk : nullptr;
  // K tile: 16 blocks of 1 KB, two per wave; dS^T tile: 32 blocks of 1 KB, four per wave.  In
  // LDS the dS^T tile is two row-major swizzled 64 x 128 tiles side by side (queries 0..127 and
  // 128..255 of the workgroup): 16-byte chunk c of row r of half hr is chunk c % 8 of key r in
  // query block 2 hr + c / 8
  int ld_voff_k[2], ld_voff_s[4], ld_blk_s[4];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = (w * 2 + r) * 4 + (lane >> 4);
    ld_voff_k[r] = (int)(row * kl_bytes) + (((lane & 15) ^ swz16(row)) << 4);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int blk = w * 4 + r, hr = blk >> 4, row = (blk & 15) * 4 + (lane >> 4);
    const int c = (lane & 15) ^ swz16(row);
    ld_blk_s[r] = 2 * hr + (c >> 3);
    ld_voff_s[r] = (c & 7) * kDsChunkBytes + row * 16;
  }
  auto issue = [&](int tile, StageDs& dst) __attribute__((always_inline)) {
    const int k0 = tile * BN;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + k0 * kl_bytes, k_extent - k0 * kl_bytes);
    const int64_t kb = k0 / kDsBlock, qlo = ds_qlo(p, kb);
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(sg + ds_row_start(p, kb) * kDsBlockBytes, (nqb - qlo) * kDsBlockBytes);
    const int rel0 = (int)(q0 / kDsBlock - qlo);  // this tile's first query block in the row
    // a block before the row's first (none of its pairs is visible) gets an offset past the end
    int voff_s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      voff_s[r] = rel0 + ld_blk_s[r] >= 0 ? (rel0 + ld_blk_s[r]) * kDsBlockBytes + ld_voff_s[r] : 0x7fffffff;
#pragma unroll
    for (int r = 0; r < 2; ++r) load_lds16(rk, &dst.k[(w * 2 + r) * 1024], ld_voff_k[r]);
#pragma unroll
    for (int r = 0; r < 4; ++r) load_lds16(rs, &dst.s[(w * 4 + r) * 1024], voff_s[r]);
    if (segs && w == 0) load_lds4(make_rsrc(segk_row + k0, (int64_t)(p.Lk - k0) * 4), &dst.seg[0], lane * 4);
  };
  int tlo0, thi0;
  tr_offsets(lane, 0, tlo0, thi0);
  // wave w's queries: half-row w / 4, column block w % 4 of it
  const int s_half = (w >> 2) * 16384;
  const int tlo_s = tlo0 ^ ((w & 3) << 6), thi_s = thi0 ^ ((w & 3) << 6);

  auto tile = [&](auto sc, int it) __attribute__((always_inline)) {
    StageDs& cur = stage(sc);
    const int k0 = (t_begin + it) * BN;
    // this tile's loads done (the next tile's may still be in flight), then every wave's
    if (it + 1 < ntiles) {
      if (segs && w == 0) wait_vmcnt<7>();
      else wait_vmcnt<6>();
    } else {
      wait_vmcnt<0>();
    }
    block_barrier();
    if (it + 2 < ntiles) issue(t_begin + it + 2, stage(DsStage<(decltype(sc)::value + 2) % 3>{}));
    bool active = wave_rows;
    bool need_mask = (k0 + BN > p.Lk) || (k0 < kbeg) || (k0 + BN > kend);
    if (p.causal) {
      active = active && (p.k_offset + k0 <= p.q_offset + wr1);
      need_mask = need_mask || (p.k_offset + k0 + BN - 1 > p.q_offset + wr0);
    }
    if (segs) {
      const int32_t ts0 = cur.seg[0], ts1 = cur.seg[min(BN, p.Lk - k0) - 1];
      active = active && !(ts1 < wseg0 || ts0 > wseg1);
      need_mask = need_mask || !(ts0 == ts1 && wseg0 == wseg1 && ts0 == wseg0);
    }
    if (!active) return;

    // dS^T operand of 16-key group g: keys 16g + 8(e/4) + 4*h32 + e%4 (element e) of query c32
    bf16x8 dsb[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) dsb[g] = read_xt(cur.s + s_half + g * 4096, tlo_s, thi_s);
    if (need_mask) {
      // key kl = 32 kb + 8 g4 + 4 h32 + j is visible iff kl < lim (end of the keys, causal limit)
      // and its segment is this lane's query's; element 4 (g4 & 1) + j of dsb[2 kb + g4 / 2]
      int64_t lim64 = (int64_t)p.Lk - k0;
      if (p.causal) lim64 = imin64(lim64, gq - p.k_offset - k0 + 1);
      const int limt = (int)imax64(imin64(lim64, BN), 0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int lim = limt - kb * 32 - 4 * h32;
        const int32_t* segt = &cur.seg[kb * 32 + 4 * h32];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          u32x4 x = __builtin_bit_cast(u32x4, dsb[2 * kb + u]);
#pragma unroll
          for (int eh = 0; eh < 2; ++eh) {
            const int g4 = 2 * u + eh;
            i32x4 ks = {myseg, myseg, myseg, myseg};
            if (segs) ks = *reinterpret_cast<const i32x4*>(segt + 8 * g4);
            bool vis[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) vis[j] = (8 * g4 + j < lim) & (ks[j] == myseg);
            x[2 * eh] &= (vis[0] ? 0xFFFFu : 0u) | (vis[1] ? 0xFFFF0000u : 0u);
            x[2 * eh + 1] &= (vis[2] ? 0xFFFFu : 0u) | (vis[3] ? 0xFFFF0000u : 0u);
          }
          dsb[2 * kb + u] = __builtin_bit_cast(bf16x8, x);
        }
      }
    }
    // dQ^T += K^T dS^T (K^T operands by transposing reads, two ahead)
    {
      bf16x8 kf[3];
      auto kread = [&](int n) {
        return read_xt(cur.k + (n >> 2) * 4096, tlo0 ^ ((n & 3) << 6), thi0 ^ ((n & 3) << 6));
      };
      kf[0] = kread(0);
      kf[1] = kread(1);
#pragma unroll
      for (int n = 0; n < 16; ++n) {  // n = 16-key group * 4 + feature block
        if (n + 2 < 16) kf[(n + 2) % 3] = kread(n + 2);
        __builtin_amdgcn_sched_barrier(0);
        acc[n & 3] = mfma_32x32x16(kf[n % 3], dsb[n >> 2], acc[n & 3]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if (ntiles > 0) issue(t_begin, lds_s0);
  if (ntiles > 1) issue(t_begin + 1, lds_s1);
  int it = 0;
  for (; it + 3 <= ntiles; it += 3) {
    tile(DsStage<0>{}, it);
    tile(DsStage<1>{}, it + 1);
    tile(DsStage<2>{}, it + 2);
  }
  if (it < ntiles) tile(DsStage<0>{}, it);
  if (it + 1 < ntiles) tile(DsStage<1>{}, it + 1);
  __syncthreads();
  // staging for the epilogue: 16 KB per wave, three waves to a stage object
  StageDs& st = w < 3 ? lds_s0 : (w < 6 ? lds_s1 : lds_s2);
  dq_epilogue(p, reinterpret_cast<uint8_t*>(&st) + (w % 3) * 16384, acc, b, hh, wr0, h32, segs);
}

// ------------------------------------------------------------------------------ dK / dV
// swap23 exchanges bits 2 and 3 of an index: the dK/dV kernel keeps query t of a tile in LDS row
// swap23(t) of its Q and dO tiles (the per-query rows stay in query order).  Lane half h of a 32 x 32 accumulator holds
// rows 16u + 4h + {0..3} and 16u + 8 + 4h + {0..3} in operand u, which are then queries
// 16u + 8h + {0..7}: eight consecutive queries, one 16-byte piece of a stored dS^T row.  Sums over
// queries are unchanged up to their order, and both dK/dV variants use the same order.
__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x >> 1) & 4) | ((x << 1) & 8); }
// A workgroup owns 256 keys and has 8 waves, two per SIMD: wave w owns the 32 keys k0 + 32 w.  It
// keeps their dK^T and dV^T accumulators (128 registers) and their K rows as MFMA operands (32
// registers) for the whole pass; their V rows sit in LDS.  All eight waves walk the visible
// 64-query tiles together, each tile as two 32-query sub-tiles, so every Q and dO tile brought
// into LDS feeds the products of 256 keys: half the bytes loaded per MFMA of a 128-key workgroup,
// and each wave's sums are complete at the end (nothing to exchange).
constexpr int BQ = 32;   // queries per sub-tile
constexpr int BQT = 64;  // queries per tile (two sub-tiles)
constexpr int BKV = 256; // keys per workgroup
constexpr int kDkdvWaves = 8;
constexpr int kQTileBytes = BQ * 256;  // 32 rows x 128 bf16
// One stage of the query-tile ring: the Q and dO rows of 64 queries (row-major swizzled, sub-tile
// u at u * kQTileBytes) and the queries' lse * log2(e), delta and segment ids.  The two stages
// and the V rows are LDS objects of their own, and the tile loop is
// unrolled by two so that every access names its stage at compile time: the compiler makes a
// transposing LDS read wait for every load into LDS in flight unless it can tell that the read's
// object differs from theirs, and the next tile's loads are in flight for most of a step.
struct StageQO {
  uint8_t q[2 * kQTileBytes];
  uint8_t o[2 * kQTileBytes];
  float lse2[64];
  float dlt[64];
  int32_t seg[64];
};
static_assert(offsetof(StageQO, dlt) == offsetof(StageQO, lse2) + 256 &&
                  offsetof(StageQO, seg) == offsetof(StageQO, lse2) + 512,
              "the three query-row arrays are consecutive");
constexpr int kVBytes = BKV * 256;  // V rows of the workgroup's keys, 8 KB per wave
// after the loop each wave stages its bf16 output rows (8 KB) in its own V rows
static_assert(kVBytes == kDkdvWaves * 32 * D * 2, "a wave's bf16 staging rows fill its V rows");

template <int S>
using StageC = std::integral_constant<int, S>;

// kStoreDs: also write dS^T of every visited (key, query) sub-tile to the stored-dS matrix (bf16,
// zero where masked), for bwd_dq_ds_kernel.
template <bool kStoreDs>
__global__ __launch_bounds__(kDkdvWaves * kWave) void bwd_dkdv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) StageQO lds_qo0;
  __shared__ __attribute__((aligned(1024))) StageQO lds_qo1;
  __shared__ __attribute__((aligned(1024))) uint8_t lds_v[kVBytes];
  auto stage = [&](auto sc) __attribute__((always_inline)) -> StageQO& {
    if constexpr (decltype(sc)::value == 0) return lds_qo0;
    else return lds_qo1;
  };
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, h32 = lane >> 5;
  const int nkt = (p.Lk + BKV - 1) / BKV;
  int lbh, kt;
  const bool segs = p.seg_q != nullptr;
  map_block(blockIdx.x, nkt, p.bh_count, false, segs, lbh, kt);
  const int bh = p.bh0 + lbh;
  const int b = bh / p.H, hh = bh - b * p.H;
  const int k0 = kt * BKV;
  const int klast = min(k0 + BKV, p.Lk) - 1;
  const int wk0 = k0 + w * 32, wk1 = min(wk0 + 32, p.Lk) - 1;
  const bool wave_keys = wk1 >= wk0;
  const int krow = wk0 + c32;
  // stored dS^T: the rows of blocks of this workgroup's four key blocks (those past the pair's
  // last key block fall outside the resource and their stores are dropped).  Lane (c32, h32)
  // writes key w*32 + c32 of them, chunks 2u + h32 of a sub-tile.
  __amdgpu_buffer_rsrc_t rds;
  int ds_wave = 0;   // the wave's part of the store offsets (its key block's row and keys); uniform
  int ds_qlo_w = 0;  // the first query block stored in the wave's key block's row
  if constexpr (kStoreDs) {
    const int64_t kb0 = k0 / kDsBlock, nkb = (p.Lk + kDsBlock - 1) / kDsBlock;
    const int64_t row0 = ds_row_start(p, kb0), kbw = kb0 + (w >> 1);
    rds = make_rsrc(reinterpret_cast<const uint8_t*>(p.ds) + (int64_t)lbh * ds_slot_bytes(p) + row0 * kDsBlockBytes,
                    (ds_row_start(p, imin64(kb0 + 4, nkb)) - row0) * kDsBlockBytes);
    ds_qlo_w = (int)ds_qlo(p, kbw);
    ds_wave = (int)((ds_row_start(p, kbw) - row0 - ds_qlo_w) * kDsBlockBytes) + (w & 1) * 32 * 16;
  }

  // this wave's 32 V rows into its 8 KB of LDS (8 blocks of 1 KB; rows past the end read as zero),
  // in flight during the query-range search; only this wave reads them
  uint8_t* const vw = lds_v + w * 8192;
  {
    const uint8_t* vgb = reinterpret_cast<const uint8_t*>(p.v + b * p.sv.b + hh * p.sv.h);
    const int64_t vlb = p.sv.l * 2;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vgb + (int64_t)wk0 * vlb, (int64_t)(p.Lk - 1 - wk0) * vlb + 256);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = r * 4 + (lane >> 4);
      const int c = (lane & 15) ^ swz16(row);
      load_lds16(rv, vw + r * 1024, (int)(row * vlb) + c * 16);
    }
  }
  // this wave's K rows as the B operands of S = Q K^T: fragment sd holds features
  // 16 sd + 8 h32 .. + 7 of key krow (zero past the end)
  bf16x8 kreg[8];
  {
    const uint16_t* kg = p.k + b * p.sk.b + hh * p.sk.h + (int64_t)krow * p.sk.l;
#pragma unroll
    for (int sd = 0; sd < 8; ++sd) {
      u32x4 a = {0u, 0u, 0u, 0u};
      if (krow < p.Lk) a = *reinterpret_cast<const u32x4*>(kg + sd * 16 + h32 * 8);
      kreg[sd] = as_bf16x8(a);
    }
  }

  // queries that can see any key of this workgroup
  int qbeg = 0, qend = p.Lq;
  if (p.causal) qbeg = (int)imin64(p.Lq, imax64(0, p.k_offset + k0 - p.q_offset));
  if (segs) {
    const int32_t* segq = p.seg_q + (int64_t)b * p.Lq;
    const int32_t s_last = p.seg_k[(int64_t)b * p.Lk + klast];
    if (causal_self_segments(p.seg_q, p.seg_k, p.Lq, p.Lk, p.q_offset, p.k_offset, p.causal)) {
      // the first key's segment starts no later than the key: the causal limit starts the range
      qend = min(qend, s_last == INT32_MAX ? p.Lq : wave_lower_bound(segq, p.Lq, s_last + 1));
    } else {
      int lo, hi;
      segment_range(segq, p.Lq, p.seg_k[(int64_t)b * p.Lk + k0], s_last, lo, hi);
      qbeg = max(qbeg, lo);
      qend = min(qend, hi);
    }
  }
  const int t_begin = qbeg / BQT;
  const int ntiles = (qend > qbeg) ? (qend + BQT - 1) / BQT - t_begin : 0;

  int32_t wseg0 = 0, wseg1 = 0;
  if (segs && wave_keys) {
    wseg0 = p.seg_k[(int64_t)b * p.Lk + wk0];
    wseg1 = p.seg_k[(int64_t)b * p.Lk + wk1];
  }
  const int32_t myseg = segs ? p.seg_k[(int64_t)b * p.Lk + min(krow, p.Lk - 1)] : 0;
  // k_offset - q_offset for the causal mask, in 32 bits: a masked tile has some query no later than
  // some key of the wave and some query at or after the wave's first key, which bounds it to
  // (-2^30, 2^30 + 32) there; clamping outside that range changes no mask
  const int kq = (int)imax64(-(int64_t(1) << 30), imin64((int64_t(1) << 30) + 64, p.k_offset - p.q_offset));
  const int krh = krow - 8 * h32;  // this lane's key less the first query it holds in a sub-tile

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;

  const uint8_t* qg = reinterpret_cast<const uint8_t*>(p.q + b * p.sq.b + hh * p.sq.h);
  const uint8_t* og = reinterpret_cast<const uint8_t*>(p.dout + b * p.sdo.b + hh * p.sdo.h);
  const int64_t ql_bytes = p.sq.l * 2, ol_bytes = p.sdo.l * 2;
  const int64_t q_extent = (int64_t)(p.Lq - 1) * ql_bytes + 256, o_extent = (int64_t)(p.Lq - 1) * ol_bytes + 256;
  const float* lse2_row = p.lse2 + ((int64_t)b * p.H + hh) * p.Lq;
  const float* dlt_row = p.delta + ((int64_t)b * p.H + hh) * p.Lq;
  const int32_t* segq_row = segs ? p.seg_q + (int64_t)b * p.Lq : nullptr;
  // per q-tile: 16 blocks of 1 KB for Q and 16 for dO, two of each per wave
  // (LDS row r holds query swap23(r) of the tile)
  const int ld_row0 = w * 8 + (lane >> 4), ld_row1 = ld_row0 + 4;
  const int ld_voff_q0 = (int)(swap23(ld_row0) * ql_bytes) + (((lane & 15) ^ swz16(ld_row0)) << 4);
  const int ld_voff_q1 = (int)(swap23(ld_row1) * ql_bytes) + (((lane & 15) ^ swz16(ld_row1)) << 4);
  const int ld_voff_o0 = (int)(swap23(ld_row0) * ol_bytes) + (((lane & 15) ^ swz16(ld_row0)) << 4);
  const int ld_voff_o1 = (int)(swap23(ld_row1) * ol_bytes) + (((lane & 15) ^ swz16(ld_row1)) << 4);
  auto issue = [&](int tile, StageQO& dst) __attribute__((always_inline)) {
    const int q0 = tile * BQT;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg + q0 * ql_bytes, q_extent - q0 * ql_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(og + q0 * ol_bytes, o_extent - q0 * ol_bytes);
    load_lds16(rq, &dst.q[(2 * w) * 1024], ld_voff_q0);
    load_lds16(rq, &dst.q[(2 * w + 1) * 1024], ld_voff_q1);
    load_lds16(ro, &dst.o[(2 * w) * 1024], ld_voff_o0);
    load_lds16(ro, &dst.o[(2 * w + 1) * 1024], ld_voff_o1);
    // the query rows, one 4-byte load per wave and no branch: wave 0 lse2, wave 1 delta, the
    // others the segment ids (each the same bytes; without segment ids, lse2 again into the
    // unused segment slot).  A branch per wave here leaves the compiler unable to tell which
    // stage the loads in flight write, and it then makes LDS reads of the other stage wait.
    const int64_t rem = (int64_t)(p.Lq - q0) * 4;
    const void* row_src = w == 0 ? static_cast<const void*>(lse2_row + q0)
                                 : (w == 1 ? static_cast<const void*>(dlt_row + q0)
                                           : (segs ? static_cast<const void*>(segq_row + q0)
                                                   : static_cast<const void*>(lse2_row + q0)));
    load_lds4(make_rsrc(row_src, rem), reinterpret_cast<uint8_t*>(&dst.lse2[0]) + min(w, 2) * 256, lane * 4);
  };
  // Row-major operand (Q, dO, V rows; row c32, chunk 2*sd + h32): the XOR swizzle leaves bit 0 of
  // an even chunk index alone, so the offset is a per-lane base plus ((2*sd) ^ swizzle) * 16.
  // Transposing reads (Q^T, dO^T) for feature block db differ from block 0's offsets by an XOR of
  // db into chunk bits 2..3.
  const int rswz = swz16(c32 & 15);
  const int rbase = c32 * 256 + (((h32 ^ rswz) & 1) << 4);
  auto roff = [&](int sd) { return rbase + (((2 * sd) ^ (rswz & 14)) << 4); };
  int tlo0, thi0;
  tr_offsets(lane, 0, tlo0, thi0);

  // Query tiles are visited from the last one down: every workgroup of a head then starts on the
  // same tile and they move through Q and dO together, so each tile is fetched into L2 once and
  // read there by all of them.
  const int t_last = t_begin + ntiles - 1;
  // One tile: stage S holds it, the other stage receives the next one.
  auto step = [&](auto sc, int it) __attribute__((always_inline)) {
    StageQO& cur = stage(sc);
    const int q0t = (t_last - it) * BQT;
    wait_vmcnt<0>();
    __syncthreads();
    if (it + 1 < ntiles) issue(t_last - it - 1, stage(StageC<1 - decltype(sc)::value>{}));
    // sub-tile u2: queries q0t + 32 u2 .. + 31 (none when past the end)
    auto sub = [&](int u2) __attribute__((always_inline)) {
      const int q0 = q0t + BQ * u2;
      if (q0 >= p.Lq) return;
      const uint8_t* qt = cur.q + u2 * kQTileBytes;
      const uint8_t* ot = cur.o + u2 * kQTileBytes;
      bool active = wave_keys;
      bool need_mask = false;
      if (p.causal) {
        active = active && (p.q_offset + q0 + BQ - 1 >= p.k_offset + wk0);
        need_mask = p.k_offset + wk1 > p.q_offset + q0;
      }
      if (segs) {
        const int32_t ts0 = cur.seg[BQ * u2], ts1 = cur.seg[BQ * u2 + min(BQ, p.Lq - q0) - 1];
        active = active && !(ts1 < wseg0 || ts0 > wseg1);
        need_mask = need_mask || !(ts0 == ts1 && wseg0 == wseg1 && ts0 == wseg0);
      }
      if (!active) return;

      // S = Q K^T and dP = dO V^T (32 queries x 32 keys); the three LDS fragments of feature step
      // sd + 1 are read while the two MFMAs of step sd run
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
      {
        bf16x8 f[2][3];
        auto rd = [&](int sd, bf16x8 (&d)[3]) {
          const int o = roff(sd);
          d[0] = as_bf16x8(*reinterpret_cast<const u32x4*>(qt + o));
          d[1] = as_bf16x8(*reinterpret_cast<const u32x4*>(ot + o));
          d[2] = as_bf16x8(*reinterpret_cast<const u32x4*>(vw + o));
        };
        rd(0, f[0]);
#pragma unroll
        for (int sd = 0; sd < 8; ++sd) {
          if (sd + 1 < 8) rd(sd + 1, f[(sd + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
          s = mfma_32x32x16(f[sd & 1][0], kreg[sd], s);
          dp = mfma_32x32x16(f[sd & 1][1], f[sd & 1][2], dp);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // lane owns key krow; element i = 4g + j is LDS row acc_row(i, h32) of the sub-tile, query
      // q0 + 16(g/2) + 8*h32 + 4(g%2) + j (the per-query rows are kept in query order)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r4 = BQ * u2 + 16 * (g >> 1) + 4 * (g & 1) + 8 * h32;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&cur.lse2[r4]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&cur.dlt[r4]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * g + j;
          s[i] = __builtin_fmaf(s[i], p.scale_log2, -l4[j]);
          dp[i] = dp[i] - d4[j];
        }
      }
      if (need_mask) {
        // element i = 4g + j holds LDS row 8g + 4*h32 + j, query ql = 16(g/2) + 8*h32 + 4(g%2) + j,
        // visible iff q_offset + q0 + ql >= k_offset + krow (causal), i.e.
        // 16(g/2) + 4(g%2) + j >= lo, and its segment matches this lane's key; masked scores get
        // exponent -inf (a select).  lo stays in 32 bits: a tile needing the causal mask has
        // kq + krow - q0 in (-2^31 + 32, 63)
        const int lo = p.causal ? kq + (krh - q0) : -BQ;
        // the segment ids of this lane's queries, all four groups read under one branch; the lane
        // half's offset 8 * h32 comes from threadIdx.x itself (a value kept for the loop was spilled)
        i32x4 qs[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) qs[g] = i32x4{myseg, myseg, myseg, myseg};
        if (segs) {
          const int32_t* segt = &cur.seg[BQ * u2] + ((threadIdx.x >> 2) & 8);
#pragma unroll
          for (int g = 0; g < 4; ++g) qs[g] = *reinterpret_cast<const i32x4*>(segt + 16 * (g >> 1) + 4 * (g & 1));
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool vis = (16 * (g >> 1) + 4 * (g & 1) + j >= lo) & (qs[g][j] == myseg);
            s[4 * g + j] = vis ? s[4 * g + j] : -INFINITY;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = fast_exp2(s[i]);
        dp[i] *= s[i];
      }
      const bf16x8 pb[2] = {pack8(s, 0), pack8(s, 1)};
      const bf16x8 dsb[2] = {pack8(dp, 0), pack8(dp, 1)};
      // a visible pair's query block is never before its key block's first stored one (the causal
      // test above bounds it); the check keeps a conservative segment test from writing elsewhere
      if (kStoreDs && q0 / kDsBlock >= ds_qlo_w) {
        // dsb[u] holds queries q0 + 16u + 8*h32 + 0..7: chunk (q0 % 64) / 8 + 2u + h32 of this
        // lane's key in the stored layout.  The stores are marked non-temporal (cache policy
        // bit nt): nothing reads dS again before the dQ kernel, and measured, that kernel then
        // runs 3-4% faster (the dK/dV kernel is unchanged).
        // the lane's part (row c32, chunk + h32) comes from threadIdx.x itself: a value kept for the
        // loop is spilled, and its reload would wait for the next tile's loads
        const int tx = (int)threadIdx.x;
        const int off = ds_wave + (q0 / kDsBlock) * kDsBlockBytes + ((q0 % kDsBlock) / 8) * kDsChunkBytes +
                        ((tx & 31) << 4) + ((tx & 32) << 5);
#pragma unroll
        for (int u = 0; u < 2; ++u)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, dsb[u]), rds, off + 2 * u * kDsChunkBytes,
                                                 0, kCachePolicyNT);
      }
      // dV^T += dO^T P, dK^T += Q^T dS (transposed operands by transposing reads, one step ahead)
      {
        bf16x8 g[2][2];
        auto rdt = [&](int n, bf16x8 (&d)[2]) {
          const int u = n >> 2, db = n & 3;
          d[0] = read_xt(ot + u * 4096, tlo0 ^ (db << 6), thi0 ^ (db << 6));
          d[1] = read_xt(qt + u * 4096, tlo0 ^ (db << 6), thi0 ^ (db << 6));
        };
        rdt(0, g[0]);
#pragma unroll
        for (int n = 0; n < 8; ++n) {  // n = 16-query group * 4 + feature block
          if (n + 1 < 8) rdt(n + 1, g[(n + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
          const int u = n >> 2, db = n & 3;
          dv[db] = mfma_32x32x16(g[n & 1][0], pb[u], dv[db]);
          dk[db] = mfma_32x32x16(g[n & 1][1], dsb[u], dk[db]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    sub(0);
    sub(1);
  };
  if (ntiles > 0) issue(t_last, lds_qo0);
  int it = 0;
  for (; it + 2 <= ntiles; it += 2) {
    step(StageC<0>{}, it);
    step(StageC<1>{}, it + 1);
  }
  if (it < ntiles) step(StageC<0>{}, it);
  wait_vmcnt<0>();  // this wave's V rows, when no tile was visited
  __syncthreads();

  const int rows_valid = max(0, min(32, p.Lk - wk0));
  if (p.dk_acc) {
    // backward ring step: dK, dV += this query block's share, in float32.  Lane c32 owns key row
    // wk0 + c32; accumulator element 4g + j of block db is feature db*32 + 8g + 4*h32 + j, so each
    // (db, g) is one 16-byte read-add-write of the row (rows belong to this wave alone).
    auto add_row = [&](const f32x16 (&acc)[4], float mul, float* row) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4* a = reinterpret_cast<f32x4*>(row + db * 32 + 8 * g + 4 * h32);
          f32x4 x = *a;
#pragma unroll
          for (int j = 0; j < 4; ++j) x[j] = __builtin_fmaf(acc[db][4 * g + j], mul, x[j]);
          *a = x;
        }
    };
    if (c32 < rows_valid) {
      add_row(dk, p.scale, p.dk_acc + b * p.sdka.b + hh * p.sdka.h + (int64_t)krow * p.sdka.l);
      add_row(dv, 1.f, p.dv_acc + b * p.sdva.b + hh * p.sdva.h + (int64_t)krow * p.sdva.l);
    }
  } else {
    if (p.rope.on) {  // dK' -> dK (inverse RoPE of the key rows) before rounding to bf16
      const bool restart = segs && p.rope.restart;
      const int64_t pos = rope_row_position(restart ? p.seg_k + (int64_t)b * p.Lk : nullptr, p.Lk, wk0, restart,
                                            p.rope.k_pos_offset);
      rope_unrotate_acc(dk, pos, p.rope, h32);
    }
    // staging rows: the wave's own V rows (the row helpers have block-wide barriers: every wave
    // takes part)
    store_rows_bf16(vw, dk, p.scale, p.dk + b * p.sdk.b + hh * p.sdk.h + wk0 * p.sdk.l, p.sdk.l, rows_valid);
    store_rows_bf16(vw, dv, 1.f, p.dv + b * p.sdv.b + hh * p.sdv.h + wk0 * p.sdv.l, p.sdv.l, rows_valid);
  }
}

}  // namespace

hipError_t launch_attn_bwd(const BwdParams& params, hipStream_t stream) {
  if (params.B == 0 || params.H == 0) return hipSuccess;
  BwdParams p = params;
  const int BH = p.B * p.H;
  if (p.Lq > 0 && !p.delta_ready) {
    const int64_t rows = (int64_t)BH * p.Lq;
    LWM_LAUNCH("bwd_delta", bwd_delta_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), stream, p);
  }
  const int nkt = (p.Lk + BKV - 1) / BKV;
  if (p.ds && p.Lq > 0 && p.Lk > 0) {
    // stored dS: per pass of ds_heads (batch, head) pairs, dK/dV (writing dS^T), then dQ from it
    const int nqt = (p.Lq + kDsQueries - 1) / kDsQueries;
    for (int bh0 = 0; bh0 < BH; bh0 += p.ds_heads) {
      p.bh0 = bh0;
      p.bh_count = min(p.ds_heads, BH - bh0);
      LWM_LAUNCH("bwd_dkdv", bwd_dkdv_kernel<true>, dim3(nkt * p.bh_count), dim3(kDkdvWaves * kWave), stream, p);
      LWM_LAUNCH("bwd_dq_ds", bwd_dq_ds_kernel, dim3(nqt * p.bh_count), dim3(kDsWaves * kWave), stream, p);
    }
    return hipGetLastError();
  }
  p.ds = nullptr;
  p.bh0 = 0;
  p.bh_count = BH;
  if (p.Lq > 0) {
    const int nqt = (p.Lq + 127) / 128;
    LWM_LAUNCH("bwd_dq", bwd_dq_kernel, dim3(nqt * BH), dim3(kThreads), stream, p);
  }
  if (p.Lk > 0)
    LWM_LAUNCH("bwd_dkdv", bwd_dkdv_kernel<false>, dim3(nkt * BH), dim3(kDkdvWaves * kWave), stream, p);
  return hipGetLastError();
}

}  // namespace lwm
