// Blockwise attention backward for gfx950 (bf16 operands, float32 accumulation).
//
// For the loss sum(dO * O) of the forward defined in include/lwm_attn.h (causal: "Inside Large
// World Model ...", section "Core Architecture"; packing: "LWM：突破 100 万 Token 的开源大模型",
// section 概述 (b); blockwise evaluation: the same page, section 配置参数), with
// P = exp(S - lse) recomputed from the forward's saved logsumexp:
//     delta_i = sum_d dO_id O_id
//     dV = P^T dO,   dP = dO V^T,   dS = P o (dP - delta),   dQ = scale dS K,   dK = scale dS^T Q.
//
// Three kernels, no atomics (the result is deterministic):
//  * delta: one pass over dO and O (HBM-bound); also stores lse * log2(e) for the other two.
//  * dQ: a workgroup per 128-query tile walks the visible 64-key tiles like the forward does,
//    with scores transposed (S^T = K Q^T) so each lane owns one query: P^T and dS^T are formed in
//    registers and feed dQ^T += K^T dS^T directly; K^T operands come from the row-major K tile by
//    transposing LDS reads.
//  * dK/dV: a workgroup per 128-key tile (32 keys per wave) walks the visible 64-query tiles with
//    scores in the other orientation (S = Q K^T, each lane owns one key): P and dS feed
//    dV^T += dO^T P and dK^T += Q^T dS directly; Q^T and dO^T operands come from the row-major tiles
//    by transposing LDS reads.
//  With fused RoPE (lwm_blockattn_bwd_rope) the dQ and dK/dV kernels rotate their float32 dQ', dK'
//  accumulators back by -angle just before the one rounding to bf16, so the stored gradients are
//  w.r.t. the pre-RoPE Q and K.
//  Tiles travel HBM -> LDS by buffer loads that write LDS directly (double-buffered).  Recomputing
//  S and dP in both kernels costs two extra products over the five the method needs; in exchange
//  no partial dQ is ever written to or reduced through memory.

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
  int bh, qt;
  map_block(blockIdx.x, nqt, p.B * p.H, true, bh, qt);
  const int b = bh / p.H, hh = bh - b * p.H;
  const int q0 = qt * BM;
  const int qlast = min(q0 + BM, p.Lq) - 1;
  const bool segs = p.seg_q != nullptr;

  int kbeg = 0, kend = p.Lk;
  if (p.causal) kend = (int)imax64(0, imin64(kend, p.q_offset + qlast - p.k_offset + 1));
  if (segs) {
    int lo, hi;
    segment_range(p.seg_k + (int64_t)b * p.Lk, p.Lk, p.seg_q[(int64_t)b * p.Lq + q0], p.seg_q[(int64_t)b * p.Lq + qlast],
                  lo, hi);
    kbeg = max(kbeg, lo);
    kend = min(kend, hi);
  }
  const int t_begin = kbeg / BN;
  const int ntiles = (kend > kbeg) ? (kend + BN - 1) / BN - t_begin : 0;

  const int wr0 = q0 + w * MW, wr1 = min(wr0 + MW, p.Lq) - 1;
  const bool wave_rows = wr1 >= wr0;
  int32_t wseg0 = 0, wseg1 = 0;
  if (segs && wave_rows) {
    wseg0 = p.seg_q[(int64_t)b * p.Lq + wr0];
    wseg1 = p.seg_q[(int64_t)b * p.Lq + wr1];
  }
  const int qrow = wr0 + c32;
  const int64_t gq = p.q_offset + qrow;
  const int32_t myseg = segs ? p.seg_q[(int64_t)b * p.Lq + min(qrow, p.Lq - 1)] : 0;
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
  const int rows_valid = max(0, min(32, p.Lq - wr0));
  if (p.dq_acc) {  // backward ring step: dQ += this shard's share, in float32
    uint8_t* stage_w = reinterpret_cast<uint8_t*>(&sm) + w * (32 * D * 4);
    add_rows_f32(stage_w, acc, p.scale, p.dq_acc + b * p.sdqa.b + hh * p.sdqa.h + wr0 * p.sdqa.l, p.sdqa.l,
                 rows_valid);
  } else {
    if (p.rope.on) {  // dQ' -> dQ (inverse RoPE of the query rows) before the one rounding to bf16
      const bool restart = segs && p.rope.restart;
      const int64_t pos = rope_row_position(restart ? p.seg_q + (int64_t)b * p.Lq : nullptr, p.Lq, wr0, restart,
                                            p.rope.q_pos_offset);
      rope_unrotate_acc(acc, pos, p.rope, h32);
    }
    uint8_t* stage_w = reinterpret_cast<uint8_t*>(&sm) + w * (32 * D * 2);
    store_rows_bf16(stage_w, acc, p.scale, p.dq + b * p.sdq.b + hh * p.sdq.h + wr0 * p.sdq.l, p.sdq.l, rows_valid);
  }
}

// ------------------------------------------------------------------------------ dK / dV
// A workgroup owns 128 keys and has 8 waves, two per SIMD: wave w handles the 32 keys
// k0 + 32 (w % 4) against the query half w / 4 of every 64-query tile, so each wave keeps one
// 32-key dK^T and dV^T accumulator pair (128 registers) and the SIMD's two waves cover each
// other's LDS and dependency waits.  The two partial sums of a key block are added through LDS at
// the end.  The workgroup's K and V tiles sit in LDS for the whole pass.
constexpr int BQ = 64;   // queries per tile
constexpr int kDkdvWaves = 8;
// One stage of the query-tile ring: the Q and dO rows of 64 queries (row-major swizzled) and the
// queries' lse * log2(e), delta and segment ids.  The two stages and the workgroup's K / V rows are
// LDS objects of their own, and the tile loop is unrolled by two so that every access names its
// stage at compile time: the compiler makes a transposing LDS read wait for every load into LDS in
// flight unless it can tell that the read's object differs from theirs, and the next tile's loads
// are in flight for most of a step.
struct StageQO {
  uint8_t q[kTileBytes];
  uint8_t o[kTileBytes];
  float lse2[BQ];
  float dlt[BQ];
  int32_t seg[BQ];
};
constexpr int kKVBytes = 4 * kTileBytes;  // K (128 rows) then V (128 rows)
// after the loop: the partial-sum exchange (dK^T partials in the K/V area, dV^T partials in the two
// stages' Q / dO areas) and each wave's epilogue staging rows (16 KB: waves 0..3 in the K/V area,
// 4..7 in the stages) reuse the same three objects
static_assert(kKVBytes == 4 * 4 * 4 * 64 * 16, "dK partials of 4 key blocks fill the K/V area");
static_assert(kTileBytes == 4 * 4 * 64 * 16, "one feature block of dV partials fills a Q or dO area");
static_assert(kTileBytes >= 32 * D * 4, "a wave's staging rows (float32) fit a Q or dO area");

template <int S>
using StageC = std::integral_constant<int, S>;

__global__ __launch_bounds__(kDkdvWaves * kWave) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int BK = 128;
  __shared__ __attribute__((aligned(1024))) StageQO lds_qo0;
  __shared__ __attribute__((aligned(1024))) StageQO lds_qo1;
  __shared__ __attribute__((aligned(1024))) uint8_t lds_kv[kKVBytes];
  auto stage = [&](auto sc) __attribute__((always_inline)) -> StageQO& {
    if constexpr (decltype(sc)::value == 0) return lds_qo0;
    else return lds_qo1;
  };
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, h32 = lane >> 5;
  const int kb = w & 3, qh = w >> 2;  // key block of 32, query half of each 64-query tile
  const int nkt = (p.Lk + BK - 1) / BK;
  int bh, kt;
  map_block(blockIdx.x, nkt, p.B * p.H, false, bh, kt);
  const int b = bh / p.H, hh = bh - b * p.H;
  const int k0 = kt * BK;
  const int klast = min(k0 + BK, p.Lk) - 1;
  const bool segs = p.seg_q != nullptr;

  // queries that can see any key of this tile
  int qbeg = 0, qend = p.Lq;
  if (p.causal) qbeg = (int)imin64(p.Lq, imax64(0, p.k_offset + k0 - p.q_offset));
  if (segs) {
    int lo, hi;
    segment_range(p.seg_q + (int64_t)b * p.Lq, p.Lq, p.seg_k[(int64_t)b * p.Lk + k0], p.seg_k[(int64_t)b * p.Lk + klast],
                  lo, hi);
    qbeg = max(qbeg, lo);
    qend = min(qend, hi);
  }
  const int t_begin = qbeg / BQ;
  const int ntiles = (qend > qbeg) ? (qend + BQ - 1) / BQ - t_begin : 0;

  const int wk0 = k0 + kb * 32, wk1 = min(wk0 + 32, p.Lk) - 1;
  const bool wave_keys = wk1 >= wk0;
  int32_t wseg0 = 0, wseg1 = 0;
  if (segs && wave_keys) {
    wseg0 = p.seg_k[(int64_t)b * p.Lk + wk0];
    wseg1 = p.seg_k[(int64_t)b * p.Lk + wk1];
  }
  const int krow = wk0 + c32;
  const int64_t gk = p.k_offset + krow;
  const int32_t myseg = segs ? p.seg_k[(int64_t)b * p.Lk + min(krow, p.Lk - 1)] : 0;

  // the workgroup's K and V (128 rows each) into LDS: 32 blocks of 1 KB per tensor, 4 per wave
  {
    const uint8_t* kgb = reinterpret_cast<const uint8_t*>(p.k + b * p.sk.b + hh * p.sk.h);
    const uint8_t* vgb = reinterpret_cast<const uint8_t*>(p.v + b * p.sv.b + hh * p.sv.h);
    const int64_t klb = p.sk.l * 2, vlb = p.sv.l * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kgb + k0 * klb, (int64_t)(p.Lk - 1 - k0) * klb + 256);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vgb + k0 * vlb, (int64_t)(p.Lk - 1 - k0) * vlb + 256);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int blk = w * 4 + r;
      const int row = blk * 4 + (lane >> 4);
      const int c = (lane & 15) ^ swz16(row);
      load_lds16(rk, &lds_kv[blk * 1024], (int)(row * klb) + c * 16);
      load_lds16(rv, &lds_kv[2 * kTileBytes + blk * 1024], (int)(row * vlb) + c * 16);
    }
  }
  const uint8_t* kw = lds_kv + kb * 8192;  // this wave's 32 keys
  const uint8_t* vw = lds_kv + 2 * kTileBytes + kb * 8192;

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
  // per q-tile: 16 blocks of 1 KB for Q and 16 for dO, two per wave
  const int ld_row0 = (w * 2) * 4 + (lane >> 4), ld_row1 = ld_row0 + 4;
  const int ld_voff_q0 = (int)(ld_row0 * ql_bytes) + (((lane & 15) ^ swz16(ld_row0)) << 4);
  const int ld_voff_q1 = (int)(ld_row1 * ql_bytes) + (((lane & 15) ^ swz16(ld_row1)) << 4);
  const int ld_voff_o0 = (int)(ld_row0 * ol_bytes) + (((lane & 15) ^ swz16(ld_row0)) << 4);
  const int ld_voff_o1 = (int)(ld_row1 * ol_bytes) + (((lane & 15) ^ swz16(ld_row1)) << 4);
  auto issue = [&](int tile, StageQO& dst) __attribute__((always_inline)) {
    const int q0 = tile * BQ;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qg + q0 * ql_bytes, q_extent - q0 * ql_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(og + q0 * ol_bytes, o_extent - q0 * ol_bytes);
    load_lds16(rq, &dst.q[(w * 2) * 1024], ld_voff_q0);
    load_lds16(rq, &dst.q[(w * 2 + 1) * 1024], ld_voff_q1);
    load_lds16(ro, &dst.o[(w * 2) * 1024], ld_voff_o0);
    load_lds16(ro, &dst.o[(w * 2 + 1) * 1024], ld_voff_o1);
    const int64_t rem = (int64_t)(p.Lq - q0) * 4;
    if (w == 0) load_lds4(make_rsrc(lse2_row + q0, rem), &dst.lse2[0], lane * 4);
    if (w == 1) load_lds4(make_rsrc(dlt_row + q0, rem), &dst.dlt[0], lane * 4);
    if (segs && w == 2) load_lds4(make_rsrc(segq_row + q0, rem), &dst.seg[0], lane * 4);
  };
  // Row-major operand (Q, dO, K, V rows; row c32 within its 32-row block, chunk 2*sd + h32): the
  // XOR swizzle leaves bit 0 of an even chunk index alone, so the offset is a per-lane base plus
  // ((2*sd) ^ swizzle) * 16.  Transposing reads (Q^T, dO^T) for feature block db differ from block
  // 0's offsets by an XOR of db into chunk bits 2..3.
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
    const int q0 = (t_last - it) * BQ;
    wait_vmcnt<0>();
    __syncthreads();
    if (it + 1 < ntiles) issue(t_last - it - 1, stage(StageC<1 - decltype(sc)::value>{}));
    const uint8_t* qt = cur.q + qh * 8192;  // this wave's 32 queries
    const uint8_t* ot = cur.o + qh * 8192;
    const int wq0 = q0 + qh * 32;
    bool active = wave_keys && (wq0 < p.Lq);
    bool need_mask = false;
    if (p.causal) {
      active = active && (p.q_offset + wq0 + 31 >= p.k_offset + wk0);
      need_mask = p.k_offset + wk1 > p.q_offset + wq0;
    }
    if (segs) {
      const int32_t ts0 = cur.seg[qh * 32], ts1 = cur.seg[min(qh * 32 + 32, p.Lq - q0) - 1];
      active = active && !(ts1 < wseg0 || ts0 > wseg1);
      need_mask = need_mask || !(ts0 == ts1 && wseg0 == wseg1 && ts0 == wseg0);
    }
    if (!active) return;

    // S = Q K^T and dP = dO V^T (32 queries x 32 keys); the four operand fragments of feature
    // step sd + 1 are read while the two MFMAs of step sd run
    f32x16 s, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
    {
      bf16x8 f[2][4];
      auto rd = [&](int sd, bf16x8 (&d)[4]) {
        const int o = roff(sd);
        d[0] = as_bf16x8(*reinterpret_cast<const u32x4*>(qt + o));
        d[1] = as_bf16x8(*reinterpret_cast<const u32x4*>(kw + o));
        d[2] = as_bf16x8(*reinterpret_cast<const u32x4*>(ot + o));
        d[3] = as_bf16x8(*reinterpret_cast<const u32x4*>(vw + o));
      };
      rd(0, f[0]);
#pragma unroll
      for (int sd = 0; sd < 8; ++sd) {
        if (sd + 1 < 8) rd(sd + 1, f[(sd + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        s = mfma_32x32x16(f[sd & 1][0], f[sd & 1][1], s);
        dp = mfma_32x32x16(f[sd & 1][2], f[sd & 1][3], dp);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // lane owns key krow; element i is query wq0 + acc_row(i, h32)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int r4 = qh * 32 + 8 * g + 4 * h32;
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
      // element i holds query ql = qh*32 + 8*(i/4) + 4*h32 + i%4, visible iff ql >= lo (causal)
      // and its segment matches this lane's key; masked scores get exponent -inf (a select)
      int lo = -BQ;
      if (p.causal) lo = (int)imax64(-BQ, imin64(BQ, gk - p.q_offset - q0));
      lo -= qh * 32 + 4 * h32;
      const int32_t* segt = &cur.seg[qh * 32 + 4 * h32];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        i32x4 qs = {myseg, myseg, myseg, myseg};
        if (segs) qs = *reinterpret_cast<const i32x4*>(segt + 8 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool vis = (8 * g + j >= lo) & (qs[j] == myseg);
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
  if (ntiles > 0) issue(t_last, lds_qo0);
  int it = 0;
  for (; it + 2 <= ntiles; it += 2) {
    step(StageC<0>{}, it);
    step(StageC<1>{}, it + 1);
  }
  if (it < ntiles) step(StageC<0>{}, it);
  __syncthreads();
  // add the second query half's partial sums (waves 4..7) to the first's (waves 0..3) via LDS:
  // dK^T partials in the K/V area [key block][db][16 groups of 4][64 lanes], dV^T partials of
  // feature block db in the Q (db even) or dO (db odd) area of stage db / 2, [key block][group][lane]
  auto xdk = [&](int db, int g) __attribute__((always_inline)) {
    return reinterpret_cast<f32x4*>(lds_kv) + ((kb * 4 + db) * 4 + g) * 64 + lane;
  };
  auto xdv = [&](int db, int g) __attribute__((always_inline)) {
    uint8_t* area = db == 0 ? lds_qo0.q : db == 1 ? lds_qo0.o : db == 2 ? lds_qo1.q : lds_qo1.o;
    return reinterpret_cast<f32x4*>(area) + (kb * 4 + g) * 64 + lane;
  };
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        *xdk(db, g) = f32x4{dk[db][4 * g], dk[db][4 * g + 1], dk[db][4 * g + 2], dk[db][4 * g + 3]};
        *xdv(db, g) = f32x4{dv[db][4 * g], dv[db][4 * g + 1], dv[db][4 * g + 2], dv[db][4 * g + 3]};
      }
  }
  __syncthreads();
  if (qh == 0) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 a = *xdk(db, g);
        const f32x4 c = *xdv(db, g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dk[db][4 * g + j] += a[j];
          dv[db][4 * g + j] += c[j];
        }
      }
  }
  __syncthreads();
  // waves 0..3 store (the row helpers have block-wide barriers: every wave takes part)
  const int rows_valid = qh == 0 ? max(0, min(32, p.Lk - wk0)) : 0;
  // staging rows (16 KB per wave): waves 0..3 in the K/V area, 4..7 in the stages' Q / dO areas
  uint8_t* const stage_w = w < 4 ? lds_kv + w * (32 * D * 4)
                                 : (w == 4 ? lds_qo0.q : w == 5 ? lds_qo0.o : w == 6 ? lds_qo1.q : lds_qo1.o);
  if (p.dk_acc) {  // backward ring step: dK, dV += this query block's share, in float32
    add_rows_f32(stage_w, dk, p.scale, p.dk_acc + b * p.sdka.b + hh * p.sdka.h + wk0 * p.sdka.l, p.sdka.l, rows_valid);
    add_rows_f32(stage_w, dv, 1.f, p.dv_acc + b * p.sdva.b + hh * p.sdva.h + wk0 * p.sdva.l, p.sdva.l, rows_valid);
  } else {
    if (p.rope.on && qh == 0) {  // dK' -> dK (inverse RoPE of the key rows) before rounding to bf16
      const bool restart = segs && p.rope.restart;
      const int64_t pos = rope_row_position(restart ? p.seg_k + (int64_t)b * p.Lk : nullptr, p.Lk, wk0, restart,
                                            p.rope.k_pos_offset);
      rope_unrotate_acc(dk, pos, p.rope, h32);
    }
    store_rows_bf16(stage_w, dk, p.scale, p.dk + b * p.sdk.b + hh * p.sdk.h + wk0 * p.sdk.l, p.sdk.l, rows_valid);
    store_rows_bf16(stage_w, dv, 1.f, p.dv + b * p.sdv.b + hh * p.sdv.h + wk0 * p.sdv.l, p.sdv.l, rows_valid);
  }
}

}  // namespace

hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t stream) {
  if (p.B == 0 || p.H == 0) return hipSuccess;
  if (p.Lq > 0) {
    const int64_t rows = (int64_t)p.B * p.Lq * p.H;
    LWM_LAUNCH("bwd_delta", bwd_delta_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), stream, p);
    const int nqt = (p.Lq + 127) / 128;
    LWM_LAUNCH("bwd_dq", bwd_dq_kernel, dim3(nqt * p.B * p.H), dim3(kThreads), stream, p);
  }
  if (p.Lk > 0) {
    const int nkt = (p.Lk + 127) / 128;
    LWM_LAUNCH("bwd_dkdv", bwd_dkdv_kernel, dim3(nkt * p.B * p.H), dim3(kDkdvWaves * kWave), stream, p);
  }
  return hipGetLastError();
}

}  // namespace lwm
