// Blockwise causal attention forward and ring step for gfx950.
//
// Method: blockwise self-attention over query and key chunks ("LWM：突破 100 万 Token 的开源大模型",
// section 配置参数) with the exact online softmax, causal ("Inside Large World Model ...", section
// "Core Architecture") and packing ("LWM：突破 100 万 Token 的开源大模型", section 概述 (b)) masks,
// and the ring step that folds one KV shard into a running (O, lse) state ("开源巨兽LWM：如何用
// RingAttention撬动百万Token多模态世界", section 3.1).
//
// Design (bf16 path):
//  * A workgroup of 4 waves owns BM = 4 * 32 * QB query rows of one (batch, head); each wave owns
//    32 * QB rows whose Q fragments stay in registers for the whole pass.
//  * K and V tiles of 64 keys stream HBM -> registers -> LDS, double-buffered: the global loads of
//    tile j+1 are in flight while tile j is computed.  K is stored row-major with a 16-byte-chunk
//    XOR swizzle; V is stored transposed (feature-major) with the keys of each 16-key group
//    permuted to match the MFMA accumulator layout, so P never leaves registers.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: each lane then
//    holds one query column, so the row max / row sum are in-lane plus a single exchange between
//    the two wave halves, and the O^T accumulator's rescale is a per-lane multiply.
//  * P^T (rounded to bf16) is the B operand of O^T += V^T P^T straight from the accumulator
//    registers.  l sums the bf16-rounded p (v_dot2_f32_bf16), so O is a true convex combination.
//  * The running max is only raised when a row's new max exceeds it by more than 2^8 (log2
//    domain); in between p <= 256, which is exact in fp32 and keeps rescales rare.
//  * Tiles wholly outside the causal / segment range are never visited; the mask is evaluated
//    only on tiles that straddle a boundary or the ragged end.
//  * Workgroups are numbered longest-first, and when B*H is a multiple of 8 the (batch, head)
//    pairs are dealt to the 8 XCDs so the query tiles sharing one head's K/V run on one L2.
#include <float.h>

#include "attn_common.hpp"
#include "profile.hpp"

namespace lwm {
namespace {

constexpr int BN = 64;                 // keys per tile (bf16 path)
constexpr int kTileBytes = BN * 256;   // one K or V tile: 64 rows x 128 bf16
constexpr float kRescaleSlack = 8.0f;  // log2 units: p <= 2^8 between rescales

// Two stages of (K tile, V tile, 64 segment ids); 2 workgroups fit in one CU's LDS.
struct SmemBf16 {
  uint8_t kv[2][2][kTileBytes];
  int32_t seg[2][BN];
};
static_assert(sizeof(SmemBf16) <= 80 * 1024, "two workgroups per CU must fit in LDS");
static_assert(sizeof(SmemBf16) >= kWaves * 32 * D * 4, "epilogue staging must fit");

// Key range [kbeg, kend) that can be visible to query rows [r0, r1] (inclusive).
__device__ inline void key_range(const FwdParams& p, int b, int r0, int r1, int& kbeg, int& kend) {
  kbeg = 0;
  kend = p.Lk;
  if (p.causal) {
    const int64_t lim = p.q_offset + r1 - p.k_offset + 1;
    kend = (int)imax64(0, imin64(kend, lim));
  }
  if (p.seg_q) {
    int lo, hi;
    segment_range(p.seg_k + (int64_t)b * p.Lk, p.Lk, p.seg_q[(int64_t)b * p.Lq + r0], p.seg_q[(int64_t)b * p.Lq + r1],
                  lo, hi);
    kbeg = max(kbeg, lo);
    kend = min(kend, hi);
  }
}

// ---------------------------------------------------------------------------- bf16 kernel
// Streams K/V tiles HBM -> LDS with buffer loads that write LDS directly (no staging registers,
// no per-tile address arithmetic beyond a scalar tile base; rows past the end read as zero).
// The swizzle of a tile is chosen by the source address each lane loads.
template <int QB>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(FwdParams p) {
  constexpr int MW = 32 * QB;
  constexpr int BM = kWaves * MW;
  __shared__ __attribute__((aligned(1024))) SmemBf16 sm;

  // the wave index is uniform; say so, so LDS bases derived from it stay in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, h32 = lane >> 5;
  const int nqt = (p.Lq + BM - 1) / BM;
  int bh, qt;
  map_block(blockIdx.x, nqt, p.B * p.H, true, bh, qt);
  const int b = bh / p.H, hh = bh - b * p.H;
  const int q0 = qt * BM;
  const int qlast = min(q0 + BM, p.Lq) - 1;

  int kbeg, kend;
  key_range(p, b, q0, qlast, kbeg, kend);
  const int t_begin = kbeg / BN;
  const int ntiles = (kend > kbeg) ? (kend + BN - 1) / BN - t_begin : 0;

  const int wr0 = q0 + w * MW;
  const int wr1 = min(wr0 + MW, p.Lq) - 1;  // may be < wr0 for a ragged last tile
  const bool wave_rows = wr1 >= wr0;
  const bool segs = p.seg_q != nullptr;
  int32_t wseg0 = 0, wseg1 = 0;
  if (segs && wave_rows) {
    wseg0 = p.seg_q[(int64_t)b * p.Lq + wr0];
    wseg1 = p.seg_q[(int64_t)b * p.Lq + wr1];
  }

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q) + b * p.sq.b + hh * p.sq.h;
  const uint8_t* kg = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(p.k) + b * p.sk.b + hh * p.sk.h);
  const uint8_t* vg = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(p.v) + b * p.sv.b + hh * p.sv.h);
  const int64_t kl_bytes = p.sk.l * 2, vl_bytes = p.sv.l * 2;
  const int64_t k_extent = (int64_t)(p.Lk - 1) * kl_bytes + 256, v_extent = (int64_t)(p.Lk - 1) * vl_bytes + 256;
  const int32_t* segk_row = segs ? p.seg_k + (int64_t)b * p.Lk : nullptr;

  int qrow[QB];
  int64_t gq[QB];
  int32_t myseg[QB];
  bf16x8 qreg[QB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qrow[qb] = wr0 + qb * 32 + c32;
    gq[qb] = p.q_offset + qrow[qb];
    myseg[qb] = segs ? p.seg_q[(int64_t)b * p.Lq + min(qrow[qb], p.Lq - 1)] : 0;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qrow[qb] < p.Lq) v = *reinterpret_cast<const u32x4*>(qg + qrow[qb] * p.sq.l + s * 16 + h32 * 8);
      qreg[qb][s] = as_bf16x8(v);
    }
  }

  // running state: O^T accumulators, row max m (log2-scaled), partial row sum l (this half's keys)
  f32x16 acc[QB][4];
  float m[QB], l[QB], m_init[QB];
  const bool ring = p.mode == 1;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[qb][db][i] = 0.f;
    m[qb] = -INFINITY;
    l[qb] = 0.f;
  }
  uint8_t* stage_w = reinterpret_cast<uint8_t*>(&sm) + w * (32 * D * 4);
  if (ring && ntiles > 0) {
    float* oag = p.o_acc + b * p.soa.b + hh * p.soa.h;
    const float* lag = p.lse_acc + ((int64_t)b * p.H + hh) * p.Lq;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int r0 = wr0 + qb * 32;
      load_rows_f32(stage_w, acc[qb], oag + r0 * p.soa.l, p.soa.l, max(0, min(32, p.Lq - r0)));
      const float ls = qrow[qb] < p.Lq ? lag[qrow[qb]] : -INFINITY;
      m[qb] = ls * kLog2e;
      l[qb] = h32 == 0 ? 1.f : 0.f;
    }
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) m_init[qb] = m[qb];

  // ---- per-lane load plan: wave w fills 1 KB blocks w*4 .. w*4+3 of each tile (4 rows per block);
  // lane l of a block holds row 4*blk + l/16, physical chunk l%16 = logical chunk ^ swz16(row).
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

  // ---- per-lane LDS read offsets (constant over tiles)
  int koff[8];  // K operand for feature step sd: row c32 (+32 per key block), chunk 2*sd + h32
#pragma unroll
  for (int sd = 0; sd < 8; ++sd) koff[sd] = rm_offset(c32, 2 * sd + h32);
  int vlo[4], vhi[4];  // V^T operand for feature block db (+4096 per 16-key group)
#pragma unroll
  for (int db = 0; db < 4; ++db) tr_offsets(lane, db, vlo[db], vhi[db]);

  if (ntiles > 0) issue(t_begin, 0);

  auto tile = [&](int st, int it) {
    const int k0 = (t_begin + it) * BN;
    wait_vmcnt<0>();   // this wave's loads of tile `it` have landed in LDS
    __syncthreads();   // ... and every other wave's; everyone is done with tile it-1
    if (it + 1 < ntiles) issue(t_begin + it + 1, st ^ 1);
    const uint8_t* kt = sm.kv[st][0];
    const uint8_t* vt = sm.kv[st][1];

    // does this wave see any key of the tile, and does it need the element mask?
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

    // ---- S^T = K Q^T: [2 key blocks][QB query blocks] of 32x32.  K fragments are read two
    // feature steps ahead of the MFMAs that consume them (scheduling barriers keep the order).
    f32x16 s[2][QB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][qb][i] = 0.f;
    {
      bf16x8 kf[3][2];
      auto kread = [&](int sd, bf16x8 (&dst)[2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) dst[kb] = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + kb * 8192 + koff[sd]));
      };
      kread(0, kf[0]);
      kread(1, kf[1]);
#pragma unroll
      for (int sd = 0; sd < 8; ++sd) {
        if (sd + 2 < 8) kread(sd + 2, kf[(sd + 2) % 3]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma_32x32x16(kf[sd % 3][kb], qreg[qb][sd], s[kb][qb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kl = kb * 32 + acc_row(i, h32);
          const int key = k0 + kl;
          const bool in_range = key < p.Lk;
          const int32_t ks = segs ? sm.seg[st][kl] : 0;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const bool vis = in_range & (!p.causal | (p.k_offset + key <= gq[qb])) & (!segs | (ks == myseg[qb]));
            s[kb][qb][i] = vis ? s[kb][qb][i] : -INFINITY;
          }
        }
    }

    // ---- online softmax (log2 domain), lazily rescaled
    float mx[QB];
    bool need_rescale = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // balanced tree over the 32 in-lane scores (short dependency chains), then the lane pair
      float t[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const f32x16& a = s[c >> 2][qb];
        const int o = (c & 3) * 4;
        t[c] = fmaxf(fmaxf(a[o], a[o + 1]), fmaxf(a[o + 2], a[o + 3]));
      }
      const float v = pair_max(fmaxf(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])), fmaxf(fmaxf(t[4], t[5]), fmaxf(t[6], t[7]))));
      mx[qb] = v * p.scale_log2;
      need_rescale = need_rescale || (mx[qb] > m[qb] + kRescaleSlack);
    }
    if (__any(need_rescale)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float mnew = fmaxf(m[qb], mx[qb]);
        const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m[qb] - mnew);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[qb][db][i] *= alpha;
        l[qb] *= alpha;
        m[qb] = mnew;
      }
    }

    // p = exp2(s * scale_log2 - m), rounded to bf16; l += sum of the rounded values
    bf16x8 pb[2][2][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float moff = (m[qb] == -INFINITY) ? 0.f : m[qb];
      float lsum[4] = {0.f, 0.f, 0.f, 0.f};  // independent partial sums (short chains)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          u32x4 packed;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float e0 = fast_exp2(__builtin_fmaf(s[kb][qb][u * 8 + 2 * j], p.scale_log2, -moff));
            const float e1 = fast_exp2(__builtin_fmaf(s[kb][qb][u * 8 + 2 * j + 1], p.scale_log2, -moff));
            const uint32_t word = pack_bf16x2(e0, e1);
            lsum[j] = sum_bf16x2(word, lsum[j]);
            packed[j] = word;
          }
          pb[kb][u][qb] = as_bf16x8(packed);
        }
      l[qb] += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    }

    // ---- O^T += V^T P^T (V^T operands by transposing reads of the row-major V tile, issued
    // two operands ahead of their MFMAs)
    {
      bf16x8 vf[3];
      auto vread = [&](int n) { return read_xt(vt + (n >> 2) * 4096, vlo[n & 3], vhi[n & 3]); };
      vf[0] = vread(0);
      vf[1] = vread(1);
#pragma unroll
      for (int n = 0; n < 16; ++n) {  // n = 16-key group * 4 + feature block
        if (n + 2 < 16) vf[(n + 2) % 3] = vread(n + 2);
        __builtin_amdgcn_sched_barrier(0);
        const int g = n >> 2, db = n & 3;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][db] = mfma_32x32x16(vf[n % 3], pb[g >> 1][g & 1][qb], acc[qb][db]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  for (int it = 0; it < ntiles; ++it) tile(it & 1, it);
  __syncthreads();  // all waves are done reading tiles before the epilogue reuses the LDS

  // ---- epilogue: O = acc / l, lse = (m + log2 l) ln 2
  uint16_t* og = static_cast<uint16_t*>(p.o);
  float* lse_row = p.lse ? p.lse + ((int64_t)b * p.H + hh) * p.Lq : nullptr;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r0 = wr0 + qb * 32;
    const int rows_valid = max(0, min(32, p.Lq - r0));
    const float lt = pair_sum(l[qb]);
    const bool any = (lt > 0.f) && (m[qb] != -INFINITY);
    const float inv = any ? 1.f / lt : 0.f;
    const float lse = any ? (m[qb] + log2f(lt)) * kLn2 : -INFINITY;
    if (!ring) {
      if (og) store_rows_bf16(stage_w, acc[qb], inv, og + b * p.so.b + hh * p.so.h + r0 * p.so.l, p.so.l, rows_valid);
      if (lse_row && h32 == 0 && qrow[qb] < p.Lq) lse_row[qrow[qb]] = lse;
    } else {
      float* lag = p.lse_acc + ((int64_t)b * p.H + hh) * p.Lq;
      float* oag = p.o_acc + b * p.soa.b + hh * p.soa.h + r0 * p.soa.l;
      uint16_t* ofg = og ? og + b * p.so.b + hh * p.so.h + r0 * p.so.l : nullptr;
      if (ntiles > 0) {
        // a row that saw nothing new keeps its state bit for bit
        const bool untouched = (m[qb] == m_init[qb]) && (lt == 1.f);
        const float sc = untouched ? 1.f : inv;
        store_rows_f32(stage_w, acc[qb], sc, oag, p.soa.l, rows_valid);
        if (h32 == 0 && qrow[qb] < p.Lq && !untouched) lag[qrow[qb]] = lse;
        if (ofg) store_rows_bf16(stage_w, acc[qb], sc, ofg, p.so.l, rows_valid);
      } else if (ofg) {
        // nothing visible in this shard for the whole tile: the bf16 copy is the state itself
        f32x16 tmp[4];
        load_rows_f32(stage_w, tmp, oag, p.soa.l, rows_valid);
        store_rows_bf16(stage_w, tmp, 1.f, ofg, p.so.l, rows_valid);
      }
    }
  }
}

// ---------------------------------------------------------------------------- fp32 kernel
// Same structure on v_mfma_f32_32x32x2_f32 (float32 everywhere, no rounding of P); 32-key
// tiles, one query block per wave, fresh state only.
constexpr int BN32 = 32;
constexpr int kPad32 = D + 1;  // LDS row pitch (floats): rows land on distinct banks

struct SmemF32 {
  float k[2][BN32 * kPad32];
  float v[2][BN32 * kPad32];
  int32_t seg[2][BN32];
};

__global__ __launch_bounds__(kThreads, 1) void attn_fwd_f32_kernel(FwdParams p) {
  constexpr int MW = 32, BM = kWaves * MW;
  __shared__ SmemF32 sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c32 = lane & 31, h32 = lane >> 5;
  const int nqt = (p.Lq + BM - 1) / BM;
  int bh, qt;
  map_block(blockIdx.x, nqt, p.B * p.H, true, bh, qt);
  const int b = bh / p.H, hh = bh - b * p.H;
  const int q0 = qt * BM;
  const int qlast = min(q0 + BM, p.Lq) - 1;
  int kbeg, kend;
  key_range(p, b, q0, qlast, kbeg, kend);
  const int t_begin = kbeg / BN32;
  const int ntiles = (kend > kbeg) ? (kend + BN32 - 1) / BN32 - t_begin : 0;
  const bool segs = p.seg_q != nullptr;

  const float* __restrict__ qg = static_cast<const float*>(p.q) + b * p.sq.b + hh * p.sq.h;
  const float* __restrict__ kg = static_cast<const float*>(p.k) + b * p.sk.b + hh * p.sk.h;
  const float* __restrict__ vg = static_cast<const float*>(p.v) + b * p.sv.b + hh * p.sv.h;

  const int qrow = q0 + w * MW + c32;
  const int64_t gq = p.q_offset + qrow;
  const int32_t myseg = segs ? p.seg_q[(int64_t)b * p.Lq + min(qrow, p.Lq - 1)] : 0;
  float qreg[64];  // feature 2*s + h32
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (qrow < p.Lq) v = *reinterpret_cast<const f32x4*>(qg + qrow * p.sq.l + c * 4);
    qreg[2 * c] = v[h32];
    qreg[2 * c + 1] = v[2 + h32];
  }

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  float m = -INFINITY, l = 0.f;

  f32x4 kst[4], vst[4];
  int32_t segst = -1;
  auto gload = [&](int tile) {
    const int k0 = tile * BN32;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = r * kThreads + tid;  // 32 keys x 32 chunks of 4 floats
      const int key = k0 + (e >> 5), c = e & 31;
      kst[r] = key < p.Lk ? *reinterpret_cast<const f32x4*>(kg + key * p.sk.l + c * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
      vst[r] = key < p.Lk ? *reinterpret_cast<const f32x4*>(vg + key * p.sv.l + c * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (segs && tid < BN32) segst = (k0 + tid < p.Lk) ? p.seg_k[(int64_t)b * p.Lk + k0 + tid] : -1;
  };
  auto swrite = [&](int st) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = r * kThreads + tid;
      const int key = e >> 5, c = e & 31;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sm.k[st][key * kPad32 + c * 4 + j] = kst[r][j];
        sm.v[st][key * kPad32 + c * 4 + j] = vst[r][j];
      }
    }
    if (segs && tid < BN32) sm.seg[st][tid] = segst;
  };

  if (ntiles > 0) {
    gload(t_begin);
    swrite(0);
    __syncthreads();
  }
  const int wr0 = q0 + w * MW, wr1 = min(wr0 + MW, p.Lq) - 1;
  for (int it = 0; it < ntiles; ++it) {
    const int st = it & 1;
    const int k0 = (t_begin + it) * BN32;
    if (it + 1 < ntiles) gload(t_begin + it + 1);
    bool active = wr1 >= wr0;
    if (p.causal) active = active && (p.k_offset + k0 <= p.q_offset + wr1);
    if (active) {
      f32x16 s;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
      for (int sd = 0; sd < 64; ++sd) s = mfma_32x32x2_f32(sm.k[st][c32 * kPad32 + 2 * sd + h32], qreg[sd], s);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kl = acc_row(i, h32);
        const int key = k0 + kl;
        bool vis = key < p.Lk && key >= kbeg && key < kend;
        if (p.causal) vis = vis && (p.k_offset + key <= gq);
        if (segs) vis = vis && (sm.seg[st][kl] == myseg);
        if (!vis) s[i] = -INFINITY;
      }
      float v = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) v = fmaxf(v, s[i]);
      v = fmaxf(v, swap_halves(v)) * p.scale_log2;
      if (__any(v > m)) {
        const float mnew = fmaxf(m, v);
        const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m - mnew);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
        l *= alpha;
        m = mnew;
      }
      const float moff = (m == -INFINITY) ? 0.f : m;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = exp2f(__builtin_fmaf(s[i], p.scale_log2, -moff));
        l += s[i];
      }
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int t = 0; t < 16; ++t)
          acc[db] = mfma_32x32x2_f32(sm.v[st][acc_row(t, h32) * kPad32 + db * 32 + c32], s[t], acc[db]);
    }
    if (it + 1 < ntiles) swrite(st ^ 1);
    __syncthreads();
  }

  const float lt = l + swap_halves(l);
  const bool any = (lt > 0.f) && (m != -INFINITY);
  const float inv = any ? 1.f / lt : 0.f;
  const float lse = any ? (m + log2f(lt)) * kLn2 : -INFINITY;
  uint8_t* stage_w = reinterpret_cast<uint8_t*>(&sm) + w * (32 * D * 4);
  float* og = static_cast<float*>(p.o) + b * p.so.b + hh * p.so.h + wr0 * p.so.l;
  store_rows_f32(stage_w, acc, inv, og, p.so.l, max(0, min(32, p.Lq - wr0)));
  if (p.lse && h32 == 0 && qrow < p.Lq) p.lse[((int64_t)b * p.H + hh) * p.Lq + qrow] = lse;
}
static_assert(sizeof(SmemF32) >= kWaves * 32 * D * 4, "epilogue staging must fit");

}  // namespace

hipError_t launch_attn_fwd(const FwdParams& p, bool bf16, hipStream_t stream) {
  if (p.Lq == 0 || p.B == 0 || p.H == 0) return hipSuccess;
  if (bf16) {
    constexpr int QB = 1, BM = kWaves * 32 * QB;
    const int nqt = (p.Lq + BM - 1) / BM;
    LWM_LAUNCH(p.mode == 1 ? "ring_step_bf16" : "attn_fwd_bf16", attn_fwd_bf16_kernel<QB>, dim3(nqt * p.B * p.H),
               dim3(kThreads), stream, p);
  } else {
    const int nqt = (p.Lq + 127) / 128;
    LWM_LAUNCH("attn_fwd_f32", attn_fwd_f32_kernel, dim3(nqt * p.B * p.H), dim3(kThreads), stream, p);
  }
  return hipGetLastError();
}

}  // namespace lwm
