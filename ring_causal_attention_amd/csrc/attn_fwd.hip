// Blockwise causal attention forward and ring step for gfx950.
//
// Method: blockwise self-attention over query and key chunks ("LWM：突破 100 万 Token 的开源大模型",
// section 配置参数) with the exact online softmax, causal ("Inside Large World Model ...", section
// "Core Architecture") and packing ("LWM：突破 100 万 Token 的开源大模型", section 概述 (b)) masks,
// and the ring step that folds one KV shard into a running (O, lse) state ("开源巨兽LWM：如何用
// RingAttention撬动百万Token多模态世界", section 3.1).
//
// Design (bf16 path):
//  * A workgroup of 4 waves owns 128 query rows of one (batch, head); each wave owns 32 rows whose
//    Q fragments stay in registers for the whole pass.  Two workgroups share a CU.
//  * K and V tiles of 64 keys go HBM -> LDS with buffer loads that write LDS directly (rows past
//    the end read as zero), row-major with a 16-byte-chunk XOR swizzle chosen by the address each
//    lane loads from.  K runs one tile ahead of V; each has its own double buffer.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: each lane holds
//    one query column, so the row max / row sum are in-lane plus one exchange between the two
//    wave halves (v_permlane32_swap), and the O^T rescale is a per-lane multiply.
//  * Software pipeline: the 16 MFMAs of S_(j+1) are interleaved with the softmax of tile j, one
//    slice of vector work behind each MFMA, so a wave keeps its matrix core busy while it does
//    the exponentials; then O^T += V_j^T P_j^T with V^T operands from transposing LDS reads
//    (ds_read_b64_tr_b16) and P^T (bf16) straight from registers.
//  * l sums the bf16-rounded p, so O is a true convex combination.  The running max is only
//    raised when a row's new max exceeds it by more than 2^8 (log2 domain); in between p <= 256,
//    exact in fp32, and rescales stay rare.
//  * Key tiles outside the workgroup's causal / segment range are never visited.  Inside it, a
//    tile is masked element-wise only when it straddles a boundary or the ragged end (a tile one
//    wave sees nothing of is computed fully masked: there are few, and the pipeline stays
//    branch-free).
//  * Fused RoPE (lwm_blockattn_fwd_rope): q holds the pre-RoPE queries and each wave rotates its
//    rows' fragments in registers right after loading them (the standalone RoPE kernel's
//    arithmetic from rope_dev.hpp, so the bits are those of a separate pass), optionally storing
//    the rotated rows for the backward.  Keys are not rotated here: every query tile streams them
//    again, and rotating each visit would add a third to the loop's vector work.
//  * Workgroups are numbered longest-first, and when B*H is a multiple of 8 the (batch, head)
//    pairs are dealt to the 8 XCDs so the query tiles sharing one head's K/V run on one L2.  In a
//    packed row a tile's work is its position inside its segment, so there each query tile is
//    dealt to every (batch, head) before the next one (tile-major order).
//  * When both sides share one segment array and offset under the causal mask (packed
//    self-attention), one search over the ids gives the key range; the Q rows are loaded first
//    so that their loads overlap it.
#include <float.h>

#include <type_traits>

#include "attn_common.hpp"
#include "profile.hpp"
#include "rope_dev.hpp"

namespace lwm {
namespace {

constexpr int BN = 64;                 // keys per tile (bf16 path)
constexpr int kTileBytes = BN * 256;   // one K or V tile: 64 rows x 128 bf16
constexpr float kRescaleSlack = 8.0f;  // log2 units: p <= 2^8 between rescales

// Key range [kbeg, kend) that can be visible to query rows [r0, r1] (inclusive).
__device__ inline void key_range(const FwdParams& p, int b, int r0, int r1, int& kbeg, int& kend) {
  kbeg = 0;
  kend = p.Lk;
  if (p.causal) {
    const int64_t lim = p.q_offset + r1 - p.k_offset + 1;
    kend = (int)imax64(0, imin64(kend, lim));
  }
  if (p.seg_q) {
    const int32_t* segk = p.seg_k + (int64_t)b * p.Lk;
    if (causal_self_segments(p.seg_q, p.seg_k, p.Lq, p.Lk, p.q_offset, p.k_offset, p.causal)) {
      // one array and offset for both sides: the last row's segment reaches at least the row
      // itself, so the causal limit already ends the range
      kbeg = max(kbeg, wave_lower_bound(segk, p.Lk, segk[r0]));
    } else {
      int lo, hi;
      segment_range(segk, p.Lk, p.seg_q[(int64_t)b * p.Lq + r0], p.seg_q[(int64_t)b * p.Lq + r1], lo, hi);
      kbeg = max(kbeg, lo);
      kend = min(kend, hi);
    }
  }
}

// ---------------------------------------------------------------------------- bf16 kernel
// Software-pipelined over key tiles: while the MFMAs of S_(j+1) = K_(j+1) Q^T run, the same wave
// issues the softmax of tile j (independent VALU work), so the matrix cores and the vector ALUs
// of a SIMD work at the same time even within one wave; O += V_j^T P_j follows.  K runs one tile
// ahead of V, so K tiles and V tiles (with their segment ids) are double-buffered separately.
struct SmemSp {
  union {
    struct {
      uint8_t k[2][kTileBytes];
      uint8_t v[2][kTileBytes];
      int32_t seg[2][BN];
    } t;
    uint8_t stage_rows[kWaves][32 * D * 4];  // epilogue staging (fp32 rows), after the loop
  };
};
static_assert(sizeof(SmemSp) <= 80 * 1024, "two workgroups per CU must fit in LDS");

template <bool kSegs, bool kRing, bool kRope = false>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(FwdParams p) {
  static_assert(!(kRing && kRope), "the ring step takes rotated queries");
  constexpr int BM = kWaves * 32;
  __shared__ __attribute__((aligned(1024))) SmemSp sm;

  // the wave index is uniform; say so, so LDS bases derived from it stay in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, h32 = lane >> 5;
  const int nqt = (p.Lq + BM - 1) / BM;
  int bh, qt;
  map_block(blockIdx.x, nqt, p.B * p.H, true, kSegs, bh, qt);
  const int b = bh / p.H, hh = bh - b * p.H;
  const int q0 = qt * BM;
  const int qlast = min(q0 + BM, p.Lq) - 1;
  const int wr0 = q0 + w * 32;
  const int wr1 = min(wr0 + 32, p.Lq) - 1;  // may be < wr0 for a ragged last tile
  const bool wave_rows = wr1 >= wr0;

  // the wave's Q rows first: their loads are in flight during the key-range search
  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q) + b * p.sq.b + hh * p.sq.h;
  const int qrow = wr0 + c32;
  const int64_t gq = p.q_offset + qrow;
  bf16x8 qreg[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (qrow < p.Lq) v = *reinterpret_cast<const u32x4*>(qg + qrow * p.sq.l + s * 16 + h32 * 8);
    qreg[s] = as_bf16x8(v);
  }

  int kbeg, kend;
  key_range(p, b, q0, qlast, kbeg, kend);
  const int t_begin = kbeg / BN;
  const int ntiles = (kend > kbeg) ? (kend + BN - 1) / BN - t_begin : 0;

  int32_t wseg0 = 0, wseg1 = 0;
  if (kSegs && wave_rows) {
    wseg0 = p.seg_q[(int64_t)b * p.Lq + wr0];
    wseg1 = p.seg_q[(int64_t)b * p.Lq + wr1];
  }

  const uint8_t* kg = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(p.k) + b * p.sk.b + hh * p.sk.h);
  const uint8_t* vg = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(p.v) + b * p.sv.b + hh * p.sv.h);
  const int64_t kl_bytes = p.sk.l * 2, vl_bytes = p.sv.l * 2;
  const int64_t k_extent = (int64_t)(p.Lk - 1) * kl_bytes + 256, v_extent = (int64_t)(p.Lk - 1) * vl_bytes + 256;
  const int32_t* segk_row = kSegs ? p.seg_k + (int64_t)b * p.Lk : nullptr;
  const int32_t myseg = kSegs ? p.seg_q[(int64_t)b * p.Lq + min(qrow, p.Lq - 1)] : 0;
  if constexpr (kRope) {
    // q holds the pre-RoPE rows: rotate them here (the standalone RoPE kernel's arithmetic, so
    // the bits equal those of a separate RoPE pass) and hand the rotated rows on if asked
    const bool restart = kSegs && p.rope.restart;
    const int64_t pos = rope_row_position(restart ? p.seg_q + (int64_t)b * p.Lq : nullptr, p.Lq, wr0, restart,
                                          p.rope.q_pos_offset);
    rope_rotate_frags(qreg, pos, p.rope, h32);
    if (p.q_rot && qrow < p.Lq) {
      uint16_t* qr = static_cast<uint16_t*>(p.q_rot) + b * p.sqr.b + hh * p.sqr.h + (int64_t)qrow * p.sqr.l;
#pragma unroll
      for (int s = 0; s < 8; ++s) *reinterpret_cast<u32x4*>(qr + s * 16 + h32 * 8) = as_u32x4(qreg[s]);
    }
  }

  // running state: O^T accumulators, row max m (log2-scaled), partial row sum l (this half's keys)
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  float m = -INFINITY, l = 0.f;
  uint8_t* stage_w = sm.stage_rows[w];
  if (kRing && ntiles > 0) {
    load_rows_f32(stage_w, acc, p.o_acc + b * p.soa.b + hh * p.soa.h + wr0 * p.soa.l, p.soa.l,
                  max(0, min(32, p.Lq - wr0)));
    const float ls = qrow < p.Lq ? p.lse_acc[((int64_t)b * p.H + hh) * p.Lq + qrow] : -INFINITY;
    m = ls * kLog2e;
    l = h32 == 0 ? 1.f : 0.f;
  }
  const float m_init = m;

  // ---- loads: wave w fills 1 KB blocks w*4 .. w*4+3 of a tile (4 rows per block); lane l of a
  // block holds row 4*blk + l/16, physical chunk l%16 = logical chunk ^ swz16(row).
  auto ld_off = [&](int r, int64_t row_bytes) {
    const int row = (w * 4 + r) * 4 + (lane >> 4);
    return (int)(row * row_bytes) + (((lane & 15) ^ swz16(row)) << 4);
  };
  auto issue_k = [&](int j) {  // K tile j -> k[j & 1]
    const int k0 = (t_begin + j) * BN;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kg + k0 * kl_bytes, k_extent - k0 * kl_bytes);
#pragma unroll
    for (int r = 0; r < 4; ++r) load_lds16(rk, &sm.t.k[j & 1][(w * 4 + r) * 1024], ld_off(r, kl_bytes));
  };
  auto issue_v = [&](int j) {  // V tile j and its segment ids -> v[j & 1], seg[j & 1]
    const int k0 = (t_begin + j) * BN;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vg + k0 * vl_bytes, v_extent - k0 * vl_bytes);
#pragma unroll
    for (int r = 0; r < 4; ++r) load_lds16(rv, &sm.t.v[j & 1][(w * 4 + r) * 1024], ld_off(r, vl_bytes));
    if (kSegs && w == 0) load_lds4(make_rsrc(segk_row + k0, (int64_t)(p.Lk - k0) * 4), &sm.t.seg[j & 1][0], lane * 4);
  };

  // ---- LDS operand offsets.  K row c32, chunk 2*sd + h32: the XOR swizzle leaves bit 0 of an
  // even chunk index alone, so the offset is a per-lane base plus ((2*sd) ^ swizzle) * 16.  The
  // V^T offsets of feature block db differ from block 0's by an XOR of db into chunk bits 2..3.
  const int kswz = swz16(c32 & 15);
  const int krow_base = c32 * 256 + (((h32 ^ kswz) & 1) << 4);
  int koff[8];
#pragma unroll
  for (int sd = 0; sd < 8; ++sd) koff[sd] = krow_base + (((2 * sd) ^ (kswz & 14)) << 4);
  int vlo0, vhi0;
  tr_offsets(lane, 0, vlo0, vhi0);

  auto kread = [&](const uint8_t* kt, int q) __attribute__((always_inline)) {  // fragment of MFMA q = 2*sd + kb
    return as_bf16x8(*reinterpret_cast<const u32x4*>(kt + (q & 1) * 8192 + koff[q >> 1]));
  };
  // S_j^T = K_j Q^T into s, alone (pipeline prologue)
  auto mma_s = [&](int j, f32x16 (&s)[2]) __attribute__((always_inline)) {
    const uint8_t* kt = sm.t.k[j & 1];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) s[q & 1] = mfma_32x32x16(kread(kt, q), qreg[q >> 1], s[q & 1]);
  };

  // Does tile j need the element mask (ragged end, range edges, causal diagonal, segment edges)?
  auto need_mask = [&](int j) __attribute__((always_inline)) {
    const int k0 = (t_begin + j) * BN;
    bool nm = (k0 + BN > p.Lk) || (k0 < kbeg) || (k0 + BN > kend) || !wave_rows;
    if (p.causal) nm = nm || (p.k_offset + k0 + BN - 1 > p.q_offset + wr0);
    if (kSegs) {
      const int32_t ts0 = sm.t.seg[j & 1][0], ts1 = sm.t.seg[j & 1][min(BN, p.Lk - k0) - 1];
      nm = nm || !(ts0 == ts1 && wseg0 == wseg1 && ts0 == wseg0);
    }
    return nm;
  };
  // Element i of key block kb holds tile key kl = kb*32 + 8*(i/4) + 4*h32 + i%4; it is visible iff
  // kl < lim (ragged end, range end, causal limit) and its segment matches this lane's query.
  auto apply_mask = [&](int j, f32x16 (&s)[2]) __attribute__((always_inline)) {
    const int k0 = (t_begin + j) * BN;
    int64_t lim64 = (int64_t)min(p.Lk, kend) - k0;
    if (p.causal) lim64 = imin64(lim64, gq - p.k_offset - k0 + 1);
    const int lim = wave_rows ? (int)imax64(imin64(lim64, BN), 0) - 4 * h32 : -BN;
    const int32_t* segt = &sm.t.seg[j & 1][4 * h32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        i32x4 ks = {0, 0, 0, 0};
        if (kSegs) ks = *reinterpret_cast<const i32x4*>(segt + kb * 32 + 8 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool vis = (kb * 32 + 8 * g + r < lim) & (!kSegs | (ks[r] == myseg));
          s[kb][4 * g + r] = vis ? s[kb][4 * g + r] : -INFINITY;
        }
      }
  };

  // Online softmax of tile j in 16 slices, so that one slice of vector work can be issued behind
  // each MFMA of the next tile's scores.  Branch-free: the running max is raised (lazily, by more
  // than the slack) only when some row of the wave needs it, and alpha, the factor the accumulator
  // must be scaled by, is exactly 1 otherwise.  Leaves P_j^T (bf16) in pb.
  bf16x8 pb[2][2];
  struct SoftmaxState {
    float t4[4];
    float alpha, moff;
    float lsum[4];
    u32x4 packed[2][2];
  };
  auto softmax_slice = [&](int q, const f32x16 (&s)[2], SoftmaxState& x) __attribute__((always_inline)) {
    if (q < 4) {  // maximum of 8 of the 32 in-lane scores (three-input maxima)
      const f32x16& a = s[q >> 1];
      const int o = (q & 1) * 8;
      float t = fmaxf(fmaxf(a[o], a[o + 1]), a[o + 2]);
      t = fmaxf(fmaxf(t, a[o + 3]), a[o + 4]);
      t = fmaxf(fmaxf(t, a[o + 5]), a[o + 6]);
      x.t4[q] = fmaxf(t, a[o + 7]);
    } else if (q == 4) {  // row max over the lane pair, lazy raise of the running max
      const float mx = pair_max(fmaxf(fmaxf(fmaxf(x.t4[0], x.t4[1]), x.t4[2]), x.t4[3])) * p.scale_log2;
      const bool raise = __any(mx > m + kRescaleSlack);
      const float mnew = raise ? fmaxf(m, mx) : m;
      x.alpha = (!raise || mnew == -INFINITY) ? 1.f : fast_exp2(m - mnew);
      m = mnew;
      x.moff = (mnew == -INFINITY) ? 0.f : mnew;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) x.lsum[jj] = 0.f;
    } else if (q < 13) {  // p = exp2(s * scale_log2 - m) for 4 scores, rounded to bf16 pairs
      const int e = q - 5;  // 0..7: block kb = e / 4, 8-element half u = (e / 2) % 2, word pair (e % 2) * 2
      const int kb = e >> 2, u = (e >> 1) & 1;
#pragma unroll
      for (int jj = (e & 1) * 2; jj < (e & 1) * 2 + 2; ++jj) {
        const float e0 = fast_exp2(__builtin_fmaf(s[kb][u * 8 + 2 * jj], p.scale_log2, -x.moff));
        const float e1 = fast_exp2(__builtin_fmaf(s[kb][u * 8 + 2 * jj + 1], p.scale_log2, -x.moff));
        const uint32_t word = pack_bf16x2(e0, e1);
        x.lsum[jj] = sum_bf16x2(word, x.lsum[jj]);
        x.packed[kb][u][jj] = word;
        // keep the work in this slice: without a use here the compiler sinks it past the MFMAs
        asm volatile("" ::"v"(word), "v"(x.lsum[jj]));
      }
    } else if (q == 13) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u) pb[kb][u] = as_bf16x8(x.packed[kb][u]);
      l = __builtin_fmaf(l, x.alpha, (x.lsum[0] + x.lsum[1]) + (x.lsum[2] + x.lsum[3]));
    }
  };
  auto rescale = [&](float alpha) __attribute__((always_inline)) {
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    }
  };
  // O^T += V_j^T P_j^T (V^T operands by transposing reads, issued two MFMAs ahead)
  auto mma_pv = [&](int j) __attribute__((always_inline)) {
    const uint8_t* vt = sm.t.v[j & 1];
    bf16x8 vf[3];
    auto vread = [&](int n) { return read_xt(vt + (n >> 2) * 4096, vlo0 ^ ((n & 3) << 6), vhi0 ^ ((n & 3) << 6)); };
    vf[0] = vread(0);
    vf[1] = vread(1);
#pragma unroll
    for (int n = 0; n < 16; ++n) {  // n = 16-key group * 4 + feature block
      if (n + 2 < 16) vf[(n + 2) % 3] = vread(n + 2);
      __builtin_amdgcn_sched_barrier(0);
      const int g = n >> 2, db = n & 3;
      acc[db] = mfma_32x32x16(vf[n % 3], pb[g >> 1][g & 1], acc[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One step of the pipeline.  On entry s_cur = S_j (raw), K_(j+1) and V_j are in LDS.  Loads of
  // K_(j+2) and V_(j+1) go into the buffers of K_j and V_(j-1), whose last readers finished before
  // the previous step's barrier, and are waited for at the end of the step.
  auto step = [&](int j, f32x16 (&s_cur)[2], f32x16 (&s_next)[2], auto has_next) __attribute__((always_inline)) {
    constexpr bool kNext = decltype(has_next)::value;
    if (j + 2 < ntiles) issue_k(j + 2);
    if (j + 1 < ntiles) issue_v(j + 1);
    if (need_mask(j)) apply_mask(j, s_cur);
    SoftmaxState x;
    // the half with the vector work runs at raised wave priority: when this SIMD's other wave is
    // in its pure-MFMA half, the softmax instructions issue first and the MFMAs fill around them
    __builtin_amdgcn_s_setprio(1);
    if constexpr (kNext) {
      // MFMA q of S_(j+1) (K fragments four MFMAs ahead), then softmax slice q of tile j
      const uint8_t* kt = sm.t.k[(j + 1) & 1];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s_next[kb][i] = 0.f;
      constexpr int kAhead = 3;  // K fragments read this many MFMAs ahead
      bf16x8 kf[kAhead + 1];
#pragma unroll
      for (int q = 0; q < kAhead; ++q) kf[q] = kread(kt, q);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (q + kAhead < 16) kf[(q + kAhead) % (kAhead + 1)] = kread(kt, q + kAhead);
        s_next[q & 1] = mfma_32x32x16(kf[q % (kAhead + 1)], qreg[q >> 1], s_next[q & 1]);
        softmax_slice(q, s_cur, x);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 16; ++q) softmax_slice(q, s_cur, x);
    }
    rescale(x.alpha);
    __builtin_amdgcn_s_setprio(0);
    mma_pv(j);
    wait_vmcnt<0>();
    __syncthreads();
  };

  if (ntiles > 0) {
    f32x16 s0[2], s1[2];
    issue_k(0);
    issue_v(0);
    if (ntiles > 1) issue_k(1);
    wait_vmcnt<0>();
    __syncthreads();
    mma_s(0, s0);
    __syncthreads();  // K_0 is read by every wave before step 0 reloads its buffer
    int j = 0;
    for (; j + 2 < ntiles; j += 2) {
      step(j, s0, s1, std::true_type{});
      step(j + 1, s1, s0, std::true_type{});
    }
    if (j + 1 < ntiles) {
      step(j, s0, s1, std::true_type{});
      step(j + 1, s1, s0, std::false_type{});
    } else {
      step(j, s0, s1, std::false_type{});
    }
  }

  // ---- epilogue: O = acc / l, lse = (m + log2 l) ln 2 (LDS now holds the staging rows)
  uint16_t* og = static_cast<uint16_t*>(p.o);
  const int rows_valid = max(0, min(32, p.Lq - wr0));
  const float lt = pair_sum(l);
  const bool any = (lt > 0.f) && (m != -INFINITY);
  const float inv = any ? 1.f / lt : 0.f;
  const float lse = any ? (m + log2f(lt)) * kLn2 : -INFINITY;
  if constexpr (!kRing) {
    if (og) store_rows_bf16(stage_w, acc, inv, og + b * p.so.b + hh * p.so.h + wr0 * p.so.l, p.so.l, rows_valid);
    if (p.lse && h32 == 0 && qrow < p.Lq) p.lse[((int64_t)b * p.H + hh) * p.Lq + qrow] = lse;
  } else {
    float* lag = p.lse_acc + ((int64_t)b * p.H + hh) * p.Lq;
    float* oag = p.o_acc + b * p.soa.b + hh * p.soa.h + wr0 * p.soa.l;
    uint16_t* ofg = og ? og + b * p.so.b + hh * p.so.h + wr0 * p.so.l : nullptr;
    if (ntiles > 0) {
      // a row that saw nothing new keeps its state bit for bit
      const bool untouched = (m == m_init) && (lt == 1.f);
      const float sc = untouched ? 1.f : inv;
      store_rows_f32(stage_w, acc, sc, oag, p.soa.l, rows_valid);
      if (h32 == 0 && qrow < p.Lq && !untouched) lag[qrow] = lse;
      if (ofg) store_rows_bf16(stage_w, acc, sc, ofg, p.so.l, rows_valid);
    } else if (ofg) {
      // nothing visible in this shard for the whole tile: the bf16 copy is the state itself
      f32x16 tmp[4];
      load_rows_f32(stage_w, tmp, oag, p.soa.l, rows_valid);
      store_rows_bf16(stage_w, tmp, 1.f, ofg, p.so.l, rows_valid);
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
  map_block(blockIdx.x, nqt, p.B * p.H, true, p.seg_q != nullptr, bh, qt);
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
    const int nqt = (p.Lq + kWaves * 32 - 1) / (kWaves * 32);
    const dim3 grid(nqt * p.B * p.H), block(kThreads);
    const bool segs = p.seg_q != nullptr;
    if (p.mode == 1) {
      if (segs) LWM_LAUNCH("ring_step_bf16", (attn_fwd_bf16_kernel<true, true>), grid, block, stream, p);
      else LWM_LAUNCH("ring_step_bf16", (attn_fwd_bf16_kernel<false, true>), grid, block, stream, p);
    } else if (p.rope.on) {
      if (segs) LWM_LAUNCH("attn_fwd_rope_bf16", (attn_fwd_bf16_kernel<true, false, true>), grid, block, stream, p);
      else LWM_LAUNCH("attn_fwd_rope_bf16", (attn_fwd_bf16_kernel<false, false, true>), grid, block, stream, p);
    } else {
      if (segs) LWM_LAUNCH("attn_fwd_bf16", (attn_fwd_bf16_kernel<true, false>), grid, block, stream, p);
      else LWM_LAUNCH("attn_fwd_bf16", (attn_fwd_bf16_kernel<false, false>), grid, block, stream, p);
    }
  } else {
    const int nqt = (p.Lq + 127) / 128;
    LWM_LAUNCH("attn_fwd_f32", attn_fwd_f32_kernel, dim3(nqt * p.B * p.H), dim3(kThreads), stream, p);
  }
  return hipGetLastError();
}

}  // namespace lwm
