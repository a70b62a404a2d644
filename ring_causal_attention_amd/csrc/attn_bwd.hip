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
//  * delta: one pass over dO and O (HBM-bound).
//  * dQ: a workgroup per 128-query tile walks the visible 64-key tiles like the forward does,
//    with scores transposed (S^T = K Q^T) so each lane owns one query: P^T and dS^T are formed
//    in registers and feed dQ^T += K^T dS^T directly (K is staged both row-major and transposed).
//  * dK/dV: a workgroup per 128-key tile (32 keys per wave) walks the visible 32-query tiles with
//    scores in the other orientation (S = Q K^T, each lane owns one key): P and dS feed
//    dV^T += dO^T P and dK^T += Q^T dS directly (Q and dO are staged both row-major and transposed).
//  Recomputing S and dP in both kernels costs two extra products over the five the method needs;
//  in exchange no partial dQ is ever written to or reduced through memory.
#include "attn_common.hpp"
#include "profile.hpp"

namespace lwm {
namespace {

constexpr int BNQ = 64;  // keys per tile in the dQ kernel
constexpr int BQK = 32;  // queries per tile in the dK/dV kernel

__device__ __forceinline__ float lse_log2(const float* lse_row, int q, int Lq) {
  // +inf for rows without any visible key or past the end: exp2(s - inf) = 0 for every s
  if (q >= Lq) return INFINITY;
  const float v = lse_row[q];
  return v == -INFINITY ? INFINITY : v * kLog2e;
}

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
  if (r < rows && c == 0) p.delta[((int64_t)b * p.H + h) * p.Lq + i] = acc;
}

// ------------------------------------------------------------------------------ dQ
struct SmemDq {
  u32x4 k[2][BNQ * 16];       // row-major K, rm_index
  u32x4 kt[2][D * (BNQ / 8)]; // transposed K, t64_index
  u32x4 v[2][BNQ * 16];       // row-major V, rm_index
  int32_t seg[2][BNQ];
};

__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(BwdParams p) {
  constexpr int MW = 32, BM = kWaves * MW;
  __shared__ SmemDq sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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
  const int t_begin = kbeg / BNQ;
  const int ntiles = (kend > kbeg) ? (kend + BNQ - 1) / BNQ - t_begin : 0;

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
  const float lse2 = lse_log2(p.lse + ((int64_t)b * p.H + hh) * p.Lq, qrow, p.Lq);
  const float dlt = qrow < p.Lq ? p.delta[((int64_t)b * p.H + hh) * p.Lq + qrow] : 0.f;

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

  const uint16_t* kg = p.k + b * p.sk.b + hh * p.sk.h;
  const uint16_t* vg = p.v + b * p.sv.b + hh * p.sv.h;
  const int ld_q = tid >> 4, ld_c = tid & 15;
  u32x4 kst[4], vst[4];
  int32_t segst = -1;
  auto gload = [&](int tile) {
    const int k0 = tile * BNQ;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = k0 + 4 * ld_q + r;  // K: quad ld_q, chunk ld_c
      kst[r] = kk < p.Lk ? *reinterpret_cast<const u32x4*>(kg + kk * p.sk.l + ld_c * 8) : u32x4{0u, 0u, 0u, 0u};
      const int kv = k0 + r * 16 + ld_q;  // V: row r*16 + ld_q, chunk ld_c
      vst[r] = kv < p.Lk ? *reinterpret_cast<const u32x4*>(vg + kv * p.sv.l + ld_c * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    if (segs && tid < BNQ) segst = (k0 + tid < p.Lk) ? p.seg_k[(int64_t)b * p.Lk + k0 + tid] : -1;
  };
  auto swrite = [&](int st) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sm.k[st][rm_index(4 * ld_q + r, ld_c)] = kst[r];
      sm.v[st][rm_index(r * 16 + ld_q, ld_c)] = vst[r];
    }
    write_transposed_quad<BNQ>(sm.kt[st], ld_q, ld_c, kst);
    if (segs && tid < BNQ) sm.seg[st][tid] = segst;
  };

  if (ntiles > 0) {
    gload(t_begin);
    swrite(0);
    __syncthreads();
  }
  for (int it = 0; it < ntiles; ++it) {
    const int st = it & 1;
    const int k0 = (t_begin + it) * BNQ;
    if (it + 1 < ntiles) gload(t_begin + it + 1);
    bool active = wave_rows;
    bool need_mask = (k0 + BNQ > p.Lk) || (k0 < kbeg) || (k0 + BNQ > kend);
    if (p.causal) {
      active = active && (p.k_offset + k0 <= p.q_offset + wr1);
      need_mask = need_mask || (p.k_offset + k0 + BNQ - 1 > p.q_offset + wr0);
    }
    if (segs) {
      const int32_t ts0 = sm.seg[st][0], ts1 = sm.seg[st][min(BNQ, p.Lk - k0) - 1];
      active = active && !(ts1 < wseg0 || ts0 > wseg1);
      need_mask = need_mask || !(ts0 == ts1 && wseg0 == wseg1 && ts0 == wseg0);
    }
    if (active) {
      f32x16 s[2], dp[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = dp[kb][i] = 0.f;
#pragma unroll
      for (int sd = 0; sd < 8; ++sd)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int idx = rm_index(kb * 32 + c32, 2 * sd + h32);
          s[kb] = mfma_32x32x16(as_bf16x8(sm.k[st][idx]), qreg[sd], s[kb]);
          dp[kb] = mfma_32x32x16(as_bf16x8(sm.v[st][idx]), doreg[sd], dp[kb]);
        }
      bf16x8 dsb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kl = kb * 32 + acc_row(i, h32);
          bool vis = true;
          if (need_mask) {
            const int key = k0 + kl;
            vis = key < p.Lk;
            if (p.causal) vis = vis && (p.k_offset + key <= gq);
            if (segs) vis = vis && (sm.seg[st][kl] == myseg);
          }
          const float pr = vis ? fast_exp2(__builtin_fmaf(s[kb][i], p.scale_log2, -lse2)) : 0.f;
          s[kb][i] = pr * (dp[kb][i] - dlt);
        }
        dsb[kb][0] = pack8(s[kb], 0);
        dsb[kb][1] = pack8(s[kb], 1);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const bf16x8 a = as_bf16x8(sm.kt[st][t64_index(db * 32 + c32, (kb * 2 + u) * 2 + h32)]);
            acc[db] = mfma_32x32x16(a, dsb[kb][u], acc[db]);
          }
    }
    if (it + 1 < ntiles) swrite(st ^ 1);
    __syncthreads();
  }
  uint8_t* stage_w = reinterpret_cast<uint8_t*>(&sm) + w * (32 * D * 2);
  store_rows_bf16(stage_w, acc, p.scale, p.dq + b * p.sdq.b + hh * p.sdq.h + wr0 * p.sdq.l, p.sdq.l,
                  max(0, min(32, p.Lq - wr0)));
}

// ------------------------------------------------------------------------------ dK / dV
struct SmemDkdv {
  u32x4 q[2][BQK * 16];        // row-major Q tile, rm_index
  u32x4 qt[2][D * (BQK / 8)];  // transposed Q tile, t32_index
  u32x4 o[2][BQK * 16];        // row-major dO tile
  u32x4 ot[2][D * (BQK / 8)];  // transposed dO tile
  float lse2[2][BQK];
  float dlt[2][BQK];
  int32_t seg[2][BQK];
};

__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int NW = 32, BK = kWaves * NW;
  __shared__ SmemDkdv sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c32 = lane & 31, h32 = lane >> 5;
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
  const int t_begin = qbeg / BQK;
  const int ntiles = (qend > qbeg) ? (qend + BQK - 1) / BQK - t_begin : 0;

  const int wk0 = k0 + w * NW, wk1 = min(wk0 + NW, p.Lk) - 1;
  const bool wave_keys = wk1 >= wk0;
  int32_t wseg0 = 0, wseg1 = 0;
  if (segs && wave_keys) {
    wseg0 = p.seg_k[(int64_t)b * p.Lk + wk0];
    wseg1 = p.seg_k[(int64_t)b * p.Lk + wk1];
  }
  const int krow = wk0 + c32;
  const int64_t gk = p.k_offset + krow;
  const int32_t myseg = segs ? p.seg_k[(int64_t)b * p.Lk + min(krow, p.Lk - 1)] : 0;

  bf16x8 kreg[8], vreg[8];
  {
    const uint16_t* kg = p.k + b * p.sk.b + hh * p.sk.h + (int64_t)krow * p.sk.l;
    const uint16_t* vg = p.v + b * p.sv.b + hh * p.sv.h + (int64_t)krow * p.sv.l;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
      if (krow < p.Lk) {
        a = *reinterpret_cast<const u32x4*>(kg + s * 16 + h32 * 8);
        c = *reinterpret_cast<const u32x4*>(vg + s * 16 + h32 * 8);
      }
      kreg[s] = as_bf16x8(a);
      vreg[s] = as_bf16x8(c);
    }
  }
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[db][i] = dv[db][i] = 0.f;

  // loader: threads 0..127 stage Q, 128..255 stage dO; each holds one quad of rows x one chunk
  const bool ld_do = tid >= 128;
  const int ld_q = (tid >> 4) & 7, ld_c = tid & 15;
  const uint16_t* src = ld_do ? p.dout + b * p.sdo.b + hh * p.sdo.h : p.q + b * p.sq.b + hh * p.sq.h;
  const int64_t src_l = ld_do ? p.sdo.l : p.sq.l;
  const float* lse_row = p.lse + ((int64_t)b * p.H + hh) * p.Lq;
  const float* dlt_row = p.delta + ((int64_t)b * p.H + hh) * p.Lq;
  u32x4 rst[4];
  float l2st = 0.f, dst = 0.f;
  int32_t segst = -1;
  auto gload = [&](int tile) {
    const int q0 = tile * BQK;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qq = q0 + 4 * ld_q + r;
      rst[r] = qq < p.Lq ? *reinterpret_cast<const u32x4*>(src + qq * src_l + ld_c * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < BQK) {
      const int qq = q0 + tid;
      l2st = lse_log2(lse_row, qq, p.Lq);
      dst = qq < p.Lq ? dlt_row[qq] : 0.f;
      if (segs) segst = qq < p.Lq ? p.seg_q[(int64_t)b * p.Lq + qq] : -1;
    }
  };
  auto swrite = [&](int st) {
    u32x4* rm = ld_do ? sm.o[st] : sm.q[st];
    u32x4* tr = ld_do ? sm.ot[st] : sm.qt[st];
#pragma unroll
    for (int r = 0; r < 4; ++r) rm[rm_index(4 * ld_q + r, ld_c)] = rst[r];
    write_transposed_quad<BQK>(tr, ld_q, ld_c, rst);
    if (tid < BQK) {
      sm.lse2[st][tid] = l2st;
      sm.dlt[st][tid] = dst;
      if (segs) sm.seg[st][tid] = segst;
    }
  };

  if (ntiles > 0) {
    gload(t_begin);
    swrite(0);
    __syncthreads();
  }
  for (int it = 0; it < ntiles; ++it) {
    const int st = it & 1;
    const int q0 = (t_begin + it) * BQK;
    if (it + 1 < ntiles) gload(t_begin + it + 1);
    bool active = wave_keys;
    bool need_mask = false;
    if (p.causal) {
      active = active && (p.q_offset + q0 + BQK - 1 >= p.k_offset + wk0);
      need_mask = p.k_offset + wk1 > p.q_offset + q0;
    }
    if (segs) {
      const int32_t ts0 = sm.seg[st][0], ts1 = sm.seg[st][min(BQK, p.Lq - q0) - 1];
      active = active && !(ts1 < wseg0 || ts0 > wseg1);
      need_mask = need_mask || !(ts0 == ts1 && wseg0 == wseg1 && ts0 == wseg0);
    }
    if (active) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
      for (int sd = 0; sd < 8; ++sd) {
        const int idx = rm_index(c32, 2 * sd + h32);
        s = mfma_32x32x16(as_bf16x8(sm.q[st][idx]), kreg[sd], s);
        dp = mfma_32x32x16(as_bf16x8(sm.o[st][idx]), vreg[sd], dp);
      }
      // lane owns key krow; element i is query q0 + acc_row(i, h32)
      f32x16 pm, ds;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r4 = 8 * g + 4 * h32;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse2[st][r4]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sm.dlt[st][r4]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * g + j;
          bool vis = true;
          if (need_mask) {
            const int ql = r4 + j;
            if (p.causal) vis = gk <= p.q_offset + q0 + ql;
            if (segs) vis = vis && (sm.seg[st][ql] == myseg);
          }
          const float pr = vis ? fast_exp2(__builtin_fmaf(s[i], p.scale_log2, -l4[j])) : 0.f;
          pm[i] = pr;
          ds[i] = pr * (dp[i] - d4[j]);
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 pb = pack8(pm, u);
        const bf16x8 dsb = pack8(ds, u);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int ti = t32_index(db * 32 + c32, u * 2 + h32);
          dv[db] = mfma_32x32x16(as_bf16x8(sm.ot[st][ti]), pb, dv[db]);
          dk[db] = mfma_32x32x16(as_bf16x8(sm.qt[st][ti]), dsb, dk[db]);
        }
      }
    }
    if (it + 1 < ntiles) swrite(st ^ 1);
    __syncthreads();
  }
  static_assert(sizeof(SmemDkdv) >= kWaves * 32 * D * 2, "epilogue staging must fit");
  uint8_t* stage_w = reinterpret_cast<uint8_t*>(&sm) + w * (32 * D * 2);
  const int rows_valid = max(0, min(32, p.Lk - wk0));
  store_rows_bf16(stage_w, dk, p.scale, p.dk + b * p.sdk.b + hh * p.sdk.h + wk0 * p.sdk.l, p.sdk.l, rows_valid);
  store_rows_bf16(stage_w, dv, 1.f, p.dv + b * p.sdv.b + hh * p.sdv.h + wk0 * p.sdv.l, p.sdv.l, rows_valid);
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
    LWM_LAUNCH("bwd_dkdv", bwd_dkdv_kernel, dim3(nkt * p.B * p.H), dim3(kThreads), stream, p);
  }
  return hipGetLastError();
}

}  // namespace lwm
