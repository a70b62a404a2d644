// Blockwise feed-forward block for gfx950: y = (silu(x W_gate^T) * (x W_up^T)) W_down^T.
//
// Method: the feed-forward half of the blockwise transformer is evaluated in chunks of rows
// along the sequence ("LWM：突破 100 万 Token 的开源大模型", section 配置参数: scan_mlp /
// scan_mlp_chunk_size); the block itself is the LLaMA one the PyTorch port loads (same page,
// section 运行 PyTorch 模型).  Weights use the nn.Linear layout [out_features, in_features].
//
// Two GEMM kernels per chunk, both "row times row" (C[m, n] = sum_k A[m, k] B[n, k]) so that
// every MFMA operand is a 16-byte piece of a K-contiguous row:
//  * gate/up: one workgroup computes a 128 x 128 tile of both x W_gate^T and x W_up^T and writes
//    h = silu(gate) * up in bf16 (the chunk's intermediate activations, in the workspace);
//  * down: y = h W_down^T, 128 x 128 tiles.
// Four waves per workgroup (2 x 2 tiles of 64 x 64), two workgroups per CU.  K advances in
// slabs of 32 through a 3-stage LDS ring filled by buffer loads that write LDS directly (rows past
// the end read as zero); LDS rows are 64 bytes with the 16-byte chunk c of row r stored at
// c ^ ((r >> 2) & 3), so the 16 rows one ds_read_b128 pass touches hit 16 distinct bank groups.
// Workgroups are dealt to the 8 XCDs in contiguous ranges and, inside a range, walk 8 row tiles
// by 8 column tiles together, so the operand slabs they stream at the same time are shared in L2.
#include "attn_common.hpp"
#include "profile.hpp"

namespace lwm {
namespace {

constexpr int FBM = 128, FBN = 128, FBK = 32;  // workgroup tile and K slab
constexpr int kFfnStages = 3;
constexpr int kFfnWaves = 4;
constexpr int kRowBytes = FBK * 2;  // 64

__device__ __forceinline__ int swz4(int r) { return (r >> 2) & 3; }
// byte offset of 16-byte chunk c of row r in a slab
__device__ __forceinline__ int slab_off(int r, int c) { return r * kRowBytes + ((c ^ swz4(r)) << 4); }

template <bool kDual>
struct SmemFfn {
  uint8_t a[kFfnStages][FBM * kRowBytes];
  uint8_t b[kFfnStages][(kDual ? 2 : 1) * FBN * kRowBytes];
};
static_assert(sizeof(SmemFfn<true>) <= 80 * 1024, "two workgroups per CU");

// Grid position -> (row tile, column tile).  When the grid is a multiple of 8, XCD x (the block
// ids congruent to x mod 8) gets a contiguous range of the logical order; the logical order walks
// groups of 8 row tiles column by column.
__device__ __forceinline__ void ffn_tile(int bid, int n_m, int n_n, int& tm, int& tn) {
  const int total = n_m * n_n;
  int logical = bid;
  if ((total & 7) == 0) logical = (bid & 7) * (total >> 3) + (bid >> 3);
  constexpr int G = 8;
  const int per_group = G * n_n;
  const int group = logical / per_group;
  const int first_m = group * G;
  const int gsize = min(n_m - first_m, G);
  const int in_group = logical - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// kDual: out = silu(A B_gate^T) * (A B_up^T) (b0 = W_gate, b1 = W_up), else out = A B0^T.
// A [M, K] (lda), B* [N, K] (ldb), out [M, N] (ldo); bf16, leading dimensions in elements.
template <bool kDual>
__global__ __launch_bounds__(kFfnWaves * kWave, 2) void ffn_gemm_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                                       const uint16_t* __restrict__ B0,
                                                                       const uint16_t* __restrict__ B1, int64_t ldb,
                                                                       uint16_t* __restrict__ out, int64_t ldo, int M,
                                                                       int N, int K) {
  __shared__ __attribute__((aligned(1024))) SmemFfn<kDual> sm;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, h32 = lane >> 5;
  const int wm = w & 1, wn = w >> 1;
  const int n_m = (M + FBM - 1) / FBM, n_n = (N + FBN - 1) / FBN;
  int tm, tn;
  ffn_tile(blockIdx.x, n_m, n_n, tm, tn);
  const int m0 = tm * FBM, n0 = tn * FBN;
  const int64_t a_bytes = lda * 2, b_bytes = ldb * 2;
  // rows past M / N read as zero through the buffer ranges
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (int64_t)m0 * lda, (int64_t)(M - m0 - 1) * a_bytes + (int64_t)K * 2);
  const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(B0 + (int64_t)n0 * ldb, (int64_t)(N - n0 - 1) * b_bytes + (int64_t)K * 2);
  const __amdgpu_buffer_rsrc_t rb1 =
      kDual ? make_rsrc(B1 + (int64_t)n0 * ldb, (int64_t)(N - n0 - 1) * b_bytes + (int64_t)K * 2) : rb0;
  const int nk = K / FBK;

  // load plan: 1 KB blocks of 16 rows; lane l writes row 16*blk + l/4, chunk slot l%4, which
  // holds logical chunk (l%4) ^ swz4(row)
  auto src_off = [&](int blk, int64_t row_bytes) {
    const int row = blk * 16 + (lane >> 2);
    return (int)(row * row_bytes) + (((lane & 3) ^ swz4(row)) << 4);
  };
  constexpr int kBBlocks = (kDual ? 2 : 1) * FBN / 16;  // 16 or 8
  constexpr int kBPerWave = kBBlocks / kFfnWaves;       // 4 or 2
  const int a_off[2] = {src_off(w * 2, a_bytes), src_off(w * 2 + 1, a_bytes)};
  int b_off[kBPerWave];
#pragma unroll
  for (int r = 0; r < kBPerWave; ++r) b_off[r] = src_off((w * kBPerWave + r) % (FBN / 16), b_bytes);
  auto issue = [&](int t) {
    const int st = t % kFfnStages;
    const int kb = t * FBK * 2;  // byte offset of the slab along K
#pragma unroll
    for (int r = 0; r < 2; ++r)
      load_lds16(ra, &sm.a[st][(w * 2 + r) * 1024], a_off[r] + kb);
#pragma unroll
    for (int r = 0; r < kBPerWave; ++r) {
      const int blk = w * kBPerWave + r;  // blocks 0..7: B0 rows, 8..15: B1 rows
      load_lds16(blk < FBN / 16 ? rb0 : rb1, &sm.b[st][blk * 1024], b_off[r] + kb);
    }
  };
  constexpr int kLoadsPerStage = 2 + kBPerWave;

  constexpr int NB = kDual ? 2 : 1;  // B operands per output tile
  f32x16 acc[NB][2][2];              // [gate/up][m block][n block]
#pragma unroll
  for (int g = 0; g < NB; ++g)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][mb][nb][i] = 0.f;

  int aoff[2][2], boff[2][2];  // [k16 step][block]: LDS offsets of this lane's fragments
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      aoff[s][x] = slab_off(wm * 64 + x * 32 + c32, 2 * s + h32);
      boff[s][x] = slab_off(wn * 64 + x * 32 + c32, 2 * s + h32);
    }

  if (nk > 0) issue(0);
  if (nk > 1) issue(1);
  for (int t = 0; t < nk; ++t) {
    const int st = t % kFfnStages;
    if (t + 1 < nk) wait_vmcnt<kLoadsPerStage>();
    else wait_vmcnt<0>();
    __syncthreads();  // slab t is in LDS for every wave; every wave is done with slab t-1
    if (t + 2 < nk) issue(t + 2);
    const uint8_t* at = sm.a[st];
    const uint8_t* bt = sm.b[st];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 af[2], bf[NB][2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        af[x] = as_bf16x8(*reinterpret_cast<const u32x4*>(at + aoff[s][x]));
#pragma unroll
        for (int g = 0; g < NB; ++g)
          bf[g][x] = as_bf16x8(*reinterpret_cast<const u32x4*>(bt + g * FBN * kRowBytes + boff[s][x]));
      }
#pragma unroll
      for (int g = 0; g < NB; ++g)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) acc[g][mb][nb] = mfma_32x32x16(bf[g][nb], af[mb], acc[g][mb][nb]);
    }
  }

  // epilogue: the accumulators hold C^T blocks, so element i of a block is row m = c32 and
  // column n = 8*(i/4) + 4*h32 + i%4: four consecutive columns per group of 4, one 8-byte store
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + wm * 64 + mb * 32 + c32;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 64 + nb * 32 + 8 * q + 4 * h32;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[0][mb][nb][4 * q + e];
          if constexpr (kDual) {
            // silu(g) * u with silu(g) = g / (1 + 2^(-g log2 e)); the exponent's overflow to +inf
            // gives -0 for large negative g, the right limit
            v[e] = v[e] * __builtin_amdgcn_rcpf(1.f + fast_exp2(-v[e] * kLog2e)) * acc[1][mb][nb][4 * q + e];
          }
        }
        if (m < M && n < N)  // N is a multiple of 32, so the 4 columns are all in range
          *reinterpret_cast<u32x2*>(out + (int64_t)m * ldo + n) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
  }
}

}  // namespace

hipError_t launch_ffn(const FfnParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  for (int64_t r0 = 0; r0 < p.rows; r0 += p.chunk) {
    const int m = (int)(p.rows - r0 < p.chunk ? p.rows - r0 : p.chunk);
    const uint16_t* x = p.x + r0 * p.ldx;
    uint16_t* y = p.y + r0 * p.ldy;
    // h = silu(x W_gate^T) * (x W_up^T): [m, d_ff] in the workspace (leading dimension d_ff)
    {
      const int n_m = (m + FBM - 1) / FBM, n_n = (p.d_ff + FBN - 1) / FBN;
      LWM_LAUNCH("ffn_gate_up", ffn_gemm_kernel<true>, dim3(n_m * n_n), dim3(kFfnWaves * kWave), stream, x, p.ldx,
                 p.w_gate, p.w_up, p.ldw, p.h, (int64_t)p.d_ff, m, p.d_ff, p.d_model);
    }
    // y = h W_down^T: [m, d_model]
    {
      const int n_m = (m + FBM - 1) / FBM, n_n = (p.d_model + FBN - 1) / FBN;
      LWM_LAUNCH("ffn_down", ffn_gemm_kernel<false>, dim3(n_m * n_n), dim3(kFfnWaves * kWave), stream,
                 (const uint16_t*)p.h, (int64_t)p.d_ff, p.w_down, (const uint16_t*)nullptr, p.ldwd, y, p.ldy, m,
                 p.d_model, p.d_ff);
    }
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lwm
