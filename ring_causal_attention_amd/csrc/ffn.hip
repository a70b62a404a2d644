// Blockwise feed-forward block for gfx950: y = (silu(x W_gate^T) * (x W_up^T)) W_down^T.
//
// Method: the feed-forward half of the blockwise transformer is evaluated in chunks of rows
// along the sequence ("LWM：突破 100 万 Token 的开源大模型", section 配置参数: scan_mlp /
// scan_mlp_chunk_size); the block itself is the LLaMA one the PyTorch port loads (same page,
// section 运行 PyTorch 模型).  Weights use the nn.Linear layout [out_features, in_features].
//
// Two GEMM kernels per chunk, both "row times row" (C[m, n] = sum_k A[m, k] B[n, k]) so that
// every MFMA operand is a 16-byte piece of a K-contiguous row:
//  * gate/up: one workgroup computes a 256 x 128 tile of both x W_gate^T and x W_up^T and writes
//    h = silu(gate) * up in bf16 (the chunk's intermediate activations, in the workspace);
//  * down: y = h W_down^T in 256 x 256 tiles.
// One workgroup of four waves per CU, one wave per SIMD: a wave owns 128 rows x 64 columns of
// both operand tiles (256 float32 accumulators, held in the accumulation registers), so a k step
// reads 8 operand fragments for 16 MFMAs.  K advances in slabs of 32 through a 4-stage LDS ring
// (128 KB) filled by buffer loads that write LDS directly (rows past the end read as zero); LDS
// rows are 64 bytes with the 16-byte chunk c of row r stored at c ^ ((r >> 2) & 3), so the 16
// rows one ds_read_b128 pass touches hit 16 distinct bank groups.  With a single wave per SIMD
// the instruction stream is the schedule: the slab's loads and the next step's fragment reads are
// spread one per MFMA pair, one barrier per slab, each wave waiting only for its own loads of
// the slab it is about to read (slabs further ahead stay in flight).
// Workgroups are dealt to the 8 XCDs in contiguous ranges and, inside a range, walk 8 row tiles
// by the column tiles, so the operand slabs they stream at the same time are shared in L2.
#include <type_traits>

#include "attn_common.hpp"
#include "profile.hpp"

namespace lwm {
namespace {

constexpr int FBN = 128, FBK = 32;  // operand tile rows (per B tile) and K slab
constexpr int kFfnWaves = 4;
constexpr int kRowBytes = FBK * 2;  // 64

__device__ __forceinline__ int swz4(int r) { return (r >> 2) & 3; }
// byte offset of 16-byte chunk c of row r in a slab
__device__ __forceinline__ int slab_off(int r, int c) { return r * kRowBytes + ((c ^ swz4(r)) << 4); }

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

// C = A B^T for one workgroup tile of (64 kMB) rows x two 128-row operand tiles B0, B1.
// kSwiGLU: out = silu(A B0^T) * (A B1^T) with B0 = W_gate, B1 = W_up: tile (64 kMB) x 128.
// Otherwise out = A B0^T in tiles of (64 kMB) x 256, B1 = B0 + 128 rows being the second half.
// A [M, K] (lda), B* [N, K] (ldb), out [M, N] (ldo); bf16, leading dimensions in elements;
// K a multiple of 32.  Waves form a 2 x 2 grid: wave (wm, wn) owns rows wm*32*kMB .. +32*kMB
// and columns wn*64 .. +64 of both operand tiles.
template <bool kSwiGLU, int kMB, int kStages, int kOcc>
__global__ __launch_bounds__(kFfnWaves * kWave, kOcc) void ffn_gemm_kernel(const uint16_t* __restrict__ A, int64_t lda,
                                                                          const uint16_t* __restrict__ B0,
                                                                          const uint16_t* __restrict__ B1, int64_t ldb,
                                                                          uint16_t* __restrict__ out, int64_t ldo,
                                                                          int M, int N, int K) {
  constexpr int FBM = 64 * kMB;
  constexpr int kABytes = FBM * kRowBytes, kBBytes = 2 * FBN * kRowBytes;
  static_assert(kStages * (kABytes + kBBytes) <= 160 * 1024 / kOcc, "LDS per CU");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages][kABytes + kBBytes];
  constexpr int kTileN = kSwiGLU ? FBN : 2 * FBN;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, h32 = lane >> 5;
  const int wm = w & 1, wn = w >> 1;
  const int n_m = (M + FBM - 1) / FBM, n_n = (N + kTileN - 1) / kTileN;
  int tm, tn;
  ffn_tile(blockIdx.x, n_m, n_n, tm, tn);
  const int m0 = tm * FBM, n0 = tn * kTileN;
  const int n1 = kSwiGLU ? n0 : n0 + FBN;  // first row of the second operand tile
  const int64_t a_bytes = lda * 2, b_bytes = ldb * 2;
  // rows past M / N read as zero through the buffer ranges
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (int64_t)m0 * lda, (int64_t)(M - m0 - 1) * a_bytes + (int64_t)K * 2);
  const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(B0 + (int64_t)n0 * ldb, (int64_t)(N - n0 - 1) * b_bytes + (int64_t)K * 2);
  const __amdgpu_buffer_rsrc_t rb1 = make_rsrc(B1 + (int64_t)n1 * ldb, (int64_t)(N - n1 - 1) * b_bytes + (int64_t)K * 2);
  const int nk = K / FBK;

  // load plan: 1 KB blocks of 16 rows; lane l writes row 16*blk + l/4, chunk slot l%4, which
  // holds logical chunk (l%4) ^ swz4(row).  Each wave loads kMB blocks of A and 4 of B.
  auto src_off = [&](int blk, int64_t row_bytes) {
    const int row = blk * 16 + (lane >> 2);
    return (int)(row * row_bytes) + (((lane & 3) ^ swz4(row)) << 4);
  };
  constexpr int kBPerWave = 2 * FBN / 16 / kFfnWaves;  // 4
  constexpr int kLoads = kMB + kBPerWave;              // per wave and slab
  int a_off[kMB], b_off[kBPerWave];
#pragma unroll
  for (int r = 0; r < kMB; ++r) a_off[r] = src_off(w * kMB + r, a_bytes);
#pragma unroll
  for (int r = 0; r < kBPerWave; ++r) b_off[r] = src_off((w * kBPerWave + r) % (FBN / 16), b_bytes);
  // load r (0 .. kLoads-1) of slab t: A blocks first, then B blocks (0..7: B0 rows, 8..15: B1 rows)
  auto issue_one = [&](int t, int r) {
    uint8_t* st = smem[t % kStages];
    const int kb = t * FBK * 2;  // byte offset of the slab along K
    if (r < kMB) {
      load_lds16(ra, st + (w * kMB + r) * 1024, a_off[r] + kb);
    } else {
      const int blk = w * kBPerWave + (r - kMB);
      load_lds16(blk < FBN / 16 ? rb0 : rb1, st + kABytes + blk * 1024, b_off[r - kMB] + kb);
    }
  };
  auto issue = [&](int t) {
#pragma unroll
    for (int r = 0; r < kLoads; ++r) issue_one(t, r);
  };

  f32x16 acc[2][kMB][2];  // [operand tile][m block][n block]
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][mb][nb][i] = 0.f;

  int aoff[kMB], boff[2];  // LDS offsets of this lane's fragments for k16 step 0 (step 1: ^ 32)
#pragma unroll
  for (int x = 0; x < kMB; ++x) aoff[x] = slab_off(wm * 32 * kMB + x * 32 + c32, h32);
#pragma unroll
  for (int x = 0; x < 2; ++x) boff[x] = slab_off(wn * 64 + x * 32 + c32, h32);
  // chunk 2s + h32 of a row: slot (2s + h32) ^ swz = (h32 ^ swz) ^ 2s, i.e. offset ^ (32 s)

  struct Frag {
    bf16x8 a[kMB], b[2][2];
  };
  // fragment r (0 .. kMB+3) of k16 step s of slab t: A blocks first, then B0, B1 blocks
  auto read_one = [&](int t, int s, Frag& f, int r) {
    const uint8_t* st = smem[t % kStages];
    if (r < kMB) {
      f.a[r] = as_bf16x8(*reinterpret_cast<const u32x4*>(st + (aoff[r] ^ (32 * s))));
    } else {
      const int g = (r - kMB) >> 1, x = (r - kMB) & 1;
      f.b[g][x] = as_bf16x8(*reinterpret_cast<const u32x4*>(st + kABytes + g * FBN * kRowBytes + (boff[x] ^ (32 * s))));
    }
  };
  auto read = [&](int t, int s, Frag& f) {
#pragma unroll
    for (int r = 0; r < kMB + 4; ++r) read_one(t, s, f, r);
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[g][mb][nb] = mfma_32x32x16(f.b[g][nb], f.a[mb], acc[g][mb][nb]);
  };
  // mma(f) with the loads of slab t_load (when kLoad) and the step-s_read fragment reads of slab
  // t_read spread between the MFMAs: one wave per SIMD issues in order, so a burst of loads or
  // reads would leave the matrix unit idle while it drains
  constexpr int kMfmas = 4 * kMB;
  static_assert(kMfmas >= 2 * kLoads && kMfmas >= 2 * (kMB + 4), "one load and one read per MFMA pair");
  auto mma_interleaved = [&](auto kLoad, const Frag& f, int t_load, int t_read, int s_read, Frag& fr) {
#pragma unroll
    for (int i = 0; i < kMfmas; ++i) {
      const int g = i / (2 * kMB), mb = (i / 2) % kMB, nb = i % 2;
      acc[g][mb][nb] = mfma_32x32x16(f.b[g][nb], f.a[mb], acc[g][mb][nb]);
      if constexpr (decltype(kLoad)::value) {
        if ((i & 1) == 0 && i / 2 < kLoads) issue_one(t_load, i / 2);
      }
      if ((i & 1) == 1 && i / 2 < kMB + 4) read_one(t_read, s_read, fr, i / 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // every stage starts loading; slab t lives in stage t % kStages and slab t + kStages is issued
  // once every wave has read slab t
#pragma unroll
  for (int t = 0; t < kStages; ++t)
    if (t < nk) issue(t);
  wait_groups<kLoads>(min(nk - 1, kStages - 1));
  block_barrier();
  Frag f0, f1;
  read(0, 0, f0);
  // one slab: MFMAs of step 0 (reading step 1), barrier, MFMAs of step 1 (reading step 0 of the
  // next slab and, while slabs remain, loading slab t + kStages into the stage slab t used)
  auto slab = [&](auto kLoad, int t) {
    mma_interleaved(std::false_type{}, f0, 0, t, 1, f1);
    wait_groups<kLoads>(min(nk - 1, t + kStages - 1) - (t + 1));  // slab t + 1 has landed
    wait_lgkm0();                                                // this wave's reads of slab t are done
    block_barrier();
    mma_interleaved(kLoad, f1, t + kStages, t + 1, 0, f0);
  };
  int t = 0;
  for (; t + kStages < nk; ++t) slab(std::true_type{}, t);
  for (; t + 1 < nk; ++t) slab(std::false_type{}, t);
  // last slab
  mma_interleaved(std::false_type{}, f0, 0, nk - 1, 1, f1);
  mma(f1);

  // epilogue: the accumulators hold C^T blocks, so element i of a block is row m = c32 and
  // column n = 8*(i/4) + 4*h32 + i%4: four consecutive columns per group of 4, one 8-byte store
  constexpr int kOut = kSwiGLU ? 1 : 2;
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
    const int m = m0 + wm * 32 * kMB + mb * 32 + c32;
#pragma unroll
    for (int g = 0; g < kOut; ++g)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + g * FBN + wn * 64 + nb * 32 + 8 * q + 4 * h32;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = acc[g][mb][nb][4 * q + e];
            if constexpr (kSwiGLU) {
              // silu(g) * u with silu(g) = g / (1 + 2^(-g log2 e)); the exponent's overflow to +inf
              // gives -0 for large negative g, the right limit
              v[e] = v[e] * __builtin_amdgcn_rcpf(1.f + fast_exp2(-v[e] * kLog2e)) * acc[1][mb][nb][4 * q + e];
            }
          }
          if (m < M && n < N)  // N is a multiple of 32, so the 4 columns are all in range
            *reinterpret_cast<u32x2*>(out + (int64_t)m * ldo + n) =
                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
  }
}

// tile height (64 kMB rows), LDS stages and workgroups per CU of both products
constexpr int kGateMB = 4, kGateStages = 4, kGateOcc = 1;
constexpr int kDownMB = 4, kDownStages = 4, kDownOcc = 1;

}  // namespace

hipError_t launch_ffn(const FfnParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  for (int64_t r0 = 0; r0 < p.rows; r0 += p.chunk) {
    const int m = (int)(p.rows - r0 < p.chunk ? p.rows - r0 : p.chunk);
    const uint16_t* x = p.x + r0 * p.ldx;
    uint16_t* y = p.y + r0 * p.ldy;
    // h = silu(x W_gate^T) * (x W_up^T): [m, d_ff] in the workspace (leading dimension d_ff)
    {
      constexpr int FBM = 64 * kGateMB;
      const int n_m = (m + FBM - 1) / FBM, n_n = (p.d_ff + FBN - 1) / FBN;
      LWM_LAUNCH("ffn_gate_up", (ffn_gemm_kernel<true, kGateMB, kGateStages, kGateOcc>), dim3(n_m * n_n), dim3(kFfnWaves * kWave), stream, x, p.ldx,
                 p.w_gate, p.w_up, p.ldw, p.h, (int64_t)p.d_ff, m, p.d_ff, p.d_model);
    }
    // y = h W_down^T: [m, d_model]
    {
      constexpr int FBM = 64 * kDownMB;
      const int n_m = (m + FBM - 1) / FBM, n_n = (p.d_model + 2 * FBN - 1) / (2 * FBN);
      LWM_LAUNCH("ffn_down", (ffn_gemm_kernel<false, kDownMB, kDownStages, kDownOcc>), dim3(n_m * n_n), dim3(kFfnWaves * kWave), stream,
                 (const uint16_t*)p.h, (int64_t)p.d_ff, p.w_down, p.w_down, p.ldwd, y, p.ldy, m, p.d_model, p.d_ff);
    }
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lwm
