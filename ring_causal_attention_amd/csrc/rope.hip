// RoPE with theta scaled to the context length ("[论文解读] World Model on Million-Length Video
// And Language With Blockwise RingAttention", section 提出的方法), applied to a [B, L, H, D]
// tensor in place or out of place, forward or inverse.
//
// HBM-bound: every element is read and written once.  A workgroup owns kTok consecutive tokens
// of one batch row.  It finds the kTok positions once (restarting ones by a single segment search
// per workgroup), forms the kTok x D/2 angles once (double precision: position times inv_freq,
// reduced modulo pi/2) and their sine/cosine (rounded to single precision) in LDS, then streams
// all H heads of those tokens with 16-byte vector loads and stores, so the trigonometry is shared
// by every head instead of being repeated per element.
#include "kernels.hpp"
#include "profile.hpp"
#include "rope_dev.hpp"

namespace lwm {
namespace {

constexpr int kTok = 4;
constexpr int kThreads = 256;

template <typename T>
struct Vec;
template <>
struct Vec<uint16_t> {  // bf16: 8 elements per 16 bytes
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float (&x)[N]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_lo(w[j]);
      x[2 * j + 1] = bf16_hi(w[j]);
    }
  }
  __device__ static void store(uint16_t* p, const float (&x)[N]) {
    u32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
    *reinterpret_cast<u32x4*>(p) = w;
  }
};
template <>
struct Vec<float> {  // fp32: 4 elements per 16 bytes
  static constexpr int N = 4;
  __device__ static void load(const float* p, float (&x)[N]) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = w[j];
  }
  __device__ static void store(float* p, const float (&x)[N]) {
    f32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = x[j];
    *reinterpret_cast<f32x4*>(p) = w;
  }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void rope_kernel(RopeParams p) {
  // (cos, sin) per token and pair.  Pair i is kept at slot (i % P) * (half / P) + i / P, where P is
  // the number of pairs one 16-byte chunk rotates: the lanes of a wave handle consecutive chunks
  // c and read pair c * P + j together, which then sit in consecutive slots (no LDS bank aliasing).
  __shared__ float2 cs[kTok][kMaxRopeHalf];
  constexpr int N = Vec<T>::N;
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * kTok;
  const int half = p.D / 2;
  const int ntok = min(kTok, p.L - t0);
  const int P = p.layout == 0 ? N : N / 2;  // pairs per chunk: (i, i + D/2) or (2i, 2i + 1)
  const int nck = half / P;                 // chunks

  // ---- phase 0: the kTok tokens' positions, once per workgroup.  With restarting positions the
  // first token's segment start comes from one wave-wide search; a later token's segment starts
  // at the last id change at or before it, else at the first token's start.
  __shared__ int64_t tpos[kTok];
  if (threadIdx.x < kWave) {
    int first0 = 0;
    const int32_t* srow = p.seg ? p.seg + (int64_t)b * p.L : nullptr;
    if (!p.pos && srow) first0 = wave_lower_bound(srow, t0 + 1, srow[t0]);
    const int tt = threadIdx.x;
    if (tt < ntok) {
      const int t = t0 + tt;
      int64_t pos = t;
      if (p.pos) {
        pos = p.pos[(int64_t)b * p.L + t];
      } else if (srow) {
        int start = first0;
        for (int u = 1; u <= tt; ++u)
          if (srow[t0 + u] != srow[t0 + u - 1]) start = t0 + u;
        pos = t - start;
      }
      tpos[tt] = pos + p.pos_offset;
    }
  }
  __syncthreads();

  // ---- phase 1: angles (double), sin/cos (float) for kTok tokens x D/2 pairs; consecutive lanes
  // fill consecutive slots
  for (int e = threadIdx.x; e < ntok * half; e += kThreads) {
    const int tt = e / half, slot = e - tt * half;
    const int i = (slot % nck) * P + slot / nck;  // the pair kept at this slot
    float s, c;
    rope_cos_sin(tpos[tt], p.inv_freq[i], c, s);
    cs[tt][slot] = make_float2(c, p.inverse ? -s : s);
  }
  __syncthreads();

  // ---- phase 2: rotate every head of the kTok tokens, 16 bytes at a time
  const T* __restrict__ x = static_cast<const T*>(p.x);
  T* __restrict__ y = static_cast<T*>(p.y);
  if (p.layout == 0) {
    // pairs (i, i + D/2): chunk c of the first half with chunk c of the second half
    const int nchunk = half / N;
    const int items = ntok * p.H * nchunk;
    for (int e = threadIdx.x; e < items; e += kThreads) {
      const int c = e % nchunk;
      const int rest = e / nchunk;
      const int h = rest % p.H, tt = rest / p.H;
      const int64_t t = t0 + tt;
      const T* xs = x + b * p.xsB + t * p.xsL + h * p.xsH + c * N;
      T* ys = y + b * p.ysB + t * p.ysL + h * p.ysH + c * N;
      float a[N], bb[N];
      Vec<T>::load(xs, a);
      Vec<T>::load(xs + half, bb);
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const float2 r = cs[tt][j * nck + c];
        rope_rotate(a[j], bb[j], r.x, r.y, a[j], bb[j]);
      }
      Vec<T>::store(ys, a);
      Vec<T>::store(ys + half, bb);
    }
  } else {
    // pairs (2i, 2i + 1): each 16-byte chunk holds N/2 whole pairs
    const int nchunk = p.D / N;
    const int items = ntok * p.H * nchunk;
    for (int e = threadIdx.x; e < items; e += kThreads) {
      const int c = e % nchunk;
      const int rest = e / nchunk;
      const int h = rest % p.H, tt = rest / p.H;
      const int64_t t = t0 + tt;
      const T* xs = x + b * p.xsB + t * p.xsL + h * p.xsH + c * N;
      T* ys = y + b * p.ysB + t * p.ysL + h * p.ysH + c * N;
      float a[N];
      Vec<T>::load(xs, a);
#pragma unroll
      for (int j = 0; j < N / 2; ++j) {
        const float2 r = cs[tt][j * nck + c];
        rope_rotate(a[2 * j], a[2 * j + 1], r.x, r.y, a[2 * j], a[2 * j + 1]);
      }
      Vec<T>::store(ys, a);
    }
  }
}

}  // namespace

hipError_t launch_rope(const RopeParams& p, bool bf16, hipStream_t stream) {
  if (p.L == 0 || p.B == 0 || p.H == 0) return hipSuccess;
  dim3 grid((p.L + kTok - 1) / kTok, p.B);
  if (bf16) LWM_LAUNCH("rope_bf16", rope_kernel<uint16_t>, grid, dim3(kThreads), stream, p);
  else LWM_LAUNCH("rope_f32", rope_kernel<float>, grid, dim3(kThreads), stream, p);
  return hipGetLastError();
}

}  // namespace lwm
