// Matrix-core rate probe (instrumentation, not part of the attention method).
//
// The attention kernels are priced against the bf16 MFMA peak the part is rated for (256 CUs x
// 4096 flop per clock x 2.4 GHz).  How close a kernel can come also depends on what the matrix
// cores sustain at the clock the chip holds under that load, and that clock depends on the
// operand values: the power a multiply array draws grows with how many of its input bits toggle.
// This kernel measures it directly: each wave issues nothing but v_mfma_f32_32x32x16_bf16 on four
// independent accumulator chains, with A and B operands rotating over eight register-resident
// fragments each (read once from memory before the loop), so no memory access, LDS access or
// vector-ALU work competes with the MFMAs inside the timed loop.  Timing one launch gives the
// sustained rate for the operand values the caller supplies (random N(0,1) bf16 like the
// attention's Q, K, V and dO, or a constant for contrast).
#include <hip/hip_runtime.h>

#include "profile.hpp"

namespace lwm {
namespace {

typedef __bf16 pbf16x8 __attribute__((ext_vector_type(8)));
typedef float pf32x16 __attribute__((ext_vector_type(16)));

constexpr int kFrags = 8;  // A and B fragments per lane

// LDS reserved per workgroup: 96 KB, so a CU (160 KB of LDS) runs one workgroup at a time and
// each of its four waves has a SIMD's matrix core to itself.  Two waves issuing identical MFMA
// streams on one SIMD settle, depending on how they happen to start, either into one wave
// streaming while the other waits or into the two alternating, and measured on the part the
// alternating pattern sustains 20-30% less; one wave per SIMD has no such choice.
constexpr int kPadFloats = 96 * 1024 / 4;

__global__ __launch_bounds__(256) void mfma_probe_kernel(const pbf16x8* __restrict__ src, float* __restrict__ sink,
                                                         int iters) {
  __shared__ float pad[kPadFloats];
  const int gt = blockIdx.x * blockDim.x + threadIdx.x;
  pbf16x8 a[kFrags], b[kFrags];
#pragma unroll
  for (int r = 0; r < kFrags; ++r) {
    a[r] = src[(size_t)gt * (2 * kFrags) + r];
    b[r] = src[(size_t)gt * (2 * kFrags) + kFrags + r];
  }
  // accumulators start from operand values, so that they hold data-like bits from the first MFMA
  pf32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = (float)a[(c + i) % kFrags][i % 8];
  for (int it = 0; it < iters; it += kFrags) {
#pragma unroll
    for (int k = 0; k < kFrags; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + c) % kFrags], b[(3 * c + k) % kFrags], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  // the lane's sum goes out through the reserved LDS, which keeps the reservation in the kernel
  pad[threadIdx.x * 64] = s;
  __syncthreads();
  sink[gt] = pad[threadIdx.x * 64];
}

}  // namespace

hipError_t launch_mfma_probe(const void* src, float* sink, int blocks, int iters, hipStream_t stream) {
  LWM_LAUNCH("mfma_probe", mfma_probe_kernel, dim3(blocks), dim3(256), stream, static_cast<const pbf16x8*>(src), sink,
             iters);
  return hipGetLastError();
}

}  // namespace lwm
