// Kernel parameter blocks and launchers (internal to the library; the public surface is the
// C ABI in include/lwm_attn.h).  Strides are in elements; the feature stride is 1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lwm {

constexpr int kMaxRopeHalf = 128;
constexpr int kHeadDim = 128;  // the attention kernels are written for D = 128

struct RopeParams {
  const void* x;
  void* y;
  const int32_t* pos;
  const int32_t* seg;
  int64_t pos_offset;
  int B, L, H, D;
  int64_t xsB, xsL, xsH;
  int64_t ysB, ysL, ysH;
  int layout;   // 0: (i, i + D/2), 1: (2i, 2i + 1)
  int inverse;  // rotate by -angle
  double inv_freq[kMaxRopeHalf];
};

struct Strides {
  int64_t b, l, h;
};

// RoPE applied inside the attention kernels.  Row t of the query (key) operand has position
// q_pos_offset + t (k_pos_offset + t), or that offset plus t minus the first index of t's segment
// when `restart` is set; inv_freq[i] = theta^(-2i/D).
struct RopeFuse {
  int on;       // 0: the operands are already rotated, nothing is fused
  int layout;   // 0: (i, i + D/2), 1: (2i, 2i + 1)
  int restart;  // positions restart at each segment (segment ids given)
  int64_t q_pos_offset, k_pos_offset;
  double inv_freq[kHeadDim / 2];
};

// Forward / ring-step attention.  mode 0: fresh state, writes o (+ lse).  mode 1: ring step,
// state read from and written back to o_acc / lse_acc, o optional (bf16 copy of the result).
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  Strides sq, sk, sv;
  int B, H, Lq, Lk;
  const int32_t* seg_q;
  const int32_t* seg_k;
  int64_t q_offset, k_offset;
  int causal;
  float scale_log2;  // scale * log2(e)
  void* o;
  Strides so;
  float* lse;
  float* o_acc;
  Strides soa;
  float* lse_acc;
  int mode;
  // rope.on: q holds the pre-RoPE queries; each workgroup rotates its rows as it loads them and,
  // when q_rot is set, stores the rotated rows there (bf16 path, fresh state only)
  RopeFuse rope;
  void* q_rot;
  Strides sqr;
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  Strides sq, sk, sv, so, sdo;
  const float* lse;
  float* delta;  // workspace [B, H, Lq]: rowsum(dout * o)
  float* lse2;   // workspace [B, H, Lq]: lse * log2(e), +inf where lse = -inf
  int B, H, Lq, Lk;
  const int32_t* seg_q;
  const int32_t* seg_k;
  int64_t q_offset, k_offset;
  int causal;
  float scale;
  float scale_log2;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  Strides sdq, sdk, sdv;
  // backward ring step: when set, the gradients are added into these float32 tensors instead
  // of being stored to dq / dk / dv
  float* dq_acc;
  float* dk_acc;
  float* dv_acc;
  Strides sdqa, sdka, sdva;
  // set when delta and lse2 already hold this query block's values (a later step of one ring)
  int delta_ready;
  // rope.on: dq and dk are rotated back (inverse RoPE) before they are stored, so they are
  // gradients w.r.t. the pre-RoPE Q and K (stored outputs only, not the ring accumulators)
  RopeFuse rope;
  // Stored dS (ds != nullptr): the (batch, head) pairs go through in passes of ds_heads; in each
  // pass the dK/dV kernel also writes dS^T (bf16) of pair bh0 + j into slot j (64 x 64 blocks: up
  // to Lk rounded up to 64 rows of ds_ld = Lq rounded up to 256 values), and a dQ kernel then
  // forms dQ from it and K alone instead of recomputing S and dP.
  uint16_t* ds;
  int64_t ds_ld;
  int ds_heads;
  // causal compaction of the slots: key block kb stores query blocks from
  // qlo(kb) = clamp(kb + ds_shift, 0, ds_ld / 64) on (ds_shift = floor((k_offset - q_offset) / 64),
  // or -2^40 without the causal mask, which stores every block); ds_slot_blocks blocks per slot
  int64_t ds_shift;
  int64_t ds_slot_blocks;
  // the (batch, head) pairs one launch covers: bh0 .. bh0 + bh_count - 1 (set by launch_attn_bwd)
  int bh0, bh_count;
};

// Blockwise feed-forward block (bf16): y = (silu(x W_gate^T) * (x W_up^T)) W_down^T over chunks
// of `chunk` rows; h is the [chunk, d_ff] workspace (leading dimension d_ff).  Leading
// dimensions are in elements.
struct FfnParams {
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* w_gate;
  const uint16_t* w_up;
  int64_t ldw;
  const uint16_t* w_down;
  int64_t ldwd;
  uint16_t* y;
  int64_t ldy;
  uint16_t* h;
  int64_t rows, chunk;
  int d_model, d_ff;
};

hipError_t launch_rope(const RopeParams& p, bool bf16, hipStream_t stream);
hipError_t launch_attn_fwd(const FwdParams& p, bool bf16, hipStream_t stream);
hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t stream);
hipError_t launch_ffn(const FfnParams& p, hipStream_t stream);

}  // namespace lwm
