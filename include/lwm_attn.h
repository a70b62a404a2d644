/*
 * lwm_attn.h - C ABI of the MI355X (gfx950) blockwise causal ring-attention library.
 *
 * What the library computes, and where the pages state it:
 *
 *  - RoPE with theta scaled to the context length: "[论文解读] World Model on Million-Length
 *    Video And Language With Blockwise RingAttention", section 提出的方法 (theta is a per-model
 *    setting; "LWM：突破 100 万 Token 的开源大模型", section 脚本运行说明, shows theta=50000000).
 *  - Self-attention computed blockwise over query and key chunks: "LWM：突破 100 万 Token 的
 *    开源大模型", section 配置参数 (scan_query_chunk_size / scan_key_chunk_size).
 *  - Autoregressive (causal) attention: "Inside Large World Model: UC Berkeley Multimodal
 *    Model that can Understand 1 Hour Long Videos", section "Core Architecture".
 *  - Masked sequence packing (segments of one packed row attend only within themselves):
 *    "LWM：突破 100 万 Token 的开源大模型", section 概述, item (b).
 *  - RingAttention: KV blocks travel around a ring of devices while each keeps its query
 *    block, compute overlapping transfer: "开源巨兽LWM：如何用RingAttention撬动百万Token多模态
 *    世界", section 3.1; sequence-parallel mesh axis: "LWM：突破 100 万 Token 的开源大模型",
 *    section 配置参数.  One ring step folds one KV shard into a running (O, logsumexp) state.
 *
 * The pages give no formula.  The library computes, per batch b and head h, for query i
 * (global index q_offset + i) and key j (global index k_offset + j):
 *     visible(i, j) = (!causal || k_offset + j <= q_offset + i) && (seg_q[i] == seg_k[j])
 *     S_ij = scale * <Q'_i, K'_j>,   P = softmax over visible j,   O_i = sum_j P_ij V_j,
 *     lse_i = ln sum_{visible j} exp(S_ij)          (natural log, float32)
 * A row with no visible key gets O = 0 and lse = -inf.  Q' and K' are the RoPE-rotated
 * operands: callers apply lwm_rope_apply first.
 *
 * Conventions for every entry point:
 *  - Tensors are described by lwm_tensor4: element strides sB, sL, sH; the D (feature)
 *    stride is 1.  The data pointer is device memory (hipMalloc / torch CUDA tensors) and must
 *    be 16-byte aligned; sB, sL, sH must be multiples of 16 bytes worth of elements (8 for bf16,
 *    4 for fp32).  Segment-id and position arrays are device int32 [B, L], contiguous.
 *    lse arrays are device float32 [B, H, Lq], contiguous.
 *  - The caller owns every buffer (including the backward workspace).  The library allocates
 *    no device memory and keeps no state besides its code objects and a thread-local error
 *    string.
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is enqueued
 *    asynchronously on it; inputs must stay alive until it completes.
 *  - Arguments are validated on the host before anything is launched.  A failed check
 *    returns a negative lwm_status, launches nothing, and leaves a message readable through
 *    lwm_last_error() on the calling thread.  Faults inside kernels surface at the caller's
 *    next synchronisation of `stream`.
 *  - Segment ids must be non-decreasing along each row (contiguous packing).  The mask
 *    itself is evaluated element by element, but the key-tile range each query tile visits
 *    is found by binary search, so other id orders give unspecified (memory-safe) results.
 *  - Outputs must not overlap inputs, except that lwm_rope_apply may run in place (y == x).
 */
#ifndef LWM_ATTN_H
#define LWM_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LWM_ABI_VERSION 8

typedef enum {
  LWM_OK = 0,
  LWM_ERR_INVALID_ARG = -1, /* null pointer, shape/stride mismatch, misalignment, bad value */
  LWM_ERR_UNSUPPORTED = -2, /* valid request the kernels do not implement (e.g. D != 128)     */
  LWM_ERR_WORKSPACE = -3,   /* backward workspace missing or smaller than required           */
  LWM_ERR_HIP = -4          /* the HIP runtime refused a launch; message has its error text  */
} lwm_status;

typedef enum { LWM_BF16 = 0, LWM_FP32 = 1 } lwm_dtype;

typedef enum {
  LWM_ROPE_HALF = 0,        /* feature i pairs with i + D/2 (LLaMA / HF convention, default) */
  LWM_ROPE_INTERLEAVED = 1  /* feature 2i pairs with 2i + 1                                 */
} lwm_rope_layout;

/* A [B, L, H, D] tensor view.  Element strides; the D stride is 1. */
typedef struct lwm_tensor4 {
  void* ptr;
  int32_t dtype; /* lwm_dtype */
  int32_t reserved;
  int64_t B, L, H, D;
  int64_t sB, sL, sH;
} lwm_tensor4;

/* Version of this ABI (LWM_ABI_VERSION of the built library). */
int lwm_abi_version(void);

/* Message of the last failed call on this thread; "" after a successful call. Never NULL. */
const char* lwm_last_error(void);

/*
 * RoPE (theta scaled to context length; see the header comment for the source).
 * For every token t of batch row b the position is
 *     p = pos_offset + (pos ? pos[b*L + t] : seg ? t - first(b, t) : t)
 * where first(b, t) is the index of the first token of t's segment (positions restart at
 * each packed segment).  inv_freq_i = theta^(-2i/D); the angle p * inv_freq_i is formed and
 * reduced in double precision to r = angle - k*pi/2 (|r| <= pi/4), whose sine and cosine are summed
 * from their Taylor series in double precision and rounded once to single precision.
 * Each pair (x_a, x_b) (layout selects the pairing) becomes
 *     (x_a cos - x_b sin,  x_a sin + x_b cos)       (inverse != 0: rotate by -angle).
 * x, y: same dtype (bf16: result rounded to nearest even; fp32) and shape [B, L, H, D] with
 * D even, 16 <= D <= 256, D % 16 == 0.  y may be x (in place).  theta > 0.
 */
int lwm_rope_apply(const lwm_tensor4* x, const lwm_tensor4* y, const int32_t* pos,
                   const int32_t* seg, int64_t pos_offset, double theta, int32_t layout,
                   int32_t inverse, void* stream);

/*
 * Blockwise attention forward: O = softmax(scale * Q K^T + mask) V and lse (natural log).
 * q [B, Lq, H, 128], k and v [B, Lk, H, 128], o [B, Lq, H, 128]: all bf16, or all fp32.
 * seg_q [B, Lq] and seg_k [B, Lk] are both NULL (one segment) or both given.
 * q_offset / k_offset: global index of the first query / key (>= 0).  causal: 0 or 1.
 * scale: > 0, or 0 for 1/sqrt(D).  lse: float32 [B, H, Lq] (NULL to skip).
 * bf16 path: P is rounded to bf16 before P*V, every sum is accumulated in float32, and O is
 * rounded to bf16 at the end.  fp32 path: float32 throughout.
 */
int lwm_blockattn_fwd(const lwm_tensor4* q, const lwm_tensor4* k, const lwm_tensor4* v,
                      const int32_t* seg_q, const int32_t* seg_k, int64_t q_offset,
                      int64_t k_offset, int32_t causal, float scale, const lwm_tensor4* o,
                      float* lse, void* stream);

/*
 * Bytes of workspace lwm_blockattn_bwd (and lwm_ring_step_bwd) needs for these sizes: two float32
 * rows per query (D_i and lse_i * log2(e)), each array rounded up to 256 bytes; at least 256.
 * Depends on B, H and Lq only; Lk and D are accepted for symmetry with the call.
 */
size_t lwm_blockattn_bwd_workspace_size(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D);

/*
 * Bytes of workspace with room for the stored-dS backward over heads_per_pass (batch, head)
 * pairs at a time, for a call with these sizes, offsets and causal flag:
 * lwm_blockattn_bwd_workspace_size() plus heads_per_pass slots.  A slot holds one pair's dS^T
 * (bf16) in 64 x 64 blocks: Lk rounded up to 64 key rows by ldq = Lq rounded up to 256 queries,
 * less, under the causal mask, the blocks of query blocks before a key block's first visible
 * query (q_offset + q >= k_offset + k): key block kb keeps query blocks from
 * clamp(kb + floor((k_offset - q_offset) / 64), 0, ldq / 64) on (about half of a square slot).
 * heads_per_pass is clamped to B * H; the minimum size comes back for heads_per_pass <= 0, empty
 * sizes, offsets outside [0, 2^40], Lq above 2^21 or nothing to store (no stored-dS path),
 * SIZE_MAX if the size does not fit in a size_t.  How a larger workspace is used is described at
 * lwm_blockattn_bwd.
 */
size_t lwm_blockattn_bwd_workspace_size_ds(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                                           int64_t q_offset, int64_t k_offset, int32_t causal,
                                           int64_t heads_per_pass);

/*
 * Blockwise attention backward (bf16 only).  The pages train the model with RingAttention at
 * up to a million tokens ("LWM：突破 100 万 Token 的开源大模型", section 概述; the context is grown
 * step by step during training, "[论文解读] World Model on Million-Length Video And Language With
 * Blockwise RingAttention", section 提出的方法), so the attention's gradients are part of the
 * method; they are not written out there.  This is the gradient of the loss sum(dout * O) of
 * the forward defined above (the textbook backward of softmax attention):
 *     D_i = sum_d dout_id O_id,  P = exp(S - lse),  dV = P^T dout,  dP = dout V^T,
 *     dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
 * q, k, v, seg_*, offsets, causal, scale as in lwm_blockattn_fwd; o and lse are that call's
 * outputs; dout like o.  dq [B, Lq, H, 128], dk and dv [B, Lk, H, 128] (bf16) are written
 * (not accumulated) and are gradients w.r.t. the operands given (the rotated Q', K'); apply
 * lwm_rope_apply(inverse=1) to dq and dk for gradients w.r.t. the pre-RoPE Q and K.
 * workspace: device memory of at least lwm_blockattn_bwd_workspace_size() bytes, 256-byte
 * aligned; its contents on entry do not matter.  When it also holds G >= min(B * H, 8) slots
 * (lwm_blockattn_bwd_workspace_size_ds), the backward stores dS instead of recomputing it: in
 * passes over G (batch, head) pairs (a multiple of 8 unless G = B * H), the dK/dV kernel also
 * writes each pair's dS^T (bf16, as the products use it) into the slots, and dQ = scale dS K
 * is formed from them, which replaces the recomputation of S and dP for dQ (5 products instead
 * of 7, plus two bytes of dS per visible pair written and read).  Both paths give the same
 * results; with less room the recomputing path runs.  Status: LWM_ERR_INVALID_ARG for NULL or
 * misaligned pointers and mismatched shapes, LWM_ERR_UNSUPPORTED for fp32 operands, D != 128 or
 * launch grids beyond 2^31 - 1 workgroups, LWM_ERR_WORKSPACE for a short or misaligned
 * workspace, LWM_ERR_HIP if a launch fails.
 */
int lwm_blockattn_bwd(const lwm_tensor4* q, const lwm_tensor4* k, const lwm_tensor4* v,
                      const lwm_tensor4* o, const float* lse, const lwm_tensor4* dout,
                      const int32_t* seg_q, const int32_t* seg_k, int64_t q_offset,
                      int64_t k_offset, int32_t causal, float scale, const lwm_tensor4* dq,
                      const lwm_tensor4* dk, const lwm_tensor4* dv, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * lwm_blockattn_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation and
 * kernels, with the workspace taken from a static device array the library holds on each GPU
 * until the process ends (16 MiB: B * H * Lq <= 2^21 query rows).  No workspace argument; every
 * other argument, result and status as for lwm_blockattn_bwd, plus LWM_ERR_UNSUPPORTED when
 * B * H * Lq exceeds 2^21.  Allocates nothing (its first call on a device looks up that device's
 * array address).  The array is shared by every call on one GPU and is fully rewritten before
 * it is read, so nothing must be cleared between calls; calls that may run concurrently on one
 * GPU (different streams or threads without ordering) race on it and must be serialised by the
 * caller.
 */
int lwm_blockattn_bwd_noalloc(const lwm_tensor4* q, const lwm_tensor4* k, const lwm_tensor4* v,
                              const lwm_tensor4* o, const float* lse, const lwm_tensor4* dout,
                              const int32_t* seg_q, const int32_t* seg_k, int64_t q_offset,
                              int64_t k_offset, int32_t causal, float scale, const lwm_tensor4* dq,
                              const lwm_tensor4* dk, const lwm_tensor4* dv, void* stream);

/*
 * One ring step (bf16): fold KV shard (k_shard, v_shard) into the running state of the
 * query block.  The state is the normalised partial output o_acc (float32 [B, Lq, H, 128],
 * described by a lwm_tensor4 of dtype LWM_FP32) and lse_acc (float32 [B, H, Lq]); before the
 * first step the caller sets o_acc = 0 and lse_acc = -inf.  After the step they hold exactly
 * (up to rounding) the attention of each query over all keys folded in so far:
 *     lse' = ln(e^lse + e^lse_shard),  o' = e^(lse - lse') o + e^(lse_shard - lse') o_shard.
 * Rows that see no key of this shard keep their state bit for bit.  k_offset is the global
 * index of the shard's first key; seg_*, causal, scale as in lwm_blockattn_fwd.  o_final:
 * NULL, or a bf16 [B, Lq, H, 128] view that receives the merged state rounded to bf16 (pass
 * it on the last step).  Shards that are entirely in the causal future may be skipped by the
 * caller; passing them is a valid no-op for the state.
 */
int lwm_ring_step(const lwm_tensor4* q, const lwm_tensor4* k_shard, const lwm_tensor4* v_shard,
                  const int32_t* seg_q, const int32_t* seg_k, int64_t q_offset, int64_t k_offset,
                  int32_t causal, float scale, const lwm_tensor4* o_acc, float* lse_acc,
                  const lwm_tensor4* o_final, void* stream);

/*
 * Backward ring step (bf16): add one KV shard's share of the gradients.  On the pages the
 * sequence is cut into blocks held by devices in a ring, each device computing on one block
 * while the next one arrives ("开源巨兽LWM：如何用RingAttention撬动百万Token多模态世界", section
 * 3.1); in the backward pass the query block (with its dout, O and lse) stays and each visiting
 * KV shard picks up this block's contribution to its dK, dV on the way:
 *     P = exp(scale Q K_shard^T - lse) on the shard's visible keys,  D_i = sum_d dout_id O_id,
 *     dq_acc += scale dS K_shard,  dk_acc += scale dS^T Q,  dv_acc += P^T dout,
 * with dS = P o (dout V_shard^T - D).  o and lse must be the forward's results over *all*
 * shards (e.g. lwm_ring_step's final state), so summing the steps over every shard gives
 * exactly lwm_blockattn_bwd's gradients.  q, dout, o: bf16 [B, Lq, H, 128]; k_shard, v_shard:
 * bf16 [B, Lk, H, 128]; k_offset is the global index of the shard's first key; seg_*, causal,
 * scale as in lwm_blockattn_fwd.  dq_acc (like q) and dk_acc, dv_acc (like k_shard) are
 * float32 lwm_tensor4 views that are read and added to (the caller zeroes them before the first
 * step); results are w.r.t. the rotated operands, as for lwm_blockattn_bwd.  workspace: at
 * least lwm_blockattn_bwd_workspace_size(B, H, Lq, Lk, D) bytes, 256-byte aligned (room for
 * stored dS, sized by lwm_blockattn_bwd_workspace_size_ds with the shard's Lk, is used as in
 * lwm_blockattn_bwd); the call writes D and the rescaled lse of the query block into it, ahead
 * of any dS slots.  Both depend on the query block only,
 * so the steps of one ring after the first may pass flags = LWM_RING_BWD_REUSE_WORKSPACE to use
 * what the first step wrote instead of recomputing it (same workspace, and the same q, o, lse,
 * dout and shape as that step; the library cannot check this).  flags: 0 or
 * LWM_RING_BWD_REUSE_WORKSPACE.  Errors as for lwm_blockattn_bwd, LWM_ERR_INVALID_ARG for other
 * flags; a shard wholly in the causal future adds zero.
 */
#define LWM_RING_BWD_REUSE_WORKSPACE 1
int lwm_ring_step_bwd(const lwm_tensor4* q, const lwm_tensor4* k_shard, const lwm_tensor4* v_shard,
                      const lwm_tensor4* o, const float* lse, const lwm_tensor4* dout,
                      const int32_t* seg_q, const int32_t* seg_k, int64_t q_offset,
                      int64_t k_offset, int32_t causal, float scale, const lwm_tensor4* dq_acc,
                      const lwm_tensor4* dk_acc, const lwm_tensor4* dv_acc, void* workspace,
                      size_t workspace_bytes, int32_t flags, void* stream);

/*
 * RoPE inside the attention kernels (the two entry points below).  RoPE with theta scaled to
 * the context length is the same operation as lwm_rope_apply ("[论文解读] World Model on
 * Million-Length Video And Language With Blockwise RingAttention", section 提出的方法); the
 * position of query row t is q_pos_offset + t and of key row t is k_pos_offset + t, or, when
 * restart is 1, that offset plus t minus the first index of t's segment in seg_q (seg_k):
 * positions restart at each packed segment ("LWM：突破 100 万 Token 的开源大模型", section 概述,
 * item (b)).  restart = 1 needs segment ids.  theta > 0 and finite; |offsets| <= 2^40.
 */
typedef struct lwm_rope_args {
  double theta;
  int32_t layout;  /* lwm_rope_layout */
  int32_t restart; /* 0 or 1 */
  int64_t q_pos_offset;
  int64_t k_pos_offset;
} lwm_rope_args;

/*
 * Forward with RoPE applied inside the call (bf16 only): q and k are the pre-RoPE operands.
 * Computes exactly what lwm_rope_apply on q (offset q_pos_offset, seg = restart ? seg_q : NULL),
 * lwm_rope_apply on k (likewise), then lwm_blockattn_fwd on the rotated pair compute, bit for bit.
 * The queries are rotated by each workgroup as it loads them into registers; the keys, which
 * every query tile streams again, are rotated once by a pass into k_rot.
 * k_rot: required bf16 output like k (the rotated keys; it may be k itself, with equal strides,
 * for an in-place rotation).  q_rot: NULL or a bf16 output like q that receives the rotated
 * queries (what lwm_blockattn_bwd_rope takes).  Other arguments and errors as for
 * lwm_blockattn_fwd; rope may not be NULL.  Outputs overlap no input (except k_rot == k).
 */
int lwm_blockattn_fwd_rope(const lwm_tensor4* q, const lwm_tensor4* k, const lwm_tensor4* v,
                           const int32_t* seg_q, const int32_t* seg_k, int64_t q_offset,
                           int64_t k_offset, int32_t causal, float scale, const lwm_rope_args* rope,
                           const lwm_tensor4* o, float* lse, const lwm_tensor4* q_rot,
                           const lwm_tensor4* k_rot, void* stream);

/*
 * Backward with the inverse RoPE applied inside the call (bf16 only): q_rot and k_rot are the
 * rotated operands the forward used (lwm_blockattn_fwd_rope's q_rot and k_rot); dq and dk are
 * the gradients w.r.t. the pre-RoPE Q and K.  The result is lwm_blockattn_bwd's followed by
 * lwm_rope_apply(inverse = 1) on dq and dk, except that dQ' and dK' are rotated back in float32
 * inside the kernels and rounded to bf16 once (the separate route rounds twice).  dv is
 * lwm_blockattn_bwd's bit for bit.  Arguments, workspace and errors as for lwm_blockattn_bwd;
 * rope (as given to the forward) may not be NULL.
 */
int lwm_blockattn_bwd_rope(const lwm_tensor4* q_rot, const lwm_tensor4* k_rot, const lwm_tensor4* v,
                           const lwm_tensor4* o, const float* lse, const lwm_tensor4* dout,
                           const int32_t* seg_q, const int32_t* seg_k, int64_t q_offset,
                           int64_t k_offset, int32_t causal, float scale, const lwm_rope_args* rope,
                           const lwm_tensor4* dq, const lwm_tensor4* dk, const lwm_tensor4* dv,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Blockwise feed-forward block: the transformer half that follows each attention, computed in
 * chunks of rows along the sequence ("LWM：突破 100 万 Token 的开源大模型", section 配置参数,
 * scan_mlp and scan_mlp_chunk_size; section 脚本运行说明 uses chunks of 8192).  The block is the
 * LLaMA one the PyTorch port of the models loads (same page, section 运行 PyTorch 模型):
 *     h = silu(x W_gate^T) * (x W_up^T),   y = h W_down^T,   silu(z) = z / (1 + e^-z),
 * no biases.  Chunks are independent, so the result does not depend on `chunk` beyond rounding.
 *
 * All operands are bf16, row-major device matrices with leading dimensions in elements:
 *   x       [rows, d_model]   leading dimension ldx  >= d_model
 *   w_gate  [d_ff, d_model]   leading dimension ldw  >= d_model (nn.Linear layout [out, in])
 *   w_up    [d_ff, d_model]   leading dimension ldw
 *   w_down  [d_model, d_ff]   leading dimension ldwd >= d_ff
 *   y       [rows, d_model]   leading dimension ldy  >= d_model (output; overlaps no input)
 * Accumulation is float32; h is rounded to bf16 (it is the chunk's stored activation) and y is
 * rounded to bf16 once.  d_model and d_ff must be multiples of 32; leading dimensions multiples
 * of 8 and below 2^22; pointers 16-byte aligned.  `workspace` (caller-owned device memory, 256-
 * byte aligned, at least lwm_blockwise_ffn_workspace_size bytes) holds one chunk's h.  rows = 0
 * is a no-op.  Status: LWM_ERR_INVALID_ARG for NULL or misaligned pointers and bad sizes,
 * LWM_ERR_UNSUPPORTED for sizes outside the ranges above, LWM_ERR_WORKSPACE for a short or
 * misaligned workspace, LWM_ERR_HIP if a launch fails.
 */
size_t lwm_blockwise_ffn_workspace_size(int64_t rows, int64_t d_ff, int64_t chunk);
int lwm_blockwise_ffn(const void* x, int64_t rows, int64_t d_model, int64_t ldx, const void* w_gate,
                      const void* w_up, int64_t ldw, const void* w_down, int64_t ldwd, int64_t d_ff,
                      void* y, int64_t ldy, int64_t chunk, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Kernel timing (instrumentation, not part of the method).  While enabled, every kernel the
 * library launches is bracketed by two HIP events recorded on its launch stream, so durations
 * are those of the kernels themselves.  lwm_profile_count / lwm_profile_get wait for the
 * recorded events, then report per kernel name the summed milliseconds and launch count since
 * the last lwm_profile_reset.  Names returned stay valid until the next reset.  Host-side state
 * only (HIP events, no device memory); thread-safe.  Returns LWM_OK, LWM_ERR_INVALID_ARG for a
 * bad index or NULL output, LWM_ERR_HIP if an event could not be resolved.
 */
int lwm_profile_enable(int32_t on);
int lwm_profile_reset(void);
int lwm_profile_count(void);
int lwm_profile_get(int32_t index, const char** name, double* total_ms, int64_t* launches);

/*
 * Matrix-core rate probe (instrumentation, not part of the method).  Launches `blocks`
 * workgroups of four waves (64 lanes each) on `stream`.  Every wave runs `iters` rounds of four
 * independent v_mfma_f32_32x32x16_bf16 (a 32x16 by 16x32 bf16 product added into a 32x32
 * float32 accumulator, 32768 flop), with A and B operands rotating over eight fragments each
 * that every lane reads once, before the loop, from `src`; the loop itself does nothing else.
 * A launch therefore performs blocks * 4 * iters * 4 * 32768 flop, and its duration on the
 * stream gives the rate the matrix cores sustain for those operand values (the clock the chip
 * holds depends on them).  Each workgroup reserves 96 KB of LDS, so a CU runs one at a time and
 * each of its waves has a SIMD's matrix core to itself; on a 256-CU part 256 blocks fill the
 * chip once, 512 twice.
 *   src:  device bf16, blocks * 256 * 128 values (lane t of the grid reads values
 *         128 t .. 128 t + 127: eight A fragments of 8, then eight B fragments of 8),
 *         16-byte aligned, owned by the caller.
 *   sink: device float32, blocks * 256 values, written with each lane's sum of its final
 *         accumulators (so the products cannot be optimised away).
 *   iters: a positive multiple of 8, at most 2^24 (with blocks <= 4096, a launch stays within
 *          about 20 s on a 256-CU part).
 * Returns LWM_OK, LWM_ERR_INVALID_ARG for a NULL or misaligned pointer, blocks outside
 * [1, 4096] or a bad iters, LWM_ERR_HIP if the launch fails.
 */
int lwm_probe_mfma_bf16(const void* src, void* sink, int32_t blocks, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LWM_ATTN_H */
