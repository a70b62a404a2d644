// C ABI of the library: argument validation on the host, then dispatch to the gfx950 kernels.
// Every check runs before anything is launched; a failed check returns a negative status and
// leaves a message for lwm_last_error() on the calling thread.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/lwm_attn.h"
#include "kernels.hpp"

namespace lwm {
// matrix-core rate probe (probe.hip): instrumentation, kept apart from the kernels' header
hipError_t launch_mfma_probe(const void* src, float* sink, int blocks, int iters, hipStream_t stream);
}  // namespace lwm

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return LWM_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(LWM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t elem_size(int32_t dtype) { return dtype == LWM_BF16 ? 2 : 4; }

// Shape, stride and alignment rules shared by every tensor argument.
int check_tensor(const lwm_tensor4* t, const char* name) {
  if (!t) return fail(LWM_ERR_INVALID_ARG, "%s: descriptor is NULL", name);
  if (t->dtype != LWM_BF16 && t->dtype != LWM_FP32) return fail(LWM_ERR_UNSUPPORTED, "%s: unknown dtype %d", name, t->dtype);
  if (t->B < 0 || t->L < 0 || t->H < 0 || t->D < 0) return fail(LWM_ERR_INVALID_ARG, "%s: negative size", name);
  if (t->B > 65535 || t->L > (int64_t(1) << 30) || t->H > 65535)
    return fail(LWM_ERR_UNSUPPORTED, "%s: sizes beyond B<=65535, L<=2^30, H<=65535", name);
  const int64_t vec = 16 / (int64_t)elem_size(t->dtype);
  if (t->sB % vec || t->sL % vec || t->sH % vec)
    return fail(LWM_ERR_INVALID_ARG, "%s: strides must be multiples of %lld elements (16 bytes)", name, (long long)vec);
  if (t->sB < 0 || t->sL < 0 || t->sH < 0) return fail(LWM_ERR_INVALID_ARG, "%s: negative stride", name);
  if (t->sL * (int64_t)elem_size(t->dtype) >= (int64_t(1) << 24))
    return fail(LWM_ERR_UNSUPPORTED, "%s: row stride of 16 MiB or more (tiles use 32-bit offsets)", name);
  const bool empty = t->B == 0 || t->L == 0 || t->H == 0;
  if (!empty) {
    if (!t->ptr) return fail(LWM_ERR_INVALID_ARG, "%s: data pointer is NULL", name);
    if (reinterpret_cast<uintptr_t>(t->ptr) % 16) return fail(LWM_ERR_INVALID_ARG, "%s: data pointer not 16-byte aligned", name);
    if (t->sH < t->D && t->H > 1) return fail(LWM_ERR_INVALID_ARG, "%s: head stride overlaps features", name);
  }
  return LWM_OK;
}

int check_same(const lwm_tensor4* a, const lwm_tensor4* b, const char* an, const char* bn, bool same_L) {
  if (a->dtype != b->dtype) return fail(LWM_ERR_UNSUPPORTED, "%s and %s: mixed dtypes", an, bn);
  if (a->B != b->B || a->H != b->H || a->D != b->D || (same_L && a->L != b->L))
    return fail(LWM_ERR_INVALID_ARG, "%s [%lld,%lld,%lld,%lld] and %s [%lld,%lld,%lld,%lld]: shape mismatch", an,
                (long long)a->B, (long long)a->L, (long long)a->H, (long long)a->D, bn, (long long)b->B,
                (long long)b->L, (long long)b->H, (long long)b->D);
  return LWM_OK;
}

lwm::Strides strides(const lwm_tensor4* t) { return lwm::Strides{t->sB, t->sL, t->sH}; }

int check_scale(float scale, int64_t D, float* scale_out) {
  if (!std::isfinite(scale) || scale < 0.f) return fail(LWM_ERR_INVALID_ARG, "scale must be finite and >= 0 (0 = 1/sqrt(D))");
  *scale_out = scale == 0.f ? (float)(1.0 / std::sqrt((double)D)) : scale;
  return LWM_OK;
}

// Checks common to forward, backward and ring step; fills the shared part of the parameters.
int check_attention(const lwm_tensor4* q, const lwm_tensor4* k, const lwm_tensor4* v, const int32_t* seg_q,
                    const int32_t* seg_k, int64_t q_offset, int64_t k_offset, int32_t causal) {
  int s;
  if ((s = check_tensor(q, "q")) || (s = check_tensor(k, "k")) || (s = check_tensor(v, "v"))) return s;
  if ((s = check_same(q, k, "q", "k", false)) || (s = check_same(k, v, "k", "v", true))) return s;
  if (q->D != lwm::kHeadDim) return fail(LWM_ERR_UNSUPPORTED, "head dimension %lld: only 128 is implemented", (long long)q->D);
  if ((seg_q == nullptr) != (seg_k == nullptr)) return fail(LWM_ERR_INVALID_ARG, "seg_q and seg_k must both be given or both NULL");
  if (q_offset < 0 || k_offset < 0 || q_offset > (int64_t(1) << 40) || k_offset > (int64_t(1) << 40))
    return fail(LWM_ERR_INVALID_ARG, "offsets must be in [0, 2^40]");
  if (causal != 0 && causal != 1) return fail(LWM_ERR_INVALID_ARG, "causal must be 0 or 1");
  // launch grids: (query tiles or key tiles of 128 rows) x B x H workgroups, each below 2^31
  const int64_t tiles = ((q->L > k->L ? q->L : k->L) + 127) / 128 + 1;
  if (q->B * q->H > ((int64_t(1) << 31) - 1) / tiles)
    return fail(LWM_ERR_UNSUPPORTED, "grid too large: B*H*ceil(max(Lq, Lk)/128) must stay below 2^31");
  return LWM_OK;
}

// Validates the fused-RoPE arguments and fills the kernels' copy (D = 128: 64 frequencies,
// computed exactly as lwm_rope_apply computes them).
int check_rope(const lwm_rope_args* r, bool have_segs, lwm::RopeFuse* out) {
  if (!r) return fail(LWM_ERR_INVALID_ARG, "rope is NULL");
  if (!(r->theta > 0.0) || !std::isfinite(r->theta)) return fail(LWM_ERR_INVALID_ARG, "theta must be finite and > 0");
  if (r->layout != LWM_ROPE_HALF && r->layout != LWM_ROPE_INTERLEAVED)
    return fail(LWM_ERR_INVALID_ARG, "unknown RoPE layout %d", r->layout);
  if (r->restart != 0 && r->restart != 1) return fail(LWM_ERR_INVALID_ARG, "restart must be 0 or 1");
  if (r->restart && !have_segs) return fail(LWM_ERR_INVALID_ARG, "restart = 1 needs seg_q and seg_k");
  const int64_t lim = int64_t(1) << 40;
  if (r->q_pos_offset < -lim || r->q_pos_offset > lim || r->k_pos_offset < -lim || r->k_pos_offset > lim)
    return fail(LWM_ERR_INVALID_ARG, "position offsets must be in [-2^40, 2^40]");
  *out = lwm::RopeFuse{};
  out->on = 1;
  out->layout = r->layout;
  out->restart = r->restart;
  out->q_pos_offset = r->q_pos_offset;
  out->k_pos_offset = r->k_pos_offset;
  for (int i = 0; i < lwm::kHeadDim / 2; ++i) out->inv_freq[i] = std::pow(r->theta, -2.0 * i / (double)lwm::kHeadDim);
  return LWM_OK;
}

}  // namespace

extern "C" {

int lwm_abi_version(void) { return LWM_ABI_VERSION; }

const char* lwm_last_error(void) { return g_err; }

int lwm_rope_apply(const lwm_tensor4* x, const lwm_tensor4* y, const int32_t* pos, const int32_t* seg,
                   int64_t pos_offset, double theta, int32_t layout, int32_t inverse, void* stream) {
  int s;
  if ((s = check_tensor(x, "x")) || (s = check_tensor(y, "y"))) return s;
  if ((s = check_same(x, y, "x", "y", true))) return s;
  if (x->D < 16 || x->D > 2 * lwm::kMaxRopeHalf || x->D % 16)
    return fail(LWM_ERR_UNSUPPORTED, "RoPE feature size %lld: need 16 <= D <= 256, D %% 16 == 0", (long long)x->D);
  if (!(theta > 0.0) || !std::isfinite(theta)) return fail(LWM_ERR_INVALID_ARG, "theta must be finite and > 0");
  if (layout != LWM_ROPE_HALF && layout != LWM_ROPE_INTERLEAVED) return fail(LWM_ERR_INVALID_ARG, "unknown RoPE layout %d", layout);
  if (inverse != 0 && inverse != 1) return fail(LWM_ERR_INVALID_ARG, "inverse must be 0 or 1");
  if (pos_offset < -(int64_t(1) << 40) || pos_offset > (int64_t(1) << 40)) return fail(LWM_ERR_INVALID_ARG, "pos_offset out of range");
  if (x->ptr == y->ptr && (x->sB != y->sB || x->sL != y->sL || x->sH != y->sH))
    return fail(LWM_ERR_INVALID_ARG, "in-place RoPE needs identical strides");
  lwm::RopeParams p{};
  p.x = x->ptr;
  p.y = y->ptr;
  p.pos = pos;
  p.seg = pos ? nullptr : seg;
  p.pos_offset = pos_offset;
  p.B = (int)x->B;
  p.L = (int)x->L;
  p.H = (int)x->H;
  p.D = (int)x->D;
  p.xsB = x->sB; p.xsL = x->sL; p.xsH = x->sH;
  p.ysB = y->sB; p.ysL = y->sL; p.ysH = y->sH;
  p.layout = layout;
  p.inverse = inverse;
  for (int i = 0; i < p.D / 2; ++i) p.inv_freq[i] = std::pow(theta, -2.0 * i / (double)p.D);
  return hip_status(lwm::launch_rope(p, x->dtype == LWM_BF16, static_cast<hipStream_t>(stream)), "rope launch");
}

int lwm_blockattn_fwd(const lwm_tensor4* q, const lwm_tensor4* k, const lwm_tensor4* v, const int32_t* seg_q,
                      const int32_t* seg_k, int64_t q_offset, int64_t k_offset, int32_t causal, float scale,
                      const lwm_tensor4* o, float* lse, void* stream) {
  int s;
  if ((s = check_attention(q, k, v, seg_q, seg_k, q_offset, k_offset, causal))) return s;
  if ((s = check_tensor(o, "o")) || (s = check_same(q, o, "q", "o", true))) return s;
  float sc;
  if ((s = check_scale(scale, q->D, &sc))) return s;
  if (lse && reinterpret_cast<uintptr_t>(lse) % 4) return fail(LWM_ERR_INVALID_ARG, "lse not 4-byte aligned");
  lwm::FwdParams p{};
  p.q = q->ptr; p.k = k->ptr; p.v = v->ptr;
  p.sq = strides(q); p.sk = strides(k); p.sv = strides(v);
  p.B = (int)q->B; p.H = (int)q->H; p.Lq = (int)q->L; p.Lk = (int)k->L;
  p.seg_q = seg_q; p.seg_k = seg_k;
  p.q_offset = q_offset; p.k_offset = k_offset; p.causal = causal;
  p.scale_log2 = sc * 1.4426950408889634f;
  p.o = o->ptr; p.so = strides(o);
  p.lse = lse;
  p.mode = 0;
  return hip_status(lwm::launch_attn_fwd(p, q->dtype == LWM_BF16, static_cast<hipStream_t>(stream)), "forward launch");
}

int lwm_blockattn_fwd_rope(const lwm_tensor4* q, const lwm_tensor4* k, const lwm_tensor4* v, const int32_t* seg_q,
                           const int32_t* seg_k, int64_t q_offset, int64_t k_offset, int32_t causal, float scale,
                           const lwm_rope_args* rope, const lwm_tensor4* o, float* lse, const lwm_tensor4* q_rot,
                           const lwm_tensor4* k_rot, void* stream) {
  int s;
  if ((s = check_attention(q, k, v, seg_q, seg_k, q_offset, k_offset, causal))) return s;
  if (q->dtype != LWM_BF16) return fail(LWM_ERR_UNSUPPORTED, "the fused-RoPE forward is implemented for bf16 only");
  if ((s = check_tensor(o, "o")) || (s = check_same(q, o, "q", "o", true))) return s;
  if ((s = check_tensor(k_rot, "k_rot")) || (s = check_same(k, k_rot, "k", "k_rot", true))) return s;
  if (k_rot->ptr == k->ptr && (k_rot->sB != k->sB || k_rot->sL != k->sL || k_rot->sH != k->sH))
    return fail(LWM_ERR_INVALID_ARG, "k_rot == k (in place) needs identical strides");
  if (q_rot) {
    if ((s = check_tensor(q_rot, "q_rot")) || (s = check_same(q, q_rot, "q", "q_rot", true))) return s;
    if (q_rot->ptr && q_rot->ptr == q->ptr) return fail(LWM_ERR_INVALID_ARG, "q_rot must not overlap q");
  }
  float sc;
  if ((s = check_scale(scale, q->D, &sc))) return s;
  if (lse && reinterpret_cast<uintptr_t>(lse) % 4) return fail(LWM_ERR_INVALID_ARG, "lse not 4-byte aligned");
  lwm::RopeFuse rf;
  if ((s = check_rope(rope, seg_q != nullptr, &rf))) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // the keys: one RoPE pass into k_rot (what lwm_rope_apply would do)
  lwm::RopeParams rp{};
  rp.x = k->ptr;
  rp.y = k_rot->ptr;
  rp.pos = nullptr;
  rp.seg = rope->restart ? seg_k : nullptr;
  rp.pos_offset = rope->k_pos_offset;
  rp.B = (int)k->B; rp.L = (int)k->L; rp.H = (int)k->H; rp.D = (int)k->D;
  rp.xsB = k->sB; rp.xsL = k->sL; rp.xsH = k->sH;
  rp.ysB = k_rot->sB; rp.ysL = k_rot->sL; rp.ysH = k_rot->sH;
  rp.layout = rope->layout;
  rp.inverse = 0;
  for (int i = 0; i < rp.D / 2; ++i) rp.inv_freq[i] = rf.inv_freq[i];
  if ((s = hip_status(lwm::launch_rope(rp, true, st), "rope launch"))) return s;
  // the queries: rotated inside the forward kernel
  lwm::FwdParams p{};
  p.q = q->ptr; p.k = k_rot->ptr; p.v = v->ptr;
  p.sq = strides(q); p.sk = strides(k_rot); p.sv = strides(v);
  p.B = (int)q->B; p.H = (int)q->H; p.Lq = (int)q->L; p.Lk = (int)k->L;
  p.seg_q = seg_q; p.seg_k = seg_k;
  p.q_offset = q_offset; p.k_offset = k_offset; p.causal = causal;
  p.scale_log2 = sc * 1.4426950408889634f;
  p.o = o->ptr; p.so = strides(o);
  p.lse = lse;
  p.mode = 0;
  p.rope = rf;
  p.q_rot = q_rot ? q_rot->ptr : nullptr;
  if (q_rot) p.sqr = strides(q_rot);
  return hip_status(lwm::launch_attn_fwd(p, true, st), "forward launch");
}

size_t lwm_blockattn_bwd_workspace_size(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D) {
  (void)Lk;
  (void)D;
  if (B <= 0 || H <= 0 || Lq <= 0) return 256;
  const size_t rows = (size_t)B * (size_t)H * (size_t)Lq * sizeof(float);
  return 2 * ((rows + 255) / 256 * 256);  // delta, then lse * log2(e)
}

}  // extern "C"

namespace {

// Stored dS: one (batch, head) pair's dS^T in 64 x 64 blocks (8 KB), rows of Lq rounded up to 256
// values.  Under the causal mask key block kb is seen by no query block before
// qlo(kb) = clamp(kb + shift, 0, nqb), shift = floor((k_offset - q_offset) / 64), and its row starts
// there (the kernels use the same closed forms).  The kernels address a workgroup's rows with
// 32-bit offsets, so rows are at most kMaxDsLd values.
constexpr int64_t kMaxDsLd = int64_t(1) << 21;
constexpr int64_t kDsNoShift = -(int64_t(1) << 40);  // without the causal mask: every block stored
int64_t ds_row_len(int64_t Lq) { return (Lq + 255) / 256 * 256; }
int64_t ds_shift(int64_t q_offset, int64_t k_offset, int32_t causal) {
  if (!causal) return kDsNoShift;
  const int64_t d = k_offset - q_offset;
  return d >= 0 ? d / 64 : -((-d + 63) / 64);  // floor(d / 64)
}
// Blocks stored for key blocks 0 .. kb - 1 (rows of nqb blocks less the causally invisible ones).
int64_t ds_row_start(int64_t kb, int64_t nqb, int64_t c) {
  const int64_t a = std::max<int64_t>(0, -c), e = std::max(a, nqb - c);
  const int64_t m = std::min(std::max(kb, a), e);
  const int64_t lo_sum = (m - a) * c + (a + m - 1) * (m - a) / 2;
  return kb * nqb - (lo_sum + nqb * std::max<int64_t>(0, kb - e));
}
int64_t ds_slot_blocks(int64_t Lq, int64_t Lk, int64_t shift) {
  return ds_row_start((Lk + 63) / 64, ds_row_len(Lq) / 64, shift);
}

}  // namespace

extern "C" {

size_t lwm_blockattn_bwd_workspace_size_ds(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                                           int64_t q_offset, int64_t k_offset, int32_t causal,
                                           int64_t heads_per_pass) {
  const size_t base = lwm_blockattn_bwd_workspace_size(B, H, Lq, Lk, D);
  if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || heads_per_pass <= 0) return base;
  const int64_t ld = ds_row_len(Lq);
  const int64_t kOff = int64_t(1) << 40;  // the offsets the calls accept
  if (ld > kMaxDsLd || Lk > (int64_t(1) << 31) || q_offset < 0 || k_offset < 0 || q_offset > kOff || k_offset > kOff)
    return base;
  const size_t slot = (size_t)ds_slot_blocks(Lq, Lk, ds_shift(q_offset, k_offset, causal)) * 8192;
  if (slot == 0) return base;
  const size_t heads = (size_t)(heads_per_pass < B * H ? heads_per_pass : B * H);
  if (heads > (SIZE_MAX - base) / slot) return SIZE_MAX;
  return base + heads * slot;
}

}  // extern "C"

namespace {

// Checks shared by the backward and the backward ring step; fills every parameter but the
// gradient outputs.
int prepare_bwd(const lwm_tensor4* q, const lwm_tensor4* k, const lwm_tensor4* v, const lwm_tensor4* o,
                const float* lse, const lwm_tensor4* dout, const int32_t* seg_q, const int32_t* seg_k,
                int64_t q_offset, int64_t k_offset, int32_t causal, float scale, void* workspace,
                size_t workspace_bytes, lwm::BwdParams* p) {
  int s;
  if ((s = check_attention(q, k, v, seg_q, seg_k, q_offset, k_offset, causal))) return s;
  if (q->dtype != LWM_BF16) return fail(LWM_ERR_UNSUPPORTED, "backward is implemented for bf16 only");
  if ((s = check_tensor(o, "o")) || (s = check_same(q, o, "q", "o", true))) return s;
  if ((s = check_tensor(dout, "dout")) || (s = check_same(q, dout, "q", "dout", true))) return s;
  float sc;
  if ((s = check_scale(scale, q->D, &sc))) return s;
  const bool empty = q->B == 0 || q->H == 0 || (q->L == 0 && k->L == 0);
  if (!empty && !lse && q->L > 0) return fail(LWM_ERR_INVALID_ARG, "lse is NULL");
  const size_t need = lwm_blockattn_bwd_workspace_size(q->B, q->H, q->L, k->L, q->D);
  if (!empty && (!workspace || workspace_bytes < need))
    return fail(LWM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (workspace && reinterpret_cast<uintptr_t>(workspace) % 256) return fail(LWM_ERR_WORKSPACE, "workspace not 256-byte aligned");
  *p = lwm::BwdParams{};
  p->q = static_cast<const uint16_t*>(q->ptr);
  p->k = static_cast<const uint16_t*>(k->ptr);
  p->v = static_cast<const uint16_t*>(v->ptr);
  p->o = static_cast<const uint16_t*>(o->ptr);
  p->dout = static_cast<const uint16_t*>(dout->ptr);
  p->sq = strides(q); p->sk = strides(k); p->sv = strides(v); p->so = strides(o); p->sdo = strides(dout);
  p->lse = lse;
  p->delta = static_cast<float*>(workspace);
  p->lse2 = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) + need / 2) : nullptr;
  // Room after the two rows for the stored dS^T of at least min(B*H, 8) (batch, head) pairs: the
  // dK/dV kernel writes dS and dQ is formed from it.  Passes take whole multiples of 8 pairs (one
  // per XCD) unless every pair fits in one.
  if (!empty && workspace && q->L > 0 && k->L > 0 && ds_row_len(q->L) <= kMaxDsLd) {
    const int64_t ld = ds_row_len(q->L), BH = q->B * q->H, shift = ds_shift(q_offset, k_offset, causal);
    const int64_t blocks = ds_slot_blocks(q->L, k->L, shift);
    const size_t slot = (size_t)std::max<int64_t>(blocks, 1) * 8192;
    const size_t room = (workspace_bytes - need) / slot;
    int64_t g = room < (size_t)BH ? (int64_t)room : BH;
    if (g < BH && g >= 8) g &= ~int64_t(7);
    if (g >= (BH < 8 ? BH : 8)) {
      p->ds = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + need);
      p->ds_ld = ld;
      p->ds_heads = (int)g;
      p->ds_shift = shift;
      p->ds_slot_blocks = blocks;
    }
  }
  p->B = (int)q->B; p->H = (int)q->H; p->Lq = (int)q->L; p->Lk = (int)k->L;
  p->seg_q = seg_q; p->seg_k = seg_k;
  p->q_offset = q_offset; p->k_offset = k_offset; p->causal = causal;
  p->scale = sc;
  p->scale_log2 = sc * 1.4426950408889634f;
  return LWM_OK;
}

// A float32 gradient accumulator with the shape of `like` (q for dQ, k for dK and dV).
int check_acc(const lwm_tensor4* acc, const lwm_tensor4* like, const char* name) {
  int s;
  if ((s = check_tensor(acc, name))) return s;
  if (acc->dtype != LWM_FP32) return fail(LWM_ERR_INVALID_ARG, "%s must be float32", name);
  if (acc->B != like->B || acc->L != like->L || acc->H != like->H || acc->D != like->D)
    return fail(LWM_ERR_INVALID_ARG, "%s: shape mismatch", name);
  return LWM_OK;
}

}  // namespace

extern "C" {

int lwm_blockattn_bwd(const lwm_tensor4* q, const lwm_tensor4* k, const lwm_tensor4* v, const lwm_tensor4* o,
                      const float* lse, const lwm_tensor4* dout, const int32_t* seg_q, const int32_t* seg_k,
                      int64_t q_offset, int64_t k_offset, int32_t causal, float scale, const lwm_tensor4* dq,
                      const lwm_tensor4* dk, const lwm_tensor4* dv, void* workspace, size_t workspace_bytes,
                      void* stream) {
  lwm::BwdParams p;
  int s;
  if ((s = prepare_bwd(q, k, v, o, lse, dout, seg_q, seg_k, q_offset, k_offset, causal, scale, workspace,
                       workspace_bytes, &p)))
    return s;
  if ((s = check_tensor(dq, "dq")) || (s = check_same(q, dq, "q", "dq", true))) return s;
  if ((s = check_tensor(dk, "dk")) || (s = check_same(k, dk, "k", "dk", true))) return s;
  if ((s = check_tensor(dv, "dv")) || (s = check_same(v, dv, "v", "dv", true))) return s;
  p.dq = static_cast<uint16_t*>(dq->ptr);
  p.dk = static_cast<uint16_t*>(dk->ptr);
  p.dv = static_cast<uint16_t*>(dv->ptr);
  p.sdq = strides(dq); p.sdk = strides(dk); p.sdv = strides(dv);
  return hip_status(lwm::launch_attn_bwd(p, static_cast<hipStream_t>(stream)), "backward launch");
}

}  // extern "C"

namespace {

// Workspace of lwm_blockattn_bwd_noalloc: a static device array, one copy per GPU, held until the
// process ends.  It holds the same two float32 rows per query (D_i, lse_i * log2 e) as the
// caller-owned workspace of lwm_blockattn_bwd, for up to kStaticBwdRows query rows (B * H * Lq).
constexpr int64_t kStaticBwdRows = int64_t(1) << 21;
constexpr size_t kStaticBwdBytes = 2 * (size_t)kStaticBwdRows * sizeof(float);
static __device__ __align__(256) uint8_t scratch[kStaticBwdBytes];

// Device address of `scratch` on each GPU, taken once per device with that device current (in
// host code the array's name is only a stand-in for the symbol, never a device address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LWM_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(LWM_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return fail(LWM_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LWM_OK;
}

}  // namespace

extern "C" {

int lwm_blockattn_bwd_noalloc(const lwm_tensor4* q, const lwm_tensor4* k, const lwm_tensor4* v,
                              const lwm_tensor4* o, const float* lse, const lwm_tensor4* dout,
                              const int32_t* seg_q, const int32_t* seg_k, int64_t q_offset, int64_t k_offset,
                              int32_t causal, float scale, const lwm_tensor4* dq, const lwm_tensor4* dk,
                              const lwm_tensor4* dv, void* stream) {
  if (q && q->B > 0 && q->H > 0 && q->L > 0 && q->B * q->H > kStaticBwdRows / q->L)
    return fail(LWM_ERR_UNSUPPORTED, "B*H*Lq = %lld query rows exceed the static workspace's %lld",
                (long long)(q->B * q->H * q->L), (long long)kStaticBwdRows);
  void* ws = nullptr;
  int s;
  if ((s = static_scratch(&ws))) return s;
  // exactly the two rows per query: the static array has no room for stored dS
  const size_t bytes = q ? lwm_blockattn_bwd_workspace_size(q->B, q->H, q->L, 0, q->D) : kStaticBwdBytes;
  return lwm_blockattn_bwd(q, k, v, o, lse, dout, seg_q, seg_k, q_offset, k_offset, causal, scale, dq, dk, dv, ws,
                           bytes, stream);
}

int lwm_blockattn_bwd_rope(const lwm_tensor4* q_rot, const lwm_tensor4* k_rot, const lwm_tensor4* v,
                           const lwm_tensor4* o, const float* lse, const lwm_tensor4* dout, const int32_t* seg_q,
                           const int32_t* seg_k, int64_t q_offset, int64_t k_offset, int32_t causal, float scale,
                           const lwm_rope_args* rope, const lwm_tensor4* dq, const lwm_tensor4* dk,
                           const lwm_tensor4* dv, void* workspace, size_t workspace_bytes, void* stream) {
  lwm::BwdParams p;
  int s;
  if ((s = prepare_bwd(q_rot, k_rot, v, o, lse, dout, seg_q, seg_k, q_offset, k_offset, causal, scale, workspace,
                       workspace_bytes, &p)))
    return s;
  if ((s = check_tensor(dq, "dq")) || (s = check_same(q_rot, dq, "q_rot", "dq", true))) return s;
  if ((s = check_tensor(dk, "dk")) || (s = check_same(k_rot, dk, "k_rot", "dk", true))) return s;
  if ((s = check_tensor(dv, "dv")) || (s = check_same(v, dv, "v", "dv", true))) return s;
  if ((s = check_rope(rope, seg_q != nullptr, &p.rope))) return s;
  p.dq = static_cast<uint16_t*>(dq->ptr);
  p.dk = static_cast<uint16_t*>(dk->ptr);
  p.dv = static_cast<uint16_t*>(dv->ptr);
  p.sdq = strides(dq); p.sdk = strides(dk); p.sdv = strides(dv);
  return hip_status(lwm::launch_attn_bwd(p, static_cast<hipStream_t>(stream)), "backward launch");
}

int lwm_ring_step_bwd(const lwm_tensor4* q, const lwm_tensor4* k_shard, const lwm_tensor4* v_shard,
                      const lwm_tensor4* o, const float* lse, const lwm_tensor4* dout, const int32_t* seg_q,
                      const int32_t* seg_k, int64_t q_offset, int64_t k_offset, int32_t causal, float scale,
                      const lwm_tensor4* dq_acc, const lwm_tensor4* dk_acc, const lwm_tensor4* dv_acc,
                      void* workspace, size_t workspace_bytes, int32_t flags, void* stream) {
  lwm::BwdParams p;
  int s;
  if (flags != 0 && flags != LWM_RING_BWD_REUSE_WORKSPACE)
    return fail(LWM_ERR_INVALID_ARG, "flags must be 0 or LWM_RING_BWD_REUSE_WORKSPACE");
  if ((s = prepare_bwd(q, k_shard, v_shard, o, lse, dout, seg_q, seg_k, q_offset, k_offset, causal, scale, workspace,
                       workspace_bytes, &p)))
    return s;
  if ((s = check_acc(dq_acc, q, "dq_acc")) || (s = check_acc(dk_acc, k_shard, "dk_acc")) ||
      (s = check_acc(dv_acc, k_shard, "dv_acc")))
    return s;
  p.dq_acc = static_cast<float*>(dq_acc->ptr);
  p.dk_acc = static_cast<float*>(dk_acc->ptr);
  p.dv_acc = static_cast<float*>(dv_acc->ptr);
  p.sdqa = strides(dq_acc); p.sdka = strides(dk_acc); p.sdva = strides(dv_acc);
  p.delta_ready = flags == LWM_RING_BWD_REUSE_WORKSPACE;
  return hip_status(lwm::launch_attn_bwd(p, static_cast<hipStream_t>(stream)), "backward ring step launch");
}

int lwm_ring_step(const lwm_tensor4* q, const lwm_tensor4* k_shard, const lwm_tensor4* v_shard, const int32_t* seg_q,
                  const int32_t* seg_k, int64_t q_offset, int64_t k_offset, int32_t causal, float scale,
                  const lwm_tensor4* o_acc, float* lse_acc, const lwm_tensor4* o_final, void* stream) {
  int s;
  if ((s = check_attention(q, k_shard, v_shard, seg_q, seg_k, q_offset, k_offset, causal))) return s;
  if (q->dtype != LWM_BF16) return fail(LWM_ERR_UNSUPPORTED, "ring step is implemented for bf16 only");
  if ((s = check_tensor(o_acc, "o_acc"))) return s;
  if (o_acc->dtype != LWM_FP32) return fail(LWM_ERR_INVALID_ARG, "o_acc must be float32");
  if (o_acc->B != q->B || o_acc->L != q->L || o_acc->H != q->H || o_acc->D != q->D)
    return fail(LWM_ERR_INVALID_ARG, "o_acc shape must equal q's");
  if (o_final) {
    if ((s = check_tensor(o_final, "o_final")) || (s = check_same(q, o_final, "q", "o_final", true))) return s;
  }
  const bool empty = q->B == 0 || q->L == 0 || q->H == 0;
  if (!empty && !lse_acc) return fail(LWM_ERR_INVALID_ARG, "lse_acc is NULL");
  if (lse_acc && reinterpret_cast<uintptr_t>(lse_acc) % 4) return fail(LWM_ERR_INVALID_ARG, "lse_acc not 4-byte aligned");
  float sc;
  if ((s = check_scale(scale, q->D, &sc))) return s;
  lwm::FwdParams p{};
  p.q = q->ptr; p.k = k_shard->ptr; p.v = v_shard->ptr;
  p.sq = strides(q); p.sk = strides(k_shard); p.sv = strides(v_shard);
  p.B = (int)q->B; p.H = (int)q->H; p.Lq = (int)q->L; p.Lk = (int)k_shard->L;
  p.seg_q = seg_q; p.seg_k = seg_k;
  p.q_offset = q_offset; p.k_offset = k_offset; p.causal = causal;
  p.scale_log2 = sc * 1.4426950408889634f;
  p.o = o_final ? o_final->ptr : nullptr;
  if (o_final) p.so = strides(o_final);
  p.lse = nullptr;
  p.o_acc = static_cast<float*>(o_acc->ptr);
  p.soa = strides(o_acc);
  p.lse_acc = lse_acc;
  p.mode = 1;
  return hip_status(lwm::launch_attn_fwd(p, true, static_cast<hipStream_t>(stream)), "ring step launch");
}

size_t lwm_blockwise_ffn_workspace_size(int64_t rows, int64_t d_ff, int64_t chunk) {
  if (rows <= 0 || d_ff <= 0 || chunk <= 0) return 256;
  const size_t bytes = (size_t)(chunk < rows ? chunk : rows) * (size_t)d_ff * 2;
  return (bytes + 255) / 256 * 256;
}

int lwm_blockwise_ffn(const void* x, int64_t rows, int64_t d_model, int64_t ldx, const void* w_gate,
                      const void* w_up, int64_t ldw, const void* w_down, int64_t ldwd, int64_t d_ff, void* y,
                      int64_t ldy, int64_t chunk, void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 0 || rows > (int64_t(1) << 31) - 1) return fail(LWM_ERR_INVALID_ARG, "rows must be in [0, 2^31)");
  if (chunk < 1) return fail(LWM_ERR_INVALID_ARG, "chunk must be >= 1");
  if (d_model <= 0 || d_ff <= 0 || d_model % 32 || d_ff % 32)
    return fail(LWM_ERR_UNSUPPORTED, "d_model and d_ff must be positive multiples of 32 (got %lld, %lld)",
                (long long)d_model, (long long)d_ff);
  const struct {
    const char* name;
    int64_t ld, min;
  } lds[] = {{"ldx", ldx, d_model}, {"ldw", ldw, d_model}, {"ldwd", ldwd, d_ff}, {"ldy", ldy, d_model}};
  for (const auto& l : lds) {
    if (l.ld < l.min) return fail(LWM_ERR_INVALID_ARG, "%s = %lld is below the row length %lld", l.name, (long long)l.ld, (long long)l.min);
    if (l.ld % 8) return fail(LWM_ERR_INVALID_ARG, "%s must be a multiple of 8 elements (16 bytes)", l.name);
    if (l.ld >= (int64_t(1) << 22))
      return fail(LWM_ERR_UNSUPPORTED, "%s: rows of 8 MiB or more (tiles use 32-bit offsets)", l.name);
  }
  if (rows == 0) return ok();
  const struct {
    const char* name;
    const void* p;
  } ptrs[] = {{"x", x}, {"w_gate", w_gate}, {"w_up", w_up}, {"w_down", w_down}, {"y", y}};
  for (const auto& q : ptrs) {
    if (!q.p) return fail(LWM_ERR_INVALID_ARG, "%s is NULL", q.name);
    if (reinterpret_cast<uintptr_t>(q.p) % 16) return fail(LWM_ERR_INVALID_ARG, "%s not 16-byte aligned", q.name);
  }
  const size_t need = lwm_blockwise_ffn_workspace_size(rows, d_ff, chunk);
  if (!workspace || workspace_bytes < need)
    return fail(LWM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(LWM_ERR_WORKSPACE, "workspace not 256-byte aligned");
  lwm::FfnParams p{};
  p.x = static_cast<const uint16_t*>(x); p.ldx = ldx;
  p.w_gate = static_cast<const uint16_t*>(w_gate); p.w_up = static_cast<const uint16_t*>(w_up); p.ldw = ldw;
  p.w_down = static_cast<const uint16_t*>(w_down); p.ldwd = ldwd;
  p.y = static_cast<uint16_t*>(y); p.ldy = ldy;
  p.h = static_cast<uint16_t*>(workspace);
  p.rows = rows; p.chunk = chunk < rows ? chunk : rows;
  p.d_model = (int)d_model; p.d_ff = (int)d_ff;
  return hip_status(lwm::launch_ffn(p, static_cast<hipStream_t>(stream)), "feed-forward launch");
}

int lwm_probe_mfma_bf16(const void* src, void* sink, int32_t blocks, int32_t iters, void* stream) {
  if (!src || !sink) return fail(LWM_ERR_INVALID_ARG, "src and sink must not be NULL");
  if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(sink) % 4)
    return fail(LWM_ERR_INVALID_ARG, "src must be 16-byte and sink 4-byte aligned");
  // bounded so that one launch stays within seconds (4096 blocks of 2^24 rounds: about 20 s on a 256-CU part)
  if (blocks < 1 || blocks > 4096) return fail(LWM_ERR_INVALID_ARG, "blocks must be in [1, 4096]");
  if (iters < 8 || iters % 8 || iters > (1 << 24)) return fail(LWM_ERR_INVALID_ARG, "iters must be a positive multiple of 8, at most 2^24");
  return hip_status(lwm::launch_mfma_probe(src, static_cast<float*>(sink), blocks, iters, static_cast<hipStream_t>(stream)),
                    "MFMA probe launch");
}

}  // extern "C"
