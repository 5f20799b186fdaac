// Host side of the C ABI declared in include/seer.h: argument validation,
// workspace layout and kernel launch. Nothing here allocates device memory or
// synchronizes the host.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>
#include <string>

#include "seer.h"
#include "seer_internal.h"

namespace {

thread_local std::string g_last_error;

seer_status fail(seer_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
seer_status fail(seer_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

seer_status ok() {
  g_last_error.clear();
  return SEER_OK;
}

constexpr int kBlock = 64;
constexpr long long kMaxSeqAttn = 1LL << 22;    // 65536 key blocks (16-bit on-chip list)
constexpr int kMaxNbGate = 16384;               // one score row in LDS (64 KiB)
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

long long nblocks(const seer_shape* s) { return (static_cast<long long>(s->seq_len) + kBlock - 1) / kBlock; }

// Shape checks shared by every call. Sets *empty when there is nothing to do.
seer_status check_shape(const seer_shape* s, bool* empty) {
  if (s == nullptr) return fail(SEER_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch < 0 || s->heads_q < 0 || s->heads_kv < 0 || s->seq_len < 0 || s->head_dim < 0)
    return fail(SEER_ERR_SHAPE, "negative size (batch %d, heads_q %d, heads_kv %d, seq_len %d, head_dim %d)",
                s->batch, s->heads_q, s->heads_kv, s->seq_len, s->head_dim);
  if (s->block != kBlock) return fail(SEER_ERR_SHAPE, "block must be 64 (got %d)", s->block);
  if (s->heads_q > 0 && (s->heads_kv == 0 || s->heads_q % s->heads_kv != 0))
    return fail(SEER_ERR_SHAPE, "heads_q (%d) must be a positive multiple of heads_kv (%d)", s->heads_q,
                s->heads_kv);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(SEER_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", s->head_dim);
  if (s->seq_len > kMaxSeqAttn)
    return fail(SEER_ERR_UNSUPPORTED, "seq_len %d exceeds the supported maximum %lld", s->seq_len, kMaxSeqAttn);
  const long long rows = static_cast<long long>(s->batch) * s->heads_q * nblocks(s);
  if (rows > 0x7fffffffLL)
    return fail(SEER_ERR_SHAPE, "batch * heads_q * blocks = %lld exceeds the launch limit", rows);
  *empty = (s->batch == 0 || s->heads_q == 0 || s->seq_len == 0);
  return SEER_OK;
}

seer_status check_device() {
  static std::once_flag once[64];
  static bool good[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SEER_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(SEER_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  std::call_once(once[dev], [dev]() {
    hipDeviceProp_t prop;
    good[dev] = hipGetDeviceProperties(&prop, dev) == hipSuccess && strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  });
  if (!good[dev]) return fail(SEER_ERR_UNSUPPORTED, "device %d is not a gfx950 (MI355X) GPU", dev);
  return SEER_OK;
}

// Workgroup order of the attention kernels (see attn_kernels.hip). Measured on
// MI355X at 32k and 128k tokens: KV-group-major order keeps one group's K/V
// in the Infinity Cache; for block-sparse rows, head-major inside the group
// additionally keeps rows of similar density together.
int attn_sched(int mode) { return mode == 0 ? 3 : 2; }

seer::AttnArgs attn_args(const seer_shape* s, const void* q, const void* k, const void* v, int mode) {
  seer::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.B = s->batch;
  a.Hq = s->heads_q;
  a.Hkv = s->heads_kv;
  a.S = s->seq_len;
  a.D = s->head_dim;
  a.nb = static_cast<int>(nblocks(s));
  a.group = s->heads_q / s->heads_kv;
  a.hs = s->seq_len;
  a.ntri = static_cast<long long>(a.nb) * (a.nb + 1) / 2;
  a.scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(s->head_dim)));
  a.sched = attn_sched(mode);
  return a;
}

seer_status check_qkv(const void* q, const void* k, const void* v) {
  if (q == nullptr || k == nullptr || (v == nullptr))
    return fail(SEER_ERR_INVALID_ARG, "q, k and v must be non-NULL device pointers");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
    return fail(SEER_ERR_INVALID_ARG, "q, k and v must be 16-byte aligned");
  return SEER_OK;
}

seer_status check_out(void* out, seer_dtype dt, float* lse) {
  if (out == nullptr) return fail(SEER_ERR_INVALID_ARG, "out must be a non-NULL device pointer");
  if (dt != SEER_F32 && dt != SEER_BF16) return fail(SEER_ERR_INVALID_ARG, "out_dtype %d is not SEER_F32/SEER_BF16", dt);
  if (!aligned(out, dt == SEER_F32 ? 16 : 8)) return fail(SEER_ERR_INVALID_ARG, "out is misaligned for its dtype");
  if (lse != nullptr && !aligned(lse, 4)) return fail(SEER_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  return SEER_OK;
}

struct GateLayout {
  size_t qp, kp, qg, kg, scores, total;
};

GateLayout gate_layout(const seer_shape* s, int dg, int wk_per_kv, bool want_scores) {
  const size_t B = s->batch, Hq = s->heads_q, Hkv = s->heads_kv, D = s->head_dim, nb = nblocks(s);
  const size_t hwk = wk_per_kv ? Hkv : Hq;
  GateLayout L{};
  size_t off = 0;
  L.qp = off; off += align_up(B * Hq * nb * D * 4);
  L.kp = off; off += align_up(B * Hkv * nb * 3 * D * 4);
  L.qg = off; off += align_up(B * Hq * nb * dg * 4);
  L.kg = off; off += align_up(B * hwk * nb * dg * 4);
  L.scores = off; off += want_scores ? 0 : align_up(B * Hq * nb * nb * 4);
  L.total = off;
  return L;
}

struct DistillLayout {
  GateLayout g;       // pooled, projected and logits (scores segment always present)
  size_t dqg, dkg, row_loss, total;
};

DistillLayout distill_layout(const seer_shape* s, int dg, int wk_per_kv) {
  const size_t B = s->batch, Hq = s->heads_q, nb = nblocks(s);
  DistillLayout L{};
  L.g = gate_layout(s, dg, wk_per_kv, false);
  size_t off = L.g.total;
  L.dqg = off; off += align_up(B * Hq * nb * dg * 4);
  L.dkg = off; off += align_up(B * Hq * nb * dg * 4);
  L.row_loss = off; off += align_up(B * Hq * nb * 4);
  L.total = off;
  return L;
}

seer_status fill_topk(const seer_shape* shape, seer_mask_mode mode, int32_t topk_k, const int32_t* topk_per_head,
                      seer::TopkTable* tk) {
  if (mode != SEER_MASK_TOPK) return SEER_OK;
  if (shape->heads_q > seer::kMaxTopkHeads)
    return fail(SEER_ERR_UNSUPPORTED, "top-k supports at most %d query heads", seer::kMaxTopkHeads);
  for (int h = 0; h < shape->heads_q; ++h) {
    const int kv = topk_per_head ? topk_per_head[h] : topk_k;
    if (kv < 1) return fail(SEER_ERR_INVALID_ARG, "top-k value %d (head %d) must be >= 1", kv, h);
    tk->k[h] = kv;
  }
  return SEER_OK;
}

seer::DecodeGateArgs decode_gate_args(const seer_shape* s, int wk_per_kv_head) {
  seer::DecodeGateArgs a{};
  a.B = s->batch;
  a.Hq = s->heads_q;
  a.Hkv = s->heads_kv;
  a.S = s->seq_len;
  a.D = s->head_dim;
  a.nb = static_cast<int>(nblocks(s));
  a.group = s->heads_kv > 0 ? s->heads_q / s->heads_kv : 1;
  a.wk_per_kv = wk_per_kv_head != 0;
  a.scale = static_cast<float>(1.0 / sqrt(static_cast<double>(s->head_dim)));
  return a;
}

seer_status check_rope(float rope_theta) {
  if (!isfinite(rope_theta) || rope_theta < 0.f)
    return fail(SEER_ERR_INVALID_ARG, "rope_theta must be 0 (no RoPE) or a finite positive base (got %g)",
                static_cast<double>(rope_theta));
  return SEER_OK;
}

}  // namespace

// Scratch of the allocation-free entry point (seer_decode_attn_fwd_noalloc):
// one copy per device, held until the process ends.
static __device__ __align__(256) unsigned char scratch[SEER_NOALLOC_SCRATCH_BYTES];

namespace {

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[64];

// Device address of the current device's `scratch`, looked up on the first
// call on that device.
seer_status scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SEER_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(SEER_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot]() { slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch)); });
  if (slot.err != hipSuccess || slot.ptr == nullptr)
    return fail(SEER_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(slot.err));
  *ptr = slot.ptr;
  return SEER_OK;
}

}  // namespace

extern "C" {

const char* seer_status_string(seer_status s) {
  switch (s) {
    case SEER_OK: return "SEER_OK";
    case SEER_ERR_INVALID_ARG: return "SEER_ERR_INVALID_ARG";
    case SEER_ERR_SHAPE: return "SEER_ERR_SHAPE";
    case SEER_ERR_UNSUPPORTED: return "SEER_ERR_UNSUPPORTED";
    case SEER_ERR_WORKSPACE: return "SEER_ERR_WORKSPACE";
    case SEER_ERR_HIP: return "SEER_ERR_HIP";
  }
  return "SEER_ERR_UNKNOWN";
}

const char* seer_last_error(void) { return g_last_error.c_str(); }

const char* seer_version(void) { return "seer-mi355x 0.1.0 (gfx950)"; }

// ---------------------------------------------------------------------------
size_t seer_gate_workspace_size(const seer_shape* shape, int32_t gate_dim, int32_t wk_per_kv_head,
                                int32_t want_scores) {
  bool empty = false;
  if (check_shape(shape, &empty) != SEER_OK || gate_dim <= 0) return 0;
  return gate_layout(shape, gate_dim, wk_per_kv_head != 0, want_scores != 0).total;
}

// hs: tokens between consecutive heads' rows of q and k (seq_len, or the packed
// length of a varlen batch); launch = false only validates.
static seer_status gate_impl(const seer_shape* shape, long long hs, int32_t gate_dim, int32_t wk_per_kv_head,
                             float rope_theta, const void* q, const void* k, const float* w_q, const float* w_k,
                             seer_mask_mode mode, float threshold, int32_t topk_k, const int32_t* topk_per_head,
                             float* scores, uint8_t* block_mask, void* workspace, size_t workspace_bytes,
                             void* hip_stream, bool launch) {
  bool empty = false;
  seer_status st = check_shape(shape, &empty);
  if (st != SEER_OK) return st;
  if (gate_dim < 16 || gate_dim > 256 || gate_dim % 16 != 0)
    return fail(SEER_ERR_UNSUPPORTED, "gate_dim must be a multiple of 16 in [16, 256] (got %d)", gate_dim);
  if (mode != SEER_MASK_THRESHOLD && mode != SEER_MASK_TOPK)
    return fail(SEER_ERR_INVALID_ARG, "mask mode %d is not SEER_MASK_THRESHOLD/SEER_MASK_TOPK", mode);
  if (mode == SEER_MASK_THRESHOLD && !isfinite(threshold))
    return fail(SEER_ERR_INVALID_ARG, "threshold must be finite");
  if ((st = check_rope(rope_theta)) != SEER_OK) return st;
  seer::TopkTable tk{};
  if ((st = fill_topk(shape, mode, topk_k, topk_per_head, &tk)) != SEER_OK) return st;
  if (nblocks(shape) > kMaxNbGate)
    return fail(SEER_ERR_UNSUPPORTED, "the gate supports at most %d blocks per sequence", kMaxNbGate);
  if (empty) return ok();
  st = check_qkv(q, k, k);
  if (st != SEER_OK) return st;
  if (w_q == nullptr || w_k == nullptr) return fail(SEER_ERR_INVALID_ARG, "w_q and w_k must be non-NULL");
  if (block_mask == nullptr) return fail(SEER_ERR_INVALID_ARG, "block_mask must be non-NULL");
  if (scores != nullptr && !aligned(scores, 4)) return fail(SEER_ERR_INVALID_ARG, "scores must be 4-byte aligned");
  const GateLayout L = gate_layout(shape, gate_dim, wk_per_kv_head != 0, scores != nullptr);
  if (workspace == nullptr || workspace_bytes < L.total || !aligned(workspace, kAlign))
    return fail(SEER_ERR_WORKSPACE, "workspace must be %zu bytes, 256-byte aligned (got %zu at %p)", L.total,
                workspace_bytes, workspace);
  st = check_device();
  if (st != SEER_OK || !launch) return st;

  char* ws = static_cast<char*>(workspace);
  seer::GateArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.wq = w_q;
  a.wk = w_k;
  a.qp = reinterpret_cast<float*>(ws + L.qp);
  a.kp = reinterpret_cast<float*>(ws + L.kp);
  a.qg = reinterpret_cast<float*>(ws + L.qg);
  a.kg = reinterpret_cast<float*>(ws + L.kg);
  a.scores = scores ? scores : reinterpret_cast<float*>(ws + L.scores);
  a.mask = block_mask;
  a.skip_scores = scores == nullptr;
  a.B = shape->batch;
  a.Hq = shape->heads_q;
  a.Hkv = shape->heads_kv;
  a.S = shape->seq_len;
  a.hs = hs;
  a.D = shape->head_dim;
  a.nb = static_cast<int>(nblocks(shape));
  a.Dg = gate_dim;
  a.group = shape->heads_q / shape->heads_kv;
  a.wk_per_kv = wk_per_kv_head != 0;
  a.scale = static_cast<float>(1.0 / sqrt(static_cast<double>(shape->head_dim)));
  a.mode = mode == SEER_MASK_TOPK ? 1 : 0;
  a.threshold = threshold;
  a.rope_base = rope_theta > 0.f ? static_cast<double>(rope_theta) / shape->block : 0.0;
  hipError_t e = seer::launch_gate(a, tk, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(SEER_ERR_HIP, "gate launch failed: %s", hipGetErrorString(e));
  return ok();
}

seer_status seer_gate_fwd(const seer_shape* shape, int32_t gate_dim, int32_t wk_per_kv_head, float rope_theta,
                          const void* q, const void* k, const float* w_q, const float* w_k, seer_mask_mode mode,
                          float threshold, int32_t topk_k, const int32_t* topk_per_head, float* scores,
                          uint8_t* block_mask, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return gate_impl(shape, shape ? shape->seq_len : 0, gate_dim, wk_per_kv_head, rope_theta, q, k, w_q, w_k, mode,
                   threshold, topk_k, topk_per_head, scores, block_mask, workspace, workspace_bytes, hip_stream, true);
}

// ---------------------------------------------------------------------------
seer_status seer_decode_compress_k(const seer_shape* shape, int32_t wk_per_kv_head, const void* k_cache,
                                   const float* w_k, int32_t block_begin, float* kcomp, int32_t kcomp_blocks,
                                   void* hip_stream) {
  bool empty = false;
  seer_status st = check_shape(shape, &empty);
  if (st != SEER_OK) return st;
  const int nb = static_cast<int>(nblocks(shape));
  if (block_begin < 0 || block_begin > nb)
    return fail(SEER_ERR_INVALID_ARG, "block_begin %d outside [0, %d]", block_begin, nb);
  if (kcomp_blocks < nb)
    return fail(SEER_ERR_INVALID_ARG, "kcomp_blocks (%d) is smaller than the cache's %d blocks", kcomp_blocks, nb);
  if (empty || block_begin == nb) return ok();
  if (k_cache == nullptr || !aligned(k_cache, 16))
    return fail(SEER_ERR_INVALID_ARG, "k_cache must be a non-NULL, 16-byte aligned device pointer");
  if (w_k == nullptr || kcomp == nullptr || !aligned(kcomp, 16))
    return fail(SEER_ERR_INVALID_ARG, "w_k and kcomp must be non-NULL (kcomp 16-byte aligned)");
  if ((st = check_device()) != SEER_OK) return st;
  seer::DecodeGateArgs a = decode_gate_args(shape, wk_per_kv_head);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.wk = w_k;
  a.kcomp = kcomp;
  a.kcomp_blocks = kcomp_blocks;
  a.block_begin = block_begin;
  hipError_t e = seer::launch_decode_kcomp(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(SEER_ERR_HIP, "decode K compression launch failed: %s", hipGetErrorString(e));
  return ok();
}

seer_status seer_decode_gate_fwd(const seer_shape* shape, int32_t wk_per_kv_head, const void* q, const float* kcomp,
                                 int32_t kcomp_blocks, seer_mask_mode mode, float threshold, int32_t topk_k,
                                 const int32_t* topk_per_head, float* scores, uint8_t* block_mask,
                                 void* hip_stream) {
  bool empty = false;
  seer_status st = check_shape(shape, &empty);
  if (st != SEER_OK) return st;
  if (mode != SEER_MASK_THRESHOLD && mode != SEER_MASK_TOPK)
    return fail(SEER_ERR_INVALID_ARG, "mask mode %d is not SEER_MASK_THRESHOLD/SEER_MASK_TOPK", mode);
  if (mode == SEER_MASK_THRESHOLD && !isfinite(threshold))
    return fail(SEER_ERR_INVALID_ARG, "threshold must be finite");
  seer::TopkTable tk{};
  if ((st = fill_topk(shape, mode, topk_k, topk_per_head, &tk)) != SEER_OK) return st;
  const int nb = static_cast<int>(nblocks(shape));
  if (nb > kMaxNbGate) return fail(SEER_ERR_UNSUPPORTED, "the gate supports at most %d blocks", kMaxNbGate);
  if (kcomp_blocks < nb)
    return fail(SEER_ERR_INVALID_ARG, "kcomp_blocks (%d) is smaller than the cache's %d blocks", kcomp_blocks, nb);
  if (empty) return ok();
  if (q == nullptr || kcomp == nullptr || block_mask == nullptr || scores == nullptr || !aligned(kcomp, 16) ||
      !aligned(q, 16))
    return fail(SEER_ERR_INVALID_ARG, "q and kcomp (16-byte aligned), scores and block_mask must be non-NULL");
  if (!aligned(scores, 4)) return fail(SEER_ERR_INVALID_ARG, "scores must be 4-byte aligned");
  if ((st = check_device()) != SEER_OK) return st;
  seer::DecodeGateArgs a = decode_gate_args(shape, wk_per_kv_head);
  a.q = static_cast<const uint16_t*>(q);
  a.kcomp = const_cast<float*>(kcomp);
  a.kcomp_blocks = kcomp_blocks;
  a.scores = scores;
  a.mask = block_mask;
  a.mode = mode == SEER_MASK_TOPK ? 1 : 0;
  a.threshold = threshold;
  hipError_t e = seer::launch_decode_gate(a, tk, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(SEER_ERR_HIP, "decode gate launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t seer_decode_attn_workspace_size(const seer_shape* shape) {
  bool empty = false;
  if (check_shape(shape, &empty) != SEER_OK || empty) return 0;
  return seer::decode_workspace_bytes(shape->batch, shape->heads_q, shape->heads_kv, static_cast<int>(nblocks(shape)),
                                      shape->head_dim);
}

static seer_status decode_attn_impl(const seer_shape* shape, const void* q, const void* k_cache,
                                    const void* v_cache, const uint8_t* block_mask, void* out, seer_dtype out_dtype,
                                    float* lse, float* gt, void* workspace, size_t workspace_bytes,
                                    void* hip_stream) {
  bool empty = false;
  seer_status st = check_shape(shape, &empty);
  if (st != SEER_OK) return st;
  if (out_dtype != SEER_F32 && out_dtype != SEER_BF16)
    return fail(SEER_ERR_INVALID_ARG, "out_dtype %d is not SEER_F32/SEER_BF16", out_dtype);
  if (shape->heads_q > 0 && shape->heads_q / shape->heads_kv > seer::kDecodeMaxGroup)
    return fail(SEER_ERR_UNSUPPORTED, "decode attention supports at most %d query heads per KV head",
                seer::kDecodeMaxGroup);
  if (gt != nullptr && block_mask != nullptr)
    return fail(SEER_ERR_INVALID_ARG, "the 1D max-pooled map (gt) is produced only in dense mode (block_mask NULL)");
  if (empty) return ok();
  if ((st = check_qkv(q, k_cache, v_cache)) != SEER_OK) return st;
  if ((st = check_out(out, out_dtype, lse)) != SEER_OK) return st;
  if (gt != nullptr && !aligned(gt, 4)) return fail(SEER_ERR_INVALID_ARG, "gt must be 4-byte aligned");
  const size_t need = seer_decode_attn_workspace_size(shape);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16))
    return fail(SEER_ERR_WORKSPACE, "workspace must be %zu bytes, 16-byte aligned (got %zu at %p)", need,
                workspace_bytes, workspace);
  if ((st = check_device()) != SEER_OK) return st;
  seer::DecodeAttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.mask = block_mask;
  a.out = out;
  a.lse = lse;
  a.gt = gt;
  a.part = static_cast<float*>(workspace);
  a.B = shape->batch;
  a.Hq = shape->heads_q;
  a.Hkv = shape->heads_kv;
  a.S = shape->seq_len;
  a.D = shape->head_dim;
  a.nb = static_cast<int>(nblocks(shape));
  a.group = shape->heads_q / shape->heads_kv;
  a.out_bf16 = out_dtype == SEER_BF16;
  a.scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(shape->head_dim)));
  seer::decode_split(a.B, a.Hkv, a.nb, &a.nsplit, &a.bps);
  {
    // block lists after the partials (16-byte aligned)
    const size_t part_bytes = static_cast<size_t>(a.B) * a.Hq * a.nsplit * (a.D + 2) * sizeof(float);
    char* base = static_cast<char*>(workspace) + (part_bytes + 15) / 16 * 16;
    a.blist = reinterpret_cast<uint32_t*>(base);
    a.bcount = reinterpret_cast<int*>(base + static_cast<size_t>(a.B) * a.Hkv * a.nb * sizeof(uint32_t));
  }
  hipError_t e = seer::launch_decode_attn(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(SEER_ERR_HIP, "decode attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

seer_status seer_decode_attn_fwd(const seer_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                                 const uint8_t* block_mask, void* out, seer_dtype out_dtype, float* lse, float* gt,
                                 void* workspace, size_t workspace_bytes, void* hip_stream) {
  return decode_attn_impl(shape, q, k_cache, v_cache, block_mask, out, out_dtype, lse, gt, workspace,
                          workspace_bytes, hip_stream);
}

// Allocation-free variant: the kernels' scratch (per-split partials and the
// per-KV-group block lists) lives in `scratch`, a fixed array in each device's
// copy of this library. Host code must not pass the array's name to a kernel:
// on the host it only stands for the symbol. Its device address is looked up
// once per device (with that device current) and kept.
seer_status seer_decode_attn_fwd_noalloc(const seer_shape* shape, const void* q, const void* k_cache,
                                         const void* v_cache, const uint8_t* block_mask, void* out,
                                         seer_dtype out_dtype, float* lse, float* gt, void* hip_stream) {
  bool empty = false;
  seer_status st = check_shape(shape, &empty);
  if (st != SEER_OK) return st;
  if (empty) return decode_attn_impl(shape, q, k_cache, v_cache, block_mask, out, out_dtype, lse, gt, nullptr, 0,
                                     hip_stream);
  const size_t need = seer_decode_attn_workspace_size(shape);
  if (need > SEER_NOALLOC_SCRATCH_BYTES)
    return fail(SEER_ERR_UNSUPPORTED,
                "decode attention of this shape needs %zu bytes of scratch, more than the %zu bytes the "
                "allocation-free entry point holds; use seer_decode_attn_fwd with a workspace",
                need, static_cast<size_t>(SEER_NOALLOC_SCRATCH_BYTES));
  void* ptr = nullptr;
  if ((st = scratch_address(&ptr)) != SEER_OK) return st;
  return decode_attn_impl(shape, q, k_cache, v_cache, block_mask, out, out_dtype, lse, gt, ptr,
                          SEER_NOALLOC_SCRATCH_BYTES, hip_stream);
}

// ---------------------------------------------------------------------------
size_t seer_gate_distill_workspace_size(const seer_shape* shape, int32_t gate_dim, int32_t wk_per_kv_head) {
  bool empty = false;
  if (check_shape(shape, &empty) != SEER_OK || gate_dim <= 0) return 0;
  return distill_layout(shape, gate_dim, wk_per_kv_head != 0).total;
}

seer_status seer_gate_distill_bwd(const seer_shape* shape, int32_t gate_dim, int32_t wk_per_kv_head,
                                  float rope_theta, const void* q, const void* k, const float* w_q,
                                  const float* w_k, const float* gt, float* loss, float* grad_wq,
                                  float* grad_wk, void* workspace, size_t workspace_bytes, void* hip_stream) {
  bool empty = false;
  seer_status st = check_shape(shape, &empty);
  if (st != SEER_OK) return st;
  if (gate_dim < 16 || gate_dim > 256 || gate_dim % 16 != 0)
    return fail(SEER_ERR_UNSUPPORTED, "gate_dim must be a multiple of 16 in [16, 256] (got %d)", gate_dim);
  if ((st = check_rope(rope_theta)) != SEER_OK) return st;
  if (nblocks(shape) > kMaxNbGate)
    return fail(SEER_ERR_UNSUPPORTED, "the gate supports at most %d blocks per sequence", kMaxNbGate);
  if (loss == nullptr || grad_wq == nullptr || grad_wk == nullptr)
    return fail(SEER_ERR_INVALID_ARG, "loss, grad_wq and grad_wk must be non-NULL");
  if (empty) return ok();
  if ((st = check_qkv(q, k, k)) != SEER_OK) return st;
  if (w_q == nullptr || w_k == nullptr || gt == nullptr)
    return fail(SEER_ERR_INVALID_ARG, "w_q, w_k and gt must be non-NULL");
  if (!aligned(gt, 4) || !aligned(loss, 4) || !aligned(grad_wq, 4) || !aligned(grad_wk, 4))
    return fail(SEER_ERR_INVALID_ARG, "gt, loss and the gradients must be 4-byte aligned");
  const DistillLayout L = distill_layout(shape, gate_dim, wk_per_kv_head != 0);
  if (workspace == nullptr || workspace_bytes < L.total || !aligned(workspace, kAlign))
    return fail(SEER_ERR_WORKSPACE, "workspace must be %zu bytes, 256-byte aligned (got %zu at %p)", L.total,
                workspace_bytes, workspace);
  st = check_device();
  if (st != SEER_OK) return st;

  char* ws = static_cast<char*>(workspace);
  seer::GateArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.wq = w_q;
  a.wk = w_k;
  a.qp = reinterpret_cast<float*>(ws + L.g.qp);
  a.kp = reinterpret_cast<float*>(ws + L.g.kp);
  a.qg = reinterpret_cast<float*>(ws + L.g.qg);
  a.kg = reinterpret_cast<float*>(ws + L.g.kg);
  a.scores = reinterpret_cast<float*>(ws + L.g.scores);
  a.dqg = reinterpret_cast<float*>(ws + L.dqg);
  a.dkg = reinterpret_cast<float*>(ws + L.dkg);
  a.row_loss = reinterpret_cast<float*>(ws + L.row_loss);
  a.gt = gt;
  a.loss = loss;
  a.grad_wq = grad_wq;
  a.grad_wk = grad_wk;
  a.B = shape->batch;
  a.Hq = shape->heads_q;
  a.Hkv = shape->heads_kv;
  a.S = shape->seq_len;
  a.hs = shape->seq_len;
  a.D = shape->head_dim;
  a.nb = static_cast<int>(nblocks(shape));
  a.Dg = gate_dim;
  a.group = shape->heads_q / shape->heads_kv;
  a.wk_per_kv = wk_per_kv_head != 0;
  a.scale = static_cast<float>(1.0 / sqrt(static_cast<double>(shape->head_dim)));
  a.rope_base = rope_theta > 0.f ? static_cast<double>(rope_theta) / shape->block : 0.0;
  hipError_t e = seer::launch_gate_distill(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(SEER_ERR_HIP, "distillation launch failed: %s", hipGetErrorString(e));
  return ok();
}

// ---------------------------------------------------------------------------
size_t seer_attn_workspace_size(const seer_shape* shape) {
  bool empty = false;
  if (check_shape(shape, &empty) != SEER_OK || empty) return 0;
  return seer::sparse_plan(shape->batch, shape->heads_kv, shape->heads_q / shape->heads_kv,
                           static_cast<int>(nblocks(shape)), shape->head_dim)
      .workspace_bytes;
}

static seer_status attn_impl(const seer_shape* shape, long long hs, const void* q, const void* k, const void* v,
                             const uint8_t* block_mask, void* out, seer_dtype out_dtype, float* lse,
                             void* workspace, size_t workspace_bytes, void* hip_stream, bool launch) {
  bool empty = false;
  seer_status st = check_shape(shape, &empty);
  if (st != SEER_OK) return st;
  if (out_dtype != SEER_F32 && out_dtype != SEER_BF16)
    return fail(SEER_ERR_INVALID_ARG, "out_dtype %d is not SEER_F32/SEER_BF16", out_dtype);
  if (empty) return ok();
  if ((st = check_qkv(q, k, v)) != SEER_OK) return st;
  if ((st = check_out(out, out_dtype, lse)) != SEER_OK) return st;
  seer::AttnArgs a = attn_args(shape, q, k, v, block_mask ? 0 : 1);
  if (block_mask != nullptr) {
    const seer::SparsePlan pl = seer::sparse_plan(a.B, a.Hkv, a.group, a.nb, a.D);
    a.xcd = pl.xcd;
    a.chunk = pl.chunk;
    a.nchunk = pl.nchunk;
    a.rotate = pl.rotate;
    a.items_per_group = pl.items_per_group;
    a.njobs = pl.njobs;
    a.slots_per_head = pl.slots_per_head;
    const long long items = static_cast<long long>(a.B) * a.Hkv * a.items_per_group;
    if (items > 0x7fffffffLL)
      return fail(SEER_ERR_SHAPE, "%lld block-sparse work items exceed the launch limit", items);
    const size_t need = pl.workspace_bytes;
    if (need > 0) {
      if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16))
        return fail(SEER_ERR_WORKSPACE, "workspace must be %zu bytes, 16-byte aligned (got %zu at %p)", need,
                    workspace_bytes, workspace);
      if (pl.xcd) {
        const size_t slots = static_cast<size_t>(a.B) * a.Hq * pl.slots_per_head;
        a.part_o16 = static_cast<uint16_t*>(workspace);
        a.part_l = reinterpret_cast<float*>(a.part_o16 + slots * 64 * a.D);
        a.xcd_ctr = reinterpret_cast<int*>(a.part_l + slots * 64);
      } else if (pl.xcd_rows) {
        a.xcd_work = static_cast<int*>(workspace);
      } else if (pl.rows) {
        a.rows = 1;
        a.xcd_ctr = static_cast<int*>(workspace);
      } else {
        a.part_o = static_cast<float*>(workspace);
        a.part_l = a.part_o + static_cast<size_t>(items) * 64 * a.D;
      }
    }
  }
  if ((st = check_device()) != SEER_OK || !launch) return st;
  a.hs = hs;
  a.mask = block_mask;
  a.out = out;
  a.lse = lse;
  a.out_bf16 = out_dtype == SEER_BF16;
  hipError_t e = seer::launch_attn(a, block_mask ? 0 : 1, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(SEER_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

seer_status seer_block_sparse_attn_fwd(const seer_shape* shape, const void* q, const void* k, const void* v,
                                       const uint8_t* block_mask, void* out, seer_dtype out_dtype, float* lse,
                                       void* workspace, size_t workspace_bytes, void* hip_stream) {
  return attn_impl(shape, shape ? shape->seq_len : 0, q, k, v, block_mask, out, out_dtype, lse, workspace,
                   workspace_bytes, hip_stream, true);
}

// ---------------------------------------------------------------------------
size_t seer_gt_workspace_size(const seer_shape* shape) {
  bool empty = false;
  if (check_shape(shape, &empty) != SEER_OK) return 0;
  const size_t nb = nblocks(shape);
  return align_up(static_cast<size_t>(shape->batch) * shape->heads_q * (nb * (nb + 1) / 2) * kBlock * sizeof(float));
}

static seer_status gt_impl(const seer_shape* shape, long long hs, const void* q, const void* k, const void* v,
                           void* out, seer_dtype out_dtype, float* lse, float* gt, void* workspace,
                           size_t workspace_bytes, void* hip_stream, bool launch) {
  bool empty = false;
  seer_status st = check_shape(shape, &empty);
  if (st != SEER_OK) return st;
  if (out_dtype != SEER_F32 && out_dtype != SEER_BF16)
    return fail(SEER_ERR_INVALID_ARG, "out_dtype %d is not SEER_F32/SEER_BF16", out_dtype);
  if (empty) return ok();
  if ((st = check_qkv(q, k, v)) != SEER_OK) return st;
  if ((st = check_out(out, out_dtype, lse)) != SEER_OK) return st;
  if (gt == nullptr || !aligned(gt, 4)) return fail(SEER_ERR_INVALID_ARG, "gt must be a non-NULL, 4-byte aligned device pointer");
  const size_t need = seer_gt_workspace_size(shape);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16))
    return fail(SEER_ERR_WORKSPACE, "workspace must be %zu bytes, 16-byte aligned (got %zu at %p)", need,
                workspace_bytes, workspace);
  if ((st = check_device()) != SEER_OK || !launch) return st;
  seer::AttnArgs a = attn_args(shape, q, k, v, 2);
  a.hs = hs;
  a.out = out;
  a.lse = lse;
  a.out_bf16 = out_dtype == SEER_BF16;
  a.rmax = static_cast<float*>(workspace);
  a.gt = gt;
  hipError_t e = seer::launch_attn(a, 2, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(SEER_ERR_HIP, "ground-truth attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

seer_status seer_attn_maxpool_gt(const seer_shape* shape, const void* q, const void* k, const void* v, void* out,
                                 seer_dtype out_dtype, float* lse, float* gt, void* workspace,
                                 size_t workspace_bytes, void* hip_stream) {
  return gt_impl(shape, shape ? shape->seq_len : 0, q, k, v, out, out_dtype, lse, gt, workspace, workspace_bytes,
                 hip_stream, true);
}

// ---------------------------------------------------------------------------
// Varlen (packed) batches: each sequence is a batch-1 problem at its token
// offset, with the packed length as the head stride; sequences run one after
// another on the stream and share the workspace. Every sequence is validated
// before anything is enqueued.
static seer_status check_varlen(const seer_varlen* vl, long long* total) {
  if (vl == nullptr) return fail(SEER_ERR_INVALID_ARG, "varlen descriptor is NULL");
  if (vl->num_seqs < 0) return fail(SEER_ERR_SHAPE, "num_seqs %d is negative", vl->num_seqs);
  if (vl->num_seqs > 0 && vl->cu_seqlens == nullptr) return fail(SEER_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if (vl->num_seqs > 0 && vl->cu_seqlens[0] != 0) return fail(SEER_ERR_SHAPE, "cu_seqlens[0] must be 0");
  for (int i = 0; i < vl->num_seqs; ++i)
    if (vl->cu_seqlens[i + 1] < vl->cu_seqlens[i])
      return fail(SEER_ERR_SHAPE, "cu_seqlens must be non-decreasing (entry %d)", i + 1);
  *total = vl->num_seqs > 0 ? vl->cu_seqlens[vl->num_seqs] : 0;
  return SEER_OK;
}

static seer_shape varlen_shape(const seer_varlen* vl, int i) {
  seer_shape s{};
  s.batch = 1;
  s.heads_q = vl->heads_q;
  s.heads_kv = vl->heads_kv;
  s.seq_len = vl->cu_seqlens[i + 1] - vl->cu_seqlens[i];
  s.head_dim = vl->head_dim;
  s.block = vl->block;
  return s;
}

// Sequences of a packed batch that share launches: non-empty, at most max_nb
// blocks, longest first (stable), cut into batches of kVarlenMaxSeqs.
static std::vector<int> varlen_shared(const seer_varlen* vl, long long max_nb) {
  std::vector<int> idx;
  for (int i = 0; i < vl->num_seqs; ++i) {
    const long long len = static_cast<long long>(vl->cu_seqlens[i + 1]) - vl->cu_seqlens[i];
    if (len > 0 && (len + kBlock - 1) / kBlock <= max_nb) idx.push_back(i);
  }
  std::stable_sort(idx.begin(), idx.end(), [vl](int a, int b) {
    return vl->cu_seqlens[a + 1] - vl->cu_seqlens[a] > vl->cu_seqlens[b + 1] - vl->cu_seqlens[b];
  });
  return idx;
}

// Element offset of each sequence's [Hq, nb_i, nb_i] block map.
static std::vector<long long> varlen_map_offsets(const seer_varlen* vl) {
  std::vector<long long> off(static_cast<size_t>(vl->num_seqs) + 1, 0);
  for (int i = 0; i < vl->num_seqs; ++i) {
    const long long nb = (static_cast<long long>(vl->cu_seqlens[i + 1]) - vl->cu_seqlens[i] + kBlock - 1) / kBlock;
    off[i + 1] = off[i] + static_cast<long long>(vl->heads_q) * nb * nb;
  }
  return off;
}

// Launch table of sequences idx[from .. from+n-1]; *rmax_floats receives the
// ground-truth scratch those sequences need (floats). False if the rows
// exceed the launch limit.
static bool varlen_table(const seer_varlen* vl, const std::vector<int>& idx, size_t from, int n,
                         const std::vector<long long>& moff, seer::VarlenTable* t, long long* rmax_floats) {
  long long rows = 0, rmax = 0;
  t->n = n;
  for (int k = 0; k < n; ++k) {
    const int i = idx[from + k];
    const long long len = static_cast<long long>(vl->cu_seqlens[i + 1]) - vl->cu_seqlens[i];
    const long long nb = (len + kBlock - 1) / kBlock;
    t->row_start[k] = static_cast<int>(rows);
    t->tok[k] = vl->cu_seqlens[i];
    t->len[k] = static_cast<int>(len);
    t->map_off[k] = moff[i];
    t->rmax_off[k] = rmax;
    rows += static_cast<long long>(vl->heads_q) * nb;
    rmax += static_cast<long long>(vl->heads_q) * (nb * (nb + 1) / 2) * kBlock;
    if (rows > 0x7fffffffLL) return false;
  }
  t->row_start[n] = static_cast<int>(rows);
  *rmax_floats = rmax;
  return true;
}

// Ground-truth scratch (bytes) of the largest shared launch of a packed batch.
static size_t varlen_gt_batch_bytes(const seer_varlen* vl) {
  const std::vector<int> idx = varlen_shared(vl, 1LL << 40);
  const std::vector<long long> moff = varlen_map_offsets(vl);
  size_t need = 0;
  for (size_t from = 0; from < idx.size(); from += seer::kVarlenMaxSeqs) {
    const int n = static_cast<int>(std::min<size_t>(seer::kVarlenMaxSeqs, idx.size() - from));
    seer::VarlenTable t{};
    long long rmax = 0;
    varlen_table(vl, idx, from, n, moff, &t, &rmax);
    need = std::max(need, align_up(static_cast<size_t>(rmax) * sizeof(float)));
  }
  return need;
}

// Runs of a packed batch whose gate shares launches: consecutive sequences of
// at most kGateVarlenMaxBlocks blocks and at most kGateVarlenMaxSeqs of them
// non-empty; a longer sequence is a run of its own on the batch-1 path.
struct GateRun {
  int first, end;     // sequences [first, end)
  bool single;        // one sequence on the batch-1 path
};

static long long varlen_nb(const seer_varlen* vl, int i) {
  return (static_cast<long long>(vl->cu_seqlens[i + 1]) - vl->cu_seqlens[i] + kBlock - 1) / kBlock;
}

static std::vector<GateRun> gate_runs(const seer_varlen* vl) {
  std::vector<GateRun> runs;
  int i = 0;
  while (i < vl->num_seqs) {
    const long long nb = varlen_nb(vl, i);
    if (nb == 0) { ++i; continue; }
    if (nb > seer::kGateVarlenMaxBlocks) { runs.push_back({i, i + 1, true}); ++i; continue; }
    int j = i, cnt = 0;
    while (j < vl->num_seqs && cnt < seer::kGateVarlenMaxSeqs) {
      const long long nj = varlen_nb(vl, j);
      if (nj > seer::kGateVarlenMaxBlocks) break;
      cnt += nj > 0;
      ++j;
    }
    runs.push_back({i, j, false});
    i = j;
  }
  return runs;
}

// Workspace of a shared run: each intermediate holds the run's sequences one
// after another (and, without a scores output, the logits maps).
static GateLayout gate_run_layout(const seer_varlen* vl, const GateRun& r, int dg, int wk_per_kv, bool want_scores) {
  size_t nbs = 0, nb2 = 0;
  for (int i = r.first; i < r.end; ++i) {
    const size_t nb = static_cast<size_t>(varlen_nb(vl, i));
    nbs += nb;
    nb2 += nb * nb;
  }
  const size_t Hq = vl->heads_q, Hkv = vl->heads_kv, D = vl->head_dim, hwk = wk_per_kv ? Hkv : Hq;
  GateLayout L{};
  size_t off = 0;
  L.qp = off; off += align_up(Hq * nbs * D * 4);
  L.kp = off; off += align_up(Hkv * nbs * 3 * D * 4);
  L.qg = off; off += align_up(Hq * nbs * dg * 4);
  L.kg = off; off += align_up(hwk * nbs * dg * 4);
  L.scores = off; off += want_scores ? 0 : align_up(Hq * nb2 * 4);
  L.total = off;
  return L;
}

static size_t gate_varlen_need(const seer_varlen* vl, int dg, int wk_per_kv, bool want_scores) {
  size_t need = 0;
  for (const GateRun& r : gate_runs(vl)) {
    size_t n;
    if (r.single) {
      const seer_shape s = varlen_shape(vl, r.first);
      n = gate_layout(&s, dg, wk_per_kv, want_scores).total;
    } else {
      n = gate_run_layout(vl, r, dg, wk_per_kv, want_scores).total;
    }
    need = std::max(need, n);
  }
  return need;
}

size_t seer_varlen_map_elements(const seer_varlen* vl) {
  long long total = 0;
  if (check_varlen(vl, &total) != SEER_OK) return 0;
  size_t n = 0;
  for (int i = 0; i < vl->num_seqs; ++i) {
    const size_t nb = (static_cast<size_t>(vl->cu_seqlens[i + 1] - vl->cu_seqlens[i]) + kBlock - 1) / kBlock;
    n += static_cast<size_t>(vl->heads_q > 0 ? vl->heads_q : 0) * nb * nb;
  }
  return n;
}

size_t seer_gate_varlen_workspace_size(const seer_varlen* vl, int32_t gate_dim, int32_t wk_per_kv_head,
                                       int32_t want_scores) {
  long long total = 0;
  if (check_varlen(vl, &total) != SEER_OK) return 0;
  size_t need = 0;
  for (int i = 0; i < vl->num_seqs; ++i) {     // every sequence's own requirement (its argument checks)
    const seer_shape s = varlen_shape(vl, i);
    const size_t n = seer_gate_workspace_size(&s, gate_dim, wk_per_kv_head, want_scores);
    need = n > need ? n : need;
  }
  return std::max(need, gate_varlen_need(vl, gate_dim, wk_per_kv_head != 0, want_scores != 0));
}

size_t seer_attn_varlen_workspace_size(const seer_varlen* vl) {
  long long total = 0;
  if (check_varlen(vl, &total) != SEER_OK) return 0;
  size_t need = 0;
  for (int i = 0; i < vl->num_seqs; ++i) {
    const seer_shape s = varlen_shape(vl, i);
    const size_t n = seer_attn_workspace_size(&s);
    need = n > need ? n : need;
  }
  return need;
}

size_t seer_gt_varlen_workspace_size(const seer_varlen* vl) {
  long long total = 0;
  if (check_varlen(vl, &total) != SEER_OK) return 0;
  return varlen_gt_batch_bytes(vl);
}

seer_status seer_gate_varlen_fwd(const seer_varlen* vl, int32_t gate_dim, int32_t wk_per_kv_head, float rope_theta,
                                 const void* q, const void* k, const float* w_q, const float* w_k,
                                 seer_mask_mode mode, float threshold, int32_t topk_k,
                                 const int32_t* topk_per_head, float* scores, uint8_t* block_mask, void* workspace,
                                 size_t workspace_bytes, void* hip_stream) {
  long long total = 0;
  seer_status st = check_varlen(vl, &total);
  if (st != SEER_OK) return st;
  const std::vector<long long> moff = varlen_map_offsets(vl);
  auto seq = [&](int i, bool launch) {
    const seer_shape s = varlen_shape(vl, i);
    const size_t t0 = static_cast<size_t>(vl->cu_seqlens[i]) * vl->head_dim;
    return gate_impl(&s, total, gate_dim, wk_per_kv_head, rope_theta,
                     q ? static_cast<const uint16_t*>(q) + t0 : nullptr,
                     k ? static_cast<const uint16_t*>(k) + t0 : nullptr, w_q, w_k, mode, threshold, topk_k,
                     topk_per_head, scores ? scores + moff[i] : nullptr, block_mask ? block_mask + moff[i] : nullptr,
                     workspace, workspace_bytes, hip_stream, launch);
  };
  const std::vector<GateRun> runs = gate_runs(vl);
  if (runs.empty()) return ok();
  const size_t need = gate_varlen_need(vl, gate_dim, wk_per_kv_head != 0, scores != nullptr);
  if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, kAlign))
    return fail(SEER_ERR_WORKSPACE, "workspace must be %zu bytes, 256-byte aligned (got %zu at %p)", need,
                workspace_bytes, workspace);
  // every sequence's arguments first, then the launches
  for (int i = 0; i < vl->num_seqs; ++i)
    if (vl->cu_seqlens[i + 1] > vl->cu_seqlens[i] && (st = seq(i, false)) != SEER_OK) return st;
  seer::TopkTable tk{};
  const seer_shape s0 = varlen_shape(vl, runs[0].first);
  if ((st = fill_topk(&s0, mode, topk_k, topk_per_head, &tk)) != SEER_OK) return st;
  for (const GateRun& r : runs) {
    if (r.single) {
      if ((st = seq(r.first, true)) != SEER_OK) return st;
      continue;
    }
    // the run in one launch per stage: the batch-1 arguments at its first
    // sequence, the intermediates of its sequences one after another
    const GateLayout L = gate_run_layout(vl, r, gate_dim, wk_per_kv_head != 0, scores != nullptr);
    seer::GateVarlenTable t{};
    int max_nb = 0;
    long long nbs = 0, pps = 0, lps = 0, nb2 = 0;
    t.n = r.end - r.first;
    for (int i = r.first; i < r.end; ++i) {
      const int k = i - r.first;
      const long long nb = varlen_nb(vl, i);
      const long long T = (nb + seer::kGateTile - 1) / seer::kGateTile;
      t.tokp[k] = vl->cu_seqlens[i] - vl->cu_seqlens[r.first];
      t.nbp[k] = static_cast<int>(nbs);
      t.pp[k] = static_cast<int>(pps);
      t.lp[k] = static_cast<int>(lps);
      t.mp[k] = nb2;
      nbs += nb;
      pps += T;
      lps += T * (T + 1) / 2 * vl->heads_q;
      nb2 += nb * nb;
      max_nb = std::max(max_nb, static_cast<int>(nb));
    }
    if (lps > 0x7fffffffLL || static_cast<long long>(vl->heads_q) * nbs > 0x7fffffffLL)
      return fail(SEER_ERR_UNSUPPORTED, "packed batch too large for one gate launch");
    t.tokp[t.n] = vl->cu_seqlens[r.end] - vl->cu_seqlens[r.first];
    t.nbp[t.n] = static_cast<int>(nbs);
    t.pp[t.n] = static_cast<int>(pps);
    t.lp[t.n] = static_cast<int>(lps);
    t.mp[t.n] = nb2;
    char* ws = static_cast<char*>(workspace);
    const size_t t0 = static_cast<size_t>(vl->cu_seqlens[r.first]) * vl->head_dim;
    seer::GateArgs a{};
    a.q = static_cast<const uint16_t*>(q) + t0;
    a.k = static_cast<const uint16_t*>(k) + t0;
    a.wq = w_q;
    a.wk = w_k;
    a.qp = reinterpret_cast<float*>(ws + L.qp);
    a.kp = reinterpret_cast<float*>(ws + L.kp);
    a.qg = reinterpret_cast<float*>(ws + L.qg);
    a.kg = reinterpret_cast<float*>(ws + L.kg);
    a.scores = scores ? scores + moff[r.first] : reinterpret_cast<float*>(ws + L.scores);
    a.mask = block_mask + moff[r.first];
    a.skip_scores = scores == nullptr;
    a.B = 1;
    a.Hq = vl->heads_q;
    a.Hkv = vl->heads_kv;
    a.hs = total;
    a.D = vl->head_dim;
    a.Dg = gate_dim;
    a.group = vl->heads_q / vl->heads_kv;
    a.wk_per_kv = wk_per_kv_head != 0;
    a.scale = static_cast<float>(1.0 / sqrt(static_cast<double>(vl->head_dim)));
    a.mode = mode == SEER_MASK_TOPK ? 1 : 0;
    a.threshold = threshold;
    a.rope_base = rope_theta > 0.f ? static_cast<double>(rope_theta) / vl->block : 0.0;
    const hipError_t e = seer::launch_gate_varlen(a, tk, t, max_nb, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(SEER_ERR_HIP, "varlen gate launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

seer_status seer_block_sparse_attn_varlen_fwd(const seer_varlen* vl, const void* q, const void* k, const void* v,
                                              const uint8_t* block_mask, void* out, seer_dtype out_dtype, float* lse,
                                              void* workspace, size_t workspace_bytes, void* hip_stream) {
  long long total = 0;
  seer_status st = check_varlen(vl, &total);
  if (st != SEER_OK) return st;
  const size_t esize = out_dtype == SEER_BF16 ? 2 : 4;
  // Sequences whose rows are one work item each (all of them in dense mode,
  // up to 1024 blocks in block-sparse mode) share launches; longer ones run
  // on their own (key-chunked or XCD-owned paths).
  const long long max_shared = block_mask != nullptr ? 1024 : (1LL << 40);
  const std::vector<int> shared = varlen_shared(vl, max_shared);
  const std::vector<long long> moff = varlen_map_offsets(vl);
  std::vector<char> is_shared(static_cast<size_t>(vl->num_seqs), 0);
  for (int i : shared) is_shared[i] = 1;
  for (int pass = 0; pass < 2; ++pass) {
    for (int i = 0; i < vl->num_seqs; ++i) {
      const seer_shape s = varlen_shape(vl, i);
      const size_t tok = static_cast<size_t>(vl->cu_seqlens[i]);
      const size_t t0 = tok * vl->head_dim;
      if (s.seq_len == 0 || (pass == 1 && is_shared[i])) continue;
      st = attn_impl(&s, total, q ? static_cast<const uint16_t*>(q) + t0 : nullptr,
                     k ? static_cast<const uint16_t*>(k) + t0 : nullptr,
                     v ? static_cast<const uint16_t*>(v) + t0 : nullptr, block_mask ? block_mask + moff[i] : nullptr,
                     out ? static_cast<char*>(out) + t0 * esize : nullptr, out_dtype, lse ? lse + tok : nullptr,
                     workspace, workspace_bytes, hip_stream, pass == 1);
      if (st != SEER_OK) return st;
    }
    for (size_t from = 0; from < shared.size(); from += seer::kVarlenMaxSeqs) {
      const int n = static_cast<int>(std::min<size_t>(seer::kVarlenMaxSeqs, shared.size() - from));
      seer::VarlenTable t{};
      long long rmax = 0;
      if (!varlen_table(vl, shared, from, n, moff, &t, &rmax))
        return fail(SEER_ERR_SHAPE, "the rows of a shared varlen launch exceed the launch limit");
      if (pass == 0) continue;
      const seer_shape s = varlen_shape(vl, shared[from]);
      seer::AttnArgs a = attn_args(&s, q, k, v, block_mask ? 0 : 1);
      a.hs = total;
      a.mask = block_mask;
      a.out = out;
      a.lse = lse;
      a.out_bf16 = out_dtype == SEER_BF16;
      a.chunk = seer::varlen_chunk_blocks();
      a.nchunk = 1;
      a.rotate = 1;
      hipError_t e = seer::launch_attn_varlen(a, t, block_mask ? 0 : 1, static_cast<hipStream_t>(hip_stream));
      if (e != hipSuccess) return fail(SEER_ERR_HIP, "varlen attention launch failed: %s", hipGetErrorString(e));
    }
  }
  return ok();
}

seer_status seer_attn_maxpool_gt_varlen(const seer_varlen* vl, const void* q, const void* k, const void* v,
                                        void* out, seer_dtype out_dtype, float* lse, float* gt, void* workspace,
                                        size_t workspace_bytes, void* hip_stream) {
  long long total = 0;
  seer_status st = check_varlen(vl, &total);
  if (st != SEER_OK) return st;
  const size_t esize = out_dtype == SEER_BF16 ? 2 : 4;
  const std::vector<long long> moff = varlen_map_offsets(vl);
  // every sequence is validated as the batch-1 call, then all run in shared launches
  for (int i = 0; i < vl->num_seqs; ++i) {
    const seer_shape s = varlen_shape(vl, i);
    const size_t tok = static_cast<size_t>(vl->cu_seqlens[i]);
    const size_t t0 = tok * vl->head_dim;
    if (s.seq_len == 0) continue;
    st = gt_impl(&s, total, q ? static_cast<const uint16_t*>(q) + t0 : nullptr,
                 k ? static_cast<const uint16_t*>(k) + t0 : nullptr, v ? static_cast<const uint16_t*>(v) + t0 : nullptr,
                 out ? static_cast<char*>(out) + t0 * esize : nullptr, out_dtype, lse ? lse + tok : nullptr,
                 gt ? gt + moff[i] : nullptr, workspace, workspace_bytes, hip_stream, false);
    if (st != SEER_OK) return st;
  }
  const size_t need = varlen_gt_batch_bytes(vl);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16)))
    return fail(SEER_ERR_WORKSPACE, "workspace must be %zu bytes, 16-byte aligned (got %zu at %p)", need,
                workspace_bytes, workspace);
  const std::vector<int> shared = varlen_shared(vl, 1LL << 40);
  for (size_t from = 0; from < shared.size(); from += seer::kVarlenMaxSeqs) {
    const int n = static_cast<int>(std::min<size_t>(seer::kVarlenMaxSeqs, shared.size() - from));
    seer::VarlenTable t{};
    long long rmax = 0;
    if (!varlen_table(vl, shared, from, n, moff, &t, &rmax))
      return fail(SEER_ERR_SHAPE, "the rows of a shared varlen launch exceed the launch limit");
  }
  for (size_t from = 0; from < shared.size(); from += seer::kVarlenMaxSeqs) {
    const int n = static_cast<int>(std::min<size_t>(seer::kVarlenMaxSeqs, shared.size() - from));
    seer::VarlenTable t{};
    long long rmax = 0;
    varlen_table(vl, shared, from, n, moff, &t, &rmax);
    const seer_shape s = varlen_shape(vl, shared[from]);
    seer::AttnArgs a = attn_args(&s, q, k, v, 2);
    a.hs = total;
    a.out = out;
    a.lse = lse;
    a.out_bf16 = out_dtype == SEER_BF16;
    a.rmax = static_cast<float*>(workspace);
    a.gt = gt;
    hipError_t e = seer::launch_attn_varlen(a, t, 2, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(SEER_ERR_HIP, "varlen ground-truth launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // extern "C"
