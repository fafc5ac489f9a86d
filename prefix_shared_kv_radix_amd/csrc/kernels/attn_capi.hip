// C entry points of the device path: argument checks on the host, then
// kernel launches on the caller's stream. Nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>
#include <vector>

#include "attn_args.hpp"
#include "host/radix_host.hpp"
#include "radix_attn.h"

using radix::set_error;
using radix_launch::AttnArgs;
using radix_launch::StoreArgs;

namespace {

constexpr float kLog2e = 1.4426950408889634f;

#define REQUIRE(cond, msg) \
  do {                     \
    if (!(cond)) {         \
      set_error(msg);      \
      return RADIX_E_INVAL; \
    }                      \
  } while (0)

enum class Kind { None, GqaF32, GqaBf16, GqaFp8, MlaBf16, MlaFp8 };

Kind classify(const radix_attn_shape *s) {
  if (!s || s->num_kv_heads <= 0 || s->num_q_heads <= 0 || s->num_q_heads % s->num_kv_heads)
    return Kind::None;
  const int G = s->num_q_heads / s->num_kv_heads;
  const bool g_ok = G == 1 || G == 2 || G == 4 || G == 8;
  if (!s->v_is_k_prefix && g_ok) {
    if (s->q_dtype == RADIX_F32 && s->kv_dtype == RADIX_F32 && s->head_dim_qk == 64 &&
        s->head_dim_v == 64)
      return Kind::GqaF32;
    if (s->q_dtype == RADIX_BF16 && s->kv_dtype == RADIX_BF16 && s->head_dim_qk == 128 &&
        s->head_dim_v == 128)
      return Kind::GqaBf16;
    if (s->q_dtype == RADIX_BF16 && s->kv_dtype == RADIX_FP8_E4M3 && s->head_dim_qk == 128 &&
        s->head_dim_v == 128)
      return Kind::GqaFp8;
  }
  if (s->v_is_k_prefix && s->num_kv_heads == 1 && s->num_q_heads == 128 && s->head_dim_qk == 576 &&
      s->head_dim_v == 512 && s->q_dtype == RADIX_BF16) {
    if (s->kv_dtype == RADIX_BF16) return Kind::MlaBf16;
    if (s->kv_dtype == RADIX_FP8_E4M3) return Kind::MlaFp8;
  }
  return Kind::None;
}

int elem_bytes(int dtype) { return dtype == RADIX_F32 ? 4 : dtype == RADIX_BF16 ? 2 : 1; }

// GQA with bf16 queries (bf16 or fp8 K/V): matrix-core tiles, in-kernel merge
bool gqa_mfma(Kind k) { return k == Kind::GqaBf16 || k == Kind::GqaFp8; }

radix_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return RADIX_OK;
  set_error(std::string(what) + ": " + hipGetErrorString(e));
  return RADIX_E_HIP;
}

radix_status check_kv(const radix_attn_shape *s, const radix_kv_buffers *kv) {
  REQUIRE(kv && kv->k_pool && kv->num_slots > 0, "missing K/V pool");
  REQUIRE(s->v_is_k_prefix || kv->v_pool, "missing V pool");
  REQUIRE(s->kv_dtype != RADIX_FP8_E4M3 || kv->kv_scale, "fp8 pool needs per-token scales");
  return RADIX_OK;
}

StoreArgs store_args(const radix_attn_shape *s, const radix_kv_buffers *kv, const void *k_new,
                     const void *v_new, const float *scale_new) {
  StoreArgs a{};
  const int eb = elem_bytes(s->kv_dtype);
  a.k_new = static_cast<const uint8_t *>(k_new);
  a.v_new = s->v_is_k_prefix ? nullptr : static_cast<const uint8_t *>(v_new);
  a.scale_new = s->kv_dtype == RADIX_FP8_E4M3 ? scale_new : nullptr;
  a.k_pool = static_cast<uint8_t *>(kv->k_pool);
  a.v_pool = static_cast<uint8_t *>(kv->v_pool);
  a.kv_scale = kv->kv_scale;
  a.k_row_bytes = s->num_kv_heads * s->head_dim_qk * eb;
  a.v_row_bytes = s->num_kv_heads * s->head_dim_v * eb;
  return a;
}

AttnArgs attn_args(const radix_attn_shape *s, const radix_kv_buffers *kv, const void *q,
                   const int32_t *rtt, int32_t stride, const int32_t *rows, void *out,
                   float *lse) {
  AttnArgs a{};
  a.q = q;
  a.k_pool = kv->k_pool;
  a.v_pool = kv->v_pool;
  a.rtt = rtt;
  a.rtt_stride = stride;
  a.req_rows = rows;
  a.out = out;
  a.lse = lse;
  a.Hq = s->num_q_heads;
  a.Hkv = s->num_kv_heads;
  a.scale_log2 = s->sm_scale * kLog2e;
  a.num_splits = 1;
  a.whole_reqs = 0;
  a.kv_scale = kv->kv_scale;
  return a;
}

// ---------------------------------------------------------------- event timing
enum KernelId {
  K_STORE = 0,
  K_DECODE_TAIL = 1,
  K_EXTEND_VALU = 2,
  K_SEGMENT_VALU = 3,
  K_EXTEND_MFMA = 4,
  K_SEGMENT_MFMA = 5,
  K_COMBINE = 6,
  K_MLA_DECODE = 7,
  K_MLA_COMBINE = 8,
  K_DECODE_FUSED = 9,
  K_COUNT = 10
};
const char *const kKernelNames[K_COUNT] = {
    "kv_store", "decode_tail_valu", "extend_valu", "segment_valu", "extend_mfma",
    "segment_mfma", "combine", "mla_decode", "mla_combine", "decode_fused"};

struct Profiler {
  std::vector<hipEvent_t> ev;
  std::vector<int32_t> ids;
  int32_t cap = 0, used = 0;
};
Profiler g_prof;

}  // namespace

namespace radix_launch {
thread_local LaunchEvents g_launch_events;
}

namespace {

// Times the one launch made in its scope while timing is enabled: the launch carries
// the event pair, so the events hold the kernel's own start and end. A scope that
// launches nothing records both events itself (zero duration).
struct Timed {
  int32_t slot = -1;
  hipStream_t s;
  Timed(int32_t id, hipStream_t stream) : s(stream) {
    if (g_prof.used < g_prof.cap) {
      slot = g_prof.used++;
      g_prof.ids[slot] = id;
      radix_launch::g_launch_events = {g_prof.ev[2 * slot], g_prof.ev[2 * slot + 1], false};
    }
  }
  ~Timed() {
    if (slot < 0) return;
    if (!radix_launch::g_launch_events.used) {
      (void)hipEventRecord(g_prof.ev[2 * slot], s);
      (void)hipEventRecord(g_prof.ev[2 * slot + 1], s);
    }
    radix_launch::g_launch_events = {};
  }
};

// Launch-shape tuning (overridable at build time).
#ifndef RADIX_TAIL_CHUNK
#define RADIX_TAIL_CHUNK 768
#endif
#ifndef RADIX_TAIL_UNSPLIT
#define RADIX_TAIL_UNSPLIT 1024
#endif
#ifndef RADIX_TAIL_WAVES
#define RADIX_TAIL_WAVES 2048
#endif

// Private-tail chunking: one chunk per request when the tails are short (<= 1024 keys)
// and the batch alone gives ~2048 waves; otherwise 768-key chunks (more for very long
// tails), which the work-queue kernel spreads evenly over the GPU whatever the mix of
// request lengths.
constexpr int kTailChunk = RADIX_TAIL_CHUNK;
int auto_splits(int batch, int hkv, int private_len) {
  if (private_len <= RADIX_TAIL_UNSPLIT && batch * hkv >= RADIX_TAIL_WAVES) return 1;
  int s = (private_len + kTailChunk - 1) / kTailChunk;
  if (s > 64) s = 64;
  return s < 1 ? 1 : s;
}

// MLA: one block per request and key chunk, 4 waves; enough chunks for >= 256 blocks,
// at least 512 keys per chunk.
int mla_splits(int batch, int max_seq_len) {
  int s = (256 + batch - 1) / (batch > 0 ? batch : 1);
  const int cap = max_seq_len / 512 > 1 ? max_seq_len / 512 : 1;
  if (s > cap) s = cap;
  return s < 1 ? 1 : s;
}

int private_len_bound(int max_seq_len, const radix_decode_plan *plan) {
  const bool use_plan = plan && plan->num_segments > 0;
  const int p = max_seq_len - (use_plan ? plan->min_private_start : 0);
  return p < 1 ? 1 : p;
}

#ifndef RADIX_FUSED_LATE_PCT
#define RADIX_FUSED_LATE_PCT 10
#endif
#ifndef RADIX_FUSED_LATE_SPLITS
#define RADIX_FUSED_LATE_SPLITS 2
#endif

// How the private keys of a decode step are cut: requests [0, whole_reqs) in one part,
// the others in `splits` parts of equal length. A caller's num_splits applies to every
// request. Automatically, the bf16 step with a plan keeps short tails whole but cuts
// those of the last requests in launch order: their waves are the ones that start
// when the first waves finish, and whole tails there leave most of the GPU idle while
// the last few run.
struct TailCut {
  int splits, whole_reqs;
};
TailCut tail_cut(const radix_attn_shape *shape, int batch, int max_seq_len,
                 const radix_decode_plan *plan, int num_splits) {
  if (num_splits > 0) return {num_splits, num_splits == 1 ? batch : 0};
  const int plen = private_len_bound(max_seq_len, plan);
  const int s = auto_splits(batch, shape->num_kv_heads, plen);
  const bool fused = plan && plan->num_segments > 0 && gqa_mfma(classify(shape));
  const int late = batch * RADIX_FUSED_LATE_PCT / 100;
  if (s > 1 || !fused || late == 0 || RADIX_FUSED_LATE_SPLITS < 2 ||
      plen < 32 * RADIX_FUSED_LATE_SPLITS)
    return {s, s == 1 ? batch : 0};
  return {RADIX_FUSED_LATE_SPLITS, batch - late};
}

// True if the kernels may read p: device memory, or host memory pinned and mapped into
// the device's address space at the same address (a pageable pointer would fault).
bool device_readable(const void *p) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();   // clear the sticky error of the failed query
    return false;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) return true;
  return at.type == hipMemoryTypeHost && at.devicePointer == p;
}

// bf16 decode workspace: counters at a fixed place (the first 256 KiB), so a workspace
// reused by calls of other shapes never finds partial data where counters are expected:
// the in-kernel merge's arrival counters (one int32 per (request, KV head)), then the
// private-tail kernel's work queue (16 counters, 128 bytes apart) in the last 2 KiB;
// partials follow.
constexpr int64_t kCounterInts = 1 << 16;
constexpr size_t kMergeCounterBytes = kCounterInts * sizeof(int32_t);
constexpr int64_t kQueueInts = 512;
constexpr int64_t kMergeCounters = kCounterInts - kQueueInts;

// partial outputs [batch, Hq, parts, Dv] and their lse [batch, Hq, parts], fp32, rounded
// up to 256 bytes
size_t partials_bytes(const radix_attn_shape *shape, int32_t batch, size_t parts) {
  const size_t b = static_cast<size_t>(batch) * shape->num_q_heads * parts *
                   (static_cast<size_t>(shape->head_dim_v) + 1) * sizeof(float);
  return (b + 255) / 256 * 256;
}

// ---------------------------------------------------------------- no-allocation decode
// Scratch of radix_attn_decode_noalloc: a device array of the library itself, so that
// callers that cannot allocate device memory (code under graph capture, serving loops
// that forbid it) need no workspace. Each device holds its own copy for the life of the
// process. In host code `scratch` names a host-side stand-in; the kernels get the
// device address that hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void zero_words_kernel(uint32_t *p, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    p[i] = 0u;
}

// Streaming read of n16 16-byte words, eight non-temporal loads in flight per lane (the
// fastest simple read pattern measured: ≈ 6.2 TB/s, against ≈ 5.4 with default-policy
// loads); the XOR of everything read reaches memory only if it equals a fixed constant,
// so the loads stay.
constexpr unsigned kProbeBlocks = 8192;
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4 *p, int64_t n16,
                                                         uint32_t *sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      typedef unsigned u4 __attribute__((ext_vector_type(4)));
      const u4 w = __builtin_nontemporal_load(reinterpret_cast<const u4 *>(p + i + k * stride));
      v[k] = uint4{w[0], w[1], w[2], w[3]};
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch. The first call on a device looks it up and
// clears the merge-counter region with a fill kernel on `s` (ordered before the call's
// decode launch); the decode kernels leave that region zero after every call.
radix_status scratch_for_current_device(hipStream_t s, void **out) {
  int dev = 0;
  radix_status st = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (st != RADIX_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device index above the scratch table");
    return RADIX_E_INVAL;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (st != RADIX_OK) return st;
    const int64_t words = static_cast<int64_t>(kMergeCounterBytes / sizeof(uint32_t));
    zero_words_kernel<<<dim3(64), dim3(256), 0, s>>>(static_cast<uint32_t *>(p), words);
    st = hip_status(hipGetLastError(), "scratch clear launch");
    if (st != RADIX_OK) return st;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RADIX_OK;
}

}  // namespace

extern "C" {



radix_status radix_attn_supported(const radix_attn_shape *shape, int is_decode) {
  Kind k = classify(shape);
  if (k == Kind::None) {
    set_error("unsupported attention shape/dtype combination");
    return RADIX_E_UNSUPPORTED;
  }
  if (!is_decode && (k == Kind::MlaBf16 || k == Kind::MlaFp8)) {
    set_error("MLA extend is not part of this library");
    return RADIX_E_UNSUPPORTED;
  }
  return RADIX_OK;
}

radix_status radix_kv_store(const radix_attn_shape *shape, const radix_kv_buffers *kv,
                            const void *k_new, const void *v_new, const float *scale_new,
                            const int32_t *slots, int64_t num_tokens, void *stream) {
  if (radix_attn_supported(shape, 1) != RADIX_OK) return RADIX_E_UNSUPPORTED;
  radix_status st = check_kv(shape, kv);
  if (st != RADIX_OK) return st;
  REQUIRE(num_tokens >= 0 && num_tokens <= 0x7fffffff, "token count out of range");
  if (num_tokens == 0) return RADIX_OK;
  REQUIRE(k_new && slots, "missing new rows or slots");
  REQUIRE(shape->v_is_k_prefix || v_new, "missing new V rows");
  REQUIRE(shape->kv_dtype != RADIX_FP8_E4M3 || scale_new, "missing new fp8 scales");
  StoreArgs a = store_args(shape, kv, k_new, v_new, scale_new);
  a.slots = slots;
  a.mode = 0;
  Timed t(K_STORE, static_cast<hipStream_t>(stream));
  return hip_status(radix_launch::kv_store(a, num_tokens, static_cast<hipStream_t>(stream)),
                    "kv_store launch");
}

radix_status radix_attn_decode_workspace_size(const radix_attn_shape *shape, int32_t batch,
                                              int32_t max_seq_len,
                                              const radix_decode_plan *plan,
                                              int32_t num_splits, size_t *bytes) {
  REQUIRE(shape && bytes && batch >= 0 && max_seq_len >= 0 && num_splits >= 0,
          "bad workspace query");
  if (shape->v_is_k_prefix) {  // MLA: partials only when a request's keys are split
    const int ns = num_splits > 0 ? num_splits : mla_splits(batch, max_seq_len);
    *bytes = ns == 1 ? 0
                     : static_cast<size_t>(batch) * shape->num_q_heads * ns *
                           (static_cast<size_t>(shape->head_dim_v) + 1) * sizeof(float);
    return RADIX_OK;
  }
  num_splits = tail_cut(shape, batch, max_seq_len, plan, num_splits).splits;
  const bool use_plan = plan && plan->num_segments > 0;
  const size_t shared = use_plan ? static_cast<size_t>(plan->max_parts) : 0;
  const size_t parts = shared + static_cast<size_t>(num_splits);
  const bool bf16 = shape->q_dtype == RADIX_BF16;
  if (!use_plan && num_splits == 1) {
    // single pass, nothing to merge (bf16: the counter region still holds the work queue)
    *bytes = bf16 ? kMergeCounterBytes : 0;
    return RADIX_OK;
  }
  // bf16: the counters occupy a fixed region in front
  *bytes = (bf16 ? kMergeCounterBytes : 0) + partials_bytes(shape, batch, parts);
  return RADIX_OK;
}

radix_status radix_attn_extend(const radix_attn_shape *shape, const radix_kv_buffers *kv,
                               const void *q, const void *k_new, const void *v_new,
                               const float *scale_new, const int32_t *req_to_token,
                               int32_t rtt_stride, const int32_t *req_rows,
                               const int32_t *prefix_lens, const int32_t *extend_lens,
                               const int32_t *cu_extend, int32_t batch, int32_t total_extend,
                               int32_t max_extend, void *out, float *lse_out, void *stream) {
  if (radix_attn_supported(shape, 0) != RADIX_OK) return RADIX_E_UNSUPPORTED;
  radix_status st = check_kv(shape, kv);
  if (st != RADIX_OK) return st;
  REQUIRE(batch >= 0 && total_extend >= 0 && max_extend >= 0, "negative sizes");
  if (batch == 0 || total_extend == 0) return RADIX_OK;
  REQUIRE(q && out && req_to_token && rtt_stride > 0 && prefix_lens && extend_lens && cu_extend,
          "missing extend argument");
  REQUIRE(max_extend <= total_extend, "max_extend exceeds total_extend");
  REQUIRE(!k_new || shape->v_is_k_prefix || v_new, "missing new V rows");
  REQUIRE(!k_new || shape->kv_dtype != RADIX_FP8_E4M3 || scale_new, "missing new fp8 scales");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (k_new) {
    StoreArgs sa = store_args(shape, kv, k_new, v_new, scale_new);
    sa.rtt = const_cast<int32_t *>(req_to_token);
    sa.rtt_stride = rtt_stride;
    sa.req_rows = req_rows;
    sa.prefix_lens = prefix_lens;
    sa.cu_extend = cu_extend;
    sa.batch = batch;
    sa.mode = 2;
    Timed t(K_STORE, s);
    st = hip_status(radix_launch::kv_store(sa, total_extend, s), "kv_store launch");
    if (st != RADIX_OK) return st;
  }
  AttnArgs a = attn_args(shape, kv, q, req_to_token, rtt_stride, req_rows, out, lse_out);
  a.prefix_lens = prefix_lens;
  a.extend_lens = extend_lens;
  a.cu_extend = cu_extend;
  a.batch = batch;
  a.num_splits = 1;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  const Kind kind = classify(shape);
  if (gqa_mfma(kind)) {
    Timed t(K_EXTEND_MFMA, s);
    return hip_status(radix_launch::mfma(G, kind == Kind::GqaFp8, a, max_extend * G, batch,
                                         static_cast<int64_t>(total_extend) * G, s),
                      "extend launch");
  }
  Timed t(K_EXTEND_VALU, s);
  return hip_status(radix_launch::valu(false, G, 1, a, total_extend, 1, s), "extend launch");
}

radix_status radix_attn_decode(const radix_attn_shape *shape, const radix_kv_buffers *kv,
                               const void *q, const void *k_new, const void *v_new,
                               const float *scale_new, const int32_t *new_slots,
                               int32_t *req_to_token, int32_t rtt_stride,
                               const int32_t *req_rows, const int32_t *seq_lens, int32_t batch,
                               int32_t max_seq_len, const radix_decode_plan *plan,
                               int32_t num_splits, void *out, float *lse_out, void *workspace,
                               size_t workspace_bytes, void *stream) {
  if (radix_attn_supported(shape, 1) != RADIX_OK) return RADIX_E_UNSUPPORTED;
  radix_status st = check_kv(shape, kv);
  if (st != RADIX_OK) return st;
  REQUIRE(batch >= 0 && max_seq_len >= 0 && num_splits >= 0, "negative sizes");
  if (batch == 0) return RADIX_OK;
  REQUIRE(q && out && req_to_token && rtt_stride > 0 && seq_lens, "missing decode argument");
  REQUIRE(max_seq_len >= 1 && max_seq_len <= rtt_stride, "max_seq_len outside [1, rtt_stride]");
  REQUIRE(!k_new || shape->v_is_k_prefix || v_new, "missing new V rows");
  REQUIRE(!k_new || shape->kv_dtype != RADIX_FP8_E4M3 || scale_new, "missing new fp8 scales");
  REQUIRE(!new_slots || device_readable(new_slots),
          "new_slots must be device memory or pinned (device-mapped) host memory");
  const bool use_plan = plan && plan->num_segments > 0;
  if (use_plan) {
    REQUIRE(plan->seg_row && plan->seg_start && plan->seg_end && plan->seg_member_off &&
                plan->seg_members && plan->seg_member_slot && plan->seg_split_off &&
                plan->seg_member_part && plan->seg_items && plan->req_num_shared &&
                plan->req_num_parts &&
                plan->req_private_start && plan->num_member_entries > 0 &&
                plan->max_members > 0 && plan->max_shared > 0 &&
                plan->num_seg_items >= plan->num_segments && plan->max_parts >= plan->max_shared &&
                plan->max_seg_splits > 0,
            "incomplete decode plan");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Kind kind = classify(shape);
  if (kind == Kind::MlaBf16 || kind == Kind::MlaFp8) {
    const int nsplit = num_splits > 0 ? num_splits : mla_splits(batch, max_seq_len);
    size_t need = 0;
    radix_attn_decode_workspace_size(shape, batch, max_seq_len, plan, nsplit, &need);
    REQUIRE(nsplit == 1 || (workspace && workspace_bytes >= need), "decode workspace too small");
    REQUIRE(!use_plan || plan->req_order, "decode plan without req_order");
    if (k_new) {  // the MLA kernel reads every key from the pool: store the new row first
      StoreArgs sa = store_args(shape, kv, k_new, v_new, scale_new);
      sa.new_slots = new_slots;
      sa.rtt = req_to_token;
      sa.rtt_stride = rtt_stride;
      sa.req_rows = req_rows;
      sa.seq_lens = seq_lens;
      sa.mode = new_slots ? 1 : 3;
      Timed t(K_STORE, s);
      st = hip_status(radix_launch::kv_store(sa, batch, s), "kv_store launch");
      if (st != RADIX_OK) return st;
    }
    radix_launch::MlaArgs m{};
    m.q = static_cast<const uint16_t *>(q);
    m.kv = kv->k_pool;
    m.kv_scale = kv->kv_scale;
    m.rtt = req_to_token;
    m.rtt_stride = rtt_stride;
    m.req_rows = req_rows;
    m.seq_lens = seq_lens;
    m.req_order = use_plan ? plan->req_order : nullptr;
    m.batch = batch;
    m.nsplit = nsplit;
    m.split_chunk = ((max_seq_len + nsplit - 1) / nsplit + 31) / 32 * 32;
    m.parts = nsplit;
    m.ws_o = nsplit > 1 ? static_cast<float *>(workspace) : nullptr;
    m.ws_lse = nsplit > 1 ? m.ws_o + static_cast<size_t>(batch) * shape->num_q_heads * nsplit *
                                         shape->head_dim_v
                          : nullptr;
    m.out = static_cast<uint16_t *>(out);
    m.lse = lse_out;
    m.scale_log2 = shape->sm_scale * kLog2e;
    m.fp8 = kind == Kind::MlaFp8;
    {
      Timed t(K_MLA_DECODE, s);
      st = hip_status(radix_launch::mla(m, s), "mla launch");
    }
    if (st != RADIX_OK || nsplit == 1) return st;
    AttnArgs c = attn_args(shape, kv, q, req_to_token, rtt_stride, req_rows, out, lse_out);
    c.num_splits = nsplit;
    c.parts = nsplit;
    c.part_base = 0;
    c.ws_o = m.ws_o;
    c.ws_lse = m.ws_lse;
    Timed t(K_MLA_COMBINE, s);
    return hip_status(radix_launch::combine(true, c, batch, shape->head_dim_v, s), "combine launch");
  }

  const TailCut cut = tail_cut(shape, batch, max_seq_len, use_plan ? plan : nullptr, num_splits);
  const int splits = cut.splits;
  const int max_shared = use_plan ? plan->max_parts : 0;   // segment partials per request
  const int parts = max_shared + splits;
  const bool direct = !use_plan && splits == 1;
  size_t need = 0;
  radix_attn_decode_workspace_size(shape, batch, max_seq_len, plan, splits, &need);
  REQUIRE((direct && !gqa_mfma(kind)) || (workspace && workspace_bytes >= need),
          "decode workspace too small");
  REQUIRE(direct || !gqa_mfma(kind) ||
              static_cast<int64_t>(batch) * shape->num_kv_heads <= kMergeCounters,
          "batch * num_kv_heads above the merge counter capacity (65024)");
  char *ws_parts = static_cast<char *>(workspace) + (gqa_mfma(kind) ? kMergeCounterBytes : 0);
  float *ws_o = direct ? nullptr : reinterpret_cast<float *>(ws_parts);
  float *ws_lse = direct ? nullptr
                         : ws_o + static_cast<size_t>(batch) * shape->num_q_heads * parts *
                                      shape->head_dim_v;

  AttnArgs a = attn_args(shape, kv, q, req_to_token, rtt_stride, req_rows, out, lse_out);
  a.seq_lens = seq_lens;
  a.num_splits = splits;
  a.whole_reqs = cut.whole_reqs;
  {
    const int plen = private_len_bound(max_seq_len, use_plan ? plan : nullptr);
    a.split_chunk = ((plen + splits - 1) / splits + 15) & ~15;
  }
  a.parts = parts;
  a.part_base = max_shared;
  a.ws_o = ws_o;
  a.ws_lse = ws_lse;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_slots = new_slots;
  a.rtt_mut = req_to_token;
  a.scale_new = scale_new;
  const bool bf16 = gqa_mfma(kind);
  const bool fp8 = kind == Kind::GqaFp8;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  if (use_plan) {
    a.seg_row = plan->seg_row;
    a.seg_start = plan->seg_start;
    a.seg_end = plan->seg_end;
    a.seg_member_off = plan->seg_member_off;
    a.seg_members = plan->seg_members;
    a.seg_member_slot = plan->seg_member_slot;
    a.seg_split_off = plan->seg_split_off;
    a.seg_member_part = plan->seg_member_part;
    a.seg_items = plan->seg_items;
    a.num_segments = plan->num_segments;
    a.req_num_parts = plan->req_num_parts;
    a.private_start = plan->req_private_start;
  }
  if (bf16) {
    // one launch per step: partials are merged in-kernel by their last producer
    a.merge_cnt = direct ? nullptr : static_cast<int32_t *>(workspace);
    a.tail_queue = static_cast<int32_t *>(workspace) + kMergeCounters;
    Timed t(use_plan ? K_DECODE_FUSED : K_DECODE_TAIL, s);
    if (use_plan)
      return hip_status(radix_launch::decode_fused(
                            G, fp8, a, plan->max_members * G,
                            static_cast<unsigned>(plan->num_seg_items),
                            static_cast<unsigned>(batch), static_cast<unsigned>(splits), s),
                        "decode launch");
    return hip_status(radix_launch::decode_tail_bf16(G, fp8, a, static_cast<unsigned>(batch),
                                                     static_cast<unsigned>(splits), s),
                      "decode launch");
  }
  if (use_plan) {
    Timed t(K_SEGMENT_VALU, s);
    st = hip_status(radix_launch::valu(false, G, 2, a, plan->num_member_entries,
                                                       plan->max_seg_splits, s),
                    "segment launch");
    if (st != RADIX_OK) return st;
  }
  if (splits == 1) {
    Timed t(K_DECODE_TAIL, s);
    return hip_status(radix_launch::valu(false, G, 3, a, batch, 1, s), "decode launch");
  }
  {
    Timed t(K_DECODE_TAIL, s);
    st = hip_status(radix_launch::valu(false, G, 0, a, batch, splits, s), "decode launch");
  }
  if (st != RADIX_OK) return st;
  Timed t(K_COMBINE, s);
  return hip_status(radix_launch::combine(false, a, batch, shape->head_dim_v, s), "combine launch");
}

radix_status radix_attn_decode_noalloc(const radix_attn_shape *shape, const radix_kv_buffers *kv,
                                       const void *q, const void *k_new, const void *v_new,
                                       const float *scale_new, const int32_t *new_slots,
                                       int32_t *req_to_token, int32_t rtt_stride,
                                       const int32_t *req_rows, const int32_t *seq_lens,
                                       int32_t batch, int32_t max_seq_len,
                                       const radix_decode_plan *plan, int32_t num_splits,
                                       void *out, float *lse_out, void *stream) {
  if (radix_attn_supported(shape, 1) != RADIX_OK) return RADIX_E_UNSUPPORTED;
  REQUIRE(batch >= 0 && max_seq_len >= 0 && num_splits >= 0, "negative sizes");
  if (batch == 0) return RADIX_OK;
  size_t need = 0;
  radix_status st = radix_attn_decode_workspace_size(shape, batch, max_seq_len, plan, num_splits,
                                                     &need);
  if (st != RADIX_OK) return st;
  if (need > kScratchBytes) {
    set_error("decode needs " + std::to_string(need) + " bytes of scratch, more than the " +
              std::to_string(kScratchBytes) + " built into the library");
    return RADIX_E_INVAL;
  }
  void *ws = nullptr;
  st = scratch_for_current_device(static_cast<hipStream_t>(stream), &ws);
  if (st != RADIX_OK) return st;
  return radix_attn_decode(shape, kv, q, k_new, v_new, scale_new, new_slots, req_to_token,
                           rtt_stride, req_rows, seq_lens, batch, max_seq_len, plan, num_splits,
                           out, lse_out, ws, kScratchBytes, stream);
}

size_t radix_attn_decode_noalloc_max_bytes(void) { return kScratchBytes; }

radix_status radix_probe_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream) {
  REQUIRE(buf && sink, "read probe: missing buffer or sink");
  REQUIRE(bytes > 0 && bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(buf) & 15) == 0,
          "read probe: buffer must be 16-byte aligned, a positive multiple of 16 bytes");
  read_probe_kernel<<<dim3(kProbeBlocks), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4 *>(buf), bytes / 16, sink);
  return hip_status(hipGetLastError(), "read probe launch");
}

radix_status radix_fence_create(radix_fence **out) {
  REQUIRE(out, "null output pointer");
  hipEvent_t e = nullptr;
  radix_status st = hip_status(
      hipEventCreateWithFlags(&e, hipEventDisableTiming | hipEventDisableSystemFence),
      "hipEventCreateWithFlags");
  if (st != RADIX_OK) return st;
  *out = reinterpret_cast<radix_fence *>(e);
  return RADIX_OK;
}

radix_status radix_fence_record(radix_fence *fence, void *stream) {
  REQUIRE(fence, "null fence");
  return hip_status(hipEventRecord(reinterpret_cast<hipEvent_t>(fence),
                                   static_cast<hipStream_t>(stream)),
                    "hipEventRecord");
}

radix_status radix_fence_wait(radix_fence *fence) {
  REQUIRE(fence, "null fence");
  return hip_status(hipEventSynchronize(reinterpret_cast<hipEvent_t>(fence)), "hipEventSynchronize");
}

void radix_fence_destroy(radix_fence *fence) {
  if (fence) (void)hipEventDestroy(reinterpret_cast<hipEvent_t>(fence));
}

radix_status radix_profile_enable(int32_t capacity) {
  REQUIRE(capacity >= 0, "negative profiling capacity");
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.ids.assign(capacity, 0);
  g_prof.cap = 0;
  g_prof.used = 0;
  for (int32_t i = 0; i < 2 * capacity; ++i) {
    hipEvent_t e;
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) {
      for (hipEvent_t x : g_prof.ev) (void)hipEventDestroy(x);
      g_prof.ev.clear();
      return hip_status(err, "hipEventCreate");
    }
    g_prof.ev.push_back(e);
  }
  g_prof.cap = capacity;
  return RADIX_OK;
}

radix_status radix_profile_read(int32_t *kernel_ids, float *ms, int32_t cap, int32_t *count) {
  REQUIRE(count && cap >= 0 && (cap == 0 || (kernel_ids && ms)), "bad profiling read");
  const int32_t n = g_prof.used < cap ? g_prof.used : cap;
  for (int32_t i = 0; i < n; ++i) {
    hipError_t err = hipEventSynchronize(g_prof.ev[2 * i + 1]);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms[i], g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
    if (err != hipSuccess) return hip_status(err, "event timing");
    kernel_ids[i] = g_prof.ids[i];
  }
  *count = n;
  g_prof.used = 0;
  return RADIX_OK;
}

const char *radix_kernel_name(int32_t kernel_id) {
  return (kernel_id >= 0 && kernel_id < K_COUNT) ? kKernelNames[kernel_id] : "";
}

}  // extern "C"
