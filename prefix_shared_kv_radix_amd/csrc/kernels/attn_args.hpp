// Argument blocks and launchers of the attention kernels (internal).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace radix_launch {

// Event pair that the next launch on this thread stamps with its own start and end
// (kernel timing); null when timing is off.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;
};
extern thread_local LaunchEvents g_launch_events;

template <typename... KArgs, typename... Args>
inline void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                   Args... args) {
  LaunchEvents &e = g_launch_events;
  if (e.start && !e.used) {
    e.used = true;
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e.start, e.stop, 0, args...);
  } else {
    kernel<<<grid, block, shmem, s>>>(args...);
  }
}

struct StoreArgs {
  const uint8_t *k_new, *v_new;
  const float *scale_new;
  uint8_t *k_pool, *v_pool;
  float *kv_scale;
  const int32_t *slots;      // mode 0
  const int32_t *new_slots;  // mode 1
  int32_t *rtt;
  int rtt_stride;
  const int32_t *req_rows;
  const int32_t *seq_lens;     // mode 1, 3
  const int32_t *prefix_lens;  // mode 2
  const int32_t *cu_extend;    // mode 2
  int batch;
  int k_row_bytes, v_row_bytes;  // multiples of 16
  int mode;  // 0 explicit slots, 1 decode append, 2 extend (slots from rows), 3 decode (slot from row)
};

struct AttnArgs {
  const void *q;
  const void *k_pool, *v_pool;
  const int32_t *rtt;
  int rtt_stride;
  const int32_t *req_rows;
  const int32_t *seq_lens, *private_start;                  // decode
  const int32_t *prefix_lens, *extend_lens, *cu_extend;     // extend
  int batch;
  const int32_t *seg_row, *seg_start, *seg_end, *seg_member_off, *seg_members, *seg_member_slot;
  // key chunks of segment s: seg_split_off[s] .. seg_split_off[s+1]-1; a member's partial
  // of chunk k of its segment is seg_member_part[entry] + k
  const int32_t *seg_split_off, *seg_member_part;
  // one record per chunk: {lo, hi, member offset, member count, row, segment, chunk, 0}
  const int32_t *seg_items;
  int num_segments;
  const int32_t *req_num_parts;   // segment partials of each request (NULL: none)
  int num_splits;   // private splits of each request at or past whole_reqs
  int whole_reqs;   // requests [0, whole_reqs) read their private keys as one part
  int split_chunk;  // keys per private split, when a request has num_splits > 1
  int parts, part_base;  // partial slots per (request, head); private ones start at part_base
  // decode: the new token's K/V (read directly for the last position and stored by the
  // tail kernel) and its slot (appended to the slot list); all NULL when already stored
  const void *k_new, *v_new;
  const int32_t *new_slots;
  int32_t *rtt_mut;
  // fp8 K/V: one fp32 scale per slot (K and V rows of every KV head) and the new token's
  float *kv_scale;
  const float *scale_new;
  void *out;
  float *lse;
  float *ws_o, *ws_lse;
  // bf16 decode: arrival counters [batch, Hkv] of the in-kernel merge (zero between calls)
  int32_t *merge_cnt;
  // bf16 private-tail kernel: work queue {next ticket, finished waves} (zero between calls)
  int32_t *tail_queue;
  int Hq, Hkv;
  float scale_log2;
};

struct MlaArgs {
  const uint16_t *q;       // [batch, 128, 576] bf16
  const void *kv;          // [slots, 576] bf16, or E4M3 bytes
  const float *kv_scale;   // [slots] (fp8)
  const int32_t *rtt;
  int rtt_stride;
  const int32_t *req_rows;
  const int32_t *seq_lens;
  const int32_t *req_order;  // [batch] or NULL: requests sharing a prefix are consecutive
  int batch, nsplit, split_chunk, parts;
  float *ws_o, *ws_lse;      // partials when nsplit > 1
  uint16_t *out;             // [batch, 128, 512] bf16 when nsplit == 1
  float *lse;
  float scale_log2;
  int fp8;
};

hipError_t kv_store(const StoreArgs &a, int64_t T, hipStream_t stream);
hipError_t mla(const MlaArgs &a, hipStream_t s);
// mode 0: decode private tail split -> partial, 1: extend (one block per token),
// 2: shared segment -> partial, 3: decode private tail -> final output (merges shared partials)
hipError_t valu(bool bf16, int G, int mode, const AttnArgs &a, unsigned items, unsigned splits,
                hipStream_t s);
// extend attention with bf16 MFMA tiles (128 or 256 query rows, chosen per batch, x 64-key
// tiles; total_rows = the batch's extend tokens x query heads per KV head); fp8: K/V bytes
// times their slot's scale, rounded to bf16 as the tiles are staged
hipError_t mfma(int G, bool fp8, const AttnArgs &a, int max_rows, unsigned items,
                int64_t total_rows, hipStream_t s);
// bf16 decode over the private keys of each request (split into `splits` chunks): output
// written directly, or partials merged in-kernel by the last producer (merge_cnt); fp8 K/V
// rows are converted exactly and their scale applied to the score and the probability
hipError_t decode_tail_bf16(int G, bool fp8, const AttnArgs &a, unsigned batch, unsigned splits,
                            hipStream_t s);
hipError_t combine(bool bf16, const AttnArgs &a, int batch, int Dv, hipStream_t s);
// one launch: shared-segment MFMA tiles + private-tail waves; the last producer of each
// (request, KV head) merges its partials (merge_cnt)
hipError_t decode_fused(int G, bool fp8, const AttnArgs &a, int max_rows, unsigned seg_items,
                        unsigned n_items, unsigned nsplit, hipStream_t s);

}  // namespace radix_launch
