// Argument blocks and launchers of the attention kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace radix_launch {

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
  int num_segments;
  const int32_t *req_num_shared;
  int num_splits, parts, part_base;
  void *out;
  float *lse;
  float *ws_o, *ws_lse;
  int Hq, Hkv;
  float scale_log2;
};

hipError_t kv_store(const StoreArgs &a, int64_t T, hipStream_t stream);
// mode 0: decode private tail (split-KV), 1: extend (one block per token), 2: shared segment
hipError_t valu(bool bf16, int G, int mode, const AttnArgs &a, unsigned items, unsigned splits,
                hipStream_t s);
hipError_t mfma(int G, bool seg, const AttnArgs &a, int max_rows, unsigned items, hipStream_t s);
hipError_t combine(bool bf16, const AttnArgs &a, int batch, int Dv, hipStream_t s);

}  // namespace radix_launch
