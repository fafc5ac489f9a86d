/*
 * radix_attn.h — C ABI of the radix-shared KV attention library (MI355X / gfx950).
 *
 * What it computes. Requests share K/V through a radix tree of token
 * sequences: every edge holds a run of tokens plus the K/V slots of those
 * tokens, lookups match token by token and split an edge where requests
 * diverge, running requests pin their path with reference counts, and the
 * least recently used unpinned leaves are evicted first when the one slot
 * pool shared by cache and running requests runs short
 * (page "49 · RadixAttention, eviction và cache churn", §2 and §4; SGLang
 * overview, "SGLang: Mô Hình Lập Trình và Phương Pháp", RadixAttention).
 * Attention reads each request's keys through its per-request slot list
 * (req_to_token), both for extend (all new prompt tokens at once against
 * the cached prefix) and for decode (one new token per request per step)
 * (AWS blog "Improve performance of Falcon models with Amazon SageMaker",
 * sections on the KV cache and on batching).
 *
 * Conventions for every call:
 *  - No exception or abort crosses this ABI. Every call that can fail returns
 *    a radix_status; radix_last_error() gives a thread-local message.
 *  - RADIX_E_INVAL: a bad argument; nothing launched and no state changed.
 *  - RADIX_E_NOMEM: not enough free + evictable slots; no state changed.
 *  - Host objects (pool, tree) are owned by the library (create/destroy) and
 *    are thread-compatible: one thread at a time per object.
 *  - Device buffers (pools, queries, outputs, slot lists, workspaces) are owned
 *    by the caller. The library keeps no device pointer past a call and never
 *    allocates device memory in attention calls. Device work is enqueued on
 *    the caller's stream and is asynchronous; host calls are synchronous.
 *  - Slots are int32 indices into the caller's K/V pool rows.
 */
#ifndef RADIX_ATTN_H
#define RADIX_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RADIX_OK = 0,
  RADIX_E_INVAL = 1,
  RADIX_E_NOMEM = 2,
  RADIX_E_HIP = 3,
  RADIX_E_UNSUPPORTED = 4
} radix_status;

typedef enum {
  RADIX_F32 = 0,
  RADIX_BF16 = 1,
  RADIX_FP8_E4M3 = 2 /* OCP E4M3FN byte, one fp32 scale per token row */
} radix_dtype;

/* Thread-local text describing the last non-OK status returned on this thread. */
const char *radix_last_error(void);

/* Library version string. */
const char *radix_version(void);

/* ======================================================================
 * Slot pool (host). One pool serves cached and running requests alike
 * (page 4 §4). The free list is FIFO and starts as 0..num_slots-1.
 * ====================================================================== */
typedef struct radix_kv_pool radix_kv_pool;

/* num_slots >= 0. *out receives the new pool. */
radix_status radix_kv_pool_create(int64_t num_slots, radix_kv_pool **out);
/* Releases the caller's handle (NULL: no-op). The pool's memory lives on while any tree
 * created on it is alive and is freed with the last of them, so pool and trees may be
 * destroyed in either order; the handle must not be used after this call. */
void radix_kv_pool_destroy(radix_kv_pool *pool);
/* Take n slots from the head of the free list into out_slots[n]. All or nothing:
 * RADIX_E_NOMEM if fewer than n are free. */
radix_status radix_kv_pool_alloc(radix_kv_pool *pool, int64_t n, int32_t *out_slots);
/* Append slots[n] to the tail of the free list in the given order. RADIX_E_INVAL
 * (nothing freed) on an index out of range, a slot already free, or a repeat. */
radix_status radix_kv_pool_free(radix_kv_pool *pool, const int32_t *slots, int64_t n);
int64_t radix_kv_pool_num_free(const radix_kv_pool *pool);
int64_t radix_kv_pool_num_slots(const radix_kv_pool *pool);
/* Copy the free list, head first, into out[cap]; *n receives its length.
 * RADIX_E_INVAL if cap is too small (nothing copied, *n still set). */
radix_status radix_kv_pool_free_list(const radix_kv_pool *pool, int32_t *out, int64_t cap,
                                     int64_t *n);

/* ======================================================================
 * Radix tree over int32 token ids (host) — page 4 §2, §4, §5.
 * A node handle (radix_node) stays valid while the node is pinned.
 * The tree keeps a logical clock that advances once per match and insert;
 * least recently used means smallest clock value, ties broken by the
 * lexicographically smaller root-to-node token path.
 * ====================================================================== */
typedef struct radix_tree radix_tree;
typedef int64_t radix_node; /* 0 = root */

/* The tree draws slots from (and returns them to) `pool` and keeps the pool's memory
 * alive until the tree is destroyed (see radix_kv_pool_destroy). */
radix_status radix_tree_create(radix_kv_pool *pool, radix_tree **out);
/* Destroys the tree (NULL: no-op) and returns every cached slot to the pool, then
 * drops the tree's hold on the pool (freeing it if its handle was destroyed already). */
void radix_tree_destroy(radix_tree *tree);

/* Length of the longest cached prefix of tok[n]; changes nothing (the match may end
 * inside an edge). Used for longest-prefix-first ordering. */
radix_status radix_tree_peek(const radix_tree *tree, const int32_t *tok, int64_t n,
                             int64_t *matched);
/* Longest cached prefix of tok[n], walking token by token; an edge matched only
 * partly is split so the match ends on a node. Refreshes the clock of every node on
 * the matched path. out_slots[n] receives the *matched slots; *last the deepest
 * matched node (root if none). */
radix_status radix_tree_match(radix_tree *tree, const int32_t *tok, int64_t n, int64_t *matched,
                              int32_t *out_slots, radix_node *last);
/* Pin (+1) / unpin (-1) a node and all its ancestors. Pinned nodes are never evicted.
 * RADIX_E_INVAL on a stale handle or an unpin below zero. */
radix_status radix_tree_lock(radix_tree *tree, radix_node node);
radix_status radix_tree_unlock(radix_tree *tree, radix_node node);
/* Take n slots from the pool, evicting unpinned leaves least recently used first
 * (whole nodes; a node whose children are all gone becomes a candidate) until enough
 * are free. All or nothing: RADIX_E_NOMEM if free + evictable < n. */
radix_status radix_tree_alloc(radix_tree *tree, int64_t n, int32_t *out_slots);
/* Insert a finished sequence tok[n] whose K/V live in slots[n] (page 4 §2: the whole
 * path, outputs included, stays). Tokens already cached keep the tree's slots;
 * *already_cached receives how many leading tokens were cached before the call. The
 * tree adopts slots[*already_cached:n]; the caller still owns the rest. */
radix_status radix_tree_insert(radix_tree *tree, const int32_t *tok, const int32_t *slots,
                               int64_t n, int64_t *already_cached);
/* Evict unpinned leaves (LRU first) until at least n_tokens slots are freed or
 * nothing is evictable; *freed receives the count. */
radix_status radix_tree_evict(radix_tree *tree, int64_t n_tokens, int64_t *freed);

typedef struct {
  int64_t cached_tokens;
  int64_t evictable_tokens;
  int64_t num_nodes; /* excluding the root */
  int64_t evicted_tokens_total;
  int64_t tick;
  int64_t pinned_tokens; /* cached tokens on pinned nodes (= cached - evictable) */
} radix_tree_stats;
radix_status radix_tree_stats_get(const radix_tree *tree, radix_tree_stats *out);

/* Admission order of n waiting requests (page 4 §5). policy 0 = first come first
 * served; 1 = longest cached prefix first (peek lengths, stable: ties keep arrival
 * order). tok[i] points at request i's tokens, len[i] their count; out_order[n]
 * receives request indices. */
radix_status radix_sched_order(const radix_tree *tree, const int32_t *const *tok,
                               const int64_t *len, int64_t n, int32_t policy,
                               int64_t *out_order);

/* Data-parallel routing: which of n_workers workers (one GPU each, each with its own
 * pool and tree) serves a request of tok[n]. The SGLang feature article gives data
 * parallel attention (§一: batches spread over independent data-parallel workers, so
 * KV is not stored twice) and names a cache-aware load balancer (§五, heading only);
 * the rule below is this library's reading of it.
 *   policy 0: round robin over *rr_counter (incremented);
 *   policy 1: cache-aware. If the loads are imbalanced (max - min > balance_abs and
 *             max > balance_rel * min) the least loaded worker; otherwise the worker
 *             whose tree holds the longest cached prefix of tok (peek: nothing
 *             changes), ties to the smaller load, then the lower index;
 *   policy 2: least loaded (ties: lower index).
 * loads[n_workers] is the caller's load measure (e.g. requests queued this round).
 * *out_worker receives the worker, *out_matched (may be NULL) that worker's cached
 * prefix length. E_INVAL on bad arguments or an unknown policy. */
radix_status radix_route(const radix_tree *const *trees, int32_t n_workers, const int64_t *loads,
                         const int32_t *tok, int64_t n, int32_t policy, int64_t balance_abs,
                         double balance_rel, int64_t *rr_counter, int32_t *out_worker,
                         int64_t *out_matched);

/* Request lifecycle (page 4 §2, §4).
 * admit: match tok[n], pin the matched path, take n - matched new slots (evicting
 *        as needed). out_row[n] receives the slot of every prompt position
 *        (cached then new); *prefix_len the matched length; *node the pinned
 *        node. On RADIX_E_NOMEM the pin is released, *prefix_len is still set and
 *        the request stays waiting (the match's splits and clock refresh remain).
 * finish: insert tok[n] (prompt + generated tokens) with row[n]; give back to the
 *        pool the slots row[prefix_len:already_cached] that duplicate tokens
 *        another request cached meanwhile; unpin `node`. */
radix_status radix_req_admit(radix_tree *tree, const int32_t *tok, int64_t n, int32_t *out_row,
                             int64_t *prefix_len, radix_node *node);
radix_status radix_req_finish(radix_tree *tree, const int32_t *tok, const int32_t *row, int64_t n,
                              int64_t prefix_len, radix_node node, int64_t *already_cached);

/* Batched lifecycle for a round (same semantics as calling radix_req_admit /
 * radix_req_finish per request in order). Request i's tokens are
 * tok[tok_off[i] .. tok_off[i+1]).
 * admit_batch: admits requests 0, 1, ... in order until max_batch are admitted or
 *   one cannot get its slots (it is left waiting, un-pinned); *admitted receives the
 *   count. Admitted request i's slots go to rows[i*row_stride ...], its matched
 *   length to prefix_len[i], its pinned node to nodes[i]. row_stride must be at
 *   least the longest prompt.
 * finish_batch: finishes n requests; request i's tokens (prompt + outputs) are
 *   tok[tok_off[i] .. tok_off[i+1]) and its slots rows[i*row_stride ...] of the same
 *   count; already_cached[i] (may be NULL) receives the insert's count. */
radix_status radix_req_admit_batch(radix_tree *tree, const int32_t *tok, const int64_t *tok_off,
                                   int64_t n, int64_t max_batch, int32_t *rows,
                                   int64_t row_stride, int64_t *prefix_len, radix_node *nodes,
                                   int64_t *admitted);
radix_status radix_req_finish_batch(radix_tree *tree, const int32_t *tok, const int64_t *tok_off,
                                    const int32_t *rows, int64_t row_stride,
                                    const int64_t *prefix_len, const radix_node *nodes, int64_t n,
                                    int64_t *already_cached);

/* ======================================================================
 * Decode plan from the tree: shared segments.
 * Requests running on one tree node read the same slots for that node's
 * tokens. A segment is a chain of tree nodes with the same set of at least
 * `min_members` running requests below it; its keys are read once for all of
 * them (the one-KV-read-many-query-heads idea of the SGLang feature article,
 * §一, applied to the requests sharing a radix-tree path). The rest of each
 * request's keys (positions from req_private_start on) is private.
 *
 * nodes[batch]: each request's admission node (pinned). A segment longer than
 * split_keys keys is cut into ceil(len / split_keys) key chunks (split_keys <= 0:
 * one chunk per segment); every chunk is a separate unit of work with its own
 * partial result per member, so a long shared prefix is spread over several
 * blocks while a short one stays whole. Outputs (host arrays, capacities in
 * brackets):
 *   seg_row[cap_seg]      a member (batch index) whose slot list holds the segment
 *   seg_start/seg_end     key positions [start, end) of the segment
 *   seg_member_off[cap_seg+1], seg_members[cap_mem], seg_member_slot[cap_mem]
 *                         CSR of members; seg_member_slot = the segment's rank
 *                         on that member's path (0 = nearest the root)
 *   seg_split_off[cap_seg+1]  prefix sums of the chunk counts: segment s has
 *                         chunks seg_split_off[s] .. seg_split_off[s+1]-1
 *   seg_member_part[cap_mem]  the member's partial index of the segment's chunk
 *                         0 (chunk k: + k); a request's partials of all its
 *                         segments are 0 .. req_num_parts-1, root-most first
 *   seg_items[cap_items*8]  one record per chunk i (i = seg_split_off[s] + k):
 *                         {lo, hi, member offset, member count, row, s, k, 0};
 *                         chunk k of segment s covers key positions [lo, hi) =
 *                         [start + k*clen, min(end, start + (k+1)*clen)) with clen =
 *                         ceil(len / chunks) rounded up to 64 (trailing chunks may be
 *                         empty: lo = hi = end)
 *   req_num_shared[batch] segments on the request's path, req_num_parts[batch]
 *                         their chunks, req_private_start[batch]
 *   req_order[batch]      batch indices, requests with the same root-most shared
 *                         segment consecutive (then those without one)
 *   *num_segments, *num_member_entries, *max_members, *max_shared,
 *   *num_seg_items (= seg_split_off[num_segments]), *max_parts (largest
 *   req_num_parts), *max_seg_splits (most chunks of one segment)
 * RADIX_E_INVAL if a capacity is too small (the needed counts are still written
 * to *num_segments, *num_member_entries and *num_seg_items). cap_seg >= 2*batch
 * and cap_mem >= batch*max-path-segments always suffice.
 * ====================================================================== */
radix_status radix_tree_decode_plan(const radix_tree *tree, const radix_node *nodes,
                                    int32_t batch, int32_t min_members, int32_t split_keys,
                                    int32_t cap_seg, int32_t cap_mem, int32_t cap_items,
                                    int32_t *seg_row, int32_t *seg_start, int32_t *seg_end,
                                    int32_t *seg_member_off, int32_t *seg_members,
                                    int32_t *seg_member_slot, int32_t *seg_split_off,
                                    int32_t *seg_member_part, int32_t *seg_items,
                                    int32_t *req_num_shared,
                                    int32_t *req_num_parts, int32_t *req_private_start,
                                    int32_t *req_order, int32_t *num_segments,
                                    int32_t *num_member_entries, int32_t *max_members,
                                    int32_t *max_shared, int32_t *num_seg_items,
                                    int32_t *max_parts, int32_t *max_seg_splits);

/* ======================================================================
 * Device side (HIP, gfx950). All pointers below marked "dev" are device
 * pointers; everything is enqueued on `stream` (a hipStream_t; NULL = the
 * default stream).
 * ====================================================================== */
typedef struct {
  int32_t num_q_heads;   /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;  /* Hkv */
  int32_t head_dim_qk;   /* Dqk */
  int32_t head_dim_v;    /* Dv */
  int32_t q_dtype;       /* radix_dtype: F32 | BF16; also the output dtype */
  int32_t kv_dtype;      /* radix_dtype: F32 | BF16 | FP8_E4M3 */
  int32_t v_is_k_prefix; /* 1: V is the first Dv dims of the K row (MLA; v_pool unused) */
  float sm_scale;        /* score = sm_scale * <q, k> */
} radix_attn_shape;

typedef struct {
  void *k_pool;    /* dev [num_slots, Hkv, Dqk] in kv_dtype */
  void *v_pool;    /* dev [num_slots, Hkv, Dv] in kv_dtype; NULL when v_is_k_prefix */
  float *kv_scale; /* dev [num_slots] per-token scale, FP8 only; else NULL */
  int64_t num_slots;
} radix_kv_buffers;

/* Shared-segment plan on the device (the arrays of radix_tree_decode_plan). */
typedef struct {
  int32_t num_segments;
  int32_t num_member_entries;                   /* length of seg_members */
  const int32_t *seg_row, *seg_start, *seg_end; /* dev [num_segments] */
  const int32_t *seg_member_off;                /* dev [num_segments + 1] */
  const int32_t *seg_members, *seg_member_slot; /* dev [num_member_entries] */
  const int32_t *seg_split_off;                 /* dev [num_segments + 1] */
  const int32_t *seg_member_part;               /* dev [num_member_entries] */
  const int32_t *seg_items;                     /* dev [num_seg_items * 8] chunk records */
  const int32_t *req_num_shared;                /* dev [batch] */
  const int32_t *req_num_parts;                 /* dev [batch] */
  const int32_t *req_private_start;             /* dev [batch] */
  const int32_t *req_order;                     /* dev [batch] or NULL */
  int32_t max_members;                          /* host: largest member count */
  int32_t max_shared;                           /* host: largest req_num_shared */
  int32_t max_seg_len;                          /* host: longest segment in tokens */
  int32_t min_private_start;                    /* host: smallest req_private_start */
  int32_t num_seg_items;                        /* host: total segment chunks */
  int32_t max_parts;                            /* host: largest req_num_parts */
  int32_t max_seg_splits;                       /* host: most chunks of one segment */
} radix_decode_plan;

/* Shapes compiled into this library (anything else: RADIX_E_UNSUPPORTED):
 *   q F32, kv F32,  Dqk = Dv = 64,   Hq/Hkv in {1, 2, 4, 8}      (extend, decode)
 *   q BF16, kv BF16 or FP8_E4M3, Dqk = Dv = 128, Hq/Hkv in {1, 2, 4, 8}
 *       (extend, decode; fp8: one scale per token for its K and V rows)
 *   q BF16, kv BF16 or FP8_E4M3, Dqk = 576, Dv = 512, Hkv = 1,
 *       Hq = 128, v_is_k_prefix = 1                              (decode, store)  */
radix_status radix_attn_supported(const radix_attn_shape *shape, int is_decode);

/* Store K/V rows (one per token, all KV heads) at their slots. Defining passages: the
 * K/V of every processed token is kept in a cache and reused instead of recomputed
 * (AWS blog "Improve performance of Falcon models with Amazon SageMaker", section on
 * the KV cache); each radix-tree edge holds the K/V of its tokens (page "49 ·
 * RadixAttention, eviction và cache churn", §2). fp8: KV Cache FP8 with one scale per
 * token (SGLang feature article, §一).
 * Errors: E_UNSUPPORTED for a shape outside the compiled set, E_INVAL for missing
 * buffers or a negative count; nothing is launched then. Async on `stream`:
 * k_pool[slots[t]] = k_new[t], v_pool[slots[t]] = v_new[t], kv_scale[slots[t]] = scale_new[t].
 * k_new dev [T, Hkv, Dqk], v_new dev [T, Hkv, Dv] (ignored when v_is_k_prefix),
 * scale_new dev [T] (FP8 only). Slots must be distinct and < num_slots. */
radix_status radix_kv_store(const radix_attn_shape *shape, const radix_kv_buffers *kv,
                            const void *k_new, const void *v_new, const float *scale_new,
                            const int32_t *slots, int64_t num_tokens, void *stream);

/* Workspace bytes radix_attn_decode needs (split-KV partial results and, for bf16, the
 * merge counters; the split-and-merge of a long key range follows from the exact
 * log-sum-exp merge of softmax partials) for `batch` requests of at most
 * `max_seq_len` tokens with `plan` (NULL = no shared segments; only its host
 * fields are read: num_segments, max_parts, min_private_start) and
 * `num_splits` private splits (0 = the count radix_attn_decode chooses itself).
 * 0 bytes means the call needs no workspace. */
radix_status radix_attn_decode_workspace_size(const radix_attn_shape *shape, int32_t batch,
                                              int32_t max_seq_len,
                                              const radix_decode_plan *plan,
                                              int32_t num_splits, size_t *bytes);

/* Extend attention (prefill of new tokens against each request's cached prefix).
 * Defining passages: prefill processes all of a prompt's tokens at once
 * (AWS blog "Improve performance of Falcon models with Amazon SageMaker", sections on
 * the KV cache and on prefill vs decode); only the part after the cached prefix is
 * computed, the shared part being reused (page "49 · RadixAttention, eviction và
 * cache churn", §2). Errors: E_UNSUPPORTED (shape not compiled, or MLA), E_INVAL
 * (missing buffers, negative sizes, max_extend > total_extend); nothing is launched.
 * No workspace: each query tile (128 or 256 rows, chosen from the batch's average extend
 * length) reads the whole key range itself.
 * Request b (rows req_rows[b] of req_to_token, or b when req_rows is NULL) has
 * prefix_lens[b] cached tokens and extend_lens[b] new ones; its new tokens are
 * rows cu_extend[b] .. cu_extend[b+1]-1 of q/k_new/v_new/out. New token i sits
 * at position prefix_lens[b] + i and attends keys 0 .. prefix_lens[b] + i
 * (causal, itself included), all read through req_to_token[row][pos]: the
 * caller has already written the new tokens' slots into the rows.
 * When k_new is not NULL the new rows are first stored at those slots.
 *   q dev [T, Hq, Dqk] (q_dtype), out dev [T, Hq, Dv] (q_dtype), lse_out dev [T, Hq]
 *   fp32 natural-log log-sum-exp of the scaled scores, or NULL.
 *   req_to_token dev [rows, rtt_stride] int32; prefix_lens, extend_lens dev [batch];
 *   cu_extend dev [batch+1]. Host scalars: total_extend = T, max_extend = max
 *   extend_lens (grid sizing); values above it are an error of the caller. */
radix_status radix_attn_extend(const radix_attn_shape *shape, const radix_kv_buffers *kv,
                               const void *q, const void *k_new, const void *v_new,
                               const float *scale_new, const int32_t *req_to_token,
                               int32_t rtt_stride, const int32_t *req_rows,
                               const int32_t *prefix_lens, const int32_t *extend_lens,
                               const int32_t *cu_extend, int32_t batch, int32_t total_extend,
                               int32_t max_extend, void *out, float *lse_out, void *stream);

/* Decode attention, one new token per request per step over the cached keys
 * (AWS blog "Improve performance of Falcon models with Amazon SageMaker", sections on
 * the KV cache and on continuous batching; decode cost is KV memory traffic, SGLang
 * feature article §一). Errors: E_UNSUPPORTED, E_INVAL (missing buffers, bad sizes,
 * workspace too small, pageable new_slots, incomplete plan); nothing is launched.
 * Request b's query (position seq_lens[b]-1) attends keys
 * 0 .. seq_lens[b]-1 read through req_to_token[row]. When new_slots is not NULL,
 * req_to_token[row][seq_lens[b]-1] = new_slots[b] and the new K/V row
 * (k_new/v_new/scale_new dev [batch, Hkv, *]) is stored at that slot; the query
 * attends the new row itself (read from k_new/v_new). new_slots [batch] int32 may be
 * device memory or pinned host memory mapped into the device (then no copy to the
 * device is needed; the host must not change it until the call's work has run);
 * any other pointer is E_INVAL.
 * With a plan, each key chunk of a shared segment is read once for all the
 * segment's members (one partial result per member and chunk) and keys from
 * req_private_start[b] on are read per request; without a plan (NULL)
 * every request reads all its keys. A request's private keys are cut into
 * `num_splits` equal chunks of a common length (0 = choose: one chunk when the
 * tails are short and the batch fills the GPU, else 768-key chunks; with a plan and
 * bf16 K/V, one chunk cuts the tails of the last tenth of the batch, once they
 * reach 64 keys, in two); all partial results are merged exactly by their
 * log-sum-exp.
 *   q dev [batch, Hq, Dqk]; out dev [batch, Hq, Dv]; lse_out dev [batch, Hq] or NULL;
 *   workspace dev, at least radix_attn_decode_workspace_size bytes. bf16 K/V: the
 *   partial results are merged inside the one decode launch by whichever block
 *   finishes a request last, counted in the workspace's first 256 KiB (int32 per
 *   request and KV head; batch * Hkv <= 65024, else E_INVAL), whose last 2 KiB
 *   hold the work queue of the private-tail kernel, so a bf16 decode always needs a
 *   workspace; that region must be zero before the first call on a workspace (e.g.
 *   allocate it zeroed) and every call leaves it zero. A workspace serves one call
 *   at a time.
 *   max_seq_len: host bound on seq_lens (grid sizing). */
radix_status radix_attn_decode(const radix_attn_shape *shape, const radix_kv_buffers *kv,
                               const void *q, const void *k_new, const void *v_new,
                               const float *scale_new, const int32_t *new_slots,
                               int32_t *req_to_token, int32_t rtt_stride,
                               const int32_t *req_rows, const int32_t *seq_lens, int32_t batch,
                               int32_t max_seq_len, const radix_decode_plan *plan,
                               int32_t num_splits, void *out, float *lse_out, void *workspace,
                               size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops or harnesses that forbid hipMalloc): radix_attn_decode with the same
 * arguments and results, but no workspace argument. Its partial results and merge
 * counters live in a device array built into the library, one per GPU, of
 * radix_attn_decode_noalloc_max_bytes() bytes (64 MiB), held by each GPU the library
 * runs on until the process ends. A call whose workspace would exceed that size
 * (radix_attn_decode_workspace_size) returns RADIX_E_INVAL and launches nothing.
 * Allocates nothing: the first call on a device looks up that device's array and
 * clears its counters with a fill kernel on `stream`; every call leaves them clear.
 * All calls on one GPU share its array, so calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller. The stream's
 * device must be the current device. */
radix_status radix_attn_decode_noalloc(const radix_attn_shape *shape, const radix_kv_buffers *kv,
                                       const void *q, const void *k_new, const void *v_new,
                                       const float *scale_new, const int32_t *new_slots,
                                       int32_t *req_to_token, int32_t rtt_stride,
                                       const int32_t *req_rows, const int32_t *seq_lens,
                                       int32_t batch, int32_t max_seq_len,
                                       const radix_decode_plan *plan, int32_t num_splits,
                                       void *out, float *lse_out, void *stream);
/* Size in bytes of the built-in scratch array of radix_attn_decode_noalloc. */
size_t radix_attn_decode_noalloc_max_bytes(void);

/* ======================================================================
 * Step fences for a scheduler that runs one batch ahead of the GPU (SGLang
 * feature article, §二: the host prepares the next batch's metadata while the
 * GPU runs the current one, so the GPU never waits for the scheduler). A fence
 * marks a point in a stream; waiting on it blocks the host until the work
 * enqueued before it has finished. Unlike a default HIP event it makes device
 * writes visible at device scope only (no system-scope cache writeback between
 * steps): read device results on the host through a copy, not through mapped
 * memory. Errors: E_INVAL on a NULL fence, E_HIP from the runtime.
 * ====================================================================== */
typedef struct radix_fence radix_fence;
radix_status radix_fence_create(radix_fence **out);
radix_status radix_fence_record(radix_fence *fence, void *stream);
radix_status radix_fence_wait(radix_fence *fence);
void radix_fence_destroy(radix_fence *fence);

/* ======================================================================
 * Practical HBM read ceiling for measurement tools (not part of the attention
 * path): reads `bytes` (a positive multiple of 16) from the device buffer `buf`
 * (16-byte aligned) once, with every lane keeping eight non-temporal 16-byte loads in
 * flight, on `stream`. `sink` is a device array of at least 8192 uint32 that the kernel
 * writes only when the XOR of everything read equals a fixed constant; its
 * contents are not meaningful. Time it with events on the same stream.
 * Errors: RADIX_E_INVAL for a missing pointer, a misaligned buffer or a bad size;
 * a launch failure as the HIP status.
 * ====================================================================== */
radix_status radix_probe_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

/* ======================================================================
 * Kernel timing for measurement tools. While enabled, every kernel the
 * attention calls launch is bracketed by two HIP events recorded on the
 * launch stream (up to `capacity` launches; later ones are not recorded).
 * radix_profile_enable(0) disables timing and releases the events.
 * radix_profile_read waits for the recorded events, writes up to `cap`
 * (kernel id, milliseconds) pairs and starts a new recording.
 * ====================================================================== */
radix_status radix_profile_enable(int32_t capacity);
radix_status radix_profile_read(int32_t *kernel_ids, float *ms, int32_t cap, int32_t *count);
/* Name of a kernel id reported by radix_profile_read ("" if unknown). */
const char *radix_kernel_name(int32_t kernel_id);

#ifdef __cplusplus
}
#endif
#endif /* RADIX_ATTN_H */
