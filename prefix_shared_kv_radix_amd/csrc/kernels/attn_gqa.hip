// gfx950 kernels for attention over a radix-shared, token-granular KV pool.
//
// A request's keys are read through its slot list (req_to_token); K/V rows
// live in one pool shared by every request (page "49 · RadixAttention,
// eviction và cache churn", §2 and §4). All kernels compute plain causal
// softmax attention, merged exactly through log-sum-exp where the key range
// is split:
//   o = sum_s 2^(L_s - L) o_s,  L = log2 sum_s 2^(L_s),  L_s = m_s + log2 l_s
// (scores are kept in the log2 domain: s * sm_scale * log2(e)).
//
// Kernels
//   kv_store_kernel   writes new K/V rows at their slots (and, for decode,
//                     appends the new slot to the request's slot list).
//   attn_valu_kernel  one query token (all query heads of one KV head)
//                     against a key range: 16 lanes per 256-byte row,
//                     16-byte loads, DPP row reductions, online softmax in
//                     registers, cross-wave merge in LDS. Used for the
//                     private tail of decode (split-KV) and for fp32.
//   attn_mfma_kernel  128 or 256 query rows x 64-key tiles with bf16 MFMA
//                     (32x32x16): S^T = K Q^T keeps a query row per lane so
//                     the softmax is lane-local; P^T feeds O^T = V^T P^T
//                     straight from registers. Query rows are either a
//                     request's new tokens x heads (extend, causal) or the
//                     members of a shared radix segment x heads (decode: one
//                     read of the segment's KV serves every member).
//   combine_kernel    merges per-request partial results.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "attn_args.hpp"
#include "radix_attn.h"

using namespace radix_dev;
using radix_launch::AttnArgs;
using radix_launch::StoreArgs;

namespace {

#ifndef RADIX_VALU_STAGES
#define RADIX_VALU_STAGES 3
#endif
constexpr int kValuStages = RADIX_VALU_STAGES;  // register buffers in the VALU kernel's ring

__device__ __forceinline__ int find_owner(const int32_t *off, int n, int t) {
  // largest i in [0, n) with off[i] <= t
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ const int32_t *rtt_row_of(const AttnArgs &a, int b) {
  int row = a.req_rows ? a.req_rows[b] : b;
  return a.rtt + static_cast<int64_t>(row) * a.rtt_stride;
}

// ------------------------------------------------------------------ KV store
__global__ void kv_store_kernel(StoreArgs a) {
  const int64_t t = blockIdx.x;
  int slot;
  if (a.mode == 0) {
    slot = a.slots[t];
  } else if (a.mode == 2) {
    int b = find_owner(a.cu_extend, a.batch, static_cast<int>(t));
    int row = a.req_rows ? a.req_rows[b] : b;
    slot = a.rtt[static_cast<int64_t>(row) * a.rtt_stride + a.prefix_lens[b] + (t - a.cu_extend[b])];
  } else {
    int row = a.req_rows ? a.req_rows[t] : static_cast<int>(t);
    int64_t at = static_cast<int64_t>(row) * a.rtt_stride + a.seq_lens[t] - 1;
    if (a.mode == 1) {
      slot = a.new_slots[t];
      if (threadIdx.x == 0) a.rtt[at] = slot;
    } else {
      slot = a.rtt[at];
    }
  }
  const int kc = a.k_row_bytes >> 4, vc = a.v_row_bytes >> 4;
  const u32x4 *ks = reinterpret_cast<const u32x4 *>(a.k_new + t * a.k_row_bytes);
  u32x4 *kd = reinterpret_cast<u32x4 *>(a.k_pool + static_cast<int64_t>(slot) * a.k_row_bytes);
  for (int c = threadIdx.x; c < kc; c += blockDim.x) kd[c] = ks[c];
  if (a.v_new) {
    const u32x4 *vs = reinterpret_cast<const u32x4 *>(a.v_new + t * a.v_row_bytes);
    u32x4 *vd = reinterpret_cast<u32x4 *>(a.v_pool + static_cast<int64_t>(slot) * a.v_row_bytes);
    for (int c = threadIdx.x; c < vc; c += blockDim.x) vd[c] = vs[c];
  }
  if (a.scale_new && threadIdx.x == 0) a.kv_scale[slot] = a.scale_new[t];
}

// ------------------------------------------------------------------ VALU kernel
template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void unpack(const u32x4 &w, float *x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
  }
  __device__ static void store(void *p, const float *x) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{x[0], x[1], x[2], x[3]};
  }
};
template <> struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ static void unpack(const u32x4 &w, float *x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
  }
  __device__ static void store(void *p, const float *x) {
    *reinterpret_cast<u32x4 *>(p) = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                          pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
  }
};

// four consecutive values at idx (a multiple of 4)
template <typename T> __device__ __forceinline__ void store_out4(void *out, int64_t idx, f32x4 v);
template <> __device__ __forceinline__ void store_out4<float>(void *out, int64_t idx, f32x4 v) {
  *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + idx) = v;
}
template <> __device__ __forceinline__ void store_out4<uint16_t>(void *out, int64_t idx, f32x4 v) {
  *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(out) + idx) =
      u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ mask) << 2,
                                                                 __builtin_bit_cast(int, x)));
}

// One wave = one query token (the G query heads of one KV head) against one key range.
// 16 lanes cover a 256-byte K (or V) row with 16-byte loads, so a wave takes 4 rows per
// load and 16 rows per iteration; the next iteration's slot indices and K/V rows are in
// flight while the current one is computed. The four 16-lane groups (different rows,
// same dims) are merged with cross-lane exchanges at the end; no LDS, no barriers.
// Work item w = blockIdx.x * 4 + wave, decomposed as ((item * nsplit + split) * Hkv + kvh).
// MODE 0: decode private tail, one of several splits -> partial (o, lse) in the workspace
// MODE 1: extend (fp32 path), item = new token -> final output
// MODE 2: decode shared segment (fp32 path), item = (segment, member) entry -> partial
// MODE 3: decode private tail, single split -> final output, merged with the request's
//         shared-segment partials (written earlier on the same stream)
// In MODE 0 and 3 the newest key (position seq_len-1) is read from k_new/v_new when given,
// and the split-0 wave stores it into the pool and appends its slot to the slot list.
template <typename T, int D, int G, int MODE>
__device__ __forceinline__ void valu_body(const AttnArgs &a, int w, int n_items, int nsplit) {
  constexpr int EPL = Vec16<T>::N;
  static_assert(D / EPL == 16, "16 lanes per row");
  constexpr bool TAIL = MODE == 0 || MODE == 3;
  const int lane = threadIdx.x & 63, grp = lane >> 4, sub = lane & 15;
  if (w >= n_items * nsplit * a.Hkv) return;
  const int kvh = w % a.Hkv;
  const int split = (w / a.Hkv) % nsplit;
  const int item = w / (a.Hkv * nsplit);

  int b, lo, hi, part = 0;
  int pieces = nsplit;   // key chunks of this item's range
  int64_t q_row;
  const int32_t *rtt_row;
  if (MODE == 1) {
    b = find_owner(a.cu_extend, a.batch, item);
    const int i = item - a.cu_extend[b];
    lo = 0;
    hi = a.prefix_lens[b] + i + 1;
    q_row = item;
    rtt_row = rtt_row_of(a, b);
  } else if (TAIL) {
    b = item;
    hi = a.seq_lens[b];
    lo = a.private_start ? a.private_start[b] : 0;
    q_row = b;
    rtt_row = rtt_row_of(a, b);
    part = a.part_base + split;
  } else {
    // item = member entry; split = key chunk of its segment (nsplit = most chunks of a
    // segment: the waves past this segment's own count have no work)
    const int sg = find_owner(a.seg_member_off, a.num_segments, item);
    pieces = a.seg_split_off[sg + 1] - a.seg_split_off[sg];
    if (split >= pieces) return;
    b = a.seg_members[item];
    const int32_t *rec = a.seg_items + static_cast<int64_t>(a.seg_split_off[sg] + split) * 8;
    lo = rec[0];   // the chunk's own key range (below, split 0 of one chunk)
    hi = rec[1];
    q_row = b;
    rtt_row = rtt_row_of(a, rec[4]);
    part = a.seg_member_part[item] + split;
  }
  // TAIL: common chunk length (a.split_chunk) so uneven requests spread evenly;
  // MODE 2: [lo, hi) is already this chunk
  const int chunk = (TAIL && nsplit > 1) ? a.split_chunk : ((hi - lo + 15) & ~15);
  const int s_lo = lo + (MODE == 2 ? 0 : split * chunk);
  const int s_hi = min(hi, s_lo + chunk);

  const int64_t row_bytes = static_cast<int64_t>(a.Hkv) * D * sizeof(T);
  const char *kb = reinterpret_cast<const char *>(a.k_pool) + kvh * D * sizeof(T) + sub * 16;
  const char *vb = reinterpret_cast<const char *>(a.v_pool) + kvh * D * sizeof(T) + sub * 16;
  const bool fuse_new = TAIL && a.k_new != nullptr;
  const char *knew = nullptr, *vnew = nullptr;
  if (fuse_new) {
    const int64_t off = (static_cast<int64_t>(b) * a.Hkv + kvh) * D * sizeof(T) + sub * 16;
    knew = reinterpret_cast<const char *>(a.k_new) + off;
    vnew = reinterpret_cast<const char *>(a.v_new) + off;
    if (split == 0 && grp == 0) {
      const int64_t at = static_cast<int64_t>(a.req_rows ? a.req_rows[b] : b) * a.rtt_stride + hi - 1;
      const int64_t slot = a.new_slots ? a.new_slots[b] : a.rtt[at];
      if (a.new_slots && kvh == 0 && sub == 0) a.rtt_mut[at] = static_cast<int32_t>(slot);
      *reinterpret_cast<u32x4 *>(const_cast<char *>(kb) + slot * row_bytes) = ldg16(knew);
      *reinterpret_cast<u32x4 *>(const_cast<char *>(vb) + slot * row_bytes) = ldg16(vnew);
    }
  }

  float qf[G][EPL];
  {
    const T *qp = reinterpret_cast<const T *>(a.q) + (q_row * a.Hq + kvh * G) * D + sub * EPL;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      Vec16<T>::unpack(ldg16(qp + h * D), qf[h]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[h][e] *= a.scale_log2;
    }
  }
  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  // ring of NB register buffers: iteration t (16 rows) is computed while the K/V rows of
  // iterations t+1 .. t+NB-1 and the slot indices of iteration t+NB are in flight
  constexpr int NB = kValuStages;
  u32x4 kbuf[NB][4], vbuf[NB][4];
  int32_t sbuf[NB][4];
  // Loads are unconditional (no branches around them, so the compiler can count the
  // loads in flight): rows past the range read a clamped slot-list entry / slot 0 and
  // are masked after the load.
  const int last = s_hi - 1;   // >= 0: s_hi >= 1 always
  auto load_slots = [&](int base, int32_t *sl) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = base + u * 4 + grp;
      const int32_t v = rtt_row[min(r, last)];
      sl[u] = (r < s_hi && !(fuse_new && r == hi - 1)) ? v : 0;
    }
  };
  auto load_kv = [&](int base, const int32_t *sl, u32x4 *kd, u32x4 *vd) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = base + u * 4 + grp;
      const bool newest = fuse_new && r == hi - 1;
      const char *kp = newest ? knew : kb + static_cast<int64_t>(sl[u]) * row_bytes;
      const char *vp = newest ? vnew : vb + static_cast<int64_t>(sl[u]) * row_bytes;
      kd[u] = ldg16(kp);
      vd[u] = ldg16(vp);
    }
  };
  auto compute = [&](int base, const u32x4 *kr, const u32x4 *vr) {
    float p[4][G];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float kf[EPL];
      Vec16<T>::unpack(kr[u], kf);
      const bool valid = base + u * 4 + grp < s_hi;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d = fmaf(qf[h][e], kf[e], d);
        d = sum16(d);
        p[u][h] = valid ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mx = fmaxf(fmaxf(p[0][h], p[1][h]), fmaxf(p[2][h], p[3][h]));
      const float mn = fmaxf(m[h], mx);
      const float alpha = exp2f(m[h] - mn);
#pragma unroll
      for (int u = 0; u < 4; ++u) p[u][h] = exp2f(p[u][h] - mn);
      l[h] = l[h] * alpha + ((p[0][h] + p[1][h]) + (p[2][h] + p[3][h]));
      m[h] = mn;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool valid = base + u * 4 + grp < s_hi;
      u32x4 w = vr[u];
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] = valid ? w[c] : 0u;   // masked rows may hold NaN
      float vf[EPL];
      Vec16<T>::unpack(w, vf);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p[u][h], vf[e], acc[h][e]);
    }
  };

  // Step t computes iteration t (buffer t % NB). Before that it issues, in this order,
  // the slot indices of iteration t+NB and the K/V rows of iteration t+NB-1 (whose slots
  // came one step earlier). Loads return in issue order, so waiting for those slots
  // never waits for the K/V rows issued one step earlier: NB-1 iterations stay in flight.
#pragma unroll
  for (int j = 0; j < NB; ++j) load_slots(s_lo + 16 * j, sbuf[j]);
#pragma unroll
  for (int j = 0; j + 1 < NB; ++j) load_kv(s_lo + 16 * j, sbuf[j], kbuf[j], vbuf[j]);
  for (int base = s_lo; base < s_hi; base += 16 * NB) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int it = base + 16 * j;
      if (it >= s_hi) break;
      const int jl = (j + NB - 1) % NB;
      const int ahead = it + 16 * (NB - 1);
      load_slots(ahead + 16, sbuf[j]);
      load_kv(ahead, sbuf[jl], kbuf[jl], vbuf[jl]);
      compute(it, kbuf[j], vbuf[j]);
    }
  }

  // merge the four 16-lane groups (same dims, other rows); afterwards every lane holds
  // the wave's state for its 8 (bf16) or 4 (fp32) dims of every head
#pragma unroll
  for (int mask = 16; mask <= 32; mask <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = shfl_xor_f(m[h], mask), lo_ = shfl_xor_f(l[h], mask);
      const float mn = fmaxf(m[h], mo);
      const float wa = exp2f(m[h] - mn), wb = exp2f(mo - mn);
      l[h] = l[h] * wa + lo_ * wb;
      m[h] = mn;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * wa + shfl_xor_f(acc[h][e], mask) * wb;
    }
  }

  // lane group g writes heads g, g+4, ...; dims sub*EPL .. sub*EPL+EPL-1
  const int nshared = (MODE == 3 && a.req_num_parts) ? a.req_num_parts[b] : 0;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if ((h & 3) != grp) continue;
    const int head = kvh * G + h;
    float M = m[h], L = l[h];
    float O[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) O[e] = acc[h][e];
    if (MODE == 3) {
      // shared-segment partials (o normalised, lse in log2 units), four at a time
      const int64_t hp = (static_cast<int64_t>(b) * a.Hq + head) * a.parts;
      for (int p0 = 0; p0 < nshared; p0 += 4) {
        float pl[4];
        f32x4 po[4][EPL / 4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool ok = p0 + j < nshared;
          pl[j] = ok ? a.ws_lse[hp + p0 + j] : -INFINITY;
#pragma unroll
          for (int c = 0; c < EPL / 4; ++c)
            po[j][c] = ok ? *reinterpret_cast<const f32x4 *>(a.ws_o + (hp + p0 + j) * D + sub * EPL + 4 * c)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float mn = fmaxf(M, pl[j]);
          const float wa = exp2f(M - mn), wb = exp2f(pl[j] - mn);
          L = L * wa + wb;
          M = mn;
#pragma unroll
          for (int c = 0; c < EPL / 4; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) O[4 * c + e] = O[4 * c + e] * wa + po[j][c][e] * wb;
        }
      }
    }
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.f / L;
    const float lse2 = empty ? -INFINITY : M + log2f(L);
#pragma unroll
    for (int e = 0; e < EPL; ++e) O[e] *= inv;
    if (MODE == 1 || MODE == 3) {
      Vec16<T>::store(reinterpret_cast<T *>(a.out) + (q_row * a.Hq + head) * D + sub * EPL, O);
      if (a.lse && sub == 0) a.lse[q_row * a.Hq + head] = lse2 * kLn2;
    } else {
      const int64_t pi = (static_cast<int64_t>(b) * a.Hq + head) * a.parts + part;
#pragma unroll
      for (int c = 0; c < EPL / 4; ++c)
        *reinterpret_cast<f32x4 *>(a.ws_o + pi * D + sub * EPL + 4 * c) =
            f32x4{O[4 * c], O[4 * c + 1], O[4 * c + 2], O[4 * c + 3]};
      if (sub == 0) a.ws_lse[pi] = lse2;
    }
  }
}

template <typename T, int D, int G, int MODE>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnArgs a, int n_items, int nsplit) {
  valu_body<T, D, G, MODE>(a, blockIdx.x * 4 + (threadIdx.x >> 6), n_items, nsplit);
}

// ------------------------------------------------------------------ bf16 decode tail
// One wave = one decode query (the G query heads of one KV head) over one key chunk,
// for bf16 K/V with 128 dims. Sixteen lanes cover a 256-byte row (16 bytes each, so one
// load instruction reads four whole rows), and an iteration of 16 rows gives every lane
// four rows (r, r+4, r+8 and r+12 of the iteration).
//   q.k  : v_dot2_f32_bf16 on packed pairs, then a 4-step DPP sum over the 16 lanes
//   p.v  : p of two rows packed to bf16, V dims of the two rows paired with byte
//          permutes, v_dot2_f32_bf16 per dim (fp32 accumulation)
// The running maximum is refreshed only when some head's tile maximum exceeds it by
// more than 2^8 (numerator and denominator share the stale maximum, so nothing is lost).
// A request whose keys all fall in this one chunk (no shared segment, one chunk) writes
// its output directly. Otherwise the wave writes a partial and arrives at the request's
// merge counter; whichever producer of the request arrives last (this wave, another
// chunk, or a shared-segment tile) merges every partial into the output, so no second
// launch is needed. The newest key is read from k_new/v_new; the chunk-0 wave stores it
// at its slot and appends the slot to the slot list after its own loop (no other wave
// of this launch reads that slot or list entry).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
// Merges every partial of up to NR requests (bs[0 .. n-1], wave-uniform, n >= 1; nparts[r]
// = request bs[r]'s segment-chunk partial count) for the G query heads of KV head kvh
// into the bf16 output (and lse): lane -> 8 dims of one head, 512 values per pass.
// Partials of shared-segment chunks come first ([0, nparts)), then the private chunks
// ([part_base, part_base + num_splits)); an empty partial has lse -inf and weight 0.
// The first four partials of all NR requests are loaded before any is folded, so the
// merges take one memory round trip rather than one per request. Called by the last
// producer to arrive, after its counter read.
// Private parts of request b, and the private-tail items of a step whose first `whole`
// requests are read in one part and the rest in nsplit parts each.
__device__ __forceinline__ int tail_parts(const AttnArgs &a, int b) {
  return b < a.whole_reqs ? 1 : a.num_splits;
}
__host__ __device__ __forceinline__ int tail_items(int whole, int n_items, int nsplit, int hkv) {
  return (whole + (n_items - whole) * nsplit) * hkv;
}

template <int G, int NR>
__device__ __forceinline__ void merge_requests_bf16(const AttnArgs &a, const int (&bs)[NR],
                                                    const int (&nparts)[NR], int n, int kvh) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < (G * 128 + 511) / 512; ++c) {
    const int e = c * 512 + lane * 8;
    if (e >= G * 128) break;
    const int head = kvh * G + e / 128, d = e % 128;
    float pl[NR][4];
    f32x4 pa[NR][4], pb[NR][4];
    // partials p0 .. p0+3 of request slot r (slots past n repeat request 0; indices past
    // the request's count re-read its partial 0 with weight 0): loads never branch
    auto load4 = [&](int r, int p0) {
      const int b = r < n ? bs[r] : bs[0];
      const int ns = r < n ? nparts[r] : nparts[0];
      const int total = ns + tail_parts(a, b);
      const int64_t base = (static_cast<int64_t>(b) * a.Hq + head) * a.parts;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = p0 + j < total ? p0 + j : 0;
        const int64_t pi = base + (idx < ns ? idx : a.part_base + idx - ns);
        const float l = ld_dev1(a.ws_lse + pi);
        pl[r][j] = p0 + j < total ? l : -INFINITY;
        pa[r][j] = ld_dev(a.ws_o + pi * 128 + d);
        pb[r][j] = ld_dev(a.ws_o + pi * 128 + d + 4);
      }
    };
    auto fold4 = [&](int r, float &M, float &L, f32x4 &O0, f32x4 &O1) {
      float mx = M;
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = fmaxf(mx, pl[r][j]);
      const float alpha = exp2f(M - mx);
      L *= alpha;
      O0 *= alpha;
      O1 *= alpha;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float wj = exp2f(pl[r][j] - mx);
        L += wj;
        if (wj > 0.f) {
          O0 += pa[r][j] * wj;
          O1 += pb[r][j] * wj;
        }
      }
      M = mx;
    };
#pragma unroll
    for (int r = 0; r < NR; ++r) load4(r, 0);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (r >= n) break;
      const int b = bs[r];
      float M = kNegBig, L = 0.f;
      f32x4 O0 = f32x4{0.f, 0.f, 0.f, 0.f}, O1 = O0;
      fold4(r, M, L, O0, O1);
      for (int p0 = 4; p0 < nparts[r] + tail_parts(a, b); p0 += 4) {   // more than 4 partials
        load4(r, p0);
        fold4(r, M, L, O0, O1);
      }
      const float inv = 1.f / L;
      uint16_t *op = reinterpret_cast<uint16_t *>(a.out) + (static_cast<int64_t>(b) * a.Hq + head) * 128 + d;
      *reinterpret_cast<u32x4 *>(op) =
          u32x4{pack2bf(O0[0] * inv, O0[1] * inv), pack2bf(O0[2] * inv, O0[3] * inv),
                pack2bf(O1[0] * inv, O1[1] * inv), pack2bf(O1[2] * inv, O1[3] * inv)};
      if (a.lse && d == 0) a.lse[static_cast<int64_t>(b) * a.Hq + head] = (M + log2f(L)) * kLn2;
    }
  }
}

#ifndef RADIX_TAIL_STAGES
#define RADIX_TAIL_STAGES 3
#endif



__device__ __forceinline__ int32_t take_ticket(int32_t *q);

// One private-tail item w = (request, split, KV head) on one wave. With a work queue
// (queue != NULL) the wave draws its next ticket into `ticket` (lane 0) once its keys
// are read, so the atomic's latency overlaps the rest of the item.
template <bool FP8> struct RowOf { typedef u32x4 type; };   // one lane's part of a row
template <> struct RowOf<true> { typedef u32x2 type; };

template <int G, bool FP8>
__device__ __forceinline__ void tail_bf16_body(const AttnArgs &a, int w, int n_items, int nsplit,
                                               int32_t *queue = nullptr, int32_t *ticket = nullptr) {
  constexpr int D = 128;
  // bf16 rows: 16 bytes per lane; fp8 rows: 8 bytes per lane (the same 8 dims), converted
  // exactly to bf16 pairs, the row's scale applied to its score and probability
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int LB = 8 * EB;
  using RowT = typename RowOf<FP8>::type;
  constexpr int NB = RADIX_TAIL_STAGES;
  constexpr float kGrow = 8.f;
  int lane = threadIdx.x & 63;
  // opaque per call, so that the values derived from the lane index are computed for each
  // item instead of being kept live across the work-queue loop (register pressure)
  asm volatile("" : "+v"(lane));
  // 16 lanes per 256-byte row: lane sub holds dims 8*sub .. 8*sub+7 of a row; the four
  // row groups r4 take rows r4, r4+4, r4+8 and r4+12 of each 16-row iteration
  const int r4 = lane >> 4, sub = lane & 15;
  w = __builtin_amdgcn_readfirstlane(w);   // one work item per wave: its indices are scalar
  // items: (request, KV head) for the requests read whole, then (request, split, KV head)
  const int whole = min(a.whole_reqs, n_items);
  if (w >= tail_items(whole, n_items, nsplit, a.Hkv)) return;
  const bool one = w < whole * a.Hkv;
  const int wr = one ? w : w - whole * a.Hkv;
  const int ns_tail = one ? 1 : nsplit;   // private parts of this request
  const int kvh = wr % a.Hkv;
  const int split = (wr / a.Hkv) % ns_tail;
  const int b = (one ? 0 : whole) + wr / (a.Hkv * ns_tail);

  const int hi = a.seq_lens[b];
  const int lo = a.private_start ? a.private_start[b] : 0;
  const int64_t q_row = b;
  const int32_t *rtt_row = rtt_row_of(a, b);
  const int part = a.part_base + split;
  const int chunk = ns_tail > 1 ? a.split_chunk : ((hi - lo + 15) & ~15);
  const int s_lo = lo + split * chunk;
  const int s_hi = min(hi, s_lo + chunk);

  const int64_t row_bytes = static_cast<int64_t>(a.Hkv) * D * EB;
  const char *kb = reinterpret_cast<const char *>(a.k_pool) + kvh * D * EB + sub * LB;
  const char *vb = reinterpret_cast<const char *>(a.v_pool) + kvh * D * EB + sub * LB;
  const bool fuse_new = a.k_new != nullptr;
  const char *knew = nullptr, *vnew = nullptr;
  // the new token's slot: read now (new_slots may be pinned host memory), used at the end
  const bool store_new = fuse_new && split == 0;
  const int64_t new_at = static_cast<int64_t>(a.req_rows ? a.req_rows[b] : b) * a.rtt_stride + hi - 1;
  int32_t new_slot = 0;
  float sc_new = 1.f;
  if (fuse_new) {
    const int64_t off = (static_cast<int64_t>(b) * a.Hkv + kvh) * D * EB + sub * LB;
    knew = reinterpret_cast<const char *>(a.k_new) + off;
    vnew = reinterpret_cast<const char *>(a.v_new) + off;
    if (store_new) new_slot = a.new_slots ? a.new_slots[b] : a.rtt[new_at];
    if (FP8) sc_new = a.scale_new[b];
  }
  const int ns_b = a.req_num_parts ? a.req_num_parts[b] : 0;
  const int expected = ns_b + ns_tail;   // producers of this request's output

  // q: G heads x this lane's 8 dims, packed bf16 pairs (unscaled)
  uint32_t qp[G][4];
  {
    const char *qb = reinterpret_cast<const char *>(a.q) + (q_row * a.Hq + kvh * G) * D * 2 + sub * 16;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const u32x4 x = ldg16(qb + h * D * 2);
#pragma unroll
      for (int c = 0; c < 4; ++c) qp[h][c] = x[c];
    }
  }
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  // Pool rows of this chunk: [s_lo, pool_hi); the newest key (position hi-1, not yet in
  // the pool when fused) is folded in once after the loop from k_new/v_new.
  // Iteration t covers rows base .. base+15; this lane takes rows base + 4k + r4 (k < 4).
  // Every load is unconditional: rows past pool_hi re-read the chunk's
  // last pool row (finite, stored), and their weight is exactly 0.
  const int pool_hi = fuse_new ? min(s_hi, hi - 1) : s_hi;
  const int last = pool_hi - 1;
  // With up to 4 query heads per KV head the ring's loads are issued as asm and waited
  // for explicitly: each step waits for exactly the slots it is about to use (the K/V
  // rows of the step being computed are older, so they have landed too), keeping NB-1
  // iterations in flight during the arithmetic. The compiler's own wait placement for
  // this ring also waits for the next iteration's rows (its merge at the loop head is
  // conservative), which halves the loads in flight. The counts assume that no other
  // vector memory operation is issued inside the ring, so register spills (scratch
  // accesses) would break them: the build rejects these kernels if they use scratch.
  // With 8 heads the kernel spills, and the compiler places the waits.
  constexpr bool kOwnWaits = G <= 4;
  static_assert(NB >= 3, "the slot wait covers the rows being computed only for NB >= 3");
  // loads of one iteration's rows: K and V (and, fp8, the rows' scales) for 4 rows
  constexpr int kRowLoads = FP8 ? 12 : 8;
  RowT kbuf[NB][4], vbuf[NB][4];
  float cbuf[NB][4];   // fp8: the rows' scales
  int32_t sbuf[NB][4];
  auto load_slots = [&](int base, int32_t *sl) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int32_t *p = rtt_row + min(base + 4 * k + r4, last);
      sl[k] = kOwnWaits ? ld_async4(p) : *p;
    }
  };
  auto load_kv = [&](const int32_t *sl, RowT *kd, RowT *vd, float *cd) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const char *kp = kb + static_cast<int64_t>(sl[k]) * row_bytes;
      const char *vp = vb + static_cast<int64_t>(sl[k]) * row_bytes;
      if constexpr (FP8) {
        kd[k] = kOwnWaits ? ld_async8(kp) : *reinterpret_cast<const u32x2 *>(kp);
        vd[k] = kOwnWaits ? ld_async8(vp) : *reinterpret_cast<const u32x2 *>(vp);
        cd[k] = kOwnWaits ? ld_async4f(a.kv_scale + sl[k]) : a.kv_scale[sl[k]];
      } else {
        kd[k] = kOwnWaits ? ld_async16<0>(kp) : ldg16(kp);
        vd[k] = kOwnWaits ? ld_async16<0>(vp) : ldg16(vp);
      }
    }
  };
  // wait until at most N loads are outstanding; sl and the rows of one ring stage are
  // tied to the wait so that no use of them is scheduled before it
  auto wait_ring = [&](auto n, int32_t *sl, RowT *kd, RowT *vd, float *cd) {
    if constexpr (kOwnWaits && FP8)
      asm volatile("s_waitcnt vmcnt(%16)"
                   : "+v"(sl[0]), "+v"(sl[1]), "+v"(sl[2]), "+v"(sl[3]), "+v"(kd[0]), "+v"(kd[1]),
                     "+v"(kd[2]), "+v"(kd[3]), "+v"(vd[0]), "+v"(vd[1]), "+v"(vd[2]), "+v"(vd[3]),
                     "+v"(cd[0]), "+v"(cd[1]), "+v"(cd[2]), "+v"(cd[3])
                   : "n"(decltype(n)::value)
                   : "memory");
    else if constexpr (kOwnWaits)
      asm volatile("s_waitcnt vmcnt(%12)"
                   : "+v"(sl[0]), "+v"(sl[1]), "+v"(sl[2]), "+v"(sl[3]), "+v"(kd[0]), "+v"(kd[1]),
                     "+v"(kd[2]), "+v"(kd[3]), "+v"(vd[0]), "+v"(vd[1]), "+v"(vd[2]), "+v"(vd[3])
                   : "n"(decltype(n)::value)
                   : "memory");
  };
  // a lane's 8 dims of a row as 4 packed bf16 pairs
  auto words = [](const RowT &r, uint32_t (&w)[4]) {
    if constexpr (FP8) {
      w[0] = fp8x2_to_bf16x2<false>(r[0]);
      w[1] = fp8x2_to_bf16x2<true>(r[0]);
      w[2] = fp8x2_to_bf16x2<false>(r[1]);
      w[3] = fp8x2_to_bf16x2<true>(r[1]);
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) w[c] = r[c];
    }
  };
  // rows k = 0..3 of this lane (row base + 4k + r4) with valid flags `vmask` bit k; cr:
  // the rows' scales (fp8)
  auto compute = [&](int vmask, const RowT *kr, const RowT *vr, const float *cr) {
    float s[4][G];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t kw[4];
      words(kr[k], kw);
      const float sk = FP8 ? a.scale_log2 * cr[k] : a.scale_log2;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) d = dot2bf(qp[h][c], kw[c], d);
        d = sum16(d);
        s[k][h] = ((vmask >> k) & 1) ? d * sk : -INFINITY;
      }
    }
    bool grow = false;
#pragma unroll
    for (int h = 0; h < G; ++h)
      grow |= fmaxf(fmaxf(s[0][h], s[1][h]), fmaxf(s[2][h], s[3][h])) > m[h] + kGrow;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], fmaxf(fmaxf(s[0][h], s[1][h]), fmaxf(s[2][h], s[3][h])));
        const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);
        m[h] = mn;
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
      }
    }
    uint32_t pp[2][G];   // probabilities of rows (0, 1) and (2, 3), packed bf16 pairs
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float p[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) p[k] = __builtin_amdgcn_exp2f(s[k][h] - m[h]);
      l[h] += (p[0] + p[1]) + (p[2] + p[3]);
      if constexpr (FP8) {   // the value rows' scales go with their probabilities
        pp[0][h] = pack2bf(p[0] * cr[0], p[1] * cr[1]);
        pp[1][h] = pack2bf(p[2] * cr[2], p[3] * cr[3]);
      } else {
        pp[0][h] = pack2bf(p[0], p[1]);
        pp[1][h] = pack2bf(p[2], p[3]);
      }
    }
    uint32_t vw[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k) words(vr[k], vw[k]);
    // pair dim e of row 2i with dim e of row 2i+1
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t a0 = vw[2 * i][c], a1 = vw[2 * i + 1][c];
        const uint32_t lo2 = __builtin_amdgcn_perm(a1, a0, 0x05040100u);   // {row.lo, row'.lo}
        const uint32_t hi2 = __builtin_amdgcn_perm(a1, a0, 0x07060302u);   // {row.hi, row'.hi}
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][2 * c] = dot2bf(pp[i][h], lo2, acc[h][2 * c]);
          acc[h][2 * c + 1] = dot2bf(pp[i][h], hi2, acc[h][2 * c + 1]);
        }
      }
  };

  // Step t computes iteration t (buffer t % NB). Before that it issues, in this order,
  // the slot indices of iteration t+NB and the K/V rows of iteration t+NB-1 (whose slots
  // came one step earlier). Loads return in issue order, so waiting for those slots
  // never waits for the K/V rows issued one step earlier: NB-1 iterations stay in flight.
  // The last group of NB steps runs whole (steps past the end are fully masked): an
  // early exit inside it makes the compiler rotate the ring through registers that still
  // have loads in flight, which costs a wait for them every step.
  if (pool_hi > s_lo) {   // (uniform) no pool rows: nothing to load
    // the compiler's loads (q) land before the ring starts, so that it places no wait
    // for them inside the loop
    if constexpr (kOwnWaits) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(qp[h][c]));
    }
    // issue order, the same before and inside the loop: step t loads the slots of
    // iteration t+NB, then the rows of iteration t+NB-1 (whose slots came one step
    // earlier), then computes iteration t
    load_slots(s_lo, sbuf[0]);
#pragma unroll
    for (int j = 1; j < NB; ++j) {
      load_slots(s_lo + 16 * j, sbuf[j]);
      if (j == 1)
        wait_ring(std::integral_constant<int, 4>{}, sbuf[0], kbuf[0], vbuf[0], cbuf[0]);
      else
        wait_ring(std::integral_constant<int, kRowLoads + 4>{}, sbuf[j - 1], kbuf[j - 1],
                  vbuf[j - 1], cbuf[j - 1]);
      load_kv(sbuf[j - 1], kbuf[j - 1], vbuf[j - 1], cbuf[j - 1]);
    }
    for (int base = s_lo; base < pool_hi; base += 16 * NB) {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int it = base + 16 * j;
        const int jl = (j + NB - 1) % NB;
        load_slots(it + 16 * NB, sbuf[j]);
        // younger than the slots of iteration t+NB-1: the rows of t+NB-2 (kRowLoads loads)
        // and the slots just issued (4); the rows of t are older, so they have landed
        wait_ring(std::integral_constant<int, kRowLoads + 4>{}, sbuf[jl], kbuf[j], vbuf[j],
                  cbuf[j]);
        load_kv(sbuf[jl], kbuf[jl], vbuf[jl], cbuf[jl]);
        int vmask = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) vmask |= (it + 4 * k + r4 < pool_hi) << k;
        compute(vmask, kbuf[j], vbuf[j], cbuf[j]);
      }
    }
    // loads past the end are still in flight into the ring: let them land before the
    // ring's registers can be reused
#pragma unroll
    for (int j = 0; j < NB; ++j)
      wait_ring(std::integral_constant<int, 0>{}, sbuf[j], kbuf[j], vbuf[j], cbuf[j]);
  }
  if (fuse_new && hi - 1 >= s_lo && hi - 1 < s_hi) {   // (uniform) the newest key
    RowT kr[4], vr[4];
    float cr[4];
    kr[0] = *reinterpret_cast<const RowT *>(knew);
    vr[0] = *reinterpret_cast<const RowT *>(vnew);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      kr[k] = kr[0];
      vr[k] = vr[0];
      cr[k] = sc_new;
    }
    compute(r4 == 0 ? 1 : 0, kr, vr, cr);
  }

  if (queue) *ticket = take_ticket(queue);
  // the new token's row goes to its slot now (no wave reads it: the newest key is taken
  // from k_new/v_new), so its loads and stores overlap the reduction below
  if (store_new && r4 == 0) {
    if (a.new_slots && kvh == 0 && sub == 0) a.rtt_mut[new_at] = new_slot;
    char *kd = const_cast<char *>(kb) + static_cast<int64_t>(new_slot) * row_bytes;
    char *vd = const_cast<char *>(vb) + static_cast<int64_t>(new_slot) * row_bytes;
    *reinterpret_cast<RowT *>(kd) = *reinterpret_cast<const RowT *>(knew);
    *reinterpret_cast<RowT *>(vd) = *reinterpret_cast<const RowT *>(vnew);
    if (FP8 && kvh == 0 && sub == 0) a.kv_scale[new_slot] = sc_new;
  }
  // merge counter of this (request, KV head), read now for the single-chunk fold below
  // so that its round trip overlaps the cross-lane reduction (a stale, lower count only
  // means the ordinary path: own partial and arrival)
  int32_t *cnt = a.merge_cnt + static_cast<int64_t>(b) * a.Hkv + kvh;
  const bool may_fold = ns_tail == 1 && ns_b > 0;
  int seen = 0;
  if (may_fold && lane == 0) seen = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // merge the 4 row groups (lanes l, l^16, l^32 and l^48 hold the same dims)
#pragma unroll
  for (int mask = 16; mask <= 32; mask <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = shfl_xor_f(m[h], mask), lo_ = shfl_xor_f(l[h], mask);
      const float mn = fmaxf(m[h], mo);
      const float wa = exp2f(m[h] - mn), wb = exp2f(mo - mn);
      l[h] = l[h] * wa + lo_ * wb;
      m[h] = mn;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = acc[h][e] * wa + shfl_xor_f(acc[h][e], mask) * wb;
    }
  }

  // A single private chunk whose shared-segment partials are all written already (the
  // segment tiles run ahead of the tail waves) merges them straight into its output:
  // no partial of its own, no arrival. The counter then holds exactly ns_b arrivals and
  // no producer of this request is left, so the wave resets it.
  bool fold = false;
  if (may_fold) {
    fold = __builtin_amdgcn_readfirstlane(seen) == ns_b;
    if (fold && lane == 0) reset_counter(cnt);
  }

  // group r4 writes heads r4, r4 + 4, ...: 8 dims each
  const bool direct = expected == 1 || fold;
#pragma unroll
  for (int h = 0; h < G; ++h) {
      if ((h & 3) != r4) continue;
      const int head = kvh * G + h;
      const int d0 = sub * 8;
      float M = m[h], L = l[h];
      float O[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) O[e] = acc[h][e];
      if (fold) {   // shared partials: o normalised, lse in log2 units
        const int64_t hp = (static_cast<int64_t>(b) * a.Hq + head) * a.parts;
        for (int p0 = 0; p0 < ns_b; p0 += 4) {
          float pl[4];
          f32x4 po[4][2];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool ok = p0 + j < ns_b;
            pl[j] = ok ? ld_dev1(a.ws_lse + hp + p0 + j) : -INFINITY;
#pragma unroll
            for (int c = 0; c < 2; ++c)
              po[j][c] = ok ? ld_dev(a.ws_o + (hp + p0 + j) * D + d0 + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float mn = fmaxf(M, pl[j]);
            const float wa = __builtin_amdgcn_exp2f(M - mn), wb = __builtin_amdgcn_exp2f(pl[j] - mn);
            L = L * wa + wb;
            M = mn;
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
              for (int e = 0; e < 4; ++e) O[4 * c + e] = O[4 * c + e] * wa + po[j][c][e] * wb;
          }
        }
      }
      const bool empty = !(L > 0.f);
      const float inv = empty ? 0.f : 1.f / L;
      const float lse2 = empty ? -INFINITY : M + log2f(L);
      if (direct) {
        uint16_t *op = reinterpret_cast<uint16_t *>(a.out) + (q_row * a.Hq + head) * D + d0;
        *reinterpret_cast<u32x4 *>(op) = u32x4{pack2bf(O[0] * inv, O[1] * inv), pack2bf(O[2] * inv, O[3] * inv),
                                               pack2bf(O[4] * inv, O[5] * inv), pack2bf(O[6] * inv, O[7] * inv)};
        if (a.lse && d0 == 0) a.lse[q_row * a.Hq + head] = lse2 * kLn2;
      } else {
        const int64_t pi = (static_cast<int64_t>(b) * a.Hq + head) * a.parts + part;
        float *wp = a.ws_o + pi * D + d0;
        st_dev(wp, f32x4{O[0] * inv, O[1] * inv, O[2] * inv, O[3] * inv});
        st_dev(wp + 4, f32x4{O[4] * inv, O[5] * inv, O[6] * inv, O[7] * inv});
        if (d0 == 0) st_dev1(a.ws_lse + pi, lse2);
      }
    }
  if (direct) return;
  // arrive; the last producer merges (uniform branch: one counter per wave)
  wait_stores();
  int before = 0;
  if (lane == 0) before = arrive(cnt);
  before = __builtin_amdgcn_readfirstlane(before);
  if (before == expected - 1) {
    if (lane == 0) reset_counter(cnt);
    const int bs[1] = {b}, nps[1] = {ns_b};
    merge_requests_bf16<G, 1>(a, bs, nps, 1, kvh);
  }
}

// Private-tail decode as a work queue: the grid holds only as many blocks as fit on the
// GPU at once. Wave i first takes item i (request, split, KV head); when there are more
// items than waves, it then takes further items by ticket until it draws one past the
// end. Items differ widely in length (empty, partial and full chunks); launched as one
// block per four items, the hardware's in-order block dispatch leaves CUs idle behind
// long-running blocks, which the queue avoids.
// The queue has kTailShards counters, 128 bytes apart (atomics on one address are
// serialised, and thousands of waves draw at about the same time): wave i draws from
// shard k = i % S (S = kTailShards, or nwaves if smaller), whose ticket t names item
// nwaves + k + t * S.
// Every wave of shard k draws exactly one ticket past the shard's last item and stops,
// so the shard's counter ends at exactly (its items) + (its waves): the wave that draws
// the final value is the last to touch that counter and resets it for the next call.
constexpr int kTailShards = 16;
constexpr int kTailShardStride = 32;   // int32 elements between shard counters

__device__ __forceinline__ int32_t take_ticket(int32_t *q) {
  int32_t t = 0;
  if ((threadIdx.x & 63) == 0)
    t = __hip_atomic_fetch_add(q, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return t;   // lane 0's value; read with readfirstlane where it is used
}

template <int G, bool FP8>
__global__ __launch_bounds__(256, G >= 8 ? 1 : 2) void tail_bf16_kernel(AttnArgs a, int n_items,
                                                                        int nsplit) {
  const int total = tail_items(min(a.whole_reqs, n_items), n_items, nsplit, a.Hkv);
  const int nwaves = static_cast<int>(gridDim.x) * 4;
  int w = static_cast<int>(blockIdx.x) * 4 + static_cast<int>(threadIdx.x >> 6);
  w = __builtin_amdgcn_readfirstlane(w);
  const int shards = nwaves < kTailShards ? nwaves : kTailShards;   // each has >= 1 wave
  const int k = w % shards;
  int32_t *queue = total > nwaves ? a.tail_queue + k * kTailShardStride : nullptr;   // uniform
  // final counter value of shard k: its items past the first round plus its waves
  const int rest = total - nwaves - k;
  const int last = (rest > 0 ? (rest + shards - 1) / shards : 0) +
                   (nwaves - k + shards - 1) / shards - 1;
  while (w < total) {
    int32_t ticket = 0;
    tail_bf16_body<G, FP8>(a, w, n_items, nsplit, queue, &ticket);
    if (!queue) break;
    const int t = __builtin_amdgcn_readfirstlane(ticket);
    if (t == last && (threadIdx.x & 63) == 0)
      __hip_atomic_store(queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    w = nwaves + k + t * shards;
  }
}

// ------------------------------------------------------------------ MFMA kernel
constexpr int MF_D = 128;
constexpr int MF_BM = 128;   // query rows per four-wave block (4 waves x 32)
constexpr int MF_BN = 64;    // keys per tile
constexpr int MF_TILE = MF_BN * MF_D * 2;   // bytes of one K (or V) tile: 64 rows x 256 B

// Byte offset of 16-byte chunk c of row r in a 64 x 256-byte tile. Chunks are XOR-swizzled
// by a 4-bit function of the row so that, with 64 four-byte banks, the K operand reads
// (16 lanes = 16 consecutive rows per b128 pass) and the V transpose reads (32 lanes
// over 4 rows x 8 chunks per b64 pass) each touch every bank at most once.
__device__ __forceinline__ int mf_row_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int mf_swz(int r, int c) { return r * 256 + ((c ^ mf_row_swz(r)) << 4); }


// Direct global -> LDS load of 16 bytes per lane; NT = 1: non-temporal (cache-policy
// bit 2 of the instruction, `nt`), for rows that no other block reads.
template <int NT = 0>
__device__ __forceinline__ void lds_load16(const void *g, uint8_t *lds_base) {
  __builtin_amdgcn_global_load_lds(g, reinterpret_cast<__attribute__((address_space(3))) void *>(
                                          reinterpret_cast<uintptr_t>(lds_base)),
                                   16, 0, NT ? 2 : 0);
}

// The sixteen V^T operand reads of one 32-key block for all four 32-dim value blocks, and
// the wait for them: r[4*dvb + 2*qq + p] = transposed read at b[dvb][p] + OFF + 4096*qq
// (keys OFF/256 + 16*qq .. +15; key rows are 256 bytes apart), the key offsets as
// immediate offsets of the reads. Written as assembly: the compiler orders its own form of
// this read behind every outstanding global->LDS load (vmcnt(0)), which would wait for the
// next tile's prefetch in the middle of the current one.
template <int OFF>
__device__ __forceinline__ void lds_tr16_k32(u32x2 (&r)[16], const uint32_t (&b)[4][2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%24\n\t"
      "ds_read_b64_tr_b16 %1, %17 offset:%24\n\t"
      "ds_read_b64_tr_b16 %2, %16 offset:%25\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:%25\n\t"
      "ds_read_b64_tr_b16 %4, %18 offset:%24\n\t"
      "ds_read_b64_tr_b16 %5, %19 offset:%24\n\t"
      "ds_read_b64_tr_b16 %6, %18 offset:%25\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:%25\n\t"
      "ds_read_b64_tr_b16 %8, %20 offset:%24\n\t"
      "ds_read_b64_tr_b16 %9, %21 offset:%24\n\t"
      "ds_read_b64_tr_b16 %10, %20 offset:%25\n\t"
      "ds_read_b64_tr_b16 %11, %21 offset:%25\n\t"
      "ds_read_b64_tr_b16 %12, %22 offset:%24\n\t"
      "ds_read_b64_tr_b16 %13, %23 offset:%24\n\t"
      "ds_read_b64_tr_b16 %14, %22 offset:%25\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:%25\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
        "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
      : "v"(b[0][0]), "v"(b[0][1]), "v"(b[1][0]), "v"(b[1][1]), "v"(b[2][0]), "v"(b[2][1]),
        "v"(b[3][0]), "v"(b[3][1]), "n"(OFF), "n"(OFF + 4096)
      : "memory");
}

// Shared-segment chunks of at most this many keys stage their slot list in LDS.
constexpr int kSegSlotCap = 2048;

// 32 * NW query rows (NW waves x 32; shared-segment tiles: 4 waves) against 64-key
// tiles, bf16 MFMA 32x32x16.
//   S^T = K Q^T : A = K rows from LDS, B = Q in registers; a lane holds one query row
//                 (column) and 16 keys, so the row softmax is lane-local plus one
//                 exchange with lane ^ 32.
//   O^T += V^T P^T : A = V^T read from the row-major V tile with the LDS transpose read
//                 (ds_read_b64_tr_b16), B = P straight from the S^T registers (the key
//                 order inside each 16-key step is permuted identically on both sides).
// K/V tiles go global -> LDS with direct 16-byte loads, two stages: tile t+1 is in flight
// while tile t is multiplied. Query rows are a request's new tokens x heads (extend,
// causal) or the members of a shared radix segment x heads (decode partials).
template <int G, bool SEG, bool FP8, int NW = 4>
__device__ __forceinline__ void mfma_body(const AttnArgs &a, int tile, int item, int kvh,
                                          uint8_t (*smem)[2][MF_TILE], int32_t *slot_lds = nullptr) {
  static_assert(NW == 4 || (NW == 8 && !SEG), "segment tiles use four waves");
  constexpr int BM = 32 * NW;    // query rows per block
  constexpr int RPW = 64 / NW;   // rows of each 64-key tile that one wave loads
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;

  int lo, hi, mem_off = 0, nrows, P = 0, b = 0, ks = 0;
  const int32_t *rtt_row;
  if (!SEG) {
    b = item;
    P = a.prefix_lens[b];
    const int E = a.extend_lens[b];
    nrows = E * G;
    if (tile * BM >= nrows) return;
    const int i_last = min(E - 1, (tile * BM + BM - 1) / G);
    lo = 0;
    hi = P + i_last + 1;
    rtt_row = rtt_row_of(a, b);
  } else {
    // item = one key chunk of a segment: its record gives the key range, members and
    // slot row in one (uniform) load
    const int32_t *rec = a.seg_items + static_cast<int64_t>(item) * 8;
    lo = rec[0];
    hi = rec[1];
    mem_off = rec[2];
    nrows = rec[3] * G;
    ks = rec[6];
    if (tile * BM >= nrows) return;
    rtt_row = rtt_row_of(a, rec[4]);
  }

  // this lane's query row
  const int R = tile * BM + wave * 32 + n;
  const int qi = R / G, hg = R % G;
  const bool rvalid = R < nrows;
  int64_t q_tok;
  int qpos;
  if (!SEG) {
    q_tok = a.cu_extend[b] + (rvalid ? qi : 0);
    qpos = P + qi;
  } else {
    q_tok = rvalid ? a.seg_members[mem_off + qi] : 0;
    qpos = 0x7fffffff;
  }
  const int head = kvh * G + hg;

  bf16x8 qb[MF_D / 16];
  {
    const uint16_t *qp = reinterpret_cast<const uint16_t *>(a.q) + (q_tok * a.Hq + head) * MF_D + 8 * h;
#pragma unroll
    for (int s = 0; s < MF_D / 16; ++s) {
      const u32x4 w = rvalid ? ldg16(qp + 16 * s) : u32x4{0, 0, 0, 0};
      qb[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  // running max of the scaled scores (log2 domain) and the row sum; the max is kept
  // stale until a tile's maximum exceeds it by more than 2^8 (numerator and denominator
  // share it, so the result is the same and the accumulators are rarely rescaled)
  float m_run = kNegBig, l_run = 0.f;
  const float sc = a.scale_log2;   // > 0
  // first query position among this wave's rows: tiles wholly at or before it need no
  // causal mask (wave-uniform)
  const int wave_q0 = SEG ? 0x7fffffff : P + (tile * BM + wave * 32) / G;
  const bool wave_active = tile * BM + wave * 32 < nrows;   // wave-uniform

  // loaders: wave w fills rows 16w .. 16w+15 of each tile, 4 rows per instruction;
  // lane i lands at byte 16*i of the instruction's 1 KB, i.e. row +i/16, physical chunk
  // i%16, so it fetches logical chunk (i%16) ^ mf_row_swz(row) of that row.
  // fp8 K/V: rows of 128 bytes. Wave w stages its rows 16w .. 16w+15 raw, eight rows per
  // direct load (lane i: row +i/8, 16-byte chunk i%8) into one linear staging tile, then
  // converts those same chunks (times the row's scale, rounded to bf16) into the swizzled
  // bf16 tile that the matrix code below reads; the bf16 tile is single-buffered (the next
  // tile's raw bytes are in flight in the staging tile while it is used).
  constexpr int EB = FP8 ? 1 : 2;
  constexpr int NSL = FP8 ? RPW / 8 : RPW / 4;   // slot-list entries per lane per tile
  const int64_t row_bytes = static_cast<int64_t>(a.Hkv) * MF_D * EB;
  const char *kb = reinterpret_cast<const char *>(a.k_pool) + kvh * MF_D * EB;
  const char *vb = reinterpret_cast<const char *>(a.v_pool) + kvh * MF_D * EB;
  uint8_t *stg = smem[1][0];   // fp8 staging: K rows 0..63 (8 KB), then V rows
  const int last = hi - 1;
  int32_t sl[NSL];
  float rsc[NSL];   // fp8: scales of the rows this lane stages
  auto load_slots = [&](int kt) {
#pragma unroll
    for (int j = 0; j < NSL; ++j) {
      const int r = FP8 ? wave * RPW + 8 * j + (lane >> 3) : wave * RPW + 4 * j + (lane >> 4);
      sl[j] = rtt_row[min(kt + r, last)];
    }
  };
  // byte offset of a slot's row plus this lane's chunk: one unsigned 32 x 32 -> 64-bit
  // multiply-add (slots are non-negative), shared by the K and V loads
  auto row_off = [&](int32_t slot, uint32_t chunk_bytes) {
    return static_cast<uint64_t>(static_cast<uint32_t>(slot)) * static_cast<uint32_t>(row_bytes) +
           chunk_bytes;
  };
  // a shared-segment chunk with a single tile of rows is the only reader of its K/V
  // rows: those loads go non-temporal (agent decode step ≈ 7 % faster); chunks read by
  // several row tiles, and extend tiles, keep them in the XCD's L2 for the other tiles
  const bool nt_rows = SEG && nrows <= BM;   // block-uniform
  auto issue = [&](int stage) {
#pragma unroll
    for (int j = 0; j < NSL; ++j) {
      if constexpr (FP8) {
        const uint64_t off = row_off(sl[j], (lane & 7) * 16u);
        if (nt_rows) {
          lds_load16<1>(kb + off, stg + (wave * RPW + 8 * j) * 128);
          lds_load16<1>(vb + off, stg + 8192 + (wave * RPW + 8 * j) * 128);
        } else {
          lds_load16(kb + off, stg + (wave * RPW + 8 * j) * 128);
          lds_load16(vb + off, stg + 8192 + (wave * RPW + 8 * j) * 128);
        }
        rsc[j] = a.kv_scale[sl[j]];
      } else {
        const int r = wave * RPW + 4 * j + (lane >> 4);
        const int c = (lane & 15) ^ mf_row_swz(r);
        const uint64_t off = row_off(sl[j], c * 16u);
        if (nt_rows) {
          lds_load16<1>(kb + off, &smem[stage][0][(wave * RPW + 4 * j) * 256]);
          lds_load16<1>(vb + off, &smem[stage][1][(wave * RPW + 4 * j) * 256]);
        } else {
          lds_load16(kb + off, &smem[stage][0][(wave * RPW + 4 * j) * 256]);
          lds_load16(vb + off, &smem[stage][1][(wave * RPW + 4 * j) * 256]);
        }
      }
    }
  };
  // fp8: staged chunks of this lane -> bf16 tile (the caller has waited for the loads)
  auto convert = [&]() {
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < NSL; ++j) {
        const int r = wave * RPW + 8 * j + (lane >> 3), c = lane & 7;
#pragma unroll
        for (int kv = 0; kv < 2; ++kv) {
          const u32x4 raw = *reinterpret_cast<const u32x4 *>(stg + kv * 8192 + r * 128 + c * 16);
          u32x4 lo16, hi16;
          fp8x16_to_bf16(raw, rsc[j], lo16, hi16);
          *reinterpret_cast<u32x4 *>(&smem[0][kv][mf_swz(r, 2 * c)]) = lo16;
          *reinterpret_cast<u32x4 *>(&smem[0][kv][mf_swz(r, 2 * c + 1)]) = hi16;
        }
      }
    }
  };

  // ---- one 64-key tile, as two 32-key blocks mb = 0, 1 whose phases overlap: block 1's
  // scores are formed on the matrix cores while block 0's softmax runs on the vector
  // ALUs, and block 0's PV products while block 1's softmax runs (the two interleaved
  // instruction by instruction), so a wave keeps both units busy by itself.
  // Ragged or causal-diagonal block: keys past the range or past the row's position -> -inf.
  auto mask = [&](f32x16 &sb, int kb0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kb0 + 8 * (i >> 2) + 4 * h + (i & 3);
      sb[i] = (key < hi && key <= qpos) ? sb[i] : -INFINITY;
    }
  };
  // P of block mb against the running maximum as it stands, packed to bf16 for the PV
  // product, and its fp32 row sum (two chains; this lane's 16 keys). The maximum is
  // raised, and the accumulators rescaled, only when some lane's probabilities in the
  // block sum past 2^8 or overflow (the first block, whose maximum is still the start
  // value): every p is at most that sum, so p <= 2^8 whenever the block is kept.
  bf16x8 pb[2][2];
  auto exp_pack = [&](const f32x16 &sb, int mb) {
    float ra = 0.f, rb = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 8 * j + 2 * e;
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sb[i], sc, -m_run));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sb[i + 1], sc, -m_run));
        w[e] = pack2bf(p0, p1);
        ra += p0;
        rb += p1;
      }
      pb[mb][j] = __builtin_bit_cast(bf16x8, w);
    }
    return ra + rb;
  };
  auto softmax_tail = [&](const f32x16 &sb, int mb, float rs) {
    if (__builtin_amdgcn_ballot_w64(!(rs <= 256.f)) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sb[i], sb[i + 1]));
      mx = fmaxf(mx, xor32(mx)) * sc;
      const float mn = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d) o[d] *= alpha;
      rs = exp_pack(sb, mb);
    }
    l_run += rs;   // this half-wave's keys; the halves are added once, after the loop
  };
  // V^T operand: in each 16-lane group g, source lane s reads 4 dims of key row
  // base + 4*(g>>1) + (s>>2) (+8 for the second read); the transpose hands lane s the
  // 4 keys of value dim 16*(g&1) + s of the 32-dim block. Chunk of value block dvb =
  // 4*dvb + cl, and rows 16q + x (x < 16) share x's swizzle: one lane base per (dvb, row
  // vrow0 or vrow0 + 8), keys 16q as constant offsets of the reads.
  const int vg = lane >> 4, vs16 = lane & 15;
  const int vrow0 = 4 * (vg >> 1) + (vs16 >> 2);
  const int vcl = 2 * (vg & 1) + ((vs16 & 3) >> 1), vhalf = vs16 & 1;
  auto v_bases = [&](const uint8_t *Vt, uint32_t (&vbs)[4][2]) {
    const uint32_t vbase = lds_addr(Vt);
#pragma unroll
    for (int dvb = 0; dvb < 4; ++dvb)
#pragma unroll
      for (int p = 0; p < 2; ++p) vbs[dvb][p] = vbase + mf_swz(vrow0 + 8 * p, 4 * dvb + vcl) + 8 * vhalf;
  };
  // O^T += V^T P^T over block mb's keys (16-key steps q = 2mb, 2mb + 1): rv[4*dvb + 2*qq + p]
  // holds the transposed read at base (dvb, p), keys 16*(2mb + qq)
  auto pv = [&](const u32x2 (&rv)[16], int mb) {
#pragma unroll
    for (int dvb = 0; dvb < 4; ++dvb)
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const u32x4 w = u32x4{rv[4 * dvb + 2 * qq][0], rv[4 * dvb + 2 * qq][1],
                              rv[4 * dvb + 2 * qq + 1][0], rv[4 * dvb + 2 * qq + 1][1]};
        o[dvb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pb[mb][qq],
                                                         o[dvb], 0, 0, 0);
      }
  };

  // the matrix and softmax work of one 64-key tile in LDS stage `stage`; DIAG: ragged or
  // causal-diagonal tile (a compile-time variant, so each body is one straight block in
  // which the scheduler can interleave the two units' instructions)
  auto tile_body = [&](auto DIAG, int kt, int stage) {
    // DIAG: std::true_type / std::false_type, or a run-time bool (fp8 extend, whose
    // conversion pass leaves no registers for two copies of the body)
    auto maybe_mask = [&](f32x16 &sb, int kb0) {
      if constexpr (std::is_same<decltype(DIAG), bool>::value) {
        if (DIAG) mask(sb, kb0);
      } else if constexpr (decltype(DIAG)::value) {
        mask(sb, kb0);
      }
    };
    const uint8_t *Kt = smem[stage][0];
    uint32_t vbs[4][2];
    v_bases(smem[stage][1], vbs);
    f32x16 st0, st1;
    bf16x8 ka[MF_D / 16];
    // S^T of block 0; each K operand of block 0 is refilled with block 1's right after
    // the MFMA that used it, so the reads overlap the MFMAs
#pragma unroll
    for (int s = 0; s < MF_D / 16; ++s)
      ka[s] = *reinterpret_cast<const bf16x8 *>(Kt + mf_swz(n, 2 * s + h));
    st0 = f32x16{};
#pragma unroll
    for (int s = 0; s < MF_D / 16; ++s) {
      st0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qb[s], st0, 0, 0, 0);
      ka[s] = *reinterpret_cast<const bf16x8 *>(Kt + mf_swz(32 + n, 2 * s + h));
    }
    // block 1's scores on the matrix cores, block 0's softmax on the vector ALUs
    st1 = f32x16{};
#pragma unroll
    for (int s = 0; s < MF_D / 16; ++s)
      st1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qb[s], st1, 0, 0, 0);
    if constexpr (FP8 && !SEG) {
      // fp8 extend (its mask test is a branch): the two blocks one after the other
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int s = 0; s < MF_D / 16; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      maybe_mask(st0, kt);
      maybe_mask(st1, kt + 32);
      softmax_tail(st0, 0, exp_pack(st0, 0));
      softmax_tail(st1, 1, exp_pack(st1, 1));
      u32x2 rv[16];
      lds_tr16_k32<0>(rv, vbs);
      pv(rv, 0);
      lds_tr16_k32<8192>(rv, vbs);
      pv(rv, 1);
      return;
    }
    maybe_mask(st0, kt);
    float rs = exp_pack(st0, 0);
    // 8 LDS reads, (MFMA, LDS read) x 8, then (MFMA, 7 vector instructions) x 8
    // (masks: 0x100 LDS read, 0x008 MFMA, 0x002 VALU)
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int s = 0; s < MF_D / 16; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int s = 0; s < MF_D / 16; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
    }
    softmax_tail(st0, 0, rs);
    // V^T operands of keys 0..31 and 32..63
    u32x2 rv0[16], rv1[16];
    lds_tr16_k32<0>(rv0, vbs);
    lds_tr16_k32<8192>(rv1, vbs);
    // block 0's PV products on the matrix cores, block 1's softmax on the vector ALUs
    pv(rv0, 0);
    maybe_mask(st1, kt + 32);
    rs = exp_pack(st1, 1);
#pragma unroll
    for (int s = 0; s < MF_D / 16; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
    }
    softmax_tail(st1, 1, rs);
    pv(rv1, 1);
  };
  // one 64-key tile in LDS stage `stage` (the other stage receives the next tile)
  auto tile_step = [&](auto DIAG, int kt, int stage) {
    const bool more = kt + MF_BN < hi;
    if (more) {
      issue(stage ^ 1);
      if (kt + 2 * MF_BN < hi) load_slots(kt + 2 * MF_BN);
    }
    // a wave whose 32 rows are all past the block's rows (small shared segments) only
    // loads (and, fp8, converts) its share of each tile and keeps the barriers, leaving
    // the SIMD to others
    if (wave_active) tile_body(DIAG, kt, stage);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (FP8 && more) {   // the next tile's bytes have landed and nobody reads this tile now
      convert();
      lds_barrier();
    }
  };
  // Tiles starting at or before `lim` are whole and wholly at or before this wave's first
  // query position, so they need no mask; the ragged or causal-diagonal ones come last.
  // Waves differ in where they switch to the masked body, but all run the same tiles and
  // barriers.
  const int lim = min(hi - MF_BN, wave_q0 - (MF_BN - 1));
  bool ring = false;
  if constexpr (SEG && !FP8)   // (uniform) chunks of one row tile
    ring = slot_lds != nullptr && hi - lo <= kSegSlotCap && nrows <= BM;
  if (ring) {
    // Shared-segment chunk of one row tile, bf16: its tiles wait on memory, not on the
    // matrix cores, so the chunk runs as 32-key tiles through a four-deep ring (three
    // tiles, 48 KB, in flight instead of one 64-key tile). Its slot list is staged in LDS
    // first, so the loop issues only tile loads and waits for exact counts of them.
    // (Chunks of several row tiles keep the 64-key tiles, whose two blocks overlap their
    // matrix and softmax work.)
    const int n32 = (hi - lo + 31) / 32;
    for (int c = wave; c < (n32 + 1) / 2; c += 4)   // 64 entries per wave instruction
      __builtin_amdgcn_global_load_lds(rtt_row + min(lo + 64 * c + lane, last),
                                       reinterpret_cast<__attribute__((address_space(3))) void *>(
                                           reinterpret_cast<uintptr_t>(slot_lds + 64 * c)),
                                       4, 0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint8_t *ring_lds = smem[0][0];   // stage s: K at 16 KB * s, V 8 KB after it
    auto issue32 = [&](int t, int stage) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // lane i lands at byte 16*i of the 4-row group (row +i/16, physical chunk i%16)
        const int r = wave * 8 + 4 * j + (lane >> 4);
        const uint64_t off = row_off(slot_lds[32 * t + r], ((lane & 15) ^ mf_row_swz(r)) * 16u);
        uint8_t *dst = ring_lds + 16384 * stage + (wave * 8 + 4 * j) * 256;
        if (nt_rows) {
          lds_load16<1>(kb + off, dst);
          lds_load16<1>(vb + off, dst + 8192);
        } else {
          lds_load16(kb + off, dst);
          lds_load16(vb + off, dst + 8192);
        }
      }
    };
    // waits until at most n later tiles' loads (4 per lane each) are outstanding
    auto wait_tiles = [&](int n) {
      if (n >= 2)
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else if (n == 1)
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    // (barriers that leave later tiles' loads in flight: __syncthreads() would wait for
    // them; a tile's own loads are waited for explicitly first)
    for (int t = 0; t < 3 && t < n32; ++t) issue32(t, t);
    wait_tiles(min(n32, 3) - 1);
    lds_barrier();
    for (int t = 0; t < n32; ++t) {
      if (t + 3 < n32) issue32(t + 3, (t + 3) & 3);
      if (wave_active) {
        const int kt = lo + 32 * t;
        const uint8_t *Kt = ring_lds + 16384 * (t & 3);
        bf16x8 ka[MF_D / 16];
#pragma unroll
        for (int s = 0; s < MF_D / 16; ++s)
          ka[s] = *reinterpret_cast<const bf16x8 *>(Kt + mf_swz(n, 2 * s + h));
        f32x16 st0 = f32x16{};
#pragma unroll
        for (int s = 0; s < MF_D / 16; ++s)
          st0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qb[s], st0, 0, 0, 0);
        if (kt + 32 > hi) mask(st0, kt);   // (uniform) ragged last tile
        softmax_tail(st0, 0, exp_pack(st0, 0));
        uint32_t vbs[4][2];
        v_bases(Kt + 8192, vbs);
        u32x2 rv[16];
        lds_tr16_k32<0>(rv, vbs);
        pv(rv, 0);
      }
      wait_tiles(min(n32 - 1, t + 3) - (t + 1));   // tile t+1 has landed
      lds_barrier();
    }
  } else {
  if (lo < hi) {
    load_slots(lo);
    issue(0);
    if (lo + MF_BN < hi) load_slots(lo + MF_BN);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (FP8 && lo < hi) {
    convert();
    lds_barrier();
  }
  if constexpr (SEG) {
    int kt = lo, t = 0;
    for (; kt <= lim; kt += MF_BN, ++t) tile_step(std::false_type{}, kt, FP8 ? 0 : t & 1);
    for (; kt < hi; kt += MF_BN, ++t) tile_step(std::true_type{}, kt, FP8 ? 0 : t & 1);
  } else if constexpr (FP8) {
    for (int kt = lo; kt < hi; kt += MF_BN) tile_step(kt > lim, kt, 0);
  } else {
    // extend: two tiles per trip, so each copy's LDS stage (and with it the operand
    // addresses' stage offset) is a constant
    int kt = lo;
    for (; kt + MF_BN <= lim; kt += 2 * MF_BN) {
      tile_step(std::false_type{}, kt, 0);
      tile_step(std::false_type{}, kt + MF_BN, 1);
    }
    for (; kt + MF_BN < hi; kt += 2 * MF_BN) {
      tile_step(std::true_type{}, kt, 0);
      tile_step(std::true_type{}, kt + MF_BN, 1);
    }
    if (kt < hi) tile_step(std::true_type{}, kt, 0);
  }
  }

  l_run += xor32(l_run);
  if (!SEG && !rvalid) return;
  const bool empty = !(l_run > 0.f);
  const float inv = empty ? 0.f : 1.f / l_run;
  const float lse2 = empty ? -INFINITY : m_run + log2f(l_run);
  if (!SEG) {
    uint16_t *op = reinterpret_cast<uint16_t *>(a.out) + (q_tok * a.Hq + head) * MF_D;
#pragma unroll
    for (int dvb = 0; dvb < 4; ++dvb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dv = dvb * 32 + 8 * g4 + 4 * h;
        const u32x2 w = u32x2{pack_bf16x2(o[dvb][4 * g4] * inv, o[dvb][4 * g4 + 1] * inv),
                              pack_bf16x2(o[dvb][4 * g4 + 2] * inv, o[dvb][4 * g4 + 3] * inv)};
        *reinterpret_cast<u32x2 *>(op + dv) = w;
      }
    if (a.lse && h == 0) a.lse[q_tok * a.Hq + head] = lse2 * kLn2;
  } else {
    // partial of this key range for every member row, then one arrival per member
    // request (its head-0 lane); a member whose other producers have all arrived is
    // merged here by the whole wave
    // the lanes that arrive for a member request read its partial count now, so that
    // load overlaps the partial stores
    const bool arriver = rvalid && hg == 0 && h == 0;
    const int np_q = arriver ? a.req_num_parts[q_tok] : 0;
    int last_b = -1;
    if (rvalid) {
      const int part = a.seg_member_part[mem_off + qi] + ks;
      const int64_t pi = (q_tok * a.Hq + head) * a.parts + part;
      float *wp = a.ws_o + pi * MF_D;
#pragma unroll
      for (int dvb = 0; dvb < 4; ++dvb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dv = dvb * 32 + 8 * g4 + 4 * h;
          st_dev(wp + dv, f32x4{o[dvb][4 * g4] * inv, o[dvb][4 * g4 + 1] * inv,
                                o[dvb][4 * g4 + 2] * inv, o[dvb][4 * g4 + 3] * inv});
        }
      if (h == 0) st_dev1(a.ws_lse + pi, lse2);
    }
    wait_stores();
    if (arriver) {
      const int bq = static_cast<int>(q_tok);
      int32_t *cnt = a.merge_cnt + static_cast<int64_t>(bq) * a.Hkv + kvh;
      if (arrive(cnt) == np_q + tail_parts(a, bq) - 1) {
        reset_counter(cnt);
        last_b = bq;
      }
    }
    // requests this wave completed, merged NR at a time (fewer for 8 heads per KV head,
    // whose merge pass covers two 512-value halves)
    constexpr int NR = G >= 8 ? 2 : 4;
    uint64_t pending = __builtin_amdgcn_ballot_w64(last_b >= 0);
    while (pending) {
      int bs[NR], nps[NR], n = 0;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (pending) {
          const int l = __builtin_ctzll(pending);
          pending &= pending - 1;
          bs[r] = __builtin_amdgcn_readlane(last_b, l);
          nps[r] = __builtin_amdgcn_readlane(np_q, l);
          ++n;
        } else {
          bs[r] = bs[0];
          nps[r] = nps[0];
        }
      }
      merge_requests_bf16<G, NR>(a, bs, nps, n, kvh);
    }
  }
}

// Blocks of one launch in 1-D order: consecutive logical blocks (the tiles that read the
// same K/V rows) are placed on the same XCD, since block b runs on XCD b % 8.
__device__ __forceinline__ int xcd_logical(int bid, int nblocks) {
  const int per = (nblocks + 7) / 8;
  return (bid & 7) * per + (bid >> 3);
}

// Blocks of the shared-segment part of a fused decode launch: every XCD gets room for
// ceil(groups / 8) groups of `tiles` blocks.
__host__ __device__ __forceinline__ int seg_block_count(int tiles, int groups) {
  return 8 * tiles * ((groups + 7) / 8);
}

// extend: logical block -> (tile, request, kvh), tile fastest and in decreasing order:
// a causal request's last row tiles have the most keys, and dispatching them first keeps
// the launch from ending on its longest blocks. NW waves (32 * NW query rows) share each
// K/V tile; launched with four (the eight-wave tiles run in the persistent kernel below)
template <int G, bool FP8, int NW>
__global__ __launch_bounds__(64 * NW, 2) void attn_mfma_kernel(AttnArgs a, int tiles, int items) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2][2][MF_TILE];   // [stage][K, V]
  const int nblocks = tiles * items * a.Hkv;
  const int lb = xcd_logical(blockIdx.x, nblocks);
  if (lb >= nblocks) return;
  mfma_body<G, false, FP8, NW>(a, tiles - 1 - lb % tiles, (lb / tiles) % items,
                               lb / (tiles * items), smem);
}

// Persistent extend with eight-wave blocks, as many as are resident at once (P per XCD).
// The logical blocks are split into 8 contiguous ranges, one per XCD as the non-persistent
// launch maps them; block j of an XCD walks its range in snake order (j, 2P-1-j, 2P+j,
// 4P-1-j, ...), so that the long row tiles (late query rows see more keys) and the short
// ones of the same requests share out evenly, and it skips row tiles past a request's end.
template <int G, bool FP8>
__global__ __launch_bounds__(512, 2) void attn_mfma_persist_kernel(AttnArgs a, int tiles, int items) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2][2][MF_TILE];   // [stage][K, V]
  const int nblocks = tiles * items * a.Hkv;
  const int per = (nblocks + 7) / 8;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3, P = gridDim.x >> 3;
  // logical block k of this block's walk, or -1 past its end (the walk is increasing)
  auto at = [&](int k) {
    const int idx = (k & 1) ? (k + 1) * P - 1 - j : k * P + j;
    const int lb = xcd * per + idx;
    return idx < per && lb < nblocks ? lb : -1;
  };
  bool first = true;
  for (int k = 0;; ++k) {
    const int lb = at(k);
    if (lb < 0) break;
    const int tile = tiles - 1 - lb % tiles, item = (lb / tiles) % items;
    // a row tile is 256 query rows (8 waves x 32); past the request's rows: skip
    if (tile * 256 >= a.extend_lens[item] * G) continue;   // block-uniform
    // every wave is done with the previous row tile's K/V before this one's loads land
    if (!first) lds_barrier();
    first = false;
    mfma_body<G, false, FP8, 8>(a, tile, item, lb / (tiles * items), smem);
  }
}

// One decode step with a plan: blocks [0, seg_blocks) are shared-segment MFMA tiles,
// the rest are private-tail waves (4 per block); both write partials, and the last
// producer of each (request, KV head) merges them into the output (arrival counter).
// Matrix-core work and the memory-bound tail overlap.
template <int G, bool FP8>
__global__ __launch_bounds__(256, 2) void decode_fused_kernel(AttnArgs a, int tiles, int seg_items,
                                                             int n_items, int nsplit) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2][2][MF_TILE];
  __shared__ int32_t slot_lds[kSegSlotCap];
  const int groups = seg_items * a.Hkv;   // (chunk, KV head) pairs, `tiles` blocks each
  const int seg_blocks = seg_block_count(tiles, groups);
  if (static_cast<int>(blockIdx.x) < seg_blocks) {
    // Block b runs on XCD b % 8 as the (b / 8)-th there. Group g = (chunk, KV head), KV
    // head fastest, chunks in plan order (longest keys first), goes to XCD g % 8 whole:
    // its tiles read the same K/V rows, through one L2. The longest groups are dispatched
    // first on every XCD.
    const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
    const int g = xcd + 8 * (k / tiles);
    if (g >= groups) return;
    mfma_body<G, true, FP8>(a, k % tiles, g / a.Hkv, g % a.Hkv, smem, FP8 ? nullptr : slot_lds);
  } else {
    tail_bf16_body<G, FP8>(a, (blockIdx.x - seg_blocks) * 4 + (threadIdx.x >> 6), n_items, nsplit);
  }
}

// ------------------------------------------------------------------ combine
// Merges the partials of every (request, head) into the output. One wave covers 256
// consecutive values of a request's [Hq, Dv] output (lane: 4 dims of one head); the
// partials are taken 8 at a time with all their loads issued before any is used, and
// folded into a running (M, L, O) in the log2 domain. An empty partial has lse -inf and
// weight exactly 0 (its stored values are not read into the sum).
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a, int Dv, int batch) {
  const int lane = threadIdx.x & 63;
  const int per_req = (a.Hq * Dv + 255) / 256;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= batch * per_req) return;
  const int b = w / per_req;
  const int e = (w % per_req) * 256 + lane * 4;
  if (e >= a.Hq * Dv) return;
  const int head = e / Dv, d = e % Dv;
  const int ns = a.req_num_parts ? a.req_num_parts[b] : 0;
  const int total = ns + tail_parts(a, b);
  const int64_t base = (static_cast<int64_t>(b) * a.Hq + head) * a.parts;
  float M = kNegBig, L = 0.f;
  f32x4 O = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < total; p0 += 8) {
    float pl[8];
    f32x4 po[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = p0 + j;
      const int64_t pi = base + (idx < ns ? idx : a.part_base + idx - ns);
      const bool ok = idx < total;
      pl[j] = ok ? a.ws_lse[pi] : -INFINITY;
      po[j] = ok ? *reinterpret_cast<const f32x4 *>(a.ws_o + pi * Dv + d) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mx = M;
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, pl[j]);
    const float alpha = exp2f(M - mx);
    L *= alpha;
    O *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float wj = exp2f(pl[j] - mx);
      L += wj;
      const f32x4 c = wj > 0.f ? po[j] * wj : f32x4{0.f, 0.f, 0.f, 0.f};
      O += c;
    }
    M = mx;
  }
  const float inv = 1.f / L;
  store_out4<T>(a.out, (static_cast<int64_t>(b) * a.Hq + head) * Dv + d, O * inv);
  if (a.lse && d == 0) a.lse[static_cast<int64_t>(b) * a.Hq + head] = (M + log2f(L)) * kLn2;
}

}  // namespace

// ====================================================================== launchers
namespace radix_launch {

hipError_t kv_store(const StoreArgs &a, int64_t T, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  launch(kv_store_kernel, dim3(static_cast<unsigned>(T)), dim3(128), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D, int G>
static hipError_t launch_valu(int mode, const AttnArgs &a, unsigned items, unsigned splits,
                              hipStream_t stream) {
  const uint64_t waves = static_cast<uint64_t>(items) * splits * a.Hkv;
  if (waves > 0x7fffffffull) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>((waves + 3) / 4)), block(256);
  const int n = static_cast<int>(items), ns = static_cast<int>(splits);
  if (mode == 0) launch(attn_valu_kernel<T, D, G, 0>, grid, block, 0, stream, a, n, ns);
  else if (mode == 1) launch(attn_valu_kernel<T, D, G, 1>, grid, block, 0, stream, a, n, ns);
  else if (mode == 2) launch(attn_valu_kernel<T, D, G, 2>, grid, block, 0, stream, a, n, ns);
  else launch(attn_valu_kernel<T, D, G, 3>, grid, block, 0, stream, a, n, ns);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t valu_g(int G, int mode, const AttnArgs &a, unsigned items, unsigned splits,
                         hipStream_t s) {
  switch (G) {
    case 1: return launch_valu<T, D, 1>(mode, a, items, splits, s);
    case 2: return launch_valu<T, D, 2>(mode, a, items, splits, s);
    case 4: return launch_valu<T, D, 4>(mode, a, items, splits, s);
    case 8: return launch_valu<T, D, 8>(mode, a, items, splits, s);
  }
  return hipErrorInvalidValue;
}

template <int G, bool FP8>
static hipError_t launch_tail(const AttnArgs &a, unsigned items, unsigned splits, hipStream_t stream) {
  if (static_cast<uint64_t>(items) * splits * a.Hkv > 0x7fffffffull) return hipErrorInvalidValue;
  const int whole = a.whole_reqs < static_cast<int>(items) ? a.whole_reqs : static_cast<int>(items);
  const uint64_t waves = tail_items(whole, static_cast<int>(items), static_cast<int>(splits), a.Hkv);
  if (!a.tail_queue) return hipErrorInvalidValue;
  // blocks resident at once on this device (cached per device)
  static std::atomic<int> resident[64];   // one table per kernel instantiation
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int fit = dev < 64 ? resident[dev].load(std::memory_order_relaxed) : 0;
  if (fit == 0) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, tail_bf16_kernel<G, FP8>, 256, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    fit = per_cu * cus > 0 ? per_cu * cus : 1;
    if (dev < 64) resident[dev].store(fit, std::memory_order_relaxed);
  }
  const uint64_t blocks = (waves + 3) / 4;
  dim3 grid(static_cast<unsigned>(blocks < static_cast<uint64_t>(fit) ? blocks : fit)), block(256);
  const int n = static_cast<int>(items), ns = static_cast<int>(splits);
  launch(tail_bf16_kernel<G, FP8>, grid, block, 0, stream, a, n, ns);
  return hipGetLastError();
}

template <bool FP8>
static hipError_t tail_g(int G, const AttnArgs &a, unsigned batch, unsigned splits, hipStream_t s) {
  switch (G) {
    case 1: return launch_tail<1, FP8>(a, batch, splits, s);
    case 2: return launch_tail<2, FP8>(a, batch, splits, s);
    case 4: return launch_tail<4, FP8>(a, batch, splits, s);
    case 8: return launch_tail<8, FP8>(a, batch, splits, s);
  }
  return hipErrorInvalidValue;
}

hipError_t decode_tail_bf16(int G, bool fp8, const AttnArgs &a, unsigned batch, unsigned splits,
                            hipStream_t s) {
  if (batch == 0) return hipSuccess;
  return fp8 ? tail_g<true>(G, a, batch, splits, s) : tail_g<false>(G, a, batch, splits, s);
}

hipError_t valu(bool bf16, int G, int mode, const AttnArgs &a, unsigned items, unsigned splits,
                hipStream_t s) {
  if (items == 0) return hipSuccess;
  return bf16 ? valu_g<uint16_t, 128>(G, mode, a, items, splits, s)
              : valu_g<float, 64>(G, mode, a, items, splits, s);
}

// Compute units of the current device (cached per device; 256 if the query fails).
static int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  int c = dev < 64 ? cached[dev].load(std::memory_order_relaxed) : 0;
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      return 256;
    if (dev < 64) cached[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

template <int G, bool FP8, int NW>
static hipError_t launch_mfma(const AttnArgs &a, int max_rows, unsigned items, hipStream_t s) {
  const unsigned tiles = static_cast<unsigned>((max_rows + 32 * NW - 1) / (32 * NW));
  const uint64_t n = static_cast<uint64_t>(tiles) * items * a.Hkv;
  if (n > 0x7fffffffull) return hipErrorInvalidValue;
  if constexpr (NW == 8) {
    // persistent: the blocks resident at once on this device (cached per device),
    // rounded down to a multiple of the 8 XCDs
    static std::atomic<int> resident[64];   // one table per kernel instantiation
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int fit = dev < 64 ? resident[dev].load(std::memory_order_relaxed) : 0;
    if (fit == 0) {
      int per_cu = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_mfma_persist_kernel<G, FP8>, 512, 0);
      if (e != hipSuccess) return e;
      fit = per_cu * device_cus() >= 8 ? per_cu * device_cus() : 8;
      if (dev < 64) resident[dev].store(fit, std::memory_order_relaxed);
    }
    const uint64_t per = (n + 7) / 8, pmax = static_cast<uint64_t>(fit / 8);
    dim3 grid(static_cast<unsigned>(8 * (per < pmax ? per : pmax))), block(512);
    launch(attn_mfma_persist_kernel<G, FP8>, grid, block, 0, s, a, static_cast<int>(tiles),
           static_cast<int>(items));
  } else {
    dim3 grid(static_cast<unsigned>(8 * ((n + 7) / 8))), block(64 * NW);
    launch(attn_mfma_kernel<G, FP8, NW>, grid, block, 0, s, a, static_cast<int>(tiles),
           static_cast<int>(items));
  }
  return hipGetLastError();
}

template <int G, bool FP8>
static hipError_t launch_fused(const AttnArgs &a, unsigned tiles, unsigned seg_items,
                               unsigned n_items, unsigned nsplit, hipStream_t s) {
  const uint64_t groups = static_cast<uint64_t>(seg_items) * a.Hkv;
  const uint64_t seg_blocks = 8ull * tiles * ((groups + 7) / 8);   // = seg_block_count()
  if (seg_blocks > 0x7fffffffull) return hipErrorInvalidValue;
  if (static_cast<uint64_t>(n_items) * nsplit * a.Hkv > 0x7fffffffull) return hipErrorInvalidValue;
  const int whole = a.whole_reqs < static_cast<int>(n_items) ? a.whole_reqs : static_cast<int>(n_items);
  const uint64_t tail_blocks =
      (tail_items(whole, static_cast<int>(n_items), static_cast<int>(nsplit), a.Hkv) + 3ull) / 4;
  if (seg_blocks + tail_blocks > 0x7fffffffull) return hipErrorInvalidValue;
  launch(decode_fused_kernel<G, FP8>, dim3(static_cast<unsigned>(seg_blocks + tail_blocks)),
         dim3(256), 0, s, a, tiles, seg_items, n_items, nsplit);
  return hipGetLastError();
}

template <bool FP8>
static hipError_t fused_g(int G, const AttnArgs &a, unsigned tiles, unsigned seg_items,
                          unsigned n_items, unsigned nsplit, hipStream_t s) {
  switch (G) {
    case 1: return launch_fused<1, FP8>(a, tiles, seg_items, n_items, nsplit, s);
    case 2: return launch_fused<2, FP8>(a, tiles, seg_items, n_items, nsplit, s);
    case 4: return launch_fused<4, FP8>(a, tiles, seg_items, n_items, nsplit, s);
    case 8: return launch_fused<8, FP8>(a, tiles, seg_items, n_items, nsplit, s);
  }
  return hipErrorInvalidValue;
}

hipError_t decode_fused(int G, bool fp8, const AttnArgs &a, int max_rows, unsigned seg_items,
                        unsigned n_items, unsigned nsplit, hipStream_t s) {
  const unsigned tiles = static_cast<unsigned>((max_rows + MF_BM - 1) / MF_BM);
  return fp8 ? fused_g<true>(G, a, tiles, seg_items, n_items, nsplit, s)
             : fused_g<false>(G, a, tiles, seg_items, n_items, nsplit, s);
}

template <bool FP8, int NW>
static hipError_t mfma_g(int G, const AttnArgs &a, int max_rows, unsigned items, hipStream_t s) {
  switch (G) {
    case 1: return launch_mfma<1, FP8, NW>(a, max_rows, items, s);
    case 2: return launch_mfma<2, FP8, NW>(a, max_rows, items, s);
    case 4: return launch_mfma<4, FP8, NW>(a, max_rows, items, s);
    case 8: return launch_mfma<8, FP8, NW>(a, max_rows, items, s);
  }
  return hipErrorInvalidValue;
}

// Eight-wave blocks (256 query rows) halve the K/V tile traffic when requests fill them;
// they run as a persistent grid (one block per CU) that walks a static share of the row
// tiles. Four-wave blocks (two per CU, placed by the hardware dispatcher as others end)
// serve the batches that grid handles badly:
//  - short extends (on average under 3/4 of a 256-row tile);
//  - a longest request with more than twice the average rows: the static walk cannot
//    balance a few long requests against many short ones (a re-extend batch of that kind
//    took 4.46 ms that way against 2.52 ms as a four-wave grid);
//  - fewer than 8 row tiles of 256 rows per CU: a walk of a few tiles per block leaves
//    the uneven tile lengths unbalanced and each tile's prologue uncovered (chat-tree
//    turn batches, about 5 tiles per CU: 0.216 of the matrix peak against 0.237).
hipError_t mfma(int G, bool fp8, const AttnArgs &a, int max_rows, unsigned items,
                int64_t total_rows, hipStream_t s) {
  if (items == 0 || max_rows <= 0) return hipSuccess;
  const bool wide = total_rows >= static_cast<int64_t>(items) * (3 * 2 * MF_BM / 4) &&
                    2 * total_rows >= static_cast<int64_t>(items) * max_rows &&
                    total_rows * a.Hkv >= static_cast<int64_t>(8) * (2 * MF_BM) * device_cus();
  if (fp8) return wide ? mfma_g<true, 8>(G, a, max_rows, items, s) : mfma_g<true, 4>(G, a, max_rows, items, s);
  return wide ? mfma_g<false, 8>(G, a, max_rows, items, s) : mfma_g<false, 4>(G, a, max_rows, items, s);
}

hipError_t combine(bool bf16, const AttnArgs &a, int batch, int Dv, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  const uint64_t waves = static_cast<uint64_t>(batch) * ((a.Hq * Dv + 255) / 256);
  if (waves > 0x7fffffffull) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>((waves + 3) / 4)), block(256);
  if (bf16) launch(combine_kernel<uint16_t>, grid, block, 0, s, a, Dv, batch);
  else launch(combine_kernel<float>, grid, block, 0, s, a, Dv, batch);
  return hipGetLastError();
}

}  // namespace radix_launch
