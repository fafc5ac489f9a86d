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
//   attn_mfma_kernel  128 query rows x 64-key tiles with bf16 MFMA
//                     (32x32x16): S^T = K Q^T keeps a query row per lane so
//                     the softmax is lane-local; P^T feeds O^T = V^T P^T
//                     straight from registers. Query rows are either a
//                     request's new tokens x heads (extend, causal) or the
//                     members of a shared radix segment x heads (decode: one
//                     read of the segment's KV serves every member).
//   combine_kernel    merges per-request partial results.
#include "common.hpp"
#include "attn_args.hpp"
#include "radix_attn.h"

using namespace radix_dev;
using radix_launch::AttnArgs;
using radix_launch::StoreArgs;

namespace {

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

template <typename T> __device__ __forceinline__ void store_out(void *out, int64_t idx, float v);
template <> __device__ __forceinline__ void store_out<float>(void *out, int64_t idx, float v) {
  reinterpret_cast<float *>(out)[idx] = v;
}
template <> __device__ __forceinline__ void store_out<uint16_t>(void *out, int64_t idx, float v) {
  reinterpret_cast<uint16_t *>(out)[idx] = static_cast<uint16_t>(f32_to_bf16_bits(v));
}

// MODE 0: decode private tail (per request, split-KV)
// MODE 1: extend, one block per new token
// MODE 2: decode shared segment, one block per (segment, member) entry
template <typename T, int D, int G, int MODE>
__global__ __launch_bounds__(256) void attn_valu_kernel(AttnArgs a) {
  constexpr int EPL = Vec16<T>::N;
  static_assert(D / EPL == 16, "16 lanes per row");
  const int item = blockIdx.x, kvh = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4, sub = lane & 15;

  int b, lo, hi, part = 0;
  int64_t q_row;
  const int32_t *rtt_row;
  if (MODE == 1) {
    b = find_owner(a.cu_extend, a.batch, item);
    int i = item - a.cu_extend[b];
    lo = 0;
    hi = a.prefix_lens[b] + i + 1;
    q_row = item;
    rtt_row = rtt_row_of(a, b);
  } else if (MODE == 0) {
    b = item;
    hi = a.seq_lens[b];
    lo = a.private_start ? a.private_start[b] : 0;
    q_row = b;
    rtt_row = rtt_row_of(a, b);
    part = a.part_base + split;
  } else {
    int s = find_owner(a.seg_member_off, a.num_segments, item);
    b = a.seg_members[item];
    lo = a.seg_start[s];
    hi = a.seg_end[s];
    q_row = b;
    rtt_row = rtt_row_of(a, a.seg_row[s]);
    part = a.seg_member_slot[item];
  }
  const int n = hi - lo;
  const int nsplit = static_cast<int>(gridDim.z);
  const int chunk = ((n + nsplit - 1) / nsplit + 63) & ~63;
  const int s_lo = lo + split * chunk;
  const int s_hi = min(hi, s_lo + chunk);

  float qf[G][EPL];
  const T *qp = reinterpret_cast<const T *>(a.q) + (q_row * a.Hq + kvh * G) * D + sub * EPL;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    Vec16<T>::unpack(ldg16(qp + h * D), qf[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[h][e] *= a.scale_log2;
  }
  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  const int64_t row_bytes = static_cast<int64_t>(a.Hkv) * D * sizeof(T);
  const char *kb = reinterpret_cast<const char *>(a.k_pool) + kvh * D * sizeof(T) + sub * 16;
  const char *vb = reinterpret_cast<const char *>(a.v_pool) + kvh * D * sizeof(T) + sub * 16;

  for (int base = s_lo + wave * 16; base < s_hi; base += 64) {
    u32x4 kr[4], vr[4];
    bool valid[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int r = base + u * 4 + grp;
      valid[u] = r < s_hi;
      kr[u] = u32x4{0, 0, 0, 0};
      vr[u] = u32x4{0, 0, 0, 0};
      if (valid[u]) {
        int64_t slot = rtt_row[r];
        kr[u] = ldg16(kb + slot * row_bytes);
        vr[u] = ldg16(vb + slot * row_bytes);
      }
    }
    float s[4][G];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float kf[EPL];
      Vec16<T>::unpack(kr[u], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d = fmaf(qf[h][e], kf[e], d);
        d = sum16(d);
        s[u][h] = valid[u] ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = fmaxf(fmaxf(s[0][h], s[1][h]), fmaxf(s[2][h], s[3][h]));
      float mn = fmaxf(m[h], mx);
      float alpha = exp2f(m[h] - mn);
      float p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) p[u] = exp2f(s[u][h] - mn);
      l[h] = l[h] * alpha + (p[0] + p[1]) + (p[2] + p[3]);
      m[h] = mn;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float vf[EPL];
      Vec16<T>::unpack(vr[u], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float p = exp2f(s[u][h] - m[h]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
    }
  }

  // merge the 16 (wave, lane-group) states, one head at a time
  __shared__ float sm_m[16], sm_l[16];
  __shared__ float sm_acc[16][D];
  const int st = wave * 4 + grp;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (sub == 0) {
      sm_m[st] = m[h];
      sm_l[st] = l[h];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) sm_acc[st][sub * EPL + e] = acc[h][e];
    __syncthreads();
    for (int d = tid; d < D; d += 256) {
      float M = kNegBig;
#pragma unroll
      for (int x = 0; x < 16; ++x) M = fmaxf(M, sm_m[x]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const float w = exp2f(sm_m[x] - M);
        L = fmaf(sm_l[x], w, L);
        O = fmaf(sm_acc[x][d], w, O);
      }
      const int head = kvh * G + h;
      const bool empty = !(L > 0.f);
      const float o = empty ? 0.f : O / L;
      const float lse2 = empty ? -INFINITY : M + log2f(L);
      if (MODE == 1 || (MODE == 0 && a.ws_o == nullptr)) {
        store_out<T>(a.out, (q_row * a.Hq + head) * D + d, o);
        if (a.lse && d == 0) a.lse[q_row * a.Hq + head] = lse2 * kLn2;
      } else {
        const int64_t pi = (static_cast<int64_t>(b) * a.Hq + head) * a.parts + part;
        a.ws_o[pi * D + d] = o;
        if (d == 0) a.ws_lse[pi] = lse2;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ MFMA kernel
constexpr int MF_D = 128;
constexpr int MF_BM = 128;   // query rows per block (4 waves x 32)
constexpr int MF_BN = 64;    // keys per tile
constexpr int MF_KS = MF_D + 8;    // K tile row stride (bf16 elements)
constexpr int MF_VS = MF_BN + 4;   // V^T tile row stride (bf16 elements)

template <int G, bool SEG>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[MF_BN * MF_KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[MF_D * MF_VS];

  const int tile = blockIdx.x, item = blockIdx.y, kvh = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;

  int lo, hi, mem_off = 0, nrows, P = 0, b = 0;
  const int32_t *rtt_row;
  if (!SEG) {
    b = item;
    P = a.prefix_lens[b];
    const int E = a.extend_lens[b];
    nrows = E * G;
    if (tile * MF_BM >= nrows) return;
    const int i_last = min(E - 1, (tile * MF_BM + MF_BM - 1) / G);
    lo = 0;
    hi = P + i_last + 1;
    rtt_row = rtt_row_of(a, b);
  } else {
    mem_off = a.seg_member_off[item];
    nrows = (a.seg_member_off[item + 1] - mem_off) * G;
    if (tile * MF_BM >= nrows) return;
    lo = a.seg_start[item];
    hi = a.seg_end[item];
    rtt_row = rtt_row_of(a, a.seg_row[item]);
  }

  // this lane's query row
  const int R = tile * MF_BM + wave * 32 + n;
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
      u32x4 w = rvalid ? ldg16(qp + 16 * s) : u32x4{0, 0, 0, 0};
      qb[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_run = kNegBig, l_run = 0.f;

  const int64_t row_bytes = static_cast<int64_t>(a.Hkv) * MF_D * 2;
  const char *kb = reinterpret_cast<const char *>(a.k_pool) + kvh * MF_D * 2;
  const char *vb = reinterpret_cast<const char *>(a.v_pool) + kvh * MF_D * 2;
  const int lr = tid >> 4, lc = tid & 15;   // loader: row within 16, 16-byte chunk

  for (int kt = lo; kt < hi; kt += MF_BN) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = lr + 16 * u;
      const int key = kt + r;
      u32x4 kv = u32x4{0, 0, 0, 0}, vv = u32x4{0, 0, 0, 0};
      if (key < hi) {
        const int64_t slot = rtt_row[key];
        kv = ldg16(kb + slot * row_bytes + lc * 16);
        vv = ldg16(vb + slot * row_bytes + lc * 16);
      }
      *reinterpret_cast<u32x4 *>(&Ks[r * MF_KS + lc * 8]) = kv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[(lc * 8 + 2 * e) * MF_VS + r] = static_cast<uint16_t>(vv[e] & 0xffffu);
        Vt[(lc * 8 + 2 * e + 1) * MF_VS + r] = static_cast<uint16_t>(vv[e] >> 16);
      }
    }
    __syncthreads();

    f32x16 st[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      st[mb] = f32x16{};
#pragma unroll
      for (int s = 0; s < MF_D / 16; ++s) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(&Ks[(mb * 32 + n) * MF_KS + 16 * s + 8 * h]);
        st[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[s], st[mb], 0, 0, 0);
      }
    }
    float mx = kNegBig;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kt + mb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        float v = st[mb][i] * a.scale_log2;
        v = (key < hi && key <= qpos) ? v : -INFINITY;
        st[mb][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, xor32(mx));
    const float mn = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - mn);
    m_run = mn;
    float rs = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = exp2f(st[mb][i] - mn);
        st[mb][i] = p;
        rs += p;
      }
    rs += xor32(rs);
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] *= alpha;

    bf16x8 pb[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = pack_bf16x2(st[mb][8 * j + 2 * e], st[mb][8 * j + 2 * e + 1]);
        pb[mb][j] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
    for (int dvb = 0; dvb < 4; ++dvb) {
      const uint16_t *vrow = &Vt[(dvb * 32 + n) * MF_VS + 4 * h];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x2 lo2 = *reinterpret_cast<const u32x2 *>(vrow + mb * 32 + 16 * j);
          const u32x2 hi2 = *reinterpret_cast<const u32x2 *>(vrow + mb * 32 + 16 * j + 8);
          const u32x4 w = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
          o[dvb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pb[mb][j],
                                                           o[dvb], 0, 0, 0);
        }
    }
  }

  if (!rvalid) return;
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
    const int part = a.seg_member_slot[mem_off + qi];
    const int64_t pi = (q_tok * a.Hq + head) * a.parts + part;
    float *wp = a.ws_o + pi * MF_D;
#pragma unroll
    for (int dvb = 0; dvb < 4; ++dvb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dv = dvb * 32 + 8 * g4 + 4 * h;
        *reinterpret_cast<f32x4 *>(wp + dv) =
            f32x4{o[dvb][4 * g4] * inv, o[dvb][4 * g4 + 1] * inv, o[dvb][4 * g4 + 2] * inv,
                  o[dvb][4 * g4 + 3] * inv};
      }
    if (h == 0) a.ws_lse[pi] = lse2;
  }
}

// ------------------------------------------------------------------ combine
template <typename T>
__global__ __launch_bounds__(128) void combine_kernel(AttnArgs a, int Dv) {
  const int b = blockIdx.x, head = blockIdx.y;
  const int ns = a.req_num_shared ? a.req_num_shared[b] : 0;
  const int64_t base = (static_cast<int64_t>(b) * a.Hq + head) * a.parts;
  float M = -INFINITY;
  for (int p = 0; p < ns; ++p) M = fmaxf(M, a.ws_lse[base + p]);
  for (int s = 0; s < a.num_splits; ++s) M = fmaxf(M, a.ws_lse[base + a.part_base + s]);
  float L = 0.f;
  for (int p = 0; p < ns; ++p) L += exp2f(a.ws_lse[base + p] - M);
  for (int s = 0; s < a.num_splits; ++s) L += exp2f(a.ws_lse[base + a.part_base + s] - M);
  const float inv = 1.f / L;
  for (int d = threadIdx.x; d < Dv; d += blockDim.x) {
    float o = 0.f;
    for (int p = 0; p < ns; ++p)
      o = fmaf(exp2f(a.ws_lse[base + p] - M), a.ws_o[(base + p) * Dv + d], o);
    for (int s = 0; s < a.num_splits; ++s) {
      const int64_t pi = base + a.part_base + s;
      const float w = exp2f(a.ws_lse[pi] - M);
      if (w > 0.f) o = fmaf(w, a.ws_o[pi * Dv + d], o);
    }
    store_out<T>(a.out, (static_cast<int64_t>(b) * a.Hq + head) * Dv + d, o * inv);
  }
  if (a.lse && threadIdx.x == 0) a.lse[static_cast<int64_t>(b) * a.Hq + head] = (M + log2f(L)) * kLn2;
}

}  // namespace

// ====================================================================== launchers
namespace radix_launch {

hipError_t kv_store(const StoreArgs &a, int64_t T, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  kv_store_kernel<<<dim3(static_cast<unsigned>(T)), dim3(128), 0, stream>>>(a);
  return hipGetLastError();
}

template <typename T, int D, int G>
static hipError_t launch_valu(int mode, const AttnArgs &a, unsigned items, unsigned splits,
                              hipStream_t stream) {
  dim3 grid(items, a.Hkv, splits), block(256);
  if (mode == 0) attn_valu_kernel<T, D, G, 0><<<grid, block, 0, stream>>>(a);
  else if (mode == 1) attn_valu_kernel<T, D, G, 1><<<grid, block, 0, stream>>>(a);
  else attn_valu_kernel<T, D, G, 2><<<grid, block, 0, stream>>>(a);
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

hipError_t valu(bool bf16, int G, int mode, const AttnArgs &a, unsigned items, unsigned splits,
                hipStream_t s) {
  if (items == 0) return hipSuccess;
  return bf16 ? valu_g<uint16_t, 128>(G, mode, a, items, splits, s)
              : valu_g<float, 64>(G, mode, a, items, splits, s);
}

template <int G>
static hipError_t launch_mfma(bool seg, const AttnArgs &a, unsigned tiles, unsigned items,
                              hipStream_t s) {
  dim3 grid(tiles, items, a.Hkv), block(256);
  if (seg) attn_mfma_kernel<G, true><<<grid, block, 0, s>>>(a);
  else attn_mfma_kernel<G, false><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t mfma(int G, bool seg, const AttnArgs &a, int max_rows, unsigned items, hipStream_t s) {
  if (items == 0 || max_rows <= 0) return hipSuccess;
  const unsigned tiles = static_cast<unsigned>((max_rows + MF_BM - 1) / MF_BM);
  switch (G) {
    case 1: return launch_mfma<1>(seg, a, tiles, items, s);
    case 2: return launch_mfma<2>(seg, a, tiles, items, s);
    case 4: return launch_mfma<4>(seg, a, tiles, items, s);
    case 8: return launch_mfma<8>(seg, a, tiles, items, s);
  }
  return hipErrorInvalidValue;
}

hipError_t combine(bool bf16, const AttnArgs &a, int batch, int Dv, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  dim3 grid(batch, a.Hq), block(128);
  if (bf16) combine_kernel<uint16_t><<<grid, block, 0, s>>>(a, Dv);
  else combine_kernel<float><<<grid, block, 0, s>>>(a, Dv);
  return hipGetLastError();
}

}  // namespace radix_launch
