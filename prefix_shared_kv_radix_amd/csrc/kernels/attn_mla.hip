// MLA decode on gfx950: 128 query heads against one latent KV head whose rows hold
// 576 dims (512 latent + 64 rope); the values are the first 512 dims of the same
// row (SGLang feature article, §一: MLA keeps a single KV head, so one block
// processes many query heads and each KV row is read once for all of them).
// Requests sharing a radix-tree prefix run at the same time on the same XCD, so the
// shared rows come from that XCD's L2 after the first read.
// KV rows are bf16, or OCP E4M3 bytes with one fp32 scale per token (KV cache FP8,
// same section), dequantised to bf16 as they are staged into LDS.
//
// Block = one request's 128 heads over one key range; 4 waves x 32 heads. Per
// 32-key tile: S^T = K Q^T (MFMA 32x32x16, query head per lane column), online
// softmax in registers, O^T += V^T P^T (MFMA, 16 blocks of 32 value dims). Tiles
// are double-buffered in LDS: the next tile's rows are loaded into registers
// while the current one is multiplied. With one chunk per request the block
// writes the output; with several, partials (o, lse) that combine_kernel merges.
#include "attn_args.hpp"
#include "common.hpp"

using namespace radix_dev;
using radix_launch::MlaArgs;

namespace {

constexpr int kDqk = 576, kDv = 512, kHeads = 128;
constexpr int kBN = 32;              // keys per tile
constexpr int kKS = kDqk + 8;        // K tile row stride (bf16 elements)
constexpr int kVS = kBN + 4;         // V^T tile row stride (bf16 elements)
constexpr float kRescaleLog2 = 8.f;  // tolerated growth of the running max before rescaling

__device__ __forceinline__ float xor32f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ 32) << 2,
                                                                 __builtin_bit_cast(int, x)));
}

// Staging of one tile: thread t loads key (t >> 3), chunk group (t & 7) = 144 bytes of
// a bf16 row (9 x 16 B) or 72 bytes of an fp8 row (9 x 8 B).
template <bool FP8> struct Stage;
template <> struct Stage<false> {
  u32x4 w[9];
  float scale;
  __device__ void load(const uint8_t *row) {
#pragma unroll
    for (int i = 0; i < 9; ++i) w[i] = *reinterpret_cast<const u32x4 *>(row + 16 * i);
  }
  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < 9; ++i) w[i] = u32x4{0, 0, 0, 0};
  }
  __device__ u32x4 bf16x8(int i) const { return w[i]; }
};
template <> struct Stage<true> {
  u32x2 w[9];
  float scale;
  __device__ void load(const uint8_t *row) {
#pragma unroll
    for (int i = 0; i < 9; ++i) w[i] = *reinterpret_cast<const u32x2 *>(row + 8 * i);
  }
  __device__ void zero() {
#pragma unroll
    for (int i = 0; i < 9; ++i) w[i] = u32x2{0, 0};
    scale = 0.f;
  }
  __device__ u32x4 bf16x8(int i) const {
    const uint32_t a = w[i][0], b = w[i][1];
    return u32x4{pack_bf16x2(fp8_to_f32<0>(a) * scale, fp8_to_f32<1>(a) * scale),
                 pack_bf16x2(fp8_to_f32<2>(a) * scale, fp8_to_f32<3>(a) * scale),
                 pack_bf16x2(fp8_to_f32<0>(b) * scale, fp8_to_f32<1>(b) * scale),
                 pack_bf16x2(fp8_to_f32<2>(b) * scale, fp8_to_f32<3>(b) * scale)};
  }
};

template <bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBN * kKS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][kDv * kVS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;

  // ---- work item: requests in plan order (members of one shared segment are
  // consecutive) spread so that consecutive items land on one XCD; each request's
  // keys [0, seq_len) are cut into nsplit chunks
  const int items = a.batch * a.nsplit;
  const int per_xcd = (items + 7) / 8;
  const int pos = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (pos >= items) return;
  const int split = pos % a.nsplit;
  const int b = a.req_order ? a.req_order[pos / a.nsplit] : pos / a.nsplit;
  const int L = a.seq_lens[b];
  const int lo = split * a.split_chunk;
  const int hi = min(L, lo + a.split_chunk);
  const int part = split;
  const int32_t *rtt_row = a.rtt + static_cast<int64_t>(a.req_rows ? a.req_rows[b] : b) * a.rtt_stride;

  // ---- Q (B operand of S^T = K Q^T): this lane's head, dims 16s + 8h .. +7
  const int head = wave * 32 + n;
  bf16x8 qb[kDqk / 16];
  {
    const uint16_t *qp = a.q + (static_cast<int64_t>(b) * kHeads + head) * kDqk + 8 * h;
#pragma unroll
    for (int s = 0; s < kDqk / 16; ++s) qb[s] = __builtin_bit_cast(bf16x8, ldg16(qp + 16 * s));
  }
  f32x16 o[kDv / 32];
#pragma unroll
  for (int i = 0; i < kDv / 32; ++i) o[i] = f32x16{};
  float m_run = kNegBig, l_run = 0.f;

  // ---- staging
  constexpr int kRowBytes = FP8 ? kDqk : 2 * kDqk;
  const int skey = tid >> 3, sgrp = tid & 7;
  const uint8_t *kv = static_cast<const uint8_t *>(a.kv);
  Stage<FP8> st;
  auto fetch = [&](int kt) {
    const int key = kt + skey;
    if (key < hi) {
      const int64_t slot = rtt_row[key];
      st.load(kv + slot * kRowBytes + sgrp * (FP8 ? 72 : 144));
      if (FP8) st.scale = a.kv_scale[slot];
    } else {
      st.zero();
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int c = sgrp * 9 + i;            // 16-byte chunk (8 dims) of the 576-dim row
      const u32x4 w = st.bf16x8(i);
      *reinterpret_cast<u32x4 *>(&Ks[buf][skey * kKS + c * 8]) = w;
      if (c < kDv / 8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Vt[buf][(c * 8 + 2 * e) * kVS + skey] = static_cast<uint16_t>(w[e] & 0xffffu);
          Vt[buf][(c * 8 + 2 * e + 1) * kVS + skey] = static_cast<uint16_t>(w[e] >> 16);
        }
      }
    }
  };

  const int ntiles = hi > lo ? (hi - lo + kBN - 1) / kBN : 0;
  if (ntiles > 0) {
    fetch(lo);
    stash(0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int kt = lo + t * kBN;
    if (t + 1 < ntiles) fetch(kt + kBN);

    f32x16 sc = f32x16{};
#pragma unroll
    for (int s = 0; s < kDqk / 16; ++s) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(&Ks[buf][n * kKS + 16 * s + 8 * h]);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[s], sc, 0, 0, 0);
    }
    float mx = kNegBig;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kt + 8 * (i >> 2) + 4 * h + (i & 3);
      const float v = key < hi ? sc[i] * a.scale_log2 : -INFINITY;
      sc[i] = v;
      mx = fmaxf(mx, v);
    }
    mx = fmaxf(mx, xor32f(mx));
    // rescale the accumulators only when some head's maximum grew noticeably
    const bool grow = mx > m_run + kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mn = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - mn);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < kDv / 32; ++d) o[d] *= alpha;
      m_run = mn;
    }
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = exp2f(sc[i] - m_run);
      sc[i] = p;
      rs += p;
    }
    l_run += rs + xor32f(rs);
    bf16x8 pb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(sc[8 * j + 2 * e], sc[8 * j + 2 * e + 1]);
      pb[j] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int d = 0; d < kDv / 32; ++d) {
      const uint16_t *vrow = &Vt[buf][(d * 32 + n) * kVS + 4 * h];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x2 lo2 = *reinterpret_cast<const u32x2 *>(vrow + 16 * j);
        const u32x2 hi2 = *reinterpret_cast<const u32x2 *>(vrow + 16 * j + 8);
        const u32x4 w = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pb[j], o[d],
                                                        0, 0, 0);
      }
    }
    if (t + 1 < ntiles) stash(buf ^ 1);
    __syncthreads();
  }

  // ---- partial (normalised o, lse in log2 units) or, for a single part, the output
  const bool empty = !(l_run > 0.f);
  const float inv = empty ? 0.f : 1.f / l_run;
  const float lse2 = empty ? -INFINITY : m_run + log2f(l_run);
  if (a.parts == 1 && a.out) {
    uint16_t *op = a.out + (static_cast<int64_t>(b) * kHeads + head) * kDv;
#pragma unroll
    for (int d = 0; d < kDv / 32; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dv = d * 32 + 8 * g4 + 4 * h;
        *reinterpret_cast<u32x2 *>(op + dv) =
            u32x2{pack_bf16x2(o[d][4 * g4] * inv, o[d][4 * g4 + 1] * inv),
                  pack_bf16x2(o[d][4 * g4 + 2] * inv, o[d][4 * g4 + 3] * inv)};
      }
    if (a.lse && h == 0) a.lse[static_cast<int64_t>(b) * kHeads + head] = lse2 * kLn2;
    return;
  }
  const int64_t pi = (static_cast<int64_t>(b) * kHeads + head) * a.parts + part;
  float *wp = a.ws_o + pi * kDv;
#pragma unroll
  for (int d = 0; d < kDv / 32; ++d)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int dv = d * 32 + 8 * g4 + 4 * h;
      *reinterpret_cast<f32x4 *>(wp + dv) = f32x4{o[d][4 * g4] * inv, o[d][4 * g4 + 1] * inv,
                                                  o[d][4 * g4 + 2] * inv, o[d][4 * g4 + 3] * inv};
    }
  if (h == 0) a.ws_lse[pi] = lse2;
}

}  // namespace

namespace radix_launch {

unsigned mla_blocks(const MlaArgs &a) {
  return static_cast<unsigned>(8 * ((a.batch * a.nsplit + 7) / 8));
}

hipError_t mla(const MlaArgs &a, hipStream_t s) {
  const unsigned blocks = mla_blocks(a);
  if (blocks == 0) return hipSuccess;
  if (a.fp8) mla_decode_kernel<true><<<dim3(blocks), dim3(256), 0, s>>>(a);
  else mla_decode_kernel<false><<<dim3(blocks), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace radix_launch
