// MLA decode on gfx950: 128 query heads against one latent KV head whose rows hold
// 576 dims (512 latent + 64 rope); the values are the first 512 dims of the same
// row (SGLang feature article, §一: MLA keeps a single KV head, so one block
// processes many query heads and each KV row is read once for all of them).
// Requests sharing a radix-tree prefix run at the same time on the same XCD, so the
// shared rows come from that XCD's L2 after the first read.
// KV rows are bf16, or OCP E4M3 bytes with one fp32 scale per token (KV cache FP8,
// same section): the bytes are staged raw and converted exactly to bf16, and each
// key's scale multiplies its score and its probability.
//
// Block = one request's 128 heads over one key range, 8 waves. Waves w and w+4 share
// the 32 heads 32*(w%4) .. +31 and split the work by dimension: wave half 0 takes QK
// dims 0..287 and value dims 0..255, half 1 the rest. Per 32-key tile each wave forms
// a partial S^T = K Q^T over its dims (MFMA 32x32x16, query head per lane column),
// the pair swaps partials through LDS and both add them in the same order, so both
// run the identical online softmax; then O^T += V^T P^T over the wave's value dims.
// Per wave that is 72 registers of Q and 128 accumulator registers of O, which fits
// two waves per SIMD. bf16 tiles are double-buffered in LDS (rows go straight from
// global memory to LDS); fp8 rows go straight to one of two staging tiles, and each
// tile is converted into the free bf16 buffer while the previous tile's values are
// multiplied. With one
// chunk per request the block writes the output; with several, partials (o, lse)
// that combine_kernel merges.
#include <type_traits>

#include "attn_args.hpp"
#include "common.hpp"

using namespace radix_dev;
using radix_launch::MlaArgs;

namespace {

constexpr int kDqk = 576, kDv = 512, kHeads = 128;
constexpr int kBN = 32;              // keys per tile
constexpr int kHalfQK = kDqk / 2;    // QK dims per wave
constexpr int kHalfV = kDv / 2;      // value dims per wave
constexpr float kRescaleLog2 = 8.f;
#ifndef RADIX_MLA_FENCE
#define RADIX_MLA_FENCE 3   // score MFMAs between scheduling fences (bounds live K operands)
#endif  // tolerated growth of the running max before rescaling

__device__ __forceinline__ float xor32f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ 32) << 2,
                                                                 __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ void lds_load16(const void *g, uint8_t *lds_base) {
  __builtin_amdgcn_global_load_lds(g, reinterpret_cast<__attribute__((address_space(3))) void *>(
                                          reinterpret_cast<uintptr_t>(lds_base)),
                                   16, 0, 0);
}

// Four transposed LDS reads at b0 + OFF0, b1 + OFF0, b0 + OFF1, b1 + OFF1 (immediate
// offsets) and the wait for them. Written as assembly: the compiler orders its own form
// of this read behind every outstanding global->LDS load (vmcnt(0)), which would wait
// for the next tile's prefetch in the middle of the current one.
template <int OFF0, int OFF1>
__device__ __forceinline__ void lds_tr16_x4_imm(u32x2 (&r)[4], uint32_t b0, uint32_t b1) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %1, %5 offset:%6\n\t"
      "ds_read_b64_tr_b16 %2, %4 offset:%7\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(b0), "v"(b1), "n"(OFF0), "n"(OFF1)
      : "memory");
}

// Tile layout in LDS (bf16, 36 KB per 32 keys): region A holds dims 0..511 of key r as
// one 1 KB row, 16-byte chunk c at r*1024 + 16*(c ^ fA(r)); region B holds the rope
// dims 512..575 as 128-byte rows after it, chunk 64+c at 32768 + r*128 + 16*(c ^ fB(r)).
// fA mixes both 2-bit fields of the row so that the score reads (16 rows, one chunk)
// and the transposed value reads (8 rows, 4 chunks) both fall on distinct banks; fB
// does the same for the 128-byte rows. One 1 KB wave-wide direct load fills one
// region-A row, so each load's slot is one scalar.
constexpr int kTileB = kBN * 2 * kDqk;   // 36 KB
constexpr int kRegB = kBN * 1024;        // start of region B
__device__ __forceinline__ int fA(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int fB(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int offA(int r, int c) { return r * 1024 + ((c ^ fA(r)) << 4); }
__device__ __forceinline__ int offB(int r, int c) { return kRegB + r * 128 + ((c ^ fB(r)) << 4); }

// fp8 staging: two raw tiles (one converting while the next lands), 24 KB each
constexpr int kStgB = 8 * 3072;

template <bool FP8, int HALF>
__device__ __forceinline__ void mla_body(const MlaArgs &a, uint8_t (*smem)[kTileB], uint8_t *stg,
                                         float *scl, f32x4 (*xs)[4][64], int wave, int b, int lo,
                                         int hi, int part) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int hg = wave & 3;
  const int n = lane & 31, h = lane >> 5;
  const int32_t *rtt_row = a.rtt + static_cast<int64_t>(a.req_rows ? a.req_rows[b] : b) * a.rtt_stride;

  // ---- Q (B operand of S^T = K Q^T): this lane's head, dims HALF*288 + 16s + 8h .. +7
  const int head = hg * 32 + n;
  bf16x8 qb[kHalfQK / 16];
  {
    const uint16_t *qp = a.q + (static_cast<int64_t>(b) * kHeads + head) * kDqk + kHalfQK * HALF + 8 * h;
#pragma unroll
    for (int s = 0; s < kHalfQK / 16; ++s) qb[s] = __builtin_bit_cast(bf16x8, ldg16(qp + 16 * s));
  }
  f32x16 o[kHalfV / 32];
#pragma unroll
  for (int i = 0; i < kHalfV / 32; ++i) o[i] = f32x16{};
  float m_run = kNegBig, l_run = 0.f;

  // ---- tile loads. bf16: region-A row J by wave J % 8 (lane i brings logical chunk
  // i ^ fA(J)); region B by waves 0..3 (lane i: row 8*wave + i/8, chunk i%8 ^ fB(row)).
  // Lane r holds the slot of row r (lanes 32..63 repeat).
  // fp8: the raw 576-byte rows go straight to a staging tile, the tile's 32 key scales
  // to a scale array; once landed, the rows are converted exactly to bf16 (every E4M3
  // value is a bf16 value) into the bf16 buffer the matrix code reads next, and each
  // key's scale is applied to its score and its probability instead. Wave w stages rows
  // 4w .. 4w+3, lane i bringing 16-byte chunks c = i%16 + 16k (k = 0, 1, 2; third-batch
  // lanes past chunk 35 bring a duplicate) of row 4w + i/16 to staging byte
  // 3072w + 1024k + 16i, so the thread that converts a chunk is the one that loaded it, at
  // offsets fixed per thread.
  const uint8_t *kv = static_cast<const uint8_t *>(a.kv);
  const int last = hi - 1;
  int32_t sl, sl_next = 0;
  auto load_slots = [&](int kt) { sl = rtt_row[min(kt + (lane & 31), last)]; };
  // fp8 loop: the next tile's slots are fetched before this tile's rows are issued (into
  // their own register, taken over after the end-of-tile wait), so no wait for them can
  // land behind the row loads; lane offset recomputed here rather than kept live
  auto load_next_slots = [&](int kt) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    sl_next = rtt_row[min(kt + (ln & 31), last)];
  };
  // bf16: rows into buffer `stage`; fp8: tile index `stage` -> staging tile stage & 1,
  // scale slot stage & 3
  auto issue = [&](int kt, int stage) {
    if (FP8) {
      int ln = lane;   // recomputed, not kept live (a spill reload here would wait on loads)
      asm volatile("" : "+v"(ln));
      const int r = 4 * wave + (ln >> 4);
      const int64_t slot = __builtin_amdgcn_ds_bpermute(r << 2, sl);
      const uint8_t *src = kv + slot * kDqk + (ln & 15) * 16;
      uint8_t *dst = stg + kStgB * (stage & 1) + 3072 * wave;
      lds_load16(src, dst);
      lds_load16(src + 256, dst + 1024);
      lds_load16(src + ((ln & 15) < 4 ? 512 : 0), dst + 2048);
      if (wave == 0)
        __builtin_amdgcn_global_load_lds(
            a.kv_scale + sl,
            reinterpret_cast<__attribute__((address_space(3))) void *>(
                reinterpret_cast<uintptr_t>(scl + 64 * (stage & 3))),
            4, 0, 0);
    } else {
#pragma unroll
      for (int jj = 0; jj < kBN / 8; ++jj) {
        const int J = wave + 8 * jj;
        const int64_t slot = __builtin_amdgcn_readlane(sl, J);
        lds_load16(kv + slot * (2 * kDqk) + ((lane ^ fA(J)) << 4), &smem[stage][J * 1024]);
      }
      if (wave < 4) {
        const int r = 8 * wave + (lane >> 3);
        const int64_t slot = __builtin_amdgcn_ds_bpermute(r << 2, sl);
        lds_load16(kv + slot * (2 * kDqk) + 1024 + (((lane & 7) ^ fB(r)) << 4),
                   &smem[stage][kRegB + wave * 1024]);
      }
    }
  };
  // fp8: one staged chunk (16 E4M3 bytes) -> its two bf16 chunks at o0, o1 of `dst`
  auto conv_store = [&](const u32x4 &w, uint8_t *dst, int o0, int o1) {
    const u32x4 lo16 = u32x4{fp8x2_to_bf16x2<false>(w[0]), fp8x2_to_bf16x2<true>(w[0]),
                             fp8x2_to_bf16x2<false>(w[1]), fp8x2_to_bf16x2<true>(w[1])};
    const u32x4 hi16 = u32x4{fp8x2_to_bf16x2<false>(w[2]), fp8x2_to_bf16x2<true>(w[2]),
                             fp8x2_to_bf16x2<false>(w[3]), fp8x2_to_bf16x2<true>(w[3])};
    *reinterpret_cast<u32x4 *>(dst + o0) = lo16;
    *reinterpret_cast<u32x4 *>(dst + o1) = hi16;
  };
  // this thread's chunks: row 4*wave + lane/16, fp8 chunk lane%16 + 16k -> bf16 chunks
  // 2c, 2c+1; the row swizzle only touches the low four chunk bits, so batch k (k < 2)
  // sits 512k bytes further. The lane-derived offsets are recomputed at each use
  // (cheap) rather than held in registers across the loop.
  auto conv_piece = [&](const u32x4 &w, uint8_t *dst, int k) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int cr = 4 * wave + (ln >> 4), i16 = ln & 15;
    if (k < 2) {
      conv_store(w, dst, cr * 1024 + (((2 * i16) ^ fA(cr)) << 4) + 512 * k,
                 cr * 1024 + (((2 * i16 + 1) ^ fA(cr)) << 4) + 512 * k);
    } else if (i16 < 4) {   // batch 2: rope chunks 32..35
      conv_store(w, dst, offB(cr, 2 * i16), offB(cr, 2 * i16 + 1));
    }
  };
  auto conv_src = [&](int t, int k) {   // staged chunk k of tile t (landed, visible)
    return *reinterpret_cast<const u32x4 *>(stg + kStgB * (t & 1) + 3072 * wave + 1024 * k +
                                            16 * lane);
  };

  // bf16: tile t+1's loads are in flight while tile t is used (two LDS buffers).
  // fp8: tile t+2's raw bytes are in flight while tile t is used, and tile t+1 (landed at
  // the last barrier) is converted into the other bf16 buffer by the same waves, its
  // pieces placed between tile t's value blocks (key scales: four buffers, tile t in t % 4).
  const int ntiles = hi > lo ? (hi - lo + kBN - 1) / kBN : 0;
  if (ntiles > 0) {
    load_slots(lo);
    issue(lo, 0);
    if (ntiles > 1) {
      load_slots(lo + kBN);
      if (FP8) {
        issue(lo + kBN, 1);
        if (ntiles > 2) load_slots(lo + 2 * kBN);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (FP8 && ntiles > 0) {   // tile 0 into buffer 0
    uint8_t *d0 = smem[0];
#pragma unroll
    for (int k = 0; k < 3; ++k) conv_piece(conv_src(0, k), d0, k);
    __syncthreads();
  }
  // V^T operand from the tile: in 16-lane group g, source lane s reads 4 value dims of
  // key row 16j + 4*(g>>1) + (s>>2) (+8 for the second read)
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int kt = lo + t * kBN;
    if (FP8) {   // staging tile t & 1 held tile t, converted during the last iteration
      // unconditional (clamped: past the end it re-reads the last slot), so no join of
      // paths forces an early copy of the loaded register (a wait behind the row loads)
      load_next_slots(kt + 3 * kBN);
      if (t + 2 < ntiles) issue(kt + 2 * kBN, t + 2);
    } else if (t + 1 < ntiles) {
      issue(kt + kBN, buf ^ 1);
      if (t + 2 < ntiles) load_slots(kt + 2 * kBN);
    }
    const uint8_t *T = smem[buf];
    // lane-derived LDS offsets are recomputed each tile (cheap VALU) rather than held
    // in registers across the loop
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int n = ln & 31, h = ln >> 5, g = ln >> 4, s16 = ln & 15;
    const int vrow = 4 * (g >> 1) + (s16 >> 2);

    // Region-A chunk c = 16q + r of row n sits at n*1024 + 256q + ((r ^ fA(n)) << 4):
    // the swizzle only touches the low 4 bits, so the score reads need one lane base per
    // r (8 of them: r = 2i + h) and take q as a constant offset.
    const uint8_t *kbase[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kbase[i] = T + n * 1024 + (((2 * i + h) ^ fA(n)) << 4);
    // fp8: tile t+1's conversion into the other buffer, in pieces between the value
    // blocks below (on the last tile it re-converts stale staging bytes into that free
    // buffer, which nothing reads again)
    uint8_t *cdst = smem[buf ^ 1];
    u32x4 cw{};
    f32x16 sc = f32x16{};
#pragma unroll
    for (int s = 0; s < kHalfQK / 16; ++s) {
      constexpr int c0 = (kHalfQK / 8) * HALF;
      const int cs = c0 + 2 * s;   // chunk of the h = 0 lanes (even)
      const bf16x8 ka = cs < 64
          ? *reinterpret_cast<const bf16x8 *>(kbase[(cs & 15) >> 1] + 256 * (cs >> 4))
          : *reinterpret_cast<const bf16x8 *>(T + offB(n, cs - 64 + h));
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[s], sc, 0, 0, 0);
      if (s % RADIX_MLA_FENCE == RADIX_MLA_FENCE - 1) __builtin_amdgcn_sched_barrier(0);
    }
    // swap partial scores with the other half of the pair; both add own + other (the
    // barrier orders LDS only: the next tile's loads stay in flight)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      xs[wave][q][lane] = f32x4{sc[4 * q], sc[4 * q + 1], sc[4 * q + 2], sc[4 * q + 3]};
    lds_barrier();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 other = xs[wave ^ 4][q][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[4 * q + e] += other[e];
    }

    if (kt + kBN > hi) {   // (uniform) ragged last tile
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kt + 8 * (i >> 2) + 4 * h + (i & 3);
        sc[i] = key < hi ? sc[i] : -INFINITY;
      }
    }
    // fp8: each key's scale (> 0) on its score; keys of sc[i]: 8*(i>>2) + 4h + (i&3)
    const float *ks = scl + 64 * (t & 3) + 4 * h;
    if (FP8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 s4 = *reinterpret_cast<const f32x4 *>(ks + 8 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[4 * q + e] *= s4[e];
      }
    }
    // raw scores: the scale (> 0) is applied to the maximum and inside the exponent
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sc[i], sc[i + 1]));
    mx = fmaxf(mx, xor32f(mx)) * a.scale_log2;
    // rescale the accumulators only when some head's maximum grew noticeably
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleLog2) != 0) {
      const float mn = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < kHalfV / 32; ++d) o[d] *= alpha;
      m_run = mn;
    }
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sc[i], a.scale_log2, -m_run));
      sc[i] = p;
      rs += p;
    }
    l_run += rs;   // this half's keys; the two halves are added after the loop
    if (FP8) {   // the value rows' scales go with their probabilities
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 s4 = *reinterpret_cast<const f32x4 *>(ks + 8 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[4 * q + e] *= s4[e];
      }
    }
    bf16x8 pb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = cvt_bf16x2(sc[8 * j + 2 * e], sc[8 * j + 2 * e + 1]);
      pb[j] = __builtin_bit_cast(bf16x8, w);
    }
    // V^T operands of one value-dim block (4 transposed reads) at a time. The chunk of
    // block d is 16q + 4(d % 4) + lane bits with q = 2*HALF + d/4, and rows 16j + vrow
    // share vrow's swizzle: one lane base per (d % 4, row vrow or vrow + 8), the rest
    // constant offsets.
    const uint32_t tb = lds_addr(T);
    const int cl = 2 * (g & 1) + ((s16 & 3) >> 1), hb = (s16 & 1);
    uint32_t vb[4][2];
#pragma unroll
    for (int dm = 0; dm < 4; ++dm)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int r = vrow + 8 * p;
        vb[dm][p] = tb + r * 1024 + (((4 * dm + cl) ^ fA(r)) << 4) + 8 * hb;
      }
    // value block d (compile-time): keys 16j + row at +16384 j, dims at +256 q, both as
    // immediate offsets of the reads
    auto pv_block = [&](auto dc) {
      constexpr int d = decltype(dc)::value;
      constexpr int q256 = 256 * (2 * HALF + (d >> 2));
      u32x2 rv[4];
      lds_tr16_x4_imm<q256, 16384 + q256>(rv, vb[d & 3][0], vb[d & 3][1]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 w = u32x4{rv[2 * j][0], rv[2 * j][1], rv[2 * j + 1][0], rv[2 * j + 1][1]};
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pb[j], o[d],
                                                        0, 0, 0);
      }
    };
    static_assert(kHalfV / 32 == 8, "eight value blocks per wave");
    pv_block(std::integral_constant<int, 0>{});
    if (FP8) cw = conv_src(t + 1, 0);
    pv_block(std::integral_constant<int, 1>{});
    pv_block(std::integral_constant<int, 2>{});
    if (FP8) {
      conv_piece(cw, cdst, 0);
      cw = conv_src(t + 1, 1);
    }
    pv_block(std::integral_constant<int, 3>{});
    pv_block(std::integral_constant<int, 4>{});
    if (FP8) {
      conv_piece(cw, cdst, 1);
      cw = conv_src(t + 1, 2);
    }
    pv_block(std::integral_constant<int, 5>{});
    pv_block(std::integral_constant<int, 6>{});
    if (FP8) conv_piece(cw, cdst, 2);
    pv_block(std::integral_constant<int, 7>{});
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (FP8) sl = sl_next;
  }

  // ---- partial (normalised o, lse in log2 units) or, for a single part, the output;
  // each wave of the pair writes its value dims, half 0 the lse
  l_run += xor32f(l_run);
  const bool empty = !(l_run > 0.f);
  const float inv = empty ? 0.f : 1.f / l_run;
  const float lse2 = empty ? -INFINITY : m_run + log2f(l_run);
  if (a.parts == 1 && a.out) {
    uint16_t *op = a.out + (static_cast<int64_t>(b) * kHeads + head) * kDv + kHalfV * HALF;
#pragma unroll
    for (int d = 0; d < kHalfV / 32; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dv = d * 32 + 8 * g4 + 4 * h;
        *reinterpret_cast<u32x2 *>(op + dv) =
            u32x2{cvt_bf16x2(o[d][4 * g4] * inv, o[d][4 * g4 + 1] * inv),
                  cvt_bf16x2(o[d][4 * g4 + 2] * inv, o[d][4 * g4 + 3] * inv)};
      }
    if (a.lse && h == 0 && HALF == 0) a.lse[static_cast<int64_t>(b) * kHeads + head] = lse2 * kLn2;
    return;
  }
  const int64_t pi = (static_cast<int64_t>(b) * kHeads + head) * a.parts + part;
  float *wp = a.ws_o + pi * kDv + kHalfV * HALF;
#pragma unroll
  for (int d = 0; d < kHalfV / 32; ++d)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int dv = d * 32 + 8 * g4 + 4 * h;
      *reinterpret_cast<f32x4 *>(wp + dv) = f32x4{o[d][4 * g4] * inv, o[d][4 * g4 + 1] * inv,
                                                  o[d][4 * g4 + 2] * inv, o[d][4 * g4 + 3] * inv};
    }
  if (h == 0 && HALF == 0) a.ws_lse[pi] = lse2;
}

template <bool FP8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_decode_kernel(MlaArgs a) {
  // bf16 tiles double-buffered; fp8 adds two raw staging tiles and four tiles' key scales
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2][kTileB];
  __shared__ __attribute__((aligned(16))) f32x4 xs[8][4][64];   // partial scores per wave
  __shared__ __attribute__((aligned(1024))) uint8_t stage[FP8 ? 2 * kStgB + 4 * 64 * 4 : 16];
  float *scl = reinterpret_cast<float *>(stage + 2 * kStgB);

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
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave < 4) mla_body<FP8, 0>(a, smem, stage, scl, xs, wave, b, lo, hi, split);
  else mla_body<FP8, 1>(a, smem, stage, scl, xs, wave, b, lo, hi, split);
}

}  // namespace

namespace radix_launch {

unsigned mla_blocks(const MlaArgs &a) {
  return static_cast<unsigned>(8 * ((a.batch * a.nsplit + 7) / 8));
}

hipError_t mla(const MlaArgs &a, hipStream_t s) {
  const unsigned blocks = mla_blocks(a);
  if (blocks == 0) return hipSuccess;
  if (a.fp8) launch(mla_decode_kernel<true>, dim3(blocks), dim3(512), 0, s, a);
  else launch(mla_decode_kernel<false>, dim3(blocks), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace radix_launch
