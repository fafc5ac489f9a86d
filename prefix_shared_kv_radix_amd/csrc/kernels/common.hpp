// Device helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace radix_dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running-max start value: finite, so exp2(start - m) is 0 and never NaN.
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Two floats -> packed bf16 pair (lo in the low half) with the hardware conversion.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// OCP E4M3FN byte -> float via the gfx950 hardware conversion (byte `sel` of w).
template <int SEL>
__device__ __forceinline__ float fp8_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w), SEL);
}

// Two E4M3FN bytes of w (bytes 0,1 or, with HI, 2,3) -> a packed bf16 pair, exactly:
// every E4M3 value (4 significant bits, exponents -9..8) is a bf16 value, and a scale
// operand of 1 leaves it unchanged.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, HI));
}

// Sixteen E4M3FN bytes times `scale`, rounded to bf16 (nearest even): two 16-byte rows
// of packed bf16 pairs, lo = values 0..7, hi = values 8..15.
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4 &w, float scale, u32x4 &lo, u32x4 &hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), false);
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[i]), true);
    out[2 * i] = cvt_bf16x2(a[0] * scale, a[1] * scale);
    out[2 * i + 1] = cvt_bf16x2(b[0] * scale, b[1] * scale);
  }
  lo = u32x4{out[0], out[1], out[2], out[3]};
  hi = u32x4{out[4], out[5], out[6], out[7]};
}

// Sum over each group of 16 consecutive lanes; every lane of the group gets the sum.
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float sum16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xF, 0xF, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x140, 0xF, 0xF, true));
  return x;
}

// Value held by lane (lane ^ 32).
__device__ __forceinline__ float xor32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(((threadIdx.x & 63) ^ 32) << 2,
                                                                 __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ u32x4 ldg16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

// Loads whose completion the compiler does not track: the caller waits for them with
// an explicit s_waitcnt that names the destination registers (see the private-tail
// ring). Nothing may read or copy the destination before that wait. The K/V row loads
// (8 and 16 bytes) are non-temporal: a private tail's rows are read once per step, and
// streaming them past the caches' retention reads about 5 % faster (measured on the
// decode steps); slots and scales keep the default policy.
__device__ __forceinline__ int32_t ld_async4(const int32_t *p) {
  int32_t v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ float ld_async4f(const float *p) {
  float v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}
__device__ __forceinline__ u32x2 ld_async8(const void *p) {
  u32x2 v;
  asm volatile("global_load_dwordx2 %0, %1, off nt" : "=v"(v) : "v"(p) : "memory");
  return v;
}
template <int OFF>
__device__ __forceinline__ u32x4 ld_async16(const void *p) {
  u32x4 v;
  asm volatile("global_load_dwordx4 %0, %1, off offset:%2 nt" : "=v"(v) : "v"(p), "n"(OFF) : "memory");
  return v;
}

// Partial results merged by another block (possibly on another XCD, whose L2 is not
// kept coherent with this one): written and read with device-scope relaxed atomic
// accesses, which the compiler emits as sc1 loads/stores (served past the XCD's L2)
// without any whole-cache writeback or invalidate.
// The ordering rests on the GFX942 memory model of the LLVM AMDGPU backend's user guide
// (gfx950 follows it): a monotonic agent-scope load or store is a global load/store with
// sc1 set, so it is coherent across XCDs; "s_waitcnt vmcnt(0)" returns only once this
// wave's earlier stores have completed at that scope; and an agent-scope atomic
// read-modify-write is performed at the same coherence point. A producer therefore
// stores its partial (sc1), waits for vmcnt(0), then increments the counter; the
// consumer that reads the final count issues its sc1 loads of the partials only
// after that atomic has returned, so they see every producer's data.
typedef float f32x2 __attribute__((ext_vector_type(2)));
// One 16-byte store with the same cache policy (sc1) that a device-scope relaxed atomic
// store gets: a pair of 8-byte atomic stores reached HBM as partial-line writes, about
// twice the bytes. The compiler does not track this store, so its own waits can only
// get stricter; callers wait for it with wait_stores() before publishing (arrive()).
// A store of more than 8 bytes needs one wait state before a vector ALU instruction
// may overwrite its data registers; the compiler adds it only for stores it emits
// itself, so the block carries its own.
__device__ __forceinline__ void st_dev(float *p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ f32x4 ld_dev(const float *p) {
  const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
  const f32x2 a = __builtin_bit_cast(
      f32x2, __hip_atomic_load(const_cast<uint64_t *>(q), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const f32x2 b = __builtin_bit_cast(
      f32x2, __hip_atomic_load(const_cast<uint64_t *>(q + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return f32x4{a[0], a[1], b[0], b[1]};
}
__device__ __forceinline__ void st_dev1(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev1(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this wave's stores are complete (device-visible for sc1 stores), so an
// atomic issued afterwards is ordered after them. A workgroup-scope fence does not wait
// for stores on this target, and an agent-scope one would also write back the L2.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Arrival counter of a merge: returns the count before this arrival (relaxed, device scope).
__device__ __forceinline__ int arrive(int32_t *c) {
  return __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_counter(int32_t *c) {
  __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations complete, then
// s_barrier. Unlike __syncthreads() it does not wait for outstanding global loads, so a
// prefetch of the next tile stays in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace radix_dev
