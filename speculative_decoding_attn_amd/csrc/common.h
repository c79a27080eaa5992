// Device-side helpers shared by the gfx950 kernels: vector types for the bf16
// MFMA operands, bf16 conversion, wave64 reductions, status plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace eagle {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
// s_waitcnt immediate for "vmcnt(0)" with expcnt and lgkmcnt left at their maxima
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32 fp32) += A(32x16 bf16) * B(16x32 bf16).  Lane l supplies A row l%32 and
// B column l%32, each with k = 8*(l/32) .. 8*(l/32)+7; it receives D column l%32,
// rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 x) { return __builtin_bit_cast(u32x4, x); }

// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ bf16x2 to_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_convertvector(v, bf16x2);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, to_bf16x2(a, b));
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t x) {
  return __builtin_bit_cast(float, (uint32_t)x << 16);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N-1>{}):
// a loop whose index is a compile-time constant in every iteration (register arrays
// indexed with it stay in registers, whatever the size of the body).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Waits until at most N vector-memory operations of this wave are outstanding
// (loads complete in issue order), for loads the compiler does not track.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit counter");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// global -> LDS copy of 16 bytes per lane: lane i's bytes land at LDS byte address
// m0 + 16*i, one contiguous KiB per wave.  Issued through inline assembly: for the
// compiler's own form of this load it waits for every outstanding load before any
// later LDS read, which would drain the pipeline each block.  Completion is waited
// for with wait_vmcnt<N>() and published to the other waves with a barrier.
// (m0 is a reserved register to the compiler, hence the warning about its clobber;
// the kernels' assembly is checked to use m0 nowhere else.  The s_nop is the wait
// state the ISA asks for between an SALU write of m0 and an LDS DMA that reads it.)
// p read from the first lane: a wave-uniform pointer the compiler keeps in SGPRs.
// readfirstlane returns a signed int, so each half goes through uint32_t: the low half
// must be zero-extended (a sign extension would set the high half to all ones).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return (T*)(uintptr_t)((uint64_t)lo | ((uint64_t)hi << 32));
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_byte_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_byte_addr))
               : "memory", "m0");
}
// The same copy with the non-temporal cache policy, for data read exactly once (a
// weight stream): its lines are not kept in the caches at the expense of operands
// that are reused, such as the hidden rows every workgroup re-reads from L2.
__device__ __forceinline__ void dma16_nt(const void* src, uint32_t lds_byte_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_byte_addr))
               : "memory", "m0");
}
// The same non-temporal copy from a wave-uniform base address plus a per-lane byte
// offset (the scalar-base form of the load): the base is kept in scalar registers,
// so a stream that advances by whole blocks costs no vector instruction per load.
__device__ __forceinline__ void dma16_nt_s(const void* base, uint32_t off, uint32_t lds_byte_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(off), "s"(uniform_ptr(base)),
                 "s"(__builtin_amdgcn_readfirstlane(lds_byte_addr))
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}

// Ancestor-or-self bitmask of node i (bit a set for every a on the root path of
// i).  Walks at most 64 parent links and stops at any link that breaks the tree
// rules, so it is memory-safe for any parent content.
__device__ __forceinline__ uint64_t ancestor_mask(const int32_t* par, int i, int N) {
  uint64_t m = 0;
  int n = i;
  for (int step = 0; step < 64; ++step) {
    if (n < 0 || n >= N) break;
    m |= 1ull << n;
    int p = par[n];
    if (p >= n) break;
    n = p;
  }
  return m;
}

}  // namespace eagle
