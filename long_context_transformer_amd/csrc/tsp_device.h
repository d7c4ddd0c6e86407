// tsp_device.h -- device helpers shared by the gfx950 kernels of the TSP rank-shard layer.
//
// CDNA4 (gfx950) specifics used here:
//  * wave64; bf16 MFMA v_mfma_f32_32x32x16_bf16: operand A gives row i = lane%32,
//    operand B gives column j = lane%32, each lane supplying 8 bf16 of the reduction
//    dimension selected by lane/32; the 32x32 fp32 result puts column j = lane%32 and
//    rows 8*(r/4) + 4*(lane/32) + r%4 in accumulator register r (r = 0..15).
//    Only the pairing "lane group g, element e of A meets lane group g, element e of
//    B" matters for the reduction, so any consistent relabelling of the reduction
//    index between the two operands gives the same product.
//  * 8 XCDs: consecutive workgroup ids are dealt round-robin to the XCDs, each with
//    its own L2; xcd_remap gives every XCD a contiguous range of logical work items
//    so that items sharing operands share an L2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace tsp {

typedef uint16_t bf16_t;  // storage type of a bfloat16 in global memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

// Two fp32 -> packed bf16 pair (round to nearest even; gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

__device__ __forceinline__ bf16_t to_bf16(float x) {
  __bf16 v = (__bf16)x;
  return __builtin_bit_cast(bf16_t, v);
}

// 16-byte global -> LDS copies (global_load_lds_dwordx4): lane i's 16 bytes land at LDS
// byte address `lds` + 16 i, where `lds` is the same for the whole wave (it goes to M0).
// Issued from inline assembly on purpose: the compiler then neither tracks these writes
// nor inserts its own conservative waits before LDS reads; callers order them with
// explicit s_waitcnt vmcnt (loads retire in order) and s_barrier. Nothing else in these
// kernels uses M0. A scalar write of M0 needs one wait state before an LDS DMA reads it
// (the compiler puts an s_nop 0 there for its own global_load_lds), hence the s_nop.
//   dma16_sbase: address = uniform 64-bit base + per-lane 32-bit byte offset
//   dma16_vaddr: address = per-lane 64-bit pointer
__device__ __forceinline__ void dma16_sbase(const void* base, uint32_t voff, uint32_t lds) {
  // The base must sit in SGPRs: read it from the first lane (free when already scalar).
  // readfirstlane returns int: each half is taken as uint32_t before widening, so the low
  // half is zero-extended.
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  const uint64_t ps = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(ps), "s"(lds) : "memory");
}
// 4-byte form of dma16_sbase (global_load_lds_dword): one lane per 128-byte line pulls lines
// into the caches ahead of their 16-byte loads; its LDS destination is scratch nobody reads.
__device__ __forceinline__ void dma4_sbase(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  const uint64_t ps = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(ps), "s"(lds) : "memory");
}
__device__ __forceinline__ void dma16_vaddr(const void* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "s"(lds) : "memory");
}
// LDS byte address of a pointer into a __shared__ array, made wave-uniform.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}

// max(v of this lane, v of lane ^ 32) in registers (v_permlane32_swap exchanges the upper
// half of the first operand with the lower half of the second; with both holding v, the
// pair's max is the max across the two half-waves). Inline assembly: this compiler folds
// a max of the intrinsic's two results to its first result. The s_nops give the wait
// states around the permute. Inputs are finite or -inf.
__device__ __forceinline__ float max_swap32(float v) {
  uint32_t x = __builtin_bit_cast(uint32_t, v), y = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1" : "+v"(x), "+v"(y));
  return __builtin_bit_cast(float, x);
}

// Lanes 16..31 of x trade places with lanes 0..15 of y, and lanes 48..63 of x with lanes
// 32..47 of y (v_permlane16_swap), with the wait states around the permute.
__device__ __forceinline__ void swap16(uint32_t& x, uint32_t& y) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// s_waitcnt immediate that waits until at most `vm` vector-memory loads of this wave are
// in flight, leaving the export and LDS counters unconstrained.
constexpr int waitcnt_vm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (15 << 8); }

// Global position of local row i of rank r, for chunk length C and fold D.
// Rows 0..C-1 are chunk r, rows C..2C-1 are the mirror chunk 2D-1-r.
__host__ __device__ __forceinline__ int64_t zigzag_pos(int64_t i, int64_t C, int r, int D) {
  return i < C ? (int64_t)r * C + i : (int64_t)(2 * D - 1 - r) * C + (i - C);
}

// Bijection of [0, n) that maps the workgroups of XCD x (blockIdx % 8 == x) onto a
// contiguous block of logical ids, in dispatch order.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int x = bid % kNumXcd;
  const int local = bid / kNumXcd;
  const int q = n / kNumXcd;
  const int rem = n % kNumXcd;
  const int start = x * q + (x < rem ? x : rem);
  return start + local;
}

}  // namespace tsp
