// LDS plumbing shared by the backward kernels (gfx950): LDS-direct tile
// copies, the row / transpose read helpers and the 16-byte-slot swizzle.
#pragma once

#include "fa_common.h"

namespace fa {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x4 lds_u4;
typedef __attribute__((address_space(3))) const f32x4 lds_f4;
typedef __attribute__((address_space(3))) u32x4 lds_u4_out;

// Slot swizzle for tiles read both row-wise (16 consecutive rows, one 16-byte
// slot each) and by transpose reads (4 consecutive rows x 4 slots): the
// 16-byte slot of chunk c in row r is c ^ swz(r).  It depends on r % 16 only,
// and swz(r + 4) = swz(r) ^ 1, swz(r + 8) = swz(r) ^ 2 when r % 16 < 4 resp. 8.
template <int ROW_BYTES>
__device__ __forceinline__ constexpr int swz(int r) {
  return ROW_BYTES == 256 ? (4 * (r & 3) | ((r >> 2) & 3)) : (4 * ((r >> 1) & 1) | ((r >> 2) & 3));
}

__device__ __forceinline__ void lds_copy(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_copy4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("buffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds) : "memory");
}
// vmcnt(0) as the compiler's own wait instruction (vmcnt 0, expcnt 7,
// lgkmcnt 15 in the gfx9 encoding), so its wait-count tracking knows that
// every earlier vector memory load has completed and adds no wait of its
// own for registers loaded before (an asm wait is opaque to it, and it then
// kept a vmcnt(0) in every iteration, which also waited for the copies just
// issued for the next tile); the empty asm keeps memory accesses in place.
__device__ __forceinline__ void wait_loads() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// Hides a lane constant from the optimizer so that it stays one register
// instead of being re-derived at every use.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// A transpose read: four bf16 of one column, 4 consecutive rows; two of them
// make the 8-element operand.  Arguments are LDS byte addresses.
__device__ __forceinline__ bf16x8 tr_pair(uint32_t a0, uint32_t a1) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)a0);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)a1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ bf16x8 lds_row16(uint32_t a) { return __builtin_bit_cast(bf16x8, *(lds_u4*)(uintptr_t)a); }

}  // namespace fa
