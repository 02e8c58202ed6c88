// Global-to-LDS loads and LDS fragment reads for gfx950, shared by the GEMM
// and the rank-r kernels.
#pragma once

#include "common.hpp"

namespace lora {

typedef __attribute__((address_space(3))) char lds_char;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Values the compiler cannot prove uniform are moved to scalar registers.
__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Buffer descriptor as four scalar words (base, stride 0, byte size, format)
// for the inline-assembly load below; every input is uniform.  bytes is
// clamped to [0, 2^31 - 1].
__device__ __forceinline__ i32x4 rsrc_words(const void* p, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7fffffff) bytes = 0x7fffffff;
  const uint64_t base = (uint64_t)uni64(reinterpret_cast<int64_t>(p));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return i32x4{(int)(uint32_t)base, (int)((base >> 32) & 0xffff), n, 0x00020000};
}

// Range-checked buffer access to a row-major [rows, ld] operand (raw buffer,
// stride 0): a 16-byte access at a byte offset at or past the descriptor's
// size loads zeros, and a store there is dropped.  Epilogues address rows
// past the last one this way without per-lane branches.  bytes is clamped
// to [0, 2^31 - 1].
typedef __amdgpu_buffer_rsrc_t brsrc;
__device__ __forceinline__ brsrc make_rsrc(const void* p, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7fffffff) bytes = 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// Byte offset of element (m, n) of a row-major [M, ld] operand of es-byte
// elements; rows at or past M get an offset past every descriptor (2^31), so
// their accesses read zero or are dropped.  For m < M the offset is below
// 2^31 because every operand is smaller than 2 GiB.
__device__ __forceinline__ uint32_t row_off(int64_t m, int64_t M, int64_t ld, int64_t n, int es) {
  return m < M ? (uint32_t)((m * ld + n) * es) : 0x80000000u;
}
__device__ __forceinline__ u32x4 buf_load16(brsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void buf_store16(brsrc r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store16f(brsrc r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}

// 16 bytes per lane from global memory into LDS: lane i writes bytes
// lds_addr + 16 i .. + 15 with the bytes at voff + soff of the descriptor;
// offsets past the descriptor's size read zero.
// Issued as inline assembly so that the compiler does not wait for these
// loads before unrelated LDS reads (it cannot tell ring slots apart); the
// kernels wait with an explicit vmcnt and a barrier before they read a slot,
// and they issue no other vector-memory loads while such loads are in flight.
// lds_addr and soff must be uniform; they are moved to scalar registers here
// (a no-op when they already are) because the instruction takes them there.
__device__ __forceinline__ void dma16(const i32x4& r, uint32_t voff, uint32_t lds_addr, uint32_t soff = 0) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  soff = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :
               : "v"(voff), "s"(r), "s"(lds_addr), "s"(soff)
               : "memory", "m0");
}

// 4 bytes per lane: lane i writes bytes lds_addr + 4 i .. + 3 with the dword
// at voff of the descriptor (zero past its size); same rules as dma16.
__device__ __forceinline__ void dma4(const i32x4& r, uint32_t voff, uint32_t lds_addr) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(lds_addr)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N) (N <= 63), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) { return (uint32_t)(uintptr_t)p; }
__device__ __forceinline__ u32x4 lds_read16(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(p);
}
// ds_read_b64_tr_b16: lane 16 g + i receives element i % 4 of the 8 bytes
// that lanes 16 g + 4 j + i / 4 (j = 0..3) point at, as elements j.
__device__ __forceinline__ uint64_t lds_read_tr(const lds_char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(uint64_t, v);
}
// Two transposing reads (rows r and r + 4 of a K-group of 8) as one 8-value operand.
__device__ __forceinline__ bf16x8 lds_read_tr8(const lds_char* p, int second_off) {
  const uint64_t lo = lds_read_tr(p);
  const uint64_t hi = lds_read_tr(p + second_off);
  u32x4 v;
  v[0] = (uint32_t)lo;
  v[1] = (uint32_t)(lo >> 32);
  v[2] = (uint32_t)hi;
  v[3] = (uint32_t)(hi >> 32);
  return __builtin_bit_cast(bf16x8, v);
}
// The same with the two reads at addresses of their own.
__device__ __forceinline__ bf16x8 lds_read_tr8(const lds_char* p, const lds_char* q) {
  const uint64_t lo = lds_read_tr(p);
  const uint64_t hi = lds_read_tr(q);
  u32x4 v;
  v[0] = (uint32_t)lo;
  v[1] = (uint32_t)(lo >> 32);
  v[2] = (uint32_t)hi;
  v[3] = (uint32_t)(hi >> 32);
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace lora
