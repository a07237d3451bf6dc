// Internal definitions shared by the HIP translation units of liboscar.
// The pool layout implemented here is the one documented in include/oscar.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar {

constexpr int kPage = 16;  // tokens per page

__host__ __device__ constexpr int int2_block_bytes(int d, int ng) { return 8 * d + 128 * ng; }
__host__ __device__ constexpr int bf16_block_bytes(int d) { return 64 * d; }

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Remap the dispatch id so that each XCD receives one contiguous range
// of logical work units: units of one (sequence, KV head) then share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int q = nblocks / kXcd, r = nblocks % kXcd;
  const int xcd = bid % kXcd, idx = bid / kXcd;
  return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// dword 3 of a gfx950 buffer descriptor for raw (untyped) access: 32-bit
// data format, no swizzle; loads at offsets past num_records read zero and
// stores there are dropped
constexpr int kBufferFlags = 0x00020000;

// a wave-uniform pointer held in scalar registers
__device__ __forceinline__ void* uniform_ptr(const void* q) {
  const uint64_t u = (uint64_t)q;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (void*)(((uint64_t)hi << 32) | lo);
}

// DPP row rotate (within 16-lane rows): lane i reads lane (i + n) % 16.
template <int N>
__device__ __forceinline__ float dpp_row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}

}  // namespace oscar
