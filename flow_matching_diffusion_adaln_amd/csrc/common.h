// Internal helpers shared by the gfx950 kernels of the DiT block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define DIT_LOG2E 1.4426950408889634f

namespace dit {

// bf16 bit pattern -> float (exact)
__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// low / high bf16 halves of a packed dword -> float
__device__ __forceinline__ float lo2f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi2f(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// two floats -> packed bf16 dword, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Segment (stream) of a row: rows [0, e0) are stream 0, [e0, e1) stream 1, rest stream 2.
__device__ __forceinline__ int stream_of(int row, int e0, int e1) {
  return (row >= e0) + (row >= e1);
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on
// XCD i % 8).  Map the hardware id to a logical id so that each XCD works on
// one contiguous range of logical ids, which then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int hw_id, int total) {
  const int per = total / 8, rem = total % 8;
  const int x = hw_id % 8, loc = hw_id / 8;
  return x * per + (x < rem ? x : rem) + loc;
}

}  // namespace dit
