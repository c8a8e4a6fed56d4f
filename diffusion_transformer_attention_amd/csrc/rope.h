// The rotary turn of one channel pair, shared by the pack kernel and the
// attention kernel's query load so both round the same way ("Parallelism
// Acceleration Guide", vLLM-Omni docs, "How to parallelize a new model": the
// image and text rotary tables; the turn is this library's reading,
// RoFormer's rotary embedding in interleaved form):
//   y[2i] = x[2i] cos - x[2i+1] sin,  y[2i+1] = x[2i] sin + x[2i+1] cos
// in float32, rounded to bf16 (nearest, ties to even).
#pragma once
#include <hip/hip_runtime.h>

namespace ditattn {

__device__ __forceinline__ float rope_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float rope_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ unsigned rope_pack2(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  return (unsigned)__builtin_bit_cast(unsigned short, x) |
         ((unsigned)__builtin_bit_cast(unsigned short, y) << 16);
}

// One 32-bit word holds the pair (x[2i], x[2i+1]) in its low and high halves.
__device__ __forceinline__ unsigned rope_turn_pair(unsigned w, float c, float s) {
  const float x0 = rope_lo(w), x1 = rope_hi(w);
  return rope_pack2(fmaf(x0, c, -(x1 * s)), fmaf(x0, s, x1 * c));
}

}  // namespace ditattn
