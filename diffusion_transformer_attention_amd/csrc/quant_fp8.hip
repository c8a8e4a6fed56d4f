// Per-(b, h) quantization of bf16 [B,H,N,D] to 8-bit floating point, OCP
// E4M3 (FP8 low precision as the last step of the latency ladder in "Multi-GPU
// parallelism: spreading one step over several cards", section "Combining:
// what xDiT does"; the format and per-head scaling are this library's
// reading of it):
//   descale[b,h] = amax / 448 (float32, correctly rounded; 1 for an all-zero
//                  head), amax = max |x| over the head
//   code         = E4M3(clamp(x / descale, -448, 448)), the quotient correctly
//                  rounded in float32, the conversion round-to-nearest-even
// Four launches: zero the descale buffer, which then holds amax as float
// bits (a non-negative float orders like its bit pattern, so an unsigned
// atomic max is exact and order-independent); one pass for amax; one pass
// writing the codes; last, amax -> descale in place.  HBM-bound: x is read twice and
// the codes written once (5 bytes per element).
#include "launch.h"

namespace ditattn {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;  // 16-byte vectors (8 elements) per thread per block step
constexpr float kE4M3Max = 448.0f;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__global__ void zero_kernel(float* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// Block b handles head b / bph and strides over it, so a head takes at most
// kAmaxBlocks atomics (thousands of atomics on one address serialize at L2).
constexpr int kAmaxBlocks = 64;

__global__ __launch_bounds__(kThreads) void amax_kernel(const u32x4* __restrict__ x,
                                                       unsigned* __restrict__ amax,
                                                       int64_t vec_per_head, int bph) {
  const int bh = blockIdx.x / bph;
  const int chunk = blockIdx.x - bh * bph;
  const u32x4* src = x + (int64_t)bh * vec_per_head;
  float m = 0.0f;
  const int64_t step = (int64_t)bph * kVec * kThreads;
  for (int64_t base = (int64_t)chunk * kVec * kThreads; base < vec_per_head; base += step) {
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      if (i < vec_per_head) {
        const u32x4 v = src[i];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          m = fmaxf(m, __uint_as_float((v[w] & 0x7fffu) << 16));
          m = fmaxf(m, __uint_as_float(v[w] & 0x7fff0000u));
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  __shared__ float wmax[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, wmax[w]);
    atomicMax(amax + bh, __float_as_uint(m));
  }
}

__device__ __forceinline__ float descale_of(unsigned amax_bits) {
  const float a = __uint_as_float(amax_bits);
  return a > 0.0f ? __fdiv_rn(a, kE4M3Max) : 1.0f;
}

__device__ __forceinline__ float quotient(float v, float d) {
  return fminf(fmaxf(__fdiv_rn(v, d), -kE4M3Max), kE4M3Max);
}

__global__ __launch_bounds__(kThreads) void quant_kernel(const u32x4* __restrict__ x,
                                                        u32x2* __restrict__ codes,
                                                        const unsigned* __restrict__ amax,
                                                        int64_t vec_per_head, int bph) {
  const int bh = blockIdx.x / bph;
  const int chunk = blockIdx.x - bh * bph;
  const float d = descale_of(amax[bh]);
  const u32x4* src = x + (int64_t)bh * vec_per_head;
  u32x2* dst = codes + (int64_t)bh * vec_per_head;
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const int64_t i = ((int64_t)chunk * kVec + u) * kThreads + threadIdx.x;
    if (i < vec_per_head) {
      const u32x4 v = src[i];
      unsigned out[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned w0 = v[2 * h], w1 = v[2 * h + 1];
        unsigned r = __builtin_amdgcn_cvt_pk_fp8_f32(quotient(__uint_as_float(w0 << 16), d),
                                                     quotient(__uint_as_float(w0 & 0xffff0000u), d),
                                                     0, false);
        r = __builtin_amdgcn_cvt_pk_fp8_f32(quotient(__uint_as_float(w1 << 16), d),
                                            quotient(__uint_as_float(w1 & 0xffff0000u), d), r, true);
        out[h] = r;
      }
      dst[i] = u32x2{out[0], out[1]};
    }
  }
}

__global__ void finalize_kernel(float* __restrict__ descale, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) descale[i] = descale_of(__float_as_uint(descale[i]));
}

}  // namespace

hipError_t launch_quant_fp8(const void* x, void* codes, float* descale, int B, int H, int N, int D,
                            hipStream_t stream) {
  const int nbh = B * H;
  const int64_t vec_per_head = (int64_t)N * D / 8;
  const int64_t per_block = (int64_t)kVec * kThreads;
  const int64_t bph = (vec_per_head + per_block - 1) / per_block;
  if (bph * nbh > 0x7fffffff) return hipErrorInvalidValue;
  const unsigned small = (unsigned)((nbh + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(zero_kernel, dim3(small), dim3(kThreads), 0, stream, descale, nbh);
  if (bph > 0) {  // N == 0: every head is empty, amax stays 0 and descale becomes 1
    const int64_t abph = bph < kAmaxBlocks ? bph : kAmaxBlocks;
    hipLaunchKernelGGL(amax_kernel, dim3((unsigned)(abph * nbh)), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(x), reinterpret_cast<unsigned*>(descale),
                       vec_per_head, (int)abph);
    hipLaunchKernelGGL(quant_kernel, dim3((unsigned)(bph * nbh)), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(x), static_cast<u32x2*>(codes),
                       reinterpret_cast<const unsigned*>(descale), vec_per_head, (int)bph);
  }
  hipLaunchKernelGGL(finalize_kernel, dim3(small), dim3(kThreads), 0, stream, descale, nbh);
  return hipGetLastError();
}

}  // namespace ditattn
