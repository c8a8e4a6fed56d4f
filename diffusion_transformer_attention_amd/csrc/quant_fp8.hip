// Per-(b, h) quantization of bf16 [B,H,N,D] to 8-bit floating point, OCP
// E4M3 (FP8 low precision as the last step of the latency ladder in "Multi-GPU
// parallelism: spreading one step over several cards", section "Combining:
// what xDiT does"; the format and per-head scaling are this library's
// reading of it):
//   descale[b,h] = amax / 448 (float32, correctly rounded; 1 for an all-zero
//                  head), amax = max |x| over the head
//   code         = E4M3(clamp(x / descale, -448, 448)), the quotient correctly
//                  rounded in float32, the conversion round-to-nearest-even
// Three launches for one or two tensors (q and k of one attention call
// together): clear the descale words; one pass for amax, whose blocks fold
// their maxima into the head's word with an unsigned atomic max of
// (amax bits | 0x80000000) (a non-negative float orders like its bit pattern,
// so the max is exact and order-independent, and the set top bit marks the
// word as an amax); one pass writing the codes, in which every block turns
// the word into the descale itself -- a word with the top bit clear is
// already the descale -- and the first block of each head stores it (every
// block would store the same value, so the order of these stores does not
// matter).  HBM-bound: x is read twice and the codes written once (5 bytes
// per element).
// Power-of-two form (q and k of one attention call, for the fp8 product that
// takes E8M0 scales): x' = float32(x * pre) with pre = scale * log2(e) for q
// and 1 for k; descale = the smallest 2^e (e >= -126) with max |x'| <= 448 *
// 2^e (1 for an all-zero head); code = E4M3(x' / descale), the quotient
// exact.  max |x'| = float32(amax * pre), rounding being monotonic, so the
// same amax pass serves.
#include "launch.h"

namespace ditattn {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;  // 16-byte vectors (8 elements) per thread per block step
constexpr float kE4M3Max = 448.0f;
constexpr unsigned kAmaxTag = 0x80000000u;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// One or two tensors of the same [B,H] head grid.
struct QuantJob {
  const u32x4* x[2];
  u32x2* codes[2];
  unsigned* word[2];       // the descale buffers, as words
  int64_t vec_per_head[2];  // 16-byte vectors per head (0: empty tensor)
  int blocks[2];            // blocks per head of the pass
  float pre[2];             // power-of-two form: factor applied to x first
  int ntensors, nbh;
  int pow2;                 // power-of-two descales
};

// Block ids: tensor 0's heads first, then tensor 1's; within a tensor, head
// then chunk.
__device__ __forceinline__ void block_of(const QuantJob& j, int& t, int& bh, int& chunk) {
  int b = blockIdx.x;
  t = 0;
  const int n0 = j.nbh * j.blocks[0];
  if (b >= n0) {
    t = 1;
    b -= n0;
  }
  bh = b / j.blocks[t];
  chunk = b - bh * j.blocks[t];
}

// Clear every descale word; an empty tensor's heads get their final descale 1.
__global__ void init_kernel(QuantJob j) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  for (int t = 0; t < j.ntensors; ++t)
    if (i < j.nbh) j.word[t][i] = j.vec_per_head[t] > 0 ? 0u : __float_as_uint(1.0f);
}

// Block b of a head strides over it, so a head takes at most kAmaxBlocks
// atomics (thousands of atomics on one address serialize at L2).
constexpr int kAmaxBlocks = 64;

__global__ __launch_bounds__(kThreads) void amax_kernel(QuantJob j) {
  int t, bh, chunk;
  block_of(j, t, bh, chunk);
  const int64_t vph = j.vec_per_head[t];
  const u32x4* src = j.x[t] + (int64_t)bh * vph;
  float m = 0.0f;
  const int64_t step = (int64_t)j.blocks[t] * kVec * kThreads;
  for (int64_t base = (int64_t)chunk * kVec * kThreads; base < vph; base += step) {
    u32x4 v[kVec];
#pragma unroll
    for (int u = 0; u < kVec; ++u) {  // all loads first
      const int64_t i = base + u * kThreads + threadIdx.x;
      v[u] = i < vph ? src[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kVec; ++u)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        m = fmaxf(m, __uint_as_float((v[u][w] & 0x7fffu) << 16));
        m = fmaxf(m, __uint_as_float(v[u][w] & 0x7fff0000u));
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
    atomicMax(j.word[t] + bh, __float_as_uint(m) | kAmaxTag);
  }
}

__device__ __forceinline__ float descale_of(unsigned amax_bits) {
  const float a = __uint_as_float(amax_bits);
  return a > 0.0f ? __fdiv_rn(a, kE4M3Max) : 1.0f;
}

// Smallest power of two d (d >= 2^-126) with a <= 448 d, for a >= 0 (1 for
// a = 0).  a = (1 + M 2^-23) 2^k and 448 = 1.75 2^8, so d = 2^(k-8) when
// M <= 0.75 2^23 and 2^(k-7) otherwise; subnormal a takes 2^-126.
__device__ __forceinline__ float pow2_descale_of(float a) {
  if (!(a > 0.0f)) return 1.0f;
  const unsigned bits = __float_as_uint(a);
  const int E = (int)(bits >> 23), M = (int)(bits & 0x7fffffu);
  int e = E == 0 ? -126 : (E - 127) - (M <= 0x600000 ? 8 : 7);
  e = e < -126 ? -126 : e;
  return __uint_as_float((unsigned)(e + 127) << 23);
}

// The head's descale from its word: an amax (top bit set) or the descale.
__device__ __forceinline__ float descale_from_word(unsigned w, float pre, int pow2) {
  if (!(w & kAmaxTag)) return __uint_as_float(w);
  const unsigned a = w & ~kAmaxTag;
  return pow2 ? pow2_descale_of(__fmul_rn(__uint_as_float(a), pre)) : descale_of(a);
}

__device__ __forceinline__ float quotient(float v, float d) {
  return fminf(fmaxf(__fdiv_rn(v, d), -kE4M3Max), kE4M3Max);
}

__global__ __launch_bounds__(kThreads) void quant_kernel(QuantJob j) {
  int t, bh, chunk;
  block_of(j, t, bh, chunk);
  const int64_t vph = j.vec_per_head[t];
  const float pre = j.pre[t];
  const float d = descale_from_word(__atomic_load_n(j.word[t] + bh, __ATOMIC_RELAXED), pre, j.pow2);
  // x' = x * pre in the power-of-two form (pre = 1 otherwise: x' = x exactly)
  auto xv = [&](unsigned bits) { return __fmul_rn(__uint_as_float(bits), pre); };
  const u32x4* src = j.x[t] + (int64_t)bh * vph;
  u32x2* dst = j.codes[t] + (int64_t)bh * vph;
  u32x4 v[kVec];
#pragma unroll
  for (int u = 0; u < kVec; ++u) {  // all loads first
    const int64_t i = ((int64_t)chunk * kVec + u) * kThreads + threadIdx.x;
    v[u] = i < vph ? src[i] : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const int64_t i = ((int64_t)chunk * kVec + u) * kThreads + threadIdx.x;
    if (i < vph) {
      unsigned out[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned w0 = v[u][2 * h], w1 = v[u][2 * h + 1];
        unsigned r = __builtin_amdgcn_cvt_pk_fp8_f32(quotient(xv(w0 << 16), d),
                                                     quotient(xv(w0 & 0xffff0000u), d), 0, false);
        r = __builtin_amdgcn_cvt_pk_fp8_f32(quotient(xv(w1 << 16), d),
                                            quotient(xv(w1 & 0xffff0000u), d), r, true);
        out[h] = r;
      }
      // streaming store: the codes are not read again by this call
      // (non-temporal: 78.2 -> 74.9 us for the q and k of B1 H10 N32768 D128;
      // non-temporal loads of x as well measured slower)
      __builtin_nontemporal_store(u32x2{out[0], out[1]}, dst + i);
    }
  }
  if (chunk == 0 && threadIdx.x == 0)
    __atomic_store_n(j.word[t] + bh, __float_as_uint(d), __ATOMIC_RELAXED);
}

}  // namespace

namespace {
hipError_t launch_quant(const void* const* x, void* const* codes, float* const* descale,
                        const int* N, int ntensors, int B, int H, int D, const float* pre, int pow2,
                        hipStream_t stream) {
  QuantJob j{};
  j.ntensors = ntensors;
  j.nbh = B * H;
  j.pow2 = pow2;
  const int64_t per_block = (int64_t)kVec * kThreads;
  int64_t qblocks = 0, ablocks = 0;
  for (int t = 0; t < ntensors; ++t) {
    j.x[t] = static_cast<const u32x4*>(x[t]);
    j.codes[t] = static_cast<u32x2*>(codes[t]);
    j.word[t] = reinterpret_cast<unsigned*>(descale[t]);
    j.vec_per_head[t] = (int64_t)N[t] * D / 8;
    j.pre[t] = pre[t];
    const int64_t bph = (j.vec_per_head[t] + per_block - 1) / per_block;
    if (bph * j.nbh > 0x3fffffff) return hipErrorInvalidValue;
    qblocks += bph * j.nbh;
    ablocks += (bph < kAmaxBlocks ? bph : kAmaxBlocks) * j.nbh;
  }
  const unsigned small = (unsigned)((j.nbh + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(init_kernel, dim3(small), dim3(kThreads), 0, stream, j);
  if (qblocks > 0) {  // an empty tensor has 0 blocks; its descale is already final
    QuantJob a = j;
    for (int t = 0; t < ntensors; ++t) {
      const int64_t bph = (j.vec_per_head[t] + per_block - 1) / per_block;
      a.blocks[t] = (int)(bph < kAmaxBlocks ? bph : kAmaxBlocks);
      j.blocks[t] = (int)bph;
    }
    hipLaunchKernelGGL(amax_kernel, dim3((unsigned)ablocks), dim3(kThreads), 0, stream, a);
    hipLaunchKernelGGL(quant_kernel, dim3((unsigned)qblocks), dim3(kThreads), 0, stream, j);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_quant_fp8_n(const void* const* x, void* const* codes, float* const* descale,
                              const int* N, int ntensors, int B, int H, int D,
                              hipStream_t stream) {
  const float one[2] = {1.0f, 1.0f};
  return launch_quant(x, codes, descale, N, ntensors, B, H, D, one, 0, stream);
}

hipError_t launch_quant_fp8(const void* x, void* codes, float* descale, int B, int H, int N, int D,
                            hipStream_t stream) {
  return launch_quant_fp8_n(&x, &codes, &descale, &N, 1, B, H, D, stream);
}

hipError_t launch_quant_fp8_mx(const void* q, const void* k, void* q_codes, void* k_codes,
                               float* q_descale, float* k_descale, int B, int H, int Nq, int Nkv,
                               int D, float c0, hipStream_t stream) {
  const void* x[2] = {q, k};
  void* c[2] = {q_codes, k_codes};
  float* ds[2] = {q_descale, k_descale};
  const int n[2] = {Nq, Nkv};
  const float pre[2] = {c0, 1.0f};
  return launch_quant(x, c, ds, n, 2, B, H, D, pre, 1, stream);
}

}  // namespace ditattn
