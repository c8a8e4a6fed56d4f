// Joint text + image sequence with rotary position embedding ("Parallelism
// Acceleration Guide", vLLM-Omni docs, section "How to parallelize a new
// model": a dual-stream model attends jointly over its concatenated text and
// image tokens; the text stays whole on every sequence-parallel rank).
//
// For each (b, h) the output holds the Nt text tokens of head h0 + h of the
// text tensor [B,Ht,Nt,D], then the Ni image tokens of head h of the image
// tensor [B,H,Ni,D].  A part whose cosine/sine tables ([N, D/2] float32) are
// given has every channel pair (2i, 2i+1) of token n turned by that token's
// angle for pair i:
//   y[2i] = x[2i] cos - x[2i+1] sin,  y[2i+1] = x[2i] sin + x[2i+1] cos
// computed in float32 and rounded to bf16 (nearest, ties to even); a part
// without tables is copied bit for bit.
//
// HBM-bound: every element is read and written once; each lane moves 16
// bytes (four channel pairs) per step with one float4 of cosines and one of
// sines, which the heads of a launch share through L2.  One launch packs up
// to three tensors (q, k, v): blockIdx.y picks the tensor.
#include "launch.h"
#include "rope.h"

namespace ditattn {
namespace {

constexpr int kThreads = 256;
constexpr int kTok = 64;  // tokens per workgroup

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct PackSet {
  RopePackTensor t[3];
};

template <int D>
__global__ __launch_bounds__(kThreads) void rope_pack_kernel(PackSet set, int H, int Ht, int h0,
                                                             int Nt, int Ni, int ntt) {
  constexpr int CPT = D / 8;  // 16-byte chunks per token
  // Uniform selection keeps the pointers in scalar registers.
  const RopePackTensor a = blockIdx.y == 0 ? set.t[0] : blockIdx.y == 1 ? set.t[1] : set.t[2];
  const int bh = blockIdx.x / ntt;
  const int tt = blockIdx.x - bh * ntt;
  const int b = bh / H, h = bh - b * H;
  const int N = Nt + Ni;
  const __bf16* txt =
      Nt ? static_cast<const __bf16*>(a.txt) + ((int64_t)b * Ht + h0 + h) * Nt * D : nullptr;
  const __bf16* img = Ni ? static_cast<const __bf16*>(a.img) + ((int64_t)b * H + h) * Ni * D : nullptr;
  __bf16* out = static_cast<__bf16*>(a.out) + ((int64_t)b * H + h) * N * D;
#pragma unroll
  for (int it = 0; it < kTok * CPT / kThreads; ++it) {
    const int i = it * kThreads + threadIdx.x;
    const int n = tt * kTok + i / CPT, c = i % CPT;
    if (n >= N) continue;
    const bool is_txt = n < Nt;
    const int m = is_txt ? n : n - Nt;
    const u32x4 x = *reinterpret_cast<const u32x4*>((is_txt ? txt : img) + (int64_t)m * D + 8 * c);
    const float* ct = is_txt ? a.cos_txt : a.cos_img;
    const float* st = is_txt ? a.sin_txt : a.sin_img;
    u32x4 y = x;
    if (ct) {
      const f32x4 cv = *reinterpret_cast<const f32x4*>(ct + (int64_t)m * (D / 2) + 4 * c);
      const f32x4 sv = *reinterpret_cast<const f32x4*>(st + (int64_t)m * (D / 2) + 4 * c);
#pragma unroll
      for (int p = 0; p < 4; ++p) y[p] = rope_turn_pair(x[p], cv[p], sv[p]);
    }
    *reinterpret_cast<u32x4*>(out + ((int64_t)n * D + 8 * c)) = y;
  }
}

}  // namespace

hipError_t launch_rope_pack(const RopePackTensor* tensors, int ntensors, int B, int H, int Ht,
                            int h0, int Nt, int Ni, int D, hipStream_t stream) {
  PackSet set{};
  for (int i = 0; i < ntensors; ++i) set.t[i] = tensors[i];
  const int ntt = (Nt + Ni + kTok - 1) / kTok;
  const int64_t gx = (int64_t)B * H * ntt;
  if (gx > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)gx, (unsigned)ntensors);
  switch (D) {
    case 32:
      hipLaunchKernelGGL(rope_pack_kernel<32>, grid, dim3(kThreads), 0, stream, set, H, Ht, h0, Nt,
                         Ni, ntt);
      break;
    case 64:
      hipLaunchKernelGGL(rope_pack_kernel<64>, grid, dim3(kThreads), 0, stream, set, H, Ht, h0, Nt,
                         Ni, ntt);
      break;
    default:
      hipLaunchKernelGGL(rope_pack_kernel<128>, grid, dim3(kThreads), 0, stream, set, H, Ht, h0,
                         Nt, Ni, ntt);
      break;
  }
  return hipGetLastError();
}

}  // namespace ditattn
