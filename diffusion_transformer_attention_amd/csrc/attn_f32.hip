// float32 non-causal attention with log-sum-exp, on the vector ALUs.
//
// Serves float32 inputs (the handbook's four-card Ulysses simulation runs in
// float32: "Multi-GPU parallelism: spreading one step over several cards",
// section "Sequence parallelism: Ulysses and Ring").  It is not a
// performance path: one thread owns one query row, K/V tiles are staged in
// LDS and read as broadcasts, and the softmax is the block-wise running
// max / running sum of the Ring paragraph, in float32 throughout.
#include <math.h>

#include "launch.h"

namespace ditattn {
namespace {

constexpr int kRows = 64;  // query rows per workgroup (one wave)
constexpr int kTK = 32;    // keys per LDS tile

template <int D>
__global__ __launch_bounds__(kRows) void attn_f32_kernel(const float* __restrict__ Q,
                                                         const float* __restrict__ K,
                                                         const float* __restrict__ V,
                                                         float* __restrict__ O,
                                                         float* __restrict__ LSE, int Nq, int Nkv,
                                                         int n_qtiles, float c) {
  __shared__ float Ks[kTK][D];
  __shared__ float Vs[kTK][D];
  const int bh = blockIdx.x / n_qtiles;
  const int qt = blockIdx.x - bh * n_qtiles;
  const int tid = threadIdx.x;
  const int qi = qt * kRows + tid;
  const float* Kb = K + (int64_t)bh * Nkv * D;
  const float* Vb = V + (int64_t)bh * Nkv * D;

  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qi < Nq ? Q[((int64_t)bh * Nq + qi) * D + d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int k0 = 0; k0 < Nkv; k0 += kTK) {
    __syncthreads();
    for (int e = tid; e < kTK * D; e += kRows) {
      const int j = e / D, d = e - j * D;
      const bool in = k0 + j < Nkv;
      Ks[j][d] = in ? Kb[(int64_t)(k0 + j) * D + d] : 0.f;
      Vs[j][d] = in ? Vb[(int64_t)(k0 + j) * D + d] : 0.f;
    }
    __syncthreads();
    float s[kTK];
    float mt = m;
#pragma unroll
    for (int j = 0; j < kTK; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(q[d], Ks[j][d], acc);
      s[j] = (k0 + j < Nkv) ? acc : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float alpha = __builtin_amdgcn_exp2f((m - mt) * c);  // m = -inf on the first tile -> 0
    m = mt;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < kTK; ++j) {
      const float p = __builtin_amdgcn_exp2f((s[j] - m) * c);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, Vs[j][d], o[d]);
    }
  }
  if (qi < Nq) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) O[((int64_t)bh * Nq + qi) * D + d] = o[d] * inv;
    if (LSE) LSE[(int64_t)bh * Nq + qi] = (m * c + __builtin_amdgcn_logf(l)) * 0.6931471805599453f;
  }
}

template <int D>
hipError_t launch_d(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                    int H, int Nq, int Nkv, float c, hipStream_t stream) {
  const int n_qtiles = (Nq + kRows - 1) / kRows;
  const int64_t grid = (int64_t)B * H * n_qtiles;
  hipLaunchKernelGGL(attn_f32_kernel<D>, dim3((unsigned)grid), dim3(kRows), 0, stream, q, k, v, o,
                     lse, Nq, Nkv, n_qtiles, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                           int B, int H, int Nq, int Nkv, int D, float scale,
                           hipStream_t stream) {
  const float c = scale * 1.4426950408889634f;  // softmax in base 2: exp(x*scale) = 2^(x*c)
  switch (D) {
    case 32: return launch_d<32>(q, k, v, o, lse, B, H, Nq, Nkv, c, stream);
    case 64: return launch_d<64>(q, k, v, o, lse, B, H, Nq, Nkv, c, stream);
    default: return launch_d<128>(q, k, v, o, lse, B, H, Nq, Nkv, c, stream);
  }
}

}  // namespace ditattn
