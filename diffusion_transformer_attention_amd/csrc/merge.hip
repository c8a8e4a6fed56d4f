// Exact log-sum-exp merge of attention partials over disjoint key blocks
// ("Multi-GPU parallelism: spreading one step over several cards", section
// "Sequence parallelism: Ulysses and Ring", Ring paragraph: each block's
// local attention is merged with a log-sum-exp).
//
//   M = max_i LSE_i,  LSE = M + ln sum_i exp(LSE_i - M),
//   O = sum_i exp(LSE_i - M) O_i / sum_i exp(LSE_i - M)
//
// HBM-bound: every partial is read once and the result written once.  One
// thread owns four consecutive channels (one 16-byte load per partial) of one
// row; the D/4 threads of a row read the same nblk LSE values from cache.  Up
// to eight partials are loaded before any arithmetic so their loads overlap.
#include <math.h>

#include "launch.h"

namespace ditattn {
namespace {

constexpr int kThreads = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// NB > 0: nblk == NB known at compile time, so every partial's load is issued
// before the arithmetic (NB loads in flight per thread); NB == 0: any nblk.
template <bool OUT_F32, int NB>
__global__ __launch_bounds__(kThreads) void merge_kernel(const float* __restrict__ o_parts,
                                                         const float* __restrict__ lse_parts,
                                                         int nblk, void* __restrict__ o,
                                                         float* __restrict__ lse, int64_t rows,
                                                         int log2_tpr, int D) {
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kLn2 = 0.6931471805599453f;
  const int n = NB > 0 ? NB : nblk;
  const int64_t total = rows << log2_tpr;
  for (int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x; gid < total;
       gid += (int64_t)gridDim.x * kThreads) {
    const int64_t row = gid >> log2_tpr;
    const int c4 = (int)(gid & ((1 << log2_tpr) - 1)) * 4;
    float M = -INFINITY;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float tot = 0.f;
    if (NB > 0) {
      float li[NB > 0 ? NB : 1];
      f32x4 x[NB > 0 ? NB : 1];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        li[i] = lse_parts[(int64_t)i * rows + row];
        x[i] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(o_parts + ((int64_t)i * rows + row) * D + c4));
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) M = fmaxf(M, li[i]);
      if (M != -INFINITY) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const float w = __builtin_amdgcn_exp2f((li[i] - M) * kLog2e);  // li = -inf -> 0
          tot += w;
          acc += w * x[i];
        }
        acc *= 1.0f / tot;
      }
    } else {
      for (int i = 0; i < n; ++i) M = fmaxf(M, lse_parts[(int64_t)i * rows + row]);
      if (M != -INFINITY) {
        for (int i = 0; i < n; ++i) {
          const float li = lse_parts[(int64_t)i * rows + row];
          const float w = __builtin_amdgcn_exp2f((li - M) * kLog2e);
          const f32x4 x = __builtin_nontemporal_load(
              reinterpret_cast<const f32x4*>(o_parts + ((int64_t)i * rows + row) * D + c4));
          tot += w;
          acc += w * x;
        }
        acc *= 1.0f / tot;
      }
    }
    const int64_t off = row * D + c4;
    if (OUT_F32) {
      __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(static_cast<float*>(o) + off));
    } else {
      bf16x4 b = {(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
      // streaming store, as for float32 O (531 -> 485 us for 4 partials of
      // [1,40,32768,128] into bf16, bit-identical)
      __builtin_nontemporal_store(__builtin_bit_cast(unsigned long long, b),
                                  reinterpret_cast<unsigned long long*>(static_cast<__bf16*>(o) + off));
    }
    if (lse && c4 == 0)
      lse[row] = (M == -INFINITY) ? -INFINITY : M + __builtin_amdgcn_logf(tot) * kLn2;
  }
}

template <bool OUT_F32, int NB>
void launch_nb(dim3 grid, hipStream_t stream, const float* o_parts, const float* lse_parts,
               int nblk, void* o, float* lse, int64_t rows, int log2_tpr, int D) {
  hipLaunchKernelGGL((merge_kernel<OUT_F32, NB>), grid, dim3(kThreads), 0, stream, o_parts,
                     lse_parts, nblk, o, lse, rows, log2_tpr, D);
}

template <bool OUT_F32>
void launch_any(dim3 grid, hipStream_t stream, const float* o_parts, const float* lse_parts,
                int nblk, void* o, float* lse, int64_t rows, int log2_tpr, int D) {
  switch (nblk) {
    case 1: return launch_nb<OUT_F32, 1>(grid, stream, o_parts, lse_parts, nblk, o, lse, rows, log2_tpr, D);
    case 2: return launch_nb<OUT_F32, 2>(grid, stream, o_parts, lse_parts, nblk, o, lse, rows, log2_tpr, D);
    case 3: return launch_nb<OUT_F32, 3>(grid, stream, o_parts, lse_parts, nblk, o, lse, rows, log2_tpr, D);
    case 4: return launch_nb<OUT_F32, 4>(grid, stream, o_parts, lse_parts, nblk, o, lse, rows, log2_tpr, D);
    case 5: return launch_nb<OUT_F32, 5>(grid, stream, o_parts, lse_parts, nblk, o, lse, rows, log2_tpr, D);
    case 6: return launch_nb<OUT_F32, 6>(grid, stream, o_parts, lse_parts, nblk, o, lse, rows, log2_tpr, D);
    case 7: return launch_nb<OUT_F32, 7>(grid, stream, o_parts, lse_parts, nblk, o, lse, rows, log2_tpr, D);
    case 8: return launch_nb<OUT_F32, 8>(grid, stream, o_parts, lse_parts, nblk, o, lse, rows, log2_tpr, D);
    default: return launch_nb<OUT_F32, 0>(grid, stream, o_parts, lse_parts, nblk, o, lse, rows, log2_tpr, D);
  }
}

}  // namespace

hipError_t launch_merge(const float* o_parts, const float* lse_parts, int nblk, void* o,
                        float* lse, int64_t rows, int D, bool o_f32, hipStream_t stream) {
  const int tpr = D / 4;  // D in {32, 64, 128}: a power of two
  int log2_tpr = 0;
  while ((1 << log2_tpr) < tpr) ++log2_tpr;
  const int64_t threads = rows * tpr;
  int64_t blocks = (threads + kThreads - 1) / kThreads;
  if (blocks > (1 << 20)) blocks = 1 << 20;
  const dim3 grid((unsigned)blocks);
  if (o_f32)
    launch_any<true>(grid, stream, o_parts, lse_parts, nblk, o, lse, rows, log2_tpr, D);
  else
    launch_any<false>(grid, stream, o_parts, lse_parts, nblk, o, lse, rows, log2_tpr, D);
  return hipGetLastError();
}

}  // namespace ditattn
