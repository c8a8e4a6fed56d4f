// Ulysses seq<->head exchange as it lands on one device: a batched copy of
// contiguous runs ("Multi-GPU parallelism: spreading one step over several
// cards", section "Sequence parallelism: Ulysses and Ring", the
// all_to_all_heads / all_to_all_tokens of the four-card simulation).
//
// Both layouts are rank-stacked, so every (rank r, rank s, b, head h' of the
// group) pair moves one contiguous run of Ns*D elements (Ns = N/P):
//   seq->head  dst chunk c = ((r*B + b)*g + h')*P + s   (dst is contiguous in c)
//              src chunk   = (s*B + b)*H + r*g + h'
//   head->seq  dst chunk c = (s*B + b)*H + r*g + h'
//              src chunk   = ((r*B + b)*g + h')*P + s
// with g = H/P.  Pure data movement: bit-exact for any element type.
#include "launch.h"

namespace ditattn {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

struct ChunkMap {
  int P, B, H, g;
  bool head2seq;
  __device__ int64_t src_chunk(int64_t c) const {
    if (!head2seq) {
      const int64_t s = c % P;
      int64_t t = c / P;
      const int64_t hh = t % g;
      t /= g;
      const int64_t b = t % B;
      const int64_t r = t / B;
      return (s * B + b) * H + r * g + hh;
    }
    const int64_t h = c % H;
    const int64_t t = c / H;
    const int64_t b = t % B;
    const int64_t s = t / B;
    const int64_t r = h / g, hh = h % g;
    return ((r * B + b) * g + hh) * P + s;
  }
};

// Each block copies kUnroll*kThreads vectors per step of its grid-stride loop
// inside one chunk; blockIdx.y walks the chunks.
template <typename VecT>
__global__ __launch_bounds__(kThreads) void permute_kernel(const VecT* __restrict__ in,
                                                           VecT* __restrict__ out, ChunkMap map,
                                                           int64_t nchunks, int64_t chunk_vecs) {
  for (int64_t c = blockIdx.y; c < nchunks; c += gridDim.y) {
    const VecT* src = in + map.src_chunk(c) * chunk_vecs;
    VecT* dst = out + c * chunk_vecs;
    const int64_t step = (int64_t)gridDim.x * kThreads * kUnroll;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll; base < chunk_vecs; base += step) {
      VecT v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + u * kThreads + threadIdx.x;
        if (i < chunk_vecs) v[u] = __builtin_nontemporal_load(src + i);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = base + u * kThreads + threadIdx.x;
        if (i < chunk_vecs) __builtin_nontemporal_store(v[u], dst + i);
      }
    }
  }
}

template <typename VecT>
hipError_t launch_typed(const void* in, void* out, ChunkMap map, int64_t nchunks,
                        int64_t chunk_vecs, hipStream_t stream) {
  const int64_t per_block = (int64_t)kThreads * kUnroll;
  int64_t gx = (chunk_vecs + per_block - 1) / per_block;
  if (gx > 4096) gx = 4096;
  int64_t gy = nchunks < 65535 ? nchunks : 65535;
  hipLaunchKernelGGL(permute_kernel<VecT>, dim3((unsigned)gx, (unsigned)gy), dim3(kThreads), 0,
                     stream, static_cast<const VecT*>(in), static_cast<VecT*>(out), map, nchunks,
                     chunk_vecs);
  return hipGetLastError();
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

}  // namespace

hipError_t launch_permute(const void* in, void* out, int P, int B, int H, int N, int D,
                          int elem_bytes, bool head2seq, hipStream_t stream) {
  ChunkMap map{P, B, H, H / P, head2seq};
  const int64_t nchunks = (int64_t)P * B * H;
  const int64_t chunk_bytes = (int64_t)(N / P) * D * elem_bytes;
  const uintptr_t a = reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out);
  if (chunk_bytes % 16 == 0 && a % 16 == 0)
    return launch_typed<u32x4>(in, out, map, nchunks, chunk_bytes / 16, stream);
  if (chunk_bytes % 8 == 0 && a % 8 == 0)
    return launch_typed<unsigned long long>(in, out, map, nchunks, chunk_bytes / 8, stream);
  if (chunk_bytes % 4 == 0 && a % 4 == 0)
    return launch_typed<unsigned int>(in, out, map, nchunks, chunk_bytes / 4, stream);
  if (chunk_bytes % 2 == 0 && a % 2 == 0)
    return launch_typed<unsigned short>(in, out, map, nchunks, chunk_bytes / 2, stream);
  return launch_typed<unsigned char>(in, out, map, nchunks, chunk_bytes, stream);
}

}  // namespace ditattn
