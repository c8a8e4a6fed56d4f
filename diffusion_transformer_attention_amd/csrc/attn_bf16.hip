// bf16 non-causal attention with log-sum-exp on the CDNA4 matrix cores.
//
// What is computed ("Multi-GPU parallelism: spreading one step over several
// cards", section "Sequence parallelism: Ulysses and Ring": each rank runs
// full attention over all tokens of its heads, and the Ring paragraph's
// block-wise online softmax; the miles_diffusion USP pull request, "Ring
// kernel selection": the kernel returns the LSE):
//   O[i]   = sum_j exp(s_ij - m_i) v_j / l_i,   s_ij = scale * q_i . k_j
//   LSE[i] = m_i + ln l_i
// with the running max m and running sum l updated block by block.
//
// Work decomposition (gfx950, wave64, one workgroup of 4 waves per CU):
//  * a workgroup owns 256 query rows of one (b, h); each wave owns 64 of
//    them as two 32-row blocks, so every K or V fragment read from LDS feeds
//    two MFMAs;
//  * keys are staged in 64-key LDS tiles (3 stages each for K and V, each a
//    separate LDS array so the compiler can tell a stage being loaded from
//    the stages being read) with global_load_lds_dwordx4, which writes LDS
//    without staging registers;
//    the 16-byte chunks of each row are XOR-swizzled so that the K reads
//    (ds_read_b128, 32 rows at one column) and the V reads
//    (ds_read_b64_tr_b16, 4 rows x 32 bytes per 16 lanes) hit distinct banks;
//  * contractions are v_mfma_f32_32x32x16_bf16 on transposed products:
//      S^T (keys x queries) = K . Q^T      A = K (LDS), B = Q^T (registers)
//      O^T (chans x queries) += V^T . P^T  A = V^T (LDS transposing read),
//                                          B = P^T (registers)
//    so each lane holds one query column of S^T and O^T: softmax statistics
//    are per-lane scalars and the S^T accumulator becomes the P^T operand in
//    registers;
//  * the key loop runs in 32-key slots, software-pipelined: slot s issues
//    the QK^T MFMAs of step s+1 and the PV MFMAs of step s-1 while the
//    vector ALUs do the softmax of step s; the three are independent and
//    share one basic block, and scheduling hints interleave the MFMAs with
//    the softmax instructions and the LDS reads;
//  * softmax in base 2: p = 2^(s*c - m*c) with c = scale*log2(e).  Two row
//    sums: lb of the bf16-rounded p that the PV product multiplies (via
//    v_dot2_f32_bf16), which normalises O, so O stays an exact convex
//    combination of the V rows whatever the rounding of its dominant
//    weight; and l of the float32 p, which gives the LSE (the rounded sum
//    would carry 2^-9 errors into rows dominated by a few keys);
//  * fixed reference max: each row's max m is taken from its first 32-key
//    step (while O is still zero) and then held.  O and l accumulate
//    p = 2^(s*c - m*c) against that same m, so O/l and m*c + log2(l) are
//    exact whatever m is, and O is never rescaled in the loop.  p stays below
//    2^64 unless a later score exceeds m by more than 64 (base 2); a row
//    that does sets a flag, and the workgroup then recomputes its tile in
//    two passes: the exact row max first, then the same loop with that max
//    (p <= 1).  Typical inputs never take that path;
//  * keys >= Nkv load a clamped in-range row and score -inf; the last,
//    partial key tile is peeled out of the loop; query rows >= Nq load a
//    clamped row and are not stored;
//  * workgroup ids are remapped so the query tiles of a head run on one XCD
//    and share its L2 while they stream the same K/V.
#include <math.h>

#include "launch.h"

namespace ditattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;              // two waves per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kQB = 1;                 // 32-row query blocks per wave
constexpr int kBM = 32 * kQB * kWaves; // query rows per workgroup
constexpr int kBN = 64;                // keys per LDS tile (two 32-key steps)
constexpr int kStages = 3;             // LDS stages for K and for V (tile t uses stage t % 3)
constexpr float kHeadroom = 64.0f;     // largest score excess over m (base 2) the loop accepts

template <int D>
struct Geo {
  static constexpr int KS = D / 16;            // k-steps of Q.K^T
  static constexpr int DB = D / 32;            // 32-channel blocks of O^T
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int ROWB = D * 2;           // bytes per row
  static constexpr int TILE = kBN * ROWB;      // bytes per K or V tile
  static constexpr int PIECES = TILE / 1024;  // 1 KB pieces per tile (one load instruction each)
};

// Chunk swizzles (chunk index XOR f(row)).  K: the 16 rows read together
// by ds_read_b128 land in 16 distinct 16-byte bank slots.  V: the 4 rows x
// 4 chunks read by 32 lanes of ds_read_b64_tr_b16 land in 16 distinct slots.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  constexpr int CPR = D / 8, RPL = 16 / CPR;
  return (row / RPL) & (CPR - 1);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  constexpr int CPR = D / 8;
  return (4 * (row & 3)) & (CPR - 1);
}

// Workgroups are dispatched round-robin over the 8 XCDs (id i -> XCD i % 8).
// Hand each XCD a contiguous range of tiles (a bijection on [0, total)).
__device__ __forceinline__ int remap_xcd(int i, int total) {
  const int x = i & 7, j = i >> 3;
  const int q = total >> 3, r = total & 7;
  return x * q + (x < r ? x : r) + j;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max (or sum) of x over lanes l and l^32.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS pointers are 32-bit address-space-3 pointers throughout.
typedef __attribute__((address_space(3))) char lds_t;
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// global_load_lds writes LDS asynchronously and is counted by vmcnt: each
// wave waits for its own loads (s_waitcnt vmcnt(0); gfx9 encoding: vmcnt
// bits [3:0] and [15:14] zero, expcnt 7 and lgkmcnt 15 = no wait) before the
// barrier that publishes the tile to the other waves.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
}

// Stage one 64-key tile of K (or V) into LDS: the wave's LOADS instructions
// each write 1 KB contiguously (lane i -> bytes [16i, 16i+16)); the global
// source of each lane is the chunk whose swizzled position that is.
template <int D, bool IS_V>
__device__ __forceinline__ void stage_tile(const __bf16* __restrict__ G, int k0, int Nkv,
                                           lds_t* buf, int wave, int lane) {
  using Gm = Geo<D>;
#pragma unroll
  for (int n = 0; n < (Gm::PIECES + kWaves - 1) / kWaves; ++n) {
    const int inst = n * kWaves + wave;
    if (Gm::PIECES % kWaves != 0 && inst >= Gm::PIECES) break;
    const int p = inst * 64 + lane;
    const int row = p / Gm::CPR, pc = p % Gm::CPR;
    const int lc = pc ^ (IS_V ? swz_v<D>(row) : swz_k<D>(row));
    const int key = min(k0 + row, Nkv - 1);
    __builtin_amdgcn_global_load_lds(G + (int64_t)key * D + lc * 8, LDS_PTR(buf + inst * 1024), 16,
                                     0, 0);
  }
}

template <int D>
struct Frags {
  f32x16 o[kQB][Geo<D>::DB];
  bf16x8 q[kQB][Geo<D>::KS];
  float m[kQB], l[kQB], lb[kQB];
};

// S^T for one 32-key step: keys rows [sub*32, sub*32+32) of the K stage.
template <int D>
__device__ __forceinline__ void qk_step(f32x16 (&S)[kQB], const lds_t* kst, const int (&koff)[Geo<D>::KS],
                                        const bf16x8 (&q)[kQB][Geo<D>::KS]) {
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) S[qb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < Geo<D>::KS; ++ks) {
    const bf16x8 a = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kst + koff[ks]);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) S[qb] = mfma32(a, q[qb][ks], S[qb]);
  }
}

// Softmax of one 32-key step against the row's reference max.  A row with
// no reference yet (m = -inf, so O and l are still zero) takes this step's
// max.  A row whose scores exceed its reference by more than kHeadroom
// raises `flag`: its O can no longer be kept without rescaling.
// key0: index of the step's first key; keys >= Nkv are masked when MASK.
// S is only read (copied into registers first).
template <int D, bool MASK>
__device__ __forceinline__ void softmax_step(const f32x16 (&S)[kQB], bf16x8 (&P)[kQB][2],
                                             Frags<D>& f, float c, int key0, int Nkv, int half,
                                             bool& flag) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    float s[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = S[qb][r];
    if (MASK) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[r] = (key0 + 8 * (r >> 2) + 4 * half + (r & 3) < Nkv) ? s[r] : -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = pair_max(mx);
    const float m_old = f.m[qb];
    const bool over = (mx - m_old) * c > kHeadroom;   // true when m_old = -inf
    flag |= over && (m_old != -INFINITY);
    const float m_use = over ? mx : m_old;
    f.m[qb] = m_use;
    float l = f.l[qb], lb = f.lb[qb];
    const float mc = m_use * c;
#pragma unroll
    for (int hc = 0; hc < 2; ++hc) {
      bf16x8 pv;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * hc + j], c, -mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * hc + j + 1], c, -mc));
        const bf16x2 pk = {(__bf16)p0, (__bf16)p1};
        l += p0 + p1;
        lb = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, lb, false);
        pv[j] = pk[0];
        pv[j + 1] = pk[1];
      }
      P[qb][hc] = pv;
    }
    f.l[qb] = l;
    f.lb[qb] = lb;
  }
}

// Row max of one 32-key step (exact-max pass).
template <bool MASK>
__device__ __forceinline__ void rowmax_step(const f32x16 (&S)[kQB], float (&m)[kQB], int key0,
                                            int Nkv, int half) {
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float v = S[qb][r];
      mx = fmaxf(mx, (!MASK || key0 + 8 * (r >> 2) + 4 * half + (r & 3) < Nkv) ? v : -INFINITY);
    }
    m[qb] = fmaxf(m[qb], pair_max(mx));
  }
}

// O^T += V^T P^T for one 32-key step: value rows [sub*32, sub*32+32) of the V stage.
// MFMA k index 8*half + j <-> key 16*hc + 8*(j/4) + 4*half + (j%4) of the step.
template <int D>
__device__ __forceinline__ void pv_step(Frags<D>& f, const bf16x8 (&P)[kQB][2], const lds_t* vst,
                                        const int (&voff)[Geo<D>::DB]) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int hc = 0; hc < 2; ++hc)
#pragma unroll
    for (int db = 0; db < Geo<D>::DB; ++db) {
      const lds_t* base = vst + voff[db] + 16 * hc * Geo<D>::ROWB;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(base));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(base + 8 * Geo<D>::ROWB));
      const bf16x4 blo = __builtin_bit_cast(bf16x4, lo), bhi = __builtin_bit_cast(bf16x4, hi);
      const bf16x8 a = {blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) f.o[qb][db] = mfma32(a, P[qb][hc], f.o[qb][db]);
    }
}

// Everything one pass over the keys needs.
template <int D>
struct PassCtx {
  const __bf16* Kb;
  const __bf16* Vb;
  lds_t *k0, *k1, *k2;  // K stages (separate scalars: never an indexed array)
  lds_t *v0, *v1, *v2;  // V stages
  int Nkv, ntiles, wave, lane, half;
  float c;
  int koff[Geo<D>::KS];
  int voff[Geo<D>::DB];
};

// Stage of tile t: PH = t % 3 when known at compile time, else -1.
__device__ __forceinline__ lds_t* stage_of(lds_t* s0, lds_t* s1, lds_t* s2, int PH, int t) {
  const int i = PH >= 0 ? PH % kStages : t % kStages;
  return i == 0 ? s0 : (i == 1 ? s1 : s2);
}
#define KSTAGE(x, PH, t) stage_of((x).k0, (x).k1, (x).k2, (PH), (t))
#define VSTAGE(x, PH, t) stage_of((x).v0, (x).v1, (x).v2, (PH), (t))

// Ask the scheduler to interleave one slot's 32 MFMAs with its LDS reads and
// its softmax VALU work (groups are filled in order; empty ones are skipped).
__device__ __forceinline__ void interleave_slot() {
#pragma unroll
  for (int i = 0; i < 16 * kQB; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // five VALU
  }
}

// One 32-key slot: QK^T of the next step into Sn, PV of the previous step
// from Pp, softmax of this step from Sc into Pc.
template <int D, bool MASK>
__device__ __forceinline__ void slot(Frags<D>& f, const f32x16 (&Sc)[kQB], f32x16 (&Sn)[kQB],
                                     const bf16x8 (&Pp)[kQB][2], bf16x8 (&Pc)[kQB][2],
                                     const lds_t* k_next, const lds_t* v_prev,
                                     const PassCtx<D>& x, int key0, bool& flag) {
  qk_step<D>(Sn, k_next, x.koff, f.q);
  pv_step<D>(f, Pp, v_prev, x.voff);
  softmax_step<D, MASK>(Sc, Pc, f, x.c, key0, x.Nkv, x.half, flag);
  interleave_slot();
}

// One 64-key tile t = slots 2t and 2t+1.  PH = t % 3 when known at compile
// time (the unrolled main loop: every LDS stage is then a distinct array and
// the loads into stage t+2 overlap the reads of the others), or -1.
// On entry S0 holds S^T of step 2t and Pa holds P of step 2t-1; on exit S0
// holds S^T of step 2t+2 (garbage past the last tile, never used) and Pa
// holds P of step 2t+1.
template <int D, int PH, bool MASK>
__device__ __forceinline__ void tile_trip(int t, Frags<D>& f, f32x16 (&S0)[kQB], f32x16 (&S1)[kQB],
                                          bf16x8 (&Pa)[kQB][2], bf16x8 (&Pb)[kQB][2],
                                          const PassCtx<D>& x, bool& flag) {
  using Gm = Geo<D>;
  tile_barrier();  // K_{t+1}, V_t landed; every wave is done with tile t-1
  const int p2 = PH >= 0 ? PH + 2 : -1, p1 = PH >= 0 ? PH + 1 : -1;
  if (t + 2 < x.ntiles)
    stage_tile<D, false>(x.Kb, (t + 2) * kBN, x.Nkv, KSTAGE(x, p2, t + 2), x.wave, x.lane);
  if (t + 1 < x.ntiles)
    stage_tile<D, true>(x.Vb, (t + 1) * kBN, x.Nkv, VSTAGE(x, p1, t + 1), x.wave, x.lane);
  const lds_t* kcur = KSTAGE(x, PH, t);
  const lds_t* knext = KSTAGE(x, p1, t + 1);
  const lds_t* vcur = VSTAGE(x, PH, t);
  const lds_t* vprev = VSTAGE(x, p2, t + 2);  // stage of tile t-1
  const int key0 = t * kBN;
  slot<D, MASK>(f, S0, S1, Pa, Pb, kcur + 32 * Gm::ROWB, vprev + 32 * Gm::ROWB, x, key0, flag);
  slot<D, MASK>(f, S1, S0, Pb, Pa, knext, vcur, x, key0 + 32, flag);
}

// One full pass over the keys: stage, the unmasked tiles (unrolled by the
// stage count), the partial last tile (if any) with masking, then the PV of
// the last step.
template <int D>
__device__ __forceinline__ void run_pass(Frags<D>& f, const PassCtx<D>& x, bool& flag) {
  using Gm = Geo<D>;
  // The first slot multiplies P = 0 by the V stage of tile -1 (stage 2): zero
  // it so no stale Inf/NaN bit pattern can turn 0 * V into NaN.
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  for (int i = threadIdx.x; i < Gm::TILE / 16; i += kThreads)
    reinterpret_cast<__attribute__((address_space(3))) u32x4*>(x.v2)[i] = u32x4{0u, 0u, 0u, 0u};
  stage_tile<D, false>(x.Kb, 0, x.Nkv, x.k0, x.wave, x.lane);
  if (x.ntiles > 1) stage_tile<D, false>(x.Kb, kBN, x.Nkv, x.k1, x.wave, x.lane);
  stage_tile<D, true>(x.Vb, 0, x.Nkv, x.v0, x.wave, x.lane);
  f32x16 S0[kQB], S1[kQB];
  bf16x8 Pa[kQB][2], Pb[kQB][2];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) Pa[qb][0] = Pa[qb][1] = bf16x8{};
  tile_barrier();  // K tile 0 (and K 1, V 0) landed
  qk_step<D>(S0, x.k0, x.koff, f.q);
  const bool partial = (x.Nkv % kBN) != 0;
  const int nfull = partial ? x.ntiles - 1 : x.ntiles;
  int t = 0;
  for (; t + kStages <= nfull; t += kStages) {
    tile_trip<D, 0, false>(t, f, S0, S1, Pa, Pb, x, flag);
    tile_trip<D, 1, false>(t + 1, f, S0, S1, Pa, Pb, x, flag);
    tile_trip<D, 2, false>(t + 2, f, S0, S1, Pa, Pb, x, flag);
  }
  for (; t < nfull; ++t) tile_trip<D, -1, false>(t, f, S0, S1, Pa, Pb, x, flag);
  if (partial) tile_trip<D, -1, true>(t, f, S0, S1, Pa, Pb, x, flag);
  pv_step<D>(f, Pa, VSTAGE(x, -1, x.ntiles - 1) + 32 * Gm::ROWB, x.voff);
}

// Exact row max over all keys (only when the fixed-reference loop flagged).
template <int D>
__device__ __forceinline__ void exact_max_pass(Frags<D>& f, const PassCtx<D>& x) {
  using Gm = Geo<D>;
  float m[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) m[qb] = -INFINITY;
  for (int t = 0; t < x.ntiles; ++t) {
    __syncthreads();  // every wave is done reading the stage
    stage_tile<D, false>(x.Kb, t * kBN, x.Nkv, x.k0, x.wave, x.lane);
    tile_barrier();  // landed
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 S[kQB];
      qk_step<D>(S, x.k0 + sub * 32 * Gm::ROWB, x.koff, f.q);
      if (t * kBN + kBN > x.Nkv)
        rowmax_step<true>(S, m, t * kBN + sub * 32, x.Nkv, x.half);
      else
        rowmax_step<false>(S, m, t * kBN + sub * 32, x.Nkv, x.half);
    }
  }
  __syncthreads();
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) f.m[qb] = m[qb];
}

template <int D, bool OUT_F32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void attn_fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                          const __bf16* __restrict__ V, void* __restrict__ Oout,
                          float* __restrict__ LSE, int Nq, int Nkv, int n_qtiles, int total_tiles,
                          float c) {
  using Gm = Geo<D>;
  __shared__ __attribute__((aligned(1024))) char k0s[Gm::TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[Gm::TILE];
  __shared__ __attribute__((aligned(1024))) char k2s[Gm::TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[Gm::TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[Gm::TILE];
  __shared__ __attribute__((aligned(1024))) char v2s[Gm::TILE];

  const int tile = remap_xcd(blockIdx.x, total_tiles);
  const int bh = tile / n_qtiles;
  const int qt = tile - bh * n_qtiles;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, half = lane >> 5;

  const __bf16* Qb = Q + (int64_t)bh * Nq * D;
  PassCtx<D> x;
  x.Kb = K + (int64_t)bh * Nkv * D;
  x.Vb = V + (int64_t)bh * Nkv * D;
  x.k0 = (lds_t*)k0s; x.k1 = (lds_t*)k1s; x.k2 = (lds_t*)k2s;
  x.v0 = (lds_t*)v0s; x.v1 = (lds_t*)v1s; x.v2 = (lds_t*)v2s;
  x.Nkv = Nkv;
  x.ntiles = (Nkv + kBN - 1) / kBN;
  x.wave = wave;
  x.lane = lane;
  x.half = half;
  x.c = c;

  // Per-lane LDS byte offsets (independent of the step).
#pragma unroll
  for (int ks = 0; ks < Gm::KS; ++ks)
    x.koff[ks] = col * Gm::ROWB + (((2 * ks + half) ^ swz_k<D>(col)) << 4);
  {
    const int g = lane >> 4, t = lane & 15;
    const int row = 4 * (g >> 1) + (t >> 2);
#pragma unroll
    for (int db = 0; db < Gm::DB; ++db) {
      const int ce = db * 32 + 16 * (g & 1) + 4 * (t & 3);
      x.voff[db] = row * Gm::ROWB + (((ce >> 3) ^ swz_v<D>(row)) << 4) + (ce & 7) * 2;
    }
  }

  Frags<D> f;
  const int qrow0 = qt * kBM + wave * (32 * kQB) + col;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int row = min(qrow0 + 32 * qb, Nq - 1);
#pragma unroll
    for (int ks = 0; ks < Gm::KS; ++ks)
      f.q[qb][ks] = *reinterpret_cast<const bf16x8*>(Qb + (int64_t)row * D + ks * 16 + half * 8);
    f.m[qb] = -INFINITY;
    f.l[qb] = 0.f;
    f.lb[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < Gm::DB; ++db) f.o[qb][db] = f32x16{};
  }

  // Second attempt only if some row's scores outgrew its reference max:
  // then redo the tile with the exact row max (all waves decide together).
  for (int attempt = 0;; ++attempt) {
    bool flag = false;
    run_pass<D>(f, x, flag);
    if (attempt == 1 || !__syncthreads_or(flag)) break;
    exact_max_pass<D>(f, x);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      f.l[qb] = 0.f;
      f.lb[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < Gm::DB; ++db) f.o[qb][db] = f32x16{};
    }
  }

  // Epilogue: O = O^T / lb, LSE = (m*c + log2 l) * ln 2.
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float l_tot = pair_sum(f.l[qb]);
    const float inv = 1.0f / pair_sum(f.lb[qb]);
    const int qrow = qrow0 + 32 * qb;
    if (qrow < Nq) {
      const int64_t obase = ((int64_t)bh * Nq + qrow) * D;
#pragma unroll
      for (int db = 0; db < Gm::DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = db * 32 + 8 * g + 4 * half;
          const f32x4 val = {f.o[qb][db][4 * g] * inv, f.o[qb][db][4 * g + 1] * inv,
                             f.o[qb][db][4 * g + 2] * inv, f.o[qb][db][4 * g + 3] * inv};
          if (OUT_F32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(Oout) + obase + d0) = val;
          } else {
            const bf16x4 b = {(__bf16)val[0], (__bf16)val[1], (__bf16)val[2], (__bf16)val[3]};
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(Oout) + obase + d0) = b;
          }
        }
      if (LSE && half == 0)
        LSE[(int64_t)bh * Nq + qrow] =
            (f.m[qb] * c + __builtin_amdgcn_logf(l_tot)) * 0.6931471805599453f;
    }
  }
}

template <int D, bool OUT_F32>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int Nq, int Nkv, float c, hipStream_t stream) {
  const int n_qtiles = (Nq + kBM - 1) / kBM;
  const int64_t total = (int64_t)B * H * n_qtiles;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, OUT_F32>), dim3((unsigned)total), dim3(kThreads), 0,
                     stream, static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), o, lse, Nq, Nkv, n_qtiles, (int)total, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Nq, int Nkv, int D, float scale, bool o_f32,
                            hipStream_t stream) {
  const float c = scale * 1.4426950408889634f;
  if (o_f32) {
    switch (D) {
      case 32: return launch_d<32, true>(q, k, v, o, lse, B, H, Nq, Nkv, c, stream);
      case 64: return launch_d<64, true>(q, k, v, o, lse, B, H, Nq, Nkv, c, stream);
      default: return launch_d<128, true>(q, k, v, o, lse, B, H, Nq, Nkv, c, stream);
    }
  }
  switch (D) {
    case 32: return launch_d<32, false>(q, k, v, o, lse, B, H, Nq, Nkv, c, stream);
    case 64: return launch_d<64, false>(q, k, v, o, lse, B, H, Nq, Nkv, c, stream);
    default: return launch_d<128, false>(q, k, v, o, lse, B, H, Nq, Nkv, c, stream);
  }
}

}  // namespace ditattn
