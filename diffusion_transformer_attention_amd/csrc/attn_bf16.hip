// bf16 non-causal attention with log-sum-exp on the CDNA4 matrix cores.
//
// What is computed ("Multi-GPU parallelism: spreading one step over several
// cards", section "Sequence parallelism: Ulysses and Ring": each rank runs
// full attention over all tokens of its heads, and the Ring paragraph's
// block-wise softmax; the miles_diffusion USP pull request, "Ring kernel
// selection": the kernel returns the LSE):
//   O[i]   = sum_j exp(s_ij - m_i) v_j / l_i,   s_ij = scale * q_i . k_j
//   LSE[i] = m_i + ln l_i
//
// Work decomposition (gfx950, wave64):
//  * a workgroup of 8 waves (two per SIMD, so one wave's softmax overlaps
//    the other's MFMAs) owns 256 query rows of one (b, h); each wave owns
//    32 rows as two 16-row blocks;
//  * keys are staged in 64-key LDS tiles (3 stages each for K and V, each a
//    separate LDS array so the compiler can tell the stage being loaded from
//    the stages being read) with buffer_load_dwordx4 ... lds, which writes
//    LDS without staging registers; the buffer descriptor is rebased per
//    tile in scalar registers, so each lane's offset is loop-invariant and
//    rows past Nkv are out of range and arrive as zeros; the 16-byte chunks
//    of each row are XOR-swizzled so the K reads (ds_read_b128, 16 rows at
//    one column) and the V reads (ds_read_b64_tr_b16, 8 rows x 32 bytes per
//    32 lanes) hit distinct banks;
//  * contractions are v_mfma_f32_16x16x32_bf16 on transposed products:
//      S^T (keys x queries) = K . Q^T      A = K (LDS), B = Q^T (registers)
//      O^T (chans x queries) += V^T . P^T  A = V^T (LDS transposing read),
//                                          B = P^T (registers)
//    so each lane holds one query column and four consecutive keys or
//    channels of a 16x16 block: the softmax works per lane, the S^T
//    accumulator becomes the P^T operand in registers, and a 32x32 score
//    tile is four independent accumulators (short MFMA dependency chains);
//  * the key loop runs in 32-key slots, software-pipelined: slot s issues
//    the QK^T MFMAs of step s+1 and the PV MFMAs of step s-1 while the
//    vector ALUs do the softmax of step s; the slot is laid out as groups
//    fenced by scheduling barriers, each issuing LDS reads ahead of their
//    MFMAs, one QK^T and one PV MFMA and a share of the softmax;
//  * softmax in base 2: p = 2^(s*c - m*c) with c = scale*log2(e).  Two row
//    sums: lb of the bf16-rounded p that the PV product multiplies
//    normalises O, so O stays an exact convex combination of the V rows
//    whatever the rounding of its dominant weight; it comes from the matrix
//    cores (one more PV MFMA per query block, with an all-ones V^T block),
//    which frees the vector ALUs that bound the loop.  l of the float32 p
//    gives the LSE (the rounded sum would carry errors of up to 2^-8 into
//    rows dominated by a few keys);
//  * fixed reference max: each row's reference m is the max of its first
//    32-key step and is then held.  O and l accumulate p against that same m,
//    so O/l and m*c + log2(l) are exact whatever m is, and the loop never
//    rescales O nor tracks a running max.  Because l >= every p, a pass that
//    ends with l < 2^40 (and finite) never held a p >= 2^40 and never
//    overflowed; a row that ends above raises a flag and the workgroup
//    recomputes its tile in two passes: the exact row max first, then the
//    same loop with that max (p <= 1).  Typical inputs never take that path;
//  * keys >= Nkv arrive as zero rows and score -inf; the last, partial key
//    tile is peeled out of the loop; query rows >= Nq load a clamped row and
//    are not stored;
//  * workgroup ids are remapped so the query tiles of a head run on one XCD
//    and share its L2 while they stream the same K/V.
#include <math.h>

#include <atomic>

#include "launch.h"
#include "rope.h"

namespace ditattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// LDS pointers are 32-bit address-space-3 pointers throughout.
typedef __attribute__((address_space(3))) char lds_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) const u32x4 lds_cu32x4;
typedef __attribute__((address_space(3))) int lds_i32;

constexpr int kWaves = 8;               // two waves per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kQB = 2;                  // 16-row query blocks per wave (1: half-height tiles)
constexpr int kBM = 16 * kQB * kWaves;  // query rows per workgroup
constexpr int kBN = 64;                 // keys per LDS tile (two 32-key slots)
static_assert(kBM == kFwdQueryTile && kBN == kFwdKeyTile, "launch.h tile sizes");
constexpr int kStages = 3;              // LDS stages for K and for V (tile t uses stage t % 3)
constexpr float kMaxSum = 1099511627776.0f;  // 2^40: a larger row sum means the pass must be redone
constexpr float kMinSum = 1.0f / kMaxSum;     // fp8 mode 2 without a reference max: a smaller one too

template <int D>
struct Geo {
  static constexpr int KS = D / 32;        // 32-wide k-steps of Q.K^T
  static constexpr int DB = D / 16;        // 16-channel blocks of O^T
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int ROWB = D * 2;       // bytes per row
  static constexpr int TILE = kBN * ROWB;  // bytes per K or V tile
  static constexpr int PIECES = TILE / 1024;  // 1 KB pieces per tile (one load instruction each)
};

// Chunk swizzles (chunk index XOR f(row)).  K: the 16 rows read together by
// ds_read_b128 land in 16 distinct 16-byte bank slots.  V: the 8 rows x 2
// chunks read by 32 lanes of ds_read_b64_tr_b16 land in 16 distinct slots.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  constexpr int CPR = D / 8, RPL = 16 / CPR;
  return (row / RPL) & (CPR - 1);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  constexpr int CPR = D / 8;
  return (2 * (row & 7)) & (CPR - 1);
}

// The Q.K^T operands.  bf16: K rows of 2D bytes, fragments of 8 channels
// (v_mfma_f32_16x16x32_bf16, D/32 k-steps).  fp8 (OCP E4M3, D = 128 only):
// K rows of 128 bytes, one fragment of 32 channels per lane covering all of
// D in one v_mfma_f32_16x16x128_f8f6f4 (lane group g holds channels
// 32g .. 32g+31 of its key row in A and of its query column in B: the
// instruction pairs byte j of lane group g in A with the same byte of the
// same group in B, checked on gfx950).
template <int D, int F8>
struct QKOps;

template <int D>
struct QKOps<D, 0> {
  using Frag = bf16x8;
  static constexpr int KS = D / 32;       // k-steps (fragments per 16-key block)
  static constexpr int ROWB = D * 2;      // bytes per K row
  static constexpr int TILE = kBN * ROWB;
  static constexpr int PIECES = TILE / 1024;
  __device__ static int swz(int row) { return swz_k<D>(row); }
  // byte offset of fragment ks within a 16-row block: row c16, chunk 4ks + g
  __device__ static int frag_off(int c16, int g, int ks) {
    return c16 * ROWB + (((4 * ks + g) ^ swz(c16)) << 4);
  }
  __device__ static Frag load(const lds_t* blk, int off) {
    return *reinterpret_cast<const lds_bf16x8*>(blk + off);
  }
  __device__ static Frag load_q(const void* row, int g, int ks) {
    return *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(row) + ks * 32 + g * 8);
  }
  __device__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static f32x4 mma_s(Frag a, Frag b, f32x4 c, int, int) { return mma(a, b, c); }
};

template <int D>
struct QKOps<D, 1> {
  static_assert(D == 128, "fp8 Q.K^T is built for head dim 128");
  using Frag = i32x8;
  static constexpr int KS = 1;
  static constexpr int ROWB = D;
  static constexpr int TILE = kBN * ROWB;
  static constexpr int PIECES = TILE / 1024;
  // Chunk swizzle of the 128-byte rows: with it the fragment reads (16 rows
  // at one chunk per 16 lanes) meet no bank conflict.  Counted on gfx950 with
  // SQ_LDS_BANK_CONFLICT: (row >> 1) & 7, row & 7 and others cost 4 extra
  // cycles per ds_read_b128, this one none.
  __device__ static int swz(int row) { return 2 * (row & 3) + ((row >> 2) & 1); }
  // first 16 bytes of the lane's 32: row c16, chunk 2g; the second chunk
  // 2g + 1 sits at (offset ^ 16).
  __device__ static int frag_off(int c16, int g, int) { return c16 * ROWB + (((2 * g) ^ swz(c16)) << 4); }
  __device__ static Frag load(const lds_t* blk, int off) {
    const u32x4 lo = *reinterpret_cast<lds_cu32x4*>(blk + off);
    const u32x4 hi = *reinterpret_cast<lds_cu32x4*>(blk + (off ^ 16));
    return Frag{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                (int)hi[3]};
  }
  __device__ static Frag load_q(const void* row, int g, int) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(row) + 32 * g);
    const u32x4 lo = p[0], hi = p[1];
    return Frag{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                (int)hi[3]};
  }
  __device__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
  __device__ static f32x4 mma_s(Frag a, Frag b, f32x4 c, int, int) { return mma(a, b, c); }
};

// fp8 with power-of-two per-head scales (mode 2): the same operands, and the
// instruction multiplies the products by 2^(sa - 127) * 2^(sb - 127) (E8M0
// bytes sa for the keys, sb for the queries), so that with the softmax
// constant folded into the query codes the accumulator holds base-2 scores.
template <int D>
struct QKOps<D, 2> : QKOps<D, 1> {
  using Frag = typename QKOps<D, 1>::Frag;
  __device__ static f32x4 mma_s(Frag a, Frag b, f32x4 c, int sa, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
  }
};

// Workgroups are dispatched round-robin over the 8 XCDs (id i -> XCD i % 8).
// Hand each XCD a contiguous range of tiles (a bijection on [0, total)).
__device__ __forceinline__ int remap_xcd(int i, int total) {
  const int x = i & 7, j = i >> 3;
  const int q = total >> 3, r = total & 7;
  return x * q + (x < r ? x : r) + j;
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max / sum over the four lanes that hold the same query (l, l^16, l^32, l^48).
__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// Buffer loads into LDS complete asynchronously and are counted by vmcnt: each
// wave waits for its own loads (s_waitcnt vmcnt(0); gfx9 encoding: vmcnt
// bits [3:0] and [15:14] zero, expcnt 7 and lgkmcnt 15 = no wait) before the
// barrier that publishes the tile to the other waves.
// WAITN > 0: wait only until at most WAITN memory operations are left, for
// the first waits of a tile whose loads were issued before the previous
// tile's WAITN output stores (vmcnt retires in order, so the loads are then
// done and the stores may still be in flight).
template <int WAITN = 0>
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | (WAITN & 15) | ((WAITN >> 4) << 14));
  __syncthreads();
}

// A stream of 64-key tiles of K (or V) in key order.  The keys of one (b, h)
// lie in segments (a single segment for contiguous keys; one per Ulysses
// token shard otherwise, each of at least a tile), the end of one segment
// `jump` bytes before the start of the next.  p is the next tile's first row,
// left the rows from there to the end of its segment and rem the rows from
// there to the end of the stream: moving to the next tile is a few scalar
// operations, with no division to find the segment.
struct TileStream {
  const char* p;
  int left;
  int next;  // rows of each later segment
  int rem;
};

// Stage the stream's next tile into LDS and advance.  Each load instruction
// writes 1 KB contiguously (lane i -> bytes [16i, 16i+16)); voff[n] is the
// byte offset, within a tile, of the global chunk whose swizzled position
// that is (see piece_offsets; its row is voff[n] / ROWB).  The descriptor
// covers the tile's rows up to the end of its segment, so rows past the end
// of the stream read as zero (its 32-bit size is at most one tile).  A tile
// that runs past the end of its segment into the next one (shards whose
// length is not a multiple of the tile) takes its later rows from the next
// segment through per-lane offsets.  `straddle` is a
// compile-time constant after inlining (the pass context's str), false in
// every launch whose segments are whole tiles, so their code has no such
// branch.
template <int ROWB, int PIECES>
__device__ __forceinline__ void stage_next(TileStream& s, int64_t jump, lds_t* buf, int wave,
                                           const int* voff, bool straddle) {
  constexpr int kLogRowB = __builtin_ctz(ROWB);
  static_assert((1 << kLogRowB) == ROWB, "row bytes a power of two");
  const int take = min(s.left, kBN);  // rows from the current segment
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)s.p, (short)0, take * ROWB, 0x00020000);
  if (!straddle || take == kBN || s.rem <= take) {
#pragma unroll
    for (int n = 0; n < (PIECES + kWaves - 1) / kWaves; ++n) {
      const int inst = n * kWaves + wave;
      if (PIECES % kWaves != 0 && inst >= PIECES) break;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(buf + inst * 1024), 16, voff[n], 0, 0,
          0);
    }
  } else {
    // rows [take, min(kBN, rem)) from the next segment, which starts at
    // p + take*ROWB + jump: one descriptor based at p that reaches that far
    // (the launch keeps jump + a tile below 2^31 bytes), the lanes of those
    // rows adding jump to their offset; rows past the end of the stream fall
    // outside the record and read as zero
    const __amdgpu_buffer_rsrc_t rsrc2 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)s.p, (short)0, (int)jump + min(kBN, s.rem) * ROWB, 0x00020000);
#pragma unroll
    for (int n = 0; n < (PIECES + kWaves - 1) / kWaves; ++n) {
      const int inst = n * kWaves + wave;
      if (PIECES % kWaves != 0 && inst >= PIECES) break;
      const int off = voff[n] + ((voff[n] >> kLogRowB) >= take ? (int)jump : 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc2, (__attribute__((address_space(3))) void*)(buf + inst * 1024), 16, off, 0, 0, 0);
    }
  }
  s.p += kBN * ROWB;
  s.left -= kBN;
  if (straddle) {
    s.rem -= kBN;
    if (s.left <= 0) {  // past the end of a segment: into the next one
      s.p += jump;
      s.left += s.next;
    }
  } else if (s.left == 0) {  // end of a segment: on to the next one
    s.p += jump;
    s.left = s.next;
  }
}

// Per-lane source offsets of the wave's load pieces (loop-invariant).
template <int ROWB, int PIECES, typename Swz>
__device__ __forceinline__ void piece_offsets(int* voff, int wave, int lane, Swz swz) {
  constexpr int CPR = ROWB / 16;
#pragma unroll
  for (int n = 0; n < (PIECES + kWaves - 1) / kWaves; ++n) {
    const int p = (n * kWaves + wave) * 64 + lane;
    const int row = p / CPR, pc = p % CPR;
    voff[n] = row * ROWB + (pc ^ swz(row)) * 16;
  }
}

template <int D, int F8, int QB = kQB>
struct Frags {
  using QK = QKOps<D, F8>;
  f32x4 o[QB][Geo<D>::DB];           // O^T blocks: lane holds channels 16db+4g+r of its query
  typename QK::Frag q[QB][QK::KS];   // Q^T operand of the lane's query (bf16: channels 32ks+8g..+7)
  float m[QB], l[QB];
  f32x4 lb[QB];                      // sum of the bf16 p: an all-ones V^T block, every row alike
};

// Everything one pass over the keys needs.
template <int D, int F8>
struct PassCtx {
  using QK = QKOps<D, F8>;
  const char* Kb;    // keys / values of this (b, h): segment 0
  const char* Vb;
  int kseg;          // keys per K segment (Nkv for contiguous keys)
  int vfirst, vnext; // keys of the first V segment and of each later one
  int64_t kjump;     // bytes from the end of one K segment to the start of the next
  int64_t vjump;     // the same for V
  TileStream ks, vs; // the next K / V tile to stage
  lds_t *k0, *k1, *k2;  // K stages (separate scalars: never an indexed array)
  lds_t *v0, *v1, *v2;  // V stages
  int Nkv, ntiles, wave, lane, g;
  float c;
  int sa, sb;       // E8M0 scales of the key and query products (fp8 mode 2)
  bool str;          // segments may end inside a tile (set from a template parameter)
  // Fragment offsets, each plus the LDS address of stage 0 and held in a
  // register the compiler cannot see through: a read of stage j is then
  // that register plus the constant (stage j - stage 0 + in-tile offset),
  // which the instruction encodes, so the key loop does no address
  // arithmetic (and the reads keep the stage array as their object, so the
  // compiler still knows they do not touch the stage being loaded).
  int kof[QK::KS];       // K fragment (ks): byte offset within a 16-key block + kbase
  int vxo[Geo<D>::DB];   // V^T fragment (db): byte offset within a 32-key step + vbase
  int kbase, vbase;      // LDS addresses of the stages k0 and v0
  // The lane's query rows (one per 16-row block) of this unit and of the
  // next one (null: the next unit's queries are loaded by begin_tile).
  const char* cq[2];
  const char* nq[2];
  bool nqv;              // nq holds the next unit's rows
  lds_i32* anyw;         // one word per wave for any_row_flagged
  int kld[(QK::PIECES + kWaves - 1) / kWaves];      // K load-piece source offsets
  int vld[(Geo<D>::PIECES + kWaves - 1) / kWaves];  // V load-piece source offsets
};

// Stage of tile t: PH = t % 3 when known at compile time, else -1.
__device__ __forceinline__ lds_t* stage_of(lds_t* s0, lds_t* s1, lds_t* s2, int PH, int t) {
  const int i = PH >= 0 ? PH % kStages : t % kStages;
  return i == 0 ? s0 : (i == 1 ? s1 : s2);
}
#define KSTAGE(x, PH, t) stage_of((x).k0, (x).k1, (x).k2, (PH), (t))
#define VSTAGE(x, PH, t) stage_of((x).v0, (x).v1, (x).v2, (PH), (t))

// S^T of one 32-key step (rows [0, 32) at kst): S[kb][qb] holds keys
// 16kb + 4g + r for the lane's query of block qb.
template <int D, int F8, int QB>
__device__ __forceinline__ void qk_step(f32x4 (&S)[2][QB], const lds_t* kst,
                                        const PassCtx<D, F8>& x, const Frags<D, F8, QB>& f) {
  using QK = QKOps<D, F8>;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) S[kb][qb] = f32x4{};
#pragma unroll
  for (int ks = 0; ks < QK::KS; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const typename QK::Frag a = QK::load(kst - x.kbase + kb * 16 * QK::ROWB, x.kof[ks]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) S[kb][qb] = QK::mma_s(a, f.q[qb][ks], S[kb][qb], x.sa, x.sb);
    }
}

// Row max of one 32-key step (reference max / exact-max pass); keys >= Nkv
// excluded when MASK.
template <bool MASK, int QB>
__device__ __forceinline__ void rowmax_step(const f32x4 (&S)[2][QB], float (&m)[QB], int key0,
                                            int Nkv, int g) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = !MASK || key0 + 16 * kb + 4 * g + r < Nkv;
        mx = fmaxf(mx, ok ? S[kb][qb][r] : -INFINITY);
      }
    m[qb] = fmaxf(m[qb], quad_max(mx));
  }
}

// One 32-key slot: QK^T of the next step into Sn (K rows at k_next), PV of
// the previous step from Pp (V rows at v_prev), softmax of this step from Sc
// into Pc.  Laid out as 16 groups fenced by sched_barrier(0): group g runs
// the QK^T MFMAs [g NQK/16, (g+1) NQK/16) (index i: ks = i / 2QB, kb =
// (i / QB) % 2, qb = i % QB), the PV MFMAs [g NPV/16, (g+1) NPV/16)
// (index j: db = j / QB, qb = j % QB) and the softmax scores
// [g NS/16, (g+1) NS/16) (index e: qb = e / 8, kb = (e / 4) % 2, r = e % 4),
// and issues the LDS reads of the fragments first needed LA groups later.
// The P^T operand of block qb packs the keys 4g + r (kb 0) and 16 + 4g + r
// (kb 1): MFMA k index 8g + j <-> key 4g + j (j < 4), 16 + 4g + j - 4 (j >= 4).
// NOQK: the last slot of a pass, which has no next step: no QK^T MFMAs and
// no K fragment reads.
template <int D, int F8, bool MASK, bool NOQK = false, bool FB = false, int QB>
__device__ __forceinline__ void slot(Frags<D, F8, QB>& f, const f32x4 (&Sc)[2][QB], f32x4 (&Sn)[2][QB],
                                     const bf16x8 (&Pp)[QB], bf16x8 (&Pc)[QB],
                                     const lds_t* k_next, const lds_t* v_prev,
                                     const PassCtx<D, F8>& x, int key0) {
  using Gm = Geo<D>;
  using QK = QKOps<D, F8>;
  constexpr int NG = 16;                       // groups
  constexpr int NQK = 2 * QB * QK::KS;        // QK^T MFMAs
  constexpr int NPV = QB * Gm::DB;            // PV MFMAs
  constexpr int NS = 8 * QB;                  // softmax scores per lane
  constexpr int NKF = 2 * QK::KS;              // K fragments (ks, kb), ks-major
  constexpr int NVF = Gm::DB;                  // V^T fragments (db)
  constexpr int LA = 1;                        // read lookahead, in groups
  typename QK::Frag kf[NKF];
  bf16x8 vf[NVF];
  auto load_k = [&](int i) {
    kf[i] = QK::load(k_next - x.kbase + (i & 1) * 16 * QK::ROWB, x.kof[i >> 1]);
  };
  auto load_v = [&](int i) {
    const lds_t* base = v_prev - x.vbase + x.vxo[i];
    const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)base));
    const bf16x4 hi = __builtin_bit_cast(
        bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 16 * Gm::ROWB)));
    vf[i] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  // first group that uses K fragment f / V^T fragment f
  auto kfirst = [](int fi) { return fi * QB * NG / NQK; };
  auto vfirst = [](int fi) { return fi * QB * NG / NPV; };
#pragma unroll
  for (int fi = 0; fi < NKF; ++fi)
    if (!NOQK && kfirst(fi) < LA) load_k(fi);
#pragma unroll
  for (int fi = 0; fi < NVF; ++fi)
    if (vfirst(fi) < LA) load_v(fi);
  const bf16x8 ones8 = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                        (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
  float l[QB], mc[QB], p[QB][8];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    l[qb] = f.l[qb];
    mc[qb] = f.m[qb] * x.c;
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      if (!NOQK) Sn[kb][qb] = f32x4{};
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int fi = 0; fi < NKF; ++fi)
      if (!NOQK && kfirst(fi) >= LA && kfirst(fi) == g + LA) load_k(fi);
#pragma unroll
    for (int fi = 0; fi < NVF; ++fi)
      if (vfirst(fi) >= LA && vfirst(fi) == g + LA) load_v(fi);
#pragma unroll
    for (int i = g * NQK / NG; i < (g + 1) * NQK / NG; ++i) {
      const int ks = i / (2 * QB), kb = (i / QB) % 2, qb = i % QB;
      if (!NOQK) Sn[kb][qb] = QK::mma_s(kf[ks * 2 + kb], f.q[qb][ks], Sn[kb][qb], x.sa, x.sb);
    }
#pragma unroll
    for (int j = g * NPV / NG; j < (g + 1) * NPV / NG; ++j) {
      const int db = j / QB, qb = j % QB;
      f.o[qb][db] = mfma16(vf[db], Pp[qb], f.o[qb][db]);
    }
    // The row sums of the bf16 P^T the PV product multiplies, on the matrix
    // cores: an all-ones V^T block, one MFMA per query block.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      if (g == NG - 1 - (NG / QB) * qb) f.lb[qb] = mfma16(ones8, Pp[qb], f.lb[qb]);
#pragma unroll
    for (int e = g * NS / NG; e < (g + 1) * NS / NG; ++e) {
      const int qb = e / 8, kb = (e / 4) % 2, r = e % 4;
      float sv = Sc[kb][qb][r];
      // Pin the softmax work to its group: without the opaque copies the
      // optimizer sinks it (and the row sums) towards its uses in later
      // slots, which leaves those slots' MFMAs with no VALU work to hide.
      asm volatile("" : "+v"(sv));
      if (MASK) sv = (key0 + 16 * kb + 4 * x.g + r < x.Nkv) ? sv : -INFINITY;
      // mode 2: sv is the base-2 score; the first attempt takes no reference
      // max (m = 0), the exact-max pass (FB) subtracts the row's
      p[qb][4 * kb + r] = __builtin_amdgcn_exp2f(
          F8 == 2 ? (FB ? sv - f.m[qb] : sv) : fmaf(sv, x.c, -mc[qb]));
      if (e & 1) {
        const int j = 4 * kb + r - 1;
        const float p0 = p[qb][j], p1 = p[qb][j + 1];
        bf16x2 pk = {(__bf16)p0, (__bf16)p1};
        l[qb] += p0 + p1;
        asm volatile("" : "+v"(pk), "+v"(l[qb]));
        Pc[qb][j] = pk[0];
        Pc[qb][j + 1] = pk[1];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    f.l[qb] = l[qb];
  }
}

// Load the queries of the lane's rows (one row pointer per 16-row block) as
// the Q^T operands.
template <int D, int F8, int QB>
__device__ __forceinline__ void load_queries(Frags<D, F8, QB>& f, const char* const (&rows)[2], int g) {
  using QK = QKOps<D, F8>;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < QK::KS; ++ks) f.q[qb][ks] = QK::load_q(rows[qb], g, ks);
}

// One 64-key tile t = slots 2t and 2t+1.  PH = t % 3 when known at compile
// time (the unrolled main loop: every LDS stage is then a distinct array and
// the loads into stage t+2 overlap the reads of the others), or -1.
// On entry S0 holds S^T of step 2t and Pa holds P of step 2t-1; on exit S0
// holds S^T of step 2t+2 and Pa holds P of step 2t+1.  LAST: t is the last
// tile, so there is no step 2t+2: its slot has no QK^T, and once the first
// slot's QK^T has read the queries, the next unit's queries are loaded in
// their place (when x.nqv), a tile and the epilogue ahead of their use.
template <int D, int F8, int PH, bool MASK, int WAITN = 0, bool LAST = false, bool FB = false, int QB>
__device__ __forceinline__ void tile_trip(int t, Frags<D, F8, QB>& f, f32x4 (&S0)[2][QB], f32x4 (&S1)[2][QB],
                                          bf16x8 (&Pa)[QB], bf16x8 (&Pb)[QB],
                                          PassCtx<D, F8>& x) {
  using Gm = Geo<D>;
  using QK = QKOps<D, F8>;
  tile_barrier<WAITN>();  // K_{t+1}, V_t landed; every wave is done with tile t-1
  const int p2 = PH >= 0 ? PH + 2 : -1, p1 = PH >= 0 ? PH + 1 : -1;
  if (t + 2 < x.ntiles)  // K tile t+2 is the K stream's next tile
    stage_next<QK::ROWB, QK::PIECES>(x.ks, x.kjump, KSTAGE(x, p2, t + 2), x.wave, x.kld, x.str);
  if (t + 1 < x.ntiles)  // V tile t+1 is the V stream's next tile
    stage_next<Gm::ROWB, Gm::PIECES>(x.vs, x.vjump, VSTAGE(x, p1, t + 1), x.wave, x.vld, x.str);
  const lds_t* kcur = KSTAGE(x, PH, t);
  const lds_t* knext = KSTAGE(x, p1, t + 1);
  const lds_t* vcur = VSTAGE(x, PH, t);
  const lds_t* vprev = VSTAGE(x, p2, t + 2);  // stage of tile t-1
  const int key0 = t * kBN;
  slot<D, F8, MASK, false, FB>(f, S0, S1, Pa, Pb, kcur + 32 * QK::ROWB, vprev + 32 * Gm::ROWB, x, key0);
  if (LAST) {
    if (x.nqv) load_queries<D, F8>(f, x.nq, x.g);
    slot<D, F8, MASK, true, FB>(f, S1, S0, Pb, Pa, knext, vcur, x, key0 + 32);
  } else {
    slot<D, F8, MASK, false, FB>(f, S1, S0, Pb, Pa, knext, vcur, x, key0 + 32);
  }
}

// O^T += V^T P^T for one 32-key step (used once, after the loop).
template <int D, int F8, int QB>
__device__ __forceinline__ void pv_step(Frags<D, F8, QB>& f, const bf16x8 (&P)[QB], const lds_t* vst,
                                        const PassCtx<D, F8>& x) {
  using Gm = Geo<D>;
#pragma unroll
  for (int db = 0; db < Gm::DB; ++db) {
    const lds_t* base = vst - x.vbase + x.vxo[db];
    const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)base));
    const bf16x4 hi = __builtin_bit_cast(
        bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 16 * Gm::ROWB)));
    const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) f.o[qb][db] = mfma16(a, P[qb], f.o[qb][db]);
  }
  const bf16x8 ones8 = {(__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f,
                        (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) f.lb[qb] = mfma16(ones8, P[qb], f.lb[qb]);
}

// Stage the first K tiles (0 and 1) and V tile 0 of a pass.
template <int D, int F8>
__device__ __forceinline__ void stage_first(PassCtx<D, F8>& x) {
  using Gm = Geo<D>;
  using QK = QKOps<D, F8>;
  x.ks = TileStream{x.Kb, x.kseg, x.kseg, x.Nkv};
  x.vs = TileStream{x.Vb, x.vfirst, x.vnext, x.Nkv};
  stage_next<QK::ROWB, QK::PIECES>(x.ks, x.kjump, x.k0, x.wave, x.kld, x.str);
  if (x.ntiles > 1) stage_next<QK::ROWB, QK::PIECES>(x.ks, x.kjump, x.k1, x.wave, x.kld, x.str);
  stage_next<Gm::ROWB, Gm::PIECES>(x.vs, x.vjump, x.v0, x.wave, x.vld, x.str);
}

// Whether a row's pass must be redone with its exact max: its sum outgrew
// the bound (or is not a number); in fp8 mode 2, whose first attempt takes
// no reference max (m = 0, p = 2^s), also when the sum is tiny, all scores
// far below zero.
template <int F8>
__device__ __forceinline__ bool row_needs_exact_max(float l) {
  return !(l < kMaxSum) || (F8 == 2 && !(l > kMinSum));
}

// One full pass over the keys whose first tiles stage_first has issued: the
// unmasked tiles (unrolled by the stage count), the partial last tile (if
// any) with masking, then the PV of the last step.  Returns true if some
// row's sum outgrew its reference.  NST > 0: the first tiles were issued
// before the previous tile's NST output and LSE stores, so the first two
// waits leave those stores in flight.
template <int D, int F8, int NST, bool FB = false, int QB>
__device__ __forceinline__ bool run_pass_body(Frags<D, F8, QB>& f, PassCtx<D, F8>& x) {
  using Gm = Geo<D>;
  constexpr bool PF = NST > 0;
  // The first slot multiplies P = 0 by the V stage of tile -1 (stage 2): zero
  // it so no stale Inf/NaN bit pattern can turn 0 * V into NaN.
  for (int i = threadIdx.x; i < Gm::TILE / 16; i += kThreads)
    reinterpret_cast<lds_u32x4*>(x.v2)[i] = u32x4{0u, 0u, 0u, 0u};
  f32x4 S0[2][QB], S1[2][QB];
  bf16x8 Pa[QB], Pb[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) Pa[qb] = bf16x8{};
  tile_barrier<NST>();  // K tile 0 (and K 1, V 0) landed
  qk_step<D, F8>(S0, x.k0, x, f);
  if (f.m[0] == -INFINITY) {  // first attempt: reference max = max of step 0
    float m[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m[qb] = -INFINITY;
    if (x.Nkv < 32)
      rowmax_step<true>(S0, m, 0, x.Nkv, x.g);
    else
      rowmax_step<false>(S0, m, 0, x.Nkv, x.g);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) f.m[qb] = m[qb];
  }
  const int nmid = x.ntiles - 1;  // tiles before the last
  int t = 0;
  if (PF && nmid >= kStages) {  // no load is issued between the first wait and trip 0's
    tile_trip<D, F8, 0, false, NST, false, FB>(0, f, S0, S1, Pa, Pb, x);
    tile_trip<D, F8, 1, false, 0, false, FB>(1, f, S0, S1, Pa, Pb, x);
    tile_trip<D, F8, 2, false, 0, false, FB>(2, f, S0, S1, Pa, Pb, x);
    t = kStages;
  }
  for (; t + kStages <= nmid; t += kStages) {
    tile_trip<D, F8, 0, false, 0, false, FB>(t, f, S0, S1, Pa, Pb, x);
    tile_trip<D, F8, 1, false, 0, false, FB>(t + 1, f, S0, S1, Pa, Pb, x);
    tile_trip<D, F8, 2, false, 0, false, FB>(t + 2, f, S0, S1, Pa, Pb, x);
  }
  for (; t < nmid; ++t) tile_trip<D, F8, -1, false, 0, false, FB>(t, f, S0, S1, Pa, Pb, x);
  // the last tile, masked whether or not it is partial (one instantiation
  // for both keeps the kernel within its registers)
  tile_trip<D, F8, -1, true, 0, true, FB>(t, f, S0, S1, Pa, Pb, x);
  pv_step<D, F8>(f, Pa, VSTAGE(x, -1, x.ntiles - 1) + 32 * Gm::ROWB, x);
  bool flag = false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) flag |= row_needs_exact_max<F8>(quad_sum(f.l[qb]));
  return flag;
}

// Exact row max over all keys, taken as the reference of the rows whose sum
// outgrew theirs (only when the fixed-reference loop flagged some row); the
// other rows keep their first reference, so a row's result does not depend
// on which rows share its tile.
template <int D, int F8, int QB>
__device__ __forceinline__ void exact_max_pass(Frags<D, F8, QB>& f, PassCtx<D, F8>& x) {
  using QK = QKOps<D, F8>;
  float m[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) m[qb] = -INFINITY;
  x.ks = TileStream{x.Kb, x.kseg, x.kseg, x.Nkv};
  for (int t = 0; t < x.ntiles; ++t) {
    __syncthreads();  // every wave is done reading the stage
    stage_next<QK::ROWB, QK::PIECES>(x.ks, x.kjump, x.k0, x.wave, x.kld, x.str);
    tile_barrier();  // landed
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x4 S[2][QB];
      qk_step<D, F8>(S, x.k0 + sub * 32 * QK::ROWB, x, f);
      if (t * kBN + kBN > x.Nkv)
        rowmax_step<true>(S, m, t * kBN + sub * 32, x.Nkv, x.g);
      else
        rowmax_step<false>(S, m, t * kBN + sub * 32, x.Nkv, x.g);
    }
  }
  __syncthreads();
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
    if (row_needs_exact_max<F8>(quad_sum(f.l[qb]))) f.m[qb] = m[qb];
}

// Where the tokens of one (b, h) live.  Contiguous [B,H,N,D] tensors are one
// segment per (b, h) (qseg = Nq, kseg = Nkv, hg = htot = H, hoff = 0).  Ulysses
// token shards [P][B,H,N/P,D] hold the N tokens of head h in P segments of
// N/P rows, one per shard; the launch then covers the hg = H/P heads of one
// head group, starting at head hoff.
struct Layout {
  int qseg, kseg;  // query / key rows per segment
  int hg;          // heads covered by the launch
  int htot;        // heads in the buffers
  int hoff;        // first head of the launch
  int B;
  int tile0;       // first query tile of the launch (tiles of 16 * QB * kWaves rows)
};

// Element offset of token n of the (b, hh) head: segment n / seg.
__device__ __forceinline__ int64_t token_offset(int n, int seg, int64_t head_elems,
                                                int64_t sstride, int D) {
  if (n < seg) return head_elems + (int64_t)n * D;
  const int sg = n / seg;
  return head_elems + sg * sstride + (int64_t)(n - sg * seg) * D;
}

// Key-split launch (contiguous layout only): grid unit u computes key chunk
// u % nsplit of query tile tile0 + u / nsplit.  Chunk j holds keys
// [j*kc, min((j+1)*kc, Nkv)) with kc a multiple of the key tile, and writes
// its float32 O and LSE over those keys alone to the workspace, chunk-major:
// O at (j*rows + r - row0)*D, LSE at j*rows + r - row0, for the flat query
// row r = (b*H + h)*Nq + n.  The partials are then merged by log-sum-exp.
struct Split {
  int tile0, nsplit, kc;
  int64_t row0, rows;
};

// Joint text + image attention ("Parallelism Acceleration Guide", vLLM-Omni
// docs, "How to parallelize a new model"): the joint sequence is the Nt text
// tokens of head h0 + h of [B,Ht,Nt,D] tensors, then the Ni image tokens of
// head h of [B,H,Ni,D] tensors.  Queries are read from their parts and
// turned by the part's rotary tables ([N, D/2] float32 cosines and sines; a
// part without tables is not turned); V is read from its parts when v_txt /
// v_img are given (Nt a multiple of the key tile), else from the packed V;
// K always comes packed (turned).
struct JointArgs {
  const __bf16* q_txt;
  const __bf16* q_img;
  const __bf16* v_txt;
  const __bf16* v_img;
  const float* cos_txt;
  const float* sin_txt;
  const float* cos_img;
  const float* sin_img;
  int Nt, Ni, Ht, h0;
};

// Where one work unit's rows and keys are: the unit's head (bh), query tile
// (qt), key chunk (SPLIT), its key count and the pointers of its K and V.
struct TileInfo {
  int bh, qt, chunk, Nkv, kseg;
  int vfirst, vnext;    // V stream: rows of its first segment and of each later one
  int64_t vjump;        // bytes from the end of one V segment to the start of the next
  int64_t qhead;        // element offset of the head's segment 0 in Q and O
  const char* Kb;
  const char* Vb;
  const __bf16* qtxt;   // JOINT: the head's text and image queries
  const __bf16* qimg;
  float c;              // softmax constant (F8: times the head's descales; mode 2: unused)
};

template <int D, int F8, bool SPLIT, bool JOINT>
__device__ __forceinline__ TileInfo tile_info(int u, int total, int n_qtiles, int Nkv, const Layout& lay,
                                              const void* K, const __bf16* V, float c,
                                              const float* qds, const float* kds, const Split& sp,
                                              const JointArgs& ja) {
  constexpr int QKB = F8 ? 1 : 2;  // bytes per q / k element
  TileInfo ti;
  int tile = remap_xcd(u, total);
  if (!SPLIT) tile += lay.tile0;
  ti.chunk = 0;
  if (SPLIT) {
    const int v = tile;
    tile = sp.tile0 + v / sp.nsplit;
    ti.chunk = v - (v / sp.nsplit) * sp.nsplit;
  }
  const int kbeg = SPLIT ? ti.chunk * sp.kc : 0;  // first key of the chunk
  ti.Nkv = SPLIT ? min(sp.kc, Nkv - kbeg) : Nkv;
  ti.bh = tile / n_qtiles;
  ti.qt = tile - ti.bh * n_qtiles;
  // bh = b * hg + h'; the buffers hold head hoff + h' of batch b.
  const int bb = ti.bh / lay.hg;
  const int hh = lay.hoff + (ti.bh - bb * lay.hg);
  ti.qhead = ((int64_t)bb * lay.htot + hh) * lay.qseg * D;
  ti.Kb = static_cast<const char*>(K) + (((int64_t)bb * lay.htot + hh) * lay.kseg + kbeg) * D * QKB;
  ti.Vb = reinterpret_cast<const char*>(V + (((int64_t)bb * lay.htot + hh) * lay.kseg + kbeg) * D);
  ti.kseg = lay.kseg - kbeg;
  ti.vfirst = ti.kseg;
  ti.vnext = ti.kseg;
  // segment starts are B*H*kseg rows apart; the jump is from one segment's end
  // (only key-split launches start inside a segment, and they have one)
  ti.vjump = ((int64_t)lay.B * lay.htot - 1) * lay.kseg * D * 2;
  ti.c = F8 == 1 ? c * qds[ti.bh] * kds[ti.bh] : c;
  ti.qtxt = ti.qimg = nullptr;
  if (JOINT) {  // contiguous layout: bh = b * H + h, head h of the image, h0 + h of the text
    const int64_t th = (int64_t)bb * ja.Ht + ja.h0 + hh, ih = (int64_t)bb * lay.htot + hh;
    ti.qtxt = ja.Nt ? ja.q_txt + th * ja.Nt * D : nullptr;
    ti.qimg = ja.Ni ? ja.q_img + ih * ja.Ni * D : nullptr;
    if (ja.v_txt || ja.v_img) {  // V read from its two parts: the text rows, then the image rows
      const char* vt = ja.Nt ? reinterpret_cast<const char*>(ja.v_txt + th * ja.Nt * D) : nullptr;
      const char* vi = ja.Ni ? reinterpret_cast<const char*>(ja.v_img + ih * ja.Ni * D) : nullptr;
      if (ja.Nt) {
        ti.Vb = vt;
        ti.vfirst = ja.Nt;
        ti.vnext = ja.Ni;
        ti.vjump = vi ? (int64_t)((uintptr_t)vi - (uintptr_t)vt) - (int64_t)ja.Nt * D * 2 : 0;
      } else {
        ti.Vb = vi;
        ti.vfirst = ti.vnext = ja.Ni;
        ti.vjump = 0;
      }
    }
  }
  return ti;
}

// The lane's query row pointers of a unit, one per 16-row block (rows past
// Nq point at row Nq - 1).
template <int D, int F8, int QB>
__device__ __forceinline__ void query_rows(const char* (&rows)[2], const TileInfo& ti, const void* Q,
                                           int Nq, const Layout& lay, int64_t qsstride, int wave,
                                           int c16) {
  constexpr int QKB = F8 ? 1 : 2;
  const int qrow0 = ti.qt * (16 * QB * kWaves) + wave * (16 * QB) + c16;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = min(qrow0 + 16 * (qb < QB ? qb : 0), Nq - 1);
    rows[qb] = static_cast<const char*>(Q) + token_offset(row, lay.qseg, ti.qhead, qsstride, D) * QKB;
  }
}

// Point the pass at a unit and issue its first K / V tiles; load its queries
// when `loadq` (otherwise the previous unit's last tile has loaded them).
// JOINT: a query is a text or an image token of the joint sequence (text
// first), turned by its part's rotary table when the part has one; the
// fragment of k-step ks holds channel pairs 16 ks + 4 g .. +3 of the lane's
// token, one per 32-bit word.
template <int D, int F8, bool JOINT, int QB>
__device__ __forceinline__ void begin_tile(Frags<D, F8, QB>& f, PassCtx<D, F8>& x, const TileInfo& ti,
                                           const void* Q, int Nq, const Layout& lay,
                                           int64_t qsstride, int c16, const JointArgs& ja,
                                           bool loadq) {
  using QK = QKOps<D, F8>;
  x.Kb = ti.Kb;
  x.Vb = ti.Vb;
  x.kseg = ti.kseg;
  x.vfirst = ti.vfirst;
  x.vnext = ti.vnext;
  x.vjump = ti.vjump;
  x.Nkv = ti.Nkv;
  x.ntiles = (ti.Nkv + kBN - 1) / kBN;
  x.c = ti.c;
  stage_first<D, F8>(x);
  if (!JOINT) {
    query_rows<D, F8, QB>(x.cq, ti, Q, Nq, lay, qsstride, x.wave, c16);
    if (loadq) load_queries<D, F8>(f, x.cq, x.g);
    return;
  }
  const int qrow0 = ti.qt * (16 * QB * kWaves) + x.wave * (16 * QB) + c16;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = min(qrow0 + 16 * qb, Nq - 1);
    if constexpr (JOINT && !F8) {
      const bool txt = row < ja.Nt;
      const int m = txt ? row : row - ja.Nt;
      const __bf16* src = (txt ? ti.qtxt : ti.qimg) + (int64_t)m * D;
      const float* ct = txt ? ja.cos_txt : ja.cos_img;
      const float* st = txt ? ja.sin_txt : ja.sin_img;
#pragma unroll
      for (int ks = 0; ks < QK::KS; ++ks) {
        u32x4 w = *reinterpret_cast<const u32x4*>(src + ks * 32 + x.g * 8);
        if (ct) {
          const int pr = (int64_t)m * (D / 2) + 16 * ks + 4 * x.g;
          const f32x4 cv = *reinterpret_cast<const f32x4*>(ct + pr);
          const f32x4 sv = *reinterpret_cast<const f32x4*>(st + pr);
#pragma unroll
          for (int j = 0; j < 4; ++j) w[j] = rope_turn_pair(w[j], cv[j], sv[j]);
        }
        f.q[qb][ks] = __builtin_bit_cast(bf16x8, w);
      }
    }
  }
}

// Whether a row of any wave has `flag`: one LDS word per wave, a wait for
// the LDS write alone (s_waitcnt lgkmcnt(0); vmcnt and expcnt at their
// maxima, no wait) and s_barrier.  __syncthreads_or, and a workgroup fence,
// would also wait for every outstanding vector memory operation, here the
// next unit's query loads.  The words are next written a unit later, after
// barriers every wave has passed, so no wave still reads them then.
template <int D, int F8>
__device__ __forceinline__ bool any_row_flagged(const PassCtx<D, F8>& x, bool flag) {
  const bool w = __builtin_amdgcn_ballot_w64(flag) != 0;
  if (x.lane == 0) x.anyw[x.wave] = w;
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  int any = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) any |= x.anyw[i];
  return any != 0;
}

// Attention of the unit begin_tile pointed the pass at.  Second attempt only
// if some row's sum outgrew its reference max: then the tile is redone (all
// waves decide together) with the exact row max for those rows.  Ends with every wave done
// with the LDS stages.
// NST: output store instructions per wave still in flight from the previous
// unit (0 for the first unit).
template <int D, int F8, int NST, int QB>
__device__ __forceinline__ void compute_tile(Frags<D, F8, QB>& f, PassCtx<D, F8>& x) {
  using Gm = Geo<D>;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    f.m[qb] = F8 == 2 ? 0.0f : -INFINITY;  // mode 2: no reference max on the first attempt
    f.l[qb] = 0.f;
    f.lb[qb] = f32x4{};
#pragma unroll
    for (int db = 0; db < Gm::DB; ++db) f.o[qb][db] = f32x4{};
  }
  const bool flag = run_pass_body<D, F8, NST>(f, x);
  if (any_row_flagged(x, flag)) {
    if (x.nqv) load_queries<D, F8>(f, x.cq, x.g);  // the last tile replaced them
    exact_max_pass<D, F8>(f, x);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f.l[qb] = 0.f;
      f.lb[qb] = f32x4{};
#pragma unroll
      for (int db = 0; db < Gm::DB; ++db) f.o[qb][db] = f32x4{};
    }
    stage_first<D, F8>(x);
    run_pass_body<D, F8, 0, F8 == 2>(f, x);
    __syncthreads();
  }
}

// Store instructions per wave of one unit's epilogue: per query block, one
// per 16-channel block (float32) or per 32-channel pair of blocks (bf16),
// and one for the LSE.
template <int D, bool OUT_F32, int QB>
constexpr int kStoreInsts = QB * ((OUT_F32 ? Geo<D>::DB : Geo<D>::DB / 2) + 1);

// Epilogue of one unit: O = O^T / lb, LSE = (m*c + log2 l) * ln 2.  Every
// lane stores (a row past Nq stores row Nq - 1, which it computed from that
// row's query, so the same bits), so each wave issues exactly kStoreInsts
// stores, with or without an LSE, which the next unit's first waits count on.
// bf16 output: a lane of group g holds channels 16 db + 4 g .. +3 of its row;
// blocks 2p and 2p + 1 are exchanged between groups g and g ^ 1
// (v_permlane16_swap swaps the odd 16-lane rows of one register with the
// even rows of another), after which group g holds the 8 channels
// 16 (2p + (g & 1)) + 8 (g >> 1) .. +7 and each row's 4 lanes write its
// channels [32p, 32p + 32) as 16-byte pieces: half the instructions, and
// 64-byte row pieces instead of 32-byte ones.  The bf16 output is stored
// non-temporally (nothing in the kernel reads it back): the 64 KB of O a unit
// writes then does not displace the K/V tiles the XCD's other units are
// streaming through its L2 (cross attention over 512 keys 2.5% faster, image
// share 1%, the long shapes unchanged); the price is that a row's four
// 64-byte pieces reach memory uncombined.  Float32 output (Ring partials)
// gains nothing from it, so it is stored as usual.
template <int D, bool OUT_F32, int F8, bool SPLIT, int QB>
__device__ __forceinline__ void store_tile(const Frags<D, F8, QB>& f, const TileInfo& ti, void* Oout,
                                           float* LSE, int Nq, const Layout& lay, int64_t qsstride,
                                           const Split& sp, int wave, int c16, int g) {
  using Gm = Geo<D>;
  const int qtop = ti.qt * (16 * QB * kWaves) + wave * (16 * QB);  // the wave's first row
  const int qrow0 = qtop + c16;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = quad_sum(f.l[qb]);
    const float inv = 1.0f / f.lb[qb][0];
    const int qrow = min(qrow0 + 16 * qb, Nq - 1);
    const int64_t wrow = (int64_t)ti.chunk * sp.rows + (int64_t)ti.bh * Nq + qrow - sp.row0;
    const int64_t obase = SPLIT ? wrow * D : token_offset(qrow, lay.qseg, ti.qhead, qsstride, D);
    if (OUT_F32) {
#pragma unroll
      for (int db = 0; db < Gm::DB; ++db)
        *reinterpret_cast<f32x4*>(static_cast<float*>(Oout) + obase + db * 16 + 4 * g) =
            f.o[qb][db] * inv;
    } else {
#pragma unroll
      for (int p = 0; p < Gm::DB / 2; ++p) {
        const f32x4 a = f.o[qb][2 * p] * inv, b = f.o[qb][2 * p + 1] * inv;
        const u32x2 aw = __builtin_bit_cast(
            u32x2, bf16x4{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3]});
        const u32x2 bw = __builtin_bit_cast(
            u32x2, bf16x4{(__bf16)b[0], (__bf16)b[1], (__bf16)b[2], (__bf16)b[3]});
        const auto lo = __builtin_amdgcn_permlane16_swap(aw[0], bw[0], false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(aw[1], bw[1], false, false);
        const int ch = 32 * p + 16 * (g & 1) + 8 * (g >> 1);
        __builtin_nontemporal_store(u32x4{lo[0], hi[0], lo[1], hi[1]},
                                    reinterpret_cast<u32x4*>(static_cast<__bf16*>(Oout) + obase + ch));
      }
    }
    // The LSE goes through a buffer descriptor over the block's 16 rows from
    // its first (clamped) row r0: the lanes of groups 1-3, and all lanes when
    // LSE is null (a zero-size record), address past its end, and the
    // hardware drops those stores, so the store instruction is always issued.
    const int r0 = min(qtop + 16 * qb, Nq - 1);
    const int64_t lrow = SPLIT ? (int64_t)ti.chunk * sp.rows + (int64_t)ti.bh * Nq + r0 - sp.row0
                               : (int64_t)ti.bh * Nq + r0;
    const __amdgpu_buffer_rsrc_t lr = __builtin_amdgcn_make_buffer_rsrc(
        LSE ? (void*)(LSE + lrow) : nullptr, (short)0, LSE ? 64 : 0, 0x00020000);
    const float lse = ((F8 == 2 ? f.m[qb] : f.m[qb] * ti.c) + __builtin_amdgcn_logf(l_tot)) *
                      0.6931471805599453f;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, lse), lr,
                                          g == 0 ? (qrow - r0) * 4 : (1 << 30), 0, 0);
  }
}

// The kernel body: a persistent workgroup computes units blockIdx.x,
// blockIdx.x + gridDim.x, ... (with more units than workgroups gridDim.x is
// the compute-unit count, 256, a multiple of 8, so they all map to one XCD's
// range).  A unit's last key tile loads the next unit's queries (JOINT: the
// next unit's begin_tile loads and turns them); after the unit's last LDS
// read it issues the next unit's first K / V tiles, and only then stores the
// unit's output, so the next unit's first waits need not wait for those
// stores.  F8: q and
// k are E4M3 codes (1 byte per element) whose scores are rescaled by the
// per-(b, h) factors qds[bh] * kds[bh]; else q and k are bf16 and qds, kds
// are unused.  SPLIT: a key-split launch, total_tiles is then the number of
// units.
template <int D, bool OUT_F32, int F8, bool SPLIT = false, bool JOINT = false, int QB = kQB,
          bool STR = false>
__device__ __forceinline__ void attn_fwd_body(const void* __restrict__ Q, const void* __restrict__ K,
                                              const __bf16* __restrict__ V, void* __restrict__ Oout,
                                              float* __restrict__ LSE, int Nq, int Nkv,
                                              int n_qtiles, int total_tiles, float c, Layout lay,
                                              const float* __restrict__ qds,
                                              const float* __restrict__ kds, Split sp = {},
                                              JointArgs ja = {}) {
  using Gm = Geo<D>;
  using QK = QKOps<D, F8>;
  constexpr int QKB = F8 ? 1 : 2;  // bytes per q / k element
  __shared__ __attribute__((aligned(1024))) char k0s[QK::TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[QK::TILE];
  __shared__ __attribute__((aligned(1024))) char k2s[QK::TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[Gm::TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[Gm::TILE];
  __shared__ __attribute__((aligned(1024))) char v2s[Gm::TILE];
  __shared__ int any_words[kWaves];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  const int64_t qsstride = (int64_t)lay.B * lay.htot * lay.qseg * D;

  PassCtx<D, F8> x;
  // segment starts are B*H*kseg rows apart; the jump is from one segment's end
  // (only key-split launches start inside a segment, and they have one)
  x.kjump = ((int64_t)lay.B * lay.htot - 1) * lay.kseg * D * QKB;
  x.k0 = (lds_t*)k0s; x.k1 = (lds_t*)k1s; x.k2 = (lds_t*)k2s;
  x.v0 = (lds_t*)v0s; x.v1 = (lds_t*)v1s; x.v2 = (lds_t*)v2s;
  x.wave = wave;
  x.lane = lane;
  x.str = STR;
  x.anyw = (lds_i32*)any_words;
  x.g = g;
  piece_offsets<QK::ROWB, QK::PIECES>(x.kld, wave, lane, [](int r) { return QK::swz(r); });
  piece_offsets<Gm::ROWB, Gm::PIECES>(x.vld, wave, lane, [](int r) { return swz_v<D>(r); });
  // K fragment (ks): row c16 of a 16-key block (bf16: chunk 4ks + g).
  x.kbase = (int)(size_t)x.k0;
  x.vbase = (int)(size_t)x.v0;
#pragma unroll
  for (int ks = 0; ks < QK::KS; ++ks) {
    x.kof[ks] = QK::frag_off(c16, g, ks) + x.kbase;
    asm volatile("" : "+v"(x.kof[ks]));
  }
  // V^T fragment (db), first of two transposing reads: lane t of its 16-lane
  // group g loads row 4g + t/4, channels 16db + 4(t%4) .. +3; the second read
  // is 16 rows further (same swizzle).  Chunk (2db + a) ^ 2(row & 7), a =
  // (t%4)/2, sits at bytes 32 (db ^ (row & 7)) + 16a of the row, and the
  // row, the 16a and the in-chunk offsets occupy bits disjoint from 32 db, so
  // the offset of fragment db is vxb ^ (32 db).
  {
    const int row = 4 * g + (c16 >> 2);
    const int ce0 = 4 * (c16 & 3);
    const int vxb = row * Gm::ROWB + (((ce0 >> 3) ^ swz_v<D>(row)) << 4) + (ce0 & 7) * 2;
#pragma unroll
    for (int db = 0; db < Gm::DB; ++db) {
      x.vxo[db] = (vxb ^ (32 * db)) + x.vbase;
      asm volatile("" : "+v"(x.vxo[db]));
    }
  }

  // The next unit's query rows, which this unit's last key tile loads
  // (JOINT: begin_tile loads and turns them).
  auto point_next = [&](int un) {
    x.nqv = !JOINT && un < total_tiles;
    if (x.nqv) {
      const TileInfo tp = tile_info<D, F8, SPLIT, JOINT>(un, total_tiles, n_qtiles, Nkv, lay, K, V,
                                                         c, qds, kds, sp, ja);
      query_rows<D, F8, QB>(x.nq, tp, Q, Nq, lay, qsstride, wave, c16);
    }
  };

  Frags<D, F8, QB> f;
  int u = blockIdx.x;
  TileInfo ti =
      tile_info<D, F8, SPLIT, JOINT>(u, total_tiles, n_qtiles, Nkv, lay, K, V, c, qds, kds, sp, ja);
  // fp8 mode 2: the descales are powers of two; their biased exponent fields
  // are the E8M0 scales of the key and query products (127 = 2^0)
  auto set_scales = [&](int bh) {
    // (read into scalar registers: the head is the same for the whole workgroup)
    x.sa = F8 == 2 ? __builtin_amdgcn_readfirstlane((int)((__float_as_uint(kds[bh]) >> 23) & 0xff)) : 127;
    x.sb = F8 == 2 ? __builtin_amdgcn_readfirstlane((int)((__float_as_uint(qds[bh]) >> 23) & 0xff)) : 127;
  };
  set_scales(ti.bh);
  begin_tile<D, F8, JOINT>(f, x, ti, Q, Nq, lay, qsstride, c16, ja, true);
  point_next(u + gridDim.x);
  compute_tile<D, F8, 0>(f, x);
  for (;;) {
    const int un = u + gridDim.x;
    const bool more = un < total_tiles;
    TileInfo tn;
    if (more) {
      tn = tile_info<D, F8, SPLIT, JOINT>(un, total_tiles, n_qtiles, Nkv, lay, K, V, c, qds, kds,
                                          sp, ja);
      set_scales(tn.bh);
      begin_tile<D, F8, JOINT>(f, x, tn, Q, Nq, lay, qsstride, c16, ja, !x.nqv);
    }
    // the next unit's loads stay ahead of this unit's stores
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    store_tile<D, OUT_F32, F8, SPLIT>(f, ti, Oout, LSE, Nq, lay, qsstride, sp, wave, c16, g);
    if (!more) break;
    u = un;
    ti = tn;
    point_next(u + gridDim.x);
    compute_tile<D, F8, kStoreInsts<D, OUT_F32, QB>>(f, x);
  }
}

// QB = 1: half-height tiles (128 query rows), for the last partial round.
// STR: Ulysses token shards whose length is not a multiple of the key tile.
template <int D, bool OUT_F32, int QB = kQB, bool STR = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void attn_fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                          const __bf16* __restrict__ V, void* __restrict__ Oout,
                          float* __restrict__ LSE, int Nq, int Nkv, int n_qtiles, int total_tiles,
                          float c, Layout lay) {
  attn_fwd_body<D, OUT_F32, false, false, false, QB, STR>(Q, K, V, Oout, LSE, Nq, Nkv, n_qtiles,
                                                          total_tiles, c, lay, nullptr, nullptr);
}

// Key-split partials (float32 O and LSE into the workspace).
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void attn_fwd_bf16_split_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                const __bf16* __restrict__ V, float* __restrict__ Opart,
                                float* __restrict__ Lpart, int Nq, int Nkv, int n_qtiles,
                                int units, float c, Layout lay, Split sp) {
  attn_fwd_body<D, true, false, true>(Q, K, V, Opart, Lpart, Nq, Nkv, n_qtiles, units, c, lay,
                                      nullptr, nullptr, sp);
}

// MODE 1: any per-head descales, scores scale * qds * kds * (q . k);
// MODE 2: power-of-two descales and the softmax constant folded into the
// query codes, scores in base 2 qds * kds * (q . k) from the scaled product.
template <bool OUT_F32, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void attn_fwd_fp8_kernel(const unsigned char* __restrict__ Q, const unsigned char* __restrict__ K,
                         const __bf16* __restrict__ V, void* __restrict__ Oout,
                         float* __restrict__ LSE, int Nq, int Nkv, int n_qtiles, int total_tiles,
                         float c, Layout lay, const float* __restrict__ qds,
                         const float* __restrict__ kds) {
  attn_fwd_body<128, OUT_F32, MODE>(Q, K, V, Oout, LSE, Nq, Nkv, n_qtiles, total_tiles, c, lay,
                                    qds, kds);
}

// Joint text + image attention (JointArgs): K packed and turned in
// [B,H,Nt+Ni,D], V packed there too or read from its parts.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void attn_fwd_joint_kernel(const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                           __bf16* __restrict__ Oout, float* __restrict__ LSE, int N, int n_qtiles,
                           int total_tiles, float c, Layout lay, JointArgs ja) {
  attn_fwd_body<D, false, false, false, true>(nullptr, K, V, Oout, LSE, N, N, n_qtiles, total_tiles,
                                              c, lay, nullptr, nullptr, Split{}, ja);
}

// Workgroups of a persistent launch over `total` units: one per compute unit
// of the current device (the kernel holds a compute unit's LDS), or fewer
// when there are fewer units.  The count is read once per device.
unsigned persistent_grid(int64_t total) {
  static std::atomic<int> cus[64];  // host threads may launch at once: each reads or sets its device's count
  int dev = 0;
  int n = 256;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    int c = cus[dev].load(std::memory_order_relaxed);
    if (c <= 0 &&
        hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0)
      cus[dev].store(c, std::memory_order_relaxed);
    if (c > 0) n = c;
  }
  return (unsigned)(total < n ? total : n);
}

// Query tiles of a plain launch: whole rounds of full tiles over the
// persistent grid's slots, then, when the tiles of the last partial round
// would fill at most half the slots, those tiles as half-height ones (two
// each), which then take one round of about half the time.  Full tile t
// covers half tiles 2t and 2t + 1 of its head (its second half may lie
// past the head's last row, and then it does not exist).
struct FwdSplitRounds {
  int n_full, n_half;          // query tiles per head, full / half height
  int64_t full_units;          // full tiles of the main launch
  int half_tile0, half_units;  // half tiles of the second launch
};
FwdSplitRounds fwd_rounds(int Nq, int64_t heads) {
  FwdSplitRounds r;
  r.n_full = (Nq + kBM - 1) / kBM;
  r.n_half = (Nq + kBM / 2 - 1) / (kBM / 2);
  const int64_t total = heads * r.n_full;
  const int64_t slots = persistent_grid(total);
  const int64_t rem = slots > 0 ? total % slots : 0;
  r.full_units = total;
  r.half_tile0 = r.half_units = 0;
  if (total > slots && rem > 0 && 2 * rem <= slots) {
    r.full_units = total - rem;
    const int64_t h0 = r.full_units / r.n_full, t0 = r.full_units - h0 * r.n_full;
    const int64_t g0 = h0 * r.n_half + 2 * t0;
    r.half_tile0 = (int)g0;
    r.half_units = (int)(heads * r.n_half - g0);
  }
  return r;
}

template <int D, bool OUT_F32, bool STR = false>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o, float* lse, int Nq,
                    int Nkv, float c, const Layout& lay, hipStream_t stream) {
  const int64_t heads = (int64_t)lay.B * lay.hg;
  if (heads * ((Nq + kBM / 2 - 1) / (kBM / 2)) > 0x7fffffff) return hipErrorInvalidValue;
  const FwdSplitRounds r = fwd_rounds(Nq, heads);
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, OUT_F32, kQB, STR>), dim3(persistent_grid(r.full_units)),
                     dim3(kThreads), 0, stream, static_cast<const __bf16*>(q),
                     static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), o, lse, Nq, Nkv,
                     r.n_full, (int)r.full_units, c, lay);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || r.half_units == 0) return e;
  Layout lh = lay;
  lh.tile0 = r.half_tile0;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, OUT_F32, 1, STR>), dim3(persistent_grid(r.half_units)),
                     dim3(kThreads), 0, stream, static_cast<const __bf16*>(q),
                     static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), o, lse, Nq, Nkv,
                     r.n_half, r.half_units, c, lh);
  return hipGetLastError();
}

template <bool OUT_F32, int MODE>
hipError_t launch_fp8(const void* q, const void* k, const void* v, const float* qds,
                      const float* kds, void* o, float* lse, int Nq, int Nkv, float c,
                      const Layout& lay, hipStream_t stream) {
  const int n_qtiles = (Nq + kBM - 1) / kBM;
  const int64_t total = (int64_t)lay.B * lay.hg * n_qtiles;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<OUT_F32, MODE>), dim3(persistent_grid(total)), dim3(kThreads), 0,
                     stream, static_cast<const unsigned char*>(q),
                     static_cast<const unsigned char*>(k), static_cast<const __bf16*>(v), o, lse,
                     Nq, Nkv, n_qtiles, (int)total, c, lay, qds, kds);
  return hipGetLastError();
}

template <bool OUT_F32>
hipError_t launch_layout(const void* q, const void* k, const void* v, void* o, float* lse, int Nq,
                         int Nkv, int D, float scale, const Layout& lay, hipStream_t stream) {
  const float c = scale * 1.4426950408889634f;
  switch (D) {
    case 32: return launch_d<32, OUT_F32>(q, k, v, o, lse, Nq, Nkv, c, lay, stream);
    case 64: return launch_d<64, OUT_F32>(q, k, v, o, lse, Nq, Nkv, c, lay, stream);
    default: return launch_d<128, OUT_F32>(q, k, v, o, lse, Nq, Nkv, c, lay, stream);
  }
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Nq, int Nkv, int D, float scale, bool o_f32,
                            hipStream_t stream) {
  const Layout lay{Nq, Nkv, H, H, 0, B, 0};
  return o_f32 ? launch_layout<true>(q, k, v, o, lse, Nq, Nkv, D, scale, lay, stream)
               : launch_layout<false>(q, k, v, o, lse, Nq, Nkv, D, scale, lay, stream);
}

hipError_t launch_attn_bf16_balanced(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int B, int H, int Nq, int Nkv, int D, float scale,
                                     bool o_f32, const BalancedPlan& pl, void* workspace,
                                     hipStream_t stream) {
  if (pl.nsplit <= 1)
    return launch_attn_bf16(q, k, v, o, lse, B, H, Nq, Nkv, D, scale, o_f32, stream);
  const Layout lay{Nq, Nkv, H, H, 0, B, 0};
  const float c = scale * 1.4426950408889634f;
  const int n_qtiles = (Nq + kBM - 1) / kBM;
  hipError_t e = hipSuccess;
  if (pl.whole > 0) {  // whole tiles: exact waves of the plain kernel
    auto run = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(persistent_grid(pl.whole)), dim3(kThreads), 0, stream,
                         static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                         static_cast<const __bf16*>(v), o, lse, Nq, Nkv, n_qtiles, pl.whole, c,
                         lay);
    };
    if (o_f32) {
      if (D == 32) run(attn_fwd_bf16_kernel<32, true>);
      else if (D == 64) run(attn_fwd_bf16_kernel<64, true>);
      else run(attn_fwd_bf16_kernel<128, true>);
    } else {
      if (D == 32) run(attn_fwd_bf16_kernel<32, false>);
      else if (D == 64) run(attn_fwd_bf16_kernel<64, false>);
      else run(attn_fwd_bf16_kernel<128, false>);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  float* opart = static_cast<float*>(workspace);
  float* lpart = opart + (size_t)pl.nsplit * pl.rows * D;
  const Split sp{pl.whole, pl.nsplit, pl.kc, pl.row0, pl.rows};
  auto split = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(persistent_grid(pl.units)), dim3(kThreads), 0, stream,
                       static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                       static_cast<const __bf16*>(v), opart, lpart, Nq, Nkv, n_qtiles, pl.units,
                       c, lay, sp);
  };
  if (D == 32) split(attn_fwd_bf16_split_kernel<32>);
  else if (D == 64) split(attn_fwd_bf16_split_kernel<64>);
  else split(attn_fwd_bf16_split_kernel<128>);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  char* otail = static_cast<char*>(o) + pl.row0 * D * (o_f32 ? 4 : 2);
  return launch_merge(opart, lpart, pl.nsplit, otail, lse ? lse + pl.row0 : nullptr, pl.rows, D,
                      o_f32, stream);
}

hipError_t launch_attn_joint(const void* k_packed, const void* v_packed, const JointParts& parts,
                             void* o, float* lse, int B, int H, int Nt, int Ni, int D, float scale,
                             hipStream_t stream) {
  const int N = Nt + Ni;
  const Layout lay{N, N, H, H, 0, B, 0};
  const float c = scale * 1.4426950408889634f;
  const int n_qtiles = (N + kBM - 1) / kBM;
  const int64_t total = (int64_t)B * H * n_qtiles;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  JointArgs ja{static_cast<const __bf16*>(parts.q_txt), static_cast<const __bf16*>(parts.q_img),
               v_packed ? nullptr : static_cast<const __bf16*>(parts.v_txt),
               v_packed ? nullptr : static_cast<const __bf16*>(parts.v_img),
               parts.cos_txt, parts.sin_txt, parts.cos_img, parts.sin_img, Nt, Ni, parts.Ht,
               parts.h0};
  auto run = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(persistent_grid(total)), dim3(kThreads), 0, stream,
                       static_cast<const __bf16*>(k_packed), static_cast<const __bf16*>(v_packed),
                       static_cast<__bf16*>(o), lse, N, n_qtiles, (int)total, c, lay, ja);
  };
  switch (D) {
    case 32: run(attn_fwd_joint_kernel<32>); break;
    case 64: run(attn_fwd_joint_kernel<64>); break;
    default: run(attn_fwd_joint_kernel<128>); break;
  }
  return hipGetLastError();
}

hipError_t launch_attn_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                           const float* k_descale, void* o, float* lse, int B, int H, int Nq,
                           int Nkv, float scale, bool o_f32, hipStream_t stream) {
  const Layout lay{Nq, Nkv, H, H, 0, B, 0};
  const float c = scale * 1.4426950408889634f;
  return o_f32 ? launch_fp8<true, 1>(q, k, v, q_descale, k_descale, o, lse, Nq, Nkv, c, lay, stream)
               : launch_fp8<false, 1>(q, k, v, q_descale, k_descale, o, lse, Nq, Nkv, c, lay, stream);
}

hipError_t launch_attn_fp8_mx(const void* q, const void* k, const void* v, const float* q_descale,
                              const float* k_descale, void* o, float* lse, int B, int H, int Nq,
                              int Nkv, bool o_f32, hipStream_t stream) {
  const Layout lay{Nq, Nkv, H, H, 0, B, 0};
  return o_f32 ? launch_fp8<true, 2>(q, k, v, q_descale, k_descale, o, lse, Nq, Nkv, 1.0f, lay, stream)
               : launch_fp8<false, 2>(q, k, v, q_descale, k_descale, o, lse, Nq, Nkv, 1.0f, lay, stream);
}

hipError_t launch_attn_bf16_ulysses(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int P, int r, int B, int H, int N, int D,
                                    float scale, hipStream_t stream) {
  const int ns = N / P, hg = H / P;
  const Layout lay{ns, ns, hg, H, r * hg, B, 0};
  if (ns % kBN == 0) return launch_layout<false>(q, k, v, o, lse, N, N, D, scale, lay, stream);
  // shards that end inside a key tile: the kernels that stage such tiles from two shards
  const float c = scale * 1.4426950408889634f;
  switch (D) {
    case 32: return launch_d<32, false, true>(q, k, v, o, lse, N, N, c, lay, stream);
    case 64: return launch_d<64, false, true>(q, k, v, o, lse, N, N, c, lay, stream);
    default: return launch_d<128, false, true>(q, k, v, o, lse, N, N, c, lay, stream);
  }
}

}  // namespace ditattn
