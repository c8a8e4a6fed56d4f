// bf16 attention backward on the CDNA4 matrix cores: dQ, dK, dV from q, k, v,
// the forward's O and LSE, and the output gradient dO.
//
// What is computed (the chain rule of the forward definition; the pages'
// "Feat: USP sequence parallelism (Ulysses x Ring)" pull request, "Ring kernel
// selection": ring kernels pair with a real backward kernel; Validation:
// dQ/dK/dV against a full-sequence reference, deterministic double runs):
//   P_ij    = exp(scale q_i.k_j - LSE_i)
//   delta_i = sum_d dO_id O_id
//   dS_ij   = P_ij (dO_i.v_j - delta_i)
//   dV_j    = sum_i P_ij dO_i
//   dK_j    = scale sum_i dS_ij q_i
//   dQ_i    = scale sum_j dS_ij k_j
// With the merged LSE and the final O of a ring, a call on one K/V block gives
// that block's dK, dV and its share of dQ.
//
// Three kernels, each writing every output element once (no atomics, so the
// results are bitwise repeatable):
//  * delta_kernel: delta = rowsum(dO * O) in float32;
//  * dkdv_kernel: a workgroup of 8 waves owns 128 keys of one (b, h), 16 per
//    wave, with its K and V rows in registers; it streams the query rows in
//    64-row LDS tiles (Q, dO, LSE, delta; four stages, loaded with
//    buffer_load ... lds) and per 32-query step computes, with
//    v_mfma_f32_16x16x32_bf16,
//      S  = Q K^T and dP = dO V^T  (A = Q / dO rows from LDS, B = K / V),
//      P, dS per element in float32,
//      dV^T += dO^T P and dK^T += Q^T dS  (A = transposing LDS reads of the
//      same tiles, B = P / dS packed to bf16 from the lane's own S layout),
//    software-pipelined so that one slot holds the first product of the
//    next step, the second of the previous one and the softmax of this one.
//    V is held negated and each dP chain starts at delta, so the chain ends
//    at delta - dP and the softmax yields -dS = p (delta - dP) with one
//    multiply (dK takes the sign back in its final scale);
//  * dq_kernel: the forward's arrangement: 8 waves x 32 query rows with Q and
//    dO in registers, K and V streamed in 64-key LDS tiles (three stages);
//    per 32-key step
//      S^T = K Q^T, dP^T = V dO^T, then dQ^T += K^T dS^T,
//    each dP^T chain starting at -delta of the lane's query, so that it ends
//    at dP - delta; software-pipelined so that the next step's products
//    overlap this step's softmax and dQ^T products.
// The tiles' 16-byte chunks are XOR-swizzled per row (swz), so that both read
// patterns, ds_read_b128 of 16 rows at one column and ds_read_b64_tr_b16 of 8
// rows x 2 chunks per 32 lanes, are bank-conflict-free (head dimension 32:
// nearly so).
// Head dimensions 32, 64 and 128; every kernel is a template on it, and a
// smaller head dimension keeps the same loops with fewer channel steps.
#include <math.h>

#include "launch.h"

namespace ditattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) float lds_f32;

constexpr int TR = 64;             // rows per LDS tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int KEYS_PER_WG = 16 * kWaves;     // dkdv_kernel
constexpr int QUERIES_PER_WG = 32 * kWaves;  // dq_kernel
constexpr float kLog2e = 1.4426950408889634f;

// Sizes that follow from the head dimension D.
template <int D_>
struct G {
  static constexpr int D = D_;
  static constexpr int ROWB = 2 * D;                          // bytes per row
  static constexpr int CPR = D / 8;                           // 16-byte chunks per row
  static constexpr int KS = D / 32;                           // 32-wide k-steps over channels
  static constexpr int DB = D / 16;                           // 16-channel blocks
  static constexpr int TILE = TR * ROWB;                      // bytes per LDS tile
  static constexpr int PIECES = TILE / 1024;                  // 1 KB load instructions per tile
  static constexpr int NLD = (PIECES + kWaves - 1) / kWaves;  // of them per wave
};

// Chunk swizzle of the LDS tiles: LDS slot pc of row r holds chunk
// pc ^ swz(r).  With D = 128 (one row per 256-byte bank sweep) and D = 64
// (two) neither the row-major fragment reads (ds_read_b128) nor the
// transposing reads (ds_read_b64_tr_b16) of tr_frag meet a bank conflict;
// the D = 128 patterns were counted on gfx950 with SQ_LDS_BANK_CONFLICT, the
// others chosen on the bank map fitted to those counts.  With D = 32 (four
// rows per sweep, four chunks) no swizzle clears every pattern; this one
// leaves the fewest.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if (D == 128) return 2 * (row & 7);
  if (D == 64) return row & 6;
  return ((row >> 1) & 2) | ((row >> 3) & 1);
}

__device__ __forceinline__ int remap_xcd(int i, int total) {
  const int x = i & 7, j = i >> 3;
  const int q = total >> 3, r = total & 7;
  return x * q + (x < r ? x : r) + j;
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Loads into LDS are counted by vmcnt: wait for them (gfx9 s_waitcnt
// encoding: vmcnt 0, expcnt 7, lgkmcnt 15) before the barrier that publishes
// the tile.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
}

// Stage rows [r0, r0 + 64) of a [rows, D] bf16 matrix into a swizzled LDS
// tile: LDS slot pc of row r holds chunk pc ^ swz(r).  The descriptor ends at
// row min(nrows, r0 + TR), so rows past the end arrive as zeros (and its
// 32-bit size stays within one tile).
// Each load instruction writes 1 KB; a tile smaller than kWaves KB leaves
// the last waves idle.
template <int D>
__device__ __forceinline__ void stage_rows(const __bf16* M, int r0, int nrows, lds_t* buf,
                                           int wave, const int* voff) {
  using g = G<D>;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(M + (int64_t)r0 * D), (short)0, min(nrows - r0, TR) * g::ROWB, 0x00020000);
#pragma unroll
  for (int n = 0; n < g::NLD; ++n) {
    const int inst = n * kWaves + wave;
    if (g::PIECES % kWaves != 0 && inst >= g::PIECES) break;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(buf + inst * 1024), 16, voff[n], 0, 0, 0);
  }
}

// Stage 64 floats (rows [r0, r0 + 64) of a row vector) into LDS, lane l -> row r0 + l.
__device__ __forceinline__ void stage_vec(const float* G, int r0, int nrows, lds_f32* buf, int lane) {
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(G + r0), (short)0, min(nrows - r0, TR) * 4, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)buf, 4,
                                           4 * lane, 0, 0, 0);
}

template <int D>
__device__ __forceinline__ void piece_offsets(int* voff, int wave, int lane) {
  using g = G<D>;
#pragma unroll
  for (int n = 0; n < g::NLD; ++n) {
    const int p = (n * kWaves + wave) * 64 + lane;
    const int row = p / g::CPR, pc = p % g::CPR;
    voff[n] = row * g::ROWB + ((pc ^ swz<D>(row)) << 4);
  }
}

// Byte offset, within a 16-row block, of the A-operand fragment of k-step ks
// for a row-major tile: lane (c16, g) reads row c16, chunk 4ks + g.
template <int D>
__device__ __forceinline__ int a_off(int c16, int g, int ks) {
  return c16 * G<D>::ROWB + (((4 * ks + g) ^ swz<D>(c16)) << 4);
}

// Transposing read base: lane t of 16-lane group g reads row r = 4g + t/4,
// channels 16db + 4(t%4) .. +3 (the second read is 16 rows further, same
// swizzle), i.e. chunk 2db + a, a = (t%4)/2.  Its in-row byte offset is
// 16((2db + a) ^ swz(r)) = 32db ^ 16a ^ 16swz(r), so the channel block only
// flips bits 5 and up of it: block db is at trb ^ (32 db).
template <int D>
__device__ __forceinline__ int tr_base(int lane) {
  const int t = lane & 15, g = lane >> 4;
  const int r = 4 * g + (t >> 2);
  const int a = (t & 3) >> 1;
  return r * G<D>::ROWB + ((16 * a) ^ (16 * swz<D>(r))) + 8 * (t & 1);
}

template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const lds_t* base) {
  const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)base));
  const bf16x4 hi = __builtin_bit_cast(
      bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 16 * G<D>::ROWB)));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---------------------------------------------------------------- delta
// One group of D/8 lanes per row: lane i holds channels 8i .. 8i+7.
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const __bf16* __restrict__ O,
                                                    const __bf16* __restrict__ dO,
                                                    float* __restrict__ delta, int64_t rows) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + (threadIdx.x / LPR);
  const int i = threadIdx.x % LPR;
  float s = 0.f;
  if (row < rows) {
    const bf16x8 o = *reinterpret_cast<const bf16x8*>(O + row * D + 8 * i);
    const bf16x8 d = *reinterpret_cast<const bf16x8*>(dO + row * D + 8 * i);
#pragma unroll
    for (int j = 0; j < 8; ++j) s = fmaf((float)o[j], (float)d[j], s);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m /= 2) s += __shfl_xor(s, m, LPR);
  if (row < rows && i == 0) delta[row] = s;
}

// ---------------------------------------------------------------- dK, dV
// Software-pipelined over 32-query steps: slot s issues the S / dP MFMAs of
// step s+1, the dV / dK MFMAs of step s-1 and the P / dS of step s, laid out
// as 16 groups fenced by scheduling barriers (as in the forward kernel), so
// one wave's vector work overlaps its own matrix work.  A step's Q / dO tile
// is read from the slot before the step (S, dP) to the slot after it (dV,
// dK): four LDS stages per tensor, tile t+2 loaded while tiles t-1 .. t+1
// are live.
constexpr int kQStages = 4;

// Per-lane LDS offsets, each plus the LDS address of its tensor's stage 0, in
// registers the compiler cannot see through: a read of stage j is that
// register plus a constant below 64 KB that the instruction encodes.  The
// reads keep their stage array as their object, so the compiler still knows
// they do not touch the stage being loaded.
template <int D>
struct KVCtx {
  static constexpr int KS = G<D>::KS, DB = G<D>::DB;
  bf16x8 k[KS], v[KS];  // B operands: lane holds key c16, channels 32ks + 8g .. +7
  f32x4 dk[DB], dv[DB]; // -dK^T, dV^T blocks: lane holds channels 16db + 4g + r of key c16
  int qa[KS], oa[KS];   // row-major fragment (ks) of the Q / dO stages
  int qt[DB], ot[DB];   // transposing fragment (db) of the Q / dO stages
  int qbase, obase;     // LDS addresses of Q stage 0 and dO stage 0
  int g, lane, wave;
  int Nq, ntiles;
  float c;
  const __bf16 *Qb, *dOb;
  const float *Lb, *Db;
  int voff[G<D>::NLD];
  // stages (separate scalars: never an indexed array); a dO stage holds the
  // tile, then the tile's 64 LSE values, then its 64 delta values
  lds_t *q0, *q1, *q2, *q3, *o0, *o1, *o2, *o3;
};

template <typename T>
__device__ __forceinline__ T pick4(T a0, T a1, T a2, T a3, int i) {
  return i == 0 ? a0 : (i == 1 ? a1 : (i == 2 ? a2 : a3));
}
// Stage of tile t + k, where PH = t % 4 when known at compile time, else -1.
__device__ __forceinline__ int stage_at(int PH, int t, int k) {
  return PH >= 0 ? (PH + k) % kQStages : (t + k) % kQStages;
}
#define QST(x, i) pick4((x).q0, (x).q1, (x).q2, (x).q3, (i))
#define OST(x, i) pick4((x).o0, (x).o1, (x).o2, (x).o3, (i))
#define LST(x, i) reinterpret_cast<lds_f32*>(OST(x, i) + G<D>::TILE)
#define DST(x, i) reinterpret_cast<lds_f32*>(OST(x, i) + G<D>::TILE + 4 * TR)

// S = Q K^T and delta - dP = delta + dO (-V)^T of one 32-query step,
// unpipelined (first step).
template <int D>
__device__ __forceinline__ void sdp_step(const KVCtx<D>& x, f32x4 (&S)[2], f32x4 (&dP)[2],
                                         const lds_t* qs, const lds_t* os, const lds_f32* dt) {
  constexpr int ROWB = G<D>::ROWB;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    S[qb] = f32x4{};
    dP[qb] = *reinterpret_cast<const lds_f32x4*>(dt + 16 * qb + 4 * x.g);
  }
#pragma unroll
  for (int ks = 0; ks < G<D>::KS; ++ks)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const bf16x8 aq = *reinterpret_cast<const lds_bf16x8*>(qs - x.qbase + 16 * qb * ROWB + x.qa[ks]);
      const bf16x8 ao = *reinterpret_cast<const lds_bf16x8*>(os - x.obase + 16 * qb * ROWB + x.oa[ks]);
      S[qb] = mfma16(aq, x.k[ks], S[qb]);
      dP[qb] = mfma16(ao, x.v[ks], dP[qb]);
    }
}

// dV^T += dO^T P and -dK^T += Q^T (-dS) of one step, unpipelined (last step).
template <int D>
__device__ __forceinline__ void dvdk_step(KVCtx<D>& x, bf16x8 pp, bf16x8 dsp, const lds_t* qs,
                                          const lds_t* os) {
#pragma unroll
  for (int db = 0; db < G<D>::DB; ++db) {
    x.dv[db] = mfma16(tr_frag<D>(os - x.obase + x.ot[db]), pp, x.dv[db]);
    x.dk[db] = mfma16(tr_frag<D>(qs - x.qbase + x.qt[db]), dsp, x.dk[db]);
  }
}

// One slot: S / delta - dP of the next step into Sn / dPn (rows at qn / on,
// delta at dtn), dV / -dK of the previous step from Pp / dSp (rows at qp /
// op), P / -dS of this step from Sc / dPc into Pc / dSc (LSE at lt, query
// index q0 of the step's row 0).  There are NG = D/8 groups, as many as S / dP
// MFMAs and as dV / dK MFMAs.  Group gi runs the S / dP MFMA gi (index i: ks =
// i / 4, qb = (i / 2) % 2, S if i is even else dP), the dV / dK MFMA gi (db =
// gi / 2, dV if gi is even else dK) and a share of this step's 8 scores e
// (qb = e / 4, r = e % 4): with 16 groups score gi / 2 in odd groups, with 8
// score gi, with 4 scores 2gi and 2gi + 1; it issues the LDS reads that
// group gi + 1 needs.  The B operands pack query 4g + j (j < 4) and
// 16 + 4g + j - 4 (j >= 4) of the step: k index 8g + j of
// v_mfma_f32_16x16x32_bf16.
template <int D, bool MASK>
__device__ __forceinline__ void dkdv_slot(KVCtx<D>& x, const f32x4 (&Sc)[2], const f32x4 (&dPc)[2],
                                          f32x4 (&Sn)[2], f32x4 (&dPn)[2], bf16x8 Pp, bf16x8 dSp,
                                          bf16x8& Pc, bf16x8& dSc, const lds_t* qn, const lds_t* on,
                                          const lds_t* qp, const lds_t* op, const lds_f32* lt,
                                          const lds_f32* dtn, int q0) {
  constexpr int ROWB = G<D>::ROWB;
  constexpr int NG = G<D>::CPR;
  constexpr int SG = NG > 8 ? NG / 8 : 1;   // groups per scoring group
  constexpr int EPG = NG < 8 ? 8 / NG : 1;  // scores per scoring group
  bf16x8 fa[NG], fc[NG];
  auto load_a = [&](int i) {
    const int ks = i / 4, qb = (i / 2) % 2;
    fa[i] = (i & 1) ? *reinterpret_cast<const lds_bf16x8*>(on - x.obase + 16 * qb * ROWB + x.oa[ks])
                    : *reinterpret_cast<const lds_bf16x8*>(qn - x.qbase + 16 * qb * ROWB + x.qa[ks]);
  };
  auto load_c = [&](int j) {
    const int db = j / 2;
    fc[j] = (j & 1) ? tr_frag<D>(qp - x.qbase + x.qt[db]) : tr_frag<D>(op - x.obase + x.ot[db]);
  };
  // LSE of this step's rows 16qb + 4g + r; the next step's dP chains start
  // at its delta.
  f32x4 lse[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    lse[qb] = *reinterpret_cast<const lds_f32x4*>(lt + 16 * qb + 4 * x.g);
    dPn[qb] = *reinterpret_cast<const lds_f32x4*>(dtn + 16 * qb + 4 * x.g);
    Sn[qb] = f32x4{};
  }
  load_a(0);
  load_c(0);
  float p[8], ds[8];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    if (gi + 1 < NG) {
      load_a(gi + 1);
      load_c(gi + 1);
    }
    {
      const int ks = gi / 4, qb = (gi / 2) % 2;
      if (gi & 1)
        dPn[qb] = mfma16(fa[gi], x.v[ks], dPn[qb]);
      else
        Sn[qb] = mfma16(fa[gi], x.k[ks], Sn[qb]);
    }
    {
      const int db = gi / 2;
      if (gi & 1)
        x.dk[db] = mfma16(fc[gi], dSp, x.dk[db]);
      else
        x.dv[db] = mfma16(fc[gi], Pp, x.dv[db]);
    }
    if (gi % SG == SG - 1) {
#pragma unroll
      for (int u = 0; u < EPG; ++u) {
        const int e = (gi / SG) * EPG + u, qb = e / 4, r = e % 4;
        float sv = Sc[qb][r];
        // Pin the element's work to its group (see the forward kernel).
        asm volatile("" : "+v"(sv));
        float pv = __builtin_amdgcn_exp2f(fmaf(sv, x.c, -lse[qb][r] * kLog2e));
        if (MASK && q0 + 16 * qb + 4 * x.g + r >= x.Nq) pv = 0.f;
        p[e] = pv;
        ds[e] = pv * dPc[qb][r];  // -dS = p (delta - dP)
        if (e & 1) {
          bf16x2 pk = {(__bf16)p[e - 1], (__bf16)p[e]};
          bf16x2 dk = {(__bf16)ds[e - 1], (__bf16)ds[e]};
          asm volatile("" : "+v"(pk), "+v"(dk));
          Pc[e - 1] = pk[0];
          Pc[e] = pk[1];
          dSc[e - 1] = dk[0];
          dSc[e] = dk[1];
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D>
__device__ __forceinline__ void stage_q_tile(const KVCtx<D>& x, int t, int st) {
  const int r0 = t * TR;
  stage_rows<D>(x.Qb, r0, x.Nq, QST(x, st), x.wave, x.voff);
  stage_rows<D>(x.dOb, r0, x.Nq, OST(x, st), x.wave, x.voff);
  if (x.wave == 0) stage_vec(x.Lb, r0, x.Nq, LST(x, st), x.lane);
  if (x.wave == 1) stage_vec(x.Db, r0, x.Nq, DST(x, st), x.lane);
}

// Query tile t = steps 2t and 2t+1.  On entry S0 / dP0 hold step 2t and
// Pa / dSa hold step 2t-1; on exit S0 / dP0 hold step 2t+2 (past the last
// tile: unused) and Pa / dSa hold step 2t+1.
template <int D, int PH, bool MASK>
__device__ __forceinline__ void dkdv_tile(KVCtx<D>& x, int t, f32x4 (&S0)[2], f32x4 (&dP0)[2],
                                          f32x4 (&S1)[2], f32x4 (&dP1)[2], bf16x8& Pa, bf16x8& dSa,
                                          bf16x8& Pb, bf16x8& dSb) {
  constexpr int ROWB = G<D>::ROWB;
  tile_barrier();  // tile t+1 landed; every wave is done with tile t-2
  const int sc = stage_at(PH, t, 0), sn = stage_at(PH, t, 1), sp = stage_at(PH, t, 3);
  if (t + 2 < x.ntiles) stage_q_tile<D>(x, t + 2, stage_at(PH, t, 2));
  const lds_t* qc = QST(x, sc);
  const lds_t* oc = OST(x, sc);
  const lds_f32* lt = LST(x, sc);
  const lds_f32* dt = DST(x, sc);
  dkdv_slot<D, MASK>(x, S0, dP0, S1, dP1, Pa, dSa, Pb, dSb, qc + 32 * ROWB, oc + 32 * ROWB,
                     QST(x, sp) + 32 * ROWB, OST(x, sp) + 32 * ROWB, lt, dt + 32, t * TR);
  dkdv_slot<D, MASK>(x, S1, dP1, S0, dP0, Pb, dSb, Pa, dSa, QST(x, sn), OST(x, sn), qc, oc, lt + 32,
                     DST(x, sn), t * TR + 32);
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dkdv_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                 const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                 const float* __restrict__ LSE, const float* __restrict__ Dl,
                 float* __restrict__ dK, float* __restrict__ dV, int Nq, int Nkv, int n_ktiles,
                 int total, float c, float scale) {
  constexpr int TILE = G<D>::TILE, ROWB = G<D>::ROWB, KS = G<D>::KS, DB = G<D>::DB;
  __shared__ __attribute__((aligned(1024))) char q0s[TILE];
  __shared__ __attribute__((aligned(1024))) char q1s[TILE];
  __shared__ __attribute__((aligned(1024))) char q2s[TILE];
  __shared__ __attribute__((aligned(1024))) char q3s[TILE];
  // One LDS object per stage and tensor: the compiler tells apart at most
  // eight objects written by buffer_load ... lds when it decides which
  // reads must wait for them.
  __shared__ __attribute__((aligned(1024))) char o0s[TILE + 8 * TR];
  __shared__ __attribute__((aligned(1024))) char o1s[TILE + 8 * TR];
  __shared__ __attribute__((aligned(1024))) char o2s[TILE + 8 * TR];
  __shared__ __attribute__((aligned(1024))) char o3s[TILE + 8 * TR];

  const int tile = remap_xcd(blockIdx.x, total);
  const int bh = tile / n_ktiles;
  const int kt = tile - bh * n_ktiles;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, g = lane >> 4;

  KVCtx<D> x;
  x.g = g;
  x.lane = lane;
  x.wave = wave;
  x.Nq = Nq;
  x.ntiles = (Nq + TR - 1) / TR;
  x.c = c;
  x.Qb = Q + (int64_t)bh * Nq * D;
  x.dOb = dO + (int64_t)bh * Nq * D;
  x.Lb = LSE + (int64_t)bh * Nq;
  x.Db = Dl + (int64_t)bh * Nq;
  x.q0 = (lds_t*)q0s; x.q1 = (lds_t*)q1s; x.q2 = (lds_t*)q2s; x.q3 = (lds_t*)q3s;
  x.o0 = (lds_t*)o0s; x.o1 = (lds_t*)o1s; x.o2 = (lds_t*)o2s; x.o3 = (lds_t*)o3s;
  x.qbase = (int)(size_t)x.q0;
  x.obase = (int)(size_t)x.o0;
  const int key = kt * KEYS_PER_WG + wave * 16 + c16;
  const int krow = min(key, Nkv - 1);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    x.k[ks] = *reinterpret_cast<const bf16x8*>(K + ((int64_t)bh * Nkv + krow) * D + 32 * ks + 8 * g);
    // -V: the dP chains then hold delta - dP, and the softmax yields -dS.
    x.v[ks] = __builtin_bit_cast(
        bf16x8, __builtin_bit_cast(u32x4, *reinterpret_cast<const bf16x8*>(
                                              V + ((int64_t)bh * Nkv + krow) * D + 32 * ks + 8 * g)) ^
                    u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u});
    x.qa[ks] = a_off<D>(c16, g, ks) + x.qbase;
    x.oa[ks] = a_off<D>(c16, g, ks) + x.obase;
    asm volatile("" : "+v"(x.qa[ks]), "+v"(x.oa[ks]));
  }
  const int trb = tr_base<D>(lane);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    x.dk[db] = f32x4{};
    x.dv[db] = f32x4{};
    x.qt[db] = (trb ^ (32 * db)) + x.qbase;
    x.ot[db] = (trb ^ (32 * db)) + x.obase;
    asm volatile("" : "+v"(x.qt[db]), "+v"(x.ot[db]));
  }
  piece_offsets<D>(x.voff, wave, lane);

  // The first slot multiplies P = dS = 0 by the stage of tile -1 (stage 3):
  // zero it so no stale Inf/NaN bit pattern can turn 0 * x into NaN.
  for (int i = threadIdx.x; i < TILE / 16; i += kThreads) {
    reinterpret_cast<lds_f32x4*>(x.q3)[i] = f32x4{};
    reinterpret_cast<lds_f32x4*>(x.o3)[i] = f32x4{};
  }
  stage_q_tile<D>(x, 0, 0);
  if (x.ntiles > 1) stage_q_tile<D>(x, 1, 1);
  tile_barrier();  // tiles 0 and 1 landed, stage 3 zeroed
  f32x4 S0[2], dP0[2], S1[2], dP1[2];
  bf16x8 Pa = bf16x8{}, dSa = bf16x8{}, Pb, dSb;
  sdp_step(x, S0, dP0, x.q0, x.o0, DST(x, 0));
  const bool partial = (Nq % TR) != 0;
  const int nfull = partial ? x.ntiles - 1 : x.ntiles;
  int t = 0;
  for (; t + kQStages <= nfull; t += kQStages) {
    dkdv_tile<D, 0, false>(x, t, S0, dP0, S1, dP1, Pa, dSa, Pb, dSb);
    dkdv_tile<D, 1, false>(x, t + 1, S0, dP0, S1, dP1, Pa, dSa, Pb, dSb);
    dkdv_tile<D, 2, false>(x, t + 2, S0, dP0, S1, dP1, Pa, dSa, Pb, dSb);
    dkdv_tile<D, 3, false>(x, t + 3, S0, dP0, S1, dP1, Pa, dSa, Pb, dSb);
  }
  for (; t < nfull; ++t) dkdv_tile<D, -1, false>(x, t, S0, dP0, S1, dP1, Pa, dSa, Pb, dSb);
  if (partial) dkdv_tile<D, -1, true>(x, t, S0, dP0, S1, dP1, Pa, dSa, Pb, dSb);
  // dV / dK of the last step (rows 32 .. 63 of the last tile).
  const int sl = (x.ntiles - 1) % kQStages;
  dvdk_step<D>(x, Pa, dSa, QST(x, sl) + 32 * ROWB, OST(x, sl) + 32 * ROWB);

  if (key < Nkv) {
    const int64_t base = ((int64_t)bh * Nkv + key) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      *reinterpret_cast<f32x4*>(dK + base + 16 * db + 4 * g) = x.dk[db] * -scale;  // of -dS
      *reinterpret_cast<f32x4*>(dV + base + 16 * db + 4 * g) = x.dv[db];
    }
  }
}

// ---------------------------------------------------------------- dQ
// Software-pipelined over 32-key steps in a register budget that holds only
// half of a second S^T / dP^T set: slot s runs, in its first half, the P / dS
// of step s (all 16 scores of the lane) beside the S^T / dP^T MFMAs of step
// s+1 for key block 0, and in its second half the dQ^T MFMAs of step s beside
// those of step s+1 for key block 1.  The S^T / dP^T of step s die during the
// first half, as the second block of step s+1 starts.  A K tile is read from
// the slot before its first step (S^T) to the slot of its last (dQ^T), a V
// tile only in the two slots before its steps: three stages each, tile t+2
// loaded while t and t+1 are read.
template <int D>
struct QCtx {
  static constexpr int KS = G<D>::KS, DB = G<D>::DB;
  bf16x8 q[2][KS], o[2][KS];  // B operands: lane holds query c16 of block qb, channels 32ks + 8g ..
  f32x4 dq[2][DB];            // dQ^T blocks: lane holds channels 16db + 4g + r of its query
  float lse2[2];
  f32x4 ndel[2];              // -delta of the lane's query, in every element: the start of each dP^T chain
  int ka[KS], va[KS];         // row-major fragment (ks) of the K / V stages, + kbase / vbase (opaque)
  int kt[DB];                 // transposing fragment (db) of the K stages, + kbase (opaque)
  int kbase, vbase;           // LDS addresses of the K and V stage 0
  int g, lane, wave, Nkv, ntiles;
  float c;
  const __bf16 *Kb, *Vb;
  int voff[G<D>::NLD];
  lds_t *k0, *k1, *k2, *v0, *v1, *v2;  // stages (separate scalars: never an indexed array)
};

// Stage of tile t + k, where PH = t % 3 when known at compile time, else -1.
__device__ __forceinline__ int kv_stage_at(int PH, int t, int k) { return PH >= 0 ? (PH + k) % 3 : (t + k) % 3; }
#define KQST(x, i) pick3((x).k0, (x).k1, (x).k2, (i))
#define VQST(x, i) pick3((x).v0, (x).v1, (x).v2, (i))
template <typename T>
__device__ __forceinline__ T pick3(T a0, T a1, T a2, int i) { return i == 0 ? a0 : (i == 1 ? a1 : a2); }

// S^T and dP^T of one 32-key step, unpipelined (first step): keys at rows
// [0, 32) of kst / vst.
template <int D>
__device__ __forceinline__ void sdpt_step(const QCtx<D>& x, f32x4 (&S)[2][2], f32x4 (&dP)[2][2],
                                          const lds_t* kst, const lds_t* vst) {
  constexpr int ROWB = G<D>::ROWB;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      S[kb][qb] = f32x4{};
      dP[kb][qb] = x.ndel[qb];
    }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < G<D>::KS; ++ks) {
      const bf16x8 ak = *reinterpret_cast<const lds_bf16x8*>(kst - x.kbase + 16 * kb * ROWB + x.ka[ks]);
      const bf16x8 av = *reinterpret_cast<const lds_bf16x8*>(vst - x.vbase + 16 * kb * ROWB + x.va[ks]);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        S[kb][qb] = mfma16(ak, x.q[qb][ks], S[kb][qb]);
        dP[kb][qb] = mfma16(av, x.o[qb][ks], dP[kb][qb]);
      }
    }
}

// One slot.  Sc / dPc: S^T, dP^T - delta of this step (keys key0 ..
// key0 + 31, rows [0, 32) of kc); Sn / dPn: those of the next step (rows
// [0, 32) of kn / vn).  NG = D/8 groups, NH = NG/2 = DB per half.  Group
// gi < NH: S^T / dP^T MFMAs 2gi, 2gi + 1 of the next step's key block 0 and
// this step's scores 16gi/NH .. 16(gi+1)/NH - 1; group gi >= NH: those MFMAs
// for key block 1 and dQ^T MFMAs 2(gi - NH), 2(gi - NH) + 1.  MFMA index i of
// a block: ks = i / 4, dP^T if (i / 2) is odd, qb = i % 2; score e: qb = e /
// 8, kb = (e / 4) % 2, r = e % 4; dQ^T MFMA j: db = j / 2, qb = j % 2.
template <int D, bool MASK>
__device__ __forceinline__ void dq_slot(QCtx<D>& x, const f32x4 (&Sc)[2][2], const f32x4 (&dPc)[2][2],
                                        f32x4 (&Sn)[2][2], f32x4 (&dPn)[2][2], const lds_t* kc,
                                        const lds_t* kn, const lds_t* vn, int key0) {
  constexpr int ROWB = G<D>::ROWB, DB = G<D>::DB;
  constexpr int NG = G<D>::CPR, NH = NG / 2, EPG = 16 / NH;
  bf16x8 fa[NG], fc[DB];
  auto load_a = [&](int gi) {  // fragment used by the two MFMAs of group gi
    const int kb = gi / NH, i = 2 * (gi % NH), ks = i / 4;
    fa[gi] = ((i / 2) & 1)
                 ? *reinterpret_cast<const lds_bf16x8*>(vn - x.vbase + 16 * kb * ROWB + x.va[ks])
                 : *reinterpret_cast<const lds_bf16x8*>(kn - x.kbase + 16 * kb * ROWB + x.ka[ks]);
  };
  auto load_c = [&](int db) { fc[db] = tr_frag<D>(kc - x.kbase + x.kt[db]); };
  bf16x8 dsp[2];
  float ds[16];
  load_a(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    if (gi + 1 < NG) load_a(gi + 1);
    if (gi >= NH - 1 && gi - (NH - 1) < DB) load_c(gi - (NH - 1));  // used one group later
    {
      const int kb = gi / NH, i0 = 2 * (gi % NH);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u, ks = i / 4, qb = i % 2;
        if ((i / 2) & 1)
          dPn[kb][qb] = mfma16(fa[gi], x.o[qb][ks], ks ? dPn[kb][qb] : x.ndel[qb]);
        else
          Sn[kb][qb] = mfma16(fa[gi], x.q[qb][ks], ks ? Sn[kb][qb] : f32x4{});
      }
    }
    if (gi < NH) {
#pragma unroll
      for (int u = 0; u < EPG; ++u) {
        const int e = EPG * gi + u, qb = e / 8, kb = (e / 4) % 2, r = e % 4;
        float sv = Sc[kb][qb][r];
        asm volatile("" : "+v"(sv));
        float p = __builtin_amdgcn_exp2f(fmaf(sv, x.c, -x.lse2[qb]));
        if (MASK && key0 + 16 * kb + 4 * x.g + r >= x.Nkv) p = 0.f;
        ds[e] = p * dPc[kb][qb][r];
        if (e & 1) {
          bf16x2 pk = {(__bf16)ds[e - 1], (__bf16)ds[e]};
          asm volatile("" : "+v"(pk));
          dsp[qb][4 * kb + r - 1] = pk[0];
          dsp[qb][4 * kb + r] = pk[1];
        }
      }
    } else {
      // dQ^T += K^T dS^T; k index 8g + j <-> key 4g + j (j < 4), 16 + 4g + j - 4 (j >= 4).
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = 2 * (gi - NH) + u, db = j / 2, qb = j % 2;
        x.dq[qb][db] = mfma16(fc[db], dsp[qb], x.dq[qb][db]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D>
__device__ __forceinline__ void stage_kv_tile(const QCtx<D>& x, int t, int st) {
  stage_rows<D>(x.Kb, t * TR, x.Nkv, KQST(x, st), x.wave, x.voff);
  stage_rows<D>(x.Vb, t * TR, x.Nkv, VQST(x, st), x.wave, x.voff);
}

// Key tile t = steps 2t and 2t+1.  On entry S0 / dP0 hold step 2t; on exit
// they hold step 2t+2 (past the last tile: unused).
template <int D, int PH, bool MASK>
__device__ __forceinline__ void dq_tile(QCtx<D>& x, int t, f32x4 (&S0)[2][2], f32x4 (&dP0)[2][2],
                                        f32x4 (&S1)[2][2], f32x4 (&dP1)[2][2]) {
  constexpr int ROWB = G<D>::ROWB;
  tile_barrier();  // tile t+1 landed; every wave is done with tile t-1
  const int sc = kv_stage_at(PH, t, 0), sn = kv_stage_at(PH, t, 1);
  if (t + 2 < x.ntiles) stage_kv_tile<D>(x, t + 2, kv_stage_at(PH, t, 2));
  const lds_t* kc = KQST(x, sc);
  const lds_t* vc = VQST(x, sc);
  dq_slot<D, MASK>(x, S0, dP0, S1, dP1, kc, kc + 32 * ROWB, vc + 32 * ROWB, t * TR);
  dq_slot<D, MASK>(x, S1, dP1, S0, dP0, kc + 32 * ROWB, KQST(x, sn), VQST(x, sn), t * TR + 32);
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
               const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
               const float* __restrict__ LSE, const float* __restrict__ Dl,
               float* __restrict__ dQ, int Nq, int Nkv, int n_qtiles, int total, float c,
               float scale) {
  constexpr int TILE = G<D>::TILE, KS = G<D>::KS, DB = G<D>::DB;
  __shared__ __attribute__((aligned(1024))) char k0s[TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[TILE];
  __shared__ __attribute__((aligned(1024))) char k2s[TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[TILE];
  __shared__ __attribute__((aligned(1024))) char v2s[TILE];

  const int tile = remap_xcd(blockIdx.x, total);
  const int bh = tile / n_qtiles;
  const int qt = tile - bh * n_qtiles;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, g = lane >> 4;

  QCtx<D> x;
  x.g = g;
  x.lane = lane;
  x.wave = wave;
  x.Nkv = Nkv;
  x.ntiles = (Nkv + TR - 1) / TR;
  x.c = c;
  x.Kb = K + (int64_t)bh * Nkv * D;
  x.Vb = V + (int64_t)bh * Nkv * D;
  x.k0 = (lds_t*)k0s; x.k1 = (lds_t*)k1s; x.k2 = (lds_t*)k2s;
  x.v0 = (lds_t*)v0s; x.v1 = (lds_t*)v1s; x.v2 = (lds_t*)v2s;
  x.kbase = (int)(size_t)x.k0;
  x.vbase = (int)(size_t)x.v0;
  const int qrow0 = qt * QUERIES_PER_WG + wave * 32 + c16;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = min(qrow0 + 16 * qb, Nq - 1);
    const int64_t rb = ((int64_t)bh * Nq + row) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      x.q[qb][ks] = *reinterpret_cast<const bf16x8*>(Q + rb + 32 * ks + 8 * g);
      x.o[qb][ks] = *reinterpret_cast<const bf16x8*>(dO + rb + 32 * ks + 8 * g);
    }
    x.lse2[qb] = LSE[(int64_t)bh * Nq + row] * kLog2e;
    const float d = -Dl[(int64_t)bh * Nq + row];
    x.ndel[qb] = f32x4{d, d, d, d};
#pragma unroll
    for (int db = 0; db < DB; ++db) x.dq[qb][db] = f32x4{};
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    x.ka[ks] = a_off<D>(c16, g, ks) + x.kbase;
    x.va[ks] = a_off<D>(c16, g, ks) + x.vbase;
    asm volatile("" : "+v"(x.ka[ks]), "+v"(x.va[ks]));
  }
  const int trb = tr_base<D>(lane);
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    x.kt[db] = (trb ^ (32 * db)) + x.kbase;
    asm volatile("" : "+v"(x.kt[db]));
  }
  piece_offsets<D>(x.voff, wave, lane);

  stage_kv_tile<D>(x, 0, 0);
  if (x.ntiles > 1) stage_kv_tile<D>(x, 1, 1);
  tile_barrier();  // tiles 0 and 1 landed
  f32x4 S0[2][2], dP0[2][2], S1[2][2], dP1[2][2];
  sdpt_step<D>(x, S0, dP0, x.k0, x.v0);
  const bool partial = (Nkv % TR) != 0;
  const int nfull = partial ? x.ntiles - 1 : x.ntiles;
  int t = 0;
  for (; t + 3 <= nfull; t += 3) {
    dq_tile<D, 0, false>(x, t, S0, dP0, S1, dP1);
    dq_tile<D, 1, false>(x, t + 1, S0, dP0, S1, dP1);
    dq_tile<D, 2, false>(x, t + 2, S0, dP0, S1, dP1);
  }
  for (; t < nfull; ++t) dq_tile<D, -1, false>(x, t, S0, dP0, S1, dP1);
  if (partial) dq_tile<D, -1, true>(x, t, S0, dP0, S1, dP1);

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qrow0 + 16 * qb;
    if (row < Nq) {
      const int64_t base = ((int64_t)bh * Nq + row) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(dQ + base + 16 * db + 4 * g) = x.dq[qb][db] * scale;
    }
  }
}

}  // namespace

namespace {
template <int D>
hipError_t launch_bwd_d(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, float* delta, float* dq, float* dk,
                        float* dv, int B, int H, int Nq, int Nkv, float scale, hipStream_t stream) {
  const int64_t rows = (int64_t)B * H * Nq;
  constexpr int kRowsPerBlock = 256 / (D / 8);  // delta_kernel
  const int64_t dgrid = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int n_ktiles = (Nkv + KEYS_PER_WG - 1) / KEYS_PER_WG;
  const int n_qtiles = (Nq + QUERIES_PER_WG - 1) / QUERIES_PER_WG;
  const int64_t kv_total = (int64_t)B * H * n_ktiles, q_total = (int64_t)B * H * n_qtiles;
  if (dgrid > 0x7fffffff || kv_total > 0x7fffffff || q_total > 0x7fffffff)
    return hipErrorInvalidValue;
  const float c = scale * kLog2e;
  const __bf16* Qp = static_cast<const __bf16*>(q);
  const __bf16* Kp = static_cast<const __bf16*>(k);
  const __bf16* Vp = static_cast<const __bf16*>(v);
  const __bf16* Op = static_cast<const __bf16*>(o);
  const __bf16* dOp = static_cast<const __bf16*>(dout);
  hipLaunchKernelGGL(delta_kernel<D>, dim3((unsigned)dgrid), dim3(256), 0, stream, Op, dOp, delta,
                     rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dkdv_kernel<D>, dim3((unsigned)kv_total), dim3(kThreads), 0, stream, Qp, Kp, Vp,
                     dOp, lse, (const float*)delta, dk, dv, Nq, Nkv, n_ktiles, (int)kv_total, c,
                     scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dq_kernel<D>, dim3((unsigned)q_total), dim3(kThreads), 0, stream, Qp, Kp, Vp, dOp,
                     lse, (const float*)delta, dq, Nq, Nkv, n_qtiles, (int)q_total, c, scale);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, float* delta, float* dq,
                                float* dk, float* dv, int B, int H, int Nq, int Nkv, int D,
                                float scale, hipStream_t stream) {
  switch (D) {
    case 32:
      return launch_bwd_d<32>(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, Nq, Nkv, scale, stream);
    case 64:
      return launch_bwd_d<64>(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, Nq, Nkv, scale, stream);
    case 128:
      return launch_bwd_d<128>(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, Nq, Nkv, scale,
                               stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace ditattn
