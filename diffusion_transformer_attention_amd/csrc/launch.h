// Internal launchers behind the C ABI.  Arguments arrive already validated
// by api.cpp; each returns a hipError_t from the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ditattn {

// bf16 q/k/v; o in bf16 (o_f32 == false) or float32.  lse may be null.
hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Nq, int Nkv, int D, float scale, bool o_f32,
                            hipStream_t stream);

// Tile sizes of the bf16 / fp8 forward kernels (checked in attn_bf16.hip).
constexpr int kFwdQueryTile = 256;  // query rows per workgroup
constexpr int kFwdKeyTile = 64;     // keys per LDS stage

// Work balance of one bf16 forward over `slots` concurrent workgroups: the
// first `whole` query tiles (a multiple of slots) run whole; the remaining
// tiles are cut into nsplit key chunks of kc keys (units = tiles * nsplit
// workgroups) whose float32 partials fill ws_bytes of workspace and are
// merged into flat query rows [row0, row0 + rows).  nsplit == 1: one plain
// launch, no workspace.
struct BalancedPlan {
  int whole, nsplit, kc, units;
  int64_t row0, rows;
  size_t ws_bytes;
};
BalancedPlan balanced_plan(int B, int H, int Nq, int Nkv, int D, int slots);

hipError_t launch_attn_bf16_balanced(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int B, int H, int Nq, int Nkv, int D, float scale,
                                     bool o_f32, const BalancedPlan& plan, void* workspace,
                                     hipStream_t stream);

// Device address of this device's static scratch array (DIT_SCRATCH_BYTES
// bytes, scratch.hip), looked up on the first call per device.
hipError_t scratch_buffer(void** out, size_t* bytes);

// bf16 q/k/v/o in Ulysses token-shard layout [P][B,H,N/P,D]: attention of
// head group r (heads [r*H/P, (r+1)*H/P)) over all N tokens.  lse is
// [B,H/P,N] or null.  Requires (N/P) % 64 == 0.
hipError_t launch_attn_bf16_ulysses(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int P, int r, int B, int H, int N, int D,
                                    float scale, hipStream_t stream);

// q, k: E4M3 codes [B,H,N,D] (D = 128) with per-(b, h) float32 descales;
// v bf16; o bf16 (o_f32 == false) or float32; lse may be null.
hipError_t launch_attn_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                           const float* k_descale, void* o, float* lse, int B, int H, int Nq,
                           int Nkv, float scale, bool o_f32, hipStream_t stream);

// The same with power-of-two descales, scores in base 2 (the queries' codes
// carry scale * log2(e)): see dit_attn_fwd_fp8_mx.
hipError_t launch_attn_fp8_mx(const void* q, const void* k, const void* v, const float* q_descale,
                              const float* k_descale, void* o, float* lse, int B, int H, int Nq,
                              int Nkv, bool o_f32, hipStream_t stream);

// bf16 x [B,H,N,D] -> E4M3 codes [B,H,N,D] and float32 descale [B,H] (D % 8 == 0).
hipError_t launch_quant_fp8(const void* x, void* codes, float* descale, int B, int H, int N, int D,
                            hipStream_t stream);
// The same for 1 or 2 tensors of one [B,H] head grid (token counts N[t]) in
// three launches.
hipError_t launch_quant_fp8_n(const void* const* x, void* const* codes, float* const* descale,
                              const int* N, int ntensors, int B, int H, int D, hipStream_t stream);
// q and k of one attention call with power-of-two descales, q multiplied by
// c0 = scale * log2(e) (float32) before it is scaled (dit_quant_fp8_qk_mx).
hipError_t launch_quant_fp8_mx(const void* q, const void* k, void* q_codes, void* k_codes,
                               float* q_descale, float* k_descale, int B, int H, int Nq, int Nkv,
                               int D, float c0, hipStream_t stream);

// Backward, bf16 q/k/v/o/dout (head dim 32, 64 or 128), float32 lse in,
// delta out ([B,H,Nq]), float32 dq/dk/dv.
hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, float* delta, float* dq,
                                float* dk, float* dv, int B, int H, int Nq, int Nkv, int D,
                                float scale, hipStream_t stream);

// One tensor of a joint-sequence pack: text part [B,Ht,Nt,D] (heads h0 ..
// h0+H-1 used), image part [B,H,Ni,D], output [B,H,Nt+Ni,D], all bf16.  A
// part's rotary tables ([N, D/2] float32) may be null: that part is copied.
struct RopePackTensor {
  const void* txt;
  const void* img;
  void* out;
  const float* cos_txt;
  const float* sin_txt;
  const float* cos_img;
  const float* sin_img;
};

// Joint text + image attention reading the queries (turned in the kernel)
// and, unless v_packed is given, the values from their parts; K comes packed
// and turned in [B,H,Nt+Ni,D] (v_packed likewise).  Two-part V needs Nt a
// multiple of kFwdKeyTile.
struct JointParts {
  const void* q_txt;  // [B,Ht,Nt,D], heads h0 .. h0+H-1 used
  const void* q_img;  // [B,H,Ni,D]
  const void* v_txt;
  const void* v_img;
  const float* cos_txt;
  const float* sin_txt;
  const float* cos_img;
  const float* sin_img;
  int Ht, h0;
};
hipError_t launch_attn_joint(const void* k_packed, const void* v_packed, const JointParts& parts,
                             void* o, float* lse, int B, int H, int Nt, int Ni, int D, float scale,
                             hipStream_t stream);

// Packs 1 to 3 tensors in one launch.
hipError_t launch_rope_pack(const RopePackTensor* tensors, int ntensors, int B, int H, int Ht,
                            int h0, int Nt, int Ni, int D, hipStream_t stream);

// float32 q/k/v/o.  lse may be null.
hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                           int B, int H, int Nq, int Nkv, int D, float scale, hipStream_t stream);

hipError_t launch_merge(const float* o_parts, const float* lse_parts, int nblk, void* o,
                        float* lse, int64_t rows, int D, bool o_f32, hipStream_t stream);

// head2seq == false: seq->head; true: head->seq.
hipError_t launch_permute(const void* in, void* out, int P, int B, int H, int N, int D,
                          int elem_bytes, bool head2seq, hipStream_t stream);

}  // namespace ditattn
