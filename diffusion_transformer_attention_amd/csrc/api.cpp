// C ABI of libditattn.so: host-side argument validation, then the launch.
// Every check runs before any HIP call, so an argument error never touches
// the device.  Declarations and argument meaning: include/dit_attn.h.
#include "../../include/dit_attn.h"

#include <math.h>
#include <stdint.h>

#include "launch.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_head_dim(int D) { return D == 32 || D == 64 || D == 128; }

// B*H*N*D must stay well inside int64 (and the kernels' 64-bit offsets).
bool size_ok(int64_t a, int64_t b, int64_t c, int64_t d) {
  const int64_t lim = (int64_t)1 << 46;
  int64_t x = a;
  for (int64_t y : {b, c, d}) {
    if (y != 0 && x > lim / y) return false;
    x *= y;
  }
  return true;
}

int map_launch(hipError_t e) { return e == hipSuccess ? DIT_OK : DIT_ELAUNCH; }

// Sizes of a balanced forward (bf16 inputs); DIT_OK with *work false when
// there is nothing to compute.
int balanced_check(int B, int H, int Nq, int Nkv, int D, float scale, int o_dtype, int slots,
                   bool* work) {
  *work = false;
  if (B < 0 || H < 0 || Nq < 0 || Nkv < 0 || D <= 0 || slots < 0) return DIT_EINVAL;
  if (!(isfinite(scale) && scale > 0.0f)) return DIT_EINVAL;
  if (o_dtype != DIT_BF16 && o_dtype != DIT_F32) return DIT_EUNSUPPORTED;
  if (!supported_head_dim(D)) return DIT_EUNSUPPORTED;
  if (!size_ok(B, H, Nq, D) || !size_ok(B, H, Nkv, D)) return DIT_ERANGE;
  if (B == 0 || H == 0 || Nq == 0) return DIT_OK;
  if (Nkv == 0) return DIT_EINVAL;
  *work = true;
  return DIT_OK;
}

// Concurrent workgroups of the forward kernel: one per compute unit.
int device_slots(int slots, int* out) {
  if (slots > 0) {
    *out = slots;
    return DIT_OK;
  }
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return DIT_ELAUNCH;
  *out = n;
  return DIT_OK;
}

int attn_common(const void* q, const void* k, const void* v, void* o, float* lse, bool lse_required,
                int B, int H, int Nq, int Nkv, int D, float scale, int in_dtype, int o_dtype,
                void* stream) {
  if (B < 0 || H < 0 || Nq < 0 || Nkv < 0 || D <= 0) return DIT_EINVAL;
  if (!(isfinite(scale) && scale > 0.0f)) return DIT_EINVAL;
  if (in_dtype != DIT_BF16 && in_dtype != DIT_F32) return DIT_EUNSUPPORTED;
  if (o_dtype != DIT_BF16 && o_dtype != DIT_F32) return DIT_EUNSUPPORTED;
  if (in_dtype == DIT_F32 && o_dtype != DIT_F32) return DIT_EUNSUPPORTED;
  if (!supported_head_dim(D)) return DIT_EUNSUPPORTED;
  if (!size_ok(B, H, Nq, D) || !size_ok(B, H, Nkv, D)) return DIT_ERANGE;
  if (B == 0 || H == 0 || Nq == 0) return DIT_OK;
  if (Nkv == 0) return DIT_EINVAL;  // softmax over an empty key set is undefined
  if (!q || !k || !v || !o || (lse_required && !lse)) return DIT_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return DIT_EALIGN;
  if (lse && !aligned(lse, 4)) return DIT_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (in_dtype == DIT_BF16)
    return map_launch(ditattn::launch_attn_bf16(q, k, v, o, lse, B, H, Nq, Nkv, D, scale,
                                                o_dtype == DIT_F32, s));
  return map_launch(ditattn::launch_attn_f32(static_cast<const float*>(q),
                                             static_cast<const float*>(k),
                                             static_cast<const float*>(v),
                                             static_cast<float*>(o), lse, B, H, Nq, Nkv, D,
                                             scale, s));
}

int permute_common(const void* in, void* out, int P, int B, int H, int N, int D, int elem_bytes,
                   bool head2seq, void* stream) {
  if (P < 1 || B < 0 || H < 0 || N < 0 || D < 0) return DIT_EINVAL;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
    return DIT_EUNSUPPORTED;
  if (H % P != 0 || N % P != 0) return DIT_EINVAL;
  if (!size_ok(B, H, N, (int64_t)D * elem_bytes)) return DIT_ERANGE;
  if (B == 0 || H == 0 || N == 0 || D == 0) return DIT_OK;
  if (!in || !out) return DIT_EINVAL;
  if (!aligned(in, elem_bytes) || !aligned(out, elem_bytes)) return DIT_EALIGN;
  return map_launch(ditattn::launch_permute(in, out, P, B, H, N, D, elem_bytes, head2seq,
                                            static_cast<hipStream_t>(stream)));
}

// Sizes and table pairs shared by the joint-sequence calls.
int joint_check(int B, int H, int Ht, int h0, int Nt, int Ni, int D) {
  if (B < 0 || H < 0 || Nt < 0 || Ni < 0 || D <= 0) return DIT_EINVAL;
  if (Nt > 0 && (h0 < 0 || Ht < 1 || H > Ht || h0 > Ht - H)) return DIT_EINVAL;
  if (!supported_head_dim(D)) return DIT_EUNSUPPORTED;
  const int64_t N = (int64_t)Nt + Ni;
  if (N > 0x7fffffff || !size_ok(B, H, N, 3 * (int64_t)D) || !size_ok(B, Ht, Nt, D))
    return DIT_ERANGE;
  return DIT_OK;
}

int tables_check(const float* c, const float* s) {
  if ((c == nullptr) != (s == nullptr)) return DIT_EINVAL;
  if (c && (!aligned(c, 16) || !aligned(s, 16))) return DIT_EALIGN;
  return DIT_OK;
}

// Pointers of one packed tensor: each part present when its length is.
int part_check(const void* txt, const void* img, int Nt, int Ni) {
  if ((Nt > 0 && !txt) || (Ni > 0 && !img)) return DIT_EINVAL;
  if ((Nt > 0 && !aligned(txt, 16)) || (Ni > 0 && !aligned(img, 16))) return DIT_EALIGN;
  return DIT_OK;
}

}  // namespace

extern "C" {

int dit_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int D, float scale, int dtype, void* stream) {
  return attn_common(q, k, v, o, lse, false, B, H, N, N, D, scale, dtype, dtype, stream);
}

int dit_attn_fwd_block(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int Nq, int Nkv, int D, float scale, int in_dtype, int o_dtype,
                       void* stream) {
  return attn_common(q, k, v, o, lse, true, B, H, Nq, Nkv, D, scale, in_dtype, o_dtype, stream);
}

int dit_attn_fwd_balanced_workspace(int B, int H, int Nq, int Nkv, int D, int slots,
                                    size_t* bytes) {
  if (!bytes) return DIT_EINVAL;
  *bytes = 0;
  bool work = false;
  int rc = balanced_check(B, H, Nq, Nkv, D, 1.0f, DIT_BF16, slots, &work);
  if (rc != DIT_OK || !work) return rc;
  int n = 0;
  if ((rc = device_slots(slots, &n)) != DIT_OK) return rc;
  *bytes = ditattn::balanced_plan(B, H, Nq, Nkv, D, n).ws_bytes;
  return DIT_OK;
}

int dit_attn_fwd_balanced(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                          int H, int Nq, int Nkv, int D, float scale, int o_dtype, int slots,
                          void* workspace, size_t workspace_bytes, void* stream) {
  bool work = false;
  int rc = balanced_check(B, H, Nq, Nkv, D, scale, o_dtype, slots, &work);
  if (rc != DIT_OK || !work) return rc;
  if (!q || !k || !v || !o) return DIT_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return DIT_EALIGN;
  if (lse && !aligned(lse, 4)) return DIT_EALIGN;
  if (workspace && !aligned(workspace, 16)) return DIT_EALIGN;
  int n = 0;
  if ((rc = device_slots(slots, &n)) != DIT_OK) return rc;
  const ditattn::BalancedPlan plan = ditattn::balanced_plan(B, H, Nq, Nkv, D, n);
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes)) return DIT_EINVAL;
  return map_launch(ditattn::launch_attn_bf16_balanced(q, k, v, o, lse, B, H, Nq, Nkv, D, scale,
                                                       o_dtype == DIT_F32, plan, workspace,
                                                       static_cast<hipStream_t>(stream)));
}

int dit_attn_fwd_balanced_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int B, int H, int Nq, int Nkv, int D, float scale, int o_dtype,
                                  int slots, void* stream) {
  bool work = false;
  int rc = balanced_check(B, H, Nq, Nkv, D, scale, o_dtype, slots, &work);
  if (rc != DIT_OK || !work) return rc;
  if (!q || !k || !v || !o) return DIT_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return DIT_EALIGN;
  if (lse && !aligned(lse, 4)) return DIT_EALIGN;
  int n = 0;
  if ((rc = device_slots(slots, &n)) != DIT_OK) return rc;
  const ditattn::BalancedPlan plan = ditattn::balanced_plan(B, H, Nq, Nkv, D, n);
  if (plan.ws_bytes > DIT_SCRATCH_BYTES) return DIT_ESCRATCH;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (plan.ws_bytes > 0) {
    if (ditattn::scratch_buffer(&ws, &ws_bytes) != hipSuccess) return DIT_ELAUNCH;
    if (ws_bytes < plan.ws_bytes) return DIT_ESCRATCH;
  }
  return map_launch(ditattn::launch_attn_bf16_balanced(q, k, v, o, lse, B, H, Nq, Nkv, D, scale,
                                                       o_dtype == DIT_F32, plan, ws,
                                                       static_cast<hipStream_t>(stream)));
}

int dit_attn_merge(const float* o_parts, const float* lse_parts, int nblk, void* o, float* lse,
                   int B, int H, int N, int D, int o_dtype, void* stream) {
  if (nblk < 1 || B < 0 || H < 0 || N < 0 || D <= 0) return DIT_EINVAL;
  if (o_dtype != DIT_BF16 && o_dtype != DIT_F32) return DIT_EUNSUPPORTED;
  if (!supported_head_dim(D)) return DIT_EUNSUPPORTED;
  if (!size_ok((int64_t)nblk * B, H, N, D)) return DIT_ERANGE;
  if (B == 0 || H == 0 || N == 0) return DIT_OK;
  if (!o_parts || !lse_parts || !o) return DIT_EINVAL;
  if (!aligned(o_parts, 16) || !aligned(o, 16)) return DIT_EALIGN;
  if (!aligned(lse_parts, 4) || (lse && !aligned(lse, 4))) return DIT_EALIGN;
  return map_launch(ditattn::launch_merge(o_parts, lse_parts, nblk, o, lse,
                                          (int64_t)B * H * N, D, o_dtype == DIT_F32,
                                          static_cast<hipStream_t>(stream)));
}

int dit_attn_fwd_ulysses(const void* q, const void* k, const void* v, void* o, float* lse, int P,
                         int r, int B, int H, int N, int D, float scale, int dtype, void* stream) {
  if (P < 1 || r < 0 || r >= P || B < 0 || H < 0 || N < 0 || D <= 0) return DIT_EINVAL;
  if (!(isfinite(scale) && scale > 0.0f)) return DIT_EINVAL;
  if (H % P != 0 || N % P != 0) return DIT_EINVAL;
  if (dtype != DIT_BF16) return DIT_EUNSUPPORTED;
  if (!supported_head_dim(D)) return DIT_EUNSUPPORTED;
  if ((N / P) % 64 != 0) {  // key tiles that span two shards (never three) ...
    if (N / P < 64) return DIT_EUNSUPPORTED;
    // ... reached through 32-bit offsets from one shard into the next
    if (((int64_t)B * H - 1) * (N / P) * D * 2 + 64 * D * 2 >= ((int64_t)1 << 31))
      return DIT_EUNSUPPORTED;
  }
  if (!size_ok(B, H, N, D)) return DIT_ERANGE;
  if (B == 0 || H == 0 || N == 0) return DIT_OK;
  if (!q || !k || !v || !o) return DIT_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return DIT_EALIGN;
  if (lse && !aligned(lse, 4)) return DIT_EALIGN;
  return map_launch(ditattn::launch_attn_bf16_ulysses(q, k, v, o, lse, P, r, B, H, N, D, scale,
                                                      static_cast<hipStream_t>(stream)));
}

int dit_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, float* delta, void* dq, void* dk, void* dv, int B, int H, int Nq,
                 int Nkv, int D, float scale, int dtype, int grad_dtype, void* stream) {
  if (B < 0 || H < 0 || Nq < 0 || Nkv < 0 || D <= 0) return DIT_EINVAL;
  if (!(isfinite(scale) && scale > 0.0f)) return DIT_EINVAL;
  if (dtype != DIT_BF16 || grad_dtype != DIT_F32) return DIT_EUNSUPPORTED;
  if (D != 32 && D != 64 && D != 128) return DIT_EUNSUPPORTED;
  if (!size_ok(B, H, Nq, D) || !size_ok(B, H, Nkv, D)) return DIT_ERANGE;
  if (B == 0 || H == 0) return DIT_OK;
  if (Nq == 0 || Nkv == 0) return DIT_EINVAL;
  if (!q || !k || !v || !o || !dout || !lse || !delta || !dq || !dk || !dv) return DIT_EINVAL;
  for (const void* p : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned(p, 16)) return DIT_EALIGN;
  if (!aligned(lse, 4) || !aligned(delta, 4)) return DIT_EALIGN;
  return map_launch(ditattn::launch_attn_bwd_bf16(
      q, k, v, o, dout, lse, delta, static_cast<float*>(dq), static_cast<float*>(dk),
      static_cast<float*>(dv), B, H, Nq, Nkv, D, scale, static_cast<hipStream_t>(stream)));
}

int dit_rope_pack(const void* x_txt, const void* x_img, const float* cos_txt,
                  const float* sin_txt, const float* cos_img, const float* sin_img, void* out,
                  int B, int H, int Ht, int h0, int Nt, int Ni, int D, void* stream) {
  int rc = joint_check(B, H, Ht, h0, Nt, Ni, D);
  if (rc != DIT_OK) return rc;
  if (B == 0 || H == 0 || Nt + Ni == 0) return DIT_OK;
  if ((rc = part_check(x_txt, x_img, Nt, Ni)) != DIT_OK) return rc;
  if ((rc = tables_check(cos_txt, sin_txt)) != DIT_OK) return rc;
  if ((rc = tables_check(cos_img, sin_img)) != DIT_OK) return rc;
  if (!out) return DIT_EINVAL;
  if (!aligned(out, 16)) return DIT_EALIGN;
  const ditattn::RopePackTensor t{x_txt, x_img, out, cos_txt, sin_txt, cos_img, sin_img};
  return map_launch(ditattn::launch_rope_pack(&t, 1, B, H, Ht, h0, Nt, Ni, D,
                                              static_cast<hipStream_t>(stream)));
}

int dit_attn_fwd_joint(const void* q_txt, const void* k_txt, const void* v_txt,
                       const void* q_img, const void* k_img, const void* v_img,
                       const float* cos_txt, const float* sin_txt, const float* cos_img,
                       const float* sin_img, void* workspace, void* o, float* lse, int B, int H,
                       int Ht, int h0, int Nt, int Ni, int D, float scale, void* stream) {
  int rc = joint_check(B, H, Ht, h0, Nt, Ni, D);
  if (rc != DIT_OK) return rc;
  if (!(isfinite(scale) && scale > 0.0f)) return DIT_EINVAL;
  if (B == 0 || H == 0 || Nt + Ni == 0) return DIT_OK;
  if ((rc = part_check(q_txt, q_img, Nt, Ni)) != DIT_OK) return rc;
  if ((rc = part_check(k_txt, k_img, Nt, Ni)) != DIT_OK) return rc;
  if ((rc = part_check(v_txt, v_img, Nt, Ni)) != DIT_OK) return rc;
  if ((rc = tables_check(cos_txt, sin_txt)) != DIT_OK) return rc;
  if ((rc = tables_check(cos_img, sin_img)) != DIT_OK) return rc;
  if (!workspace || !o) return DIT_EINVAL;
  if (!aligned(workspace, 16) || !aligned(o, 16)) return DIT_EALIGN;
  if (lse && !aligned(lse, 4)) return DIT_EALIGN;
  const int N = Nt + Ni;
  const int64_t elems = (int64_t)B * H * N * D;
  __bf16* ws = static_cast<__bf16*>(workspace);
  // k is packed turned into the workspace's second slot; v is read from its
  // parts when the text ends on a key-tile boundary, else packed into the
  // third slot; the queries are read and turned by the attention kernel.
  const bool v_parts = Nt % ditattn::kFwdKeyTile == 0;
  const ditattn::RopePackTensor t[2] = {
      {k_txt, k_img, ws + elems, cos_txt, sin_txt, cos_img, sin_img},
      {v_txt, v_img, ws + 2 * elems, nullptr, nullptr, nullptr, nullptr}};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = ditattn::launch_rope_pack(t, v_parts ? 1 : 2, B, H, Ht, h0, Nt, Ni, D, s);
  if (e != hipSuccess) return DIT_ELAUNCH;
  const ditattn::JointParts parts{q_txt, q_img, v_txt, v_img, cos_txt, sin_txt, cos_img, sin_img,
                                  Ht, h0};
  return map_launch(ditattn::launch_attn_joint(ws + elems, v_parts ? nullptr : ws + 2 * elems, parts,
                                               o, lse, B, H, Nt, Ni, D, scale, s));
}

int dit_quant_fp8(const void* x, void* codes, float* descale, int B, int H, int N, int D,
                  void* stream) {
  if (B < 0 || H < 0 || N < 0 || D <= 0) return DIT_EINVAL;
  if (!supported_head_dim(D)) return DIT_EUNSUPPORTED;
  if (!size_ok(B, H, N, D) || (int64_t)B * H > 0x7fffffff) return DIT_ERANGE;
  if (B == 0 || H == 0) return DIT_OK;
  if (!descale || (N > 0 && (!x || !codes))) return DIT_EINVAL;
  if (!aligned(descale, 4)) return DIT_EALIGN;
  if (N > 0 && (!aligned(x, 16) || !aligned(codes, 8))) return DIT_EALIGN;
  return map_launch(ditattn::launch_quant_fp8(x, codes, descale, B, H, N, D,
                                              static_cast<hipStream_t>(stream)));
}

int dit_quant_fp8_qk(const void* q, const void* k, void* q_codes, void* k_codes, float* q_descale,
                     float* k_descale, int B, int H, int Nq, int Nkv, int D, void* stream) {
  if (B < 0 || H < 0 || Nq < 0 || Nkv < 0 || D <= 0) return DIT_EINVAL;
  if (!supported_head_dim(D)) return DIT_EUNSUPPORTED;
  if (!size_ok(B, H, Nq, D) || !size_ok(B, H, Nkv, D) || (int64_t)B * H > 0x7fffffff)
    return DIT_ERANGE;
  if (B == 0 || H == 0) return DIT_OK;
  if (!q_descale || !k_descale || (Nq > 0 && (!q || !q_codes)) || (Nkv > 0 && (!k || !k_codes)))
    return DIT_EINVAL;
  if (!aligned(q_descale, 4) || !aligned(k_descale, 4)) return DIT_EALIGN;
  if (Nq > 0 && (!aligned(q, 16) || !aligned(q_codes, 8))) return DIT_EALIGN;
  if (Nkv > 0 && (!aligned(k, 16) || !aligned(k_codes, 8))) return DIT_EALIGN;
  const void* x[2] = {q, k};
  void* c[2] = {q_codes, k_codes};
  float* ds[2] = {q_descale, k_descale};
  const int n[2] = {Nq, Nkv};
  return map_launch(ditattn::launch_quant_fp8_n(x, c, ds, n, 2, B, H, D,
                                                static_cast<hipStream_t>(stream)));
}

int dit_attn_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                     const float* k_descale, void* o, float* lse, int B, int H, int Nq, int Nkv,
                     int D, float scale, int o_dtype, void* stream) {
  if (B < 0 || H < 0 || Nq < 0 || Nkv < 0 || D <= 0) return DIT_EINVAL;
  if (!(isfinite(scale) && scale > 0.0f)) return DIT_EINVAL;
  if (o_dtype != DIT_BF16 && o_dtype != DIT_F32) return DIT_EUNSUPPORTED;
  if (D != 128) return DIT_EUNSUPPORTED;
  if (!size_ok(B, H, Nq, D) || !size_ok(B, H, Nkv, D)) return DIT_ERANGE;
  if (B == 0 || H == 0 || Nq == 0) return DIT_OK;
  if (Nkv == 0) return DIT_EINVAL;
  if (!q || !k || !v || !q_descale || !k_descale || !o) return DIT_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return DIT_EALIGN;
  if (!aligned(q_descale, 4) || !aligned(k_descale, 4) || (lse && !aligned(lse, 4)))
    return DIT_EALIGN;
  return map_launch(ditattn::launch_attn_fp8(q, k, v, q_descale, k_descale, o, lse, B, H, Nq, Nkv,
                                             scale, o_dtype == DIT_F32,
                                             static_cast<hipStream_t>(stream)));
}

int dit_quant_fp8_qk_mx(const void* q, const void* k, void* q_codes, void* k_codes,
                        float* q_descale, float* k_descale, int B, int H, int Nq, int Nkv, int D,
                        float scale, void* stream) {
  if (B < 0 || H < 0 || Nq < 0 || Nkv < 0 || D <= 0) return DIT_EINVAL;
  if (!(isfinite(scale) && scale > 0.0f)) return DIT_EINVAL;
  if (!supported_head_dim(D)) return DIT_EUNSUPPORTED;
  if (!size_ok(B, H, Nq, D) || !size_ok(B, H, Nkv, D) || (int64_t)B * H > 0x7fffffff)
    return DIT_ERANGE;
  if (B == 0 || H == 0) return DIT_OK;
  if (!q_descale || !k_descale || (Nq > 0 && (!q || !q_codes)) || (Nkv > 0 && (!k || !k_codes)))
    return DIT_EINVAL;
  if (!aligned(q_descale, 4) || !aligned(k_descale, 4)) return DIT_EALIGN;
  if (Nq > 0 && (!aligned(q, 16) || !aligned(q_codes, 8))) return DIT_EALIGN;
  if (Nkv > 0 && (!aligned(k, 16) || !aligned(k_codes, 8))) return DIT_EALIGN;
  const float c0 = scale * 1.4426950408889634f;
  return map_launch(ditattn::launch_quant_fp8_mx(q, k, q_codes, k_codes, q_descale, k_descale, B, H,
                                                 Nq, Nkv, D, c0, static_cast<hipStream_t>(stream)));
}

int dit_attn_fwd_fp8_mx(const void* q, const void* k, const void* v, const float* q_descale,
                        const float* k_descale, void* o, float* lse, int B, int H, int Nq, int Nkv,
                        int D, int o_dtype, void* stream) {
  if (B < 0 || H < 0 || Nq < 0 || Nkv < 0 || D <= 0) return DIT_EINVAL;
  if (o_dtype != DIT_BF16 && o_dtype != DIT_F32) return DIT_EUNSUPPORTED;
  if (D != 128) return DIT_EUNSUPPORTED;
  if (!size_ok(B, H, Nq, D) || !size_ok(B, H, Nkv, D)) return DIT_ERANGE;
  if (B == 0 || H == 0 || Nq == 0) return DIT_OK;
  if (Nkv == 0) return DIT_EINVAL;
  if (!q || !k || !v || !q_descale || !k_descale || !o) return DIT_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return DIT_EALIGN;
  if (!aligned(q_descale, 4) || !aligned(k_descale, 4) || (lse && !aligned(lse, 4)))
    return DIT_EALIGN;
  return map_launch(ditattn::launch_attn_fp8_mx(q, k, v, q_descale, k_descale, o, lse, B, H, Nq,
                                                Nkv, o_dtype == DIT_F32,
                                                static_cast<hipStream_t>(stream)));
}

int ulysses_seq2head(const void* in, void* out, int P, int B, int H, int N, int D, int elem_bytes,
                     void* stream) {
  return permute_common(in, out, P, B, H, N, D, elem_bytes, false, stream);
}

int ulysses_head2seq(const void* in, void* out, int P, int B, int H, int N, int D, int elem_bytes,
                     void* stream) {
  return permute_common(in, out, P, B, H, N, D, elem_bytes, true, stream);
}

const char* dit_strerror(int code) {
  switch (code) {
    case DIT_OK: return "success";
    case DIT_EINVAL: return "invalid argument (null pointer, bad size, divisibility or scale)";
    case DIT_EUNSUPPORTED: return "unsupported head dim, dtype combination or element size";
    case DIT_EALIGN: return "misaligned pointer";
    case DIT_ELAUNCH: return "HIP launch failed";
    case DIT_ERANGE: return "tensor size out of range";
    case DIT_ESCRATCH:
      return "the work needs more scratch than the static buffer holds (DIT_SCRATCH_BYTES)";
    default: return "unknown error code";
  }
}

int dit_abi_version(void) { return DIT_ABI_VERSION; }

}  // extern "C"
