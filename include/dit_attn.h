/*
 * dit_attn.h -- C ABI of libditattn.so: one GPU's share of the attention in
 * Ulysses / Ring sequence parallelism for diffusion transformers, on AMD
 * Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [HB]  "Multi-GPU parallelism: spreading one step over several cards"
 *         (AI infra handbook), section "Sequence parallelism: Ulysses and
 *         Ring": the four-card Ulysses simulation (token partition,
 *         all_to_all_heads, per-card attention, all_to_all_tokens) and the
 *         Ring paragraph (per-block local attention merged by log-sum-exp).
 *   [PR]  "Feat: USP sequence parallelism (Ulysses x Ring) via
 *         SequenceParallelPlan; Wan enabled" (miles_diffusion pull request):
 *         Design / "Ring kernel selection" (ring kernels return the LSE);
 *         "Limitations" (everything outside the envelope fails loudly: head
 *         count divisible by the Ulysses degree, sequence length divisible by
 *         the SP degree, no mask / dropout / causal flag under SP).
 *   [HC]  [HB] section "Combining: what xDiT does": FP8 low precision is the
 *         last step of the latency ladder, on top of the parallel split and
 *         caching (the pages do not say which tensors are 8-bit).
 *   [VO]  "Parallelism Acceleration Guide" (vLLM-Omni docs), section "How
 *         to parallelize a new model": a dual-stream (text + image) model
 *         runs joint attention over the concatenated sequences; the text
 *         stays whole on every sequence-parallel rank and the image rotary
 *         tables are cut along the token axis with the image tokens.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense, row-major, with no padding.  q, k, v, o are
 *    [B, H, N, D] (batch, head, token, channel); lse is float32 [B, H, N].
 *  - Every pointer is a DEVICE pointer on the current HIP device, allocated
 *    and owned by the caller.  The library allocates no memory and keeps no
 *    state between calls (the one exception, the static scratch array of
 *    dit_attn_fwd_balanced_noalloc, is described there); calls are
 *    reentrant.  Outputs must not overlap inputs.
 *  - Every call enqueues its kernels on `stream` (a hipStream_t; NULL = the
 *    legacy default stream) and returns without synchronising.
 *  - All arguments are validated on the host BEFORE any HIP call, so an
 *    argument error leaves the device untouched.  Nothing throws across the
 *    ABI; the return value is DIT_OK or a negative code (dit_strerror).
 *  - Work with a zero batch, head or query count is a no-op that returns
 *    DIT_OK without looking at the pointers.
 *  - bf16 means bfloat16 (1-8-7), stored as 16-bit words; f32 is IEEE binary32.
 */
#ifndef DIT_ATTN_H
#define DIT_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIT_ABI_VERSION 1

typedef enum { DIT_BF16 = 0, DIT_F32 = 1 } dit_dtype;

enum {
  DIT_OK = 0,
  DIT_EINVAL = -1,       /* null pointer, negative size, Nkv == 0, scale not finite or <= 0,
                            H % P != 0, N % P != 0, nblk < 1, P < 1, r outside [0, P),
                            text head range outside [0, Ht), cos without sin, slots < 0,
                            balanced-forward workspace missing or too small */
  DIT_EUNSUPPORTED = -2, /* D not in {32, 64, 128}, a dtype combination not built, elem_bytes
                            not in {1, 2, 4, 8}, fused Ulysses shard length not a multiple
                            of 64 */
  DIT_EALIGN = -3,       /* q/k/v/o/o_parts/rotary tables not 16-byte aligned, lse not
                            4-byte aligned,
                            permute buffers not aligned to elem_bytes */
  DIT_ELAUNCH = -4,      /* the HIP runtime reported an error at launch */
  DIT_ERANGE = -5,       /* a size product does not fit the 64-bit index space */
  DIT_ESCRATCH = -6      /* dit_attn_fwd_balanced_noalloc: the plan needs more scratch than
                            the library's static buffer holds (DIT_SCRATCH_BYTES) */
};

/* Bytes of the static device scratch behind dit_attn_fwd_balanced_noalloc:
   one copy per GPU the library runs on, held until the process ends. */
#define DIT_SCRATCH_BYTES ((size_t)160 << 20)

/*
 * Non-causal full-sequence attention with log-sum-exp  ([HB] Ulysses
 * simulation: each card runs complete attention over all N tokens of its
 * heads; [PR] "Ring kernel selection": the kernel returns the LSE).
 *
 *   O[b,h,i,:]  = sum_j softmax_j(scale * q_i . k_j) v_j
 *   LSE[b,h,i]  = ln sum_j exp(scale * q_i . k_j)        (natural log, scale included)
 *
 *   q, k, v : [B,H,N,D], dtype `dtype` (DIT_BF16 or DIT_F32)
 *   o       : [B,H,N,D], same dtype as the inputs
 *   lse     : float32 [B,H,N], or NULL to skip the LSE write
 *   scale   : finite, > 0 (the usual choice is 1/sqrt(D))
 *   D       : 32, 64 or 128
 * bf16 inputs are contracted on the matrix cores with float32 accumulation;
 * softmax statistics are float32; O is rounded to bf16 (nearest-even) once.
 * There is no mask, dropout or causal flag, by design ([PR] "Limitations").
 */
int dit_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int D, float scale, int dtype, void* stream);

/*
 * One Ring step: attention of Nq queries against one K/V block of Nkv tokens,
 * returning the partial output and its LSE so that partials over disjoint
 * key blocks merge exactly ([HB] Ring paragraph; [PR] "Ring kernel
 * selection").  Same formula as dit_attn_fwd with separate lengths.
 *
 *   q : [B,H,Nq,D] in_dtype;  k, v : [B,H,Nkv,D] in_dtype;  Nkv >= 1
 *   o : [B,H,Nq,D] o_dtype (DIT_F32 keeps the partial unrounded; DIT_BF16
 *       allowed for bf16 inputs);  lse : float32 [B,H,Nq], required.
 * Built combinations: (BF16 -> F32), (BF16 -> BF16), (F32 -> F32).
 */
int dit_attn_fwd_block(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int Nq, int Nkv, int D, float scale,
                       int in_dtype, int o_dtype, void* stream);

/*
 * Work-balanced forward: the same attention as dit_attn_fwd_block (bf16
 * inputs), computed so that the last, partly filled wave of query tiles does
 * not leave compute units idle.  The query tiles (256 rows of one head) that
 * fill whole waves of `slots` concurrent workgroups run as in
 * dit_attn_fwd_block and give bit-identical rows; each remaining tile is cut
 * into key chunks whose float32 (O_j, LSE_j) are merged exactly as Ring
 * blocks are ([HB] Ring paragraph: attention of disjoint key blocks merged
 * by log-sum-exp), so those rows differ from dit_attn_fwd_block only in
 * rounding.  The cut depends on B*H, Nq, Nkv, D and slots, never on the data;
 * two calls with the same arguments give bit-identical results.
 *
 *   q        : bf16 [B,H,Nq,D];  k, v : bf16 [B,H,Nkv,D];  D in {32, 64, 128}
 *   o        : [B,H,Nq,D] in o_dtype (DIT_BF16 or DIT_F32), written
 *   lse      : float32 [B,H,Nq], written, or NULL to skip
 *   slots    : concurrent workgroups to plan for; 0 = the current device's
 *              compute-unit count (one workgroup per compute unit)
 *   workspace: device memory of at least the size that
 *              dit_attn_fwd_balanced_workspace reports for the same sizes and
 *              slots (16-byte aligned; may be NULL when that size is 0);
 *              caller-owned, overwritten, must not overlap any other argument
 * Returns DIT_EINVAL when the workspace is missing or too small.  Calls that
 * share one workspace must be ordered on one stream.
 */
int dit_attn_fwd_balanced(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int Nq, int Nkv, int D, float scale, int o_dtype,
                          int slots, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes dit_attn_fwd_balanced needs for these sizes and slots
 * (0 when the tiles already fill whole waves or a split would not pay).
 * Writes *bytes; returns DIT_OK or the error dit_attn_fwd_balanced would give
 * for the sizes.  slots = 0 queries the current device (a host-side HIP
 * attribute query; DIT_ELAUNCH if it fails).
 */
int dit_attn_fwd_balanced_workspace(int B, int H, int Nq, int Nkv, int D, int slots,
                                    size_t* bytes);

/*
 * dit_attn_fwd_balanced without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, plan, kernels and results
 * (bit for bit) as dit_attn_fwd_balanced; the key-chunk partials go to a
 * static device array of DIT_SCRATCH_BYTES (160 MiB) per GPU instead of a
 * caller workspace.  The call allocates nothing (no hipMalloc / hipFree, no
 * allocating library routine); its first call on a device looks up that
 * device's copy of the array once.
 *
 * Returns DIT_ESCRATCH, before any launch, when the plan's partials need more
 * than DIT_SCRATCH_BYTES (dit_attn_fwd_balanced_workspace reports the size;
 * the long-video shape B1 H10 N75600 D128 on 256 compute units needs 133 MB).
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (on different streams, or from different threads) race; order
 * them on one stream.  Nothing in the array has to start at zero (each call
 * writes every partial it reads), and it keeps the last call's contents.
 */
int dit_attn_fwd_balanced_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int B, int H, int Nq, int Nkv, int D, float scale, int o_dtype,
                                  int slots, void* stream);

/*
 * Attention backward: the gradients of sum(dout * O) for O = attention(q, k, v)
 * ([PR] "Ring kernel selection": the ring kernels pair with a real backward
 * kernel and return the LSE it needs; Validation: dQ/dK/dV compared against
 * a full-sequence reference, and bitwise repeatable in deterministic mode).
 * The chain rule of dit_attn_fwd's definition, with P recomputed from the
 * forward's LSE:
 *
 *   P_ij     = exp(scale * q_i . k_j - LSE_i)
 *   delta_i  = sum_d dout_id * o_id
 *   dS_ij    = P_ij * (dout_i . v_j - delta_i)
 *   dv_j = sum_i P_ij dout_i,  dk_j = scale sum_i dS_ij q_i,  dq_i = scale sum_j dS_ij k_j
 *
 *   q, o, dout : bf16 [B,H,Nq,D];  k, v : bf16 [B,H,Nkv,D];  D is 32, 64 or 128
 *                (else DIT_EUNSUPPORTED)
 *   lse        : float32 [B,H,Nq], the forward's LSE (required)
 *   delta      : float32 [B,H,Nq], written (rowsum(dout * o)); caller-owned
 *   dq         : float32 [B,H,Nq,D];  dk, dv : float32 [B,H,Nkv,D]  (written)
 *   dtype must be DIT_BF16 and grad_dtype DIT_F32.
 * For one Ring K/V block, pass the merged o and lse of the full row: dk, dv
 * are that block's gradients and dq its share (sum the shares over blocks).
 * Every output element is written once with a fixed summation order, so two
 * calls give bit-identical results.  Nq and Nkv must be >= 1 (DIT_EINVAL),
 * unless B or H is 0 (no-op).
 */
int dit_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, float* delta, void* dq, void* dk, void* dv, int B, int H,
                 int Nq, int Nkv, int D, float scale, int dtype, int grad_dtype, void* stream);

/*
 * Exact log-sum-exp merge of nblk partials over disjoint key blocks ([HB]
 * Ring paragraph: results of each K/V block merged with a log-sum-exp).
 *
 *   M   = max_i LSE_i
 *   LSE = M + ln sum_i exp(LSE_i - M)
 *   O   = sum_i exp(LSE_i - LSE) * O_i
 *
 *   o_parts   : float32 [nblk,B,H,N,D], the partials stacked contiguously
 *   lse_parts : float32 [nblk,B,H,N]
 *   o         : [B,H,N,D] in o_dtype (DIT_BF16 or DIT_F32)
 *   lse       : float32 [B,H,N], or NULL to skip
 * A block whose LSE is -inf gets weight 0; a row whose every LSE is -inf
 * gets O = 0 and LSE = -inf (never NaN).
 */
int dit_attn_merge(const float* o_parts, const float* lse_parts, int nblk,
                   void* o, float* lse, int B, int H, int N, int D, int o_dtype, void* stream);

/*
 * Attention of one Ulysses head group read straight from the token shards
 * and written straight back into them: ulysses_seq2head of q, k, v, then
 * dit_attn_fwd on head group r, then ulysses_head2seq of that group's
 * output, without the exchange buffers ([HB] Ulysses simulation: the
 * all_to_all_heads / per-card attention / all_to_all_tokens sequence of one
 * card, r being its rank).
 *
 *   q, k, v : bf16 [P][B,H,N/P,D]   rank s holds every head of tokens
 *                                   [s*N/P, (s+1)*N/P)
 *   o       : bf16 [P][B,H,N/P,D]   only heads [r*H/P, (r+1)*H/P) of every
 *                                   shard are written; the other heads are
 *                                   left untouched, so the P calls r = 0..P-1
 *                                   fill the whole output
 *   lse     : float32 [B,H/P,N] for head group r (natural log, scale
 *             included), or NULL to skip
 *   0 <= r < P;  N is the full sequence length; dtype must be DIT_BF16.
 * The O and LSE values are bit-identical to the unfused sequence above (the
 * same kernel, with different addressing).  Requires H % P == 0 and
 * N % P == 0 (DIT_EINVAL otherwise, [PR] "Limitations") and, as a limit of
 * this implementation, when N/P is not a multiple of 64, N/P >= 64 and
 * (B*H - 1)*(N/P)*D*2 + 128*D < 2^31 (DIT_EUNSUPPORTED otherwise; use the
 * unfused sequence): a 64-key tile may then span two shards, never three,
 * and the second is reached through a 32-bit offset from the first.
 */
int dit_attn_fwd_ulysses(const void* q, const void* k, const void* v, void* o, float* lse,
                         int P, int r, int B, int H, int N, int D, float scale, int dtype,
                         void* stream);

/*
 * Joint text + image sequence with rotary position embedding ([VO]): per
 * (b, h), the Nt text tokens of head h0 + h of the text tensor, then the Ni
 * image tokens of head h of the image tensor.  The pages name the rotary
 * tables but not the rotation; the reading taken is RoFormer's rotary
 * embedding in interleaved form: channels (2i, 2i+1) of token n are one pair,
 * turned by that token's angle for pair i,
 *
 *   y[2i] = x[2i] cos[n,i] - x[2i+1] sin[n,i],  y[2i+1] = x[2i] sin[n,i] + x[2i+1] cos[n,i]
 *
 * in float32, rounded to bf16 (nearest, ties to even).
 *
 *   x_txt            : bf16 [B,Ht,Nt,D]; heads h0 .. h0+H-1 are used (the
 *                      text stays replicated with all Ht heads on every rank,
 *                      the call covers one head group of it)
 *   x_img            : bf16 [B,H,Ni,D]
 *   cos_txt, sin_txt : float32 [Nt, D/2], or both NULL: text copied unturned
 *   cos_img, sin_img : float32 [Ni, D/2], or both NULL: image copied unturned
 *   out              : bf16 [B,H,Nt+Ni,D]
 * x_txt may be NULL when Nt == 0 and x_img when Ni == 0.  Requires
 * 0 <= h0, h0 + H <= Ht when Nt > 0, and one of cos / sin of a part given
 * without the other is DIT_EINVAL.  Tables must be 16-byte aligned.
 */
int dit_rope_pack(const void* x_txt, const void* x_img, const float* cos_txt,
                  const float* sin_txt, const float* cos_img, const float* sin_img, void* out,
                  int B, int H, int Ht, int h0, int Nt, int Ni, int D, void* stream);

/*
 * Joint attention ([VO]): every text and image query attends over every text
 * and image key, with the rotary embedding on queries and keys (not values).
 * The result is, bit for bit, dit_rope_pack of q and k (with the tables) and
 * of v (without), then dit_attn_fwd over the N = Nt + Ni joint tokens; the
 * call itself packs only k (turned), and v too when Nt is not a multiple of
 * 64, while the attention kernel turns the queries as it loads them and
 * reads v from its two parts.
 *
 *   q_txt, k_txt, v_txt : bf16 [B,Ht,Nt,D] (heads h0 .. h0+H-1 used)
 *   q_img, k_img, v_img : bf16 [B,H,Ni,D]
 *   tables              : as in dit_rope_pack
 *   workspace           : bf16 [3][B,H,N,D] scratch owned by the caller (the
 *                         second slot receives the packed k, the third the
 *                         packed v when Nt % 64 != 0; overwritten)
 *   o                   : bf16 [B,H,N,D], text rows first
 *   lse                 : float32 [B,H,N], or NULL to skip
 * Cross attention (image queries over text keys only) needs no packing: it
 * is dit_attn_fwd_block with Nq = Ni and Nkv = Nt.
 */
int dit_attn_fwd_joint(const void* q_txt, const void* k_txt, const void* v_txt,
                       const void* q_img, const void* k_img, const void* v_img,
                       const float* cos_txt, const float* sin_txt, const float* cos_img,
                       const float* sin_img, void* workspace, void* o, float* lse, int B, int H,
                       int Ht, int h0, int Nt, int Ni, int D, float scale, void* stream);

/*
 * Per-(b, h) quantization to 8-bit floating point for dit_attn_fwd_fp8 ([HC];
 * format and scaling are this library's reading: OCP E4M3 -- 1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits, subnormals, largest finite
 * 448, no infinities):
 *
 *   descale[b,h] = amax / 448 in float32 (correctly rounded), amax = max |x|
 *                  over the head; 1 for an all-zero (or empty) head
 *   code         = E4M3 of the float32 quotient x / descale (correctly
 *                  rounded), clamped to +-448, rounded to nearest-even
 *
 *   x       : bf16 [B,H,N,D]
 *   codes   : uint8 [B,H,N,D] E4M3 codes (written), 8-byte aligned
 *   descale : float32 [B,H] (written)
 * Deterministic (the max is exact).  NaN inputs get no special handling.
 */
int dit_quant_fp8(const void* x, void* codes, float* descale, int B, int H, int N, int D,
                  void* stream);

/*
 * dit_quant_fp8 of the queries and keys of one attention call together, in
 * three launches instead of six (same codes and descales, bit for bit):
 *
 *   q : bf16 [B,H,Nq,D] -> q_codes uint8 [B,H,Nq,D], q_descale float32 [B,H]
 *   k : bf16 [B,H,Nkv,D] -> k_codes uint8 [B,H,Nkv,D], k_descale float32 [B,H]
 *
 * Alignment and errors as dit_quant_fp8, for each tensor.  The four outputs
 * must not overlap each other or the inputs.
 */
int dit_quant_fp8_qk(const void* q, const void* k, void* q_codes, void* k_codes, float* q_descale,
                     float* k_descale, int B, int H, int Nq, int Nkv, int D, void* stream);

/*
 * FP8 attention ([HC], reading as above): scores from E4M3 queries and keys,
 *
 *   s_ij = scale * q_descale[b,h] * k_descale[b,h] * (q_i . k_j)   (codes decoded)
 *
 * then the softmax, O and LSE of dit_attn_fwd_block with P and V in bf16.
 * The products q_i . k_j run on the fp8 matrix cores
 * (v_mfma_f32_16x16x128_f8f6f4) with float32 accumulation.
 *
 *   q       : uint8 [B,H,Nq,D] E4M3 codes;  k : uint8 [B,H,Nkv,D] E4M3 codes
 *   v       : bf16 [B,H,Nkv,D];  q_descale, k_descale : float32 [B,H]
 *   o       : [B,H,Nq,D] in o_dtype (DIT_BF16 or DIT_F32)
 *   lse     : float32 [B,H,Nq] (natural log, all factors included), or NULL
 *   D must be 128.  Nkv >= 1 unless B, H or Nq is 0 (no-op).
 */
int dit_attn_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale,
                     const float* k_descale, void* o, float* lse, int B, int H, int Nq, int Nkv,
                     int D, float scale, int o_dtype, void* stream);

/*
 * FP8 with power-of-two scales, for the fp8 product that applies E8M0
 * (power-of-two) scales itself ([HC]; this library's second reading of the
 * FP8 step): the queries of one attention call are first multiplied in
 * float32 by c0 = scale * log2(e) (c0 the float32 product of the two), so
 * that the scaled products are the scores in base 2.  Per (b, h) and tensor,
 * with x' = float32(x * c0) for q and x' = k for k:
 *
 *   descale[b,h] = the smallest power of two 2^e (e >= -126) with
 *                  max |x'| <= 448 * 2^e over the head; 1 for an all-zero
 *                  (or empty) head
 *   code         = E4M3 of x' / descale (exact quotient), nearest-even
 *
 *   q : bf16 [B,H,Nq,D] -> q_codes uint8 [B,H,Nq,D], q_descale float32 [B,H]
 *   k : bf16 [B,H,Nkv,D] -> k_codes uint8 [B,H,Nkv,D], k_descale float32 [B,H]
 *   scale : the softmax scale dit_attn_fwd_fp8_mx will apply (> 0, finite)
 * Three launches, as dit_quant_fp8_qk; alignment and errors as dit_quant_fp8_qk.
 * The products x * c0 must stay within float32's range (they do unless c0 > 1
 * and |q| is within a factor c0 of the bf16 maximum): a head where one
 * overflows gets unspecified codes and descale, as does a head holding NaN.
 */
int dit_quant_fp8_qk_mx(const void* q, const void* k, void* q_codes, void* k_codes,
                        float* q_descale, float* k_descale, int B, int H, int Nq, int Nkv, int D,
                        float scale, void* stream);

/*
 * Attention of codes from dit_quant_fp8_qk_mx ([HC], reading as above): the
 * scores in base 2 are
 *
 *   s_ij = q_descale[b,h] * k_descale[b,h] * (q_i . k_j)   (codes decoded),
 *
 * P_ij = 2^s_ij / sum_j 2^s_ij, O = P V with P and V in bf16, LSE = ln 2 *
 * log2 sum_j 2^s_ij (natural log).  The descales must be powers of two
 * (normal floats), as dit_quant_fp8_qk_mx writes them: the kernel passes
 * their exponents to the fp8 matrix instruction as its E8M0 scales and starts
 * each score accumulation at minus the row's reference maximum, so the
 * softmax needs no multiply.  Arguments as dit_attn_fwd_fp8 without `scale`
 * (it is in the query codes).  D must be 128.
 */
int dit_attn_fwd_fp8_mx(const void* q, const void* k, const void* v, const float* q_descale,
                        const float* k_descale, void* o, float* lse, int B, int H, int Nq, int Nkv,
                        int D, int o_dtype, void* stream);

/*
 * Ulysses sequence -> head exchange as it lands on one device ([HB] Ulysses
 * simulation, all_to_all_heads): P token shards become P head groups.
 *
 *   in  : [P][B,H,N/P,D]  rank s holds every head of tokens [s*N/P,(s+1)*N/P)
 *   out : [P][B,H/P,N,D]  rank r holds heads [r*H/P,(r+1)*H/P) of all N tokens
 *   out[r][b,h',s*N/P+n,d] = in[s][b,r*H/P+h',n,d]
 * N is the full sequence length.  Pure data movement of elem_bytes-sized
 * elements (1, 2, 4 or 8): the result is bit-exact for any dtype.
 * Requires H % P == 0 and N % P == 0 ([PR] "Limitations": no padding).
 */
int ulysses_seq2head(const void* in, void* out, int P, int B, int H, int N, int D,
                     int elem_bytes, void* stream);

/*
 * Inverse exchange, head -> sequence ([HB] Ulysses simulation,
 * all_to_all_tokens):
 *   in  : [P][B,H/P,N,D],  out : [P][B,H,N/P,D]
 *   out[s][b,r*H/P+h',n,d] = in[r][b,h',s*N/P+n,d]
 * Same requirements and exactness as ulysses_seq2head.
 */
int ulysses_head2seq(const void* in, void* out, int P, int B, int H, int N, int D,
                     int elem_bytes, void* stream);

/* Static English text for a return code (never NULL). */
const char* dit_strerror(int code);

/* DIT_ABI_VERSION of the built library. */
int dit_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIT_ATTN_H */
