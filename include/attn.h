/*
 * attn.h -- C ABI of the exact-attention library for MI355X (gfx950).
 *
 * Computes exact scaled-dot-product attention
 *
 *     O = softmax(Q K^T * scale + mask) V
 *
 * tile by tile with an online softmax (a running row maximum m and running
 * exponential sum l), so the N x N score matrix never reaches HBM, and writes
 * the per-row log-sum-exp LSE so that the backward pass can form the
 * probabilities again from LSE instead of storing them.
 *
 * Sources (web pages, by title and section):
 *   - the unfused chain S = QK^T, S/sqrt(d_k), S + attn_mask, softmax, S V:
 *     "Step 3.7 Flash 的表现有点意外" (xxmr.cn/news/81028) §2.3;
 *   - tiling into B_r x B_c blocks and the online softmax (running m and l):
 *     "FlashAttention技术解析：优化Transformer注意力计算效率"
 *     (jsqmd.com/news/722897) §2.2; storing only O(N) statistics and
 *     recomputing P in the backward: same page §3.3;
 *   - the call surfaces that fix the argument set: F.scaled_dot_product_attention
 *     (q, k, v in [B, H, N, d], attn_mask, is_causal) and
 *     flash_attn_func(q, k, v, softmax_scale, causal, window_size,
 *     deterministic) in [B, N, H, d] -- "如何在ChatGLM2-6B中集成Flash-Attention2？
 *     实测性能提升与显存优化" (jsqmd.com/news/348824) §3 steps 3 and 4;
 *   - the tanh soft cap (score_mod) and the 2-D neighbourhood mask
 *     (mask_mod / block_mask) of FlexAttention: the PyTorch
 *     attention-options article (atyun.com/61003), sections
 *     "Score Mod示例：使用Tanh进行软上限" and "Mask Mod示例：邻域屏蔽".
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library allocates nothing and frees nothing; the backward's scratch
 *     comes in through `workspace`.
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the default
 *     stream) and return without synchronising.  Faults during execution
 *     surface at the caller's next synchronisation.
 *   - Errors are returned as attn_status; the library never aborts or prints.
 *   - The library keeps no global state; calls on different streams may run
 *     concurrently.
 */
#ifndef EXACT_ATTENTION_ATTN_H
#define EXACT_ATTENTION_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = 1,        /* invalid shape or parameter                         */
  ATTN_EUNSUPPORTED = 2,  /* valid, but outside what the kernels implement      */
  ATTN_EALIGN = 3,        /* a pointer is not 16-byte aligned                   */
  ATTN_EWORKSPACE = 4,    /* workspace missing or too small                     */
  ATTN_EHIP = 5,          /* a kernel launch failed (hipGetLastError)           */
  ATTN_ESCRATCH = 6       /* attn_decode_static: the call needs more scratch
                             than ATTN_DECODE_SCRATCH_BYTES                     */
} attn_status;

typedef enum { ATTN_FP32 = 0, ATTN_FP16 = 1, ATTN_BF16 = 2 } attn_dtype;

/* d is always the contiguous (innermost) dimension. */
typedef enum {
  ATTN_BHND = 0,  /* [B, H, N, d]: the scaled_dot_product_attention layout      */
  ATTN_BNHD = 1   /* [B, N, H, d]: the flash_attn_func ("bshd") layout           */
} attn_layout;

typedef struct {
  int32_t B;       /* batch                                                     */
  int32_t Hq;      /* query heads                                               */
  int32_t Hkv;     /* key/value heads; Hq % Hkv == 0; q-head h reads kv-head    */
                   /* h / (Hq / Hkv) (grouped-query attention)                  */
  int32_t Nq;      /* query rows per head, >= 0                                 */
  int32_t Nk;      /* key rows per head, >= 0                                   */
  int32_t d;       /* head dimension: 8 <= d <= 128, d % 8 == 0                 */
  attn_dtype dtype;   /* element type of q, k, v, o and dout                   */
  attn_layout layout; /* layout of q, k, v, o, dout, dq, dk, dv; lse is always */
                      /* a contiguous [B, Hq, Nq] float array                  */
  float scale;     /* softmax scale; <= 0 or NaN means 1/sqrt(d) (real d)       */
  int32_t causal;  /* non-zero: key j is visible to query i iff j <= i;         */
                   /* requires Nq == Nk                                         */
  /* Optional additive float mask in logit units, added after scaling:
   *   element (b, h, i, j) is mask[b*mask_sb + h*mask_sh + i*mask_sq + j].
   * A stride of 0 broadcasts that dimension.  -INFINITY entries exclude a key.
   * NULL = no mask. */
  const float* mask;
  int64_t mask_sb, mask_sh, mask_sq;
  /* Optional [B] int32 valid key counts: keys j >= kv_lens[b] are excluded.
   * Values are clamped to [0, Nk].  NULL = all Nk keys are valid.  The rows
   * of k and v past kv_lens[b] are never read into a result (they may hold
   * anything, NaN and infinities included), except by attn_quantize_fp8,
   * whose 64-row block scales span them. */
  const int32_t* kv_lens;
  /* Local attention and the soft cap; a zero-filled tail means none of them.
   * Query row i sits at position p = i in attn_fwd / attn_bwd and at
   * p = L - Nq + i in attn_decode (L = kv_lens[b] or Nk).
   *   window != 0: sliding window (flash_attn_func's window_size =
   *     (window_left, window_right)): key j is visible iff
   *     p - window_left <= j <= p + window_right; a negative bound leaves its
   *     side open.  Combines with causal (which then caps the right side).
   *   grid_cols > 0: 2-D neighbourhood: position t is the cell
   *     (t / grid_cols, t % grid_cols) of a row-major grid, and key j is
   *     visible iff |row(p) - row(j)| < nbr_rows and
   *     |col(p) - col(j)| < nbr_cols (both >= 1).  attn_fwd / attn_bwd only.
   *   softcap > 0: the scaled logit s = scale * q.k becomes
   *     softcap * tanh(s / softcap) before the additive mask.  0 = off.
   * A key excluded by any rule is excluded (the rules intersect).  With a
   * window or grid, attn_fwd / attn_bwd need Nq == Nk and Nq + Nk < 2^29;
   * attn_decode always needs Nq + Nk < 2^29. */
  int32_t window;
  int32_t window_left, window_right;
  int32_t grid_cols, nbr_rows, nbr_cols;
  float softcap;
} attn_params;

/* Host-only check of *p (no GPU call) for attn_fwd (for_backward == 0) or
 * attn_bwd (for_backward != 0).  Returns ATTN_OK, ATTN_EINVAL (null p,
 * shapes out of range (B, Nq, Nk < 0; Hq, Hkv, d < 1), Hq % Hkv != 0, causal,
 * window or grid with Nq != Nk, bad enum, negative mask stride, grid_cols < 0,
 * grid_cols > 0 with nbr_rows or nbr_cols < 1, softcap negative or not
 * finite, or so small that 2 * scale * log2(e) / softcap overflows) or
 * ATTN_EUNSUPPORTED (d outside [8, 128] or d % 8 != 0; a window or grid with
 * Nq + Nk >= 2^29).  The forward and the backward accept the same params.
 * B == 0, Nq == 0 and Nk == 0 are valid: the first two make a call a no-op,
 * the last makes every row fully masked. */
attn_status attn_validate(const attn_params* p, int for_backward);

/* Forward pass.
 *   q:   [B, Hq, Nq, d] or [B, Nq, Hq, d] (p->layout), p->dtype
 *   k,v: [B, Hkv, Nk, d] or [B, Nk, Hkv, d], p->dtype
 *   o:   output, q's shape and layout, p->dtype (rounded to nearest even)
 *   lse: output, [B, Hq, Nq] float: natural-log log-sum-exp of the scaled,
 *        masked logits of each row; -INFINITY (and o = 0) for a row whose
 *        keys are all excluded.
 * q, k, v, o, lse must be 16-byte aligned.  Returns ATTN_OK once the kernel
 * is enqueued; ATTN_EINVAL / ATTN_EUNSUPPORTED / ATTN_EALIGN without
 * enqueueing anything; ATTN_EHIP if the launch failed. */
attn_status attn_fwd(const attn_params* p, const void* q, const void* k,
                     const void* v, void* o, float* lse, void* stream);

/* Bytes of device workspace attn_bwd needs for *p (0 if p is invalid): two
 * [B, Hq, Nq rounded up to 128] float arrays (D and -LSE*log2(e)); for
 * 16-bit inputs whose q-heads of a kv-head are split over several
 * work-groups, fp32 partial dK and dV sums; for bf16 inputs, fp16 copies of
 * q, dout and k, and 32 KB of per-block maxima and scales. */
size_t attn_bwd_workspace_bytes(const attn_params* p);

/* Backward pass: gradients of <dout, O> with O = attention(q, k, v), with the
 * probabilities formed again from the forward's lse (FlashAttention技术解析
 * §3.3).  With D_i = sum_c dout_ic o_ic:
 *   dP = dout V^T, dS = P * (dP - D), dq = scale dS K,
 *   dk = scale dS^T Q, dv = P^T dout,
 * where dk, dv sum over the q-heads sharing a kv-head.
 *   o, lse: the forward's outputs for the same inputs and params
 *   dout:   q's shape, layout and dtype
 *   dq:     q's shape and layout; dk, dv: k's shape and layout
 *   grad_dtype: element type of dq, dk, dv: ATTN_FP32 or p->dtype
 *   workspace: device memory of at least attn_bwd_workspace_bytes(p) bytes,
 *              16-byte aligned; its contents on entry do not matter.
 * The additive mask (p->mask, the same one the forward took), kv_lens,
 * causal, the window, the grid and the soft cap (whose derivative
 * 1 - tanh^2(s / softcap) multiplies dS) and all three dtypes are supported
 * (fp32 inputs take an all-fp32 path).  The result is deterministic: no
 * atomics.  bf16 inputs run the products that take P or dS on fp16 operands
 * (11-bit significands, the precision the 2e-2 tolerance of the causal GQA
 * case needs); the fp16 copies of q, k, v and dout are scaled by powers of
 * two found on the device from each tensor's largest magnitude and the
 * scales are undone exactly, so bf16 inputs above 65504 or below 2^-14 are
 * handled (fully for largest magnitudes within [2^-27, 2^42]). */
attn_status attn_bwd(const attn_params* p, const void* q, const void* k,
                     const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv,
                     attn_dtype grad_dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Bytes of device workspace attn_decode needs for *p (0 if p is not a valid
 * decode problem): the fp32 partial outputs and log-sum-exps of the key
 * splits, [n_splits, B, Hq, Nq, d] and [n_splits, B, Hq, Nq]. */
size_t attn_decode_workspace_bytes(const attn_params* p);

/* Decode attention: a few new queries (Nq, typically 1..16) against a long
 * key/value cache, split over the keys and merged through the log-sum-exp
 * (FlashDecoding; FlashAttention技术解析 §5.2, decode phase).  Computes the
 * same O and LSE as attn_fwd for:
 *   q: [B,Hq,Nq,d] / [B,Nq,Hq,d]; k, v: [B,Hkv,Nk,d] / [B,Nk,Hkv,d] (the
 *      cache); o: q's shape; lse: [B,Hq,Nq] fp32
 *   kv_lens: optional per-batch count of valid cache entries
 *   causal: the Nq queries are the last Nq positions of the sequence: query
 *      i sees keys j <= L - Nq + i, with L = kv_lens[b] (or Nk).  Unlike
 *      attn_fwd, Nq may differ from Nk.
 *   window / softcap: as for attn_fwd, at position p = L - Nq + i; with a
 *      bounded window_left only the last Nq + window_left keys are read.
 * 16-bit dtypes only, no additive mask and no grid (ATTN_EUNSUPPORTED
 * otherwise); Nq + Nk < 2^29; other parameters as for attn_fwd.
 *   workspace: device memory of at least attn_decode_workspace_bytes(p)
 *              bytes, 16-byte aligned; its contents on entry do not matter.
 * Deterministic: the splits are merged in a fixed order. */
attn_status attn_decode(const attn_params* p, const void* q, const void* k,
                        const void* v, void* o, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Size of the fixed device scratch of attn_decode_static: 16 MiB, one copy
 * per GPU, held from the library's load until the process ends. */
#define ATTN_DECODE_SCRATCH_BYTES (16u << 20)

/* attn_decode without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The key splits'
 * partial outputs go to a static device array of ATTN_DECODE_SCRATCH_BYTES
 * instead; results are those of attn_decode, bit for bit.
 *   Arguments, layouts and errors as for attn_decode (no workspace); the
 *   stream must belong to the current device, whose copy of the scratch is
 *   used.  Returns ATTN_ESCRATCH, before enqueueing anything, when
 *   attn_decode_workspace_bytes(p) > ATTN_DECODE_SCRATCH_BYTES; ATTN_EHIP if
 *   the scratch's device address cannot be obtained.
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (nothing in it needs clearing): calls that may overlap on
 * one GPU (different streams, different host threads) race and must be
 * ordered by the caller. */
attn_status attn_decode_static(const attn_params* p, const void* q, const void* k,
                               const void* v, void* o, float* lse, void* stream);

/* FP8 block quantisation for attn_fwd_fp8 (the FP8 variant of
 * "FlashAttention技术解析：优化Transformer注意力计算效率" (jsqmd.com/news/722897)
 * §4.2 item 3 and §6.3 item 2: FP8 matrix operands, one scale per block).
 * Every 64 consecutive rows of one (batch, head) of q, k and v form a block
 * with scale s = amax / 448 (1 for an all-zero block), computed in fp32, and
 * each element becomes the OCP FP8 E4M3FN code of fp32(x * (448 / amax)),
 * rounded to nearest even; the value a code stands for is code * s.
 *   q, k, v:  as for attn_fwd, element type p->dtype (any of the three)
 *   q8, k8:   outputs, E4M3 codes, q's and k's shape and layout (1 byte each)
 *   vt8:      output, v's codes transposed: [B, Hkv, d, ldv] bytes with
 *             ldv = Nk rounded up to 64 (keys contiguous; columns past Nk 0)
 *   q_scale:  output, [B, Hq, ceil(Nq / 64)] float
 *   k_scale, v_scale: outputs, [B, Hkv, ceil(Nk / 64)] float
 * Needs d % 16 == 0 (ATTN_EUNSUPPORTED otherwise); every pointer 16-byte
 * aligned.  p's mask, window, grid and soft cap are ignored. */
attn_status attn_quantize_fp8(const attn_params* p, const void* q, const void* k,
                              const void* v, void* q8, void* k8, void* vt8, float* q_scale,
                              float* k_scale, float* v_scale, void* stream);

/* FP8 forward on the outputs of attn_quantize_fp8: the same O and LSE as
 * attn_fwd on the dequantised inputs (code * block scale), with both matrix
 * products on FP8 operands: the probabilities are rounded to E4M3 for the
 * product with V (relative error up to 2^-4 per probability), the softmax
 * statistics stay fp32.
 *   p->dtype: the element type of o (ATTN_BF16 or ATTN_FP16); p->layout: the
 *   layout of q8, k8 and o; causal, kv_lens, GQA and scale as for attn_fwd.
 *   o: output, q's shape and layout; lse: output, [B, Hq, Nq] float.
 * ATTN_EUNSUPPORTED for an fp32 output, an additive mask, a window, a grid,
 * a soft cap or d % 16 != 0. */
attn_status attn_fwd_fp8(const attn_params* p, const void* q8, const void* k8,
                         const void* vt8, const float* q_scale, const float* k_scale,
                         const float* v_scale, void* o, float* lse, void* stream);

/* Static, human-readable name of a status code. */
const char* attn_status_string(attn_status s);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_ATTN_H */
