/*
 * abg.h - C ABI of the biased multi-query attention library (libabg.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation is AlphaGenome's sequence attention as described on the web
 * page "Making Full-Context AlphaGenome Fit on an RTX 3090"
 * (twigslot.github.io):
 *
 *   - section "Why stock FlashAttention was not a drop-in replacement":
 *     Q [B,S,8,128], K [B,S,1,128], V [B,S,1,Dv] with one K/V head shared by
 *     the 8 query heads; a compact learned bias with one cell per 16
 *     positions on each axis; the logit equation
 *         L_ij = cap * tanh((scale * q_i . k_j + bias[i/16, j/16]) / cap)
 *     with cap 5 and scale 1/sqrt(128); softmax over keys; times V; BF16
 *     matrix products with FP32 accumulation.
 *   - section "Profiling pointed at one very large object": the compact bias
 *     is a projection of a compact pair representation, repeated 16x along
 *     both sequence axes in the dense implementation.
 *   - section "Online softmax, one block at a time": the output is computed
 *     tile by tile with running max / denominator / numerator, and the dense
 *     logits and the dense repeated bias never exist.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors) owned by the caller.  Tensors are dense, row-major,
 *     contiguous, 16-byte aligned.  The library never allocates, frees or
 *     synchronizes; it only enqueues kernels on `stream` (a hipStream_t
 *     passed as void*, NULL = the null stream) and returns.
 *   - Every argument is validated on the host before any HIP call; a non-OK
 *     status means nothing was enqueued.  abg_last_error() then gives a
 *     thread-local message naming the argument.
 *   - ABG_ERR_DEVICE means the HIP runtime rejected the launch; the message
 *     carries the HIP error string.  Kernel faults surface, as usual for HIP,
 *     at the caller's next synchronization.
 *   - Calls are thread-safe; results are deterministic (no atomics).
 */
#ifndef ABG_H
#define ABG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ABG_ABI_VERSION 1

typedef enum abg_status {
  ABG_OK = 0,
  ABG_ERR_NULL = 1,        /* a required pointer is NULL                         */
  ABG_ERR_SHAPE = 2,       /* a size is out of range or sizes are inconsistent   */
  ABG_ERR_UNSUPPORTED = 3, /* valid request that this library does not implement */
  ABG_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                   */
  ABG_ERR_VALUE = 5,       /* a scalar argument is not finite or out of range    */
  ABG_ERR_DEVICE = 6,      /* the HIP runtime reported an error                  */
  ABG_ERR_ALIAS = 7        /* the output overlaps an input (appended after the   */
                           /* first six codes, which keep their values)          */
} abg_status;

typedef enum abg_dtype {
  ABG_F32 = 0,  /* IEEE float32 inputs, float32 products                   */
  ABG_BF16 = 1  /* bfloat16 inputs, bf16 products with float32 accumulation */
} abg_dtype;

/* Version of this ABI (ABG_ABI_VERSION). */
int abg_abi_version(void);

/* Static, human-readable name of a status code. */
const char* abg_status_string(int status);

/* Thread-local detail for the last non-OK status returned on this thread
 * ("" if none).  The pointer stays valid until the next library call on the
 * same thread. */
const char* abg_last_error(void);

/*
 * Pair-bias projection ("Profiling pointed at one very large object"):
 *
 *   bias[b, h, p, r] = sum_c pair[b, p, r, c] * weight[c, h]
 *
 * A plain linear map (no bias term, normalisation or activation).
 *   pair    [Bp, P, P, C]  dtype      compact pair representation(s)
 *   weight  [C, H]         dtype      projection weight, shared by all b
 *   bias    [Bp, H, P, P]  float32    written fully (products in dtype,
 *                                     accumulated in float32)
 * Limits: Bp >= 1; 1 <= P <= 65536; 8 <= C <= 512 with C % 8 == 0; H == 8.
 * bias must not overlap pair or weight.
 */
abg_status abg_pair_bias_project(const void* pair, const void* weight, float* bias,
                                 int64_t Bp, int64_t P, int64_t C, int64_t H,
                                 abg_dtype dtype, void* stream);

/*
 * Biased, soft-capped multi-query attention forward
 * ("Why stock FlashAttention was not a drop-in replacement", logit equation;
 *  "Online softmax, one block at a time"):
 *
 *   x_ij  = scale * (q[b,i,h,:] . k[b,j,0,:]) + bias_b[h, i/16, j/16]
 *   L_ij  = softcap * tanh(x_ij / softcap)   (softcap > 0)
 *         = x_ij                             (softcap == 0: no cap)
 *   out[b,i,h,:] = sum_j softmax_j(L_i.) * v[b,j,0,:]
 *
 *   q     [B, S, Hq, Dk]  dtype
 *   k     [B, S, 1, Dk]   dtype   (one K head shared by all query heads)
 *   v     [B, S, 1, Dv]   dtype   (one V head shared by all query heads)
 *   bias  float32 compact bias; batch item b reads the [Hq, P, P] block
 *         (P = ceil(S/16): a last cell of fewer than 16 positions still has
 *         its row and column) at  bias + (b / bias_group) * bias_batch_stride
 *         (elements).
 *         bias_batch_stride = 0 shares one bias by every item; bias_group is
 *         the number of consecutive items that share a block (e.g. 2 for a
 *         REF/ALT pair).
 *   out   [B, S, Hq, Dv]  dtype, written fully; must not overlap any input.
 *
 * Non-causal, no masks.  Limits (v1): B >= 1; 1 <= S <= 262144 (any
 * length: a sequence may end inside a 64-key tile); Hq == 8; Dk == 128; Dv == 128, or Dv == 192 (the released
 * checkpoint's value width, same page, section "Why stock FlashAttention
 * was not a drop-in replacement") for ABG_BF16 with softcap > 0;
 * bias_group >= 1 and bias_batch_stride == 0 or in [Hq*P^2, 2^40] (a
 * multiple of 4); scale finite; softcap finite and >= 0.  Any other request returns
 * ABG_ERR_UNSUPPORTED, ABG_ERR_SHAPE or ABG_ERR_VALUE before anything is
 * enqueued.
 *
 * Range (ABG_BF16 with softcap > 0): the bias cell scales the soft-cap's
 * exponential by 2^(2 log2(e) bias / softcap), clamped to 2^+-100, so a
 * bias beyond +-34.66 softcap counts as +-34.66 softcap: the logit is
 * saturated there and the result is unchanged, unless the pre-cap score
 * scale * q.k itself exceeds about 30.8 softcap in magnitude with the
 * opposite sign.
 */
abg_status abg_biased_mqa_fwd(const void* q, const void* k, const void* v,
                              const float* bias, void* out,
                              int64_t B, int64_t S, int64_t Hq, int64_t Dk, int64_t Dv,
                              int64_t bias_batch_stride, int64_t bias_group,
                              float scale, float softcap,
                              abg_dtype dtype, void* stream);

/* Workspace bytes that abg_biased_mqa_fwd_ex needs for kv_splits key ranges:
 * 0 for kv_splits == 1, else kv_splits * B * Sq * Hq * (Dv + 1) * 4: room for
 * float32 partial numerators and denominators, which is what the float32
 * kernel stores.  The bf16 kernels store each partial row normalised by its
 * key range's row sum, in bf16, and one float per row, so they use
 * Dv * 2 + 4 of each row's (Dv + 1) * 4 bytes.  -1 for out-of-range
 * arguments (any below 1, kv_splits above 64, or a size past INT64_MAX). */
int64_t abg_biased_mqa_fwd_workspace_bytes(int64_t B, int64_t Sq, int64_t Hq, int64_t Dv,
                                           int64_t kv_splits);

/* The attention of abg_biased_mqa_fwd for a block of query positions and
 * with the keys split over several workgroups.
 *
 *   q     [B, Sq, Hq, Dk]: positions q_offset .. q_offset + Sq - 1 of a
 *         sequence of Sk positions; out [B, Sq, Hq, Dv] likewise.
 *   k, v  [B, Sk, 1, Dk] / [B, Sk, 1, Dv]; bias compact for the whole
 *         sequence, [Hq, P, P] per block as above (P = ceil(Sk/16)).  Query i uses bias
 *         row (q_offset + i) / 16 -- the per-position bias of the logit
 *         equation (page "Making Full-Context AlphaGenome Fit on an RTX 3090",
 *         section "Why stock FlashAttention was not a drop-in replacement").
 *   kv_splits  the ceil(Sk/64) key tiles are divided into kv_splits equal ranges,
 *         each computed by its own workgroups; their partial softmax states
 *         are merged afterwards by the update equations of section "Online
 *         softmax, one block at a time" (with the cap the maximum is fixed,
 *         so the partial numerators and denominators simply add; without it
 *         each range's maximum is carried).  This keeps the GPU full
 *         when B * Sq / 32 is small (short sequences, one GPU's share of the
 *         queries).  kv_splits > 1 needs a device workspace of
 *         abg_biased_mqa_fwd_workspace_bytes(...) bytes, owned by the caller,
 *         16-byte aligned, not overlapping any tensor; its contents are
 *         scratch and are overwritten.  Calls that share a workspace must be
 *         ordered on one stream.
 *
 * Limits beyond abg_biased_mqa_fwd's: 1 <= Sq <= Sk; q_offset a multiple of 16 with
 * q_offset + Sq <= Sk; 1 <= kv_splits <= 64 dividing ceil(Sk/64);
 * kv_splits > 1 needs B * Sq * Hq * Dv / 4 < 2^39.
 * abg_biased_mqa_fwd(...) equals abg_biased_mqa_fwd_ex(..., NULL, 0, B, S, S,
 * 0, ..., 1, ...). */
abg_status abg_biased_mqa_fwd_ex(const void* q, const void* k, const void* v,
                                 const float* bias, void* out,
                                 void* workspace, int64_t workspace_bytes,
                                 int64_t B, int64_t Sq, int64_t Sk, int64_t q_offset,
                                 int64_t Hq, int64_t Dk, int64_t Dv,
                                 int64_t bias_batch_stride, int64_t bias_group,
                                 int64_t kv_splits, float scale, float softcap,
                                 abg_dtype dtype, void* stream);

/* Bytes of device scratch that abg_biased_mqa_fwd_ex_noalloc holds per GPU. */
#define ABG_NOALLOC_SCRATCH_BYTES (64LL << 20)

/* abg_biased_mqa_fwd_ex for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, meaning and results as abg_biased_mqa_fwd_ex
 * without the workspace: with kv_splits > 1 the partial numerators and
 * denominators go to a scratch array that the library itself holds, one copy
 * per GPU, from the first call on that GPU until the process ends
 * (ABG_NOALLOC_SCRATCH_BYTES = 64 MiB each).  The call allocates and frees
 * nothing.
 *
 * Limit: abg_biased_mqa_fwd_workspace_bytes(B, Sq, Hq, Dv, kv_splits) <=
 * ABG_NOALLOC_SCRATCH_BYTES; a larger request returns ABG_ERR_SHAPE before
 * anything is enqueued (at Dv = 128 that is B * Sq <= 4064 query positions
 * with kv_splits = 4, <= 2032 with 8: a 2048-position sequence in 4 key
 * ranges, or one GPU's 1024 of 8192 query positions in 8).  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents; each call writes all of the partials it
 * reads before reading them, so nothing needs clearing, but calls that may
 * overlap in time on one GPU (different streams, different threads without
 * ordering) race on the array and must be serialised by the caller, e.g. by
 * issuing them on one stream.  The first call on a device looks up the
 * array's device address (hipGetSymbolAddress); a failure there returns
 * ABG_ERR_DEVICE. */
abg_status abg_biased_mqa_fwd_ex_noalloc(const void* q, const void* k, const void* v,
                                         const float* bias, void* out,
                                         int64_t B, int64_t Sq, int64_t Sk, int64_t q_offset,
                                         int64_t Hq, int64_t Dk, int64_t Dv,
                                         int64_t bias_batch_stride, int64_t bias_group,
                                         int64_t kv_splits, float scale, float softcap,
                                         abg_dtype dtype, void* stream);

/* abg_biased_mqa_fwd_ex with the bias projected inside the attention kernel
 * from the pair representation, so that the compact bias is never written
 * out (page "Making Full-Context AlphaGenome Fit on an RTX 3090", section
 * "Why stock FlashAttention was not a drop-in replacement": the bias is the
 * pair representation projected per head, one value per 16 x 16 block).
 * Each workgroup projects, tile by tile, the cells its queries and keys
 * use: cell (p, c) of head h is sum_ch pair[p, c, ch] * weight[ch, h], bf16
 * products summed in float32 -- the value abg_pair_bias_project writes.
 *
 *   pair    [., P, P, C]  bf16, P = ceil(Sk/16); batch item b reads the
 *           block at  pair + (b / pair_group) * pair_batch_stride
 *           (elements; 0 shares one block by every item)
 *   weight  [C, Hq]       bf16
 *
 * Limits beyond abg_biased_mqa_fwd_ex's: dtype ABG_BF16 with softcap > 0;
 * Dv == 128 or 192; C == 128; pair_batch_stride 0 or in [P*P*C, 2^40] and a
 * multiple of 8;
 * 1 <= pair_group <= B; pair and weight 16-byte aligned and not overlapping
 * out or the workspace.  kv_splits, q_offset and the workspace work as for
 * abg_biased_mqa_fwd_ex. */
abg_status abg_pair_biased_mqa_fwd(const void* q, const void* k, const void* v,
                                   const void* pair, const void* weight, void* out,
                                   void* workspace, int64_t workspace_bytes,
                                   int64_t B, int64_t Sq, int64_t Sk, int64_t q_offset,
                                   int64_t Hq, int64_t Dk, int64_t Dv, int64_t C,
                                   int64_t pair_batch_stride, int64_t pair_group,
                                   int64_t kv_splits, float scale, float softcap,
                                   abg_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ABG_H */
