/*
 * latent_tail.h -- C ABI of liblatenttail.so: the latent-MoE output tail on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages this library follows):
 *   [PR51253]  prhub report of vLLM PR #51253, "[ROCm][Perf] Kimi-K3 Shard
 *              Latent MoE up-projection for ROCm path".
 *   [PR50383]  prhub report of vLLM PR #50383 (tiered tail of the K3
 *              latent-MoE runner; column-parallel `_shard_up_proj_tail`).
 *   [PR50593]  prhub report of vLLM PR #50593, "[Kimi-K3][AMD] Fuse AttnRes
 *              state updates and norms" (bf16 storage round trip, fp32 norm
 *              variance, token-count launch heuristic, HIP graph replay).
 *
 * Conventions for every entry point:
 *   - bf16 tensors are passed as pointers to their 16-bit patterns.
 *   - Every pointer is a DEVICE pointer on the current HIP device, owned by
 *     the caller; the library keeps no pointer after a call returns.
 *   - Calls are asynchronous and stream-ordered on `stream` (a hipStream_t;
 *     NULL means the default stream; hipStreamPerThread is the calling
 *     thread's own stream).  No call synchronises the device or copies
 *     between host and device; only lt_release_scratch synchronises, and
 *     growing the internal scratch (see lt_reserve) calls hipMalloc.
 *   - The library never reads or clears the caller's pending HIP error
 *     state: launch failures come back as LT_ERR_HIP from the launch's own
 *     status.
 *   - Argument errors are reported before anything is launched; in that case
 *     no device memory has been read or written.
 *   - The library is thread-safe.  Results are bit-identical from run to run
 *     for the same arguments (no atomics, fixed reduction order).
 */
#ifndef LATENT_TAIL_H
#define LATENT_TAIL_H

#include <stdint.h>

#if defined(LT_BUILDING_LIBRARY)
#define LT_API __attribute__((visibility("default")))
#else
#define LT_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define LT_OK 0
#define LT_ERR_INVALID_ARG 1   /* an argument is out of range, NULL or overlaps */
#define LT_ERR_UNSUPPORTED 2   /* legal in principle, outside what this library handles */
#define LT_ERR_NO_MEMORY 3     /* scratch could not be (re)allocated */
#define LT_ERR_HIP 4           /* a HIP call or kernel launch failed */
#define LT_ERR_SCRATCH_LIMIT 5 /* lt_latent_tail_noalloc: T*L beyond its fixed scratch */

/* Largest latent width the kernels accept (the model's is 1024). */
#define LT_MAX_L 2048

/*
 * lt_latent_tail -- one GPU's share of the latent-MoE output tail.
 *
 * Defined by [PR50383 Key source snippets, `_shard_up_proj_tail`] and the
 * expected value of [PR51253 Key source snippets, `_check_matches_replicated`],
 * on one GPU: the tensor-parallel all-reduce of the routed latent becomes a
 * local sum over `n_partials` partials, and the final all-reduce that stitches
 * the column shards is left to the caller.  For t < T and 0 <= j < n:
 *
 *   s[t,k]  = bf16( sum_p partials[p][t][k] )               (fp32 sum)
 *   y[t,k]  = bf16( s[t,k] * rsqrt(mean_k s[t,k]^2 + eps) * norm_w[k] )
 *             (fp32 variance and scaling; y = s when norm_w == NULL)
 *   out[t][c0+j] = bf16( out[t][c0+j] + sum_k y[t,k] * W[c0+j][k] )
 *             (fp32 accumulation, one rounding: the beta-add of `addmm_`)
 *
 * Every other element of `out` -- columns outside [c0, c0+n), the padding
 * between H and ld_out, rows >= T -- is left bit-identical
 * ([PR51253 Key source snippets, `_check_writes_only_its_own_shard`]).
 * alpha is 1: the pages require a routed scaling factor of 1
 * ([PR51253 Implementation, item 2]).
 *
 * Arguments:
 *   partials    [n_partials][T][L] bf16, packed contiguous; 16-byte aligned.
 *   n_partials  >= 1.
 *   T           tokens, >= 0.
 *   L           latent width, 8 <= L <= LT_MAX_L, L % 8 == 0.
 *   norm_w      [L] bf16 RMSNorm weight, 16-byte aligned, or NULL to skip
 *               the norm ([PR50383 Key source snippets]: the norm is optional).
 *   eps         >= 0 and finite; added to the mean square inside the root.
 *   W           [H][L] bf16 row-major: the full replicated up-projection
 *               weight (rows = hidden index); 16-byte aligned.
 *   H           hidden width = rows of W = logical columns of out, >= 1.
 *   c0, n       column window: 0 <= c0, 0 <= n, c0 + n <= H.  Any window is
 *               legal (no divisibility requirement).
 *   out         [T][ld_out] bf16 shared-expert partial, updated in place on
 *               the window only; 2-byte aligned.  Must not overlap
 *               partials, norm_w or W.
 *   ld_out      row stride of out in elements, ld_out >= H.
 *   stream      hipStream_t (NULL = default stream).
 *
 * Returns LT_OK, LT_ERR_INVALID_ARG (NULL pointer where data is needed,
 * out-of-range size or window, non-finite or negative eps, out overlapping an
 * input), LT_ERR_UNSUPPORTED (L outside 8..LT_MAX_L or not a multiple of 8, a
 * misaligned pointer), LT_ERR_NO_MEMORY (the scratch of the T > skinny path
 * could not grow, or would have to grow while `stream` is being captured into
 * a graph; calls with one partial and norm_w == NULL use no scratch), or
 * LT_ERR_HIP.  T == 0 or n == 0 returns LT_OK with nothing
 * launched ([PR50383 Key source snippets]: an empty batch is a legal state).
 */
LT_API int lt_latent_tail(const void *partials, int n_partials, int64_t T, int64_t L,
                   const void *norm_w, float eps, const void *W, int64_t H,
                   int64_t c0, int64_t n, void *out, int64_t ld_out, void *stream);

/*
 * lt_latent_tail_residual -- lt_latent_tail followed by the decoder layer's
 * residual update, fused into the tail's epilogue.
 *
 * [PR50593 Key source snippets, `forward_attn_residual`]: after the MLP the
 * layer adds the MLP output to the running prefix sum (a bf16 add, one
 * rounding of the exact sum).  With the tail's result as the MLP output:
 * after updating `out` exactly as lt_latent_tail does, for t < T and
 * 0 <= j < n
 *
 *   resid[t][c0+j] = bf16( prefix[t][c0+j] + out[t][c0+j] )
 *
 * using the updated (already rounded) out, so the result equals running the
 * tail and then the separate add.  The add of the pages happens after the
 * final all-reduce of `out`; this form is for callers that own the finished
 * window (one GPU, or the full window after their own collective).
 *
 * Extra arguments (all others as in lt_latent_tail):
 *   prefix      [T][ld_prefix] bf16, read on the window; 2-byte aligned.
 *   ld_prefix   row stride of prefix in elements, >= c0 + n.
 *   resid       [T][ld_resid] bf16, written on the window only; every other
 *               element is left bit-identical.  May be `prefix` itself (with
 *               ld_resid == ld_prefix) for an in-place update; must not
 *               otherwise overlap prefix, and must not overlap partials,
 *               norm_w, W or out.  prefix must not overlap out.
 *   ld_resid    row stride of resid in elements, >= c0 + n.
 *
 * Returns the codes of lt_latent_tail; LT_ERR_INVALID_ARG also for a NULL
 * prefix or resid, a stride below c0 + n or an overlap listed above, and
 * LT_ERR_UNSUPPORTED for an odd address.  T == 0 or n == 0 returns LT_OK
 * with nothing launched.
 */
LT_API int lt_latent_tail_residual(const void *partials, int n_partials, int64_t T, int64_t L,
                                   const void *norm_w, float eps, const void *W, int64_t H,
                                   int64_t c0, int64_t n, void *out, int64_t ld_out,
                                   const void *prefix, int64_t ld_prefix, void *resid,
                                   int64_t ld_resid, void *stream);

/*
 * lt_latent_tail_noalloc -- lt_latent_tail for callers that cannot allocate
 * device memory: code being captured into a HIP graph without a prior
 * lt_reserve, tight serving loops, and harnesses that forbid hipMalloc.
 * Same arguments, results (bit for bit) and status codes as lt_latent_tail;
 * it never calls hipMalloc or hipFree, nor any allocating library routine.
 *
 * The large-token path's [T][L] bf16 latent goes to a fixed device array of
 * LT_NOALLOC_MAX_LATENT elements (16 MiB), one per GPU, held until the
 * process ends.  A call that takes that path with T * L larger than
 * LT_NOALLOC_MAX_LATENT returns LT_ERR_SCRATCH_LIMIT before anything is
 * launched (use lt_latent_tail there).  The weight-streaming path (T <=
 * skinny_max) and one partial with norm_w == NULL use no scratch and have
 * no such limit.  Every element of the array that a call reads is written
 * earlier by the same call, so no state carries over between calls.
 *
 * All calls on one GPU share its array: calls that may overlap on one GPU
 * (different streams without an ordering between them, or replays of
 * captured calls running concurrently) race on it and give wrong results.
 * Calls on one stream are ordered and safe, from any number of threads.
 * The first call on a device resolves the array's address on that device.
 */
#define LT_NOALLOC_MAX_LATENT (8u * 1024u * 1024u)
LT_API int lt_latent_tail_noalloc(const void *partials, int n_partials, int64_t T, int64_t L,
                                  const void *norm_w, float eps, const void *W, int64_t H,
                                  int64_t c0, int64_t n, void *out, int64_t ld_out,
                                  void *stream);

/*
 * lt_attn_res_zero_block -- the AttnRes state update and output RMSNorm of a
 * decoder layer, for the case of no valid blocks.
 *
 * [PR50593 Implementation, item 1]: the fused AttnRes kernel adds the delta
 * to the prefix sum in fp32, rounds the sum to bf16 storage precision and
 * uses it as the residual source from then on (the prefix is updated in
 * place), writes it to the block-residual slot of a block-write layer, and
 * applies the output RMSNorm with its variance in fp32; with zero blocks the
 * softmax has one source and the aggregated value equals the prefix.
 * [PR50593 Key source snippets, `forward_attn_residual`]: the delta stands
 * for the unfused `prefix_sum + hidden_states`.  For t < T, h < H:
 *
 *   p'[t][h]  = bf16( prefix[t][h] + delta[t][h] )   (= prefix if delta NULL)
 *   prefix[t][h] = p'[t][h]                           (only when delta != NULL)
 *   block_residual[t][block_idx][h] = p'[t][h]         (only when block_idx >= 0)
 *   out[t][h] = bf16( p'[t][h] * rsqrt(mean_h p'[t][.]^2 + eps) * norm_w[h] )
 *               (fp32 variance and scaling; out = p' when norm_w == NULL)
 *
 * The softmax aggregation over one or more valid blocks (the layer's
 * res_proj and res_norm) is not part of this call.
 *
 * Arguments (all bf16 bit patterns, device pointers, packed row-major,
 * 16-byte aligned):
 *   prefix          [T][H], read; updated in place when delta != NULL.
 *   delta           [T][H] or NULL (the pages' HAS_DELTA switch).
 *   T               tokens, >= 0.
 *   H               hidden width, H % 8 == 0, 8 <= H <= LT_ATTN_RES_MAX_H.
 *   block_residual  [T][num_slots][H]; only slot block_idx of each token is
 *                   written, every other element is left bit-identical.
 *                   May be NULL when block_idx == -1.
 *   num_slots       slots per token of block_residual, >= 0.
 *   block_idx       slot to write, -1 for none (the pages' WRITE_BLOCK
 *                   switch), < num_slots.
 *   norm_w          [H] output-norm weight, or NULL (APPLY_OUTPUT_NORM).
 *   eps             >= 0 and finite; added to the mean square inside the root.
 *   out             [T][H], written.
 *   stream          hipStream_t (NULL = default stream).
 * out must not overlap any other buffer; block_residual must not overlap
 * prefix, delta or norm_w; prefix must not overlap delta or norm_w.
 *
 * Returns LT_OK, LT_ERR_INVALID_ARG (range, NULL or overlap), LT_ERR_UNSUPPORTED
 * (H not a multiple of 8 or above LT_ATTN_RES_MAX_H, a misaligned pointer,
 * T above 2^31 - 1) or LT_ERR_HIP; errors are returned before any launch.
 * T == 0 returns LT_OK with nothing launched.
 */
#define LT_ATTN_RES_MAX_H 8192
LT_API int lt_attn_res_zero_block(void *prefix, const void *delta, int64_t T, int64_t H,
                                  void *block_residual, int64_t num_slots, int64_t block_idx,
                                  const void *norm_w, float eps, void *out, void *stream);

/*
 * lt_status_string -- human-readable name of a status code (static storage,
 * never NULL).  The pages' runner falls back silently, with one warning, when
 * a precondition of the sharded tail fails ([PR51253 Implementation, item 2];
 * [PR51253 Risks and impact, item 2] notes that this hides the lost
 * optimisation), and [PR50383 Risks and impact] flags a missing divisibility
 * check; a library cannot fall back to a path it does not own, so every
 * failed precondition is a status code the caller can name and act on.
 */
LT_API const char *lt_status_string(int status);

/*
 * lt_reserve -- pre-size the library-owned scratch used by calls with
 * T > skinny_max on `stream` of the current device: a [max_T][L] bf16 latent
 * buffer (calls with one partial and norm_w == NULL multiply the partial in
 * place and need none).  Calls that then fit never allocate, so they can be
 * captured into a HIP graph ([PR50593 Implementation, item 4]: graph capture
 * and replay at varying shapes is part of the validation there).  The buffer
 * belongs to (device, stream) -- for hipStreamPerThread to (device, calling
 * thread) -- and is shared by every call on that stream.
 *
 * Lifetime: a buffer is never freed while the library is loaded, except by
 * lt_release_scratch.  When a later call on the same stream (outside capture)
 * needs more, a larger buffer takes over and the old one is kept, so graphs
 * captured earlier stay valid and keep using the buffer they captured.  A
 * call under capture that would need to grow the buffer returns
 * LT_ERR_NO_MEMORY instead of allocating.  Replays of graphs captured on one
 * stream share that stream's buffer with each other and with eager calls, so
 * they must not run concurrently (stream order serialises them).
 * Returns LT_OK, LT_ERR_INVALID_ARG, LT_ERR_NO_MEMORY or LT_ERR_HIP.
 */
LT_API int lt_reserve(int64_t max_T, int64_t L, void *stream);

/*
 * lt_release_scratch -- synchronise the current device and free every scratch
 * buffer the library holds on it (current and replaced ones).  Every graph
 * that captured a call of the large-token path on this device becomes
 * invalid: replaying it afterwards is an error of the caller.  Needed only to
 * return the memory before process exit.  The lifetime rule exists for the
 * graph replay of [PR50593 Implementation, item 4].
 */
LT_API int lt_release_scratch(void);

/*
 * lt_set_skinny_max_tokens -- the token-count dispatcher's threshold
 * ([PR50383 Implementation, item 1]: the tail variant is chosen from the token
 * count alone).  Calls with T <= t take the weight-streaming path, the others
 * the sum+RMSNorm kernel followed by the MFMA GEMM.  t < 0 restores the
 * default (64, or the environment variable LT_SKINNY_MAX_T if set).  Returns
 * the previous threshold.  Process-wide.
 */
LT_API int64_t lt_set_skinny_max_tokens(int64_t t);

/* Current threshold (see lt_set_skinny_max_tokens; [PR50383 Implementation,
 * item 1]). */
LT_API int64_t lt_get_skinny_max_tokens(void);

/*
 * lt_path_for -- which path a call with these sizes takes:
 * 0 = nothing launched (T == 0 or n == 0; [PR50383 Key source snippets,
 * `_select_tail_tier`] treats a positive token count as the precondition of
 * every tier), 1 = weight-streaming (skinny), 2 = sum+RMSNorm kernel then
 * MFMA GEMM (the GEMM alone for one partial with norm_w == NULL).  The
 * tier is a function of the token count alone, as there.  Host-only,
 * launches nothing.
 */
LT_API int lt_path_for(int64_t T, int64_t n);

/*
 * lt_set_kernel_events -- per-kernel timing hook, the measurement that an
 * operator benchmark takes ([PR50593 Implementation, item 4] reports operator
 * latencies on gfx950).  While set (non-NULL) for the calling thread, every
 * lt_latent_tail / lt_latent_tail_residual call made from that thread records
 * the hipEvent_t `before` on its stream immediately before launching its
 * projection kernel (k_skinny, or the GEMM on the large-token path) and
 * `after` immediately after it, so the caller can time that kernel alone with
 * hipEventElapsedTime.  Pass NULL, NULL to switch it off (the default).
 * The setting is per host thread; calls from other threads are unaffected.
 * Returns LT_OK.
 */
LT_API int lt_set_kernel_events(void *before, void *after);

/* Library version string, e.g. "liblatenttail 0.2.0 gfx950".  No passage
 * defines it; it names the build in logs. */
LT_API const char *lt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LATENT_TAIL_H */
