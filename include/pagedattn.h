/*
 * libpagedattn -- paged-KV varlen flash attention for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Every pointer argument documented
 * as "device" is a HIP device pointer; "host" pointers are ordinary host
 * memory.  The library allocates no memory, keeps no global state and never
 * synchronises: each device-side call enqueues its kernels on the caller's
 * `stream` and returns at once, so the calls can be captured into a HIP
 * graph.  All argument checks run on the host BEFORE any HIP call; a call
 * that returns an error has launched nothing.
 *
 * Data types: Q/K/V/out are bf16 (stored as 16-bit words), lse is fp32.
 * The KV cache is one contiguous tensor laid out (2, num_blocks, block_size,
 * num_kv_heads, head_size): plane 0 holds keys, plane 1 values (the
 * FlashAttention backend class hierarchy in "FlashAttention 在 vLLM 中的实现分析",
 * section 2.1, and the `kv_cache.unbind(dim=0)` split of section 4).
 *
 * Semantics fixed where the pages are silent:
 *   - GQA: query head h reads KV head h / (num_heads / num_kv_heads).
 *   - causal masking is bottom-right aligned: query i (0-based) of a sequence
 *     with Lq queries and Lk keys sees keys j <= i + Lk - Lq.
 *   - lse is the natural-log log-sum-exp of the scaled scores (the backend
 *     abstraction page warns that ln and log2 LSE must not be mixed).
 *   - a query that sees no key gets out = 0 and lse = -inf.
 */
#ifndef PAGEDATTN_H_
#define PAGEDATTN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, inconsistent lengths */
  PA_ERR_UNSUPPORTED = 2,        /* a valid configuration the library does not instantiate */
  PA_ERR_WORKSPACE_TOO_SMALL = 3,/* worklist or workspace smaller than the plan needs */
  PA_ERR_HIP = 4                 /* a kernel launch failed (hipGetLastError) */
} pa_status;

/* Static string naming a status code. */
const char* pa_status_str(pa_status s);

/* Library version, (major << 16) | minor.  Major 5 added num_cus to
 * pa_attn_params (plans for 256 compute units are unchanged).  Major 4 added
 * kv_cache_fp8 to pa_attn_params (the work list is unchanged, version 3).  Major 3: tiled
 * work items of up to PA_TILED_ROWS_WIDE rows, reported in
 * pa_plan_info.tiled_rows (work-list version 3).  Major 2 added the sliding window to pa_attn_params and the
 * plan info, and the sequence's first token to the reduce items. */
int32_t pa_version(void);

/* Head sizes with a compiled kernel. */
#define PA_NUM_HEAD_SIZES 3
extern const int32_t pa_supported_head_sizes[PA_NUM_HEAD_SIZES]; /* {64, 128, 256} */

/* Shape of one attention call.
 *   batch              number of sequences B
 *   num_heads          query heads H
 *   num_kv_heads       KV heads Hkv; H % Hkv == 0
 *   head_size          D, one of pa_supported_head_sizes
 *   block_size         BS, tokens per cache block; a positive multiple of 16
 *                      (the FlashAttention backend rejects other sizes:
 *                      "FlashAttention と FlashInfer" page, 境界と失敗)
 *   num_blocks         NB, physical blocks in the cache
 *   max_blocks_per_seq columns of block_table a sequence may use
 *   block_table_stride int32 elements between block_table rows; 0 means
 *                      max_blocks_per_seq (a column slice such as the cascade
 *                      suffix view block_table[:, k:] keeps the full stride)
 *   causal             0 or 1
 *   scale              softmax scale applied to q.k (fp32, finite, > 0) */
typedef struct {
  int32_t batch;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t head_size;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t block_table_stride;
  int32_t causal;
  float scale;
  int32_t sliding_window;   /* 0: none; W > 0 (causal only): query i sees keys
                               i + Lk - Lq - (W - 1) .. i + Lk - Lq */
  int32_t kv_cache_fp8;     /* 0: bf16 cache, 1: E4M3 cache (pa_varlen_fwd_fp8).
                               Read by the planner only: in a launch with no
                               tiled items it cuts key ranges finer for the
                               smaller cache.  A plan is valid with either
                               cache; only its split count differs.  Other
                               values: PA_ERR_INVALID_ARGUMENT */
  int32_t num_cus;          /* compute units the planner schedules for (read
                               by the planner only): 0 means
                               PA_PLAN_TARGET_CUS, one whole MI355X; a
                               partitioned or smaller device passes its own
                               count (the binding reads it from the device).
                               Negative or above 65536:
                               PA_ERR_INVALID_ARGUMENT */
} pa_attn_params;

/* ------------------------------------------------------------------------
 * pa_plan_varlen -- host-side scheduling metadata (the ahead-of-time
 * schedule of "FlashAttention 在 vLLM 中的实现分析", section 7: computed from
 * batch size, query/key lengths, head counts, head size and page size, so
 * the kernels run a fixed, deterministic work list).
 *
 * Host only; makes no HIP call.  Reads host mirrors of cu_seqlens_q [B+1]
 * (cu[0] == 0, non-decreasing) and seqused_k [B] (0 <= Lk <=
 * max_blocks_per_seq * block_size).
 *   force_splits     0: the planner chooses how many KV splits each work unit
 *                    gets (for p->num_cus compute units, PA_PLAN_TARGET_CUS
 *                    when that is 0);
 *                    n >= 1: every unit is split into n ranges (ranges
 *                    shorter than one key tile are merged) -- for tests of
 *                    the split-KV reduction
 *   host_worklist    receives the int32 work list (layout below); may be
 *                    NULL to query sizes only
 *   worklist_capacity_bytes  size of host_worklist
 *   info             receives item counts and the worklist / workspace sizes
 * The caller copies the work list unchanged to device memory and passes it,
 * with `info`, to pa_varlen_fwd.
 * Errors: PA_ERR_INVALID_ARGUMENT (bad params or lengths),
 * PA_ERR_UNSUPPORTED (head size), PA_ERR_WORKSPACE_TOO_SMALL (capacity).
 * ------------------------------------------------------------------------ */
#define PA_PLAN_TARGET_CUS 256

typedef struct {
  int32_t num_small_items;   /* items for the small-row (decode) kernel     */
  int32_t num_tiled_items;   /* items for the tiled kernels (<= tiled_rows)  */
  int32_t num_reduce_items;  /* split-KV merges                              */
  int32_t num_partial_rows;  /* fp32 partial rows held in the workspace      */
  int32_t max_reduce_rows;   /* most rows of any reduce item                 */
  int32_t batch, num_heads, num_kv_heads, head_size, causal, num_tokens;
  int32_t sliding_window;    /* as planned (item key ranges start at the window) */
  int32_t tiled_rows;        /* rows per tiled row block: PA_TILED_ROWS, or
                                PA_TILED_ROWS_WIDE (8-wave workgroups sharing
                                each K/V tile) */
  size_t worklist_bytes;
  size_t workspace_bytes;
} pa_plan_info;

pa_status pa_plan_varlen(const pa_attn_params* p,
                         const int32_t* host_cu_seqlens_q,
                         const int32_t* host_seqused_k,
                         int32_t force_splits,
                         int32_t* host_worklist, size_t worklist_capacity_bytes,
                         pa_plan_info* info);

/* ------------------------------------------------------------------------
 * pa_upload_words -- copy n_words int32 words (a work list written by
 * pa_plan_varlen) from pinned host memory to device memory with a kernel on
 * `stream`.  A copy-engine transfer on the same stream makes the next kernel
 * wait for the engine's completion signal (25-40 us measured on MI355X with
 * a 100 KB work list); this copy is an ordinary kernel of the stream, so the
 * attention launch behind it starts as after any other kernel.
 *   host_src   pinned host memory mapped for the device (hipHostMalloc,
 *              torch pin_memory()), 16-byte aligned; the caller keeps it
 *              unchanged until the copy has run (an event after this call)
 *   dev_dst    device memory, 16-byte aligned, n_words int32
 * Errors: PA_ERR_INVALID_ARGUMENT (null pointers, misalignment, n_words < 0,
 * or host_src not device-mapped pinned memory), PA_ERR_HIP (launch).
 * ------------------------------------------------------------------------ */
pa_status pa_upload_words(const int32_t* host_src, int32_t* dev_dst, int64_t n_words,
                          hipStream_t stream);

/* ------------------------------------------------------------------------
 * pa_cascade_split -- host-side metadata of the two cascade passes
 * ("FlashAttention 在 vLLM 中的实现分析", section 6.3): a prefix pass in
 * which all num_tokens queries form ONE pseudo-sequence attending
 * non-causally to the common_prefix_len shared keys addressed by block-table
 * row 0, and a suffix pass in which every sequence attends causally to its
 * own remaining keys through block_table[:, common_prefix_len/BS:].
 *
 *   p                  the full (single-pass) problem; must be causal
 *   common_prefix_len  > 0, a multiple of block_size, and <= Lk_b - Lq_b for
 *                      every sequence (each query comes after the prefix)
 *   host_cu_seqlens_q, host_seqused_k   host mirrors [B+1], [B]
 * Outputs (host):
 *   prefix_p, suffix_p     params of the two passes
 *   prefix_cu_seqlens_q    [2] = {0, num_tokens}
 *   prefix_seqused_k       [1] = {common_prefix_len}
 *   suffix_seqused_k       [B] = seqused_k - common_prefix_len
 *   block_table_col0       column offset of the suffix view
 * The caller uploads the three small arrays, plans and runs each pass with
 * pa_varlen_fwd (prefix with block_table, suffix with block_table +
 * *block_table_col0) and merges with pa_merge_attn_states.  Host only.
 * ------------------------------------------------------------------------ */
pa_status pa_cascade_split(const pa_attn_params* p, int32_t common_prefix_len,
                           const int32_t* host_cu_seqlens_q, const int32_t* host_seqused_k,
                           pa_attn_params* prefix_p, pa_attn_params* suffix_p,
                           int32_t* prefix_cu_seqlens_q, int32_t* prefix_seqused_k,
                           int32_t* suffix_seqused_k, int32_t* block_table_col0);

/* ------------------------------------------------------------------------
 * pa_cascade_decide -- the host cascade decision ("FlashAttention 在 vLLM 中
 * 的实现分析", section 6.2, use_cascade_attention; section 6.1, a prefix shared
 * by every request).  Host only; reads nothing on the device.
 *
 *   p                  the full (single-pass) problem
 *   host_cu_seqlens_q, host_seqused_k   host mirrors [B+1], [B]
 *   host_block_table   host int32 [B, stride] (stride = p->block_table_stride,
 *                      or p->max_blocks_per_seq when that is 0)
 *   kv_bytes_per_elem  2 for the bf16 cache, 1 for the E4M3 cache
 * Outputs:
 *   common_prefix_len  block_size x the number of leading block-table
 *                      columns whose entry is the same physical block in
 *                      every row, cut to what every query token comes after
 *                      (<= seqused_k[b] - Lq_b, rounded down to whole
 *                      blocks); 0 when B < 2 or nothing is shared
 *   use_cascade        1 when the cascade path (pa_cascade_split + two
 *                      passes + pa_merge_attn_states) should be taken:
 *                      causal, common_prefix_len >= 256, B >= 8 (the
 *                      section's thresholds; ALiBi, sliding windows and DCP
 *                      do not exist here), and the cost model below expects
 *                      it to be faster than the single pass; else 0.
 * Cost model (this library's stand-in for the section's comparison of the
 * two paths' CTA counts): both paths are planned with pa_plan_varlen and
 * their launches priced with times fitted to this library's kernels on
 * MI355X: small-row work 7.8 us + KV bytes / 6.5 TB/s, with the single
 * pass's repeated reads of the shared blocks at 13.6 TB/s while the prefix's
 * K/V fit in 128 MB (they come from the last-level cache); tiled work
 * 10.8 us + 1.15 us per 64-key tile of its longest item per 512 items; a
 * split reduce 4.2 us; the merge 3.4 us.
 * Errors: PA_ERR_INVALID_ARGUMENT (bad params or lengths, NULL pointers).
 * ------------------------------------------------------------------------ */
pa_status pa_cascade_decide(const pa_attn_params* p, const int32_t* host_cu_seqlens_q,
                            const int32_t* host_seqused_k, const int32_t* host_block_table,
                            int32_t kv_bytes_per_elem, int32_t* common_prefix_len,
                            int32_t* use_cascade);

/* ------------------------------------------------------------------------
 * pa_reshape_and_cache -- scatter the new tokens' keys and values into the
 * paged cache ("FlashAttention 在 vLLM 中的实现分析", section 4.2, the
 * do_kv_cache_update step, and the helper-kernel table of section 8.2).
 *
 *   key, value        device bf16 [num_tokens, num_kv_heads, head_size];
 *                     head_size contiguous, heads contiguous; consecutive
 *                     tokens key_row_stride / value_row_stride elements
 *                     apart (>= num_kv_heads * head_size, multiple of 8)
 *   kv_cache          device bf16 (2, num_blocks, block_size, Hkv, D), updated
 *                     in place
 *   slot_mapping      device int64 [num_tokens]; token t goes to block
 *                     slot / block_size, offset slot % block_size; a negative
 *                     slot skips the token, and so does a slot >= num_blocks
 *                     * block_size (the kernel never writes outside the
 *                     cache).  Slots must be distinct (not checked).
 * Bit copy: the written bits equal the input bits.
 * num_tokens == 0 launches nothing and returns PA_OK.
 * ------------------------------------------------------------------------ */
pa_status pa_reshape_and_cache(const void* key, const void* value,
                               int64_t key_row_stride, int64_t value_row_stride,
                               void* kv_cache, const int64_t* slot_mapping,
                               int32_t num_tokens, int32_t num_kv_heads, int32_t head_size,
                               int32_t num_blocks, int32_t block_size, hipStream_t stream);

/* ------------------------------------------------------------------------
 * pa_varlen_fwd -- paged varlen flash attention forward
 * ("FlashAttention 在 vLLM 中的实现分析", section 4 standard call and section 5:
 * q packed [num_tokens, H, D] and delimited by cu_seqlens_q, keys of
 * sequence b are its first seqused_k[b] cache positions, addressed through
 * block_table[b][j / block_size]; tiling with an online softmax, section
 * 1.1; split-KV partials merged by LSE, section 1.3 num_splits).
 *
 *   p                 shape, as given to pa_plan_varlen
 *   plan              the info pa_plan_varlen filled for these lengths
 *   worklist          device copy of the planned work list (plan->worklist_bytes)
 *   q                 device bf16 [num_tokens, H, D], contiguous
 *   kv_cache          device bf16 (2, NB, BS, Hkv, D), contiguous
 *   cu_seqlens_q      device int32 [B+1]
 *   seqused_k         device int32 [B]
 *   block_table       device int32 [B, max_blocks_per_seq]; entries at
 *                     index < ceil(seqused_k[b] / BS) must be in [0, NB);
 *                     the rest are never read.  An entry outside [0, NB)
 *                     is not followed: its keys and values read as zeros
 *                     (no access outside the cache; the result for that
 *                     sequence is then meaningless)
 *   num_tokens        cu_seqlens_q[B]
 *   out               device bf16 [num_tokens, H, D]; every element is written
 *   lse               device fp32 [num_tokens, H] (natural log), or NULL
 *   workspace         device scratch, >= plan->workspace_bytes, 256-byte
 *                     aligned (may be NULL when that is 0)
 * The device lengths must equal the host mirrors given to the planner.
 * Errors: PA_ERR_INVALID_ARGUMENT (null pointer, plan/params mismatch),
 * PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE_TOO_SMALL, PA_ERR_HIP.
 * ------------------------------------------------------------------------ */
pa_status pa_varlen_fwd(const pa_attn_params* p, const pa_plan_info* plan,
                        const int32_t* worklist,
                        const void* q, const void* kv_cache,
                        const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                        const int32_t* block_table,
                        int32_t num_tokens, void* out, float* lse,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * FP8 KV cache.  The pages list an fp8 / fp8_e4m3 KV cache with per-head
 * quantisation scales among the FlashAttention-3 and FlashInfer backend
 * features ("FlashAttention 在 vLLM 中的实现分析", the backend section and its
 * feature table; the backend-abstraction page, kv_cache_dtype) without a
 * formula; these two calls take the plain reading:
 *   format  OCP 8-bit float E4M3 (1 sign, 4 exponent bits with bias 7,
 *           3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN,
 *           largest finite 448), one byte per element, same (2, NB, BS, Hkv,
 *           D) layout as the bf16 cache;
 *   write   code = E4M3(fp32(x) / k_scale[h]) (v_scale[h] for values), the
 *           division in IEEE fp32, rounding to nearest with ties to the even
 *           code, saturating to +-448, NaN -> 0x7F;
 *   read    key = E4M3 value * k_scale[h], value = E4M3 value * v_scale[h].
 *
 * pa_reshape_and_cache_fp8: as pa_reshape_and_cache, into an E4M3 cache.
 *   kv_cache          device uint8 (2, NB, BS, Hkv, D), updated in place
 *   k_scale, v_scale  device fp32 [num_kv_heads], > 0 and finite
 *   head_size         a multiple of 16
 * Same errors as pa_reshape_and_cache.
 * ------------------------------------------------------------------------ */
pa_status pa_reshape_and_cache_fp8(const void* key, const void* value,
                                   int64_t key_row_stride, int64_t value_row_stride,
                                   void* kv_cache, const int64_t* slot_mapping,
                                   const float* k_scale, const float* v_scale,
                                   int32_t num_tokens, int32_t num_kv_heads, int32_t head_size,
                                   int32_t num_blocks, int32_t block_size, hipStream_t stream);

/* pa_varlen_fwd_fp8: pa_varlen_fwd over an E4M3 cache (uint8, same layout),
 * with k_scale / v_scale the device fp32 [num_kv_heads] scales the cache was
 * written with.  Plan, work list and workspace are those of pa_varlen_fwd
 * (the same pa_plan_varlen call); q, out and lse are unchanged.  K and V
 * are widened to bf16 exactly; the scales are applied in fp32 (k_scale to
 * the scores, v_scale to the output).  Same errors as pa_varlen_fwd, and
 * PA_ERR_INVALID_ARGUMENT for a NULL scale pointer. */
pa_status pa_varlen_fwd_fp8(const pa_attn_params* p, const pa_plan_info* plan,
                            const int32_t* worklist,
                            const void* q, const void* kv_cache,
                            const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                            const int32_t* block_table,
                            const float* k_scale, const float* v_scale,
                            int32_t num_tokens, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * pa_varlen_fwd_ex -- pa_varlen_fwd with the options of the FA3 path the
 * pages list ("FlashAttention 在 vLLM 中的实现分析", section 1.2: the s_aux
 * argument, a learnable attention sink; the FP8 KV cache above):
 *
 *   kv_dtype   PA_KV_BF16 (the bf16 cache) or PA_KV_E4M3 (the E4M3 cache,
 *              with k_scale / v_scale as for pa_varlen_fwd_fp8)
 *   s_aux      NULL, or device fp32 [num_heads]: one sink logit per query
 *              head, in the units of the scaled scores, that joins each
 *              row's softmax denominator and carries no value:
 *                out = sum_j e^{s_j} v_j / (sum_j e^{s_j} + e^{s_aux[h]}),
 *                lse = ln(sum_j e^{s_j} + e^{s_aux[h]});
 *              a row that sees no key gets out = 0, lse = s_aux[h].  In a
 *              cascade give it to one of the two passes only.
 * The sliding window is a shape parameter (pa_attn_params.sliding_window)
 * and must equal the planned one.  Same errors as pa_varlen_fwd.
 * ------------------------------------------------------------------------ */
#define PA_KV_BF16 0
#define PA_KV_E4M3 1

typedef struct {
  int32_t kv_dtype;
  const float* k_scale;
  const float* v_scale;
  const float* s_aux;
} pa_fwd_options;

pa_status pa_varlen_fwd_ex(const pa_attn_params* p, const pa_plan_info* plan,
                           const int32_t* worklist,
                           const void* q, const void* kv_cache,
                           const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                           const int32_t* block_table, const pa_fwd_options* opt,
                           int32_t num_tokens, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * pa_varlen_fwd_noalloc -- pa_varlen_fwd_ex for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument; the split-KV
 * partials go to a scratch array compiled into the library,
 * PA_NOALLOC_SCRATCH_BYTES on every GPU the library runs on, held until the
 * process ends.  The call allocates nothing; its first call on a device
 * (after all argument checks) resolves that device's scratch address once.
 *
 *   opt        as for pa_varlen_fwd_ex, or NULL: bf16 cache, no sinks
 *   the other arguments are those of pa_varlen_fwd_ex (the work list is
 *   still the caller's device copy of the plan)
 * Calls on one GPU share its scratch, which keeps the last call's partials;
 * nothing in it needs clearing (every partial row is written before the
 * same call reads it), but calls that overlap on one GPU (on two streams, or
 * in two graphs replayed concurrently) race: the caller orders them.
 * Errors: those of pa_varlen_fwd_ex; PA_ERR_WORKSPACE_TOO_SMALL when
 * plan->workspace_bytes > PA_NOALLOC_SCRATCH_BYTES; PA_ERR_HIP when the
 * scratch address cannot be resolved.
 * ------------------------------------------------------------------------ */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)

pa_status pa_varlen_fwd_noalloc(const pa_attn_params* p, const pa_plan_info* plan,
                                const int32_t* worklist,
                                const void* q, const void* kv_cache,
                                const int32_t* cu_seqlens_q, const int32_t* seqused_k,
                                const int32_t* block_table, const pa_fwd_options* opt,
                                int32_t num_tokens, void* out, float* lse, hipStream_t stream);

/* ------------------------------------------------------------------------
 * pa_merge_attn_states -- LSE-weighted merge of two partial attentions over
 * disjoint key sets (the cascade's third step, "FlashAttention 在 vLLM 中的
 * 实现分析" section 6.3, and the merge_attn_states helper of section 8.2):
 *   M = max(lse_p, lse_s), a = exp(lse_p - M), b = exp(lse_s - M),
 *   out = (a * out_p + b * out_s) / (a + b), out_lse = M + ln(a + b);
 *   two empty partials (both -inf) give out = 0, out_lse = -inf.
 *
 *   out, prefix_out, suffix_out   device bf16 [num_tokens, num_heads, head_size]
 *                                 (out may alias either input)
 *   out_lse                       device fp32 [num_tokens, num_heads] or NULL;
 *                                 it must not alias prefix_lse or suffix_lse
 *                                 (PA_ERR_INVALID_ARGUMENT): the threads of
 *                                 one row read both weights before any of
 *                                 them writes, and that order is not kept
 *                                 across a row's threads
 *   prefix_lse, suffix_lse        device fp32 [num_tokens, num_heads]
 * head_size must be a multiple of 8 and at most 512.
 * ------------------------------------------------------------------------ */
pa_status pa_merge_attn_states(void* out, float* out_lse,
                               const void* prefix_out, const float* prefix_lse,
                               const void* suffix_out, const float* suffix_lse,
                               int32_t num_tokens, int32_t num_heads, int32_t head_size,
                               hipStream_t stream);

/* Work-list layout (int32 words):
 *   [0] PA_WORKLIST_MAGIC  [1] version  [2] num_small_items  [3] num_tiled_items
 *   [4] num_reduce_items  [5] num_partial_rows  [6] group size H/Hkv
 *   [7] causal  [8..15] reserved (0)
 * then num_small_items + num_tiled_items attention items, then the reduce
 * items, PA_ITEM_WORDS words each.
 * attention item: seq, kv_head, row0, nrows, kv_begin, kv_end,
 *   partial_row (-1: write out/lse directly), kind (0: small-row item of
 *   <= PA_SMALL_MAX_ROWS rows, 1: tiled item of <= pa_plan_info.tiled_rows
 *   rows: PA_TILED_ROWS_WIDE in launches with no small-row items at
 *   head_size <= 128 whose prefills are long, else PA_TILED_ROWS),
 *   first token of the sequence (cu_seqlens_q[seq]), Lk - Lq of the
 *   sequence, 0, 0.  Rows and key range are clipped to the sequence, so the
 *   kernels read no lengths from device memory.
 *   When both kinds are present they run as one launch: each kind longest
 *   first, the two merged in proportion to their counts; otherwise all
 *   items are one kind, longest first.
 * reduce item: seq, kv_head, row0, nrows, partial_row0, num_splits,
 *   first token of the sequence (cu_seqlens_q[seq]), 0, 0, 0, 0, 0
 *   (split s of the unit wrote rows partial_row0 + s * nrows ...)
 * A "row" of sequence b is (query token i, head-in-group g) -> row i*G + g,
 * G = H / Hkv; kv_head's query heads are kv_head*G .. kv_head*G + G-1.    */
#define PA_WORKLIST_MAGIC 0x50414731
#define PA_WORKLIST_VERSION 3
#define PA_WORKLIST_HEADER_WORDS 16
#define PA_ITEM_WORDS 12
#define PA_SMALL_MAX_ROWS 16
#define PA_TILED_ROWS 128
#define PA_TILED_ROWS_WIDE 256

#ifdef __cplusplus
}
#endif
#endif /* PAGEDATTN_H_ */
