/*
 * pkv.h -- C ABI of the MI355X (gfx950) paged-KV decode-attention library.
 *
 * The operation is the one the FlashInfer `flashinfer.xqa.xqa` reference page
 * defines (function signature, parameter list and the closing note on
 * inferred parameters): a short run of query tokens per sequence attends,
 * for every group of query heads that shares one KV head, over K/V rows
 * gathered from a paged cache through an int32 page table up to a
 * per-sequence length.  Softmax attention is exact (no approximation); the
 * result is written in place into `out`.
 *
 * The absorbed multi-head-latent-attention decode of the vLLM
 * `models/kimi_k3/nvidia/mla` page (MultiHeadLatentAttention: the decode
 * branch of `_attention`, `forward_mqa` over the latent cache, and
 * `_v_up_proj`) is the same call at another shape: one KV head whose rows are
 * `kv_lora_rank + qk_rope_head_dim` wide (576), with V the first
 * `kv_lora_rank` (512) entries of each cached row.  Pass the same pointer as
 * `k_cache` and `v_cache` and `head_dim_v < head_dim_qk` to select it.
 *
 * Conventions used throughout (each is a reading of the pages; the design
 * notes list them with their reasons):
 *   q        [batch, q_seq_len, num_q_heads, head_dim_qk]   q_dtype, dense
 *            (beam width 1: the xqa page supports only beam width 1)
 *   k_cache  NHD: [num_pages, page_size, num_kv_heads, head_dim_qk]
 *            HND: [num_pages, num_kv_heads, page_size, head_dim_qk]
 *   v_cache  same layout with head_dim_v, or == k_cache (latent cache; V is
 *            the first head_dim_v entries of each K row)
 *   page_table [batch, pages_per_seq] int32; K and V share the table
 *   seq_lens [batch] uint32; token t of sequence b lives in page
 *            page_table[b][t / page_size], slot t % page_size
 *   out      [batch, q_seq_len, num_q_heads, head_dim_v] in q_dtype (bf16
 *            for an fp8 query; e4m3fn bytes with out_fp8)
 *   sinks    [num_kv_heads, num_q_heads / num_kv_heads] fp32 or NULL
 *   mask     [batch, q_seq_len, 2 * ceil(q_seq_len / 32)] uint16 or NULL
 *
 *   Query head h uses KV head h / G, G = num_q_heads / num_kv_heads.
 *   Query token i of sequence b sits at position pos = seq_len - q_seq_len + i
 *   (the draft tokens are the last q_seq_len positions of the sequence).
 *   Token t is visible to (b, i, h) iff
 *       t < seq_len,
 *       window == 0  or  t > pos - window          (a lower bound only: the
 *                                                   window hides no token after
 *                                                   pos; those are hidden only
 *                                                   by the mask),
 *       q_seq_len == 1 or mask == NULL or t < seq_len - q_seq_len
 *                  or bit (t - (seq_len - q_seq_len)) of mask row (b, i) is 1.
 *   A mask row is read as little-endian 32-bit words, word w being
 *   row[2w] | row[2w+1] << 16; draft j is bit (j % 32) of word j / 32.
 *   logit(t) = q_scale * kv_scale / sqrt(head_dim_qk) * dot(q, k_t)
 *   out = kv_scale * sum_t e^(logit(t) - M) v_t
 *         / (sum_t e^(logit(t) - M) + [sinks] e^(sink_h - M)),
 *   sink_h = sinks[h / G][h % G], M the max over logits and sink;
 *   a query with no visible token gets out = 0.
 *
 * Ownership and threading: every pointer is caller-owned device memory
 * (`dims` and `opts` are host structs).  The decode call never allocates,
 * frees or synchronises; it enqueues its kernels on `stream` (a
 * hipStream_t; NULL is the default stream) and returns.  Calls on one
 * stream serialise; the workspace must not be shared by calls that may run
 * concurrently.  The error string is thread-local.
 *
 * Errors: every check that can be made on the host is made before any
 * launch; on failure the call returns a non-zero status, enqueues nothing
 * and leaves a message for pkv_last_error().  Device-resident data (page
 * ids, sequence lengths) is not read on the host by the decode call: a
 * page id outside [0, num_pages) makes the tokens it holds invisible and a
 * seq_len above pages_per_seq * page_size is clamped to it -- inputs that
 * are outside the contract, which pkv_validate_inputs() reports.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 7

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARGUMENT = 1,   /* malformed shapes, NULLs, bad values   */
  PKV_ERR_UNSUPPORTED = 2,        /* well-formed but not implemented        */
  PKV_ERR_WORKSPACE_TOO_SMALL = 3,
  PKV_ERR_HIP = 4,                /* a HIP runtime call failed              */
  PKV_ERR_DEVICE_DATA = 5         /* pkv_validate_inputs: bad device data   */
} pkv_status;

/* Element types.  PKV_FP8_E4M3 is the OCP 8-bit E4M3 format ("fn": no
 * infinities, S.1111.111 is NaN, largest finite 448) -- the
 * torch.float8_e4m3fn cache dtype named on the xqa page.  A cache stored as
 * raw uint8 bytes is the same thing (the Kimi-K3 MLA page views its plain
 * fp8 cache that way). */
typedef enum { PKV_F16 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

/* Cache layouts of the xqa page's `kv_layout` parameter. */
typedef enum { PKV_NHD = 0, PKV_HND = 1 } pkv_layout;

/* What the xqa page infers from tensor shapes (its closing note), passed
 * explicitly because the ABI carries no shapes. */
typedef struct pkv_dims {
  int32_t batch;          /* q.shape[0]                                     */
  int32_t num_q_heads;    /* q.shape[-2]                                    */
  int32_t head_dim_qk;    /* q.shape[-1]; also the K row width              */
  int32_t head_dim_v;     /* V row width = out.shape[-1]                    */
  int32_t pages_per_seq;  /* page_table.shape[-1]; max_seq_len = this*page  */
  int32_t num_pages;      /* k_cache.shape[0] (physical pages)              */
  int32_t q_dtype;        /* pkv_dtype: PKV_F16 or PKV_BF16 (out dtype too);
                             PKV_FP8_E4M3 for the latent cache's quantised
                             query (needs an fp8 cache; out is PKV_BF16)    */
  int32_t kv_dtype;       /* pkv_dtype: == q_dtype or PKV_FP8_E4M3          */
  uint64_t workspace_bytes; /* size of the caller's workspace buffer        */
} pkv_dims;

/* Kernel paths.  PKV_PATH_AUTO lets the planner choose.  PKV_PATH_VALU is a
 * non-default reference path: the planner never picks it (the matrix-core
 * kernel, with its rows padded to 16, is faster at every measured shape,
 * small groups included); it runs only when forced, on the split grid. */
typedef enum {
  PKV_PATH_AUTO = 0,
  PKV_PATH_VALU = 1,      /* vector-ALU dot products, head dim 128, <= 8 rows */
  PKV_PATH_MFMA = 2,      /* matrix-core tiles, up to 16 rows per KV head   */
  PKV_PATH_MFMA_MLA = 3   /* matrix-core, 64 rows, latent (aliased) cache   */
} pkv_path;

/* Optional planner overrides (A/B measurement, split-invariance tests).
 * Zero-initialised means "all automatic". */
typedef struct pkv_options {
  int32_t path;           /* pkv_path                                       */
  int32_t split_pages;    /* pages per split-KV chunk; 0 = planner's choice */
  int32_t num_cus;        /* compute units to plan for; 0 = query device    */
  int32_t target_ctas;    /* planner's grid-size goal; 0 = default          */
  void* split_event;      /* hipEvent_t or NULL: when set, it is recorded on
                             the call's stream after the split-KV kernel and
                             before the combine kernel (timing one kernel with
                             events; no work changes)                       */
  /* xqa page, parameters `q_scale` / `kv_scale`: each may be a tensor.  When
   * set, these point at one fp32 value in device memory, 4-byte aligned and
   * caller-owned, and replace the q_scale / kv_scale arguments of the call.
   * The kernels read them when they run (a captured graph replays with the
   * values current at replay time); they must be finite. */
  const float* q_scale_dev;
  const float* kv_scale_dev;
  /* Where the matrix-core stream-K plan merges the partials of a
   * (sequence, KV head) cut across waves: 0 = planner's choice (in the split
   * kernel when every wave's share is short, where the second launch would
   * dominate; else in a combine kernel), 1 = combine kernel (two launches),
   * 2 = split kernel (one launch).  Other plans always use the combine
   * kernel.  (ABI version 3.) */
  int32_t merge_mode;
  /* xqa page, `output` ("dtype of q or of the KV cache") and `rcp_out_scale`
   * ("reciprocal of the output scale"): nonzero out_fp8 writes the output as
   * E4M3 bytes (an fp8 KV cache only) holding round(out * rcp_out_scale) --
   * binary32 product, nearest even, magnitudes past 448 saturated;
   * rcp_out_scale 0 means 1.  (ABI version 4.) */
  int32_t out_fp8;
  float rcp_out_scale;
} pkv_options;

/* The plan a decode call would use (pkv_query_plan). */
typedef struct pkv_plan_info {
  int32_t path;           /* pkv_path actually selected                     */
  int32_t split_pages;    /* pages per split                                */
  int32_t max_splits;     /* grid extent over splits                        */
  int32_t rows;           /* (num_q_heads / num_kv_heads) * q_seq_len       */
  int32_t ctas_per_split_grid; /* workgroups launched by the split kernel   */
  int32_t num_cus;
  uint64_t workspace_bytes;    /* bytes the call needs                      */
  int32_t single_launch;       /* 1: one launch, no combine kernel: the
                                  split kernel merges its partials itself,
                                  or (short sequences) gives each (sequence,
                                  KV head) one wave and cuts nothing; ABI 3 */
  int32_t waves_per_workgroup; /* matrix-core stream-K: waves per workgroup,
                                  each streaming the same tokens of another
                                  KV head; ABI 5                            */
} pkv_plan_info;

/* ABI version (PKV_ABI_VERSION of the built library). */
int pkv_abi_version(void);

/* Message of the last failing call on this thread ("" if none). */
const char* pkv_last_error(void);

/* Validates host arguments and reports the plan and workspace size.  Makes
 * no device call when opts->num_cus > 0.  `dims->workspace_bytes` is
 * ignored. */
pkv_status pkv_query_plan(const pkv_dims* dims, int num_kv_heads, int page_size,
                          int window, int q_seq_len, const pkv_options* opts,
                          pkv_plan_info* info);

/* Workspace bytes a decode call with these arguments needs (0 on invalid
 * arguments; pkv_last_error() says why).  The workspace holds the split-KV
 * partial results (running max, running sum and unnormalised output per
 * split), the role of the xqa page's `workspace_buffer`, and -- for the
 * matrix-core stream-K plan -- one 8-byte counter per (sequence, KV head),
 * the role of its `semaphores`.  No initialisation is needed: a counter word
 * tagged by another call counts as zero, and a call leaves its counts at
 * zero.  Calls that share a workspace must not run concurrently. */
size_t pkv_workspace_size(const pkv_dims* dims, int num_kv_heads, int page_size,
                          int window, int q_seq_len);

/* The decode call (xqa page: `xqa(q, k_cache, v_cache, page_table, seq_lens,
 * output, workspace_buffer, semaphores, num_kv_heads, page_size, sinks,
 * q_scale, kv_scale, sliding_win_size, kv_layout, ..., q_seq_len, mask)`).
 * `window` is sliding_win_size (0 = off).  `mask` is read only when
 * q_seq_len > 1.  `workspace` must hold dims->workspace_bytes >=
 * pkv_workspace_size(...) bytes and be 256-byte aligned (it may be NULL
 * when that size is 0: on the matrix-core path, when no (sequence, KV head)
 * can span more than 17 16-token tiles and there are at most eight of them
 * per CU, each gets one wave that streams it whole).  The xqa page's
 * `semaphores` live in the workspace: on the matrix-core stream-K plan with
 * short shares the last wave to finish a piece of a (sequence, KV head)
 * merges its partials in the same launch; the other stream-K plans, the
 * latent-cache and the split-grid plans merge in a second kernel.  `sm_count` and `enable_pdl` have no counterpart (the CU count is
 * queried).  This entry point writes the output in q's dtype with scale 1;
 * the xqa page's `rcp_out_scale` and fp8 output are pkv_options.out_fp8 and
 * pkv_options.rcp_out_scale of pkv_decode_attn_ex. */
pkv_status pkv_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* page_table, const uint32_t* seq_lens,
                           void* out, void* workspace, int num_kv_heads,
                           int page_size, int layout, const float* sinks,
                           float q_scale, float kv_scale, int window,
                           int q_seq_len, const uint16_t* mask, void* stream,
                           const pkv_dims* dims);

/* As pkv_decode_attn with planner overrides (opts may be NULL). */
pkv_status pkv_decode_attn_ex(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* page_table, const uint32_t* seq_lens,
                              void* out, void* workspace, int num_kv_heads,
                              int page_size, int layout, const float* sinks,
                              float q_scale, float kv_scale, int window,
                              int q_seq_len, const uint16_t* mask, void* stream,
                              const pkv_dims* dims, const pkv_options* opts);

/* Bytes of the static scratch of pkv_decode_attn_noalloc (per GPU). */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

/* pkv_decode_attn_ex without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The partial results and counters live in
 * a static device array of PKV_NOALLOC_SCRATCH_BYTES bytes, one per GPU,
 * allocated when the library's code is loaded on that GPU and kept until the
 * process ends; this call allocates nothing.  The current device must be the
 * one the stream and the buffers belong to.  A plan needing more scratch
 * than that (pkv_query_plan's workspace_bytes) is rejected with
 * PKV_ERR_WORKSPACE_TOO_SMALL before any device work.  Every call on one GPU
 * shares its array: nothing in it needs clearing (the single-launch counters
 * carry a per-call tag), but calls that overlap in time on one GPU (two
 * streams, or two threads) race and give wrong results.  (ABI version 7.) */
pkv_status pkv_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* page_table, const uint32_t* seq_lens,
                                   void* out, int num_kv_heads, int page_size, int layout,
                                   const float* sinks, float q_scale, float kv_scale,
                                   int window, int q_seq_len, const uint16_t* mask,
                                   void* stream, const pkv_dims* dims,
                                   const pkv_options* opts);

/* Checks the device-resident inputs the decode call trusts: every page id a
 * visible token needs lies in [0, num_pages) and q_seq_len <= seq_len <=
 * pages_per_seq * page_size.  Copies seq_lens and page_table to the host and
 * synchronises `stream` (a testing and debugging aid, not for the hot path).
 * Returns PKV_ERR_DEVICE_DATA with a message naming the first offending
 * sequence, or the host-argument status of pkv_decode_attn. */
pkv_status pkv_validate_inputs(const int32_t* page_table, const uint32_t* seq_lens,
                               int num_kv_heads, int page_size, int window,
                               int q_seq_len, void* stream, const pkv_dims* dims);

/* ---- the write side of the paged cache ------------------------------ */

/* Sizes of a cache insert. */
typedef struct pkv_insert_dims {
  int32_t num_tokens;     /* N: rows to insert (slot_mapping.shape[0])      */
  int32_t num_kv_heads;   /* Hkv                                            */
  int32_t head_dim_k;     /* cache K row width Dk (multiple of 8)           */
  int32_t head_dim_k_lo;  /* leading part of the K row from k_src; the rest
                             (Dk - Dlo, from k_rope_src) -- Dlo == Dk: no
                             second source; multiple of 8                   */
  int32_t head_dim_v;     /* V row width (multiple of 8); 0: no V cache     */
  int32_t page_size;      /* 16, 32, 64 or 128                              */
  int32_t num_pages;      /* physical pages of the cache                    */
  int32_t layout;         /* pkv_layout                                     */
  int32_t src_dtype;      /* PKV_F16 or PKV_BF16: k_src, k_rope_src, v_src,
                             q_lo, q_hi, q_out                              */
  int32_t cache_dtype;    /* == src_dtype, or PKV_FP8_E4M3                  */
  int32_t num_q_heads;    /* query concat heads (used when q_out != NULL)   */
} pkv_insert_dims;

/* Inserts new tokens' rows into the paged cache (vLLM Kimi-K3 MLA page,
 * `_decode_concat_cache`: the decode step's latent cache insert at
 * slot_mapping, fused with the query concat [ql_nope | q_pe]).
 *   For token i with slot s = slot_mapping[i] (int64; page s / page_size,
 *   offset s % page_size) and KV head h:
 *     K row  = [k_src[i, h, 0:Dlo] | k_rope_src[i, h, 0:Dk-Dlo]]
 *     V row  = v_src[i, h, 0:Dv]
 *   stored at [page, offset, h] (NHD) or [page, h, offset] (HND).  A slot
 *   below 0 (padding) or at/after num_pages * page_size writes nothing.
 *   A 16-bit cache gets the source bits; an E4M3 cache gets the nearest
 *   E4M3 value of the binary32 product x * cache_scale_inv (ties to even,
 *   magnitudes past 448 saturate to 448).  cache_scale_inv_dev, when not
 *   NULL, points at the scale in device memory (read when the kernel runs)
 *   and replaces cache_scale_inv.
 *   When q_out is not NULL: q_out[i, h] = [q_lo[i, h, 0:Dlo] | q_hi[i, h,
 *   0:Dk-Dlo]] for h < num_q_heads (all [N, Hq, .] contiguous, src_dtype).
 * The latent cache is Hkv = 1, Dk = 576, Dlo = 512, Dv = 0 (V is the
 * leading 512 entries of the K row).  All tensors are contiguous device
 * memory, 16-byte aligned; one launch on `stream`; errors as for decode. */
pkv_status pkv_cache_insert(const void* k_src, const void* k_rope_src, const void* v_src,
                            const int64_t* slot_mapping, void* k_cache, void* v_cache,
                            float cache_scale_inv, const float* cache_scale_inv_dev,
                            const void* q_lo, const void* q_hi, void* q_out, void* stream,
                            const pkv_insert_dims* dims);

/* ---- the latent-attention projections around the decode ------------- */

/* Per-head product y[m, h, 0:N] = x[m, h, 0:K] . W[h] for m < M, h < H (vLLM
 * Kimi-K3 MLA page, `_attention` decode branch: BMM1, which absorbs q_nope
 * into the latent space with W_UK_T [H, qk_nope_head_dim, kv_lora_rank]
 * before the latent decode, and `_v_up_proj`, which takes the
 * kv_lora_rank-wide decode output back to v_head_dim with W_UV [H,
 * kv_lora_rank, v_head_dim]).
 *   x: element (m, h, k) at x + m * x_stride_m + h * x_stride_h + k
 *      (strides in elements, multiples of 8: e.g. the q_nope part of q);
 *   w: [H, K, N] contiguous (the page's layout);
 *   y: element (m, h, n) at y + m * y_stride_m + h * y_stride_h + n
 *      (strides multiples of 4).
 * dtype PKV_BF16 or PKV_F16 for x, w and y; fp32 accumulation, one rounding
 * (nearest even) to the output.  K must be a multiple of 32 and N of 64;
 * pointers 16-byte aligned.  One launch on `stream`. */
pkv_status pkv_head_matmul(const void* x, int64_t x_stride_m, int64_t x_stride_h, const void* w,
                           void* y, int64_t y_stride_m, int64_t y_stride_h, int M, int H, int K,
                           int N, int dtype, void* stream);

/* ---- merging attention results over disjoint key sets --------------- */

/* vLLM Kimi-K3 MLA page, chunked prefill `merge_attn_states(output,
 * prefix_output, prefix_lse, suffix_output, suffix_lse,
 * prefill_tokens_with_context)`: for token n < N and head h < H, with the
 * natural-log log-sum-exps lp = prefix_lse(n, h), ls = suffix_lse(n, h),
 * M = max(lp, ls) and w = e^(lse - M):
 *   out[n, h] = (prefix_out[n, h] w_p + suffix_out[n, h] w_s) / (w_p + w_s)
 * and, when out_lse != NULL, out_lse(n, h) = M + log(w_p + w_s).  Tokens
 * n >= num_tokens_with_prefix take the suffix alone (prefix arrays then need
 * only num_tokens_with_prefix rows).  An -inf log-sum-exp contributes
 * nothing; both -inf give zeros (and -inf).  out: [N, H, D] contiguous;
 * prefix_out and suffix_out: element (n, h, d) at x + n * stride_n +
 * h * stride_h + d, strides in elements, multiples of 8 (the page merges
 * the leading v_head_dim entries of wider rows); dtype PKV_BF16 or PKV_F16
 * for all three, D a multiple of 8, pointers 16-byte aligned.  out may be
 * suffix_out itself when that is contiguous (strides H D, D), not any other
 * overlap.  Log-sum-exps fp32 with element (n, h) at lse + n * lse_stride_n
 * + h * lse_stride_h (e.g. [H, N]: strides 1, N).  One launch on `stream`. */
pkv_status pkv_merge_attn_states(void* out, const void* prefix_out, int64_t prefix_stride_n,
                                 int64_t prefix_stride_h, const float* prefix_lse,
                                 const void* suffix_out, int64_t suffix_stride_n,
                                 int64_t suffix_stride_h, const float* suffix_lse, float* out_lse,
                                 int64_t lse_stride_n, int64_t lse_stride_h, int num_tokens,
                                 int num_heads, int head_dim, int num_tokens_with_prefix,
                                 int dtype, void* stream);

/* ---- ragged (non-paged) attention with its log-sum-exp -------------- */

/* vllm-omni TRTLLM diffusion backend page, `trtllm_ragged_attention_deepseek`
 * (queries and keys packed by `cum_seq_lens_q` / `cum_seq_lens_kv`,
 * `is_causal`, `bmm1_scale` = the softmax scale, `max_q_len`), and the vLLM
 * Kimi-K3 MLA page's chunked prefill, whose `run_prefill_new_tokens` and
 * `_compute_prefill_context` return the (output, lse) pairs that
 * `merge_attn_states` (above) combines.
 *
 * Sequence s < num_seqs owns query rows [cu_seqlens_q[s], cu_seqlens_q[s+1])
 * of q [total_q, num_q_heads, head_dim_qk] and key/value rows
 * [cu_seqlens_k[s], cu_seqlens_k[s+1]) of k [total_k, num_kv_heads,
 * head_dim_qk] and v [total_k, num_kv_heads, head_dim_v] (all contiguous);
 * query head h reads KV head h / (num_q_heads / num_kv_heads).  With Lq and
 * Lk the two lengths, query i (0-based in its sequence) sees key j iff
 * j < Lk and, when `causal`, j <= i + Lk - Lq (the queries are the last Lq
 * positions of the key sequence; Lq == Lk is the plain causal mask).
 *   out[row, h]  = sum_j softmax_j(sm_scale q.k_j) v_j   (out: [total_q,
 *                  num_q_heads, head_dim_v], dtype of q)
 *   lse(row, h)  = log sum_j e^(sm_scale q.k_j)  (natural log, fp32, element
 *                  (row, h) at lse + row * lse_stride_n + h * lse_stride_h,
 *                  e.g. [H, N]: strides 1, total_q; lse may be NULL)
 * sm_scale must be positive and finite.  K and V rows of a sequence must be
 * finite (a causal query's weight for a later key is zero, but a zero times
 * a non-finite value is not); rows outside every sequence are never used.
 * A query that sees no key gets zeros and lse = -inf.  dtype PKV_BF16 or
 * PKV_F16 for q, k, v and out; fp32 accumulation.  (head_dim_qk,
 * head_dim_v) in {(64, 64), (128, 128), (192, 128)}; total_k * num_kv_heads *
 * head_dim * 2 bytes under 2 GiB; num_seqs and num_q_heads at most 65535.
 * cu_seqlens_*: int32 device arrays of num_seqs + 1 entries, non-decreasing;
 * sequence bounds are clamped to [0, total_*] on the device, so any values
 * stay in bounds.  Queries past `max_q_len` in a sequence are not computed
 * (their rows are left unwritten): max_q_len must be at least the longest
 * Lq (the page's `max_q_len`).  Pointers 16-byte aligned (lse 4-byte).
 * Caller-owned memory, nothing allocated; one launch on `stream`.  (ABI
 * version 6.) */
pkv_status pkv_ragged_attn(const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, void* out,
                           float* lse, int64_t lse_stride_n, int64_t lse_stride_h, int num_seqs,
                           int num_q_heads, int num_kv_heads, int head_dim_qk, int head_dim_v,
                           int total_q, int total_k, int max_q_len, float sm_scale, int causal,
                           int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
