// kernels.h -- launchers of the decode kernels (host side of the HIP path).
#pragma once

#include <hip/hip_runtime.h>

#include "pkv_device.h"

namespace pkv {

// Split-KV decode on the matrix cores, up to 16 rows per KV head,
// head_dim_qk == head_dim_v in {64, 128, 256}.
hipError_t launch_split_mfma16(int q_dtype, int kv_dtype, int D, const Params& p, hipStream_t s);

// Split-KV decode over a latent cache: one KV head, up to 64 rows, 576-wide
// rows whose leading 512 entries are V.
hipError_t launch_split_mla(int q_dtype, int kv_dtype, const Params& p, hipStream_t s);

// The same on the stream-K schedule, with score and P.V work on separate
// waves and the tiles loaded straight into LDS (16-bit or fp8 caches).
hipError_t launch_split_mla_ws(int q_dtype, int kv_dtype, const Params& p, hipStream_t s);

// Split-KV decode on the vector ALUs, up to 8 rows per KV head.
hipError_t launch_split_valu(int q_dtype, int kv_dtype, int D, const Params& p, hipStream_t s);

// The write side: new tokens' rows into the paged cache at their slots.
struct InsertParams {
  const void* k_src;          // [N, Hkv, Dlo]
  const void* k_rope;         // [N, Hkv, Dk - Dlo] (or unused when Dlo == Dk)
  const void* v_src;          // [N, Hkv, Dv] (Dv == 0: no V cache)
  const int64_t* slot_mapping;  // [N]; < 0 or past the pool: skipped
  void* k_cache;
  void* v_cache;
  const void* q_lo;           // [N, Hq, Dlo]   query concat (q_out == null: none)
  const void* q_hi;           // [N, Hq, Dk - Dlo]
  void* q_out;                // [N, Hq, Dk]
  int N, Hkv, Hq, Dk, Dlo, Dv, ps, num_pages, layout;
  float scale_inv;            // E4M3 cache: stored value = round(x * scale_inv)
  const float* scale_inv_dev; // device-resident scale_inv, or null
};
hipError_t launch_cache_insert(int src_dtype, int cache_dtype, const InsertParams& p, hipStream_t s);

// Per-head products around the latent decode: y[m, h] = x[m, h] . W[h].
struct HeadMatmulParams {
  const void* x;              // element (m, h, k) at m * xs_m + h * xs_h + k
  const void* w;              // [H, K, N] row-major
  void* y;                    // element (m, h, n) at m * ys_m + h * ys_h + n
  int64_t xs_m, xs_h, ys_m, ys_h;
  int M, H, K, N;
};
hipError_t launch_head_matmul(int dtype, const HeadMatmulParams& p, hipStream_t s);

// Merge of two attention results by their log-sum-exps (natural log).
struct MergeParams {
  void* out;                  // [N, H, D] contiguous
  const void* o_p;            // prefix results: (n, h, d) at n * p_sn + h * p_sh + d
  const void* o_s;            // suffix results: (n, h, d) at n * s_sn + h * s_sh + d
  int64_t p_sn, p_sh, s_sn, s_sh;
  const float* lse_p;         // element (n, h) at n * lse_sn + h * lse_sh
  const float* lse_s;
  float* lse_out;             // same layout, or null
  int64_t lse_sn, lse_sh;
  int N, H, D, n_prefix;
};
hipError_t launch_merge_states(int dtype, const MergeParams& p, hipStream_t s);

// Attention over a ragged (non-paged) batch with its log-sum-exp.
struct RaggedParams {
  const void* q;              // [total_q, Hq, Dqk]
  const void* k;              // [total_k, Hkv, Dqk]
  const void* v;              // [total_k, Hkv, Dv]
  const int32_t* cu_q;        // [num_seqs + 1]
  const int32_t* cu_k;        // [num_seqs + 1]
  void* out;                  // [total_q, Hq, Dv]
  float* lse;                 // element (n, h) at n * lse_sn + h * lse_sh, or null
  int64_t lse_sn, lse_sh;
  int num_seqs, Hq, Hkv, G, Dqk, Dv, total_q, total_k, max_q_len, causal;
  int q_blocks;               // query blocks per (sequence, head) (set by the launcher)
  float scale_log2;           // sm_scale * log2(e)
};
hipError_t launch_ragged_attn(int dtype, const RaggedParams& p, hipStream_t s);

// Log-sum-exp merge of the split partials of every sequence that needed
// more than one split (zeros for sequences with nothing visible).
hipError_t launch_combine(int q_dtype, const Params& p, hipStream_t s);

}  // namespace pkv
