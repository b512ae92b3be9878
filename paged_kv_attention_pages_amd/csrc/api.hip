// api.hip -- the C ABI of include/pkv.h: argument checks, the split-KV
// planner, workspace layout and kernel launches.
//
// Operation: FlashInfer `flashinfer.xqa.xqa` reference page (paged-KV decode
// attention: parameters q, k_cache, v_cache, page_table, seq_lens, output,
// workspace_buffer, num_kv_heads, page_size, sinks, q_scale, kv_scale,
// sliding_win_size, kv_layout, q_seq_len, mask, and the note on the
// parameters inferred from shapes).  Errors follow the explicit-message style
// of the vllm-omni trtllm_attn backend page (metadata validation in
// `forward_cuda`): every malformed argument is rejected with a message, and
// nothing falls back silently.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/pkv.h"
#include "kernels.h"

// Scratch memory of pkv_decode_attn_noalloc: a fixed array in device global
// memory, one copy per GPU the library runs on, held until the process ends.
// On the host this name stands for a host-side shadow, not a device address:
// host code passes only the address hipGetSymbolAddress returns for the
// current GPU (scratch_of_current_device below).
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int kv_elem(int dt) { return dt == PKV_FP8_E4M3 ? 1 : 2; }

int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

struct Plan {
  int path;
  int rows;
  int split_pages;
  int max_splits;
  int num_cus;
  int sk_waves;        // > 0: stream-K over this many persistent waves
  int sk_hb;           // matrix-core stream-K: waves per workgroup, one KV head each
  size_t ws_o_bytes;   // partial outputs
  size_t ws_ml_off;    // offset of (max, sum) pairs
  size_t ws_cnt_off;   // offset of the per-unit counters (single-launch merge)
  bool fused;          // cut units merged in the split kernel (no combine launch)
  bool lat_ws;         // latent stream-K with separate score / P.V waves
  bool unit_aligned;   // matrix-core stream-K over B * Hkv waves, one per unit when even
  bool unit_whole;     // matrix-core, one wave per unit always, nothing cut (no combine)
  size_t ws_bytes;
};

// Generation of a single-launch-merge call: tags the per-unit counters so
// that words left by other calls count as zero.
std::atomic<unsigned> g_gen{0};

// Device address of `scratch` per GPU, looked up on the first no-alloc call
// made with that GPU current.
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

pkv_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(PKV_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PKV_OK;
}

// Host-side checks shared by every entry point, then the plan.
pkv_status make_plan(const pkv_dims* d, int Hkv, int ps, int layout, int window, int Tq,
                     bool aliased, const pkv_options* opts, Plan* pl) {
  if (d == nullptr) return fail(PKV_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (d->batch < 0) return fail(PKV_ERR_INVALID_ARGUMENT, "batch must be >= 0, got %d", d->batch);
  if (d->num_q_heads < 1)
    return fail(PKV_ERR_INVALID_ARGUMENT, "num_q_heads must be >= 1, got %d", d->num_q_heads);
  if (Hkv < 1) return fail(PKV_ERR_INVALID_ARGUMENT, "num_kv_heads must be >= 1, got %d", Hkv);
  if (d->num_q_heads % Hkv != 0)
    return fail(PKV_ERR_INVALID_ARGUMENT,
                "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", d->num_q_heads, Hkv);
  if (ps != 16 && ps != 32 && ps != 64 && ps != 128)
    return fail(PKV_ERR_INVALID_ARGUMENT, "page_size must be one of 16, 32, 64, 128; got %d", ps);
  if (layout != PKV_NHD && layout != PKV_HND)
    return fail(PKV_ERR_INVALID_ARGUMENT, "kv_layout must be NHD (0) or HND (1); got %d", layout);
  if (window < 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "sliding window must be >= 0 (0 = off); got %d", window);
  if (Tq < 1) return fail(PKV_ERR_INVALID_ARGUMENT, "q_seq_len must be >= 1; got %d", Tq);
  if (d->pages_per_seq < 1)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pages_per_seq must be >= 1; got %d", d->pages_per_seq);
  if (d->num_pages < 1)
    return fail(PKV_ERR_INVALID_ARGUMENT, "num_pages must be >= 1; got %d", d->num_pages);
  if (d->head_dim_qk < 1 || d->head_dim_v < 1)
    return fail(PKV_ERR_INVALID_ARGUMENT, "head dims must be >= 1; got %d / %d", d->head_dim_qk,
                d->head_dim_v);
  // an fp8 query (the latent path's quantised query input) goes with an fp8
  // cache; its output is bfloat16
  const bool q8 = d->q_dtype == PKV_FP8_E4M3;
  if (d->q_dtype != PKV_F16 && d->q_dtype != PKV_BF16 && !q8)
    return fail(PKV_ERR_INVALID_ARGUMENT, "q dtype must be float16 (0), bfloat16 (1) or "
                                          "float8_e4m3fn (2, latent cache only); got %d",
                d->q_dtype);
  if (q8 && d->kv_dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_INVALID_ARGUMENT, "an float8_e4m3fn query needs an float8_e4m3fn KV cache");
  if (d->kv_dtype != d->q_dtype && d->kv_dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_INVALID_ARGUMENT,
                "KV cache dtype must equal the query dtype or be float8_e4m3fn; got %d for q %d",
                d->kv_dtype, d->q_dtype);
  if ((int64_t)d->pages_per_seq * ps > INT32_MAX / 2)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pages_per_seq * page_size too large");

  const int G = d->num_q_heads / Hkv;
  const int64_t R64 = (int64_t)G * Tq;
  const int R = (int)(R64 > INT32_MAX ? INT32_MAX : R64);
  const int Dk = d->head_dim_qk, Dv = d->head_dim_v;
  const int want = opts ? opts->path : PKV_PATH_AUTO;
  if (want < PKV_PATH_AUTO || want > PKV_PATH_MFMA_MLA)
    return fail(PKV_ERR_INVALID_ARGUMENT, "unknown path %d", want);

  const bool std_shape = Dk == Dv && (Dk == 64 || Dk == 128 || Dk == 256) && R <= 16 && !q8;
  const bool mla_shape = Dk == 576 && Dv == 512 && aliased && R <= 64 && Tq <= 32;
  const bool valu_ok = std_shape && Dk == 128 && R <= 8;
  int path;
  if (want == PKV_PATH_AUTO) {
    if (std_shape) path = PKV_PATH_MFMA;
    else if (mla_shape) path = PKV_PATH_MFMA_MLA;
    else if (Dk == 576 && Dv == 512 && !aliased)
      return fail(PKV_ERR_UNSUPPORTED,
                  "head dims 576/512 are supported for the latent cache only (v_cache == k_cache)");
    else
      return fail(PKV_ERR_UNSUPPORTED,
                  "unsupported shape: head_dim_qk %d, head_dim_v %d, %d rows per KV head%s "
                  "(supported: equal head dims 64/128/256 with <= 16 rows and a 16-bit query, "
                  "or the 576/512 latent cache with <= 64 rows and q_seq_len <= 32)",
                  Dk, Dv, R, q8 ? " with an fp8 query" : "");
  } else {
    path = want;
    if (path == PKV_PATH_MFMA && !std_shape)
      return fail(PKV_ERR_UNSUPPORTED, "matrix-core path needs equal head dims 64/128/256, "
                                       "<= 16 rows per KV head and a 16-bit query");
    if (path == PKV_PATH_VALU && !valu_ok)
      return fail(PKV_ERR_UNSUPPORTED, "vector path needs head_dim 128 and <= 8 rows per KV head");
    if (path == PKV_PATH_MFMA_MLA && !mla_shape)
      return fail(PKV_ERR_UNSUPPORTED, "latent path needs head dims 576/512, v_cache == k_cache, "
                                       "<= 64 rows and q_seq_len <= 32");
  }

  // ---- split planning: chunks of whole pages; grid sized for the CU count
  const int cus = (opts && opts->num_cus > 0) ? opts->num_cus : device_cus();
  const int64_t pps = d->pages_per_seq;
  int64_t pages_max = pps;
  if (window > 0) pages_max = std::min<int64_t>(pps, cdiv((int64_t)window + Tq - 1, ps) + 1);
  const int64_t units = (int64_t)d->batch * Hkv;
  const int64_t row_bytes = (int64_t)(Dk + (aliased ? 0 : Dv)) * kv_elem(d->kv_dtype);
  const int64_t page_bytes = (int64_t)ps * row_bytes;
  // kernels address inside one page (all KV heads) with 32-bit byte offsets
  if (page_bytes * Hkv >= (int64_t)1 << 31)
    return fail(PKV_ERR_UNSUPPORTED, "one cache page (all KV heads) must be under 2 GiB");
  const int64_t partial_bytes = (int64_t)R * Dv * 4 + (int64_t)R * 8;
  // keep each split's partial-result traffic under ~1/8 of its cache bytes,
  // and every split at least 256 tokens long
  int64_t min_pages = std::max<int64_t>(cdiv(8 * partial_bytes, page_bytes), cdiv(256, ps));
  // the matrix-core path runs one wave per split and keeps a split's page ids
  // one per lane (at most 64 pages); the others run four waves per split
  const int64_t waves_per_cta = path == PKV_PATH_MFMA ? 1 : 4;
  const int64_t max_sp = path == PKV_PATH_MFMA ? 64 : INT32_MAX;
  const int64_t target =
      (opts && opts->target_ctas > 0) ? opts->target_ctas : 32LL * cus / waves_per_cta / 4;
  int64_t sp = units > 0 ? cdiv(units * pages_max, target) : pages_max;
  sp = std::max(sp, min_pages);
  sp = std::min(sp, pages_max);
  if (opts && opts->split_pages > 0) sp = std::min<int64_t>(opts->split_pages, pages_max);
  sp = std::max<int64_t>(std::min(sp, max_sp), 1);
  const int64_t S = cdiv(pages_max, sp);
  if (S > 65535) return fail(PKV_ERR_UNSUPPORTED, "too many splits (%lld)", (long long)S);

  pl->path = path;
  pl->rows = R;
  pl->split_pages = (int)sp;
  pl->max_splits = (int)S;
  pl->num_cus = cus;
  pl->sk_waves = 0;
  pl->sk_hb = 1;
  pl->fused = false;
  pl->lat_ws = false;
  pl->unit_aligned = false;
  pl->unit_whole = false;
  pl->ws_cnt_off = 0;
  // Stream-K schedule (matrix-core path, batch <= 256, no forced split size):
  // persistent waves (measured best: one per SIMD for 16-bit caches, each
  // with a three-stage pipeline in flight); 2 partial slots per wave.
  // The latent-cache kernel runs the same schedule over 32-token tiles (64
  // for an fp8 cache) with one eight-wave workgroup per CU (its LDS ring
  // allows no more).
  // Both kernels count tiles in 32-bit integers (the tiles of one KV head
  // over all sequences, per-sequence prefixes, unit offsets), so the whole
  // tile stream must stay under 2^31 tiles; a sequence's visible tokens span
  // at most cdiv(pages_max * ps, tile) + 1 aligned tiles.  Larger problems
  // take the split grid.
  const int64_t sk_tile = path != PKV_PATH_MFMA_MLA ? 16 : d->kv_dtype == PKV_FP8_E4M3 ? 64 : 32;
  const bool sk_path = (path == PKV_PATH_MFMA || path == PKV_PATH_MFMA_MLA) &&
                       units * (cdiv(pages_max * ps, sk_tile) + 1) < ((int64_t)1 << 31);
  // (up to 256 sequences; the matrix-core kernel with head dims up to 128
  // also has a wider schedule for up to 1024)
  const int64_t sk_max_batch = path == PKV_PATH_MFMA && Dk <= 128 && Dv <= 128 ? 1024 : 256;
  if (sk_path && d->batch <= sk_max_batch && !(opts && opts->split_pages > 0)) {
    // fp8 tiles carry half the bytes for the same matrix work, so more waves
    // per CU hide the conversion work: 8 per CU for fp8, 4 for 16-bit caches
    const int64_t per_cu = path == PKV_PATH_MFMA_MLA ? 1 : d->kv_dtype == PKV_FP8_E4M3 ? 8 : 4;
    const int64_t W = (opts && opts->target_ctas > 0) ? opts->target_ctas : per_cu * cus;
    pl->sk_waves = (int)std::min<int64_t>(W, 1 << 20);
    // The waves of one workgroup stream the same tokens of sk_hb KV heads
    // side by side (the unit order is KV-head-major and Hkv divides the wave
    // count), so in an NHD cache the heads' pieces of each token row are read
    // together: up to one CU's resident waves (at most 8), a divisor of Hkv.
    pl->sk_hb = 1;
    const int64_t resident = pl->sk_waves >= cus ? std::min<int64_t>(8, pl->sk_waves / cus) : 8;
    if (path == PKV_PATH_MFMA && pl->sk_waves % Hkv == 0)
      for (int h = (int)std::min<int64_t>(resident, Hkv); h > 1; --h)
        if (Hkv % h == 0) {
          pl->sk_hb = h;
          break;
        }
    pl->split_pages = 0;
    pl->max_splits = 0;
    // the latent kernel keeps 64 padded rows per slot, its partial outputs
    // in the P.V waves' register order (see combine.hip)
    pl->lat_ws = path == PKV_PATH_MFMA_MLA;
    const size_t nrow = (size_t)2 * pl->sk_waves * (pl->lat_ws ? 64 : R);
    pl->ws_o_bytes = nrow * Dv * sizeof(float);
    pl->ws_ml_off = (pl->ws_o_bytes + 255) & ~(size_t)255;
    pl->ws_bytes = pl->ws_ml_off + nrow * 2 * sizeof(float);
    // The matrix-core kernel can merge cut units itself (one launch), with
    // one 8-byte counter per unit after the partials.  The merge then sits
    // at the end of the waves' shares, behind a few device-scope memory
    // round trips; that beats a second launch only when the shares are
    // short (measured, 64 sequences x 8 KV heads: 3 us per call gained at
    // 16-128 tokens, even at 256, 1 us lost at 512 and more), so by default
    // it is used when no wave's share can exceed 8 tiles.  The latent-cache
    // kernel leaves the merge of its 64-row partials to the combine kernel.
    const int mode = opts ? opts->merge_mode : 0;
    // Short sequences: when no unit can span more than 17 tiles (at most 256
    // cached tokens a sequence, or within the window), one wave per unit
    // streams it whole in one launch -- nothing is cut, no partial is
    // written and no combine runs -- and the units' start latencies (query,
    // page ids, first tiles) overlap instead of following one another in a
    // wave's share.  Up to eight units per CU.
    int64_t span = pages_max * ps;   // most tokens a unit can see
    if (window > 0) span = std::min<int64_t>(span, (int64_t)window + Tq - 1);
    if (path == PKV_PATH_MFMA && mode == 0 && !(opts && opts->target_ctas > 0) &&
        cdiv(span, 16) + 1 <= 17 && units <= 8 * (int64_t)cus) {
      pl->unit_whole = true;
      pl->sk_waves = (int)units;
      pl->sk_hb = 1;
      const int64_t res = std::min<int64_t>(8, units / cus);
      for (int h = (int)std::min<int64_t>(res, Hkv); h > 1; --h)
        if (Hkv % h == 0) {
          pl->sk_hb = h;
          break;
        }
      pl->ws_o_bytes = pl->ws_ml_off = pl->ws_bytes = 0;
      return PKV_OK;
    }
    // With a window every unit spans at most cdiv(window + Tq - 1, 16) + 1
    // tiles, and where the sequences reach past the window the units are of
    // (nearly) equal length.  Then one wave per whole unit is as balanced as
    // equal shares, cuts nothing and leaves the merge pass nothing to do
    // (measured, fp8 + window 4096 + sinks, 1024 units of 4096 tokens: the
    // call 200 -> 182 us).  The plan launches B * Hkv waves and workspace for
    // equal shares over them; the kernels choose between the two on the
    // device, from the lengths (sk_units_even), so a batch of mostly short
    // sequences still gets equal shares.  Used by default when the units give
    // every CU two to eight waves (more would only grow the equal-shares
    // workspace, two partial slots per unit).
    if (path == PKV_PATH_MFMA && window > 0 && mode == 0 && !(opts && opts->target_ctas > 0) &&
        units >= 2 * (int64_t)cus && units <= 8 * (int64_t)cus) {
      pl->unit_aligned = true;
      pl->sk_waves = (int)units;
      pl->sk_hb = 1;
      const int64_t res = std::min<int64_t>(8, units / cus);
      for (int h = (int)std::min<int64_t>(res, Hkv); h > 1; --h)
        if (Hkv % h == 0) {
          pl->sk_hb = h;
          break;
        }
      const size_t nrow_u = (size_t)2 * pl->sk_waves * R;
      pl->ws_o_bytes = nrow_u * Dv * sizeof(float);
      pl->ws_ml_off = (pl->ws_o_bytes + 255) & ~(size_t)255;
      pl->ws_bytes = pl->ws_ml_off + nrow_u * 2 * sizeof(float);
      return PKV_OK;
    }
    const int64_t max_tiles = units * cdiv(pages_max * ps, 16);
    pl->fused = path == PKV_PATH_MFMA &&
                (mode == 2 || (mode == 0 && max_tiles <= 8 * (int64_t)pl->sk_waves));
    if (pl->fused) {
      pl->ws_cnt_off = (pl->ws_bytes + 255) & ~(size_t)255;
      pl->ws_bytes = pl->ws_cnt_off + (size_t)units * sizeof(unsigned long long);
    }
    return PKV_OK;
  }
  const size_t nrow = (size_t)d->batch * Hkv * S * R;
  if (S > 1) {
    pl->ws_o_bytes = nrow * Dv * sizeof(float);
    pl->ws_ml_off = (pl->ws_o_bytes + 255) & ~(size_t)255;
    pl->ws_bytes = pl->ws_ml_off + nrow * 2 * sizeof(float);
  } else {
    pl->ws_o_bytes = pl->ws_ml_off = pl->ws_bytes = 0;
  }
  return PKV_OK;
}

bool misaligned(const void* p, size_t a) { return ((uintptr_t)p % a) != 0; }

pkv_status decode(const void* q, const void* k, const void* v, const int32_t* page_table,
                  const uint32_t* seq_lens, void* out, void* workspace, int Hkv, int ps,
                  int layout, const float* sinks, float q_scale, float kv_scale, int window,
                  int Tq, const uint16_t* mask, void* stream, const pkv_dims* d,
                  const pkv_options* opts) {
  Plan pl;
  const bool aliased = v != nullptr && v == k && d != nullptr && d->head_dim_v < d->head_dim_qk;
  pkv_status st = make_plan(d, Hkv, ps, layout, window, Tq, aliased, opts, &pl);
  if (st != PKV_OK) return st;
  if (d->batch == 0) return PKV_OK;
  if (!q || !k || !v || !page_table || !seq_lens || !out)
    return fail(PKV_ERR_INVALID_ARGUMENT, "q, k_cache, v_cache, page_table, seq_lens and out "
                                          "must not be NULL");
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16))
    return fail(PKV_ERR_INVALID_ARGUMENT, "q, k_cache, v_cache and out must be 16-byte aligned");
  if (!std::isfinite(q_scale) || !std::isfinite(kv_scale))
    return fail(PKV_ERR_INVALID_ARGUMENT, "q_scale and kv_scale must be finite");
  if (opts && (misaligned(opts->q_scale_dev, 4) || misaligned(opts->kv_scale_dev, 4)))
    return fail(PKV_ERR_INVALID_ARGUMENT, "device q_scale / kv_scale must be 4-byte aligned");
  const bool out_fp8 = opts && opts->out_fp8;
  const float rcp_out = (opts && opts->rcp_out_scale != 0.f) ? opts->rcp_out_scale : 1.f;
  if (out_fp8 && d->kv_dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_INVALID_ARGUMENT, "an float8_e4m3fn output needs an float8_e4m3fn KV cache "
                                          "(the output dtype is q's or the cache's)");
  if (!std::isfinite(rcp_out) || rcp_out <= 0.f)
    return fail(PKV_ERR_INVALID_ARGUMENT, "rcp_out_scale must be finite and positive");
  if (pl.ws_bytes > 0) {
    if (workspace == nullptr)
      return fail(PKV_ERR_WORKSPACE_TOO_SMALL, "workspace is NULL; %zu bytes needed", pl.ws_bytes);
    if (d->workspace_bytes < pl.ws_bytes)
      return fail(PKV_ERR_WORKSPACE_TOO_SMALL, "workspace holds %llu bytes; %zu needed",
                  (unsigned long long)d->workspace_bytes, pl.ws_bytes);
    if (misaligned(workspace, 256))
      return fail(PKV_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  }

  pkv::Params p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.page_table = page_table;
  p.seq_lens = seq_lens;
  p.out = out;
  p.ws_o = pl.ws_bytes ? (float*)workspace : nullptr;
  p.ws_ml = pl.ws_bytes ? (float2*)((char*)workspace + pl.ws_ml_off) : nullptr;
  p.sinks = sinks;
  p.mask = Tq > 1 ? mask : nullptr;
  const int64_t Dk = d->head_dim_qk, Dv = d->head_dim_v;
  const int64_t vrow = pl.path == PKV_PATH_MFMA_MLA ? Dk : Dv;
  if (layout == PKV_NHD) {
    p.k_page = (int64_t)ps * Hkv * Dk; p.k_slot = (int64_t)Hkv * Dk; p.k_head = Dk;
    p.v_page = (int64_t)ps * Hkv * vrow; p.v_slot = (int64_t)Hkv * vrow; p.v_head = vrow;
  } else {
    p.k_page = (int64_t)Hkv * ps * Dk; p.k_slot = Dk; p.k_head = (int64_t)ps * Dk;
    p.v_page = (int64_t)Hkv * ps * vrow; p.v_slot = vrow; p.v_head = (int64_t)ps * vrow;
  }
  p.B = d->batch;
  p.Tq = Tq;
  p.Hq = d->num_q_heads;
  p.Hkv = Hkv;
  p.G = d->num_q_heads / Hkv;
  p.R = pl.rows;
  p.Dqk = (int)Dk;
  p.Dv = (int)Dv;
  p.ps = ps;
  p.ps_shift = __builtin_ctz((unsigned)ps);
  p.pps = d->pages_per_seq;
  p.num_pages = d->num_pages;
  p.window = window;
  p.mask_words16 = ((Tq + 31) / 32) * 2;
  p.split_pages = pl.split_pages;
  p.max_splits = pl.max_splits;
  p.sk_waves = pl.sk_waves;
  p.sk_hb = pl.sk_hb;
  p.sk_shift = pl.path != PKV_PATH_MFMA_MLA ? 4 : d->kv_dtype == PKV_FP8_E4M3 && pl.lat_ws ? 6 : 5;
  p.qk_scale_log2 = (float)((double)q_scale * (double)kv_scale / std::sqrt((double)Dk) *
                            1.4426950408889634);
  p.out_scale = kv_scale;
  p.q_scale_dev = opts ? opts->q_scale_dev : nullptr;
  p.kv_scale_dev = opts ? opts->kv_scale_dev : nullptr;
  p.q_scale = q_scale;
  p.kv_scale = kv_scale;
  p.qk_unit = (float)(1.4426950408889634 / std::sqrt((double)Dk));
  p.fused = pl.fused ? 1 : 0;
  p.ws_lanes = pl.lat_ws ? 1 : 0;
  p.sk_units = pl.unit_whole ? 2 : pl.unit_aligned ? 1 : 0;
  p.out_fp8 = out_fp8 ? 1 : 0;
  p.rcp_out_scale = rcp_out;
  p.ws_cnt = pl.fused ? (unsigned long long*)((char*)workspace + pl.ws_cnt_off) : nullptr;
  p.gen = pl.fused ? g_gen.fetch_add(1, std::memory_order_relaxed) + 1u : 0u;
  if (p.B > 65535 || Hkv > 65535)
    return fail(PKV_ERR_UNSUPPORTED, "batch and num_kv_heads must be <= 65535");

  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  switch (pl.path) {
    case PKV_PATH_VALU: e = pkv::launch_split_valu(d->q_dtype, d->kv_dtype, (int)Dk, p, s); break;
    case PKV_PATH_MFMA_MLA:
      // the stream-K schedule: the wave-specialised kernel; the split grid:
      // the kernel that stages tiles in registers
      e = pl.lat_ws ? pkv::launch_split_mla_ws(d->q_dtype, d->kv_dtype, p, s)
              : pkv::launch_split_mla(d->q_dtype, d->kv_dtype, p, s);
      break;
    default: e = pkv::launch_split_mfma16(d->q_dtype, d->kv_dtype, (int)Dk, p, s); break;
  }
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "split-KV launch failed: %s", hipGetErrorString(e));
  if (opts && opts->split_event) {
    e = hipEventRecord((hipEvent_t)opts->split_event, s);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "event record failed: %s", hipGetErrorString(e));
  }
  if (!pl.fused && !pl.unit_whole) {
    // an fp8 query's output is bfloat16
    e = pkv::launch_combine(d->q_dtype == PKV_FP8_E4M3 ? PKV_BF16 : d->q_dtype, p, s);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "combine launch failed: %s", hipGetErrorString(e));
  }
  g_err.clear();
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_last_error(void) { return g_err.c_str(); }

pkv_status pkv_query_plan(const pkv_dims* dims, int num_kv_heads, int page_size, int window,
                          int q_seq_len, const pkv_options* opts, pkv_plan_info* info) {
  if (info == nullptr) return fail(PKV_ERR_INVALID_ARGUMENT, "info is NULL");
  Plan pl;
  // the latent shape is only reachable with an aliased cache; assume it
  const bool aliased = dims != nullptr && dims->head_dim_v < dims->head_dim_qk;
  pkv_status st = make_plan(dims, num_kv_heads, page_size, PKV_NHD, window, q_seq_len, aliased,
                            opts, &pl);
  if (st != PKV_OK) return st;
  info->path = pl.path;
  info->split_pages = pl.split_pages;
  info->max_splits = pl.max_splits;
  info->rows = pl.rows;
  info->ctas_per_split_grid =
      pl.sk_waves > 0 ? pl.sk_waves : pl.max_splits * num_kv_heads * dims->batch;
  info->num_cus = pl.num_cus;
  info->workspace_bytes = pl.ws_bytes;
  info->single_launch = pl.fused || pl.unit_whole ? 1 : 0;
  info->waves_per_workgroup = pl.path == PKV_PATH_MFMA_MLA ? 8 : pl.sk_waves > 0 ? pl.sk_hb : 1;
  g_err.clear();
  return PKV_OK;
}

size_t pkv_workspace_size(const pkv_dims* dims, int num_kv_heads, int page_size, int window,
                          int q_seq_len) {
  Plan pl;
  const bool aliased = dims != nullptr && dims->head_dim_v < dims->head_dim_qk;
  if (make_plan(dims, num_kv_heads, page_size, PKV_NHD, window, q_seq_len, aliased, nullptr,
                &pl) != PKV_OK)
    return 0;
  return pl.ws_bytes;
}

pkv_status pkv_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* page_table, const uint32_t* seq_lens, void* out,
                           void* workspace, int num_kv_heads, int page_size, int layout,
                           const float* sinks, float q_scale, float kv_scale, int window,
                           int q_seq_len, const uint16_t* mask, void* stream,
                           const pkv_dims* dims) {
  return decode(q, k_cache, v_cache, page_table, seq_lens, out, workspace, num_kv_heads,
                page_size, layout, sinks, q_scale, kv_scale, window, q_seq_len, mask, stream,
                dims, nullptr);
}

pkv_status pkv_decode_attn_ex(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* page_table, const uint32_t* seq_lens, void* out,
                              void* workspace, int num_kv_heads, int page_size, int layout,
                              const float* sinks, float q_scale, float kv_scale, int window,
                              int q_seq_len, const uint16_t* mask, void* stream,
                              const pkv_dims* dims, const pkv_options* opts) {
  return decode(q, k_cache, v_cache, page_table, seq_lens, out, workspace, num_kv_heads,
                page_size, layout, sinks, q_scale, kv_scale, window, q_seq_len, mask, stream,
                dims, opts);
}

pkv_status pkv_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* page_table, const uint32_t* seq_lens,
                                   void* out, int num_kv_heads, int page_size, int layout,
                                   const float* sinks, float q_scale, float kv_scale, int window,
                                   int q_seq_len, const uint16_t* mask, void* stream,
                                   const pkv_dims* dims, const pkv_options* opts) {
  if (dims == nullptr) return fail(PKV_ERR_INVALID_ARGUMENT, "dims is NULL");
  // the same plan decode() makes, to size the scratch before any device call
  Plan pl;
  const bool aliased = v_cache != nullptr && v_cache == k_cache && dims->head_dim_v < dims->head_dim_qk;
  pkv_status st = make_plan(dims, num_kv_heads, page_size, layout, window, q_seq_len, aliased,
                            opts, &pl);
  if (st != PKV_OK) return st;
  if (pl.ws_bytes > PKV_NOALLOC_SCRATCH_BYTES)
    return fail(PKV_ERR_WORKSPACE_TOO_SMALL,
                "this call needs %zu bytes of scratch; pkv_decode_attn_noalloc has %zu "
                "(call pkv_decode_attn_ex with a workspace instead)",
                pl.ws_bytes, (size_t)PKV_NOALLOC_SCRATCH_BYTES);
  if (dims->batch == 0) return PKV_OK;
  void* ws = nullptr;
  if (pl.ws_bytes > 0) {
    st = scratch_of_current_device(&ws);
    if (st != PKV_OK) return st;
  }
  pkv_dims d = *dims;
  d.workspace_bytes = PKV_NOALLOC_SCRATCH_BYTES;
  return decode(q, k_cache, v_cache, page_table, seq_lens, out, ws, num_kv_heads, page_size,
                layout, sinks, q_scale, kv_scale, window, q_seq_len, mask, stream, &d, opts);
}

pkv_status pkv_validate_inputs(const int32_t* page_table, const uint32_t* seq_lens,
                               int num_kv_heads, int page_size, int window, int q_seq_len,
                               void* stream, const pkv_dims* dims) {
  Plan pl;
  const bool aliased = dims != nullptr && dims->head_dim_v < dims->head_dim_qk;
  pkv_options o{};
  o.num_cus = 256;  // the plan is not used; avoid a device query
  pkv_status st = make_plan(dims, num_kv_heads, page_size, PKV_NHD, window, q_seq_len, aliased,
                            &o, &pl);
  if (st != PKV_OK) return st;
  if (dims->batch == 0) return PKV_OK;
  if (!page_table || !seq_lens)
    return fail(PKV_ERR_INVALID_ARGUMENT, "page_table and seq_lens must not be NULL");
  const int B = dims->batch, pps = dims->pages_per_seq;
  std::vector<uint32_t> L(B);
  std::vector<int32_t> T((size_t)B * pps);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(L.data(), seq_lens, sizeof(uint32_t) * B, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(T.data(), page_table, sizeof(int32_t) * T.size(), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "copying metadata failed: %s", hipGetErrorString(e));
  const int64_t cap = (int64_t)pps * page_size;
  for (int b = 0; b < B; ++b) {
    const int64_t Lb = L[b];
    if (Lb > cap)
      return fail(PKV_ERR_DEVICE_DATA, "sequence %d: seq_len %lld exceeds pages_per_seq * "
                                       "page_size = %lld", b, (long long)Lb, (long long)cap);
    if (Lb < q_seq_len)
      return fail(PKV_ERR_DEVICE_DATA, "sequence %d: seq_len %lld is shorter than q_seq_len %d",
                  b, (long long)Lb, q_seq_len);
    int64_t lo = 0;
    if (window > 0) lo = std::max<int64_t>(0, Lb - q_seq_len + 1 - window);
    for (int64_t pg = lo / page_size; pg < cdiv(Lb, page_size); ++pg) {
      const int32_t id = T[(size_t)b * pps + pg];
      if (id < 0 || id >= dims->num_pages)
        return fail(PKV_ERR_DEVICE_DATA, "sequence %d: page_table[%d][%lld] = %d is outside "
                                         "[0, %d)", b, b, (long long)pg, id, dims->num_pages);
    }
  }
  g_err.clear();
  return PKV_OK;
}

pkv_status pkv_cache_insert(const void* k_src, const void* k_rope_src, const void* v_src,
                            const int64_t* slot_mapping, void* k_cache, void* v_cache,
                            float cache_scale_inv, const float* cache_scale_inv_dev,
                            const void* q_lo, const void* q_hi, void* q_out, void* stream,
                            const pkv_insert_dims* d) {
  if (d == nullptr) return fail(PKV_ERR_INVALID_ARGUMENT, "dims is NULL");
  if (d->num_tokens < 0) return fail(PKV_ERR_INVALID_ARGUMENT, "num_tokens must be >= 0");
  if (d->num_kv_heads < 1) return fail(PKV_ERR_INVALID_ARGUMENT, "num_kv_heads must be >= 1");
  const int Dk = d->head_dim_k, Dlo = d->head_dim_k_lo, Dv = d->head_dim_v;
  if (Dk < 8 || Dk % 8 || Dlo < 8 || Dlo % 8 || Dlo > Dk || Dv < 0 || Dv % 8)
    return fail(PKV_ERR_INVALID_ARGUMENT,
                "head dims must be multiples of 8 with 8 <= head_dim_k_lo <= head_dim_k "
                "(got k %d, k_lo %d, v %d)", Dk, Dlo, Dv);
  const int ps = d->page_size;
  if (ps != 16 && ps != 32 && ps != 64 && ps != 128)
    return fail(PKV_ERR_INVALID_ARGUMENT, "page_size must be one of 16, 32, 64, 128; got %d", ps);
  if (d->num_pages < 1) return fail(PKV_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
  if (d->layout != PKV_NHD && d->layout != PKV_HND)
    return fail(PKV_ERR_INVALID_ARGUMENT, "kv_layout must be NHD (0) or HND (1); got %d", d->layout);
  if (d->src_dtype != PKV_F16 && d->src_dtype != PKV_BF16)
    return fail(PKV_ERR_INVALID_ARGUMENT, "source dtype must be float16 or bfloat16; got %d",
                d->src_dtype);
  if (d->cache_dtype != d->src_dtype && d->cache_dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_INVALID_ARGUMENT,
                "cache dtype must equal the source dtype or be float8_e4m3fn; got %d for %d",
                d->cache_dtype, d->src_dtype);
  if (q_out != nullptr && (d->num_q_heads < 1 || q_lo == nullptr || (Dlo < Dk && q_hi == nullptr)))
    return fail(PKV_ERR_INVALID_ARGUMENT, "the query concat needs num_q_heads >= 1, q_lo and "
                                          "(when head_dim_k_lo < head_dim_k) q_hi");
  if (!std::isfinite(cache_scale_inv))
    return fail(PKV_ERR_INVALID_ARGUMENT, "cache_scale_inv must be finite");
  if (d->num_tokens == 0) {
    g_err.clear();
    return PKV_OK;
  }
  if (!k_src || !slot_mapping || !k_cache || (Dlo < Dk && !k_rope_src) || (Dv > 0 && (!v_src || !v_cache)))
    return fail(PKV_ERR_INVALID_ARGUMENT, "k_src, slot_mapping, k_cache (and k_rope_src when "
                                          "head_dim_k_lo < head_dim_k, v_src and v_cache when "
                                          "head_dim_v > 0) must not be NULL");
  for (const void* ptr : {k_src, k_rope_src, v_src, (const void*)k_cache, (const void*)v_cache, q_lo,
                          q_hi, (const void*)q_out})
    if (misaligned(ptr, 16))
      return fail(PKV_ERR_INVALID_ARGUMENT, "insert tensors must be 16-byte aligned");
  if (misaligned(slot_mapping, 8) || misaligned(cache_scale_inv_dev, 4))
    return fail(PKV_ERR_INVALID_ARGUMENT, "slot_mapping must be 8-byte and the device scale "
                                          "4-byte aligned");
  pkv::InsertParams p{};
  p.k_src = k_src;
  p.k_rope = k_rope_src;
  p.v_src = v_src;
  p.slot_mapping = slot_mapping;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.q_lo = q_lo;
  p.q_hi = q_hi;
  p.q_out = q_out;
  p.N = d->num_tokens;
  p.Hkv = d->num_kv_heads;
  p.Hq = q_out != nullptr ? d->num_q_heads : 0;
  p.Dk = Dk;
  p.Dlo = Dlo;
  p.Dv = Dv;
  p.ps = ps;
  p.num_pages = d->num_pages;
  p.layout = d->layout;
  p.scale_inv = cache_scale_inv;
  p.scale_inv_dev = cache_scale_inv_dev;
  const int64_t items = (int64_t)p.N * std::max<int64_t>((int64_t)p.Hkv * std::max(Dk, Dv), (int64_t)p.Hq * Dk) / 8;
  if (items >= ((int64_t)1 << 31))
    return fail(PKV_ERR_UNSUPPORTED, "insert too large: %lld 16-byte items in one part (limit 2^31)",
                (long long)items);
  const hipError_t e = pkv::launch_cache_insert(d->src_dtype, d->cache_dtype, p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "cache insert launch failed: %s", hipGetErrorString(e));
  g_err.clear();
  return PKV_OK;
}

pkv_status pkv_head_matmul(const void* x, int64_t xs_m, int64_t xs_h, const void* w, void* y,
                           int64_t ys_m, int64_t ys_h, int M, int H, int K, int N, int dtype,
                           void* stream) {
  if (M < 0 || H < 1 || K < 32 || K % 32 || N < 64 || N % 64)
    return fail(PKV_ERR_INVALID_ARGUMENT, "head_matmul needs M >= 0, H >= 1, K a multiple of 32 "
                                          "and N a multiple of 64 (got M %d, H %d, K %d, N %d)",
                M, H, K, N);
  if (dtype != PKV_F16 && dtype != PKV_BF16)
    return fail(PKV_ERR_INVALID_ARGUMENT, "head_matmul dtype must be float16 or bfloat16; got %d",
                dtype);
  if (xs_m % 8 || xs_h % 8 || ys_m % 4 || ys_h % 4 || xs_m < 0 || xs_h < 0 || ys_m < 0 || ys_h < 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "head_matmul strides must be non-negative, x's multiples "
                                          "of 8 and y's of 4 elements");
  if (M == 0) {
    g_err.clear();
    return PKV_OK;
  }
  if (!x || !w || !y) return fail(PKV_ERR_INVALID_ARGUMENT, "x, w and y must not be NULL");
  if (misaligned(x, 16) || misaligned(w, 16) || misaligned(y, 16))
    return fail(PKV_ERR_INVALID_ARGUMENT, "x, w and y must be 16-byte aligned");
  if ((int64_t)H > 65535 || (int64_t)N / 64 > 65535)
    return fail(PKV_ERR_UNSUPPORTED, "head_matmul: H and N / 64 must be <= 65535");
  pkv::HeadMatmulParams p{};
  p.x = x;
  p.w = w;
  p.y = y;
  p.xs_m = xs_m;
  p.xs_h = xs_h;
  p.ys_m = ys_m;
  p.ys_h = ys_h;
  p.M = M;
  p.H = H;
  p.K = K;
  p.N = N;
  const hipError_t e = pkv::launch_head_matmul(dtype, p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "head_matmul launch failed: %s", hipGetErrorString(e));
  g_err.clear();
  return PKV_OK;
}

pkv_status pkv_merge_attn_states(void* out, const void* o_p, int64_t p_sn, int64_t p_sh,
                                 const float* lse_p, const void* o_s, int64_t s_sn, int64_t s_sh,
                                 const float* lse_s, float* lse_out, int64_t lse_sn, int64_t lse_sh,
                                 int N, int H, int D, int n_prefix, int dtype, void* stream) {
  if (N < 0 || H < 1 || D < 8 || D % 8 || n_prefix < 0 || n_prefix > N)
    return fail(PKV_ERR_INVALID_ARGUMENT, "merge_attn_states needs N >= 0, H >= 1, head_dim a "
                                          "multiple of 8 and 0 <= num_tokens_with_prefix <= N "
                                          "(got N %d, H %d, D %d, prefix %d)", N, H, D, n_prefix);
  if (dtype != PKV_F16 && dtype != PKV_BF16)
    return fail(PKV_ERR_INVALID_ARGUMENT, "merge_attn_states dtype must be float16 or bfloat16");
  if (lse_sn < 0 || lse_sh < 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "log-sum-exp strides must be non-negative");
  if (p_sn < 0 || p_sh < 0 || s_sn < 0 || s_sh < 0 || p_sn % 8 || p_sh % 8 || s_sn % 8 || s_sh % 8)
    return fail(PKV_ERR_INVALID_ARGUMENT, "output strides must be non-negative multiples of 8 "
                                          "elements");
  if (N == 0) {
    g_err.clear();
    return PKV_OK;
  }
  if (!out || !o_s || !lse_s || (n_prefix > 0 && (!o_p || !lse_p)))
    return fail(PKV_ERR_INVALID_ARGUMENT, "out, suffix_out, suffix_lse (and the prefix arrays when "
                                          "num_tokens_with_prefix > 0) must not be NULL");
  if (misaligned(out, 16) || misaligned(o_p, 16) || misaligned(o_s, 16) || misaligned(lse_p, 4) ||
      misaligned(lse_s, 4) || misaligned(lse_out, 4))
    return fail(PKV_ERR_INVALID_ARGUMENT, "outputs must be 16-byte and log-sum-exps 4-byte aligned");
  if ((int64_t)N * H * (D / 8) >= ((int64_t)1 << 31))
    return fail(PKV_ERR_UNSUPPORTED, "merge_attn_states: too many elements (limit 2^34)");
  pkv::MergeParams p{};
  p.out = out;
  p.o_p = o_p;
  p.o_s = o_s;
  p.p_sn = p_sn;
  p.p_sh = p_sh;
  p.s_sn = s_sn;
  p.s_sh = s_sh;
  p.lse_p = lse_p;
  p.lse_s = lse_s;
  p.lse_out = lse_out;
  p.lse_sn = lse_sn;
  p.lse_sh = lse_sh;
  p.N = N;
  p.H = H;
  p.D = D;
  p.n_prefix = n_prefix;
  const hipError_t e = pkv::launch_merge_states(dtype, p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "merge_attn_states launch failed: %s", hipGetErrorString(e));
  g_err.clear();
  return PKV_OK;
}

pkv_status pkv_ragged_attn(const void* q, const void* k, const void* v, const int32_t* cu_q,
                           const int32_t* cu_k, void* out, float* lse, int64_t lse_sn,
                           int64_t lse_sh, int num_seqs, int Hq, int Hkv, int Dqk, int Dv,
                           int total_q, int total_k, int max_q_len, float sm_scale, int causal,
                           int dtype, void* stream) {
  if (num_seqs < 0 || total_q < 0 || total_k < 0 || max_q_len < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv)
    return fail(PKV_ERR_INVALID_ARGUMENT, "ragged_attn needs num_seqs, total_q, total_k, max_q_len "
                                          ">= 0 and num_q_heads a multiple of num_kv_heads (got %d, "
                                          "%d, %d, %d; %d, %d)", num_seqs, total_q, total_k,
                max_q_len, Hq, Hkv);
  if (!((Dqk == 64 && Dv == 64) || (Dqk == 128 && Dv == 128) || (Dqk == 192 && Dv == 128)))
    return fail(PKV_ERR_UNSUPPORTED, "ragged_attn supports head dims (qk, v) = (64, 64), "
                                     "(128, 128) and (192, 128), not (%d, %d)", Dqk, Dv);
  if (dtype != PKV_F16 && dtype != PKV_BF16)
    return fail(PKV_ERR_INVALID_ARGUMENT, "ragged_attn dtype must be float16 or bfloat16");
  if (causal != 0 && causal != 1)
    return fail(PKV_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (!(sm_scale > 0.f) || sm_scale == __builtin_inff())
    return fail(PKV_ERR_INVALID_ARGUMENT, "sm_scale must be positive and finite");
  if (lse_sn < 0 || lse_sh < 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "log-sum-exp strides must be non-negative");
  if (num_seqs > 65535 || Hq > 65535)
    return fail(PKV_ERR_UNSUPPORTED, "ragged_attn: at most 65535 sequences and query heads");
  // the kernel addresses K and V through buffer resources with 32-bit offsets
  // (q, out and lse use 64-bit offsets)
  if ((int64_t)total_k * Hkv * (Dqk > Dv ? Dqk : Dv) * 2 >= ((int64_t)1 << 31))
    return fail(PKV_ERR_UNSUPPORTED, "ragged_attn: K/V tensors must be under 2 GiB");
  if (num_seqs == 0 || max_q_len == 0 || total_q == 0) {
    g_err.clear();
    return PKV_OK;
  }
  if (!q || !out || !cu_q || !cu_k || (total_k > 0 && (!k || !v)))
    return fail(PKV_ERR_INVALID_ARGUMENT, "q, out, cu_seqlens_q, cu_seqlens_k (and k, v when "
                                          "total_k > 0) must not be NULL");
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16) ||
      misaligned(lse, 4) || misaligned(cu_q, 4) || misaligned(cu_k, 4))
    return fail(PKV_ERR_INVALID_ARGUMENT, "q, k, v, out must be 16-byte aligned, lse and "
                                          "cu_seqlens 4-byte aligned");
  pkv::RaggedParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.cu_q = cu_q;
  p.cu_k = cu_k;
  p.out = out;
  p.lse = lse;
  p.lse_sn = lse_sn;
  p.lse_sh = lse_sh;
  p.num_seqs = num_seqs;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.Dqk = Dqk;
  p.Dv = Dv;
  p.total_q = total_q;
  p.total_k = total_k;
  p.max_q_len = max_q_len;
  p.causal = causal;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  const hipError_t e = pkv::launch_ragged_attn(dtype, p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "ragged_attn launch failed: %s", hipGetErrorString(e));
  g_err.clear();
  return PKV_OK;
}

}  // extern "C"
