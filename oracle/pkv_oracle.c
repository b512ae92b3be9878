/*
 * pkv_oracle.c -- plain fp64 CPU oracle for paged-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the HIP path is checked against.  Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load it; the
 * library's own decode path never calls it.  It shares no code, header,
 * table or constant with the HIP path.
 *
 * What it computes (exact softmax attention over a paged cache):
 *   FlashInfer `flashinfer.xqa.xqa` reference page -- the signature, the
 *   shapes and dtypes of q / k_cache / v_cache / page_table / seq_lens /
 *   output, `num_kv_heads`, `page_size`, `sinks`, `q_scale`, `kv_scale`,
 *   `sliding_win_size`, `kv_layout`, `q_seq_len`, `mask`, and the closing
 *   note (head_group_ratio = num_q_heads / num_kv_heads,
 *   max_seq_len = pages_per_seq * page_size).
 *   vLLM `models/kimi_k3/nvidia/mla` page, MultiHeadLatentAttention: the
 *   latent cache row is [kv_c_normed | k_pe] (the key-concat/cache-insert
 *   step), attention runs over it as one KV head (`get_kv_cache_spec`,
 *   `forward_mqa`), and its output is kv_lora_rank wide (`_v_up_proj`), so V
 *   is the leading head_dim_v entries of each cached row (`v_from_k`).
 *
 * Readings taken where the pages leave a step open (each is listed in the
 * design notes):
 *   - logit = q_scale * kv_scale / sqrt(head_dim_qk) * q.k: q_scale and
 *     kv_scale multiply the query and the dequantised cache, and the softmax
 *     scale is the usual 1/sqrt(head dim) (the xqa call has no separate
 *     softmax-scale argument; the vllm-omni trtllm_attn page passes the
 *     softmax scale as the first-matmul scale and 1.0 as the second).
 *   - V is dequantised with the same kv_scale as K.
 *   - a sink is a logit-domain value: it adds e^(sink - M) to the softmax
 *     denominator and nothing to the numerator, once per (sequence, query
 *     token, head); head h uses sinks[h / G][h % G].
 *   - window W > 0 bounds visibility from below only: position pos sees t
 *     only if t > pos - W.  No upper bound comes from the window; tokens
 *     after pos are hidden only by the draft mask (and t < seq_len), so a
 *     NULL mask with q_seq_len > 1 lets every draft see every other draft.
 *   - the q_seq_len draft tokens are the last positions of the sequence; a
 *     mask row is little-endian 32-bit words made of uint16 pairs, bit j set
 *     means draft j is visible; tokens before the drafts are always visible;
 *     a NULL mask (or q_seq_len == 1) hides nothing.
 *   - no visible token: the output row is zero.
 * Unused page-table entries and slots outside the visible range are never
 * read (they may hold anything, including out-of-range ids and NaN).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- storage-format decoders, written from the format definitions ---- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits; exponent 0 is subnormal (f * 2^-24), 31 is infinity / NaN. */
double pkvo_decode_f16(uint16_t h)
{
  int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 15 - 10);
  return s ? -v : v;
}

/* bfloat16: the upper half of an IEEE 754 binary32 -- 1 sign bit, 8
 * exponent bits (bias 127), 7 fraction bits; exponent 0 is subnormal
 * (f * 2^-133), 255 is infinity / NaN. */
double pkvo_decode_bf16(uint16_t b)
{
  int s = (b >> 15) & 1, e = (b >> 7) & 0xff, f = b & 0x7f;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133);
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(128 + f), e - 127 - 7);
  return s ? -v : v;
}

/* OCP 8-bit floating point, E4M3 ("fn"): 1 sign bit, 4 exponent bits
 * (bias 7), 3 fraction bits; exponent 0 is subnormal (f * 2^-9); there is
 * no infinity and only S.1111.111 is NaN, so the largest finite value is
 * 1.75 * 2^8 = 448. */
double pkvo_decode_e4m3fn(uint8_t x)
{
  int s = (x >> 7) & 1, e = (x >> 3) & 0xf, f = x & 7;
  double v;
  if (e == 15 && f == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)f, -9);
  else
    v = ldexp((double)(8 + f), e - 7 - 3);
  return s ? -v : v;
}

/* dtype codes of this oracle (its own; not shared with the library) */
enum { PKVO_F16 = 0, PKVO_BF16 = 1, PKVO_E4M3 = 2 };
enum { PKVO_NHD = 0, PKVO_HND = 1 };

typedef struct pkvo_problem {
  int batch, q_seq_len, num_q_heads, num_kv_heads;
  int head_dim_qk, head_dim_v;
  int page_size, pages_per_seq, num_pages;
  int q_dtype, kv_dtype, layout;
  int window;      /* 0 = off */
  int v_from_k;    /* V row = first head_dim_v entries of the K row */
  int num_threads; /* <= 0: OpenMP default */
  double q_scale, kv_scale;
} pkvo_problem;

static double load_elem(const void *base, int dtype, size_t idx)
{
  switch (dtype) {
  case PKVO_F16:
    return pkvo_decode_f16(((const uint16_t *)base)[idx]);
  case PKVO_BF16:
    return pkvo_decode_bf16(((const uint16_t *)base)[idx]);
  default:
    return pkvo_decode_e4m3fn(((const uint8_t *)base)[idx]);
  }
}

/* Element index of entry d of the row (page, slot, kv head) in a cache
 * whose rows are `row` elements wide.
 *   NHD: [num_pages, page_size, num_kv_heads, row]
 *   HND: [num_pages, num_kv_heads, page_size, row] */
static size_t cache_index(const pkvo_problem *p, int page, int slot, int kvh,
                          int row, int d)
{
  size_t P = (size_t)page, S = (size_t)slot, H = (size_t)kvh;
  size_t ps = (size_t)p->page_size, nh = (size_t)p->num_kv_heads;
  if (p->layout == PKVO_NHD)
    return ((P * ps + S) * nh + H) * (size_t)row + (size_t)d;
  return ((P * nh + H) * ps + S) * (size_t)row + (size_t)d;
}

/* Visibility of token t to query token i of sequence b (length L). */
static int is_visible(const pkvo_problem *p, const uint16_t *mask, int b,
                      int i, long L, long t)
{
  long Tq = p->q_seq_len;
  long pos = L - Tq + i;
  if (t < 0 || t >= L)
    return 0;
  if (p->window > 0 && !(t > pos - p->window))
    return 0;
  if (Tq > 1 && mask != NULL && t >= L - Tq) {
    long j = t - (L - Tq);
    long words16 = ((Tq + 31) / 32) * 2;
    const uint16_t *row = mask + ((size_t)b * Tq + i) * words16;
    uint32_t w = (uint32_t)row[2 * (j / 32)] |
                 ((uint32_t)row[2 * (j / 32) + 1] << 16);
    if (!((w >> (j % 32)) & 1u))
      return 0;
  }
  return 1;
}

/* out: [batch, q_seq_len, num_q_heads, head_dim_v] doubles.
 * Returns 0, or 1 + b for the first sequence b whose visible tokens need a
 * page id outside [0, num_pages), or -1 on malformed problem sizes. */
int pkvo_decode(const pkvo_problem *p, const void *q, const void *k_cache,
                const void *v_cache, const int32_t *page_table,
                const uint32_t *seq_lens, const float *sinks,
                const uint16_t *mask, double *out)
{
  if (p->batch < 0 || p->q_seq_len < 1 || p->num_kv_heads < 1 ||
      p->num_q_heads % p->num_kv_heads != 0 || p->head_dim_qk < 1 ||
      p->head_dim_v < 1 || p->page_size < 1 || p->pages_per_seq < 0 ||
      (p->v_from_k && p->head_dim_v > p->head_dim_qk))
    return -1;
  const int Tq = p->q_seq_len, Hq = p->num_q_heads;
  const int G = Hq / p->num_kv_heads;
  const int Dk = p->head_dim_qk, Dv = p->head_dim_v;
  const int krow = Dk, vrow = p->v_from_k ? Dk : Dv;
  const void *vbase = p->v_from_k ? k_cache : v_cache;
  const double c = p->q_scale / sqrt((double)Dk);
  const long items = (long)p->batch * Tq * Hq;
  int bad = 0;

#ifdef _OPENMP
  int nt = p->num_threads > 0 ? p->num_threads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
#endif
  for (long it = 0; it < items; ++it) {
    const int h = (int)(it % Hq);
    const int i = (int)((it / Hq) % Tq);
    const int b = (int)(it / ((long)Hq * Tq));
    const int kvh = h / G, g = h % G;
    long L = (long)seq_lens[b];
    if (L > (long)p->pages_per_seq * p->page_size)
      L = (long)p->pages_per_seq * p->page_size; /* outside the contract */
    double *o = out + (size_t)it * Dv;
    const size_t qoff = (size_t)it * Dk;

    double *logit = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    char *vis = (char *)calloc((size_t)(L > 0 ? L : 1), 1);
    double M = -INFINITY;
    int any = 0, my_bad = 0;

    /* logits of the visible tokens, dereferencing the page table */
    for (long t = 0; t < L; ++t) {
      if (!is_visible(p, mask, b, i, L, t))
        continue;
      int32_t page = page_table[(size_t)b * p->pages_per_seq + t / p->page_size];
      int slot = (int)(t % p->page_size);
      if (page < 0 || page >= p->num_pages) {
        my_bad = 1;
        continue;
      }
      double dot = 0.0;
      for (int d = 0; d < Dk; ++d) {
        double qd = load_elem(q, p->q_dtype, qoff + (size_t)d);
        double kd = p->kv_scale *
                    load_elem(k_cache, p->kv_dtype,
                              cache_index(p, page, slot, kvh, krow, d));
        dot += qd * kd;
      }
      logit[t] = c * dot;
      vis[t] = 1;
      any = 1;
      if (logit[t] > M)
        M = logit[t];
    }

    for (int d = 0; d < Dv; ++d)
      o[d] = 0.0;
    if (any) {
      double sink = 0.0;
      if (sinks != NULL) {
        sink = (double)sinks[(size_t)kvh * G + g];
        if (sink > M)
          M = sink;
      }
      double den = sinks != NULL ? exp(sink - M) : 0.0;
      for (long t = 0; t < L; ++t) {
        if (!vis[t])
          continue;
        double w = exp(logit[t] - M);
        den += w;
        int32_t page =
            page_table[(size_t)b * p->pages_per_seq + t / p->page_size];
        int slot = (int)(t % p->page_size);
        for (int d = 0; d < Dv; ++d)
          o[d] += w * p->kv_scale *
                  load_elem(vbase, p->kv_dtype,
                            cache_index(p, page, slot, kvh, vrow, d));
      }
      for (int d = 0; d < Dv; ++d)
        o[d] /= den;
    }
    free(logit);
    free(vis);
    if (my_bad) {
#ifdef _OPENMP
#pragma omp critical
#endif
      {
        if (bad == 0 || b + 1 < bad)
          bad = b + 1;
      }
    }
  }
  return bad;
}

/* Number of threads the OpenMP runtime would use (for reporting). */
int pkvo_max_threads(void)
{
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ==================================================================== */
/* The cache write side: insert the new tokens' rows at slot_mapping.   */
/*                                                                      */
/* vLLM `models/kimi_k3/nvidia/mla` page, `_decode_concat_cache`: one   */
/* fused step builds the decode query [ql_nope | q_pe] and writes each  */
/* new token's latent row [kv_c_normed | k_pe] into the paged cache at  */
/* its slot_mapping entry; a quantised (fp8) cache stores the row times */
/* `cache_scale_inv` (the reciprocal of the cache scale, `_k_scale_inv`,*/
/* precomputed in `process_weights_after_loading`).  The same write for */
/* a K/V cache (the xqa page's k_cache / v_cache layouts) is the step   */
/* just before decode attention.                                        */
/*                                                                      */
/* Readings (listed in the design notes):                               */
/*   - a slot is page * page_size + offset; a negative slot (padding)   */
/*     or one past num_pages * page_size writes nothing;                */
/*   - a 16-bit cache of the source dtype receives the source bits;     */
/*   - an E4M3 cache receives the nearest E4M3 value (ties to the even  */
/*     code) of the binary32 product value * cache_scale_inv, with      */
/*     magnitudes beyond the largest finite value 448 stored as +-448   */
/*     (saturation) and NaN as S.1111.111.                              */
/* ==================================================================== */

/* OCP E4M3 ("fn") encoder, by definition: the representable value nearest
 * to x (searched over every finite code), ties to the code with an even
 * last fraction bit; |x| >= 448 saturates to 448; NaN gives 0x7F. */
uint8_t pkvo_encode_e4m3fn(float xf)
{
  const double x = (double)xf;
  if (isnan(x))
    return 0x7f;
  const int s = signbit(x) ? 0x80 : 0;
  const double a = fabs(x);
  if (a >= 448.0)
    return (uint8_t)(s | 0x7e);
  int best = 0;
  double bd = a; /* distance to code 0 (+0) */
  for (int c = 1; c <= 0x7e; ++c) {
    const double d = fabs(pkvo_decode_e4m3fn((uint8_t)c) - a);
    if (d < bd || (d == bd && (c & 1) == 0)) {
      best = c;
      bd = d;
    }
  }
  return (uint8_t)(s | best);
}

typedef struct pkvo_insert {
  int num_tokens, num_kv_heads;
  int head_dim_k;    /* cache K row width                                   */
  int head_dim_k_lo; /* leading part of the K row from k_src; the rest from k_rope */
  int head_dim_v;    /* V row width; 0: no V cache (latent cache)            */
  int page_size, num_pages, layout;
  int src_dtype, cache_dtype;
  float cache_scale_inv;
} pkvo_insert;

static size_t insert_index(const pkvo_insert *p, int64_t page, int off, int h, int D, int d)
{
  if (p->layout == PKVO_NHD)
    return (((size_t)page * p->page_size + off) * p->num_kv_heads + h) * D + d;
  return (((size_t)page * p->num_kv_heads + h) * p->page_size + off) * D + d;
}

static void insert_elem(const pkvo_insert *p, void *cache, size_t idx, uint16_t bits)
{
  if (p->cache_dtype == PKVO_E4M3) {
    const double v = p->src_dtype == PKVO_F16 ? pkvo_decode_f16(bits) : pkvo_decode_bf16(bits);
    const float y = (float)v * p->cache_scale_inv; /* one binary32 rounding */
    ((uint8_t *)cache)[idx] = pkvo_encode_e4m3fn(y);
  } else {
    ((uint16_t *)cache)[idx] = bits;
  }
}

/* k_src [N, Hkv, Dlo], k_rope [N, Hkv, Dk - Dlo] (NULL when Dlo == Dk),
 * v_src [N, Hkv, Dv] (NULL when Dv == 0), slot_mapping [N].  Returns 0, or
 * -1 for malformed sizes. */
int pkvo_cache_insert(const pkvo_insert *p, const uint16_t *k_src, const uint16_t *k_rope,
                      const uint16_t *v_src, const int64_t *slot_mapping, void *k_cache,
                      void *v_cache)
{
  if (p->num_tokens < 0 || p->num_kv_heads < 1 || p->head_dim_k < 1 ||
      p->head_dim_k_lo < 1 || p->head_dim_k_lo > p->head_dim_k || p->head_dim_v < 0 ||
      p->page_size < 1 || p->num_pages < 1)
    return -1;
  const int H = p->num_kv_heads, Dk = p->head_dim_k, Dlo = p->head_dim_k_lo, Dv = p->head_dim_v;
  for (int i = 0; i < p->num_tokens; ++i) {
    const int64_t s = slot_mapping[i];
    if (s < 0 || s >= (int64_t)p->num_pages * p->page_size)
      continue;
    const int64_t page = s / p->page_size;
    const int off = (int)(s % p->page_size);
    for (int h = 0; h < H; ++h) {
      for (int d = 0; d < Dk; ++d) {
        const uint16_t bits = d < Dlo ? k_src[((size_t)i * H + h) * Dlo + d]
                                      : k_rope[((size_t)i * H + h) * (Dk - Dlo) + (d - Dlo)];
        insert_elem(p, k_cache, insert_index(p, page, off, h, Dk, d), bits);
      }
      for (int d = 0; d < Dv; ++d)
        insert_elem(p, v_cache, insert_index(p, page, off, h, Dv, d),
                    v_src[((size_t)i * H + h) * Dv + d]);
    }
  }
  return 0;
}
