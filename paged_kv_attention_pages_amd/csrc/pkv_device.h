// pkv_device.h -- device-side building blocks shared by the decode kernels.
//
// Kernel parameter block, sequence/split geometry, element conversions and
// the matrix-core (MFMA) wrappers for gfx950.  Everything here is HIP-path
// code; the CPU oracle shares none of it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// element codes (match pkv_dtype in include/pkv.h)
enum : int { kF16 = 0, kBF16 = 1, kFP8 = 2 };

// Parameters of one decode call, passed by value to every kernel.
struct Params {
  const void* q;              // [B, Tq, Hq, Dqk]
  const void* k;              // paged K cache
  const void* v;              // paged V cache (== k for the latent cache)
  const int32_t* page_table;  // [B, pps]
  const uint32_t* seq_lens;   // [B]
  void* out;                  // [B, Tq, Hq, Dv]
  float* ws_o;                // [B, Hkv, S, R, Dv] unnormalised partial outputs
  float2* ws_ml;              // [B, Hkv, S, R] (running max in log2 units, sum)
  const float* sinks;         // [Hkv, G] or null
  const uint16_t* mask;       // [B, Tq, mask_words16] or null
  int64_t k_page, k_slot, k_head;  // element strides of the K cache
  int64_t v_page, v_slot, v_head;  // element strides of the V cache
  int B, Tq, Hq, Hkv, G, R, Dqk, Dv;
  int ps, pps, num_pages, window, mask_words16;
  int ps_shift;               // log2(ps): page sizes are powers of two
  int split_pages, max_splits;
  int sk_waves;               // > 0: stream-K schedule over that many waves
                              // (or workgroups, for the latent-cache kernel)
  int sk_shift;               // stream-K tiles are 1 << sk_shift tokens
  int sk_hb;                  // matrix-core stream-K: waves (KV heads) per workgroup
  float qk_scale_log2;        // q_scale * kv_scale / sqrt(Dqk) * log2(e)
  float out_scale;            // kv_scale (V dequantisation, applied once)
  // device-resident scales (null: the host values above hold)
  const float* q_scale_dev;
  const float* kv_scale_dev;
  float q_scale, kv_scale;    // host values, for a kernel that reads one scale
  float qk_unit;              // Dqk^-1/2 * log2(e)
  // single-launch merge (matrix-core stream-K): per-unit counters and the
  // call's generation; fused == 0 leaves the merge to the combine kernel
  unsigned long long* ws_cnt; // [B * Hkv]
  unsigned gen;
  int fused;
  // E4M3 output (xqa `output` in the KV dtype): stored value =
  // round(out * rcp_out_scale); 0 = 16-bit output in q's dtype
  int out_fp8;
  float rcp_out_scale;
  // latent stream-K partials in the P.V waves' register order, 64 rows a
  // slot (split_mla_ws.hip; merged by combine_lat_kernel)
  int ws_lanes;
  // matrix-core stream-K over sk_waves == B * Hkv waves: 1 = when the units
  // are even (sk_units_even) each unit gets one wave and nothing is cut (the
  // combine then finds nothing to merge), otherwise equal shares as usual;
  // 2 = each unit gets one wave always (short sequences; no combine runs)
  int sk_units;
};

// Scales from device memory when the call passed them there: every kernel
// calls this first, so all of them see the same values.
__device__ __forceinline__ void resolve_scales(Params& p) {
  if (p.q_scale_dev != nullptr || p.kv_scale_dev != nullptr) {
    const float qs = p.q_scale_dev != nullptr ? *p.q_scale_dev : p.q_scale;
    const float ks = p.kv_scale_dev != nullptr ? *p.kv_scale_dev : p.kv_scale;
    p.qk_scale_log2 = qs * ks * p.qk_unit;
    p.out_scale = ks;
  }
}

// Token range of sequence b that any of its query rows can see, and the
// split-KV chunking of the pages that hold it.  Shared by the split and the
// combine kernels so both agree on the number of splits of a sequence.
struct SeqGeom {
  int L;        // length, clamped to pps * ps
  int lo;       // first token visible to the earliest query row
  int p0;       // first page holding a visible token
  int npages;   // pages from p0 through the one holding token L-1
  int nsplits;  // ceil(npages / split_pages)
};

__device__ __forceinline__ SeqGeom seq_geom(const Params& p, int b) {
  SeqGeom g;
  uint32_t Lraw = p.seq_lens[b];
  int cap = p.pps * p.ps;
  g.L = Lraw > (uint32_t)cap ? cap : (int)Lraw;
  int lo = 0;
  if (p.window > 0) {
    lo = g.L - p.Tq + 1 - p.window;
    lo = lo < 0 ? 0 : lo;
  }
  g.lo = lo;
  if (g.L <= lo) {
    g.p0 = 0;
    g.npages = 0;
    g.nsplits = 0;
    return g;
  }
  g.p0 = lo / p.ps;
  g.npages = (g.L + p.ps - 1) / p.ps - g.p0;
  g.nsplits = p.split_pages > 0 ? (g.npages + p.split_pages - 1) / p.split_pages : 0;
  return g;
}

// ------------------------------------------------------- stream-K schedule
// The stream-K tiles (1 << sk_shift tokens, aligned) that a sequence's query
// rows can see, [tile0, tile0 + ntiles).
__device__ __forceinline__ int seq_tiles(const Params& p, int b, int* tile0) {
  const SeqGeom g = seq_geom(p, b);
  const int sh = p.sk_shift, m = (1 << sh) - 1;
  *tile0 = g.lo >> sh;
  return g.L > g.lo ? ((g.L + m) >> sh) - (g.lo >> sh) : 0;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// Stream-K tile space: unit (b, kvh) owns the visible tiles of sequence b
// for KV head kvh; units are laid end to end KV-head-major, so unit (b, kvh)
// starts at kvh * T1 + pre_b, with T1 the tiles of one KV head over all
// sequences and pre_b the tiles of the sequences before b.  Wave w of W takes
// tiles [w T / W, (w+1) T / W), T = Hkv T1; when Hkv divides W, waves w and
// w + k W / Hkv take the same tiles of KV heads kvh and kvh + k.
// Lane l holds pre_b and n_b of sequences b = l + 64 c, c < C (B <= 64 C):
// C = 4 (up to 256 sequences) everywhere; the matrix-core kernel and its
// combine also come with C = 16 (up to 1024 sequences, 32 more registers).
constexpr int kSkMaxBatch = 256;
constexpr int kSkMaxBatchWide = 1024;
template <int C>
struct SkSchedC {
  int64_t T;     // total tiles
  int T1;        // tiles of one KV head
  int pre[C];    // exclusive prefix of tiles per sequence (lane's sequences)
  int cnt[C];    // tiles per sequence
};
using SkSched = SkSchedC<4>;

// First global tile of unit (b, kvh), given pre_b.
template <int C>
__device__ __forceinline__ int64_t sk_unit_start(const SkSchedC<C>& s, int kvh, int pre) {
  return (int64_t)kvh * s.T1 + pre;
}

template <int C = 4>
__device__ __forceinline__ SkSchedC<C> sk_schedule(const Params& p) {
  SkSchedC<C> s;
  const int lane = threadIdx.x & 63;
  int carry = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int b = lane + 64 * c;
    int t0;
    const int n = (64 * c < p.B && b < p.B) ? seq_tiles(p, b, &t0) : 0;
    const int inc = wave_scan(n) + carry;
    s.pre[c] = inc - n;
    s.cnt[c] = n;
    carry = __builtin_amdgcn_readlane(inc, 63);
  }
  s.T1 = carry;
  s.T = (int64_t)carry * p.Hkv;
  return s;
}

// Waves that get work: at most one per 8 tiles, so every wave with work has
// at least 8 tiles (and none in 0 .. W_eff-1 is empty); the rest exit.
__device__ __forceinline__ int sk_waves_eff(int64_t T, int W) {
  const int64_t cap = T / 8 > 0 ? T / 8 : 1;
  return (int)(cap < W ? cap : W);
}

// First tile of wave w of W: floor(w T / W).
__device__ __forceinline__ int64_t sk_wave_start(int64_t T, int w, int W) {
  return (T * (int64_t)w) / W;
}

// The wave whose range holds global tile x: the largest w with start(w) <= x.
__device__ __forceinline__ int sk_wave_of(int64_t T, int64_t x, int W) {
  return (int)(((x + 1) * (int64_t)W + T - 1) / T) - 1;
}

// Whether the units are even enough to give each its own wave: the longest
// unit's tiles times the unit count within 5/4 of all tiles, i.e. one wave
// per unit takes at most a quarter longer than equal shares of the same
// tiles (which pay for their cuts and a merge pass instead).  Empty units
// count, as waves with nothing to do.  Wave-uniform.
template <int C>
__device__ __forceinline__ bool sk_units_even(const Params& p, const SkSchedC<C>& s) {
  int mx = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) mx = max(mx, s.cnt[c]);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mx = max(mx, __shfl_xor(mx, d));
  mx = __builtin_amdgcn_readfirstlane(mx);
  return 4 * (int64_t)mx * p.B <= 5 * (int64_t)s.T1;
}

// Unit holding global tile x (x < T): sequence b, KV head kvh, its first
// global tile, and its tile count.  Wave-uniform.
struct SkUnit {
  int b, kvh, ntiles;
  int64_t start;
};

// pre_b and n_b of sequence b (wave-uniform b): read every chunk's lane and
// select on the scalar side, so the per-lane arrays are never indexed
// dynamically (which would put them in scratch memory).
template <int C>
__device__ __forceinline__ void sk_seq_of(const SkSchedC<C>& s, int b, int* pre, int* n) {
  const int ln = b & 63, c = b >> 6;
  int pr = 0, nn = 0;
#pragma unroll
  for (int k = 0; k < C; ++k) {
    const int pk = __builtin_amdgcn_readlane(s.pre[k], ln), nk = __builtin_amdgcn_readlane(s.cnt[k], ln);
    pr = c == k ? pk : pr;
    nn = c == k ? nk : nn;
  }
  *pre = pr;
  *n = nn;
}

template <int C>
__device__ __forceinline__ SkUnit sk_locate(const Params& p, const SkSchedC<C>& s, int64_t x) {
  SkUnit u;
  u.kvh = (int)(x / s.T1);
  const int xr = (int)(x - (int64_t)u.kvh * s.T1);
  // last sequence whose first tile is <= xr (it has tiles, since xr < T1)
  int best = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int b = (threadIdx.x & 63) + 64 * c;
    const bool ok = b < p.B && s.pre[c] <= xr;
    const uint64_t m = __ballot(ok);
    if (m != 0) best = 64 * c + 63 - __builtin_clzll(m);
  }
  u.b = best;
  int pre, n;
  sk_seq_of(s, best, &pre, &n);
  u.ntiles = n;
  u.start = sk_unit_start(s, u.kvh, pre);
  return u;
}

// ---------------------------------------------------------------- vectors
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// D(16x16) += A(16x32) * B(32x16).  Lane l supplies A[l%16][8(l/16)..+8] and
// B[8(l/16)..+8][l%16] as eight 16-bit values in four dwords; it receives
// D[4(l/16)+i][l%16], i = 0..3.
template <int QT>
__device__ __forceinline__ f32x4 mfma_k32(uint4 a, uint4 b, f32x4 c) {
  if constexpr (QT == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// D(16x16) += A(16x16) * B(16x16).  Lane l supplies A[l%16][4(l/16)..+4] and
// B[4(l/16)..+4][l%16] as four 16-bit values in two dwords.
template <int QT>
__device__ __forceinline__ f32x4 mfma_k16(uint2 a, uint2 b, f32x4 c) {
  if constexpr (QT == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a),
                                                     __builtin_bit_cast(bf16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// ------------------------------------------------------------ buffer loads
// Raw buffer loads through a resource that spans one cache page: offsets are
// 32-bit and relative to the page, and a resource with zero size makes every
// load return zeros without touching memory -- used for pipeline slots past
// the end of a split and for page ids outside the cache, so that every
// pipeline step issues the same number of loads.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Cache policy of the K/V stream: non-temporal ("nt"), so the caches do not
// keep lines that are read once.  Measured on the Llama-3-8B-shaped GQA
// decode: split kernel 193.7 us with the default policy, 173.8 us with nt.
constexpr int kStreamPolicy = 2;

// N 32-bit words at byte offset voff + soff (K/V stream: non-temporal unless
// the caller asks for another policy)
template <int N, int POL = kStreamPolicy>
__device__ __forceinline__ void buf_load(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint32_t* w) {
  if constexpr (N >= 4) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 4 * i, soff, POL);
      w[i] = a[0]; w[i + 1] = a[1]; w[i + 2] = a[2]; w[i + 3] = a[3];
    }
  } else if constexpr (N == 2) {
    u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, POL);
    w[0] = a[0]; w[1] = a[1];
  } else {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, POL);
  }
}

// ------------------------------------------------------------ conversions
// Two fp32 -> packed 16-bit pair (round to nearest even), low half = x.
template <int QT>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  if constexpr (QT == kBF16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 v = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// The two 16-bit values of a packed pair, widened to fp32 (exact).
template <int QT>
__device__ __forceinline__ float2 unpack2(uint32_t w) {
  if constexpr (QT == kBF16) {
    return make_float2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
  } else {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 h = __builtin_bit_cast(f16x2, w);
    return make_float2((float)h[0], (float)h[1]);
  }
}

// ------------------------------------------------------------ output stores
// Four consecutive output elements starting at element e (e % 4 == 0): in
// q's dtype, or as E4M3 bytes of value * rcp_out_scale (binary32 product,
// clamped to +-448 with NaN kept, then v_cvt_pk_fp8_f32's round to nearest
// even).
__device__ __forceinline__ float sat448(float x) { return x != x ? x : fminf(fmaxf(x, -448.f), 448.f); }

template <int QT>
__device__ __forceinline__ void store_out4(const Params& p, int64_t e, float a, float b, float c, float d) {
  if (p.out_fp8) {
    const float s = p.rcp_out_scale;
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a * s), sat448(b * s), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c * s), sat448(d * s), w, true);
    *(uint32_t*)((uint8_t*)p.out + e) = w;
  } else {
    *(uint2*)((uint16_t*)p.out + e) = make_uint2(pack2<QT>(a, b), pack2<QT>(c, d));
  }
}

// One output element.
template <int QT>
__device__ __forceinline__ void store_out1(const Params& p, int64_t e, float a) {
  if (p.out_fp8)
    ((uint8_t*)p.out)[e] =
        (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(sat448(a * p.rcp_out_scale), 0.f, 0, false) & 0xff);
  else
    ((uint16_t*)p.out)[e] = (uint16_t)(pack2<QT>(a, 0.f) & 0xffffu);
}

// Softmax reference slack (log2 units): a kernel moves its running
// reference max only when a tile's max passes it by more than this, so the
// probabilities stay below 2^kSlack -- held by bf16, f16 and the fp32
// accumulators with unchanged relative precision -- and the accumulators
// are rescaled far less often.  Normalisation and the split merge are exact
// for any reference.
constexpr float kSlack = 8.f;

// Four OCP e4m3fn bytes -> four fp32 (exact).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* f) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

// Four e4m3fn bytes -> two dwords of the 16-bit compute type.  Every e4m3fn
// value is exact in bf16 and in f16, so this conversion is exact: gfx950's
// v_cvt_scalef32_pk_{bf16,f16}_fp8 with scale 1.0 converts two bytes per
// instruction (a probe over every code in every byte position matched the
// fp32 route bit for bit, NaN codes to NaN).
template <int QT>
__device__ __forceinline__ uint2 fp8x4_to_16(uint32_t w) {
  if constexpr (QT == kBF16) {
    const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
  } else {
    const f16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    const f16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
  }
}

// 16-bit element e (0..7) of a uint4, as the low 16 bits of a dword.
__device__ __forceinline__ uint32_t half_of(const uint4& v, int e) {
  uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// Butterfly max across the four 16-lane rows of a wave (lanes l, l^16,
// l^32, l^48): every lane ends with the max of its column.  gfx950's
// v_permlane16_swap / v_permlane32_swap exchange 16-lane rows and 32-lane
// halves between two registers in the VALU; with the value in both
// operands, each lane ends up holding itself in one result and its partner
// (l ^ 16, resp. l ^ 32) in the other, so no LDS round trip is needed.
__device__ __forceinline__ float2 row_partner16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float2 row_partner32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float max_across_rows(float x) {
  float2 a = row_partner16(x);
  x = fmaxf(a.x, a.y);
  a = row_partner32(x);
  return fmaxf(a.x, a.y);
}

__device__ __forceinline__ float sum_across_rows(float x) {
  float2 a = row_partner16(x);
  x = a.x + a.y;
  a = row_partner32(x);
  return a.x + a.y;
}

// Row r of the (G * Tq) rows sharing one KV head: query token r / G, head
// kvh * G + r % G.
__device__ __forceinline__ int64_t q_row_offset(const Params& p, int b, int kvh, int r) {
  int iq = r / p.G, gh = r - iq * p.G;
  return ((int64_t)(b * p.Tq + iq) * p.Hq + kvh * p.G + gh);
}

// Visibility of token t to query row r (the window and the spec-decode mask;
// t < L is part of the test).  Written without branches or short-circuit
// operators: the result feeds a select, and divergent early returns here
// were structured wrongly by the compiler for the first element of the
// score fragment (the bit test was dropped), so every term is evaluated and
// combined with bitwise operators.
struct RowVis {
  int lo;          // first visible token (the window is a lower bound only), may be negative
  int draft0;      // first draft position L - Tq (mask applies from here)
  uint32_t bits;   // draft mask bits of this row (all ones without a mask)
  __device__ __forceinline__ bool operator()(int t, int L) const {
    const uint32_t sh = (uint32_t)(t - draft0) & 31u;
    const bool in_range = (t >= lo) & (t < L);
    const bool drafted = (t < draft0) | (((bits >> sh) & 1u) != 0u);
    return in_range & drafted;
  }
};

__device__ __forceinline__ RowVis row_vis(const Params& p, int b, int L, int r) {
  RowVis v;
  int iq = r / p.G;
  v.lo = p.window > 0 ? L - p.Tq + iq - p.window + 1 : INT32_MIN;
  if (p.Tq > 1 && p.mask != nullptr) {
    v.draft0 = L - p.Tq;
    const uint16_t* row = p.mask + ((int64_t)b * p.Tq + iq) * p.mask_words16;
    v.bits = (uint32_t)row[0] | ((uint32_t)row[1] << 16);
  } else {
    v.draft0 = INT32_MAX;
    v.bits = 0xffffffffu;
  }
  return v;
}

}  // namespace pkv
