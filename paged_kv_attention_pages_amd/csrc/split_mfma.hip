// split_mfma.hip -- split-KV paged decode attention on the gfx950 matrix cores,
// for up to 16 query rows per KV head (rows = head group x query tokens).
//
// One wave handles one (sequence, KV head, split); a split is a run of at most
// 64 pages (FlashInfer xqa page: multi-block decode through a
// `workspace_buffer`; here the partials go to the workspace and a combine
// kernel merges them).  The page ids of the split are read once, one per
// lane, and broadcast with v_readlane; the cache is streamed through a
// register pipeline of 16-token tiles (2 to 4 stages, by tile size): while
// tile t is being computed the next tiles are in flight, and every step
// issues the same number of buffer loads so the wait counts stay static.
//
// Per 16-token tile, with the rows padded to 16:
//   S^T (16 tokens x 16 rows) = K (16 x D) . Q^T (D x 16)  -- 16x16x32 MFMAs
//   O^T (D x 16 rows)        += V^T (D x 16) . P^T (16 x 16) -- 16x16x16 MFMAs
// Putting the tokens on the M side of both products leaves every lane with
// one query row (l % 16) in both S^T and O^T, so P never leaves registers
// and the softmax rescale is per lane.  K and V come straight from HBM into
// the operand registers with 16-byte loads; the dimension order inside the
// dot products is permuted so that each lane's loads are contiguous
// (the sums do not depend on the order).
#include "pkv_device.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

// 16-byte chunk (8 elements) of the head dimension that lane group g feeds
// into QK k-step s.  16-bit caches: chunk 4s+g.  fp8 caches: chunks 8u+2g and
// 8u+2g+1 for steps 2u and 2u+1, so one 16-byte load serves two steps.  In
// both cases load i of lane group g starts at byte 64 i + 16 g of the row.
template <int KT>
__device__ __forceinline__ int qk_chunk(int s, int g) {
  if constexpr (KT == kFP8)
    return 8 * (s >> 1) + 2 * g + (s & 1);
  else
    return 4 * s + g;
}

template <int KT, int D>
struct Tile {
  static constexpr int ELEM = KT == kFP8 ? 1 : 2;
  static constexpr int KSTEPS = D / 32;
  static constexpr int KLOADS = KT == kFP8 ? KSTEPS / 2 : KSTEPS;  // 16-byte loads per lane
  static constexpr int DT = D / 16;                // O^T tiles = V elements per lane/token
  static constexpr int VW = DT * ELEM / 4;         // V words per lane per token
  // pipeline depth: as many 16-token tiles in flight as fit beside the
  // accumulator and Q in the 256 architected VGPRs (bf16 D=128: 3 stages of
  // 32 registers; fp8 D=128: 4 of 16; bf16 D=256: 2 of 64)
  static constexpr int REGS = 4 * KLOADS + 4 * VW;
  static constexpr int STAGES = REGS >= 64 ? 2 : REGS >= 32 ? 3 : 4;
  uint32_t k[KLOADS][4];
  uint32_t v[4][VW];
};

// Per-wave constants of the tile loads.
struct Stream {
  int my_page;      // page id of split page `lane` (lanes >= pages in split: -1)
  int pg_begin;     // first page of the split (sequence-relative)
  int tile_end;     // one past the last 16-token tile of the split
  int k_lane;       // lane part of the K byte offset inside a page
  int v_lane;       // lane part of the V byte offset inside a page
  uint32_t k_page_bytes, v_page_bytes;
};

template <int KT, int D>
__device__ __forceinline__ void load_tile(const Params& p, const Stream& st, int t,
                                          Tile<KT, D>& T) {
  using TT = Tile<KT, D>;
  const int tok0 = t << 4;
  const int j = (tok0 >> p.ps_shift) - st.pg_begin;
  int page = __builtin_amdgcn_readlane(st.my_page, j & 63);
  const bool ok = t < st.tile_end && (unsigned)page < (unsigned)p.num_pages;
  page = ok ? page : 0;
  const int slot0 = tok0 & (p.ps - 1);
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc((const uint8_t*)p.k + (int64_t)page * p.k_page * TT::ELEM, ok ? st.k_page_bytes : 0u);
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc((const uint8_t*)p.v + (int64_t)page * p.v_page * TT::ELEM, ok ? st.v_page_bytes : 0u);
  const int ks = slot0 * (int)p.k_slot * TT::ELEM;
  const int vs = slot0 * (int)p.v_slot * TT::ELEM;
  // fp8 K: each load takes half of 16 rows' 128-byte lines and the next load
  // the other half, so these loads keep the default policy (the lines stay
  // cached for their second half); measured 193 -> 189 us on the fp8
  // window/sinks workload, while non-temporal loads stay faster for the
  // 16-bit caches' full-line K loads
  constexpr int kKPolicy = KT == kFP8 ? 0 : kStreamPolicy;
#pragma unroll
  for (int i = 0; i < TT::KLOADS; ++i) buf_load<4, kKPolicy>(rk, st.k_lane + 64 * i, ks, T.k[i]);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    buf_load<TT::VW>(rv, st.v_lane, vs + kk * (int)p.v_slot * TT::ELEM, T.v[kk]);
}

// Online-softmax state and accumulator of one wave (row n = lane % 16).
template <int D>
struct Acc {
  float m, l;
  f32x4 o[D / 16];
};

template <int QT, int KT, int D>
__device__ __forceinline__ void compute_tile(const Params& p, const SeqGeom& sg, const RowVis& vis,
                                             int lo_last, int mask_from, const uint4* qb, int g,
                                             int t, Tile<KT, D>& T, Acc<D>& A) {
  using TT = Tile<KT, D>;
  constexpr int KSTEPS = TT::KSTEPS, DT = TT::DT;
  const int tok0 = t << 4;
  const bool edge = tok0 < lo_last || tok0 + 16 > mask_from;
  if (edge) {
    // tokens no row can see may hold anything (NaN): clear their V so a zero
    // weight cannot turn into NaN inside the P.V product
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int tk = tok0 + 4 * g + kk;
      const bool keep = (tk >= sg.lo) & (tk < sg.L);
#pragma unroll
      for (int w = 0; w < TT::VW; ++w) T.v[kk][w] = keep ? T.v[kk][w] : 0u;
    }
  }
  // ---- S^T = K . Q^T
  f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    uint4 a;
    if constexpr (KT == kFP8) {
      const uint32_t* w = T.k[s >> 1];
      const uint2 lo = fp8x4_to_16<QT>((s & 1) ? w[2] : w[0]);
      const uint2 hi = fp8x4_to_16<QT>((s & 1) ? w[3] : w[1]);
      a = make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
      a = make_uint4(T.k[s][0], T.k[s][1], T.k[s][2], T.k[s][3]);
    }
    s4 = mfma_k32<QT>(a, qb[s], s4);
  }
  // ---- online softmax over this tile (row n, tokens 4g+i)
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float xi = s4[i] * p.qk_scale_log2;
    x[i] = (!edge || vis(tok0 + 4 * g + i, sg.L)) ? xi : kNegInf;
  }
  float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  tmax = max_across_rows(tmax);
  // the reference A.m moves only when the tile max passes it by kSlack
  const bool bump = tmax > A.m + kSlack;
  const float m_new = bump ? tmax : A.m;
  const float m_ref = m_new == kNegInf ? 0.f : m_new;
  // raw v_exp_f32: every argument is <= kSlack (or -inf), and weights below
  // the fp32 normal range may flush to zero without changing the result
  const float alpha = bump ? __builtin_amdgcn_exp2f(A.m - m_ref) : 1.f;
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(x[i] - m_ref);
  // the sum takes the rounded probabilities that P . V uses, so the output
  // is an exact weighted mean of the V rows
  const uint2 pb = make_uint2(pack2<QT>(pr[0], pr[1]), pack2<QT>(pr[2], pr[3]));
  const float2 r0 = unpack2<QT>(pb.x), r1 = unpack2<QT>(pb.y);
  A.l = A.l * alpha + ((r0.x + r0.y) + (r1.x + r1.y));
  A.m = m_new;
  // the reference rarely moves after the first tiles: rescale only then
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
    for (int j = 0; j < DT; ++j) A.o[j] *= alpha;
  }
  // ---- O^T += V^T . P^T
  // operand of dim j: element j of the lane's V chunk for its four tokens
  if constexpr (KT == kFP8) {
    // dims j and j + 1 (bytes b, b + 1 of a word) of two tokens: one byte
    // permute per token pair puts [t0 b, t1 b, t0 b+1, t1 b+1] in a word,
    // whose low and high byte pairs convert (exactly) to the (t0, t1)
    // operand halves of the two dims
#pragma unroll
    for (int j = 0; j < DT; j += 2) {
      const int wi = j >> 2, b = j & 3;
      const uint32_t sel = (uint32_t)b | ((uint32_t)(b + 4) << 8) | ((uint32_t)(b + 1) << 16) |
                           ((uint32_t)(b + 5) << 24);
      const uint2 c01 = fp8x4_to_16<QT>(__builtin_amdgcn_perm(T.v[1][wi], T.v[0][wi], sel));
      const uint2 c23 = fp8x4_to_16<QT>(__builtin_amdgcn_perm(T.v[3][wi], T.v[2][wi], sel));
      A.o[j] = mfma_k16<QT>(make_uint2(c01.x, c23.x), pb, A.o[j]);
      A.o[j + 1] = mfma_k16<QT>(make_uint2(c01.y, c23.y), pb, A.o[j + 1]);
    }
  } else {
    // element j of tokens 0, 1 (2, 3) into one word with one byte permute:
    // the low (j even) or high (j odd) halves of the two tokens' words
#pragma unroll
    for (int j = 0; j < DT; ++j) {
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t w01 = __builtin_amdgcn_perm(T.v[1][j >> 1], T.v[0][j >> 1], sel);
      const uint32_t w23 = __builtin_amdgcn_perm(T.v[3][j >> 1], T.v[2][j >> 1], sel);
      A.o[j] = mfma_k16<QT>(make_uint2(w01, w23), pb, A.o[j]);
    }
  }
}

// Everything one wave needs to stream a run of tiles of one (sequence, KV
// head) unit and to finish it.
template <int KT, int D>
struct Unit {
  static constexpr int KSTEPS = D / 32;
  SeqGeom sg;
  RowVis vis;
  int b, kvh, lo_last, mask_from;
  bool row_ok;
  uint4 qb[KSTEPS];
};

template <int KT, int D>
__device__ __forceinline__ void setup_unit(const Params& p, int b, int kvh, Unit<KT, D>& U) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  U.b = b;
  U.kvh = kvh;
  U.sg = seq_geom(p, b);
  // Q^T operand of row n (zero rows pad the group to 16)
  U.row_ok = n < p.R;
  const uint16_t* qrow = (const uint16_t*)p.q + q_row_offset(p, b, kvh, U.row_ok ? n : 0) * p.Dqk;
#pragma unroll
  for (int s = 0; s < Unit<KT, D>::KSTEPS; ++s)
    U.qb[s] = U.row_ok ? *(const uint4*)(qrow + qk_chunk<KT>(s, g) * 8) : make_uint4(0, 0, 0, 0);
  U.vis = row_vis(p, b, U.sg.L, U.row_ok ? n : 0);
  // tiles wholly inside [lo_last_row, mask_from) need no per-element test
  U.lo_last = p.window > 0 ? U.sg.L - p.window : INT32_MIN;
  U.mask_from = (p.Tq > 1 && p.mask != nullptr) ? U.sg.L - p.Tq : U.sg.L;
}

// Stream the sequence tiles [tile_from, tile_to) of the unit into A.  Runs of
// at most 64 pages share one vector load of their page ids (one per lane);
// each run goes through the NS-stage pipeline.  With PRE, page0_ids holds
// the unit's page ids from page 0 on (lane l: page l, loaded early by the
// caller) and serves a run that starts at page 0.
template <int QT, int KT, int D, bool PRE = false>
__device__ __forceinline__ void stream_tiles(const Params& p, const Unit<KT, D>& U, int tile_from,
                                             int tile_to, Acc<D>& A, int page0_ids = -1) {
  using TT = Tile<KT, D>;
  constexpr int NS = TT::STAGES, DT = TT::DT;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int tiles_per_page = p.ps >> 4;
  Stream st;
  st.k_lane = (int)((n * p.k_slot + U.kvh * p.k_head) * TT::ELEM) + 16 * g;
  st.v_lane = (int)((4 * g * p.v_slot + U.kvh * p.v_head + (int64_t)DT * n) * TT::ELEM);
  st.k_page_bytes = (uint32_t)(p.k_page * TT::ELEM);
  st.v_page_bytes = (uint32_t)(p.v_page * TT::ELEM);
  for (int run = tile_from; run < tile_to;) {
    st.pg_begin = run / tiles_per_page;
    const int run_end = min(tile_to, (st.pg_begin + 64) * tiles_per_page);
    const int pg_last = (run_end - 1) / tiles_per_page;
    st.tile_end = run_end;
    if (PRE && st.pg_begin == 0)
      st.my_page = lane <= pg_last ? page0_ids : -1;
    else
      st.my_page = lane <= pg_last - st.pg_begin
                       ? p.page_table[(int64_t)U.b * p.pps + st.pg_begin + lane] : -1;
    TT buf[NS];
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) {
      load_tile<KT, D>(p, st, run + k, buf[k]);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int t = run; t < run_end; t += NS) {
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        load_tile<KT, D>(p, st, t + k + NS - 1, buf[(k + NS - 1) % NS]);
        if (k == 0 || t + k < run_end)
          compute_tile<QT, KT, D>(p, U.sg, U.vis, U.lo_last, U.mask_from, U.qb, g, t + k, buf[k], A);
      }
    }
    run = run_end;
  }
}

// Finish a unit: the normalised output when this wave saw all of it
// (complete), else the partial (m, l, o) in workspace row `prow`.
template <int QT, int KT, int D>
__device__ __forceinline__ void finish_unit(const Params& p, const Unit<KT, D>& U, Acc<D>& A,
                                            bool complete, int64_t prow) {
  constexpr int DT = D / 16;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const float l = sum_across_rows(A.l);
  if (!U.row_ok) return;
  // lane (n, g) holds dims DT*(4g+i) + j of row n
  if (complete) {
    float num = 1.f, den = l;
    if (p.sinks != nullptr) {
      const float sk = p.sinks[U.kvh * p.G + n % p.G] * kLog2e;
      const float Mf = fmaxf(A.m, sk);
      num = A.m == kNegInf ? 0.f : exp2f(A.m - Mf);
      den = l * num + exp2f(sk - Mf);
    }
    const float inv = den > 0.f ? p.out_scale * num / den : 0.f;
    const int64_t ob = q_row_offset(p, U.b, U.kvh, n) * p.Dv;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < DT; j += 4)
        store_out4<QT>(p, ob + DT * (4 * g + i) + j, A.o[j][i] * inv, A.o[j + 1][i] * inv,
                       A.o[j + 2][i] * inv, A.o[j + 3][i] * inv);
  } else {
    float* o = p.ws_o + prow * p.Dv;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < DT; j += 4)
        *(float4*)(o + DT * (4 * g + i) + j) =
            make_float4(A.o[j][i], A.o[j + 1][i], A.o[j + 2][i], A.o[j + 3][i]);
    if (g == 0) p.ws_ml[prow] = make_float2(A.m, l);
  }
}

// ---- single-launch merge of cut stream-K units
//
// The waves that share a cut unit each leave their partial (m, l, o) in the
// workspace with device-scope stores, wait until those stores have
// completed, and count on the unit's counter; the wave that brings the count
// to the number of pieces merges all of them.  The stores and the merging
// wave's loads are device-scope accesses (sc1: coherent across the XCDs'
// L2 caches, as the compiler lowers agent-scope relaxed atomics), so no
// cache write-back or invalidate is needed.  This is the role the xqa page
// gives its `semaphores` buffer.
//
// Counter word of a unit: (call generation << 32) | pieces counted.  A word
// from another call (another generation, or bytes another plan left there)
// counts as zero; the merging wave resets the count, so replays of a captured
// call with the same generation start from zero too.

// Device-scope (sc1) 8-byte store and load of two floats.
__device__ __forceinline__ void st_dev(float* p, float a, float b) {
  __hip_atomic_store((unsigned long long*)p, __builtin_bit_cast(unsigned long long, make_float2(a, b)),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_dev(const float* p) {
  return __builtin_bit_cast(float2, __hip_atomic_load((unsigned long long*)p, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT));
}

// Write this wave's partial of its rows to workspace slot `slot` with
// device-scope stores (the wave waits for them before it counts the piece).
template <int D>
__device__ __forceinline__ void store_partial_dev(const Params& p, bool row_ok, const Acc<D>& A, float l,
                                                  int64_t prow) {
  constexpr int DT = D / 16;
  const int g = (threadIdx.x & 63) >> 4;
  if (row_ok) {
    float* o = p.ws_o + prow * p.Dv;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < DT; j += 2) st_dev(o + DT * (4 * g + i) + j, A.o[j][i], A.o[j + 1][i]);
    if (g == 0) st_dev((float*)(p.ws_ml + prow), A.m, l);
  }
}

// A cut piece whose count (and possibly the merge of its unit) waits until
// the wave has streamed the rest of its share.
struct Pending {
  int b, kvh, w0, w1;
  int64_t slot0;
};

// Count this piece on the unit's counter; true (on every lane) for the wave
// that counts the last of `pieces`.  The compare-and-swap loop makes progress
// whenever any of the unit's waves succeeds; its bound only guards against a
// counter word that something else keeps changing.
__device__ __forceinline__ bool count_piece(const Params& p, int unit, int pieces) {
  int last = 0;
  if ((threadIdx.x & 63) == 0) {
    unsigned long long* c = p.ws_cnt + unit;
    const unsigned long long gen = (unsigned long long)p.gen << 32;
    // first try: this call's generation with nothing counted yet (right for
    // the first wave to arrive); a failed swap returns the word to retry with
    unsigned long long cur = gen;
    for (int it = 0; it < (1 << 16); ++it) {
      const unsigned long long next = (cur & ~0xffffffffull) == gen ? cur + 1 : gen | 1ull;
      if (__hip_atomic_compare_exchange_strong(c, &cur, next, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)) {
        last = (int)(next & 0xffffffffull) == pieces;
        break;
      }
    }
  }
  last = __builtin_amdgcn_readfirstlane(last);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return last != 0;
}

// Merge the unit's pieces into the output, reading every slot (this wave's
// own too) with device-scope loads in slot order -- so the sums, and the
// output bits, do not depend on which wave happened to finish last -- then
// reset the unit's count.  Slots: `slot0` for the first wave w0 of the unit,
// then 2 w for every later wave up to w1.
template <int QT, int D>
__device__ __forceinline__ void merge_unit(const Params& p, const Pending& u) {
  constexpr int DT = D / 16;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const bool row_ok = n < p.R;
  const int64_t slot0 = u.slot0;
  const int w0 = u.w0, w1 = u.w1;
  float M = kNegInf, den = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int j = 0; j < DT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // slots in groups of kGroup: the group's loads are all issued before any is
  // used, so a group costs one memory round trip
  constexpr int kGroup = D >= 256 ? 1 : 256 / D;
  for (int wb = w0; wb <= w1 && row_ok; wb += kGroup) {
    float2 ml[kGroup];
    f32x4 os[kGroup][DT];
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      const int w = min(wb + k, w1);
      const int64_t prow = (w == w0 ? slot0 : 2 * (int64_t)w) * p.R + n;
      ml[k] = ld_dev((const float*)(p.ws_ml + prow));
      const float* o = p.ws_o + prow * p.Dv;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < DT; j += 2) {
          const float2 v = ld_dev(o + DT * (4 * g + i) + j);
          os[k][j][i] = v.x;
          os[k][j + 1][i] = v.y;
        }
    }
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      if (wb + k > w1) break;
      const float Mn = fmaxf(M, ml[k].x);
      const float a1 = M == kNegInf ? 0.f : exp2f(M - Mn);
      const float a2 = ml[k].x == kNegInf ? 0.f : exp2f(ml[k].x - Mn);
      den = den * a1 + ml[k].y * a2;
#pragma unroll
      for (int j = 0; j < DT; ++j) acc[j] = acc[j] * a1 + os[k][j] * a2;
      M = Mn;
    }
  }
  if (row_ok) {
    float num = 1.f;
    if (p.sinks != nullptr) {
      const float sk = p.sinks[u.kvh * p.G + n % p.G] * kLog2e;
      const float Mf = fmaxf(M, sk);
      num = M == kNegInf ? 0.f : exp2f(M - Mf);
      den = den * num + exp2f(sk - Mf);
    }
    const float inv = den > 0.f ? p.out_scale * num / den : 0.f;
    const int64_t ob = q_row_offset(p, u.b, u.kvh, n) * p.Dv;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < DT; j += 4)
        store_out4<QT>(p, ob + DT * (4 * g + i) + j, acc[j][i] * inv, acc[j + 1][i] * inv,
                       acc[j + 2][i] * inv, acc[j + 3][i] * inv);
  }
  if (lane == 0)
    __hip_atomic_store(p.ws_cnt + (u.b * p.Hkv + u.kvh), (unsigned long long)p.gen << 32,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Zero the outputs of one (sequence, KV head) unit's rows.
__device__ __forceinline__ void zero_unit(const Params& p, int b, int kvh) {
  const int lane = threadIdx.x & 63;
  for (int r = 0; r < p.R; ++r) {
    const int64_t ob = q_row_offset(p, b, kvh, r) * p.Dv;
    for (int d = 4 * lane; d < p.Dv; d += 256) store_out4<kBF16>(p, ob + d, 0.f, 0.f, 0.f, 0.f);
  }
}

// Zero the outputs of the sequences with no visible token (they have no
// tiles, so no wave meets them): wave w takes sequences w, w + W, ...
template <int SC>
__device__ __forceinline__ void zero_empty_units(const Params& p, const SkSchedC<SC>& S, int w, int W) {
  const int lane = threadIdx.x & 63;
  for (int b = w; b < p.B; b += W) {
    int pre, n;
    sk_seq_of(S, b, &pre, &n);
    if (n != 0) continue;
    for (int kvh = 0; kvh < p.Hkv; ++kvh)
      for (int r = 0; r < p.R; ++r) {
        const int64_t ob = q_row_offset(p, b, kvh, r) * p.Dv;
        for (int d = 4 * lane; d < p.Dv; d += 256) store_out4<kBF16>(p, ob + d, 0.f, 0.f, 0.f, 0.f);
      }
  }
}

template <int D>
__device__ __forceinline__ void reset(Acc<D>& A) {
  A.m = kNegInf;
  A.l = 0.f;
#pragma unroll
  for (int j = 0; j < D / 16; ++j) A.o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

}  // namespace

// Grid schedule: one wave per (split, KV head, sequence); a split is
// `split_pages` pages of the sequence's visible span.
template <int QT, int KT, int D>
__global__ __launch_bounds__(64) void split_mfma16_kernel(Params p) {
  resolve_scales(p);
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const SeqGeom sg = seq_geom(p, b);
  if (split >= sg.nsplits) return;
  const int pg_begin = sg.p0 + split * p.split_pages;
  const int pg_end = min(pg_begin + p.split_pages, sg.p0 + sg.npages);
  const int tile_begin = max(pg_begin * p.ps, sg.lo) >> 4;
  const int tile_end = (min(pg_end * p.ps, sg.L) + 15) >> 4;
  Unit<KT, D> U;
  setup_unit<KT, D>(p, b, kvh, U);
  Acc<D> A;
  reset<D>(A);
  stream_tiles<QT, KT, D>(p, U, tile_begin, tile_end, A);
  const int64_t prow = (((int64_t)b * p.Hkv + kvh) * p.max_splits + split) * p.R + (threadIdx.x & 15);
  finish_unit<QT, KT, D>(p, U, A, sg.nsplits == 1, prow);
}

// Stream-K schedule: wave w of W takes an equal share of the tile stream of
// all units; units wholly inside its share are finished here, the first and
// the last (when cut) leave partials in workspace slots 2w and 2w+1.  With
// p.fused the wave that completes a cut unit merges it (see merge_unit);
// otherwise the combine kernel does.
// FUSED selects the single-launch merge at compile time, so the two-launch
// kernel carries none of its code or registers; SC is the schedule's chunk
// count (4: up to 256 sequences, 16: up to 1024).
template <int QT, int KT, int D, bool FUSED, int SC>
// (two waves per SIMD: the register budget keeps the accumulators in
// architected VGPRs instead of moving them through AGPRs every tile)
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void split_mfma16_sk_kernel(Params p) {
  resolve_scales(p);
  // workgroup (head group hg, position j) of sk_hb waves: wave i takes share
  // j of KV head hg * sk_hb + i's part of the tile stream (W / Hkv waves per
  // head), i.e. the same tokens as its neighbours, of another KV head
  int w = blockIdx.x;
  if (p.sk_hb > 1) {
    const int W1 = p.sk_waves / p.Hkv, hg = blockIdx.x / W1, j = blockIdx.x - hg * W1;
    w = (hg * p.sk_hb + (int)(threadIdx.x >> 6)) * W1 + j;
  }
  // the wave index is uniform across the wave; saying so keeps the schedule,
  // the tile indices and the buffer resources built from them in scalar
  // registers (a value derived from threadIdx counts as per-lane, and a
  // per-lane buffer resource costs a loop around every load)
  w = __builtin_amdgcn_readfirstlane(w);
  if (p.sk_units == 2) {
    // short units (at most 17 tiles): wave w = kvh * B + b streams all of
    // unit (b, kvh) and needs no schedule, so its first memory round trip
    // fetches the length, the query rows and the first page ids together
    if (w >= p.sk_waves) return;
    const int kvh = w / p.B, b = w - kvh * p.B, lane = threadIdx.x & 63;
    const int page0_ids = lane < p.pps ? p.page_table[(int64_t)b * p.pps + lane] : -1;
    Unit<KT, D> U;
    setup_unit<KT, D>(p, b, kvh, U);
    int tile0;
    const int n = seq_tiles(p, b, &tile0);
    if (n == 0) {
      zero_unit(p, b, kvh);
      return;
    }
    Acc<D> A;
    reset<D>(A);
    stream_tiles<QT, KT, D, true>(p, U, tile0, tile0 + n, A, page0_ids);
    finish_unit<QT, KT, D>(p, U, A, true, 0);
    return;
  }
  const SkSchedC<SC> S = sk_schedule<SC>(p);
  const int W = sk_waves_eff(S.T, p.sk_waves);
  int64_t x0, x1;
  if (p.sk_units == 1 && sk_units_even(p, S)) {
    // one wave per unit when the units are even: wave w = kvh * B + b
    // streams all of unit (b, kvh) (the KV-head-major unit order); an empty
    // unit gets zeros
    if (w >= p.sk_waves) return;
    const int kvh = w / p.B, b = w - kvh * p.B;
    int pre, n;
    sk_seq_of(S, b, &pre, &n);
    if (n == 0) {
      zero_unit(p, b, kvh);
      return;
    }
    x0 = sk_unit_start(S, kvh, pre);
    x1 = x0 + n;
  } else {
    if (w >= W) return;
    x0 = sk_wave_start(S.T, w, W);
    x1 = sk_wave_start(S.T, w + 1, W);
  }
  if (FUSED) zero_empty_units(p, S, w, W);
  Unit<KT, D> U;
  Acc<D> A;
  // cut pieces (at most the share's first and last) counted after the loop,
  // when their partial stores have long completed
  Pending pend[2];
  int npend = 0;
  for (int64_t x = x0; x < x1;) {
    const SkUnit u = sk_locate(p, S, x);
    const int64_t seg_end = min(x1, u.start + u.ntiles);
    setup_unit<KT, D>(p, u.b, u.kvh, U);
    reset<D>(A);
    int tile0;
    seq_tiles(p, u.b, &tile0);
    stream_tiles<QT, KT, D>(p, U, tile0 + (int)(x - u.start), tile0 + (int)(seg_end - u.start), A);
    const bool complete = x == u.start && seg_end == u.start + u.ntiles;
    const int slot = 2 * w + (x == x0 ? 0 : 1);
    if (complete || !FUSED) {
      finish_unit<QT, KT, D>(p, U, A, complete, (int64_t)slot * p.R + (threadIdx.x & 15));
    } else {
      const float l = sum_across_rows(A.l);
      store_partial_dev<D>(p, U.row_ok, A, l, (int64_t)slot * p.R + (threadIdx.x & 15));
      Pending& pd = pend[npend == 0 ? 0 : 1];
      pd.b = u.b;
      pd.kvh = u.kvh;
      pd.w0 = sk_wave_of(S.T, u.start, W);
      pd.w1 = sk_wave_of(S.T, u.start + u.ntiles - 1, W);
      pd.slot0 = sk_wave_start(S.T, pd.w0, W) == u.start ? 2 * (int64_t)pd.w0 : 2 * (int64_t)pd.w0 + 1;
      ++npend;
    }
    x = seg_end;
  }
  if (FUSED && npend > 0) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the partial stores have completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    for (int k = 0; k < npend; ++k) {
      const Pending& pd = pend[k];
      if (count_piece(p, pd.b * p.Hkv + pd.kvh, pd.w1 - pd.w0 + 1)) merge_unit<QT, D>(p, pd);
    }
  }
}

template <int QT, int KT, int D>
hipError_t launch_split_mfma16(const Params& p, hipStream_t stream) {
  if (p.sk_waves > 0) {
    const dim3 grid(p.sk_waves / p.sk_hb), block(64 * p.sk_hb);
    if (p.B <= kSkMaxBatch) {
      if (p.fused)
        hipLaunchKernelGGL((split_mfma16_sk_kernel<QT, KT, D, true, 4>), grid, block, 0, stream, p);
      else
        hipLaunchKernelGGL((split_mfma16_sk_kernel<QT, KT, D, false, 4>), grid, block, 0, stream, p);
    } else if constexpr (D <= 128) {
      // the wide schedule's registers fit beside head dims up to 128 only
      if (p.fused)
        hipLaunchKernelGGL((split_mfma16_sk_kernel<QT, KT, D, true, 16>), grid, block, 0, stream, p);
      else
        hipLaunchKernelGGL((split_mfma16_sk_kernel<QT, KT, D, false, 16>), grid, block, 0, stream, p);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    dim3 grid(p.max_splits, p.Hkv, p.B);
    hipLaunchKernelGGL((split_mfma16_kernel<QT, KT, D>), grid, dim3(64), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_split_mfma16(int q_dtype, int kv_dtype, int D, const Params& p, hipStream_t s) {
  if (p.sk_waves == 0 && p.split_pages > 64) return hipErrorInvalidValue;
  if (p.sk_waves > 0 && p.B > kSkMaxBatchWide) return hipErrorInvalidValue;
  if (p.sk_waves > 0 && (p.sk_hb < 1 || p.sk_hb > 8 || p.sk_waves % p.sk_hb ||
                         (p.sk_hb > 1 && (p.sk_waves % p.Hkv || p.Hkv % p.sk_hb))))
    return hipErrorInvalidValue;
#define PKV_CASE(QT, KT, DD) \
  if (q_dtype == QT && kv_dtype == KT && D == DD) return launch_split_mfma16<QT, KT, DD>(p, s);
  PKV_CASE(kBF16, kBF16, 128)
  PKV_CASE(kF16, kF16, 128)
  PKV_CASE(kBF16, kFP8, 128)
  PKV_CASE(kF16, kFP8, 128)
  PKV_CASE(kBF16, kBF16, 64)
  PKV_CASE(kF16, kF16, 64)
  PKV_CASE(kBF16, kFP8, 64)
  PKV_CASE(kF16, kFP8, 64)
  PKV_CASE(kBF16, kBF16, 256)
  PKV_CASE(kF16, kF16, 256)
  PKV_CASE(kBF16, kFP8, 256)
  PKV_CASE(kF16, kFP8, 256)
#undef PKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
