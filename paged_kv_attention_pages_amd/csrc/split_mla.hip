// split_mla.hip -- split-KV decode over a latent (MLA) cache on the gfx950
// matrix cores: one KV head, up to 64 query rows, 576-wide cached rows of
// which the first 512 entries are V.
//
// vLLM `models/kimi_k3/nvidia/mla` page, MultiHeadLatentAttention: the decode
// branch of `_attention` runs multi-query attention of the absorbed queries
// [q_nope . W_UK_T | q_pe] over the latent cache rows [kv_c_normed | k_pe]
// (`forward_mqa`), and the kv_lora_rank-wide result is what `_v_up_proj`
// projects back -- so V is the leading kv_lora_rank entries of each K row.
//
// A workgroup of eight waves (two per SIMD) processes 32-token tiles.  The
// tile (32 cached rows, 36 KB) is loaded as whole contiguous rows -- wave w
// fetches rows 4w .. 4w + 3 -- and written once into a three-deep LDS ring;
// everything else reads it from there.  Wave w owns query rows
// 16 (w mod 4) .. + 15 and half of the dimensions, h = w / 4:
//   1. partial scores over dims [288 h, 288 h + 288) (nine 16x16x32 MFMA per
//      16-token block; half 1 holds the rope dims):
//        S^T_h (32 tokens x 16 rows) = K[:, 288 h ..] . Q[rows, 288 h ..]^T
//   2. the two halves swap their partials through LDS (2 KB per wave) and
//      both run the same online softmax of their 16 rows in registers;
//   3. O^T (256 dims [256 h, 256 h + 256) x 16 rows) += V^T . P^T, V^T read
//      from the LDS tile by column (token along the MFMA K dimension).
// One barrier per tile.  LDS writes per tile are the 36 KB tile and 16 KB of
// partial scores -- the LDS writes at about a third of its read rate on
// gfx950, so reads carry the operand traffic.  The 64 accumulator
// registers per lane keep the working set in the 256 VGPRs of a
// two-waves-per-SIMD budget.
// This kernel serves the grid schedule, one (sequence, split) per workgroup
// (batches above the stream-K limit, or a forced split size); the stream-K
// schedule runs the wave-specialised kernel of split_mla_ws.hip.
#include "pkv_device.h"
#include "kernels.h"

namespace pkv {

namespace {
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

constexpr int kDqk = 576, kDv = 512;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kQkHalf = kDqk / 2;             // 288 score dims per half
constexpr int kQkSteps = kQkHalf / 32;        // 9 MFMA K steps
constexpr int kPvHalf = kDv / 2;              // 256 output dims per half
constexpr int kTileTok = 32;                  // tokens per tile
constexpr int kTileShift = 5;
// LDS tile: two halves of 16 rows; a half holds the first 1024 bytes of its
// rows (dims 0 .. 511) at 1024 bytes per row, then the last 128 bytes (the
// rope dims) at 128 bytes per row.  The 16-byte chunks of a row are
// XOR-swizzled (swz_lo / swz_hi) so that the K reads (sixteen rows, one
// chunk), the transposed V reads (eight rows, 32 bytes each) and the row
// stores each hit distinct banks.
constexpr int kLoBytes = 1024, kHiBytes = 128;
constexpr int kHiOff = 16 * kLoBytes;         // rope part of a half
constexpr int kHalfBytes = 16 * (kLoBytes + kHiBytes);
constexpr int kTileBytes = 2 * kHalfBytes;
constexpr int kRing = 3;                      // LDS tiles in flight
constexpr int kLoadRing = 3;                  // register tiles in flight per wave
static_assert(kLoadRing == kRing, "the step loop indexes the LDS ring by its unroll index");
static_assert(kQkHalf % 32 == 0 && kPvHalf % 64 == 0, "latent row split");

struct Smem {
  uint8_t tile[kRing][kTileBytes];           // 32 rows of the cache, layout above
  f32x4 sp[2][4][2][2][64];                  // partial scores [parity][row block][half][token block]
};

// Query slice of this wave: B operands of S^T = K . Q^T.
struct QRegs {
  uint4 k[kQkSteps];   // row 16 rb + n, dims 288 h + 32 s + 8 g .. + 8
};

// This wave's share of one tile on its way to LDS: rows 4w + (lane / 16),
// bytes 16 (lane mod 16) + 256 j (j < 4) and 1024 + 8 (lane mod 16) of a
// 16-bit row; of an fp8 row (576 bytes), bytes 16 (lane mod 16) + 256 j
// (j < 2) in a[0..1] and 512 + 4 (lane mod 16) in b.x.
struct LTile {
  uint4 a[4];
  uint2 b;
};

// The token range [tok_lo, tok_hi) of one (sequence, KV head) that one
// workgroup processes, and what every wave needs to process it.
struct Piece {
  int b, kvh, L;
  int tok_lo, tok_hi;
  int lo_last;     // tokens >= lo_last pass every row's window
  int mask_from;   // tokens >= mask_from are subject to the draft mask
  int lane_row;    // byte offset of this lane's loads inside its tile block
  uint32_t page_bytes;
  RowVis vis;      // visibility of this lane's row (16 rb + n)
};

struct Acc {
  f32x4 o[16];     // [m][i]: dims 256 h + 16 m + 4 g + i, row 16 rb + n
  float m;         // running reference max (log2 units)
  f32x4 lsum;      // P . ones: every element holds the row sum of the rounded probabilities
};

// Per-lane LDS byte offsets inside a tile slot, fixed for the kernel.
struct LdsOff {
  int k[9];   // K fragment of step s, half 0 (half 1: + kHalfBytes)
  int v[8];   // transposed V read of MFMA m (k = m mod 8; + 256 (m / 8)), half 0
};

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Workgroup barrier that orders LDS only: the release fence waits for this
// wave's LDS operations, not for its outstanding global loads, so the tile
// prefetch stays in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Chunk swizzles of row r (0 .. 15) of a half tile: chunk c of the low part
// sits at c ^ swz_lo(r) (within its aligned group of 16), chunk c of the rope
// part at c ^ swz_hi(r).  swz_lo was chosen by measuring the K-read and
// transposed-V-read rates of candidate tables on gfx950: with it both run at
// the full rate of their instruction (about 205 and 175 bytes per clock per
// CU), where a plain r or a bit-rotation of r slows one of them by 30-40%.
__device__ __forceinline__ int swz_lo(int r) { return (r ^ (r << 1)) & 15; }
__device__ __forceinline__ int swz_hi(int r) { return (r >> 1) & 7; }
// byte offset of 16-byte chunk c of a row's low part, chunk-swizzled
__device__ __forceinline__ int lo_chunk(int r, int c) { return r * kLoBytes + 16 * ((c & ~15) | ((c & 15) ^ swz_lo(r))); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed LDS read (ds_read_b64_tr_b16).  In each group of 16 lanes, lane
// a + 4 j supplies the address of four 16-bit elements; lane 4 a + e
// receives element e of lanes a, a + 4, a + 8, a + 12, in that order.
__device__ __forceinline__ uint2 lds_read_tr16(const uint8_t* addr) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(addr));
  return __builtin_bit_cast(uint2, v);
}

// Score step s reads chunk c = 36 h + 4 s + g of row n of each half: with
// s = j + 4 i that is chunk (36 h + g + 4 j) + 16 i of the low part (the
// swizzle leaves the + 16 i alone), except steps 7 and 8 of half 1, which
// are the rope chunks g and 4 + g.  V read m of lane (n, g) covers row
// 4 g + n / 4 of each half, chunk 32 h + 2 m + (n / 2 mod 2), byte 8 (n mod 2).
__device__ __forceinline__ LdsOff lds_offsets() {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4, h = wave_id() >> 2;
  LdsOff o;
  const int c0 = 36 * h + g;
#pragma unroll
  for (int j = 0; j < 4; ++j) o.k[j] = lo_chunk(n, c0 + 4 * j);
#pragma unroll
  for (int s = 4; s < 7; ++s) o.k[s] = o.k[s & 3] + 256 * (s >> 2);
  const int hi = kHiOff + n * kHiBytes;
  o.k[7] = h ? hi + 16 * (g ^ swz_hi(n)) : o.k[3] + 256;
  o.k[8] = h ? hi + 16 * ((4 + g) ^ swz_hi(n)) : o.k[0] + 512;
  const int r = 4 * g + (n >> 2), bsel = (n >> 1) & 1;
#pragma unroll
  for (int k = 0; k < 8; ++k) o.v[k] = lo_chunk(r, 32 * h + 2 * k + bsel) + 8 * (n & 1);
  return o;
}

template <bool KV8>
__device__ __forceinline__ void setup_piece(const Params& p, int b, int kvh, int tok_lo, int tok_hi,
                                            Piece& P) {
  constexpr int E = KV8 ? 1 : 2;  // bytes per cache element
  const int lane = threadIdx.x & 63, n = lane & 15, w = wave_id();
  const SeqGeom sg = seq_geom(p, b);
  P.b = b;
  P.kvh = kvh;
  P.L = sg.L;
  P.tok_lo = tok_lo;
  P.tok_hi = tok_hi;
  P.lo_last = p.window > 0 ? sg.L - p.window : INT32_MIN;
  P.mask_from = (p.Tq > 1 && p.mask != nullptr) ? sg.L - p.Tq : sg.L;
  // this lane's row inside the wave's 16-token block: 4 (w mod 4) + lane / 16
  P.lane_row = (int)(((4 * (w & 3) + (lane >> 4)) * p.k_slot + kvh * p.k_head) * E) + 16 * n;
  P.page_bytes = (uint32_t)(p.k_page * E);
  const int own = 16 * (w & 3) + n;
  P.vis = row_vis(p, b, sg.L, own < p.R ? own : 0);
}

// This wave's slice of its 16 query rows (zeros for rows >= R); an fp8
// query (Q8) is converted exactly to QT.
template <int QT, bool Q8>
__device__ __forceinline__ void load_q(const Params& p, const Piece& P, QRegs& Q) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4, w = wave_id();
  const int row = 16 * (w & 3) + n, h = w >> 2;
  const bool ok = row < p.R;
  const int64_t qoff = q_row_offset(p, P.b, P.kvh, ok ? row : 0) * kDqk;
#pragma unroll
  for (int s = 0; s < kQkSteps; ++s) {
    const int64_t e = qoff + kQkHalf * h + 32 * s + 8 * g;
    if constexpr (Q8) {
      const uint2 raw = ok ? *(const uint2*)((const uint8_t*)p.q + e) : make_uint2(0, 0);
      const uint2 lo = fp8x4_to_16<QT>(raw.x), hi = fp8x4_to_16<QT>(raw.y);
      Q.k[s] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
      Q.k[s] = ok ? *(const uint4*)((const uint16_t*)p.q + e) : make_uint4(0, 0, 0, 0);
    }
  }
}

// Issue this wave's loads of tile t: rows 4w .. 4w + 3 lie in the 16-token
// block w / 4, so one page per wave and tile.  The run's page ids sit one
// per lane in my_page for pages pg_begin ..; a block outside the run or on
// a page id outside the cache reads through an empty resource (zeros, no
// memory access), and rows outside [tok_lo, tok_hi) get an offset past the
// end of the page, which also reads zeros -- so the invisible rows, which
// may hold anything, never reach the arithmetic.
template <bool KV8>
__device__ __forceinline__ void load_tile(const Params& p, const Piece& P, int my_page, int pg_begin,
                                          bool live, int t, LTile& T) {
  constexpr int E = KV8 ? 1 : 2;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int tok16 = t * kTileTok + 16 * (w >> 2);
  const int pg = tok16 >> p.ps_shift;
  const int rel = pg - pg_begin;
  int page = -1;
  if (live && rel >= 0 && rel < 64) page = __builtin_amdgcn_readlane(my_page, rel);
  const bool ok = (unsigned)page < (unsigned)p.num_pages;
  const uint8_t* base = (const uint8_t*)p.k + (ok ? (int64_t)page * p.k_page * E : 0);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, ok ? P.page_bytes : 0u);
  const int soff = (int)((tok16 - (pg << p.ps_shift)) * p.k_slot * E);
  const int tok = tok16 + 4 * (w & 3) + (lane >> 4);
  const bool in = tok >= P.tok_lo && tok < P.tok_hi;
  const int va = in ? P.lane_row : (int)0x80000000u;
  if constexpr (KV8) {
    const int vb = in ? P.lane_row + 512 - 12 * (lane & 15) : (int)0x80000000u;
#pragma unroll
    for (int j = 0; j < 2; ++j) buf_load<4>(rs, va + 256 * j, soff, (uint32_t*)&T.a[j]);
    buf_load<1>(rs, vb, soff, (uint32_t*)&T.b);
  } else {
    const int vb = in ? P.lane_row + 1024 - 8 * (lane & 15) : (int)0x80000000u;
#pragma unroll
    for (int j = 0; j < 4; ++j) buf_load<4>(rs, va + 256 * j, soff, (uint32_t*)&T.a[j]);
    buf_load<2>(rs, vb, soff, (uint32_t*)&T.b);
  }
}

// Write this wave's rows of a tile into LDS ring slot `slot`; fp8 rows are
// converted exactly to QT on the way (the LDS tile is 16-bit either way).
template <int QT, bool KV8>
__device__ __forceinline__ void store_tile(const LTile& T, int slot, Smem& sm) {
  const int lane = threadIdx.x & 63, n = lane & 15, w = wave_id();
  const int r = 4 * (w & 3) + (lane >> 4);   // row in half tile w / 4
  uint8_t* half = sm.tile[slot] + (w >> 2) * kHalfBytes;
  uint8_t* hi = half + kHiOff + r * kHiBytes + 16 * ((n >> 1) ^ swz_hi(r)) + 8 * (n & 1);
  if constexpr (KV8) {
    // fp8 bytes 16 n + 256 j .. + 16 are elements of 16-bit chunks 2 n + 32 j
    // and 2 n + 32 j + 1; rope elements 4 n .. 4 n + 3 fill half a chunk
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint2 e0 = fp8x4_to_16<QT>(T.a[j].x), e1 = fp8x4_to_16<QT>(T.a[j].y);
      const uint2 e2 = fp8x4_to_16<QT>(T.a[j].z), e3 = fp8x4_to_16<QT>(T.a[j].w);
      *(uint4*)(half + lo_chunk(r, 2 * n + 32 * j)) = make_uint4(e0.x, e0.y, e1.x, e1.y);
      *(uint4*)(half + lo_chunk(r, 2 * n + 32 * j + 1)) = make_uint4(e2.x, e2.y, e3.x, e3.y);
    }
    *(uint2*)hi = fp8x4_to_16<QT>(T.b.x);
  } else {
    // chunk n + 16 j lands at 16 j + (n ^ swz_lo(r))
    uint8_t* lo = half + lo_chunk(r, n);
#pragma unroll
    for (int j = 0; j < 4; ++j) *(uint4*)(lo + 256 * j) = T.a[j];
    *(uint2*)hi = T.b;
  }
}

// One tile from LDS ring slot `slot`: partial scores, swap, softmax, P . V.
// `par` selects the partial-score buffer (tile parity).
template <int QT>
__device__ __forceinline__ void score_tile(const Params& p, const Piece& P, const QRegs& Q, const LdsOff& L,
                                           int t, int slot, Smem& sm, f32x4 (&s4)[2]) {
  // ---- 1. partial scores over dims [288 h, 288 h + 288): the 18 K
  // fragments (two 16-token blocks x nine steps) are read kAhead ahead of
  // their MFMA, so LDS latency overlaps the matrix work
  const uint8_t* tl = sm.tile[slot];
  constexpr int kFrags = 2 * kQkSteps, kAhead = 4;
  auto frag = [&](int j) { return *(const uint4*)(tl + (j / kQkSteps) * kHalfBytes + L.k[j % kQkSteps]); };
  uint4 kf[kAhead];
#pragma unroll
  for (int j = 0; j < kAhead; ++j) kf[j] = frag(j);
  s4[0] = s4[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kFrags; ++j) {
    const uint4 cur = kf[j % kAhead];
    if (j + kAhead < kFrags) kf[j % kAhead] = frag(j + kAhead);
    s4[j / kQkSteps] = mfma_k32<QT>(cur, Q.k[j % kQkSteps], s4[j / kQkSteps]);
  }
  // keep the order: kAhead reads, then (MFMA, read) pairs, then the last MFMAs
  __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
  for (int j = 0; j < kFrags - kAhead; ++j) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
}

template <int QT>
__device__ __forceinline__ void finish_tile(const Params& p, const Piece& P, const LdsOff& L, int t, int slot,
                                            int par, const f32x4 (&s4)[2], Smem& sm, Acc& A) {
  const int lane = threadIdx.x & 63, g = lane >> 4, w = wave_id();
  const int rb = w & 3, h = w >> 2;
  const int tok0 = t * kTileTok;
  // ---- 2. the other half's partials (the sum a + b is the same bits on both sides)
  f32x4 sc[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) sc[tb] = s4[tb] + sm.sp[par][rb][h ^ 1][tb][lane];
  // the first V^T operands (step 3) are read now, under the softmax
  const uint8_t* tl = sm.tile[slot];
  auto vread = [&](int m) {
    const int o = L.v[m & 7] + 256 * (m >> 3);
    const uint2 v0 = lds_read_tr16(tl + o), v1 = lds_read_tr16(tl + kHalfBytes + o);
    return make_uint4(v0.x, v0.y, v1.x, v1.y);
  };
  constexpr int kVAhead = 3;
  uint4 vf[kVAhead];
#pragma unroll
  for (int j = 0; j < kVAhead; ++j) vf[j] = vread(j);
  float x[2][4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[tb][i] = sc[tb][i] * p.qk_scale_log2;
  // tiles that hold an invisible token for some row (window, draft mask,
  // the ends of the piece) mask; the others are visible to every row
  if (tok0 < max(P.tok_lo, P.lo_last) || tok0 + kTileTok > min(P.tok_hi, P.mask_from)) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tok0 + 16 * tb + 4 * g + i;
        const bool v = (tok >= P.tok_lo) & (tok < P.tok_hi) & P.vis(tok, P.L);
        x[tb][i] = v ? x[tb][i] : kNegInf;
      }
  }
  float tmax = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                     fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
  tmax = max_across_rows(tmax);
  // the reference A.m moves only when the tile max passes it by kSlack
  const bool bump = tmax > A.m + kSlack;
  const float m_new = bump ? tmax : A.m;
  const float m_ref = m_new == kNegInf ? 0.f : m_new;
  const float alpha = bump ? __builtin_amdgcn_exp2f(A.m - m_ref) : 1.f;
  float pr[2][4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[tb][i] = __builtin_amdgcn_exp2f(x[tb][i] - m_ref);
  // P^T operand: MFMA K index 8 g + c <-> token 4 g + c (c < 4) or
  // 16 + 4 g + c - 4.  The row sum takes the rounded probabilities, so the
  // output is an exact weighted mean of the V rows; it comes from one more
  // MFMA against a tile of ones (all 32 tokens, no cross-lane reduction)
  const uint4 pw = make_uint4(pack2<QT>(pr[0][0], pr[0][1]), pack2<QT>(pr[0][2], pr[0][3]),
                              pack2<QT>(pr[1][0], pr[1][1]), pack2<QT>(pr[1][2], pr[1][3]));
  A.m = m_new;
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
    for (int m = 0; m < 16; ++m) A.o[m] *= alpha;
    A.lsum *= alpha;
  }
  // ---- 3. O^T += V^T . P^T over dims [256 h, 256 h + 256), 16 (MFMA m) at
  // a time.  The V^T operand comes from two transposed reads, one per half
  // tile: lane a + 4 j of group g supplies dims 16 m + 4 a .. + 4 of token
  // 16 hh + 4 g + j, so lane n of group g receives dim 16 m + n of tokens
  // 16 hh + 4 g + (0 .. 3) -- MFMA K index 8 g + 4 hh + j, as in P^T.
  // Reads run kVAhead MFMAs ahead.
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const uint4 cur = vf[m % kVAhead];
    if (m + kVAhead < 16) vf[m % kVAhead] = vread(m + kVAhead);
    A.o[m] = mfma_k32<QT>(cur, pw, A.o[m]);
  }
#pragma unroll
  for (int m = 0; m + kVAhead < 16; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kVAhead, 0);
  const uint32_t one2 = QT == kBF16 ? 0x3f803f80u : 0x3c003c00u;
  A.lsum = mfma_k32<QT>(make_uint4(one2, one2, one2, one2), pw, A.lsum);
}

// A run: tiles [begin, end) whose pages (at most 64, from pg_begin) have
// their ids one per lane in my_page.
struct Run {
  int begin, end, pg_begin, my_page;
};

__device__ __forceinline__ Run open_run(const Params& p, const Piece& P, int run, int t_to) {
  Run r;
  r.begin = run;
  r.pg_begin = (run * kTileTok) / p.ps;
  r.end = min(t_to, ((r.pg_begin + 64) * p.ps) >> kTileShift);
  const int pg_last = (min(r.end * kTileTok, P.tok_hi) - 1) / p.ps;
  const int lane = threadIdx.x & 63;
  r.my_page = lane <= pg_last - r.pg_begin ? p.page_table[(int64_t)P.b * p.pps + r.pg_begin + lane] : -1;
  return r;
}

// Tiles [R.begin, t_to) of a piece, run by run.  Per run: the first two
// tiles go to LDS before the loop; in step t the workgroup scores tile t,
// swaps partials (the one barrier), finishes tile t, writes tile t + 2 into
// the ring slot freed by tile t - 1 and issues the loads of tile
// t + 2 + kLoadRing.  The register ring holds kLoadRing tiles in flight per
// wave; the loop is unrolled by kLoadRing to index it statically.
template <int QT, bool KV8>
__device__ __forceinline__ void stream_piece(const Params& p, const Piece& P, const QRegs& Q, const LdsOff& L, Run R,
                                             int t_to, Smem& sm, Acc& A) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int rb = w & 3, h = w >> 2;
  while (true) {
    const int tb0 = R.begin, te = R.end;
    LTile lr[kLoadRing];
    LTile first[2];
    load_tile<KV8>(p, P, R.my_page, R.pg_begin, tb0 < te, tb0, first[0]);
    load_tile<KV8>(p, P, R.my_page, R.pg_begin, tb0 + 1 < te, tb0 + 1, first[1]);
#pragma unroll
    for (int k = 0; k < kLoadRing; ++k)
      load_tile<KV8>(p, P, R.my_page, R.pg_begin, tb0 + 2 + k < te, tb0 + 2 + k, lr[k]);
    // the ring may still be read by the previous run or piece
    lds_barrier();
    store_tile<QT, KV8>(first[0], 0, sm);
    store_tile<QT, KV8>(first[1], 1, sm);
    lds_barrier();
    for (int t = tb0; t < te; t += kLoadRing) {
#pragma unroll
      for (int k = 0; k < kLoadRing; ++k) {
        const int tt = t + k;
        const bool act = k == 0 || tt < te;
        const int i = tt - tb0;
        const int slot = k, par = i & 1;   // i mod kRing == k: runs start at slot 0
        f32x4 s4[2];
        if (act) {
          score_tile<QT>(p, P, Q, L, tt, slot, sm, s4);
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) sm.sp[par][rb][h][tb][lane] = s4[tb];
          lds_barrier();
          finish_tile<QT>(p, P, L, tt, slot, par, s4, sm, A);
          // tile tt + 2 into the slot tile tt - 1 used (every wave finished
          // tile tt - 1 before it reached this step's barrier); stored after
          // this tile's work, so a late load stalls the wave only once the
          // step's matrix work is done, and still ahead of the next barrier
          store_tile<QT, KV8>(lr[k], (i + 2) % kRing, sm);
        }
        // issued on every step, live or not, so the wait counts before the
        // stores stay exact and kLoadRing tiles remain in flight
        load_tile<KV8>(p, P, R.my_page, R.pg_begin, tt + 2 + kLoadRing < te, tt + 2 + kLoadRing, lr[k]);
      }
    }
    if (te >= t_to) break;
    R = open_run(p, P, te, t_to);
  }
}

__device__ __forceinline__ void reset(Acc& A) {
  A.m = kNegInf;
  A.lsum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < 16; ++m) A.o[m] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Normalised output when this workgroup saw the whole unit, else the
// partial (m, l, o) in workspace rows prow0 + row.
template <int QT>
__device__ __forceinline__ void finish_piece(const Params& p, const Piece& P, Acc& A, bool complete,
                                             int64_t prow0) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4, w = wave_id();
  const int row = 16 * (w & 3) + n, h = w >> 2;
  const float l = A.lsum[0];
  if (row >= p.R) return;
  // lane (n, g) holds dims 256 h + 16 m + 4 g + i of its row
  if (complete) {
    float num = 1.f, den = l;
    if (p.sinks != nullptr) {
      const float sk = p.sinks[P.kvh * p.G + row % p.G] * kLog2e;
      const float Mf = fmaxf(A.m, sk);
      num = A.m == kNegInf ? 0.f : exp2f(A.m - Mf);
      den = l * num + exp2f(sk - Mf);
    }
    const float inv = den > 0.f ? p.out_scale * num / den : 0.f;
    const int64_t ob = q_row_offset(p, P.b, P.kvh, row) * kDv + kPvHalf * h + 4 * g;
#pragma unroll
    for (int m = 0; m < 16; ++m)
      store_out4<QT>(p, ob + 16 * m, A.o[m][0] * inv, A.o[m][1] * inv, A.o[m][2] * inv, A.o[m][3] * inv);
  } else {
    float* o = p.ws_o + (prow0 + row) * kDv + kPvHalf * h + 4 * g;
#pragma unroll
    for (int m = 0; m < 16; ++m)
      *(float4*)(o + 16 * m) = make_float4(A.o[m][0], A.o[m][1], A.o[m][2], A.o[m][3]);
    if (h == 0 && g == 0) p.ws_ml[prow0 + row] = make_float2(A.m, l);
  }
}

}  // namespace

// Grid schedule: one workgroup per (split, KV head, sequence).  QT: the
// operand and output type; KV8: fp8 cache; Q8: fp8 query.
template <int QT, bool KV8, bool Q8>
__global__ __launch_bounds__(kThreads) void split_mla_kernel(Params p) {
  resolve_scales(p);
  __shared__ Smem sm;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const SeqGeom sg = seq_geom(p, b);
  if (split >= sg.nsplits) return;
  const int pg_begin = sg.p0 + split * p.split_pages;
  const int pg_end = min(pg_begin + p.split_pages, sg.p0 + sg.npages);
  const int tok_lo = max(pg_begin * p.ps, sg.lo), tok_hi = min(pg_end * p.ps, sg.L);
  Piece P;
  setup_piece<KV8>(p, b, kvh, tok_lo, tok_hi, P);
  const int t_to = (tok_hi + kTileTok - 1) >> kTileShift;
  const Run R = open_run(p, P, tok_lo >> kTileShift, t_to);
  QRegs Q;
  load_q<QT, Q8>(p, P, Q);
  Acc A;
  reset(A);
  const LdsOff L = lds_offsets();
  stream_piece<QT, KV8>(p, P, Q, L, R, t_to, sm, A);
  finish_piece<QT>(p, P, A, sg.nsplits == 1,
                   (((int64_t)b * p.Hkv + kvh) * p.max_splits + split) * p.R);
}

template <int QT, bool KV8, bool Q8>
hipError_t launch_split_mla(const Params& p, hipStream_t stream) {
  if (p.sk_waves > 0) return hipErrorInvalidValue;   // stream-K: split_mla_ws.hip
  dim3 grid(p.max_splits, p.Hkv, p.B);
  hipLaunchKernelGGL((split_mla_kernel<QT, KV8, Q8>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

// 16-bit query and cache; 16-bit query and fp8 cache; fp8 query and cache
// (bf16 operands and output).
hipError_t launch_split_mla(int q_dtype, int kv_dtype, const Params& p, hipStream_t s) {
  if (kv_dtype == kFP8) {
    if (q_dtype == kFP8) return launch_split_mla<kBF16, true, true>(p, s);
    if (q_dtype == kBF16) return launch_split_mla<kBF16, true, false>(p, s);
    if (q_dtype == kF16) return launch_split_mla<kF16, true, false>(p, s);
    return hipErrorInvalidValue;
  }
  if (q_dtype != kv_dtype) return hipErrorInvalidValue;
  if (q_dtype == kBF16) return launch_split_mla<kBF16, false, false>(p, s);
  if (q_dtype == kF16) return launch_split_mla<kF16, false, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
