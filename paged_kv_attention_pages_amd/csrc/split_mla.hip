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
// Work split inside a workgroup of eight waves (two per SIMD): the waves
// divide the cached row by DIMENSION, not the query rows.  Wave w loads, for
// every token of a 32-token tile, latent dims [64w, 64w + 64) and rope dims
// [512 + 8w, 512 + 8w + 8) -- so every byte of the cache is loaded by
// exactly one wave and never shared through LDS.
// Per tile:
//   1. each wave forms partial scores over its dims for all 64 query rows
//        S^T_w (32 tokens x 64 rows) = K_w (32 x 72) . Q_w^T
//      (two token blocks x four row blocks of three 16x16x32 MFMA; the
//      8 rope dims ride in one whose other 24 K entries are zero -- a
//      16x16x16 MFMA feeding a 16x16x32 one as its accumulator read the
//      last two result registers before they were written on gfx950);
//   2. the partials go through LDS to the wave that owns the row block
//      (waves 0..3 own rows 16w .. 16w + 15), which sums the eight of them
//      and runs the online softmax of its rows;
//   3. the probabilities P (16-bit) and the rescale factors of all rows go
//      back through LDS, and every wave accumulates
//        O^T_w (64 dims x 64 rows) += V_w^T (64 x 32 tokens) . P^T
//      with one 16x16x32 MFMA per (4-dim group, row block).
// V_w^T needs the tile transposed (token along the MFMA K dimension): each
// wave stages its own 32 x 64 block in LDS in row order and reads it back by
// column, a wave-private round trip.  Sixty-four accumulator registers per
// lane keep the whole working set in the 256 VGPRs of a two-waves-per-SIMD
// budget, so the accumulators never move through AGPRs.
// The workgroup runs stream-K over 32-token tiles of all (sequence, KV head)
// units (one workgroup per CU), or one (sequence, split) per workgroup under
// the grid schedule.
#include "pkv_device.h"
#include "kernels.h"

namespace pkv {

namespace {
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

constexpr int kDqk = 576, kDv = 512;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kVw = kDv / kWaves;             // 64 latent dims per wave
constexpr int kRw = (kDqk - kDv) / kWaves;    // 8 rope dims per wave
constexpr int kTileTok = 32;                  // tokens per tile
constexpr int kTileShift = 5;
constexpr int kRowChunks = kVw / 8 + 1;       // staged token row: 8 chunks + 1 pad chunk
static_assert(kVw == 64 && kRw == 8, "dimension split assumes the 576/512 latent row");

// Staging, P and the rescale factors are double-buffered by tile parity:
// tile t's P . V runs while tile t + 1's softmax is computed.
struct Smem {
  uint4 t[2][kWaves][kTileTok * kRowChunks];  // per-wave staging for the V transpose
  f32x4 s[4][kWaves][2][64];                  // partial scores [row block][from wave][token block]
  uint4 pm[2][4][64];                         // P^T operand of each row block
  float alpha[2][16][4];                      // rescale factor of row 16 rb + n at [n][rb]
  float2 ml[64];                              // (max, sum) per row at the end of a unit
};

// This wave's slice of the query rows: B operands of S^T = K . Q^T.
struct QRegs {
  uint4 k[4][2];   // [row block][k step]: row 16 rb + n, dims 64 w + 32 st + 8 g .. + 8
  uint4 r[4];      // [row block]: row 16 rb + n, dims 512 + 8 w .. + 8 (g == 0; else 0)
};

// One tile of this wave's cache slice, as A operands of S^T = K . Q^T.
struct KTile {
  uint4 k[2][2];   // [token block][k step]: token 16 tb + n, dims 64 w + 32 st + 8 g .. + 8
  uint4 r[2];      // [token block]: token 16 tb + n, dims 512 + 8 w .. + 8 (g == 0; else 0)
};

// The token range [tok_lo, tok_hi) of one (sequence, KV head) that one
// workgroup processes, and what every wave needs to process it.
struct Piece {
  int b, kvh, L;
  int tok_lo, tok_hi;
  int lo_last;     // tokens >= lo_last pass every row's window
  int mask_from;   // tokens >= mask_from are subject to the draft mask
  int lane_k;      // byte offset of this lane's latent chunk inside a token row
  int lane_r;      // byte offset of this lane's rope chunk inside a token row (g == 0)
  uint32_t page_bytes;
  RowVis vis;      // visibility of this lane's row in the wave's own row block
};

struct Acc {
  f32x4 o[4][4];   // [row block][dim group e]: dims 64 w + 4 (4 g + i) + e, row 16 rb + n
  float m, l;      // running max (log2 units) and this lane's part of the sum (waves 0..3)
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

__device__ __forceinline__ void setup_piece(const Params& p, int b, int kvh, int tok_lo, int tok_hi,
                                            Piece& P) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4, w = wave_id();
  const SeqGeom sg = seq_geom(p, b);
  P.b = b;
  P.kvh = kvh;
  P.L = sg.L;
  P.tok_lo = tok_lo;
  P.tok_hi = tok_hi;
  P.lo_last = p.window > 0 ? sg.L - p.window : INT32_MIN;
  P.mask_from = (p.Tq > 1 && p.mask != nullptr) ? sg.L - p.Tq : sg.L;
  P.lane_k = (int)((n * p.k_slot + kvh * p.k_head + kVw * w + 8 * g) * 2);
  P.lane_r = g == 0 ? (int)((n * p.k_slot + kvh * p.k_head + kDv + kRw * w) * 2)
                    : (int)0x80000000u;
  P.page_bytes = (uint32_t)(p.k_page * 2);
  const int own = 16 * (w & 3) + n;
  P.vis = row_vis(p, b, sg.L, own < p.R ? own : 0);
}

// This wave's slice of the 64 query rows (zeros for rows >= R).
__device__ __forceinline__ void load_q(const Params& p, const Piece& P, QRegs& Q) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4, w = wave_id();
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int row = 16 * rb + n;
    const bool ok = row < p.R;
    const uint16_t* qrow = (const uint16_t*)p.q + q_row_offset(p, P.b, P.kvh, ok ? row : 0) * kDqk;
#pragma unroll
    for (int st = 0; st < 2; ++st)
      Q.k[rb][st] = ok ? *(const uint4*)(qrow + kVw * w + 32 * st + 8 * g) : make_uint4(0, 0, 0, 0);
    Q.r[rb] = ok && g == 0 ? *(const uint4*)(qrow + kDv + kRw * w) : make_uint4(0, 0, 0, 0);
  }
}

// Issue the loads of tile t (tokens 32 t .. 32 t + 31).  The run's page ids
// sit one per lane in my_page for pages pg_begin ..; a token block outside
// the run or on a page id outside the cache reads through an empty resource
// (zeros, no memory access), and tokens outside [tok_lo, tok_hi) get an
// offset past the end of the page, which also reads zeros -- so the
// invisible rows, which may hold anything, never reach the arithmetic.
__device__ __forceinline__ void load_tile(const Params& p, const Piece& P, int my_page, int pg_begin,
                                          bool live, int t, KTile& T) {
  const int n = threadIdx.x & 15;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int tok16 = t * kTileTok + 16 * tb;
    const int pg = tok16 / p.ps;
    const int rel = pg - pg_begin;
    int page = -1;
    if (live && rel >= 0 && rel < 64) page = __builtin_amdgcn_readlane(my_page, rel);
    const bool ok = (unsigned)page < (unsigned)p.num_pages;
    const uint16_t* base = (const uint16_t*)p.k + (ok ? (int64_t)page * p.k_page : 0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, ok ? P.page_bytes : 0u);
    const int soff = (int)((tok16 - pg * p.ps) * p.k_slot * 2);
    const int tok = tok16 + n;
    const bool in = tok >= P.tok_lo && tok < P.tok_hi;
    const int vk = in ? P.lane_k : (int)0x80000000u;
    const int vr = in ? P.lane_r : (int)0x80000000u;
#pragma unroll
    for (int st = 0; st < 2; ++st) buf_load<4>(rs, vk + 64 * st, soff, (uint32_t*)&T.k[tb][st]);
    buf_load<4>(rs, vr, soff, (uint32_t*)&T.r[tb]);
  }
}

// O^T += V^T . P^T for the tile staged in buffer `buf`, after rescaling the
// accumulators by that tile's factors.  Every wave, its own 64 dims.
template <int QT>
__device__ __forceinline__ void pv_tile(int buf, Smem& sm, Acc& A) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4, w = wave_id();
  // V^T operand source: token sigma(8 g + c) of this wave's block, dims 4 n .. 4 n + 4,
  // where the MFMA K index 8 g + c maps to token 4 g + c (c < 4) or 16 + 4 g + c - 4
  const uint2* rows2 = (const uint2*)sm.t[buf][w];
  uint2 vt[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int tk = c < 4 ? 4 * g + c : 16 + 4 * g + (c - 4);
    vt[c] = rows2[tk * (2 * kRowChunks) + n];
  }
  uint4 pb[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) pb[rb] = sm.pm[buf][rb][lane];
  const float4 al = *(const float4*)&sm.alpha[buf][n][0];
  const float alr[4] = {al.x, al.y, al.z, al.w};
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    if (__builtin_amdgcn_ballot_w64(alr[rb] != 1.f) != 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) A.o[rb][e] *= alr[rb];
    }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // 16-bit element e of each staged chunk, two tokens per dword
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    uint32_t a[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = (e >> 1) ? vt[2 * q].y : vt[2 * q].x;
      const uint32_t hi = (e >> 1) ? vt[2 * q + 1].y : vt[2 * q + 1].x;
      a[q] = __builtin_amdgcn_perm(hi, lo, sel);
    }
    const uint4 av = make_uint4(a[0], a[1], a[2], a[3]);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) A.o[rb][e] = mfma_k32<QT>(av, pb[rb], A.o[rb][e]);
  }
}

// Tile t: scores and softmax of t, and P . V of the previous tile (pv_prev)
// next to this tile's score product.
template <int QT>
__device__ __forceinline__ void compute_tile(const Params& p, const Piece& P, const QRegs& Q,
                                             const KTile& T, int t, bool pv_prev, Smem& sm, Acc& A) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4, w = wave_id();
  const int tok0 = t * kTileTok;
  const int cur = t & 1;

  // ---- 1. partial scores over this wave's dims; stage the tile for the transpose
  uint4* st_rows = sm.t[cur][w];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int st = 0; st < 2; ++st) st_rows[(16 * tb + n) * kRowChunks + 4 * st + g] = T.k[tb][st];
  f32x4 s[2][4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      f32x4 a = mfma_k32<QT>(T.r[tb], Q.r[rb], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int st = 0; st < 2; ++st) a = mfma_k32<QT>(T.k[tb][st], Q.k[rb][st], a);
      s[tb][rb] = a;
    }
  // every partial goes through LDS (also the owner's own: uniform code, no
  // branches, and the owner's eight reads issue back to back)
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) sm.s[rb][w][tb][lane] = s[tb][rb];
  // ---- the previous tile's O^T += V^T . P^T: its staging, P and factors
  // were published by the previous step's barriers, and running it here
  // keeps the matrix cores busy while the LDS absorbs this tile's writes
  if (pv_prev) pv_tile<QT>(cur ^ 1, sm, A);
  lds_barrier();

  // ---- 2. waves 0..3: sum the eight partials of row block w; online softmax
  if (w < 4) {
    f32x4 sc[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      // eight reads in flight, then a pairwise sum in a fixed order; one
      // token block at a time to bound the registers held by the reads
      f32x4 part[kWaves];
#pragma unroll
      for (int src = 0; src < kWaves; ++src) part[src] = sm.s[w][src][tb][lane];
      const f32x4 a01 = part[0] + part[1], a23 = part[2] + part[3];
      const f32x4 a45 = part[4] + part[5], a67 = part[6] + part[7];
      sc[tb] = (a01 + a23) + (a45 + a67);
      __builtin_amdgcn_sched_barrier(0);
    }
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
    // P^T operand (K index 8 g + c <-> the token order of the V^T operand);
    // the sum takes the rounded probabilities, so the output is an exact
    // weighted mean of the V rows and the rounding error scales with |V - out|
    const uint4 pw = make_uint4(pack2<QT>(pr[0][0], pr[0][1]), pack2<QT>(pr[0][2], pr[0][3]),
                                pack2<QT>(pr[1][0], pr[1][1]), pack2<QT>(pr[1][2], pr[1][3]));
    const float2 r0 = unpack2<QT>(pw.x), r1 = unpack2<QT>(pw.y);
    const float2 r2 = unpack2<QT>(pw.z), r3 = unpack2<QT>(pw.w);
    A.l = A.l * alpha + (((r0.x + r0.y) + (r1.x + r1.y)) + ((r2.x + r2.y) + (r3.x + r3.y)));
    A.m = m_new;
    sm.pm[cur][w][lane] = pw;
    if (g == 0) sm.alpha[cur][n][w] = alpha;
  }
  lds_barrier();
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

// Tiles [R.begin, t_to) of a piece, run by run; within a run an NS-deep
// register pipeline keeps NS - 1 tiles' loads in flight while one is
// computed.  The first run's page ids come in already loaded.
template <int QT, int NS>
__device__ __forceinline__ void stream_piece(const Params& p, const Piece& P, const QRegs& Q, Run R,
                                             int t_to, Smem& sm, Acc& A) {
  const int t_first = R.begin;
  while (true) {
    KTile buf[NS];
#pragma unroll
    for (int k = 0; k < NS - 1; ++k) {
      load_tile(p, P, R.my_page, R.pg_begin, R.begin + k < R.end, R.begin + k, buf[k]);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int t = R.begin; t < R.end; t += NS) {
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int tl = t + k + NS - 1;
        load_tile(p, P, R.my_page, R.pg_begin, tl < R.end, tl, buf[(k + NS - 1) % NS]);
        if (k == 0 || t + k < R.end) compute_tile<QT>(p, P, Q, buf[k], t + k, t + k > t_first, sm, A);
      }
    }
    if (R.end >= t_to) break;
    R = open_run(p, P, R.end, t_to);
  }
  // drain: the last tile's P . V (its P is visible after the last barrier)
  if (t_to > t_first) pv_tile<QT>((t_to - 1) & 1, sm, A);
}

__device__ __forceinline__ void reset(Acc& A) {
  A.m = kNegInf;
  A.l = 0.f;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int e = 0; e < 4; ++e) A.o[rb][e] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Normalised output when this workgroup saw the whole unit, else the
// partial (m, l, o) in workspace rows prow0 + row.
template <int QT>
__device__ __forceinline__ void finish_piece(const Params& p, const Piece& P, Acc& A, Smem& sm,
                                             bool complete, int64_t prow0) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4, w = wave_id();
  const float l = sum_across_rows(A.l);
  if (w < 4 && g == 0) sm.ml[16 * w + n] = make_float2(A.m, l);
  lds_barrier();
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int row = 16 * rb + n;
    if (row >= p.R) continue;
    const float2 ml = sm.ml[row];
    // lane (n, g) holds dims 64 w + 16 g + 4 i + e of this row
    if (complete) {
      float num = 1.f, den = ml.y;
      if (p.sinks != nullptr) {
        const float sk = p.sinks[P.kvh * p.G + row % p.G] * kLog2e;
        const float Mf = fmaxf(ml.x, sk);
        num = ml.x == kNegInf ? 0.f : exp2f(ml.x - Mf);
        den = ml.y * num + exp2f(sk - Mf);
      }
      const float inv = den > 0.f ? p.out_scale * num / den : 0.f;
      uint16_t* o = (uint16_t*)p.out + q_row_offset(p, P.b, P.kvh, row) * kDv + kVw * w + 16 * g;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *(uint4*)(o + 8 * h) =
            make_uint4(pack2<QT>(A.o[rb][0][2 * h] * inv, A.o[rb][1][2 * h] * inv),
                       pack2<QT>(A.o[rb][2][2 * h] * inv, A.o[rb][3][2 * h] * inv),
                       pack2<QT>(A.o[rb][0][2 * h + 1] * inv, A.o[rb][1][2 * h + 1] * inv),
                       pack2<QT>(A.o[rb][2][2 * h + 1] * inv, A.o[rb][3][2 * h + 1] * inv));
    } else {
      float* o = p.ws_o + (prow0 + row) * kDv + kVw * w + 16 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(float4*)(o + 4 * i) = make_float4(A.o[rb][0][i], A.o[rb][1][i], A.o[rb][2][i], A.o[rb][3][i]);
      if (w == rb && g == 0) p.ws_ml[prow0 + row] = ml;
    }
  }
}

constexpr int kStages = 3;

}  // namespace

// Grid schedule: one workgroup per (split, KV head, sequence).
template <int QT>
__global__ __launch_bounds__(kThreads) void split_mla_kernel(Params p) {
  __shared__ Smem sm;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const SeqGeom sg = seq_geom(p, b);
  if (split >= sg.nsplits) return;
  const int pg_begin = sg.p0 + split * p.split_pages;
  const int pg_end = min(pg_begin + p.split_pages, sg.p0 + sg.npages);
  const int tok_lo = max(pg_begin * p.ps, sg.lo), tok_hi = min(pg_end * p.ps, sg.L);
  Piece P;
  setup_piece(p, b, kvh, tok_lo, tok_hi, P);
  const int t_to = (tok_hi + kTileTok - 1) >> kTileShift;
  const Run R = open_run(p, P, tok_lo >> kTileShift, t_to);
  QRegs Q;
  load_q(p, P, Q);
  Acc A;
  reset(A);
  stream_piece<QT, kStages>(p, P, Q, R, t_to, sm, A);
  finish_piece<QT>(p, P, A, sm, sg.nsplits == 1,
                   (((int64_t)b * p.Hkv + kvh) * p.max_splits + split) * p.R);
}

// Stream-K schedule over 32-token tiles: workgroup w of W takes an equal
// share of the tile stream of all units; units wholly inside its share are
// finished here, the first and the last (when cut) leave partials in
// workspace slots 2w and 2w+1.
template <int QT>
__global__ __launch_bounds__(kThreads) void split_mla_sk_kernel(Params p) {
  __shared__ Smem sm;
  // the schedule's per-sequence tile prefix sums and counts live in LDS, so
  // the unit loop carries no per-lane schedule state
  __shared__ int sk_pre[kSkMaxBatch], sk_cnt[kSkMaxBatch];
  const int lane = threadIdx.x & 63;
  int64_t T;
  {
    const SkSched S = sk_schedule(p);
    T = S.T;
    if (wave_id() == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sk_pre[lane + 64 * c] = S.pre[c];
        sk_cnt[lane + 64 * c] = S.cnt[c];
      }
    }
  }
  lds_barrier();
  const int wg = blockIdx.x, W = sk_waves_eff(T, gridDim.x);
  if (wg >= W) return;
  // the host keeps the tile stream under 2^31 tiles for this kernel
  const int x0 = (int)sk_wave_start(T, wg, W), x1 = (int)sk_wave_start(T, wg + 1, W);
  const int Hkv = p.Hkv;
  for (int x = x0; x < x1;) {
    Piece P;
    QRegs Q;
    Acc A;
    // unit holding global tile x: the last sequence whose first tile is <= x
    int b = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int bb = lane + 64 * c;
      const bool ok = bb < p.B && sk_pre[bb] * Hkv <= x;
      const uint64_t m = __ballot(ok);
      if (m != 0) b = 64 * c + 63 - __builtin_clzll(m);
    }
    const int pre = sk_pre[b], ntiles = sk_cnt[b];
    const int kvh = (x - pre * Hkv) / ntiles;
    const int ustart = pre * Hkv + kvh * ntiles;
    const int seg_end = min(x1, ustart + ntiles);
    const SeqGeom sg = seq_geom(p, b);
    const int tile0 = sg.lo >> kTileShift;
    const int t_from = tile0 + (x - ustart), t_to = tile0 + (seg_end - ustart);
    const int tok_lo = max(t_from * kTileTok, sg.lo), tok_hi = min(t_to * kTileTok, sg.L);
    setup_piece(p, b, kvh, tok_lo, tok_hi, P);
    const Run R = open_run(p, P, t_from, t_to);
    load_q(p, P, Q);
    reset(A);
    stream_piece<QT, kStages>(p, P, Q, R, t_to, sm, A);
    const bool complete = x == ustart && seg_end == ustart + ntiles;
    const int slot = 2 * wg + (x == x0 ? 0 : 1);
    finish_piece<QT>(p, P, A, sm, complete, (int64_t)slot * p.R);
    x = seg_end;
  }
}

template <int QT>
hipError_t launch_split_mla(const Params& p, hipStream_t stream) {
  if (p.sk_waves > 0) {
    if (p.sk_shift != kTileShift || p.B > kSkMaxBatch) return hipErrorInvalidValue;
    hipLaunchKernelGGL((split_mla_sk_kernel<QT>), dim3(p.sk_waves), dim3(kThreads), 0, stream, p);
  } else {
    dim3 grid(p.max_splits, p.Hkv, p.B);
    hipLaunchKernelGGL((split_mla_kernel<QT>), grid, dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_split_mla(int q_dtype, const Params& p, hipStream_t s) {
  if (q_dtype == kBF16) return launch_split_mla<kBF16>(p, s);
  if (q_dtype == kF16) return launch_split_mla<kF16>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
