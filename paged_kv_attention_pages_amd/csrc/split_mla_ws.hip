// split_mla_ws.hip -- latent (MLA) split-KV decode with wave-specialised
// roles, for 16-bit latent caches: one KV head's 576-wide rows, of which the
// first 512 entries are V, and up to 64 query rows.
//
// vLLM `models/kimi_k3/nvidia/mla` page, MultiHeadLatentAttention: the decode
// branch of `_attention` runs multi-query attention of the absorbed queries
// over the latent cache rows [kv_c_normed | k_pe] (`forward_mqa`), and the
// kv_lora_rank-wide result is what `_v_up_proj` projects back -- so V is the
// leading kv_lora_rank entries of each K row.
//
// A workgroup of eight waves runs stream-K over 32-token tiles (one workgroup
// per CU).  The tiles enter a four-slot LDS ring straight from HBM: each tile
// row goes in with buffer loads that write LDS (16 bytes per lane, no
// register staging), issued three tiles ahead.  The waves split the work by
// role, and the two roles work on neighbouring tiles in the same step:
//   score waves 0..3 (one per SIMD): wave rb computes the scores of query rows
//     16 rb .. + 15 against all 32 tokens of tile t + 1 over all 576 dims,
//     S^T (32 tokens x 16 rows) = K . Q^T, 36 16x16x32 MFMAs with the query
//     slice held in registers, runs the rows' online softmax, and leaves the
//     16-bit probabilities and the rows' rescale factors in LDS;
//   P.V waves 4..7 (one per SIMD): wave (rh, dh) takes rows 32 rh .. + 31 and
//     value dims 256 dh .. + 255 of tile t: it rescales its accumulators and
//     adds O^T (256 dims x 32 rows) += V^T . P^T as 32x32x16 MFMAs with V^T
//     from transposed LDS reads; these waves also issue the tile loads.
// One barrier per step.  Per tile the LDS serves 144 KB of K reads, 64 KB of
// V reads and 12 KB of probability traffic -- against about 290 KB read and
// 52 KB written when every wave did both products for its own rows.
//
// The loads that write LDS are issued through a short asm block: the
// compiler would otherwise wait for every outstanding one before each LDS
// read and each barrier.  The P.V waves count their own loads (a fixed nine
// per tile) with explicit vmcnt waits; the score waves issue no tile loads,
// so the compiler's waits on their query loads stay exact.  Page ids are
// read with scalar loads (constant address space), which do not use vmcnt.
#include "pkv_device.h"
#include "kernels.h"

namespace pkv {

namespace {
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

constexpr int kDqk = 576, kDv = 512;
constexpr int kThreads = 512;
constexpr int kTileTok = 32;
constexpr int kQkSteps = kDqk / 32;           // 18 K steps of the score product
// LDS tile: two halves of 16 rows; a half holds the first 1024 bytes of its
// rows (dims 0 .. 511) at a 1024-byte pitch, then the last 128 bytes (the
// rope dims) at a 128-byte pitch.  The 16-byte chunks of a row are
// XOR-swizzled (swz_lo / swz_hi), so that K reads (sixteen rows, one chunk
// each), transposed V reads (four rows, 32 bytes each) and the row loads
// spread over the banks.
constexpr int kLoBytes = 1024, kHiBytes = 128;
constexpr int kHiOff = 16 * kLoBytes;
constexpr int kHalfBytes = 16 * (kLoBytes + kHiBytes);   // 18432
constexpr int kTileBytes = 2 * kHalfBytes;                // 36864
constexpr int kRing = 4;
constexpr int kLoadsPerWave = 9;              // 32 row loads + 4 rope loads per tile, over 4 waves

struct Smem {
  uint8_t tile[kRing][kTileBytes];
  // probabilities (four 16-bit values) [parity][row block][token half][g / 2][n][g % 2]:
  // 16 bytes at [..][h][n] are tokens 16 tb + 8 h .. + 7 of row 16 rb + n
  uint2 p[2][4][2][2][16][2];
  float alpha[2][64];                         // per-row rescale of the P.V accumulators
  float2 ml[2][64];                           // (m, l) of rows whose piece ends at this tile
};

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(4))) const int32_t const_i32;

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// swz_lo is the linear map over the four row bits r0..r3 that XORs the
// chunk index with 4 r0 ^ 8 r1 ^ 3 r2 ^ 2 r3.  It was chosen with per-pattern
// bank-conflict counters on gfx950: 16-byte reads serve the lanes in four
// groups of 16 that mix both halves of the wave, 8-byte (and transposed)
// reads in two groups of 32, and with this map the K reads (one chunk of 16
// rows per 16 lanes) and the transposed V reads (four rows x four chunks
// per 32 lanes) both run without conflicts, where the tables r ^ 2r and
// the 2-bit transpose each conflict on one of the two.
__device__ __forceinline__ int swz_lo(int r) {
  return ((r & 1) ? 4 : 0) ^ ((r & 2) ? 8 : 0) ^ ((r & 4) ? 3 : 0) ^ ((r & 8) ? 2 : 0);
}
__device__ __forceinline__ int swz_hi(int r) { return (r >> 1) & 7; }
// byte offset of 16-byte chunk c of row r's low part, chunk-swizzled
__device__ __forceinline__ int lo_chunk(int r, int c) {
  return r * kLoBytes + 16 * ((c & ~15) | ((c & 15) ^ swz_lo(r)));
}

// 32-bit LDS address of a shared-memory pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Buffer resource over `bytes` bytes at `base` (raw, stride 0): offsets at or
// past `bytes` read as zeros without touching memory.
__device__ __forceinline__ i32x4 rsrc4(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from memory into LDS (buffer_load_dwordx4 ... lds, non-
// temporal): lane l's bytes, at byte voff + soff of the resource, land at
// lds + 16 l.  M0 carries the LDS address and is restored afterwards.  No
// register receives data, so nothing in the compiler's view waits for it;
// the caller waits with vmcnt.
__device__ __forceinline__ void load_to_lds(const i32x4& rs, uint32_t lds, int voff, int soff) {
  int save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds), "v"(voff), "s"(rs), "s"(soff)
      : "memory");
}

// Wait until at most N of this wave's vector memory operations are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// Workgroup barrier for LDS: this wave's LDS (and scalar) operations are
// complete first; outstanding vector memory operations stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Transposed LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, lane
// a + 4 j supplies the address of four 16-bit elements and lane 4 a + e
// receives element e of lanes a, a + 4, a + 8, a + 12, in that order.
__device__ __forceinline__ uint2 lds_read_tr16(const uint8_t* addr) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(addr));
  return __builtin_bit_cast(uint2, v);
}

// D(32x32) += A(32x16) * B(16x32).  Lane l supplies A[l%32][8(l/32)..+8] and
// B[8(l/32)..+8][l%32]; it receives D[8(i/4) + 4(l/32) + i%4][l%32] in i.
template <int QT>
__device__ __forceinline__ f32x16 mfma_32x32(uint4 a, uint4 b, f32x16 c) {
  if constexpr (QT == kBF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// The unit (sequence b, KV head kvh) holding global stream-K tile x: its
// global tiles [ustart, uend), the sequence tile of its first global tile,
// its length and its first visible token.
struct UnitPos {
  int b, kvh, ustart, uend, tile0, L, lo;
};

// The sequence length is read with a scalar load (constant address space):
// a vector load here would make the compiler wait for every outstanding
// vector memory operation, the in-flight tile loads included.  L and lo
// follow seq_geom.
__device__ __forceinline__ UnitPos locate(const Params& p, const SkSched& S, int x) {
  const SkUnit su = sk_locate(p, S, x);
  UnitPos u;
  u.b = su.b;
  u.kvh = su.kvh;
  u.ustart = (int)su.start;
  u.uend = (int)su.start + su.ntiles;
  const uint32_t Lraw = ((__attribute__((address_space(4))) const uint32_t*)p.seq_lens)[su.b];
  const int cap = p.pps * p.ps;
  u.L = Lraw > (uint32_t)cap ? cap : (int)Lraw;
  u.lo = p.window > 0 ? max(0, u.L - p.Tq + 1 - p.window) : 0;
  u.tile0 = u.lo >> 5;
  return u;
}

// ---------------------------------------------------------------- tile loads
// The P.V waves' load cursor: the next global tile to load, its unit and the
// page ids of its two 16-row halves (-1: nothing to read).  The page ids are
// read one step before the tile's loads are issued, so the scalar loads
// never hold up the issue.
struct LoadCursor {
  UnitPos u;
  int t;
  int pid0, pid1;
};

__device__ __forceinline__ void fetch_page_ids(const Params& p, int x1, LoadCursor& c) {
  c.pid0 = c.pid1 = -1;
  if (c.t >= x1) return;
  const int tok0 = (c.u.tile0 + (c.t - c.u.ustart)) << 5;
  const const_i32* row = (const const_i32*)p.page_table + (int64_t)c.u.b * p.pps;
  if (tok0 < c.u.L) c.pid0 = row[tok0 >> p.ps_shift];
  if (tok0 + 16 < c.u.L) c.pid1 = row[(tok0 + 16) >> p.ps_shift];
}

// Move the cursor to tile t (the next one, or the first of the share).
__device__ __forceinline__ void advance(const Params& p, const SkSched& S, int x1, int t, LoadCursor& c) {
  c.t = t;
  if (t < x1 && t >= c.u.uend) c.u = locate(p, S, t);
  fetch_page_ids(p, x1, c);
}

// Per-lane parts of a P.V wave's tile loads, fixed for the kernel: the
// byte offset inside a row of the 16-byte chunk that lane l loads for low
// rows 4 a + pw (chunk l, swizzled so that it lands at its place), and the
// row and rope offset of the lane's rope load (rows 8 (pw & 1) + l / 8).
struct LoadLanes {
  int lo[4];
  int rope_row, rope_col;
};

__device__ __forceinline__ LoadLanes load_lanes(int pw) {
  const int lane = threadIdx.x & 63;
  LoadLanes ll;
#pragma unroll
  for (int a = 0; a < 4; ++a) ll.lo[a] = 16 * ((lane & ~15) | ((lane & 15) ^ swz_lo(4 * a + pw)));
  ll.rope_row = 8 * (pw & 1) + (lane >> 3);
  ll.rope_col = kLoBytes + 16 * ((lane & 7) ^ swz_hi(ll.rope_row));
  return ll;
}

// Issue this P.V wave's nine loads of the cursor's tile into ring slot
// `slot_lds`: rows pw, pw + 4, ..., pw + 28 (one 1024-byte low part each;
// rows 4 k + pw lie in half k / 4) and rope block pw (rows 8 (pw & 1) .. + 7
// of half pw / 2).  The row offset goes in the scalar offset, so a tile whose
// 32 rows are all visible needs no per-lane arithmetic; on a tile that
// crosses the sequence's visible span [lo, L) the rows outside read as
// zeros (an offset past the page), and so do pages with ids outside the
// cache and tiles past the share (empty resource).
__device__ __forceinline__ void load_tile(const Params& p, const LoadCursor& c, const LoadLanes& ll,
                                          uint32_t slot_lds, int pw) {
  const int tok0 = (c.u.tile0 + (c.t - c.u.ustart)) << 5;
  const uint32_t page_bytes = (uint32_t)(p.k_page * 2);
  const int row_bytes = (int)(p.k_slot * 2);
  const int head_off = (int)(c.u.kvh * p.k_head * 2);
  const int pmask = p.ps - 1;
  const bool ok0 = (unsigned)c.pid0 < (unsigned)p.num_pages, ok1 = (unsigned)c.pid1 < (unsigned)p.num_pages;
  const i32x4 rs0 = rsrc4((const uint8_t*)p.k + (ok0 ? (int64_t)c.pid0 * page_bytes : 0), ok0 ? page_bytes : 0u);
  const i32x4 rs1 = rsrc4((const uint8_t*)p.k + (ok1 ? (int64_t)c.pid1 * page_bytes : 0), ok1 ? page_bytes : 0u);
  if (tok0 >= c.u.lo && tok0 + kTileTok <= c.u.L) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int hf = k >> 2, rr = 4 * (k & 3) + pw;
      const int soff = ((tok0 + 16 * hf + rr) & pmask) * row_bytes + head_off;
      load_to_lds(hf ? rs1 : rs0, slot_lds + hf * kHalfBytes + rr * kLoBytes, ll.lo[k & 3], soff);
    }
    const int hf = pw >> 1;
    const int soff = ((tok0 + 16 * hf + 8 * (pw & 1)) & pmask) * row_bytes + head_off;
    load_to_lds(hf ? rs1 : rs0, slot_lds + hf * kHalfBytes + kHiOff + 8 * (pw & 1) * kHiBytes,
                (ll.rope_row - 8 * (pw & 1)) * row_bytes + ll.rope_col, soff);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int hf = k >> 2, rr = 4 * (k & 3) + pw;
      const int tok = tok0 + 16 * hf + rr;
      const bool in = tok >= c.u.lo && tok < c.u.L;
      const int voff = in ? (tok & pmask) * row_bytes + head_off + ll.lo[k & 3] : (int)0x80000000u;
      load_to_lds(hf ? rs1 : rs0, slot_lds + hf * kHalfBytes + rr * kLoBytes, voff, 0);
    }
    const int hf = pw >> 1;
    const int tok = tok0 + 16 * hf + ll.rope_row;
    const bool in = tok >= c.u.lo && tok < c.u.L;
    const int voff = in ? (tok & pmask) * row_bytes + head_off + ll.rope_col : (int)0x80000000u;
    load_to_lds(hf ? rs1 : rs0, slot_lds + hf * kHalfBytes + kHiOff + 8 * (pw & 1) * kHiBytes, voff, 0);
  }
}

// ---------------------------------------------------------------- score waves
struct QRegs {
  uint4 k[kQkSteps];   // row 16 rb + n, dims 32 s + 8 g .. + 8
};

__device__ __forceinline__ void load_q(const Params& p, const UnitPos& u, int rb, QRegs& Q) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int row = 16 * rb + n;
  const bool ok = row < p.R;
  const uint16_t* q = (const uint16_t*)p.q + q_row_offset(p, u.b, u.kvh, ok ? row : 0) * kDqk + 8 * g;
#pragma unroll
  for (int s = 0; s < kQkSteps; ++s) Q.k[s] = ok ? *(const uint4*)(q + 32 * s) : make_uint4(0, 0, 0, 0);
}

// Score step for tile t (in ring slot tl): S^T of rows 16 rb .. + 15
// against the tile's 32 tokens over all 576 dims, then the online softmax of
// those rows.  K fragment (tb, s) of lane (n, g) is chunk 4 s + g of row
// 16 tb + n (steps 16 and 17: rope chunks g and 4 + g); the reads run kAhead
// MFMAs ahead.  Lane (n, g) ends with tokens 16 tb + 4 g + i of row n; the
// wave keeps the row's running reference max m (log2 units) and its sum l
// of the rounded probabilities, and leaves in LDS the probabilities (16-bit)
// and the factor alpha by which the P.V waves rescale their accumulators.
struct RowState {
  float m, l;
};

template <int QT>
__device__ __forceinline__ void score_tile(const Params& p, const UnitPos& u, const RowVis& vis, int lo_last,
                                           int mask_from, const QRegs& Q, const uint8_t* tl, int rb, int par, int t,
                                           Smem& sm, RowState& st) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  int base[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) base[i] = n * kLoBytes + 16 * ((4 * i + g) ^ swz_lo(n));
  const int hi0 = kHiOff + n * kHiBytes + 16 * (g ^ swz_hi(n));
  const int hi1 = kHiOff + n * kHiBytes + 16 * ((4 + g) ^ swz_hi(n));
  auto frag = [&](int j) {
    const int s = j >> 1, tb = j & 1;
    const int o = s < 16 ? base[s & 3] + 256 * (s >> 2) : (s == 16 ? hi0 : hi1);
    return *(const uint4*)(tl + tb * kHalfBytes + o);
  };
  constexpr int kFrags = 2 * kQkSteps, kAhead = 6;
  uint4 kf[kAhead];
#pragma unroll
  for (int j = 0; j < kAhead; ++j) kf[j] = frag(j);
  f32x4 s4[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int j = 0; j < kFrags; ++j) {
    const uint4 cur = kf[j % kAhead];
    if (j + kAhead < kFrags) kf[j % kAhead] = frag(j + kAhead);
    s4[j & 1] = mfma_k32<QT>(cur, Q.k[j >> 1], s4[j & 1]);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
  for (int j = 0; j < kFrags - kAhead; ++j) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
  // ---- online softmax of row n over tokens 16 tb + 4 g + i
  float x[2][4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[tb][i] = s4[tb][i] * p.qk_scale_log2;
  // tiles that hold a token invisible to some row (window, draft mask, the
  // sequence's ends) mask; the others are visible to every row
  const int tok0 = (u.tile0 + (t - u.ustart)) << 5;
  if (tok0 < lo_last || tok0 + kTileTok > mask_from) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[tb][i] = vis(tok0 + 16 * tb + 4 * g + i, u.L) ? x[tb][i] : kNegInf;
  }
  float tmax = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                     fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
  tmax = max_across_rows(tmax);
  // the reference moves only when the tile max passes it by kSlack
  const bool bump = tmax > st.m + kSlack;
  const float m_new = bump ? tmax : st.m;
  const float m_ref = m_new == kNegInf ? 0.f : m_new;
  const float alpha = bump ? __builtin_amdgcn_exp2f(st.m - m_ref) : 1.f;
  float tsum = 0.f;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const uint32_t w0 = pack2<QT>(__builtin_amdgcn_exp2f(x[tb][0] - m_ref), __builtin_amdgcn_exp2f(x[tb][1] - m_ref));
    const uint32_t w1 = pack2<QT>(__builtin_amdgcn_exp2f(x[tb][2] - m_ref), __builtin_amdgcn_exp2f(x[tb][3] - m_ref));
    // the sum takes the rounded probabilities, so the output is an exact
    // weighted mean of the V rows
    const float2 r0 = unpack2<QT>(w0), r1 = unpack2<QT>(w1);
    tsum += (r0.x + r0.y) + (r1.x + r1.y);
    sm.p[par][rb][tb][g >> 1][n][g & 1] = make_uint2(w0, w1);
  }
  tsum = sum_across_rows(tsum);
  st.l = st.l * alpha + tsum;
  st.m = m_new;
  if (g == 0) sm.alpha[par][16 * rb + n] = alpha;
}

// Score waves: tile t in step t - 1 (the prologue step for x0).  The query
// slice of the next unit is loaded one step before it is needed.  When a
// tile ends the workgroup's piece of its unit, the rows' (m, l) go to LDS for
// the P.V waves, which finish the piece one step later.
template <int QT>
__device__ __forceinline__ void score_role(const Params& p, const SkSched& S, int x0, int x1, Smem& sm) {
  const int rb = wave_id(), lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int row = 16 * rb + n;
  UnitPos cur = locate(p, S, x0), nxt = cur;
  QRegs Q, Qn;
  load_q(p, cur, rb, Q);
  RowVis vis{};
  int lo_last = 0, mask_from = 0;
  RowState st{kNegInf, 0.f};
  auto step = [&](int t) {
    if (t >= cur.uend) {
      cur = nxt;
      Q = Qn;
    }
    if (t == x0 || t == cur.ustart) {
      vis = row_vis(p, cur.b, cur.L, row < p.R ? row : 0);
      lo_last = p.window > 0 ? cur.L - p.window : INT32_MIN;
      mask_from = (p.Tq > 1 && p.mask != nullptr) ? cur.L - p.Tq : cur.L;
      st.m = kNegInf;
      st.l = 0.f;
    }
    if (t + 1 < x1 && t + 1 >= cur.uend) {
      nxt = locate(p, S, t + 1);
      load_q(p, nxt, rb, Qn);
    }
    const int i = t - x0;
    score_tile<QT>(p, cur, vis, lo_last, mask_from, Q, sm.tile[i & 3], rb, i & 1, t, sm, st);
    if ((t + 1 == cur.uend || t + 1 == x1) && g == 0) sm.ml[i & 1][row] = make_float2(st.m, st.l);
  };
  lds_barrier();            // tile x0 is in LDS
  step(x0);
  lds_barrier();            // probabilities of x0 are in LDS; tile x0 + 1 is in LDS
  for (int x = x0; x < x1; ++x) {
    if (x + 1 < x1) step(x + 1);
    lds_barrier();
  }
}

// ---------------------------------------------------------------- P.V waves
struct PvState {
  f32x16 o[8];     // dims 256 dh + 32 j + 8 (i / 4) + 4 h + i % 4 of row 32 rh + (lane % 32)
};

// Per-lane LDS offsets of the transposed V reads: read (cc, j) of lane (s, G)
// takes row 8 h + 4 cc + s / 4 of a half tile, dims 256 dh + 32 j + 16 (G % 2)
// + 4 (s % 4) .. + 4; the XOR of the chunk index with the row's swizzle only
// touches its low four bits, so j = a + 4 (a < 4) is a 256-byte step from j = a.
struct VOff {
  int o[2][4];
};

__device__ __forceinline__ VOff v_offsets(int dh) {
  const int lane = threadIdx.x & 63, s = lane & 15, G = lane >> 4, h = lane >> 5;
  VOff v;
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    const int rr = 8 * h + 4 * cc + (s >> 2);
    const int e = 2 * (G & 1) + ((s & 3) >> 1);   // chunk bits 0..1
#pragma unroll
    for (int a = 0; a < 4; ++a) v.o[cc][a] = lo_chunk(rr, 32 * dh + 4 * a + e) + 8 * (s & 1);
  }
  return v;
}

// P.V step for tile x (ring slot tl): rescale by the rows' alpha, then
// O^T (256 dims x 32 rows) += V^T . P^T as 32x32x16 MFMAs, token step ts
// outer so that consecutive MFMAs feed different accumulators.  K index
// 8 h + c of token step ts is token 16 ts + 8 h + c in both operands.
template <int QT>
__device__ __forceinline__ void pv_tile(const VOff& vo, const uint8_t* tl, int rh, int par, Smem& sm, PvState& A) {
  const int lane = threadIdx.x & 63, col = lane & 31, h = lane >> 5;
  const int rb = 2 * rh + (col >> 4), n = col & 15;
  const float alpha = sm.alpha[par][32 * rh + col];
  uint4 pw[2];
#pragma unroll
  for (int ts = 0; ts < 2; ++ts) pw[ts] = *(const uint4*)&sm.p[par][rb][ts][h][n][0];
  auto vread = [&](int q) {
    const int ts = q >> 3, jb = q & 7;
    const int o = ts * kHalfBytes + 256 * (jb >> 2);
    const uint2 a = lds_read_tr16(tl + o + vo.o[0][jb & 3]);
    const uint2 b = lds_read_tr16(tl + o + vo.o[1][jb & 3]);
    return make_uint4(a.x, a.y, b.x, b.y);
  };
  constexpr int kVAhead = 4;
  uint4 vf[kVAhead];
#pragma unroll
  for (int q = 0; q < kVAhead; ++q) vf[q] = vread(q);
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) A.o[j] *= alpha;
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const uint4 cur = vf[q % kVAhead];
    if (q + kVAhead < 16) vf[q % kVAhead] = vread(q + kVAhead);
    A.o[q & 7] = mfma_32x32<QT>(cur, pw[q >> 3], A.o[q & 7]);
  }
#pragma unroll
  for (int q = 0; q + kVAhead < 16; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kVAhead, 0);
}

// The normalised output rows (the unit was whole in this share) or the
// partial (m, l, o) in workspace slot `slot`.  A slot holds 64 (m, l) rows
// and the four P.V waves' accumulators in register order -- wave pw's
// element (j, 4 q + e) of lane l at float ((pw * 32 + 4 j + q) * 64 + l) * 4
// + e -- so that every store instruction writes 1 KB contiguously.
template <int QT>
__device__ __forceinline__ void pv_finish(const Params& p, const UnitPos& u, int rh, int dh, const PvState& A,
                                          float2 ml, bool complete, int64_t slot) {
  const int lane = threadIdx.x & 63, col = lane & 31, h = lane >> 5;
  const int row = 32 * rh + col;
  if (row >= p.R) return;
  const int dbase = 256 * dh + 4 * h;
  if (complete) {
    float num = 1.f, den = ml.y;
    if (p.sinks != nullptr) {
      const float sk = p.sinks[u.kvh * p.G + row % p.G] * kLog2e;
      const float Mf = fmaxf(ml.x, sk);
      num = ml.x == kNegInf ? 0.f : exp2f(ml.x - Mf);
      den = ml.y * num + exp2f(sk - Mf);
    }
    const float inv = den > 0.f ? p.out_scale * num / den : 0.f;
    const int64_t ob = q_row_offset(p, u.b, u.kvh, row) * kDv + dbase;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        store_out4<QT>(p, ob + 32 * j + 8 * q, A.o[j][4 * q] * inv, A.o[j][4 * q + 1] * inv,
                       A.o[j][4 * q + 2] * inv, A.o[j][4 * q + 3] * inv);
  } else {
    float* o = p.ws_o + (slot * 4 + 2 * rh + dh) * (32 * 64 * 4) + 4 * lane;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(float4*)(o + (4 * j + q) * 256) =
            make_float4(A.o[j][4 * q], A.o[j][4 * q + 1], A.o[j][4 * q + 2], A.o[j][4 * q + 3]);
    if (dh == 0 && h == 0) p.ws_ml[slot * 64 + row] = ml;
  }
}

template <int QT>
__device__ __forceinline__ void pv_role(const Params& p, const SkSched& S, int x0, int x1, int wg, Smem& sm) {
  const int pwv = wave_id() - 4, rh = pwv >> 1, dh = pwv & 1;
  const int lane = threadIdx.x & 63;
  const uint32_t ring = lds_addr(&sm.tile[0][0]);
  const VOff vo = v_offsets(dh);
  const LoadLanes ll = load_lanes(pwv);
  // loads run three tiles ahead of the P.V step
  LoadCursor lc;
  lc.u = locate(p, S, x0);
  advance(p, S, x1, x0, lc);
  auto issue = [&]() {
    load_tile(p, lc, ll, ring + ((lc.t - x0) & 3) * kTileBytes, pwv);
    advance(p, S, x1, lc.t + 1, lc);
  };
  issue();
  issue();
  issue();
  wait_vm<2 * kLoadsPerWave>();   // tile x0 is in LDS
  lds_barrier();
  wait_vm<kLoadsPerWave>();       // tile x0 + 1 is in LDS
  lds_barrier();
  UnitPos cur = locate(p, S, x0);
  PvState A;
#pragma unroll
  for (int j = 0; j < 8; ++j) A.o[j] = f32x16{};
  for (int x = x0; x < x1; ++x) {
    issue();                      // tile x + 3
    if (x >= cur.uend) {
      cur = locate(p, S, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) A.o[j] = f32x16{};
    }
    const int i = x - x0;
    pv_tile<QT>(vo, sm.tile[i & 3], rh, i & 1, sm, A);
    wait_vm<kLoadsPerWave>();     // tile x + 2 is in LDS (x + 3 may stay in flight)
    // the piece's stores go after the wait, so that the wait never covers them
    if (x + 1 == cur.uend || x + 1 == x1) {
      const int first = max(x0, cur.ustart);
      const bool complete = first == cur.ustart && x + 1 == cur.uend;
      pv_finish<QT>(p, cur, rh, dh, A, sm.ml[i & 1][32 * rh + (lane & 31)], complete,
                    2 * wg + (first == x0 ? 0 : 1));
    }
    lds_barrier();
  }
  wait_vm<0>();                   // no load into LDS outlives the workgroup
}

}  // namespace

// Stream-K over 32-token tiles: workgroup w of W takes an equal share of the
// tile stream of all units; units wholly inside its share are finished
// here, the first and the last (when cut) leave partials in workspace slots
// 2w and 2w+1 for combine_lat_kernel.
template <int QT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void split_mla_ws_kernel(Params p) {
  resolve_scales(p);
  __shared__ Smem sm;
  const SkSched S = sk_schedule(p);
  const int wg = blockIdx.x, W = sk_waves_eff(S.T, gridDim.x);
  if (wg >= W) return;
  // the host keeps the tile stream under 2^31 tiles for this kernel
  const int x0 = (int)sk_wave_start(S.T, wg, W), x1 = (int)sk_wave_start(S.T, wg + 1, W);
  if (wave_id() < 4)
    score_role<QT>(p, S, x0, x1, sm);
  else
    pv_role<QT>(p, S, x0, x1, wg, sm);
}

hipError_t launch_split_mla_ws(int q_dtype, const Params& p, hipStream_t s) {
  if (p.sk_waves <= 0 || p.sk_shift != 5 || p.B > kSkMaxBatch || p.Dqk != kDqk || p.Dv != kDv || p.R > 64 ||
      !p.ws_lanes)
    return hipErrorInvalidValue;
  if (q_dtype == kBF16)
    hipLaunchKernelGGL((split_mla_ws_kernel<kBF16>), dim3(p.sk_waves), dim3(kThreads), 0, s, p);
  else if (q_dtype == kF16)
    hipLaunchKernelGGL((split_mla_ws_kernel<kF16>), dim3(p.sk_waves), dim3(kThreads), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
