// split_mla_ws.hip -- latent (MLA) split-KV decode with wave-specialised
// roles: one KV head's 576-wide rows, of which the first 512 entries are V,
// and up to 64 query rows; 16-bit or e4m3fn latent caches.
//
// vLLM `models/kimi_k3/nvidia/mla` page, MultiHeadLatentAttention: the decode
// branch of `_attention` runs multi-query attention of the absorbed queries
// over the latent cache rows [kv_c_normed | k_pe] (`forward_mqa`), and the
// kv_lora_rank-wide result is what `_v_up_proj` projects back -- so V is the
// leading kv_lora_rank entries of each K row.  The same page reads a uint8
// cache as e4m3fn (`_attn_read_kv_cache`) and accepts a quantised query for
// it.
//
// A workgroup of eight waves runs stream-K over tiles of 32 tokens (16-bit
// cache) or 64 tokens (fp8 cache), one workgroup per CU; either tile is
// 36 KB.  The tiles enter a four-slot LDS ring straight from HBM: each tile
// row goes in with buffer loads that write LDS (16 bytes per lane, no
// register staging), issued three tiles ahead.  The waves split the work by
// role, and the two roles work on neighbouring tiles in the same step:
//   score waves 0..3 (one per SIMD): wave rb computes the scores of query rows
//     16 rb .. + 15 against all tokens of tile t + 1 over all 576 dims,
//     S^T (tokens x 16 rows) = K . Q^T, as 16x16x32 MFMAs with the query
//     slice held in registers, runs the rows' online softmax, and leaves the
//     16-bit probabilities and the rows' rescale factors in LDS;
//   P.V waves 4..7 (one per SIMD): wave (rh, dh) takes rows 32 rh .. + 31 and
//     value dims 256 dh .. + 255 of tile t (of an fp8 tile: wave w takes all
//     64 rows and dims 128 w .. + 127): it rescales its accumulators and adds
//     O^T += V^T . P^T as 32x32x16 MFMAs with V^T from transposed LDS reads;
//     these waves also issue the tile loads.
// One barrier per step.  For a 16-bit tile the LDS serves 144 KB of K reads,
// 64 KB of V reads and 12 KB of probability traffic -- against about 290 KB
// read and 52 KB written when every wave did both products for its own rows.
// An fp8 tile holds twice the tokens at the same bytes.  Its V fragments
// are read as bytes and converted exactly to the 16-bit operand type in
// registers (every e4m3fn value is exact in bf16 and f16), and so are its K
// fragments for a 16-bit query.  With an fp8 query the scores run on the
// fp8 matrix instruction (v_mfma_f32_16x16x128_f8f6f4) on the bytes
// themselves: measured on random e4m3fn operands it sums its 128 products
// with relative errors up to ~1e-4 of the sum of their magnitudes (the
// 16-bit route is exact up to fp32 rounding), far below the quantisation of
// the fp8 inputs.  Where attention is peaky (large logits) the error reaches
// the output: against the same query as bf16 (the exact route) outputs
// differed by up to 3.9e-3 at an output rms of 0.14, a fifth of the
// fp8-cache parity bound.
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
constexpr int kQkSteps = kDqk / 32;           // 18 K steps of the score product
// 16-bit tile (32 tokens): two halves of 16 rows; a half holds the first
// 1024 bytes of its rows (dims 0 .. 511) at a 1024-byte pitch, then the last
// 128 bytes (the rope dims) at a 128-byte pitch.  The 16-byte chunks of a
// row are XOR-swizzled (swz_lo / swz_hi), so that K reads (sixteen rows, one
// chunk each), transposed V reads (four rows, 32 bytes each) and the row
// loads spread over the banks.
constexpr int kLoBytes = 1024, kHiBytes = 128;
constexpr int kHiOff = 16 * kLoBytes;
constexpr int kHalfBytes = 16 * (kLoBytes + kHiBytes);   // 18432
constexpr int kTileBytes = 2 * kHalfBytes;                // 36864
constexpr int kRing = 4;
constexpr int kLoadsPerWave = 9;              // 36 loads of 1 KB per tile, over 4 waves
// fp8 tile (64 tokens): the first 512 bytes of each row at a 512-byte pitch
// (32 KB, ring slot i & 3), and the 64 rope bytes of each row at a 64-byte
// pitch (4 KB, in a ring of three slots of its own, i % 3: a tile's rope
// part is dead once the score waves are through with it, a step before its
// V part).  Chunk swizzles swz_lo (low part) and swz8_hi (rope part).
constexpr int kLo8Row = 512, kHi8Row = 64;
constexpr int kLo8Slot = 64 * kLo8Row;       // 32768
constexpr int kHi8Slot = 64 * kHi8Row;       // 4096
constexpr int kHi8Ring = 3;

template <bool KV8>
struct Fmt {
  static constexpr int kTok = KV8 ? 64 : 32;  // tokens per tile
  static constexpr int kTB = kTok / 16;       // 16-token blocks per tile
  static constexpr int kShift = KV8 ? 6 : 5;
  static constexpr int kRingBytes = KV8 ? kRing * kLo8Slot + kHi8Ring * kHi8Slot : kRing * kTileBytes;
};

template <bool KV8>
struct Smem {
  uint8_t ring[Fmt<KV8>::kRingBytes];
  // probabilities (four 16-bit values) [parity][row block][16-token block][g / 2][n][g % 2]:
  // 16 bytes at [..][h][n] are tokens 16 tb + 8 h .. + 7 of row 16 rb + n
  uint2 p[2][4][Fmt<KV8>::kTB][2][16][2];
  float alpha[2][64];                         // per-row rescale of the P.V accumulators
  float2 ml[2][64];                           // (m, l) of rows whose piece ends at this tile
};
static_assert(sizeof(Smem<false>) <= 160 * 1024 && sizeof(Smem<true>) <= 160 * 1024, "LDS budget");

// Ring slot i of a workgroup's tiles: its low part (or the whole 16-bit
// tile) and, for an fp8 tile, its rope part.
template <bool KV8>
__device__ __forceinline__ uint8_t* slot_lo(Smem<KV8>& sm, int i) {
  return sm.ring + (i & 3) * (KV8 ? kLo8Slot : kTileBytes);
}
__device__ __forceinline__ uint8_t* slot_hi8(Smem<true>& sm, int i3) {
  return sm.ring + kRing * kLo8Slot + i3 * kHi8Slot;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
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
// fp8 tile: chunk c (0..31) of row r's low part sits at
// (c & ~15) | ((c & 15) ^ swz_lo(r)), as in the 16-bit tile (its rows are
// 512 bytes, also a multiple of the 256 bytes the banks span), and the
// 16-byte K reads take the same pattern as there.  The transposed V reads
// (bytes) take two neighbouring chunks (2c, 2c + 1) of eight rows 8k .. 8k + 7
// per 32 lanes: swz_lo of those rows differs in its bits 1..3, so each pair
// stays together and the eight pairs land on different banks.  Rope chunk
// c (0..3) of row r sits at c ^ swz8_hi(r): rope rows lie four to 256
// bytes, and swz8_hi separates the rows that a 16-byte read takes from one
// such line.
__device__ __forceinline__ int swz8_hi(int r) { return (r >> 2) & 3; }

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

// Transposed LDS read of bytes (ds_read_b64_tr_b8), measured on gfx950: in
// each group of 16 lanes, lane a + 2 j (a < 2, j < 8) supplies the address
// of eight bytes and lane 8 a + e receives byte e of lanes a, a + 2, ...,
// a + 14, in that order.
__device__ __forceinline__ uint2 lds_read_tr8(const uint8_t* addr) {
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(addr));
  return __builtin_bit_cast(uint2, v);
}

// Eight e4m3fn bytes -> eight 16-bit values of the operand type (exact).
template <int QT>
__device__ __forceinline__ uint4 fp8x8_to_16(uint2 w) {
  const uint2 lo = fp8x4_to_16<QT>(w.x), hi = fp8x4_to_16<QT>(w.y);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
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
template <bool KV8>
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
  u.tile0 = u.lo >> Fmt<KV8>::kShift;
  return u;
}

// ---------------------------------------------------------------- tile loads
// The P.V waves' load cursor: the next global tile to load, its unit and the
// page ids of its 16-row blocks (-1: nothing to read).  The page ids are
// read one step before the tile's loads are issued, so the scalar loads
// never hold up the issue.
template <bool KV8>
struct LoadCursor {
  UnitPos u;
  int t;
  int pid[Fmt<KV8>::kTB];
};

template <bool KV8>
__device__ __forceinline__ void fetch_page_ids(const Params& p, int x1, LoadCursor<KV8>& c) {
#pragma unroll
  for (int q = 0; q < Fmt<KV8>::kTB; ++q) c.pid[q] = -1;
  if (c.t >= x1) return;
  const int tok0 = (c.u.tile0 + (c.t - c.u.ustart)) << Fmt<KV8>::kShift;
  const const_i32* row = (const const_i32*)p.page_table + (int64_t)c.u.b * p.pps;
#pragma unroll
  for (int q = 0; q < Fmt<KV8>::kTB; ++q)
    if (tok0 + 16 * q < c.u.L) c.pid[q] = row[(tok0 + 16 * q) >> p.ps_shift];
}

// Move the cursor to tile t (the next one, or the first of the share).
template <bool KV8>
__device__ __forceinline__ void advance(const Params& p, const SkSched& S, int x1, int t, LoadCursor<KV8>& c) {
  c.t = t;
  if (t < x1 && t >= c.u.uend) c.u = locate<KV8>(p, S, t);
  fetch_page_ids<KV8>(p, x1, c);
}

// Per-lane parts of a P.V wave's tile loads, fixed for the kernel.
// 16-bit tile: the byte offset inside a row of the 16-byte chunk that lane l
// loads for low rows 4 a + pw (chunk l, swizzled so that it lands at its
// place), and the row and rope offset of the lane's rope load (rows
// 8 (pw & 1) + l / 8).  fp8 tile: the offset from the first of the two rows
// of a low-part load (row l / 32, chunk l % 32 swizzled; [i & 1] for the
// wave's load i, whose rows differ in bit 3), and from the first row of the
// wave's rope load (row l / 4, rope chunk l % 4 swizzled).
struct LoadLanes {
  int lo[4];
  int rope_row, rope_col;
};

template <bool KV8>
__device__ __forceinline__ LoadLanes load_lanes(const Params& p, int pw) {
  const int lane = threadIdx.x & 63;
  LoadLanes ll;
  if constexpr (KV8) {
    const int row_bytes = (int)p.k_slot;
    const int r7 = 2 * pw + (lane >> 5);       // row & 7 of the lane's low rows
#pragma unroll
    for (int a = 0; a < 2; ++a) ll.lo[a] = (lane >> 5) * row_bytes + 16 * ((lane & 31) ^ swz_lo(r7 + 8 * a));
    ll.lo[2] = ll.lo[3] = 0;
    ll.rope_row = lane >> 2;
    ll.rope_col = kLo8Row + 16 * ((lane & 3) ^ swz8_hi(lane >> 2));
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a) ll.lo[a] = 16 * ((lane & ~15) | ((lane & 15) ^ swz_lo(4 * a + pw)));
    ll.rope_row = 8 * (pw & 1) + (lane >> 3);
    ll.rope_col = kLoBytes + 16 * ((lane & 7) ^ swz_hi(ll.rope_row));
  }
  return ll;
}

// Issue this P.V wave's nine loads of the cursor's tile into ring slot `lo`
// (and `hi`, the rope slot of an fp8 tile).
// 16-bit tile: rows pw, pw + 4, ..., pw + 28 (one 1024-byte low part each;
// rows 4 k + pw lie in half k / 4) and rope block pw (rows 8 (pw & 1) .. + 7
// of half pw / 2).
// fp8 tile: low parts of rows 2 k, 2 k + 1 for k = pw + 4 i (i < 8; rows of
// 16-row block k / 8) and the rope parts of rows 16 pw .. + 15.
// The row offset goes in the scalar offset, so a tile whose rows are all
// visible needs no per-lane arithmetic; on a tile that crosses the
// sequence's visible span [lo, L) the rows outside read as zeros (an offset
// past the page), and so do pages with ids outside the cache and tiles past
// the share (empty resource).
template <bool KV8>
__device__ __forceinline__ void load_tile(const Params& p, const LoadCursor<KV8>& c, const LoadLanes& ll,
                                          uint32_t lo_lds, uint32_t hi_lds, int pw) {
  constexpr int kTB = Fmt<KV8>::kTB, kTok = Fmt<KV8>::kTok;
  constexpr int esz = KV8 ? 1 : 2;
  const int tok0 = (c.u.tile0 + (c.t - c.u.ustart)) << Fmt<KV8>::kShift;
  const uint32_t page_bytes = (uint32_t)(p.k_page * esz);
  const int row_bytes = (int)(p.k_slot * esz);
  const int head_off = (int)(c.u.kvh * p.k_head * esz);
  const int pmask = p.ps - 1;
  // the resource of 16-row block q (built from its scalar page id, so that
  // it stays in scalar registers)
  auto rs = [&](int pid) {
    const bool ok = (unsigned)pid < (unsigned)p.num_pages;
    return rsrc4((const uint8_t*)p.k + (ok ? (int64_t)pid * page_bytes : 0), ok ? page_bytes : 0u);
  };
  const bool whole = tok0 >= c.u.lo && tok0 + kTok <= c.u.L;
  const int lane = threadIdx.x & 63;
  if constexpr (KV8) {
    const i32x4 r0 = rs(c.pid[0]), r1 = rs(c.pid[1]), r2 = rs(c.pid[2]), r3 = rs(c.pid[3]);
    const i32x4 rp = pw == 0 ? r0 : pw == 1 ? r1 : pw == 2 ? r2 : r3;   // rope block pw
    if (whole) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = pw + 4 * i;                // rows 2 k, 2 k + 1 of block i / 2 (as pw < 4)
        const int soff = ((tok0 + 2 * k) & pmask) * row_bytes + head_off;
        load_to_lds(i < 2 ? r0 : i < 4 ? r1 : i < 6 ? r2 : r3, lo_lds + 1024 * k, ll.lo[i & 1], soff);
      }
      const int soff = ((tok0 + 16 * pw) & pmask) * row_bytes + head_off;
      load_to_lds(rp, hi_lds + 1024 * pw, ll.rope_row * row_bytes + ll.rope_col, soff);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = pw + 4 * i;
        const int tok = tok0 + 2 * k + (lane >> 5);
        const bool in = tok >= c.u.lo && tok < c.u.L;
        const int voff = in ? (tok & pmask) * row_bytes + head_off + ll.lo[i & 1] - (lane >> 5) * row_bytes
                            : (int)0x80000000u;
        load_to_lds(i < 2 ? r0 : i < 4 ? r1 : i < 6 ? r2 : r3, lo_lds + 1024 * k, voff, 0);
      }
      const int tok = tok0 + 16 * pw + ll.rope_row;
      const bool in = tok >= c.u.lo && tok < c.u.L;
      const int voff = in ? (tok & pmask) * row_bytes + head_off + ll.rope_col : (int)0x80000000u;
      load_to_lds(rp, hi_lds + 1024 * pw, voff, 0);
    }
  } else {
    const i32x4 r0 = rs(c.pid[0]), r1 = rs(c.pid[1]);
    if (whole) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int hf = k >> 2, rr = 4 * (k & 3) + pw;
        const int soff = ((tok0 + 16 * hf + rr) & pmask) * row_bytes + head_off;
        load_to_lds(hf ? r1 : r0, lo_lds + hf * kHalfBytes + rr * kLoBytes, ll.lo[k & 3], soff);
      }
      const int hf = pw >> 1;
      const int soff = ((tok0 + 16 * hf + 8 * (pw & 1)) & pmask) * row_bytes + head_off;
      load_to_lds(hf ? r1 : r0, lo_lds + hf * kHalfBytes + kHiOff + 8 * (pw & 1) * kHiBytes,
                  (ll.rope_row - 8 * (pw & 1)) * row_bytes + ll.rope_col, soff);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int hf = k >> 2, rr = 4 * (k & 3) + pw;
        const int tok = tok0 + 16 * hf + rr;
        const bool in = tok >= c.u.lo && tok < c.u.L;
        const int voff = in ? (tok & pmask) * row_bytes + head_off + ll.lo[k & 3] : (int)0x80000000u;
        load_to_lds(hf ? r1 : r0, lo_lds + hf * kHalfBytes + rr * kLoBytes, voff, 0);
      }
      const int hf = pw >> 1;
      const int tok = tok0 + 16 * hf + ll.rope_row;
      const bool in = tok >= c.u.lo && tok < c.u.L;
      const int voff = in ? (tok & pmask) * row_bytes + head_off + ll.rope_col : (int)0x80000000u;
      load_to_lds(hf ? r1 : r0, lo_lds + hf * kHalfBytes + kHiOff + 8 * (pw & 1) * kHiBytes, voff, 0);
    }
  }
}

// ---------------------------------------------------------------- score waves
struct QRegs {
  uint4 k[kQkSteps];   // row 16 rb + n, dims q_dim(s, g) .. + 8
};

// The dims that lane group g supplies for K step s of the score product:
// 32 s + 8 g .. + 8 over a 16-bit tile; over an fp8 tile, whose K fragments
// are read 16 bytes (two steps) at a time, 64 (s / 2) + 16 g + 8 (s % 2)
// .. + 8.  Either way the steps' dims cover all 576 once, and the K
// fragments take the same dims.
template <bool KV8>
__device__ __forceinline__ int q_dim(int s, int g) {
  return KV8 ? 64 * (s >> 1) + 16 * g + 8 * (s & 1) : 32 * s + 8 * g;
}

// Element offset of this lane's query row (zeros for rows >= R).
__device__ __forceinline__ int64_t q_lane_offset(const Params& p, const UnitPos& u, int rb, bool& ok) {
  const int lane = threadIdx.x & 63, n = lane & 15;
  const int row = 16 * rb + n;
  ok = row < p.R;
  return q_row_offset(p, u.b, u.kvh, ok ? row : 0) * kDqk;
}

// An fp8 query (Q8) is converted exactly to QT.
template <int QT, bool KV8, bool Q8>
__device__ __forceinline__ uint4 q_step(const Params& p, int64_t e, bool ok, int s) {
  const int64_t d = e + q_dim<KV8>(s, (threadIdx.x & 63) >> 4);
  if constexpr (Q8) {
    const uint2 raw = ok ? *(const uint2*)((const uint8_t*)p.q + d) : make_uint2(0, 0);
    return fp8x8_to_16<QT>(raw);
  } else {
    return ok ? *(const uint4*)((const uint16_t*)p.q + d) : make_uint4(0, 0, 0, 0);
  }
}

// An fp8 query over an fp8 cache keeps its bytes: the scores then run on the
// fp8 matrix instructions (16x16x128), and lane group g supplies bytes
// 16 h .. + 15 of dims 128 s + 32 g .. + 32 in k[2 s + h] (s < 4), and of the
// rope dims 512 + 32 g .. + 32 in k[8 + h] (zeros for g >= 2).
constexpr int kQ8Regs = 10;

__device__ __forceinline__ uint4 q8_part(const Params& p, int64_t e, bool ok, int k) {
  const int g = (threadIdx.x & 63) >> 4, s = k >> 1, h = k & 1;
  const bool live = ok && (s < 4 || g < 2);
  return live ? *(const uint4*)((const uint8_t*)p.q + e + 128 * s + 32 * g + 16 * h) : make_uint4(0, 0, 0, 0);
}

template <int QT, bool KV8, bool Q8>
__device__ __forceinline__ void load_q(const Params& p, const UnitPos& u, int rb, QRegs& Q) {
  bool ok;
  const int64_t e = q_lane_offset(p, u, rb, ok);
  if constexpr (KV8 && Q8) {
#pragma unroll
    for (int k = 0; k < kQ8Regs; ++k) Q.k[k] = q8_part(p, e, ok, k);
  } else {
#pragma unroll
    for (int s = 0; s < kQkSteps; ++s) Q.k[s] = q_step<QT, KV8, Q8>(p, e, ok, s);
  }
}

// The next unit's query slice, loaded a step before the unit starts.  A
// 16-bit query over a 16-bit cache: all of it.  An fp8 query: its bytes,
// converted when the unit starts.  A 16-bit query over an fp8 cache (whose
// score step holds more registers): the first half, the second half being
// loaded when the unit starts -- its first use is 36 MFMAs into the step.
template <bool KV8, bool Q8>
struct QNext {
  static constexpr int kPre = KV8 && !Q8 ? kQkSteps / 2 : KV8 ? kQ8Regs : kQkSteps;
  uint4 k[Q8 && !KV8 ? 1 : kPre];
  uint2 raw[Q8 && !KV8 ? kQkSteps : 1];
};

template <int QT, bool KV8, bool Q8>
__device__ __forceinline__ void prefetch_q(const Params& p, const UnitPos& u, int rb, QNext<KV8, Q8>& N) {
  bool ok;
  const int64_t e = q_lane_offset(p, u, rb, ok);
#pragma unroll
  for (int s = 0; s < QNext<KV8, Q8>::kPre; ++s) {
    if constexpr (KV8 && Q8)
      N.k[s] = q8_part(p, e, ok, s);
    else if constexpr (Q8)
      N.raw[s] = ok ? *(const uint2*)((const uint8_t*)p.q + e + q_dim<KV8>(s, (threadIdx.x & 63) >> 4))
                    : make_uint2(0, 0);
    else
      N.k[s] = q_step<QT, KV8, false>(p, e, ok, s);
  }
}

template <int QT, bool KV8, bool Q8>
__device__ __forceinline__ void take_q(const Params& p, const UnitPos& u, int rb, const QNext<KV8, Q8>& N,
                                       QRegs& Q) {
  constexpr int kPre = QNext<KV8, Q8>::kPre;
#pragma unroll
  for (int s = 0; s < kPre; ++s) {
    if constexpr (Q8 && !KV8)
      Q.k[s] = fp8x8_to_16<QT>(N.raw[s]);
    else
      Q.k[s] = N.k[s];
  }
  if constexpr (kPre < kQkSteps && !(KV8 && Q8)) {
    bool ok;
    const int64_t e = q_lane_offset(p, u, rb, ok);
#pragma unroll
    for (int s = kPre; s < kQkSteps; ++s) Q.k[s] = q_step<QT, KV8, Q8>(p, e, ok, s);
  }
}

// Score step for tile t (low slot tl, rope slot th of an fp8 tile): S^T of
// rows 16 rb .. + 15 against the tile's tokens over all 576 dims, then the
// online softmax of those rows.  16-bit tile: K fragment (tb, s) of lane
// (n, g) is chunk 4 s + g of row 16 tb + n (steps 16 and 17: rope chunks g
// and 4 + g).  fp8 tile: it is bytes 8 (g % 2) .. + 7 of chunk 2 s + g / 2
// of row 16 tb + n (steps 16 and 17: rope chunk 2 (s - 16) + g / 2),
// converted to QT.  The reads run kAhead MFMAs ahead.  Lane (n, g) ends with
// tokens 16 tb + 4 g + i of row n; the wave keeps the row's running
// reference max m (log2 units) and its sum l of the rounded probabilities,
// and leaves in LDS the probabilities (16-bit) and the factor alpha by which
// the P.V waves rescale their accumulators.
struct RowState {
  float m, l;
};

template <int QT, bool KV8, bool Q8>
__device__ __forceinline__ void score_tile(const Params& p, const UnitPos& u, const RowVis& vis, int lo_last,
                                           int mask_from, const QRegs& Q, const uint8_t* tl, const uint8_t* th,
                                           int rb, int par, int t, Smem<KV8>& sm, RowState& st) {
  constexpr int kTB = Fmt<KV8>::kTB, kTok = Fmt<KV8>::kTok;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  f32x4 s4[kTB];
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) s4[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (KV8 && Q8) {
    // fp8 query and cache: S^T on v_mfma_f32_16x16x128_f8f6f4, K and Q as
    // bytes.  K fragment (tb, s) of lane (n, g): dims 128 s + 32 g .. + 32 of
    // row 16 tb + n, i.e. chunks 8 s + 2 g + h (h = 0, 1), chunk c at
    // 16 (c / 16) + ((c % 16) ^ swz_lo(n)); s = 4: rope chunks 2 g + h of
    // lanes g < 2 (zeros for the others, whose query bytes are zeros).
    int kb8[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int h = 0; h < 2; ++h) kb8[a][h] = n * kLo8Row + 16 * ((8 * a + 2 * g + h) ^ swz_lo(n));
    const int hb[2] = {n * kHi8Row + 16 * ((2 * (g & 1)) ^ swz8_hi(n)),
                       n * kHi8Row + 16 * ((2 * (g & 1) + 1) ^ swz8_hi(n))};
    auto frag = [&](int s, int tb) {
      uint4 a, b;
      if (s < 4) {
        a = *(const uint4*)(tl + tb * 16 * kLo8Row + kb8[s & 1][0] + 256 * (s >> 1));
        b = *(const uint4*)(tl + tb * 16 * kLo8Row + kb8[s & 1][1] + 256 * (s >> 1));
      } else {
        a = *(const uint4*)(th + tb * 16 * kHi8Row + hb[0]);
        b = *(const uint4*)(th + tb * 16 * kHi8Row + hb[1]);
        if (g >= 2) a = b = make_uint4(0, 0, 0, 0);
      }
      return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    };
    auto qop = [&](int s) {
      const uint4 a = Q.k[2 * s], b = Q.k[2 * s + 1];
      return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    };
    constexpr int kSteps8 = 5;
    i32x8 kf[2][kTB];
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) kf[0][tb] = frag(0, tb);
#pragma unroll
    for (int s = 0; s < kSteps8; ++s) {
      if (s + 1 < kSteps8) {
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb) kf[(s + 1) & 1][tb] = frag(s + 1, tb);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb)
        s4[tb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf[s & 1][tb], qop(s), s4[tb], 0, 0, 0, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if constexpr (KV8) {
    // fragment pair (tb, sp) of lane (n, g): the 16 bytes of chunk 4 sp + g
    // of row 16 tb + n, i.e. dims 64 sp + 16 g .. + 16 -- K steps 2 sp and
    // 2 sp + 1 (sp = 8: rope chunk g).  Chunk 4 sp + g sits at
    // 16 (sp / 4) + ((4 (sp % 4) + g) ^ swz_lo(n)): per-lane offsets for
    // sp % 4, and 256 (sp / 4) and 8192 tb as immediates.
    int kb[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) kb[a] = n * kLo8Row + 16 * ((4 * a + g) ^ swz_lo(n));
    const int hb = n * kHi8Row + 16 * (g ^ swz8_hi(n));
    auto frag = [&](int j) {
      const int sp = j / kTB, tb = j % kTB;
      if (sp < 8) return *(const uint4*)(tl + tb * 16 * kLo8Row + kb[sp & 3] + 256 * (sp >> 2));
      return *(const uint4*)(th + tb * 16 * kHi8Row + hb);
    };
    // 36 reads of 16 bytes, each converted into the operands of two MFMAs
    // (K steps 2 sp and 2 sp + 1 of token block tb).  Step sp's four reads
    // are issued a block ahead, and the four blocks' MFMAs alternate, so
    // that no MFMA waits for the one before it; the scheduling barriers keep
    // the compiler from regrouping the blocks.
    constexpr int kPairs = kQkSteps / 2;
    uint4 kf[2][kTB];
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) kf[0][tb] = frag(tb);
#pragma unroll
    for (int sp = 0; sp < kPairs; ++sp) {
      if (sp + 1 < kPairs) {
#pragma unroll
        for (int tb = 0; tb < kTB; ++tb) kf[(sp + 1) & 1][tb] = frag((sp + 1) * kTB + tb);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb)
        s4[tb] = mfma_k32<QT>(fp8x8_to_16<QT>(make_uint2(kf[sp & 1][tb].x, kf[sp & 1][tb].y)), Q.k[2 * sp],
                              s4[tb]);
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb)
        s4[tb] = mfma_k32<QT>(fp8x8_to_16<QT>(make_uint2(kf[sp & 1][tb].z, kf[sp & 1][tb].w)),
                              Q.k[2 * sp + 1], s4[tb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
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
  }
  // ---- online softmax of row n over tokens 16 tb + 4 g + i
  float x[kTB][4];
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[tb][i] = s4[tb][i] * p.qk_scale_log2;
  // tiles that hold a token invisible to some row (window, draft mask, the
  // sequence's ends) mask; the others are visible to every row
  const int tok0 = (u.tile0 + (t - u.ustart)) << Fmt<KV8>::kShift;
  if (tok0 < lo_last || tok0 + kTok > mask_from) {
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[tb][i] = vis(tok0 + 16 * tb + 4 * g + i, u.L) ? x[tb][i] : kNegInf;
  }
  float tmax = kNegInf;
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb)
    tmax = fmaxf(tmax, fmaxf(fmaxf(x[tb][0], x[tb][1]), fmaxf(x[tb][2], x[tb][3])));
  tmax = max_across_rows(tmax);
  // the reference moves only when the tile max passes it by kSlack
  const bool bump = tmax > st.m + kSlack;
  const float m_new = bump ? tmax : st.m;
  const float m_ref = m_new == kNegInf ? 0.f : m_new;
  const float alpha = bump ? __builtin_amdgcn_exp2f(st.m - m_ref) : 1.f;
  float tsum = 0.f;
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) {
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
template <int QT, bool KV8, bool Q8>
__device__ __forceinline__ void score_role(const Params& p, const SkSched& S, int x0, int x1, Smem<KV8>& sm) {
  const int rb = wave_id(), lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int row = 16 * rb + n;
  UnitPos cur = locate<KV8>(p, S, x0), nxt = cur;
  QRegs Q;
  QNext<KV8, Q8> Qn;
  load_q<QT, KV8, Q8>(p, cur, rb, Q);
  RowVis vis{};
  int lo_last = 0, mask_from = 0;
  RowState st{kNegInf, 0.f};
  int i3 = 0;                                  // rope slot of the next tile (fp8)
  auto step = [&](int t) {
    if (t >= cur.uend) {
      cur = nxt;
      take_q<QT, KV8, Q8>(p, cur, rb, Qn, Q);
    }
    if (t == x0 || t == cur.ustart) {
      vis = row_vis(p, cur.b, cur.L, row < p.R ? row : 0);
      lo_last = p.window > 0 ? cur.L - p.window : INT32_MIN;
      mask_from = (p.Tq > 1 && p.mask != nullptr) ? cur.L - p.Tq : cur.L;
      st.m = kNegInf;
      st.l = 0.f;
    }
    if (t + 1 < x1 && t + 1 >= cur.uend) {
      nxt = locate<KV8>(p, S, t + 1);
      prefetch_q<QT, KV8, Q8>(p, nxt, rb, Qn);
    }
    const int i = t - x0;
    const uint8_t* th = nullptr;
    if constexpr (KV8) {
      th = slot_hi8(sm, i3);
      i3 = i3 == kHi8Ring - 1 ? 0 : i3 + 1;
    }
    score_tile<QT, KV8, Q8>(p, cur, vis, lo_last, mask_from, Q, slot_lo(sm, i), th, rb, i & 1, t, sm, st);
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
// 16-bit tile: wave (rh, dh) holds dims 256 dh + 32 j + 8 (i / 4) + 4 h + i % 4
// of row 32 rh + (lane % 32) in o[j].  fp8 tile: wave w holds dims
// 128 w + 32 jd + 8 (i / 4) + 4 h + i % 4 of row 32 rb + (lane % 32) in
// o[4 rb + jd] -- all 64 rows and a quarter of the dims, so that each V byte
// is converted once per tile.
struct PvState {
  f32x16 o[8];
};

// Per-lane LDS offsets of the transposed V reads.
// 16-bit tile: read (cc, j) of lane (s, G) takes row 8 h + 4 cc + s / 4 of a
// half tile, dims 256 dh + 32 j + 16 (G % 2) + 4 (s % 4) .. + 4; the XOR of
// the chunk index with the row's swizzle only touches its low four bits, so
// j = a + 4 (a < 4) is a 256-byte step from j = a.
// fp8 tile: read jd of wave w's lane (s, G) takes row 8 h + s / 2 of a
// 16-row block, dims 128 w + 32 jd + 16 (G % 2) + 8 (s % 2) .. + 8, i.e. byte
// 8 (s % 2) of chunk 8 w + 2 jd + G % 2; with tr8 lane (s, G) then holds dim
// 128 w + 32 jd + (lane % 32) of tokens 8 h .. + 7.
struct VOff {
  int o[8];
};

template <bool KV8>
__device__ __forceinline__ VOff v_offsets(int dh, int w) {
  const int lane = threadIdx.x & 63, s = lane & 15, G = lane >> 4, h = lane >> 5;
  VOff v;
  if constexpr (KV8) {
    const int rr = 8 * h + (s >> 1);
#pragma unroll
    for (int jd = 0; jd < 4; ++jd) {
      const int c = 8 * w + 2 * jd + (G & 1);
      v.o[jd] = rr * kLo8Row + 16 * ((c & ~15) | ((c & 15) ^ swz_lo(rr))) + 8 * (s & 1);
    }
    v.o[4] = v.o[5] = v.o[6] = v.o[7] = 0;
  } else {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const int rr = 8 * h + 4 * cc + (s >> 2);
      const int e = 2 * (G & 1) + ((s & 3) >> 1);   // chunk bits 0..1
#pragma unroll
      for (int a = 0; a < 4; ++a) v.o[4 * cc + a] = lo_chunk(rr, 32 * dh + 4 * a + e) + 8 * (s & 1);
    }
  }
  return v;
}

// P.V step for tile x (ring slot tl): rescale by the rows' alpha, then
// O^T += V^T . P^T as 32x32x16 MFMAs, token step ts outer so that
// consecutive MFMAs feed different accumulators.  K index 8 h + c of token
// step ts is token 16 ts + 8 h + c in both operands.
template <int QT, bool KV8>
__device__ __forceinline__ void pv_tile(const VOff& vo, const uint8_t* tl, int rh, int par, Smem<KV8>& sm,
                                        PvState& A) {
  constexpr int kTB = Fmt<KV8>::kTB;
  const int lane = threadIdx.x & 63, col = lane & 31, h = lane >> 5;
  const int n = col & 15;
  if constexpr (KV8) {
    // both 32-row blocks: each converted V fragment feeds two MFMAs
    const float al0 = sm.alpha[par][col], al1 = sm.alpha[par][32 + col];
    uint4 pw[2][kTB];
#pragma unroll
    for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
      for (int ts = 0; ts < kTB; ++ts) pw[rb2][ts] = *(const uint4*)&sm.p[par][2 * rb2 + (col >> 4)][ts][h][n][0];
    auto vread = [&](int ts, int jd) { return lds_read_tr8(tl + ts * 16 * kLo8Row + vo.o[jd]); };
    // token step ts: four reads (one per 32-dim block) issued a step ahead,
    // then eight MFMAs on different accumulators
    uint2 vf[2][4];
#pragma unroll
    for (int jd = 0; jd < 4; ++jd) vf[0][jd] = vread(0, jd);
    if (__builtin_amdgcn_ballot_w64(al0 != 1.f || al1 != 1.f) != 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        A.o[j] *= al0;
        A.o[4 + j] *= al1;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ts = 0; ts < kTB; ++ts) {
      if (ts + 1 < kTB) {
#pragma unroll
        for (int jd = 0; jd < 4; ++jd) vf[(ts + 1) & 1][jd] = vread(ts + 1, jd);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jd = 0; jd < 4; ++jd) {
        const uint4 a = fp8x8_to_16<QT>(vf[ts & 1][jd]);
        A.o[jd] = mfma_32x32<QT>(a, pw[0][ts], A.o[jd]);
        A.o[4 + jd] = mfma_32x32<QT>(a, pw[1][ts], A.o[4 + jd]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    const int rb = 2 * rh + (col >> 4);
    const float alpha = sm.alpha[par][32 * rh + col];
    uint4 pw[kTB];
#pragma unroll
    for (int ts = 0; ts < kTB; ++ts) pw[ts] = *(const uint4*)&sm.p[par][rb][ts][h][n][0];
    auto vread = [&](int q) {
      const int ts = q >> 3, jb = q & 7;
      const int o = ts * kHalfBytes + 256 * (jb >> 2);
      const uint2 a = lds_read_tr16(tl + o + vo.o[jb & 3]);
      const uint2 b = lds_read_tr16(tl + o + vo.o[4 + (jb & 3)]);
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
}

// The normalised output rows (the unit was whole in this share) or the
// partial (m, l, o) in workspace slot `slot`.  A slot holds 64 (m, l) rows
// and the accumulators in the 16-bit tile's P.V register order -- element
// (j, 4 q + e) of lane l of wave (rh, dh) at float
// (((2 rh + dh) * 32 + 4 j + q) * 64 + l) * 4 + e -- so that every store
// instruction writes 1 KB contiguously.  Row block rh of this wave: its
// accumulators acc[k] hold the dims 256 dh + 32 (j0 + k) ..; write_ml: this
// wave writes the rows' (m, l).
template <int QT, int NJ>
__device__ __forceinline__ void finish_rows(const Params& p, const UnitPos& u, int rh, int dh, int j0,
                                            const f32x16* acc, float2 ml, bool complete, int64_t slot,
                                            bool write_ml) {
  const int lane = threadIdx.x & 63, col = lane & 31, h = lane >> 5;
  const int row = 32 * rh + col;
  if (row >= p.R) return;
  if (complete) {
    float num = 1.f, den = ml.y;
    if (p.sinks != nullptr) {
      const float sk = p.sinks[u.kvh * p.G + row % p.G] * kLog2e;
      const float Mf = fmaxf(ml.x, sk);
      num = ml.x == kNegInf ? 0.f : exp2f(ml.x - Mf);
      den = ml.y * num + exp2f(sk - Mf);
    }
    const float inv = den > 0.f ? p.out_scale * num / den : 0.f;
    const int64_t ob = q_row_offset(p, u.b, u.kvh, row) * kDv + 256 * dh + 32 * j0 + 4 * h;
#pragma unroll
    for (int k = 0; k < NJ; ++k)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        store_out4<QT>(p, ob + 32 * k + 8 * q, acc[k][4 * q] * inv, acc[k][4 * q + 1] * inv,
                       acc[k][4 * q + 2] * inv, acc[k][4 * q + 3] * inv);
  } else {
    float* o = p.ws_o + (slot * 4 + 2 * rh + dh) * (32 * 64 * 4) + 4 * lane + 4 * j0 * 256;
#pragma unroll
    for (int k = 0; k < NJ; ++k)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(float4*)(o + (4 * k + q) * 256) =
            make_float4(acc[k][4 * q], acc[k][4 * q + 1], acc[k][4 * q + 2], acc[k][4 * q + 3]);
    if (write_ml && h == 0) p.ws_ml[slot * 64 + row] = ml;
  }
}

// 16-bit tile: wave (rh, dh), one row block; fp8 tile: wave w, both row
// blocks, dims 128 w .. + 127 (dh = w / 2, j0 = 4 (w % 2)).
template <int QT, bool KV8>
__device__ __forceinline__ void pv_finish(const Params& p, const UnitPos& u, int rh, int dh, int w,
                                          const PvState& A, float2 ml0, float2 ml1, bool complete,
                                          int64_t slot) {
  if constexpr (KV8) {
    finish_rows<QT, 4>(p, u, 0, w >> 1, 4 * (w & 1), &A.o[0], ml0, complete, slot, w == 0);
    finish_rows<QT, 4>(p, u, 1, w >> 1, 4 * (w & 1), &A.o[4], ml1, complete, slot, w == 0);
  } else {
    finish_rows<QT, 8>(p, u, rh, dh, 0, &A.o[0], ml0, complete, slot, dh == 0);
  }
}

template <int QT, bool KV8>
__device__ __forceinline__ void pv_role(const Params& p, const SkSched& S, int x0, int x1, int wg, Smem<KV8>& sm) {
  const int pwv = wave_id() - 4, rh = pwv >> 1, dh = pwv & 1;
  const int lane = threadIdx.x & 63;
  const VOff vo = v_offsets<KV8>(dh, pwv);
  const LoadLanes ll = load_lanes<KV8>(p, pwv);
  // loads run three tiles ahead of the P.V step
  LoadCursor<KV8> lc;
  lc.u = locate<KV8>(p, S, x0);
  advance<KV8>(p, S, x1, x0, lc);
  int i3 = 0;                                  // rope slot of the next tile to load (fp8)
  auto issue = [&]() {
    const int i = lc.t - x0;
    uint32_t hi = 0;
    if constexpr (KV8) {
      hi = lds_addr(slot_hi8(sm, i3));
      i3 = i3 == kHi8Ring - 1 ? 0 : i3 + 1;
    }
    load_tile<KV8>(p, lc, ll, lds_addr(slot_lo(sm, i)), hi, pwv);
    advance<KV8>(p, S, x1, lc.t + 1, lc);
  };
  issue();
  issue();
  issue();
  wait_vm<2 * kLoadsPerWave>();   // tile x0 is in LDS
  lds_barrier();
  wait_vm<kLoadsPerWave>();       // tile x0 + 1 is in LDS
  lds_barrier();
  UnitPos cur = locate<KV8>(p, S, x0);
  PvState A;
#pragma unroll
  for (int j = 0; j < 8; ++j) A.o[j] = f32x16{};
  for (int x = x0; x < x1; ++x) {
    issue();                      // tile x + 3
    if (x >= cur.uend) {
      cur = locate<KV8>(p, S, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) A.o[j] = f32x16{};
    }
    const int i = x - x0;
    pv_tile<QT, KV8>(vo, slot_lo(sm, i), rh, i & 1, sm, A);
    wait_vm<kLoadsPerWave>();     // tile x + 2 is in LDS (x + 3 may stay in flight)
    // the piece's stores go after the wait, so that the wait never covers them
    if (x + 1 == cur.uend || x + 1 == x1) {
      const int first = max(x0, cur.ustart);
      const bool complete = first == cur.ustart && x + 1 == cur.uend;
      const float2 ml0 = sm.ml[i & 1][(KV8 ? 0 : 32 * rh) + (lane & 31)];
      const float2 ml1 = KV8 ? sm.ml[i & 1][32 + (lane & 31)] : ml0;
      pv_finish<QT, KV8>(p, cur, rh, dh, pwv, A, ml0, ml1, complete, 2 * wg + (first == x0 ? 0 : 1));
    }
    lds_barrier();
  }
  wait_vm<0>();                   // no load into LDS outlives the workgroup
}

}  // namespace

// Stream-K over tiles of 32 (16-bit cache) or 64 (fp8 cache) tokens:
// workgroup w of W takes an equal share of the tile stream of all units;
// units wholly inside its share are finished here, the first and the last
// (when cut) leave partials in workspace slots 2w and 2w+1 for
// combine_lat_kernel.  QT: operand and output type; KV8: fp8 cache; Q8:
// fp8 query.
template <int QT, bool KV8, bool Q8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void split_mla_ws_kernel(Params p) {
  resolve_scales(p);
  __shared__ Smem<KV8> sm;
  const SkSched S = sk_schedule(p);
  const int wg = blockIdx.x, W = sk_waves_eff(S.T, gridDim.x);
  if (wg >= W) return;
  // the host keeps the tile stream under 2^31 tiles for this kernel
  const int x0 = (int)sk_wave_start(S.T, wg, W), x1 = (int)sk_wave_start(S.T, wg + 1, W);
  if (wave_id() < 4)
    score_role<QT, KV8, Q8>(p, S, x0, x1, sm);
  else
    pv_role<QT, KV8>(p, S, x0, x1, wg, sm);
}

template <int QT, bool KV8, bool Q8>
hipError_t launch_ws(const Params& p, hipStream_t s) {
  hipLaunchKernelGGL((split_mla_ws_kernel<QT, KV8, Q8>), dim3(p.sk_waves), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

// 16-bit query and cache; 16-bit query and fp8 cache; fp8 query and cache
// (bf16 operands and output).
hipError_t launch_split_mla_ws(int q_dtype, int kv_dtype, const Params& p, hipStream_t s) {
  const bool kv8 = kv_dtype == kFP8;
  if (p.sk_waves <= 0 || p.sk_shift != (kv8 ? Fmt<true>::kShift : Fmt<false>::kShift) || p.B > kSkMaxBatch ||
      p.Dqk != kDqk || p.Dv != kDv || p.R > 64 || !p.ws_lanes)
    return hipErrorInvalidValue;
  if (kv8) {
    if (q_dtype == kFP8) return launch_ws<kBF16, true, true>(p, s);
    if (q_dtype == kBF16) return launch_ws<kBF16, true, false>(p, s);
    if (q_dtype == kF16) return launch_ws<kF16, true, false>(p, s);
    return hipErrorInvalidValue;
  }
  if (q_dtype != kv_dtype) return hipErrorInvalidValue;
  if (q_dtype == kBF16) return launch_ws<kBF16, false, false>(p, s);
  if (q_dtype == kF16) return launch_ws<kF16, false, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
