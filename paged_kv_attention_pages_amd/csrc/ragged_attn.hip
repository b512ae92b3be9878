// ragged_attn.hip -- attention over a ragged (non-paged) batch with its
// log-sum-exp, on the gfx950 matrix cores: the prefill-side attention whose
// (output, lse) pairs the chunked-prefill merge combines.
//
// vllm-omni TRTLLM diffusion backend page: `trtllm_ragged_attention_deepseek`
// takes queries, keys and values packed by `cum_seq_lens_q` /
// `cum_seq_lens_kv`, `is_causal`, and `bmm1_scale` as the softmax scale.
// vLLM Kimi-K3 MLA page, chunked prefill: `run_prefill_new_tokens` (causal
// over the new tokens) and `_compute_prefill_context` (over the cached
// context) each return (output, lse), merged by `merge_attn_states`.
//
// Sequence s owns query rows [cu_q[s], cu_q[s+1]) and key/value rows
// [cu_k[s], cu_k[s+1]); query head h reads KV head h / (Hq / Hkv).  Query i
// of a sequence (Lq queries, Lk keys) sees key j < Lk, and, when causal,
// only j <= i + Lk - Lq: the queries are the last Lq positions of the key
// sequence (for the new-token attention Lq == Lk, the plain causal mask).
//
// A workgroup of eight waves takes 32 consecutive queries per wave of one
// (sequence, query head) -- a query block -- or, for causal calls, two
// blocks of the same pair one after the other.  It loads each tile of 8
// keys per wave of K and V once -- 16-byte loads spread over its threads,
// into registers and then into a two-stage LDS ring -- and every wave reads
// its matrix operands from LDS, with the key tokens on the M side of both
// products as in the decode kernels.  The output is normalised in the kernel
// (no split).
#include "kernels.h"
#include "pkv_device.h"

namespace pkv {

namespace {

constexpr float kNegInfR = -__builtin_inff();
constexpr float kLn2 = 0.6931471805599453f;
// a wave takes kSub sub-blocks of 16 queries (one per MFMA column block)
// against each K/V tile its workgroup loads
constexpr int kSub = 2;
constexpr int kQueriesPerWave = 16 * kSub;

typedef short rs16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) rs16x4 lds_rs16x4;

// Transposed LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, lane
// a + 4 j supplies the address of four 16-bit elements, and lane 4 a + e
// receives element e of lanes a, a + 4, a + 8, a + 12, in that order.
__device__ __forceinline__ uint2 lds_tr16(const uint8_t* addr) {
  const rs16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_rs16x4*)(addr));
  return __builtin_bit_cast(uint2, v);
}

// Workgroup barrier that orders LDS only (the global prefetch stays in
// flight across it).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// 16-byte chunk c of key row r sits at chunk c ^ (r mod 8) of the row's LDS
// slot, so the K fragment reads (16 rows, one chunk) and the transposed V
// reads (16 rows, 32 bytes) spread over the banks.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7); }

// Maxima of finite-or-minus-infinity scores.  The IEEE-mode lowering of
// fmaxf quiets each operand with an extra v_max_f32 x, x first; these take
// one instruction per two or three operands.
__device__ __forceinline__ float vmax2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// The maximum over the four 16-lane row groups (lanes n, n + 16, n + 32,
// n + 48 hold the same query row).
__device__ __forceinline__ float row_max4(float x) {
  float2 a = row_partner16(x);
  x = vmax2(a.x, a.y);
  a = row_partner32(x);
  return vmax2(a.x, a.y);
}

// Online-softmax state of one 16-query sub-block: the reference max (log2
// units), the O^T accumulators, and lsum = P . ones, i.e. every element of
// lsum holds the lane's row sum of the rounded probabilities (the matrix
// cores add them, in the same products as the V sums).
template <int DV>
struct RAcc {
  float m;
  f32x4 o[DV / 16];
  f32x4 lsum;
};

}  // namespace

// One query block (32 NW queries of a (sequence, head)) on a workgroup of
// NW waves: the workgroup loads each 8 NW-key tile of K and V once (16-byte
// loads spread over its threads, straight into registers, then into a
// two-stage LDS ring), and every wave reads its matrix operands from LDS.
// Wave w holds queries 32 w .. 32 w + 31 as two 16-query sub-blocks.  Per
// tile, 32 keys at a time, and sub-block:
//   S^T (2 x 16 keys x 16 queries) = K . Q^T   -- 16x16x32 MFMAs from LDS
//   online softmax of the 32 keys per lane
//   O^T (Dv x 16 queries) += V^T . P^T          -- 16x16x32 MFMAs, V^T by
//                                                  transposed LDS reads
// The MFMA contraction index 8 g + c of P.V stands for key 4 g + c of the
// first 16-key block (c < 4) or 16 + 4 g + c - 4 of the second: the order in
// which the lane holds its scores, and the order of the two transposed reads.
template <int DQK, int DV, int NW>
constexpr int ragged_stage_bytes() { return 8 * NW * (DQK + DV) * 2; }

template <int QT, int DQK, int DV, int NW>
__device__ __forceinline__ void ragged_item(const RaggedParams& p, uint8_t* lds, int pair, int qblk) {
  constexpr int kThreadsWg = 64 * NW, kQueriesPerWg = NW * kQueriesPerWave;
  constexpr int KSTEPS = DQK / 32, DT = DV / 16;
  constexpr int KC = DQK / 8, VC = DV / 8;              // 16-byte chunks per row
  constexpr int KROW = DQK * 2, VROW = DV * 2;          // LDS bytes per key row
  constexpr int TK = 8 * NW;                            // keys per tile (halves of 32)
  constexpr int KBYTES = TK * KROW, STAGE = KBYTES + TK * VROW;
  constexpr int KI = TK * KC / kThreadsWg, NCH = TK * (KC + VC) / kThreadsWg;  // chunks per thread
  static_assert(TK * KC % kThreadsWg == 0 && TK * VC % kThreadsWg == 0, "whole K and V loads per thread");
  static_assert(STAGE == ragged_stage_bytes<DQK, DV, NW>(), "stage size");
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane((int)(tid >> 6));
  const int s = pair / p.Hq, h = pair - s * p.Hq, kvh = h / p.G;
  // sequence bounds, clamped to the tensors so that any cu_seqlens stay in bounds
  const int q0 = min(max(p.cu_q[s], 0), p.total_q), q1 = min(max(p.cu_q[s + 1], q0), p.total_q);
  const int k0 = min(max(p.cu_k[s], 0), p.total_k), k1 = min(max(p.cu_k[s + 1], k0), p.total_k);
  const int Lq = q1 - q0, Lk = k1 - k0;
  const int Lrun = min(Lq, p.max_q_len);   // queries computed (the rest stay unwritten)
  const int qwg = qblk * kQueriesPerWg;
  if (qwg >= Lrun) return;                 // whole workgroup: no barrier is left waiting
  const int off = p.causal ? Lk - Lq : 0;  // query i sees keys < i + 1 + off (causal)
  const int i0 = qwg + kQueriesPerWave * w;
  const bool has_rows = i0 < Lrun;         // wave-uniform; a wave without rows still loads
  int lim[kSub], lim_lo[kSub];
  bool row_ok[kSub];
#pragma unroll
  for (int b = 0; b < kSub; ++b) {
    const int i = i0 + 16 * b + n;
    row_ok[b] = i < Lrun;
    lim[b] = p.causal ? min(Lk, max(i + 1 + off, 0)) : Lk;
    lim_lo[b] = p.causal ? min(Lk, max(i0 + 16 * b + 1 + off, 0)) : Lk;
  }
  // one past the last key the wave's (the workgroup's) rows see
  const int kend_w = p.causal ? min(Lk, max(min(i0 + kQueriesPerWave, Lrun) + off, 0)) : Lk;
  const int kend = p.causal ? min(Lk, max(min(qwg + kQueriesPerWg, Lrun) + off, 0)) : Lk;
  const int nt = (kend + TK - 1) / TK;
  // Q^T operands of the rows (zeros past the computed queries)
  uint4 qb[kSub][KSTEPS];
#pragma unroll
  for (int b = 0; b < kSub; ++b) {
    const uint16_t* qrow =
        (const uint16_t*)p.q + ((int64_t)(q0 + (row_ok[b] ? i0 + 16 * b + n : 0)) * p.Hq + h) * DQK;
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st)
      qb[b][st] = row_ok[b] ? *(const uint4*)(qrow + (4 * st + g) * 8) : make_uint4(0, 0, 0, 0);
  }
  // resources over the sequence's rows of this KV head's K and V, bounded by
  // the end of the tensors (offsets are 32-bit: the host checks the sizes)
  const int k_tok = p.Hkv * DQK * 2, v_tok = p.Hkv * DV * 2;   // bytes per key row
  const uint8_t* kb = (const uint8_t*)p.k + (int64_t)k0 * k_tok + (int64_t)kvh * DQK * 2;
  const uint8_t* vb = (const uint8_t*)p.v + (int64_t)k0 * v_tok + (int64_t)kvh * DV * 2;
  const uint32_t k_bytes = (uint32_t)((int64_t)(p.total_k - k0) * k_tok - kvh * DQK * 2);
  const uint32_t v_bytes = (uint32_t)((int64_t)(p.total_k - k0) * v_tok - kvh * DV * 2);
  // this thread's chunks of a tile: i < KI are K chunks, the rest V chunks
  int crow[NCH], cvoff[NCH], clds[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int x = tid + kThreadsWg * i;
    if (i < KI) {
      crow[i] = x / KC;
      const int c = x - crow[i] * KC;
      cvoff[i] = crow[i] * k_tok + 16 * c;
      clds[i] = crow[i] * KROW + 16 * swz(crow[i], c);
    } else {
      const int y = x - TK * KC;
      crow[i] = y / VC;
      const int c = y - crow[i] * VC;
      cvoff[i] = crow[i] * v_tok + 16 * c;
      clds[i] = KBYTES + crow[i] * VROW + 16 * swz(crow[i], c);
    }
  }
  uint4 stg[NCH];
  auto gload = [&](int t) {
    const bool live = t < nt;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int so = live ? t * TK * (i < KI ? k_tok : v_tok) : 0;
      // past the last tile the resource has size zero: the load returns
      // zeros and the wait counts stay the same on every step (the size is
      // a scalar select, so the resource stays in scalar registers)
      const __amdgpu_buffer_rsrc_t r = make_rsrc(i < KI ? kb : vb, live ? (i < KI ? k_bytes : v_bytes) : 0u);
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, cvoff[i], so, 0);
      stg[i] = make_uint4(a[0], a[1], a[2], a[3]);
    }
  };
  // keys past the last one the workgroup's rows see are stored as zeros, so
  // a zero weight never meets a non-finite value (only the last tile has
  // such keys: the test is wave-uniform)
  auto lwrite = [&](auto stage_c, int t) {
    constexpr int SG = decltype(stage_c)::value;
    uint8_t* base = lds + SG * STAGE;
    if (t * TK + TK <= kend) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) *(uint4*)(base + clds[i]) = stg[i];
    } else {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const bool keep = t * TK + crow[i] < kend;
        *(uint4*)(base + clds[i]) = keep ? stg[i] : make_uint4(0, 0, 0, 0);
      }
    }
  };
  // Per-lane LDS offsets of the operand reads, split so that everything
  // that varies with the step, the key block or the stage is an immediate.
  // K fragment of step st: row n, chunk (4 st + g) ^ (n mod 8) = 4 (st ^ b)
  // + (g ^ (n mod 4)) with b = bit 2 of n; st ^ b is st + b for even st and
  // st - b for odd st.
  const int kb_bit = (n >> 2) & 1;
  const int kofs_e = n * KROW + 16 * (g ^ (n & 3)) + 64 * kb_bit;
  const int kofs_o = kofs_e - 128 * kb_bit;
  // transposed V read of dims 16 jd .. + 15: lane (a + 4 jj) of its group
  // addresses key r0 = 4 g + jj (r0 + 16 for the second block, the same
  // swizzle), dims 16 jd + 4 a .. + 3, i.e. chunk c = 2 jd + a / 2 at
  // c ^ m, m = r0 mod 8; with mm = m / 2 that is 2 ((jd & ~3) + ((jd & 3) ^
  // mm)) + (a / 2 ^ m mod 2): one base per value of jd mod 4.
  const int va = n & 3, vjj = n >> 2;
  const int vr0 = 4 * g + vjj, vm = vr0 & 7;
  int vofs[4];
#pragma unroll
  for (int qd = 0; qd < 4; ++qd)
    vofs[qd] = KBYTES + vr0 * VROW + 32 * (qd ^ (vm >> 1)) + 16 * ((va >> 1) ^ (vm & 1)) + 8 * (va & 1);
  RAcc<DV> A[kSub];
#pragma unroll
  for (int b = 0; b < kSub; ++b) {
    A[b].m = kNegInfR;
    A[b].lsum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jd = 0; jd < DT; ++jd) A[b].o[jd] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  using Stage0 = std::integral_constant<int, 0>;
  using Stage1 = std::integral_constant<int, 1>;
  gload(0);
  lwrite(Stage0{}, 0);
  gload(1);
  lds_sync();
  // one tile; its LDS stage SG = t mod 2 is a compile-time constant, so
  // every operand read is a per-lane base plus an immediate offset
  auto tile = [&](auto stage_c, int t) {
    constexpr int SG = decltype(stage_c)::value;
#pragma unroll
    for (int hf = 0; hf < TK / 32; ++hf) {
    const uint8_t* kt = lds + SG * STAGE + hf * 32 * KROW;
    const uint8_t* vt = lds + SG * STAGE + hf * 32 * VROW;
    const int key0 = t * TK + 32 * hf;
    if (has_rows && key0 < kend_w) {
      // ---- S^T of both 16-key blocks for both sub-blocks
      f32x4 sc[kSub][2];
#pragma unroll
      for (int b = 0; b < kSub; ++b) sc[b][0] = sc[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const uint4 kf = *(const uint4*)(kt + kb2 * 16 * KROW + 64 * st + ((st & 1) ? kofs_o : kofs_e));
#pragma unroll
          for (int b = 0; b < kSub; ++b) sc[b][kb2] = mfma_k32<QT>(kf, qb[b][st], sc[b][kb2]);
        }
      // ---- online softmax per sub-block over the 32 keys (row n; keys
      // t TK + 16 kb2 + 4 g + i)
      uint4 pw[kSub];
#pragma unroll
      for (int b = 0; b < kSub; ++b) {
        // raw scores; the scale (> 0) enters once, in the exponent.  Only
        // a tile that reaches past some row's last key (wave-uniform test)
        // needs the causal mask.
        float x[8];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[4 * kb2 + i] = sc[b][kb2][i];
        if (key0 + 32 > lim_lo[b]) {
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (key0 + 16 * kb2 + 4 * g + i >= lim[b]) x[4 * kb2 + i] = kNegInfR;
        }
        float tmax = vmax3(vmax3(x[0], x[1], x[2]), vmax3(x[3], x[4], x[5]), vmax2(x[6], x[7]));
        tmax = row_max4(tmax) * p.scale_log2;
        const bool bump = tmax > A[b].m + kSlack;
        const float m_new = bump ? tmax : A[b].m;
        const float m_ref = m_new == kNegInfR ? 0.f : m_new;
        const float alpha = bump ? __builtin_amdgcn_exp2f(A[b].m - m_ref) : 1.f;
        float pr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], p.scale_log2, -m_ref));
        pw[b] = make_uint4(pack2<QT>(pr[0], pr[1]), pack2<QT>(pr[2], pr[3]),
                           pack2<QT>(pr[4], pr[5]), pack2<QT>(pr[6], pr[7]));
        A[b].m = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
          for (int jd = 0; jd < DT; ++jd) A[b].o[jd] *= alpha;
          A[b].lsum *= alpha;
        }
      }
      // ---- O^T += V^T . P^T, 16 dims at a time
#pragma unroll
      for (int jd = 0; jd < DT; ++jd) {
        const uint8_t* va0 = vt + vofs[jd & 3] + 32 * (jd & ~3);
        const uint2 v0 = lds_tr16(va0);
        const uint2 v1 = lds_tr16(va0 + 16 * VROW);
        const uint4 vop = make_uint4(v0.x, v0.y, v1.x, v1.y);
#pragma unroll
        for (int b = 0; b < kSub; ++b) A[b].o[jd] = mfma_k32<QT>(vop, pw[b], A[b].o[jd]);
      }
      // the row sums: P . ones (1.0 in the operand type)
      const uint32_t one2 = QT == kBF16 ? 0x3f803f80u : 0x3c003c00u;
#pragma unroll
      for (int b = 0; b < kSub; ++b)
        A[b].lsum = mfma_k32<QT>(make_uint4(one2, one2, one2, one2), pw[b], A[b].lsum);
    }
    }
    // the next tile into the stage tile t - 1 used (every wave finished it
    // before the last barrier), then the loads of the one after
    if (t + 1 < nt) lwrite(std::integral_constant<int, 1 - SG>{}, t + 1);
    gload(t + 2);
    lds_sync();
  };
  for (int t = 0; t < nt; t += 2) {
    tile(Stage0{}, t);
    if (t + 1 < nt) tile(Stage1{}, t + 1);
  }
#pragma unroll
  for (int b = 0; b < kSub; ++b) {
    const float l = A[b].lsum[0];
    if (!row_ok[b]) continue;
    const int i = i0 + 16 * b + n;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    // lane (n, g) holds dims 16 jd + 4 g + ii of row i
    uint16_t* orow = (uint16_t*)p.out + ((int64_t)(q0 + i) * p.Hq + h) * DV;
#pragma unroll
    for (int jd = 0; jd < DT; ++jd)
      *(uint2*)(orow + 16 * jd + 4 * g) =
          make_uint2(pack2<QT>(A[b].o[jd][0] * inv, A[b].o[jd][1] * inv),
                     pack2<QT>(A[b].o[jd][2] * inv, A[b].o[jd][3] * inv));
    if (p.lse != nullptr && g == 0)
      p.lse[(int64_t)(q0 + i) * p.lse_sn + (int64_t)h * p.lse_sh] =
          l > 0.f ? (A[b].m + log2f(l)) * kLn2 : kNegInfR;
  }
}

// Workgroups are dealt to the 8 XCDs round robin (id mod 8); every query
// block of one (sequence, head) pair gets an id of the same residue, so they
// share one XCD's L2 and its copy of the pair's K/V rows: XCD x takes pairs
// x, x + 8, ... in order.  Causal blocks differ in cost (block j sees j + 1
// blocks of keys), so a causal workgroup takes two blocks of its pair, j from
// the end and j from the start, one after the other: every workgroup then has
// the same work, and a pair takes half as many workgroups.  Other calls take
// one block per workgroup, the pair's blocks side by side (they read the
// same K/V rows at about the same time).
template <int QT, int DQK, int DV, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) void ragged_attn_kernel(RaggedParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * ragged_stage_bytes<DQK, DV, NW>()];
  const int xcd = blockIdx.x & 7, jw = blockIdx.x >> 3;
  const int per_pair = p.causal ? (p.q_blocks + 1) / 2 : p.q_blocks;
  const int pl = jw / per_pair, jj = jw - pl * per_pair;
  const int pair = 8 * pl + xcd;
  if (pair >= p.num_seqs * p.Hq) return;
  ragged_item<QT, DQK, DV, NW>(p, lds, pair, p.q_blocks - 1 - jj);
  if (p.causal && jj != p.q_blocks - 1 - jj) ragged_item<QT, DQK, DV, NW>(p, lds, pair, jj);
}

// Eight-wave workgroups (256 queries, 64-key tiles): one tile load serves
// 256 queries.  (Causal calls had run four waves, 128 queries, so that rows
// seeing different key counts idle less at the diagonal; with two blocks per
// causal workgroup eight waves measured 6% faster on the 4 x 4096 causal
// prefill.)
template <int QT, int DQK, int DV>
static hipError_t launch_ragged(const RaggedParams& p, hipStream_t s) {
  constexpr int nw = 8;
  RaggedParams q = p;
  q.q_blocks = (p.max_q_len + 32 * nw - 1) / (32 * nw);
  // workgroups: pairs per XCD (rounded up) x workgroups per pair, per XCD
  const int64_t per_xcd = ((int64_t)p.num_seqs * p.Hq + 7) / 8;
  const int64_t per_pair = p.causal ? (q.q_blocks + 1) / 2 : q.q_blocks;
  const int64_t n = 8 * per_xcd * per_pair;
  if (n >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((ragged_attn_kernel<QT, DQK, DV, nw>), dim3((unsigned)n), dim3(64 * nw), 0, s, q);
  return hipGetLastError();
}

hipError_t launch_ragged_attn(int dtype, const RaggedParams& p, hipStream_t s) {
#define PKV_RCASE(QT, A, B) \
  if (dtype == QT && p.Dqk == A && p.Dv == B) return launch_ragged<QT, A, B>(p, s);
  PKV_RCASE(kBF16, 128, 128)
  PKV_RCASE(kF16, 128, 128)
  PKV_RCASE(kBF16, 192, 128)
  PKV_RCASE(kF16, 192, 128)
  PKV_RCASE(kBF16, 64, 64)
  PKV_RCASE(kF16, 64, 64)
#undef PKV_RCASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
