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
// A workgroup of four waves takes 64 consecutive queries of one (sequence,
// query head); wave w takes rows 16 w .. 16 w + 15, so the four waves stream
// the same K/V rows (the later ones from cache).  Per 16-key tile, with the
// key tokens on the M side of both products as in the decode kernels:
//   S^T (16 keys x 16 queries) = K (16 x Dqk) . Q^T   -- 16x16x32 MFMAs
//   O^T (Dv x 16 queries)     += V^T (Dv x 16) . P^T  -- 16x16x16 MFMAs
// so lane l keeps query l % 16 in both results and the online softmax is
// per lane.  K and V come from HBM straight into the operand registers with
// 16-byte buffer loads; the next tile's loads are issued before this tile's
// matrix work.  The output is normalised in the kernel (no split).
#include "kernels.h"
#include "pkv_device.h"

namespace pkv {

namespace {

constexpr float kNegInfR = -__builtin_inff();
constexpr float kLn2 = 0.6931471805599453f;
// a wave takes kSub sub-blocks of 16 queries (one per MFMA column block)
// against each K/V tile it loads; a workgroup holds four waves
constexpr int kSub = 2;
constexpr int kQueriesPerWave = 16 * kSub;
constexpr int kQueriesPerWg = 4 * kQueriesPerWave;

// N 32-bit words at byte offset voff + soff with the default cache policy:
// the K/V rows of a (sequence, head) are read again by every query block.
template <int N>
__device__ __forceinline__ void rbuf_load(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint32_t* w) {
  if constexpr (N == 4) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
  } else {
    static_assert(N == 2, "16-bit V rows of 64 or 128 dims");
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    w[0] = a[0]; w[1] = a[1];
  }
}

template <int DQK, int DV>
struct RTile {
  static constexpr int KSTEPS = DQK / 32;   // 16x16x32 steps of S^T
  static constexpr int DT = DV / 16;        // O^T tiles (V elements per lane and token)
  static constexpr int VW = DT / 2;         // V words per lane and token (16-bit)
  uint32_t k[KSTEPS][4];
  uint32_t v[4][VW];
};

// The loads of 16-key tile t: lane (n, g) takes key n's 16-byte chunk
// 4 s + g of step s, and the DT values at dims DT n .. of keys 4 g + kk.  A
// tile past the block's last one reads through an empty resource (zeros, no
// memory access), so every step issues the same loads.
template <int DQK, int DV>
__device__ __forceinline__ void load_rtile(const __amdgpu_buffer_rsrc_t& rk,
                                           const __amdgpu_buffer_rsrc_t& rv,
                                           const __amdgpu_buffer_rsrc_t& rz, bool live, int t,
                                           int k_lane, int v_lane, int k_tok, int v_tok,
                                           RTile<DQK, DV>& T) {
  using TT = RTile<DQK, DV>;
  const int ks = live ? (t << 4) * k_tok : 0, vs = live ? (t << 4) * v_tok : 0;
#pragma unroll
  for (int s = 0; s < TT::KSTEPS; ++s) rbuf_load<4>(live ? rk : rz, k_lane + 64 * s, ks, T.k[s]);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) rbuf_load<TT::VW>(live ? rv : rz, v_lane, vs + kk * v_tok, T.v[kk]);
}

template <int DV>
struct RAcc {
  float m, l;
  f32x4 o[DV / 16];
};

// Keys at or past kend (one past the last key any row of the wave sees)
// get zero V, since a zero weight times a non-finite value would not be zero.
template <int DQK, int DV>
__device__ __forceinline__ void clear_v_past(int kend, int g, int t, RTile<DQK, DV>& T) {
  const int tok0 = t << 4;
  if (tok0 + 16 > kend) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bool keep = tok0 + 4 * g + kk < kend;
#pragma unroll
      for (int w = 0; w < RTile<DQK, DV>::VW; ++w) T.v[kk][w] = keep ? T.v[kk][w] : 0u;
    }
  }
}

// One 16-key tile for one 16-query sub-block.  lim: this lane's row sees
// keys < lim; lim_lo: the smallest lim of the sub-block's rows (tiles below
// it need no mask).
template <int QT, int DQK, int DV>
__device__ __forceinline__ void rcompute(float scale_log2, int lim, int lim_lo,
                                         const uint4* qb, int g, int t, const RTile<DQK, DV>& T,
                                         RAcc<DV>& A) {
  using TT = RTile<DQK, DV>;
  constexpr int DT = TT::DT;
  const int tok0 = t << 4;
  f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < TT::KSTEPS; ++s)
    s4 = mfma_k32<QT>(make_uint4(T.k[s][0], T.k[s][1], T.k[s][2], T.k[s][3]), qb[s], s4);
  const bool edge = tok0 + 16 > lim_lo;
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float xi = s4[i] * scale_log2;
    x[i] = (!edge || tok0 + 4 * g + i < lim) ? xi : kNegInfR;
  }
  float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  tmax = max_across_rows(tmax);
  // the reference A.m moves only when the tile max passes it by kSlack
  const bool bump = tmax > A.m + kSlack;
  const float m_new = bump ? tmax : A.m;
  const float m_ref = m_new == kNegInfR ? 0.f : m_new;
  const float alpha = bump ? __builtin_amdgcn_exp2f(A.m - m_ref) : 1.f;
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = __builtin_amdgcn_exp2f(x[i] - m_ref);
  // the sum takes the rounded probabilities that P . V uses
  const uint2 pb = make_uint2(pack2<QT>(pr[0], pr[1]), pack2<QT>(pr[2], pr[3]));
  const float2 r0 = unpack2<QT>(pb.x), r1 = unpack2<QT>(pb.y);
  A.l = A.l * alpha + ((r0.x + r0.y) + (r1.x + r1.y));
  A.m = m_new;
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
    for (int j = 0; j < DT; ++j) A.o[j] *= alpha;
  }
  // element j of keys 0, 1 (2, 3) into one word with one byte permute
#pragma unroll
  for (int j = 0; j < DT; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t w01 = __builtin_amdgcn_perm(T.v[1][j >> 1], T.v[0][j >> 1], sel);
    const uint32_t w23 = __builtin_amdgcn_perm(T.v[3][j >> 1], T.v[2][j >> 1], sel);
    A.o[j] = mfma_k16<QT>(make_uint2(w01, w23), pb, A.o[j]);
  }
}

}  // namespace

template <int QT, int DQK, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void ragged_attn_kernel(RaggedParams p) {
  using TT = RTile<DQK, DV>;
  constexpr int KSTEPS = TT::KSTEPS, DT = TT::DT;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // workgroups are dealt to the 8 XCDs round robin (id mod 8); every query
  // block of one (sequence, head) pair gets an id of the same residue, so
  // they share one XCD's L2 and its copy of the pair's K/V rows: XCD x takes
  // pairs x, x + 8, ..., each pair's blocks from the last (causal: the most
  // keys) to the first, so the cheap blocks fill the tail
  const int wg = blockIdx.x, xcd = wg & 7, j = wg >> 3;
  const int pair = 8 * (j / p.q_blocks) + xcd;
  const int qblk = p.q_blocks - 1 - (j - (j / p.q_blocks) * p.q_blocks);
  if (pair >= p.num_seqs * p.Hq) return;
  const int s = pair / p.Hq, h = pair - s * p.Hq, kvh = h / p.G;
  // sequence bounds, clamped to the tensors so that any cu_seqlens stay in bounds
  const int q0 = min(max(p.cu_q[s], 0), p.total_q), q1 = min(max(p.cu_q[s + 1], q0), p.total_q);
  const int k0 = min(max(p.cu_k[s], 0), p.total_k), k1 = min(max(p.cu_k[s + 1], k0), p.total_k);
  const int Lq = q1 - q0, Lk = k1 - k0;
  const int Lrun = min(Lq, p.max_q_len);   // queries computed (the rest stay unwritten)
  // wave w: queries i0 .. i0 + 31, as sub-blocks b = 0, 1 of 16 rows that
  // share every K/V tile the wave loads
  const int i0 = qblk * kQueriesPerWg + kQueriesPerWave * w;
  if (i0 >= Lrun) return;
  const int off = p.causal ? Lk - Lq : 0;  // query i sees keys < i + 1 + off (causal)
  int lim[kSub], lim_lo[kSub];
  bool row_ok[kSub];
#pragma unroll
  for (int b = 0; b < kSub; ++b) {
    const int i = i0 + 16 * b + n;
    row_ok[b] = i < Lrun;
    lim[b] = p.causal ? min(Lk, max(i + 1 + off, 0)) : Lk;
    lim_lo[b] = p.causal ? min(Lk, max(i0 + 16 * b + 1 + off, 0)) : Lk;
  }
  const int kend = p.causal ? min(Lk, max(min(i0 + kQueriesPerWave, Lrun) + off, 0)) : Lk;
  const int nt = (kend + 15) >> 4;
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
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)((int64_t)(p.total_k - k0) * k_tok - kvh * DQK * 2));
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)((int64_t)(p.total_k - k0) * v_tok - kvh * DV * 2));
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(kb, 0u);
  const int k_lane = n * k_tok + 16 * g;
  const int v_lane = 4 * g * v_tok + DT * n * 2;
  RAcc<DV> A[kSub];
#pragma unroll
  for (int b = 0; b < kSub; ++b) {
    A[b].m = kNegInfR;
    A[b].l = 0.f;
#pragma unroll
    for (int j = 0; j < DT; ++j) A[b].o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  TT buf[2];
  load_rtile<DQK, DV>(rk, rv, rz, 0 < nt, 0, k_lane, v_lane, k_tok, v_tok, buf[0]);
  for (int t = 0; t < nt; t += 2) {
    load_rtile<DQK, DV>(rk, rv, rz, t + 1 < nt, t + 1, k_lane, v_lane, k_tok, v_tok, buf[1]);
    clear_v_past<DQK, DV>(kend, g, t, buf[0]);
#pragma unroll
    for (int b = 0; b < kSub; ++b)
      rcompute<QT, DQK, DV>(p.scale_log2, lim[b], lim_lo[b], qb[b], g, t, buf[0], A[b]);
    load_rtile<DQK, DV>(rk, rv, rz, t + 2 < nt, t + 2, k_lane, v_lane, k_tok, v_tok, buf[0]);
    if (t + 1 < nt) {
      clear_v_past<DQK, DV>(kend, g, t + 1, buf[1]);
#pragma unroll
      for (int b = 0; b < kSub; ++b)
        rcompute<QT, DQK, DV>(p.scale_log2, lim[b], lim_lo[b], qb[b], g, t + 1, buf[1], A[b]);
    }
  }
#pragma unroll
  for (int b = 0; b < kSub; ++b) {
    const float l = sum_across_rows(A[b].l);
    if (!row_ok[b]) continue;
    const int i = i0 + 16 * b + n;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    // lane (n, g) holds dims DT (4 g + ii) + j of row i
    uint16_t* orow = (uint16_t*)p.out + ((int64_t)(q0 + i) * p.Hq + h) * DV;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int j = 0; j < DT; j += 4)
        *(uint2*)(orow + DT * (4 * g + ii) + j) =
            make_uint2(pack2<QT>(A[b].o[j][ii] * inv, A[b].o[j + 1][ii] * inv),
                       pack2<QT>(A[b].o[j + 2][ii] * inv, A[b].o[j + 3][ii] * inv));
    if (p.lse != nullptr && g == 0)
      p.lse[(int64_t)(q0 + i) * p.lse_sn + (int64_t)h * p.lse_sh] =
          l > 0.f ? (A[b].m + log2f(l)) * kLn2 : kNegInfR;
  }
}

template <int QT, int DQK, int DV>
static hipError_t launch_ragged(const RaggedParams& p, hipStream_t s) {
  RaggedParams q = p;
  q.q_blocks = (p.max_q_len + kQueriesPerWg - 1) / kQueriesPerWg;
  const int64_t groups = ((int64_t)p.num_seqs * p.Hq + 7) / 8;
  const int64_t n = 8 * groups * q.q_blocks;
  if (n >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((ragged_attn_kernel<QT, DQK, DV>), dim3((unsigned)n), dim3(256), 0, s, q);
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
