// split_mfma.hip -- split-KV paged decode attention on the gfx950 matrix cores,
// for up to 16 query rows per KV head (rows = head group x query tokens).
//
// One workgroup (4 waves) handles one (sequence, KV head, split); the split
// is a run of `split_pages` pages (FlashInfer xqa page: the multi-block
// decode with a `workspace_buffer`; here the partials go to the workspace
// and a combine kernel merges them).  Each wave takes every fourth 16-token
// tile of the split, keeps its own online-softmax state, and the four waves
// merge through LDS at the end.
//
// Per 16-token tile a wave computes, with the rows padded to 16:
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
// 8u+2g+1 for steps 2u and 2u+1, so one 16-byte load serves two steps.
template <int KT>
__device__ __forceinline__ int qk_chunk(int s, int g) {
  if constexpr (KT == kFP8)
    return 8 * (s >> 1) + 2 * g + (s & 1);
  else
    return 4 * s + g;
}

template <int N>
__device__ __forceinline__ void load_words(const uint8_t* src, uint32_t* w) {
  if constexpr (N == 8) {
    uint4 a = *(const uint4*)src, b = *(const uint4*)(src + 16);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else if constexpr (N == 4) {
    uint4 a = *(const uint4*)src;
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  } else if constexpr (N == 2) {
    uint2 a = *(const uint2*)src;
    w[0] = a.x; w[1] = a.y;
  } else {
    w[0] = *(const uint32_t*)src;
  }
}

template <int KT, int D>
struct Tile {
  static constexpr int ELEM = KT == kFP8 ? 1 : 2;
  static constexpr int KSTEPS = D / 32;
  static constexpr int KLOADS = KT == kFP8 ? KSTEPS / 2 : KSTEPS;  // uint4 per lane
  static constexpr int DT = D / 16;                // O^T tiles = V elements per lane/token
  static constexpr int VW = DT * ELEM / 4;         // V words per lane per token
  uint4 k[KLOADS];
  uint32_t v[4][VW];
  int tok0;
  bool valid;
};

template <int QT, int KT, int D>
__device__ __forceinline__ void load_tile(const Params& p, int b, int kvh, int t, int n, int g,
                                          Tile<KT, D>& T) {
  using TT = Tile<KT, D>;
  T.tok0 = t << 4;
  const int page = p.page_table[(int64_t)b * p.pps + T.tok0 / p.ps];
  T.valid = (unsigned)page < (unsigned)p.num_pages;
  if (!T.valid) return;
  const int slot0 = T.tok0 % p.ps;
  const uint8_t* kb = (const uint8_t*)p.k +
      ((int64_t)page * p.k_page + (int64_t)(slot0 + n) * p.k_slot + (int64_t)kvh * p.k_head) * TT::ELEM;
#pragma unroll
  for (int i = 0; i < TT::KLOADS; ++i) {
    const int chunk = KT == kFP8 ? 8 * i + 2 * g : 4 * i + g;
    T.k[i] = *(const uint4*)(kb + chunk * 8 * TT::ELEM);
  }
  const uint8_t* vb = (const uint8_t*)p.v +
      ((int64_t)page * p.v_page + (int64_t)(slot0 + 4 * g) * p.v_slot + (int64_t)kvh * p.v_head +
       (int64_t)TT::DT * n) * TT::ELEM;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    load_words<TT::VW>(vb + (int64_t)kk * p.v_slot * TT::ELEM, T.v[kk]);
}

}  // namespace

template <int QT, int KT, int D>
__global__ __launch_bounds__(256) void split_mfma16_kernel(Params p) {
  using TT = Tile<KT, D>;
  constexpr int KSTEPS = TT::KSTEPS, DT = TT::DT;
  constexpr int SROW = D + 4;  // LDS row stride (floats), padded
  __shared__ float s_acc[4][16 * SROW];
  __shared__ float s_m[4][16], s_l[4][16], s_M[16], s_L[16];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const SeqGeom sg = seq_geom(p, b);
  if (split >= sg.nsplits) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;

  const int pg_begin = sg.p0 + split * p.split_pages;
  const int pg_end = min(pg_begin + p.split_pages, sg.p0 + sg.npages);
  const int tok_begin = max(pg_begin * p.ps, sg.lo);
  const int tok_end = min(pg_end * p.ps, sg.L);
  const int tile_begin = tok_begin >> 4, tile_end = (tok_end + 15) >> 4;

  // Q^T operand of row n (zero rows pad the group to 16)
  const bool row_ok = n < p.R;
  uint4 qb[KSTEPS];
  {
    const uint16_t* qrow =
        (const uint16_t*)p.q + q_row_offset(p, b, kvh, row_ok ? n : 0) * p.Dqk;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      qb[s] = row_ok ? *(const uint4*)(qrow + qk_chunk<KT>(s, g) * 8) : make_uint4(0, 0, 0, 0);
  }
  const RowVis vis = row_vis(p, b, sg.L, row_ok ? n : 0);
  // tiles wholly inside [lo_last_row, mask_from) need no per-element test
  const int lo_last = p.window > 0 ? sg.L - p.window : INT32_MIN;
  const int mask_from = (p.Tq > 1 && p.mask != nullptr) ? sg.L - p.Tq : sg.L;

  float m = kNegInf, l = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int j = 0; j < DT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  TT cur, nxt;
  int t = tile_begin + wave;
  if (t < tile_end) load_tile<QT, KT, D>(p, b, kvh, t, n, g, cur);
  while (t < tile_end) {
    const int tn = t + 4;
    if (tn < tile_end) load_tile<QT, KT, D>(p, b, kvh, tn, n, g, nxt);
    if (cur.valid) {
      const int tok0 = cur.tok0;
      const bool edge = tok0 < lo_last || tok0 + 16 > mask_from;
      if (edge) {
        // tokens no row can see may hold anything (NaN): clear their V so a
        // zero weight cannot turn into NaN inside the P.V product
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int tk = tok0 + 4 * g + kk;
          if (tk < sg.lo || tk >= sg.L)
#pragma unroll
            for (int w = 0; w < TT::VW; ++w) cur.v[kk][w] = 0u;
        }
      }
      // ---- S^T = K . Q^T
      f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        uint4 a;
        if constexpr (KT == kFP8) {
          const uint4& w = cur.k[s >> 1];
          uint2 lo = fp8x4_to_16<QT>((s & 1) ? w.z : w.x);
          uint2 hi = fp8x4_to_16<QT>((s & 1) ? w.w : w.y);
          a = make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
          a = cur.k[s];
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
      const float m_new = fmaxf(m, tmax);
      const float m_ref = m_new == kNegInf ? 0.f : m_new;
      const float alpha = exp2f(m - m_ref);
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = exp2f(x[i] - m_ref);
      l = l * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      m = m_new;
#pragma unroll
      for (int j = 0; j < DT; ++j) acc[j] *= alpha;
      const uint2 pb = make_uint2(pack2<QT>(pr[0], pr[1]), pack2<QT>(pr[2], pr[3]));
      // ---- O^T += V^T . P^T
      uint32_t v16[4][DT / 2];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if constexpr (KT == kFP8) {
#pragma unroll
          for (int w = 0; w < TT::VW; ++w) {
            uint2 c = fp8x4_to_16<QT>(cur.v[kk][w]);
            v16[kk][2 * w] = c.x;
            v16[kk][2 * w + 1] = c.y;
          }
        } else {
#pragma unroll
          for (int w = 0; w < DT / 2; ++w) v16[kk][w] = cur.v[kk][w];
        }
      }
#pragma unroll
      for (int j = 0; j < DT; ++j) {
        const int sh = 16 * (j & 1);
        const uint32_t e0 = (v16[0][j >> 1] >> sh) & 0xffffu, e1 = (v16[1][j >> 1] >> sh) & 0xffffu;
        const uint32_t e2 = (v16[2][j >> 1] >> sh) & 0xffffu, e3 = (v16[3][j >> 1] >> sh) & 0xffffu;
        acc[j] = mfma_k16<QT>(make_uint2(e0 | (e1 << 16), e2 | (e3 << 16)), pb, acc[j]);
      }
    }
    t = tn;
    cur = nxt;
  }

  // ---- merge the four waves (LDS), then write a partial or the output
  l = sum_across_rows(l);
  if (g == 0) {
    s_m[wave][n] = m;
    s_l[wave][n] = l;
  }
  __syncthreads();
  float M = fmaxf(fmaxf(s_m[0][n], s_m[1][n]), fmaxf(s_m[2][n], s_m[3][n]));
  float Ltot = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (s_m[w][n] != kNegInf) Ltot += s_l[w][n] * exp2f(s_m[w][n] - M);
  const float sc = m == kNegInf ? 0.f : exp2f(m - M);
  // lane (n, g) holds dims DT*(4g+i) + j of row n
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < DT; ++j) s_acc[wave][n * SROW + DT * (4 * g + i) + j] = acc[j][i] * sc;
  if (wave == 0 && g == 0) {
    s_M[n] = M;
    s_L[n] = Ltot;
  }
  __syncthreads();

  const bool final_out = sg.nsplits == 1;
  for (int e4 = threadIdx.x; e4 < 16 * (D / 4); e4 += 256) {
    const int row = e4 / (D / 4), d = (e4 % (D / 4)) * 4;
    if (row >= p.R) continue;
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 a = *(const float4*)&s_acc[w][row * SROW + d];
      sum.x += a.x; sum.y += a.y; sum.z += a.z; sum.w += a.w;
    }
    if (final_out) {
      const float Mr = s_M[row], Lr = s_L[row];
      float num = 1.f, den = Lr;
      if (p.sinks != nullptr) {
        const int gh = row % p.G;
        const float sk = p.sinks[kvh * p.G + gh] * kLog2e;
        const float Mf = fmaxf(Mr, sk);
        num = Mr == kNegInf ? 0.f : exp2f(Mr - Mf);
        den = Lr * num + exp2f(sk - Mf);
      }
      const float inv = den > 0.f ? p.out_scale * num / den : 0.f;
      uint16_t* o = (uint16_t*)p.out + q_row_offset(p, b, kvh, row) * p.Dv + d;
      *(uint2*)o = make_uint2(pack2<QT>(sum.x * inv, sum.y * inv), pack2<QT>(sum.z * inv, sum.w * inv));
    } else {
      const int64_t prow = (((int64_t)b * p.Hkv + kvh) * p.max_splits + split) * p.R + row;
      *(float4*)(p.ws_o + prow * p.Dv + d) = sum;
      if (d == 0) p.ws_ml[prow] = make_float2(s_M[row], s_L[row]);
    }
  }
}

template <int QT, int KT, int D>
hipError_t launch_split_mfma16(const Params& p, hipStream_t stream) {
  dim3 grid(p.max_splits, p.Hkv, p.B);
  hipLaunchKernelGGL((split_mfma16_kernel<QT, KT, D>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_split_mfma16(int q_dtype, int kv_dtype, int D, const Params& p, hipStream_t s) {
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
