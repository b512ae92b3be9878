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
// One workgroup (4 waves) handles one (sequence, split).  Each 16-token tile
// of the latent cache is loaded once into LDS (16-byte loads, prefetched
// into registers during the previous tile's math) and read by all four
// waves; wave w owns query rows 16w..16w+15 and computes
//   S^T (16 tokens x 16 rows) = K (16 x 576) . Q^T      -- 18 MFMA 16x16x32
//   O^T (512 x 16 rows)      += V^T (512 x 16) . P^T    -- 32 MFMA 16x16x16
// with V^T read from the same LDS rows as K, so each cached byte leaves HBM
// once and serves both products.
#include "pkv_device.h"
#include "kernels.h"

namespace pkv {

namespace {
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
}  // namespace

template <int QT, int DQK, int DV>
__global__ __launch_bounds__(256) void split_mla_kernel(Params p) {
  constexpr int KSTEPS = DQK / 32;            // 18
  constexpr int DT = DV / 16;                 // 32 O^T tiles; V dims per lane
  constexpr int CH = DQK / 8;                 // 72 16-byte chunks per row
  constexpr int STRIDE = CH + 1;              // LDS row stride in chunks (pad)
  constexpr int TILE_CHUNKS = 16 * CH;        // 1152
  constexpr int PER_THREAD = (TILE_CHUNKS + 255) / 256;  // 5
  static_assert(DT % 8 == 0, "V width must be a multiple of 128");
  __shared__ uint4 s_k[16 * STRIDE];

  const int split = blockIdx.x, b = blockIdx.z;
  const int kvh = blockIdx.y;
  const SeqGeom sg = seq_geom(p, b);
  if (split >= sg.nsplits) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int row = wave * 16 + n;

  const int pg_begin = sg.p0 + split * p.split_pages;
  const int pg_end = min(pg_begin + p.split_pages, sg.p0 + sg.npages);
  const int tok_begin = max(pg_begin * p.ps, sg.lo);
  const int tok_end = min(pg_end * p.ps, sg.L);
  const int tile_begin = tok_begin >> 4, tile_end = (tok_end + 15) >> 4;

  const bool row_ok = row < p.R;
  uint4 qb[KSTEPS];
  {
    const uint16_t* qrow =
        (const uint16_t*)p.q + q_row_offset(p, b, kvh, row_ok ? row : 0) * p.Dqk;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      qb[s] = row_ok ? *(const uint4*)(qrow + (4 * s + g) * 8) : make_uint4(0, 0, 0, 0);
  }
  const RowVis vis = row_vis(p, b, sg.L, row_ok ? row : 0);
  const int lo_last = p.window > 0 ? sg.L - p.window : INT32_MIN;
  const int mask_from = (p.Tq > 1 && p.mask != nullptr) ? sg.L - p.Tq : sg.L;

  float m = kNegInf, l = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int j = 0; j < DT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // cooperative tile load: chunk c = tid + 256 i -> (token c / CH, chunk c % CH)
  uint4 pre[PER_THREAD];
  auto load = [&](int t, bool& valid) {
    const int tok0 = t << 4;
    const int page = p.page_table[(int64_t)b * p.pps + tok0 / p.ps];
    valid = (unsigned)page < (unsigned)p.num_pages;
    if (!valid) return;
    const int slot0 = tok0 % p.ps;
    const uint16_t* base = (const uint16_t*)p.k + (int64_t)page * p.k_page + (int64_t)kvh * p.k_head;
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int c = tid + 256 * i;
      if (c < TILE_CHUNKS) {
        const int tk = c / CH, ch = c - tk * CH;
        const int tok = tok0 + tk;
        // rows no query can see may hold anything (NaN): load zeros instead
        if (tok >= sg.lo && tok < sg.L)
          pre[i] = *(const uint4*)(base + (int64_t)(slot0 + tk) * p.k_slot + ch * 8);
        else
          pre[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };

  bool valid_cur = false, valid_nxt = false;
  if (tile_begin < tile_end) load(tile_begin, valid_cur);
  for (int t = tile_begin; t < tile_end; ++t) {
    __syncthreads();  // previous tile's readers are done with s_k
    if (valid_cur) {
#pragma unroll
      for (int i = 0; i < PER_THREAD; ++i) {
        const int c = tid + 256 * i;
        if (c < TILE_CHUNKS) {
          const int tk = c / CH, ch = c - tk * CH;
          s_k[tk * STRIDE + ch] = pre[i];
        }
      }
    }
    __syncthreads();
    if (t + 1 < tile_end) load(t + 1, valid_nxt);
    if (valid_cur) {
      const int tok0 = t << 4;
      const bool edge = tok0 < lo_last || tok0 + 16 > mask_from || tok0 < sg.lo || tok0 + 16 > sg.L;
      // ---- S^T = K . Q^T (A: token n, chunk 4s+g)
      f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) s4 = mfma_k32<QT>(s_k[n * STRIDE + 4 * s + g], qb[s], s4);
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
      // ---- O^T += V^T . P^T; lane (n, g) feeds dims DT*n + j of tokens 4g+kk
#pragma unroll
      for (int q8 = 0; q8 < DT / 8; ++q8) {
        uint4 vv[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) vv[kk] = s_k[(4 * g + kk) * STRIDE + (DT / 8) * n + q8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t a0 = half_of(vv[0], e) | (half_of(vv[1], e) << 16);
          const uint32_t a1 = half_of(vv[2], e) | (half_of(vv[3], e) << 16);
          acc[8 * q8 + e] = mfma_k16<QT>(make_uint2(a0, a1), pb, acc[8 * q8 + e]);
        }
      }
    }
    valid_cur = valid_nxt;
  }

  // ---- epilogue: each wave owns its rows; no cross-wave merge
  l = sum_across_rows(l);
  if (!row_ok) return;
  const bool final_out = sg.nsplits == 1;
  // lane (n, g) holds dims DT*(4g+i) + j for i = 0..3, j = 0..DT-1
  if (final_out) {
    float num = 1.f, den = l;
    if (p.sinks != nullptr) {
      const float sk = p.sinks[kvh * p.G + row % p.G] * kLog2e;
      const float Mf = fmaxf(m, sk);
      num = m == kNegInf ? 0.f : exp2f(m - Mf);
      den = l * num + exp2f(sk - Mf);
    }
    const float inv = den > 0.f ? p.out_scale * num / den : 0.f;
    uint16_t* o = (uint16_t*)p.out + q_row_offset(p, b, kvh, row) * p.Dv;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < DT; j += 4)
        *(uint2*)(o + DT * (4 * g + i) + j) =
            make_uint2(pack2<QT>(acc[j][i] * inv, acc[j + 1][i] * inv),
                       pack2<QT>(acc[j + 2][i] * inv, acc[j + 3][i] * inv));
  } else {
    const int64_t prow = (((int64_t)b * p.Hkv + kvh) * p.max_splits + split) * p.R + row;
    float* o = p.ws_o + prow * p.Dv;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < DT; j += 4)
        *(float4*)(o + DT * (4 * g + i) + j) =
            make_float4(acc[j][i], acc[j + 1][i], acc[j + 2][i], acc[j + 3][i]);
    if (g == 0) p.ws_ml[prow] = make_float2(m, l);
  }
}

template <int QT>
hipError_t launch_split_mla(const Params& p, hipStream_t stream) {
  dim3 grid(p.max_splits, p.Hkv, p.B);
  hipLaunchKernelGGL((split_mla_kernel<QT, 576, 512>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_split_mla(int q_dtype, const Params& p, hipStream_t s) {
  if (q_dtype == kBF16) return launch_split_mla<kBF16>(p, s);
  if (q_dtype == kF16) return launch_split_mla<kF16>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
