// split_valu.hip -- split-KV paged decode attention on the vector ALUs, for
// head groups of up to 8 query rows and head_dim 128.
//
// Decode with few rows per KV head does ~4 flops per cached byte, far below
// the matrix-core ridge, so this path keeps the contraction on the VALU:
// 16 lanes share one token, each owning 8 head dims (one 16-byte load of K
// and of V); a wave covers 4 tokens per step and 16 per tile.
//   q.k : v_dot2 on 16-bit pairs (fp8 K converted exactly first), then a
//         16-lane DPP butterfly (quad_perm, row_ror) -- every lane of the
//         group ends with the full score of every row;
//   P.V : per-lane fp32 FMAs into an [rows x 8 dims] accumulator;
// online softmax per tile, and the four token slots of a wave and the four
// waves of the workgroup merge at the end.  Workgroup = (sequence, KV head,
// split), as in the matrix-core path.
#include "pkv_device.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}

// sum over the 16 lanes of a DPP row; every lane gets the total
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x124>(x);  // row_ror 4
  x += dpp<0x128>(x);  // row_ror 8
  return x;
}

template <int QT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (QT == kBF16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  } else {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                  false);
  }
}

// 8 elements of the compute type (4 dwords) -> 8 floats
template <int QT>
__device__ __forceinline__ void widen8(const uint4& w, float* f) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (QT == kBF16) {
      f[2 * i] = __uint_as_float(a[i] << 16);
      f[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
    } else {
      typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
      f16x2 h = __builtin_bit_cast(f16x2, a[i]);
      f[2 * i] = (float)h[0];
      f[2 * i + 1] = (float)h[1];
    }
  }
}

template <int KT>
struct VTile {
  // per step j (token tok0 + 4j + slot): this lane's 8 dims of K and V
  uint4 k[4];
  uint4 v[4];   // fp8: only .x/.y used (8 bytes)
  int tok0;
  bool valid;
};

template <int KT>
__device__ __forceinline__ void vload(const Params& p, int b, int kvh, int t, int slot, int c,
                                      VTile<KT>& T) {
  constexpr int ELEM = KT == kFP8 ? 1 : 2;
  T.tok0 = t << 4;
  const int page = p.page_table[(int64_t)b * p.pps + T.tok0 / p.ps];
  T.valid = (unsigned)page < (unsigned)p.num_pages;
  if (!T.valid) return;
  const int slot0 = T.tok0 % p.ps;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = slot0 + 4 * j + slot;
    const uint8_t* kb = (const uint8_t*)p.k +
        ((int64_t)page * p.k_page + (int64_t)s * p.k_slot + (int64_t)kvh * p.k_head + 8 * c) * ELEM;
    const uint8_t* vb = (const uint8_t*)p.v +
        ((int64_t)page * p.v_page + (int64_t)s * p.v_slot + (int64_t)kvh * p.v_head + 8 * c) * ELEM;
    if constexpr (KT == kFP8) {
      uint2 a = *(const uint2*)kb, d = *(const uint2*)vb;
      T.k[j] = make_uint4(a.x, a.y, 0u, 0u);
      T.v[j] = make_uint4(d.x, d.y, 0u, 0u);
    } else {
      // non-temporal: the K/V stream is read once
      const u32x4 a = __builtin_nontemporal_load((const u32x4*)kb);
      const u32x4 d = __builtin_nontemporal_load((const u32x4*)vb);
      T.k[j] = make_uint4(a[0], a[1], a[2], a[3]);
      T.v[j] = make_uint4(d[0], d[1], d[2], d[3]);
    }
  }
}

template <int QT, int KT>
__device__ __forceinline__ uint4 to16x8(const uint4& raw) {
  if constexpr (KT == kFP8) {
    uint2 lo = fp8x4_to_16<QT>(raw.x), hi = fp8x4_to_16<QT>(raw.y);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  } else {
    return raw;
  }
}

}  // namespace

template <int QT, int KT, int NR>
__global__ __launch_bounds__(256) void split_valu_kernel(Params p) {
  resolve_scales(p);
  constexpr int D = 128;
  __shared__ float s_acc[4][NR][D];
  __shared__ float s_m[4][NR], s_l[4][NR];

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const SeqGeom sg = seq_geom(p, b);
  if (split >= sg.nsplits) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane >> 4, c = lane & 15;  // token slot in a step, 8-dim chunk

  const int pg_begin = sg.p0 + split * p.split_pages;
  const int pg_end = min(pg_begin + p.split_pages, sg.p0 + sg.npages);
  const int tok_begin = max(pg_begin * p.ps, sg.lo);
  const int tok_end = min(pg_end * p.ps, sg.L);
  const int tile_begin = tok_begin >> 4, tile_end = (tok_end + 15) >> 4;

  uint4 q[NR];
  RowVis vis[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const bool ok = r < p.R;
    const uint16_t* qrow = (const uint16_t*)p.q + q_row_offset(p, b, kvh, ok ? r : 0) * p.Dqk;
    q[r] = ok ? *(const uint4*)(qrow + 8 * c) : make_uint4(0, 0, 0, 0);
    vis[r] = row_vis(p, b, sg.L, ok ? r : 0);
  }
  const int lo_last = p.window > 0 ? sg.L - p.window : INT32_MIN;
  const int mask_from = (p.Tq > 1 && p.mask != nullptr) ? sg.L - p.Tq : sg.L;

  float m[NR], l[NR], acc[NR][8];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }

  VTile<KT> cur, nxt;
  int t = tile_begin + wave;
  if (t < tile_end) vload<KT>(p, b, kvh, t, slot, c, cur);
  while (t < tile_end) {
    const int tn = t + 4;
    if (tn < tile_end) vload<KT>(p, b, kvh, tn, slot, c, nxt);
    if (cur.valid) {
      const int tok0 = cur.tok0;
      const bool edge = tok0 < lo_last || tok0 + 16 > mask_from;
      float x[4][NR];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 k = to16x8<QT, KT>(cur.k[j]);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          float s = dot2<QT>(q[r].x, k.x, 0.f);
          s = dot2<QT>(q[r].y, k.y, s);
          s = dot2<QT>(q[r].z, k.z, s);
          s = dot2<QT>(q[r].w, k.w, s);
          x[j][r] = sum16(s) * p.qk_scale_log2;
        }
        if (edge) {
          const int tk = tok0 + 4 * j + slot;
#pragma unroll
          for (int r = 0; r < NR; ++r) x[j][r] = vis[r](tk, sg.L) ? x[j][r] : kNegInf;
          // a token no row sees may hold NaN: keep it out of the P.V sum
          if (tk < sg.lo || tk >= sg.L) cur.v[j] = make_uint4(0, 0, 0, 0);
        }
      }
      float vf[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j) widen8<QT>(to16x8<QT, KT>(cur.v[j]), vf[j]);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float tmax = fmaxf(fmaxf(x[0][r], x[1][r]), fmaxf(x[2][r], x[3][r]));
        tmax = max_across_rows(tmax);
        const float m_new = fmaxf(m[r], tmax);
        const float m_ref = m_new == kNegInf ? 0.f : m_new;
        const float alpha = exp2f(m[r] - m_ref);
        float pr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) pr[j] = exp2f(x[j][r] - m_ref);
        l[r] = l[r] * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
        m[r] = m_new;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float a = acc[r][e] * alpha;
          a = fmaf(pr[0], vf[0][e], a);
          a = fmaf(pr[1], vf[1][e], a);
          a = fmaf(pr[2], vf[2][e], a);
          a = fmaf(pr[3], vf[3][e], a);
          acc[r][e] = a;
        }
      }
    }
    t = tn;
    cur = nxt;
  }

  // ---- fold the four token slots of the wave (m is uniform across slots)
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    l[r] = sum_across_rows(l[r]);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = sum_across_rows(acc[r][e]);
  }
  // ---- merge the four waves
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      s_m[wave][r] = m[r];
      s_l[wave][r] = l[r];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const float M = fmaxf(fmaxf(s_m[0][r], s_m[1][r]), fmaxf(s_m[2][r], s_m[3][r]));
    const float sc = m[r] == kNegInf ? 0.f : exp2f(m[r] - M);
    if (slot == 0)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][r][8 * c + e] = acc[r][e] * sc;
  }
  __syncthreads();
  const bool final_out = sg.nsplits == 1;
  for (int idx = threadIdx.x; idx < NR * (D / 4); idx += 256) {
    const int r = idx / (D / 4), d = (idx % (D / 4)) * 4;
    if (r >= p.R) continue;
    const float M = fmaxf(fmaxf(s_m[0][r], s_m[1][r]), fmaxf(s_m[2][r], s_m[3][r]));
    float Ltot = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (s_m[w][r] != kNegInf) Ltot += s_l[w][r] * exp2f(s_m[w][r] - M);
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 a = *(const float4*)&s_acc[w][r][d];
      sum.x += a.x; sum.y += a.y; sum.z += a.z; sum.w += a.w;
    }
    if (final_out) {
      float num = 1.f, den = Ltot;
      if (p.sinks != nullptr) {
        const float sk = p.sinks[kvh * p.G + r % p.G] * kLog2e;
        const float Mf = fmaxf(M, sk);
        num = M == kNegInf ? 0.f : exp2f(M - Mf);
        den = Ltot * num + exp2f(sk - Mf);
      }
      const float inv = den > 0.f ? p.out_scale * num / den : 0.f;
      store_out4<QT>(p, q_row_offset(p, b, kvh, r) * p.Dv + d, sum.x * inv, sum.y * inv, sum.z * inv,
                     sum.w * inv);
    } else {
      const int64_t prow = (((int64_t)b * p.Hkv + kvh) * p.max_splits + split) * p.R + r;
      *(float4*)(p.ws_o + prow * p.Dv + d) = sum;
      if (d == 0) p.ws_ml[prow] = make_float2(M, Ltot);
    }
  }
}

template <int QT, int KT>
hipError_t launch_valu_rows(const Params& p, hipStream_t s) {
  dim3 grid(p.max_splits, p.Hkv, p.B);
  if (p.R <= 1) hipLaunchKernelGGL((split_valu_kernel<QT, KT, 1>), grid, dim3(256), 0, s, p);
  else if (p.R <= 2) hipLaunchKernelGGL((split_valu_kernel<QT, KT, 2>), grid, dim3(256), 0, s, p);
  else if (p.R <= 4) hipLaunchKernelGGL((split_valu_kernel<QT, KT, 4>), grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((split_valu_kernel<QT, KT, 8>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_split_valu(int q_dtype, int kv_dtype, int D, const Params& p, hipStream_t s) {
  if (D != 128 || p.R > 8) return hipErrorInvalidValue;
  if (q_dtype == kBF16 && kv_dtype == kBF16) return launch_valu_rows<kBF16, kBF16>(p, s);
  if (q_dtype == kF16 && kv_dtype == kF16) return launch_valu_rows<kF16, kF16>(p, s);
  if (q_dtype == kBF16 && kv_dtype == kFP8) return launch_valu_rows<kBF16, kFP8>(p, s);
  if (q_dtype == kF16 && kv_dtype == kFP8) return launch_valu_rows<kF16, kFP8>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
