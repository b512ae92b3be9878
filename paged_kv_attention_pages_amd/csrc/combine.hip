// combine.hip -- merge of split-KV partial results.
//
// Each split s of a (sequence, KV head) left, per query row, its running max
// m_s (log2 units), its running sum l_s and its unnormalised output o_s.  The
// exact softmax over the union of the splits is
//   M   = max(max_s m_s, sink),
//   out = kv_scale * sum_s 2^(m_s - M) o_s / (sum_s 2^(m_s - M) l_s + 2^(sink - M)),
// the same log-sum-exp merge the vLLM Kimi-K3 MLA page applies to prefix and
// suffix attention states (`merge_attn_states`).  The sink enters here once
// per row, never per split.  Sequences that fit one split were finished by
// the split kernel; sequences with nothing visible get zeros.
#include "pkv_device.h"
#include "kernels.h"

namespace pkv {

namespace {
constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
}  // namespace

// grid (rows, Hkv, B), one wave per row; lane handles 4 consecutive dims
template <int QT>
__global__ __launch_bounds__(64) void combine_kernel(Params p) {
  resolve_scales(p);
  const int r = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const SeqGeom sg = seq_geom(p, b);
  if (sg.nsplits == 1) return;
  const int lane = threadIdx.x;
  const int64_t ob = q_row_offset(p, b, kvh, r) * p.Dv;
  if (sg.nsplits == 0) {
    for (int d = lane * 4; d < p.Dv; d += 256) store_out4<QT>(p, ob + d, 0.f, 0.f, 0.f, 0.f);
    return;
  }
  const int64_t base = ((int64_t)b * p.Hkv + kvh) * p.max_splits * p.R + r;  // split stride R
  float M = kNegInf;
  for (int s = 0; s < sg.nsplits; ++s) M = fmaxf(M, p.ws_ml[base + (int64_t)s * p.R].x);
  float sk = kNegInf;
  if (p.sinks != nullptr) sk = p.sinks[kvh * p.G + r % p.G] * kLog2e;
  const float Mf = fmaxf(M, sk);
  float den = p.sinks != nullptr ? exp2f(sk - Mf) : 0.f;
  for (int s = 0; s < sg.nsplits; ++s) {
    const float2 ml = p.ws_ml[base + (int64_t)s * p.R];
    if (ml.x != kNegInf) den += ml.y * exp2f(ml.x - Mf);
  }
  const float inv = den > 0.f ? p.out_scale / den : 0.f;
  for (int d = lane * 4; d < p.Dv; d += 256) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < sg.nsplits; ++s) {
      const int64_t prow = base + (int64_t)s * p.R;
      const float mx = p.ws_ml[prow].x;
      if (mx == kNegInf) continue;
      const float w = exp2f(mx - Mf);
      const float4 v = *(const float4*)(p.ws_o + prow * p.Dv + d);
      a.x += w * v.x; a.y += w * v.y; a.z += w * v.z; a.w += w * v.w;
    }
    store_out4<QT>(p, ob + d, a.x * inv, a.y * inv, a.z * inv, a.w * inv);
  }
}

// Stream-K schedule: unit (b, kvh) was cut across waves w0..w1 when its tiles
// span more than one wave's share.  Wave w0 left its piece in slot 2 w0 (when
// the unit is its first) or 2 w0 + 1 (its last); every later wave up to w1
// has the unit first and left slot 2 w.  Units held by one wave were finished
// by the split kernel; units with no tiles get zeros here.  Under the
// one-wave-per-unit plan with even units nothing was cut and every wave exits.
// One wave per (unit, group of 64 / (DV / 8) rows): each row's DV / 8 lanes
// hold 8 consecutive dims.  The slots are merged in chunks of 8 whose (m, l)
// pairs and partial outputs are all loaded before any is used -- one memory
// round trip per chunk -- with the running reference moved between chunks.
template <int QT, int DV, int SC>
__global__ __launch_bounds__(64) void combine_sk_kernel(Params p) {
  constexpr int LPR = DV / 8, RPW = 64 / LPR, CH = 8;
  resolve_scales(p);
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, li = lane % LPR;
  const int r = blockIdx.x * RPW + lane / LPR;
  const bool row_ok = r < p.R;
  const int rr = row_ok ? r : 0;  // lanes past the last row read row 0 and store nothing
  const SkSchedC<SC> S = sk_schedule<SC>(p);
  // the split kernel gave every unit a wave of its own: nothing was cut
  if (p.sk_units && sk_units_even(p, S)) return;
  const int W = sk_waves_eff(S.T, p.sk_waves);
  int pre, n;
  sk_seq_of(S, b, &pre, &n);
  const int64_t ob = q_row_offset(p, b, kvh, rr) * DV + 8 * li;
  if (n == 0) {
    if (row_ok) {
      store_out4<QT>(p, ob, 0.f, 0.f, 0.f, 0.f);
      store_out4<QT>(p, ob + 4, 0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  const int64_t us = sk_unit_start(S, kvh, pre), ue = us + n;
  const int w0 = sk_wave_of(S.T, us, W), w1 = sk_wave_of(S.T, ue - 1, W);
  if (w0 == w1) return;
  const int64_t slot0 = sk_wave_start(S.T, w0, W) == us ? 2 * (int64_t)w0 : 2 * (int64_t)w0 + 1;
  const int nslots = w1 - w0 + 1;
  // the sink term enters once: as the starting reference with weight 1
  float M = kNegInf, den = 0.f;
  if (p.sinks != nullptr) {
    M = p.sinks[kvh * p.G + rr % p.G] * kLog2e;
    den = 1.f;
  }
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  for (int j0 = 0; j0 < nslots; j0 += CH) {
    float2 ml[CH];
    float4 v[CH][2];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      // slots past the last are read as slot0 (in bounds) and weighted 0
      const int j = j0 + u;
      const int64_t prow = (j >= nslots ? slot0 : j == 0 ? slot0 : 2 * (int64_t)(w0 + j)) * p.R + rr;
      ml[u] = p.ws_ml[prow];
      const float4* src = (const float4*)(p.ws_o + prow * DV + 8 * li);
      v[u][0] = src[0];
      v[u][1] = src[1];
    }
    float Mc = M;
#pragma unroll
    for (int u = 0; u < CH; ++u)
      if (j0 + u < nslots) Mc = fmaxf(Mc, ml[u].x);
    if (Mc == kNegInf) continue;  // nothing visible so far
    const float scale = exp2f(M - Mc);  // 0 when M is -inf
    den *= scale;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] *= scale;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const float wu = (j0 + u < nslots && ml[u].x != kNegInf) ? exp2f(ml[u].x - Mc) : 0.f;
      den += wu * ml[u].y;
      acc[0] += wu * v[u][0].x; acc[1] += wu * v[u][0].y; acc[2] += wu * v[u][0].z; acc[3] += wu * v[u][0].w;
      acc[4] += wu * v[u][1].x; acc[5] += wu * v[u][1].y; acc[6] += wu * v[u][1].z; acc[7] += wu * v[u][1].w;
    }
    M = Mc;
  }
  if (!row_ok) return;
  const float inv = den > 0.f ? p.out_scale / den : 0.f;
  store_out4<QT>(p, ob, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  store_out4<QT>(p, ob + 4, acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
}

// Stream-K merge of the latent kernel's partials (split_mla_ws.hip), which
// sit in the P.V waves' register order: slot s holds, for P.V wave pw (rows
// 32 (pw / 2) .., dims 256 (pw % 2) ..), element (j, 4 q + e) of lane l at
// float ((s * 4 + pw) * 32 + 4 j + q) * 256 + 4 l + e, where lane l holds row
// 32 (pw / 2) + l % 32 and dims 256 (pw % 2) + 32 j + 8 q + 4 (l / 32) + e;
// (m, l) of row r at ws_ml[64 s + r].  One wave per (unit, P.V block, j):
// each lane merges 16 values of its row over the unit's slots, in chunks of 8
// slots loaded together (one memory round trip per chunk), and every load
// instruction reads 1 KB contiguously.
template <int QT>
__global__ __launch_bounds__(64) void combine_lat_kernel(Params p) {
  constexpr int CH = 8;
  resolve_scales(p);
  const int pw = blockIdx.x >> 3, j = blockIdx.x & 7, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int r = 32 * (pw >> 1) + (lane & 31);
  const bool row_ok = r < p.R;
  const int rr = row_ok ? r : 0;  // lanes past the last row read row 0 and store nothing
  const SkSched S = sk_schedule(p);
  const int W = sk_waves_eff(S.T, p.sk_waves);
  int pre, n;
  sk_seq_of(S, b, &pre, &n);
  const int64_t ob = q_row_offset(p, b, kvh, rr) * p.Dv + 256 * (pw & 1) + 32 * j + 4 * h;
  if (n == 0) {
    if (row_ok)
#pragma unroll
      for (int q = 0; q < 4; ++q) store_out4<QT>(p, ob + 8 * q, 0.f, 0.f, 0.f, 0.f);
    return;
  }
  const int64_t us = sk_unit_start(S, kvh, pre), ue = us + n;
  const int w0 = sk_wave_of(S.T, us, W), w1 = sk_wave_of(S.T, ue - 1, W);
  if (w0 == w1) return;
  const int64_t slot0 = sk_wave_start(S.T, w0, W) == us ? 2 * (int64_t)w0 : 2 * (int64_t)w0 + 1;
  const int nslots = w1 - w0 + 1;
  float M = kNegInf, den = 0.f;
  if (p.sinks != nullptr) {
    M = p.sinks[kvh * p.G + rr % p.G] * kLog2e;
    den = 1.f;
  }
  float acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = 0.f;
  for (int j0 = 0; j0 < nslots; j0 += CH) {
    float2 ml[CH];
    float4 v[CH][4];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int js = j0 + u;
      const int64_t slot = js >= nslots || js == 0 ? slot0 : 2 * (int64_t)(w0 + js);
      ml[u] = p.ws_ml[slot * 64 + rr];
      const float4* src = (const float4*)(p.ws_o + ((slot * 4 + pw) * 32 + 4 * j) * 256) + lane;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[u][q] = src[64 * q];
    }
    float Mc = M;
#pragma unroll
    for (int u = 0; u < CH; ++u)
      if (j0 + u < nslots) Mc = fmaxf(Mc, ml[u].x);
    if (Mc == kNegInf) continue;
    const float scale = exp2f(M - Mc);
    den *= scale;
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] *= scale;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const float wu = (j0 + u < nslots && ml[u].x != kNegInf) ? exp2f(ml[u].x - Mc) : 0.f;
      den += wu * ml[u].y;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[4 * q] += wu * v[u][q].x;
        acc[4 * q + 1] += wu * v[u][q].y;
        acc[4 * q + 2] += wu * v[u][q].z;
        acc[4 * q + 3] += wu * v[u][q].w;
      }
    }
    M = Mc;
  }
  if (!row_ok) return;
  const float inv = den > 0.f ? p.out_scale / den : 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    store_out4<QT>(p, ob + 8 * q, acc[4 * q] * inv, acc[4 * q + 1] * inv, acc[4 * q + 2] * inv,
                   acc[4 * q + 3] * inv);
}

hipError_t launch_combine(int q_dtype, const Params& p, hipStream_t s) {
  dim3 grid(p.R, p.Hkv, p.B);
  if (p.ws_lanes) {
    if (p.Dv != 512 || p.R > 64) return hipErrorInvalidValue;
    const dim3 lgrid(32, p.Hkv, p.B);
    if (q_dtype == kBF16)
      hipLaunchKernelGGL((combine_lat_kernel<kBF16>), lgrid, dim3(64), 0, s, p);
    else
      hipLaunchKernelGGL((combine_lat_kernel<kF16>), lgrid, dim3(64), 0, s, p);
    return hipGetLastError();
  }
  if (p.sk_waves > 0) {
    const bool wide = p.B > kSkMaxBatch;
    if (p.B > kSkMaxBatchWide) return hipErrorInvalidValue;
#define PKV_COMBINE_SK(DV)                                                                   \
  if (p.Dv == DV) {                                                                          \
    const dim3 ugrid((p.R + 64 / (DV / 8) - 1) / (64 / (DV / 8)), p.Hkv, p.B);              \
    if (q_dtype == kBF16 && !wide)                                                           \
      hipLaunchKernelGGL((combine_sk_kernel<kBF16, DV, 4>), ugrid, dim3(64), 0, s, p);       \
    else if (!wide)                                                                          \
      hipLaunchKernelGGL((combine_sk_kernel<kF16, DV, 4>), ugrid, dim3(64), 0, s, p);        \
    else if (q_dtype == kBF16)                                                               \
      hipLaunchKernelGGL((combine_sk_kernel<kBF16, DV, 16>), ugrid, dim3(64), 0, s, p);      \
    else                                                                                     \
      hipLaunchKernelGGL((combine_sk_kernel<kF16, DV, 16>), ugrid, dim3(64), 0, s, p);       \
    return hipGetLastError();                                                                \
  }
    PKV_COMBINE_SK(64)
    PKV_COMBINE_SK(128)
    PKV_COMBINE_SK(256)
    PKV_COMBINE_SK(512)
#undef PKV_COMBINE_SK
    return hipErrorInvalidValue;
  } else if (q_dtype == kBF16) {
    hipLaunchKernelGGL((combine_kernel<kBF16>), grid, dim3(64), 0, s, p);
  } else {
    hipLaunchKernelGGL((combine_kernel<kF16>), grid, dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace pkv
