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
// by the split kernel; units with no tiles get zeros here.
// Grid (Hkv, B, row groups of 4); wave v merges row 4 * group + v.  Lane j
// reads the (m, l) of slot j (in groups of 64), so the max and the
// denominator are wave reductions; the slot weights are then broadcast with
// readlane and eight slots' partial outputs are loaded at a time.
template <int QT>
__global__ __launch_bounds__(256) void combine_sk_kernel(Params p) {
  resolve_scales(p);
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.z * 4 + (threadIdx.x >> 6);
  if (r >= p.R) return;
  const SkSched S = sk_schedule(p);
  const int W = sk_waves_eff(S.T, p.sk_waves);
  int pre, n;
  sk_seq_of(S, b, &pre, &n);
  const int64_t ob = q_row_offset(p, b, kvh, r) * p.Dv;
  if (n == 0) {
    for (int d = lane; d < p.Dv; d += 64) store_out1<QT>(p, ob + d, 0.f);
    return;
  }
  const int64_t us = sk_unit_start(S, kvh, pre), ue = us + n;
  const int w0 = sk_wave_of(S.T, us, W), w1 = sk_wave_of(S.T, ue - 1, W);
  if (w0 == w1) return;
  const int64_t slot0 = sk_wave_start(S.T, w0, W) == us ? 2 * (int64_t)w0 : 2 * (int64_t)w0 + 1;
  const int nslots = w1 - w0 + 1;
  auto row_of = [&](int j) -> int64_t {
    return (j == 0 ? slot0 : 2 * (int64_t)(w0 + j)) * p.R + r;
  };
  float sk = kNegInf;
  if (p.sinks != nullptr) sk = p.sinks[kvh * p.G + r % p.G] * kLog2e;
  float M = sk;
  for (int j0 = 0; j0 < nslots; j0 += 64) {
    const int j = j0 + lane;
    M = fmaxf(M, j < nslots ? p.ws_ml[row_of(j)].x : kNegInf);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d));
  float den = p.sinks != nullptr ? exp2f(sk - M) : 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  const int per_lane = p.Dv >> 6;  // Dv in {64, 128, 256, 512}
  for (int j0 = 0; j0 < nslots; j0 += 64) {
    const int j = j0 + lane;
    float wt = 0.f, lsum = 0.f;
    if (j < nslots) {
      const float2 ml = p.ws_ml[row_of(j)];
      wt = ml.x == kNegInf ? 0.f : exp2f(ml.x - M);
      lsum = wt * ml.y;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) lsum += __shfl_xor(lsum, d);
    den += lsum;
    const int cnt = min(64, nslots - j0);
    for (int jb = 0; jb < cnt; jb += 8) {
      float v[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool ok = jb + u < cnt;
        const float* src = p.ws_o + row_of(j0 + (ok ? jb + u : 0)) * p.Dv + lane;
#pragma unroll
        for (int k = 0; k < 8; ++k) v[u][k] = (ok && k < per_lane) ? src[64 * k] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        // lanes past the last slot hold weight 0 (and their loads are zeros)
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), jb + u));
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] += wj * v[u][k];
      }
    }
  }
  const float inv = den > 0.f ? p.out_scale / den : 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k < per_lane) store_out1<QT>(p, ob + lane + 64 * k, acc[k] * inv);
}

hipError_t launch_combine(int q_dtype, const Params& p, hipStream_t s) {
  dim3 grid(p.R, p.Hkv, p.B);
  if (p.sk_waves > 0) {
    if (p.Dv > 512) return hipErrorInvalidValue;
    dim3 ugrid(p.Hkv, p.B, (p.R + 3) / 4);
    if (q_dtype == kBF16)
      hipLaunchKernelGGL((combine_sk_kernel<kBF16>), ugrid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((combine_sk_kernel<kF16>), ugrid, dim3(256), 0, s, p);
  } else if (q_dtype == kBF16) {
    hipLaunchKernelGGL((combine_kernel<kBF16>), grid, dim3(64), 0, s, p);
  } else {
    hipLaunchKernelGGL((combine_kernel<kF16>), grid, dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace pkv
