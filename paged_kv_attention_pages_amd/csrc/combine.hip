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
  const int r = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const SeqGeom sg = seq_geom(p, b);
  if (sg.nsplits == 1) return;
  const int lane = threadIdx.x;
  uint16_t* o = (uint16_t*)p.out + q_row_offset(p, b, kvh, r) * p.Dv;
  if (sg.nsplits == 0) {
    for (int d = lane * 4; d < p.Dv; d += 256) *(uint2*)(o + d) = make_uint2(0u, 0u);
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
    *(uint2*)(o + d) = make_uint2(pack2<QT>(a.x * inv, a.y * inv), pack2<QT>(a.z * inv, a.w * inv));
  }
}

hipError_t launch_combine(int q_dtype, const Params& p, hipStream_t s) {
  dim3 grid(p.R, p.Hkv, p.B);
  if (q_dtype == kBF16)
    hipLaunchKernelGGL((combine_kernel<kBF16>), grid, dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL((combine_kernel<kF16>), grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace pkv
