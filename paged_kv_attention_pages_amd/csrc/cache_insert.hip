// cache_insert.hip -- the write side of the paged cache: the new tokens'
// rows go to their slots (slot = page * page_size + offset), with a
// quantising store for an E4M3 cache, and, in the same launch, the latent
// attention's decode query concat.
//
// vLLM `models/kimi_k3/nvidia/mla` page, `_decode_concat_cache`: one fused
// step writes each decode token's latent row [kv_c_normed | k_pe] into the
// paged cache at its slot_mapping entry (an fp8 cache stores the row times
// `cache_scale_inv`, the reciprocal of the cache scale) and builds the query
// [ql_nope | q_pe].  For a K/V cache in the xqa page's NHD / HND layouts the
// same store is the step just before decode attention.
//
// Work item: 8 elements (16 source bytes) of one row.  Grid: x over the
// items of the largest part (256 per block), y = part (0: K rows, 1: V rows,
// 2: query concat).  Consecutive lanes take consecutive items of a row, so
// the source reads and the cache stores are contiguous runs.  Item indices
// are 32-bit (the host keeps every part under 2^31 items).
#include <algorithm>

#include "pkv_device.h"
#include "kernels.h"

namespace pkv {

namespace {

// Eight 16-bit source values times s as E4M3 bytes: binary32 products,
// magnitudes clamped to the largest finite value 448 (NaN passes through),
// then v_cvt_pk_fp8_f32, which rounds to nearest even.
template <int ST>
__device__ __forceinline__ uint2 to_e4m3x8(const uint4& v, float s) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float2 t = unpack2<ST>(w[i]);
    f[2 * i] = t.x * s;
    f[2 * i + 1] = t.y * s;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = f[i] != f[i] ? f[i] : fminf(fmaxf(f[i], -448.f), 448.f);
  uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
  uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
  return make_uint2(lo, hi);
}

template <int ST, bool FP8>
__global__ __launch_bounds__(256) void cache_insert_kernel(InsertParams p) {
  const int part = blockIdx.y;
  const uint32_t item = blockIdx.x * 256u + threadIdx.x;
  if (part == 2) {  // query concat: q_out[i, h] = [q_lo[i, h] | q_hi[i, h]]
    const uint32_t per_row = (uint32_t)p.Dk >> 3;
    if (item >= (uint32_t)p.N * (uint32_t)p.Hq * per_row) return;
    const uint32_t row = item / per_row, d = (item - row * per_row) * 8;
    const uint16_t* src = (int)d < p.Dlo ? (const uint16_t*)p.q_lo + (int64_t)row * p.Dlo + d
                                         : (const uint16_t*)p.q_hi + (int64_t)row * (p.Dk - p.Dlo) + (d - p.Dlo);
    *(uint4*)((uint16_t*)p.q_out + (int64_t)row * p.Dk + d) = *(const uint4*)src;
    return;
  }
  const int D = part == 0 ? p.Dk : p.Dv;
  const uint32_t per_row = (uint32_t)D >> 3, per_token = (uint32_t)p.Hkv * per_row;
  if (item >= (uint32_t)p.N * per_token) return;
  const uint32_t i = item / per_token, rem = item - i * per_token;
  const uint32_t h = rem / per_row, d = (rem - h * per_row) * 8;
  const int64_t slot = p.slot_mapping[i];
  if (slot < 0 || slot >= (int64_t)p.num_pages * p.ps) return;  // padding / outside the pool
  const int64_t page = slot / p.ps;
  const int off = (int)(slot - page * p.ps);
  const int64_t row = (int64_t)i * p.Hkv + h;
  const uint16_t* src;
  if (part == 0)
    src = (int)d < p.Dlo ? (const uint16_t*)p.k_src + row * p.Dlo + d
                         : (const uint16_t*)p.k_rope + row * (p.Dk - p.Dlo) + (d - p.Dlo);
  else
    src = (const uint16_t*)p.v_src + row * p.Dv + d;
  const uint4 v = *(const uint4*)src;
  const int64_t e = p.layout == 0 ? ((page * p.ps + off) * p.Hkv + h) * D + d
                                  : ((page * p.Hkv + h) * p.ps + off) * D + d;
  void* cache = part == 0 ? p.k_cache : p.v_cache;
  if constexpr (FP8) {
    const float s = p.scale_inv_dev != nullptr ? *p.scale_inv_dev : p.scale_inv;
    *(uint2*)((uint8_t*)cache + e) = to_e4m3x8<ST>(v, s);
  } else {
    *(uint4*)((uint16_t*)cache + e) = v;
  }
}

}  // namespace

hipError_t launch_cache_insert(int src_dtype, int cache_dtype, const InsertParams& p, hipStream_t s) {
  const int64_t items_k = (int64_t)p.N * p.Hkv * (p.Dk / 8);
  const int64_t items_v = (int64_t)p.N * p.Hkv * (p.Dv / 8);
  const int64_t items_q = p.q_out != nullptr ? (int64_t)p.N * p.Hq * (p.Dk / 8) : 0;
  const int64_t items = std::max(items_k, std::max(items_v, items_q));
  if (items == 0) return hipSuccess;
  if (items >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((items + 255) / 256), items_q > 0 ? 3 : p.Dv > 0 ? 2 : 1);
  const bool fp8 = cache_dtype == kFP8;
  if (src_dtype == kBF16 && fp8)
    hipLaunchKernelGGL((cache_insert_kernel<kBF16, true>), grid, dim3(256), 0, s, p);
  else if (src_dtype == kBF16)
    hipLaunchKernelGGL((cache_insert_kernel<kBF16, false>), grid, dim3(256), 0, s, p);
  else if (fp8)
    hipLaunchKernelGGL((cache_insert_kernel<kF16, true>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((cache_insert_kernel<kF16, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pkv
