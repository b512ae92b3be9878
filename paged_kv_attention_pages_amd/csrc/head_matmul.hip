// head_matmul.hip -- the per-head products on either side of the latent
// (MLA) decode kernel:
//   y[m, h, 0:N] = x[m, h, 0:K] . W[h]      (W[h]: K x N, row-major)
// vLLM `models/kimi_k3/nvidia/mla` page, MultiHeadLatentAttention `_attention`
// decode branch: BMM1 absorbs q_nope into the latent space with W_UK_T
// ([heads, qk_nope_head_dim, kv_lora_rank]); `_v_up_proj` takes the
// kv_lora_rank-wide attention output back to v_head_dim with W_UV
// ([heads, kv_lora_rank, v_head_dim]).
//
// One wave per (64 output columns, head); it walks all M rows in blocks of
// 32.  Matrix cores, transposed so the weight is the A operand:
//   y^T (64 x 32) = W^T (64 x K) . x^T (K x 32)      16x16x32 MFMAs
// x^T's operand is a 16-byte load of 8 consecutive k of one row; W^T's
// operand gathers 8 rows of one weight column (2-byte loads: 16 lanes read
// 32 contiguous bytes of a weight row), so the weights are read once per
// wave and row block in their stored layout.  Each lane ends up with 4
// consecutive output columns of one row: 8-byte stores.  fp32 accumulation,
// one rounding to the output dtype.
#include "pkv_device.h"
#include "kernels.h"

namespace pkv {

namespace {

template <int QT>
__global__ __launch_bounds__(64) void head_matmul_kernel(HeadMatmulParams p) {
  const int lane = threadIdx.x, n = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 64, h = blockIdx.y;
  const uint16_t* w = (const uint16_t*)p.w + (int64_t)h * p.K * p.N + n0;
  const uint16_t* x = (const uint16_t*)p.x + (int64_t)h * p.xs_h;
  uint16_t* y = (uint16_t*)p.y + (int64_t)h * p.ys_h + n0;
  for (int m0 = 0; m0 < p.M; m0 += 32) {
    f32x4 acc[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t][0] = acc[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // rows of this block that exist (others read row 0 and are not stored)
    const int ma = m0 + n, mb = m0 + 16 + n;
    const uint16_t* xa = x + (int64_t)(ma < p.M ? ma : 0) * p.xs_m + 8 * g;
    const uint16_t* xb = x + (int64_t)(mb < p.M ? mb : 0) * p.xs_m + 8 * g;
    for (int k0 = 0; k0 < p.K; k0 += 32) {
      const uint4 ba = *(const uint4*)(xa + k0), bb = *(const uint4*)(xb + k0);
      // W^T operand of column block t: lane (n, g) takes W[k0 + 8 g + e][16 t + n], e < 8
      const uint16_t* wk = w + (int64_t)(k0 + 8 * g) * p.N + n;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t a[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a[e] = (uint32_t)wk[(int64_t)(2 * e) * p.N + 16 * t] |
                 ((uint32_t)wk[(int64_t)(2 * e + 1) * p.N + 16 * t] << 16);
        const uint4 av = make_uint4(a[0], a[1], a[2], a[3]);
        acc[t][0] = mfma_k32<QT>(av, ba, acc[t][0]);
        acc[t][1] = mfma_k32<QT>(av, bb, acc[t][1]);
      }
    }
    // lane (n, g) holds y^T[16 t + 4 g + i][row]: columns 16 t + 4 g .. + 3
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int m = r == 0 ? ma : mb;
      if (m >= p.M) continue;
      uint16_t* yr = y + (int64_t)m * p.ys_m;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        *(uint2*)(yr + 16 * t + 4 * g) = make_uint2(pack2<QT>(acc[t][r][0], acc[t][r][1]),
                                                    pack2<QT>(acc[t][r][2], acc[t][r][3]));
    }
  }
}

}  // namespace

hipError_t launch_head_matmul(int dtype, const HeadMatmulParams& p, hipStream_t s) {
  if (p.M == 0) return hipSuccess;
  const dim3 grid((unsigned)(p.N / 64), (unsigned)p.H);
  if (dtype == kBF16)
    hipLaunchKernelGGL((head_matmul_kernel<kBF16>), grid, dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL((head_matmul_kernel<kF16>), grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace pkv
