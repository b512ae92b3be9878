"""GPU parity of the latent-attention projections (pkv_head_matmul) and of the
whole absorbed decode: q_nope . W_UK_T, the query concat, the latent decode,
then . W_UV -- against the oracle's multi-head attention with K and V
materialised from the latent cache (random weights).

Head products: fp32 accumulation and one rounding, so each output is within
half an output ulp of the fp64 product plus the fp32 sum error, bounded by
K 2^-24 sum_k |x_k w_k| (the standard bound for a K-term float sum).
"""
import math

import pytest
import torch

import oracle
import paged_kv_attention_pages_amd as pkv
from paged_kv_attention_pages_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ulp(ref, dtype):
    mant = {torch.bfloat16: 7, torch.float16: 10}[dtype]
    e = torch.floor(torch.log2(ref.abs().clamp(min=2.0 ** -14)))
    return torch.exp2(e - mant)


def _check_products(y, x, w, label):
    """y (device, rounded) against the fp64 product: half an ulp of the output
    dtype at the larger of the two magnitudes, plus the fp32 sum bound."""
    ref = oracle.head_matmul(x, w)
    got = y.double().cpu()
    K = x.shape[-1]
    sum_bound = K * 2.0 ** -24 * oracle.head_matmul(x.double().abs(), w.double().abs())
    allow = 0.5 * _ulp(torch.maximum(ref.abs(), got.abs()), y.dtype) + sum_bound
    ratio = ((got - ref).abs() / allow).max().item()
    print(f"[parity] {label}: max error / allowance = {ratio:.3f}", flush=True)
    assert ratio <= 1.0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("M, H, K, N", [(32, 64, 128, 512), (32, 64, 512, 128), (1, 3, 32, 64),
                                        (45, 5, 96, 192), (200, 2, 64, 64)])
def test_head_matmul_matches_oracle(M, H, K, N, dtype):
    g = torch.Generator().manual_seed(M + H + K + N)
    x = torch.randn(M, H, K, generator=g).to(dtype)
    w = (torch.randn(H, K, N, generator=g) / math.sqrt(K)).to(dtype)
    y = pkv.head_matmul(x.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    _check_products(y, x, w, f"head_matmul {M}x{H}x{K}x{N} {dtype}")


def test_head_matmul_strided_views():
    # x is the q_nope slice of q [M, H, 192]; y a slice of a wider buffer
    g = torch.Generator().manual_seed(7)
    q = torch.randn(20, 8, 192, generator=g).to(torch.bfloat16).to(DEV)
    w = (torch.randn(8, 128, 512, generator=g) / math.sqrt(128)).to(torch.bfloat16).to(DEV)
    buf = torch.full((20, 8, 576), float("nan"), dtype=torch.bfloat16, device=DEV)
    pkv.head_matmul(q[..., :128], w, buf[..., :512])
    torch.cuda.synchronize()
    _check_products(buf[..., :512], q[..., :128].cpu(), w.cpu(), "head_matmul strided")
    assert torch.isnan(buf[..., 512:].float()).all()        # nothing written past the view


def test_absorbed_latent_decode_matches_materialised_attention():
    w = synth.WORKLOADS["mla"].replace(batch=4, seq_len_range=(50, 1500))
    inp = synth.make_inputs(w, 31, DEV, poison=False)
    g = torch.Generator().manual_seed(32)
    B, H, P, L, V = w.batch, w.num_q_heads, 128, 512, 128
    q_nope = torch.randn(B, H, P, generator=g).to(torch.bfloat16)
    q_pe = inp["q"].reshape(B, H, 576)[:, :, L:].contiguous()
    w_uk_t = (torch.randn(H, P, L, generator=g) / math.sqrt(P)).to(torch.bfloat16)
    w_uv = (torch.randn(H, L, V, generator=g) / math.sqrt(L)).to(torch.bfloat16)
    # GPU: BMM1, the query concat (the insert's fused form, no rows to insert),
    # the latent decode, the up-projection
    ql = pkv.head_matmul(q_nope.to(DEV), w_uk_t.to(DEV))
    mqa_q = torch.empty(B, H, 576, dtype=torch.bfloat16, device=DEV)
    none = torch.full((B,), -1, dtype=torch.int64, device=DEV)
    dummy = torch.zeros(B, 1, L, dtype=torch.bfloat16, device=DEV)
    dummy_pe = torch.zeros(B, 1, 64, dtype=torch.bfloat16, device=DEV)
    pkv.cache_insert(inp["k_cache"], None, none, dummy, k_rope=dummy_pe, page_size=w.page_size,
                     q_lo=ql, q_hi=q_pe.to(DEV), q_out=mqa_q)
    lat = torch.empty(B, 1, H, L, dtype=torch.bfloat16, device=DEV)
    pkv.decode_attn(mqa_q.view(B, 1, H, 576), inp["k_cache"], inp["k_cache"], inp["page_table"],
                    inp["seq_lens"], lat, num_kv_heads=1, page_size=w.page_size,
                    q_scale=math.sqrt(576 / 192), kv_layout=w.kv_layout, head_dim_v=L)
    out = pkv.head_matmul(lat.view(B, H, L), w_uv.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.mla_materialised(q_nope, q_pe, inp["k_cache"], inp["page_table"].cpu(),
                                  inp["seq_lens"].cpu(), w_uk_t, w_uv, page_size=w.page_size,
                                  softmax_scale=192 ** -0.5)
    err = (out.double().cpu() - ref).abs().max().item()
    rms = ref.pow(2).mean().sqrt().item()
    print(f"[parity] absorbed-vs-materialised max_abs={err:.3e} rms_ref={rms:.3e}", flush=True)
    # three bf16 roundings (absorbed query, latent output, projection) on
    # O(0.1-1) values: the decode's own bound 1e-2 covers them
    assert err <= 1e-2
