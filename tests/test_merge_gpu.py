"""GPU parity of pkv_merge_attn_states against the oracle's fp64 merge.

The kernel forms the weights in fp32 as exponentials of differences in
[-88, 0] (smaller ones underflow to weights below 2^-126): the argument's
rounding costs at most 88 2^-24 ~ 5.3e-6 relative and the exponential a few
fp32 ulps, the normalised weight w / (w_p + w_s) twice that, ~1.1e-5.  Two
products are summed and rounded once to the output dtype: each output is
within half an output ulp of the fp64 merge plus 2e-5 (|o_p| + |o_s|), and
each log-sum-exp within 1e-5 (1 + |lse|).
"""
import pytest
import torch

import oracle
import paged_kv_attention_pages_amd as pkv

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ulp(ref, dtype):
    mant = {torch.bfloat16: 7, torch.float16: 10}[dtype]
    e = torch.floor(torch.log2(ref.abs().clamp(min=2.0 ** -14)))
    return torch.exp2(e - mant)


def _inputs(N, H, D, dtype, seed, inf_frac=0.1, lse_scale=4.0, lse_nh=False):
    g = torch.Generator().manual_seed(seed)
    po = torch.randn(N, H, D, generator=g).to(dtype)
    so = torch.randn(N, H, D, generator=g).to(dtype)
    shape = (N, H) if lse_nh else (H, N)
    pl = torch.randn(*shape, generator=g) * lse_scale
    sl = torch.randn(*shape, generator=g) * lse_scale
    pl[torch.rand(*shape, generator=g) < inf_frac] = float("-inf")
    sl[torch.rand(*shape, generator=g) < inf_frac] = float("-inf")
    if lse_nh:               # [N, H] storage seen as [H, N] (strides 1, H)
        pl, sl = pl.t(), sl.t()
    return po, pl, so, sl


def _check(out, lse, po, pl, so, sl, n_pre, label):
    ref, ref_lse = oracle.merge_attn_states(po, pl, so, sl, n_pre)
    got = out.double().cpu()
    mag = so.double().abs() + torch.cat([po.double().abs()[:n_pre],
                                         torch.zeros_like(so.double()[n_pre:])])
    allow = 0.5 * _ulp(torch.maximum(ref.abs(), got.abs()), out.dtype) + 2e-5 * mag
    ratio = ((got - ref).abs() / allow).max().item() if got.numel() else 0.0
    print(f"[parity] {label}: max error / allowance = {ratio:.3f}", flush=True)
    assert ratio <= 1.0
    if lse is not None:
        gl = lse.double().cpu()
        fin = torch.isfinite(ref_lse)
        assert torch.equal(torch.isfinite(gl), fin)
        assert (gl[~fin] == float("-inf")).all()
        assert ((gl[fin] - ref_lse[fin]).abs() <= 1e-5 * (1 + ref_lse[fin].abs())).all()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("N, H, D, n_pre", [(37, 16, 128, 37), (37, 16, 128, 20), (5, 3, 512, 0),
                                            (1, 1, 8, 1), (300, 128, 128, 250), (64, 16, 576, 64)])
def test_merge_matches_oracle(N, H, D, n_pre, dtype):
    po, pl, so, sl = _inputs(N, H, D, dtype, seed=N * 7 + H + D + n_pre)
    out = torch.full((N, H, D), float("nan"), dtype=dtype, device=DEV)
    lse = torch.full((H, N), float("nan"), device=DEV)
    pkv.merge_attn_states(out, po.to(DEV), pl.to(DEV), so.to(DEV), sl.to(DEV), n_pre, lse)
    torch.cuda.synchronize()
    _check(out, lse, po, pl, so, sl, n_pre, f"merge {N}x{H}x{D} prefix {n_pre} {dtype}")


def test_merge_without_prefix_arrays_takes_the_suffix():
    po, pl, so, sl = _inputs(9, 4, 64, torch.bfloat16, seed=3)
    out = torch.empty(9, 4, 64, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(4, 9, device=DEV)
    pkv.merge_attn_states(out, None, None, so.to(DEV), sl.to(DEV), 0, lse)
    torch.cuda.synchronize()
    fin = torch.isfinite(sl).t()[..., None].expand(9, 4, 64)
    assert torch.equal(out.cpu()[fin], so[fin])           # weight 1, exactly the suffix
    assert (out.cpu()[~fin] == 0).all()
    assert torch.equal(lse.cpu().isfinite(), sl.isfinite())


def test_merge_nh_lse_layout_in_place_and_large_lse():
    # log-sum-exps stored [N, H]; output aliases the suffix; log-sum-exps of
    # magnitude ~ 200 (e^lse overflows fp32: the max is subtracted first)
    N, H, D = 40, 8, 256
    po, pl, so, sl = _inputs(N, H, D, torch.float16, seed=11, lse_scale=200.0, lse_nh=True)
    s_dev = so.to(DEV)
    lse = torch.empty(N, H, device=DEV).t()
    pkv.merge_attn_states(s_dev, po.to(DEV), pl.to(DEV), s_dev, sl.to(DEV), N, lse)
    torch.cuda.synchronize()
    _check(s_dev, lse, po, pl, so, sl, N, "merge [N,H] lse, in place, |lse| ~ 200")


def test_merge_both_empty_gives_zeros_and_no_lse_output():
    N, H, D = 6, 2, 32
    po, pl, so, sl = _inputs(N, H, D, torch.bfloat16, seed=5, inf_frac=1.1)
    out = torch.full((N, H, D), 7.0, dtype=torch.bfloat16, device=DEV)
    pkv.merge_attn_states(out, po.to(DEV), pl.to(DEV), so.to(DEV), sl.to(DEV))
    torch.cuda.synchronize()
    assert (out == 0).all()


def test_merge_empty_call_is_a_noop():
    out = torch.empty(0, 4, 64, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(4, 0, device=DEV)
    pkv.merge_attn_states(out, out, lse, out, lse, 0, lse)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_merge_strided_results(dtype):
    # the page merges the leading v_head_dim (128) entries of 192-wide prefix
    # rows and 256-wide suffix rows
    N, H, D = 50, 16, 128
    po, pl, so, sl = _inputs(N, H, D, dtype, seed=21)
    g = torch.Generator().manual_seed(22)
    pw = torch.randn(N, H, 192, generator=g).to(dtype)
    sw = torch.randn(N, H, 256, generator=g).to(dtype)
    pw[..., :D] = po
    sw[..., :D] = so
    out = torch.empty(N, H, D, dtype=dtype, device=DEV)
    lse = torch.empty(H, N, device=DEV)
    pkv.merge_attn_states(out, pw.to(DEV)[..., :D], pl.to(DEV), sw.to(DEV)[..., :D], sl.to(DEV), 31, lse)
    torch.cuda.synchronize()
    _check(out, lse, po, pl, so, sl, 31, f"merge strided {dtype}")


def test_merge_rejects_aliasing_a_strided_suffix():
    sw = torch.zeros(4, 2, 128, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(2, 4, device=DEV)
    with pytest.raises(pkv.PkvError, match="contiguous"):
        pkv.merge_attn_states(sw[..., :64], None, None, sw[..., :64], lse, 0)
