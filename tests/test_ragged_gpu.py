"""GPU parity of pkv_ragged_attn (ragged, non-paged attention with its
log-sum-exp) against the oracle's fp64 ragged attention.

Outputs: the max-abs bound of the decode path (1e-2 bf16, 4e-3 f16 on N(0,1)
inputs), with half an output ulp where the dtype cannot hold the exact value
that closely.  Log-sum-exps: the kernel sums the probabilities after their
rounding to the 16-bit operand type, each within the unit roundoff u of its
exact value (u = 2^-8 for bf16, 2^-11 for f16), so the sum is too and
|lse - ref| <= -log(1 - u) ~ u, plus fp32 slack.
"""
import math

import pytest
import torch

import oracle
import paged_kv_attention_pages_amd as pkv
from paged_kv_attention_pages_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {torch.bfloat16: 1e-2, torch.float16: 4e-3}
LSE_TOL = {torch.bfloat16: 2.0 ** -8 + 1e-5, torch.float16: 2.0 ** -11 + 1e-5}


def _half_ulp(ref, dtype):
    mant = {torch.bfloat16: 7, torch.float16: 10}[dtype]
    e = torch.floor(torch.log2(ref.abs().clamp(min=2.0 ** -14)))
    return 0.5 * torch.exp2(e - mant)


def _check(out, lse, ref, ref_lse, dtype, label):
    got = out.double().cpu()
    assert not torch.isnan(got).any(), f"{label}: NaN in output"
    d = (got - ref).abs()
    allowed = torch.clamp(_half_ulp(ref, dtype) + 0.5 * TOL[dtype], min=TOL[dtype])
    err = d.max().item() if d.numel() else 0.0
    print(f"[parity] ragged {label}: max_abs={err:.3e}", flush=True)
    assert not (d > allowed).any(), f"{label}: max abs err {err}"
    if lse is not None:
        gl = lse.double().cpu()
        fin = torch.isfinite(ref_lse)
        assert torch.equal(torch.isfinite(gl), fin), f"{label}: -inf rows differ"
        assert (gl[~fin] == float("-inf")).all()
        lerr = (gl[fin] - ref_lse[fin]).abs().max().item() if fin.any() else 0.0
        print(f"[parity] ragged {label}: lse max_abs={lerr:.3e}", flush=True)
        assert lerr <= LSE_TOL[dtype]


def _run(lens_q, lens_k, Hq, Hkv, Dqk, Dv, dtype, causal, seed, scale=None, max_q_len=None):
    inp = synth.make_ragged(lens_q, lens_k, Hq, Hkv, Dqk, Dv, dtype, seed, DEV)
    scale = Dqk ** -0.5 if scale is None else scale
    mq = inp["max_q_len"] if max_q_len is None else max_q_len
    out, lse = pkv.ragged_attn(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_q"],
                               inp["cu_seqlens_k"], max_q_len=mq, sm_scale=scale, causal=causal,
                               return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.ragged_attn(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_q_host"],
                                      inp["cu_seqlens_k_host"], sm_scale=scale, causal=causal)
    return out, lse, ref, ref_lse


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("dims", [(128, 128), (192, 128), (64, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_parity(dtype, dims, causal):
    # ragged lengths across several 64-query blocks and 16-key tiles, with
    # ragged tails, a single query, more keys than queries, and (causal) a
    # sequence with fewer keys than queries (its first rows see nothing)
    lens_q = [1, 17, 64, 130, 5, 40]
    lens_k = [1, 17, 64, 130, 300, 23] if causal else [9, 1, 64, 77, 300, 0]
    out, lse, ref, ref_lse = _run(lens_q, lens_k, 8, 2, dims[0], dims[1], dtype, causal, seed=3)
    _check(out, lse, ref, ref_lse, dtype, f"{dtype} {dims} causal={causal}")


@pytest.mark.parametrize("Hq, Hkv", [(4, 4), (16, 1), (6, 3)])
def test_ragged_head_groupings(Hq, Hkv):
    out, lse, ref, ref_lse = _run([33, 70], [33, 90], Hq, Hkv, 128, 128, torch.bfloat16, True, seed=4)
    _check(out, lse, ref, ref_lse, torch.bfloat16, f"Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("lens", [[300], [300, 260, 129, 385], [640, 1, 129], [0, 511, 128]])
def test_ragged_causal_block_pairs(lens):
    # a causal workgroup takes query blocks j and last - j of one pair: odd
    # and even block counts (3, 4, 5 and 4 blocks of 128 queries), sequences
    # shorter than max_q_len (their later blocks have no rows) and empty ones
    out, lse, ref, ref_lse = _run(lens, lens, 8, 2, 192, 128, torch.bfloat16, True, seed=8)
    _check(out, lse, ref, ref_lse, torch.bfloat16, f"pairs {lens}")


def test_ragged_long_sequence_and_scale():
    # 1000 queries over 1500 keys (16 query blocks of 64, 94 key tiles); a
    # larger softmax scale sharpens the weights
    out, lse, ref, ref_lse = _run([1000], [1500], 2, 1, 192, 128, torch.bfloat16, True, seed=5,
                                  scale=0.2)
    _check(out, lse, ref, ref_lse, torch.bfloat16, "long")


def test_ragged_empty_cases():
    # no keys at all: zeros and -inf; a zero-length query range between others
    out, lse, ref, ref_lse = _run([3, 0, 4], [0, 5, 0], 2, 2, 64, 64, torch.float16, False, seed=6)
    assert torch.equal(out[:3].cpu(), torch.zeros_like(out[:3].cpu()))
    _check(out, lse, ref, ref_lse, torch.float16, "empty")
    # nothing to do: no sequences / no queries
    q = torch.zeros((0, 2, 64), dtype=torch.float16, device=DEV)
    kv = torch.zeros((0, 2, 64), dtype=torch.float16, device=DEV)
    cu = torch.zeros(1, dtype=torch.int32, device=DEV)
    o = pkv.ragged_attn(q, kv, kv, cu, cu, max_q_len=0, sm_scale=1.0)
    assert o.shape == (0, 2, 64)


def test_ragged_rows_past_max_q_len_are_not_written():
    inp = synth.make_ragged([40], [40], 2, 2, 64, 64, torch.bfloat16, 7, DEV)
    out = torch.full((40, 2, 64), 7.0, dtype=torch.bfloat16, device=DEV)
    pkv.ragged_attn(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                    max_q_len=16, sm_scale=0.125, causal=True, out=out)
    torch.cuda.synchronize()
    ref, _ = oracle.ragged_attn(inp["q"], inp["k"], inp["v"], [0, 40], [0, 40], sm_scale=0.125,
                                causal=True)
    assert (out[16:].float() == 7.0).all()
    _check(out[:16], None, ref[:16], None, torch.bfloat16, "max_q_len")


def test_chunked_prefill_pipeline_matches_causal_attention():
    # Kimi-K3 chunked prefill on the GPU: new tokens over the cached context
    # (not causal) and over themselves (causal), merged by their log-sum-exps
    # with pkv_merge_attn_states, equal causal attention over context + new
    C, N, Hq, Hkv, D = 300, 90, 8, 8, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    q = torch.randn((N, Hq, 192), generator=g, device=DEV).to(torch.bfloat16)
    k = torch.randn((C + N, Hkv, 192), generator=g, device=DEV).to(torch.bfloat16)
    v = torch.randn((C + N, Hkv, D), generator=g, device=DEV).to(torch.bfloat16)
    scale = 192 ** -0.5
    cu_n = torch.tensor([0, N], dtype=torch.int32, device=DEV)
    cu_c = torch.tensor([0, C], dtype=torch.int32, device=DEV)
    ctx_o, ctx_l = pkv.ragged_attn(q, k[:C].contiguous(), v[:C].contiguous(), cu_n, cu_c,
                                   max_q_len=N, sm_scale=scale, causal=False, return_lse=True)
    new_o, new_l = pkv.ragged_attn(q, k[C:].contiguous(), v[C:].contiguous(), cu_n, cu_n,
                                   max_q_len=N, sm_scale=scale, causal=True, return_lse=True)
    out = torch.empty_like(new_o)
    out_lse = torch.empty_like(new_l)
    pkv.merge_attn_states(out, ctx_o, ctx_l, new_o, new_l, output_lse=out_lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.ragged_attn(q, k, v, [0, N], [0, C + N], sm_scale=scale, causal=True)
    # two roundings of each part to bf16 before the merge: twice the bound
    got = out.double().cpu()
    d = (got - ref).abs().max().item()
    print(f"[parity] chunked prefill pipeline: max_abs={d:.3e}", flush=True)
    assert d <= 2 * TOL[torch.bfloat16]
    assert (out_lse.double().cpu() - ref_lse).abs().max().item() <= 2 * LSE_TOL[torch.bfloat16]


def test_ragged_bad_arguments_are_rejected():
    inp = synth.make_ragged([4], [4], 2, 2, 64, 64, torch.bfloat16, 8, DEV)
    with pytest.raises(pkv.PkvError):     # head dims not supported
        x = torch.zeros((4, 2, 96), dtype=torch.bfloat16, device=DEV)
        pkv.ragged_attn(x, x, x, inp["cu_seqlens_q"], inp["cu_seqlens_k"], max_q_len=4,
                        sm_scale=1.0)
    with pytest.raises(pkv.PkvError):     # Hq not a multiple of Hkv
        k3 = torch.zeros((4, 3, 64), dtype=torch.bfloat16, device=DEV)
        pkv.ragged_attn(inp["q"], k3, k3, inp["cu_seqlens_q"], inp["cu_seqlens_k"], max_q_len=4,
                        sm_scale=1.0)
    with pytest.raises(pkv.PkvError):     # non-finite scale
        pkv.ragged_attn(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                        max_q_len=4, sm_scale=math.inf)


def test_ragged_graph_capture_replays_match_eager():
    # the call allocates nothing and issues one kernel, so it can be captured;
    # each replay, with eager work in between, gives the eager result
    inp = synth.make_ragged([70, 33], [90, 33], 4, 2, 128, 128, torch.bfloat16, 9, DEV)
    out = torch.empty((103, 4, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((4, 103), dtype=torch.float32, device=DEV)

    def call():
        pkv.ragged_attn(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                        max_q_len=70, sm_scale=0.1, causal=True, out=out, lse=lse)

    call()
    torch.cuda.synchronize()
    want, want_lse = out.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                                   # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for _ in range(3):
        out.fill_(0)
        lse.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want) and torch.equal(lse, want_lse)


# the two ragged bench workloads, at their full sizes: qk 192 / v 128, 64 heads,
# 4 x 4096 new tokens (causal) and 2 x 1024 queries over 16384 keys
FULL = {
    "ragged_prefill": dict(lens_q=[4096] * 4, lens_k=[4096] * 4, causal=True),
    "ragged_context": dict(lens_q=[1024] * 2, lens_k=[16384] * 2, causal=False),
}


@pytest.mark.parametrize("name", list(FULL))
def test_ragged_full_size_sampled(name):
    # one launch at the full size; sampled (sequence, query, head) outputs and
    # log-sum-exps against the oracle, each computed alone: query i of a
    # causal sequence attends exactly its first i + 1 + Lk - Lq keys
    cfg = FULL[name]
    H, Dqk, Dv = 64, 192, 128
    print(f"[case] ragged full {name}", flush=True)
    inp = synth.make_ragged(cfg["lens_q"], cfg["lens_k"], H, H, Dqk, Dv, torch.bfloat16, 1, DEV)
    scale = Dqk ** -0.5
    out, lse = pkv.ragged_attn(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_q"],
                               inp["cu_seqlens_k"], max_q_len=inp["max_q_len"], sm_scale=scale,
                               causal=cfg["causal"], return_lse=True)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    cq, ck = inp["cu_seqlens_q_host"], inp["cu_seqlens_k_host"]
    g = torch.Generator().manual_seed(2)
    worst = 0.0
    for s in range(len(cfg["lens_q"])):
        Lq, Lk = cfg["lens_q"][s], cfg["lens_k"][s]
        queries = sorted({0, Lq - 1, *torch.randint(0, Lq, (4,), generator=g).tolist()})
        for i in queries:
            h = int(torch.randint(0, H, (1,), generator=g))
            n = min(Lk, i + 1 + Lk - Lq) if cfg["causal"] else Lk
            row = cq[s] + i
            q1 = inp["q"][row:row + 1, h:h + 1].cpu()
            k1 = inp["k"][ck[s]:ck[s] + n, h:h + 1].cpu()
            v1 = inp["v"][ck[s]:ck[s] + n, h:h + 1].cpu()
            ref, ref_lse = oracle.ragged_attn(q1, k1, v1, [0, 1], [0, n], sm_scale=scale,
                                              causal=False)
            got = out[row, h].double().cpu()
            d = (got - ref[0, 0]).abs()
            allowed = torch.clamp(_half_ulp(ref[0, 0], torch.bfloat16) + 0.5 * TOL[torch.bfloat16],
                                  min=TOL[torch.bfloat16])
            assert not (d > allowed).any(), f"{name} seq {s} query {i} head {h}: {d.max().item()}"
            assert abs(float(lse[h, row]) - float(ref_lse[0, 0])) <= LSE_TOL[torch.bfloat16]
            worst = max(worst, d.max().item())
    print(f"[parity] ragged full {name}: max_abs={worst:.3e}", flush=True)
