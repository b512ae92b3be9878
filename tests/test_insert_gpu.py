"""GPU parity of the cache write side (pkv_cache_insert) against the oracle.

The insert is byte work: every cache byte after the call must equal the
oracle's, bit for bit (16-bit caches: the source bits; E4M3 caches: the
round-to-nearest-even code of the binary32 product, saturated at 448).
Untouched slots, padding (-1) and slots past the pool must keep their bytes.
"""
import pytest
import torch

import oracle
import paged_kv_attention_pages_amd as pkv
from paged_kv_attention_pages_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    t = t.detach().cpu()
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.uint8)


def _case(layout, src, cache, N=37, Hkv=4, D=128, ps=16, P=40, seed=0):
    g = torch.Generator().manual_seed(seed)
    shape = (P, ps, Hkv, D) if layout == "NHD" else (P, Hkv, ps, D)
    kc = (torch.randn(shape, generator=g) * 4).to(cache)
    vc = (torch.randn(shape, generator=g) * 4).to(cache)
    k = (torch.randn(N, Hkv, D, generator=g) * 3).to(src)
    v = (torch.randn(N, Hkv, D, generator=g) * 3).to(src)
    slots = torch.randperm(P * ps, generator=g)[:N].to(torch.int64)
    slots[3] = -1
    slots[7] = P * ps + 5
    return kc, vc, k, v, slots


@pytest.mark.parametrize("ps", [16, 64])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("src, cache", [(torch.bfloat16, torch.bfloat16), (torch.float16, torch.float16),
                                        (torch.bfloat16, torch.float8_e4m3fn),
                                        (torch.float16, torch.float8_e4m3fn)])
def test_insert_matches_oracle(layout, src, cache, ps):
    print(f"[case] insert {layout} {src} -> {cache} ps={ps}", flush=True)
    kc, vc, k, v, slots = _case(layout, src, cache, ps=ps)
    s_inv = 7.5 if cache == torch.float8_e4m3fn else 1.0
    want_k, want_v = oracle.cache_insert(kc, vc, slots, k, v=v, page_size=ps, kv_layout=layout,
                                         cache_scale_inv=s_inv)
    gk, gv = kc.to(DEV), vc.to(DEV)
    pkv.cache_insert(gk, gv, slots.to(DEV), k.to(DEV), v=v.to(DEV), page_size=ps,
                     kv_layout=layout, cache_scale_inv=s_inv)
    torch.cuda.synchronize()
    assert torch.equal(_bits(gk), _bits(want_k))
    assert torch.equal(_bits(gv), _bits(want_v))


def test_insert_e4m3_rounding_and_saturation_vectors():
    # every midpoint between adjacent E4M3 values, one bf16 step either side
    # of it, values past 448 and NaN, through a scale of 1
    vals = [oracle.decode_e4m3fn(c) for c in range(0x7f)]
    mids = torch.tensor([(a + b) / 2 for a, b in zip(vals, vals[1:])], dtype=torch.float32)
    src = torch.cat([mids, -mids]).to(torch.bfloat16)
    up = (src.view(torch.int16) + 1).view(torch.bfloat16)   # the next bf16 away from zero
    src = torch.cat([src, up, torch.tensor([448.0, 460.0, 1e4, -1e4, 3e38, float("nan")],
                                           dtype=torch.bfloat16)])
    n = -(-src.numel() // 64)
    src = torch.cat([src, torch.zeros(n * 64 - src.numel(), dtype=torch.bfloat16)]).view(n, 1, 64)
    kc = torch.zeros(n, 16, 1, 64, dtype=torch.float8_e4m3fn)
    slots = torch.arange(n, dtype=torch.int64) * 16
    want, _ = oracle.cache_insert(kc, None, slots, src, page_size=16)
    g = kc.to(DEV)
    pkv.cache_insert(g, None, slots.to(DEV), src.to(DEV), page_size=16)
    torch.cuda.synchronize()
    got, ref = _bits(g).flatten(), _bits(want).flatten()
    nan_g = (got & 0x7F) == 0x7F
    nan_r = (ref & 0x7F) == 0x7F
    assert torch.equal(nan_g, nan_r)                       # NaN stays NaN (either sign)
    assert torch.equal(got[~nan_g], ref[~nan_r])


def test_insert_latent_row_and_query_concat():
    # latent cache: one KV head, row [kv_c_normed (512) | k_pe (64)], no V
    # cache; the same launch builds the decode query [ql_nope | q_pe]
    g = torch.Generator().manual_seed(4)
    N, Hq, P, ps = 33, 16, 12, 64
    cache = torch.randn(P, ps, 1, 576, generator=g).to(torch.bfloat16)
    kvc = torch.randn(N, 1, 512, generator=g).to(torch.bfloat16)
    kpe = torch.randn(N, 1, 64, generator=g).to(torch.bfloat16)
    ql = torch.randn(N, Hq, 512, generator=g).to(torch.bfloat16)
    qp = torch.randn(N, Hq, 64, generator=g).to(torch.bfloat16)
    slots = torch.randperm(P * ps, generator=g)[:N].to(torch.int64)
    slots[0] = -1
    want, _ = oracle.cache_insert(cache, None, slots, kvc, k_rope=kpe, page_size=ps)
    gc = cache.to(DEV)
    qo = torch.full((N, Hq, 576), float("nan"), dtype=torch.bfloat16, device=DEV)
    pkv.cache_insert(gc, None, slots.to(DEV), kvc.to(DEV), k_rope=kpe.to(DEV), page_size=ps,
                     q_lo=ql.to(DEV), q_hi=qp.to(DEV), q_out=qo)
    torch.cuda.synchronize()
    assert torch.equal(_bits(gc), _bits(want))
    assert torch.equal(_bits(qo), _bits(torch.cat([ql, qp], dim=-1)))


def test_insert_device_scale_and_empty_call():
    kc, vc, k, v, slots = _case("NHD", torch.bfloat16, torch.float8_e4m3fn, seed=5)
    want_k, want_v = oracle.cache_insert(kc, vc, slots, k, v=v, page_size=16, cache_scale_inv=3.25)
    gk, gv = kc.to(DEV), vc.to(DEV)
    s = torch.tensor([3.25], dtype=torch.float32, device=DEV)
    pkv.cache_insert(gk, gv, slots.to(DEV), k.to(DEV), v=v.to(DEV), page_size=16, cache_scale_inv=s)
    empty = torch.empty(0, dtype=torch.int64, device=DEV)
    pkv.cache_insert(gk, gv, empty, k[:0].to(DEV), v=v[:0].to(DEV), page_size=16)
    torch.cuda.synchronize()
    assert torch.equal(_bits(gk), _bits(want_k)) and torch.equal(_bits(gv), _bits(want_v))


@pytest.mark.parametrize("name", ["llama3_8b_gqa", "fp8_window_sinks"])
def test_insert_then_decode(name):
    # the decode step's order: write each sequence's new token at position L,
    # then attend over L + 1 tokens; the GPU pair against the oracle pair
    w = synth.WORKLOADS[name].replace(batch=4, seq_len_range=(100, 700))
    w = w.replace(window=min(w.window, 300)) if w.window else w
    L = synth.draw_seq_lens(w, 6)
    inp = synth.make_inputs(w, 6, DEV, seq_lens=L + 1, poison=False)
    B, Hkv, D, ps = w.batch, w.num_kv_heads, w.head_dim_qk, w.page_size
    g = torch.Generator().manual_seed(6)
    k = torch.randn(B, Hkv, D, generator=g).to(w.q_dtype)
    v = torch.randn(B, Hkv, D, generator=g).to(w.q_dtype)
    pt = inp["page_table_host"]
    slots = torch.tensor([int(pt[b, int(L[b]) // ps]) * ps + int(L[b]) % ps for b in range(B)],
                         dtype=torch.int64)
    s_inv = 1.0 / w.kv_scale
    kc, vc = oracle.cache_insert(inp["k_cache"], inp["v_cache"], slots, k, v=v, page_size=ps,
                                 kv_layout=w.kv_layout, cache_scale_inv=s_inv)
    pkv.cache_insert(inp["k_cache"], inp["v_cache"], slots.to(DEV), k.to(DEV), v=v.to(DEV),
                     page_size=ps, kv_layout=w.kv_layout, cache_scale_inv=s_inv)
    torch.cuda.synchronize()
    assert torch.equal(_bits(inp["k_cache"]), _bits(kc)) and torch.equal(_bits(inp["v_cache"]), _bits(vc))
    out = torch.full((B, 1, w.num_q_heads, D), float("nan"), dtype=w.q_dtype, device=DEV)
    pkv.decode_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"], inp["seq_lens"], out,
                    num_kv_heads=Hkv, page_size=ps, sinks=inp["sinks"], q_scale=w.q_scale,
                    kv_scale=w.kv_scale, sliding_win_size=w.window, kv_layout=w.kv_layout)
    ref = oracle.decode(inp["q"], kc, vc, inp["page_table"], inp["seq_lens"], sinks=inp["sinks"],
                        **synth.decode_kwargs(w))
    tol = 2e-2 if w.kv_dtype == torch.float8_e4m3fn else 1e-2
    err = (out.double().cpu() - ref).abs().max().item()
    print(f"[parity] insert-then-decode {name} max_abs={err:.3e}", flush=True)
    assert err <= tol
