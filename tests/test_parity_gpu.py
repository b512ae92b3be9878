"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (max-abs on N(0,1) inputs): 4e-3 for fp16, 1e-2 for bf16, 2e-2
for an fp8 cache (the oracle reads the same e4m3fn bytes and kv_scale).  An
output whose own rounding to the output dtype approaches the bound (bf16
values of magnitude >= 2, f16 >= 8) may be off by half an ulp plus half the
tolerance (see assert_parity).
Index work is checked exactly: single-token sequences must return their V
row bit for bit, page permutation and NHD/HND must not change a single bit,
NaN poison in every unused page and invisible slot must never reach the
output, and every output element must be written (outputs start as NaN).
"""
import math

import pytest
import torch

import oracle
import paged_kv_attention_pages_amd as pkv
from paged_kv_attention_pages_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def tol_for(w):
    if w.kv_dtype == torch.float8_e4m3fn:
        return 2e-2
    return 4e-3 if w.q_dtype == torch.float16 else 1e-2


def keep_from(w, L):
    """Start of the range any query row can see (the window reading)."""
    if w.window <= 0:
        return None
    return (L - w.q_seq_len + 1 - w.window).clamp(min=0)


def make(w, seed, seq_lens=None):
    L = synth.draw_seq_lens(w, seed) if seq_lens is None else torch.as_tensor(seq_lens)
    return synth.make_inputs(w, seed, DEV, seq_lens=L, keep_from=keep_from(w, L))


def out_dtype(w):
    """The output dtype: q's, bfloat16 for an fp8 query."""
    return torch.bfloat16 if w.q_dtype == torch.float8_e4m3fn else w.q_dtype


def run_gpu(w, inp, **kw):
    B = inp["q"].shape[0]
    out = torch.full((B, w.q_seq_len, w.num_q_heads, w.head_dim_v), float("nan"),
                     dtype=out_dtype(w), device=DEV)
    pkv.decode_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"], inp["seq_lens"],
                    out, num_kv_heads=w.num_kv_heads, page_size=w.page_size, sinks=inp["sinks"],
                    q_scale=w.q_scale, kv_scale=w.kv_scale, sliding_win_size=w.window,
                    kv_layout=w.kv_layout, q_seq_len=w.q_seq_len, mask=inp["mask"],
                    head_dim_v=w.head_dim_v, **kw)
    torch.cuda.synchronize()
    return out


def _take(t, idx):
    """Rows idx of a small per-sequence tensor, on the host (uint16 has no index kernel)."""
    if t is None:
        return None
    t = t.cpu()
    if t.dtype == torch.uint16:
        return t.view(torch.int16)[idx].view(torch.uint16)
    return t[idx]


def run_oracle(w, inp, idx=None):
    sel = (lambda t: t) if idx is None else (lambda t: _take(t, idx))
    return oracle.decode(sel(inp["q"]), inp["k_cache"], None if w.v_from_k else inp["v_cache"],
                         sel(inp["page_table"]), sel(inp["seq_lens"]), sinks=inp["sinks"],
                         mask=sel(inp["mask"]), head_dim_v=w.head_dim_v, v_from_k=w.v_from_k,
                         **synth.decode_kwargs(w))


def out_half_ulp(ref, dtype):
    """Half the spacing of the output dtype at |ref|: the error of the correctly
    rounded output itself."""
    mant = {torch.bfloat16: 7, torch.float16: 10}[dtype]
    e = torch.floor(torch.log2(ref.abs().clamp(min=2.0 ** -14)))
    return 0.5 * torch.exp2(e - mant)


def assert_parity(w, got, ref, label=""):
    """Max-abs error within the tolerance.  Where the output dtype cannot hold
    the exact value to that accuracy (bf16 |out| >= 2, f16 |out| >= 8: half a
    unit in the last place approaches the bound), the allowance is that
    half-ulp plus half the tolerance -- the correctly rounded exact value
    passes, a value one ulp further off does not."""
    got = got.double().cpu()
    assert not torch.isnan(got).any(), f"{label}: NaN in output (unwritten or poisoned)"
    tol = tol_for(w)
    d = (got - ref).abs()
    allowed = torch.clamp(out_half_ulp(ref, out_dtype(w)) + 0.5 * tol, min=tol)
    err = d.max().item()
    at = ref.flatten()[d.flatten().argmax()].item()
    rms = ref.pow(2).mean().sqrt().item()
    n_fmt = int((d > tol).sum())
    print(f"[parity] {label} max_abs={err:.3e} tol={tol:.0e} rms_ref={rms:.3e} "
          f"ref_at_max={at:.4f} beyond_tol_by_format={n_fmt}", flush=True)
    bad = d > allowed
    assert not bad.any(), (f"{label}: max abs err {err} (reference there {at}); "
                           f"{int(bad.sum())} elements beyond the allowance")


# ---------------------------------------------------------------- small cases

SMALL = {
    "tiny": synth.WORKLOADS["tiny"],
    "gqa": synth.WORKLOADS["llama3_8b_gqa"].replace(batch=6, seq_len_range=(1, 1500)),
    "fp8": synth.WORKLOADS["fp8_window_sinks"].replace(
        batch=5, num_q_heads=16, num_kv_heads=2, seq_len_range=(100, 1200), window=300),
    "spec": synth.WORKLOADS["spec_decode"].replace(batch=5, seq_len_range=(4, 1200)),
    "mla": synth.WORKLOADS["mla"].replace(batch=3, seq_len_range=(1, 900)),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("split", [0, 1, 1000])
def test_small_parity(name, split):
    w = SMALL[name]
    print(f"[case] small {name} split_pages={split}", flush=True)
    inp = make(w, seed=31)
    got = run_gpu(w, inp, split_pages=split)
    assert_parity(w, got, run_oracle(w, inp), f"{name}/split{split}")


@pytest.mark.parametrize("name", ["tiny", "gqa", "fp8"])
@pytest.mark.parametrize("split", [0, 1])
def test_valu_path_parity(name, split):
    w = SMALL[name]
    print(f"[case] valu {name} split_pages={split}", flush=True)
    inp = make(w, seed=32)
    got = run_gpu(w, inp, path="valu", split_pages=split)
    assert_parity(w, got, run_oracle(w, inp), f"valu/{name}/split{split}")


@pytest.mark.parametrize("ps", [16, 32, 64, 128])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_page_sizes_and_layouts(ps, layout, path):
    w = SMALL["gqa"].replace(page_size=ps, kv_layout=layout, seq_len_range=(1, 700), batch=4)
    print(f"[case] ps={ps} {layout} {path}", flush=True)
    inp = make(w, seed=33 + ps)
    got = run_gpu(w, inp, path=path, split_pages=2)
    assert_parity(w, got, run_oracle(w, inp), f"ps{ps}/{layout}/{path}")


@pytest.mark.parametrize("D", [64, 256])
def test_other_head_dims(D):
    w = SMALL["gqa"].replace(head_dim_qk=D, head_dim_v=D, batch=3, seq_len_range=(1, 600))
    print(f"[case] head_dim {D}", flush=True)
    inp = make(w, seed=40 + D)
    got = run_gpu(w, inp, split_pages=3)
    assert_parity(w, got, run_oracle(w, inp), f"D{D}")


def test_fp16_query_fp8_cache():
    w = SMALL["fp8"].replace(q_dtype=torch.float16)
    print("[case] f16 q + fp8 cache", flush=True)
    inp = make(w, seed=41)
    for path in ("mfma", "valu"):
        got = run_gpu(w, inp, path=path, split_pages=2)
        assert_parity(w, got, run_oracle(w, inp), f"f16q-fp8/{path}")


@pytest.mark.parametrize("kind", ["causal", "random", "ones", None])
@pytest.mark.parametrize("W", [0, 50])
def test_spec_decode_masks(kind, W):
    w = SMALL["spec"].replace(mask=kind, window=W)
    print(f"[case] spec mask={kind} window={W}", flush=True)
    inp = make(w, seed=42)
    got = run_gpu(w, inp, split_pages=1)
    assert_parity(w, got, run_oracle(w, inp), f"spec/{kind}/W{W}")


def test_spec_16_rows_one_kv_head_per_query_head():
    # q_seq_len 16 with group 1: a full 16-row tile of query tokens
    w = SMALL["spec"].replace(num_q_heads=4, num_kv_heads=4, q_seq_len=16, mask="random",
                              seq_len_range=(16, 700))
    print("[case] spec Tq=16 G=1", flush=True)
    inp = make(w, seed=43)
    got = run_gpu(w, inp, split_pages=2)
    assert_parity(w, got, run_oracle(w, inp), "spec/Tq16")


def test_window_sinks_multi_split():
    w = SMALL["fp8"].replace(window=700, seq_len_range=(1, 2500), batch=6)
    print("[case] fp8 window 700 sinks, 1-page splits", flush=True)
    inp = make(w, seed=44)
    got = run_gpu(w, inp, split_pages=1)
    assert_parity(w, got, run_oracle(w, inp), "fp8/W700")


# ---------------------------------------------------------------- exact checks

@pytest.mark.parametrize("name", ["tiny", "gqa", "mla"])
def test_single_token_returns_v_row_exactly(name):
    w = SMALL[name].replace(sinks=False, window=0)
    B = 3
    inp = make(w.replace(batch=B, fixed_seq_lens=(1,) * B, seq_len_range=None, num_pages=None),
               seed=45)
    got = run_gpu(w, inp)
    t0 = inp["page_table_host"][:, 0].to(torch.int64)
    src = inp["k_cache"] if w.v_from_k else inp["v_cache"]
    for b in range(B):
        for h in range(w.num_q_heads):
            kvh = h // w.group
            row = src[t0[b], 0, kvh] if w.kv_layout == "NHD" else src[t0[b], kvh, 0]
            assert torch.equal(got[b, 0, h], row[: w.head_dim_v].to(w.q_dtype)), (b, h)


@pytest.mark.parametrize("path", ["mfma", "valu"])
def test_fp8_every_code_decodes_exactly(path):
    # one-token sequences whose V rows hold all 256 e4m3fn codes: out must be
    # exactly the decoded value (e4m3fn is a subset of bf16), NaN for NaN codes
    w = SMALL["fp8"].replace(sinks=False, window=0, num_q_heads=2, num_kv_heads=1, kv_scale=1.0)
    B = 2
    inp = make(w.replace(batch=B, fixed_seq_lens=(1,) * B, seq_len_range=None), seed=46)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(2, 128)
    v = inp["v_cache"].view(torch.uint8)
    k = inp["k_cache"].view(torch.uint8)
    for b in range(B):
        pg = int(inp["page_table_host"][b, 0])
        v[pg, 0, 0] = codes[b].to(DEV)
        k[pg, 0, 0] = 0x38  # 1.0, finite scores
    torch.cuda.synchronize()
    got = run_gpu(w, inp, path=path).float().cpu()
    want = codes.view(torch.float8_e4m3fn).float()
    for b in range(B):
        for h in range(2):
            g, r = got[b, 0, h], want[b]
            assert torch.equal(torch.isnan(g), torch.isnan(r))
            ok = ~torch.isnan(r)
            assert torch.equal(g[ok], r[ok]), (b, h)
    # cross-check the oracle's decoder on the same codes
    for c in range(256):
        o = oracle.decode_e4m3fn(c)
        r = float(want.flatten()[c])
        assert (math.isnan(o) and math.isnan(r)) or o == r


def test_empty_and_ragged_sequences():
    w = SMALL["gqa"].replace(batch=8)
    lens = [0, 1, 15, 16, 17, 63, 65, 1023]
    inp = make(w, seed=47, seq_lens=lens)
    for split in (0, 1):
        got = run_gpu(w, inp, split_pages=split)
        assert torch.equal(got[0].float().cpu(), torch.zeros_like(got[0].float().cpu()))
        assert_parity(w, got, run_oracle(w, inp), f"ragged/split{split}")


def test_window_one_and_window_ge_len():
    w = SMALL["gqa"].replace(batch=4, seq_len_range=(1, 500))
    inp = make(w, seed=48)
    base = run_gpu(w, inp)
    wide = run_gpu(w.replace(window=10_000), inp)
    assert torch.equal(base, wide)
    one = run_gpu(w.replace(window=1), inp)
    torch.testing.assert_close(one.double().cpu(), run_oracle(w.replace(window=1), inp),
                               rtol=0, atol=1e-2)


def test_no_visible_draft_row_gives_zeros():
    # seq_len == q_seq_len and an all-zero mask row: query 0 sees nothing
    w = SMALL["spec"].replace(batch=2, fixed_seq_lens=(4, 4), seq_len_range=None, mask="causal")
    inp = make(w, seed=49)
    inp["mask"].view(torch.int16)[:, 0] = 0
    got = run_gpu(w, inp)
    assert torch.equal(got[:, 0].float().cpu(), torch.zeros_like(got[:, 0].float().cpu()))
    assert_parity(w, got, run_oracle(w, inp), "zero-row")


def test_page_permutation_is_bit_identical():
    w = SMALL["gqa"]
    inp = make(w, seed=50)
    base = run_gpu(w, inp, split_pages=2)
    P = inp["num_pages"]
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(5))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(P)
    inp2 = dict(inp)
    perm_d = perm.to(DEV)
    inp2["k_cache"] = inp["k_cache"][perm_d].contiguous()
    inp2["v_cache"] = inp["v_cache"][perm_d].contiguous()
    inp2["page_table"] = inv.to(DEV)[inp["page_table"].long()].to(torch.int32)
    assert torch.equal(run_gpu(w, inp2, split_pages=2), base)


def test_nhd_and_hnd_are_bit_identical():
    w = SMALL["gqa"].replace(kv_layout="NHD")
    inp = make(w, seed=51)
    a = run_gpu(w, inp, split_pages=2)
    inp2 = dict(inp)
    inp2["k_cache"] = inp["k_cache"].transpose(1, 2).contiguous()
    inp2["v_cache"] = inp["v_cache"].transpose(1, 2).contiguous()
    b = run_gpu(w.replace(kv_layout="HND"), inp2, split_pages=2)
    assert torch.equal(a, b)


def test_validate_inputs_reports_bad_page_ids():
    w = SMALL["gqa"]
    inp = make(w, seed=52)
    kw = dict(num_kv_heads=w.num_kv_heads, page_size=w.page_size)
    pkv.validate_inputs(inp["q"], inp["k_cache"], inp["page_table"], inp["seq_lens"], **kw)
    bad = inp["page_table"].clone()
    bad[2, 0] = inp["num_pages"] + 5
    with pytest.raises(pkv.PkvError, match="sequence 2"):
        pkv.validate_inputs(inp["q"], inp["k_cache"], bad, inp["seq_lens"], **kw)


def test_bad_arguments_raise():
    w = SMALL["gqa"]
    inp = make(w, seed=53)
    with pytest.raises(pkv.PkvError, match="page_size"):
        run_gpu(w.replace(page_size=48), inp)


# ---------------------------------------------------------------- full sizes

def _sample(L, k=6):
    order = torch.argsort(L)
    pick = [int(order[0]), int(order[-1])] + [int(i) for i in order[torch.linspace(
        1, len(L) - 2, k - 2).long()]]
    return torch.tensor(sorted(set(pick)))


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_full_size_sampled_parity(name):
    w = synth.WORKLOADS[name]
    print(f"[case] full {name}", flush=True)
    inp = make(w, seed=1)
    got = run_gpu(w, inp)
    L = inp["seq_lens_host"]
    idx = torch.arange(len(L)) if len(L) <= 8 else _sample(L, 6 if name != "mla" else 4)
    ref = run_oracle(w, inp, idx)
    assert_parity(w, got[idx.to(DEV)], ref, f"full/{name}")
    assert not torch.isnan(got).any()


def test_full_size_sampled_parity_fp8_latent():
    # the fp8 latent workload (fp8 query and cache, 32 sequences of 4096 to
    # 16384 tokens, 64 heads) on the schedule the benchmark times
    w = synth.WORKLOADS["mla_fp8"]
    print("[case] full mla_fp8", flush=True)
    inp = make(w, seed=1)
    got = run_gpu(w, inp)
    idx = _sample(inp["seq_lens_host"], 4)
    assert_parity(w, got[idx.to(DEV)], run_oracle(w, inp, idx), "full/mla_fp8")
    assert not torch.isnan(got).any()


def test_full_size_sampled_parity_512_sequences():
    # the Llama-3-8B decode shape at 512 sequences: the wide stream-K schedule
    w = synth.WORKLOADS["llama3_8b_gqa"].replace(batch=512)
    print("[case] full llama3_8b_gqa batch 512", flush=True)
    inp = make(w, seed=2)
    plan = pkv.query_plan(batch=512, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                          head_dim_qk=128, head_dim_v=128, pages_per_seq=inp["page_table"].shape[1],
                          page_size=w.page_size)
    assert plan["split_pages"] == 0
    got = run_gpu(w, inp)
    idx = _sample(inp["seq_lens_host"], 6)
    assert_parity(w, got[idx.to(DEV)], run_oracle(w, inp, idx), "full/gqa-b512")
    assert not torch.isnan(got).any()


# ---------------------------------------------------------------- exact visible sets

def _probe(w, inp):
    """q = 0 and V[t] = onehot(t): out[b, i, h, d] = 1/|visible| if token d is visible."""
    inp["q"].zero_()
    src = inp["k_cache"] if w.v_from_k else inp["v_cache"]
    # write raw bits: 1.0 is 0x38 (e4m3fn), 0x3F80 (bf16), 0x3C00 (f16)
    if src.dtype == torch.float8_e4m3fn:
        src, one = src.view(torch.uint8), 0x38
    else:
        src, one = src.view(torch.int16), (0x3F80 if src.dtype == torch.bfloat16 else 0x3C00)
    src.zero_()
    for b in range(inp["q"].shape[0]):
        L = int(inp["seq_lens_host"][b])
        for t in range(L):
            pg, sl = int(inp["page_table_host"][b, t // w.page_size]), t % w.page_size
            if w.kv_layout == "NHD":
                src[pg, sl, :, t] = one
            else:
                src[pg, :, sl, t] = one
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", [
    ("spec", "causal", "mfma", 0), ("spec", "random", "mfma", 0), ("spec", "zero", "mfma", 0),
    ("spec", "random", "mfma", 9), ("spec2", "causal", "valu", 0), ("spec2", "random", "valu", 7),
    ("gqa", None, "mfma", 5), ("gqa", None, "valu", 5), ("fp8", None, "mfma", 11),
    ("fp8", None, "valu", 11), ("mla", None, "mfma_mla", 0), ("mla4", "random", "mfma_mla", 0),
])
def test_visible_sets_exact(case):
    name, mask, path, W = case
    base = {
        "spec": SMALL["spec"].replace(num_q_heads=8, num_kv_heads=2),
        "spec2": SMALL["spec"].replace(num_q_heads=4, num_kv_heads=2),
        "gqa": SMALL["gqa"], "fp8": SMALL["fp8"].replace(kv_scale=1.0, sinks=False),
        "mla": SMALL["mla"], "mla4": SMALL["mla"].replace(num_q_heads=16, q_seq_len=4),
    }[name]
    w = base.replace(batch=3, fixed_seq_lens=(20, 37, 100), seq_len_range=None, page_size=16,
                     window=W, mask=("causal" if mask == "zero" else mask) if base.q_seq_len > 1 or name == "mla4" else None)
    print(f"[case] visible-set {case}", flush=True)
    inp = make(w, seed=60)
    if mask == "zero":
        inp["mask"].view(torch.int16).zero_()
    _probe(w, inp)
    got = run_gpu(w, inp, path=path, split_pages=1).float().cpu()
    ref = run_oracle(w, inp)
    vis_got = got > 0
    vis_ref = ref > 0
    assert torch.equal(vis_got, vis_ref), f"visible sets differ at {torch.nonzero(vis_got != vis_ref)[:8].tolist()}"
    torch.testing.assert_close(got.double(), ref, rtol=2 ** -7, atol=0)


# ---------------------------------------------------------------- stream-K schedule

@pytest.mark.parametrize("W", [1, 3, 7, 64, 5000])
@pytest.mark.parametrize("name", ["gqa", "fp8", "spec", "tiny"])
def test_stream_k_wave_counts(name, W):
    # 1 wave finishes every unit itself; 3 and 7 cut units across many waves;
    # 5000 waves exceed the tile count, so most waves are empty
    w = SMALL[name]
    print(f"[case] stream-K {name} waves={W}", flush=True)
    inp = make(w, seed=70)
    got = run_gpu(w, inp, target_ctas=W)
    assert_parity(w, got, run_oracle(w, inp), f"sk/{name}/W{W}")


@pytest.mark.parametrize("hkv, W, single", [(8, 64, False), (8, 64, True), (6, 48, False),
                                             (6, 768, False), (2, 10, False), (8, 12, False),
                                             (8, 40, True), (4, 2048, True)])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_stream_k_head_grouped_workgroups(hkv, W, single, kv):
    # workgroups of several waves, one KV head each, over the KV-head-major
    # unit order (2, 3, 4, 6 and 8 heads per workgroup and the one-wave
    # fallback), with both merges
    base = SMALL["gqa"] if kv == "bf16" else SMALL["fp8"]
    w = base.replace(num_kv_heads=hkv, num_q_heads=4 * hkv, batch=5, seq_len_range=(1, 700),
                     kv_layout="NHD")
    inp = make(w, seed=72)
    p = pkv.query_plan(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=hkv,
                       head_dim_qk=128, head_dim_v=128, pages_per_seq=inp["page_table"].shape[1],
                       page_size=w.page_size, q_dtype=w.q_dtype, kv_dtype=w.kv_dtype,
                       window=w.window, target_ctas=W, single_launch=single)
    print(f"[case] head groups {kv} Hkv={hkv} waves={W} single={single}: "
          f"{p['waves_per_workgroup']} per workgroup", flush=True)
    got = run_gpu(w, inp, target_ctas=W, single_launch=single)
    assert_parity(w, got, run_oracle(w, inp), f"hg/{kv}/Hkv{hkv}/W{W}")


def test_stream_k_empty_sequences_and_split_invariance():
    w = SMALL["gqa"].replace(batch=8)
    lens = [0, 1, 15, 0, 17, 63, 1023, 0]
    inp = make(w, seed=71, seq_lens=lens)
    ref = run_oracle(w, inp)
    outs = [run_gpu(w, inp, target_ctas=W) for W in (1, 5, 37, 2048)]
    for o in outs:
        assert_parity(w, o, ref, "sk-empty")
        assert torch.equal(o[0].float().cpu(), torch.zeros_like(o[0].float().cpu()))


@pytest.mark.parametrize("D", [64, 256])
@pytest.mark.parametrize("W", [5, 0])
def test_stream_k_other_head_dims(D, W):
    w = SMALL["gqa"].replace(head_dim_qk=D, head_dim_v=D, batch=3, seq_len_range=(1, 600))
    print(f"[case] stream-K head_dim {D} waves={W}", flush=True)
    inp = make(w, seed=80 + D)
    got = run_gpu(w, inp, target_ctas=W)
    assert_parity(w, got, run_oracle(w, inp), f"sk-D{D}-W{W}")


def test_repeated_calls_reuse_workspace():
    # workspace contents on entry are arbitrary: a garbage-filled workspace,
    # reused across calls, must give the same result every time
    w = SMALL["spec"]
    inp = make(w, seed=81)
    ref = run_oracle(w, inp)
    plan = pkv.query_plan(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                          head_dim_qk=128, head_dim_v=128, pages_per_seq=inp["page_table"].shape[1],
                          page_size=w.page_size, q_seq_len=w.q_seq_len, target_ctas=7)
    ws = torch.randint(0, 255, (plan["workspace_bytes"],), dtype=torch.uint8, device=DEV)
    for _ in range(3):
        out = torch.full((w.batch, w.q_seq_len, w.num_q_heads, 128), float("nan"),
                         dtype=w.q_dtype, device=DEV)
        pkv.decode_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"],
                        inp["seq_lens"], out, ws, num_kv_heads=w.num_kv_heads,
                        page_size=w.page_size, kv_layout=w.kv_layout, q_seq_len=w.q_seq_len,
                        mask=inp["mask"], target_ctas=7)
        torch.cuda.synchronize()
        assert_parity(w, out, ref, "ws-reuse")


def test_default_workspace_per_stream():
    # two calls in flight on two streams with the default workspace: each
    # stream has its own, so neither overwrites the other's partials
    w = SMALL["gqa"].replace(batch=4, seq_len_range=(600, 1500))
    print("[case] default workspace on two streams", flush=True)
    a, b = make(w, seed=82), make(w, seed=83)
    ref_a, ref_b = run_oracle(w, a), run_oracle(w, b)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for inp, s in ((a, s1), (b, s2)):
        out = torch.full((w.batch, 1, w.num_q_heads, 128), float("nan"), dtype=w.q_dtype, device=DEV)
        outs.append(out)
    torch.cuda.synchronize()
    for _ in range(3):
        for inp, s, out in ((a, s1, outs[0]), (b, s2, outs[1])):
            with torch.cuda.stream(s):
                pkv.decode_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"],
                                inp["seq_lens"], out, num_kv_heads=w.num_kv_heads,
                                page_size=w.page_size, kv_layout=w.kv_layout)
    torch.cuda.synchronize()
    keys = [k for k in pkv._ws_cache if k[1] in (s1.cuda_stream, s2.cuda_stream)]
    assert len(keys) == 2
    assert pkv._ws_cache[keys[0]].data_ptr() != pkv._ws_cache[keys[1]].data_ptr()
    assert_parity(w, outs[0], ref_a, "ws-stream1")
    assert_parity(w, outs[1], ref_b, "ws-stream2")


# ---------------------------------------------------------------- single-launch merge

def _ulps_apart(a, b, dtype):
    """Largest distance between two outputs in units of the output dtype's
    spacing at the larger magnitude."""
    a, b = a.double().cpu(), b.double().cpu()
    mant = {torch.bfloat16: 7, torch.float16: 10}[dtype]
    e = torch.floor(torch.log2(torch.maximum(a.abs(), b.abs()).clamp(min=2.0 ** -14)))
    return ((a - b).abs() / torch.exp2(e - mant)).max().item()


@pytest.mark.parametrize("W", [0, 3, 64])
@pytest.mark.parametrize("name", ["tiny", "gqa", "fp8", "spec"])
def test_single_launch_matches_two_launches(name, W):
    # the split kernel's own merge (the last wave of a unit) against the
    # combine kernel on the same partials: both within the bound, and at most
    # one output ulp apart (the merges sum in a different order)
    w = SMALL[name]
    print(f"[case] single-launch {name} waves={W}", flush=True)
    inp = make(w, seed=90)
    one = run_gpu(w, inp, target_ctas=W, single_launch=True)
    two = run_gpu(w, inp, target_ctas=W, single_launch=False)
    ref = run_oracle(w, inp)
    assert_parity(w, one, ref, f"one-launch/{name}/W{W}")
    assert_parity(w, two, ref, f"two-launch/{name}/W{W}")
    assert _ulps_apart(one, two, w.q_dtype) <= 1.0
    # the merge reads the slots in a fixed order, whichever wave finishes last
    for _ in range(3):
        assert torch.equal(run_gpu(w, inp, target_ctas=W, single_launch=True), one)


def test_single_launch_sees_each_calls_partials():
    # new queries on every call through one workspace: a merge that read a
    # partial left by the previous call (a stale line in some cache) would
    # differ from the two-launch result of the same call
    w = SMALL["gqa"].replace(batch=4, seq_len_range=(300, 1500))
    inp = make(w, seed=91)
    plan = pkv.query_plan(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                          head_dim_qk=128, head_dim_v=128, pages_per_seq=inp["page_table"].shape[1],
                          page_size=w.page_size, target_ctas=96, single_launch=True)
    assert plan["single_launch"] == 1
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(91)
    for call in range(12):
        inp["q"] = torch.randn(inp["q"].shape, generator=g, device=DEV).to(w.q_dtype)
        one = torch.full((w.batch, 1, w.num_q_heads, 128), float("nan"), dtype=w.q_dtype, device=DEV)
        pkv.decode_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"],
                        inp["seq_lens"], one, ws, num_kv_heads=w.num_kv_heads,
                        page_size=w.page_size, kv_layout=w.kv_layout, target_ctas=96,
                        single_launch=True)
        two = run_gpu(w, inp, target_ctas=96, single_launch=False)
        assert not torch.isnan(one).any(), f"call {call}: NaN"
        assert _ulps_apart(one, two, w.q_dtype) <= 1.0, f"call {call}"
    assert_parity(w, one, run_oracle(w, inp), "one-launch/last-call")


# ---------------------------------------------------------------- latent (MLA) path

MLA_SMALL = SMALL["mla"].replace(batch=3, seq_len_range=(1, 700))


@pytest.mark.parametrize("ps", [16, 32, 64, 128])
@pytest.mark.parametrize("layout", ["NHD", "HND"])
@pytest.mark.parametrize("split", [0, 3])
def test_mla_page_sizes_and_layouts(ps, layout, split):
    # split 0: stream-K over 32-token tiles; split 3: grid schedule whose
    # 3-page splits start mid-tile when the page holds 16 tokens
    w = MLA_SMALL.replace(page_size=ps, kv_layout=layout)
    print(f"[case] mla ps={ps} {layout} split={split}", flush=True)
    inp = make(w, seed=90 + ps)
    got = run_gpu(w, inp, split_pages=split)
    assert_parity(w, got, run_oracle(w, inp), f"mla/ps{ps}/{layout}/split{split}")


@pytest.mark.parametrize("variant", ["window_sinks", "f16", "rows20", "rows40", "spec2_random",
                                     "spec4_causal"])
@pytest.mark.parametrize("split", [0, 1])
def test_mla_variants(variant, split):
    w = {
        "window_sinks": MLA_SMALL.replace(window=100, sinks=True, seq_len_range=(1, 900)),
        "f16": MLA_SMALL.replace(q_dtype=torch.float16, kv_dtype=torch.float16),
        "rows20": MLA_SMALL.replace(num_q_heads=20),
        "rows40": MLA_SMALL.replace(num_q_heads=40, sinks=True),
        "spec2_random": MLA_SMALL.replace(num_q_heads=32, q_seq_len=2, mask="random",
                                          seq_len_range=(2, 700)),
        "spec4_causal": MLA_SMALL.replace(num_q_heads=16, q_seq_len=4, mask="causal", window=40,
                                          seq_len_range=(4, 700)),
    }[variant]
    print(f"[case] mla {variant} split={split}", flush=True)
    inp = make(w, seed=95)
    got = run_gpu(w, inp, split_pages=split)
    assert_parity(w, got, run_oracle(w, inp), f"mla/{variant}/split{split}")


def test_mla_empty_and_ragged_sequences():
    w = MLA_SMALL.replace(batch=9)
    lens = [0, 1, 31, 32, 33, 0, 64, 65, 700]
    inp = make(w, seed=96, seq_lens=lens)
    ref = run_oracle(w, inp)
    for split, W in ((0, 0), (0, 5), (1, 0)):
        got = run_gpu(w, inp, split_pages=split, target_ctas=W)
        for b in (0, 5):
            assert torch.equal(got[b].float().cpu(), torch.zeros_like(got[b].float().cpu()))
        assert_parity(w, got, ref, f"mla-ragged/split{split}/W{W}")


MLA_FP8 = MLA_SMALL.replace(kv_dtype=torch.float8_e4m3fn, kv_scale=0.05, kv_gen_scale=1.0 / 0.05)


@pytest.mark.parametrize("q", ["bf16", "f16", "fp8"])
@pytest.mark.parametrize("ps", [16, 32, 64, 128])
@pytest.mark.parametrize("split", [0, 3])
def test_mla_fp8_cache(q, ps, split):
    # an e4m3fn latent cache, with a 16-bit query or the quantised (e4m3fn)
    # query of the latent path, whose output is bfloat16; split 0: stream-K
    # over 64-token tiles (one to four pages each), split 3: the split grid
    qd = {"bf16": torch.bfloat16, "f16": torch.float16, "fp8": torch.float8_e4m3fn}[q]
    w = MLA_FP8.replace(q_dtype=qd, page_size=ps)
    print(f"[case] mla fp8 cache, q {q}, ps={ps} split={split}", flush=True)
    inp = make(w, seed=98 + ps)
    got = run_gpu(w, inp, split_pages=split)
    assert got.dtype == out_dtype(w)
    assert_parity(w, got, run_oracle(w, inp), f"mla-fp8/q{q}/ps{ps}/split{split}")


@pytest.mark.parametrize("variant", ["window_sinks_q8", "spec4_q8", "ragged_q8", "W7_q16", "W1_q8",
                                     "W300_q8", "rows20_q16"])
def test_mla_fp8_variants(variant):
    base = MLA_FP8.replace(q_dtype=torch.float8_e4m3fn)
    kw, lens = {}, None
    if variant == "W1_q8":          # one workgroup: every unit switch in one share
        w, kw = base, dict(target_ctas=1)
    elif variant == "W300_q8":      # more workgroups than tiles of some units
        w, kw = base.replace(seq_len_range=(1, 400)), dict(target_ctas=300)
    elif variant == "rows20_q16":   # 20 query rows: partial row blocks in both roles
        w = MLA_FP8.replace(num_q_heads=20)
    elif variant == "window_sinks_q8":
        w = base.replace(window=100, sinks=True, seq_len_range=(1, 900), q_scale=1.3)
    elif variant == "spec4_q8":
        w = base.replace(num_q_heads=16, q_seq_len=4, mask="causal", seq_len_range=(4, 700))
    elif variant == "ragged_q8":
        w = base.replace(batch=9)
        lens = [0, 1, 31, 32, 33, 0, 64, 65, 700]
    else:
        w = MLA_FP8
        kw = dict(target_ctas=7)
    print(f"[case] mla fp8 {variant}", flush=True)
    inp = make(w, seed=99, seq_lens=lens)
    got = run_gpu(w, inp, **kw)
    assert_parity(w, got, run_oracle(w, inp), f"mla-fp8/{variant}")


@pytest.mark.parametrize("split", [0, 3])
def test_mla_fp8_query_matches_its_bf16_image(split):
    # An fp8 query takes the fp8 matrix instruction for the scores on the
    # stream-K kernel (inexact sums, ~1e-4 of the products' magnitudes) and
    # the exact conversion on the split grid; the same query as bf16 (an exact
    # image) goes through the exact route.  On the grid the outputs are
    # identical; on stream-K they differ by the fp8 sums' error, which peaky
    # attention (large logits) carries into the output -- bounded here by a
    # quarter of the parity tolerance.
    w = MLA_FP8.replace(q_dtype=torch.float8_e4m3fn, batch=6, seq_len_range=(1, 2000))
    print(f"[case] fp8 query vs its bf16 image, split={split}", flush=True)
    inp = make(w, seed=71)
    got8 = run_gpu(w, inp, split_pages=split).float()
    w16 = w.replace(q_dtype=torch.bfloat16)
    inp16 = dict(inp, q=inp["q"].to(torch.bfloat16))
    got16 = run_gpu(w16, inp16, split_pages=split).float()
    diff = (got8 - got16).abs().max().item()
    rms = got16.pow(2).mean().sqrt().item()
    print(f"[parity] fp8-vs-bf16-query split={split} max_diff={diff:.3e} rms={rms:.3e}", flush=True)
    if split:
        assert diff == 0.0          # the same exact route
    else:
        assert diff <= 0.25 * tol_for(w)
    assert_parity(w, got8.to(torch.bfloat16), run_oracle(w, inp), f"q8-image/split{split}")


def test_mla_fp8_query_rejected_off_the_latent_path():
    w = SMALL["fp8"].replace(q_dtype=torch.float8_e4m3fn)
    inp = make(w, seed=100)
    with pytest.raises(pkv.PkvError, match="fp8 query|16-bit query"):
        run_gpu(w, inp)


@pytest.mark.parametrize("W", [1, 3, 7, 64, 5000])
def test_mla_stream_k_workgroup_counts(W):
    w = MLA_SMALL
    print(f"[case] mla stream-K workgroups={W}", flush=True)
    inp = make(w, seed=97)
    got = run_gpu(w, inp, target_ctas=W)
    assert_parity(w, got, run_oracle(w, inp), f"mla-sk/W{W}")


# ---------------------------------------------------------------- schedules and capture

@pytest.mark.parametrize("name,B", [("gqa", 1100), ("mla", 300)])
def test_batch_above_schedule_limit_uses_split_grid(name, B):
    # the stream-K schedule keeps per-sequence prefix sums for up to 1024
    # sequences (matrix-core path) or 256 (latent path); larger batches take
    # the split grid
    w = (SMALL["gqa"] if name == "gqa" else MLA_SMALL).replace(batch=B, seq_len_range=(0, 200))
    print(f"[case] batch {B} {name}", flush=True)
    inp = make(w, seed=98)
    plan = pkv.query_plan(batch=B, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                          head_dim_qk=w.head_dim_qk, head_dim_v=w.head_dim_v,
                          pages_per_seq=inp["page_table"].shape[1], page_size=w.page_size,
                          q_dtype=w.q_dtype, kv_dtype=w.kv_dtype)
    assert plan["max_splits"] > 0  # grid schedule
    got = run_gpu(w, inp)
    assert_parity(w, got, run_oracle(w, inp), f"batch{B}/{name}")


@pytest.mark.parametrize("B", [257, 512, 1024])
@pytest.mark.parametrize("kind", ["gqa", "fp8", "spec", "gqa_single_launch", "d64"])
def test_stream_k_wide_batches(kind, B):
    # more than 256 sequences: the matrix-core kernel and its combine run the
    # 16-chunk schedule (lanes hold the prefix sums of 16 sequences each);
    # lengths from 0 give empty sequences, which must come out as zeros
    base = {"gqa": SMALL["gqa"], "fp8": SMALL["fp8"], "spec": SMALL["spec"],
            "gqa_single_launch": SMALL["gqa"],
            "d64": SMALL["gqa"].replace(head_dim_qk=64, head_dim_v=64)}[kind]
    w = base.replace(batch=B, seq_len_range=(4, 300))
    kw = {"single_launch": True} if kind == "gqa_single_launch" else {}
    print(f"[case] stream-K batch {B} {kind}", flush=True)
    L = synth.draw_seq_lens(w, 100 + B)
    if kind != "spec":          # (drafts need q_seq_len <= seq_len)
        L[::97] = 0
    inp = make(w, seed=100 + B, seq_lens=L)
    plan = pkv.query_plan(batch=B, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                          head_dim_qk=w.head_dim_qk, head_dim_v=w.head_dim_v,
                          pages_per_seq=inp["page_table"].shape[1], page_size=w.page_size,
                          q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, window=w.window,
                          q_seq_len=w.q_seq_len, **kw)
    assert plan["split_pages"] == 0 and plan["max_splits"] == 0  # stream-K
    got = run_gpu(w, inp, **kw)
    ref = run_oracle(w, inp)
    assert_parity(w, got, ref, f"sk-wide/{kind}/B{B}")
    if kind != "spec":
        L = inp["seq_lens"].cpu()
        assert bool((L == 0).any())
        assert torch.equal(got[L == 0].float().cpu(), torch.zeros_like(got[L == 0].float().cpu()))


@pytest.mark.parametrize("name", ["gqa", "spec", "mla", "fp8_unit_waves", "mla_fp8", "fp8_short"])
def test_graph_replay_matches_eager(name):
    # a captured call (workspace passed in, so nothing is allocated inside the
    # capture) replayed several times, with eager work between the replays;
    # fp8_unit_waves: a window and two units per CU (one wave per unit);
    # fp8_short: a 200-token window, one wave per short unit, no workspace
    kw = dict(num_cus=2) if name == "fp8_unit_waves" else {}
    w = MLA_SMALL if name == "mla" else SMALL[name.split("_")[0]]
    if name == "fp8_short":
        w = w.replace(window=200)
    if name == "mla_fp8":
        w = MLA_FP8.replace(q_dtype=torch.float8_e4m3fn)
    print(f"[case] graph replay {name}", flush=True)
    inp = make(w, seed=99)
    plan = pkv.query_plan(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                          head_dim_qk=w.head_dim_qk, head_dim_v=w.head_dim_v,
                          pages_per_seq=inp["page_table"].shape[1], page_size=w.page_size,
                          q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, window=w.window,
                          q_seq_len=w.q_seq_len, **kw)
    ws = torch.empty(max(plan["workspace_bytes"], 256), dtype=torch.uint8, device=DEV)
    out = torch.full((w.batch, w.q_seq_len, w.num_q_heads, w.head_dim_v), float("nan"),
                     dtype=out_dtype(w), device=DEV)

    def call():
        pkv.decode_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"],
                        inp["seq_lens"], out, ws, num_kv_heads=w.num_kv_heads,
                        page_size=w.page_size, sinks=inp["sinks"], q_scale=w.q_scale,
                        kv_scale=w.kv_scale, sliding_win_size=w.window, kv_layout=w.kv_layout,
                        q_seq_len=w.q_seq_len, mask=inp["mask"], head_dim_v=w.head_dim_v, **kw)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    assert_parity(w, eager, run_oracle(w, inp), f"graph-eager/{name}")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))
        ws.random_(0, 255)           # eager work between replays, workspace garbage
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager call"


@pytest.mark.parametrize("name", ["gqa", "fp8", "mla", "short"])
def test_device_resident_scales(name):
    # the xqa page's q_scale / kv_scale may be tensors: one fp32 value in
    # device memory, read when the kernels run (short: one wave per unit)
    base = {"gqa": SMALL["gqa"], "fp8": SMALL["fp8"], "mla": MLA_SMALL,
            "short": SMALL["fp8"].replace(window=200)}[name]
    w = base.replace(q_scale=0.7, kv_scale=base.kv_scale * 1.3)
    print(f"[case] device scales {name}", flush=True)
    inp = make(w, seed=100)
    ref = run_oracle(w, inp)
    qs = torch.tensor([w.q_scale], dtype=torch.float32, device=DEV)
    ks = torch.tensor([w.kv_scale], dtype=torch.float32, device=DEV)
    out = torch.full((w.batch, w.q_seq_len, w.num_q_heads, w.head_dim_v), float("nan"),
                     dtype=w.q_dtype, device=DEV)
    for split in (0, 1):
        pkv.decode_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"],
                        inp["seq_lens"], out, num_kv_heads=w.num_kv_heads, page_size=w.page_size,
                        sinks=inp["sinks"], q_scale=qs, kv_scale=ks, sliding_win_size=w.window,
                        kv_layout=w.kv_layout, q_seq_len=w.q_seq_len, mask=inp["mask"],
                        head_dim_v=w.head_dim_v, split_pages=split)
        torch.cuda.synchronize()
        assert_parity(w, out, ref, f"dev-scales/{name}/split{split}")
    # a captured call picks up new values at replay
    w2 = w.replace(q_scale=1.1, kv_scale=w.kv_scale * 0.8)
    ref2 = run_oracle(w2, inp)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    plan = pkv.query_plan(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                          head_dim_qk=w.head_dim_qk, head_dim_v=w.head_dim_v,
                          pages_per_seq=inp["page_table"].shape[1], page_size=w.page_size,
                          q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, window=w.window,
                          q_seq_len=w.q_seq_len)
    ws = torch.empty(max(plan["workspace_bytes"], 256), dtype=torch.uint8, device=DEV)
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pkv.decode_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"],
                            inp["seq_lens"], out, ws, num_kv_heads=w.num_kv_heads,
                            page_size=w.page_size, sinks=inp["sinks"], q_scale=qs, kv_scale=ks,
                            sliding_win_size=w.window, kv_layout=w.kv_layout,
                            q_seq_len=w.q_seq_len, mask=inp["mask"], head_dim_v=w.head_dim_v)
    torch.cuda.current_stream().wait_stream(s)
    qs.fill_(w2.q_scale)
    ks.fill_(w2.kv_scale)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert_parity(w2, out, ref2, f"dev-scales-replay/{name}")


def test_device_scale_arguments_checked():
    w = SMALL["gqa"]
    inp = make(w, seed=101)
    out = torch.empty((w.batch, 1, w.num_q_heads, 128), dtype=w.q_dtype, device=DEV)
    for bad in (torch.ones(2, device=DEV), torch.ones(1, dtype=torch.float16, device=DEV),
                torch.ones(1)):
        with pytest.raises(pkv.PkvError, match="q_scale tensor"):
            pkv.decode_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"],
                            inp["seq_lens"], out, num_kv_heads=w.num_kv_heads,
                            page_size=w.page_size, kv_layout=w.kv_layout, q_scale=bad)


# ---------------------------------------------------------------- fp8 output (rcp_out_scale)

@pytest.mark.parametrize("rcp", [1.0, 6.0])
@pytest.mark.parametrize("mode", ["sk", "grid", "valu", "one_launch", "short", "latent_sk",
                                  "latent_grid"])
def test_fp8_output_with_rcp_out_scale(mode, rcp):
    # an fp8 cache may write an fp8 output holding round(out * rcp_out_scale);
    # the decoded output / rcp is within the bound plus half an E4M3 step
    # (latent: fp8 query and cache, whole units from the split kernel and cut
    # ones from the combine; short: a 200-token window, one wave per unit)
    w = (MLA_FP8.replace(q_dtype=torch.float8_e4m3fn) if mode.startswith("latent")
         else SMALL["fp8"].replace(window=200) if mode == "short" else SMALL["fp8"])
    print(f"[case] fp8 output {mode} rcp={rcp}", flush=True)
    inp = make(w, seed=95)
    B = inp["q"].shape[0]
    out = torch.full((B, w.q_seq_len, w.num_q_heads, w.head_dim_v), float("nan"),
                     dtype=torch.float8_e4m3fn, device=DEV)
    kw = {"sk": {}, "grid": {"split_pages": 3}, "valu": {"path": "valu"},
          "one_launch": {"single_launch": True, "target_ctas": 7}, "short": {},
          "latent_sk": {"target_ctas": 5}, "latent_grid": {"split_pages": 3}}[mode]
    pkv.decode_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"], inp["seq_lens"],
                    out, num_kv_heads=w.num_kv_heads, page_size=w.page_size, sinks=inp["sinks"],
                    q_scale=w.q_scale, kv_scale=w.kv_scale, sliding_win_size=w.window,
                    kv_layout=w.kv_layout, q_seq_len=w.q_seq_len, mask=inp["mask"],
                    rcp_out_scale=rcp, head_dim_v=w.head_dim_v, **kw)
    torch.cuda.synchronize()
    ref = run_oracle(w, inp)
    got = out.cpu().to(torch.float64) / rcp
    assert not torch.isnan(got).any()
    scaled = (ref * rcp).abs().clamp(min=2.0 ** -6)
    half_step = 0.5 * torch.exp2(torch.floor(torch.log2(scaled)) - 3) / rcp   # 3 fraction bits
    allowed = tol_for(w) + half_step
    err = ((got - ref).abs() - allowed).max().item()
    print(f"[parity] fp8-out/{mode}/rcp{rcp} worst margin {err:.3e}", flush=True)
    assert err <= 0.0


def test_fp8_output_needs_an_fp8_cache():
    w = SMALL["gqa"]
    inp = make(w, seed=96)
    out = torch.empty((w.batch, 1, w.num_q_heads, 128), dtype=torch.float8_e4m3fn, device=DEV)
    with pytest.raises(pkv.PkvError, match="dtype"):
        pkv.decode_attn(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"],
                        inp["seq_lens"], out, num_kv_heads=w.num_kv_heads, page_size=w.page_size,
                        kv_layout=w.kv_layout)


@pytest.mark.parametrize("kind, lens, kw", [
    ("tiny", [37, 100], {}),
    ("gqa", [0, 1, 255, 256, 17, 128, 64, 200], {}),
    ("gqa", [0, 1, 255, 256, 17, 128, 64, 200], {"num_cus": 8}),     # 8 units a CU: 8 heads a group
    ("gqa", [0, 1, 255, 256, 17, 128, 64, 200], {"num_cus": 16}),    # 4 heads a group
    ("fp8", [700, 2000, 5, 0, 1200], {}),                              # window 200: short spans
    ("spec", [4, 5, 130, 256], {}),
    ("d64", [1, 64, 65, 250], {}),
    ("d256", [1, 64, 65, 250], {}),
    ("wide", [(37 * i) % 257 for i in range(600)], {}),                # 600 sequences: wide schedule
    ("win16", [3000, 10, 150, 0, 215, 1], {}),                         # 188 table pages, window 200
])
def test_short_sequences_one_wave_per_unit(kind, lens, kw):
    # every unit spans at most 17 tiles (256 cached tokens, or a window that
    # short): one wave per unit, whole, in one launch with no workspace
    base = {"tiny": SMALL["tiny"], "gqa": SMALL["gqa"], "fp8": SMALL["fp8"].replace(window=200),
            "spec": SMALL["spec"],
            "d64": SMALL["gqa"].replace(head_dim_qk=64, head_dim_v=64),
            "d256": SMALL["gqa"].replace(head_dim_qk=256, head_dim_v=256),
            "wide": SMALL["gqa"].replace(num_q_heads=8, num_kv_heads=2),
            "win16": SMALL["gqa"].replace(page_size=16, kv_layout="NHD", window=200)}[kind]
    w = base.replace(batch=len(lens), seq_len_range=(1, max(lens)))
    print(f"[case] short units {kind} lens={lens[:8]} ({len(lens)}) {kw}", flush=True)
    inp = make(w, seed=70 + len(lens), seq_lens=lens)
    plan = pkv.query_plan(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                          head_dim_qk=w.head_dim_qk, head_dim_v=w.head_dim_v,
                          pages_per_seq=inp["page_table"].shape[1], page_size=w.page_size,
                          q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, window=w.window,
                          q_seq_len=w.q_seq_len, **kw)
    assert plan["single_launch"] == 1 and plan["workspace_bytes"] == 0, plan
    assert plan["ctas_per_split_grid"] == w.batch * w.num_kv_heads
    got = run_gpu(w, inp, **kw)
    assert_parity(w, got, run_oracle(w, inp), f"short/{kind}")


def _units_even(w, lens):
    """Which schedule the one-wave-per-unit plan runs: with 16-token tiles of
    the visible span [max(0, L - Tq + 1 - window), L), one wave per unit
    when 4 * max(tiles) * B <= 5 * sum(tiles), equal shares otherwise."""
    n = []
    for L in lens:
        lo = max(0, L - w.q_seq_len + 1 - w.window)
        n.append((L + 15) // 16 - lo // 16 if L > lo else 0)
    return 4 * max(n) * len(lens) <= 5 * sum(n)


@pytest.mark.parametrize("kv, hkv, cus, lens, even", [
    ("fp8", 2, 4, [600, 1600, 900, 1300, 700], True),
    ("fp8", 8, 16, [0, 700, 800, 900, 1000, 1100, 1200, 1300, 1400, 1500], True),
    ("fp8", 4, 4, [250, 300, 301, 1000, 1200], True),
    ("fp8", 8, 16, [0, 1, 299, 300, 301, 2000, 0, 17], False),
    ("fp8", 6, 8, [5, 700, 0, 1200, 64], False),
    ("bf16", 8, 8, [1000, 1500, 400, 333, 1200], True),
    ("bf16", 1, 2, [0, 0, 33, 900, 4000], False),
    ("spec", 4, 2, [290, 3000, 1200, 301], True),
    ("spec", 4, 4, [0, 3, 4, 300, 1200, 301], False),
])
def test_stream_k_one_wave_per_windowed_unit(kv, hkv, cus, lens, even):
    # with a window and two to eight units per CU the plan launches one wave
    # per (sequence, KV head) unit; the kernels give each unit its own wave
    # when the units are even (here: empty units, units shorter than the
    # window and units cut by it) and equal shares otherwise
    base = {"fp8": SMALL["fp8"], "bf16": SMALL["gqa"].replace(window=300),
            "spec": SMALL["spec"].replace(window=280)}[kv]
    w = base.replace(num_kv_heads=hkv, num_q_heads=(base.num_q_heads // base.num_kv_heads) * hkv,
                     batch=len(lens), seq_len_range=(1, 4000))
    assert _units_even(w, lens) == even
    inp = make(w, seed=90 + hkv, seq_lens=lens)
    p = pkv.query_plan(batch=w.batch, num_q_heads=w.num_q_heads, num_kv_heads=hkv,
                       head_dim_qk=w.head_dim_qk, head_dim_v=w.head_dim_v,
                       pages_per_seq=inp["page_table"].shape[1], page_size=w.page_size,
                       q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, window=w.window,
                       q_seq_len=w.q_seq_len, num_cus=cus)
    print(f"[case] unit waves {kv} Hkv={hkv} cus={cus} lens={lens} even={even}: {p}", flush=True)
    assert p["ctas_per_split_grid"] == w.batch * hkv and p["single_launch"] == 0
    ref = run_oracle(w, inp)
    got = run_gpu(w, inp, num_cus=cus)
    assert_parity(w, got, ref, f"unit/{kv}/Hkv{hkv}/even{even}")
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.equal(got[b].float().cpu(), torch.zeros_like(got[b].float().cpu()))
    # the same call planned as equal shares (forced wave count) agrees
    other = run_gpu(w, inp, target_ctas=7)
    assert_parity(w, other, ref, f"unit-vs-shares/{kv}/Hkv{hkv}")
