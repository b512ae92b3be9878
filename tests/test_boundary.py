"""Host-side tests of the C-ABI library (no GPU needed).

- libpkv.so loads and exports every function include/pkv.h declares;
- the ctypes structs of the binding match the header's layout (a tiny C
  program built with gcc prints sizeof/offsetof);
- argument validation rejects what the xqa page rules out, with a message,
  before anything is launched;
- the split planner's choices (paths, split sizes, workspace sizes).
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import paged_kv_attention_pages_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"pkv_decode_attn", "pkv_workspace_size", "pkv_last_error",
            "pkv_validate_inputs"} <= set(names)
    L = pkv.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", pkv.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (pkv_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    assert pkv.lib().pkv_abi_version() == 7


def test_struct_layouts_match_header(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text("""
#include <stddef.h>
#include <stdio.h>
#include "pkv.h"
#define F(T, m) printf(#T "." #m " %zu\\n", offsetof(T, m));
int main(void) {
  printf("pkv_dims %zu\\n", sizeof(pkv_dims));
  printf("pkv_options %zu\\n", sizeof(pkv_options));
  printf("pkv_plan_info %zu\\n", sizeof(pkv_plan_info));
  F(pkv_dims, workspace_bytes) F(pkv_dims, kv_dtype) F(pkv_options, target_ctas) F(pkv_options, split_event) F(pkv_options, q_scale_dev) F(pkv_options, kv_scale_dev)
  F(pkv_options, merge_mode) F(pkv_options, rcp_out_scale)
  printf("pkv_insert_dims %zu\\n", sizeof(pkv_insert_dims));
  F(pkv_insert_dims, num_q_heads) F(pkv_insert_dims, cache_dtype)
  F(pkv_plan_info, workspace_bytes) F(pkv_plan_info, num_cus) F(pkv_plan_info, single_launch)
  F(pkv_plan_info, waves_per_workgroup)
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(prog), "-o", str(exe)],
                   check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    assert int(got["pkv_dims"]) == ctypes.sizeof(pkv.Dims)
    assert int(got["pkv_options"]) == ctypes.sizeof(pkv.Options)
    assert int(got["pkv_plan_info"]) == ctypes.sizeof(pkv.PlanInfo)
    assert int(got["pkv_dims.workspace_bytes"]) == pkv.Dims.workspace_bytes.offset
    assert int(got["pkv_dims.kv_dtype"]) == pkv.Dims.kv_dtype.offset
    assert int(got["pkv_options.target_ctas"]) == pkv.Options.target_ctas.offset
    assert int(got["pkv_options.split_event"]) == pkv.Options.split_event.offset
    assert int(got["pkv_options.q_scale_dev"]) == pkv.Options.q_scale_dev.offset
    assert int(got["pkv_options.kv_scale_dev"]) == pkv.Options.kv_scale_dev.offset
    assert int(got["pkv_plan_info.workspace_bytes"]) == pkv.PlanInfo.workspace_bytes.offset
    assert int(got["pkv_plan_info.num_cus"]) == pkv.PlanInfo.num_cus.offset
    assert int(got["pkv_options.merge_mode"]) == pkv.Options.merge_mode.offset
    assert int(got["pkv_options.rcp_out_scale"]) == pkv.Options.rcp_out_scale.offset
    assert int(got["pkv_insert_dims"]) == ctypes.sizeof(pkv.InsertDims)
    assert int(got["pkv_insert_dims.num_q_heads"]) == pkv.InsertDims.num_q_heads.offset
    assert int(got["pkv_insert_dims.cache_dtype"]) == pkv.InsertDims.cache_dtype.offset
    assert int(got["pkv_plan_info.single_launch"]) == pkv.PlanInfo.single_launch.offset
    assert int(got["pkv_plan_info.waves_per_workgroup"]) == pkv.PlanInfo.waves_per_workgroup.offset


BASE = dict(batch=64, num_q_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
            pages_per_seq=128, page_size=64, q_dtype=torch.bfloat16, num_cus=256)


def plan(**kw):
    a = dict(BASE)
    a.update(kw)
    return pkv.query_plan(**a)


def test_plan_paths():
    assert plan()["path"] == pkv.PATH_MFMA
    assert plan(path="valu")["path"] == pkv.PATH_VALU
    mla = plan(batch=32, num_q_heads=64, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
               pages_per_seq=256)
    assert mla["path"] == pkv.PATH_MFMA_MLA and mla["rows"] == 64
    spec = plan(q_seq_len=4)
    assert spec["rows"] == 16 and spec["path"] == pkv.PATH_MFMA
    fp8 = plan(batch=128, num_q_heads=64, kv_dtype=torch.float8_e4m3fn, page_size=32,
               pages_per_seq=1024, window=4096)
    assert fp8["rows"] == 8


def test_plan_window_bounds_splits():
    # a 4096-token window over 32-token pages touches at most 129 pages
    p = plan(batch=128, num_q_heads=64, kv_dtype=torch.float8_e4m3fn, page_size=32,
             pages_per_seq=1024, window=4096, path="valu")
    assert p["split_pages"] * p["max_splits"] >= 129
    assert (p["max_splits"] - 1) * p["split_pages"] < 129


def test_plan_stream_k():
    # default matrix-core plan: persistent waves, 4 per CU, two partial slots each
    p = plan()
    assert p["split_pages"] == 0 and p["ctas_per_split_grid"] == 4 * 256
    assert p["workspace_bytes"] >= 2 * 1024 * 4 * (128 * 4 + 8)
    assert plan(target_ctas=100)["ctas_per_split_grid"] == 100
    # the matrix-core schedule runs up to 1024 sequences (head dims <= 128),
    # beyond that the grid schedule; head dim 256 and the latent path stop at 256
    assert plan(batch=300)["split_pages"] == 0
    assert plan(batch=1024)["split_pages"] == 0
    assert plan(batch=1025)["split_pages"] > 0
    assert plan(batch=300, head_dim_qk=256, head_dim_v=256)["split_pages"] > 0
    lat = dict(num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512)
    assert plan(batch=256, **lat)["split_pages"] == 0
    assert plan(batch=257, **lat)["split_pages"] > 0


def test_plan_one_wave_per_short_unit():
    # caches of at most 256 tokens a sequence (or a window that short): one
    # wave per (sequence, KV head), whole, one launch, no workspace
    short = plan(batch=2, num_q_heads=4, num_kv_heads=1, pages_per_seq=16, page_size=16)
    assert short["ctas_per_split_grid"] == 2 and short["single_launch"] == 1
    assert short["workspace_bytes"] == 0 and short["split_pages"] == 0
    assert plan(batch=64, pages_per_seq=4, page_size=64)["workspace_bytes"] == 0          # 256 tokens
    assert plan(batch=64, pages_per_seq=5, page_size=64)["workspace_bytes"] > 0           # 320
    assert plan(batch=64, pages_per_seq=128, page_size=64, window=200)["workspace_bytes"] == 0
    assert plan(batch=64, pages_per_seq=4, page_size=64, num_cus=2)["workspace_bytes"] > 0  # > 8 / CU
    wide = plan(batch=64, pages_per_seq=4, page_size=64)     # 512 units: 2 per CU, 2 heads a group
    assert wide["ctas_per_split_grid"] == 512 and wide["waves_per_workgroup"] == 2
    # forced merges and wave counts keep their plans
    assert plan(batch=64, pages_per_seq=4, page_size=64, target_ctas=100)["workspace_bytes"] > 0
    mla = plan(batch=2, num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
               pages_per_seq=4, page_size=64)
    assert mla["workspace_bytes"] > 0                      # the latent path keeps stream-K
    # the edges: a window reaching 256 tokens (window + q_seq_len - 1) or one
    # more; exactly eight units per CU or one more; an explicit merge choice;
    # the vector path
    assert plan(batch=8, pages_per_seq=128, page_size=64, window=253, q_seq_len=4)["workspace_bytes"] == 0
    assert plan(batch=8, pages_per_seq=128, page_size=64, window=254, q_seq_len=4)["workspace_bytes"] > 0
    assert plan(batch=256, pages_per_seq=4, page_size=64, num_cus=256)["workspace_bytes"] == 0  # 2048 units
    assert plan(batch=257, pages_per_seq=4, page_size=64, num_cus=256)["workspace_bytes"] > 0
    for merge in (True, False):
        p = plan(batch=64, pages_per_seq=4, page_size=64, single_launch=merge)
        assert p["workspace_bytes"] > 0 and p["single_launch"] == (1 if merge else 0)
    valu = plan(batch=2, pages_per_seq=4, page_size=64, path="valu")   # the split grid
    assert valu["path"] == pkv.PATH_VALU and valu["split_pages"] == 4 and valu["single_launch"] == 0


def test_plan_one_wave_per_windowed_unit():
    # with a window, the merge chosen by default and no forced wave count, a
    # batch of at least two units per CU gets B * Hkv waves (the kernels run
    # one per unit when the units are even) with workspace for equal shares
    # over them, and head-grouped workgroups of up to units / CUs waves
    fp8 = dict(batch=128, num_q_heads=64, num_kv_heads=8, kv_dtype=torch.float8_e4m3fn)
    p = plan(window=4096, **fp8)
    assert p["ctas_per_split_grid"] == 1024 and p["waves_per_workgroup"] == 4
    assert p["single_launch"] == 0
    assert p["workspace_bytes"] >= 2 * 1024 * 8 * (128 * 4 + 8)
    assert plan(window=0, **fp8)["ctas_per_split_grid"] == 2048           # no window
    assert plan(window=4096, **dict(fp8, batch=63))["ctas_per_split_grid"] == 2048  # 504 units
    assert plan(window=4096, **dict(fp8, batch=64))["ctas_per_split_grid"] == 512
    assert plan(window=4096, **dict(fp8, batch=64))["waves_per_workgroup"] == 2
    assert plan(window=4096, target_ctas=300, **fp8)["ctas_per_split_grid"] == 300
    assert plan(window=4096, single_launch=True, **fp8)["ctas_per_split_grid"] == 2048
    assert plan(window=4096, batch=256, num_q_heads=32, num_kv_heads=8)["waves_per_workgroup"] == 8
    assert plan(window=4096, batch=300, num_q_heads=6, num_kv_heads=6)["waves_per_workgroup"] == 6
    # up to eight units per CU; beyond, equal shares over the usual waves
    assert plan(window=4096, batch=256, num_q_heads=32, num_kv_heads=8)["ctas_per_split_grid"] == 2048
    assert plan(window=4096, batch=257, num_q_heads=32, num_kv_heads=8)["ctas_per_split_grid"] == 1024
    lat = dict(batch=256, num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512)
    assert plan(window=4096, **lat)["ctas_per_split_grid"] == 256          # latent: its own plan


def test_plan_stream_k_tile_count_edge():
    # the stream-K kernels count tiles (16 tokens; 32 for the latent cache)
    # in 32-bit integers: the last problem under 2^31 tiles keeps stream-K,
    # the next page per sequence moves to the split grid
    big = dict(batch=256, pages_per_seq=262143)          # 2048 units x (4 * pps + 1) tiles
    assert plan(**big)["split_pages"] == 0
    assert 2048 * (4 * 262143 + 1) < 2 ** 31
    p = plan(**dict(big, pages_per_seq=262144))
    assert p["split_pages"] > 0 and p["max_splits"] > 0
    assert 2048 * (4 * 262144 + 1) >= 2 ** 31
    lat = dict(batch=256, num_q_heads=16, num_kv_heads=1, head_dim_qk=576, head_dim_v=512)
    assert plan(**lat, pages_per_seq=4194303)["split_pages"] == 0
    assert plan(**lat, pages_per_seq=4194304)["split_pages"] > 0


def test_plan_latent_fp8_cache_and_query():
    # the latent path takes an e4m3fn cache with a 16-bit or e4m3fn query
    lat = dict(head_dim_qk=576, head_dim_v=512, num_kv_heads=1, num_q_heads=64)
    for q in (torch.bfloat16, torch.float16, torch.float8_e4m3fn):
        p = plan(q_dtype=q, kv_dtype=torch.float8_e4m3fn, **lat)
        assert p["path"] == 3 and p["ctas_per_split_grid"] == 256


def test_plan_head_grouped_workgroups():
    # the matrix-core stream-K plan puts up to a CU's resident waves (4 for
    # 16-bit caches, 8 for fp8; up to 8 below one wave per CU) in one
    # workgroup, one KV head each, when the KV head count divides the wave
    # count: a divisor of Hkv
    assert plan()["waves_per_workgroup"] == 4
    assert plan(kv_dtype=torch.float8_e4m3fn)["waves_per_workgroup"] == 8
    assert plan(target_ctas=2048)["waves_per_workgroup"] == 8
    assert plan(target_ctas=512)["waves_per_workgroup"] == 2
    assert plan(target_ctas=64)["waves_per_workgroup"] == 8
    assert plan(num_kv_heads=2, num_q_heads=8)["waves_per_workgroup"] == 2
    assert plan(num_kv_heads=1, num_q_heads=4)["waves_per_workgroup"] == 1
    assert plan(num_kv_heads=6, num_q_heads=24, target_ctas=48)["waves_per_workgroup"] == 6
    assert plan(num_kv_heads=6, num_q_heads=24, target_ctas=768)["waves_per_workgroup"] == 3
    assert plan(num_kv_heads=6, num_q_heads=24)["waves_per_workgroup"] == 1   # 6 does not divide 1024
    assert plan(target_ctas=12)["waves_per_workgroup"] == 1                   # 8 does not divide 12
    assert plan(split_pages=4)["waves_per_workgroup"] == 1                    # split grid


def test_plan_single_launch_merge():
    # the matrix-core stream-K plan can merge in the split kernel, with one
    # 8-byte counter per (sequence, KV head) after the partials; by default
    # it does when no wave's share can exceed 16 tiles; the split grid and
    # the latent path keep the combine kernel
    one, two = plan(single_launch=True), plan(single_launch=False)
    assert one["single_launch"] == 1 and two["single_launch"] == 0
    assert one["workspace_bytes"] >= two["workspace_bytes"] + 64 * 8 * 8
    assert plan()["single_launch"] == 0                       # 8 K tokens: two launches
    assert plan(pages_per_seq=2)["single_launch"] == 1        # 128 tokens: one launch
    assert plan(pages_per_seq=4, target_ctas=64)["single_launch"] == 0
    assert plan(batch=1100, single_launch=True)["single_launch"] == 0
    assert plan(split_pages=4, single_launch=True)["single_launch"] == 0
    mla = plan(batch=32, num_q_heads=64, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
               pages_per_seq=256, single_launch=True)
    assert mla["single_launch"] == 0


def test_plan_forced_split_and_workspace():
    p = plan(split_pages=1)
    assert p["split_pages"] == 1 and p["max_splits"] == 128
    rows = 4
    want_o = 64 * 8 * 128 * rows * 128 * 4
    assert p["workspace_bytes"] >= want_o + 64 * 8 * 128 * rows * 8
    assert plan(split_pages=128)["split_pages"] == 64   # one page id per lane
    one = plan(split_pages=128, path="valu")
    assert one["max_splits"] == 1 and one["workspace_bytes"] == 0
    assert pkv.workspace_size(**{k: v for k, v in BASE.items() if k != "num_cus"}) > 0


def test_plan_split_sizes_multiple_of_pages_and_at_least_256_tokens():
    for ps in (16, 32, 64, 128):
        p = plan(page_size=ps, pages_per_seq=8192 // ps, path="valu")
        assert p["split_pages"] * ps >= 256
        assert p["split_pages"] * p["max_splits"] >= 8192 // ps


@pytest.mark.parametrize("kw, status, msg", [
    (dict(page_size=48), 1, "page_size"),
    (dict(num_kv_heads=5), 1, "multiple of num_kv_heads"),
    (dict(window=-1), 1, "window"),
    (dict(q_seq_len=0), 1, "q_seq_len"),
    (dict(head_dim_qk=96, head_dim_v=96), 2, "unsupported shape"),
    (dict(q_dtype=torch.float8_e4m3fn, kv_dtype=torch.bfloat16), 1, "float8_e4m3fn KV cache"),
    (dict(q_dtype=torch.float8_e4m3fn, kv_dtype=torch.float8_e4m3fn), 2, "fp8 query"),
    (dict(q_seq_len=5), 2, "rows"),
    (dict(path="valu", q_seq_len=4), 2, "vector path"),
    (dict(path="mfma_mla"), 2, "latent path"),
    (dict(kv_dtype=torch.float16), 1, "KV cache dtype"),
    (dict(pages_per_seq=0), 1, "pages_per_seq"),
])
def test_plan_rejects(kw, status, msg):
    with pytest.raises(pkv.PkvError) as e:
        plan(**kw)
    assert e.value.status == status
    assert msg in str(e.value)


def _raw_decode(**over):
    """Call pkv_decode_attn directly with fake pointers; validation must fail first."""
    d = pkv.Dims(64, 32, 128, 128, 128, 1000, 1, 1, 1 << 30)
    args = dict(q=8192, k=8192, v=8192, pt=8192, sl=8192, out=8192, ws=8192, hkv=8, ps=64,
                layout=0, sinks=None, qs=1.0, ks=1.0, win=0, tq=1, mask=None, stream=None, dims=d)
    args.update(over)
    L = pkv.lib()
    st = L.pkv_decode_attn(*[ctypes.c_void_p(a) if isinstance(a, int) else a for a in (
        args["q"], args["k"], args["v"], args["pt"], args["sl"], args["out"], args["ws"])],
        args["hkv"], args["ps"], args["layout"], args["sinks"], args["qs"], args["ks"],
        args["win"], args["tq"], args["mask"], args["stream"], ctypes.byref(args["dims"]))
    return st, L.pkv_last_error().decode()


def test_decode_rejects_before_launch():
    assert _raw_decode(ps=12)[0] == 1
    assert _raw_decode(layout=7)[0] == 1
    st, msg = _raw_decode(q=None)
    assert st == 1 and "NULL" in msg
    st, msg = _raw_decode(q=8200)
    assert st == 1 and "aligned" in msg
    st, msg = _raw_decode(dims=pkv.Dims(64, 32, 128, 128, 128, 1000, 1, 1, 16))
    assert st == 3 and "workspace" in msg
    st, msg = _raw_decode(qs=float("nan"))
    assert st == 1 and "finite" in msg
    st, msg = _raw_decode(dims=pkv.Dims(64, 32, 128, 128, 128, 1000, 0, 1, 1 << 30))
    assert st == 1 and "KV cache dtype" in msg


def test_zero_batch_is_a_noop():
    st, msg = _raw_decode(dims=pkv.Dims(0, 32, 128, 128, 128, 1000, 1, 1, 0), q=None, out=None)
    assert st == 0, msg


def test_binding_rejects_cpu_tensors():
    q = torch.zeros(2, 1, 4, 128, dtype=torch.float16)
    k = torch.zeros(4, 16, 1, 128, dtype=torch.float16)
    with pytest.raises(pkv.PkvError, match="GPU"):
        pkv.decode_attn(q, k, k, torch.zeros(2, 4, dtype=torch.int32),
                        torch.zeros(2, dtype=torch.int32), torch.empty_like(q),
                        num_kv_heads=1, page_size=16)


def _insert_dims(**kw):
    d = dict(num_tokens=4, num_kv_heads=2, head_dim_k=128, head_dim_k_lo=128, head_dim_v=128,
             page_size=16, num_pages=8, layout=0, src_dtype=1, cache_dtype=1, num_q_heads=0)
    d.update(kw)
    return pkv.InsertDims(**d)


@pytest.mark.parametrize("kw, msg", [
    (dict(head_dim_k=100), "multiples of 8"),
    (dict(head_dim_k_lo=136), "multiples of 8"),
    (dict(head_dim_v=12), "multiples of 8"),
    (dict(page_size=8), "page_size"),
    (dict(layout=3), "kv_layout"),
    (dict(src_dtype=2), "source dtype"),
    (dict(cache_dtype=0), "cache dtype"),
    (dict(num_kv_heads=0), "num_kv_heads"),
    (dict(num_tokens=-1), "num_tokens"),
])
def test_cache_insert_rejects_bad_sizes(kw, msg):
    # checked on the host before any device call
    L = pkv.lib()
    st = L.pkv_cache_insert(None, None, None, None, None, None, 1.0, None, None, None, None, None,
                            ctypes.byref(_insert_dims(**kw)))
    assert st == 1 and msg in L.pkv_last_error().decode()


def test_cache_insert_null_tensors_and_bad_scale():
    L = pkv.lib()
    st = L.pkv_cache_insert(None, None, None, None, None, None, 1.0, None, None, None, None, None,
                            ctypes.byref(_insert_dims()))
    assert st == 1 and "must not be NULL" in L.pkv_last_error().decode()
    st = L.pkv_cache_insert(None, None, None, None, None, None, float("inf"), None, None, None,
                            None, None, ctypes.byref(_insert_dims()))
    assert st == 1 and "finite" in L.pkv_last_error().decode()
    # nothing to insert: no device call, success
    assert L.pkv_cache_insert(None, None, None, None, None, None, 1.0, None, None, None, None, None,
                              ctypes.byref(_insert_dims(num_tokens=0))) == 0


@pytest.mark.parametrize("M, H, K, N, dtype, msg", [
    (-1, 4, 32, 64, 1, "M >= 0"),
    (4, 0, 32, 64, 1, "H >= 1"),
    (4, 4, 48, 64, 1, "multiple of 32"),
    (4, 4, 32, 96, 1, "multiple of 64"),
    (4, 4, 32, 64, 2, "float16 or bfloat16"),
])
def test_head_matmul_rejects_bad_sizes(M, H, K, N, dtype, msg):
    L = pkv.lib()
    st = L.pkv_head_matmul(None, 8 * 32, 32, None, None, 64, 64, M, H, K, N, dtype, None)
    assert st == 1 and msg in L.pkv_last_error().decode()


def test_head_matmul_rejects_strides_and_nulls():
    L = pkv.lib()
    assert L.pkv_head_matmul(None, 12, 32, None, None, 64, 64, 4, 4, 32, 64, 1, None) == 1
    assert "strides" in L.pkv_last_error().decode()
    assert L.pkv_head_matmul(None, 128, 32, None, None, 64, 64, 4, 4, 32, 64, 1, None) == 1
    assert "must not be NULL" in L.pkv_last_error().decode()
    assert L.pkv_head_matmul(None, 128, 32, None, None, 64, 64, 0, 4, 32, 64, 1, None) == 0


@pytest.mark.parametrize("N, H, D, n_pre, dtype, msg", [
    (-1, 2, 64, 0, 1, "N >= 0"),
    (4, 0, 64, 0, 1, "H >= 1"),
    (4, 2, 60, 0, 1, "multiple of 8"),
    (4, 2, 64, 5, 1, "num_tokens_with_prefix <= N"),
    (4, 2, 64, -1, 1, "num_tokens_with_prefix <= N"),
    (4, 2, 64, 2, 2, "float16 or bfloat16"),
])
def test_merge_attn_states_rejects_bad_sizes(N, H, D, n_pre, dtype, msg):
    L = pkv.lib()
    st = L.pkv_merge_attn_states(None, None, H * D, D, None, None, H * D, D, None, None, 1, N, N, H,
                                 D, n_pre, dtype, None)
    assert st == 1 and msg in L.pkv_last_error().decode()


def _merge(lse_sn=1, p_sn=128, s_sh=64, N=4, n_pre=2):
    return pkv.lib().pkv_merge_attn_states(None, None, p_sn, 64, None, None, 128, s_sh, None, None,
                                           lse_sn, 4, N, 2, 64, n_pre, 1, None)


def test_merge_attn_states_nulls_strides_and_empty():
    L = pkv.lib()
    assert _merge() == 1 and "must not be NULL" in L.pkv_last_error().decode()
    assert _merge(lse_sn=-1) == 1 and "non-negative" in L.pkv_last_error().decode()
    assert _merge(p_sn=12) == 1 and "multiples of 8" in L.pkv_last_error().decode()
    assert _merge(s_sh=-8) == 1 and "multiples of 8" in L.pkv_last_error().decode()
    assert _merge(N=0, n_pre=0) == 0


def _ragged(num_seqs=2, Hq=4, Hkv=2, Dqk=128, Dv=128, total_q=10, total_k=12, max_q_len=8,
            sm_scale=0.1, causal=1, dtype=1, lse_sn=1, lse_sh=10):
    return pkv.lib().pkv_ragged_attn(None, None, None, None, None, None, None, lse_sn, lse_sh,
                                     num_seqs, Hq, Hkv, Dqk, Dv, total_q, total_k, max_q_len,
                                     sm_scale, causal, dtype, None)


@pytest.mark.parametrize("kw, status, msg", [
    (dict(num_seqs=-1), 1, "num_seqs"),
    (dict(Hq=6, Hkv=4), 1, "multiple of num_kv_heads"),
    (dict(Dqk=96, Dv=96), 2, "head dims"),
    (dict(Dqk=192, Dv=192), 2, "head dims"),
    (dict(dtype=2), 1, "float16 or bfloat16"),
    (dict(causal=2), 1, "causal must be 0 or 1"),
    (dict(sm_scale=float("nan")), 1, "finite"),
    (dict(sm_scale=0.0), 1, "positive"),
    (dict(sm_scale=-0.5), 1, "positive"),
    (dict(lse_sh=-1), 1, "non-negative"),
    (dict(num_seqs=70000), 2, "65535"),
    (dict(total_k=1 << 22, Hkv=2, Hq=4), 2, "2 GiB"),
    (dict(), 1, "must not be NULL"),
])
def test_ragged_attn_rejects_before_launch(kw, status, msg):
    st = _ragged(**kw)
    assert st == status and msg in pkv.lib().pkv_last_error().decode()


def test_ragged_attn_empty_calls_do_nothing():
    assert _ragged(num_seqs=0) == 0
    assert _ragged(max_q_len=0) == 0
    assert _ragged(total_q=0) == 0
