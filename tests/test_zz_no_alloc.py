"""The allocation-free decode entry point (pkv_decode_attn_noalloc).

Its partial results live in the library's static per-GPU scratch instead of
a workspace.  It runs the same plan and kernels as pkv_decode_attn_ex, so on
the GPU its output must equal that entry point's bit for bit (and both stay
within the oracle tolerance), on two calls in a row, the second smaller, so
the second reads scratch the first one left behind.  On the CPU: the scratch
size in the header matches the binding, and an oversized plan is rejected
before any device work.
"""
import ctypes
import os
import subprocess

import pytest
import torch

import paged_kv_attention_pages_amd as pkv
from tests.test_parity_gpu import DEV, SMALL, assert_parity, make, run_gpu, run_oracle

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "pkv.h")


def test_scratch_size_matches_header(tmp_path):
    prog = tmp_path / "size.c"
    prog.write_text('#include <stdio.h>\n#include "pkv.h"\n'
                    'int main(void) { printf("%zu\\n", PKV_NOALLOC_SCRATCH_BYTES); return 0; }\n')
    exe = tmp_path / "size"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(prog), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    assert int(out) == pkv.NOALLOC_SCRATCH_BYTES == 96 << 20


def _noalloc_host_call(batch, pages_per_seq):
    # host-only call: NULL buffers, the CU count given (no device query)
    d = pkv.Dims(batch, 32, 128, 128, pages_per_seq, 1, 1, 1, 0)
    o = pkv.Options()
    o.num_cus = 256
    L = pkv.lib()
    st = L.pkv_decode_attn_noalloc(None, None, None, None, None, None, 8, 16, 0, None, 1.0, 1.0,
                                   0, 1, None, None, ctypes.byref(d), ctypes.byref(o))
    return st, L.pkv_last_error().decode()


def test_oversized_plan_is_rejected_before_device_work():
    # 4096 sequences take the split grid, whose partials exceed the scratch
    need = pkv.query_plan(batch=4096, num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
                          head_dim_v=128, pages_per_seq=1024, page_size=16,
                          num_cus=256)["workspace_bytes"]
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    st, msg = _noalloc_host_call(4096, 1024)
    assert st == 3, msg                      # PKV_ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in msg and str(need) in msg
    # an empty batch succeeds without touching the device
    st, msg = _noalloc_host_call(0, 1024)
    assert st == 0, msg


CASES = {
    "gqa": dict(),
    "fp8": dict(),
    "spec": dict(),
    "mla": dict(),
    "gqa_single_launch": dict(single_launch=True, target_ctas=7),
    "gqa_split_grid": dict(split_pages=2),
    # a window and two units per CU: one wave per (sequence, KV head)
    "fp8_unit_waves": dict(num_cus=2),
    # fp8 query and latent cache (64-token tiles), four workgroups
    "mla_fp8": dict(target_ctas=4),
    # at most 256 tokens a sequence: one wave per unit, no scratch at all
    "gqa_short": dict(),
}


@pytest.mark.gpu
@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_matches_workspace_entry_point(case):
    name = case.split("_")[0]
    kw = CASES[case]
    w1 = SMALL[name]
    if case == "mla_fp8":
        w1 = w1.replace(q_dtype=torch.float8_e4m3fn, kv_dtype=torch.float8_e4m3fn, kv_scale=0.05,
                        kv_gen_scale=1.0 / 0.05)
    if case == "gqa_short":
        w1 = w1.replace(seq_len_range=(1, 256))
    lo, hi = w1.seq_len_range
    w2 = w1.replace(batch=max(1, w1.batch - 2), seq_len_range=(lo, max(lo, hi // 3)))
    for step, (w, seed) in enumerate(((w1, 201), (w2, 202))):
        print(f"[case] noalloc {case} call {step + 1} batch {w.batch}", flush=True)
        inp = make(w, seed=seed)
        want = run_gpu(w, inp, **kw)
        got = torch.full_like(want, float("nan"))
        pkv.decode_attn_noalloc(inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"],
                                inp["seq_lens"], got, num_kv_heads=w.num_kv_heads,
                                page_size=w.page_size, sinks=inp["sinks"], q_scale=w.q_scale,
                                kv_scale=w.kv_scale, sliding_win_size=w.window,
                                kv_layout=w.kv_layout, q_seq_len=w.q_seq_len, mask=inp["mask"],
                                head_dim_v=w.head_dim_v, **kw)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), case
        assert_parity(w, got, run_oracle(w, inp), f"noalloc/{case}/{step + 1}")
