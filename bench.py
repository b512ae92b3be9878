"""Benchmark: paged GQA decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--batch B]

A step is one decode call (split-KV kernel + combine kernel) over one batch
of the workload, with every input already resident in HBM.  The default
workload is the Llama-3-8B-shaped GQA decode (batch 64, 32 query heads on 8
KV heads, head_dim 128, bf16, HND, 64-token pages, lengths uniform in
[1024, 8192]).  Caches larger than the 256 MB last-level cache are timed as
they are; smaller ones rotate through replicas totalling >= 1.5 GB so that
each call reads cold data.

Reported (one JSON line on stdout):
  value        effective KV bandwidth, algorithmic KV bytes / wall time per
               call (GB/s) over K back-to-back calls with no events between
               them; us_per_call and the fraction of the 8 TB/s HBM peak
               beside it
  roofline     the split-KV kernel alone, from a second pass of K calls with
               HIP events on the launch stream around it: algorithmic KV
               bytes per launch / its mean time, against the HBM peak
  cpu_baseline the fp64 oracle on a bounded sample of the same batch, on the
               host cores (a reported baseline, not the target)
  host_us_per_call  the host side of a call (binding + launch), each call
               timed alone after a synchronisation, median of up to 100
  configs      (default run) the other decode configurations measured the same
               way in the same run -- tiny, fp8 + window + sinks, speculative
               decode, latent (MLA) and its fp8 form: us/call, effective GB/s,
               % of HBM peak, the split-KV kernel's fraction of peak (and, for
               the latent kernel, of the bf16 matrix-core peak), the combine
               time and an oracle baseline on a smaller sample
Each workload's seed is its number in the list of configurations.
Algorithmic KV bytes = sum over sequences of (tokens some query row can see)
x num_kv_heads x (head_dim_qk + head_dim_v) x element size; a latent cache
row serves as K and V and counts once.

    python bench.py --workload insert_prefill | insert_prefill_fp8 |
                    insert_decode | insert_latent_decode

times the cache write side instead (pkv_cache_insert: new tokens' rows into
their slots): value = bytes read + bytes written per call / wall time.

    python bench.py --workload latent_absorb | latent_up_proj

times the latent-attention projections around the decode (pkv_head_matmul:
BMM1 with W_UK_T, the up-projection with W_UV) for the latent workload's 32
decode tokens and 64 heads; value = bytes read + written / wall time (the
weights dominate).

    python bench.py --workload merge_chunked_prefill

times the merge of two attention results by their log-sum-exps
(pkv_merge_attn_states) for a chunked prefill of 8192 tokens, 128 heads,
head dim 128; value = bytes read + written / wall time.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published


def kv_bytes_of(w, L: torch.Tensor) -> int:
    if w.window > 0:
        lo = (L - w.q_seq_len + 1 - w.window).clamp(min=0)
        vis = (L - lo).clamp(min=0)
    else:
        vis = L
    elem = 1 if w.kv_dtype == torch.float8_e4m3fn else 2
    row = w.head_dim_qk + (0 if w.v_from_k else w.head_dim_v)
    return int(vis.sum()) * w.num_kv_heads * row * elem


def measured_traffic(workload: str, forced: bool):
    """HBM bytes per launch of the split kernel from the committed counter runs.

    The record holds FETCH_SIZE/WRITE_SIZE (KiB per dispatch) with their copy-
    kernel scale factors and a hash of the kernel sources; it is used only for
    the default plan and only while those sources are unchanged (else None).
    """
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if forced or not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload)
    if rec is None:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return int(rec["fetch_kib_per_dispatch"] * rec["fetch_scale"] * 1024
               + rec["write_kib_per_dispatch"] * rec["write_scale"] * 1024)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b_gqa")
    ap.add_argument("--path", default=None, help="auto | valu | mfma | mfma_mla")
    ap.add_argument("--split-pages", type=int, default=0)
    ap.add_argument("--target-ctas", type=int, default=0)
    ap.add_argument("--batch", type=int, default=0,
                    help="number of sequences of the named decode workload (0: its own)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure only the named workload (the default run also measures the other "
                         "decode configurations and reports them under 'configs')")
    ap.add_argument("--config-cpu-seconds", type=float, default=5.0,
                    help="approximate CPU time budget of each other configuration's oracle baseline")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (paged decode "
              "attention shards over sequences and KV heads with no exchange; see the design "
              "notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.workload in INSERT_WORKLOADS:
        return bench_insert(args)
    if args.workload in PROJ_WORKLOADS:
        return bench_proj(args)
    if args.workload in MERGE_WORKLOADS:
        return bench_merge(args)
    if args.workload in RAGGED_WORKLOADS:
        return bench_ragged(args)

    import paged_kv_attention_pages_amd as pkv
    from paged_kv_attention_pages_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rec = measure_decode(args.workload, args, args.cpu_seconds, headline=True)
    if args.workload == "llama3_8b_gqa" and not args.no_configs and not (args.path or args.split_pages or
                                                                          args.target_ctas or args.batch):
        # every other decode configuration, measured in the same run
        cfgs = {}
        for name in ["tiny", "fp8_window_sinks", "spec_decode", "mla", "mla_fp8"]:
            torch.cuda.empty_cache()
            cfgs[name] = measure_decode(name, args, args.config_cpu_seconds, headline=False)
        rec["configs"] = cfgs
    print(json.dumps(rec), flush=True)


# The seed of each decode workload: its number in the list of synthetic
# configurations (the fp8 latent form shares the latent workload's draw).
SEEDS = {"tiny": 1, "llama3_8b_gqa": 2, "fp8_window_sinks": 3, "spec_decode": 4, "mla": 5,
         "mla_fp8": 5}


def measure_decode(name, args, cpu_budget, headline):
    """One decode workload: wall time over K back-to-back calls, then an
    evented pass that splits each call into the split-KV kernel and the
    combine; the oracle on a bounded sample of the same batch.  Returns the
    JSON record (the top-level line for the headline workload, a compact
    sub-record otherwise)."""
    import paged_kv_attention_pages_amd as pkv
    from paged_kv_attention_pages_amd import synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[name]
    if headline and args.batch:
        w = w.replace(batch=args.batch)
    seed = SEEDS.get(name, 1)
    L = synth.draw_seq_lens(w, seed)
    kf = (L - w.q_seq_len + 1 - w.window).clamp(min=0) if w.window > 0 else None
    inp = synth.make_inputs(w, seed=seed, device=dev, seq_lens=L, keep_from=kf)
    cache_bytes = inp["k_cache"].numel() * inp["k_cache"].element_size()
    if not w.v_from_k:
        cache_bytes += inp["v_cache"].numel() * inp["v_cache"].element_size()
    n_rep = max(1, math.ceil(1.5e9 / cache_bytes)) if cache_bytes < 1.0e9 else 1
    reps = [inp]
    for _ in range(n_rep - 1):
        k2 = inp["k_cache"].clone()
        reps.append(dict(inp, k_cache=k2, v_cache=k2 if w.v_from_k else inp["v_cache"].clone()))
    kv_bytes = kv_bytes_of(w, L)
    B = L.numel()
    # an fp8 query's output is bfloat16
    out_dt = torch.bfloat16 if w.q_dtype == torch.float8_e4m3fn else w.q_dtype
    out = torch.empty((B, w.q_seq_len, w.num_q_heads, w.head_dim_v), dtype=out_dt, device=dev)
    plan = pkv.query_plan(batch=B, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                          head_dim_qk=w.head_dim_qk, head_dim_v=w.head_dim_v,
                          pages_per_seq=inp["page_table"].shape[1], page_size=w.page_size,
                          q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, window=w.window,
                          q_seq_len=w.q_seq_len, path=args.path, split_pages=args.split_pages,
                          target_ctas=args.target_ctas)
    ws = torch.empty(max(plan["workspace_bytes"], 256), dtype=torch.uint8, device=dev)

    def call(i, ev=None):
        r = reps[i % n_rep]
        pkv.decode_attn(r["q"], r["k_cache"], r["v_cache"], r["page_table"], r["seq_lens"], out,
                        ws, num_kv_heads=w.num_kv_heads, page_size=w.page_size, sinks=r["sinks"],
                        q_scale=w.q_scale, kv_scale=w.kv_scale, sliding_win_size=w.window,
                        kv_layout=w.kv_layout, q_seq_len=w.q_seq_len, mask=r["mask"],
                        head_dim_v=w.head_dim_v, path=args.path, split_pages=args.split_pages,
                        target_ctas=args.target_ctas, split_event=ev)

    K, W = args.steps, args.warmup
    for i in range(W):
        call(i)
    print(f"[bench] {w.name}: warmup done ({W} calls), timing {K}", file=sys.stderr, flush=True)
    # pass 1 -- the metric: K calls back to back, no events inside (a timing
    # event on the stream costs several microseconds per call)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        call(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    # pass 2 -- the breakdown: the same K calls with HIP events on the launch
    # stream before the call, between the split and combine kernels, and after
    ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_m = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    for e in ev_m:  # create the device events before handing their handles over
        e.record()
    torch.cuda.synchronize()
    for i in range(K):
        ev_s[i].record()
        call(i, ev_m[i])
        ev_e[i].record()
    torch.cuda.synchronize()
    call_ms = [ev_s[i].elapsed_time(ev_e[i]) for i in range(K)]
    split_ms = [ev_s[i].elapsed_time(ev_m[i]) for i in range(K)]
    comb_ms = [ev_m[i].elapsed_time(ev_e[i]) for i in range(K)]
    split_mean = statistics.fmean(split_ms)
    # pass 3 -- the host side: each call timed alone on the host after a
    # synchronisation (binding + launch, with an empty launch queue)
    host = []
    for i in range(min(K, 100)):
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        call(i)
        host.append(time.perf_counter() - h0)
    torch.cuda.synchronize()
    host_us = statistics.median(host) * 1e6
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = kv_bytes / (split_mean * 1e-3) / 1e9
    print(f"[bench] {w.name}: {ms_per_step * 1e3:.1f} us/call wall, evented pass: call median "
          f"{statistics.median(call_ms) * 1e3:.1f} us (split {split_mean * 1e3:.1f} us, combine "
          f"{statistics.fmean(comb_ms) * 1e3:.1f} us), host {host_us:.1f} us per call, "
          f"{value:.0f} GB/s effective, plan {plan}",
          file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp, L, cpu_budget)
    traffic = measured_traffic(w.name, bool(args.path or args.split_pages or args.target_ctas))
    path = pkv.PATH_NAMES.get(plan["path"], plan["path"])
    del reps, inp
    dtype = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float8_e4m3fn: "fp8"}[w.q_dtype]
    if w.kv_dtype == torch.float8_e4m3fn:
        dtype += "+fp8kv"
    cfg = {
        "workload": w.name, "seed": seed, "batch": B, "q_seq_len": w.q_seq_len,
        "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
        "head_dim_qk": w.head_dim_qk, "head_dim_v": w.head_dim_v,
        "kv_layout": w.kv_layout, "page_size": w.page_size,
        "seq_len_range": list(w.seq_len_range) if w.seq_len_range else list(w.fixed_seq_lens),
        "window": w.window, "sinks": w.sinks, "mask": w.mask,
        "kv_dtype": str(w.kv_dtype).replace("torch.", ""),
        "kv_bytes_per_call": kv_bytes, "cache_replicas": n_rep, "path": path,
        "split_pages": plan["split_pages"], "max_splits": plan["max_splits"],
        "single_launch": bool(plan["single_launch"]),
    }
    if not headline:
        sub = {
            "config": cfg, "dtype": dtype, "us_per_call": round(ms_per_step * 1e3, 2),
            "us_per_call_evented_median": round(statistics.median(call_ms) * 1e3, 2),
            "us_per_call_evented_p10_p90": [round(q * 1e3, 2) for q in _p10_p90(call_ms)],
            "effective_gbs": round(value, 2), "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "split_us_mean": round(split_mean * 1e3, 2),
            "split_frac_hbm_peak": round(achieved / HBM_PEAK_GBS, 4),
            "combine_us_mean": round(statistics.fmean(comb_ms) * 1e3, 2),
            "host_us_per_call": round(host_us, 2),
            "traffic": traffic, "cpu_baseline": cpu,
        }
        if path == "mfma_mla":
            # matrix-core work: every visible token x rows x (Dqk + Dv) x 2 flop
            vis = int((L - ((L - w.q_seq_len + 1 - w.window).clamp(min=0) if w.window > 0 else 0)).sum())
            flops = 2.0 * vis * w.num_q_heads * w.q_seq_len * (w.head_dim_qk + w.head_dim_v)
            sub["split_mfma_frac"] = round(flops / (split_mean * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        return sub
    return {
        "metric": "effective KV GB/s (% of HBM peak) + us/call, paged GQA decode attention",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "us_per_call": round(ms_per_step * 1e3, 2),
        "us_per_call_evented_median": round(statistics.median(call_ms) * 1e3, 2),
        "us_per_call_evented_p10_p90": [round(q * 1e3, 2) for q in _p10_p90(call_ms)],
        "host_us_per_call": round(host_us, 2),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "config": cfg,
        "roofline": {
            "kernel": "split-KV decode (" + path + ")",
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes": kv_bytes, "launch_us_mean": round(split_mean * 1e3, 2),
        },
        "cpu_baseline": cpu,
    }


# The write side (cache insert).  Shapes: the prefill inserts write one
# 32 K-token prompt's K/V rows of the Llama-3-8B-shaped cache (8 KV heads,
# head_dim 128, HND, 64-token pages); the decode inserts write one token per
# sequence of the decode workloads (GQA: 64 sequences; latent: 32 sequences,
# row [512 | 64] plus the 64-head query concat).
INSERT_WORKLOADS = {
    "insert_prefill": dict(N=32768, Hkv=8, Dk=128, Dlo=128, Dv=128, ps=64, layout="HND",
                           cache=torch.bfloat16, Hq=0),
    "insert_prefill_fp8": dict(N=32768, Hkv=8, Dk=128, Dlo=128, Dv=128, ps=64, layout="HND",
                               cache=torch.float8_e4m3fn, Hq=0),
    "insert_decode": dict(N=64, Hkv=8, Dk=128, Dlo=128, Dv=128, ps=64, layout="HND",
                          cache=torch.bfloat16, Hq=0),
    "insert_latent_decode": dict(N=32, Hkv=1, Dk=576, Dlo=512, Dv=0, ps=64, layout="NHD",
                                 cache=torch.bfloat16, Hq=64),
}


PROJ_WORKLOADS = {
    "latent_absorb": dict(M=32, H=64, K=128, N=512),
    "latent_up_proj": dict(M=32, H=64, K=512, N=128),
}


def bench_proj(args):
    import paged_kv_attention_pages_amd as pkv
    cfg = PROJ_WORKLOADS[args.workload]
    M, H, K, N = cfg["M"], cfg["H"], cfg["K"], cfg["N"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev).manual_seed(1)
    x = torch.randn(M, H, K, generator=g, device=dev).to(torch.bfloat16)
    # weights rotate through replicas totalling >= 1 GB (read from HBM each call)
    wb = H * K * N * 2
    n_rep = min(128, max(1, math.ceil(1.0e9 / wb)))
    ws = [(torch.randn(H, K, N, generator=g, device=dev) / math.sqrt(K)).to(torch.bfloat16)
          for _ in range(n_rep)]
    y = torch.empty(M, H, N, dtype=torch.bfloat16, device=dev)
    nbytes = wb + M * H * (K + N) * 2
    K_, W_ = args.steps, args.warmup
    for i in range(W_):
        pkv.head_matmul(x, ws[i % n_rep], y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K_):
        pkv.head_matmul(x, ws[i % n_rep], y)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K_
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K_)]
    for i, (a, b) in enumerate(ev):
        a.record()
        pkv.head_matmul(x, ws[i % n_rep], y)
        b.record()
    torch.cuda.synchronize()
    kern_ms = statistics.fmean(a.elapsed_time(b) for a, b in ev)
    value = nbytes / (ms * 1e-3) / 1e9
    flops = 2.0 * M * H * K * N
    print(f"[bench] {args.workload}: {ms * 1e3:.2f} us/call wall, evented {kern_ms * 1e3:.2f} us, "
          f"{value:.0f} GB/s", file=sys.stderr, flush=True)
    rec = {
        "metric": "latent projection GB/s (bytes read + written) + us/call",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K_, "warmup": W_,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "us_per_call": round(ms * 1e3, 2),
        "config": {"workload": args.workload, "tokens": M, "heads": H, "k": K, "n": N,
                   "bytes_per_call": nbytes, "flops_per_call": flops, "weight_replicas": n_rep},
        "roofline": {"kernel": "head matmul", "bound": "hbm",
                     "achieved": round(nbytes / (kern_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(nbytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes": nbytes,
                     "launch_us_mean": round(kern_ms * 1e3, 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


MERGE_WORKLOADS = {
    # chunked prefill of 8192 new tokens, 128 heads, value head dim 128
    "merge_chunked_prefill": dict(N=8192, H=128, D=128),
}


def bench_merge(args):
    import paged_kv_attention_pages_amd as pkv
    cfg = MERGE_WORKLOADS[args.workload]
    N, H, D = cfg["N"], cfg["H"], cfg["D"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev).manual_seed(1)
    po = torch.randn(N, H, D, generator=g, device=dev).to(torch.bfloat16)
    so = torch.randn(N, H, D, generator=g, device=dev).to(torch.bfloat16)
    pl = torch.randn(H, N, generator=g, device=dev) * 4
    sl = torch.randn(H, N, generator=g, device=dev) * 4
    out = torch.empty_like(so)
    lse = torch.empty_like(sl)
    # two outputs read, one written; two log-sum-exps read, one written
    nbytes = 3 * N * H * D * 2 + 3 * N * H * 4

    def call():
        pkv.merge_attn_states(out, po, pl, so, sl, N, lse)

    K_, W_ = args.steps, args.warmup
    for _ in range(W_):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K_):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K_
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K_)]
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    kern_ms = statistics.fmean(a.elapsed_time(b) for a, b in ev)
    value = nbytes / (ms * 1e-3) / 1e9
    print(f"[bench] {args.workload}: {ms * 1e3:.2f} us/call wall, evented {kern_ms * 1e3:.2f} us, "
          f"{value:.0f} GB/s", file=sys.stderr, flush=True)
    rec = {
        "metric": "attention-state merge GB/s (bytes read + written) + us/call",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K_, "warmup": W_,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "us_per_call": round(ms * 1e3, 2),
        "config": {"workload": args.workload, "tokens": N, "heads": H, "head_dim": D,
                   "bytes_per_call": nbytes},
        "roofline": {"kernel": "merge states", "bound": "hbm",
                     "achieved": round(nbytes / (kern_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(nbytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes": nbytes,
                     "launch_us_mean": round(kern_ms * 1e3, 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


# Ragged (non-paged) attention: the new-token attention of a chunked
# prefill at the latent model's materialised head shape (qk 192 = 128 nope +
# 64 rope, v 128), one GPU's 64-head share, 4 sequences of 4096 new tokens,
# causal; and the context attention of 1024 new tokens over 16384 cached
# context tokens (not causal).
RAGGED_WORKLOADS = {
    "ragged_prefill": dict(lens_q=[4096] * 4, lens_k=[4096] * 4, H=64, Hkv=64, Dqk=192, Dv=128,
                           causal=True),
    "ragged_context": dict(lens_q=[1024] * 2, lens_k=[16384] * 2, H=64, Hkv=64, Dqk=192, Dv=128,
                           causal=False),
}
MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_ragged(args):
    import paged_kv_attention_pages_amd as pkv
    from paged_kv_attention_pages_amd import synth
    cfg = RAGGED_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    H, Hkv, Dqk, Dv = cfg["H"], cfg["Hkv"], cfg["Dqk"], cfg["Dv"]
    inp = synth.make_ragged(cfg["lens_q"], cfg["lens_k"], H, Hkv, Dqk, Dv, torch.bfloat16, 1, dev)
    # visible (query, key) pairs per head; two products of Dqk and Dv per pair
    pairs = 0
    for lq, lk in zip(cfg["lens_q"], cfg["lens_k"]):
        pairs += sum(min(lk, max(0, i + lk - lq + 1)) for i in range(lq)) if cfg["causal"] else lq * lk
    flops = 2 * pairs * H * (Dqk + Dv)
    out = torch.empty((inp["q"].shape[0], H, Dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((H, inp["q"].shape[0]), dtype=torch.float32, device=dev)

    def call():
        pkv.ragged_attn(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                        max_q_len=inp["max_q_len"], sm_scale=Dqk ** -0.5, causal=cfg["causal"],
                        out=out, lse=lse)

    K_, W_ = args.steps, args.warmup
    for _ in range(W_):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K_):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K_
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K_)]
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    kern_ms = statistics.fmean(a.elapsed_time(b) for a, b in ev)
    value = flops / (ms * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    print(f"[bench] {args.workload}: {ms * 1e3:.1f} us/call wall, evented {kern_ms * 1e3:.1f} us, "
          f"{value:.1f} TFLOP/s", file=sys.stderr, flush=True)
    cpu = None
    if not getattr(args, "no_cpu_baseline", True):
        cpu = ragged_cpu_baseline(cfg, inp, args.cpu_seconds)
    rec = {
        "metric": "ragged attention TFLOP/s (visible query-key pairs) + us/call",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K_, "warmup": W_,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "us_per_call": round(ms * 1e3, 2),
        "config": {"workload": args.workload, "seqs": len(cfg["lens_q"]), "lens_q": cfg["lens_q"][0],
                   "lens_k": cfg["lens_k"][0], "heads": H, "kv_heads": Hkv, "head_dim_qk": Dqk,
                   "head_dim_v": Dv, "causal": cfg["causal"], "flops_per_call": flops},
        "roofline": {"kernel": "ragged attention (mfma)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(args.workload, False), "algorithmic_flops": flops,
                     "launch_us_mean": round(kern_ms * 1e3, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def ragged_cpu_baseline(cfg, inp, budget_s):
    """The fp64 oracle on a bounded sample of the ragged workload: the last
    queries of the first sequence (the ones that see the most keys), one head
    at a time, as many heads as fit in the budget; TFLOP/s of the same
    algorithmic flop count."""
    import oracle
    Lq, Lk = cfg["lens_q"][0], cfg["lens_k"][0]
    nq = min(Lq, 64)
    q = inp["q"][Lq - nq:Lq].cpu()
    k = inp["k"][:Lk].cpu()
    v = inp["v"][:Lk].cpu()
    G = cfg["H"] // cfg["Hkv"]
    flops = 0
    t0 = time.perf_counter()
    heads = 0
    for h in range(cfg["H"]):
        kv = h // G
        # queries Lq - nq .. Lq - 1 of the sequence (aligned to the end of
        # its Lk keys, as in the full call) over their keys
        oracle.ragged_attn(q[:, h:h + 1], k[:, kv:kv + 1], v[:, kv:kv + 1], [0, nq], [0, Lk],
                           sm_scale=cfg["Dqk"] ** -0.5, causal=cfg["causal"])
        heads += 1
        for i in range(Lq - nq, Lq):
            vis = min(Lk, max(0, i + Lk - Lq + 1)) if cfg["causal"] else Lk
            flops += 2 * vis * (cfg["Dqk"] + cfg["Dv"])
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": torch.get_num_threads(),
            "kind": "oracle",
            "sample": f"last {nq} queries of sequence 0 over its {Lk} keys, {heads} of {cfg['H']} heads, fp64"}


def bench_insert(args):
    import paged_kv_attention_pages_amd as pkv
    cfg = INSERT_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    N, Hkv, Dk, Dlo, Dv, ps, Hq = (cfg[k] for k in ("N", "Hkv", "Dk", "Dlo", "Dv", "ps", "Hq"))
    g = torch.Generator(device=dev).manual_seed(1)
    P = 2 * (N + ps - 1) // ps + 1
    shape = (lambda D: (P, ps, Hkv, D)) if cfg["layout"] == "NHD" else (lambda D: (P, Hkv, ps, D))
    kc = torch.zeros(shape(Dk), dtype=cfg["cache"], device=dev)
    vc = torch.zeros(shape(Dv), dtype=cfg["cache"], device=dev) if Dv else None
    k = torch.randn(N, Hkv, Dlo, generator=g, device=dev).to(torch.bfloat16)
    kr = torch.randn(N, Hkv, Dk - Dlo, generator=g, device=dev).to(torch.bfloat16) if Dlo < Dk else None
    v = torch.randn(N, Hkv, Dv, generator=g, device=dev).to(torch.bfloat16) if Dv else None
    slots = torch.randperm(P * ps, generator=torch.Generator().manual_seed(2))[:N].to(dev)
    ql = torch.randn(N, Hq, Dlo, generator=g, device=dev).to(torch.bfloat16) if Hq else None
    qh = torch.randn(N, Hq, Dk - Dlo, generator=g, device=dev).to(torch.bfloat16) if Hq else None
    qo = torch.empty(N, Hq, Dk, dtype=torch.bfloat16, device=dev) if Hq else None
    elem = 1 if cfg["cache"] == torch.float8_e4m3fn else 2
    rows = N * Hkv * (Dk + Dv)
    nbytes = rows * 2 + rows * elem + N * 8 + (N * Hq * Dk * 4 if Hq else 0)
    # sources larger than a few MB rotate through replicas totalling >= 1 GB,
    # so that each call reads them from HBM, not from the last-level cache
    n_rep = min(16, max(1, math.ceil(1.0e9 / (rows * 2)))) if rows * 2 > (8 << 20) else 1
    srcs = [(k, kr, v)] + [(k.clone(), None if kr is None else kr.clone(), None if v is None else v.clone())
                           for _ in range(n_rep - 1)]

    def call(i):
        a, b, c = srcs[i % n_rep]
        pkv.cache_insert(kc, vc, slots, a, k_rope=b, v=c, page_size=ps, kv_layout=cfg["layout"],
                         cache_scale_inv=20.0 if elem == 1 else 1.0, q_lo=ql, q_hi=qh, q_out=qo)

    K, W = args.steps, args.warmup
    for i in range(W):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        call(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for i, (a, b) in enumerate(ev):
        a.record()
        call(i)
        b.record()
    torch.cuda.synchronize()
    kern_ms = statistics.fmean(a.elapsed_time(b) for a, b in ev)
    value = nbytes / (ms * 1e-3) / 1e9
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    print(f"[bench] {args.workload}: {ms * 1e3:.2f} us/call wall, evented {kern_ms * 1e3:.2f} us, "
          f"{value:.0f} GB/s", file=sys.stderr, flush=True)
    rec = {
        "metric": "paged-cache insert GB/s (bytes read + written) + us/call",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" + ("->fp8" if elem == 1 else ""), "data": "synthetic",
        "us_per_call": round(ms * 1e3, 2),
        "config": {"workload": args.workload, "num_tokens": N, "num_kv_heads": Hkv,
                   "head_dim_k": Dk, "head_dim_k_lo": Dlo, "head_dim_v": Dv, "page_size": ps,
                   "kv_layout": cfg["layout"], "cache_dtype": str(cfg["cache"]).replace("torch.", ""),
                   "query_concat_heads": Hq, "bytes_per_call": nbytes, "source_replicas": n_rep},
        "roofline": {"kernel": "cache insert", "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes": nbytes,
                     "launch_us_mean": round(kern_ms * 1e3, 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def _p10_p90(xs):
    ys = sorted(xs)
    pick = lambda f: ys[min(len(ys) - 1, max(0, int(round(f * (len(ys) - 1)))))]
    return pick(0.1), pick(0.9)


def cpu_baseline(w, inp, L, budget_s):
    """The oracle (as is) on the first n sequences of the batch, n sized to the budget."""
    import oracle
    from paged_kv_attention_pages_amd import synth

    cores = len(os.sched_getaffinity(0))
    k_host = inp["k_cache"].cpu()
    v_host = None if w.v_from_k else inp["v_cache"].cpu()
    kw = dict(head_dim_v=w.head_dim_v, v_from_k=w.v_from_k, num_threads=cores,
              **synth.decode_kwargs(w))
    sel = lambda t, n: None if t is None else t[:n].cpu()

    def run(n, threads):
        t = time.perf_counter()
        oracle.decode(sel(inp["q"], n), k_host, v_host, sel(inp["page_table"], n),
                      sel(inp["seq_lens"], n), sinks=None if inp["sinks"] is None else inp["sinks"].cpu(),
                      mask=sel(inp["mask"], n), **dict(kw, num_threads=threads))
        return time.perf_counter() - t

    t1 = run(1, cores)
    n = int(max(1, min(L.numel(), budget_s / max(t1, 1e-3))))
    dt = run(n, cores) if n > 1 else t1
    sample_bytes = kv_bytes_of(w, L[:n])
    print(f"[bench] oracle: {n} sequences in {dt:.2f} s on {cores} threads", file=sys.stderr,
          flush=True)
    rec = {"value": round(sample_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
           "kind": "oracle", "ms_per_sequence": round(dt * 1e3 / n, 2),
           "sample": f"first {n} of {L.numel()} sequences of the same batch (all heads), fp64"}
    if w.name in ("tiny", "llama3_8b_gqa"):
        # the same oracle on one thread, on a sample a third of the budget allows
        t1s = run(1, 1)
        n1 = int(max(1, min(L.numel(), budget_s / 3 / max(t1s, 1e-3))))
        dt1 = run(n1, 1) if n1 > 1 else t1s
        rec["one_thread"] = {"value": round(kv_bytes_of(w, L[:n1]) / dt1 / 1e9, 4), "unit": "GB/s",
                             "ms_per_sequence": round(dt1 * 1e3 / n1, 2),
                             "sample": f"first {n1} sequences"}
        print(f"[bench] oracle: {n1} sequences in {dt1:.2f} s on 1 thread", file=sys.stderr,
              flush=True)
    return rec


if __name__ == "__main__":
    main()
