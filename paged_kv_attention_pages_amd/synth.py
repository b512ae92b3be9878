"""Seeded synthetic inputs for paged-KV decode attention.

This module builds inputs only -- sequence lengths, page assignments, cache
contents, queries, sinks and masks -- and holds none of the attention
arithmetic.  Tests, the benchmark and the smoke check take their inputs
from here, so the HIP path and the oracle always see the same bytes.

The five workloads are the synthetic configurations the library is measured
and checked on: a tiny fp16 case, a Llama-3-8B-shaped GQA decode, an fp8 cache
with a sliding window and sinks, a speculative decode with a bit-packed
causal mask, and the absorbed-MLA latent decode of one GPU's head share.
Values are N(0, 1) (fp8 caches hold e4m3fn(N(0, 1) / kv_scale)); physical
pages are handed out through a seeded random permutation; every page-table
entry a sequence does not need points at a NaN-filled poison page, and slots
past a sequence's end are NaN too, so any stray read shows up in the output.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    q_dtype: torch.dtype
    kv_dtype: torch.dtype
    kv_layout: str
    page_size: int
    seq_len_range: tuple = None      # inclusive (lo, hi), drawn uniformly
    fixed_seq_lens: tuple = None     # explicit lengths instead of a range
    num_pages: int = None            # physical pages (default: needed + 1)
    q_seq_len: int = 1
    window: int = 0
    sinks: bool = False
    q_scale: float = 1.0
    kv_scale: float = 1.0
    kv_gen_scale: float = 1.0        # cache values = N(0,1) * this, then cast
    mask: str = None                 # None | "causal" | "random" | "ones"
    v_from_k: bool = False           # latent cache: V = leading Dv of K row

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


WORKLOADS = {
    "tiny": Workload(
        name="tiny", batch=2, num_q_heads=4, num_kv_heads=1, head_dim_qk=128,
        head_dim_v=128, q_dtype=torch.float16, kv_dtype=torch.float16, kv_layout="NHD",
        page_size=16, fixed_seq_lens=(37, 100), num_pages=16),
    "llama3_8b_gqa": Workload(
        name="llama3_8b_gqa", batch=64, num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
        head_dim_v=128, q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, kv_layout="HND",
        page_size=64, seq_len_range=(1024, 8192)),
    "fp8_window_sinks": Workload(
        name="fp8_window_sinks", batch=128, num_q_heads=64, num_kv_heads=8,
        head_dim_qk=128, head_dim_v=128, q_dtype=torch.bfloat16,
        kv_dtype=torch.float8_e4m3fn, kv_layout="NHD", page_size=32,
        seq_len_range=(4096, 32768), window=4096, sinks=True, q_scale=1.0,
        kv_scale=0.05, kv_gen_scale=1.0 / 0.05),
    "spec_decode": Workload(
        name="spec_decode", batch=32, num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
        head_dim_v=128, q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, kv_layout="NHD",
        page_size=64, seq_len_range=(2048, 16384), q_seq_len=4, mask="causal"),
    # softmax scale 192^-0.5 (qk_nope 128 + rope 64) over 576-wide rows:
    # q_scale = sqrt(576 / 192) turns the library's 1/sqrt(576) into it.
    "mla": Workload(
        name="mla", batch=32, num_q_heads=64, num_kv_heads=1, head_dim_qk=576,
        head_dim_v=512, q_dtype=torch.bfloat16, kv_dtype=torch.bfloat16, kv_layout="NHD",
        page_size=64, seq_len_range=(4096, 16384), q_scale=math.sqrt(576.0 / 192.0),
        v_from_k=True),
    # the latent path's fp8 form: e4m3fn cache (kv_scale 0.05) and e4m3fn query
    "mla_fp8": Workload(
        name="mla_fp8", batch=32, num_q_heads=64, num_kv_heads=1, head_dim_qk=576,
        head_dim_v=512, q_dtype=torch.float8_e4m3fn, kv_dtype=torch.float8_e4m3fn,
        kv_layout="NHD", page_size=64, seq_len_range=(4096, 16384),
        q_scale=math.sqrt(576.0 / 192.0), kv_scale=0.05, kv_gen_scale=1.0 / 0.05, v_from_k=True),
}

# the order the workloads are listed in the specification of the benchmark
WORKLOAD_ORDER = ["tiny", "llama3_8b_gqa", "fp8_window_sinks", "spec_decode", "mla"]

NAN_BITS = {torch.float16: 0x7E00, torch.bfloat16: 0x7FC0, torch.float8_e4m3fn: 0x7F}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def draw_seq_lens(w: Workload, seed: int) -> torch.Tensor:
    """Sequence lengths (int64, CPU): the fixed list or uniform integers."""
    if w.fixed_seq_lens is not None:
        return torch.tensor(w.fixed_seq_lens, dtype=torch.int64)
    lo, hi = w.seq_len_range
    return torch.randint(lo, hi + 1, (w.batch,), generator=_gen(seed * 1000 + 1, "cpu"))


def pack_mask_bits(visible: torch.Tensor) -> torch.Tensor:
    """Pack a boolean [B, Tq, Tq] draft-visibility matrix into uint16 words.

    Row (b, i) becomes ceil(Tq/32) little-endian 32-bit words stored as
    uint16 pairs (low half first); draft j is bit j % 32 of word j // 32.
    """
    B, Tq, _ = visible.shape
    nw = (Tq + 31) // 32
    words = np.zeros((B, Tq, nw * 2), dtype=np.uint16)
    v = visible.cpu().numpy().astype(bool)
    for j in range(Tq):
        w32, bit = divmod(j, 32)
        half, hb = divmod(bit, 16)
        words[:, :, 2 * w32 + half] |= (v[:, :, j].astype(np.uint16) << np.uint16(hb))
    return torch.from_numpy(words)


def draft_visibility(kind: str, batch: int, q_seq_len: int, seed: int) -> torch.Tensor:
    """Boolean [B, Tq, Tq]: causal (j <= i), all ones, or seeded random."""
    if kind == "causal":
        m = torch.tril(torch.ones(q_seq_len, q_seq_len, dtype=torch.bool))
        return m.expand(batch, q_seq_len, q_seq_len).clone()
    if kind == "ones":
        return torch.ones(batch, q_seq_len, q_seq_len, dtype=torch.bool)
    if kind == "random":
        g = _gen(seed * 1000 + 7, "cpu")
        return torch.rand(batch, q_seq_len, q_seq_len, generator=g) < 0.5
    raise ValueError(f"unknown mask kind {kind!r}")


def _fill_values(dst: torch.Tensor, w: Workload, g: torch.Generator, chunk: int = 1 << 26):
    """Fill a cache tensor with N(0,1) * kv_gen_scale cast to its dtype, in chunks."""
    flat = dst.view(-1)
    for s in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - s)
        x = torch.randn(n, generator=g, device=dst.device, dtype=torch.float32)
        if w.kv_gen_scale != 1.0:
            x.mul_(w.kv_gen_scale)
        flat[s:s + n] = x.to(dst.dtype)


def _nan_of(dtype, device):
    return torch.tensor(NAN_BITS[dtype], dtype=torch.int32).to(
        torch.uint8 if dtype == torch.float8_e4m3fn else torch.int16).view(dtype).to(device)


def make_inputs(w: Workload, seed: int, device="cpu", *, seq_lens=None, keep_from=None,
                poison=True):
    """Build one batch of inputs for workload ``w``.

    seq_lens: optional explicit lengths (overrides the workload's draw).
    keep_from: optional per-sequence first token to keep; earlier tokens of
        the sequence are overwritten with NaN (callers pass the start of the
        visible range when a window hides the beginning of a sequence).
    Returns a dict of tensors on ``device`` plus the host copies of the
    lengths and page table and the poison page id.
    """
    dev = torch.device(device)
    L = draw_seq_lens(w, seed) if seq_lens is None else torch.as_tensor(seq_lens, dtype=torch.int64)
    B = L.numel()
    ps = w.page_size
    need = [(int(x) + ps - 1) // ps for x in L]
    total = sum(need)
    num_pages = w.num_pages if w.num_pages is not None else total + 1
    if num_pages < total + 1:
        raise ValueError(f"{num_pages} physical pages cannot hold {total} pages plus a poison page")
    # table width = the longest length the workload allows (max_seq_len)
    cap = w.seq_len_range[1] if (seq_lens is None and w.seq_len_range) else int(L.max()) if B else 0
    pps = max((cap + ps - 1) // ps, max(need) if need else 0, 1)
    perm = torch.randperm(num_pages, generator=_gen(seed * 1000 + 2, "cpu"))
    poison_page = int(perm[total])
    table = torch.full((B, pps), poison_page, dtype=torch.int32)
    off = 0
    for b in range(B):
        table[b, :need[b]] = perm[off:off + need[b]].to(torch.int32)
        off += need[b]

    Hkv, Dk, Dv = w.num_kv_heads, w.head_dim_qk, w.head_dim_v
    if w.kv_layout == "NHD":
        kshape, vshape = (num_pages, ps, Hkv, Dk), (num_pages, ps, Hkv, Dv)
    else:
        kshape, vshape = (num_pages, Hkv, ps, Dk), (num_pages, Hkv, ps, Dv)
    gdev = _gen(seed * 1000 + 3, dev)
    k_cache = torch.empty(kshape, dtype=w.kv_dtype, device=dev)
    _fill_values(k_cache, w, gdev)
    if w.v_from_k:
        v_cache = k_cache
    else:
        v_cache = torch.empty(vshape, dtype=w.kv_dtype, device=dev)
        _fill_values(v_cache, w, gdev)

    q = torch.randn((B, w.q_seq_len, w.num_q_heads, Dk), generator=gdev, device=dev,
                    dtype=torch.float32).to(w.q_dtype)
    sinks = None
    if w.sinks:
        sinks = torch.randn((Hkv, w.group), generator=_gen(seed * 1000 + 4, "cpu"),
                            dtype=torch.float32).to(dev)
    mask = None
    if w.mask is not None and w.q_seq_len > 1:
        mask = pack_mask_bits(draft_visibility(w.mask, B, w.q_seq_len, seed)).to(dev)

    if poison:
        nan = _nan_of(w.kv_dtype, dev)
        caches = [k_cache] if w.v_from_k else [k_cache, v_cache]
        used = torch.zeros(num_pages, dtype=torch.bool)
        used[perm[:total]] = True
        whole = [int(x) for x in torch.nonzero(~used).flatten()]   # unused pages
        partial = []                                               # (page, first, end) slots
        kf = None if keep_from is None else torch.as_tensor(keep_from, dtype=torch.int64)
        for b in range(B):
            Lb = int(L[b])
            if Lb % ps:
                partial.append((int(table[b, need[b] - 1]), Lb % ps, ps))
            if kf is not None and int(kf[b]) > 0:
                first = min(int(kf[b]), Lb)
                whole.extend(int(x) for x in table[b, :first // ps])
                if first % ps:
                    partial.append((int(table[b, first // ps]), 0, first % ps))
        for c in caches:
            if whole:
                c[torch.tensor(whole, device=dev)] = nan
            for page, s0, s1 in partial:
                _poison_slots(c, w.kv_layout, page, s0, s1, nan)

    return {
        "q": q, "k_cache": k_cache, "v_cache": v_cache,
        # uint32 on the xqa page; int32 holds the same bits for these lengths
        "page_table": table.to(dev), "seq_lens": L.to(torch.int32).to(dev),
        "sinks": sinks, "mask": mask,
        "seq_lens_host": L.clone(), "page_table_host": table.clone(),
        "num_pages": num_pages, "poison_page": poison_page,
    }


def _poison_slots(cache, layout, page, s0, s1, nan):
    if layout == "NHD":
        cache[page, s0:s1] = nan
    else:
        cache[page, :, s0:s1] = nan


def decode_kwargs(w: Workload) -> dict:
    """The scalar decode arguments of a workload, by the xqa page's names."""
    return dict(num_kv_heads=w.num_kv_heads, page_size=w.page_size, kv_layout=w.kv_layout,
                q_scale=w.q_scale, kv_scale=w.kv_scale, sliding_win_size=w.window,
                q_seq_len=w.q_seq_len)


def make_ragged(lens_q, lens_k, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, dtype,
                seed, device="cpu"):
    """Inputs of a ragged (non-paged) attention: q [sum lens_q, Hq, Dqk] and
    k, v [sum lens_k, Hkv, D] ~ N(0, 1) in ``dtype``, and the int32 prefix sums
    cu_seqlens_q / cu_seqlens_k [num_seqs + 1] (host copies in *_host)."""
    dev = torch.device(device)
    cq = [0] + [int(x) for x in np.cumsum(lens_q)] if len(lens_q) else [0]
    ck = [0] + [int(x) for x in np.cumsum(lens_k)] if len(lens_k) else [0]
    g = _gen(seed * 1000 + 7, dev)
    q = torch.randn((cq[-1], num_q_heads, head_dim_qk), generator=g, device=dev).to(dtype)
    k = torch.randn((ck[-1], num_kv_heads, head_dim_qk), generator=g, device=dev).to(dtype)
    v = torch.randn((ck[-1], num_kv_heads, head_dim_v), generator=g, device=dev).to(dtype)
    return {"q": q, "k": k, "v": v,
            "cu_seqlens_q": torch.tensor(cq, dtype=torch.int32, device=dev),
            "cu_seqlens_k": torch.tensor(ck, dtype=torch.int32, device=dev),
            "cu_seqlens_q_host": cq, "cu_seqlens_k_host": ck,
            "max_q_len": max([int(x) for x in lens_q], default=0)}
