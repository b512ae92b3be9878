"""fp64 CPU oracle for paged-KV decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The library's decode path never does; the two
share no code (this wrapper loads ``pkv_oracle.c`` compiled by gcc, with
``-O2 -fopenmp`` and no fast-math).

The definition it follows, and the readings taken where the pages leave a
step open, are stated in the header of ``pkv_oracle.c``.  Every function
here is pinned by ``tests/test_oracle_pins.py`` against things other than
itself: the format definitions' own values, library conversions, a dense
brute-force attention on gathered pages, closed forms and invariants.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB = os.path.join(_HERE, "libpkv_oracle.so")
_lock = threading.Lock()
_lib = None

DTYPE_CODE = {torch.float16: 0, torch.bfloat16: 1, torch.float8_e4m3fn: 2, torch.uint8: 2}
LAYOUT_CODE = {"NHD": 0, "HND": 1}


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int), ("q_seq_len", ctypes.c_int),
        ("num_q_heads", ctypes.c_int), ("num_kv_heads", ctypes.c_int),
        ("head_dim_qk", ctypes.c_int), ("head_dim_v", ctypes.c_int),
        ("page_size", ctypes.c_int), ("pages_per_seq", ctypes.c_int),
        ("num_pages", ctypes.c_int), ("q_dtype", ctypes.c_int),
        ("kv_dtype", ctypes.c_int), ("layout", ctypes.c_int),
        ("window", ctypes.c_int), ("v_from_k", ctypes.c_int),
        ("num_threads", ctypes.c_int),
        ("q_scale", ctypes.c_double), ("kv_scale", ctypes.c_double),
    ]


class _Insert(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int), ("num_kv_heads", ctypes.c_int),
        ("head_dim_k", ctypes.c_int), ("head_dim_k_lo", ctypes.c_int),
        ("head_dim_v", ctypes.c_int), ("page_size", ctypes.c_int),
        ("num_pages", ctypes.c_int), ("layout", ctypes.c_int),
        ("src_dtype", ctypes.c_int), ("cache_dtype", ctypes.c_int),
        ("cache_scale_inv", ctypes.c_float),
    ]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, fp64, OpenMP, no fast-math)."""
    with _lock:
        if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            tmp = _LIB + f".tmp{os.getpid()}"
            subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                            "-Wall", _SRC, "-o", tmp, "-lm"], check=True)
            os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        for name in ("pkvo_decode_f16", "pkvo_decode_bf16"):
            getattr(lib, name).restype = ctypes.c_double
            getattr(lib, name).argtypes = [ctypes.c_uint16]
        lib.pkvo_decode_e4m3fn.restype = ctypes.c_double
        lib.pkvo_decode_e4m3fn.argtypes = [ctypes.c_uint8]
        lib.pkvo_decode.restype = ctypes.c_int
        lib.pkvo_decode.argtypes = [ctypes.POINTER(_Problem)] + [ctypes.c_void_p] * 8
        lib.pkvo_max_threads.restype = ctypes.c_int
        lib.pkvo_encode_e4m3fn.restype = ctypes.c_uint8
        lib.pkvo_encode_e4m3fn.argtypes = [ctypes.c_float]
        lib.pkvo_cache_insert.restype = ctypes.c_int
        lib.pkvo_cache_insert.argtypes = [ctypes.POINTER(_Insert)] + [ctypes.c_void_p] * 6
        _lib = lib
    return _lib


def decode_f16(bits: int) -> float:
    return _load().pkvo_decode_f16(bits)


def decode_bf16(bits: int) -> float:
    return _load().pkvo_decode_bf16(bits)


def decode_e4m3fn(bits: int) -> float:
    return _load().pkvo_decode_e4m3fn(bits)


def max_threads() -> int:
    return _load().pkvo_max_threads()


def _raw(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor's storage bits (no value conversion)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy()
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return t.view(torch.uint8).numpy()
    return t.numpy()


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode(q, k_cache, v_cache, page_table, seq_lens, *, num_kv_heads, page_size,
           kv_layout="NHD", sinks=None, q_scale=1.0, kv_scale=1.0, sliding_win_size=0,
           q_seq_len=1, mask=None, head_dim_v=None, v_from_k=False, num_pages=None,
           num_threads=0):
    """Exact attention in fp64.  q: [B, q_seq_len, Hq, Dqk] (or [B, Hq, Dqk]).

    Returns a float64 tensor [B, q_seq_len, Hq, Dv].  ``v_from_k`` takes V as
    the first ``head_dim_v`` entries of each K row (the latent cache).
    """
    B = q.shape[0]
    Hq, Dqk = q.shape[-2], q.shape[-1]
    Tq = q_seq_len
    assert q.numel() == B * Tq * Hq * Dqk, "q does not hold batch*q_seq_len*Hq*Dqk elements"
    if head_dim_v is None:
        head_dim_v = Dqk if (v_from_k or v_cache is None) else v_cache.shape[-1]
    p = _Problem()
    p.batch, p.q_seq_len, p.num_q_heads, p.num_kv_heads = B, Tq, Hq, num_kv_heads
    p.head_dim_qk, p.head_dim_v = Dqk, head_dim_v
    p.page_size, p.pages_per_seq = page_size, page_table.shape[-1]
    p.num_pages = k_cache.shape[0] if num_pages is None else num_pages
    p.q_dtype, p.kv_dtype = DTYPE_CODE[q.dtype], DTYPE_CODE[k_cache.dtype]
    p.layout = LAYOUT_CODE[kv_layout]
    p.window, p.v_from_k, p.num_threads = sliding_win_size, 1 if v_from_k else 0, num_threads
    p.q_scale, p.kv_scale = float(q_scale), float(kv_scale)

    qa = _raw(q)
    ka = _raw(k_cache)
    va = None if (v_from_k or v_cache is None) else _raw(v_cache)
    pt = np.ascontiguousarray(page_table.detach().cpu().to(torch.int32).numpy())
    sl = np.ascontiguousarray(seq_lens.detach().cpu().reshape(-1).to(torch.int64).numpy().astype(np.uint32))
    sk = None if sinks is None else np.ascontiguousarray(sinks.detach().cpu().to(torch.float32).numpy())
    mk = None
    if mask is not None:
        mk = np.ascontiguousarray(mask.detach().cpu().view(torch.int16).numpy())
    out = np.zeros((B, Tq, Hq, head_dim_v), dtype=np.float64)
    rc = _load().pkvo_decode(ctypes.byref(p), _ptr(qa), _ptr(ka), _ptr(va), _ptr(pt), _ptr(sl),
                             _ptr(sk), _ptr(mk), _ptr(out))
    if rc < 0:
        raise ValueError("oracle: malformed problem sizes")
    if rc > 0:
        raise ValueError(f"oracle: sequence {rc - 1} needs a page id outside [0, num_pages)")
    return torch.from_numpy(out)


def encode_e4m3fn(x: float) -> int:
    """E4M3 code of the binary32 value nearest to x (ties to even, saturating at 448)."""
    return _load().pkvo_encode_e4m3fn(x)


def cache_insert(k_cache, v_cache, slot_mapping, k, k_rope=None, v=None, *, page_size,
                 kv_layout="NHD", cache_scale_inv=1.0):
    """The write side: new tokens' rows into copies of the caches at slot_mapping.

    k [N, Hkv, Dlo] (16-bit), k_rope [N, Hkv, Dk - Dlo] or None, v [N, Hkv, Dv] or
    None (latent cache), slot_mapping [N] int64.  Returns host copies of the
    updated (k_cache, v_cache) with the input caches' dtypes.
    """
    N = slot_mapping.shape[0]
    Hkv = k.shape[-2]
    Dlo = k.shape[-1]
    Dk = k_cache.shape[-1]
    Dv = 0 if v is None else v.shape[-1]
    p = _Insert()
    p.num_tokens, p.num_kv_heads, p.head_dim_k, p.head_dim_k_lo, p.head_dim_v = N, Hkv, Dk, Dlo, Dv
    p.page_size, p.num_pages, p.layout = page_size, k_cache.shape[0], LAYOUT_CODE[kv_layout]
    p.src_dtype, p.cache_dtype = DTYPE_CODE[k.dtype], DTYPE_CODE[k_cache.dtype]
    p.cache_scale_inv = float(cache_scale_inv)
    kc = k_cache.detach().to("cpu").clone()
    vc = None if v_cache is None else v_cache.detach().to("cpu").clone()
    ka, ra, va = _raw(k), None if k_rope is None else _raw(k_rope), None if v is None else _raw(v)
    sm = np.ascontiguousarray(slot_mapping.detach().cpu().to(torch.int64).numpy())
    kc_raw = kc.view(torch.int16 if kc.element_size() == 2 else torch.uint8).numpy()
    vc_raw = None if vc is None else vc.view(torch.int16 if vc.element_size() == 2 else torch.uint8).numpy()
    rc = _load().pkvo_cache_insert(ctypes.byref(p), _ptr(ka), _ptr(ra), _ptr(va), _ptr(sm),
                                   _ptr(kc_raw), _ptr(vc_raw))
    if rc < 0:
        raise ValueError("oracle: malformed insert sizes")
    return kc, vc


def head_matmul(x, w):
    """y[m, h] = x[m, h] . w[h] in fp64 (torch's matmul on the decoded values).

    The per-head products of the vLLM Kimi-K3 MLA page around its latent
    decode: BMM1 with W_UK_T and `_v_up_proj` with W_UV.
    """
    xd = x.detach().to("cpu", torch.float64)
    wd = w.detach().to("cpu", torch.float64)
    return torch.matmul(xd.transpose(0, 1), wd).transpose(0, 1).contiguous()


def mla_materialised(q_nope, q_pe, kv_cache, page_table, seq_lens, w_uk_t, w_uv, *, page_size,
                     kv_lora_rank=512, softmax_scale):
    """Multi-head attention with the keys and values materialised from the latent
    cache, in fp64 -- the form the absorbed decode must equal (vLLM Kimi-K3 MLA
    page: K_nope = kv_c . W_UK, K = [K_nope | k_pe], V = kv_c . W_UV).

    q_nope [B, H, P], q_pe [B, H, R], kv_cache [pages, page_size, 1, kv_lora_rank + R]
    (rows [kv_c | k_pe]), w_uk_t [H, P, L], w_uv [H, L, V].  Returns [B, H, V].
    """
    B, H, _ = q_nope.shape
    L = kv_lora_rank
    cache = kv_cache.detach().to("cpu", torch.float64).reshape(-1, kv_cache.shape[-1])
    wuk = w_uk_t.detach().to("cpu", torch.float64)          # [H, P, L]
    wuv = w_uv.detach().to("cpu", torch.float64)            # [H, L, V]
    qn = q_nope.detach().to("cpu", torch.float64)
    qp = q_pe.detach().to("cpu", torch.float64)
    out = torch.zeros(B, H, wuv.shape[-1], dtype=torch.float64)
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        t = torch.arange(n)
        rows = cache[page_table[b].to(torch.int64)[t // page_size] * page_size + t % page_size]
        kv_c, k_pe = rows[:, :L], rows[:, L:]
        for h in range(H):
            k_nope = kv_c @ wuk[h].T                        # [n, P]
            v = kv_c @ wuv[h]                               # [n, V]
            logits = softmax_scale * (k_nope @ qn[b, h] + k_pe @ qp[b, h])
            out[b, h] = torch.softmax(logits, dim=0) @ v
    return out


def merge_attn_states(prefix_out, prefix_lse, suffix_out, suffix_lse, num_tokens_with_prefix=None):
    """fp64 merge of two attention results by their natural-log log-sum-exps.

    vLLM Kimi-K3 MLA page, chunked prefill `merge_attn_states`: with
    M = max(lp, ls) and w = e^(lse - M), out = (o_p w_p + o_s w_s) / (w_p + w_s)
    and lse = M + log(w_p + w_s); tokens at or past num_tokens_with_prefix
    take the suffix alone; both -inf give zeros and -inf.  Outputs [N, H, D],
    log-sum-exps [H, N].  Returns (out fp64 [N, H, D], lse fp64 [H, N]).
    """
    so = suffix_out.detach().to("cpu", torch.float64)
    sl = suffix_lse.detach().to("cpu", torch.float64)
    N, H, D = so.shape
    n_pre = N if num_tokens_with_prefix is None else int(num_tokens_with_prefix)
    po = torch.zeros_like(so)
    pl = torch.full_like(sl, float("-inf"))
    if n_pre > 0:
        po[:n_pre] = prefix_out.detach().to("cpu", torch.float64)[:n_pre]
        pl[:, :n_pre] = prefix_lse.detach().to("cpu", torch.float64)[:, :n_pre]
    out = torch.zeros_like(so)
    lse = torch.full_like(sl, float("-inf"))
    for n in range(N):
        for h in range(H):
            lp, ls = float(pl[h, n]), float(sl[h, n])
            M = max(lp, ls)
            if M == float("-inf"):
                continue
            wp = 0.0 if lp == float("-inf") else math.exp(lp - M)
            ws = 0.0 if ls == float("-inf") else math.exp(ls - M)
            acc = torch.zeros(D, dtype=torch.float64)
            if wp:
                acc += po[n, h] * wp
            if ws:
                acc += so[n, h] * ws
            out[n, h] = acc / (wp + ws)
            lse[h, n] = M + math.log(wp + ws)
    return out, lse


def ragged_attn(q, k, v, cu_seqlens_q, cu_seqlens_k, *, sm_scale, causal):
    """fp64 attention over a ragged (non-paged) batch, with its log-sum-exp.

    FlashInfer `trtllm_ragged_attention_deepseek` call of the vllm-omni TRTLLM
    backend (`cum_seq_lens_q` / `cum_seq_lens_kv`, `is_causal`, `bmm1_scale`
    as the softmax scale), and the vLLM Kimi-K3 MLA page's chunked prefill,
    whose `run_prefill_new_tokens` and `_compute_prefill_context` return the
    (output, lse) pairs that `merge_attn_states` combines.

    Sequence s owns query rows [cu_q[s], cu_q[s+1]) and key/value rows
    [cu_k[s], cu_k[s+1]).  Query head h reads KV head h // (Hq / Hkv).  With
    Lq, Lk the two lengths, query i (0-based in its sequence) sees key j iff
    j < Lk and, when causal, j <= i + Lk - Lq (the queries are the last Lq
    positions of the key sequence).  logit = sm_scale * q . k; out = softmax
    weighted mean of the visible V rows; lse = natural log of the sum of
    e^logit.  A row that sees nothing gets zeros and lse = -inf.

    q [Nq, Hq, Dqk], k [Nk, Hkv, Dqk], v [Nk, Hkv, Dv].  Returns
    (out fp64 [Nq, Hq, Dv], lse fp64 [Hq, Nq]).
    """
    qd = q.detach().to("cpu", torch.float64)
    kd = k.detach().to("cpu", torch.float64)
    vd = v.detach().to("cpu", torch.float64)
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    Nq, Hq, _ = qd.shape
    Hkv, Dv = kd.shape[1], vd.shape[2]
    G = Hq // Hkv
    out = torch.zeros(Nq, Hq, Dv, dtype=torch.float64)
    lse = torch.full((Hq, Nq), float("-inf"), dtype=torch.float64)
    for s in range(len(cq) - 1):
        Lq, Lk = cq[s + 1] - cq[s], ck[s + 1] - ck[s]
        for h in range(Hq):
            kh = kd[ck[s]:ck[s + 1], h // G]              # [Lk, Dqk]
            vh = vd[ck[s]:ck[s + 1], h // G]              # [Lk, Dv]
            for i in range(Lq):
                n = Lk if not causal else max(0, min(Lk, i + Lk - Lq + 1))
                if n == 0:
                    continue
                logits = sm_scale * (kh[:n] @ qd[cq[s] + i, h])
                m = float(logits.max())
                e = torch.exp(logits - m)
                den = float(e.sum())
                out[cq[s] + i, h] = (e @ vh[:n]) / den
                lse[h, cq[s] + i] = m + math.log(den)
    return out, lse
