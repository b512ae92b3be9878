"""Paged-KV decode attention for MI355X (gfx950): Python binding of libpkv.so.

A thin ctypes layer over the C ABI declared in ``include/pkv.h``: it reads
shapes, dtypes, device pointers and the current HIP stream from torch tensors
and passes them through.  Every step of the attention runs in the library's
HIP kernels; there is no Python or CPU fallback, and calling into a missing
library raises.

``decode_attn`` mirrors the parameters of FlashInfer's ``flashinfer.xqa.xqa``
(reference page: q, k_cache, v_cache, page_table, seq_lens, output,
workspace_buffer, num_kv_heads, page_size, sinks, q_scale, kv_scale,
sliding_win_size, kv_layout, q_seq_len, mask).  The workspace, when not
given, is cached per (device, stream) and grown on demand, as the vllm-omni
trtllm_attn backend page does with its attention workspace (``_get_workspace``);
calls on different streams never share one.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = ["ragged_attn", "decode_attn", "workspace_size", "query_plan", "validate_inputs", "library_path",
           "PATH_AUTO", "PATH_VALU", "PATH_MFMA", "PATH_MFMA_MLA", "PkvError"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpkv.so")

PATH_AUTO, PATH_VALU, PATH_MFMA, PATH_MFMA_MLA = 0, 1, 2, 3
PATH_NAMES = {PATH_VALU: "valu", PATH_MFMA: "mfma", PATH_MFMA_MLA: "mfma_mla"}
_STATUS = {0: "PKV_OK", 1: "PKV_ERR_INVALID_ARGUMENT", 2: "PKV_ERR_UNSUPPORTED",
           3: "PKV_ERR_WORKSPACE_TOO_SMALL", 4: "PKV_ERR_HIP", 5: "PKV_ERR_DEVICE_DATA"}
_DTYPE = {torch.float16: 0, torch.bfloat16: 1, torch.float8_e4m3fn: 2, torch.uint8: 2}
_LAYOUT = {"NHD": 0, "HND": 1}


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64)]


PKV_ERR_WORKSPACE_TOO_SMALL = 3

# bytes of the static per-GPU scratch of pkv_decode_attn_noalloc
NOALLOC_SCRATCH_BYTES = 96 << 20


class Options(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("split_pages", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("target_ctas", ctypes.c_int32),
                ("split_event", ctypes.c_void_p), ("q_scale_dev", ctypes.c_void_p),
                ("kv_scale_dev", ctypes.c_void_p), ("merge_mode", ctypes.c_int32),
                ("out_fp8", ctypes.c_int32), ("rcp_out_scale", ctypes.c_float)]


class InsertDims(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim_k", ctypes.c_int32), ("head_dim_k_lo", ctypes.c_int32),
                ("head_dim_v", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("src_dtype", ctypes.c_int32), ("cache_dtype", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("split_pages", ctypes.c_int32),
                ("max_splits", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("ctas_per_split_grid", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64), ("single_launch", ctypes.c_int32),
                ("waves_per_workgroup", ctypes.c_int32)]


_lib = None
_lib_lock = threading.Lock()
_vp = ctypes.c_void_p


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libpkv.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lib_lock:
            if _lib is None:
                if not os.path.exists(_LIB_PATH):
                    raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                                       "`python -m paged_kv_attention_pages_amd.build`")
                L = ctypes.CDLL(_LIB_PATH)
                L.pkv_abi_version.restype = ctypes.c_int
                L.pkv_last_error.restype = ctypes.c_char_p
                L.pkv_query_plan.restype = ctypes.c_int
                L.pkv_query_plan.argtypes = [ctypes.POINTER(Dims), ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.POINTER(Options),
                                             ctypes.POINTER(PlanInfo)]
                L.pkv_workspace_size.restype = ctypes.c_size_t
                L.pkv_workspace_size.argtypes = [ctypes.POINTER(Dims), ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_int]
                dec = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                       _vp, ctypes.c_float, ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp, _vp,
                       ctypes.POINTER(Dims)]
                L.pkv_decode_attn.restype = ctypes.c_int
                L.pkv_decode_attn.argtypes = dec
                L.pkv_decode_attn_ex.restype = ctypes.c_int
                L.pkv_decode_attn_ex.argtypes = dec + [ctypes.POINTER(Options)]
                L.pkv_decode_attn_noalloc.restype = ctypes.c_int
                L.pkv_decode_attn_noalloc.argtypes = dec[:6] + dec[7:] + [ctypes.POINTER(Options)]
                L.pkv_validate_inputs.restype = ctypes.c_int
                L.pkv_validate_inputs.argtypes = [_vp, _vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_int, _vp, ctypes.POINTER(Dims)]
                L.pkv_head_matmul.restype = ctypes.c_int
                L.pkv_head_matmul.argtypes = [_vp, ctypes.c_int64, ctypes.c_int64, _vp, _vp,
                                              ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, _vp]
                L.pkv_merge_attn_states.restype = ctypes.c_int
                i64 = ctypes.c_int64
                L.pkv_merge_attn_states.argtypes = [_vp, _vp, i64, i64, _vp, _vp, i64, i64, _vp,
                                                    _vp, i64, i64, ctypes.c_int, ctypes.c_int,
                                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp]
                ci = ctypes.c_int
                L.pkv_ragged_attn.restype = ctypes.c_int
                L.pkv_ragged_attn.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, i64, i64, ci, ci,
                                              ci, ci, ci, ci, ci, ci, ctypes.c_float, ci, ci, _vp]
                L.pkv_cache_insert.restype = ctypes.c_int
                L.pkv_cache_insert.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp,
                                               _vp, _vp, _vp, _vp, ctypes.POINTER(InsertDims)]
                _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise PkvError(status, lib().pkv_last_error().decode())


def _ptr(t):
    # a plain int: ctypes converts it for c_void_p arguments
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _current_stream(dev: int) -> int:
    """Handle of torch's current stream on device index `dev`."""
    if _raw_stream is not None:
        return _raw_stream(dev)
    return torch.cuda.current_stream(dev).cuda_stream


_get_device = getattr(torch._C, "_cuda_getDevice", None)


def _call_on(dev: int, fn, *args):
    """fn(*args) with device `dev` current (switching only when it is not)."""
    if (_get_device() if _get_device is not None else torch.cuda.current_device()) == dev:
        return fn(*args)
    with torch.cuda.device(dev):
        return fn(*args)


def _dims(q, k_cache, page_table, head_dim_v, q_seq_len, workspace_bytes=0) -> Dims:
    d = Dims()
    d.batch = q.shape[0]
    d.num_q_heads = q.shape[-2]
    d.head_dim_qk = q.shape[-1]
    d.head_dim_v = head_dim_v
    d.pages_per_seq = page_table.shape[-1]
    d.num_pages = k_cache.shape[0]
    if q.dtype not in (torch.float16, torch.bfloat16, torch.float8_e4m3fn):
        raise PkvError(1, f"q dtype must be float16, bfloat16 or float8_e4m3fn (latent cache), "
                          f"got {q.dtype}")
    if k_cache.dtype not in _DTYPE:
        raise PkvError(1, f"unsupported KV cache dtype {k_cache.dtype}")
    d.q_dtype = _DTYPE[q.dtype]
    d.kv_dtype = _DTYPE[k_cache.dtype]
    d.workspace_bytes = workspace_bytes
    return d


def _options(path=None, split_pages=0, num_cus=0, target_ctas=0, split_event=None,
             q_scale_dev=None, kv_scale_dev=None, single_launch=None, out_fp8=False,
             rcp_out_scale=1.0):
    if not (path or split_pages or num_cus or target_ctas or split_event or q_scale_dev
            or kv_scale_dev or single_launch is not None or out_fp8):
        return None
    o = Options()
    o.path = {None: 0, "auto": 0, "valu": 1, "mfma": 2, "mfma_mla": 3}.get(path, path)
    o.split_pages, o.num_cus, o.target_ctas = split_pages, num_cus, target_ctas
    o.split_event = split_event
    o.q_scale_dev, o.kv_scale_dev = q_scale_dev, kv_scale_dev
    o.merge_mode = 0 if single_launch is None else 2 if single_launch else 1
    o.out_fp8 = 1 if out_fp8 else 0
    o.rcp_out_scale = float(rcp_out_scale)
    return o


def _scale_arg(x, name, device):
    """A scale given as a float, or (as the xqa page allows) a one-element fp32
    device tensor: returns (host value, device pointer or None)."""
    if isinstance(x, torch.Tensor):
        if (x.dtype != torch.float32 or x.numel() != 1 or x.device != device):
            raise PkvError(1, f"{name} tensor must hold one float32 on {device}")
        return 1.0, x.data_ptr()
    return float(x), None


def query_plan(*, batch, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, pages_per_seq,
               page_size, q_dtype=torch.bfloat16, kv_dtype=None, num_pages=1, window=0,
               q_seq_len=1, path=None, split_pages=0, num_cus=0, target_ctas=0,
               single_launch=None) -> dict:
    """The plan the library would use (host only when num_cus > 0)."""
    d = Dims(batch, num_q_heads, head_dim_qk, head_dim_v, pages_per_seq, num_pages,
             _DTYPE[q_dtype], _DTYPE[kv_dtype or q_dtype], 0)
    info = PlanInfo()
    o = _options(path, split_pages, num_cus, target_ctas, single_launch=single_launch)
    _check(lib().pkv_query_plan(ctypes.byref(d), num_kv_heads, page_size, window, q_seq_len,
                                None if o is None else ctypes.byref(o), ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in PlanInfo._fields_}


def workspace_size(*, batch, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, pages_per_seq,
                   page_size, q_dtype=torch.bfloat16, kv_dtype=None, window=0, q_seq_len=1) -> int:
    d = Dims(batch, num_q_heads, head_dim_qk, head_dim_v, pages_per_seq, 1, _DTYPE[q_dtype],
             _DTYPE[kv_dtype or q_dtype], 0)
    return lib().pkv_workspace_size(ctypes.byref(d), num_kv_heads, page_size, window, q_seq_len)


_ws_cache: dict = {}


def _workspace(device, stream: int, nbytes: int) -> torch.Tensor:
    """The default workspace of (device, stream), grown on demand.

    Calls on one stream run in order and may share it; calls on another
    stream get their own, since two calls in flight at once would write the
    same partial slots and counters.  A workspace used on a stream other than
    torch's current one is marked with record_stream, so that dropping it
    when it grows cannot hand its memory out while a kernel still uses it.
    """
    key = (device, stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        if stream != torch.cuda.current_stream(device).cuda_stream:
            ws.record_stream(torch.cuda.ExternalStream(stream, device=device))
        _ws_cache[key] = ws
    return ws


def _shape_checks(q, k_cache, v_cache, page_table, seq_lens, output, num_kv_heads, page_size,
                  kv_layout, q_seq_len, head_dim_v, mask):
    """Shape, dtype, layout and device checks of a decode call; returns q's
    (B, Hq, Dk), the table width and the pages in the cache.  Each tensor's
    shape and dtype are read once (a call on small inputs is host-bound)."""
    qs, ks, pts = q.shape, k_cache.shape, page_table.shape
    B, Hq, Dk = qs[0], qs[-2], qs[-1]
    if q.numel() != B * q_seq_len * Hq * Dk:
        raise PkvError(1, f"q of shape {tuple(qs)} does not hold batch x q_seq_len "
                          f"({q_seq_len}) x num_q_heads x head_dim elements (beam width 1 only)")
    if kv_layout not in _LAYOUT:
        raise PkvError(1, f"kv_layout must be 'NHD' or 'HND', got {kv_layout!r}")
    if len(ks) != 4:
        raise PkvError(1, f"k_cache must be 4-D, got shape {tuple(ks)}")
    ps_dim, h_dim = (1, 2) if kv_layout == "NHD" else (2, 1)
    if ks[ps_dim] != page_size or ks[h_dim] != num_kv_heads or ks[3] != Dk:
        raise PkvError(1, f"k_cache shape {tuple(ks)} does not match {kv_layout} with "
                          f"page_size {page_size}, num_kv_heads {num_kv_heads}, head_dim {Dk}")
    kdt = k_cache.dtype
    if v_cache is not k_cache and v_cache.data_ptr() != k_cache.data_ptr():
        vs = v_cache.shape
        if vs[:3] != ks[:3] or vs[3] != head_dim_v:
            raise PkvError(1, f"v_cache shape {tuple(vs)} does not match k_cache "
                              f"{tuple(ks)} with head_dim_v {head_dim_v}")
        if v_cache.dtype != kdt:
            raise PkvError(1, "k_cache and v_cache must have the same dtype")
    if page_table.dtype != torch.int32 or len(pts) != 2 or pts[0] != B:
        raise PkvError(1, f"page_table must be int32 [batch, pages_per_seq], got "
                          f"{page_table.dtype} {tuple(pts)}")
    if seq_lens.dtype not in (torch.int32, torch.uint32) or seq_lens.numel() != B:
        raise PkvError(1, f"seq_lens must be uint32 (or int32) [batch] or [batch, 1], got "
                          f"{seq_lens.dtype} {tuple(seq_lens.shape)}")
    # an fp8 query's output is bfloat16 (or the fp8 cache's dtype)
    qdt, odt = q.dtype, output.dtype
    out16 = torch.bfloat16 if qdt == torch.float8_e4m3fn else qdt
    out_ok = odt == out16 or (odt in (torch.float8_e4m3fn, torch.uint8)
                              and kdt in (torch.float8_e4m3fn, torch.uint8))
    if not out_ok or output.numel() != B * q_seq_len * Hq * head_dim_v:
        raise PkvError(1, f"output must have q's dtype (bfloat16 for an fp8 query, or the fp8 "
                          f"cache's) and batch x q_seq_len x num_q_heads x head_dim_v elements, "
                          f"got {odt} {tuple(output.shape)}")
    if mask is not None and q_seq_len > 1:
        want = (B, q_seq_len, ((q_seq_len + 31) // 32) * 2)
        if mask.dtype not in (torch.uint16, torch.int16) or tuple(mask.shape) != want:
            raise PkvError(1, f"mask must be uint16 {want}, got {mask.dtype} {tuple(mask.shape)}")
    # q is a device tensor (checked by the caller), so dev >= 0 and a host
    # tensor (get_device() == -1) fails the comparison
    dev = q.get_device()
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("page_table", page_table), ("seq_lens", seq_lens), ("output", output),
                    ("mask", mask)):
        if t is None:
            continue
        if not t.is_contiguous():
            raise PkvError(1, f"{name} must be contiguous")
        if t.get_device() != dev:
            raise PkvError(1, f"{name} is on {t.device}, q on {q.device}")
    return B, Hq, Dk, pts[1], ks[0]


def decode_attn(q, k_cache, v_cache, page_table, seq_lens, output, workspace_buffer=None, *,
                num_kv_heads, page_size, sinks=None, q_scale=1.0, kv_scale=1.0,
                sliding_win_size=0, kv_layout="NHD", q_seq_len=1, mask=None, head_dim_v=None,
                path=None, split_pages=0, target_ctas=0, stream=None, split_event=None,
                single_launch=None, rcp_out_scale=1.0, num_cus=0):
    """Paged-KV decode attention, written in place into ``output``.

    q [B, q_seq_len, Hq, Dqk] (or [B, Hq, Dqk], or the xqa page's beam-1
    forms); caches NHD [P, page_size, Hkv, D] or HND [P, Hkv, page_size, D]
    in q's dtype or float8_e4m3fn (uint8 bytes are read as e4m3fn); pass the
    same tensor as k_cache and v_cache with head_dim_v < Dqk for a latent
    (MLA) cache whose rows start with V.  ``q_scale`` / ``kv_scale`` are
    floats or one-element float32 device tensors (read by the kernels when
    they run).  ``split_event`` (a torch.cuda.Event that has been recorded
    once) is recorded after the split-KV kernel (before the combine kernel,
    when the plan has one).  ``single_launch`` (None: the planner's choice)
    makes the matrix-core stream-K plan merge cut units in the split kernel
    (True) or in a second kernel (False).  A float8_e4m3fn ``output`` (fp8
    caches only, as the xqa page allows the cache's dtype) receives
    round(out * rcp_out_scale).  ``num_cus`` (0: the device's) is the CU
    count the planner sizes the schedule for.  Returns ``output``.
    """
    if head_dim_v is None:
        head_dim_v = output.shape[-1]
    L = lib()
    opts, d, q_scale, kv_scale = _decode_prep(
        q, k_cache, v_cache, page_table, seq_lens, output, num_kv_heads, page_size, sinks,
        q_scale, kv_scale, kv_layout, q_seq_len, mask, head_dim_v, path, split_pages,
        target_ctas, split_event, single_launch, rcp_out_scale, num_cus)
    dev = q.get_device()
    if stream is None:
        stream = _current_stream(dev)
    own_ws = workspace_buffer is None
    if own_ws:
        # the stream's cached workspace; the library rejects it (before any
        # device work) when this call needs more, and it is grown then
        workspace_buffer = _workspace(q.device, stream, 0)
    fn = L.pkv_decode_attn if opts is None else L.pkv_decode_attn_ex
    extra = () if opts is None else (ctypes.byref(opts),)
    for attempt in (0, 1):
        d.workspace_bytes = workspace_buffer.numel() * workspace_buffer.element_size()
        args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), page_table.data_ptr(),
                seq_lens.data_ptr(), output.data_ptr(), workspace_buffer.data_ptr(),
                num_kv_heads, page_size, _LAYOUT[kv_layout], _ptr(sinks), q_scale, kv_scale,
                int(sliding_win_size), int(q_seq_len), _ptr(mask if q_seq_len > 1 else None),
                stream, ctypes.byref(d)) + extra
        st = _call_on(dev, fn, *args)
        if st != PKV_ERR_WORKSPACE_TOO_SMALL or not own_ws or attempt:
            break
        info = PlanInfo()
        _check(_call_on(dev, L.pkv_query_plan, ctypes.byref(d), num_kv_heads, page_size,
                        sliding_win_size, q_seq_len, None if opts is None else ctypes.byref(opts),
                        ctypes.byref(info)))
        workspace_buffer = _workspace(q.device, stream, info.workspace_bytes)
    _check(st)
    return output


def _decode_prep(q, k_cache, v_cache, page_table, seq_lens, output, num_kv_heads, page_size,
                 sinks, q_scale, kv_scale, kv_layout, q_seq_len, mask, head_dim_v, path,
                 split_pages, target_ctas, split_event, single_launch, rcp_out_scale, num_cus=0):
    """Argument checks and the C structs of a decode call (no device work)."""
    if not q.is_cuda:
        raise PkvError(1, "decode_attn runs on the GPU only: q must be a device tensor")
    B, Hq, Dk, pages_per_seq, num_pages = _shape_checks(
        q, k_cache, v_cache, page_table, seq_lens, output, num_kv_heads, page_size, kv_layout,
        q_seq_len, head_dim_v, mask)
    if sinks is not None:
        if sinks.dtype != torch.float32 or sinks.numel() != Hq or not sinks.is_contiguous():
            raise PkvError(1, "sinks must be contiguous float32 [num_kv_heads, head_group_ratio]")
    ev = None if split_event is None else split_event.cuda_event
    q_scale_dev = kv_scale_dev = None
    if isinstance(q_scale, torch.Tensor):
        q_scale, q_scale_dev = _scale_arg(q_scale, "q_scale", q.device)
    if isinstance(kv_scale, torch.Tensor):
        kv_scale, kv_scale_dev = _scale_arg(kv_scale, "kv_scale", q.device)
    out_fp8 = output.dtype in (torch.float8_e4m3fn, torch.uint8)
    opts = _options(path, split_pages, num_cus, target_ctas, ev, q_scale_dev, kv_scale_dev,
                    single_launch, out_fp8, rcp_out_scale)
    qdt, kdt = q.dtype, k_cache.dtype
    if qdt not in (torch.float16, torch.bfloat16, torch.float8_e4m3fn):
        raise PkvError(1, f"q dtype must be float16, bfloat16 or float8_e4m3fn (latent cache), "
                          f"got {qdt}")
    if kdt not in _DTYPE:
        raise PkvError(1, f"unsupported KV cache dtype {kdt}")
    d = Dims(B, Hq, Dk, head_dim_v, pages_per_seq, num_pages, _DTYPE[qdt], _DTYPE[kdt], 0)
    return opts, d, float(q_scale), float(kv_scale)


def decode_attn_noalloc(q, k_cache, v_cache, page_table, seq_lens, output, *, num_kv_heads,
                        page_size, sinks=None, q_scale=1.0, kv_scale=1.0, sliding_win_size=0,
                        kv_layout="NHD", q_seq_len=1, mask=None, head_dim_v=None, path=None,
                        split_pages=0, target_ctas=0, stream=None, split_event=None,
                        single_launch=None, rcp_out_scale=1.0, num_cus=0):
    """``decode_attn`` without a workspace and without allocating anything.

    The partial results live in the library's static per-GPU scratch
    (``pkv_decode_attn_noalloc``): calls that overlap in time on one GPU race,
    and a plan needing more than ``NOALLOC_SCRATCH_BYTES`` raises.  Returns
    ``output``.
    """
    if head_dim_v is None:
        head_dim_v = output.shape[-1]
    L = lib()
    opts, d, q_scale, kv_scale = _decode_prep(
        q, k_cache, v_cache, page_table, seq_lens, output, num_kv_heads, page_size, sinks,
        q_scale, kv_scale, kv_layout, q_seq_len, mask, head_dim_v, path, split_pages,
        target_ctas, split_event, single_launch, rcp_out_scale, num_cus)
    dev = q.get_device()
    if stream is None:
        stream = _current_stream(dev)
    st = _call_on(dev, L.pkv_decode_attn_noalloc,
                  _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(seq_lens),
                  _ptr(output), num_kv_heads, page_size, _LAYOUT[kv_layout], _ptr(sinks),
                  float(q_scale), float(kv_scale), int(sliding_win_size), int(q_seq_len),
                  _ptr(mask if q_seq_len > 1 else None), stream, ctypes.byref(d),
                  None if opts is None else ctypes.byref(opts))
    _check(st)
    return output


def validate_inputs(q, k_cache, page_table, seq_lens, *, num_kv_heads, page_size,
                    sliding_win_size=0, q_seq_len=1, head_dim_v=None, stream=None):
    """Check the device-resident page ids and lengths (synchronises)."""
    d = _dims(q, k_cache, page_table, head_dim_v or q.shape[-1], q_seq_len)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib().pkv_validate_inputs(_ptr(page_table), _ptr(seq_lens), num_kv_heads, page_size,
                                     sliding_win_size, q_seq_len, ctypes.c_void_p(stream),
                                     ctypes.byref(d)))


def cache_insert(k_cache, v_cache, slot_mapping, k, k_rope=None, v=None, *, page_size,
                 kv_layout="NHD", cache_scale_inv=1.0, q_lo=None, q_hi=None, q_out=None,
                 stream=None):
    """Write new tokens' rows into the paged cache, in place (one launch).

    k [N, Hkv, Dlo] (and k_rope [N, Hkv, Dk - Dlo] for a K row built from two
    parts, as the latent row [kv_c_normed | k_pe]); v [N, Hkv, Dv] or None for
    a latent cache (v_cache None); slot_mapping [N] int64 (page * page_size +
    offset, negative = padding).  A float8_e4m3fn (or uint8) cache stores
    round(x * cache_scale_inv); ``cache_scale_inv`` is a float or a
    one-element float32 device tensor.  With q_out [N, Hq, Dk], also writes
    the query concat [q_lo | q_hi].  Returns k_cache.
    """
    if k.device.type != "cuda":
        raise PkvError(1, "cache_insert runs on the GPU only")
    if k.dtype not in (torch.float16, torch.bfloat16):
        raise PkvError(1, f"source dtype must be float16 or bfloat16, got {k.dtype}")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("slot_mapping", slot_mapping),
                    ("k", k), ("k_rope", k_rope), ("v", v), ("q_lo", q_lo), ("q_hi", q_hi),
                    ("q_out", q_out)):
        if t is None:
            continue
        if not t.is_contiguous():
            raise PkvError(1, f"{name} must be contiguous")
        if t.device != k.device:
            raise PkvError(1, f"{name} is on {t.device}, k on {k.device}")
    for name, t in (("k_rope", k_rope), ("v", v), ("q_lo", q_lo), ("q_hi", q_hi), ("q_out", q_out)):
        if t is not None and t.dtype != k.dtype:
            raise PkvError(1, f"{name} dtype {t.dtype} differs from k's {k.dtype}")
    if slot_mapping.dtype != torch.int64 or slot_mapping.dim() != 1:
        raise PkvError(1, "slot_mapping must be a 1-D int64 tensor")
    if k_cache.dtype not in _DTYPE or (v_cache is not None and v_cache.dtype != k_cache.dtype):
        raise PkvError(1, "caches must share one supported dtype")
    N = slot_mapping.shape[0]
    Dk = k_cache.shape[-1]
    if k.dim() != 3 or k.shape[0] != N:
        raise PkvError(1, f"k must be [N, num_kv_heads, Dlo] with N = {N}")
    Hkv, Dlo = k.shape[1], k.shape[2]
    kv_layout = kv_layout.upper()
    if kv_layout not in _LAYOUT:
        raise PkvError(1, f"kv_layout must be NHD or HND, got {kv_layout}")
    heads_at = 2 if kv_layout == "NHD" else 1
    slots_at = 1 if kv_layout == "NHD" else 2
    if (k_cache.dim() != 4 or k_cache.shape[heads_at] != Hkv or k_cache.shape[slots_at] != page_size):
        raise PkvError(1, f"k_cache must be [pages, {page_size}, {Hkv}, Dk] (NHD) or "
                          f"[pages, {Hkv}, {page_size}, Dk] (HND); got {tuple(k_cache.shape)}")
    if (k_rope is None) != (Dlo == Dk):
        raise PkvError(1, "k_rope is needed exactly when k is narrower than the cache row")
    if k_rope is not None and tuple(k_rope.shape) != (N, Hkv, Dk - Dlo):
        raise PkvError(1, f"k_rope must be [{N}, {Hkv}, {Dk - Dlo}]")
    Dv = 0
    if v is not None or v_cache is not None:
        if v is None or v_cache is None or v_cache.shape[:3] != k_cache.shape[:3]:
            raise PkvError(1, "v and v_cache go together, with k_cache's first three dims")
        Dv = v_cache.shape[-1]
        if tuple(v.shape) != (N, Hkv, Dv):
            raise PkvError(1, f"v must be [{N}, {Hkv}, {Dv}]")
    Hq = 0
    if q_out is not None:
        if q_out.dim() != 3 or q_out.shape[0] != N or q_out.shape[2] != Dk:
            raise PkvError(1, f"q_out must be [{N}, num_q_heads, {Dk}]")
        Hq = q_out.shape[1]
        if q_lo is None or tuple(q_lo.shape) != (N, Hq, Dlo):
            raise PkvError(1, f"q_lo must be [{N}, {Hq}, {Dlo}]")
        if Dlo < Dk and (q_hi is None or tuple(q_hi.shape) != (N, Hq, Dk - Dlo)):
            raise PkvError(1, f"q_hi must be [{N}, {Hq}, {Dk - Dlo}]")
    d = InsertDims(N, Hkv, Dk, Dlo, Dv, page_size, k_cache.shape[0], _LAYOUT[kv_layout],
                   _DTYPE[k.dtype], _DTYPE[k_cache.dtype], Hq)
    scale, scale_dev = _scale_arg(cache_scale_inv, "cache_scale_inv", k.device)
    if stream is None:
        stream = torch.cuda.current_stream(k.device).cuda_stream
    with torch.cuda.device(k.device):
        st = lib().pkv_cache_insert(_ptr(k), _ptr(k_rope), _ptr(v), _ptr(slot_mapping),
                                    _ptr(k_cache), _ptr(v_cache), float(scale),
                                    None if scale_dev is None else ctypes.c_void_p(scale_dev),
                                    _ptr(q_lo), _ptr(q_hi), _ptr(q_out), ctypes.c_void_p(stream),
                                    ctypes.byref(d))
    _check(st)
    return k_cache


def head_matmul(x, w, y=None, *, stream=None):
    """Per-head product y[m, h] = x[m, h] . w[h] (one launch).

    x [M, H, K] (any strides with a contiguous last dim, e.g. the q_nope
    slice of q), w [H, K, N] contiguous (the latent-attention weights W_UK_T
    or W_UV in their stored layout), y [M, H, N] (allocated when None; may
    be a strided view).  bf16 or f16 throughout.  Returns y.
    """
    if x.device.type != "cuda":
        raise PkvError(1, "head_matmul runs on the GPU only")
    if x.dim() != 3 or w.dim() != 3 or x.shape[1] != w.shape[0] or x.shape[2] != w.shape[1]:
        raise PkvError(1, f"x must be [M, H, K] and w [H, K, N]; got {tuple(x.shape)} and "
                          f"{tuple(w.shape)}")
    if x.dtype not in (torch.float16, torch.bfloat16) or w.dtype != x.dtype:
        raise PkvError(1, "x and w must share dtype float16 or bfloat16")
    if not w.is_contiguous() or x.stride(2) != 1:
        raise PkvError(1, "w must be contiguous and x's last dim contiguous")
    M, H, K = x.shape
    N = w.shape[2]
    if y is None:
        y = torch.empty((M, H, N), dtype=x.dtype, device=x.device)
    if tuple(y.shape) != (M, H, N) or y.dtype != x.dtype or y.stride(2) != 1:
        raise PkvError(1, f"y must be [{M}, {H}, {N}] of x's dtype with a contiguous last dim")
    for t in (w, y):
        if t.device != x.device:
            raise PkvError(1, "x, w and y must be on one device")
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        st = lib().pkv_head_matmul(_ptr(x), x.stride(0), x.stride(1), _ptr(w), _ptr(y), y.stride(0),
                                   y.stride(1), M, H, K, N, _DTYPE[x.dtype], ctypes.c_void_p(stream))
    _check(st)
    return y


def merge_attn_states(output, prefix_output, prefix_lse, suffix_output, suffix_lse,
                      num_tokens_with_prefix=None, output_lse=None, *, stream=None):
    """Merge two attention results over disjoint key sets by their natural-log
    log-sum-exps, in place into ``output`` (one launch).

    ``output`` [N, H, D] contiguous (bf16 or f16); the two results [>= rows,
    H, D] of the same dtype with a unit last stride (e.g. the leading
    v_head_dim entries of wider rows); log-sum-exps float32 [H, N] (any
    strides).  Tokens at or past ``num_tokens_with_prefix`` (default N) take
    the suffix alone.  ``output`` may be ``suffix_output`` itself when that is
    contiguous.  Returns ``output``.
    """
    if output.device.type != "cuda":
        raise PkvError(1, "merge_attn_states runs on the GPU only")
    if not output.is_contiguous():
        raise PkvError(1, "output must be contiguous")
    N, H, D = output.shape
    n_pre = N if num_tokens_with_prefix is None else int(num_tokens_with_prefix)
    for name, t, rows in (("prefix_output", prefix_output, n_pre), ("suffix_output", suffix_output, N)):
        if t is None and rows == 0:
            continue
        if t is None or t.dtype != output.dtype or tuple(t.shape[1:]) != (H, D) or t.shape[0] < rows \
                or t.stride(2) != 1:
            raise PkvError(1, f"{name} must be [>= {rows}, {H}, {D}] of output's dtype with unit "
                              f"last stride")
    if suffix_output.data_ptr() == output.data_ptr() and not suffix_output.is_contiguous():
        raise PkvError(1, "output may alias suffix_output only when that is contiguous")
    for name, t in (("prefix_lse", prefix_lse), ("suffix_lse", suffix_lse), ("output_lse", output_lse)):
        if t is not None and (t.dtype != torch.float32 or t.dim() != 2 or t.shape[0] != H):
            raise PkvError(1, f"{name} must be float32 [{H}, tokens]")
    if output_lse is not None and output_lse.stride() != suffix_lse.stride():
        raise PkvError(1, "output_lse must have suffix_lse's strides")
    if prefix_lse is not None and prefix_lse.stride() != suffix_lse.stride():
        raise PkvError(1, "prefix_lse and suffix_lse must share strides")
    if stream is None:
        stream = torch.cuda.current_stream(output.device).cuda_stream
    with torch.cuda.device(output.device):
        ps = (0, 0) if prefix_output is None else (prefix_output.stride(0), prefix_output.stride(1))
        st = lib().pkv_merge_attn_states(
            _ptr(output), _ptr(prefix_output), ps[0], ps[1], _ptr(prefix_lse), _ptr(suffix_output),
            suffix_output.stride(0), suffix_output.stride(1), _ptr(suffix_lse), _ptr(output_lse),
            suffix_lse.stride(1), suffix_lse.stride(0), N, H, D, n_pre, _DTYPE[output.dtype],
            ctypes.c_void_p(stream))
    _check(st)
    return output


def ragged_attn(q, k, v, cu_seqlens_q, cu_seqlens_k, *, max_q_len, sm_scale, causal=False,
                out=None, return_lse=False, lse=None, stream=None):
    """Attention over a ragged (non-paged) batch, with its natural-log
    log-sum-exp (the TRTLLM backend page's cum_seq_lens call; the Kimi-K3
    chunked prefill's new-token and context attentions).

    q [total_q, Hq, Dqk], k [total_k, Hkv, Dqk], v [total_k, Hkv, Dv]
    (contiguous, bf16 or f16, one dtype); cu_seqlens_q / cu_seqlens_k int32
    [num_seqs + 1] on the same device; ``max_q_len`` bounds every sequence's
    query count (no device sync here).  Causal: query i of a sequence sees
    keys j <= i + Lk - Lq.  Writes ``out`` [total_q, Hq, Dv] (allocated when
    None) and, with ``return_lse`` or a given ``lse`` (float32 [Hq, total_q],
    any strides), the log-sum-exps.  Returns out, or (out, lse).
    """
    if q.device.type != "cuda":
        raise PkvError(1, "ragged_attn runs on the GPU only")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 3 or not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise PkvError(1, f"{name} must be a contiguous 3-d tensor of q's dtype on q's device")
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise PkvError(1, "ragged_attn takes bfloat16 or float16")
    total_q, Hq, Dqk = q.shape
    total_k, Hkv, Dv = k.shape[0], k.shape[1], v.shape[2]
    if tuple(k.shape) != (total_k, Hkv, Dqk) or tuple(v.shape[:2]) != (total_k, Hkv):
        raise PkvError(1, "k must be [total_k, Hkv, Dqk] and v [total_k, Hkv, Dv]")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or t.dim() != 1 or t.device != q.device or not t.is_contiguous():
            raise PkvError(1, f"{name} must be a contiguous int32 vector on q's device")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise PkvError(1, "cu_seqlens_q and cu_seqlens_k need num_seqs + 1 entries each")
    if out is None:
        out = torch.empty((total_q, Hq, Dv), dtype=q.dtype, device=q.device)
    elif tuple(out.shape) != (total_q, Hq, Dv) or out.dtype != q.dtype or not out.is_contiguous():
        raise PkvError(1, f"out must be contiguous [{total_q}, {Hq}, {Dv}] of q's dtype")
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, total_q)):
        raise PkvError(1, f"lse must be float32 [{Hq}, {total_q}]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = lib().pkv_ragged_attn(
            _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(out), _ptr(lse),
            0 if lse is None else lse.stride(1), 0 if lse is None else lse.stride(0),
            cu_seqlens_q.numel() - 1, Hq, Hkv, Dqk, Dv, total_q, total_k, int(max_q_len),
            float(sm_scale), 1 if causal else 0, _DTYPE[q.dtype], ctypes.c_void_p(stream))
    _check(st)
    return (out, lse) if (return_lse or lse is not None) else out
