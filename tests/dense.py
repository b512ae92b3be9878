"""Dense brute-force attention used to pin the oracle (CPU, torch fp64).

It does not share the oracle's formulation: pages are gathered with torch
indexing into a contiguous [L, D] K/V per sequence and KV head, dtypes are
decoded by torch's own conversions, visibility is an explicit boolean matrix
the caller builds, sinks enter as an extra logit column that is dropped after
the softmax, and the softmax itself is torch.softmax (or torch's
scaled_dot_product_attention).
"""
import torch


def to_f64(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.uint8:
        t = t.view(torch.float8_e4m3fn)
    return t.to(torch.float64)


def gather_rows(cache, page_table_row, L, page_size, kvh, layout):
    """Contiguous [L, row] fp64 rows of one sequence and KV head."""
    c = to_f64(cache)
    t = torch.arange(L)
    pages = page_table_row.to(torch.int64)[t // page_size]
    slots = t % page_size
    if layout == "NHD":
        return c[pages, slots, kvh]
    return c[pages, kvh, slots]


def attention(q, K, V, visible, scale, sink=None):
    """softmax(scale * q K^T over visible keys [+ sink column]) V for one row.

    q: [D] fp64, K: [L, D], V: [L, Dv], visible: bool [L].
    """
    logits = scale * (K @ q)
    logits = torch.where(visible, logits, torch.tensor(float("-inf"), dtype=torch.float64))
    if not bool(visible.any()):
        return torch.zeros(V.shape[1], dtype=torch.float64)
    if sink is not None:
        logits = torch.cat([logits, torch.tensor([float(sink)], dtype=torch.float64)])
        p = torch.softmax(logits, dim=0)[:-1]
    else:
        p = torch.softmax(logits, dim=0)
    p = torch.where(visible, p, torch.zeros((), dtype=torch.float64))
    return p @ V


def dense_decode(inp, *, num_kv_heads, page_size, kv_layout="NHD", q_scale=1.0, kv_scale=1.0,
                 visible_fn=None, sinks=None, v_from_k=False, head_dim_v=None):
    """Brute force over all (b, i, h); visible_fn(b, i, L) -> bool [L] (default: all)."""
    q = to_f64(inp["q"])
    B, Tq, Hq, Dk = q.shape
    G = Hq // num_kv_heads
    Dv = head_dim_v or (Dk if not v_from_k else Dk)
    out = torch.zeros(B, Tq, Hq, Dv, dtype=torch.float64)
    L_all = inp["seq_lens_host"]
    table = inp["page_table_host"]
    scale = q_scale * kv_scale / (Dk ** 0.5)
    for b in range(B):
        L = int(L_all[b])
        for kvh in range(num_kv_heads):
            K = gather_rows(inp["k_cache"], table[b], L, page_size, kvh, kv_layout)
            if v_from_k:
                V = K[:, :Dv]
            else:
                V = gather_rows(inp["v_cache"], table[b], L, page_size, kvh, kv_layout)
            V = kv_scale * V
            for i in range(Tq):
                vis = torch.ones(L, dtype=torch.bool) if visible_fn is None else visible_fn(b, i, L)
                for g in range(G):
                    h = kvh * G + g
                    sink = None if sinks is None else float(sinks[kvh, g])
                    out[b, i, h] = attention(q[b, i, h], K, V, vis, scale, sink)
    return out
