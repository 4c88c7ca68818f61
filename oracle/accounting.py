"""Byte accounting.

KV-cache size: 2 (K and V) x layers x KV heads x head dim x tokens x bytes per
element -- the formula the sarnas.ru JoLT post gives under its section on how
much memory the KV cache takes, with the Llama-3.1-70B example (80 layers, 8 KV
heads, d=128, bf16 -> 327,680 bytes per token), repeated in the hegai.media
piece.

Compressed cell size: the stored tensors of one (layer group, K or V) cell of
a JoLT cache -- "A JoLT for the KV cache" (arXiv 2607.12550v4 summary) §3: the
token factor and feature factor are shared by the group's layers and heads,
the core keeps the layer and head modes at full rank, and b=0 stores no
residual.  The residual is b bits per element plus one fp32 scale per
quantised row (one row per layer, head and token).
"""


def dense_kv_bytes(n_layers, n_kv_heads, head_dim, seq_len, dtype_bytes=2):
    return 2 * n_layers * n_kv_heads * head_dim * seq_len * dtype_bytes


def cell_bytes(T, d, group_size, H, r_T, r_F, bits, factor_bytes):
    """Bytes of one stored cell: factors A (T x r_T), B (d x r_F),
    core G (|g| x H x r_T x r_F) and, when bits > 0, packed codes
    (|g| x H x T rows of d*bits/8 bytes) plus one fp32 scale per row."""
    factors = factor_bytes * (T * r_T + d * r_F + group_size * H * r_T * r_F)
    resid = group_size * H * T * (d * bits // 8 + 4 * (bits > 0))
    return factors + resid


def cache_bytes(cache):
    """Total stored bytes of a compressed cache dict."""
    fb = 4 if cache["factor_dtype"] == "f32" else 2
    gs_list = cache["group_start"]
    total = 0
    for g, pair in enumerate(cache["cells"]):
        gs = gs_list[g + 1] - gs_list[g]
        for cell in pair:
            total += cell_bytes(cache["T"], cache["d"], gs, cache["H"], cell["r_T"],
                                cell["r_F"], cell["bits"], fb)
    return total
