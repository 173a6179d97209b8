"""Oracle for PagedAttention decode (test infrastructure).

What it computes: for each sequence i with context length n (the number of
tokens whose K/V are in the cache, this step's token included) and each query
head h,

    out[i][h] = softmax(q[i][h] . K_i^T * scale) V_i

with K_i, V_i the [n][D] keys and values of the KV head that h reads.  This is
the attention formula of the dpshk.com PagedAttention article
("企业官网建设流程全解析", section 2.2), evaluated over the whole context.

That article's blockwise pseudocode normalises each block on its own and adds
the per-block results; that disagrees with its own formula whenever the context
spans more than one block, and would make the output depend on the block size.
This oracle takes the formula: ONE softmax over all n tokens.  Blocks only
decide where the rows are stored.

K_i and V_i are gathered through the block table: logical block j of sequence
i is physical block ``block_tables[i][j]``; token t sits at offset
``t % block_size`` of logical block ``t // block_size`` (page
"vLLM的诞生背景…", section "PagedAttention的破局思路"; page
"PagedAttention 与连续批处理…", section "PagedAttention：把显存做成虚拟内存":
attention finds each page through the page table).  Table entries past the
last needed block and rows past n in the last block are never read.

Query head h reads KV head ``h // (H / H_kv)`` (consecutive groups; the pages
do not mention grouped-query attention, this is the reading used for grouped
workloads).  The scale is the float32 value passed by the caller, promoted
exactly to float64.  A sequence with n = 0 yields zeros.

FP8 caches are dequantised as ``decode(code) * scale[block][kv_head]`` in
float64.  All arithmetic is float64; the result is float64 [S][H][D].
"""

import numpy as np

from .fp8_e4m3 import fp8_decode


def element_values(arr: np.ndarray) -> np.ndarray:
    """fp32 / bf16-bits / FP8-codes array -> float64 (FP8 still unscaled)."""
    if arr.dtype == np.float32 or arr.dtype == np.float64:
        return arr.astype(np.float64)
    if arr.dtype == np.uint16:
        return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if arr.dtype == np.uint8:
        return fp8_decode(arr)
    raise TypeError(f"unsupported dtype {arr.dtype}")


def gather_sequence(cache, scales, table_row, n, block_size, kv_heads=None):
    """Contiguous float64 [n][H_kv'][D] rows of one sequence.

    cache  : [num_blocks][H_kv][block_size][D]
    scales : [num_blocks][H_kv] float32 for FP8 caches, else None
    kv_heads: optional list of KV heads to keep (default: all)
    """
    nb = -(-n // block_size)
    phys = np.asarray(table_row[:nb], dtype=np.int64)
    tiles = cache[phys]                                   # [nb][H_kv][bs][D]
    if kv_heads is not None:
        tiles = tiles[:, kv_heads]
    vals = element_values(tiles)
    if scales is not None:
        sc = np.asarray(scales, dtype=np.float32)[phys]   # [nb][H_kv]
        if kv_heads is not None:
            sc = sc[:, kv_heads]
        vals = vals * sc.astype(np.float64)[:, :, None, None]
    # [nb][H][bs][D] -> [nb][bs][H][D] -> [nb*bs][H][D], then keep n rows.
    rows = vals.transpose(0, 2, 1, 3).reshape(nb * block_size, vals.shape[1], vals.shape[3])
    return rows[:n]


def _attend(qv, K, V, scale):
    """softmax(qv . K^T * scale) V for one head, float64."""
    s = (K @ qv) * scale
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def paged_attention_decode(q, key_cache, value_cache, block_tables, context_lens,
                           scale, block_size, key_scale=None, value_scale=None):
    """float64 [S][H][D] decode output.

    q            : [S][H][D] float32 or uint16 (bf16 bits)
    key/value_cache : [num_blocks][H_kv][block_size][D]
    block_tables : [S][max_blocks] integer
    context_lens : [S] integer
    scale        : softmax scale (taken as float32)
    key/value_scale : [num_blocks][H_kv] float32 for FP8 caches
    """
    qf = element_values(np.asarray(q))
    S, H, D = qf.shape
    H_kv = key_cache.shape[1]
    G = H // H_kv
    sc = float(np.float32(scale))
    out = np.zeros((S, H, D), dtype=np.float64)
    for i in range(S):
        n = int(context_lens[i])
        if n == 0:
            continue
        K = gather_sequence(key_cache, key_scale, block_tables[i], n, block_size)
        V = gather_sequence(value_cache, value_scale, block_tables[i], n, block_size)
        for h in range(H):
            g = h // G
            out[i, h] = _attend(qf[i, h], K[:, g, :], V[:, g, :], sc)
    return out


def paged_attention_decode_one(q, key_cache, value_cache, block_tables, context_lens,
                               scale, block_size, seq, head,
                               key_scale=None, value_scale=None):
    """float64 [D] output of one (sequence, query head): for sampled checks."""
    H = q.shape[1]
    H_kv = key_cache.shape[1]
    g = head // (H // H_kv)
    n = int(context_lens[seq])
    D = q.shape[2]
    if n == 0:
        return np.zeros(D, dtype=np.float64)
    qv = element_values(np.asarray(q[seq, head]))
    K = gather_sequence(key_cache, key_scale, block_tables[seq], n, block_size, [g])[:, 0, :]
    V = gather_sequence(value_cache, value_scale, block_tables[seq], n, block_size, [g])[:, 0, :]
    return _attend(qv, K, V, float(np.float32(scale)))


def paged_attention_prefill(q, key_cache, value_cache, block_tables, context_lens, scale,
                            block_size, key_scale=None, value_scale=None):
    """float64 [S][M][H][D]: the decode formula for each of M new query tokens.

    Sequence i holds n = context_lens[i] tokens, its M newest being the query
    tokens; token t sits at position n - M + t and attends to positions
    0 .. n - M + t (causal), i.e. it is a decode step whose context ends at
    its own position (dpshk.com article, section 2.2, applied per token).
    """
    q = np.asarray(q)
    M = q.shape[1]
    lens = np.asarray(context_lens, dtype=np.int64)
    assert np.all(lens >= M), "every sequence holds its query tokens"
    out = np.zeros(q.shape, dtype=np.float64)
    for t in range(M):
        out[:, t] = paged_attention_decode(q[:, t], key_cache, value_cache, block_tables,
                                           lens - M + t + 1, scale, block_size, key_scale,
                                           value_scale)
    return out
