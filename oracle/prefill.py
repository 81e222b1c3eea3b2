"""Float64 chunked prefill attention over a paged KV cache (test infrastructure).

What is computed.  A prefill step hands the model a chunk of a sequence's
new tokens at once (the pages: prefill admits a prompt and allocates
ceil(prompt / B) blocks for it, "vLLM PagedAttention：大模型推理的显存管理革命",
分配策略; prefill works on large blocks of queries, "vllm-pagedattention",
它和 FlashAttention 优化的是两张不同的账).  The chunk's K and V rows have been
written into the cache first, so sequence s holds ctx[s] tokens of which the
last n_s are the chunk.  Query i of the chunk sits at position
p = ctx[s] - n_s + i and, as every autoregressive query, sees the tokens at
positions 0..p:

    out[row, h] = sum_{t <= p} softmax_t(scale * <q[row, h], K_t>) * V_t,

with K_t, V_t found through the block table exactly as in decode ("Paged
Attention" (daiw.org), 定义).  The pages say that combining paging with a
tiled (FlashAttention-style) kernel changes how the operator moves data, not
what it computes ("Paged Attention" (daiw.org), 回顾与衔接), so this module
is the plain definition written out in float64: each query row is the decode
attention of that row over its visible prefix.

Layout (a reading; the pages give no prefill interface): the chunks of all
sequences are packed row after row, q ``[T][Hq][d]`` with sequence s owning
rows [q_start[s], q_start[s+1]); out has the same shape.
"""
import numpy as np

from .attention import decode_one
from .bits import to_f64


def chunk_positions(ctx_len, n_rows):
    """Positions of a chunk's query rows: the last n_rows of ctx_len tokens."""
    return np.arange(ctx_len - n_rows, ctx_len, dtype=np.int64)


def paged_prefill(q_bits, k_cache_bits, v_cache_bits, block_tables, ctx_lens, q_start,
                  block_size, scale, dtype, num_q_heads, num_kv_heads, rows=None):
    """Causal attention of every chunk row over its sequence's paged context.

    q_bits        ``[T][Hq][d]`` raw bits, rows grouped by sequence
    k/v_cache     ``[num_blocks][Hkv][B][d]`` raw bits
    block_tables  ``[S][max_blocks]``; entries below ceil(ctx / B) are read
    ctx_lens      ``[S]`` tokens in the cache, the chunk included
    q_start       ``[S + 1]`` row offsets; the chunk of s is rows q_start[s]..q_start[s+1]-1
    rows          optional iterable of (row, h) pairs to compute (others stay 0)
    Returns float64 ``[T][Hq][d]``.
    """
    T = q_bits.shape[0]
    d = q_bits.shape[-1]
    group = num_q_heads // num_kv_heads
    out = np.zeros((T, num_q_heads, d), dtype=np.float64)
    want = None
    if rows is not None:
        want = {}
        for r, h in rows:
            want.setdefault(int(r), []).append(int(h))
    q_all = to_f64(q_bits, dtype)
    for s in range(len(ctx_lens)):
        r0, r1 = int(q_start[s]), int(q_start[s + 1])
        if r1 == r0 or (want is not None and not any(r in want for r in range(r0, r1))):
            continue
        ctx = int(ctx_lens[s])
        pos = np.arange(ctx)
        blocks = np.asarray(block_tables[s], dtype=np.int64)[pos // block_size]
        k = to_f64(k_cache_bits[blocks, :, pos % block_size, :], dtype)   # [ctx][Hkv][d]
        v = to_f64(v_cache_bits[blocks, :, pos % block_size, :], dtype)
        for r, p in zip(range(r0, r1), chunk_positions(ctx, r1 - r0)):
            heads = range(num_q_heads) if want is None else want.get(r, [])
            for h in heads:
                g = h // group
                out[r, h] = decode_one(q_all[r, h], k[:p + 1, g], v[:p + 1, g], scale)
    return out


def prefill_flops(ctx_lens, q_start, head_dim, num_q_heads):
    """Multiply-add work of a prefill call, counted as 2 flops each: per query
    row at position p, (p + 1) dot products of length d for the scores and
    (p + 1) * d for the weighted sum, for every query head."""
    total = 0
    for s in range(len(ctx_lens)):
        n = int(q_start[s + 1]) - int(q_start[s])
        p = chunk_positions(int(ctx_lens[s]), n)
        total += int(np.sum(p + 1)) * 2 * 2 * head_dim * num_q_heads
    return total
