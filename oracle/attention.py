"""Float64 decode attention over a paged KV cache (test infrastructure).

What is computed: for each sequence s and query head h, with g the KV head
that h reads, the single-query attention over the sequence's ctx cached
tokens,

    z_t = scale * <q[s, h], K_t>,   out[s, h] = sum_t softmax(z)_t * V_t,

where token t's K and V rows are found through the block table: block
block_table[s][t // B], row t % B ("Paged Attention" (daiw.org), 直觉 and
定义).  The pages stress that paging changes only where the rows come from,
not the attention itself ("vllm-pagedattention" (chenyuan1125.github.io),
页表真正解开的…: the kernel looks up each K/V block through the table and then
does scores, softmax and the weighted sum), so this module is the plain
definition written out, in float64, on rows decoded from the cache's raw bits.

Readings (the pages are silent on these):
* query head h reads KV head h // (Hq // Hkv) (consecutive grouping);
* the new token has been written before the step, so it attends to itself
  (the context is tokens [0, ctx));
* the softmax is taken after subtracting the maximum score, which leaves
  its value unchanged and keeps exp() finite.
"""
import numpy as np

from .bits import to_f64


def _softmax_weighted_sum(z, v):
    w = np.exp(z - z.max())
    return (w @ v) / w.sum()


def decode_one(q, k_rows, v_rows, scale):
    """One query head: q ``[d]``, K and V rows ``[ctx][d]`` (all float64)."""
    z = scale * (k_rows @ q)
    return _softmax_weighted_sum(z, v_rows)


def paged_decode(q_bits, k_cache_bits, v_cache_bits, block_tables, ctx_lens,
                 block_size, scale, dtype, num_q_heads, num_kv_heads,
                 heads=None):
    """Decode attention for a batch through block tables.

    q_bits        ``[S][Hq][d]`` raw bits
    k/v_cache     ``[num_blocks][Hkv][B][d]`` raw bits
    block_tables  ``[S][max_blocks]`` ints; only entries below
                  ceil(ctx / B) are read
    heads         optional list of (s, h) pairs to compute (others stay 0);
                  lets large batches be checked on a sample
    Returns float64 ``[S][Hq][d]``.
    """
    S = len(ctx_lens)
    d = q_bits.shape[-1]
    group = num_q_heads // num_kv_heads
    out = np.zeros((S, num_q_heads, d), dtype=np.float64)
    want = None
    if heads is not None:
        want = {}
        for s, h in heads:
            want.setdefault(int(s), []).append(int(h))
    for s in range(S):
        if want is not None and s not in want:
            continue
        ctx = int(ctx_lens[s])
        pos = np.arange(ctx)
        blocks = np.asarray(block_tables[s], dtype=np.int64)[pos // block_size]
        rows = pos % block_size
        k = to_f64(k_cache_bits[blocks, :, rows, :], dtype)   # [ctx][Hkv][d]
        v = to_f64(v_cache_bits[blocks, :, rows, :], dtype)
        q = to_f64(q_bits[s], dtype)                          # [Hq][d]
        for h in (want[s] if want is not None else range(num_q_heads)):
            g = h // group
            out[s, h] = decode_one(q[h], k[:, g, :], v[:, g, :], scale)
    return out


def contiguous_decode(q_bits, k_bits, v_bits, ctx_lens, scale, dtype,
                      num_q_heads, num_kv_heads):
    """Same attention on the contiguous layout ``[S][Hkv][cap][d]``.

    The layout the pages contrast paging with: one region per sequence sized
    for its maximum length ("Paged Attention" (daiw.org), 定义, first row of
    the utilisation table).
    """
    S = len(ctx_lens)
    d = q_bits.shape[-1]
    group = num_q_heads // num_kv_heads
    out = np.zeros((S, num_q_heads, d), dtype=np.float64)
    for s in range(S):
        ctx = int(ctx_lens[s])
        k = to_f64(k_bits[s, :, :ctx, :], dtype)               # [Hkv][ctx][d]
        v = to_f64(v_bits[s, :, :ctx, :], dtype)
        q = to_f64(q_bits[s], dtype)
        for h in range(num_q_heads):
            g = h // group
            out[s, h] = decode_one(q[h], k[g], v[g], scale)
    return out


# -- split-context partition + combine ---------------------------------------
# Not on the pages.  A long context is cut into partitions of P tokens; each
# partition keeps its own maximum m_p, its sum of exponentials l_p and its
# unnormalised weighted sum o_p.  Rescaling every partition to the common
# maximum M = max_p m_p gives back the one-pass softmax exactly:
#   L = sum_p l_p * exp(m_p - M),   out = sum_p exp(m_p - M) * o_p / L.

def partition_stats(q, k_rows, v_rows, scale):
    """(m, l, o) of one partition: max score, sum of exp, weighted V sum."""
    z = scale * (k_rows @ q)
    m = z.max()
    w = np.exp(z - m)
    return m, w.sum(), w @ v_rows


def combine_partitions(stats):
    """Merge a list of (m, l, o) partition results into the attention output."""
    M = max(m for m, _, _ in stats)
    L = sum(l * np.exp(m - M) for m, l, _ in stats)
    o = sum(np.exp(m - M) * o for m, _, o in stats)
    return o / L


def split_decode_one(q, k_rows, v_rows, scale, partition):
    """``decode_one`` computed partition by partition and then combined."""
    ctx = k_rows.shape[0]
    stats = [partition_stats(q, k_rows[a:a + partition], v_rows[a:a + partition], scale)
             for a in range(0, ctx, partition)]
    return combine_partitions(stats)
