"""Replays of a workload's operation log, shared by the tests.

``oracle_replay`` runs the log through the oracle's pool model and raw-bit
cache; ``logical_streams`` rebuilds each sequence's token rows straight from
the log, without blocks, tables or slots, so it can pin the paged path.
"""
import numpy as np

from oracle.kv_store import KVStoreModel
from oracle.pool_model import BlockPoolModel


class OracleRun:
    """Pool model + cache model after a workload's log, plus what it emitted."""

    def __init__(self, wl, free_order=None):
        order = wl.free_order if free_order is None else free_order
        self.pool = BlockPoolModel(wl.num_blocks, wl.block_size, order)
        self.cache = KVStoreModel(wl.num_blocks, wl.num_kv_heads, wl.block_size,
                                  wl.head_dim, wl.dtype)
        self.slots = []        # per op: list of slots written (or [])
        self.cow = []          # every (src, dst) pair in order
        for op in wl.ops():
            self.slots.append(self.apply(wl, op))

    def apply(self, wl, op):
        kind = op[0]
        if kind == "alloc":
            _, seq, n, r0 = op
            slots = self.pool.alloc(seq, n)
            self.cache.write(slots, wl.k_rows[r0:r0 + n], wl.v_rows[r0:r0 + n])
            return slots
        if kind == "append":
            _, seq, n, r0 = op
            slots = []
            for i in range(n):
                slot, cow = self.pool.append(seq)
                if cow is not None:
                    self.cow.append(cow)
                    self.cache.copy([cow])
                self.cache.write([slot], wl.k_rows[r0 + i:r0 + i + 1],
                                 wl.v_rows[r0 + i:r0 + i + 1])
                slots.append(slot)
            return slots
        if kind == "fork":
            self.pool.fork(op[1], op[2])
            return []
        if kind == "free":
            self.pool.free(op[1])
            return []
        raise ValueError(kind)

    def tables(self, wl):
        rows, lens = self.pool.block_tables(wl.batch, wl.max_blocks)
        return np.asarray(rows, dtype=np.int32), np.asarray(lens, dtype=np.int32)

    # preemption: the pool's swap verbs plus the cache's swap images
    def swap_out(self, seq):
        """Release seq's blocks; returns (old table, host image of its blocks)."""
        table = self.pool.swap_out(seq)
        return table, self.cache.swap_image(table)

    def swap_in(self, seq, image):
        """New blocks for seq, filled from its image; returns the new table."""
        table = self.pool.swap_in(seq)
        self.cache.restore_image(table, image)
        return table


def logical_streams(wl):
    """seq -> row indices (into k_rows / v_rows) of its tokens, in order."""
    streams = {}
    for op in wl.ops():
        kind = op[0]
        if kind == "alloc":
            _, seq, n, r0 = op
            streams[seq] = list(range(r0, r0 + n))
        elif kind == "append":
            _, seq, n, r0 = op
            streams[seq].extend(range(r0, r0 + n))
        elif kind == "fork":
            streams[op[2]] = list(streams[op[1]])
        elif kind == "free":
            del streams[op[1]]
    return streams


def contiguous_layout(wl, capacity=None):
    """Dense ``[S][Hkv][cap][d]`` K and V bits of the batch, NaN past ctx."""
    from oracle.bits import NAN_BITS
    streams = logical_streams(wl)
    ctx = [len(streams[s]) for s in wl.batch]
    cap = capacity or max(ctx)
    shape = (len(wl.batch), wl.num_kv_heads, cap, wl.head_dim)
    k = np.full(shape, NAN_BITS[wl.dtype], dtype=wl.k_rows.dtype)
    v = np.full(shape, NAN_BITS[wl.dtype], dtype=wl.v_rows.dtype)
    for i, s in enumerate(wl.batch):
        rows = np.asarray(streams[s])
        k[i, :, :len(rows), :] = wl.k_rows[rows].transpose(1, 0, 2)
        v[i, :, :len(rows), :] = wl.v_rows[rows].transpose(1, 0, 2)
    return k, v, np.asarray(ctx, dtype=np.int32)
