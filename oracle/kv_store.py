"""Raw-bit KV cache model in the [block][kv_head][slot][dim] layout.

Test infrastructure only.  Holds K and V as unsigned integer arrays of the
element width, so every write, copy and swap image can be compared with the
device cache and the host buffer byte for byte.  The layout is the reading this build takes of the pages'
statement that a block is contiguous inside and blocks may sit anywhere
("Paged Attention" (daiw.org), 定义): one block holds, per KV head, its B
token rows of ``head_dim`` elements back to back.
"""
import numpy as np

from .bits import BITS_DTYPE, NAN_BITS


class KVStoreModel:
    def __init__(self, num_blocks, kv_heads, block_size, head_dim, dtype,
                 poison=True):
        shape = (num_blocks, kv_heads, block_size, head_dim)
        fill = NAN_BITS[dtype] if poison else 0
        self.dtype = dtype
        self.block_size = block_size
        self.k = np.full(shape, fill, dtype=BITS_DTYPE[dtype])
        self.v = np.full(shape, fill, dtype=BITS_DTYPE[dtype])

    def write(self, slots, k_rows, v_rows):
        """Store token rows ``[T][kv_heads][head_dim]`` at flat ``slots``.

        Slot s names block s // B, row s % B.  A negative slot is a padding
        entry and is skipped.
        """
        for t, slot in enumerate(np.asarray(slots).tolist()):
            if slot < 0:
                continue
            blk, row = divmod(slot, self.block_size)
            self.k[blk, :, row, :] = k_rows[t]
            self.v[blk, :, row, :] = v_rows[t]

    def copy(self, pairs):
        """Copy whole blocks, K and V, for each (src, dst) pair in order."""
        for src, dst in pairs:
            self.k[dst] = self.k[src]
            self.v[dst] = self.v[src]

    def gather(self, table, ctx):
        """Logical K and V rows ``[ctx][kv_heads][head_dim]`` of one sequence."""
        pos = np.arange(ctx)
        blocks = np.asarray(table, dtype=np.int64)[pos // self.block_size]
        rows = pos % self.block_size
        return self.k[blocks, :, rows, :], self.v[blocks, :, rows, :]

    # -- swap images ("vllm-paged-attention-engine" (aiqz.cc), 连续批处理：
    # 随到随走的新秩序: a preempted request's blocks are copied out to CPU
    # memory and copied back in when it resumes).  The pages fix no host
    # layout; the reading taken here is one record per listed block, in list
    # order, holding that block's K and then its V, each in the cache's own
    # [kv_head][slot][dim] order:  image[i][0] = K[blocks[i]],
    # image[i][1] = V[blocks[i]].

    def swap_image(self, blocks):
        """Host image ``[n][2][kv_heads][B][head_dim]`` (raw bits) of the
        listed blocks, K then V for each."""
        n = len(blocks)
        _, hkv, B, d = self.k.shape
        image = np.empty((n, 2, hkv, B, d), dtype=self.k.dtype)
        for i, blk in enumerate(blocks):
            image[i, 0] = self.k[blk]
            image[i, 1] = self.v[blk]
        return image

    def restore_image(self, blocks, image):
        """Write a swap image back: block ``blocks[i]`` receives record i."""
        for i, blk in enumerate(blocks):
            self.k[blk] = image[i, 0]
            self.v[blk] = image[i, 1]
