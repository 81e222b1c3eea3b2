"""Block pool model: free list, block tables, refcounts, fork, copy-on-write.

Test infrastructure only.  An independent restatement of the allocation rules
the pages describe; the parity tests replay one operation log through this
model and through the native pool and compare every table, slot and copy
pair bit for bit.

Rules, each with the passage it comes from:

* A sequence of n tokens holds ceil(n / B) blocks; prefill takes them all at
  once ("vLLM PagedAttention：大模型推理的显存管理革命" (horeb.top), 分配策略;
  "vllm-paged-attention-engine" (aiqz.cc), 分页存储设计 formula N_i).
* Allocation is all-or-nothing: when the pool cannot cover the request it is
  refused and nothing changes ("Paged Attention" (daiw.org), 读者问答 / 运维提示:
  an exhausted pool rejects new requests instead of crashing; the allocator
  of "vllm-paged-attention-engine", Python 演示, checks before it takes).
* Free blocks are taken from the front of the free list and returned to its
  back (the allocator of "vllm-paged-attention-engine", Python 演示: it takes
  the first n free blocks and appends released blocks at the end).
* A new token goes into the last block while that block has room; only a
  full last block makes the pool hand out one more block, appended to the
  table ("vllm-pagedattention" (chenyuan1125.github.io), 页表真正解开的…).
* A finished sequence gives back its blocks ("Paged Attention", 定义).
* Each physical block carries a reference count; several tables may name the
  same block and a block goes back to the free list only when its count
  reaches zero ("Paged Attention", 量化 and 工程现场 (fork);
  "vllm-pagedattention", 一块内存，如何安全地属于多条序列).
* A branch that must write into a last block that is still shared copies it
  first, points its own table at the copy and then writes; full blocks stay
  shared ("vllm-pagedattention", 一块内存，如何安全地属于多条序列;
  "vLLM PagedAttention：大模型推理的显存管理革命", 内存共享：写时复制).

Readings taken where the pages are silent:
* slot of token i = block_table[i // B] * B + i % B (flat slot index);
* a fork copies the parent's table and length and bumps every refcount;
* freeing walks the table in order, so released blocks reach the free list
  in table order;
* the copy-on-write destination is taken from the front of the free list.

Swap-out / swap-in ("vllm-paged-attention-engine" (aiqz.cc), 连续批处理：随到随走的
新秩序: under memory pressure a request's whole set of blocks is copied back
to CPU memory, and copied in again when there is room):
* swap-out hands back the table (the blocks to copy out), releases the blocks
  as a free would and keeps the sequence's id and length;
* swap-in takes ceil(len / B) blocks from the front of the free list
  (all-or-nothing) as the new table; blocks shared before come back private;
* a swapped-out sequence refuses growth, fork and table views; statistics
  count resident sequences only.
"""
from collections import deque


class PoolError(Exception):
    """Refused operation; ``code`` is one of NOBLOCKS, NOSEQ, EXISTS, INVAL."""

    def __init__(self, code, msg=""):
        super().__init__(f"{code}: {msg}")
        self.code = code


class BlockPoolModel:
    def __init__(self, num_blocks, block_size, initial_free_order=None):
        if num_blocks < 0 or block_size <= 0:
            raise PoolError("INVAL", "bad pool shape")
        if initial_free_order is None:
            initial_free_order = range(num_blocks)
        order = [int(b) for b in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise PoolError("INVAL", "free order must be a permutation")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free_list = deque(order)
        self.refcount = [0] * num_blocks
        self.tables = {}   # seq id -> list of physical block ids
        self.length = {}   # seq id -> tokens held
        self.swapped = set()

    # -- helpers -----------------------------------------------------------
    def _take(self):
        """The block at the front of the free list."""
        return self.free_list.popleft()

    def _slot(self, seq, pos):
        blk = self.tables[seq][pos // self.block_size]
        return blk * self.block_size + pos % self.block_size

    def _need(self, seq):
        if seq not in self.tables:
            raise PoolError("NOSEQ", f"unknown sequence {seq}")

    def _resident(self, seq):
        self._need(seq)
        if seq in self.swapped:
            raise PoolError("INVAL", f"sequence {seq} is swapped out")

    def _release(self, table):
        """Blocks whose count reaches zero go to the back, in table order."""
        for blk in table:
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                self.free_list.append(blk)

    # -- verbs -------------------------------------------------------------
    def alloc(self, seq, n_tokens):
        """Admit ``seq`` with ``n_tokens`` prompt tokens; returns their slots."""
        if n_tokens < 0:
            raise PoolError("INVAL", "negative length")
        if seq in self.tables:
            raise PoolError("EXISTS", f"sequence {seq} exists")
        want = -(-n_tokens // self.block_size)
        if want > len(self.free_list):
            raise PoolError("NOBLOCKS", f"need {want}, have {len(self.free_list)}")
        table = [self._take() for _ in range(want)]
        for blk in table:
            self.refcount[blk] = 1
        self.tables[seq] = table
        self.length[seq] = n_tokens
        return [self._slot(seq, i) for i in range(n_tokens)]

    def append(self, seq):
        """Reserve the next token's slot; returns (slot, cow pair or None)."""
        self._resident(seq)
        table = self.tables[seq]
        pos = self.length[seq]
        cow = None
        if pos % self.block_size == 0:
            # last block full (or no block yet): one more block at the end
            if not self.free_list:
                raise PoolError("NOBLOCKS", "no block for growth")
            blk = self._take()
            self.refcount[blk] = 1
            table.append(blk)
        elif self.refcount[table[-1]] > 1:
            # the token lands in a last block other sequences still share
            if not self.free_list:
                raise PoolError("NOBLOCKS", "no block for copy-on-write")
            src = table[-1]
            dst = self._take()
            self.refcount[src] -= 1
            self.refcount[dst] = 1
            table[-1] = dst
            cow = (src, dst)
        self.length[seq] = pos + 1
        return self._slot(seq, pos), cow

    def fork(self, parent, child):
        """``child`` starts as a copy of ``parent`` sharing every block."""
        self._need(parent)
        if child in self.tables:
            raise PoolError("EXISTS", f"sequence {child} exists")
        self._resident(parent)
        table = list(self.tables[parent])
        for blk in table:
            self.refcount[blk] += 1
        self.tables[child] = table
        self.length[child] = self.length[parent]

    def free(self, seq):
        """Drop ``seq``; blocks whose count reaches zero return to the back."""
        self._need(seq)
        self._release(self.tables.pop(seq))
        del self.length[seq]
        self.swapped.discard(seq)

    def swap_out(self, seq):
        """Release seq's blocks, keep its id and length; returns the old table."""
        self._resident(seq)
        table = self.tables[seq]
        self._release(table)
        self.tables[seq] = []
        self.swapped.add(seq)
        return list(table)

    def swap_in(self, seq):
        """Fresh blocks for a swapped-out seq; returns the new table."""
        self._need(seq)
        if seq not in self.swapped:
            raise PoolError("INVAL", f"sequence {seq} is not swapped out")
        want = -(-self.length[seq] // self.block_size)
        if want > len(self.free_list):
            raise PoolError("NOBLOCKS", f"need {want}, have {len(self.free_list)}")
        table = [self._take() for _ in range(want)]
        for blk in table:
            self.refcount[blk] = 1
        self.tables[seq] = table
        self.swapped.discard(seq)
        return list(table)

    # -- views -------------------------------------------------------------
    def block_table(self, seq):
        self._resident(seq)
        return list(self.tables[seq])

    def seq_len(self, seq):
        self._need(seq)
        return self.length[seq]

    def block_tables(self, seqs, max_blocks, pad=-1):
        """Rows of ``max_blocks`` entries (padding ``pad``) and lengths."""
        rows, lens = [], []
        for seq in seqs:
            t = self.block_table(seq)
            if len(t) > max_blocks:
                raise PoolError("INVAL", "table wider than max_blocks")
            rows.append(t + [pad] * (max_blocks - len(t)))
            lens.append(self.length[seq])
        return rows, lens

    def stats(self):
        used = sum(1 for c in self.refcount if c > 0)
        shared = sum(1 for c in self.refcount if c > 1)
        resident = [s for s in self.tables if s not in self.swapped]
        tokens = sum(self.length[s] for s in resident)
        waste = sum(len(self.tables[s]) * self.block_size - self.length[s] for s in resident)
        return {"free": len(self.free_list), "used": used, "shared": shared,
                "seqs": len(resident), "tokens": tokens, "waste_tokens": waste}
