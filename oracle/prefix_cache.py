"""Block pool with a prefix cache: content-addressed full blocks (test infrastructure).

Test infrastructure only: the parity tests replay one operation log through
this model and through the native pool and compare tables, slots, cached
token counts, copy pairs, the free list and every counter.

What the pages say.  Automatic prefix caching turns "blocks can be shared"
into "blocks can be found": a full KV block is identified by the hash of its
parent block, the block's own tokens and extra inputs such as a cache salt,
and a new request that hits an identical prefix reuses that KV and skips
the prefill of those tokens ("vllm-pagedattention" (chenyuan1125.github.io),
the passage after 一块内存，如何安全地属于多条序列).  Which cached blocks are worth
keeping is an eviction question, and prefixes of different tenants must be
kept apart by the salt (same page, closing remarks).

The model, written from that description:

* The identity of a full block is its whole content path: the salt and every
  token from the start of the sequence to the end of the block.  A hash of
  (parent identity, block tokens, salt) names exactly this path, so the
  model keys a plain dict by the tuple itself (no hash, no collisions).
* Admission with a prompt walks its full blocks from the first; every block
  found is reused (reference count + 1), the walk stops at the first block
  not found, and the remaining tokens take fresh blocks as in the plain pool.
* A block becomes findable (is registered) when it is full: at admission for
  the prompt's full blocks, or when growth token by token fills it.  It is
  registered only if its parent block is registered (or it is the first
  block) and no block holds its content path yet.
* A registered block whose count reaches zero stays in the cache and goes to
  the back of the free list like any released block; allocation takes from
  the front, and a cached block taken there is evicted (forgotten): the
  least recently released cached block goes first.  A hit on a free cached
  block takes it back off the free list.
* With the cache on, a released sequence gives back its blocks last to
  first, so a block's descendants are released (and evicted) before it.

Readings where the pages are silent: the eviction order is
least-recently-released; an admission's hit may cover the whole prompt;
plain admission and growth without token ids leave the sequence's later
blocks unregistered.
"""
from .pool_model import BlockPoolModel, PoolError


class PrefixPoolModel(BlockPoolModel):
    def __init__(self, num_blocks, block_size, initial_free_order=None):
        super().__init__(num_blocks, block_size, initial_free_order)
        self.cache = {}        # content path (salt, tokens...) -> block
        self.path_of = {}      # registered block -> its content path
        self.tokens = {}       # tracked seq -> its token ids so far
        self.salt = {}         # tracked seq -> salt
        self.counters = {"lookups": 0, "hit_blocks": 0, "registered": 0, "evictions": 0}

    # -- the free list, with eviction ---------------------------------------
    def _take(self):
        blk = self.free_list.popleft()
        if blk in self.path_of:
            del self.cache[self.path_of.pop(blk)]
            self.counters["evictions"] += 1
        return blk

    def _register(self, seq, i):
        """Register block i of seq (full) when its parent is registered and
        its content path is new."""
        table = self.tables[seq]
        if i > 0 and table[i - 1] not in self.path_of:
            return
        B = self.block_size
        path = (self.salt[seq], tuple(self.tokens[seq][:(i + 1) * B]))
        if path in self.cache:
            return
        self.cache[path] = table[i]
        self.path_of[table[i]] = path
        self.counters["registered"] += 1

    def _untrack(self, seq):
        self.tokens.pop(seq, None)
        self.salt.pop(seq, None)

    # -- verbs ---------------------------------------------------------------
    def alloc_prefix(self, seq, tokens, salt=0):
        """Admit seq with its prompt token ids; returns (cached tokens, slots)."""
        tokens = [int(t) for t in tokens]
        if seq in self.tables:
            raise PoolError("EXISTS", f"sequence {seq} exists")
        B = self.block_size
        n = len(tokens)
        hits = []
        for i in range(n // B):
            self.counters["lookups"] += 1
            blk = self.cache.get((salt, tuple(tokens[:(i + 1) * B])))
            if blk is None:
                break
            hits.append(blk)
        want = -(-n // B) - len(hits)
        revive = sum(1 for b in hits if self.refcount[b] == 0)
        if want > len(self.free_list) - revive:
            raise PoolError("NOBLOCKS", f"need {want}, have {len(self.free_list) - revive}")
        for b in hits:
            if self.refcount[b] == 0:
                self.free_list.remove(b)
            self.refcount[b] += 1
        table = list(hits)
        for _ in range(want):
            b = self._take()
            self.refcount[b] = 1
            table.append(b)
        self.tables[seq] = table
        self.length[seq] = n
        self.tokens[seq] = tokens
        self.salt[seq] = salt
        for i in range(len(hits), n // B):
            self._register(seq, i)
        self.counters["hit_blocks"] += len(hits)
        return len(hits) * B, [self._slot(seq, i) for i in range(n)]

    def append_token(self, seq, token):
        """Growth by one token whose id is known: (slot, cow pair or None)."""
        self._resident(seq)
        tracked = seq in self.tokens
        slot, cow = BlockPoolModel.append(self, seq)
        if tracked:
            self.tokens[seq].append(int(token))
            if self.length[seq] % self.block_size == 0:
                self._register(seq, len(self.tables[seq]) - 1)
        return slot, cow

    def append(self, seq):
        slot_cow = super().append(seq)
        self._untrack(seq)
        return slot_cow

    def alloc(self, seq, n_tokens):
        return super().alloc(seq, n_tokens)

    def fork(self, parent, child):
        super().fork(parent, child)
        if parent in self.tokens:
            self.tokens[child] = list(self.tokens[parent])
            self.salt[child] = self.salt[parent]

    def _release(self, table):
        """With the cache on, blocks go back last to first."""
        super()._release(list(reversed(table)))

    def free(self, seq):
        super().free(seq)
        self._untrack(seq)

    def swap_out(self, seq):
        table = super().swap_out(seq)
        self._untrack(seq)           # blocks restored by swap-in are not registered
        return table

    # -- views ---------------------------------------------------------------
    def prefix_stats(self):
        return dict(self.counters, cached_blocks=len(self.cache))

    def block_cached(self, blk):
        return 1 if blk in self.path_of else 0
