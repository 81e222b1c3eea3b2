"""Oracle pool model against the invariants and rules the pages fix.

Every rule is checked against something other than the model itself: the
logical token stream each sequence should hold (rebuilt from the op log with
no blocks at all), counting identities, and hand-derived small cases.
"""
import random

import numpy as np
import pytest

import workloads as W
from oracle.kv_store import KVStoreModel
from oracle.pool_model import BlockPoolModel, PoolError
from tests._replay import OracleRun, logical_streams


def check_invariants(pool):
    """Counting identities that hold after any sequence of operations.

    * total references = total table entries (each entry is one reference)
    * a block is free iff its count is zero; free and used are disjoint and
      together cover the pool ("Paged Attention", 量化: a block returns to the
      free list only at count zero)
    * a sequence wastes at most B - 1 slots, all in its last block
      ("Paged Attention", 定义 and 例子 / 例 2)
    """
    B = pool.block_size
    assert sum(pool.refcount) == sum(len(t) for t in pool.tables.values())
    free = set(pool.free_list)
    assert len(free) == len(pool.free_list)
    used = {b for b in range(pool.num_blocks) if pool.refcount[b] > 0}
    assert free.isdisjoint(used) and len(free) + len(used) == pool.num_blocks
    assert all(pool.refcount[b] == 0 for b in free)
    for seq, table in pool.tables.items():
        n = pool.length[seq]
        assert len(table) == -(-n // B)
        assert len(table) * B - n <= B - 1
        assert len(set(table)) == len(table)


def snapshot(pool):
    return (list(pool.free_list), list(pool.refcount),
            {s: list(t) for s, t in pool.tables.items()}, dict(pool.length))


def test_exhaustion_is_all_or_nothing():
    pool = BlockPoolModel(4, 4)
    pool.alloc(0, 9)                     # 3 blocks
    before = snapshot(pool)
    with pytest.raises(PoolError) as e:
        pool.alloc(1, 5)                 # needs 2, 1 free
    assert e.value.code == "NOBLOCKS" and snapshot(pool) == before
    pool.alloc(1, 4)                     # exactly the last block
    for _ in range(3):
        pool.append(0)                   # fills block 2 of seq 0 (slots 9..11)
    before = snapshot(pool)
    with pytest.raises(PoolError) as e:
        pool.append(0)                   # block full, pool empty
    assert e.value.code == "NOBLOCKS" and snapshot(pool) == before
    pool.fork(1, 2)                      # seq 1's block is full: shared, no copy needed
    with pytest.raises(PoolError) as e:
        pool.append(2)                   # needs a fresh block: none
    assert e.value.code == "NOBLOCKS"


def test_cow_copies_only_still_shared_partial_blocks():
    # "vllm-pagedattention", 一块内存，如何安全地属于多条序列: writing into a
    # still-shared last block copies it; full blocks stay shared.
    pool = BlockPoolModel(16, 4)
    pool.alloc("p", 6)                   # blocks [0, 1]; block 1 holds 2 tokens
    for c in ("b1", "b2", "b3"):
        pool.fork("p", c)
    assert pool.refcount[0] == 4 and pool.refcount[1] == 4
    pairs = []
    for s in ("p", "b1", "b2", "b3"):
        slot, cow = pool.append(s)
        pairs.append(cow)
    assert pairs == [(1, 2), (1, 3), (1, 4), None]
    assert pool.block_table("b3") == [0, 1]          # last writer keeps the original
    assert [pool.block_table(s)[1] for s in ("p", "b1", "b2")] == [2, 3, 4]
    assert pool.refcount[0] == 4 and pool.refcount[1] == 1
    check_invariants(pool)
    # block-aligned fork: the next token opens a new block, nothing is copied
    pool2 = BlockPoolModel(16, 4)
    pool2.alloc("p", 8)
    pool2.fork("p", "c")
    assert pool2.append("p")[1] is None and pool2.append("c")[1] is None
    assert pool2.refcount[0] == 2 and pool2.refcount[1] == 2
    check_invariants(pool2)


def test_free_returns_at_zero_refcount_in_table_order():
    pool = BlockPoolModel(8, 2)
    pool.alloc("a", 5)                   # [0, 1, 2]
    pool.fork("a", "b")
    pool.free("a")
    assert list(pool.free_list) == [3, 4, 5, 6, 7]   # still held by b
    pool.free("b")
    assert list(pool.free_list) == [3, 4, 5, 6, 7, 0, 1, 2]
    check_invariants(pool)


@pytest.mark.parametrize("code,call", [
    ("NOSEQ", lambda p: p.append(99)), ("NOSEQ", lambda p: p.free(99)),
    ("NOSEQ", lambda p: p.fork(99, 100)), ("EXISTS", lambda p: p.alloc(0, 1)),
    ("EXISTS", lambda p: p.fork(0, 0)), ("INVAL", lambda p: p.alloc(5, -1)),
])
def test_refusals_change_nothing(code, call):
    pool = BlockPoolModel(8, 4)
    pool.alloc(0, 3)
    before = snapshot(pool)
    with pytest.raises(PoolError) as e:
        call(pool)
    assert e.value.code == code and snapshot(pool) == before


def random_op(rng, live, nxt, B):
    """One random op over the live sequences (the pool may refuse it)."""
    r = rng.random()
    if r < 0.25 or not live:
        return ("alloc", nxt, rng.randint(0, 3 * B))
    if r < 0.65:
        return ("append", rng.choice(live))
    if r < 0.8:
        return ("fork", rng.choice(live), nxt)
    return ("free", rng.choice(live))


@pytest.mark.parametrize("seed", range(20))
def test_random_logs_keep_invariants_and_contents(seed):
    """Fuzz: invariants after every op, and every sequence's cache rows equal
    its logical token stream (tokens are tagged with unique values)."""
    rng = random.Random(seed)
    B = rng.choice([1, 2, 4, 8])
    nb = rng.randint(4, 24)
    order = list(range(nb))
    rng.shuffle(order)
    pool = BlockPoolModel(nb, B, order)
    cache = KVStoreModel(nb, 1, B, 1, "f32", poison=False)
    stream = {}
    tag = 1
    nxt = 0
    for _ in range(120):
        op = random_op(rng, sorted(stream), nxt, B)
        nxt += op[0] in ("alloc", "fork")
        before = snapshot(pool)
        try:
            if op[0] == "alloc":
                slots = pool.alloc(op[1], op[2])
                vals = np.arange(tag, tag + op[2], dtype=np.uint32).reshape(-1, 1, 1)
                tag += op[2]
                cache.write(slots, vals, vals)
                stream[op[1]] = list(vals.ravel())
            elif op[0] == "append":
                slot, cow = pool.append(op[1])
                if cow is not None:
                    cache.copy([cow])
                val = np.full((1, 1, 1), tag, dtype=np.uint32)
                tag += 1
                cache.write([slot], val, val)
                stream[op[1]].append(tag - 1)
            elif op[0] == "fork":
                pool.fork(op[1], op[2])
                stream[op[2]] = list(stream[op[1]])
            else:
                pool.free(op[1])
                del stream[op[1]]
        except PoolError as e:
            assert e.code == "NOBLOCKS" and snapshot(pool) == before
            if op[0] in ("alloc", "fork"):
                continue
        check_invariants(pool)
        for seq, want in stream.items():
            if seq not in pool.tables:
                continue
            k, v = cache.gather(pool.block_table(seq), pool.seq_len(seq))
            assert list(k.ravel()) == want and list(v.ravel()) == want


@pytest.mark.parametrize("make", [W.CONFIGS["tiny"],
                                  lambda: W.shared_prefix("mini_gqa", 2, 3, 40, [5, 17, 30, 3, 9, 16],
                                                          (4, 2, 16, 8, "bf16"), 64, 16),
                                  lambda: W.beam_fork("mini_beam", 2, 4, 37, (2, 2, 8, 8, "f16"), 64, 8)])
def test_workload_cache_reproduces_logical_streams(make):
    wl = make()
    run = OracleRun(wl)
    streams = logical_streams(wl)
    for s in wl.batch:
        table = run.pool.block_table(s)
        k, v = run.cache.gather(table, run.pool.seq_len(s))
        assert np.array_equal(k, wl.k_rows[streams[s]])
        assert np.array_equal(v, wl.v_rows[streams[s]])
    check_invariants(run.pool)


def test_beam_workload_copy_count():
    # 8 parents x 4 beams with a 4095-token prompt (partial last block): three
    # copies per parent; narrow rows keep the CPU cost small
    wl = W.beam_fork("beam_narrow", 8, 4, 4095, (1, 1, 8, 16, "f16"),
                     num_blocks=16384, max_blocks=256)
    run = OracleRun(wl)
    assert len(run.cow) == 24
    st = run.pool.stats()
    assert st["shared"] == 8 * 255          # full prompt blocks stay shared


# -- planted mistakes in a copy of the pool model: each must be caught ----------

def _pool_pins_pass(cls):
    """Allocator demo trace, copy-on-write scenario and content fuzz with ``cls``."""
    import tests.test_oracle_pins as pins
    saved = pins.BlockPoolModel, globals()["BlockPoolModel"]
    pins.BlockPoolModel = cls
    globals()["BlockPoolModel"] = cls
    try:
        pins.test_allocator_demo_trace()
        test_cow_copies_only_still_shared_partial_blocks()
        test_free_returns_at_zero_refcount_in_table_order()
        for seed in range(8):
            test_random_logs_keep_invariants_and_contents(seed)
        return True
    except (AssertionError, PoolError, KeyError, IndexError):
        return False
    finally:
        pins.BlockPoolModel, globals()["BlockPoolModel"] = saved


class _TakeFromBack(BlockPoolModel):
    def alloc(self, seq, n_tokens):
        self.free_list.reverse()
        try:
            return super().alloc(seq, n_tokens)
        finally:
            self.free_list.reverse()


class _ReturnToFront(BlockPoolModel):
    def free(self, seq):
        self._need(seq)
        for blk in self.tables.pop(seq):
            self.refcount[blk] -= 1
            if self.refcount[blk] == 0:
                self.free_list.appendleft(blk)
        del self.length[seq]


class _NoCopyOnWrite(BlockPoolModel):
    def append(self, seq):
        self._need(seq)
        table, pos = self.tables[seq], self.length[seq]
        if pos % self.block_size == 0:
            if not self.free_list:
                raise PoolError("NOBLOCKS")
            blk = self.free_list.popleft()
            self.refcount[blk] = 1
            table.append(blk)
        self.length[seq] = pos + 1
        return self._slot(seq, pos), None


class _ForkWithoutRefcount(BlockPoolModel):
    def fork(self, parent, child):
        self._need(parent)
        if child in self.tables:
            raise PoolError("EXISTS")
        self.tables[child] = list(self.tables[parent])
        self.length[child] = self.length[parent]


@pytest.mark.parametrize("cls", [_TakeFromBack, _ReturnToFront, _NoCopyOnWrite,
                                 _ForkWithoutRefcount], ids=lambda c: c.__name__)
def test_planted_pool_mistakes_are_caught(cls):
    assert _pool_pins_pass(BlockPoolModel)
    assert not _pool_pins_pass(cls)
