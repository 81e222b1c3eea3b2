"""Pins of the prefix-cache pool model (CPU only).

Each scenario is small enough to work out by hand from the rules the model
states (block identity = salt + content path; lookups from the first block;
registration of full blocks; eviction from the front of the free list,
releases last to first).  Planted mistakes -- a key without the parent, a key
without the salt, releases in table order, no removal of a revived block from
the free list -- must each fail one of them.
"""
import pytest

from oracle.pool_model import PoolError
from oracle.prefix_cache import PrefixPoolModel

B = 4


def prompt(*blocks, tail=()):
    """Token ids: each block given as a base value v -> v, v+1, v+2, v+3."""
    out = []
    for v in blocks:
        out += [v, v + 1, v + 2, v + 3]
    return out + list(tail)


def test_shared_system_prompt_is_reused():
    m = PrefixPoolModel(16, B)
    c0, _ = m.alloc_prefix(0, prompt(10, 20, 30, tail=(7, 8)))     # 3 full blocks + 2 tokens
    assert c0 == 0
    assert m.prefix_stats()["registered"] == 3
    c1, _ = m.alloc_prefix(1, prompt(10, 20, 30, tail=(9,)))
    assert c1 == 3 * B
    assert m.tables[1][:3] == m.tables[0][:3]
    assert m.tables[1][3] != m.tables[0][3]                      # the partial block is private
    assert [m.refcount[b] for b in m.tables[0][:3]] == [2, 2, 2]
    assert m.prefix_stats()["hit_blocks"] == 3


def test_salt_keeps_tenants_apart():
    m = PrefixPoolModel(16, B)
    m.alloc_prefix(0, prompt(10, 20), salt=1)
    c, _ = m.alloc_prefix(1, prompt(10, 20), salt=2)
    assert c == 0
    c, _ = m.alloc_prefix(2, prompt(10, 20), salt=1)
    assert c == 2 * B


def test_identity_includes_the_parent():
    m = PrefixPoolModel(16, B)
    m.alloc_prefix(0, prompt(10, 20))
    c, _ = m.alloc_prefix(1, prompt(99, 20))   # same second block under another first block
    assert c == 0
    c, _ = m.alloc_prefix(2, prompt(10, 99))   # first block matches, second does not
    assert c == B


def test_whole_prompt_hit_and_revival_from_the_free_list():
    m = PrefixPoolModel(8, B)
    _, _ = m.alloc_prefix(0, prompt(10, 20))
    t = list(m.tables[0])
    m.free(0)
    # released last to first: the second block is ahead of the first
    assert list(m.free_list)[-2:] == [t[1], t[0]]
    assert m.prefix_stats()["cached_blocks"] == 2
    c, _ = m.alloc_prefix(1, prompt(10, 20))
    assert c == 2 * B and m.tables[1] == t
    assert t[0] not in m.free_list and t[1] not in m.free_list
    assert [m.refcount[b] for b in t] == [1, 1]


def test_eviction_takes_the_least_recently_released_deepest_first():
    m = PrefixPoolModel(4, B)
    m.alloc_prefix(0, prompt(10, 20))          # blocks 0, 1
    m.alloc_prefix(1, prompt(30, 40))          # blocks 2, 3
    m.free(0)                                  # free list: 1, 0
    m.free(1)                                  # free list: 1, 0, 3, 2
    assert list(m.free_list) == [1, 0, 3, 2]
    m.alloc(2, 4)                              # takes block 1: evicts (10, 20)'s second block
    assert m.prefix_stats()["evictions"] == 1
    c, _ = m.alloc_prefix(3, prompt(10, 20))   # first block still cached, second is not
    assert c == B
    assert m.tables[3][0] == 0


def test_growth_registers_a_filled_block_and_duplicates_are_not_registered():
    m = PrefixPoolModel(16, B)
    m.alloc_prefix(0, prompt(10, tail=(1, 2)))
    m.fork(0, 1)
    for tok in (3, 4):
        m.append_token(0, tok)
        m.append_token(1, tok)                 # copy-on-write on the first token, same contents after
    st = m.prefix_stats()
    assert st["registered"] == 2                # block (10..13) and one of the two (1, 2, 3, 4) blocks
    c, _ = m.alloc_prefix(2, prompt(10, tail=(1, 2, 3, 4)))
    assert c == 2 * B
    assert m.tables[2][1] == m.tables[0][1]    # the first to fill it holds the key


def test_plain_growth_stops_registration():
    m = PrefixPoolModel(16, B)
    m.alloc_prefix(0, prompt(10, tail=(1, 2, 3)))
    m.append(0)                                 # token id unknown
    assert m.prefix_stats()["registered"] == 1
    for tok in range(4):
        m.append_token(0, tok)
    assert m.prefix_stats()["registered"] == 1


def test_refusal_changes_nothing():
    m = PrefixPoolModel(4, B)
    m.alloc_prefix(0, prompt(10, 20))
    before = (list(m.free_list), list(m.refcount), m.prefix_stats())
    with pytest.raises(PoolError) as e:
        m.alloc_prefix(1, prompt(10, 50, 60, 70))   # 1 hit + 3 new blocks, only 2 free
    assert e.value.code == "NOBLOCKS"
    # the failed walk counted its lookups; nothing else moved
    after = (list(m.free_list), list(m.refcount), m.prefix_stats())
    assert after[0] == before[0] and after[1] == before[1]
    assert after[2]["cached_blocks"] == before[2]["cached_blocks"]


# -- planted mistakes ----------------------------------------------------------

def _run_all():
    for f in (test_shared_system_prompt_is_reused, test_salt_keeps_tenants_apart,
              test_identity_includes_the_parent, test_whole_prompt_hit_and_revival_from_the_free_list,
              test_eviction_takes_the_least_recently_released_deepest_first,
              test_growth_registers_a_filled_block_and_duplicates_are_not_registered,
              test_plain_growth_stops_registration):
        f()


@pytest.mark.parametrize("mutant", ["no_parent", "no_salt", "table_order_release", "no_revival"])
def test_planted_mistakes_fail_a_pin(mutant, monkeypatch):
    if mutant == "no_parent":
        # identity = salt + this block's tokens only
        def register(self, seq, i):
            table = self.tables[seq]
            path = (self.salt[seq], tuple(self.tokens[seq][i * B:(i + 1) * B]))
            if path not in self.cache:
                self.cache[path] = table[i]
                self.path_of[table[i]] = path
                self.counters["registered"] += 1

        def alloc_np(self, seq, tokens, salt=0):
            tokens = [int(t) for t in tokens]
            n = len(tokens)
            hits = []
            for i in range(n // B):
                blk = self.cache.get((salt, tuple(tokens[i * B:(i + 1) * B])))
                if blk is None:
                    break
                hits.append(blk)
            want = -(-n // B) - len(hits)
            for b in hits:
                if self.refcount[b] == 0:
                    self.free_list.remove(b)
                self.refcount[b] += 1
            table = list(hits)
            for _ in range(want):
                b = self._take()
                self.refcount[b] = 1
                table.append(b)
            self.tables[seq], self.length[seq] = table, n
            self.tokens[seq], self.salt[seq] = tokens, salt
            for i in range(len(hits), n // B):
                self._register(seq, i)
            return len(hits) * B, []
        monkeypatch.setattr(PrefixPoolModel, "_register", register)
        monkeypatch.setattr(PrefixPoolModel, "alloc_prefix", alloc_np)
    elif mutant == "no_salt":
        orig = PrefixPoolModel.alloc_prefix
        monkeypatch.setattr(PrefixPoolModel, "alloc_prefix", lambda self, seq, tokens, salt=0: orig(self, seq, tokens, 0))
    elif mutant == "table_order_release":
        def free(self, seq):
            for blk in self.tables.pop(seq):
                self.refcount[blk] -= 1
                if self.refcount[blk] == 0:
                    self.free_list.append(blk)
            del self.length[seq]
            self._untrack(seq)
        monkeypatch.setattr(PrefixPoolModel, "free", free)
    else:
        def alloc_nr(self, seq, tokens, salt=0, _orig=PrefixPoolModel.alloc_prefix):
            self.free_list = _NoRemove(self.free_list)
            return _orig(self, seq, tokens, salt)
        monkeypatch.setattr(PrefixPoolModel, "alloc_prefix", alloc_nr)
    with pytest.raises(AssertionError):
        _run_all()


class _NoRemove(list):
    """A free list that forgets to take revived blocks off (mutant)."""

    def __init__(self, dq):
        super().__init__(dq)

    def remove(self, b):
        pass

    def popleft(self):
        return self.pop(0)
