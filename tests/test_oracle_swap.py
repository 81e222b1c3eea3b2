"""Pins of the oracle's swap verbs and of the swap image (CPU only).

* The hand-derived trace in ``golden/swap_trace.txt``.  A request that
  shares blocks gives back only its own references. A request comes back in
  ceil(len / B) fresh blocks from the front of the free list. Refusals leave
  the pool unchanged, and a swapped-out request refuses growth, fork and
  table views.
* The host image ``[n][K, V][Hkv][B][d]`` against a closed form: every cache
  element is tagged with a number computed from its coordinates. Record i
  must then hold exactly the tags of block ``blocks[i]``, K before V.
* A whole preemption cycle on a shared-prefix workload. Swap out, overwrite
  the freed blocks, swap back in. Every sequence's cache rows must equal its
  logical token stream, which is rebuilt from the op log alone, and attention
  is unchanged bit for bit.
* Planted mistakes in copies of the model each fail one of the pins above.
"""
import os

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle.bits import NAN_BITS
from oracle.kv_store import KVStoreModel
from oracle.pool_model import BlockPoolModel, PoolError
from tests._replay import OracleRun, logical_streams

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "swap_trace.txt")


def _ints(text):
    return [int(x) for x in text.split()]


def run_trace(cls, path=GOLDEN):
    """Replays the trace on a ``cls`` pool; raises AssertionError at the
    first line whose expectation does not hold."""
    pool = None
    for raw in open(path, encoding="utf-8"):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        lhs, _, rhs = (part.strip() for part in line.partition("->"))
        words = lhs.split()
        verb = words[0]
        if verb == "pool":
            pool = cls(int(words[1]), int(words[2]))
            continue
        if verb == "free_list":
            assert list(pool.free_list) == _ints(rhs), line
            continue
        if verb == "refcount":
            assert pool.refcount[int(words[1])] == int(rhs), line
            continue
        if verb == "stats":
            want = dict(zip(rhs.split()[0::2], map(int, rhs.split()[1::2])))
            st = pool.stats()
            got = {"free": st["free"], "used": st["used"], "shared": st["shared"], "seqs": st["seqs"],
                   "tokens": st["tokens"], "waste": st["waste_tokens"]}
            assert got == want, line
            continue
        call = {
            "alloc": lambda: pool.alloc(words[1], int(words[2])),
            "fork": lambda: pool.fork(words[1], words[2]),
            "free": lambda: pool.free(words[1]),
            "append": lambda: pool.append(words[1])[0],
            "swap_out": lambda: pool.swap_out(words[1]),
            "swap_in": lambda: pool.swap_in(words[1]),
            "table": lambda: pool.block_table(words[1]),
            "len": lambda: pool.seq_len(words[1]),
        }[verb]
        if rhs.startswith("refused"):
            before = (list(pool.free_list), list(pool.refcount), {s: list(t) for s, t in pool.tables.items()},
                      dict(pool.length), set(pool.swapped))
            with pytest.raises(PoolError) as e:
                call()
            assert e.value.code == rhs.split()[1], line
            after = (list(pool.free_list), list(pool.refcount), {s: list(t) for s, t in pool.tables.items()},
                     dict(pool.length), set(pool.swapped))
            assert after == before, line
            continue
        got = call()
        if not rhs:
            continue
        if verb == "alloc":
            # alloc returns slots; the trace names the table
            got = pool.tables[words[1]]
        if isinstance(got, list):
            assert got == _ints(rhs), line
        else:
            assert got == int(rhs), line
    return True


def test_swap_trace():
    assert run_trace(BlockPoolModel)


def test_swap_refusals_in_every_state():
    pool = BlockPoolModel(8, 4)
    pool.alloc(0, 5)
    pool.swap_out(0)
    for code, call in [("INVAL", lambda: pool.swap_out(0)), ("INVAL", lambda: pool.append(0)),
                       ("INVAL", lambda: pool.fork(0, 1)), ("INVAL", lambda: pool.block_tables([0], 4)),
                       ("NOSEQ", lambda: pool.swap_out(9)), ("NOSEQ", lambda: pool.swap_in(9))]:
        before = (list(pool.free_list), list(pool.refcount), dict(pool.length))
        with pytest.raises(PoolError) as e:
            call()
        assert e.value.code == code
        assert (list(pool.free_list), list(pool.refcount), dict(pool.length)) == before
    pool.swap_in(0)
    with pytest.raises(PoolError) as e:
        pool.swap_in(0)                 # resident again
    assert e.value.code == "INVAL"


# -- the host image against a closed form ----------------------------------------

def tagged_store(nb, hkv, B, d):
    """A uint32 cache whose element (b, g, r, e) holds 1 + ((b*hkv + g)*B + r)*d + e
    in K and that plus 2^30 in V."""
    st = KVStoreModel(nb, hkv, B, d, "f32", poison=False)
    tag = 1 + np.arange(nb * hkv * B * d, dtype=np.uint32).reshape(nb, hkv, B, d)
    st.k[:] = tag
    st.v[:] = tag + np.uint32(2 ** 30)
    return st


@pytest.mark.parametrize("nb,hkv,B,d", [(10, 2, 4, 3), (16, 8, 16, 8), (7, 1, 8, 5)])
def test_swap_image_closed_form(nb, hkv, B, d):
    st = tagged_store(nb, hkv, B, d)
    blocks = [nb - 1, 0, 3, 3 % nb, 1]
    img = st.swap_image(blocks)
    assert img.shape == (len(blocks), 2, hkv, B, d)
    for i, b in enumerate(blocks):
        for kv in (0, 1):
            for g in range(hkv):
                for r in range(B):
                    for e in range(d):
                        want = 1 + ((b * hkv + g) * B + r) * d + e + kv * 2 ** 30
                        assert int(img[i, kv, g, r, e]) == want
    # restore into other blocks: exactly those blocks change, to the records
    dest = [2, 5, 6, 4, 8 % nb]
    dest = list(dict.fromkeys(dest))[:len(blocks)]
    fresh = tagged_store(nb, hkv, B, d)
    fresh.restore_image(dest, img[:len(dest)])
    for j in range(nb):
        if j in dest:
            i = dest.index(j)
            assert np.array_equal(fresh.k[j], st.k[blocks[i]]) and np.array_equal(fresh.v[j], st.v[blocks[i]])
        else:
            assert np.array_equal(fresh.k[j], st.k[j]) and np.array_equal(fresh.v[j], st.v[j])


def preemption_cycle(make_store=KVStoreModel, pool_cls=BlockPoolModel, share=True):
    """Swap a third of a shared-prefix batch out and back in (oracle side).

    Returns (workload, run, output before, output after, victims)."""
    lens = np.random.default_rng(5).integers(1, 60, size=12)
    wl = W.shared_prefix("swap_oracle", 3, 4, 37, lens, (4, 2, 16, 8, "bf16"), 160, 16, share=share)
    run = OracleRun(wl)
    run.pool.__class__ = pool_cls
    run.cache.__class__ = make_store
    tables, ctx = run.tables(wl)
    before = A.paged_decode(wl.q, run.cache.k, run.cache.v, tables, ctx, wl.block_size, wl.scale, wl.dtype,
                            wl.num_q_heads, wl.num_kv_heads)
    victims = [s for s in wl.batch if s % 3 == 1]
    images = {s: run.swap_out(s) for s in victims}
    # whatever reuses the freed blocks overwrites them
    for b in range(wl.num_blocks):
        if run.pool.refcount[b] == 0:
            run.cache.k[b] = NAN_BITS[wl.dtype]
            run.cache.v[b] = NAN_BITS[wl.dtype]
    for s in victims:
        run.swap_in(s, images[s][1])
    tables, ctx = run.tables(wl)
    after = A.paged_decode(wl.q, run.cache.k, run.cache.v, tables, ctx, wl.block_size, wl.scale, wl.dtype,
                           wl.num_q_heads, wl.num_kv_heads)
    return wl, run, before, after, victims


def cycle_pins_pass(make_store=KVStoreModel, pool_cls=BlockPoolModel):
    for share in (True, False):
        wl, run, before, after, victims = preemption_cycle(make_store, pool_cls, share)
        streams = logical_streams(wl)
        for s in wl.batch:
            k, v = run.cache.gather(run.pool.block_table(s), run.pool.seq_len(s))
            if not (np.array_equal(k, wl.k_rows[streams[s]]) and np.array_equal(v, wl.v_rows[streams[s]])):
                return False
        if not np.array_equal(before, after):
            return False
        # restored sequences hold private blocks
        if any(run.pool.refcount[b] != 1 for s in victims for b in run.pool.block_table(s)):
            return False
    return True


def test_preemption_cycle_restores_streams_and_attention():
    assert cycle_pins_pass()


# -- planted mistakes: each must fail a pin -------------------------------------

class _SwapInFromBack(BlockPoolModel):
    def swap_in(self, seq):
        self.free_list.reverse()
        try:
            return super().swap_in(seq)
        finally:
            self.free_list.reverse()


class _SwapOutDropsShared(BlockPoolModel):
    def swap_out(self, seq):
        self._resident(seq)
        table = self.tables[seq]
        for blk in table:               # wrong: ignores the other holders
            if self.refcount[blk] > 0:
                self.refcount[blk] = 0
                self.free_list.append(blk)
        self.tables[seq] = []
        self.swapped.add(seq)
        return list(table)


class _GrowthWhileSwapped(BlockPoolModel):
    def _resident(self, seq):
        self._need(seq)


class _SwapOutForgetsLength(BlockPoolModel):
    def swap_out(self, seq):
        table = super().swap_out(seq)
        self.length[seq] = 0
        return table


class _SwapInReusesOldTable(BlockPoolModel):
    def swap_out(self, seq):
        self._kept = getattr(self, "_kept", {})
        self._kept[seq] = list(self.tables[seq])
        return super().swap_out(seq)

    def swap_in(self, seq):
        self._need(seq)
        if seq not in self.swapped:
            raise PoolError("INVAL")
        table = self._kept.pop(seq)
        for blk in table:
            if blk in self.free_list:
                self.free_list.remove(blk)
            self.refcount[blk] += 1
        self.tables[seq] = table
        self.swapped.discard(seq)
        return list(table)


class _ImageVBeforeK(KVStoreModel):
    def swap_image(self, blocks):
        return super().swap_image(blocks)[:, ::-1].copy()


class _ImageHeadMajor(KVStoreModel):
    def swap_image(self, blocks):
        img = super().swap_image(blocks)
        return np.ascontiguousarray(img.transpose(0, 2, 1, 3, 4)).reshape(img.shape)


class _ImageBlocksReversed(KVStoreModel):
    def swap_image(self, blocks):
        return super().swap_image(list(blocks)[::-1])


def _trace_passes(cls):
    try:
        return run_trace(cls)
    except (AssertionError, PoolError, KeyError, IndexError, ValueError, pytest.fail.Exception):
        return False


@pytest.mark.parametrize("cls", [_SwapInFromBack, _SwapOutDropsShared, _GrowthWhileSwapped,
                                 _SwapOutForgetsLength, _SwapInReusesOldTable], ids=lambda c: c.__name__)
def test_planted_swap_verb_mistakes_are_caught(cls):
    assert _trace_passes(BlockPoolModel)
    assert not _trace_passes(cls)


def _image_pins_pass(store_cls):
    try:
        orig = globals()["KVStoreModel"]
        globals()["KVStoreModel"] = store_cls
        test_swap_image_closed_form(10, 2, 4, 3)
        return True
    except AssertionError:
        return False
    finally:
        globals()["KVStoreModel"] = orig


@pytest.mark.parametrize("cls", [_ImageVBeforeK, _ImageHeadMajor, _ImageBlocksReversed], ids=lambda c: c.__name__)
def test_planted_image_mistakes_are_caught(cls):
    assert _image_pins_pass(KVStoreModel)
    assert not _image_pins_pass(cls)


@pytest.mark.parametrize("store,pool", [(_ImageVBeforeK, BlockPoolModel), (_ImageBlocksReversed, BlockPoolModel),
                                        (KVStoreModel, _SwapInReusesOldTable)],
                         ids=["v_before_k", "blocks_reversed", "reuses_old_table"])
def test_planted_mistakes_break_the_preemption_cycle(store, pool):
    assert not cycle_pins_pass(store, pool)
