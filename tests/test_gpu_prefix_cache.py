"""Prefix caching end to end on the GPU, against the oracle.

Requests that share a system prompt are admitted through
pa_seq_alloc_prefix (native pool) and PrefixPoolModel (oracle) from the same
free order.  Both must report the same cached token count, slots and tables.
Only the uncached tokens' K/V rows are then written (pa_write_kv on the
device, KVStoreModel.write in the oracle); a cached block keeps the rows the
request that first computed it wrote.  A token's K/V row is a function of
the salt and the prompt up to that token, as for a real model, so a correct
hit finds exactly the rows the request would have computed.

pa_prefill then runs each request's uncached rows over its whole context
(a whole-prompt hit runs its last row), reading the shared blocks through
the table.  A decode step follows (append_token on both pools, the new rows
written, pa_decode).  Both are checked against the float64 oracle
(oracle.prefill / oracle.attention over the model's tables and the oracle
cache).  The device cache bytes must equal the oracle's after every phase.
Freed requests leave their blocks cached; a later admission revives them
from the free list, and the test checks their rows are intact.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_147_amd as P
from oracle import attention as A
from oracle import prefill as PF
from oracle.kv_store import KVStoreModel
from oracle.prefix_cache import PrefixPoolModel
from tests._native import device_tensor
from tests._tol import assert_close
from workloads.synth import normal_bits

pytestmark = pytest.mark.gpu

B, HQ, HKV, D, DT = 16, 8, 2, 128, "bf16"
NB = 192


class Rows:
    """K/V row of each (salt, prompt prefix): the same prefix always gets the
    same row, drawn once from a seeded stream in order of first use."""

    def __init__(self, seed):
        self.rng = np.random.default_rng(seed)
        self.index = {}
        self.k, self.v = [], []

    def of(self, salt, tokens, i):
        key = (salt, tuple(tokens[:i + 1]))
        if key not in self.index:
            self.index[key] = len(self.k)
            self.k.append(normal_bits(self.rng, (HKV, D), DT))
            self.v.append(normal_bits(self.rng, (HKV, D), DT))
        j = self.index[key]
        return self.k[j], self.v[j]


class Both:
    """Native pool + device caches and model pool + oracle cache, driven together."""

    def __init__(self, seed):
        order = np.random.default_rng(seed).permutation(NB).astype(np.int32)
        self.native = P.BlockPool(NB, B, order)
        self.native.enable_prefix_cache()
        self.model = PrefixPoolModel(NB, B, order)
        self.store = KVStoreModel(NB, HKV, B, D, DT)
        self.kc = device_tensor(self.store.k, DT, "cuda")      # the same NaN poison
        self.vc = device_tensor(self.store.v, DT, "cuda")
        self.rows = Rows(seed + 1)
        self.prompt = {}

    def write(self, salt, tokens, positions, slots):
        if not positions:
            return
        k = np.stack([self.rows.of(salt, tokens, i)[0] for i in positions])
        v = np.stack([self.rows.of(salt, tokens, i)[1] for i in positions])
        self.store.write(slots, k, v)
        P.pa_write_kv(self.kc, self.vc, device_tensor(k, DT, "cuda"), device_tensor(v, DT, "cuda"),
                      torch.tensor(list(slots), dtype=torch.int64, device="cuda"))

    def admit(self, seq, tokens, salt):
        cached, slots = self.native.alloc_prefix(seq, tokens, salt)
        c_m, s_m = self.model.alloc_prefix(seq, tokens, salt)
        assert cached == c_m and list(slots) == s_m, seq
        self.prompt[seq] = (salt, list(tokens))
        n = len(tokens)
        self.write(salt, tokens, list(range(cached, n)), slots[cached:])
        return cached

    def grow(self, seq, token):
        salt, toks = self.prompt[seq]
        slot, cow = self.native.append_token(seq, token)
        assert (slot, cow) == self.model.append_token(seq, token)
        toks.append(int(token))
        self.write(salt, toks, [len(toks) - 1], [slot])

    def free(self, seq):
        self.native.free(seq)
        self.model.free(seq)
        del self.prompt[seq]

    def check_state(self, seqs):
        torch.cuda.synchronize()
        mb = max(-(-len(self.prompt[s][1]) // B) for s in seqs)
        tn, cn = self.native.block_tables(seqs, mb)
        tm, cm = self.model.block_tables(seqs, mb)
        assert np.array_equal(tn, np.asarray(tm)) and list(cn) == list(cm)
        assert list(self.native.free_list()) == list(self.model.free_list)
        assert self.native.prefix_stats() == self.model.prefix_stats()
        kd = self.kc.view(torch.int16).cpu().numpy().view(np.uint16)
        vd = self.vc.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(kd, self.store.k) and np.array_equal(vd, self.store.v)
        # every request's cache rows are the rows of its own prefix
        for s in seqs:
            salt, toks = self.prompt[s]
            k, v = self.store.gather(self.model.block_table(s), len(toks))
            want = [self.rows.of(salt, toks, i) for i in range(len(toks))]
            assert np.array_equal(k, np.stack([w[0] for w in want]))
            assert np.array_equal(v, np.stack([w[1] for w in want]))
        return np.asarray(tm, dtype=np.int32), np.asarray(cm, dtype=np.int32)


def prefill_and_check(both, seqs, cached, seed):
    tables, ctx = both.check_state(seqs)
    # rows to run: the uncached tokens, or the last one for a whole-prompt hit
    n_rows = [max(int(c) - cached[s], 1) for s, c in zip(seqs, ctx)]
    q_start = np.concatenate([[0], np.cumsum(n_rows)]).astype(np.int32)
    q = normal_bits(np.random.default_rng(seed), (int(q_start[-1]), HQ, D), DT)
    out = torch.empty((int(q_start[-1]), HQ, D), dtype=torch.float32, device="cuda")
    scale = 1 / np.sqrt(D)
    P.pa_prefill(out, device_tensor(q, DT, "cuda"), both.kc, both.vc, torch.from_numpy(tables).cuda(),
                 torch.from_numpy(ctx).cuda(), torch.from_numpy(q_start).cuda(), scale, max(n_rows))
    want = PF.paged_prefill(q, both.store.k, both.store.v, tables, ctx, q_start, B, scale, DT, HQ, HKV)
    assert_close(out.cpu().numpy(), want, DT, "prefill through cached blocks")


def decode_and_check(both, seqs, seed):
    rng = np.random.default_rng(seed)
    for s in seqs:
        both.grow(s, int(rng.integers(0, 1000)))
    tables, ctx = both.check_state(seqs)
    q = normal_bits(rng, (len(seqs), HQ, D), DT)
    out = torch.empty((len(seqs), HQ, D), dtype=torch.float32, device="cuda")
    scale = 1 / np.sqrt(D)
    P.pa_decode(out, device_tensor(q, DT, "cuda"), both.kc, both.vc, torch.from_numpy(tables).cuda(),
                torch.from_numpy(ctx).cuda(), scale)
    want = A.paged_decode(q, both.store.k, both.store.v, tables, ctx, B, scale, DT, HQ, HKV)
    assert_close(out.cpu().numpy(), want, DT, "decode through cached blocks")


def test_prefix_cache_end_to_end():
    both = Both(seed=21)
    rng = np.random.default_rng(22)
    system = [int(t) for t in rng.integers(0, 1000, size=100)]          # 6 full blocks + 4 tokens
    private = lambda n: [int(t) for t in rng.integers(1000, 2000, size=n)]
    prompts = {0: (7, system + private(37)),
               1: (7, system + private(50)),          # hits the 6 system blocks
               2: (7, system[:64] + private(20)),     # hits 4 blocks
               3: (9, system + private(30)),          # another salt: no hit
               4: (7, system[:96])}                   # the whole prompt is cached
    cached = {}
    for s, (salt, toks) in prompts.items():
        cached[s] = both.admit(s, toks, salt)
        print(f"[prefix] request {s}: {len(toks)} tokens, {cached[s]} cached", flush=True)
    assert [cached[s] for s in range(5)] == [0, 96, 64, 0, 96]
    seqs = list(prompts)
    prefill_and_check(both, seqs, cached, seed=23)
    decode_and_check(both, seqs, seed=24)
    # requests 0 and 1 finish: their private full blocks go to the free list
    # but stay cached (the system blocks are still held by request 4); a new
    # request with request 0's first 128 tokens revives two of them
    both.free(0)
    both.free(1)
    revived = both.model.tables[4][:6]
    salt, toks = 7, prompts[0][1][:128] + private(17)
    free_before = list(both.model.free_list)
    cached[5] = both.admit(5, toks, salt)
    assert cached[5] == 128
    t5 = both.model.tables[5]
    assert t5[:6] == revived and all(b in free_before for b in t5[6:8])
    seqs = [2, 3, 4, 5]
    prefill_and_check(both, seqs, cached, seed=25)
    decode_and_check(both, seqs, seed=26)
