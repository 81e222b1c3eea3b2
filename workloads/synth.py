"""Seeded synthetic workloads for paged decode attention.

This module only draws inputs: sequence lengths, a shuffled physical free
order, query rows and the K/V rows of every token the workload writes, and
it lists the pool operations (admit, grow, fork, release) in the order a
serving loop would issue them.  It holds none of the method's arithmetic:
no block counts, slots, tables, copies or attention.  Both sides of the
parity check -- the CPU oracle and the native library -- consume what it
returns and compute everything else on their own.

Values are drawn as float32 N(0, 1) and rounded once, round-to-nearest-even,
to the workload's element type; both sides receive those same bits.  Every
tensor has its own child of ``numpy.random.SeedSequence(seed)``, spawned in
the fixed order of ``_STREAMS``, so a tensor's values do not depend on the
sizes of the others (the block-size sweep draws identical Q/K/V for every B).

Operation log entries (tuples):
    ("alloc",  seq, n, row0)   admit seq with n prompt tokens; their K/V are
                               rows row0 .. row0+n-1 of k_rows / v_rows
    ("append", seq, n, row0)   n single-token growth steps, rows row0..
    ("fork",   parent, child)  child shares parent's cached tokens
    ("free",   seq)            release seq
"""
from dataclasses import dataclass, field

import numpy as np
import torch

_STREAMS = ("lengths", "free_order", "q", "k", "v", "q_rows")

_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
_BITS = {"f32": (torch.int32, np.uint32), "f16": (torch.int16, np.uint16),
         "bf16": (torch.int16, np.uint16)}


def _streams(seed):
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.default_rng(k) for name, k in zip(_STREAMS, kids)}


def normal_bits(rng, shape, dtype):
    """float32 N(0,1) draws rounded (RNE) to ``dtype``; returns raw bits."""
    x = torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32))
    tbits, nbits = _BITS[dtype]
    return x.to(_TORCH[dtype]).view(tbits).numpy().view(nbits)


@dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                    # "f32" | "f16" | "bf16"
    num_blocks: int               # physical pool size
    max_blocks: int               # block-table width
    scale: float
    free_order: np.ndarray        # initial free list, a permutation
    setup_ops: list               # ops that build the cache before the step
    step_ops: list                # the decode step's own growth ops
    batch: list                   # seq ids decoded, in batch order
    q: np.ndarray                 # [S][Hq][d] raw bits
    k_rows: np.ndarray            # [T][Hkv][d] raw bits, log order
    v_rows: np.ndarray
    info: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return len(self.batch)

    def ops(self):
        return list(self.setup_ops) + list(self.step_ops)


class _Log:
    """Accumulates ops and hands out row ranges of the K/V row arrays."""

    def __init__(self):
        self.setup, self.step, self.rows = [], [], 0

    def take(self, n):
        r0 = self.rows
        self.rows += n
        return r0


def _finish(name, log, batch, shape, streams, num_blocks, max_blocks, info):
    Hq, Hkv, d, B, dtype = shape
    rs = streams
    free_order = rs["free_order"].permutation(num_blocks).astype(np.int32)
    q = normal_bits(rs["q"], (len(batch), Hq, d), dtype)
    k_rows = normal_bits(rs["k"], (log.rows, Hkv, d), dtype)
    v_rows = normal_bits(rs["v"], (log.rows, Hkv, d), dtype)
    return Workload(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                    block_size=B, dtype=dtype, num_blocks=num_blocks,
                    max_blocks=max_blocks, scale=1.0 / float(np.sqrt(d)),
                    free_order=free_order, setup_ops=log.setup, step_ops=log.step,
                    batch=list(batch), q=q, k_rows=k_rows, v_rows=v_rows, info=info)


def independent(name, ctx_lens, shape, num_blocks, max_blocks, seed=0, info=None):
    """Sequences with their own prompts of ctx-1 tokens, then one decode step.

    Each sequence is admitted with ctx-1 prompt tokens (sequences in index
    order), then the step grows every sequence by its new token.
    """
    log = _Log()
    for s, c in enumerate(ctx_lens):
        log.setup.append(("alloc", s, int(c) - 1, log.take(int(c) - 1)))
    for s in range(len(ctx_lens)):
        log.step.append(("append", s, 1, log.take(1)))
    return _finish(name, log, range(len(ctx_lens)), shape, _streams(seed),
                   num_blocks, max_blocks, dict(info or {}, ctx=list(map(int, ctx_lens))))


def shared_prefix(name, groups, group_size, prefix, suffix_lens, shape, num_blocks,
                  max_blocks, share=True, seed=0, info=None):
    """Groups of sequences behind one common prompt prefix.

    Per group: the first member is admitted with ``prefix`` tokens; with
    ``share`` the others are forked from it, without ``share`` each admits
    its own copy of the same prefix rows.  Member j then grows by
    suffix_lens[j] - 1 tokens in setup and by its new token in the step.
    """
    log = _Log()
    batch = []
    prefix_rows = []
    for gi in range(groups):
        base = gi * group_size
        r0 = log.take(prefix)
        prefix_rows.append(r0)
        log.setup.append(("alloc", base, prefix, r0))
        for j in range(1, group_size):
            if share:
                log.setup.append(("fork", base, base + j))
            else:
                log.setup.append(("alloc", base + j, prefix, r0))
        batch.extend(range(base, base + group_size))
    suffix_lens = np.asarray(suffix_lens)
    for s in batch:
        n = int(suffix_lens[s]) - 1
        if n > 0:
            log.setup.append(("append", s, n, log.take(n)))
    for s in batch:
        log.step.append(("append", s, 1, log.take(1)))
    ctx = [prefix + int(x) for x in suffix_lens]
    return _finish(name, log, batch, shape, _streams(seed), num_blocks, max_blocks,
                   dict(info or {}, ctx=ctx, prefix=prefix, group_size=group_size,
                        share=share))


def beam_fork(name, parents, beams, prompt, shape, num_blocks, max_blocks, seed=0,
              info=None):
    """Each parent (prompt tokens) forks into ``beams`` beams that each write.

    Setup admits every parent and forks beams-1 children from it; the step
    grows beam 0, 1, ... of each parent in order by one token each, so every
    beam but the last one to write lands in a still-shared last block.
    """
    log = _Log()
    batch = []
    for p in range(parents):
        base = p * beams
        log.setup.append(("alloc", base, prompt, log.take(prompt)))
        for j in range(1, beams):
            log.setup.append(("fork", base, base + j))
        batch.extend(range(base, base + beams))
    for s in batch:
        log.step.append(("append", s, 1, log.take(1)))
    return _finish(name, log, batch, shape, _streams(seed), num_blocks, max_blocks,
                   dict(info or {}, ctx=[prompt + 1] * len(batch)))


# -- the five workloads -------------------------------------------------------

def tiny(seed=0):
    """4 sequences, ctx {7,19,33,64}, B=16, 8/8 heads, d=64, fp32, 32 blocks."""
    return independent("tiny_mha_f32", [7, 19, 33, 64], (8, 8, 64, 16, "f32"),
                       num_blocks=32, max_blocks=64 // 16, seed=seed)


def llama7b_mha(seed=0, batch=64):
    """Llama-7B-like layer: 32/32 heads, d=128, fp16, B=16, ctx U[128, 2048]."""
    rs = _streams(seed)
    ctx = rs["lengths"].integers(128, 2048, size=batch, endpoint=True)
    return independent("llama7b_mha_f16", ctx, (32, 32, 128, 16, "f16"),
                       num_blocks=8192, max_blocks=2048 // 16, seed=seed)


GQA_PREFIX = 1008            # shared system prompt, 63 blocks of 16
GQA_CAP = 8192
GQA_SIGMA = 1.0
GQA_MEAN = 512.0


def gqa_suffix_lengths(seed, batch):
    """Private lengths after the shared prefix: lognormal with mean 512.

    x = clip(rint(exp(mu + sigma Z)), 1, cap - prefix) with sigma = 1 and
    mu = ln(512) - sigma^2 / 2, so that E[exp(mu + sigma Z)] = 512.
    """
    rs = _streams(seed)
    mu = np.log(GQA_MEAN) - GQA_SIGMA ** 2 / 2
    z = rs["lengths"].standard_normal(batch)
    x = np.rint(np.exp(mu + GQA_SIGMA * z))
    return np.clip(x, 1, GQA_CAP - GQA_PREFIX).astype(np.int64)


def llama31_8b_gqa(seed=0, share=True, groups=32, group_size=8):
    """Llama-3.1-8B-like layer: 32/8 heads, d=128, bf16, B=16, batch 256.

    Groups of 8 sequences share a 1008-token prefix (forked, refcounted);
    ``share=False`` gives every sequence a private copy of the same bytes.
    """
    suffix = gqa_suffix_lengths(seed, groups * group_size)
    name = "llama31_8b_gqa_bf16" + ("" if share else "_noshare")
    return shared_prefix(name, groups, group_size, GQA_PREFIX, suffix,
                         (32, 8, 128, 16, "bf16"), num_blocks=32768,
                         max_blocks=GQA_CAP // 16, share=share, seed=seed)


SWEEP_CAP = 1024


def block_sweep(block_size, seed=0, batch=128, ctx=1000):
    """ctx 1000 x 128 sequences, 32/8 heads, d=128, bf16, B in {8, 16, 32}.

    The pool holds twice the table capacity (2 * batch * 1024 / B blocks),
    shuffled.  Q/K/V are identical for every B.
    """
    per_seq = SWEEP_CAP // block_size
    return independent(f"sweep_b{block_size}_bf16", [ctx] * batch,
                       (32, 8, 128, block_size, "bf16"),
                       num_blocks=2 * batch * per_seq, max_blocks=per_seq, seed=seed)


def llama13b_long(seed=0, batch=32):
    """LLaMA-13B-like layer: 40/40 heads, d=128, fp16, B=16, ctx 4096."""
    return independent("llama13b_long_f16", [4096] * batch, (40, 40, 128, 16, "f16"),
                       num_blocks=16384, max_blocks=4096 // 16, seed=seed)


def llama13b_beam(seed=0, parents=8, beams=4):
    """8 parents with 4095-token prompts, each forked into 4 beams."""
    return beam_fork("llama13b_beam_f16", parents, beams, 4095, (40, 40, 128, 16, "f16"),
                     num_blocks=16384, max_blocks=4096 // 16, seed=seed)


def prefill_chunks(name, prefix_lens, chunk_lens, shape, num_blocks, max_blocks, seed=0, info=None):
    """Chunked prefill: sequence s holds prefix_lens[s] cached tokens, then the
    step appends its chunk of chunk_lens[s] new tokens (their K/V written like
    any growth) and the chunk's query rows attend over the whole cache.

    The chunk rows' queries come from their own stream: ``info["q_rows"]`` is
    ``[T][Hq][d]`` raw bits, T = sum(chunk_lens), rows grouped by sequence;
    ``info["q_start"]`` holds the S + 1 row offsets.
    """
    Hq, Hkv, d, B, dtype = shape
    log = _Log()
    for s, p in enumerate(prefix_lens):
        if p > 0:
            log.setup.append(("alloc", s, int(p), log.take(int(p))))
    for s, (p, n) in enumerate(zip(prefix_lens, chunk_lens)):
        if p > 0:
            log.step.append(("append", s, int(n), log.take(int(n))))
        else:
            log.step.append(("alloc", s, int(n), log.take(int(n))))
    rs = _streams(seed)
    q_start = np.concatenate([[0], np.cumsum(chunk_lens)]).astype(np.int32)
    q_rows = normal_bits(rs["q_rows"], (int(q_start[-1]), Hq, d), dtype)
    ctx = [int(p) + int(n) for p, n in zip(prefix_lens, chunk_lens)]
    return _finish(name, log, range(len(chunk_lens)), shape, rs, num_blocks, max_blocks,
                   dict(info or {}, ctx=ctx, prefix=list(map(int, prefix_lens)),
                        chunk=list(map(int, chunk_lens)), q_rows=q_rows, q_start=q_start))


PREFILL_CHUNK = 512


def llama31_8b_prefill(seed=0, batch=16):
    """Llama-3.1-8B-like layer (32/8 heads, d=128, bf16, B=16): 16 sequences
    with cached prefixes of U{0..2048} tokens, each appending a 512-token chunk."""
    prefix = _streams(seed)["lengths"].integers(0, 2048, size=batch, endpoint=True)
    per_seq = (2048 + PREFILL_CHUNK) // 16
    return prefill_chunks("llama31_8b_prefill_bf16", prefix.tolist(), [PREFILL_CHUNK] * batch,
                          (32, 8, 128, 16, "bf16"), num_blocks=2 * batch * per_seq, max_blocks=per_seq,
                          seed=seed)


CONFIGS = {
    "tiny": tiny,
    "llama7b": llama7b_mha,
    "gqa": llama31_8b_gqa,
    "gqa_noshare": lambda seed=0: llama31_8b_gqa(seed, share=False),
    "sweep8": lambda seed=0: block_sweep(8, seed),
    "sweep16": lambda seed=0: block_sweep(16, seed),
    "sweep32": lambda seed=0: block_sweep(32, seed),
    "long13b": llama13b_long,
    "beam13b": llama13b_beam,
}

PREFILL_CONFIGS = {
    "prefill_small": lambda seed=0: prefill_chunks("prefill_small", [0, 17, 100, 300, 5], [1, 33, 64, 200, 16],
                                                   (8, 2, 128, 16, "bf16"), 160, 32, seed=seed),
    "prefill_gqa": llama31_8b_prefill,
}
