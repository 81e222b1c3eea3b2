"""Oracle pins against numbers the pages print (worked examples, demo trace)."""
import os

import numpy as np
import pytest
import torch

from oracle import capacity
from oracle.bits import to_f64
from oracle.pool_model import BlockPoolModel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GIB = 2 ** 30


def _lines(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for raw in f:
            line = raw.strip()
            if line and not line.startswith("#"):
                yield line


def _worked():
    out = []
    for line in _lines("worked_examples.txt"):
        lhs, rhs = line.split("=")
        toks = lhs.split()
        approx = toks[0] == "approx"
        if approx:
            toks = toks[1:]
        out.append((line, toks[0], [int(t) for t in toks[1:]], approx, rhs.split()))
    return out


@pytest.mark.parametrize("line,fn,args,approx,rhs", _worked(), ids=lambda x: str(x)[:40])
def test_worked_example(line, fn, args, approx, rhs):
    got = getattr(capacity, fn)(*args)
    if approx:
        value, unit, _, tol = rhs
        assert unit == "GiB"
        assert abs(got / GIB - float(value)) <= float(tol), line
    else:
        assert got == int(rhs[0]), line


def test_example1_ratio_and_concurrency_gap():
    # "Paged Attention", 例子 / 例 1 and 工程现场: 1024 vs 32768 blocks; 896 vs 56 (16x)
    assert 64 * capacity.blocks_needed(256, 16) == 1024
    assert 64 * capacity.blocks_needed(8192, 16) == 32768
    paged = capacity.max_concurrency(28672, 512, 16)
    contiguous = capacity.max_concurrency(28672, 8192, 16)
    assert paged // contiguous == 16 and paged % contiguous == 0


def test_logical_to_physical_figure():
    # "Paged Attention", 直觉: 7 tokens, block_size 4, table [0, 1]:
    # t0..t3 in block 0, t4..t6 in block 1.
    table = [0, 1]
    assert [capacity.logical_to_physical(table, t, 4) for t in range(7)] == \
        [(0, 0), (0, 1), (0, 2), (0, 3), (1, 0), (1, 1), (1, 2)]
    # "vllm-pagedattention", 页表真正解开的…: logical blocks 0,1,2 may sit in 7,1,3
    table = [7, 1, 3]
    assert capacity.logical_to_physical(table, 5, 4) == (1, 1)
    assert capacity.logical_to_physical(table, 11, 4) == (3, 3)


def test_allocator_demo_trace():
    pool = None
    names = {}
    for line in _lines("allocator_trace.txt"):
        lhs, _, rhs = line.partition("->")
        toks = lhs.split()
        want = [int(t) for t in rhs.split()]
        if toks[0] == "pool":
            pool = BlockPoolModel(int(toks[1]), int(toks[2]))
        elif toks[0] == "alloc":
            seq = names.setdefault(toks[1], len(names))
            pool.alloc(seq, int(toks[2]))
            assert pool.block_table(seq) == want, line
        elif toks[0] == "free":
            pool.free(names[toks[1]])
        elif toks[0] == "free_list":
            assert list(pool.free_list) == want, line
        elif toks[0] == "free_count":
            assert len(pool.free_list) == want[0], line
        else:
            raise AssertionError(line)


# -- bit decoding: definitions and a library cross-check ---------------------

@pytest.mark.parametrize("dtype,bits,value", [
    ("bf16", 0x3F80, 1.0), ("bf16", 0xC000, -2.0), ("bf16", 0x0001, 2.0 ** -133),
    ("bf16", 0x7F80, np.inf), ("bf16", 0x3FC0, 1.5),
    ("f16", 0x3C00, 1.0), ("f16", 0x0001, 2.0 ** -24), ("f16", 0xFC00, -np.inf),
    ("f16", 0x3555, (1 + 0x155 / 1024) * 2.0 ** -2),
    ("f32", 0x3F800000, 1.0), ("f32", 0x00000001, 2.0 ** -149),
])
def test_bits_known_patterns(dtype, bits, value):
    arr = np.array([bits], dtype=np.uint32 if dtype == "f32" else np.uint16)
    assert to_f64(arr, dtype)[0] == value


@pytest.mark.parametrize("dtype,tdt,idt", [("bf16", torch.bfloat16, torch.int16),
                                           ("f16", torch.float16, torch.int16),
                                           ("f32", torch.float32, torch.int32)])
def test_bits_match_torch(dtype, tdt, idt):
    g = torch.Generator().manual_seed(1)
    if idt is torch.int16:
        raw = torch.randint(-32768, 32767, (4096,), dtype=torch.int32, generator=g).to(torch.int16)
        bits = raw.numpy().view(np.uint16)
    else:
        raw = torch.randint(-2 ** 31, 2 ** 31 - 1, (4096,), dtype=torch.int64, generator=g).to(torch.int32)
        bits = raw.numpy().view(np.uint32)
    ref = raw.view(tdt).to(torch.float64).numpy()
    got = to_f64(bits, dtype)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
