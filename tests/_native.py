"""Replays of a workload's operation log through the native library.

``NativePoolRun`` drives only the host pool (no GPU); ``NativeDeviceRun``
also builds the device caches with pa_write_kv / pa_copy_blocks, exactly as a
serving loop would.  Nothing here imports the oracle.
"""
import numpy as np

import paged_kv_cache_147_amd as P


class NativePoolRun:
    def __init__(self, wl, free_order=None, on_write=None, on_copy=None):
        order = wl.free_order if free_order is None else free_order
        self.pool = P.BlockPool(wl.num_blocks, wl.block_size, order)
        self.slots, self.cow = [], []
        self.on_write, self.on_copy = on_write, on_copy
        for op in wl.setup_ops:
            self.slots.append(self.apply(op))
        self.step_slots = []
        for op in wl.step_ops:
            s = self.apply(op, step=True)
            self.slots.append(s)

    def apply(self, op, step=False):
        kind = op[0]
        if kind == "alloc":
            _, seq, n, r0 = op
            slots = self.pool.alloc(seq, n)
            if self.on_write:
                self.on_write(slots, r0, step)
            return list(slots)
        if kind == "append":
            _, seq, n, r0 = op
            slots, cow = self.pool.extend(seq, n)
            if cow is not None:
                self.cow.append(cow)
                if self.on_copy:
                    self.on_copy(cow, step)
            if self.on_write:
                self.on_write(slots, r0, step)
            return list(slots)
        if kind == "fork":
            self.pool.fork(op[1], op[2])
            return []
        if kind == "free":
            self.pool.free(op[1])
            return []
        raise ValueError(kind)

    def tables(self, wl):
        return self.pool.block_tables(wl.batch, wl.max_blocks)


_TORCH = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}
_INT = {"f32": "int32", "f16": "int16", "bf16": "int16"}
# quiet-NaN bit patterns: never-written slots must never reach an output
_POISON = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0}


def device_tensor(bits, dtype, device):
    """Raw uint16/uint32 bits -> device tensor of the workload dtype."""
    import torch
    signed = bits.view(np.int16 if bits.dtype == np.uint16 else np.int32)
    return torch.from_numpy(np.ascontiguousarray(signed)).to(device).view(getattr(torch, _TORCH[dtype]))


class NativeDeviceRun:
    """Pool replay plus device caches built by pa_write_kv / pa_copy_blocks.

    The step's writes are recorded separately (``step_writes``) so a timed
    decode step can re-issue them.
    """

    def __init__(self, wl, device="cuda", free_order=None):
        import torch
        self.wl, self.device = wl, device
        shape = (wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
        idt = getattr(torch, _INT[wl.dtype])
        self.k_cache = torch.full(shape, _POISON[wl.dtype], dtype=idt, device=device).view(
            getattr(torch, _TORCH[wl.dtype]))
        self.v_cache = torch.full(shape, _POISON[wl.dtype], dtype=idt, device=device).view(
            getattr(torch, _TORCH[wl.dtype]))
        self.k_rows = device_tensor(wl.k_rows, wl.dtype, device)
        self.v_rows = device_tensor(wl.v_rows, wl.dtype, device)
        self.step_writes = []   # (slots tensor, row0, n)
        self.step_copies = []   # (src, dst)
        self.pool_run = NativePoolRun(wl, free_order, on_write=self._write, on_copy=self._copy)
        tables, ctx = self.pool_run.tables(wl)
        self.tables = torch.from_numpy(tables).to(device)
        self.ctx = torch.from_numpy(ctx).to(device)
        self.ctx_host = ctx
        self.q = device_tensor(wl.q, wl.dtype, device)
        torch.cuda.synchronize()

    def _write(self, slots, r0, step):
        import torch
        n = len(slots)
        if n == 0:
            return
        st = torch.from_numpy(np.asarray(slots, dtype=np.int64)).to(self.device)
        P.pa_write_kv(self.k_cache, self.v_cache, self.k_rows[r0:r0 + n], self.v_rows[r0:r0 + n], st)
        if step:
            self.step_writes.append((st, r0, n))

    def _copy(self, pair, step):
        import torch
        pairs = torch.tensor([list(pair)], dtype=torch.int32, device=self.device)
        P.pa_copy_blocks(self.k_cache, self.v_cache, pairs)
        if step:
            self.step_copies.append(pair)

    def decode(self, out_dtype=None, partition_size=0, max_ctx=0, tables=None, ctx=None):
        import torch
        wl = self.wl
        dt = out_dtype or torch.float32
        out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), dtype=dt, device=self.device)
        P.pa_decode(out, self.q, self.k_cache, self.v_cache,
                    self.tables if tables is None else tables, self.ctx if ctx is None else ctx,
                    wl.scale, max_ctx=max_ctx, partition_size=partition_size)
        return out

    def cache_bits(self):
        import torch
        idt = getattr(torch, _INT[self.wl.dtype])
        nbits = np.uint16 if self.wl.dtype != "f32" else np.uint32
        k = self.k_cache.view(idt).cpu().numpy().view(nbits)
        v = self.v_cache.view(idt).cpu().numpy().view(nbits)
        return k, v
