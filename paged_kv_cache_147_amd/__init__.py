"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The compute path lives in ``libpagedkv.so`` (C ABI: include/pagedkv.h); this
package is its Python binding.  Build the library with
``python paged_kv_cache_147_amd/build.py``.
"""
from ._lib import (EXPORTED, PA_BF16, PA_F16, PA_F32, PA_FP8_E4M3, BlockPool, PagedKVError,  # noqa: F401
                   current_stream, pa_copy_blocks, pa_decode, pa_decode_contiguous,
                   pa_decode_static, pa_decode_static_max_bytes, pa_decode_validate,
                   pa_decode_workspace_bytes, pa_prefill, pa_swap_in,
                   pa_swap_out, pa_write_kv, pa_write_kv_fp8, raw)
