"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and
this package imports nothing from the product path.  It is a plain, slow,
obviously-correct restatement of what the pages define, computed in float64.

Pages cited throughout (by title and section):

* "Paged Attention" -- daiw.org, 从 Bit 到 AGI, chapter 8 (sections 直觉,
  定义, 例子, 量化, 工程现场：vLLM 块池怎么估容量, 动手试一试).
* "vllm-pagedattention" -- chenyuan1125.github.io (sections 页表真正解开的，
  是“逻辑连续”和“物理连续”; 一块内存，如何安全地属于多条序列;
  它和 FlashAttention 优化的是两张不同的账).
* "vllm-paged-attention-engine" -- aiqz.cc (sections KV缓存之谜,
  分页存储设计：标准册页与索引贴纸, Python 演示).
* "vLLM PagedAttention：大模型推理的显存管理革命" -- horeb.top (sections
  背景, 分配策略, 内存共享：写时复制).

Modules
-------
bits        decoding of raw fp32 / fp16 / bf16 bit patterns to float64
capacity    block counts and KV byte accounting (pinned to printed numbers)
pool_model  block pool: FIFO free list, refcounts, fork, copy-on-write
kv_store    raw-bit KV cache in the [block][kv_head][slot][dim] layout, and
            the host image of swapped-out blocks ([n][K, V][kv_head][slot][dim])
attention   float64 gather-through-block-table decode attention, the
            contiguous-layout variant, and the split-context combine

Parity status: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_*.py`` except where its docstring says "parity unpinned".
"""
